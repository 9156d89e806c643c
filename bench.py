#!/usr/bin/env python3
"""SplitZip codec benchmark on one MI355X.

One step = one pass of the whole hot path over one batch: encode the
Llama-3-8B-shaped KV cache (32 layers x {K,V} x 8 KV heads x 128 dims x
8192 tokens = 536,870,912 BF16 values, 1 GiB) into a SplitZip stream and
decode it back.  Inputs are generated on the device and resident in HBM
before the timed region; the codebook is calibrated offline (host, untimed)
on a layer-0 calibration tensor.

Prints one JSON line:
  value       uncompressed GB/s of the round trip = 2 N bytes / (encode + decode time)
  encode_GBps / decode_GBps    the two directions, timed separately
  ratio, escape_rate           compression ratio (input bytes / stream bytes) and E / N
  roofline    the dominant kernel's algorithmic bytes / average duration
              (HIP events recorded on the launch stream by the library's
              instrumentation) against the 8 TB/s HBM peak
  cpu_baseline the CPU oracle (single thread) on a bounded sample
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
WORKLOAD = "llama3_8b_kv"


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=WORKLOAD)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--core-only", action="store_true",
                   help="time only the encode+decode step (no calibration, format or transfer sections), "
                        "e.g. under a profiler")
    p.add_argument("--cpu-sample-log2", type=int, default=29,
                   help="elements of the workload the CPU oracle encodes and decodes (log2; the default, 2^29, is the "
                        "whole Llama-3-8B cache, about 12 s of single-core work)")
    p.add_argument("--ingest-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_BYTES"),
                   help="record HBM traffic per kernel from two rocprofv3 --pmc runs of this "
                        "benchmark (FETCH_SIZE, WRITE_SIZE) into profiles/traffic.json and exit")
    return p.parse_args()


def kernel_source_hash() -> str:
    """Hash of the kernel sources (every file under csrc/, in name order) with
    comments and blank space removed, so that recorded counters stay tied to
    the code, not to its commentary."""
    import re
    csrc = os.path.join(ROOT, "fp8_kv_cache_sz_amd", "csrc")
    src = ""
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, name)) as f:
                src += f.read() + "\n"
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


TRAFFIC_PATH = os.path.join(ROOT, "profiles", "traffic.json")
COPY_KERNEL = "sz_ref_copy"


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters, if they were taken
    on the current kernel source; otherwise None."""
    if not os.path.exists(TRAFFIC_PATH):
        return None
    with open(TRAFFIC_PATH) as f:
        rec = json.load(f)
    entry = rec.get(workload, {}).get(kernel)
    if not entry or entry.get("source_hash") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


# kernel templates, by their first template argument -> the names the
# library's instrumentation uses
LAUNCH_NAMES = {
    "sz_enc_dense_bf16<1>": "sz_enc_dense_bf16", "sz_enc_dense_bf16<2>": "sz_enc_dense_top8",
    "sz_enc_dense_bf16<3>": "sz_enc_dense_top15s", "sz_enc_compact<0>": "sz_enc_compact",
    "sz_enc_compact<1>": "sz_enc_compact", "sz_cal_hist<0>": "sz_cal_hist_bf16",
    "sz_cal_hist<1>": "sz_cal_hist_e5m2", "sz_cal_select<0>": "sz_cal_select",
    "sz_cal_select<1>": "sz_cal_select",
}


def short_kernel_name(name: str) -> str:
    """'void sz::(anonymous namespace)::sz_cal_hist<0>(...)' -> 'sz_cal_hist_bf16'
    (the launch name the library's instrumentation records)."""
    name = name.replace("(anonymous namespace)::", "").split("(")[0]
    if name.startswith("void "):
        name = name[5:]
    name = name.strip().split("::")[-1]
    base = name.split("<")[0]
    first = name[len(base) + 1:].split(",")[0].rstrip(">").strip() if "<" in name else ""
    return LAUNCH_NAMES.get("%s<%s>" % (base, first), base)


def _pmc_per_kernel(csv_path, counter):
    """{kernel short name: [values in KiB per dispatch]} from a rocprofv3 counter CSV."""
    import csv
    out = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = short_kernel_name(r["Kernel_Name"])
            out.setdefault(name, []).append(float(r["Counter_Value"]))
    return out


def ingest_pmc(workload, fetch_csv, write_csv, copy_bytes):
    """Turns FETCH_SIZE / WRITE_SIZE runs into HBM bytes per launch of every
    library kernel.  Each counter is scaled by what it reads for the plain
    device copy of `copy_bytes` bytes in the same run (the largest copy
    dispatch), and the record is tied to the current kernel source."""
    fetch = _pmc_per_kernel(fetch_csv, "FETCH_SIZE")
    write = _pmc_per_kernel(write_csv, "WRITE_SIZE")
    f_scale = copy_bytes / (max(fetch[COPY_KERNEL]) * 1024.0)
    w_scale = copy_bytes / (max(write[COPY_KERNEL]) * 1024.0)
    rec = {}
    if os.path.exists(TRAFFIC_PATH):
        with open(TRAFFIC_PATH) as f:
            rec = json.load(f)
    entry = {}
    for k in sorted(set(fetch) & set(write)):
        if not k.startswith("sz_"):
            continue
        fk = sum(fetch[k]) / len(fetch[k])
        wk = sum(write[k]) / len(write[k])
        entry[k] = {"source_hash": kernel_source_hash(),
                    "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                    "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
                    "bytes_per_launch": int(fk * 1024 * f_scale + wk * 1024 * w_scale)}
    rec[workload] = entry
    with open(TRAFFIC_PATH, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    return entry


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), else the machine type."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(x_dev, cb, dtype, log2_sample):
    import oracle
    import synth
    n = min(x_dev.numel(), 1 << log2_sample)
    bits = synth.as_bits_numpy(x_dev[:n])
    cbn = list(cb.exps)
    t0 = time.perf_counter()
    stream = oracle.encode(bits, dtype, cbn)
    t1 = time.perf_counter()
    back = oracle.decode(stream, dtype, n)
    t2 = time.perf_counter()
    assert (back == bits).all()
    elem = 2 if dtype == 0 else 1
    gbps = 2 * n * elem / (t2 - t0) / 1e9
    return {
        "value": round(gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": "first %d elements (%d MiB) of the workload; one encode (%.2f s) and one "
                  "decode (%.2f s), single-threaded C, host %s, %d logical CPUs"
                  % (n, n * elem >> 20, t1 - t0, t2 - t1, cpu_model(), os.cpu_count()),
    }


def main():
    args = parse_args()
    if args.ingest_pmc:
        f_csv, w_csv, copy_bytes = args.ingest_pmc
        print(json.dumps(ingest_pmc(args.workload, f_csv, w_csv, int(copy_bytes)), indent=1))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the SplitZip codec has no cross-GPU step on this path "
              "(each GPU encodes/decodes its own shard); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import fp8_kv_cache_sz_amd as sz
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x, dtype = synth.workload(args.workload, device=dev)
    cal = synth.calibration_tensor(args.workload, device="cpu")
    cb = sz.calibrate(cal)
    n = x.numel()
    elem = 2 if dtype == 0 else 1
    cap = sz.encoded_size(dtype, n, n)
    buf = torch.empty(cap, dtype=torch.uint8, device=dev)
    ws = sz.workspace(dtype, n, dev)
    ws_dec = sz.workspace(dtype, n, dev)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream(dev)

    def encode():
        sz.encode(x, cb, out=buf, ws=ws, sync=False)

    def decode(in_bytes):
        sz.decode(buf, dtype, n, out=y, ws=ws_dec, check=False, in_bytes=in_bytes)

    # first pass: learn the stream size, check the round trip
    encode()
    torch.cuda.synchronize()
    escapes = sz.read_escape_count(buf)
    size = sz.encoded_size(dtype, n, escapes)
    decode(size)
    torch.cuda.synchronize()
    if int(ws_dec[:4].cpu().view(torch.int32)[0]) != 0 or not torch.equal(
            y.view(torch.uint8), x.view(torch.uint8)):
        print("round trip mismatch", file=sys.stderr)
        sys.exit(1)

    for _ in range(args.warmup):
        encode()
        decode(size)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        encode()
        decode(size)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = 2 * n * elem / (ms_per_step * 1e-3) / 1e9

    # per-direction timing (events on the launch stream)
    def time_loop(fn, reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) / reps

    reps = max(5, args.steps)
    enc_ms = time_loop(encode, reps)
    dec_ms = time_loop(lambda: decode(size), reps)

    # per-kernel durations through the library's event instrumentation
    sz.profile_enable(True)
    for _ in range(reps):
        encode()
        decode(size)
    stats = sz.profile_collect()
    sz.profile_enable(False)
    per_kernel = {k: {"launches": c, "avg_ms": round(ms / c, 5)} for k, (c, ms) in stats.items()}
    dense = {k: v for k, v in per_kernel.items() if k.startswith(("sz_enc_dense", "sz_dec_bf16", "sz_dec_e5m2"))}
    dominant = max(dense, key=lambda k: dense[k]["avg_ms"])
    alg_bytes = int(3.5 * n) + 3 * escapes if dtype == 0 else int(1.875 * n) + 3 * escapes
    avg_s = dense[dominant]["avg_ms"] * 1e-3
    achieved = alg_bytes / avg_s / 1e9
    traffic = load_traffic(dominant, args.workload)

    calibration = formats = transfer = None
    if not args.core_only:
        calibration, formats, transfer = extra_sections(sz, x, cb, dtype, n, elem, buf, ws, ws_dec, y, dev,
                                                        time_loop, reps, enc_ms, dec_ms)

    # the library's streaming copy of the same bytes (non-temporal dwordx4, the
    # fastest plain copy shape), as the practical streaming ceiling
    alg_per_direction = alg_bytes // 2 // 16 * 16          # read half, write half
    src = torch.empty(alg_per_direction, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    # timed per launch through the library's event instrumentation, as the
    # codec kernels are, so that host gaps between launches do not count
    sz.reference_copy(src, dst)
    sz.profile_enable(True)
    for _ in range(reps):
        sz.reference_copy(src, dst)
    launches, total_ms = sz.profile_collect()["sz_ref_copy"]
    sz.profile_enable(False)
    copy_ms = total_ms / launches
    copy_gbps = 2 * src.numel() / (copy_ms * 1e-3) / 1e9
    del src, dst

    result = {
        "metric": "encode/decode GB/s (uncompressed) + % of 8 TB/s HBM peak; compression ratio",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16" if dtype == 0 else "u8",
        "data": "synthetic",
        "config": {"workload": args.workload, "description": synth.DESCRIPTION[args.workload],
                   "elements": n, "bytes": n * elem, "codebook": list(cb.exps),
                   "step": "encode + decode of the whole tensor"},
        "encode_GBps": round(n * elem / (enc_ms * 1e-3) / 1e9, 2),
        "decode_GBps": round(n * elem / (dec_ms * 1e-3) / 1e9, 2),
        "encode_ms": round(enc_ms, 4),
        "decode_ms": round(dec_ms, 4),
        "ratio": round(n * elem / size, 6),
        "escape_rate": round(escapes / n, 6),
        "escapes": escapes,
        "stream_bytes": size,
        "kernels": per_kernel,
        "calibration": calibration,
        "formats": formats,
        "transfer": transfer,
        "hbm": hbm_rates(per_kernel, args.workload),
        "page_numbers": {"encode_GBps": 613.3, "decode_GBps": 2181.8, "ratio": 1.324,
                         "hardware": "not named on the page", "workload": "real BF16 activations",
                         "note": "context only, not this workload or machine"},
        "copy_GBps": round(copy_gbps, 1),
        "copy_bytes": alg_per_direction,
        "copy_kernel": "sz_ref_copy: one non-temporal dwordx4 per lane, 4 KB per 256-lane workgroup",
        "dominant_vs_copy": round(achieved / copy_gbps, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": dominant,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(x, cb, dtype, args.cpu_sample_log2)
    print(json.dumps(result), flush=True)



def hbm_rates(per_kernel, workload):
    """Measured HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, when
    taken on the current kernel source) over this run's average duration."""
    out = {}
    for k, v in per_kernel.items():
        t = load_traffic(k, workload)
        if t:
            gbps = t / (v["avg_ms"] * 1e-3) / 1e9
            out[k] = {"bytes_per_launch": t, "GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    return out or None


def extra_sections(sz, x, cb, dtype, n, elem, buf, ws, ws_dec, y, dev, time_loop, reps, enc_ms, dec_ms):
    """Rows beyond the encode+decode step: on-device calibration, the
    ablation formats and the chunked transfer."""
    import torch
    # on-device calibration (per-tensor codebook at run time): the whole
    # tensor, and every 16th 64K block; then encode with the device codebook
    cal_ws = torch.empty(sz._native.sz_calibrate_workspace_size(dtype), dtype=torch.uint8, device=dev)
    d_cb = torch.zeros(sz.DEVICE_CODEBOOK_BYTES, dtype=torch.uint8, device=dev)
    cal_full_ms = time_loop(lambda: sz.calibrate_device(x, 1, out=d_cb, ws=cal_ws), reps)
    cal_s16_ms = time_loop(lambda: sz.calibrate_device(x, 16, out=d_cb, ws=cal_ws), reps)
    sz.calibrate_device(x, 1, out=d_cb, ws=cal_ws)
    enc_dcb_ms = time_loop(lambda: sz.encode(x, d_cb, out=buf, ws=ws, sync=False), reps)
    torch.cuda.synchronize()
    if int(ws[:4].cpu().view(torch.int32)[0]) != 0:
        print("device codebook rejected", file=sys.stderr)
        sys.exit(1)
    dyn_cb = sz.codebook_from_device(d_cb)
    calibration = {
        "device_full_ms": round(cal_full_ms, 4),
        "device_full_read_GBps": round(n * elem / (cal_full_ms * 1e-3) / 1e9, 1),
        "device_every16_ms": round(cal_s16_ms, 4),
        "encode_with_device_codebook_ms": round(enc_dcb_ms, 4),
        "calibrate_plus_encode_GBps": round(n * elem / ((cal_full_ms + enc_dcb_ms) * 1e-3) / 1e9, 1),
        "per_tensor_codebook": list(dyn_cb.exps),
        "per_tensor_codebook_equals_offline": list(dyn_cb.exps) == list(cb.exps),
    }

    # the page's ablation formats on the same tensor (BF16 only): Top-8 and
    # Top-15 with a sentinel code, against the Top-16 numbers above
    formats = None
    if dtype == 0:
        formats = {}
        for name, fmt in (("top8", sz.TOP8), ("top15_sentinel", sz.TOP15S)):
            cap_f = sz.encoded_size(dtype, n, n, fmt)
            buf_f = torch.empty(cap_f, dtype=torch.uint8, device=dev)
            _, size_f, esc_f = sz.encode(x, cb, out=buf_f, ws=ws, fmt=fmt)
            sz.decode(buf_f, dtype, n, out=y, ws=ws_dec, in_bytes=size_f, fmt=fmt)
            if not torch.equal(y.view(torch.uint8), x.view(torch.uint8)):
                print("round trip mismatch (%s)" % name, file=sys.stderr)
                sys.exit(1)
            e_ms = time_loop(lambda: sz.encode(x, cb, out=buf_f, ws=ws, sync=False, fmt=fmt), reps)
            d_ms = time_loop(lambda: sz.decode(buf_f, dtype, n, out=y, ws=ws_dec, check=False,
                                               in_bytes=size_f, fmt=fmt), reps)
            formats[name] = {
                "encode_GBps": round(n * elem / (e_ms * 1e-3) / 1e9, 1),
                "decode_GBps": round(n * elem / (d_ms * 1e-3) / 1e9, 1),
                "ratio": round(n * elem / size_f, 6),
                "escape_rate": round(esc_f / n, 6),
                "top16_decode_speedup": round(d_ms / dec_ms, 3),
                "top16_encode_speedup": round(e_ms / enc_ms, 3),
            }
            del buf_f

    # chunked transfer through pinned host memory (PCIe both ways stands in
    # for the prefill-to-decode link): raw against SplitZip-compressed, one
    # 2^24-value chunk (one Llama-3-8B layer, K and V) at a time
    chunk = min(n, 1 << 24)
    staging = sz.transfer_buffers(dtype, n, chunk, 3, dev)
    runs = {}
    for mode, book in (("raw", None), ("splitzip", cb)):
        best = None
        for _ in range(3):
            _, st = sz.transfer(x, chunk, book, depth=3, out=y, staging=staging)
            if best is None or st["total_ms"] < best["total_ms"]:
                best = st
        if not torch.equal(y.view(torch.uint8), x.view(torch.uint8)):
            print("transfer mismatch (%s)" % mode, file=sys.stderr)
            sys.exit(1)
        runs[mode] = best
    # the codec's own time per chunk (encode + decode of one chunk on the
    # device, no link), and its share of the compressed transfer's wall time
    xc = x[:chunk]
    bc = torch.empty(sz.encoded_size(dtype, chunk, chunk), dtype=torch.uint8, device=dev)
    wc_e, wc_d = sz.workspace(dtype, chunk, dev), sz.workspace(dtype, chunk, dev)
    yc = torch.empty_like(xc)

    def chunk_codec():
        sz.encode(xc, cb, out=bc, ws=wc_e, sync=False)
        sz.decode(bc, dtype, chunk, out=yc, ws=wc_d, check=False)
    codec_ms = time_loop(chunk_codec, reps)
    del bc, wc_e, wc_d, yc
    transfer = {
        "link": "PCIe via pinned host memory, device->host then host->device, pipelined (depth 3)",
        "chunk_elems": chunk,
        "chunks": runs["raw"]["chunks"],
        "raw_ms": round(runs["raw"]["total_ms"], 3),
        "raw_GBps": round(n * elem / (runs["raw"]["total_ms"] * 1e-3) / 1e9, 2),
        "splitzip_ms": round(runs["splitzip"]["total_ms"], 3),
        "splitzip_GBps": round(n * elem / (runs["splitzip"]["total_ms"] * 1e-3) / 1e9, 2),
        "wire_bytes": runs["splitzip"]["wire_bytes"],
        "wire_ratio": round(n * elem / runs["splitzip"]["wire_bytes"], 6),
        "speedup": round(runs["raw"]["total_ms"] / runs["splitzip"]["total_ms"], 4),
        "codec_ms_per_chunk": round(codec_ms, 4),
        "codec_share": round(runs["splitzip"]["chunks"] * codec_ms / runs["splitzip"]["total_ms"], 4),
    }
    del staging
    return calibration, formats, transfer


if __name__ == "__main__":
    main()
