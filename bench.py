#!/usr/bin/env python3
"""SplitZip codec benchmark on one MI355X.

One step = one pass of the whole hot path over one batch: encode a KV
payload into a SplitZip stream and decode it back.  The headline workload is
the largest single-GPU one, the long-context transfer payload (28 layers x
{K,V} x 4 KV heads x 128 dims x 65,536 tokens = 1,879,048,192 BF16 values,
3.76 GB).  Inputs are generated on the device and resident in HBM before the
timed region; each workload's codebook is calibrated offline (host,
untimed) on its own calibration tensor.

Prints one JSON line:
  value        uncompressed GB/s of the round trip = 2 N bytes / ms_per_step
               (K steps timed with perf_counter, synchronised on both sides)
  encode / decode   per direction, median and min of >= 20 runs, each
               bracketed by its own pair of HIP events on the launch stream
  ratio, escape_rate   input bytes / stream bytes, and E / N
  roofline     the dominant kernel's algorithmic bytes / its average duration
               (HIP events recorded on the launch stream by the library's
               instrumentation) against the 8 TB/s HBM peak
  copy, encoder_pattern, decoder_pattern   in-run streaming references:
               the library's plain copy, and its copies of the dense
               encoder's and the span decoder's memory patterns (same grid,
               lanes and memory instructions, trivial arithmetic) with the
               codec kernel's time relative to them
  cpu_baseline the CPU oracle (single thread) on a bounded sample
  parity       the whole GPU stream equals the oracle's stream of the whole
               tensor, byte for byte
  configs      the same per-direction figures, ratio, escape rate, oracle
               baseline and parity verdict for every workload
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
WORKLOAD = "longctx_kv"
# every workload the configs key reports, in this order
ALL_WORKLOADS = ("kv1m", "llama3_8b_kv", "longctx_kv", "stress_t3", "stress_oneexp", "stress_random",
                 "llama3_8b_kv_e5m2")


def parse_args(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=WORKLOAD)
    p.add_argument("--configs", default="all",
                   help="workloads for the per-config rows: 'all', 'none' or a comma-separated list")
    p.add_argument("--runs", type=int, default=20,
                   help="event-timed runs per direction for the median and min (at least 20)")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the oracle leg (baseline timings and the whole-stream parity checks)")
    p.add_argument("--core-only", action="store_true",
                   help="time only the encode+decode step of the headline workload (no per-config rows, "
                        "calibration, format or transfer sections), e.g. under a profiler")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the calibration, format and transfer sections (the per-config rows stay)")
    p.add_argument("--cpu-sample-log2", type=int, default=29,
                   help="elements of the headline workload the oracle baseline encodes and decodes (log2; "
                        "2^29 is about 12 s of single-core work)")
    p.add_argument("--config-sample-log2", type=int, default=25,
                   help="elements of each per-config row's oracle baseline sample (log2)")
    p.add_argument("--ingest-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_BYTES"),
                   help="record HBM traffic per kernel from two rocprofv3 --pmc runs of this "
                        "benchmark (FETCH_SIZE, WRITE_SIZE) into profiles/traffic.json and exit")
    args = p.parse_args(argv)
    args.runs = max(20, args.runs)
    return args


# the source file that defines each kernel family (every kernel also
# includes common.hpp)
KERNEL_SOURCES = (("sz_enc_", "encode.hip"), ("sz_dec_", "decode.hip"), ("sz_ref_join", "decode.hip"),
                  ("sz_cal_", "calibrate.hip"), ("sz_copy_", "transfer.hip"), ("sz_ref_", "runtime.hip"))


def kernel_source_hash(kernel: str) -> str:
    """Hash of the source that defines `kernel` and of common.hpp, with
    comments and blank space removed, so that recorded counters stay tied to
    that kernel's code, not to its commentary or to other kernels."""
    import re
    csrc = os.path.join(ROOT, "fp8_kv_cache_sz_amd", "csrc")
    files = ["common.hpp"] + [f for p, f in KERNEL_SOURCES if kernel.startswith(p)][:1]
    if len(files) == 1:
        files = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".hpp")))
    src = ""
    for name in files:
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
    if not entry or entry.get("source_hash") != kernel_source_hash(kernel):
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
        entry[k] = {"source_hash": kernel_source_hash(k),
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


def alg_bytes(dtype, n, escapes):
    """Bytes the method must move per direction: BF16 2 B in, 0.5 B of codes
    and 1 B of sign/mantissa per element; E5M2 1 + 0.5 + 0.375 B; 3 B per
    escape record."""
    return (int(3.5 * n) if dtype == 0 else int(1.875 * n)) + 3 * escapes


def median(v):
    v = sorted(v)
    m = len(v) // 2
    return v[m] if len(v) % 2 else 0.5 * (v[m - 1] + v[m])


# ---------------------------------------------------------------------------
# The oracle leg: baseline timings of the single-threaded CPU oracle on a
# bounded sample, and whole-stream parity checks against it
# ---------------------------------------------------------------------------
def oracle_baseline(bits, cb_exps, dtype, n_sample):
    """Times one oracle encode and one decode of the first n_sample elements
    (single thread, nothing else running on the host)."""
    import oracle
    part = bits[:n_sample]
    t0 = time.perf_counter()
    stream = oracle.encode(part, dtype, cb_exps)
    t1 = time.perf_counter()
    back = oracle.decode(stream, dtype, part.size)
    t2 = time.perf_counter()
    assert (back == part).all()
    elem = 2 if dtype == 0 else 1
    return {
        "value": round(2 * part.size * elem / (t2 - t0) / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": "first %d elements (%d MiB) of the workload; one encode (%.2f s) and one decode (%.2f s), "
                  "single-threaded C, host %s, %d logical CPUs"
                  % (part.size, part.size * elem >> 20, t1 - t0, t2 - t1, cpu_model(), os.cpu_count()),
    }


def oracle_parity(bits, cb_exps, dtype, gpu_stream):
    """The GPU's stream of the whole tensor against the oracle's, byte for
    byte; returns (equal, detail)."""
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    expect = oracle.encode(bits, dtype, cb_exps)
    secs = time.perf_counter() - t0
    if expect.size != gpu_stream.size:
        return False, "size %d, oracle %d" % (gpu_stream.size, expect.size)
    diff = np.flatnonzero(expect != gpu_stream)
    if diff.size:
        return False, "%d bytes differ, first at %d" % (diff.size, int(diff[0]))
    return True, "%d bytes equal (oracle encode %.1f s)" % (expect.size, secs)


def parity_all(jobs, workers=4):
    """Whole-stream parity of every collected workload, the oracle encodes
    running in parallel threads (the ctypes calls release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=workers) as pool:
        futs = {name: pool.submit(oracle_parity, *job) for name, job in jobs.items()}
        return {name: f.result() for name, f in futs.items()}


# ---------------------------------------------------------------------------
# GPU measurement
# ---------------------------------------------------------------------------
class Codec:
    """One workload resident on the device with its stream buffer, encode and
    decode workspaces and output tensor."""

    def __init__(self, sz, name, dev):
        import synth
        import torch
        self.name = name
        self.x, self.dtype = synth.workload(name, device=dev)
        self.cal = synth.calibration_tensor(name, device="cpu")
        self.cb = sz.calibrate(self.cal)
        self.n = self.x.numel()
        self.elem = 2 if self.dtype == 0 else 1
        self.sz = sz
        self.buf = torch.empty(sz.encoded_size(self.dtype, self.n, self.n), dtype=torch.uint8, device=dev)
        self.ws = sz.workspace(self.dtype, self.n, dev)
        self.ws_dec = sz.decode_workspace(self.dtype, self.n, dev)
        self.y = torch.empty_like(self.x)
        self.stream = torch.cuda.current_stream(dev)
        # first pass: learn the stream size, check the round trip
        self.encode()
        torch.cuda.synchronize()
        self.escapes = sz.read_escape_count(self.buf)
        self.size = sz.encoded_size(self.dtype, self.n, self.escapes)
        self.decode()
        torch.cuda.synchronize()
        if int(self.ws_dec[:4].cpu().view(torch.int32)[0]) != 0 or not torch.equal(
                self.y.view(torch.uint8), self.x.view(torch.uint8)):
            raise SystemExit("round trip mismatch on %s" % name)

    def encode(self):
        self.sz.encode(self.x, self.cb, out=self.buf, ws=self.ws, sync=False)

    def decode(self):
        self.sz.decode(self.buf, self.dtype, self.n, out=self.y, ws=self.ws_dec, check=False,
                       in_bytes=getattr(self, "size", None))

    def time_runs(self, fn, runs, warmup=3):
        """Per-run milliseconds: each run bracketed by its own event pair on
        the launch stream."""
        import torch
        for _ in range(warmup):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
        for a, b in ev:
            a.record(self.stream)
            fn()
            b.record(self.stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    def directions(self, runs):
        """Median and min of the encode and decode times, GB/s (uncompressed)
        and the share of the 8 TB/s peak on algorithmic bytes."""
        out = {}
        alg = alg_bytes(self.dtype, self.n, self.escapes)
        for d, fn in (("encode", self.encode), ("decode", self.decode)):
            t = self.time_runs(fn, runs)
            med, lo = median(t), min(t)
            out[d] = {"median_ms": round(med, 5), "min_ms": round(lo, 5), "runs": len(t),
                      "GBps": round(self.n * self.elem / (med * 1e-3) / 1e9, 2),
                      "GBps_best": round(self.n * self.elem / (lo * 1e-3) / 1e9, 2),
                      "alg_GBps": round(alg / (med * 1e-3) / 1e9, 1),
                      "frac_of_peak": round(alg / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        return out

    def kernel_stats(self, reps):
        """Average duration of every kernel launch through the library's event
        instrumentation."""
        sz = self.sz
        sz.profile_enable(True)
        for _ in range(reps):
            self.encode()
            self.decode()
        stats = sz.profile_collect()
        sz.profile_enable(False)
        return {k: {"launches": c, "avg_ms": round(ms / c, 5)} for k, (c, ms) in stats.items()}

    def host_copies(self):
        """The input's raw bits and the encoded stream, on the host."""
        import synth
        return synth.as_bits_numpy(self.x), self.buf[:self.size].cpu().numpy()

    def summary(self):
        return {"elements": self.n, "bytes": self.n * self.elem, "escapes": self.escapes,
                "escape_rate": round(self.escapes / self.n, 6), "stream_bytes": self.size,
                "ratio": round(self.n * self.elem / self.size, 6),
                "alg_bytes_per_direction": alg_bytes(self.dtype, self.n, self.escapes)}


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
    oracle_leg = not args.no_cpu_baseline
    if args.core_only or args.configs == "none":
        config_names = []
    elif args.configs == "all":
        config_names = [w for w in ALL_WORKLOADS if w != args.workload]
    else:
        config_names = [w for w in args.configs.split(",") if w and w != args.workload]
    parity_jobs = {}

    # ---- the headline workload: the timed steps --------------------------
    c = Codec(sz, args.workload, dev)
    n, dtype, elem = c.n, c.dtype, c.elem
    for _ in range(args.warmup):
        c.encode()
        c.decode()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        c.encode()
        c.decode()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = 2 * n * elem / (ms_per_step * 1e-3) / 1e9

    dirs = c.directions(args.runs)
    per_kernel = c.kernel_stats(args.runs)
    dense = {k: v for k, v in per_kernel.items() if k.startswith(("sz_enc_dense", "sz_dec_bf16", "sz_dec_e5m2"))}
    dominant = max(dense, key=lambda k: dense[k]["avg_ms"])
    alg = alg_bytes(dtype, n, c.escapes)
    achieved = alg / (dense[dominant]["avg_ms"] * 1e-3) / 1e9
    traffic = load_traffic(dominant, args.workload)

    calibration = formats = transfer = None
    if not args.core_only and not args.no_extras:
        calibration, formats, transfer = extra_sections(sz, c, args.runs, dirs)
    copy = reference_copy_rate(sz, alg, args.runs, dev)
    pattern = encoder_pattern_rate(sz, c.x, dtype, n, args.runs, per_kernel)
    dpattern = decoder_pattern_rate(sz, c, args.runs, per_kernel)

    headline_bits = headline_stream = None
    if oracle_leg:
        headline_bits, headline_stream = c.host_copies()
        parity_jobs[args.workload] = (headline_bits, list(c.cb.exps), dtype, headline_stream)
    head_summary = c.summary()
    del c
    torch.cuda.empty_cache()

    # ---- every other workload: per-direction rows -------------------------
    configs = {args.workload: dict(head_summary, **dirs, kernels=per_kernel, encoder_pattern=pattern,
                                  decoder_pattern=dpattern)}
    config_samples = {}
    for name in config_names:
        print("config %s" % name, file=sys.stderr, flush=True)
        w = Codec(sz, name, dev)
        row = dict(w.summary(), **w.directions(args.runs))
        row["kernels"] = w.kernel_stats(args.runs)
        row["encoder_pattern"] = encoder_pattern_rate(sz, w.x, w.dtype, w.n, args.runs, row["kernels"])
        row["decoder_pattern"] = decoder_pattern_rate(sz, w, args.runs, row["kernels"])
        configs[name] = row
        if oracle_leg:
            bits, stream = w.host_copies()
            parity_jobs[name] = (bits, list(w.cb.exps), w.dtype, stream)
            config_samples[name] = (bits, list(w.cb.exps), w.dtype)
        del w
        torch.cuda.empty_cache()

    # ---- the oracle leg ----------------------------------------------------
    cpu = None
    parity = None
    if oracle_leg:
        print("oracle baselines", file=sys.stderr, flush=True)
        cpu = oracle_baseline(headline_bits, list(parity_jobs[args.workload][1]), dtype,
                              min(n, 1 << args.cpu_sample_log2))
        configs[args.workload]["cpu_baseline"] = cpu
        for name, (bits, cbx, dt) in config_samples.items():
            configs[name]["cpu_baseline"] = oracle_baseline(bits, cbx, dt, min(bits.size, 1 << args.config_sample_log2))
        print("whole-stream parity of %d workloads" % len(parity_jobs), file=sys.stderr, flush=True)
        verdicts = parity_all(parity_jobs)
        for name, (ok, detail) in verdicts.items():
            configs[name]["parity"] = ok
            configs[name]["parity_detail"] = detail
        parity = all(ok for ok, _ in verdicts.values())

    enc, dec = dirs["encode"], dirs["decode"]
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
                   "elements": n, "bytes": n * elem, "codebook": list(parity_jobs[args.workload][1])
                   if oracle_leg else None, "step": "encode + decode of the whole tensor"},
        "encode_GBps": enc["GBps"],
        "decode_GBps": dec["GBps"],
        "encode_ms": {"median": enc["median_ms"], "min": enc["min_ms"], "runs": enc["runs"]},
        "decode_ms": {"median": dec["median_ms"], "min": dec["min_ms"], "runs": dec["runs"]},
        "encode_frac_of_peak": enc["frac_of_peak"],
        "decode_frac_of_peak": dec["frac_of_peak"],
        "ratio": head_summary["ratio"],
        "escape_rate": head_summary["escape_rate"],
        "escapes": head_summary["escapes"],
        "stream_bytes": head_summary["stream_bytes"],
        "parity": parity,
        "kernels": per_kernel,
        "hbm": hbm_rates(per_kernel, args.workload),
        "copy": copy,
        "dominant_vs_copy": round(achieved / copy["GBps"], 4),
        "encoder_pattern": pattern,
        "decoder_pattern": dpattern,
        "roofline": {
            "bound": "hbm",
            "kernel": dominant,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
        },
        "configs": configs,
        "calibration": calibration,
        "formats": formats,
        "transfer": transfer,
        "page_numbers": {"encode_GBps": 613.3, "decode_GBps": 2181.8, "ratio": 1.324,
                         "hardware": "not named on the page", "workload": "real BF16 activations",
                         "note": "context only, not this workload or machine"},
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)
    if parity is False:
        sys.exit(1)


def reference_copy_rate(sz, alg, runs, dev):
    """The library's streaming copy of half the dominant kernel's algorithmic
    bytes (read and written once, non-temporal dwordx4, the fastest plain
    copy shape), timed per launch like the codec kernels: the practical
    streaming ceiling."""
    import torch
    per_direction = alg // 2 // 16 * 16
    src = torch.empty(per_direction, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    sz.reference_copy(src, dst)
    sz.profile_enable(True)
    for _ in range(runs):
        sz.reference_copy(src, dst)
    launches, total_ms = sz.profile_collect()["sz_ref_copy"]
    sz.profile_enable(False)
    ms = total_ms / launches
    return {"GBps": round(2 * per_direction / (ms * 1e-3) / 1e9, 1), "bytes": per_direction,
            "kernel": "sz_ref_copy: one non-temporal dwordx4 per lane, 4 KB per 256-lane workgroup"}


def encoder_pattern_rate(sz, x, dtype, n, runs, per_kernel):
    """The library's reference of the dense encoder's memory pattern
    (sz_reference_split: the encoder's grid, lanes and memory instructions,
    trivial arithmetic) on the same tensor, timed per launch like the codec
    kernels: the practical ceiling of the encoder's stream mix.  None when
    the tensor is not whole 16K tiles."""
    if n % 16384:
        return None
    out = sz.reference_split(x)
    sz.profile_enable(True)
    for _ in range(runs):
        sz.reference_split(x)
    launches, total_ms = sz.profile_collect()["sz_ref_split"]
    sz.profile_enable(False)
    del out
    ms = total_ms / launches
    moved = n * (2 if dtype == 0 else 1) + n // 2 + (n if dtype == 0 else 3 * n // 8)
    dense = "sz_enc_dense_bf16" if dtype == 0 else "sz_enc_dense_e5m2"
    row = {"kernel": "sz_ref_split", "bytes": moved, "avg_ms": round(ms, 5),
           "GBps": round(moved / (ms * 1e-3) / 1e9, 1), "frac_of_peak": round(moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    if dense in per_kernel:
        row["dense_encoder_ms_vs_pattern"] = round(per_kernel[dense]["avg_ms"] / ms, 4)
    return row


def decoder_pattern_rate(sz, c, runs, per_kernel):
    """The library's reference of the span decoders' memory pattern
    (sz_reference_join: the wide-span grid, lanes and memory instructions,
    trivial arithmetic) over the code and sign/mantissa sections of the
    workload's own stream into its decode output, timed per launch: the
    practical ceiling of the decoders' stream mix.  None when the tensor is
    not whole 16K tiles or takes the narrow spans."""
    n, dtype = c.n, c.dtype
    if n % 16384 or (n + 65535) // 65536 <= 128:
        return None
    up256 = lambda v: (v + 255) // 256 * 256
    off_nib = up256(64 + 4 * ((n + 65535) // 65536))
    off_sm = off_nib + up256((n + 1) // 2)
    sm_bytes = n if dtype == 0 else 3 * n // 8
    codes, sym = c.buf[off_nib:off_nib + n // 2], c.buf[off_sm:off_sm + sm_bytes]
    sz.reference_join(codes, sym, dtype, n, out=c.y)
    sz.profile_enable(True)
    for _ in range(runs):
        sz.reference_join(codes, sym, dtype, n, out=c.y)
    launches, total_ms = sz.profile_collect()["sz_ref_join"]
    sz.profile_enable(False)
    ms = total_ms / launches
    moved = n // 2 + sm_bytes + n * (2 if dtype == 0 else 1)
    dense = "sz_dec_bf16_span" if dtype == 0 else "sz_dec_e5m2_span"
    row = {"kernel": "sz_ref_join", "bytes": moved, "avg_ms": round(ms, 5),
           "GBps": round(moved / (ms * 1e-3) / 1e9, 1), "frac_of_peak": round(moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    if dense in per_kernel:
        row["decoder_ms_vs_pattern"] = round(per_kernel[dense]["avg_ms"] / ms, 4)
    return row


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


def extra_sections(sz, c, runs, dirs):
    """Rows beyond the encode+decode step, on the headline tensor: on-device
    calibration, the ablation formats and the chunked transfer."""
    import torch
    x, cb, dtype, n, elem, dev = c.x, c.cb, c.dtype, c.n, c.elem, c.x.device
    enc_ms, dec_ms = dirs["encode"]["median_ms"], dirs["decode"]["median_ms"]

    def med(fn):
        return median(c.time_runs(fn, runs))

    # on-device calibration (per-tensor codebook at run time): the whole
    # tensor, and every 16th 64K block; then encode with the device codebook
    cal_ws = torch.empty(sz._native.sz_calibrate_workspace_size(dtype), dtype=torch.uint8, device=dev)
    d_cb = torch.zeros(sz.DEVICE_CODEBOOK_BYTES, dtype=torch.uint8, device=dev)
    cal_full_ms = med(lambda: sz.calibrate_device(x, 1, out=d_cb, ws=cal_ws))
    cal_s16_ms = med(lambda: sz.calibrate_device(x, 16, out=d_cb, ws=cal_ws))
    sz.calibrate_device(x, 1, out=d_cb, ws=cal_ws)
    enc_dcb_ms = med(lambda: sz.encode(x, d_cb, out=c.buf, ws=c.ws, sync=False))
    torch.cuda.synchronize()
    if int(c.ws[:4].cpu().view(torch.int32)[0]) != 0:
        raise SystemExit("device codebook rejected")
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
    # re-encode with the offline book: c.buf holds the measured stream again
    c.encode()

    # the page's ablation formats on the same tensor (BF16 only): Top-8 and
    # Top-15 with a sentinel code, against the Top-16 numbers
    formats = None
    if dtype == 0:
        formats = {}
        for name, fmt in (("top8", sz.TOP8), ("top15_sentinel", sz.TOP15S)):
            buf_f = torch.empty(sz.encoded_size(dtype, n, n, fmt), dtype=torch.uint8, device=dev)
            ws_f = sz.workspace(dtype, n, dev, fmt)
            _, size_f, esc_f = sz.encode(x, cb, out=buf_f, ws=ws_f, fmt=fmt)
            sz.decode(buf_f, dtype, n, out=c.y, ws=c.ws_dec, in_bytes=size_f, fmt=fmt)
            if not torch.equal(c.y.view(torch.uint8), x.view(torch.uint8)):
                raise SystemExit("round trip mismatch (%s)" % name)
            e_ms = med(lambda: sz.encode(x, cb, out=buf_f, ws=ws_f, sync=False, fmt=fmt))
            d_ms = med(lambda: sz.decode(buf_f, dtype, n, out=c.y, ws=c.ws_dec, check=False, in_bytes=size_f,
                                         fmt=fmt))
            formats[name] = {
                "encode_GBps": round(n * elem / (e_ms * 1e-3) / 1e9, 1),
                "decode_GBps": round(n * elem / (d_ms * 1e-3) / 1e9, 1),
                "ratio": round(n * elem / size_f, 6),
                "escape_rate": round(esc_f / n, 6),
                "top16_decode_speedup": round(d_ms / dec_ms, 3),
                "top16_encode_speedup": round(e_ms / enc_ms, 3),
            }
            del buf_f, ws_f

    # chunked transfer through pinned host memory (PCIe both ways stands in
    # for the prefill-to-decode link): raw against SplitZip-compressed, one
    # layer (K and V) per chunk
    chunk = min(n, 1 << 24 if c.name != "longctx_kv" else 1 << 26)
    staging = sz.transfer_buffers(dtype, n, chunk, 3, dev)
    runs_t = {}
    for mode, book in (("raw", None), ("splitzip", cb)):
        best = None
        for _ in range(3):
            _, st = sz.transfer(x, chunk, book, depth=3, out=c.y, staging=staging)
            if best is None or st["total_ms"] < best["total_ms"]:
                best = st
        if not torch.equal(c.y.view(torch.uint8), x.view(torch.uint8)):
            raise SystemExit("transfer mismatch (%s)" % mode)
        runs_t[mode] = best
    # the codec's own time per chunk (encode + decode of one chunk on the
    # device, no link), and its share of the compressed transfer's wall time
    xc = x[:chunk]
    bc = torch.empty(sz.encoded_size(dtype, chunk, chunk), dtype=torch.uint8, device=dev)
    wc_e, wc_d = sz.workspace(dtype, chunk, dev), sz.decode_workspace(dtype, chunk, dev)
    yc = torch.empty_like(xc)

    def chunk_codec():
        sz.encode(xc, cb, out=bc, ws=wc_e, sync=False)
        sz.decode(bc, dtype, chunk, out=yc, ws=wc_d, check=False)
    codec_ms = med(chunk_codec)
    del bc, wc_e, wc_d, yc
    transfer = {
        "link": "PCIe via pinned host memory, device->host then host->device, pipelined (depth 3)",
        "chunk_elems": chunk,
        "chunks": runs_t["raw"]["chunks"],
        "raw_ms": round(runs_t["raw"]["total_ms"], 3),
        "raw_GBps": round(n * elem / (runs_t["raw"]["total_ms"] * 1e-3) / 1e9, 2),
        "splitzip_ms": round(runs_t["splitzip"]["total_ms"], 3),
        "splitzip_GBps": round(n * elem / (runs_t["splitzip"]["total_ms"] * 1e-3) / 1e9, 2),
        "wire_bytes": runs_t["splitzip"]["wire_bytes"],
        "wire_ratio": round(n * elem / runs_t["splitzip"]["wire_bytes"], 6),
        "speedup": round(runs_t["raw"]["total_ms"] / runs_t["splitzip"]["total_ms"], 4),
        "codec_ms_per_chunk": round(codec_ms, 4),
        "codec_share": round(runs_t["splitzip"]["chunks"] * codec_ms / runs_t["splitzip"]["total_ms"], 4),
    }
    del staging
    torch.cuda.synchronize()
    return calibration, formats, transfer


if __name__ == "__main__":
    main()
