"""Encode and decode captured into a HIP graph (the library makes no
allocation, memset or host synchronisation inside either call, so both are
capturable).  The graph is replayed several times, with eager work and
synchronisation between replays and the input changed in place; every
replay must equal the eager result and the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


# small tensors take the fused kernels (one compaction launch, header check);
# 80M elements take the scans
@pytest.mark.parametrize("dtype,n_big", [(0, 0), (1, 0), (0, 80 << 20)])
def test_graph_replays_match_eager(dtype, n_big):
    import fp8_kv_cache_sz_amd as sz
    name = "llama3_8b_kv" if dtype == 0 else "llama3_8b_kv_e5m2"
    if n_big:
        x0 = synth.workload(name, device="cuda")[0][:n_big].contiguous()
    else:
        x0 = synth.workload(name, size="small")[0].cuda()
    cb = sz.calibrate(synth.calibration_tensor(name))
    n = x0.numel()
    x = x0.clone()
    cap = sz.encoded_size(dtype, n, n)
    buf = torch.zeros(cap, dtype=torch.uint8, device="cuda")
    ws_e = torch.zeros(sz.workspace_size(dtype, n), dtype=torch.uint8, device="cuda")
    ws_d = torch.zeros(sz.workspace_size(dtype, n), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    size_bound = cap
    stream = torch.cuda.Stream()
    # warm up on the capture stream, then capture encode + decode
    with torch.cuda.stream(stream):
        sz.encode(x, cb, out=buf, ws=ws_e, sync=False, stream=stream)
        sz.decode(buf, dtype, n, out=y, ws=ws_d, check=False, in_bytes=size_bound, stream=stream)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        sz.encode(x, cb, out=buf, ws=ws_e, sync=False, stream=stream)
        sz.decode(buf, dtype, n, out=y, ws=ws_d, check=False, in_bytes=size_bound, stream=stream)
    for rep in range(4):
        print("graph replay", rep, flush=True)
        # change the input in place (eager work between replays)
        x.copy_(torch.roll(x0, shifts=12345 * (rep + 1)))
        torch.cuda.synchronize()
        buf.fill_(0xA5)
        y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        bits = synth.as_bits_numpy(x)
        expect = oracle.encode(bits, dtype, list(cb.exps))
        got = buf[:expect.size].cpu().numpy()
        assert np.array_equal(got, expect), rep
        assert int(ws_d[:4].cpu().view(torch.int32)[0]) == 0
        assert torch.equal(y.view(torch.uint8), x.view(torch.uint8)), rep
