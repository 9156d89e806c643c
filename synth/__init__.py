"""Seeded synthetic KV-cache inputs shared by the tests, the smoke check and
the benchmark.

This module only draws random numbers and lays them out as BF16 / FP8-E5M2
tensors; it holds none of the codec's arithmetic.  Both the HIP path and the
CPU oracle are fed the tensors it returns.

Workloads (stand-ins for the real Qwen / Llama / Phi KV activations the
SplitZip page measures on, which are not available here):

* ``kv_layer``: one K (or V) tensor ``[tokens, heads, dims]`` whose channels
  carry a per-(head, dim) scale s ~ LogNormal(0, 1); values are N(0, 1) * s,
  rounded to BF16 with round-to-nearest-even.  A fraction of channels can be
  marked outliers and scaled by 50.
* ``kv_cache``: ``layers x {K, V}`` such tensors concatenated in
  (layer, K/V) order.
* escape-stress sets: Student-t values with a share of random exponents,
  a single exponent, and random bit patterns without NaN/Inf.
* the E5M2 variant of ``kv_cache`` (round-to-nearest-even to FP8 E5M2).

All draws use ``torch.Generator`` on the requested device, so a given
(seed, device) always yields the same tensor.
"""
from __future__ import annotations

import torch

BF16 = 0
E5M2 = 1


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _channel_scales(g, heads, dims, device, outlier_frac=0.0, outlier_scale=50.0):
    s = torch.exp(torch.randn((heads, dims), generator=g, device=device, dtype=torch.float32))
    if outlier_frac > 0.0:
        mask = torch.rand((heads, dims), generator=g, device=device) < outlier_frac
        s = torch.where(mask, s * outlier_scale, s)
    return s


def kv_layer_f32(g, tokens, heads, dims, device, outlier_frac=0.0, scales=None):
    """float32 [tokens, heads, dims] = N(0,1) * per-channel LogNormal(0,1) scale."""
    if scales is None:
        scales = _channel_scales(g, heads, dims, device, outlier_frac)
    z = torch.randn((tokens, heads, dims), generator=g, device=device, dtype=torch.float32)
    return z * scales


def kv_layer(seed, tokens=1024, heads=8, dims=128, device="cpu"):
    """One layer's K tensor in BF16 (the single-tensor workload and its calibration twin)."""
    g = _gen(seed, device)
    return kv_layer_f32(g, tokens, heads, dims, device).to(torch.bfloat16).reshape(-1)


def kv_cache(seed, layers, tokens, heads, dims, device="cpu", outlier_frac=0.0,
             out_dtype=torch.bfloat16, per_layer_seed=None):
    """layers x {K,V} x [tokens, heads, dims], concatenated in (layer, K/V) order.

    Each (layer, K/V) tensor draws its own channel scales and then its values.
    ``per_layer_seed(l)`` gives layer l its own generator (K then V from it);
    otherwise one generator seeded with ``seed`` runs over all tensors in order.
    """
    per = tokens * heads * dims
    out = torch.empty(layers * 2 * per, dtype=out_dtype, device=device)
    g = None if per_layer_seed else _gen(seed, device)
    for layer in range(layers):
        if per_layer_seed:
            g = _gen(per_layer_seed(layer), device)
        for kv in range(2):
            x = kv_layer_f32(g, tokens, heads, dims, device, outlier_frac)
            k = (layer * 2 + kv) * per
            out[k:k + per] = x.reshape(-1).to(out_dtype)
            del x
    return out


def layer0_calibration(seed_scales, seed_values, heads, dims, device="cpu", outlier_frac=0.001,
                       tokens=1024):
    """Calibration tensor for the full-cache workload: layer 0's K channel scales
    (drawn exactly as ``kv_cache`` draws them) with fresh values."""
    g = _gen(seed_scales, device)
    scales = _channel_scales(g, heads, dims, device, outlier_frac)
    gz = _gen(seed_values, device)
    return kv_layer_f32(gz, tokens, heads, dims, device, scales=scales).to(torch.bfloat16).reshape(-1)


def student_t_with_random_exponents(seed, n, device="cpu", df=3, frac=0.02):
    """Student-t(df) values in BF16; a ``frac`` share of elements get a uniformly
    random exponent field in [1, 254]."""
    g = _gen(seed, device)
    z = torch.randn(n, generator=g, device=device, dtype=torch.float32)
    chi2 = torch.zeros(n, device=device, dtype=torch.float32)
    for _ in range(df):
        w = torch.randn(n, generator=g, device=device, dtype=torch.float32)
        chi2 += w * w
    t = z / torch.sqrt(chi2 / df)
    bits = t.to(torch.bfloat16).view(torch.int16).to(torch.int32) & 0xFFFF
    pick = torch.rand(n, generator=g, device=device) < frac
    expo = torch.randint(1, 255, (n,), generator=g, device=device, dtype=torch.int32)
    bits = torch.where(pick, (bits & 0x807F) | (expo << 7), bits)
    return _u16_bits_to_bf16(bits)


def single_exponent(seed, n, exponent=127, device="cpu"):
    """Random sign and mantissa, every exponent field equal to ``exponent``."""
    g = _gen(seed, device)
    sign = torch.randint(0, 2, (n,), generator=g, device=device, dtype=torch.int32)
    mant = torch.randint(0, 128, (n,), generator=g, device=device, dtype=torch.int32)
    return _u16_bits_to_bf16((sign << 15) | (exponent << 7) | mant)


def random_finite_bf16(seed, n, device="cpu"):
    """Random sign, mantissa and exponent field in [0, 254] (no NaN / Inf)."""
    g = _gen(seed, device)
    sign = torch.randint(0, 2, (n,), generator=g, device=device, dtype=torch.int32)
    mant = torch.randint(0, 128, (n,), generator=g, device=device, dtype=torch.int32)
    expo = torch.randint(0, 255, (n,), generator=g, device=device, dtype=torch.int32)
    return _u16_bits_to_bf16((sign << 15) | (expo << 7) | mant)


def random_bits(seed, n, dtype=BF16, device="cpu"):
    """Uniformly random bit patterns (every pattern, NaN and Inf included)."""
    g = _gen(seed, device)
    if dtype == BF16:
        return _u16_bits_to_bf16(torch.randint(0, 65536, (n,), generator=g, device=device,
                                               dtype=torch.int32))
    return torch.randint(0, 256, (n,), generator=g, device=device, dtype=torch.int32).to(torch.uint8)


def _u16_bits_to_bf16(bits_i32):
    v = bits_i32.to(torch.int32)
    v = torch.where(v >= 32768, v - 65536, v).to(torch.int16)
    return v.view(torch.bfloat16)


def to_e5m2_bytes(x_f32):
    """float32 -> FP8 E5M2 (round to nearest even) as raw uint8 bytes."""
    try:
        y = x_f32.to(torch.float8_e5m2)
    except (RuntimeError, TypeError):
        y = x_f32.cpu().to(torch.float8_e5m2).to(x_f32.device)
    return y.view(torch.uint8)


def kv_cache_e5m2(seed, layers, tokens, heads, dims, device="cpu"):
    """E5M2 bytes of a ``kv_cache``-shaped tensor (no outlier channels)."""
    per = tokens * heads * dims
    out = torch.empty(layers * 2 * per, dtype=torch.uint8, device=device)
    g = _gen(seed, device)
    for layer in range(layers):
        for kv in range(2):
            x = kv_layer_f32(g, tokens, heads, dims, device)
            k = (layer * 2 + kv) * per
            out[k:k + per] = to_e5m2_bytes(x.reshape(-1))
            del x
    return out


# ---------------------------------------------------------------------------
# Named workloads.  ``size`` = "full" gives the published shape; "small"
# keeps the structure (same generators, every distribution feature) at a
# size the CPU oracle handles in about a second.
# ---------------------------------------------------------------------------
WORKLOADS = ("kv1m", "llama3_8b_kv", "longctx_kv", "stress_t3", "stress_oneexp",
             "stress_random", "llama3_8b_kv_e5m2")

DESCRIPTION = {
    "kv1m": "single K tensor 1024 tok x 8 heads x 128 dims (1,048,576 BF16)",
    "llama3_8b_kv": "Llama-3-8B KV cache 32 layers x {K,V} x 8 heads x 128 dims x 8192 tok (536,870,912 BF16)",
    "longctx_kv": "long-context payload 28 layers x {K,V} x 4 heads x 128 dims x 65536 tok (1,879,048,192 BF16)",
    "stress_t3": "Student-t(3) with 2% random exponents (268,435,456 BF16)",
    "stress_oneexp": "single exponent 127, random sign/mantissa (268,435,456 BF16)",
    "stress_random": "random finite BF16 bit patterns (268,435,456 BF16)",
    "llama3_8b_kv_e5m2": "Llama-3-8B KV cache in FP8 E5M2 (536,870,912 bytes)",
}


def calibration_tensor(name, device="cpu", size="full"):
    """The tensor the workload's codebook is calibrated on (dtype-matched)."""
    if name == "llama3_8b_kv":
        heads = 8
        return layer0_calibration(2, 3, heads, 128, device=device)
    if name == "llama3_8b_kv_e5m2":
        g = _gen(1, device)
        return to_e5m2_bytes(kv_layer_f32(g, 1024, 8, 128, device).reshape(-1))
    return kv_layer(1, device=device)


def workload(name, device="cpu", size="full"):
    """Returns (data tensor, dtype code).  BF16 data is a bfloat16 tensor,
    E5M2 data a uint8 tensor of raw bytes."""
    full = size == "full"
    if name == "kv1m":
        return kv_layer(0, device=device), BF16
    if name == "llama3_8b_kv":
        tokens = 8192 if full else 256
        layers = 32 if full else 2
        return kv_cache(2, layers, tokens, 8, 128, device=device, outlier_frac=0.001), BF16
    if name == "longctx_kv":
        tokens = 65536 if full else 512
        layers = 28 if full else 2
        return kv_cache(None, layers, tokens, 4, 128, device=device,
                        per_layer_seed=lambda l: 100 + l), BF16
    n = 268435456 if full else 1 << 20
    if name == "stress_t3":
        return student_t_with_random_exponents(40, n, device=device), BF16
    if name == "stress_oneexp":
        return single_exponent(41, n, 127, device=device), BF16
    if name == "stress_random":
        return random_finite_bf16(42, n, device=device), BF16
    if name == "llama3_8b_kv_e5m2":
        tokens = 8192 if full else 256
        layers = 32 if full else 2
        return kv_cache_e5m2(5, layers, tokens, 8, 128, device=device), E5M2
    raise KeyError(name)


def as_bits_numpy(t):
    """Host numpy view of the raw bits (uint16 for BF16, uint8 for E5M2)."""
    import numpy as np
    t = t.detach().reshape(-1)
    if t.device.type != "cpu":
        t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int16:
        return t.numpy().view(np.uint16)
    return t.view(torch.uint8).numpy()
