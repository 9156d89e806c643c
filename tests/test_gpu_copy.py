"""The library's reference streaming copy (sz_reference_copy), which bench.py
times as the practical streaming ceiling: it must copy every byte of ragged
sizes (partial tiles and partial workgroups) and touch nothing past the end."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 32768 - 16, 32768, 32768 + 16, 3 * 32768 + 48, 64 << 20])
def test_reference_copy(nbytes):
    import fp8_kv_cache_sz_amd as sz
    print("reference_copy", nbytes, flush=True)
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.full((nbytes + 256,), 0xA5, dtype=torch.uint8, device="cuda")
    sz.reference_copy(src, dst[:nbytes])
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 0xA5).all())


def test_reference_copy_rejects_overlap():
    import fp8_kv_cache_sz_amd as sz
    buf = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(sz.SplitZipError) as e:
        sz.reference_copy(buf[:2048], buf[1024:3072])
    assert e.value.code == -1


@pytest.mark.parametrize("dtype,tiles", [(0, 1), (0, 3), (1, 1), (1, 5)])
def test_reference_split(dtype, tiles):
    """sz_reference_split (the dense encoders' memory pattern, which bench.py
    times as their ceiling) writes exactly the bytes its header states."""
    import fp8_kv_cache_sz_amd as sz
    n = tiles * 16384
    print("reference_split", dtype, n, flush=True)
    g = torch.Generator(device="cpu").manual_seed(100 * tiles + dtype)
    raw = torch.randint(0, 256, (n * (2 if dtype == 0 else 1),), dtype=torch.uint8, generator=g)
    x = (raw.view(torch.bfloat16) if dtype == 0 else raw).cuda()
    codes, sym = sz.reference_split(x)
    torch.cuda.synchronize()
    if dtype == 0:
        b = raw.view(-1, 8, 2)                       # chunk, element, byte (low first)
        want_sym = b[:, :, 0].reshape(-1)
        want_codes = (b[:, :4, 1] ^ b[:, 4:, 1]).reshape(-1)
    else:
        b = raw.view(-1, 32)
        want_codes = (b[:, :16] ^ b[:, 16:]).reshape(-1)
        want_sym = b[:, 16:28].reshape(-1)
    assert torch.equal(codes.cpu(), want_codes)
    assert torch.equal(sym.cpu(), want_sym)


@pytest.mark.parametrize("dtype,tiles", [(0, 1), (0, 3), (1, 1), (1, 5)])
def test_reference_join(dtype, tiles):
    """sz_reference_join (the span decoders' memory pattern, which bench.py
    times as their ceiling) writes exactly the bytes its header states."""
    import fp8_kv_cache_sz_amd as sz
    n = tiles * 16384
    print("reference_join", dtype, n, flush=True)
    g = torch.Generator(device="cpu").manual_seed(200 * tiles + dtype)
    codes = torch.randint(0, 256, (n // 2,), dtype=torch.uint8, generator=g)
    sym = torch.randint(0, 256, (n if dtype == 0 else 3 * n // 8,), dtype=torch.uint8, generator=g)
    out = sz.reference_join(codes.cuda(), sym.cuda(), dtype, n)
    torch.cuda.synchronize()
    got = out.view(torch.uint8).cpu()
    if dtype == 0:
        c, s = codes.view(-1, 4), sym.view(-1, 8)
        want = torch.cat([s, c, c ^ s[:, :4]], dim=1).reshape(-1)
    else:
        c, s = codes.view(-1, 16), sym.view(-1, 12)
        want = torch.cat([c, s, c[:, :4] ^ s[:, :4]], dim=1).reshape(-1)
    assert torch.equal(got, want)
