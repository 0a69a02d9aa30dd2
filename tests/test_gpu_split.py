"""GPU parity of the weight split (flashopt_split / flashopt_reconstruct)
against the oracle: bit-exact theta' and rho on the stratified exponent sweep
(both master widths, random signs) and on edge patterns, plus exhaustive
properties over all 2^32 fp32 patterns on the GPU (32-bit: lossless; 24-bit:
within 128 fp32 ulps, 255 in the clamp band) with oracle parity on a sample
of every chunk."""
import numpy as np
import pytest
import torch

from bit_companded_adam_amd import flashopt as F
from bit_companded_adam_amd import workloads as W
from tests._gpu import host, require_gpu, u16

pytestmark = pytest.mark.gpu


def _gpu_split(x_np, mb):
    x = torch.from_numpy(x_np).cuda()
    p, r = F.flashopt_split(x, mb)
    back = F.flashopt_reconstruct(p, r, mb)
    torch.cuda.synchronize()
    return u16(p), host(r), host(back)


@pytest.mark.parametrize("mb", [24, 32])
def test_sweep_parity(orc, mb):
    require_gpu()
    x = W.split_sweep()[mb].numpy()
    p, r, back = _gpu_split(x, mb)
    hp, hr = orc.split(x, mb)
    assert (p == hp).all() and (r == hr).all()
    ob = orc.reconstruct(hp, hr, mb)
    assert (back.view(np.uint32) == ob.view(np.uint32)).all()
    exact = float(np.mean(back == x))
    rel = float(np.mean(np.abs(back.astype(np.float64) - x) / np.abs(x.astype(np.float64))))
    print(f"sweep {mb}-bit: exact fraction {exact:.7f}, mean relative error {rel:.4e}")
    if mb == 32:
        assert exact == 1.0
    else:
        assert abs(exact - 1 / 256) < 2e-4 and 5.2e-6 < rel < 5.4e-6


@pytest.mark.parametrize("mb", [24, 32])
def test_edge_patterns(orc, mb):
    require_gpu()
    lo = np.arange(1 << 16, dtype=np.uint32)
    his = np.array([0x0000, 0x0001, 0x007F, 0x0080, 0x3F80, 0x7F7F, 0x7F80, 0x7FC0, 0x7FFF,
                    0x8000, 0x8001, 0xFF7F, 0xFF80, 0xFFC0, 0xFFFF], np.uint32)
    u = ((his[:, None] << 16) | lo[None, :]).reshape(-1)
    x = u.view(np.float32)
    p, r, back = _gpu_split(x, mb)
    hp, hr = orc.split(x, mb)
    assert (p == hp).all() and (r == hr).all()
    ob = orc.reconstruct(hp, hr, mb)
    assert (back.view(np.uint32) == ob.view(np.uint32)).all()


@pytest.mark.parametrize("mb", [24, 32])
def test_exhaustive_properties(orc, mb):
    require_gpu()
    chunk = 1 << 28
    rng = np.random.default_rng(mb)
    bad = 0
    for start in range(0, 1 << 32, chunk):
        print(f"split {mb}-bit chunk {start >> 28}/16", flush=True)
        u = torch.arange(start, start + chunk, dtype=torch.int64, device="cuda").to(torch.int32)
        x = u.view(torch.float32)
        p, r = F.flashopt_split(x, mb)
        back = F.flashopt_reconstruct(p, r, mb).view(torch.int32)
        nan = torch.isnan(x)
        if mb == 32:
            bad += int(((back != u) & ~nan).sum())
        else:
            diff = (back.to(torch.int64) - u.to(torch.int64)).abs()
            low = u.to(torch.int64) & 0xFFFF
            band = (low >= 32640) & (low <= 32767)
            bad += int(((diff > 128) & ~band & ~nan).sum()) + int(((diff > 255) & band & ~nan).sum())
        # oracle parity on a sample of this chunk
        idx = torch.from_numpy(rng.integers(0, chunk, 1 << 16)).cuda()
        xs = host(x[idx])
        hp, hr = orc.split(xs, mb)
        assert (u16(p[idx]) == hp).all() and (host(r[idx]) == hr).all()
        del u, x, p, r, back
    assert bad == 0


def test_bf16_exact_values_and_zero():
    require_gpu()
    hi = torch.arange(0, 1 << 16, dtype=torch.int32, device="cuda")
    x = (hi << 16).view(torch.float32)
    x = x[~torch.isnan(x)]
    for mb in (24, 32):
        p, r = F.flashopt_split(x, mb)
        assert int((r != 0).sum()) == 0
        assert torch.equal(p.view(torch.int16).to(torch.int32) & 0xFFFF,
                           (x.view(torch.int32) >> 16) & 0xFFFF)


@pytest.mark.parametrize("mb", [24, 32])
def test_tensor_past_2_31_elements(orc, mb):
    """Split and reconstruct of 2^31 + 1101 seeded fp32 masters (N(0, 0.02^2)
    on the device), checked against the oracle at the start, around elements
    2^30 (the fp32 stream passes 2^32 bytes) and 2^31 (the bf16 stream
    does), and on the ragged tail."""
    require_gpu()
    n = (1 << 31) + 1024 + 77
    gen = torch.Generator(device="cuda").manual_seed(92 + mb)
    x = torch.randn(n, generator=gen, device="cuda").mul_(0.02)
    p, r = F.flashopt_split(x, mb)
    back = F.flashopt_reconstruct(p, r, mb)
    torch.cuda.synchronize()
    k = 1 << 12
    for lo, hi in [(0, k), ((1 << 30) - k, (1 << 30) + k), ((1 << 31) - k, (1 << 31) + k), (n - k, n)]:
        hp, hr = orc.split(host(x[lo:hi]), mb)
        assert (u16(p[lo:hi]) == hp).all() and (host(r[lo:hi]) == hr).all(), f"[{lo}, {hi})"
        ob = orc.reconstruct(hp, hr, mb)
        assert (host(back[lo:hi]).view(np.uint32) == ob.view(np.uint32)).all(), f"[{lo}, {hi})"
    print(f"split {mb}-bit, 2^31 + 1101 elements: samples bit-exact", flush=True)
    del x, p, r, back
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mb", [24, 32])
def test_split_across_launches(orc, mb, monkeypatch):
    """A split and reconstruct cut into launches of 7 workgroups
    (FLASHOPT_LAUNCH_CHUNKS, the launch-size hook; a workgroup takes 1024
    elements, 4096 in the 32-bit reconstruct): every element of a ragged
    tensor of 99 * 1024 + 333 elements matches the oracle."""
    require_gpu()
    monkeypatch.setenv("FLASHOPT_LAUNCH_CHUNKS", "7")
    n = 99 * 1024 + 333
    gen = torch.Generator(device="cuda").manual_seed(7 + mb)
    x = torch.randn(n, generator=gen, device="cuda").mul_(0.02)
    p, r = F.flashopt_split(x, mb)
    back = F.flashopt_reconstruct(p, r, mb)
    torch.cuda.synchronize()
    hp, hr = orc.split(host(x), mb)
    assert (u16(p) == hp).all() and (host(r) == hr).all()
    ob = orc.reconstruct(hp, hr, mb)
    assert (host(back).view(np.uint32) == ob.view(np.uint32)).all()
