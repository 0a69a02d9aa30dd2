"""Pins for the oracle's weight split (Alg. 1: fp32 master -> bf16 theta' +
int8/int16 rho) and its inverse.

The pages do not print the split; they fix that theta' is the bf16 rounding of
the master (page "code/gpu/equivalence.py", eq_ecc() passes the bf16 cast of
the master to the correction-bit routine), that rho is int8 for a 24-bit master and
int16 for a 32-bit one (page "code/flashsim/flash_adamw_sim.py",
FlashAdamWSim.__init__), and that a bf16-exact parameter splits to rho = 0
(FlashAdamWSim.step, state init).  What pins the oracle here:
  * 32-bit master: reconstruct(split(x)) == x for every non-NaN fp32 pattern
    (exhaustive, 2^32 - NaNs);
  * theta' equals torch's bf16 cast except at exact ties whose truncated half
    is even (library routine; the one place ties-away and ties-even differ);
  * 24-bit master: the stored value is within 128 units in the last fp32 place
    (255 in the clamp band) -- exhaustive over every low half;
  * split(reconstruct(b, rho)) == (b, rho) for every valid (bf16, rho8) pair
    (brute force, 2^24 pairs) and for all rho16 on sampled bf16 patterns;
  * on the stratified exponent sweep the 24-bit exact fraction is 1/256 and
    the mean relative error matches its closed form.
"""
import math

import numpy as np
import torch

from bit_companded_adam_amd import workloads as W
from tests._par import run_chunks

CHUNK = 1 << 24


def test_split32_roundtrip_exhaustive(orc):
    def one(start):
        u = np.arange(start, start + CHUNK, dtype=np.uint64).astype(np.uint32)
        x = u.view(np.float32)
        keep = ~np.isnan(x)
        hi, rho = orc.split(x[keep], 32)
        back = orc.reconstruct(hi, rho, 32).view(np.uint32)
        bad = np.nonzero(back != u[keep])[0]
        return int(u[keep][bad[0]]) if bad.size else None

    res = [r for r in run_chunks(one, range(0, 1 << 32, CHUNK)) if r is not None]
    assert not res, "32-bit split not lossless at patterns %r" % [hex(r) for r in res[:4]]


def _patterns_all_low_halves(hi_values):
    lo = np.arange(1 << 16, dtype=np.uint32)
    return ((np.asarray(hi_values, dtype=np.uint32)[:, None] << 16) | lo[None, :]).reshape(-1)


def _hi_sample():
    rng = np.random.default_rng(3)
    special = [0x0000, 0x0001, 0x007F, 0x0080, 0x3F80, 0x3F7F, 0x7F7E, 0x7F7F,
               0x8000, 0x8001, 0x80FF, 0xBF80, 0xFF7E, 0xFF7F]
    return np.unique(np.concatenate([special, rng.integers(0, 0x7F80, 120),
                                     rng.integers(0x8000, 0xFF80, 120)]).astype(np.uint32))


def test_theta_prime_is_bf16_cast_except_even_ties(orc):
    u = _patterns_all_low_halves(_hi_sample())
    x = u.view(np.float32)
    keep = ~np.isnan(x) & ~np.isinf(x)
    u, x = u[keep], x[keep]
    hi, _ = orc.split(x, 24)
    cast = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    lo = u & 0xFFFF
    even_tie = (lo == 0x8000) & (((u >> 16) & 1) == 0)
    # ties-away rounds an even tie up, torch's RNE keeps it: exactly these differ
    assert (hi[~even_tie] == cast[~even_tie]).all()
    assert (hi[even_tie].astype(np.int64) - cast[even_tie].astype(np.int64) == 1).all()


def test_split24_error_bound_all_low_halves(orc):
    u = _patterns_all_low_halves(_hi_sample())
    x = u.view(np.float32)
    keep = ~np.isnan(x)
    u, x = u[keep], x[keep]
    hi, rho = orc.split(x, 24)
    back = orc.reconstruct(hi, rho, 24).view(np.uint32)
    diff = np.abs(back.astype(np.int64) - u.astype(np.int64))
    lo = (u & 0xFFFF).astype(np.int64)
    clamp_band = (lo >= 32640) & (lo <= 32767)
    assert diff[~clamp_band].max() <= 128
    assert diff[clamp_band].max() <= 255
    # both halves of the split stay on the input's side of zero
    assert ((back >> 31) == (u >> 31)).all()


def test_split24_all_pairs_brute_force(orc):
    b = np.repeat(np.arange(1 << 16, dtype=np.uint32), 256).astype(np.uint16)
    r = np.tile(np.arange(-128, 128, dtype=np.int16), 1 << 16).astype(np.int8)
    exp_field = (b.astype(np.uint32) >> 7) & 0xFF
    signed_zero = (b & 0x7FFF) == 0
    valid = (exp_field != 0xFF) & ~(signed_zero & (r < 0))
    assert valid.sum() == 16_711_424
    x = orc.reconstruct(b[valid], r[valid], 24)
    b2, r2 = orc.split(x, 24)
    assert (b2 == b[valid]).all() and (r2 == r[valid]).all()


def test_split16_pairs_sampled(orc):
    rng = np.random.default_rng(5)
    hs = np.concatenate([[0x0001, 0x3F80, 0x7F7F, 0x8001, 0xFF7F],
                         rng.integers(0, 0x7F80, 60), rng.integers(0x8001, 0xFF80, 60)])
    b = np.repeat(hs.astype(np.uint16), 1 << 16)
    r = np.tile(np.arange(-32768, 32768, dtype=np.int32).astype(np.int16), hs.size)
    x = orc.reconstruct(b, r, 32)
    b2, r2 = orc.split(x, 32)
    assert (b2 == b).all() and (r2 == r).all()


def test_bf16_exact_values_split_to_zero_rho(orc):
    rng = np.random.default_rng(9)
    hi = rng.integers(0, 1 << 16, 1 << 16).astype(np.uint16)
    x = (hi.astype(np.uint32) << 16).view(np.float32)
    keep = ~np.isnan(x)
    for mb in (24, 32):
        h2, rho = orc.split(x[keep], mb)
        assert (rho == 0).all() and (h2 == hi[keep]).all()
    h, r = orc.split(np.array([0.0, -0.0], np.float32), 32)
    assert list(h) == [0x0000, 0x8000] and list(r) == [0, 0]


def _expected_mean_rel_err_24():
    """Closed form of the sweep's 24-bit mean relative error: the stored pattern
    is the input pattern moved to the nearest multiple of 256 (half to even),
    except that residuals in [32640, 32767] stop at 127 * 256; the relative
    error of a uniform 23-bit mantissa f is err(f mod 2^16) 2^-23 / (1 + f 2^-23),
    averaged over all 2^23 mantissas."""
    lo = np.arange(1 << 16, dtype=np.int64)
    D = np.where(lo >= 32768, lo - 65536, lo)
    near = np.round(D / 256.0) * 256          # numpy rounds half to even
    near = np.minimum(near, 127 * 256)
    err = np.abs(D - near)
    f = np.arange(1 << 23, dtype=np.float64)
    return float(np.mean(err[(np.arange(1 << 23) & 0xFFFF)] * 2.0 ** -23 / (1.0 + f * 2.0 ** -23)))


def test_sweep_statistics_closed_form(orc):
    sw = W.split_sweep()
    x24 = sw[24].numpy()
    assert x24.size == 64 * (1 << 16)
    hi, rho = orc.split(x24, 24)
    back = orc.reconstruct(hi, rho, 24)
    exact = float(np.mean(back == x24))
    rel = float(np.mean(np.abs(back.astype(np.float64) - x24) / np.abs(x24.astype(np.float64))))
    n = x24.size
    p = 1.0 / 256.0
    assert abs(exact - p) < 6 * math.sqrt(p * (1 - p) / n), exact
    want = _expected_mean_rel_err_24()
    assert abs(want - 64.25 * 2.0 ** -23 * math.log(2)) / want < 2e-3   # ~ E[err] ln 2
    assert abs(rel - want) / want < 5e-3, (rel, want)

    x32 = sw[32].numpy()
    h32, r32 = orc.split(x32, 32)
    assert (orc.reconstruct(h32, r32, 32).view(np.uint32) == x32.view(np.uint32)).all()
