"""Pins for the oracle's fp32 -> binary16 conversion (the per-group scale is
torch's fp16 cast of the group absmax, page "code/flashsim/quantization.py",
quantize()).

Pinned against numpy.float16 (an independent library conversion, IEEE round
to nearest even with overflow to Inf): exhaustively over every fp32 pattern
whose magnitude lies in [2^-26, 2^17) -- the band where the result is neither
a signed zero nor an infinity -- for both signs, and on random samples of
every other exponent.  NaN inputs are excluded (out of contract; the oracle
returns a canonical quiet NaN)."""
import numpy as np

from tests._par import run_chunks

CHUNK = 1 << 23


def _check(orc, lo_bits, hi_bits):
    """Compare oracle vs numpy on every pattern in [lo_bits, hi_bits)."""
    def one(start):
        u = np.arange(start, min(start + CHUNK, hi_bits), dtype=np.uint64).astype(np.uint32)
        x = u.view(np.float32)
        got = orc.f16_bits(x)
        with np.errstate(over="ignore"):       # overflow to Inf is part of what is pinned
            ref = x.astype(np.float16).view(np.uint16)
        bad = np.nonzero(got != ref)[0]
        return (int(u[bad[0]]), int(got[bad[0]]), int(ref[bad[0]])) if bad.size else None

    res = [r for r in run_chunks(one, range(lo_bits, hi_bits, CHUNK)) if r]
    assert not res, "first mismatches (pattern, oracle, numpy): %r" % res[:4]


def test_f16_exhaustive_band_positive(orc):
    _check(orc, 0x32800000, 0x48000000)       # 2^-26 .. 2^17


def test_f16_exhaustive_band_negative(orc):
    _check(orc, 0xB2800000, 0xC8000000)


def test_f16_sampled_everywhere(orc):
    rng = np.random.default_rng(0)
    u = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    keep = ~np.isnan(x)
    x = x[keep]
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert (orc.f16_bits(x) == ref).all()


def test_f16_named_cases(orc):
    # values fixed by the binary16 format itself
    cases = [
        (0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3C00), (-2.0, 0xC000),
        (65504.0, 0x7BFF),          # largest finite
        (65519.99, 0x7BFF),         # below the rounding midpoint
        (65520.0, 0x7C00),          # the midpoint ties to even -> Inf
        (2.0 ** -24, 0x0001),       # smallest subnormal
        (2.0 ** -25, 0x0000),       # exact tie between 0 and 2^-24 -> even (0)
        (1.5 * 2.0 ** -25, 0x0001),
        (2.0 ** -14, 0x0400),       # smallest normal
        (float("inf"), 0x7C00), (float("-inf"), 0xFC00),
    ]
    for v, want in cases:
        got = orc.lib().oracle_f16_from_f32(v)
        assert got == want, (v, hex(got), hex(want))


def test_f16_widening_exact(orc):
    # every non-NaN binary16 pattern widens exactly and converts back to itself
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = h.view(np.float16)
    keep = ~np.isnan(f)
    w = np.array([orc.lib().oracle_f32_from_f16(int(b)) for b in h[keep]], dtype=np.float32)
    assert (w == f[keep].astype(np.float32)).all()
    assert (orc.f16_bits(w) == h[keep]).all()
