"""GPU check of the short exact fp32 sequences the kernels use instead of the
generic correctly rounded division / sqrt expansions (flashopt_math.h):
each sweep compares against the compiler's correctly rounded operation on the
same device and must find no mismatch.  Sweeps: sqrt over every x in
[0, 2^64); reciprocal over every significand (three exponents) and every fp16
value; division by an fp16 scale over every divisor x dividend significand
pair (2^33); softsign over every |y| <= 1.5; v_cvt_pk_u8_f32 and the
magic-number int8 code rounding over all 2^32 patterns; the update division over 2^32
random pairs of its stated domain and every divisor significand at the
domain's edges; the bias-correction division through an fp64 reciprocal over
every dividend significand for 8192 divisors (the fp32 bias corrections of
eight betas up to t = 512, and hashed ones); the sqrt of that quotient with
the input scaling folded into one fp64 fma, over every dividend for 16 bias
corrections; the guarded companded momentum code against the correctly
rounded chain around every rounding boundary for 4095 fp16 divisors
(two-sided short form: trusted where its two evaluations agree)."""
import ctypes
import os

import pytest

from tests._gpu import require_gpu

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "libfastmath_check.so")
CHECKS = ["sqrt", "recip", "div_by_recip", "softsign", "cvt_pk_u8", "div_markstein", "div_bias",
          "sqrt_quot", "magic_code", "softsign_code"]


@pytest.fixture(scope="module")
def lib():
    require_gpu()
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB)
    for c in CHECKS:
        getattr(L, "fastmath_check_" + c).restype = ctypes.c_longlong
    return L


@pytest.mark.parametrize("check", CHECKS)
def test_exact(lib, check):
    bad = getattr(lib, "fastmath_check_" + check)()
    print(f"fastmath {check}: {bad} mismatches", flush=True)
    assert bad == 0


def test_softsign_code_sweep_is_sensitive(lib):
    """Taken alone (without comparing its two evaluations), the short
    momentum code disagrees with the correctly rounded chain on some of the
    swept inputs: the sweep reaches the boundaries where the two-sided test
    matters."""
    lib.fastmath_softsign_code_unguarded.restype = ctypes.c_longlong
    diff = lib.fastmath_softsign_code_unguarded()
    print(f"unguarded softsign_code: {diff} disagreements", flush=True)
    assert diff > 0
