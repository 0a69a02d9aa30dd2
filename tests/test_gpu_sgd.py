"""GPU parity of the fused FlashSGD step (flashopt_sgd_step) against the
oracle, through the C ABI.  FlashSGD appears on page
"code/flashsim/flash_adamw_sim.py" only in bytes_per_param; the library and
the oracle read its update as torch.optim.SGD with momentum, the buffer stored
with the momentum spec.  Bar as for the AdamW step: scales, rho and the bf16
parameter bit-exact, codes (or the fp32 buffer) bit-exact.  Every comparison
is free-running: the oracle steps its own state from the same seeded
parameters and zero buffer, with the same seeded gradients.
  * ragged lists (sizes 0 .. 2^17) for five storage variants and four
    momentum settings (plain, weight decay, Nesterov, dampening), 3 steps;
  * 2^20 params x 10 steps;
  * non-finite gradients next to finite lanes (NaN matches any NaN);
  * the 1.2B and 8.0B lists on group-aligned samples in the benchmark's launch
    shape.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_companded_adam_amd import flashopt as F
from bit_companded_adam_amd import workloads as W
from tests._gpu import host, require_gpu, u16

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-2, momentum=0.9, dampening=0.0, weight_decay=0.0, nesterov=False)
SETTINGS = {"plain": {}, "wd": dict(weight_decay=0.01), "nesterov": dict(nesterov=True, weight_decay=0.01),
            "dampening": dict(dampening=0.1)}
STORAGE = [(24, True, True), (32, False, True), (None, True, True), (24, True, False), (None, True, False)]
RAGGED = [0, 1, 17, 31, 32, 33, 1000, 1023, 1024, 1025, 4096 + 5, 70001, 1 << 17]


def _sid(v):
    mb, comp, qs = v
    return f"mb{mb}-{'comp' if comp else 'lin'}-{'q' if qs else 'f32'}"


def _snap(s: F.TensorState, lo=0, hi=None) -> oracle.State:
    hi = s.param.numel() if hi is None else hi
    g0, g1 = lo // 32, (hi + 31) // 32
    rho = None if s.rho is None else host(s.rho[lo:hi])
    ms = None if s.m_scales is None else u16(s.m_scales[g0:g1])
    return oracle.State(u16(s.param[lo:hi]), rho, host(s.m_codes[lo:hi]), ms, None, None)


def _start(params, mb, qs):
    """The oracle's starting states: the seeded bf16 parameters (copied before
    any step), zero correction bits and a zero momentum buffer."""
    out = []
    for p in params:
        st = oracle.State.zeros_like_param(u16(p), mb, quantize_states=qs)
        st.v_codes = st.v_scales = None
        out.append(st)
    return out


def _f16_nan(a):
    return ((a & 0x7C00) == 0x7C00) & ((a & 0x03FF) != 0)


def _bf16_nan(a):
    return ((a & 0x7F80) == 0x7F80) & ((a & 0x7F) != 0)


def _compare(got: oracle.State, want: oracle.State, label: str, nan_ok=False):
    same = got.param == want.param
    if nan_ok:
        same |= _bf16_nan(got.param) & _bf16_nan(want.param)
    assert same.all(), f"{label}: bf16 param"
    if want.rho is not None:
        assert (got.rho == want.rho).all(), f"{label}: rho"
    if want.m_scales is None:
        a, b = got.m_codes.view(np.uint32), want.m_codes.view(np.uint32)
        same = a == b
        if nan_ok:
            same |= np.isnan(got.m_codes) & np.isnan(want.m_codes)
        assert same.all(), f"{label}: fp32 buffer"
    else:
        same = got.m_scales == want.m_scales
        if nan_ok:
            same |= _f16_nan(got.m_scales) & _f16_nan(want.m_scales)
        assert same.all(), f"{label}: m scales"
        assert (got.m_codes == want.m_codes).all(), f"{label}: m codes"


def _orc_hp(t, hp, mb, comp, qs):
    return oracle.sgd_hparams(lr=hp["lr"], momentum=hp["momentum"], dampening=hp["dampening"],
                              weight_decay=hp["weight_decay"], nesterov=hp["nesterov"], step=t,
                              master_bits=mb, companded=comp, quantize_states=qs)


# each storage variant in each state layout it has (blocked: quantized only)
STORAGE_LAYOUTS = [(*v, l) for v in STORAGE for l in (("blocked", "streams") if v[2] else ("streams",))]


@pytest.mark.parametrize("setting", sorted(SETTINGS))
@pytest.mark.parametrize("mb,comp,qs,layout", STORAGE_LAYOUTS,
                         ids=[f"{_sid(v[:3])}-{v[3]}" for v in STORAGE_LAYOUTS])
def test_ragged_list(orc, mb, comp, qs, layout, setting):
    require_gpu()
    hp = dict(HP, **SETTINGS[setting])
    params = [W.init_param(n, device="cuda", seed=200 + i) for i, n in enumerate(RAGGED)]
    want = _start(params, mb, qs)
    opt = F.FlashSGD(params, master_bits=mb, companded=comp, quantize_states=qs,
                     state_layout=layout, **hp)
    for t in range(1, 4):
        grads = [W.make_grad(n, t, device="cuda", stream_id=i, factor=float(np.exp(i - 6)))
                 for i, n in enumerate(RAGGED)]
        opt.step(grads)
        torch.cuda.synchronize()
        for i, (s, w, g) in enumerate(zip(opt.states, want, grads)):
            orc.sgd_step(w, u16(g), _orc_hp(t, hp, mb, comp, qs))
            _compare(_snap(s), w, f"{_sid((mb, comp, qs))} {setting} t{t} tensor{i} n{RAGGED[i]}")


SGD_GRID = [
    ("momentum_0.5", dict(momentum=0.5), 1),
    ("momentum_0.99_step_1e6", dict(momentum=0.99, weight_decay=0.01), 1_000_000),
    ("lr_1", dict(lr=1.0, weight_decay=0.1), 1),
    ("lr_1e-6", dict(lr=1e-6), 3),
    ("nesterov_0.95", dict(momentum=0.95, nesterov=True, weight_decay=0.001), 2),
    ("lr_0", dict(lr=0.0, weight_decay=0.01), 1),
]


@pytest.mark.parametrize("mb,comp,qs", [(24, True, True), (32, False, True), (24, True, False)],
                         ids=["mb24-comp", "mb32-lin", "mb24-f32"])
@pytest.mark.parametrize("name,over,t0", SGD_GRID, ids=[h[0] for h in SGD_GRID])
def test_hyper_parameter_grid(orc, name, over, t0, mb, comp, qs):
    """Three steps from a zero buffer at step t0 (the first is the buffer's
    initialisation only when t0 = 1) under each setting."""
    require_gpu()
    hp = dict(HP, **over)
    sizes = [4096 + 5, 70001]
    params = [W.init_param(n, device="cuda", seed=60 + i) for i, n in enumerate(sizes)]
    want = _start(params, mb, qs)
    opt = F.FlashSGD(params, master_bits=mb, companded=comp, quantize_states=qs, **hp)
    opt.t = t0 - 1
    for t in range(t0, t0 + 3):
        grads = [W.make_grad(n, t, device="cuda", stream_id=i, factor=float(np.exp(i)))
                 for i, n in enumerate(sizes)]
        opt.step(grads)
        torch.cuda.synchronize()
        for i, (st, w, g) in enumerate(zip(opt.states, want, grads)):
            orc.sgd_step(w, u16(g), _orc_hp(t, hp, mb, comp, qs))
            _compare(_snap(st), w, f"{name} t{t} tensor{i}")


def test_single_tensor_10_steps(orc):
    require_gpu()
    n = 1 << 20
    hp = dict(HP, weight_decay=0.01)
    p = W.init_param(n, device="cuda", seed=31)
    (free,) = _start([p], 24, True)
    opt = F.FlashSGD([p], **hp)
    for t in range(1, 11):
        g = W.make_grad(n, t, device="cuda")
        opt.step([g])
        torch.cuda.synchronize()
        orc.sgd_step(free, u16(g), _orc_hp(t, hp, 24, True, True))
        _compare(_snap(opt.states[0]), free, f"step {t}")


@pytest.mark.parametrize("mb,comp,qs", [(24, True, True), (None, True, False)], ids=["q", "f32"])
def test_non_finite_gradients(orc, mb, comp, qs):
    """Outside the contract but defined: non-finite buffers take the
    element-wise encoders; their neighbours in the same group do not."""
    require_gpu()
    n = 16 * 1024 + 77
    p = W.init_param(n, device="cuda", seed=41)
    (want,) = _start([p], mb, qs)
    opt = F.FlashSGD([p], master_bits=mb, companded=comp, quantize_states=qs, **HP)
    for t in range(1, 4):
        g = W.make_grad(n, t).float()
        g[1603] = float("inf")
        g[2091] = float("nan")
        g[64 * 32:65 * 32] = 1e30
        g = g.to(torch.bfloat16).to("cuda")
        opt.step([g])
        torch.cuda.synchronize()
        orc.sgd_step(want, u16(g), _orc_hp(t, HP, mb, comp, qs))
        _compare(_snap(opt.states[0]), want, f"non-finite t{t}", nan_ok=True)


def _sampled_parity(orc, shapes, label, mb=24, qs=True):
    """Two steps over a whole decoder list in one list launch (the benchmark's
    launch shape); after each, group-aligned samples of every tensor (its
    first and last 2^16 elements and two random 1024-element chunks) are
    checked against the oracle stepping those slices from the same seeded
    start (step 1 initialises the buffer, step 2 reads it back)."""
    require_gpu()
    params = [W.init_param(W.numel(s), device="cuda", seed=1000 + i) for i, (_, s) in enumerate(shapes)]
    opt = F.FlashSGD(params, master_bits=mb, quantize_states=qs, **dict(HP, weight_decay=0.01))
    factors = W.grad_factors(len(shapes)).numpy()
    grads = lambda t: [W.make_grad(W.numel(s), t, device="cuda", stream_id=i, factor=float(factors[i]))
                       for i, (_, s) in enumerate(shapes)]
    rng = np.random.default_rng(9)
    ranges = []
    for s in opt.states:
        n = s.param.numel()
        r = [(0, min(n, 1 << 16)), (max(0, ((n - (1 << 16)) // 32) * 32), n)]
        if n > 4096:
            r += [(int(c) * 1024, int(c) * 1024 + 1024) for c in rng.integers(0, n // 1024 - 1, 2)]
        ranges.append(r)
    want = [_start([s.param[lo:hi] for lo, hi in rr], mb, qs) for s, rr in zip(opt.states, ranges)]
    for t in (1, 2):
        g_t = grads(t)
        gs = [[u16(g[lo:hi]) for lo, hi in rr] for g, rr in zip(g_t, ranges)]
        opt.step(g_t)
        del g_t
        torch.cuda.synchronize()
        for i, (s, rr) in enumerate(zip(opt.states, ranges)):
            for (lo, hi), w, g in zip(rr, want[i], gs[i]):
                orc.sgd_step(w, g, _orc_hp(t, dict(HP, weight_decay=0.01), mb, True, qs))
                _compare(_snap(s, lo, hi), w, f"{label} step {t} tensor {i} [{lo}, {hi})")


def test_decoder_1b_sampled(orc):
    _sampled_parity(orc, W.decoder_1b_shapes(), "1.2B")


@pytest.mark.parametrize("mb,qs", [(24, True), (32, True), (24, False)],
                         ids=["mb24", "mb32", "fp32_buffer"])
def test_decoder_8b_sampled(orc, mb, qs):
    _sampled_parity(orc, W.decoder_8b_shapes(), f"8.0B, mb {mb}, quantized {qs}", mb, qs)


def test_tensor_past_2_31_elements(orc):
    """One tensor of 2^31 + 1101 elements (offsets past 32-bit range): step 1
    through the list entry point, step 2 through the single-tensor one,
    checked at the start, on both sides of element 2^31 and on the ragged
    tail."""
    require_gpu()
    n = (1 << 31) + 1024 + 77
    mid = 1 << 31
    rr = [(0, 1 << 12), (mid - (1 << 12), mid + (1 << 12)), (((n - (1 << 12)) // 32) * 32, n)]
    hp = dict(HP, weight_decay=0.01)
    p = W.init_param(n, device="cuda", seed=78)
    want = _start([p[lo:hi] for lo, hi in rr], 24, True)
    opt = F.FlashSGD([p], **hp)
    for t in (1, 2):
        g = W.make_grad(n, t, device="cuda")
        gs = [u16(g[lo:hi]) for lo, hi in rr]
        if t == 1:
            opt.step([g])
        else:
            opt.step_tensor(0, g)
        del g
        torch.cuda.synchronize()
        for (lo, hi), w, gb in zip(rr, want, gs):
            orc.sgd_step(w, gb, _orc_hp(t, hp, 24, True, True))
            _compare(_snap(opt.states[0], lo, hi), w, f"n = 2^31 + 1101, step {t}, [{lo}, {hi})")
        print(f"2^31 + 1101 elements, step {t}: samples bit-exact", flush=True)
    del opt, p
    torch.cuda.empty_cache()
