"""GPU parity of the fused FlashAdamW step (flashopt_adamw_step, page
"code/flashsim/flash_adamw_sim.py", FlashAdamWSim.step / Alg. 4) against the
oracle, through the C ABI.

Every comparison is free-running: the oracle starts from the same seeded
parameters with zero moments (the state both sides begin from) and steps its
own state with the same seeded gradients; no value the GPU computed is ever
an input of the oracle.

Bar: fp16 scales, rho and the bf16 parameter bit-exact; codes bit-exact
(contract: >= 99.99% and never more than 1 apart); reconstructed fp32 master
within 1e-6 relative (implied by bit-exact param and rho).
  * 2^20 single tensor, 10 steps, 24-bit companded; two tensors over 64 steps.
  * ragged multi-tensor lists (sizes 0, 1, 17, ..., 70001) in one launch, all
    master widths and both companding modes, 3 steps.
  * determinism across runs and launch shapes.
  * the full 1.2B decoder list, every element, after each of two steps.
  * full-size decoder lists (1.2B and 8.0B parameters) in the launch
    configuration the benchmark times, checked on group-aligned samples: the
    first and last 2^16 elements of every tensor and random 1024-element
    chunks; the step is elementwise with group-local maxima, so any aligned
    slice is checked exactly by the oracle stepping that slice alone.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from bit_companded_adam_amd import flashopt as F
from bit_companded_adam_amd import workloads as W
from tests._gpu import code_agreement, host, require_gpu, u16

pytestmark = pytest.mark.gpu

HP = dict(W.HP_DEFAULT)


def _orc_hp(t, master_bits, companded, quantize_states=True):
    return oracle.hparams(lr=HP["lr"], betas=HP["betas"], eps=HP["eps"],
                          weight_decay=HP["weight_decay"], step=t,
                          master_bits=master_bits, companded=companded,
                          quantize_states=quantize_states)


def _snap(s: F.TensorState, lo=0, hi=None) -> oracle.State:
    """Host copy of a device state slice [lo, hi) (lo, hi multiples of 32)."""
    hi = s.param.numel() if hi is None else hi
    g0, g1 = lo // 32, (hi + 31) // 32
    opt = lambda t, f: None if t is None else f(t)
    return oracle.State(u16(s.param[lo:hi]), opt(s.rho, lambda r: host(r[lo:hi])),
                        host(s.m_codes[lo:hi]), opt(s.m_scales, lambda t: u16(t[g0:g1])),
                        host(s.v_codes[lo:hi]), opt(s.v_scales, lambda t: u16(t[g0:g1])))


def _start(params, mb, qs=True):
    """The oracle's starting states: the seeded bf16 parameters (copied before
    any step) with zero correction bits and zero moments, as the binding
    allocates them."""
    return [oracle.State.zeros_like_param(u16(p), mb, quantize_states=qs) for p in params]


def _compare(got: oracle.State, want: oracle.State, mb, label: str):
    """mb: 24 | 32 | None (no split).  fp32 moments (no scales) compare bit
    for bit; codes to the contract's bar, held here to equality."""
    assert (got.param == want.param).all(), f"{label}: bf16 param"
    if want.m_scales is None:
        for name in ("m_codes", "v_codes"):
            a, b = getattr(got, name), getattr(want, name)
            assert (a.view(np.uint32) == b.view(np.uint32)).all(), f"{label}: fp32 {name}"
    else:
        assert (got.m_scales == want.m_scales).all(), f"{label}: m scales"
        assert (got.v_scales == want.v_scales).all(), f"{label}: v scales"
        for name in ("m_codes", "v_codes"):
            agree, worst = code_agreement(getattr(got, name), getattr(want, name))
            assert worst <= 1 and agree >= 0.9999, (label, name, agree, worst)
            assert agree == 1.0, f"{label}: {name} agree {agree:.8f}"
    if mb is None:
        return
    assert (got.rho == want.rho).all(), f"{label}: rho"
    a = oracle.reconstruct(got.param, got.rho, mb).astype(np.float64)
    b = oracle.reconstruct(want.param, want.rho, mb).astype(np.float64)
    assert (np.abs(a - b) <= 1e-6 * np.abs(b)).all(), f"{label}: master"


@pytest.mark.parametrize("layout", ["blocked", "streams"])
def test_single_tensor_10_steps(orc, layout):
    """2^20 params, bf16 N(0, 0.02^2), grads N(0, 1e-3^2) fresh each step,
    24-bit master, companded, lr 1e-3, betas (0.9, 0.999), eps 1e-8, wd 0.01;
    the state in either layout."""
    require_gpu()
    n = 1 << 20
    p = W.init_param(n, device="cuda")
    (free,) = _start([p], 24)
    opt = F.FlashAdamW([p], master_bits=24, companded=True, state_layout=layout, **HP)
    for t in range(1, 11):
        g = W.make_grad(n, t, device="cuda")
        opt.step([g])
        torch.cuda.synchronize()
        orc.adamw_step(free, u16(g), _orc_hp(t, 24, True))
        _compare(_snap(opt.states[0]), free, 24, f"step {t}")
        print(f"step {t}: parity ok", flush=True)


@pytest.mark.parametrize("mb,comp,qs", [(24, True, True), (32, True, True), (24, False, True)],
                         ids=["mb24-comp", "mb32-comp", "mb24-lin"])
def test_free_running_64_steps(orc, mb, comp, qs):
    """64 steps with the oracle stepping its own state from the same start:
    every stored byte stays equal the whole way, so no rare mismatch is
    compounding."""
    require_gpu()
    sizes = [1 << 17, 50001]
    params = [W.init_param(n, device="cuda", seed=70 + i) for i, n in enumerate(sizes)]
    host_states = _start(params, mb, qs)
    opt = F.FlashAdamW(params, master_bits=mb, companded=comp, quantize_states=qs, **HP)
    for t in range(1, 65):
        grads = [W.make_grad(n, t, device="cuda", stream_id=i, factor=float(np.exp(i)))
                 for i, n in enumerate(sizes)]
        opt.step(grads)
        for h, g in zip(host_states, grads):
            orc.adamw_step(h, u16(g), _orc_hp(t, mb, comp, qs))
        if t % 16 == 0:
            torch.cuda.synchronize()
            for i, (st, h) in enumerate(zip(opt.states, host_states)):
                _compare(_snap(st), h, mb, f"free-running t{t} tensor{i}")
            print(f"step {t}: bit-exact", flush=True)


RAGGED = [0, 1, 17, 31, 32, 33, 1000, 1023, 1024, 1025, 4096 + 5, 70001, 1 << 17]


# (master_bits, companded, quantize_states): the method, the linear ablation
# of the codec, the page's master_weight_bits=None and quantize_states=False
# ablations, and their combinations
VARIANTS = [(24, True, True), (32, True, True), (24, False, True), (32, False, True),
            (None, True, True), (None, False, True), (24, True, False), (32, True, False),
            (None, True, False)]


def _vid(v):
    mb, comp, qs = v
    return f"mb{mb}-{'comp' if comp else 'lin'}-{'q' if qs else 'f32'}"


# every variant in each state layout it has (the blocked layout holds
# quantized states only)
VARIANT_LAYOUTS = [(v, layout) for v in VARIANTS for layout in (("blocked", "streams") if v[2] else ("streams",))]


@pytest.mark.parametrize("mb,comp,qs,layout", [(*v, l) for v, l in VARIANT_LAYOUTS],
                         ids=[f"{_vid(v)}-{l}" for v, l in VARIANT_LAYOUTS])
def test_ragged_list(orc, mb, comp, qs, layout):
    require_gpu()
    params = [W.init_param(n, device="cuda", seed=10 + i) for i, n in enumerate(RAGGED)]
    want = _start(params, mb, qs)
    opt = F.FlashAdamW(params, master_bits=mb, companded=comp, quantize_states=qs,
                       state_layout=layout, **HP)
    for t in range(1, 4):
        grads = [W.make_grad(n, t, device="cuda", stream_id=i, factor=float(np.exp(i - 6)))
                 for i, n in enumerate(RAGGED)]
        opt.step(grads)
        torch.cuda.synchronize()
        for i, (s, w, g) in enumerate(zip(opt.states, want, grads)):
            orc.adamw_step(w, u16(g), _orc_hp(t, mb, comp, qs))
            _compare(_snap(s), w, mb, f"{_vid((mb, comp, qs))} t{t} tensor{i} n{RAGGED[i]}")


# Hyper-parameter settings away from the default: (name, overrides, first
# step).  beta 0 (no averaging), beta2 0.9999 (a small bias correction),
# bias corrections at 1 (step 10^6; and steps 17320-17322, where the second
# one reaches 1 and the step switches to its late-training route), learning
# rates 0, 1e-10 and 1e-6 to 1 (1e-10, and 1e-2 with beta1 0.9999 at step 1,
# lie outside the short route's learning-rate range: the whole step takes the
# generic route), no weight decay, a large eps.
HP_GRID = [
    ("betas_zero", dict(betas=(0.0, 0.0)), 1),
    ("beta2_0.9999", dict(betas=(0.5, 0.9999)), 1),
    ("step_1e6", dict(betas=(0.95, 0.99)), 1_000_000),
    ("step_100", dict(), 100),
    ("step_163", dict(), 163),         # 1 - 0.9^t reaches 1 in fp32 at t = 165
    ("step_17320", dict(), 17320),     # 1 - 0.999^t reaches 1 in fp32 at t = 17321
    ("lr_1_wd_0.1", dict(lr=1.0, weight_decay=0.1), 1),
    ("lr_1e-6_wd_0", dict(lr=1e-6, weight_decay=0.0), 5),
    ("eps_1e-3", dict(eps=1e-3), 2),
    ("lr_0", dict(lr=0.0, weight_decay=0.1), 1),       # the master must come back unchanged
    # lr above 2^6 (1 - beta1^t): the whole step takes the generic route
    ("beta1_0.9999_lr_1e-2", dict(betas=(0.9999, 0.999), lr=1e-2), 1),
    # lr below 2^-32: the generic route as well
    ("lr_1e-10", dict(lr=1e-10), 1),
]


@pytest.mark.parametrize("mb,comp,qs", [(24, True, True), (32, False, True), (24, True, False)],
                         ids=["mb24-comp", "mb32-lin", "mb24-f32"])
@pytest.mark.parametrize("name,over,t0", HP_GRID, ids=[h[0] for h in HP_GRID])
def test_hyper_parameter_grid(orc, name, over, t0, mb, comp, qs):
    """Three steps from zero moments at step t0 under each setting: the host's
    scalars, the short division's domain checks and the codec across the
    hyper-parameter range."""
    require_gpu()
    hp = dict(HP, **over)
    sizes = [4096 + 5, 70001, 1 << 15]
    params = [W.init_param(n, device="cuda", seed=40 + i) for i, n in enumerate(sizes)]
    want = _start(params, mb, qs)
    init = [w.param.copy() for w in want]
    opt = F.FlashAdamW(params, master_bits=mb, companded=comp, quantize_states=qs, **hp)
    opt.t = t0 - 1
    for t in range(t0, t0 + 3):
        grads = [W.make_grad(n, t, device="cuda", stream_id=i, factor=float(np.exp(i - 1)))
                 for i, n in enumerate(sizes)]
        opt.step(grads)
        torch.cuda.synchronize()
        for i, (st, w, g) in enumerate(zip(opt.states, want, grads)):
            orc.adamw_step(w, u16(g), oracle.hparams(
                lr=hp["lr"], betas=hp["betas"], eps=hp["eps"], weight_decay=hp["weight_decay"],
                step=t, master_bits=mb, companded=comp, quantize_states=qs))
            _compare(_snap(st), w, mb, f"{name} t{t} tensor{i}")
            if hp["lr"] == 0.0:
                assert (u16(st.param) == init[i]).all(), f"{name}: lr 0 changed the parameter"


@pytest.mark.parametrize("mb,comp,qs", [(None, True, True), (24, True, False)],
                         ids=["mb_none", "fp32_states"])
def test_ablation_10_steps(orc, mb, comp, qs):
    """The two ablations over 10 steps on 2^18 + 77 params against the
    oracle."""
    require_gpu()
    n = (1 << 18) + 77
    p = W.init_param(n, device="cuda", seed=21)
    (free,) = _start([p], mb, qs)
    opt = F.FlashAdamW([p], master_bits=mb, companded=comp, quantize_states=qs, **HP)
    for t in range(1, 11):
        g = W.make_grad(n, t, device="cuda")
        opt.step([g])
        torch.cuda.synchronize()
        orc.adamw_step(free, u16(g), _orc_hp(t, mb, comp, qs))
        _compare(_snap(opt.states[0]), free, mb, f"{_vid((mb, comp, qs))} step {t}")


@pytest.mark.parametrize("comp,qs", [(True, True), (False, True), (True, False)],
                         ids=["comp", "lin", "f32-states"])
def test_fp32_params_10_steps(orc, comp, qs):
    """fp32 parameters with fp32 gradients, never split (FlashAdamWSim.step's
    use_split is false for an fp32 parameter): a ragged list over 10
    free-running steps against the oracle, every stored bit equal; the
    single-tensor launches of a second copy give the same bits."""
    require_gpu()
    sizes = [1, 33, 4096 + 5, 70001, (1 << 18) + 77]
    mk = lambda: [W.init_param(n, device="cuda", seed=300 + i, dtype=torch.float32)
                  for i, n in enumerate(sizes)]
    params, params_b = mk(), mk()
    want = [oracle.State.zeros_like_param(host(p).copy(), None, quantize_states=qs) for p in params]
    opt = F.FlashAdamW(params, master_bits=None, companded=comp, quantize_states=qs, **HP)
    opt_b = F.FlashAdamW(params_b, master_bits=None, companded=comp, quantize_states=qs, **HP)
    for t in range(1, 11):
        grads = [W.make_grad(n, t, device="cuda", stream_id=i, factor=float(np.exp(i - 2)),
                             dtype=torch.float32) for i, n in enumerate(sizes)]
        opt.step(grads)
        for i, g in enumerate(grads):
            opt_b.step_tensor(i, g)
        torch.cuda.synchronize()
        for i, (s, sb, w, g) in enumerate(zip(opt.states, opt_b.states, want, grads)):
            orc.adamw_step(w, host(g), oracle.hparams(
                lr=HP["lr"], betas=HP["betas"], eps=HP["eps"], weight_decay=HP["weight_decay"],
                step=t, master_bits=None, companded=comp, quantize_states=qs, fp32_param=True))
            label = f"fp32 params comp{comp} qs{qs} t{t} tensor{i}"
            assert (host(s.param).view(np.uint32) == w.param.view(np.uint32)).all(), label
            for name in ("m_codes", "m_scales", "v_codes", "v_scales"):
                a, b = getattr(s, name), getattr(w, name)
                if b is None:
                    continue
                assert (host(a).view(np.uint8) == b.view(np.uint8)).all(), f"{label}: {name}"
                assert (host(getattr(sb, name)).view(np.uint8) == b.view(np.uint8)).all(), \
                    f"{label}: {name} (single-tensor launch)"
            assert (host(sb.param).view(np.uint32) == w.param.view(np.uint32)).all(), \
                f"{label}: single-tensor launch"


def test_zero_and_large_gradients(orc):
    """All-zero gradients keep zero scales and codes; gradients of very
    different magnitude across tensors."""
    require_gpu()
    sizes = [4096, 4096, 4096]
    params = [W.init_param(n, device="cuda", seed=40 + i) for i, n in enumerate(sizes)]
    want = _start(params, 24)
    opt = F.FlashAdamW(params, master_bits=24, **HP)
    for t in range(1, 3):
        grads = [torch.zeros(4096, dtype=torch.bfloat16, device="cuda"),
                 W.make_grad(4096, t, device="cuda", scale=1e2),
                 W.make_grad(4096, t, device="cuda", scale=1e-30)]
        opt.step(grads)
        torch.cuda.synchronize()
        for i, (s, w, g) in enumerate(zip(opt.states, want, grads)):
            orc.adamw_step(w, u16(g), _orc_hp(t, 24, True))
            _compare(_snap(s), w, 24, f"t{t} tensor{i}")
    assert int(opt.states[0].m_scales.abs().sum()) == 0


def _f16_nan(s: np.ndarray) -> np.ndarray:
    return ((s & 0x7C00) == 0x7C00) & ((s & 0x03FF) != 0)


def _bf16_nan(x: np.ndarray) -> np.ndarray:
    return ((x & 0x7F80) == 0x7F80) & ((x & 0x7F) != 0)


def _compare_nan_aware(got: oracle.State, want: oracle.State, mb: int, label: str):
    """Like _compare, but a NaN parameter or scale matches any NaN: the pages
    fix no NaN payload or sign, and the host and the GPU make different
    default NaNs.  Everything else stays bit-exact."""
    both_nan = _bf16_nan(got.param) & _bf16_nan(want.param)
    assert ((got.param == want.param) | both_nan).all(), f"{label}: bf16 param"
    if mb is not None:
        assert (got.rho == want.rho).all(), f"{label}: rho"
    if want.m_scales is None:                 # fp32 moments
        for name in ("m_codes", "v_codes"):
            a, b = getattr(got, name), getattr(want, name)
            same = (a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))
            assert same.all(), f"{label}: fp32 {name}"
        return
    for name in ("m_scales", "v_scales"):
        a, b = getattr(got, name), getattr(want, name)
        assert ((a == b) | (_f16_nan(a) & _f16_nan(b))).all(), f"{label}: {name}"
    assert (got.m_codes == want.m_codes).all(), f"{label}: m codes"
    assert (got.v_codes == want.v_codes).all(), f"{label}: v codes"


def _edge_grad(case: str, n: int, t: int) -> torch.Tensor:
    """Gradients that drive lanes (16 consecutive elements) out of the
    short division's domain, next to lanes that stay in it."""
    g = W.make_grad(n, t).float()
    idx = torch.arange(n)
    lane = idx // 16
    if case == "tiny_mixed":
        g[(lane % 3 == 0) & (idx % 16 == 5)] *= 1e-27     # one tiny numerator in a lane
        g[lane % 7 == 1] *= 1e-30                         # whole lanes of tiny numerators
    elif case == "large_m_small_eps":
        g[lane % 5 == 2] *= 1e6                           # large |m|; eps 1e-30 is below the
                                                          # short routes' range: all lanes generic
    elif case == "eps_zero":
        g[lane % 4 == 3] = 0.0                            # 0 / 0 without eps
    elif case == "tiny_at_lr_bound":
        # lr just below 2^6 (1 - beta1^t) at t = 1 (beta1 0.9999): |m1| below
        # 2^-102, where m1 / bc1 may be inexact, must still reach the generic
        # route through its numerator
        g[(lane % 3 == 0) & (idx % 16 == 5)] *= 1e-33
        g[lane % 7 == 1] *= 1e-30
        g[lane % 11 == 4] *= 1e-35                        # bf16 subnormals among them
    elif case == "nonfinite":
        g[100 * 16 + 3] = float("inf")
        g[130 * 16 + 9] = float("nan")
        g[64 * 32:65 * 32] = 1e30                         # v and the scales overflow
    return g.to(torch.bfloat16).to("cuda")


EDGE_EPS = {"tiny_mixed": 1e-8, "large_m_small_eps": 1e-30, "eps_zero": 0.0, "nonfinite": 1e-8,
            "tiny_at_lr_bound": 1e-8}
EDGE_HP = {"tiny_at_lr_bound": dict(betas=(0.9999, 0.999), lr=6e-3)}


@pytest.mark.parametrize("mb,comp,qs", [(24, True, True), (32, False, True), (None, True, False)],
                         ids=["mb24-comp", "mb32-lin", "mbnone-f32"])
@pytest.mark.parametrize("case", sorted(EDGE_EPS))
# from step 1 (both quotients), 200 (bc1 = 1 with beta1 = 0.9) and 20001
# (both bias corrections 1): the three forms of the short route
@pytest.mark.parametrize("t0", [1, 200, 20001], ids=["t1", "t200", "t20001"])
def test_lanes_outside_short_division_domain(orc, case, mb, comp, qs, t0):
    """Lanes whose numerators or denominators leave the range where the
    kernel's short division is exact, or whose values are not finite, take
    the generic path; their neighbours in the same group do not.  Both must
    match the oracle (ragged size: 17 chunks, the last one partial)."""
    require_gpu()
    n = 16 * 1024 + 77
    hp = dict(HP, eps=EDGE_EPS[case], **EDGE_HP.get(case, {}))
    p = W.init_param(n, device="cuda", seed=90)
    (want,) = _start([p], mb, qs)
    opt = F.FlashAdamW([p], master_bits=mb, companded=comp, quantize_states=qs, **hp)
    opt.t = t0 - 1
    for t in range(t0, t0 + 3):
        g = _edge_grad(case, n, t)
        opt.step([g])
        torch.cuda.synchronize()
        orc.adamw_step(want, u16(g), oracle.hparams(
            lr=hp["lr"], betas=hp["betas"], eps=hp["eps"], weight_decay=hp["weight_decay"],
            step=t, master_bits=mb, companded=comp, quantize_states=qs))
        _compare_nan_aware(_snap(opt.states[0]), want, mb, f"{case} mb{mb} comp{comp} t{t}")


def test_deterministic_across_launch_splits():
    """The same steps leave the same bits whether a list is stepped in one
    launch or split into launches of 1 or 7 chunks (FLASHOPT_LAUNCH_CHUNKS
    forces the split that a list too long for one dispatch takes; 7 chunks
    of two wavefronts leave spare wavefronts in every launch's last
    workgroup, which must not reach into the next launch's chunks): AdamW
    list steps, single-tensor steps and FlashSGD list steps."""
    require_gpu()
    sizes = [1 << 16, 3000, 1 << 18]
    results = []
    try:
        for per in (None, "1", "7"):
            if per is None:
                os.environ.pop("FLASHOPT_LAUNCH_CHUNKS", None)
            else:
                os.environ["FLASHOPT_LAUNCH_CHUNKS"] = per
            make = lambda seed: [W.init_param(n, device="cuda", seed=seed + i) for i, n in enumerate(sizes)]
            opt = F.FlashAdamW(make(70), master_bits=24, **HP)
            single = F.FlashAdamW(make(80), master_bits=24, **HP)
            sgd = F.FlashSGD(make(90), **W.SGD_DEFAULT)
            for t in range(1, 4):
                grads = [W.make_grad(n, t, device="cuda", stream_id=i) for i, n in enumerate(sizes)]
                opt.step(grads)
                for i, g in enumerate(grads):
                    single.step_tensor(i, g)
                sgd.step(grads)
            torch.cuda.synchronize()
            out = []
            for s in opt.states + single.states:
                out.append(torch.cat([s.param.view(torch.int16).float(), s.rho.float(),
                                      s.m_codes.float(), s.v_codes.float()]).cpu())
            for s in sgd.states:
                out.append(torch.cat([s.param.view(torch.int16).float(), s.rho.float(),
                                      s.m_codes.float()]).cpu())
            results.append(out)
    finally:
        os.environ.pop("FLASHOPT_LAUNCH_CHUNKS", None)
    for r in results[1:]:
        for a, b in zip(results[0], r):
            assert torch.equal(a, b)


def _build_list(shapes, mb, comp, seed_base, qs=True, layout=None):
    params = [W.init_param(W.numel(s), device="cuda", seed=seed_base + i)
              for i, (_, s) in enumerate(shapes)]
    return F.FlashAdamW(params, master_bits=mb, companded=comp, quantize_states=qs,
                        state_layout=layout, **HP)


def _grads(shapes, t, factors):
    return [W.make_grad(W.numel(s), t, device="cuda", stream_id=i, factor=float(factors[i]))
            for i, (_, s) in enumerate(shapes)]


def _sample_ranges(n, rng, k=2):
    r = [(0, min(n, 1 << 16))]
    last = max(0, ((n - (1 << 16)) // 32) * 32)
    r.append((last, n))
    if n > 4 * 1024:
        for c in rng.integers(0, n // 1024 - 1, k):
            r.append((int(c) * 1024, int(c) * 1024 + 1024))
    return r


def _sampled_parity(orc, shapes, mb, comp, label, qs=True, layout=None):
    """Two list steps over the whole list; after each, every sample is
    compared with the oracle stepping that slice from the same seeded start
    (step 1 starts from zero moments, step 2 from non-trivial ones)."""
    opt = _build_list(shapes, mb, comp, seed_base=1000, qs=qs, layout=layout)
    factors = W.grad_factors(len(shapes)).numpy()
    rng = np.random.default_rng(7)
    ranges = [_sample_ranges(s.param.numel(), rng) for s in opt.states]
    want = [[oracle.State.zeros_like_param(u16(s.param[lo:hi]), mb, quantize_states=qs)
             for lo, hi in rr] for s, rr in zip(opt.states, ranges)]
    checked = 0
    for t in (1, 2):
        grads = _grads(shapes, t, factors)
        gs = [[u16(g[lo:hi]) for lo, hi in rr] for g, rr in zip(grads, ranges)]
        opt.step(grads)
        del grads
        torch.cuda.synchronize()
        for i, (s, rr) in enumerate(zip(opt.states, ranges)):
            for (lo, hi), w, g in zip(rr, want[i], gs[i]):
                orc.adamw_step(w, g, _orc_hp(t, mb, comp, qs))
                _compare(_snap(s, lo, hi), w, mb, f"{label} step {t} tensor {i} [{lo}, {hi})")
                checked += hi - lo
    print(f"{label}: {checked} sampled elements bit-exact over two steps", flush=True)
    del opt
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layout", ["blocked", "streams"])
def test_decoder_1b_sampled(orc, layout):
    require_gpu()
    _sampled_parity(orc, W.decoder_1b_shapes(), 24, True, f"1.2B list, 24-bit, {layout}",
                    layout=layout)


def test_decoder_1b_full(orc):
    """The whole 1.2B list (199 tensors, 1,195,991,040 elements) in one list
    launch per step, as the benchmark times it, every stored element compared
    with the oracle's OpenMP list driver (the same per-element arithmetic as
    its single-tensor step) after each of two steps."""
    require_gpu()
    shapes = W.decoder_1b_shapes()
    opt = _build_list(shapes, 24, True, seed_base=1000)
    factors = W.grad_factors(len(shapes)).numpy()
    want = [oracle.State.zeros_like_param(u16(s.param), 24) for s in opt.states]
    n = sum(s.param.numel() for s in opt.states)
    for t in (1, 2):
        grads = _grads(shapes, t, factors)
        gh = [u16(g) for g in grads]
        opt.step(grads)
        del grads
        torch.cuda.synchronize()
        threads = orc.adamw_step_list(want, gh, _orc_hp(t, 24, True))
        del gh
        for i, (s, w) in enumerate(zip(opt.states, want)):
            _compare(_snap(s), w, 24, f"1.2B full list, step {t}, tensor {i}")
        print(f"1.2B list, step {t}: all {n} elements bit-exact (oracle on {threads} threads)",
              flush=True)
    del opt
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mb,qs", [(None, True), (24, False)], ids=["mb_none", "fp32_states"])
def test_decoder_1b_sampled_ablations(orc, mb, qs):
    require_gpu()
    _sampled_parity(orc, W.decoder_1b_shapes(), mb, True, f"1.2B list, mb {mb}, quantized {qs}", qs=qs)


@pytest.mark.parametrize("mb,comp,layout", [(24, True, "blocked"), (32, True, "blocked"),
                                            (24, False, "blocked"), (24, True, "streams")])
def test_decoder_8b_sampled(orc, mb, comp, layout):
    require_gpu()
    _sampled_parity(orc, W.decoder_8b_shapes(), mb, comp,
                    f"8.0B list, {mb}-bit, companded={comp}, {layout}", layout=layout)


@pytest.mark.parametrize("mb,qs", [(None, True), (24, False)], ids=["mb_none", "fp32_states"])
def test_decoder_8b_sampled_ablations(orc, mb, qs):
    """The two ablations on the 8.0B list, in the launch the benchmark times
    for them (--master-bits 0, --fp32-states)."""
    require_gpu()
    _sampled_parity(orc, W.decoder_8b_shapes(), mb, True, f"8.0B list, mb {mb}, quantized {qs}", qs=qs)


# One tensor past 2^31 elements: element offsets, the byte offsets of the
# 16-bit streams (past 2^32 bytes at element 2^31) and the chunk arithmetic
# leave 32-bit range.  Samples: the start, both sides of element 2^31, and
# the ragged tail (the last chunk holds 77 elements).
N_PAST_2_31 = (1 << 31) + 1024 + 77


def _past_2_31_ranges(n):
    mid = 1 << 31
    return [(0, 1 << 12), (mid - (1 << 12), mid + (1 << 12)), (((n - (1 << 12)) // 32) * 32, n)]


def test_tensor_past_2_31_elements(orc):
    """Step 1 through the list entry point, step 2 through the single-tensor
    entry point, each checked against the oracle on the samples."""
    require_gpu()
    n = N_PAST_2_31
    p = W.init_param(n, device="cuda", seed=77)
    rr = _past_2_31_ranges(n)
    want = [oracle.State.zeros_like_param(u16(p[lo:hi]), 24) for lo, hi in rr]
    opt = F.FlashAdamW([p], master_bits=24, companded=True, **HP)
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
            orc.adamw_step(w, gb, _orc_hp(t, 24, True))
            _compare(_snap(opt.states[0], lo, hi), w, 24, f"n = 2^31 + 1101, step {t}, [{lo}, {hi})")
        print(f"2^31 + 1101 elements, step {t}: samples bit-exact", flush=True)
    del opt, p
    torch.cuda.empty_cache()


def test_shards_of_a_tensor_equal_the_whole_tensor():
    """The sharded design steps 32-aligned ranges of a tensor independently
    (each rank owns one range and its state).  Eight uneven shards stepped as
    views of one parameter, in one list launch, must leave the parameter,
    and states equal to the slices of the whole tensor's state, bit for bit."""
    require_gpu()
    n = (1 << 20) + 77
    cuts = [0, 32 * 1000, 32 * 1001, 32 * 7777, 32 * 8000, 32 * 15000, 32 * 20000, 32 * 32000, n]
    pw = W.init_param(n, device="cuda", seed=55)
    ps = pw.clone()
    whole = F.FlashAdamW([pw], master_bits=24, companded=True, **HP)
    shards = F.FlashAdamW([ps[a:b] for a, b in zip(cuts[:-1], cuts[1:])], master_bits=24,
                          companded=True, **HP)
    for t in range(1, 4):
        g = W.make_grad(n, t, device="cuda")
        whole.step([g])
        shards.step([g[a:b] for a, b in zip(cuts[:-1], cuts[1:])])
        torch.cuda.synchronize()
        assert torch.equal(pw.view(torch.int16), ps.view(torch.int16)), f"t{t}: param"
        ws = whole.states[0]
        for k, (a, b) in enumerate(zip(cuts[:-1], cuts[1:])):
            s = shards.states[k]
            for name in ("rho", "m_codes", "v_codes"):
                assert torch.equal(getattr(s, name), getattr(ws, name)[a:b]), f"t{t} shard {k}: {name}"
            for name in ("m_scales", "v_scales"):
                assert torch.equal(getattr(s, name), getattr(ws, name)[a // 32:(b + 31) // 32]), \
                    f"t{t} shard {k}: {name}"
