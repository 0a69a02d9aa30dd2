"""Pins for the oracle's AdamW body and its FlashAdamW step (page
"code/flashsim/flash_adamw_sim.py", FlashAdamWSim.step = Alg. 4).

* The update alone (fp32 states) is pinned to torch.optim.AdamW, an
  independent library implementation of decoupled-weight-decay AdamW with bias
  correction (its operation order differs, so within 1e-6 relative).
* The page's operation order (bias corrections as divisions, then
  (lr * mhat) / (sqrt(vhat) + eps)) is pinned bit for bit by a worked example
  derived by hand (tests/golden/adamw_literal_order.txt) in which the
  textbook folding of the bias corrections stores a different rho.
* Step 1 from a zero state has a closed form (m = (1-b1) g, v = (1-b2) g^2,
  theta1 = theta0 (1 - lr wd) - lr g / (|g| + eps)).
* With a 32-bit master the split is lossless, so K steps equal an fp32-master
  run through the (separately pinned) codec; with a 24-bit master each step
  equals that run teacher-forced from the rebuilt master.
* The OpenMP slice driver equals the per-tensor step bit for bit.
* 300 free-running steps with fp32 moments and the 32-bit master track
  torch.optim.AdamW within a derived rounding bound.
* A long trajectory with quantized states has a closed form in one special
  case: a group whose 32 elements are equal always gets the code +-127
  (momentum) or 255 (variance), whose dequantized value is exactly the
  group's fp16 scale, so the stored moments follow m <- fp16(m1) and
  v <- fp16(sqrt(v1))^2 (with the lossless 32-bit master, theta carries over
  unchanged); 40 steps of four such groups follow that recursion bit for bit.
A long trajectory with quantized states in general, or with the 24-bit
master, has no independent pin beyond this composition (parity unpinned for
it)."""
import os

import numpy as np
import pytest
import torch

HP = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)


def _bf16_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def test_update_matches_torch_adamw(orc):
    rng = np.random.default_rng(0)
    n, steps = 1 << 14, 10
    theta = (rng.standard_normal(n) * 0.02).astype(np.float32)
    p = torch.nn.Parameter(torch.from_numpy(theta.copy()))
    opt = torch.optim.AdamW([p], lr=HP["lr"], betas=HP["betas"], eps=HP["eps"],
                            weight_decay=HP["weight_decay"], foreach=False, fused=False)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    b1, b2 = HP["betas"]
    for t in range(1, steps + 1):
        g = (rng.standard_normal(n) * 1e-3 * np.exp(rng.standard_normal())).astype(np.float32)
        # teacher forcing: torch starts every step from the oracle's state
        with torch.no_grad():
            p.copy_(torch.from_numpy(theta))
        if t > 1:
            opt.state[p]["exp_avg"].copy_(torch.from_numpy(m))
            opt.state[p]["exp_avg_sq"].copy_(torch.from_numpy(v))
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        # torch evaluates m by lerp and v by addcmul: the two orders differ by
        # ulps of the terms, so tolerances scale with the terms' magnitudes
        m_terms = b1 * np.abs(m) + (1 - b1) * np.abs(g)
        th_terms = np.abs(theta) + HP["lr"] * 1.01
        hp = orc.hparams(**HP, step=t)
        theta, m, v = orc.adamw_update(theta, m, v, g, hp)
        st = opt.state[p]
        assert (np.abs(theta - p.detach().numpy()) <= 1e-6 * th_terms).all()
        assert (np.abs(m - st["exp_avg"].numpy()) <= 1e-6 * m_terms).all()
        assert np.allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-6, atol=0)


def test_golden_literal_order(orc):
    """Six elements' updates, every rounding derived by hand in the fixture
    (page "code/flashsim/flash_adamw_sim.py", FlashAdamWSim.step): their
    stored theta', rho pin the operation order, since the textbook folding
    of the bias corrections, either fold alone, a reciprocal multiply for a
    bias correction, a double-precision bias correction, lr applied last or
    the decay applied last each change at least one of them."""
    path = os.path.join(os.path.dirname(__file__), "golden", "adamw_literal_order.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 6
    f32 = lambda h: np.array([int(h, 16)], np.uint32).view(np.float32)
    for th, g, m, v, step, th1, m1, v1, hi, rho in rows:
        out = orc.adamw_update(f32(th), f32(m), f32(v), f32(g), orc.hparams(**HP, step=int(step)))
        assert [int(a.view(np.uint32)[0]) for a in out] == [int(th1, 16), int(m1, 16), int(v1, 16)]
        b, r = orc.split(out[0], 24)
        assert int(b[0]) == int(hi, 16) and int(r[0]) == int(rho)


@pytest.mark.parametrize("master_bits", [24, 32])
def test_step1_closed_form(orc, master_bits):
    rng = np.random.default_rng(2)
    n = 4096 + 13
    p0 = _bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    g = _bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32))
    st = orc.State.zeros_like_param(p0, master_bits)
    orc.adamw_step(st, g, orc.hparams(**HP, step=1, master_bits=master_bits))
    gf = _bits_to_f32(g).astype(np.float64)
    th0 = _bits_to_f32(p0).astype(np.float64)
    lr, wd, eps = HP["lr"], HP["weight_decay"], HP["eps"]
    want = th0 * (1 - lr * wd) - lr * gf / (np.abs(gf) + eps)
    got = orc.reconstruct(st.param, st.rho, master_bits).astype(np.float64)
    # float32 evaluation error is relative to the terms theta0 and lr (they
    # may cancel); the 24-bit master adds up to 128 units in the last fp32
    # place of the result (2^-16 relative) from the int8 correction
    tol = 1e-6 * (np.abs(th0) + lr)
    if master_bits == 24:
        tol = tol + 2.0 ** -15 * np.abs(want)
    assert (np.abs(got - want) <= tol).all()
    # moments at step 1 are exact products of the gradient
    c1 = np.float32(1 - HP["betas"][0])
    c2 = np.float32(1 - HP["betas"][1])
    g32 = _bits_to_f32(g)
    m1 = (c1 * g32).astype(np.float32)
    v1 = ((c2 * g32).astype(np.float32) * g32).astype(np.float32)
    pad = lambda a: np.concatenate([a, np.zeros((-a.size) % 32, np.float32)]).reshape(-1, 32)
    assert (st.m_scales == np.abs(pad(m1)).max(1).astype(np.float16).view(np.uint16)).all()
    assert (st.v_scales == np.sqrt(pad(v1)).max(1).astype(np.float16).view(np.uint16)).all()
    qm, _ = orc.quantize(m1, orc.MOMENTUM)
    qv, _ = orc.quantize(v1, orc.VARIANCE)
    assert (st.m_codes == qm).all() and (st.v_codes == qv).all()


def _fp32_master_run(orc, theta, grads, companded, steps):
    """The step as composition: fp32 master kept outside, states through the
    codec each step."""
    n = theta.size
    ms, vs = (orc.MOMENTUM, orc.VARIANCE) if companded else (orc.MOMENTUM_LINEAR, orc.VARIANCE_LINEAR)
    mq, msc = np.zeros(n, np.int8), np.zeros((n + 31) // 32, np.uint16)
    vq, vsc = np.zeros(n, np.uint8), np.zeros((n + 31) // 32, np.uint16)
    out = []
    for t in range(1, steps + 1):
        m = orc.dequantize(mq, msc, ms)
        v = orc.dequantize(vq, vsc, vs)
        theta, m, v = orc.adamw_update(theta, m, v, _bits_to_f32(grads[t - 1]),
                                       orc.hparams(**HP, step=t))
        mq, msc = orc.quantize(m, ms)
        vq, vsc = orc.quantize(v, vs)
        out.append((theta.copy(), mq.copy(), msc.copy(), vq.copy(), vsc.copy()))
    return out


@pytest.mark.parametrize("companded", [True, False])
def test_32bit_master_equals_fp32_master(orc, companded):
    rng = np.random.default_rng(3)
    n, steps = 3000 + 7, 6
    p0 = _bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    grads = [_bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32)) for _ in range(steps)]
    ref = _fp32_master_run(orc, _bits_to_f32(p0), grads, companded, steps)
    st = orc.State.zeros_like_param(p0, 32)
    for t in range(1, steps + 1):
        orc.adamw_step(st, grads[t - 1], orc.hparams(**HP, step=t, master_bits=32,
                                                      companded=companded))
        th, mq, msc, vq, vsc = ref[t - 1]
        assert (orc.reconstruct(st.param, st.rho, 32).view(np.uint32) == th.view(np.uint32)).all()
        assert (st.m_codes == mq).all() and (st.m_scales == msc).all()
        assert (st.v_codes == vq).all() and (st.v_scales == vsc).all()


def test_24bit_step_is_teacher_forced_composition(orc):
    rng = np.random.default_rng(4)
    n, steps = 2048 + 31, 5
    p0 = _bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    st = orc.State.zeros_like_param(p0, 24)
    for t in range(1, steps + 1):
        g = _bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32))
        theta = orc.reconstruct(st.param, st.rho, 24)
        m = orc.dequantize(st.m_codes, st.m_scales, orc.MOMENTUM)
        v = orc.dequantize(st.v_codes, st.v_scales, orc.VARIANCE)
        th1, m1, v1 = orc.adamw_update(theta, m, v, _bits_to_f32(g), orc.hparams(**HP, step=t))
        orc.adamw_step(st, g, orc.hparams(**HP, step=t, master_bits=24))
        hi, rho = orc.split(th1, 24)
        assert (st.param == hi).all() and (st.rho == rho).all()
        qm, sm = orc.quantize(m1, orc.MOMENTUM)
        qv, sv = orc.quantize(v1, orc.VARIANCE)
        assert (st.m_codes == qm).all() and (st.m_scales == sm).all()
        assert (st.v_codes == qv).all() and (st.v_scales == sv).all()


def test_unquantized_states_and_plain_param(orc):
    """quantize_states=False keeps fp32 moments (the weight-splitting-only
    ablation); master_bits=None rounds the updated parameter to bf16 with
    torch's cast."""
    rng = np.random.default_rng(5)
    n = 1000
    p0 = _bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    g = _bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32))
    st = orc.State.zeros_like_param(p0, None, quantize_states=False)
    orc.adamw_step(st, g, orc.hparams(**HP, step=1, master_bits=None, quantize_states=False))
    th, m, v = orc.adamw_update(_bits_to_f32(p0), np.zeros(n), np.zeros(n), _bits_to_f32(g),
                                orc.hparams(**HP, step=1))
    assert (st.m_codes == m).all() and (st.v_codes == v).all()
    assert (st.param == _bf16_bits(th)).all()


@pytest.mark.parametrize("companded,quantized", [(True, True), (False, True), (True, False)])
def test_fp32_param_equals_lossless_32bit_master(orc, companded, quantized):
    """An fp32 parameter is never split (use_split is false for it on page
    "code/flashsim/flash_adamw_sim.py", FlashAdamWSim.step): theta is the
    parameter and the update is stored unchanged.  The 32-bit master split is
    lossless, so with gradients that bf16 holds exactly the two must agree
    bit for bit at every step, the states included."""
    rng = np.random.default_rng(9)
    n, steps = 4096 + 45, 5
    theta = (rng.standard_normal(n) * 0.02).astype(np.float32)
    hi, rho = orc.split(theta, 32)
    a = orc.State.zeros_like_param(theta.copy(), None, quantize_states=quantized)
    b = orc.State.zeros_like_param(hi, 32, quantize_states=quantized)
    b.rho[:] = rho
    for t in range(1, steps + 1):
        g = _bf16_bits((rng.standard_normal(n) * 1e-3 * np.exp(rng.standard_normal())).astype(np.float32))
        orc.adamw_step(a, _bits_to_f32(g), orc.hparams(**HP, step=t, master_bits=None, companded=companded,
                                                       quantize_states=quantized, fp32_param=True))
        orc.adamw_step(b, g, orc.hparams(**HP, step=t, master_bits=32, companded=companded,
                                         quantize_states=quantized))
        assert (a.param.view(np.uint32) == orc.reconstruct(b.param, b.rho, 32).view(np.uint32)).all()
        for f in ("m_codes", "m_scales", "v_codes", "v_scales"):
            x, y = getattr(a, f), getattr(b, f)
            assert (x is None and y is None) or (x.view(np.uint8) == y.view(np.uint8)).all(), f


def test_list_driver_equals_per_tensor_steps(orc):
    rng = np.random.default_rng(6)
    sizes = [1, 31, 32, 33, 4096, 70001, 32768 * 2 + 5]
    for mb in (24, 32):
        states_a, states_b, grads = [], [], []
        for n in sizes:
            p0 = _bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
            s = orc.State.zeros_like_param(p0, mb)
            states_a.append(s)
            states_b.append(s.copy())
            grads.append(_bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32)))
        for t in (1, 2, 3):
            hp = orc.hparams(**HP, step=t, master_bits=mb)
            for s, g in zip(states_a, grads):
                orc.adamw_step(s, g, hp)
            used = orc.adamw_step_list(states_b, grads, hp, threads=4)
            assert used >= 1
        for a, b in zip(states_a, states_b):
            for f in ("param", "rho", "m_codes", "m_scales", "v_codes", "v_scales"):
                assert (getattr(a, f) == getattr(b, f)).all(), f


def test_bad_arguments_rejected(orc):
    p = np.zeros(8, np.uint16)
    st = orc.State.zeros_like_param(p, 24)
    with pytest.raises(ValueError):
        orc.adamw_step(st, p, orc.hparams(step=0))
    with pytest.raises(ValueError):
        orc.adamw_step(st, p, orc.hparams(step=1, master_bits=16))
    # an fp32 parameter is never split, so a master width is rejected for it
    f = orc.State.zeros_like_param(np.zeros(8, np.float32), None)
    hp = orc.hparams(step=1, master_bits=24, fp32_param=True)
    rc = orc.lib().oracle_adamw_step(f.param.ctypes.data, f.param.ctypes.data, None,
                                     f.m_codes.ctypes.data, f.m_scales.ctypes.data,
                                     f.v_codes.ctypes.data, f.v_scales.ctypes.data, 8,
                                     orc.ctypes.byref(hp))
    assert rc == -1


def test_long_trajectory_tracks_torch_adamw(orc):
    """300 free-running steps of the oracle's step with fp32 moments and the
    lossless 32-bit master (so its master is a plain fp32 AdamW parameter)
    against torch.optim.AdamW fed the same bf16 gradients.  Per step the two
    thetas drift apart by rounding only: the decay product and the final
    subtraction round once each (at most 2^-23 |theta| together, |theta| <
    0.25 here), the update (|u| <= 10 lr) differs by a few of its own ulps,
    and a v that differs by at most ~500 ulps (rounding error decaying with
    beta2) changes the update by under 2e-8.  Summed over 300 steps that is
    below 3e-5 absolute; a wrong bias correction, coupled weight decay or a
    dropped term moves theta by 1e-4 or more."""
    rng = np.random.default_rng(8)
    n, steps = 1 << 14, 300
    p0 = _bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    st = orc.State.zeros_like_param(p0, 32, quantize_states=False)
    p = torch.nn.Parameter(torch.from_numpy(_bits_to_f32(p0).copy()))
    opt = torch.optim.AdamW([p], lr=HP["lr"], betas=HP["betas"], eps=HP["eps"],
                            weight_decay=HP["weight_decay"], foreach=False, fused=False)
    for t in range(1, steps + 1):
        g = _bf16_bits((rng.standard_normal(n) * 1e-3 * np.exp(rng.standard_normal())).astype(np.float32))
        orc.adamw_step(st, g, orc.hparams(**HP, step=t, master_bits=32, quantize_states=False))
        p.grad = torch.from_numpy(_bits_to_f32(g).copy())
        opt.step()
        if t in (1, 10, 100, steps):
            th = orc.reconstruct(st.param, st.rho, 32).astype(np.float64)
            assert np.abs(th).max() < 0.25
            assert (np.abs(th - p.detach().numpy()) <= 3e-5).all(), t
            v_ref = opt.state[p]["exp_avg_sq"].numpy().astype(np.float64)
            assert (np.abs(st.v_codes - v_ref) <= 1e-4 * v_ref).all(), t


def test_constant_group_trajectory_closed_form(orc):
    """Four groups (the last one ragged), each holding one value repeated:
    at every step its momentum code is +-127 and its variance code 255, since
    the group maximum's fp16 rounding moves |m1| / scale and sqrt(v1) / scale
    by at most 2^-11 from 1, and dequantize(+-127) = +-scale, dequantize(255)
    = scale^2 exactly.  So the companded states follow m <- fp16(m1),
    v <- fl(fp16(sqrt(v1))^2), and with the lossless 32-bit master theta
    follows the update of page "code/flashsim/flash_adamw_sim.py"
    (FlashAdamWSim.step) in float32.  The gradients keep every moment in
    fp16's normal range, where these bounds hold."""
    rng = np.random.default_rng(13)
    sizes = [32, 32, 32, 7]
    n, steps = sum(sizes), 40
    group_of = np.repeat(np.arange(len(sizes)), sizes)
    theta0 = _bits_to_f32(_bf16_bits((rng.standard_normal(len(sizes)) * 0.5).astype(np.float32)))
    gs = [_bits_to_f32(_bf16_bits((rng.choice([-1.0, 1.0], len(sizes)) *
                                   rng.uniform(0.02, 0.2, len(sizes))).astype(np.float32)))
          for _ in range(steps)]
    st = orc.State.zeros_like_param(_bf16_bits(theta0[group_of]), 32)
    f32 = np.float32
    lr, wd, (beta1, beta2), eps = HP["lr"], HP["weight_decay"], HP["betas"], HP["eps"]
    cwd, b1, c1, b2, c2 = f32(1 - lr * wd), f32(beta1), f32(1 - beta1), f32(beta2), f32(1 - beta2)
    th, m, v = theta0.copy(), np.zeros(len(sizes), f32), np.zeros(len(sizes), f32)
    for t in range(1, steps + 1):
        g = gs[t - 1]
        orc.adamw_step(st, _bf16_bits(g[group_of]), orc.hparams(**HP, step=t, master_bits=32))
        bc1, bc2 = f32(1 - beta1 ** t), f32(1 - beta2 ** t)
        thd = th * cwd
        m1 = b1 * m + c1 * g
        v1 = b2 * v + (c2 * g) * g
        mhat, vhat = m1 / bc1, v1 / bc2
        th = thd - (f32(lr) * mhat) / (np.sqrt(vhat) + f32(eps))
        sm = np.abs(m1).astype(np.float16)
        sv = np.sqrt(v1).astype(np.float16)
        assert (np.abs(sm.astype(f32)) > 6.2e-5).all() and (sv.astype(f32) > 6.2e-5).all()
        m = np.copysign(sm.astype(f32), m1)
        v = sv.astype(f32) * sv.astype(f32)
        assert (st.m_codes == np.where(m1 < 0, -127, 127)[group_of]).all(), f"t{t}: m codes"
        assert (st.v_codes == 255).all(), f"t{t}: v codes"
        assert (st.m_scales == sm.view(np.uint16)).all(), f"t{t}: m scales"
        assert (st.v_scales == sv.view(np.uint16)).all(), f"t{t}: v scales"
        got = orc.reconstruct(st.param, st.rho, 32)
        assert (got.view(np.uint32) == th[group_of].view(np.uint32)).all(), f"t{t}: theta"
    # the states the oracle stores decode to the recursion's moments
    assert (orc.dequantize(st.m_codes, st.m_scales, orc.MOMENTUM) == m[group_of]).all()
    assert (orc.dequantize(st.v_codes, st.v_scales, orc.VARIANCE) == v[group_of]).all()

