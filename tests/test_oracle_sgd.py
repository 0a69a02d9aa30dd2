"""Pins for the oracle's FlashSGD step.  FlashSGD appears on page
"code/flashsim/flash_adamw_sim.py" only in bytes_per_param ("flash_sgd": bf16
master + rho + grad + one quantized state); its update is read as
torch.optim.SGD with momentum, the buffer stored with the momentum spec.

* The update alone (fp32 buffer) is pinned to torch.optim.SGD, an
  independent library implementation, teacher-forced step by step, for plain
  momentum, dampening and Nesterov, with and without weight decay.
* Step 1 has a closed form: the buffer is the (decayed) gradient itself.
* With a 32-bit master the split is lossless, so K steps equal an fp32-master
  composition of the (separately pinned) codec and update.
* Without quantization and without a split, the parameter is torch's bf16
  cast of the fp32 update.
* 300 free-running steps with an fp32 buffer and the 32-bit master track
  torch.optim.SGD within a derived rounding bound.
* A group whose 32 elements are equal always gets the code +-127, which
  dequantizes to exactly the group's fp16 scale, so a quantized buffer
  follows buf <- fp16(buf1): 40 steps of four such groups follow that float32
  recursion bit for bit.
A long trajectory with a quantized buffer in general, or with the 24-bit
master, has no independent pin beyond this composition (parity unpinned for
it)."""
import numpy as np
import pytest
import torch


def _bf16_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("dampening,nesterov,wd", [(0.0, False, 0.0), (0.0, False, 0.01),
                                                     (0.0, True, 0.01), (0.1, False, 0.0)])
def test_update_matches_torch_sgd(orc, dampening, nesterov, wd):
    rng = np.random.default_rng(11)
    n, steps, lr, mu = 1 << 14, 8, 1e-2, 0.9
    theta = (rng.standard_normal(n) * 0.02).astype(np.float32)
    p = torch.nn.Parameter(torch.from_numpy(theta.copy()))
    opt = torch.optim.SGD([p], lr=lr, momentum=mu, dampening=dampening, nesterov=nesterov,
                          weight_decay=wd, foreach=False)
    buf = np.zeros(n, np.float32)
    for t in range(1, steps + 1):
        g = (rng.standard_normal(n) * 1e-3 * np.exp(rng.standard_normal())).astype(np.float32)
        with torch.no_grad():
            p.copy_(torch.from_numpy(theta))
        if t > 1:
            opt.state[p]["momentum_buffer"].copy_(torch.from_numpy(buf))
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        hp = orc.sgd_hparams(lr=lr, momentum=mu, dampening=dampening, weight_decay=wd,
                             step=t, nesterov=nesterov)
        d_terms = np.abs(g) + wd * np.abs(theta)
        b_terms = mu * np.abs(buf) + d_terms
        theta_new, buf = orc.sgd_update(theta, buf, g, hp)
        tb = opt.state[p]["momentum_buffer"].numpy()
        # torch may fuse a multiply into an add (one rounding instead of two):
        # allow a few ulps of the terms
        assert (np.abs(buf - tb) <= 3e-7 * b_terms + 1e-30).all(), t
        th_terms = np.abs(theta) + lr * (b_terms + mu * b_terms)
        assert (np.abs(theta_new - p.detach().numpy()) <= 3e-7 * th_terms + 1e-30).all(), t
        theta = theta_new


@pytest.mark.parametrize("master_bits", [24, 32])
def test_step1_closed_form(orc, master_bits):
    """Step 1 from a zero state: buf = g + wd theta exactly as its fp32
    evaluation, the codes are the momentum quantizer's codes of that buffer,
    and the master is theta - lr buf."""
    rng = np.random.default_rng(12)
    n, lr, wd = 4096 + 13, 1e-2, 0.01
    p0 = _bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    g = _bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32))
    st = orc.State.zeros_like_param(p0, master_bits)
    st.m_codes[:] = 77                  # step 1 ignores the stored buffer
    st.m_scales[:] = 0x3C00
    orc.sgd_step(st, g, orc.sgd_hparams(lr=lr, momentum=0.9, weight_decay=wd, step=1,
                                        master_bits=master_bits))
    th0 = _bits_to_f32(p0)
    buf = (_bits_to_f32(g) + np.float32(wd) * th0).astype(np.float32)
    q, s = orc.quantize(buf, orc.MOMENTUM)
    assert (st.m_codes == q).all() and (st.m_scales == s).all()
    th1 = orc.reconstruct(st.param, st.rho, master_bits).astype(np.float64)
    want = th0.astype(np.float64) - lr * buf.astype(np.float64)
    tol = (1e-6 * np.abs(want) + 2.0 ** -15 * np.abs(want)) if master_bits == 24 else 1e-6 * np.abs(want)
    assert (np.abs(th1 - want) <= tol + 1e-12).all()


@pytest.mark.parametrize("companded", [True, False])
def test_32bit_master_equals_fp32_master(orc, companded):
    rng = np.random.default_rng(13)
    n, steps, lr = 3000 + 5, 6, 1e-2
    spec = orc.MOMENTUM if companded else orc.MOMENTUM_LINEAR
    p0 = _bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    grads = [_bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32)) for _ in range(steps)]
    st = orc.State.zeros_like_param(p0, 32)
    theta = _bits_to_f32(p0).copy()
    q, s = np.zeros(n, np.int8), np.zeros((n + 31) // 32, np.uint16)
    for t in range(1, steps + 1):
        hp = orc.sgd_hparams(lr=lr, momentum=0.9, weight_decay=0.01, step=t, master_bits=32,
                             companded=companded)
        buf = orc.dequantize(q, s, spec)
        theta, buf = orc.sgd_update(theta, buf, _bits_to_f32(grads[t - 1]), hp)
        q, s = orc.quantize(buf, spec)
        orc.sgd_step(st, grads[t - 1], hp)
        assert (orc.reconstruct(st.param, st.rho, 32).view(np.uint32) == theta.view(np.uint32)).all()
        assert (st.m_codes == q).all() and (st.m_scales == s).all()


def test_unquantized_buffer_and_plain_param(orc):
    rng = np.random.default_rng(14)
    n = 1000
    p0 = _bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    st = orc.State.zeros_like_param(p0, None, quantize_states=False)
    theta, buf = _bits_to_f32(p0), np.zeros(n, np.float32)
    for t in (1, 2, 3):
        g = _bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32))
        hp = orc.sgd_hparams(lr=1e-2, momentum=0.9, step=t, master_bits=None, quantize_states=False)
        theta, buf = orc.sgd_update(_bits_to_f32(st.param), buf, _bits_to_f32(g), hp)
        orc.sgd_step(st, g, hp)
        assert (st.m_codes == buf).all()
        assert (st.param == _bf16_bits(theta)).all()


def test_bad_arguments_rejected(orc):
    st = orc.State.zeros_like_param(np.zeros(64, np.uint16), 24)
    g = np.zeros(64, np.uint16)
    with pytest.raises(ValueError):
        orc.sgd_step(st, g, orc.sgd_hparams(step=0))
    with pytest.raises(ValueError):
        orc.sgd_step(st, g, orc.sgd_hparams(master_bits=16))


@pytest.mark.parametrize("dampening,nesterov,wd", [(0.0, False, 0.01), (0.0, True, 0.01), (0.1, False, 0.0)])
def test_long_trajectory_tracks_torch_sgd(orc, dampening, nesterov, wd):
    """300 free-running steps of the oracle's FlashSGD step with an fp32
    buffer and the lossless 32-bit master against torch.optim.SGD fed the
    same bf16 gradients.  The thetas drift apart by rounding only: the final
    subtraction rounds once per step (at most 2^-24 |theta|, |theta| < 0.25
    here), and the buffers' rounding differences decay with the momentum
    (a steady ~10 ulps of the buffer, times lr, per step).  Over 300 steps
    that stays below 1e-5; a dropped or misplaced momentum, dampening or
    weight-decay term moves theta by far more."""
    rng = np.random.default_rng(12)
    n, steps, lr, mu = 1 << 14, 300, 1e-2, 0.9
    p0 = _bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    st = orc.State.zeros_like_param(p0, 32, quantize_states=False)
    st.v_codes = st.v_scales = None
    p = torch.nn.Parameter(torch.from_numpy(_bits_to_f32(p0).copy()))
    opt = torch.optim.SGD([p], lr=lr, momentum=mu, dampening=dampening, nesterov=nesterov,
                          weight_decay=wd, foreach=False)
    for t in range(1, steps + 1):
        g = _bf16_bits((rng.standard_normal(n) * 1e-3 * np.exp(rng.standard_normal())).astype(np.float32))
        orc.sgd_step(st, g, orc.sgd_hparams(lr=lr, momentum=mu, dampening=dampening, weight_decay=wd,
                                            nesterov=nesterov, step=t, master_bits=32,
                                            quantize_states=False))
        p.grad = torch.from_numpy(_bits_to_f32(g).copy())
        opt.step()
        if t in (1, 10, 100, steps):
            th = orc.reconstruct(st.param, st.rho, 32).astype(np.float64)
            assert np.abs(th).max() < 0.25
            assert (np.abs(th - p.detach().numpy()) <= 1e-5).all(), t


@pytest.mark.parametrize("dampening,nesterov", [(0.1, False), (0.0, True)])
def test_constant_group_trajectory_closed_form(orc, dampening, nesterov):
    """Four groups (the last one ragged), each holding one value repeated:
    the momentum code is +-127 at every step (the fp16 rounding of the group
    maximum moves |buf1| / scale by at most 2^-11 from 1) and dequantizes to
    +-scale exactly, so the stored buffer follows buf <- fp16(buf1), and with
    the lossless 32-bit master theta follows torch.optim.SGD's order in
    float32 (d = g + wd theta; buf1 = d at step 1, else mu buf + (1 -
    dampening) d; the direction buf1, or d + mu buf1 with Nesterov)."""
    rng = np.random.default_rng(17)
    sizes = [32, 32, 32, 9]
    n, steps = sum(sizes), 40
    lr, mu, wd = 1e-2, 0.9, 0.01
    group_of = np.repeat(np.arange(len(sizes)), sizes)
    theta0 = _bits_to_f32(_bf16_bits((rng.standard_normal(len(sizes)) * 0.5).astype(np.float32)))
    gs = [_bits_to_f32(_bf16_bits((rng.choice([-1.0, 1.0], len(sizes)) *
                                   rng.uniform(0.02, 0.2, len(sizes))).astype(np.float32)))
          for _ in range(steps)]
    st = orc.State.zeros_like_param(_bf16_bits(theta0[group_of]), 32)
    f32 = np.float32
    th, buf = theta0.copy(), np.zeros(len(sizes), f32)
    for t in range(1, steps + 1):
        g = gs[t - 1]
        orc.sgd_step(st, _bf16_bits(g[group_of]),
                     orc.sgd_hparams(lr=lr, momentum=mu, dampening=dampening, weight_decay=wd,
                                     step=t, master_bits=32, nesterov=nesterov))
        d = g + f32(wd) * th
        b1 = d if t == 1 else f32(mu) * buf + f32(1 - dampening) * d
        direction = d + f32(mu) * b1 if nesterov else b1
        th = th - f32(lr) * direction
        sc = np.abs(b1).astype(np.float16)
        assert (sc.astype(f32) > 6.2e-5).all()
        buf = np.copysign(sc.astype(f32), b1)
        assert (st.m_codes == np.where(b1 < 0, -127, 127)[group_of]).all(), f"t{t}: codes"
        assert (st.m_scales == sc.view(np.uint16)).all(), f"t{t}: scales"
        got = orc.reconstruct(st.param, st.rho, 32)
        assert (got.view(np.uint32) == th[group_of].view(np.uint32)).all(), f"t{t}: theta"

