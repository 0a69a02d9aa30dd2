"""The Python binding's step driver on the GPU: the descriptor table it caches
between list steps is rebuilt whenever a gradient's storage changes, the
gradients are validated before anything is launched, no reference to them
outlives the call, and optimizers stepped from several threads on their own
streams at once give the same bits as one at a time."""
import gc
import weakref

import pytest
import torch

from bit_companded_adam_amd import flashopt as F
from bit_companded_adam_amd import workloads as W
from tests._gpu import require_gpu, u16

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
SIZES = [4096 + 5, 1 << 15]


def _params(seed):
    return [W.init_param(n, device="cuda", seed=seed + i) for i, n in enumerate(SIZES)]


def _grads(t):
    return [W.make_grad(n, t, device="cuda", stream_id=i) for i, n in enumerate(SIZES)]


def _state_bits(opt):
    out = []
    for s in opt.states:
        out += [u16(s.param), s.rho.cpu().numpy(), s.m_codes.cpu().numpy(), u16(s.m_scales),
                s.v_codes.cpu().numpy(), u16(s.v_scales)]
    return out


def test_new_gradient_tensors_rebuild_the_table():
    """Step 2 with freshly allocated gradients gives the same bits as step 2
    with the step-1 tensors refilled in place (whose cached table stays
    valid)."""
    require_gpu()
    fresh = F.FlashAdamW(_params(10), **HP)
    inplace = F.FlashAdamW(_params(10), **HP)
    g1 = _grads(1)
    fresh.step(g1)
    keep = [g.clone() for g in g1]
    inplace.step(keep)
    g2 = _grads(2)
    fresh.step(g2)                       # new storage: the table is rebuilt
    for k, g in zip(keep, g2):
        k.copy_(g)                       # same storage, new values
    inplace.step(keep)
    torch.cuda.synchronize()
    for a, b in zip(_state_bits(fresh), _state_bits(inplace)):
        assert (a == b).all()


def test_gradient_count_and_layout_are_checked_before_launch():
    require_gpu()
    opt = F.FlashAdamW(_params(20), **HP)
    g = _grads(1)
    with pytest.raises(ValueError):
        opt.step(g[:1])
    assert opt.t == 0
    opt.step(g)
    # the same storage, size and dtype seen as a non-contiguous view
    side = 64
    p2 = W.init_param(side * side, device="cuda", seed=30)
    opt2 = F.FlashAdamW([p2], **HP)
    g2 = W.make_grad(side * side, 1, device="cuda").view(side, side)
    opt2.step([g2.reshape(-1)])
    with pytest.raises(ValueError):
        opt2.step([g2.t()])
    assert opt2.t == 1


def test_gradients_are_not_kept_alive():
    require_gpu()
    opt = F.FlashSGD(_params(40), lr=1e-2, momentum=0.9)
    g = _grads(1)
    refs = [weakref.ref(x) for x in g]
    opt.step(g)
    torch.cuda.synchronize()
    del g
    gc.collect()
    assert all(r() is None for r in refs)


def test_threads_on_their_own_streams_match_sequential_steps():
    """Four host threads, each stepping its own optimizer on its own stream
    (default priority) at once, share the library's pinned staging ring:
    every state must equal the same steps run one optimizer at a time."""
    import threading

    require_gpu()
    kinds = ["adamw", "sgd", "adamw", "sgd"]

    def make(k, seed):
        params = [W.init_param(n, device="cuda", seed=seed + i) for i, n in enumerate(SIZES)]
        if k == "adamw":
            return F.FlashAdamW(params, **HP)
        return F.FlashSGD(params, lr=1e-2, momentum=0.9, weight_decay=0.01)

    grads = [[[W.make_grad(n, t, device="cuda", stream_id=10 * j + i) for i, n in enumerate(SIZES)]
              for t in range(1, 9)] for j in range(len(kinds))]
    torch.cuda.synchronize()
    seq = [make(k, 100 + 10 * j) for j, k in enumerate(kinds)]
    for j, opt in enumerate(seq):
        for g in grads[j]:
            opt.step(g)
    torch.cuda.synchronize()

    par = [make(k, 100 + 10 * j) for j, k in enumerate(kinds)]
    streams = [torch.cuda.Stream() for _ in kinds]
    torch.cuda.synchronize()
    errors = []

    def run(j):
        try:
            with torch.cuda.stream(streams[j]):
                for g in grads[j]:
                    par[j].step(g)
        except Exception as e:          # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(j,)) for j in range(len(kinds))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for j, (a, b) in enumerate(zip(seq, par)):
        for x, y in zip(_state_bits(a) if kinds[j] == "adamw" else _sgd_bits(a),
                        _state_bits(b) if kinds[j] == "adamw" else _sgd_bits(b)):
            assert (x == y).all(), f"optimizer {j} ({kinds[j]})"


def _sgd_bits(opt):
    out = []
    for s in opt.states:
        out += [u16(s.param), s.rho.cpu().numpy(), s.m_codes.cpu().numpy(), u16(s.m_scales)]
    return out


def test_list_launches_on_two_streams_use_their_own_workspaces():
    """One optimizer steps two disjoint halves of its tensors as list launches
    on two streams, alternating, with no synchronization between them: each
    stream's launches keep their own chunk table, so the results equal the
    same subset steps issued on one stream."""
    require_gpu()
    sizes = [1 << 18, 70001, 4096 + 5, 1 << 17, 3000, (1 << 18) + 77]
    half_a, half_b = [0, 2, 4], [1, 3, 5]
    mk = lambda: F.FlashAdamW([W.init_param(n, device="cuda", seed=600 + i)
                               for i, n in enumerate(sizes)], **W.HP_DEFAULT)
    two, one = mk(), mk()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    keep = []                                # no gradient memory is reused while a stream reads it
    for t in range(1, 5):
        grads = [W.make_grad(n, t, device="cuda", stream_id=i) for i, n in enumerate(sizes)]
        keep.append(grads)
        torch.cuda.synchronize()             # the gradients exist before either stream reads them
        two.step_tensors(half_a, [grads[i] for i in half_a], stream=sa)
        two.step_tensors(half_b, [grads[i] for i in half_b], stream=sb)
        one.step_tensors(half_a, [grads[i] for i in half_a])
        one.step_tensors(half_b, [grads[i] for i in half_b])
    torch.cuda.synchronize()
    assert len(two._workspaces) == 2
    for i, (x, y) in enumerate(zip(two.states, one.states)):
        for name in ("param", "rho", "m_codes", "m_scales", "v_codes", "v_scales"):
            a, b = getattr(x, name), getattr(y, name)
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"tensor {i} {name}"


def test_codec_and_split_wrappers_refuse_bad_buffers():
    """The C ABI takes plain pointers, so the binding checks caller-supplied
    buffers before it launches anything: a short or mistyped output buffer
    raises ValueError instead of being written past its end."""
    require_gpu()
    n = 1000
    x = torch.randn(n, device="cuda")
    ok_codes = torch.empty(n, dtype=torch.int8, device="cuda")
    ok_scales = torch.empty(F.n_groups(n), dtype=torch.int16, device="cuda")
    bad = [
        lambda: F.flashopt_quantize(x, F.SPEC_MOMENTUM, torch.empty(n - 1, dtype=torch.int8, device="cuda"), ok_scales),
        lambda: F.flashopt_quantize(x, F.SPEC_MOMENTUM, torch.empty(n, dtype=torch.int16, device="cuda"), ok_scales),
        lambda: F.flashopt_quantize(x, F.SPEC_MOMENTUM, ok_codes, ok_scales[:-1]),
        lambda: F.flashopt_quantize(x, F.SPEC_MOMENTUM, torch.empty(n, dtype=torch.int8), ok_scales),
        lambda: F.flashopt_dequantize(ok_codes, ok_scales, F.SPEC_MOMENTUM, torch.empty(n - 1, device="cuda")),
        lambda: F.flashopt_dequantize(ok_codes, ok_scales, F.SPEC_MOMENTUM,
                                      torch.empty(n, dtype=torch.float16, device="cuda")),
        lambda: F.flashopt_dequantize(ok_codes.view(torch.int16), ok_scales, F.SPEC_MOMENTUM),
        lambda: F.flashopt_dequantize(ok_codes, ok_scales[:-1], F.SPEC_MOMENTUM),
        lambda: F.flashopt_split(x, 24, rho=torch.empty(n, dtype=torch.int16, device="cuda")[: n // 2]),
        lambda: F.flashopt_split(x, 24, param=torch.empty(n, dtype=torch.float32, device="cuda")),
        lambda: F.flashopt_split(x, 32, rho=torch.empty(n, dtype=torch.int8, device="cuda")),
        lambda: F.flashopt_split(x, 16),
        lambda: F.flashopt_reconstruct(torch.empty(n, dtype=torch.bfloat16, device="cuda"),
                                       torch.empty(n - 1, dtype=torch.int8, device="cuda"), 24),
        lambda: F.flashopt_reconstruct(torch.empty(n, dtype=torch.bfloat16, device="cuda"),
                                       torch.empty(n, dtype=torch.int8, device="cuda"), 24,
                                       out=torch.empty(n, dtype=torch.bfloat16, device="cuda")),
    ]
    for i, call in enumerate(bad):
        with pytest.raises(ValueError):
            call()
        torch.cuda.synchronize()
    # the same calls with good buffers run
    q, s = F.flashopt_quantize(x, F.SPEC_MOMENTUM, ok_codes, ok_scales)
    F.flashopt_dequantize(q, s, F.SPEC_MOMENTUM)
    p, r = F.flashopt_split(x, 24)
    F.flashopt_reconstruct(p, r, 24)
    torch.cuda.synchronize()

