"""The capture-safe list steps (flashopt_adamw_plan / flashopt_sgd_plan,
_plan_set_step, _plan_launch; FlashAdamW.plan and FlashSGD.plan in the
binding).  A plan launch must leave the bits the list step
(flashopt_adamw_step / flashopt_sgd_step) leaves with the same tensors,
gradients and step (the list steps are checked against the oracle elsewhere,
so equality carries that parity over), and a launch captured once into a HIP
graph must replay with the scalars each set_step wrote: every replay equals
an eager list step at its own step count."""
import pytest
import torch

from bit_companded_adam_amd import flashopt as F
from bit_companded_adam_amd import workloads as W
from tests._gpu import require_gpu

pytestmark = pytest.mark.gpu

SIZES = [1, 33, 1000, 1024, 1025, 70001, 1 << 17]
# (master_bits, companded, quantize_states, parameter dtype, state layout;
# None: the binding's default, blocked for quantized states)
VARIANTS = [(24, True, True, torch.bfloat16, None), (32, False, True, torch.bfloat16, None),
            (None, True, False, torch.bfloat16, None), (None, True, True, torch.float32, None),
            (24, True, True, torch.bfloat16, "streams")]
IDS = ["mb24-comp", "mb32-lin", "mbNone-f32states", "fp32params", "mb24-comp-streams"]


def _pair(variant, seed):
    mb, comp, qs, dt, layout = variant
    pa = [W.init_param(n, device="cuda", seed=seed + i, dtype=dt) for i, n in enumerate(SIZES)]
    pb = [p.clone() for p in pa]
    make = lambda ps: F.FlashAdamW(ps, master_bits=mb, companded=comp, quantize_states=qs,
                                   state_layout=layout, **W.HP_DEFAULT)
    return make(pa), make(pb), dt


def _grads(t, dt):
    return [W.make_grad(n, t, device="cuda", stream_id=i, dtype=dt) for i, n in enumerate(SIZES)]


def _bits(x):
    if x is None:
        return None
    return x.view(torch.int16) if x.element_size() == 2 else (x.view(torch.int32) if x.element_size() == 4 else x)


def _assert_same(a: F.FlashAdamW, b: F.FlashAdamW, label):
    for i, (sa, sb) in enumerate(zip(a.states, b.states)):
        for name in ("param", "rho", "m_codes", "m_scales", "v_codes", "v_scales"):
            x, y = getattr(sa, name), getattr(sb, name)
            assert (x is None) == (y is None), f"{label} tensor {i}: {name}"
            if x is not None:
                assert torch.equal(_bits(x), _bits(y)), f"{label} tensor {i}: {name}"


@pytest.mark.parametrize("variant", VARIANTS, ids=IDS)
def test_plan_launch_equals_list_step(variant):
    """Steps 1..4 and then step 20001 (past the horizon where both bias
    corrections round to 1), each through a plan launch over fixed gradient
    buffers and through the list step."""
    require_gpu()
    a, b, dt = _pair(variant, 900)
    bufs = [torch.empty(n, dtype=dt, device="cuda") for n in SIZES]
    plan = b.plan(bufs, step=1)
    for t in (1, 2, 3, 4, 20001):
        grads = _grads(t, dt)
        a.t = t - 1
        a.step(grads)
        for buf, g in zip(bufs, grads):
            buf.copy_(g)
        if t != 1:
            plan.set_step(t)
        plan.launch()
        torch.cuda.synchronize()
        _assert_same(a, b, f"step {t}")


@pytest.mark.parametrize("variant", VARIANTS[:2], ids=IDS[:2])
def test_plan_launch_replays_from_a_hip_graph(variant):
    """One plan launch captured into a graph; four replays, each after new
    gradients are copied into the plan's buffers and set_step writes the
    next step's scalars, with eager work and a synchronize between replays:
    every replay equals the list step at its step count."""
    require_gpu()
    a, b, dt = _pair(variant, 950)
    bufs = [torch.zeros(n, dtype=dt, device="cuda") for n in SIZES]
    plan = b.plan(bufs, step=1)
    side = torch.randn(1 << 20, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.launch()
    torch.cuda.synchronize()
    _assert_same(a, b, "after capture")            # capture runs nothing
    for t in (1, 2, 3, 4):
        grads = _grads(t, dt)
        a.step(grads)
        for buf, g in zip(bufs, grads):
            buf.copy_(g)
        plan.set_step(t)
        graph.replay()
        side.mul_(1.0001).add_(t)                   # eager work between replays
        torch.cuda.synchronize()
        _assert_same(a, b, f"replay at step {t}")


def test_plan_set_step_takes_new_hyper_parameters():
    """set_step writes any hyper-parameters of the plan's variant: a learning
    rate schedule and a weight-decay change, through the C-ABI calls, over a
    list that includes an empty tensor, equal list steps given the same
    arguments."""
    require_gpu()
    sizes = [4096 + 5, 0, 70001, 33]
    pa = [W.init_param(n, device="cuda", seed=980 + i) for i, n in enumerate(sizes)]
    a = F.FlashAdamW(pa, **W.HP_DEFAULT)
    b = F.FlashAdamW([p.clone() for p in pa], **W.HP_DEFAULT)
    bufs = [torch.zeros(n, dtype=torch.bfloat16, device="cuda") for n in sizes]
    desc_b = F.descriptor_array(b.states, bufs)
    plan = torch.empty(F.flashopt_adamw_plan_bytes(len(sizes)), dtype=torch.uint8, device="cuda")
    schedule = [(1e-3, 0.01), (5e-4, 0.01), (2.5e-4, 0.0), (1e-4, 0.1)]
    base = {k: v for k, v in W.HP_DEFAULT.items() if k not in ("lr", "weight_decay")}
    info = None
    for t, (lr, wd) in enumerate(schedule, start=1):
        args = F.make_args(t, lr=lr, weight_decay=wd, state_layout=a.states[0].state_layout, **base)
        grads = [W.make_grad(n, t, device="cuda", stream_id=i) for i, n in enumerate(sizes)]
        F.flashopt_adamw_step(F.descriptor_array(a.states, grads), args, a.workspace(), None)
        for buf, g in zip(bufs, grads):
            buf.copy_(g)
        if info is None:
            info = F.flashopt_adamw_plan(desc_b, args, plan)
            assert (info.n_tensors, info.total_chunks) == (len(sizes), sum((n + 1023) // 1024 for n in sizes))
        else:
            F.flashopt_adamw_plan_set_step(info, args, plan)
        F.flashopt_adamw_plan_launch(info, plan)
        torch.cuda.synchronize()
        _assert_same(a, b, f"step {t}, lr {lr}, wd {wd}")


def test_decoder_8b_graph_replays_equal_list_steps():
    """The whole 8.0B list (290 tensors) stepped twice through one captured
    plan launch (set_step between replays) and twice through the list step
    from the same seeded start: every stored byte equal after each step
    (compared on the device)."""
    require_gpu()
    shapes = W.decoder_8b_shapes()
    sizes = [W.numel(s) for _, s in shapes]
    factors = W.grad_factors(len(shapes)).tolist()
    params = [W.init_param(n, device="cuda", seed=W.PARAM_SEED + i) for i, n in enumerate(sizes)]
    a = F.FlashAdamW(params, **W.HP_DEFAULT)
    b = F.FlashAdamW([p.clone() for p in params], **W.HP_DEFAULT)
    del params
    grads = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes]
    plan = b.plan(grads, step=1)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.launch()
    for t in (1, 2):
        for i, (g, n) in enumerate(zip(grads, sizes)):
            g.copy_(W.make_grad(n, t, device="cuda", stream_id=i, factor=factors[i]))
        a.step(grads)
        plan.set_step(t)
        graph.replay()
        torch.cuda.synchronize()
        _assert_same(a, b, f"8.0B list, step {t}")



SGD_VARIANTS = [(24, True, True, dict(weight_decay=0.0)), (32, False, True, dict(weight_decay=0.01)),
                (None, True, False, dict(nesterov=True, weight_decay=0.01)),
                (24, True, True, dict(dampening=0.1)),
                (32, True, True, dict(weight_decay=0.01, state_layout="blocked"))]
SGD_IDS = ["mb24-comp", "mb32-lin-wd", "mbNone-f32-nesterov", "mb24-comp-dampening", "mb32-comp-blocked"]


def _sgd_pair(variant, seed):
    mb, comp, qs, extra = variant
    pa = [W.init_param(n, device="cuda", seed=seed + i) for i, n in enumerate(SIZES)]
    pb = [p.clone() for p in pa]
    make = lambda ps: F.FlashSGD(ps, master_bits=mb, companded=comp, quantize_states=qs,
                                 **dict(W.SGD_DEFAULT, **extra))
    return make(pa), make(pb)


@pytest.mark.parametrize("variant", SGD_VARIANTS, ids=SGD_IDS)
def test_sgd_plan_launch_equals_list_step(variant):
    """FlashSGD: step 1 (the buffer set to the gradient) and steps 2..4
    through a plan launch and through the list step."""
    require_gpu()
    a, b = _sgd_pair(variant, 1100)
    bufs = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in SIZES]
    plan = b.plan(bufs, step=1)
    for t in (1, 2, 3, 4):
        grads = _grads(t, torch.bfloat16)
        a.step(grads)
        for buf, g in zip(bufs, grads):
            buf.copy_(g)
        if t != 1:
            plan.set_step(t)
        plan.launch()
        torch.cuda.synchronize()
        _assert_same(a, b, f"sgd step {t}")


def test_sgd_plan_launch_replays_from_a_hip_graph():
    """FlashSGD: one captured plan launch replayed at steps 1..4 (the first
    replay takes the first-step branch from the scalars set_step wrote), eager
    work between replays; every replay equals the list step."""
    require_gpu()
    a, b = _sgd_pair(SGD_VARIANTS[2], 1150)
    bufs = [torch.zeros(n, dtype=torch.bfloat16, device="cuda") for n in SIZES]
    plan = b.plan(bufs, step=2)
    side = torch.randn(1 << 20, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.launch()
    torch.cuda.synchronize()
    _assert_same(a, b, "after capture")
    for t in (1, 2, 3, 4):
        grads = _grads(t, torch.bfloat16)
        a.step(grads)
        for buf, g in zip(bufs, grads):
            buf.copy_(g)
        plan.set_step(t)
        graph.replay()
        side.mul_(1.0001).add_(t)
        torch.cuda.synchronize()
        _assert_same(a, b, f"sgd replay at step {t}")
