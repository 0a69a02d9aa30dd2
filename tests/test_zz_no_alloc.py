"""The allocation-free list step (flashopt_adamw_step_noalloc) against the
workspace list step (flashopt_adamw_step), both through the C ABI, on copies
of the same seeded states: every stored byte equal after two calls in a row,
the second with a smaller list (the device table then holds the first call's
entries beyond the second's), for three storage variants and the
chunk-blocked state layout."""
import ctypes

import numpy as np
import pytest
import torch

from bit_companded_adam_amd import flashopt as F
from bit_companded_adam_amd import workloads as W
from tests._gpu import host, require_gpu

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
BIG = [1 << 16, 3000, 70001, 1, 33, (1 << 18) + 77, 4096] * 6       # 42 tensors, ragged
SMALL_IDX = [2, 0, 5]                                                 # 3 of them, reordered


def _states(mb, qs, layout):
    return [F.TensorState(W.init_param(n, device="cuda", seed=500 + i), mb, qs, state_layout=layout)
            for i, n in enumerate(BIG)]


def _bytes(st):
    ts = (st.param.view(torch.int16), st.rho, st.m_codes, st.m_scales, st.v_codes, st.v_scales)
    return [host(t).view(np.uint8) for t in ts if t is not None]


@pytest.mark.parametrize("mb,comp,qs,layout", [(24, True, True, "streams"), (32, False, True, "streams"),
                                               (None, True, False, "streams"), (24, True, True, "blocked")],
                         ids=["mb24-comp", "mb32-lin", "mbnone-f32", "mb24-comp-blocked"])
def test_noalloc_step_equals_workspace_step(mb, comp, qs, layout):
    require_gpu()
    L = F.lib()
    ref, got = _states(mb, qs, layout), _states(mb, qs, layout)
    ws = torch.empty(max(16, F.flashopt_adamw_workspace_bytes(len(BIG))), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    calls = [(list(range(len(BIG))), 1), (SMALL_IDX, 2)]
    for call, (idx, t) in enumerate(calls):
        grads = [W.make_grad(BIG[i], t, device="cuda", stream_id=i) for i in idx]
        args = F.make_args(t, master_bits=mb, companded=comp, quantize_states=qs,
                           state_layout=layout, **HP)
        F.flashopt_adamw_step(F.descriptor_array([ref[i] for i in idx], grads), args, ws)
        desc = F.descriptor_array([got[i] for i in idx], grads)
        print(f"noalloc call {call}: {len(idx)} tensors, step {t}", flush=True)
        status = L.flashopt_adamw_step_noalloc(desc, len(idx), ctypes.byref(args), stream)
        assert status == F.FLASHOPT_OK, F.status_str(status)
        torch.cuda.synchronize()
        for i in range(len(BIG)):
            for a, b in zip(_bytes(ref[i]), _bytes(got[i])):
                assert (a == b).all(), f"call {call} tensor {i}"
