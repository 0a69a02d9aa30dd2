"""The C ABI of libflashopt.so without a GPU: the library loads, exports every
entry point include/flashopt.h declares, and rejects bad arguments with the
documented status before it touches the HIP runtime (no compute calls)."""
import ctypes
import os
import re

import pytest

from bit_companded_adam_amd import flashopt as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashopt.h")

A16 = 0x10000          # a fake, 16-byte aligned device address (never dereferenced)
MIS = 0x10001          # a fake misaligned address


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(F._LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return F.lib()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(flashopt_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert set(names) == set(F.EXPORTS)
    for name in names:
        assert hasattr(L, name), name


def test_header_compiles_as_c(tmp_path):
    """include/flashopt.h is plain C: a C11 translation unit that takes the
    address of every declared entry point, with its exact prototype,
    compiles with -Wall -Werror -pedantic (no C++ or HIP types leak into the
    boundary)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    names = _declared()
    src = ["#include \"flashopt.h\"", "typedef void (*fn)(void);", "int main(void) {", "    fn p[] = {"]
    src += [f"        (fn)&{n}," for n in names]
    src += ["    };", "    return (int)(sizeof p / sizeof p[0]) == " + str(len(names)) + " ? 0 : 1;", "}"]
    c = tmp_path / "abi.c"
    c.write_text("\n".join(src) + "\n")
    r = subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-I", os.path.join(ROOT, "include"), "-c", str(c),
                        "-o", str(tmp_path / "abi.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_abi_version_and_status_strings(L):
    ver = int(re.search(r"#define FLASHOPT_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert L.flashopt_abi_version() == ver
    for code in range(5):
        assert F.status_str(code).startswith("FLASHOPT_")
    assert "UNKNOWN" in F.status_str(99)


def test_codec_validation(L):
    q = L.flashopt_quantize
    d = L.flashopt_dequantize
    assert q(None, 0, 5, None, None, None) == F.FLASHOPT_OK          # n == 0 is a no-op
    assert q(A16, -1, 5, A16, A16, None) == F.FLASHOPT_EINVAL
    assert q(A16, 10, 8, A16, A16, None) == F.FLASHOPT_EINVAL         # unknown spec bit
    assert q(None, 10, 5, A16, A16, None) == F.FLASHOPT_EINVAL
    assert q(A16, 10, 5, None, A16, None) == F.FLASHOPT_EINVAL
    assert q(A16, 10, 5, A16, None, None) == F.FLASHOPT_EINVAL
    assert q(MIS, 10, 5, A16, A16, None) == F.FLASHOPT_EALIGN
    assert q(A16, 10, 5, A16 + 8, A16, None) == F.FLASHOPT_EALIGN
    assert q(A16, 10, 5, A16, MIS, None) == F.FLASHOPT_EALIGN
    assert d(None, None, 0, 2, None, None) == F.FLASHOPT_OK
    assert d(A16, A16, -5, 2, A16, None) == F.FLASHOPT_EINVAL
    assert d(A16, A16, 5, 2, MIS, None) == F.FLASHOPT_EALIGN


def test_split_validation(L):
    s = L.flashopt_split
    r = L.flashopt_reconstruct
    assert s(None, 0, 24, None, None, None) == F.FLASHOPT_OK
    assert s(A16, 10, 16, A16, A16, None) == F.FLASHOPT_EINVAL
    assert s(A16, 10, 0, A16, A16, None) == F.FLASHOPT_EINVAL
    assert s(A16, -1, 24, A16, A16, None) == F.FLASHOPT_EINVAL
    assert s(A16, 10, 24, A16, None, None) == F.FLASHOPT_EINVAL
    assert s(A16, 10, 32, A16 + 2, A16, None) == F.FLASHOPT_EALIGN
    assert r(A16, A16, 10, 25, A16, None) == F.FLASHOPT_EINVAL
    assert r(A16, MIS, 10, 24, A16, None) == F.FLASHOPT_EALIGN


def _tensor(numel=4096, **over):
    t = F.flashopt_tensor(A16, A16, A16, A16, A16, A16, A16, numel)
    for k, v in over.items():
        setattr(t, k, v)
    return t


def _step(L, tensors, args=None, ws=A16, ws_bytes=1 << 20):
    arr = (F.flashopt_tensor * max(1, len(tensors)))(*tensors)
    a = args or F.make_args(1)
    return L.flashopt_adamw_step(arr if tensors else None, len(tensors), ctypes.byref(a),
                                 ws, ws_bytes, None)


def test_step_validation(L):
    ok = [_tensor()]
    # hyper-parameters
    for bad in (dict(step=0), dict(master_bits=16), dict(companded=2), dict(fp32_states=2),
                dict(param_fp32=2), dict(param_fp32=1), dict(lr=-1.0),
                dict(beta1=1.0), dict(beta2=-0.1), dict(eps=-1e-8),
                dict(weight_decay=float("inf")), dict(lr=float("nan"))):
        a = F.make_args(1)
        for k, v in bad.items():
            setattr(a, k, v)
        assert _step(L, ok, a) == F.FLASHOPT_EINVAL, bad
    assert L.flashopt_adamw_step(None, 1, ctypes.byref(F.make_args(1)), A16, 1 << 20, None) == F.FLASHOPT_EINVAL
    assert L.flashopt_adamw_step(None, -1, ctypes.byref(F.make_args(1)), A16, 1 << 20, None) == F.FLASHOPT_EINVAL
    # tensors
    assert _step(L, [_tensor(numel=-1)]) == F.FLASHOPT_EINVAL
    for field in ("param", "grad", "rho", "m_codes", "m_scales", "v_codes", "v_scales"):
        assert _step(L, [_tensor(**{field: None})]) == F.FLASHOPT_EINVAL, field
        bad = MIS if field.endswith("scales") else A16 + 8
        assert _step(L, [_tensor(**{field: bad})]) == F.FLASHOPT_EALIGN, field
    # buffers a variant does not use may be NULL or unaligned: such calls get
    # past tensor validation and stop at the (too small) workspace, before
    # anything is enqueued
    none_args = F.make_args(1, master_bits=None)
    assert _step(L, [_tensor(rho=None)], none_args, ws_bytes=0) == F.FLASHOPT_EWORKSPACE
    assert _step(L, [_tensor(rho=MIS)], none_args, ws_bytes=0) == F.FLASHOPT_EWORKSPACE
    f32_args = F.make_args(1, quantize_states=False)
    assert _step(L, [_tensor(m_scales=None, v_scales=None)], f32_args, ws_bytes=0) == F.FLASHOPT_EWORKSPACE
    assert _step(L, [_tensor(m_scales=MIS)], f32_args, ws_bytes=0) == F.FLASHOPT_EWORKSPACE
    assert _step(L, [_tensor(rho=None)], f32_args, ws_bytes=0) == F.FLASHOPT_EINVAL
    assert _step(L, [_tensor(m_codes=A16 + 4)], f32_args, ws_bytes=0) == F.FLASHOPT_EALIGN
    # more than 2^31 - 1 chunks of 1024
    assert _step(L, [_tensor(numel=(1 << 41) + 1)]) == F.FLASHOPT_EINVAL
    # empty work is a no-op, even with no workspace
    assert _step(L, []) == F.FLASHOPT_OK
    assert _step(L, [_tensor(numel=0, param=None)], ws=None, ws_bytes=0) == F.FLASHOPT_OK
    # workspace
    need = F.flashopt_adamw_workspace_bytes(3)
    three = [_tensor(), _tensor(), _tensor()]
    assert need >= 3 * 64 + 4 * 4
    assert _step(L, three, ws=None) == F.FLASHOPT_EWORKSPACE
    assert _step(L, three, ws_bytes=need - 1) == F.FLASHOPT_EWORKSPACE
    assert _step(L, three, ws=A16 + 4, ws_bytes=need) == F.FLASHOPT_EALIGN
    assert F.flashopt_adamw_workspace_bytes(0) == 0


def test_noalloc_step_validation(L):
    """The allocation-free step validates like the list step, before any HIP
    call: more than 1024 tensors is EWORKSPACE (its fixed table's limit)."""
    def step(tensors, args=None, n=None):
        arr = (F.flashopt_tensor * max(1, len(tensors)))(*tensors)
        return L.flashopt_adamw_step_noalloc(arr if tensors else None,
                                             len(tensors) if n is None else n,
                                             ctypes.byref(args or F.make_args(1)), None)
    assert step([_tensor()] * 1025) == F.FLASHOPT_EWORKSPACE
    assert step([]) == F.FLASHOPT_OK
    assert step([_tensor(numel=0, param=None)]) == F.FLASHOPT_OK
    assert step([], n=-1) == F.FLASHOPT_EINVAL
    assert step([_tensor()], F.make_args(0)) == F.FLASHOPT_EINVAL
    assert step([_tensor(numel=-1)]) == F.FLASHOPT_EINVAL
    assert step([_tensor(grad=None)]) == F.FLASHOPT_EINVAL
    assert step([_tensor(v_codes=A16 + 8)]) == F.FLASHOPT_EALIGN
    assert step([_tensor(numel=(1 << 41) + 1)]) == F.FLASHOPT_EINVAL


def test_plan_validation(L):
    """The capture-safe plan calls validate like the list step, before any
    HIP call; the plan buffer has the workspace's size (a 128-byte scalar
    block, then the tables)."""
    info = F.flashopt_adamw_plan_info()
    args = F.make_args(1)

    def plan(tensors, a=None, buf=A16, nbytes=1 << 20, inf=info, n=None):
        arr = (F.flashopt_tensor * max(1, len(tensors)))(*tensors)
        return L.flashopt_adamw_plan(arr if tensors else None, len(tensors) if n is None else n,
                                     ctypes.byref(a or args), buf, nbytes,
                                     ctypes.byref(inf) if inf is not None else None, None)

    assert L.flashopt_adamw_plan_bytes(0) == 0
    for n in (1, 3, 290):
        assert L.flashopt_adamw_plan_bytes(n) == F.flashopt_adamw_workspace_bytes(n)
        assert L.flashopt_adamw_plan_bytes(n) >= 128 + n * 64 + (n + 1) * 4
    need = L.flashopt_adamw_plan_bytes(1)
    assert plan([_tensor()], inf=None) == F.FLASHOPT_EINVAL
    assert plan([], n=-1) == F.FLASHOPT_EINVAL
    assert plan([_tensor()], F.make_args(0)) == F.FLASHOPT_EINVAL
    assert plan([_tensor(numel=-1)]) == F.FLASHOPT_EINVAL
    assert plan([_tensor(grad=None)]) == F.FLASHOPT_EINVAL
    assert plan([_tensor()], buf=None) == F.FLASHOPT_EWORKSPACE
    assert plan([_tensor()], nbytes=need - 1) == F.FLASHOPT_EWORKSPACE
    assert plan([_tensor()], buf=A16 + 8, nbytes=need) == F.FLASHOPT_EALIGN
    assert plan([]) == F.FLASHOPT_OK                      # nothing to stage
    assert (info.n_tensors, info.total_chunks) == (0, 0)
    assert L.flashopt_adamw_plan_launch(ctypes.byref(info), None, None) == F.FLASHOPT_OK

    # set_step: the variant must be the plan's
    good = F.flashopt_adamw_plan_info(1, 4, 24, 1, 0, 0)
    for bad in (dict(master_bits=32), dict(companded=0), dict(fp32_states=1),
                dict(master_bits=0, param_fp32=1), dict(state_layout=1)):
        a = F.make_args(5)
        for k, v in bad.items():
            setattr(a, k, v)
        assert L.flashopt_adamw_plan_set_step(ctypes.byref(good), ctypes.byref(a), A16,
                                              None) == F.FLASHOPT_EINVAL, bad
    assert L.flashopt_adamw_plan_set_step(None, ctypes.byref(F.make_args(5)), A16, None) == F.FLASHOPT_EINVAL
    assert L.flashopt_adamw_plan_set_step(ctypes.byref(good), ctypes.byref(F.make_args(0)), A16,
                                          None) == F.FLASHOPT_EINVAL
    assert L.flashopt_adamw_plan_set_step(ctypes.byref(good), ctypes.byref(F.make_args(5)), None,
                                          None) == F.FLASHOPT_EWORKSPACE
    assert L.flashopt_adamw_plan_set_step(ctypes.byref(good), ctypes.byref(F.make_args(5)), A16 + 8,
                                          None) == F.FLASHOPT_EALIGN

    # launch: the info's fields are checked, the buffer must be there
    def launch(fields, buf=A16):
        return L.flashopt_adamw_plan_launch(ctypes.byref(F.flashopt_adamw_plan_info(*fields)), buf, None)
    for bad in ((1, 4, 16, 1, 0, 0), (1, 4, 24, 2, 0, 0), (1, 4, 24, 1, 2, 0), (1, 4, 24, 1, 0, 1),
                (1, 4, 24, 1, 0, 0, 2), (1, 4, 24, 1, 1, 0, 1),
                (-1, 4, 24, 1, 0, 0), (1, -4, 24, 1, 0, 0), (0, 4, 24, 1, 0, 0)):
        assert launch(bad) == F.FLASHOPT_EINVAL, bad
    assert launch((1, 4, 24, 1, 0, 0), buf=None) == F.FLASHOPT_EWORKSPACE
    assert launch((1, 4, 24, 1, 0, 0), buf=A16 + 8) == F.FLASHOPT_EALIGN
    assert launch((1, 0, 24, 1, 0, 0)) == F.FLASHOPT_OK    # an empty list launches nothing
    assert L.flashopt_adamw_plan_launch(None, A16, None) == F.FLASHOPT_EINVAL


def test_sgd_plan_validation(L):
    """The FlashSGD plan calls validate like flashopt_sgd_step, before any
    HIP call."""
    info = F.flashopt_sgd_plan_info()

    def plan(tensors, a=None, buf=A16, nbytes=1 << 20, inf=info):
        arr = (F.flashopt_tensor * max(1, len(tensors)))(*tensors)
        return L.flashopt_sgd_plan(arr if tensors else None, len(tensors),
                                   ctypes.byref(a or F.make_sgd_args(1)), buf, nbytes,
                                   ctypes.byref(inf) if inf is not None else None, None)

    assert L.flashopt_sgd_plan_bytes(0) == 0
    assert L.flashopt_sgd_plan_bytes(5) == F.flashopt_sgd_workspace_bytes(5)
    sgd_tensor = lambda **kw: _tensor(v_codes=None, v_scales=None, **kw)
    assert plan([sgd_tensor()], inf=None) == F.FLASHOPT_EINVAL
    assert plan([sgd_tensor()], F.make_sgd_args(1, momentum=0.0)) == F.FLASHOPT_EINVAL
    assert plan([sgd_tensor()], F.make_sgd_args(1, nesterov=True, dampening=0.1)) == F.FLASHOPT_EINVAL
    assert plan([sgd_tensor(m_codes=None)]) == F.FLASHOPT_EINVAL
    assert plan([sgd_tensor()], buf=None) == F.FLASHOPT_EWORKSPACE
    assert plan([sgd_tensor()], nbytes=L.flashopt_sgd_plan_bytes(1) - 1) == F.FLASHOPT_EWORKSPACE
    assert plan([sgd_tensor()], buf=A16 + 8) == F.FLASHOPT_EALIGN
    assert plan([]) == F.FLASHOPT_OK and (info.n_tensors, info.total_chunks) == (0, 0)

    good = F.flashopt_sgd_plan_info(1, 4, 24, 1, 0, 0)
    set_step = lambda inf, a, buf=A16: L.flashopt_sgd_plan_set_step(
        ctypes.byref(inf) if inf is not None else None, ctypes.byref(a), buf, None)
    assert set_step(good, F.make_sgd_args(3, master_bits=32)) == F.FLASHOPT_EINVAL
    assert set_step(good, F.make_sgd_args(3, companded=False)) == F.FLASHOPT_EINVAL
    assert set_step(good, F.make_sgd_args(3, quantize_states=False)) == F.FLASHOPT_EINVAL
    assert set_step(F.flashopt_sgd_plan_info(1, 4, 24, 1, 0, 1), F.make_sgd_args(3)) == F.FLASHOPT_EINVAL
    assert set_step(good, F.make_sgd_args(3, state_layout="blocked")) == F.FLASHOPT_EINVAL
    assert set_step(None, F.make_sgd_args(3)) == F.FLASHOPT_EINVAL
    assert set_step(good, F.make_sgd_args(0)) == F.FLASHOPT_EINVAL
    assert set_step(good, F.make_sgd_args(3), buf=None) == F.FLASHOPT_EWORKSPACE
    assert set_step(good, F.make_sgd_args(3), buf=A16 + 8) == F.FLASHOPT_EALIGN

    def launch(fields, buf=A16):
        return L.flashopt_sgd_plan_launch(ctypes.byref(F.flashopt_sgd_plan_info(*fields)), buf, None)
    for bad in ((1, 4, 16, 1, 0, 0), (1, 4, 24, 2, 0, 0), (1, 4, 24, 1, 2, 0), (1, 4, 24, 1, 0, 2),
                (1, 4, 24, 1, 1, 1), (1, 4, 1, 1, 0, 0), (-1, 4, 24, 1, 0, 0), (1, -4, 24, 1, 0, 0),
                (0, 4, 24, 1, 0, 0)):
        assert launch(bad) == F.FLASHOPT_EINVAL, bad
    assert launch((1, 4, 24, 1, 0, 0), buf=None) == F.FLASHOPT_EWORKSPACE
    assert launch((1, 4, 24, 1, 0, 0), buf=A16 + 8) == F.FLASHOPT_EALIGN
    assert launch((1, 0, 24, 1, 0, 0)) == F.FLASHOPT_OK
    assert L.flashopt_sgd_plan_launch(None, A16, None) == F.FLASHOPT_EINVAL


def test_binding_refuses_host_tensors(L):
    import torch
    with pytest.raises(ValueError):
        F.flashopt_quantize(torch.zeros(64), F.SPEC_MOMENTUM)
    for make in (F.FlashAdamW, F.FlashSGD):            # host parameters: refused at construction
        with pytest.raises(ValueError):
            make([torch.zeros(64, dtype=torch.bfloat16)])


def test_sgd_step_validation(L):
    def sgd(tensors, args, ws=A16, ws_bytes=1 << 20):
        arr = (F.flashopt_tensor * max(1, len(tensors)))(*tensors)
        return L.flashopt_sgd_step(arr, len(tensors), ctypes.byref(args), ws, ws_bytes, None)

    ok = [_tensor()]
    for bad in (dict(step=0), dict(momentum=0.0), dict(momentum=float("nan")), dict(lr=-1.0),
                dict(dampening=float("inf")), dict(weight_decay=float("nan")),
                dict(master_bits=16), dict(companded=2), dict(fp32_states=2), dict(nesterov=2)):
        a = F.make_sgd_args(1)
        for k, v in bad.items():
            setattr(a, k, v)
        assert sgd(ok, a) == F.FLASHOPT_EINVAL, bad
    a = F.make_sgd_args(1, nesterov=True, dampening=0.1)
    assert sgd(ok, a) == F.FLASHOPT_EINVAL                       # nesterov needs dampening 0
    # the variance streams are unused: NULL passes validation and the call
    # stops at the (too small) workspace, before anything is enqueued
    assert sgd([_tensor(v_codes=None, v_scales=None)], F.make_sgd_args(1), ws_bytes=0) == F.FLASHOPT_EWORKSPACE
    assert sgd([_tensor(m_scales=None)], F.make_sgd_args(1), ws_bytes=0) == F.FLASHOPT_EINVAL
    assert sgd([_tensor(m_scales=None)], F.make_sgd_args(1, quantize_states=False),
               ws_bytes=0) == F.FLASHOPT_EWORKSPACE
    assert sgd([_tensor(m_codes=A16 + 8)], F.make_sgd_args(1), ws_bytes=0) == F.FLASHOPT_EALIGN
    assert F.flashopt_sgd_workspace_bytes(3) == F.flashopt_adamw_workspace_bytes(3)   # both stage a scalar block


def test_single_tensor_validation(L):
    """The workspace-free single-tensor entry points validate like the list
    forms; an empty tensor is a no-op.  (No call here reaches a launch.)"""
    st = L.flashopt_adamw_step_tensor
    sg = L.flashopt_sgd_step_tensor
    a, s = F.make_args(1), F.make_sgd_args(1)
    assert st(None, ctypes.byref(a), None) == F.FLASHOPT_EINVAL
    assert st(ctypes.byref(_tensor()), None, None) == F.FLASHOPT_EINVAL
    assert st(ctypes.byref(_tensor(numel=0, param=None)), ctypes.byref(a), None) == F.FLASHOPT_OK
    assert st(ctypes.byref(_tensor(numel=-1)), ctypes.byref(a), None) == F.FLASHOPT_EINVAL
    assert st(ctypes.byref(_tensor(grad=None)), ctypes.byref(a), None) == F.FLASHOPT_EINVAL
    assert st(ctypes.byref(_tensor(rho=A16 + 8)), ctypes.byref(a), None) == F.FLASHOPT_EALIGN
    assert st(ctypes.byref(_tensor(numel=(1 << 41) + 1)), ctypes.byref(a), None) == F.FLASHOPT_EINVAL
    bad = F.make_args(0)
    assert st(ctypes.byref(_tensor()), ctypes.byref(bad), None) == F.FLASHOPT_EINVAL
    assert sg(None, ctypes.byref(s), None) == F.FLASHOPT_EINVAL
    assert sg(ctypes.byref(_tensor(numel=0, param=None)), ctypes.byref(s), None) == F.FLASHOPT_OK
    assert sg(ctypes.byref(_tensor(m_codes=A16 + 8)), ctypes.byref(s), None) == F.FLASHOPT_EALIGN
    bad_s = F.make_sgd_args(1, momentum=0.0)
    assert sg(ctypes.byref(_tensor()), ctypes.byref(bad_s), None) == F.FLASHOPT_EINVAL


def test_blocked_state_validation(L):
    """The chunk-blocked state layout: one 16-byte aligned buffer at rho, the
    other state pointers NULL, quantized states only, and the buffer size of
    flashopt_blocked_state_bytes; a bad layout code is EINVAL."""
    blocked = F.make_args(1, state_layout="blocked")
    blk = lambda **kw: _tensor(**dict(dict(m_codes=None, m_scales=None, v_codes=None, v_scales=None), **kw))
    # valid: validation passes and stops at the missing workspace
    assert _step(L, [blk()], blocked, ws_bytes=0) == F.FLASHOPT_EWORKSPACE
    assert _step(L, [blk()], F.make_args(1, master_bits=None, state_layout="blocked"),
                 ws_bytes=0) == F.FLASHOPT_EWORKSPACE
    # a stream pointer next to the block, a missing or misaligned block
    for field in ("m_codes", "m_scales", "v_codes", "v_scales"):
        assert _step(L, [blk(**{field: A16})], blocked) == F.FLASHOPT_EINVAL, field
    assert _step(L, [blk(rho=None)], blocked) == F.FLASHOPT_EINVAL
    assert _step(L, [blk(rho=A16 + 8)], blocked) == F.FLASHOPT_EALIGN
    # the blocked layout holds quantized states only; layout codes are 0 | 1
    a = F.make_args(1, quantize_states=False)
    a.state_layout = 1
    assert _step(L, [blk()], a) == F.FLASHOPT_EINVAL
    a = F.make_args(1)
    a.state_layout = 2
    assert _step(L, [_tensor()], a) == F.FLASHOPT_EINVAL
    s = F.make_sgd_args(1)
    s.state_layout = 2
    arr = (F.flashopt_tensor * 1)(_tensor())
    assert L.flashopt_sgd_step(arr, 1, ctypes.byref(s), A16, 1 << 20, None) == F.FLASHOPT_EINVAL
    one = (F.flashopt_tensor * 1)(blk(rho=None))
    assert L.flashopt_adamw_step_tensor(one, ctypes.byref(blocked), None) == F.FLASHOPT_EINVAL
    # sizes: per 1024-element chunk, rho (1024 | 2048 | 0) + codes and scales
    assert F.flashopt_blocked_state_bytes(1, 24) == 1024 + 2 * (1024 + 64)
    assert F.flashopt_blocked_state_bytes(1025, 24) == 2 * 3200
    assert F.flashopt_blocked_state_bytes(2048, 32) == 2 * (2048 + 2176)
    assert F.flashopt_blocked_state_bytes(3000, None) == 3 * 2176
    assert F.flashopt_blocked_state_bytes(1024, 24, variance=False) == 2176      # 2112 in 128-byte lines
    assert F.flashopt_blocked_state_bytes(1024, 32, variance=False) == 3200      # 3136 likewise
    assert F.flashopt_blocked_state_bytes(1024, None, variance=False) == 1152    # 1088 likewise
    assert F.flashopt_blocked_state_bytes(0, 24) == 0
    assert L.flashopt_blocked_state_bytes(10, 16, 1) == 0
