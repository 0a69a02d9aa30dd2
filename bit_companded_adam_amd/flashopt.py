"""Thin ctypes binding of libflashopt.so with the C entry points' names
(FlashAdamW and FlashSGD steps, the codec and the weight split).

Argument marshalling only: every computation runs in the HIP kernels of the
library.  Tensors are torch CUDA (HIP) tensors; outputs are allocated with
torch when not given.  Work goes to the current torch stream unless a
stream is passed.  A missing library raises at first use -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

# FLASHOPT_LIB may point at another build of the same library (experiments).
_LIB_PATH = os.environ.get("FLASHOPT_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libflashopt.so")

FLASHOPT_OK, FLASHOPT_EINVAL, FLASHOPT_EALIGN, FLASHOPT_EWORKSPACE, FLASHOPT_EHIP = range(5)
Q_SIGNED, Q_SQRT, Q_SOFTSIGN = 1, 2, 4
SPEC_MOMENTUM = Q_SIGNED | Q_SOFTSIGN
SPEC_VARIANCE = Q_SQRT
SPEC_MOMENTUM_LINEAR = Q_SIGNED
SPEC_VARIANCE_LINEAR = 0
GROUP = 32
CHUNK_ELEMS = 1024
STATE_STREAMS, STATE_BLOCKED = 0, 1
STATE_LAYOUTS = {"streams": STATE_STREAMS, "blocked": STATE_BLOCKED}

EXPORTS = ("flashopt_quantize", "flashopt_dequantize", "flashopt_split",
           "flashopt_reconstruct", "flashopt_adamw_workspace_bytes",
           "flashopt_adamw_step", "flashopt_adamw_step_tensor", "flashopt_sgd_workspace_bytes",
           "flashopt_sgd_step", "flashopt_sgd_step_tensor", "flashopt_status_str",
           "flashopt_abi_version", "flashopt_adamw_step_noalloc", "flashopt_adamw_plan_bytes",
           "flashopt_adamw_plan", "flashopt_adamw_plan_set_step", "flashopt_adamw_plan_launch",
           "flashopt_sgd_plan_bytes", "flashopt_sgd_plan", "flashopt_sgd_plan_set_step",
           "flashopt_sgd_plan_launch", "flashopt_blocked_state_bytes")


class FlashoptError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)}")
        self.status = status


class flashopt_tensor(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("rho", ctypes.c_void_p), ("m_codes", ctypes.c_void_p),
                ("m_scales", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("v_scales", ctypes.c_void_p), ("numel", ctypes.c_int64)]


class flashopt_adamw_args(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("step", ctypes.c_int64),
                ("master_bits", ctypes.c_int), ("companded", ctypes.c_int),
                ("fp32_states", ctypes.c_int), ("param_fp32", ctypes.c_int),
                ("state_layout", ctypes.c_int)]


class flashopt_adamw_plan_info(ctypes.Structure):
    _fields_ = [("n_tensors", ctypes.c_int32), ("total_chunks", ctypes.c_int32),
                ("master_bits", ctypes.c_int32), ("companded", ctypes.c_int32),
                ("fp32_states", ctypes.c_int32), ("param_fp32", ctypes.c_int32),
                ("state_layout", ctypes.c_int32)]


class flashopt_sgd_args(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("momentum", ctypes.c_double),
                ("dampening", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("step", ctypes.c_int64), ("master_bits", ctypes.c_int),
                ("companded", ctypes.c_int), ("fp32_states", ctypes.c_int),
                ("nesterov", ctypes.c_int), ("state_layout", ctypes.c_int)]


class flashopt_sgd_plan_info(ctypes.Structure):
    _fields_ = [("n_tensors", ctypes.c_int32), ("total_chunks", ctypes.c_int32),
                ("master_bits", ctypes.c_int32), ("companded", ctypes.c_int32),
                ("fp32_states", ctypes.c_int32), ("state_layout", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, u, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint, ctypes.c_int
        L.flashopt_quantize.argtypes = [vp, i64, u, vp, vp, vp]
        L.flashopt_dequantize.argtypes = [vp, vp, i64, u, vp, vp]
        L.flashopt_split.argtypes = [vp, i64, i, vp, vp, vp]
        L.flashopt_reconstruct.argtypes = [vp, vp, i64, i, vp, vp]
        L.flashopt_adamw_workspace_bytes.argtypes = [ctypes.POINTER(flashopt_tensor), i]
        L.flashopt_adamw_workspace_bytes.restype = ctypes.c_size_t
        L.flashopt_adamw_step.argtypes = [ctypes.POINTER(flashopt_tensor), i,
                                          ctypes.POINTER(flashopt_adamw_args), vp,
                                          ctypes.c_size_t, vp]
        L.flashopt_sgd_workspace_bytes.argtypes = [ctypes.POINTER(flashopt_tensor), i]
        L.flashopt_sgd_workspace_bytes.restype = ctypes.c_size_t
        L.flashopt_sgd_step.argtypes = [ctypes.POINTER(flashopt_tensor), i,
                                        ctypes.POINTER(flashopt_sgd_args), vp,
                                        ctypes.c_size_t, vp]
        L.flashopt_adamw_step_tensor.argtypes = [ctypes.POINTER(flashopt_tensor),
                                                 ctypes.POINTER(flashopt_adamw_args), vp]
        L.flashopt_adamw_step_noalloc.argtypes = [ctypes.POINTER(flashopt_tensor), i,
                                                  ctypes.POINTER(flashopt_adamw_args), vp]
        L.flashopt_sgd_step_tensor.argtypes = [ctypes.POINTER(flashopt_tensor),
                                               ctypes.POINTER(flashopt_sgd_args), vp]
        L.flashopt_adamw_plan_bytes.argtypes = [i]
        L.flashopt_adamw_plan_bytes.restype = ctypes.c_size_t
        L.flashopt_adamw_plan.argtypes = [ctypes.POINTER(flashopt_tensor), i,
                                          ctypes.POINTER(flashopt_adamw_args), vp, ctypes.c_size_t,
                                          ctypes.POINTER(flashopt_adamw_plan_info), vp]
        L.flashopt_adamw_plan_set_step.argtypes = [ctypes.POINTER(flashopt_adamw_plan_info),
                                                   ctypes.POINTER(flashopt_adamw_args), vp, vp]
        L.flashopt_adamw_plan_launch.argtypes = [ctypes.POINTER(flashopt_adamw_plan_info), vp, vp]
        L.flashopt_sgd_plan_bytes.argtypes = [i]
        L.flashopt_sgd_plan_bytes.restype = ctypes.c_size_t
        L.flashopt_sgd_plan.argtypes = [ctypes.POINTER(flashopt_tensor), i,
                                        ctypes.POINTER(flashopt_sgd_args), vp, ctypes.c_size_t,
                                        ctypes.POINTER(flashopt_sgd_plan_info), vp]
        L.flashopt_sgd_plan_set_step.argtypes = [ctypes.POINTER(flashopt_sgd_plan_info),
                                                 ctypes.POINTER(flashopt_sgd_args), vp, vp]
        L.flashopt_sgd_plan_launch.argtypes = [ctypes.POINTER(flashopt_sgd_plan_info), vp, vp]
        L.flashopt_blocked_state_bytes.argtypes = [i64, i, i]
        L.flashopt_blocked_state_bytes.restype = ctypes.c_size_t
        L.flashopt_status_str.argtypes = [i]
        L.flashopt_status_str.restype = ctypes.c_char_p
        L.flashopt_abi_version.argtypes = []
        for name in ("flashopt_quantize", "flashopt_dequantize", "flashopt_split",
                     "flashopt_reconstruct", "flashopt_adamw_step", "flashopt_sgd_step",
                     "flashopt_adamw_step_tensor", "flashopt_sgd_step_tensor",
                     "flashopt_adamw_step_noalloc", "flashopt_adamw_plan",
                     "flashopt_adamw_plan_set_step", "flashopt_adamw_plan_launch",
                     "flashopt_sgd_plan", "flashopt_sgd_plan_set_step", "flashopt_sgd_plan_launch"):
            getattr(L, name).restype = i
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().flashopt_status_str(status).decode()


def _check(status: int, where: str):
    if status != FLASHOPT_OK:
        raise FlashoptError(status, where)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def n_groups(n: int) -> int:
    return (n + GROUP - 1) // GROUP


def _buf(t: torch.Tensor, name: str, device, elem_sizes, numel: int, float32: bool = False):
    """A caller-supplied buffer's address, after the checks the C ABI cannot
    make on plain pointers: same device as the input, element width, enough
    elements (a short buffer would be written past its end on the GPU)."""
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the input on {device}")
    if float32 and t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32")
    if t.element_size() not in elem_sizes:
        raise ValueError(f"{name} must have {'/'.join(map(str, elem_sizes))}-byte elements")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, {numel} needed")
    return _dev(t, name)


def flashopt_abi_version() -> int:
    return lib().flashopt_abi_version()


# --------------------------------------------------------------- codec

def flashopt_quantize(x: torch.Tensor, spec: int, codes=None, scales=None, stream=None):
    """Group-32 quantize x (fp32); returns (codes int8|uint8, scales fp16 as int16 bits)."""
    n = x.numel()
    if x.dtype != torch.float32:
        raise ValueError("x must be float32")
    px = _dev(x, "x")
    if codes is None:
        codes = torch.empty(n, dtype=torch.int8 if spec & Q_SIGNED else torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(n_groups(n), dtype=torch.int16, device=x.device)
    pc = _buf(codes, "codes", x.device, (1,), n)
    ps = _buf(scales, "scales", x.device, (2,), n_groups(n))
    with torch.cuda.device(x.device):
        _check(lib().flashopt_quantize(px, n, spec, pc, ps, _stream(stream)), "flashopt_quantize")
    return codes, scales


def flashopt_dequantize(codes: torch.Tensor, scales: torch.Tensor, spec: int, out=None, stream=None):
    """Group-32 dequantize codes with their fp16 scales (int16 bits) into fp32."""
    n = codes.numel()
    if codes.element_size() != 1:
        raise ValueError("codes must be int8 or uint8")
    pc = _dev(codes, "codes")
    ps = _buf(scales, "scales", codes.device, (2,), n_groups(n))
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=codes.device)
    po = _buf(out, "out", codes.device, (4,), n, float32=True)
    with torch.cuda.device(codes.device):
        _check(lib().flashopt_dequantize(pc, ps, n, spec, po, _stream(stream)), "flashopt_dequantize")
    return out


# --------------------------------------------------------------- split

def rho_dtype(master_bits: int):
    if master_bits not in (24, 32):
        raise ValueError("master_bits must be 24 or 32")
    return {24: torch.int8, 32: torch.int16}[master_bits]


def flashopt_split(master: torch.Tensor, master_bits: int, param=None, rho=None, stream=None):
    """fp32 master -> (bf16 param, rho int8|int16)."""
    n = master.numel()
    if master.dtype != torch.float32:
        raise ValueError("master must be float32")
    pm = _dev(master, "master")
    rdt = rho_dtype(master_bits)
    if param is None:
        param = torch.empty(n, dtype=torch.bfloat16, device=master.device)
    if rho is None:
        rho = torch.empty(n, dtype=rdt, device=master.device)
    pp = _buf(param, "param", master.device, (2,), n)
    pr = _buf(rho, "rho", master.device, (rdt.itemsize,), n)
    with torch.cuda.device(master.device):
        _check(lib().flashopt_split(pm, n, master_bits, pp, pr, _stream(stream)), "flashopt_split")
    return param, rho


def flashopt_reconstruct(param: torch.Tensor, rho: torch.Tensor, master_bits: int, out=None,
                         stream=None):
    """(bf16 param, rho int8|int16) -> fp32 master."""
    n = param.numel()
    if param.element_size() != 2:
        raise ValueError("param must hold bf16 values")
    rdt = rho_dtype(master_bits)
    pp = _dev(param, "param")
    pr = _buf(rho, "rho", param.device, (rdt.itemsize,), n)
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=param.device)
    po = _buf(out, "out", param.device, (4,), n, float32=True)
    with torch.cuda.device(param.device):
        _check(lib().flashopt_reconstruct(pp, pr, n, master_bits, po, _stream(stream)),
               "flashopt_reconstruct")
    return out


# --------------------------------------------------------------- step

def flashopt_blocked_state_bytes(numel: int, master_bits, variance: bool = True) -> int:
    """Bytes of a chunk-blocked state buffer (FLASHOPT_STATE_BLOCKED) for
    numel elements; master_bits 24 | 32 | None."""
    return lib().flashopt_blocked_state_bytes(numel, 0 if master_bits is None else master_bits,
                                              int(variance))


class TensorState:
    """Device state of one parameter tensor: bf16 or fp32 param (updated in
    place; fp32 only without a split), rho (master_bits 24 | 32; none for
    master_bits None), and the momentum
    and variance as codes with fp16 scales, or as fp32 arrays when
    quantize_states is False.  Fresh state is zero.

    state_layout "streams" keeps rho, the codes and the scales as five
    tensors (the page's per-parameter state); "blocked" keeps the same
    values chunk by chunk in one uint8 buffer (`block`; quantized states
    only), which the step streams faster.  The attributes rho, m_codes,
    m_scales, v_codes and v_scales then return copies in the streams
    format (for reading)."""

    def __init__(self, param: torch.Tensor, master_bits=24, quantize_states: bool = True,
                 variance: bool = True, state_layout: str = "streams"):
        if param.dtype not in (torch.bfloat16, torch.float32) or not param.is_contiguous() \
                or not param.is_cuda:
            raise ValueError("param must be a contiguous bf16 or fp32 device tensor")
        if master_bits not in (24, 32, None):
            raise ValueError("master_bits must be 24, 32 or None")
        if param.dtype == torch.float32 and master_bits is not None:
            raise ValueError("an fp32 parameter is never split: use master_bits=None")
        if state_layout not in STATE_LAYOUTS:
            raise ValueError("state_layout must be 'streams' or 'blocked'")
        if state_layout == "blocked" and not quantize_states:
            raise ValueError("the blocked state layout holds quantized states only")
        n, dev = param.numel(), param.device
        self.param = param
        self.master_bits = master_bits
        self.quantize_states = quantize_states
        self.variance = variance
        self.state_layout = state_layout
        self.block = None
        if state_layout == "blocked":
            self.block = torch.zeros(max(16, flashopt_blocked_state_bytes(n, master_bits, variance)),
                                     dtype=torch.uint8, device=dev)
            return
        self._rho = None if master_bits is None else torch.zeros(n, dtype=rho_dtype(master_bits), device=dev)
        if quantize_states:
            self._m_codes = torch.zeros(n, dtype=torch.int8, device=dev)
            self._m_scales = torch.zeros(n_groups(n), dtype=torch.int16, device=dev)
            self._v_codes = torch.zeros(n, dtype=torch.uint8, device=dev) if variance else None
            self._v_scales = torch.zeros(n_groups(n), dtype=torch.int16, device=dev) if variance else None
        else:
            self._m_codes = torch.zeros(n, dtype=torch.float32, device=dev)
            self._v_codes = torch.zeros(n, dtype=torch.float32, device=dev) if variance else None
            self._m_scales = self._v_scales = None

    # ---- the blocked layout's parts, as copies in the streams format
    def _block_part(self, offset: int, width: int, dtype, count: int) -> torch.Tensor:
        """Bytes [offset, offset + width) of every chunk's block, joined, as
        `count` elements of dtype."""
        n = self.param.numel()
        chunks = (n + CHUNK_ELEMS - 1) // CHUNK_ELEMS
        size = flashopt_blocked_state_bytes(n, self.master_bits, self.variance) // max(chunks, 1)
        if n == 0:
            return torch.zeros(0, dtype=dtype, device=self.param.device)
        rows = self.block[:chunks * size].view(chunks, size)[:, offset:offset + width]
        return rows.contiguous().view(-1).view(dtype)[:count]

    def _offsets(self):
        r = {24: 1024, 32: 2048, None: 0}[self.master_bits]
        if self.variance:
            return r, r, r + 1024, r + 2048, r + 2112
        return r, r, None, r + 1024, None

    @property
    def rho(self):
        if self.block is None:
            return self._rho
        if self.master_bits is None:
            return None
        r = self._offsets()[0]
        return self._block_part(0, r, rho_dtype(self.master_bits), self.param.numel())

    @property
    def m_codes(self):
        if self.block is None:
            return self._m_codes
        return self._block_part(self._offsets()[1], CHUNK_ELEMS, torch.int8, self.param.numel())

    @property
    def v_codes(self):
        if self.block is None:
            return self._v_codes
        off = self._offsets()[2]
        return None if off is None else self._block_part(off, CHUNK_ELEMS, torch.uint8,
                                                         self.param.numel())

    @property
    def m_scales(self):
        if self.block is None:
            return self._m_scales
        return self._block_part(self._offsets()[3], 64, torch.int16, n_groups(self.param.numel()))

    @property
    def v_scales(self):
        if self.block is None:
            return self._v_scales
        off = self._offsets()[4]
        return None if off is None else self._block_part(off, 64, torch.int16,
                                                         n_groups(self.param.numel()))

    def descriptor(self, grad: torch.Tensor) -> flashopt_tensor:
        if grad.dtype != self.param.dtype or grad.numel() != self.param.numel():
            raise ValueError(f"grad must be {self.param.dtype} with the parameter's size")
        if grad.device != self.param.device:
            raise ValueError(f"grad is on {grad.device}, its parameter on {self.param.device}")
        opt = lambda t, name: 0 if t is None else _dev(t, name)
        if self.block is not None:
            return flashopt_tensor(_dev(self.param, "param"), _dev(grad, "grad"),
                                   _dev(self.block, "block"), 0, 0, 0, 0, self.param.numel())
        return flashopt_tensor(_dev(self.param, "param"), _dev(grad, "grad"),
                               opt(self._rho, "rho"), _dev(self._m_codes, "m_codes"),
                               opt(self._m_scales, "m_scales"), opt(self._v_codes, "v_codes"),
                               opt(self._v_scales, "v_scales"), self.param.numel())


def make_args(step: int, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0,
              master_bits=24, companded=True, quantize_states=True,
              param_fp32=False, state_layout="streams") -> flashopt_adamw_args:
    """master_bits 24 | 32 | None (no split); quantize_states False: fp32 m, v;
    param_fp32: fp32 parameters and gradients (needs master_bits None);
    state_layout "streams" | "blocked"."""
    return flashopt_adamw_args(lr, betas[0], betas[1], eps, weight_decay, step,
                               0 if master_bits is None else master_bits, int(companded),
                               0 if quantize_states else 1, int(param_fp32),
                               STATE_LAYOUTS[state_layout])


def flashopt_adamw_workspace_bytes(n_tensors: int) -> int:
    return lib().flashopt_adamw_workspace_bytes(None, n_tensors)


def descriptor_array(states, grads):
    arr = (flashopt_tensor * len(states))()
    for i, (s, g) in enumerate(zip(states, grads)):
        arr[i] = s.descriptor(g)
    return arr


def flashopt_adamw_step(descriptors, args: flashopt_adamw_args, workspace: torch.Tensor,
                        stream=None):
    """One fused step over a ctypes array of flashopt_tensor descriptors."""
    n = len(descriptors)
    _check(lib().flashopt_adamw_step(descriptors, n, ctypes.byref(args), _dev(workspace, "workspace"),
                                     workspace.numel() * workspace.element_size(), _stream(stream)),
           "flashopt_adamw_step")


def flashopt_adamw_step_tensor(desc: flashopt_tensor, args: flashopt_adamw_args, stream=None):
    """One tensor's step, descriptor in the kernel arguments (no workspace)."""
    _check(lib().flashopt_adamw_step_tensor(ctypes.byref(desc), ctypes.byref(args), _stream(stream)),
           "flashopt_adamw_step_tensor")


def flashopt_adamw_plan_bytes(n_tensors: int) -> int:
    return lib().flashopt_adamw_plan_bytes(n_tensors)


def flashopt_adamw_plan(descriptors, args: flashopt_adamw_args, plan: torch.Tensor,
                        stream=None) -> flashopt_adamw_plan_info:
    """Stage the scalars of args and the tables of a descriptor array into
    the device buffer `plan`; returns the plan's host info."""
    info = flashopt_adamw_plan_info()
    _check(lib().flashopt_adamw_plan(descriptors, len(descriptors), ctypes.byref(args),
                                     _dev(plan, "plan"), plan.numel() * plan.element_size(),
                                     ctypes.byref(info), _stream(stream)),
           "flashopt_adamw_plan")
    return info


def flashopt_adamw_plan_set_step(info: flashopt_adamw_plan_info, args: flashopt_adamw_args,
                                 plan: torch.Tensor, stream=None):
    _check(lib().flashopt_adamw_plan_set_step(ctypes.byref(info), ctypes.byref(args),
                                              _dev(plan, "plan"), _stream(stream)),
           "flashopt_adamw_plan_set_step")


def flashopt_adamw_plan_launch(info: flashopt_adamw_plan_info, plan: torch.Tensor, stream=None):
    _check(lib().flashopt_adamw_plan_launch(ctypes.byref(info), _dev(plan, "plan"), _stream(stream)),
           "flashopt_adamw_plan_launch")


def flashopt_sgd_plan_bytes(n_tensors: int) -> int:
    return lib().flashopt_sgd_plan_bytes(n_tensors)


def flashopt_sgd_plan(descriptors, args, plan: torch.Tensor, stream=None) -> flashopt_sgd_plan_info:
    """flashopt_adamw_plan for the FlashSGD step."""
    info = flashopt_sgd_plan_info()
    _check(lib().flashopt_sgd_plan(descriptors, len(descriptors), ctypes.byref(args),
                                   _dev(plan, "plan"), plan.numel() * plan.element_size(),
                                   ctypes.byref(info), _stream(stream)),
           "flashopt_sgd_plan")
    return info


def flashopt_sgd_plan_set_step(info: flashopt_sgd_plan_info, args, plan: torch.Tensor, stream=None):
    _check(lib().flashopt_sgd_plan_set_step(ctypes.byref(info), ctypes.byref(args),
                                            _dev(plan, "plan"), _stream(stream)),
           "flashopt_sgd_plan_set_step")


def flashopt_sgd_plan_launch(info: flashopt_sgd_plan_info, plan: torch.Tensor, stream=None):
    _check(lib().flashopt_sgd_plan_launch(ctypes.byref(info), _dev(plan, "plan"), _stream(stream)),
           "flashopt_sgd_plan_launch")


class StepPlan:
    """The capture-safe list step of a FlashAdamW or FlashSGD over fixed
    gradient buffers (flashopt_adamw_plan / flashopt_sgd_plan): launch()
    enqueues the step kernel only, so it can be recorded into a CUDA/HIP
    graph, and set_step(t), called outside any capture before a launch or
    replay, writes the scalars of step t that it uses.  The plan keeps
    references to the gradient tensors (their addresses are in its table)
    and does not change the optimizer's step counts."""

    def __init__(self, opt, grads, step: int, stream=None):
        grads = list(grads)
        if len(grads) != len(opt.states):
            raise ValueError(f"{len(grads)} gradients for {len(opt.states)} parameters")
        self.opt = opt
        self.grads = grads
        self._bytes, self._plan, self._set, self._launch = opt._plan_calls
        desc = descriptor_array(opt.states, grads)
        with torch.cuda.device(opt.device):
            self.buffer = torch.empty(max(16, self._bytes(len(desc))), dtype=torch.uint8,
                                      device=opt.device or "cuda")
            self.info = self._plan(desc, opt._args(step), self.buffer, stream)
        self.t = step

    def set_step(self, t: int, stream=None):
        with torch.cuda.device(self.opt.device):
            self._set(self.info, self.opt._args(t), self.buffer, stream)
        self.t = t

    def launch(self, stream=None):
        with torch.cuda.device(self.opt.device):
            self._launch(self.info, self.buffer, stream)


class _Stepper:
    """Common driver of FlashAdamW / FlashSGD: a list step (one launch for all
    tensors) and a per-tensor step (one launch for one tensor, each tensor
    counting its own steps as the pages' per-parameter state does)."""

    def _init_common(self):
        devices = {s.param.device for s in self.states}
        if len(devices) > 1:
            raise ValueError(f"all parameters must be on one device, got {sorted(map(str, devices))}")
        self.device = devices.pop() if devices else None
        self.t = 0
        self.ts = [0] * len(self.states)
        self._key = None
        self._desc = None
        self._workspaces = {}

    def workspace(self, stream=None) -> torch.Tensor:
        """The device workspace of list launches on `stream` (the current
        stream if None): one per stream, so that a launch on one stream never
        rewrites the chunk table that a kernel still running on another
        stream reads (a launch only reuses its own stream's workspace, after
        that stream's earlier work)."""
        key = _stream(stream)
        ws = self._workspaces.get(key)
        if ws is None:
            ws = torch.empty(self._workspace_bytes, dtype=torch.uint8, device=self.device or "cuda")
            self._workspaces[key] = ws
        return ws

    def step(self, grads, stream=None):
        """One launch over every tensor; grads[i] is the bf16 gradient of
        tensor i.  The descriptor table is rebuilt (and the grads validated)
        whenever a grad's address, size, dtype, device or contiguity differs
        from the previous step's; no reference to the grads is kept."""
        grads = list(grads)
        if len(grads) != len(self.states):
            raise ValueError(f"{len(grads)} gradients for {len(self.states)} parameters")
        key = tuple((g.data_ptr(), g.numel(), g.dtype, g.device, g.is_contiguous()) for g in grads)
        if key != self._key:
            self._desc = descriptor_array(self.states, grads)
            self._key = key
        self._check_stream(stream)
        self.t += 1
        self.ts = [self.t] * len(self.states)
        with torch.cuda.device(self.device):    # the library launches on the current device
            self._list_step(self._desc, self.t, stream)

    def step_tensor(self, i: int, grad: torch.Tensor, stream=None):
        desc = self.states[i].descriptor(grad)
        self._check_stream(stream)
        self.ts[i] += 1
        with torch.cuda.device(self.device):
            self._tensor_step(desc, self.ts[i], stream)

    def step_tensors(self, indices, grads, stream=None):
        """Step a subset of the tensors (indices, each at most once) with one
        list launch per distinct step count: the same results as
        step_tensor() on each, in fewer launches."""
        indices, grads = list(indices), list(grads)
        if len(indices) != len(grads) or len(set(indices)) != len(indices):
            raise ValueError("indices must be distinct and match the gradients")
        descs = [self.states[i].descriptor(g) for i, g in zip(indices, grads)]
        self._check_stream(stream)
        by_t = {}
        for i, d in zip(indices, descs):
            self.ts[i] += 1
            by_t.setdefault(self.ts[i], []).append(d)
        with torch.cuda.device(self.device):
            for t, ds in by_t.items():
                arr = (flashopt_tensor * len(ds))(*ds)
                self._list_step(arr, t, stream)

    def plan(self, grads, step: int, stream=None) -> "StepPlan":
        """A capture-safe list step over these gradient buffers, with the
        scalars of `step` staged (StepPlan)."""
        return StepPlan(self, grads, step, stream)

    def _check_stream(self, stream):
        dev = getattr(stream, "device", None)
        if dev is not None and self.device is not None and dev != self.device:
            raise ValueError(f"stream is on {dev}, the parameters on {self.device}")


RELEASE_BATCH_BELOW = 65536
RELEASE_STREAMS = 4


def attach_grad_release(opt, params, batch_below: int = RELEASE_BATCH_BELOW,
                        streams: int = RELEASE_STREAMS):
    """Gradient release: register a post-accumulate-grad hook on every
    parameter that runs that tensor's step as soon as its gradient is
    complete and then frees the gradient, so a full set of gradients is never
    held.  params are the optimizer's parameters, in its order.  Every
    setting below gives the same bits as a list step; the defaults (norm
    vectors and biases batched, four side streams) make the per-tensor
    launches of a 1.2B-parameter decoder list take about 1.1 times the list
    step's time on MI355X, against about 1.37 times with batch_below=0 and
    streams=1.

    batch_below > 0: a parameter with fewer elements is not launched on its
    own; its (small) gradient is kept until the backward pass ends and all
    such parameters are stepped together in one list launch, which saves a
    kernel launch per small tensor (norm vectors, biases).

    streams > 1: the single-tensor launches go round-robin to that many side
    streams, each first waiting for the backward stream's work up to the
    hook, so that the launches of tensors too small to fill the GPU overlap
    instead of running one at a time (tensors are independent).  Each
    gradient's memory is kept until its side stream has used it
    (record_stream), and when the backward pass ends the backward stream
    waits for every side stream, so later work sees the updated parameters.
    Returns the hook handles."""
    index = {id(p): i for i, p in enumerate(params)}
    pending = []
    side = [torch.cuda.Stream(device=opt.device) for _ in range(streams)] if streams > 1 else []
    turn = [0]
    queued = [False]

    def end_of_backward():
        queued[0] = False
        if pending:
            idx, grads = zip(*pending)
            pending.clear()
            opt.step_tensors(idx, grads)
        if side:
            cur = torch.cuda.current_stream(opt.device)
            for s in side:
                cur.wait_stream(s)

    def hook(p):
        if not queued[0]:              # run once when this backward pass ends
            torch.autograd.Variable._execution_engine.queue_callback(end_of_backward)
            queued[0] = True
        i = index[id(p)]
        if p.numel() < batch_below:
            pending.append((i, p.grad))
        elif side:
            s = side[turn[0] % len(side)]
            turn[0] += 1
            s.wait_stream(torch.cuda.current_stream(opt.device))
            opt.step_tensor(i, p.grad, stream=s)
            p.grad.record_stream(s)
        else:
            opt.step_tensor(i, p.grad)
        p.grad = None

    return [p.register_post_accumulate_grad_hook(hook) for p in params]


def _layout(state_layout, quantize_states: bool, default: str) -> str:
    """An optimizer's state layout: its default for quantized states, the
    streams for fp32 states (the blocked layout holds quantized states
    only)."""
    if state_layout is None:
        return default if quantize_states else "streams"
    return state_layout


class FlashAdamW(_Stepper):
    """A list of TensorStates stepped together by one launch per step.  The
    parameters share one dtype: bf16 (split per master_bits, or cast back
    with master_bits None) or fp32 (master_bits None; fp32 gradients).
    state_layout: "blocked" (the default for quantized states: in
    in-process A/B runs on the 8.0B list 0.2-2.6% faster than the streams
    for the 24-bit master, 0.5-1.5% for the 32-bit one) or "streams" (see
    TensorState); the stored values are the same."""

    def __init__(self, params, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0,
                 master_bits=24, companded=True, quantize_states=True, state_layout=None):
        state_layout = _layout(state_layout, quantize_states, "blocked")
        self.states = [TensorState(p, master_bits, quantize_states, state_layout=state_layout)
                       for p in params]
        dtypes = {s.param.dtype for s in self.states}
        if len(dtypes) > 1:
            raise ValueError("all parameters of one FlashAdamW must share a dtype (bf16 or fp32)")
        self.hp = dict(lr=lr, betas=betas, eps=eps, weight_decay=weight_decay,
                       master_bits=master_bits, companded=companded,
                       quantize_states=quantize_states,
                       param_fp32=dtypes == {torch.float32}, state_layout=state_layout)
        self._init_common()
        self._workspace_bytes = max(16, flashopt_adamw_workspace_bytes(len(self.states)))

    def _list_step(self, desc, t, stream):
        flashopt_adamw_step(desc, make_args(t, **self.hp), self.workspace(stream), stream)

    def _args(self, t):
        return make_args(t, **self.hp)

    # (a tuple of plain functions: looked up on an instance, they stay unbound)
    _plan_calls = (flashopt_adamw_plan_bytes, flashopt_adamw_plan, flashopt_adamw_plan_set_step,
                   flashopt_adamw_plan_launch)

    def _tensor_step(self, desc, t, stream):
        flashopt_adamw_step_tensor(desc, make_args(t, **self.hp), stream)


# --------------------------------------------------------------- FlashSGD

def make_sgd_args(step: int, lr=1e-2, momentum=0.9, dampening=0.0, weight_decay=0.0,
                  nesterov=False, master_bits=24, companded=True,
                  quantize_states=True, state_layout="streams") -> flashopt_sgd_args:
    return flashopt_sgd_args(lr, momentum, dampening, weight_decay, step,
                             0 if master_bits is None else master_bits, int(companded),
                             0 if quantize_states else 1, int(nesterov),
                             STATE_LAYOUTS[state_layout])


def flashopt_sgd_workspace_bytes(n_tensors: int) -> int:
    return lib().flashopt_sgd_workspace_bytes(None, n_tensors)


def flashopt_sgd_step_tensor(desc: flashopt_tensor, args: flashopt_sgd_args, stream=None):
    """One tensor's FlashSGD step, descriptor in the kernel arguments."""
    _check(lib().flashopt_sgd_step_tensor(ctypes.byref(desc), ctypes.byref(args), _stream(stream)),
           "flashopt_sgd_step_tensor")


def flashopt_sgd_step(descriptors, args: flashopt_sgd_args, workspace: torch.Tensor,
                      stream=None):
    """One fused FlashSGD step over a ctypes array of flashopt_tensor descriptors."""
    n = len(descriptors)
    _check(lib().flashopt_sgd_step(descriptors, n, ctypes.byref(args), _dev(workspace, "workspace"),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "flashopt_sgd_step")


class FlashSGD(_Stepper):
    """A list of TensorStates (momentum buffer only) stepped together by one
    launch per step.  state_layout: "streams" (the default: with one state
    the blocked layout measured 0.6-1.1% slower) or "blocked"."""

    def __init__(self, params, lr=1e-2, momentum=0.9, dampening=0.0, weight_decay=0.0,
                 nesterov=False, master_bits=24, companded=True, quantize_states=True,
                 state_layout=None):
        state_layout = _layout(state_layout, quantize_states, "streams")
        self.states = [TensorState(p, master_bits, quantize_states, variance=False,
                                   state_layout=state_layout) for p in params]
        self.hp = dict(lr=lr, momentum=momentum, dampening=dampening, weight_decay=weight_decay,
                       nesterov=nesterov, master_bits=master_bits, companded=companded,
                       quantize_states=quantize_states, state_layout=state_layout)
        self._init_common()
        self._workspace_bytes = max(16, flashopt_sgd_workspace_bytes(len(self.states)))

    def _list_step(self, desc, t, stream):
        flashopt_sgd_step(desc, make_sgd_args(t, **self.hp), self.workspace(stream), stream)

    def _args(self, t):
        return make_sgd_args(t, **self.hp)

    _plan_calls = (flashopt_sgd_plan_bytes, flashopt_sgd_plan, flashopt_sgd_plan_set_step,
                   flashopt_sgd_plan_launch)

    def _tensor_step(self, desc, t, stream):
        flashopt_sgd_step_tensor(desc, make_sgd_args(t, **self.hp), stream)
