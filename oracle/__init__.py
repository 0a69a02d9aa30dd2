"""Oracle for the FlashAdamW and FlashSGD steps: ctypes wrapper around ``liboracle.so``.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
library (``bit_companded_adam_amd``) never imports it and shares no code with it.

The C source (``flashopt_oracle.c``) follows the method pages:
``code/flashsim/quantization.py`` (quantize/dequantize, Alg. 2-3),
``code/flashsim/flash_adamw_sim.py`` (FlashAdamWSim.step, Alg. 4) and
``code/gpu/equivalence.py`` (the bf16 cast fed to the correction bits).
FlashSGD appears on the pages only in bytes_per_param; its update is read as
torch.optim.SGD with momentum (R16 in the C source).
All arrays here are numpy arrays on the host.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "flashopt_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

SIGNED, SQRT, SOFTSIGN = 1, 2, 4
MOMENTUM = SIGNED | SOFTSIGN          # Alg. 2: signed int8, softsign companding
VARIANCE = SQRT                       # Alg. 3: unsigned uint8, sqrt companding
MOMENTUM_LINEAR = SIGNED              # linear ablation
VARIANCE_LINEAR = 0
GROUP = 32

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-Wall"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (CPU only)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Tensor(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("rho", ctypes.c_void_p), ("m_codes", ctypes.c_void_p),
                ("m_scales", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("v_scales", ctypes.c_void_p), ("numel", ctypes.c_int64)]


class HParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("step", ctypes.c_int64),
                ("master_bits", ctypes.c_int), ("companded", ctypes.c_int),
                ("quantize_states", ctypes.c_int), ("fp32_param", ctypes.c_int)]


def hparams(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0, step=1,
            master_bits=24, companded=True, quantize_states=True,
            fp32_param=False) -> HParams:
    """Step hyper-parameters.  fp32_param: the parameter and its gradient are
    float32 arrays and are never split (master_bits must then be None/0)."""
    return HParams(lr, betas[0], betas[1], eps, weight_decay, step,
                   0 if master_bits is None else master_bits, int(companded),
                   int(quantize_states), int(fp32_param))


class SgdHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("momentum", ctypes.c_double),
                ("dampening", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("step", ctypes.c_int64), ("master_bits", ctypes.c_int),
                ("companded", ctypes.c_int), ("quantize_states", ctypes.c_int),
                ("nesterov", ctypes.c_int)]


def sgd_hparams(lr=1e-2, momentum=0.9, dampening=0.0, weight_decay=0.0, step=1,
                master_bits=24, companded=True, quantize_states=True,
                nesterov=False) -> SgdHParams:
    return SgdHParams(lr, momentum, dampening, weight_decay, step,
                      0 if master_bits is None else master_bits, int(companded),
                      int(quantize_states), int(nesterov))


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i64, u = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint
        L.oracle_f16_from_f32.argtypes = [ctypes.c_float]
        L.oracle_f16_from_f32.restype = ctypes.c_uint16
        L.oracle_f32_from_f16.argtypes = [ctypes.c_uint16]
        L.oracle_f32_from_f16.restype = ctypes.c_float
        L.oracle_f16_array.argtypes = [vp, i64, vp]
        L.oracle_f16_array.restype = None
        L.oracle_split.argtypes = [vp, i64, ctypes.c_int, vp, vp]
        L.oracle_reconstruct.argtypes = [vp, vp, i64, ctypes.c_int, vp]
        L.oracle_quantize.argtypes = [vp, i64, u, vp, vp]
        L.oracle_dequantize.argtypes = [vp, vp, i64, u, vp]
        L.oracle_nmse.argtypes = [vp, vp, i64]
        L.oracle_nmse.restype = ctypes.c_double
        L.oracle_adamw_update.argtypes = [vp, vp, vp, vp, i64, ctypes.POINTER(HParams)]
        L.oracle_adamw_update.restype = None
        L.oracle_adamw_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64,
                                        ctypes.POINTER(HParams)]
        L.oracle_adamw_step_list.argtypes = [ctypes.POINTER(_Tensor), ctypes.c_int,
                                             ctypes.POINTER(HParams), ctypes.c_int]
        L.oracle_sgd_update.argtypes = [vp, vp, vp, i64, ctypes.POINTER(SgdHParams)]
        L.oracle_sgd_update.restype = None
        L.oracle_sgd_step.argtypes = [vp, vp, vp, vp, vp, i64, ctypes.POINTER(SgdHParams)]
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags.c_contiguous
    return a.ctypes.data


def _ck(rc):
    if rc < 0:
        raise ValueError("oracle call rejected its arguments")
    return rc


# ----------------------------------------------------------------- codec

def f16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> binary16 bits (round to nearest even, overflow to Inf)."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    out = np.zeros(x.size, dtype=np.uint16)
    lib().oracle_f16_array(_p(x), x.size, _p(out))
    return out


def quantize(x: np.ndarray, spec: int):
    """Group-32 quantize; returns (codes int8|uint8 [n], scales fp16 bits [ceil(n/32)])."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    n = x.size
    codes = np.zeros(n, dtype=np.int8 if spec & SIGNED else np.uint8)
    scales = np.zeros((n + GROUP - 1) // GROUP, dtype=np.uint16)
    _ck(lib().oracle_quantize(_p(x), n, spec, _p(codes), _p(scales)))
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, spec: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes).reshape(-1)
    scales = np.ascontiguousarray(scales, dtype=np.uint16).reshape(-1)
    assert codes.dtype == (np.int8 if spec & SIGNED else np.uint8)
    assert scales.size == (codes.size + GROUP - 1) // GROUP
    out = np.zeros(codes.size, dtype=np.float32)
    _ck(lib().oracle_dequantize(_p(codes), _p(scales), codes.size, spec, _p(out)))
    return out


def nmse(orig: np.ndarray, recon: np.ndarray) -> float:
    orig = np.ascontiguousarray(orig, dtype=np.float32).reshape(-1)
    recon = np.ascontiguousarray(recon, dtype=np.float32).reshape(-1)
    assert orig.size == recon.size
    return lib().oracle_nmse(_p(orig), _p(recon), orig.size)


# ----------------------------------------------------------------- split

def rho_dtype(master_bits: int):
    return {24: np.int8, 32: np.int16}[master_bits]


def split(x: np.ndarray, master_bits: int):
    """fp32 master -> (bf16 bits uint16 [n], rho int8|int16 [n])."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    hi = np.zeros(x.size, dtype=np.uint16)
    rho = np.zeros(x.size, dtype=rho_dtype(master_bits))
    _ck(lib().oracle_split(_p(x), x.size, master_bits, _p(hi), _p(rho)))
    return hi, rho


def reconstruct(hi: np.ndarray, rho: np.ndarray, master_bits: int) -> np.ndarray:
    hi = np.ascontiguousarray(hi, dtype=np.uint16).reshape(-1)
    rho = np.ascontiguousarray(rho, dtype=rho_dtype(master_bits)).reshape(-1)
    assert hi.size == rho.size
    out = np.zeros(hi.size, dtype=np.float32)
    _ck(lib().oracle_reconstruct(_p(hi), _p(rho), hi.size, master_bits, _p(out)))
    return out


# ----------------------------------------------------------------- AdamW

def adamw_update(theta, m, v, g, hp: HParams):
    """AdamW body on fp32 arrays; returns new (theta, m, v)."""
    theta = np.array(theta, dtype=np.float32, copy=True).reshape(-1)
    m = np.array(m, dtype=np.float32, copy=True).reshape(-1)
    v = np.array(v, dtype=np.float32, copy=True).reshape(-1)
    g = np.ascontiguousarray(g, dtype=np.float32).reshape(-1)
    lib().oracle_adamw_update(_p(theta), _p(m), _p(v), _p(g), theta.size, ctypes.byref(hp))
    return theta, m, v


class State:
    """Host copy of one tensor's FlashAdamW state (all numpy, C-contiguous)."""

    def __init__(self, param, rho, m_codes, m_scales, v_codes, v_scales):
        self.param, self.rho = param, rho
        self.m_codes, self.m_scales = m_codes, m_scales
        self.v_codes, self.v_scales = v_codes, v_scales

    @classmethod
    def zeros_like_param(cls, param_bits: np.ndarray, master_bits=24, quantize_states=True):
        """Fresh state for a parameter given as bf16 bits (uint16) or, for an
        fp32 parameter, as a float32 array (then master_bits must be None)."""
        if param_bits.dtype == np.float32:
            assert not master_bits
        n = param_bits.size
        g = (n + GROUP - 1) // GROUP
        rho = None if not master_bits else np.zeros(n, dtype=rho_dtype(master_bits))
        if quantize_states:
            return cls(param_bits.copy(), rho, np.zeros(n, np.int8), np.zeros(g, np.uint16),
                       np.zeros(n, np.uint8), np.zeros(g, np.uint16))
        return cls(param_bits.copy(), rho, np.zeros(n, np.float32), None,
                   np.zeros(n, np.float32), None)

    def copy(self) -> "State":
        c = lambda a: None if a is None else a.copy()
        return State(c(self.param), c(self.rho), c(self.m_codes), c(self.m_scales),
                     c(self.v_codes), c(self.v_scales))


def adamw_step(state: State, grad_bits: np.ndarray, hp: HParams) -> State:
    """One FlashAdamW step on a host state (in place); returns the state.  The
    gradient is bf16 bits (uint16), or float32 for an fp32 parameter."""
    fp32 = state.param.dtype == np.float32
    assert fp32 == bool(hp.fp32_param)
    grad_bits = np.ascontiguousarray(grad_bits, dtype=np.float32 if fp32 else np.uint16).reshape(-1)
    n = state.param.size
    assert grad_bits.size == n
    _ck(lib().oracle_adamw_step(_p(state.param), _p(grad_bits), _p(state.rho),
                                _p(state.m_codes), _p(state.m_scales),
                                _p(state.v_codes), _p(state.v_scales), n,
                                ctypes.byref(hp)))
    return state


def sgd_update(theta, buf, g, hp: SgdHParams):
    """SGD-with-momentum body on fp32 arrays; returns new (theta, buf)."""
    theta = np.array(theta, dtype=np.float32, copy=True).reshape(-1)
    buf = np.array(buf, dtype=np.float32, copy=True).reshape(-1)
    g = np.ascontiguousarray(g, dtype=np.float32).reshape(-1)
    lib().oracle_sgd_update(_p(theta), _p(buf), _p(g), theta.size, ctypes.byref(hp))
    return theta, buf


def sgd_step(state: State, grad_bits: np.ndarray, hp: SgdHParams) -> State:
    """One FlashSGD step on a host state (in place; the momentum buffer is
    state.m_codes / m_scales, v is unused); returns the state."""
    grad_bits = np.ascontiguousarray(grad_bits, dtype=np.uint16).reshape(-1)
    n = state.param.size
    assert grad_bits.size == n
    _ck(lib().oracle_sgd_step(_p(state.param), _p(grad_bits), _p(state.rho),
                              _p(state.m_codes), _p(state.m_scales), n, ctypes.byref(hp)))
    return state


def adamw_step_list(states, grads, hp: HParams, threads: int = 0) -> int:
    """Step a list of host states with the OpenMP slice driver; returns threads used."""
    arr = (_Tensor * len(states))()
    for i, (s, g) in enumerate(zip(states, grads)):
        assert g.dtype == s.param.dtype and g.flags.c_contiguous and g.size == s.param.size
        arr[i] = _Tensor(_p(s.param), _p(g), _p(s.rho), _p(s.m_codes), _p(s.m_scales),
                         _p(s.v_codes), _p(s.v_scales), s.param.size)
    return _ck(lib().oracle_adamw_step_list(arr, len(states), ctypes.byref(hp), threads))
