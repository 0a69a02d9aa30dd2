"""Helpers for the GPU parity tests: device checks and bit-level host copies."""
import numpy as np
import pytest
import torch

from bit_companded_adam_amd import flashopt as F


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    F.lib()      # raises if the HIP library is missing: no fallback


def u16(t: torch.Tensor) -> np.ndarray:
    """Host copy of a 16-bit tensor as uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    """Host copy keeping the dtype (int8 / uint8 / int16 / float32)."""
    return t.detach().contiguous().cpu().numpy()


def dev_u16(a: np.ndarray, device="cuda", dtype=torch.bfloat16) -> torch.Tensor:
    """uint16 bit patterns -> device tensor of a 16-bit dtype."""
    return torch.from_numpy(a.view(np.int16).copy()).to(device).view(dtype)


def code_agreement(a: np.ndarray, b: np.ndarray):
    """(fraction equal, max |difference|) of two code arrays."""
    d = np.abs(a.astype(np.int32) - b.astype(np.int32))
    return float((d == 0).mean()) if d.size else 1.0, int(d.max()) if d.size else 0
