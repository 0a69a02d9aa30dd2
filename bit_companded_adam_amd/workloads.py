"""Seeded synthetic inputs for the FlashAdamW step, its codec and its split.

This module draws random numbers and lays out shapes; it holds none of the
method's arithmetic.  Both the HIP path's tests/benchmark and the oracle take
their inputs from here.

Workloads (all synthetic; the pages use no dataset):
  * ``battery()``      -- the seven codec test tensors of the page
    "code/gpu/equivalence.py" (battery(), CPU generator seed 7), drawn in the
    same order so the tensors are the page's own.
  * ``split_sweep()``  -- the stratified exponent sweep of the same page
    (eq_ecc(): fp32 exponent fields 1, 5, ..., 253, 2^16 uniform 23-bit
    mantissas each), with a random sign for both master widths.
  * ``decoder_1b_shapes()`` / ``decoder_8b_shapes()`` -- decoder-shaped tensor
    lists (1,195,991,040 and 8,030,257,152 parameters).
  * ``init_params`` / ``make_grads`` -- bf16 weights ~ N(0, 0.02^2); grads
    N(0, 1) * 1e-3 * f_t, f_t = exp(N(0, 1)) drawn once per tensor.
"""
from __future__ import annotations

import torch

BATTERY_SEED = 7
SWEEP_SEED = 11
PARAM_SEED = 1234
GRAD_SEED = 5678
FACTOR_SEED = 4321

# Step hyper-parameters of the single-tensor workload (2^20 params, 10 steps).
HP_DEFAULT = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
# FlashSGD step hyper-parameters (SGD with momentum)
SGD_DEFAULT = dict(lr=1e-2, momentum=0.9, dampening=0.0, weight_decay=0.01, nesterov=False)


def battery() -> dict[str, torch.Tensor]:
    """The seven fp32 CPU tensors of the codec battery, in the page's draw order."""
    g = torch.Generator(device="cpu").manual_seed(BATTERY_SEED)
    ts = {}
    ts["normal"] = torch.randn(1 << 20, generator=g)
    a = torch.randn(1 << 20, generator=g)
    b = torch.randn(1 << 20, generator=g)
    ts["heavy_tail"] = a * torch.exp(b * 3)
    ts["tiny"] = torch.randn(1 << 16, generator=g) * 1e-20
    ts["adam_v_like"] = (torch.randn(1 << 20, generator=g) * 1e-3) ** 2
    ts["nonmult32"] = torch.randn((1 << 16) + 17, generator=g)
    ts["const_groups"] = torch.ones(1 << 12) * 0.37
    u = torch.rand(1 << 16, generator=g)
    z = torch.randn(1 << 16, generator=g)
    ts["with_zeros"] = torch.where(u < 0.3, torch.zeros(1), z)
    return ts


SWEEP_EXPONENTS = list(range(1, 255, 4))     # 64 exponent buckets
SWEEP_PER_EXP = 1 << 16


def split_sweep(per_exp: int = SWEEP_PER_EXP, seed: int = SWEEP_SEED) -> dict[int, torch.Tensor]:
    """fp32 sweep inputs for both master widths: {24: x, 32: x}, each
    64 * per_exp values, bucket by bucket, random sign and mantissa."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    out = {}
    for width in (24, 32):
        parts = []
        for e in SWEEP_EXPONENTS:
            mant = torch.randint(0, 1 << 23, (per_exp,), dtype=torch.int32, generator=g)
            sign = torch.randint(0, 2, (per_exp,), dtype=torch.int32, generator=g) << 31
            parts.append(sign | (e << 23) | mant)
        out[width] = torch.cat(parts).view(torch.float32)
    return out


def decoder_1b_shapes() -> list[tuple[str, tuple[int, ...]]]:
    """199 tensors: embedding 32000x2048 and 22 layers of q/k/v/o 2048x2048,
    gate/up 2048x5632, down 5632x2048 and two RMSNorm vectors of 2048."""
    d, f, vocab, layers = 2048, 5632, 32000, 22
    shapes = [("embed", (vocab, d))]
    for i in range(layers):
        shapes += [(f"l{i}.q", (d, d)), (f"l{i}.k", (d, d)), (f"l{i}.v", (d, d)),
                   (f"l{i}.o", (d, d)), (f"l{i}.gate", (d, f)), (f"l{i}.up", (d, f)),
                   (f"l{i}.down", (f, d)), (f"l{i}.norm1", (d,)), (f"l{i}.norm2", (d,))]
    return shapes


def decoder_8b_shapes() -> list[tuple[str, tuple[int, ...]]]:
    """290 tensors: embedding and LM head 128256x4096 and 32 layers of
    q/o 4096x4096, k/v 4096x1024, gate/up 4096x14336, down 14336x4096 and two
    norm vectors of 4096."""
    d, kv, f, vocab, layers = 4096, 1024, 14336, 128256, 32
    shapes = [("embed", (vocab, d))]
    for i in range(layers):
        shapes += [(f"l{i}.q", (d, d)), (f"l{i}.k", (d, kv)), (f"l{i}.v", (d, kv)),
                   (f"l{i}.o", (d, d)), (f"l{i}.gate", (d, f)), (f"l{i}.up", (d, f)),
                   (f"l{i}.down", (f, d)), (f"l{i}.norm1", (d,)), (f"l{i}.norm2", (d,))]
    shapes.append(("lm_head", (vocab, d)))
    return shapes


def numel(shape) -> int:
    n = 1
    for s in shape:
        n *= s
    return n


def init_param(n: int, device="cpu", seed: int = PARAM_SEED, std: float = 0.02,
               dtype=torch.bfloat16) -> torch.Tensor:
    """Weights N(0, std^2) drawn in fp32, cast to dtype (bf16: torch's
    round-to-nearest-even cast; fp32: as drawn)."""
    g = torch.Generator(device=device).manual_seed(seed)
    return (torch.randn(n, generator=g, device=device) * std).to(dtype)


def grad_factors(count: int, seed: int = FACTOR_SEED) -> torch.Tensor:
    """Per-tensor lognormal(0, 1) factors, drawn once and fixed across steps."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.exp(torch.randn(count, generator=g, dtype=torch.float64))


def make_grad(n: int, step: int, device="cpu", seed: int = GRAD_SEED,
              scale: float = 1e-3, factor: float = 1.0, stream_id: int = 0,
              dtype=torch.bfloat16) -> torch.Tensor:
    """Gradient of one tensor at one step: N(0, 1) * scale * factor in fp32,
    freshly drawn from (seed, stream_id, step), cast to dtype (bf16 by
    default; fp32 for an fp32 parameter)."""
    g = torch.Generator(device=device).manual_seed(seed + 1_000_003 * stream_id + step)
    return (torch.randn(n, generator=g, device=device) * (scale * factor)).to(dtype)


def bf16_bits(t: torch.Tensor) -> torch.Tensor:
    """Reinterpret a bf16 tensor as its int16 bit patterns (no arithmetic)."""
    return t.contiguous().view(torch.int16)
