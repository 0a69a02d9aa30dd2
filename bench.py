"""Benchmark of the fused FlashAdamW step on one MI355X.

Workload: the 8,030,257,152-parameter decoder-shaped list (290 bf16 tensors:
embedding and LM head 128256x4096, 32 layers of q/o 4096x4096, k/v
4096x1024, gate/up 4096x14336, down 14336x4096, two norms of 4096), 24-bit
master (int8 rho), companded int8/uint8 states with fp16 group-32 scales;
one multi-tensor launch per step.  Inputs are synthetic and resident in HBM
before timing starts (bf16 weights ~ N(0, 0.02^2); one bf16 gradient set
N(0, 1e-3^2) times a per-tensor lognormal factor, reused by every step).

Other configurations (reported beside the default, not as its value):
--workload decoder-1b-list (199 tensors, 1,195,991,040 params), --master-bits
32 | 0 (0: no split, the page's master_weight_bits=None), --linear (linear
codec ablation), --fp32-states (quantize_states=False), --optimizer sgd (the
FlashSGD step: lr 1e-2, momentum 0.9, weight decay 0.01), --grad-release (one
single-tensor launch per tensor, the gradient-release launch pattern).
--codec times the codec and split entry points instead (one JSON line each).

Prints one JSON line: Gparam/s over the K timed steps, the roofline of the
step kernel (algorithmic bytes per param of the configuration against
8 TB/s), the oracle's throughput on host cores for a bounded sample of the
same workload, and the GPU, ROCm and clock readings.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from bit_companded_adam_amd import flashopt as F  # noqa: E402
from bit_companded_adam_amd import workloads as W  # noqa: E402

METRIC = "FlashAdamW step Gparam/s and % of HBM roofline (12.25 B/param), 1 GPU"
PEAK_HBM_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "bit_companded_adam_amd", "csrc", "flashopt_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "adamw_step_8b_traffic.json")


def bytes_per_param(master_bits: int, quantize_states: bool = True, n_states: int = 2) -> float:
    """Algorithmic HBM bytes per parameter per step: read bf16 param 2, bf16
    grad 2, rho 1|2 (none without a split), each state (m and v for AdamW, the
    momentum buffer for SGD) 1 byte plus an fp16 scale per 32 (2/32), or 4
    bytes as fp32; write all of them except the grad."""
    rho = {24: 1, 32: 2, 0: 0}[master_bits]
    states = n_states * ((1 + 2 / 32) if quantize_states else 4)
    read = 2 + 2 + rho + states
    write = 2 + rho + states
    return read + write


def kernel_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


# Peak VALU issue of MI355X: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz, one
# (non-packed) instruction per lane per cycle; a wavefront instruction
# takes 4 cycles of a SIMD.
PEAK_VALU_LANE_INSTS = 256 * 4 * 16 * 2.4e9


def _counter_record():
    """The committed rocprofv3 counter record of the default step, or None if
    the kernel source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    return rec if rec.get("kernel_sha") == kernel_sha() else None


def traffic_per_launch():
    """HBM bytes per launch from the committed counter record (or None)."""
    rec = _counter_record()
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def valu_roofline(ms_launch: float):
    """The step's second roof: its VALU wavefront instructions per launch
    (committed counter record) at the peak issue rate, against the measured
    launch time; None when the record is stale."""
    rec = _counter_record()
    if rec is None or not rec.get("valu_insts_per_launch"):
        return None
    lane_insts = rec["valu_insts_per_launch"] * 64
    achieved = lane_insts / (ms_launch * 1e-3)
    return {"bound": "alu", "achieved": achieved, "peak": PEAK_VALU_LANE_INSTS,
            "unit": "VALU lane-instructions/s", "frac": achieved / PEAK_VALU_LANE_INSTS,
            "ms_at_peak": lane_insts / PEAK_VALU_LANE_INSTS * 1e3}


WORKLOADS = {"decoder-8b-list": W.decoder_8b_shapes, "decoder-1b-list": W.decoder_1b_shapes}


def build_workload(master_bits: int, companded: bool, quantize_states: bool = True,
                   workload: str = "decoder-8b-list", optimizer: str = "adamw"):
    shapes = WORKLOADS[workload]()
    params = [W.init_param(W.numel(s), device="cuda", seed=W.PARAM_SEED + i)
              for i, (_, s) in enumerate(shapes)]
    factors = W.grad_factors(len(shapes)).tolist()
    grads = [W.make_grad(W.numel(s), 1, device="cuda", stream_id=i, factor=factors[i])
             for i, (_, s) in enumerate(shapes)]
    if optimizer == "sgd":
        opt = F.FlashSGD(params, master_bits=master_bits or None, companded=companded,
                         quantize_states=quantize_states, **W.SGD_DEFAULT)
    else:
        opt = F.FlashAdamW(params, master_bits=master_bits or None, companded=companded,
                           quantize_states=quantize_states, **W.HP_DEFAULT)
    return opt, grads


def environment() -> dict:
    """GPU name, compute units, ROCm/HIP version and the live clocks, read
    from torch and rocm-smi (best effort: fields that cannot be read are
    omitted)."""
    env = {}
    try:
        prop = torch.cuda.get_device_properties(0)
        env.update(gpu=prop.name, arch=getattr(prop, "gcnArchName", None),
                   compute_units=prop.multi_processor_count, hip=torch.version.hip)
    except Exception:
        pass
    if "rocprof" in os.environ.get("LD_PRELOAD", ""):
        return env                  # no child processes under a profiler's preload
    try:
        import subprocess
        out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                             timeout=20).stdout
        clocks = {}
        for line in out.splitlines():
            if "sclk" in line or "mclk" in line or "fclk" in line:
                key = "sclk" if "sclk" in line else ("mclk" if "mclk" in line else "fclk")
                mhz = line.split("(")[-1].rstrip(")").strip()
                clocks.setdefault(key, mhz)
        if clocks:
            env["clocks"] = clocks
    except Exception:
        pass
    return env


def time_steps(opt, grads, steps: int, warmup: int, per_tensor: bool = False,
               batch_below: int = 0):
    """per_tensor: the gradient-release launch pattern, one single-tensor
    launch per tensor (the step is then the whole sequence of launches);
    tensors with fewer than batch_below elements are instead stepped together
    in one list launch after the others (attach_grad_release's batching)."""
    small = [i for i, g in enumerate(grads) if g.numel() < batch_below]
    large = [i for i, g in enumerate(grads) if g.numel() >= batch_below]

    def one_step(stream=None):
        if per_tensor:
            for i in large:
                opt.step_tensor(i, grads[i], stream)
            if small:
                opt.step_tensors(small, [grads[i] for i in small], stream)
        else:
            opt.step(grads, stream)

    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        one_step(stream)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in evs]          # ms, one launch each
    return wall, per


def cpu_baseline(master_bits: int, target_elems: int, threads: int, min_seconds: float = 10.0,
                 companded: bool = True, quantize_states: bool = True):
    """The oracle as it is, on host threads, over a bounded sample of the
    workload: the first target_elems / 32 elements of each of 32 evenly spaced
    tensors of the 8.0B list (same distributions), steps 2, 3, ... after an
    untimed step 1, repeated for about min_seconds."""
    import oracle
    oracle.build(force=False)
    shapes = W.decoder_8b_shapes()
    pick = np.linspace(0, len(shapes) - 1, 32).astype(int)
    per = target_elems // 32
    factors = W.grad_factors(len(shapes)).numpy()
    states, g1, g2 = [], [], []
    for k, i in enumerate(pick):
        n = min(per, W.numel(shapes[i][1]))
        p = W.init_param(n, seed=W.PARAM_SEED + int(i)).view(torch.int16).numpy().view(np.uint16)
        states.append(oracle.State.zeros_like_param(p, master_bits or None, quantize_states))
        for lst, t in ((g1, 1), (g2, 2)):
            lst.append(W.make_grad(n, t, stream_id=int(i), factor=float(factors[i]))
                       .view(torch.int16).numpy().view(np.uint16))
    hp = dict(lr=W.HP_DEFAULT["lr"], betas=W.HP_DEFAULT["betas"], eps=W.HP_DEFAULT["eps"],
              weight_decay=W.HP_DEFAULT["weight_decay"], master_bits=master_bits or None,
              companded=companded, quantize_states=quantize_states)
    oracle.adamw_step_list(states, g1, oracle.hparams(step=1, **hp), threads)
    n_total = sum(s.param.size for s in states)
    steps, used = 0, 0
    t0 = time.perf_counter()
    while True:                      # steps 2, 3, ... until about min_seconds of work
        used = oracle.adamw_step_list(states, g2 if steps % 2 == 0 else g1,
                                      oracle.hparams(step=2 + steps, **hp), threads)
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": n_total * steps / dt / 1e9, "unit": "Gparam/s", "cores": used, "kind": "oracle",
            "sample": f"{n_total} params (first {per} elements of 32 of the 290 tensors of the "
                      f"8.0B list), {steps} steps in {dt:.1f} s"}


def copy_reference(gib: float = 8.0, reps: int = 5) -> float:
    """Context for the roofline: GB/s (read + write) of a plain streaming
    kernel on this GPU -- torch's elementwise negation of a gib-GiB fp32
    buffer into another (reads and writes gib GiB each)."""
    n = int(gib * (1 << 30)) // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.neg(a, out=b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.neg(a, out=b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2.0 * n * 4 / (ms * 1e-3) / 1e9


def calibrate_copy(gib: float):
    """One plain streaming kernel of known size (torch's elementwise negation,
    reading and writing gib GiB each), for scaling rocprofv3 FETCH_SIZE /
    WRITE_SIZE counters."""
    n = int(gib * (1 << 30)) // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes_read": n * 4, "calibration_copy_bytes_written": n * 4}))


def bench_codec(n: int, reps: int, warmup: int):
    """Per-launch time of flashopt_quantize / dequantize (both specs) and
    flashopt_split / reconstruct (both widths) over one flat tensor of n
    elements: fp32 N(0, 1e-3^2) values (their squares for the variance
    spec).  Algorithmic bytes per element: quantize and dequantize 4 + 1 +
    2/32; split and reconstruct 4 + 2 + 1 (24-bit) or 4 + 2 + 2 (32-bit)."""
    g = torch.Generator(device="cuda").manual_seed(W.PARAM_SEED)
    x = torch.randn(n, generator=g, device="cuda") * 1e-3
    xa = x * x
    codes = torch.empty(n, dtype=torch.int8, device="cuda")
    scales = torch.empty(F.n_groups(n), dtype=torch.int16, device="cuda")
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    param = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    rho = {24: torch.empty(n, dtype=torch.int8, device="cuda"),
           32: torch.empty(n, dtype=torch.int16, device="cuda")}
    codec = 4 + 1 + 2 / 32
    cases = [
        ("flashopt_quantize", "momentum", codec,
         lambda: F.flashopt_quantize(x, F.SPEC_MOMENTUM, codes, scales)),
        ("flashopt_dequantize", "momentum", codec,
         lambda: F.flashopt_dequantize(codes, scales, F.SPEC_MOMENTUM, out)),
        ("flashopt_quantize", "variance", codec,
         lambda: F.flashopt_quantize(xa, F.SPEC_VARIANCE, codes.view(torch.uint8), scales)),
        ("flashopt_dequantize", "variance", codec,
         lambda: F.flashopt_dequantize(codes.view(torch.uint8), scales, F.SPEC_VARIANCE, out)),
        ("flashopt_split", "24-bit", 7.0, lambda: F.flashopt_split(x, 24, param, rho[24])),
        ("flashopt_reconstruct", "24-bit", 7.0,
         lambda: F.flashopt_reconstruct(param, rho[24], 24, out)),
        ("flashopt_split", "32-bit", 8.0, lambda: F.flashopt_split(x, 32, param, rho[32])),
        ("flashopt_reconstruct", "32-bit", 8.0,
         lambda: F.flashopt_reconstruct(param, rho[32], 32, out)),
    ]
    stream = torch.cuda.current_stream()
    for op, variant, bpe, fn in cases:
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        gbs = n * bpe / (ms * 1e-3) / 1e9
        print(json.dumps({
            "metric": f"{op} ({variant}) GB/s, 1 GPU", "value": gbs, "unit": "GB/s",
            "n_gpus": 1, "steps": reps, "warmup": warmup, "ms_per_step": ms,
            "higher_is_better": True, "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": f"flat tensor of {n} elements", "op": op, "variant": variant,
                       "bytes_per_element": bpe},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "traffic": None},
        }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decoder-8b-list", choices=sorted(WORKLOADS))
    ap.add_argument("--master-bits", type=int, default=24, choices=(24, 32, 0),
                    help="0: no master split (the parameter is cast back to bf16)")
    ap.add_argument("--linear", action="store_true", help="linear (non-companded) ablation")
    ap.add_argument("--fp32-states", action="store_true",
                    help="unquantized fp32 moments (weight-splitting-only ablation)")
    ap.add_argument("--optimizer", default="adamw", choices=("adamw", "sgd"),
                    help="sgd: the FlashSGD step (momentum buffer only)")
    ap.add_argument("--batch-below", type=int, default=0,
                    help="with --grad-release: step tensors below this many elements together")
    ap.add_argument("--grad-release", action="store_true",
                    help="one single-tensor launch per tensor (the gradient-release pattern)")
    ap.add_argument("--cpu-elems", type=int, default=1 << 27,
                    help="oracle sample size for the CPU baseline (0: skip)")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", type=float, default=0.0, metavar="GIB",
                    help="only run one device copy of GIB GiB (for counter scaling) and exit")
    ap.add_argument("--no-copy-ref", action="store_true")
    ap.add_argument("--codec", action="store_true",
                    help="instead of the step, time the codec and split entry points on one "
                         "flat tensor (one JSON line each)")
    ap.add_argument("--codec-elems", type=int, default=1 << 29)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the step needs no communication, and this "
              "build measures one GPU's share (--gpus 1).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy > 0:
        calibrate_copy(args.calibrate_copy)
        return
    if args.codec:
        bench_codec(args.codec_elems, args.steps, args.warmup)
        return

    mb, comp, qs = args.master_bits, not args.linear, not args.fp32_states
    copy_gbs = None if args.no_copy_ref else copy_reference()
    opt, grads = build_workload(mb, comp, qs, args.workload, args.optimizer)
    n = sum(s.param.numel() for s in opt.states)
    n_tensors = len(opt.states)
    print(f"# workload ready: {len(opt.states)} tensors, {n} params, "
          f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated", file=sys.stderr, flush=True)

    wall, per = time_steps(opt, grads, args.steps, args.warmup, args.grad_release, args.batch_below)
    env = environment()                     # clocks read right after the timed steps
    ms_step = wall * 1e3 / args.steps
    ms_launch = float(np.mean(per))
    bpp = bytes_per_param(mb, qs, 1 if args.optimizer == "sgd" else 2)
    alg_bytes = bpp * n
    achieved = alg_bytes / (ms_launch * 1e-3) / 1e9
    print(f"# per-launch ms: mean {ms_launch:.3f} median {np.median(per):.3f} "
          f"min {min(per):.3f} max {max(per):.3f}", file=sys.stderr, flush=True)
    sizes = [s.param.numel() for s in opt.states]
    del opt, grads
    torch.cuda.empty_cache()

    cpu = None
    if args.cpu_elems > 0 and args.optimizer == "adamw":
        cpu = cpu_baseline(mb, args.cpu_elems, args.cpu_threads, args.cpu_seconds, comp, qs)
    default = (args.workload, mb, comp, qs, args.optimizer, args.grad_release) == \
        ("decoder-8b-list", 24, True, True, "adamw", False)
    name = args.workload + ("" if comp else "-linear") + ("" if qs else "-fp32-states") + \
        ("-no-split" if mb == 0 else "") + ("-flashsgd" if args.optimizer == "sgd" else "") + \
        ("-per-tensor-launches" if args.grad_release else "") + \
        (f"-batched-below-{args.batch_below}" if args.grad_release and args.batch_below else "")

    launches = 1
    if args.grad_release:
        small = sum(1 for n in sizes if n < args.batch_below)
        launches = len(sizes) - small + (1 if small else 0)
    metric = METRIC
    if args.optimizer == "sgd":      # same measure for the FlashSGD step, at its own bytes/param
        metric = f"FlashSGD step Gparam/s and % of HBM roofline ({bpp:g} B/param), 1 GPU"
    out = {
        "metric": metric,
        "value": n / (ms_step * 1e-3) / 1e9,
        "unit": "Gparam/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, "params": n, "tensors": n_tensors,
                   "master_bits": mb, "companded": comp, "quantized_states": qs,
                   "bytes_per_param": bpp,
                   "launches_per_step": launches},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic_per_launch() if default else None,
                     "copy_ref_gbs": copy_gbs},
        "valu_roofline": valu_roofline(ms_launch) if default else None,
        "cpu_baseline": cpu,
        "env": env,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
