"""Benchmark of the fused FlashAdamW step on one MI355X.

Workload: the 8,030,257,152-parameter decoder-shaped list (290 bf16 tensors:
embedding and LM head 128256x4096, 32 layers of q/o 4096x4096, k/v
4096x1024, gate/up 4096x14336, down 14336x4096, two norms of 4096), 24-bit
master (int8 rho), companded int8/uint8 states with fp16 group-32 scales
(the optimizer's default chunk-blocked state layout; --state-layout streams
keeps them as five arrays per tensor); one multi-tensor launch per step.
Inputs are synthetic and resident in HBM
before timing starts (bf16 weights ~ N(0, 0.02^2); one bf16 gradient set
N(0, 1e-3^2) times a per-tensor lognormal factor, reused by every step).

Other configurations (reported beside the default, not as its value):
--workload decoder-1b-list (199 tensors, 1,195,991,040 params), --workload
flat-2^20 (one tensor of 2^20 params: cache-resident, a latency figure),
--master-bits 32 | 0 (0: no split, the page's master_weight_bits=None),
--param-fp32 (fp32 parameters, never split), --linear (linear
codec ablation), --fp32-states (quantize_states=False), --optimizer sgd (the
FlashSGD step: lr 1e-2, momentum 0.9, weight decay 0.01), --grad-release (one
single-tensor launch per tensor, the gradient-release launch pattern).
--codec times the codec and split entry points instead (one JSON line each).

Prints one JSON line: Gparam/s over the K timed steps, the roofline of the
step kernel (algorithmic bytes per param of the configuration against
8 TB/s), the oracle's throughput on host cores (the 1.2B list in full on all
threads, and a sixteenth of it on one thread), the GPU, CPU, ROCm and
clock readings, and the board power and shader clock that sysfs reports
while the same step runs for a few more (untimed) seconds after the timed
steps.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import threading
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


def bytes_per_param(master_bits: int, quantize_states: bool = True, n_states: int = 2,
                    param_bytes: int = 2) -> float:
    """Algorithmic HBM bytes per parameter per step: read the param and its
    grad (bf16: 2 bytes each; fp32 parameters: 4), rho 1|2 (none without a
    split), each state (m and v for AdamW, the momentum buffer for SGD) 1
    byte plus an fp16 scale per 32 (2/32), or 4 bytes as fp32; write all of
    them except the grad."""
    rho = {24: 1, 32: 2, 0: 0}[master_bits]
    states = n_states * ((1 + 2 / 32) if quantize_states else 4)
    read = 2 * param_bytes + rho + states
    write = param_bytes + rho + states
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


def valu_roofline(ms_launch: float, sclk_mhz=None):
    """The step's second roof: its VALU wavefront instructions per launch
    (committed counter record) at a modelled peak issue rate (one wavefront
    instruction per SIMD every 4 cycles at 2.4 GHz), against the measured
    launch time; also at the shader clock the GPU reported right after the
    timed steps and at the clock the counters saw during the step
    (GRBM_GUI_ACTIVE cycles over the launch's duration).  The counters also
    give the VALU instructions each SIMD issued per 4 cycles of the step: a
    value above 1 means that the hardware co-issues VALU instructions and the
    one-per-4-cycles model overstates the VALU time.  None when the record is
    stale."""
    rec = _counter_record()
    if rec is None or not rec.get("valu_insts_per_launch"):
        return None
    lane_insts = rec["valu_insts_per_launch"] * 64
    achieved = lane_insts / (ms_launch * 1e-3)
    out = {"bound": "alu", "achieved": achieved, "peak": PEAK_VALU_LANE_INSTS,
           "unit": "VALU lane-instructions/s", "frac": achieved / PEAK_VALU_LANE_INSTS,
           "ms_at_peak": lane_insts / PEAK_VALU_LANE_INSTS * 1e3,
           "valu_per_element_lane": rec.get("valu_per_element_lane")}
    if sclk_mhz:
        peak_clk = PEAK_VALU_LANE_INSTS * sclk_mhz / 2400.0
        out.update(sclk_mhz=sclk_mhz, peak_at_sclk=peak_clk, frac_at_sclk=achieved / peak_clk,
                   ms_at_sclk=lane_insts / peak_clk * 1e3)
    step_clk = rec.get("sclk_mhz_during_step")
    if step_clk:
        peak_step = PEAK_VALU_LANE_INSTS * step_clk / 2400.0
        out.update(sclk_mhz_during_step=step_clk, frac_at_step_clock=achieved / peak_step,
                   valu_insts_per_simd_quad_cycle=rec.get("valu_insts_per_simd_quad_cycle"))
    return out


WORKLOADS = {"decoder-8b-list": W.decoder_8b_shapes, "decoder-1b-list": W.decoder_1b_shapes,
             "flat-2^20": lambda: [("flat", (1 << 20,))]}


def build_workload(master_bits: int, companded: bool, quantize_states: bool = True,
                   workload: str = "decoder-8b-list", optimizer: str = "adamw",
                   param_fp32: bool = False, state_layout=None):
    """state_layout None: the binding's default (chunk-blocked for
    FlashAdamW's quantized states, the per-tensor streams otherwise)."""
    shapes = WORKLOADS[workload]()
    dt = torch.float32 if param_fp32 else torch.bfloat16
    params = [W.init_param(W.numel(s), device="cuda", seed=W.PARAM_SEED + i, dtype=dt)
              for i, (_, s) in enumerate(shapes)]
    factors = W.grad_factors(len(shapes)).tolist()
    grads = [W.make_grad(W.numel(s), 1, device="cuda", stream_id=i, factor=factors[i], dtype=dt)
             for i, (_, s) in enumerate(shapes)]
    if optimizer == "sgd":
        opt = F.FlashSGD(params, master_bits=master_bits or None, companded=companded,
                         quantize_states=quantize_states, state_layout=state_layout,
                         **W.SGD_DEFAULT)
    else:
        opt = F.FlashAdamW(params, master_bits=master_bits or None, companded=companded,
                           quantize_states=quantize_states, state_layout=state_layout,
                           **W.HP_DEFAULT)
    return opt, grads


def environment() -> dict:
    """GPU name, compute units, ROCm/HIP version and the live clocks, read
    from torch and rocm-smi (best effort: fields that cannot be read are
    omitted)."""
    env = {}
    try:
        prop = torch.cuda.get_device_properties(0)
        env.update(gpu=prop.name, arch=getattr(prop, "gcnArchName", None),
                   compute_units=prop.multi_processor_count, hip_torch_build=torch.version.hip)
    except Exception:
        pass
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm_runtime"] = f.read().strip()
    except OSError:
        pass
    env["cpu_model"] = cpu_model()
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


def _mhz(text):
    """'2157Mhz' -> 2157.0 (None if unreadable)."""
    try:
        return float(str(text).lower().replace("mhz", "").strip())
    except (TypeError, ValueError):
        return None


def _gpu_hwmon():
    """(hwmon directory, DRM device directory) of the GPU torch calls device
    0, matched by PCI domain and bus (or the only GPU with a power sensor);
    (None, None) where sysfs does not show them."""
    try:
        prop = torch.cuda.get_device_properties(0)
        want = (prop.pci_domain_id, prop.pci_bus_id)
    except Exception:
        want = None
    found = []
    for card in sorted(glob.glob("/sys/class/drm/card*")):
        if not re.fullmatch(r"card\d+", os.path.basename(card)):
            continue                            # connectors such as card0-DP-1
        dev = os.path.join(card, "device")
        mons = [m for m in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*")))
                if os.path.exists(os.path.join(m, "power1_input"))]
        if not mons:
            continue
        parts = os.path.basename(os.path.realpath(dev)).split(":")   # "0000:75:00.0"
        try:
            key = (int(parts[0], 16), int(parts[1], 16))
        except (ValueError, IndexError):
            key = None
        found.append((key, mons[0], dev))
    for key, mon, dev in found:
        if want is not None and key == want:
            return mon, dev
    return (found[0][1], found[0][2]) if len(found) == 1 else (None, None)


def _read_sclk(dev):
    """The shader clock level marked current in pp_dpm_sclk, in MHz."""
    try:
        with open(os.path.join(dev, "pp_dpm_sclk")) as f:
            for line in f:
                if "*" in line:
                    return _mhz(line.split(":", 1)[1].replace("*", ""))
    except OSError:
        pass
    return None


def power_during(run, seconds: float):
    """Board power (hwmon power1_input) and shader clock (pp_dpm_sclk),
    sampled every 20 ms from sysfs while run() is called for `seconds`
    (each call runs a few more steps and returns their per-launch ms); the
    first second is dropped as the ramp.  None where sysfs has no power
    sensor for the GPU."""
    mon, dev = _gpu_hwmon()
    if mon is None or seconds <= 0:
        return None
    samples, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                with open(os.path.join(mon, "power1_input")) as f:
                    w = int(f.read()) / 1e6             # microwatts
                samples.append((time.perf_counter(), w, _read_sclk(dev)))
            except (OSError, ValueError):
                pass
            stop.wait(0.02)

    th = threading.Thread(target=sample, daemon=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    th.start()
    per = []
    while time.perf_counter() - t0 < seconds:
        per.extend(run())
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stop.set()
    th.join()
    sel = [x for x in samples if t0 + min(1.0, seconds / 3) <= x[0] <= t1]
    if not sel:
        return None
    cap = None
    try:
        with open(os.path.join(mon, "power1_cap")) as f:
            cap = int(f.read()) / 1e6
    except (OSError, ValueError):
        pass
    clk = [x[2] for x in sel if x[2]]
    return {"board_w": statistics.mean(x[1] for x in sel), "board_w_max": max(x[1] for x in sel),
            "cap_w": cap, "sclk_mhz": statistics.mean(clk) if clk else None,
            "seconds": t1 - t0, "samples": len(sel),
            "ms_per_launch_median": statistics.median(per) if per else None,
            "source": "sysfs hwmon power1_input and pp_dpm_sclk, every 20 ms"}


def time_steps(opt, grads, steps: int, warmup: int, per_tensor: bool = False,
               batch_below: int = 0, n_streams: int = 1, graph: bool = False):
    """per_tensor: the gradient-release launch pattern, one single-tensor
    launch per tensor (the step is then the whole sequence of launches);
    tensors with fewer than batch_below elements are instead stepped together
    in one list launch after the others (attach_grad_release's batching).
    n_streams > 1: the single-tensor launches go round-robin to that many
    side streams, which start after and are joined back into the timed
    stream (attach_grad_release's streams).  graph: the capture-safe list
    step (FlashAdamW.plan) captured once into a HIP graph; each step writes
    its scalars (set_step, a 128-byte copy) and replays the graph."""
    small = [i for i, g in enumerate(grads) if g.numel() < batch_below]
    large = [i for i, g in enumerate(grads) if g.numel() >= batch_below]
    side = [torch.cuda.Stream() for _ in range(n_streams)] if per_tensor and n_streams > 1 else []

    replay = None
    if graph:
        plan = opt.plan(grads, step=opt.t + 1)
        torch.cuda.synchronize()
        replay = torch.cuda.CUDAGraph()
        with torch.cuda.graph(replay):
            plan.launch()
        torch.cuda.synchronize()

    def one_step(stream=None):
        if replay is not None:
            opt.t += 1
            plan.set_step(opt.t, stream)
            replay.replay()
        elif per_tensor:
            cur = stream or torch.cuda.current_stream()
            for s in side:
                s.wait_stream(cur)
            for k, i in enumerate(large):
                opt.step_tensor(i, grads[i], side[k % len(side)] if side else stream)
            if small:
                opt.step_tensors(small, [grads[i] for i in small], stream)
            for s in side:
                cur.wait_stream(s)
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


def cpu_model() -> str:
    """The host CPU's model name with its family/model/stepping numbers (a
    virtual machine may report only the vendor's product line by name)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    if fields:
                        break                   # the first processor's block is enough
                    continue
                k, v = (x.strip() for x in line.split(":", 1))
                fields.setdefault(k, v)
    except OSError:
        return "unknown"
    name = fields.get("model name", "unknown")
    ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    return f"{name} ({', '.join(ids)})" if ids else name


def _host_list(shapes, frac: int, master_bits, quantize_states, param_fp32=False):
    """Host copies of the seeded workload's parameters (the first 1/frac of
    each tensor, 32-aligned) with fresh oracle states, and one seeded
    gradient set; generated on the GPU with the benchmark's seeds."""
    import oracle
    factors = W.grad_factors(len(shapes)).tolist()
    dt = torch.float32 if param_fp32 else torch.bfloat16
    host = (lambda t: t.cpu().numpy()) if param_fp32 else \
        (lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16))
    states, grads = [], []
    for i, (_, shp) in enumerate(shapes):
        n = W.numel(shp)
        m = n if frac == 1 else max(32, (n // frac) // 32 * 32)
        p = W.init_param(n, device="cuda", seed=W.PARAM_SEED + i, dtype=dt)[:m]
        g = W.make_grad(n, 1, device="cuda", stream_id=i, factor=factors[i], dtype=dt)[:m]
        states.append(oracle.State.zeros_like_param(host(p).copy(), master_bits or None,
                                                    quantize_states))
        grads.append(np.ascontiguousarray(host(g)))
        del p, g
    torch.cuda.empty_cache()
    return states, grads


def _time_oracle(states, grads, hp, threads, steps=3):
    """Median seconds of `steps` timed list steps (after one untimed step)."""
    import oracle
    oracle.adamw_step_list(states, grads, oracle.hparams(step=1, **hp), threads)
    times, used = [], 0
    for k in range(steps):
        t0 = time.perf_counter()
        used = oracle.adamw_step_list(states, grads, oracle.hparams(step=2 + k, **hp), threads)
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), used


def cpu_baseline(master_bits: int, companded: bool = True, quantize_states: bool = True,
                 threads: int = 0, single_frac: int = 16, param_fp32: bool = False):
    """The oracle as it is (its OpenMP list driver, unchanged) on the host's
    cores over the 1.2B decoder list in full -- the shapes of one GPU's share
    of the 8.0B list on 8 GPUs; the step is elementwise, so its rate per
    parameter is the 8.0B list's -- with the benchmark's seeded inputs: one
    untimed step, then the median of three timed steps at all host threads.
    The same on one thread over the first 1/single_frac of every tensor (the
    whole list takes about 30 s per step on one thread)."""
    import oracle
    oracle.build(force=False)
    shapes = W.decoder_1b_shapes()
    hp = dict(lr=W.HP_DEFAULT["lr"], betas=W.HP_DEFAULT["betas"], eps=W.HP_DEFAULT["eps"],
              weight_decay=W.HP_DEFAULT["weight_decay"], master_bits=master_bits or None,
              companded=companded, quantize_states=quantize_states, fp32_param=param_fp32)
    states, grads = _host_list(shapes, 1, master_bits, quantize_states, param_fp32)
    n_all = sum(s.param.size for s in states)
    dt_all, used = _time_oracle(states, grads, hp, threads)
    del states, grads
    states, grads = _host_list(shapes, single_frac, master_bits, quantize_states, param_fp32)
    n_one = sum(s.param.size for s in states)
    dt_one, _ = _time_oracle(states, grads, hp, 1)
    return {"value": n_all / dt_all / 1e9, "unit": "Gparam/s", "cores": used, "kind": "oracle",
            "sample": f"the 1.2B decoder list in full ({n_all} params, 199 tensors), median of "
                      f"3 steps ({dt_all:.2f} s each) on {used} threads",
            "single_thread": {"value": n_one / dt_one / 1e9, "unit": "Gparam/s", "cores": 1,
                              "sample": f"first 1/{single_frac} of every tensor of the 1.2B list "
                                        f"({n_one} params), median of 3 steps ({dt_one:.2f} s each)"},
            "cpu_model": cpu_model(), "host_threads": os.cpu_count()}


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
    # context: plain torch streams over the same n-element buffers -- a
    # write-only fill, a read + write negation, and a uint8 -> fp32
    # conversion, which has dequantize's mix (1 byte read, 4 written per
    # element) -- to show the memory system's ceilings for the shapes above
    cases += [
        ("reference: torch fill_ (write-only)", "fp32", 4.0, lambda: out.fill_(0.5)),
        ("reference: torch neg (read + write)", "fp32", 8.0, lambda: torch.neg(x, out=out)),
        ("reference: torch uint8 to fp32 copy_", "u8->f32", 5.0,
         lambda: out.copy_(codes.view(torch.uint8))),
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
    ap.add_argument("--batch-below", type=int, default=F.RELEASE_BATCH_BELOW,
                    help="with --grad-release: step tensors below this many elements together "
                         "(default: attach_grad_release's; 0 launches every tensor alone)")
    ap.add_argument("--grad-release", action="store_true",
                    help="one single-tensor launch per tensor (the gradient-release pattern)")
    ap.add_argument("--release-streams", type=int, default=F.RELEASE_STREAMS,
                    help="with --grad-release: spread the launches over this many streams "
                         "(default: attach_grad_release's)")
    ap.add_argument("--graph", action="store_true",
                    help="step through the capture-safe plan launch replayed from a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the oracle on the host cores")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="host threads for the oracle's all-core timing (0: all)")
    ap.add_argument("--first-step", type=int, default=1,
                    help="step count of the first (warm-up) step; from about 17321 on, with the "
                         "default betas, both bias corrections are 1 in fp32")
    ap.add_argument("--state-layout", choices=["blocked", "streams"], default=None,
                    help="optimizer state layout (default: the binding's: chunk-blocked for "
                         "FlashAdamW's quantized states, the streams otherwise)")
    ap.add_argument("--param-fp32", action="store_true",
                    help="fp32 parameters and gradients (never split; needs --master-bits 0)")
    ap.add_argument("--calibrate-copy", type=float, default=0.0, metavar="GIB",
                    help="only run one device copy of GIB GiB (for counter scaling) and exit")
    ap.add_argument("--no-copy-ref", action="store_true")
    ap.add_argument("--power-seconds", type=float, default=3.0,
                    help="after the timed steps, run the step this many more seconds while "
                         "sampling board power and shader clock (0: skip)")
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
    if args.param_fp32 and (mb != 0 or args.optimizer != "adamw"):
        print("--param-fp32 needs --master-bits 0 and the AdamW step", file=sys.stderr)
        sys.exit(2)
    copy_gbs = None if args.no_copy_ref else copy_reference()
    opt, grads = build_workload(mb, comp, qs, args.workload, args.optimizer, args.param_fp32,
                                args.state_layout)
    layout = opt.states[0].state_layout if opt.states else "streams"
    opt.t = args.first_step - 1
    opt.ts = [opt.t] * len(opt.states)
    n = sum(s.param.numel() for s in opt.states)
    n_tensors = len(opt.states)
    print(f"# workload ready: {len(opt.states)} tensors, {n} params, "
          f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated", file=sys.stderr, flush=True)

    if args.graph and (args.optimizer != "adamw" or args.grad_release):
        print("--graph times the AdamW list step (no --grad-release, no --optimizer sgd)", file=sys.stderr)
        sys.exit(2)
    wall, per = time_steps(opt, grads, args.steps, args.warmup, args.grad_release, args.batch_below,
                           args.release_streams, args.graph)
    env = environment()                     # clocks read right after the timed steps
    ms_step = wall * 1e3 / args.steps
    ms_launch = float(np.mean(per))
    power = None
    if not args.graph and "rocprof" not in os.environ.get("LD_PRELOAD", ""):
        k = max(1, min(500, int(200.0 / max(ms_launch, 1e-3))))
        power = power_during(lambda: time_steps(opt, grads, k, 0, args.grad_release,
                                                args.batch_below, args.release_streams)[1],
                             args.power_seconds)
    bpp = bytes_per_param(mb, qs, 1 if args.optimizer == "sgd" else 2, 4 if args.param_fp32 else 2)
    alg_bytes = bpp * n
    achieved = alg_bytes / (ms_launch * 1e-3) / 1e9
    print(f"# per-launch ms: mean {ms_launch:.3f} median {np.median(per):.3f} "
          f"min {min(per):.3f} max {max(per):.3f}", file=sys.stderr, flush=True)
    sizes = [s.param.numel() for s in opt.states]
    del opt, grads
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline and args.optimizer == "adamw":
        cpu = cpu_baseline(mb, comp, qs, args.cpu_threads, param_fp32=args.param_fp32)
    default = (args.workload, mb, comp, qs, args.optimizer, args.grad_release, args.param_fp32,
               args.first_step, args.graph, layout) == ("decoder-8b-list", 24, True, True, "adamw",
                                                        False, False, 1, False, "blocked")
    name = args.workload + ("" if comp else "-linear") + ("" if qs else "-fp32-states") + \
        ("-fp32-params" if args.param_fp32 else ("-no-split" if mb == 0 else "")) + \
        ("-flashsgd" if args.optimizer == "sgd" else "") + \
        ("-per-tensor-launches" if args.grad_release else "") + \
        (f"-batched-below-{args.batch_below}" if args.grad_release and args.batch_below else "") + \
        (f"-{args.release_streams}-streams" if args.grad_release and args.release_streams > 1 else "") + \
        (f"-from-step-{args.first_step}" if args.first_step != 1 else "") + \
        ("-graph-replay" if args.graph else "") + \
        (f"-{layout}-layout" if layout != ("blocked" if qs and args.optimizer == "adamw" else "streams")
         else "")

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
                   "param_dtype": "fp32" if args.param_fp32 else "bf16",
                   "first_step": args.first_step,
                   "state_layout": layout,
                   "bytes_per_param": bpp,
                   "launches_per_step": launches},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic_per_launch() if default else None,
                     "copy_ref_gbs": copy_gbs},
        "valu_roofline": valu_roofline(ms_launch, _mhz(env.get("clocks", {}).get("sclk")))
                         if default else None,
        "cpu_baseline": cpu,
        "power": power,
        "env": env,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
