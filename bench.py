#!/usr/bin/env python3
"""Throughput of one rank's TSP gated-MLP block on one MI355X.

A step is one full forward of the block over one batch of synthetic tokens:
the fused gate/up kernel over every weight shard (visited in ring order) and
the down kernel that accumulates all shards' partial outputs into the fp32 Y.
Inputs, packed weights and workspace are resident in HBM before timing.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--pass backward|attention]

Prints one JSON line. The default workload is the Llama-3-8B-shaped SwiGLU
block (T=4096 tokens, d=4096, f=14336, P=8 shards, ring start 3), reported in
TFLOP/s; ``--workload decode70b`` runs the T=16 weight-streaming workload,
reported in GB/s. An untimed clock pre-heat (~0.1 s of steps) comes before
the warmup. The ``roofline`` object is for the dominant kernel, timed with
fence-free HIP events that the library records around every kernel on the
stream the kernel runs on, over a region of as many steps right after the
timed region (which has events only at step boundaries).
``cpu_baseline`` times the fp64 oracle on a bounded sample of the same
workload on this host's cores. ``--pass backward`` times the backward instead
(one step = the gradients for a seeded output gradient; TFLOP/s over the
gradient products, the recomputed forward product not counted); its
``variants`` time, in the same process, the backward from the pre-activations
a training forward saved (no recomputation), and whole training steps
(forward + backward, TFLOP/s over both passes' algorithmic flops) with and
without saving them.
``--pass attention`` times one rank's TSP attention block instead (default
workload: the Llama-3-8B attention shape, rank 3 of 8, causal; one step =
the Q/K/V projection of the rank's tokens, attention over the context that
the other ranks' projections filled before timing, and the output
projection).
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sharded gated-MLP TFLOP/s + % bf16 MFMA peak (large T); HBM GB/s % peak (T=16)"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, published (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector / MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
KERNEL_SOURCES = {
    "gateup_tiled": ["gemm_tiled.hip", "w16.h", "common.h"],
    "down_tiled": ["gemm_tiled.hip", "w16.h", "common.h"],
    "skinny_gateup": ["gemm_skinny.hip", "common.h"],
    "skinny_down": ["gemm_skinny.hip", "common.h"],
    "gateup_f32": ["gemm_f32.hip", "common.h"],
    "down_f32": ["gemm_f32.hip", "common.h"],
    "reduce_partials": ["gemm_tiled.hip", "w16.h", "common.h"],
    "bwd_dh": ["backward.hip", "w16.h", "common.h"],
    "bwd_gateup": ["backward.hip", "w16.h", "common.h"],
    "bwd_dw_dx": ["backward.hip", "w16.h", "common.h"],
    "bwd_saved": ["backward.hip", "w16.h", "common.h"],
    "gateup_save": ["gemm_tiled.hip", "w16.h", "common.h"],
    "attn_qkv": ["attn.hip", "w16.h", "common.h"],
    "attn_core": ["attn_core.hip", "w16.h", "common.h"],
    "attn_out": ["gemm_tiled.hip", "w16.h", "common.h"],
}
METRIC_BWD = "sharded gated-MLP backward TFLOP/s (dX and weight gradients; recomputation not counted)"
METRIC_ATTN = "TSP attention block TFLOP/s, one rank (projections + causal attention over the exchanged context)"


def is_decode(w) -> bool:
    """The weight-streaming (decode-like) workloads, priced in GB/s against
    HBM: bf16 with at most 48 tokens (the skinny kernels' range)."""
    return w.dtype == "bf16" and w.T <= 48


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(kernel: str) -> str:
    """Hash of the code (comments and blank lines removed) of the sources a
    kernel is built from, and of the file-specific compiler options the build
    gives them: counter summaries stay valid across comment edits."""
    from sharded_transformer_mlp_amd.build import EXTRA_FLAGS
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sharded_transformer_mlp_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = (re.sub(r"//.*", "", line).rstrip() for line in text.splitlines())
        h.update("\n".join(line for line in lines if line.strip()).encode())
        if f in EXTRA_FLAGS:
            h.update(" ".join(EXTRA_FLAGS[f]).encode())
    return h.hexdigest()[:16]


def kernel_work(w, kernel: str, T: int):
    """Algorithmic (flops, bytes) of one launch of `kernel` on workload w."""
    es = 2 if w.dtype == "bf16" else 4
    n_gu = 2 if w.act == "swiglu" else 1
    d, f = w.d, w.f
    if kernel == "bwd_dh":                  # dH = dY.Wd^T: Wd, dY in, fp32 dH out; the same launch copies X and dY transposed
        return 2 * T * d * f, f * d * es + T * d * es + T * f * 4 + 2 * 2 * T * d * es
    if kernel == "bwd_gateup":              # recomputed gate/up product + backward epilogue
        return 2 * n_gu * T * d * f, n_gu * d * f * es + T * d * es + T * f * 4 + (n_gu + 1) * T * f * es
    if kernel == "bwd_dw_dx":               # weight gradients and dX = sum dG.Wg^T + dU.Wu^T, one launch
        return ((2 * n_gu + 2) * T * d * f + 2 * n_gu * T * d * f,
                2 * T * d * es + (n_gu + 1) * T * f * es + (n_gu + 1) * d * f * 4      # dW: X, dY, dG/dU, H in, dW out
                + n_gu * d * f * es + n_gu * T * f * es + T * d * 4)                  # dX: Wg/Wu, dG/dU in, dX out
    if kernel == "bwd_saved":               # the backward epilogue on saved pre-activations (no product)
        return 0, n_gu * T * f * 4 + T * f * 4 + (n_gu + 1) * T * f * es
    if kernel == "gateup_save":             # the gate/up product that also writes its pre-activations
        return 2 * n_gu * T * d * f, n_gu * d * f * es + T * d * es + T * f * es + n_gu * T * f * 4
    if kernel in ("gateup_tiled", "skinny_gateup", "gateup_f32"):
        flops = 2 * T * w.d * w.f * n_gu
        byts = n_gu * w.d * w.f * es + T * w.d * es + T * w.f * es      # W_gu, X, H out
    elif kernel == "reduce_partials":
        # adds the ring-group partials of a split down product into Y; its only
        # algorithmic traffic is the Y write (the partials are implementation)
        flops, byts = 0, T * w.d * 4
    else:
        flops = 2 * T * w.f * w.d
        byts = w.f * w.d * es + T * w.f * es + T * w.d * 4                 # W_d, H in, Y out
    return flops, byts


def read_traffic(workload_name: str, kernel: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel source has changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload_name}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != kernel_source_hash(kernel):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def oracle_threads(fn, *a, **kw):
    """Run a CPU-baseline body with the BLAS pool set to every CPU of this
    process's affinity mask; `cores` is the thread count the pool then
    reports (the threads the oracle's matrix products actually use)."""
    n = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:  # pragma: no cover
        return fn(*a, cores=n, **kw)
    with threadpool_limits(limits=n):
        used = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        return fn(*a, cores=max(used) if used else 1, **kw)


def cpu_baseline(w, inp, budget_s: float, dy=None):
    return oracle_threads(_cpu_baseline, w, inp, budget_s, dy)


def cpu_baseline_attn(w, inp, budget_s: float):
    return oracle_threads(_cpu_baseline_attn, w, inp, budget_s)


def _cpu_baseline(w, inp, budget_s: float, dy=None, cores=1):
    """Time the fp64 oracle on the first n token rows, n sized to ~budget_s
    (the backward when dy is given: gradients of those rows' loss)."""
    import oracle
    x = inp.x.float().numpy()
    wg = None if inp.w_gate is None else inp.w_gate.float().numpy()
    wu, wd = inp.w_up.float().numpy(), inp.w_down.float().numpy()
    order = w.order()

    g = None if dy is None else dy.float().numpy()

    def run(n):
        t = time.perf_counter()
        if g is None:
            oracle.mlp_forward(x[:n], wg, wu, wd, w.P, order, w.act)
        else:
            oracle.mlp_backward(x[:n], wg, wu, wd, g[:n], w.P, order, w.act)
        return time.perf_counter() - t

    n = min(w.T, 16)
    dt = run(n)
    while dt < 0.25 * budget_s and n < w.T:
        n = min(w.T, max(n + 1, int(n * min(8.0, 0.6 * budget_s / max(dt, 1e-3)))))
        dt = run(n)
    reps = 1
    if n == w.T and dt < 0.5 * budget_s:       # whole workload is quick: repeat it, report the mean
        reps = max(1, int(0.5 * budget_s / max(dt, 1e-3)))
        dt = sum(run(n) for _ in range(reps)) / reps
    if g is not None:
        value = oracle.backward_flops(n, w.d, w.f, w.act) / dt / 1e12
        unit = "TFLOP/s"
    elif is_decode(w):                          # decode-like: report bytes streamed per second
        value = w.bytes(n) / dt / 1e9
        unit = "GB/s"
    else:
        value = w.flops(n) / dt / 1e12
        unit = "TFLOP/s"
    what = "fp64 numpy oracle backward" if g is not None else "fp64 numpy oracle"
    return {"value": value, "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"first {n} of {w.T} token rows, full weights, {what}, "
                      f"{dt:.2f} s per pass, mean of {reps} pass(es)"}


def attn_kernel_work(w, kernel: str):
    """Algorithmic (flops, bytes) of one launch of an attention-block kernel."""
    T, d, H, Hkv, dh, P = w.T, w.d, w.H, w.Hkv, w.dh, w.P
    visible = w.rank * T + T if w.causal else w.S          # context rows the rank reads
    pairs = (w.rank * T * T + T * (T + 1) // 2) if w.causal else T * w.S
    if kernel == "attn_qkv":           # X . [Wq | Wk | Wv]: weights and X in, Q, K, V out (bf16)
        n = (H + 2 * Hkv) * dh
        return 2 * T * d * n, d * n * 2 + T * d * 2 + T * n * 2
    if kernel == "attn_core":          # Q, the visible K and V rows in, O out
        return 4 * dh * H * pairs, T * H * dh * 2 * 2 + 2 * visible * Hkv * dh * 2
    if kernel == "attn_out":           # O . Wo into fp32 Y
        return 2 * T * H * dh * d, H * dh * d * 2 + T * H * dh * 2 + T * d * 4
    if kernel == "reduce_partials":
        return 0, T * d * 4
    raise KeyError(kernel)


def _cpu_baseline_attn(w, inp, budget_s: float, cores=1):
    """Time the fp64 attention oracle on the rank's first n token rows (it
    also projects every rank's keys and values, the exchanged context, as the
    oracle does for any row count), n sized to ~budget_s."""
    import oracle.attn_oracle as ao
    X = inp.x_all.float().numpy()
    Wq, Wk, Wv, Wo = (t.float().numpy() for t in (inp.w_q, inp.w_k, inp.w_v, inp.w_o))

    def run(n):
        t = time.perf_counter()
        ao.tsp_attention(X, Wq, Wk, Wv, Wo, w.H, w.Hkv, w.P, w.rank, order=w.order(), causal=w.causal,
                         rows=list(range(n)))
        return time.perf_counter() - t

    n = min(w.T, 16)
    dt = run(n)
    while dt < 0.25 * budget_s and n < w.T:
        n = min(w.T, max(n + 1, int(n * min(8.0, 0.6 * budget_s / max(dt, 1e-3)))))
        dt = run(n)
    # flops of the sampled rows: their projections, their attention pairs
    pairs = sum(w.rank * w.T + i + 1 for i in range(n)) if w.causal else n * w.S
    flops = 4 * n * w.d * w.H * w.dh + 4 * n * w.d * w.Hkv * w.dh + 4 * w.dh * w.H * pairs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n} of the rank's {w.T} query rows (the oracle also projects the keys and values "
                      f"of all {w.S} positions), fp64 numpy attention oracle, {dt:.2f} s"}


def bench_attention(args):
    import torch
    import oracle.attn_oracle as ao
    from sharded_transformer_mlp_amd.binding import TspAttn
    from sharded_transformer_mlp_amd.inputs import attn_workload, make_attn_inputs

    name = args.workload if args.workload != "llama8b" else "attn_llama8b"
    w = attn_workload(name)
    dev = torch.device("cuda:0")
    log(f"attention workload {w.name}: generating inputs")
    inp = make_attn_inputs(w)
    x_all = inp.x_all.to(dev)
    t = time.perf_counter()
    attn = TspAttn(inp.w_q.to(dev), inp.w_k.to(dev), inp.w_v.to(dev), inp.w_o.to(dev), w.H, w.Hkv, w.P,
                   order=w.order(), causal=w.causal, T_max=w.T)
    pack_ms = (time.perf_counter() - t) * 1e3
    # the exchange, before timing: every other rank's keys and values
    for rho in range(w.P):
        if rho != w.rank:
            attn.project_kv(x_all[rho * w.T:(rho + 1) * w.T].contiguous(), rho)
    x = x_all[w.rank * w.T:(w.rank + 1) * w.T].contiguous()
    y = torch.empty(w.T, w.d, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step():
        attn.forward(x, w.rank, y)

    # pre-heat, warmup, timed region, then the kernel region (see measure_mlp)
    n_pre = preheat(step)
    log(f"pre-heat {n_pre} steps; warmup {args.warmup}, timing {args.steps} steps")
    ms, per = time_steps(step, args.steps, args.warmup)
    log(f"kernel-timing region, {args.steps} steps")
    attn.read_timing()
    attn.set_timing(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    attn.set_timing(False)
    kernels = {k: v[0] / max(v[1], 1) for k, v in attn.read_timing().items()}
    log(f"ms/step {ms:.4f}; kernels {kernels}")
    log("per-step ms: " + " ".join(f"{p:.3f}" for p in per))
    total = ao.attention_flops(w.T, w.d, w.H, w.Hkv, w.dh, w.P, w.rank, w.causal)
    value = total / (ms * 1e-3) / 1e12
    dom = max(kernels, key=lambda k: kernels[k])
    flops, byts = attn_kernel_work(w, dom)
    roof = {"bound": "mfma", "achieved": flops / (kernels[dom] * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = read_traffic(w.name, dom)
    roof.update(kernel=dom, kernel_ms=kernels[dom], algorithmic_bytes=byts, algorithmic_flops=flops)
    out = {
        "metric": METRIC_ATTN, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded normal tokens and weights, bf16-rounded)",
        "config": {"workload": w.name, "T": w.T, "S": w.S, "d": w.d, "H": w.H, "Hkv": w.Hkv, "dh": w.dh,
                   "P": w.P, "rank": w.rank, "causal": w.causal, "order": w.order(),
                   "parallelism": "one TSP rank (head-group loop on one GPU; other ranks' keys/values "
                                  "projected before timing)"},
        "pct_of_peak": value / PEAK_BF16_TFLOPS * 100.0, **step_stats(per),
        "kernels_ms": kernels, "pack_ms": pack_ms, "roofline": roof, "cpu_baseline": None, "pass": "attention",
        "env": {"gpu": torch.cuda.get_device_name(0), "torch": torch.__version__, "hip": torch.version.hip},
    }
    attn.close()
    del x_all, x, y
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline_attn(w, inp, args.cpu_budget)
    print(json.dumps(out), flush=True)


def calibrate_copy(nbytes: int = 1 << 30, reps: int = 5):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    a.fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {nbytes} bytes")


class HipEvents:
    """Timing events on a HIP stream, created through the HIP runtime that
    torch has loaded, with hipEventDisableSystemFence: a timing-only event
    then skips the system-scope release (a cache writeback and invalidation
    at every step boundary, which slows the next step's first kernel)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n: int, stream_handle: int):
        import ctypes
        import torch
        torch.cuda.init()
        path = None
        with open("/proc/self/maps") as fh:
            for line in fh:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self.c = ctypes
        hip = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [vp, vp]
        hip.hipEventSynchronize.argtypes = [vp]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        hip.hipEventDestroy.argtypes = [vp]
        self.hip, self.stream = hip, vp(stream_handle)
        self.ev = []
        for _ in range(n):
            e = vp()
            self._ok(hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE), "create")
            self.ev.append(e)

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"hipEvent {what} failed: {rc}")

    def record(self, i: int):
        self._ok(self.hip.hipEventRecord(self.ev[i], self.stream), "record")

    def elapsed_ms(self, i: int, j: int) -> float:
        self._ok(self.hip.hipEventSynchronize(self.ev[j]), "synchronize")
        t = self.c.c_float()
        self._ok(self.hip.hipEventElapsedTime(self.c.byref(t), self.ev[i], self.ev[j]), "elapsed")
        return t.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def preheat(step, seconds: float = 0.1) -> int:
    """Untimed steps for about `seconds` before the warmup: the GPU's clock
    takes ~15 ms of work to come out of idle. Returns the step count."""
    import torch
    torch.cuda.synchronize()
    t = time.perf_counter()
    step()
    torch.cuda.synchronize()
    one = max(time.perf_counter() - t, 1e-5)
    n = max(0, min(2000, int(seconds / one)))
    for _ in range(n):
        step()
    torch.cuda.synchronize()
    return n + 1


def time_steps(step, steps: int, warmup: int):
    """W untimed warmup steps, then exactly `steps` steps between two device
    synchronisations, with a (fence-free) event at every step boundary on the
    stream the steps run on. Returns (ms per step over the whole region,
    per-step ms)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = HipEvents(steps + 1, torch.cuda.current_stream().cuda_stream)
    try:
        torch.cuda.synchronize()
        evs.record(0)
        for i in range(steps):
            step()
            evs.record(i + 1)
        torch.cuda.synchronize()
        per = [evs.elapsed_ms(i, i + 1) for i in range(steps)]
        total = evs.elapsed_ms(0, steps)
    finally:
        evs.close()
    return total / steps, per


def step_stats(per):
    s = sorted(per)
    n = len(s)
    med = s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])
    return {"median_ms": med, "min_ms": s[0], "max_ms": s[-1], "first_ms": per[0]}


def measure_mlp(w, args, backward: bool = False, with_cpu: bool = False, variant: str = ""):
    """One workload's timed region, kernel region and roofline (a dict in the
    shape of the bench's JSON line). variant (with backward): "" = the
    backward recomputing the gate/up product, "saved" = the backward from the
    pre-activations a training forward kept, "train" = forward + backward
    (recomputing), "train_saved" = training forward + backward from its
    saved pre-activations."""
    import torch
    from sharded_transformer_mlp_amd.binding import TspMLP
    from sharded_transformer_mlp_amd.inputs import make_inputs, make_output_grad

    dev = torch.device("cuda:0")
    log(f"workload {w.name}: generating inputs")
    inp = make_inputs(w)
    x = inp.x.to(dev)
    wg = None if inp.w_gate is None else inp.w_gate.to(dev)
    wu, wd = inp.w_up.to(dev), inp.w_down.to(dev)
    torch.cuda.synchronize()
    t = time.perf_counter()
    mlp = TspMLP(wg, wu, wd, w.P, order=w.order(), act=w.act, T_max=w.T)
    pack_ms = (time.perf_counter() - t) * 1e3
    # the handle holds packed copies: the caller's weights are not needed again
    del wg, wu, wd
    dy = None
    if backward:
        # a step is one backward: the seeded output gradient against the
        # resident inputs and the handle's weights, gradients written into
        # preallocated fp32 tensors (the first call also allocates the
        # backward workspace, so the warmup does that)
        dy = make_output_grad(w)
        dy_dev = dy.to(dev)
        grads = {"dX": torch.empty(w.T, w.d, dtype=torch.float32, device=dev),
                 "dW_gate": None if w.act != "swiglu" else torch.empty(w.d, w.f, dtype=torch.float32, device=dev),
                 "dW_up": torch.empty(w.d, w.f, dtype=torch.float32, device=dev),
                 "dW_down": torch.empty(w.f, w.d, dtype=torch.float32, device=dev)}

        saved = None
        if variant in ("saved", "train_saved"):
            saved = torch.empty(mlp.saved_bytes(w.T), dtype=torch.uint8, device=dev)
            y = torch.empty(w.T, w.d, dtype=torch.float32, device=dev)
            mlp.forward_train(x, saved=saved, y=y)     # the step reads these
        elif variant == "train":
            y = torch.empty(w.T, w.d, dtype=torch.float32, device=dev)

        if variant == "saved":
            def step():
                mlp.backward(x, dy_dev, out=grads, saved=saved)
        elif variant == "train":
            def step():
                mlp.forward(x, y)
                mlp.backward(x, dy_dev, out=grads)
        elif variant == "train_saved":
            def step():
                mlp.forward_train(x, saved=saved, y=y)
                mlp.backward(x, dy_dev, out=grads, saved=saved)
        else:
            def step():
                mlp.backward(x, dy_dev, out=grads)
    else:
        y = torch.empty(w.T, w.d, dtype=torch.float32, device=dev)

        def step():
            mlp.forward(x, y)

    # Untimed clock pre-heat (~0.1 s of steps; the first backward also
    # allocates its workspace and unpacks the handle's weights), the W warmup
    # steps, the timed region (the headline), then a kernel region of as many
    # steps with the library recording fence-free HIP events around every
    # kernel on the stream it runs on (~5 us per step for a two-kernel step:
    # 2 % of a decode step, which is why it is a region of its own).
    n_pre = preheat(step)
    log(f"pre-heat {n_pre} steps; warmup {args.warmup}, timing {args.steps} steps")
    ms, per = time_steps(step, args.steps, args.warmup)
    log(f"kernel-timing region, {args.steps} steps")
    mlp.read_timing()
    mlp.set_timing(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    mlp.set_timing(False)
    kt = mlp.read_timing()
    kernels = {k: v[0] / max(v[1], 1) for k, v in kt.items()}
    log(f"ms/step {ms:.4f}; kernels {kernels}")
    log("per-step ms: " + " ".join(f"{p:.3f}" for p in per))

    decode = is_decode(w) and not backward
    if backward:
        import oracle
        flops_step = oracle.backward_flops(w.T, w.d, w.f, w.act)
        if variant.startswith("train"):
            flops_step += w.flops()
        value, unit = flops_step / (ms * 1e-3) / 1e12, "TFLOP/s"
    elif decode:
        value, unit = w.bytes() / (ms * 1e-3) / 1e9, "GB/s"
    else:
        value, unit = w.flops() / (ms * 1e-3) / 1e12, "TFLOP/s"
    peak = PEAK_HBM_GBS if decode else (PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS)

    dom = max(kernels, key=lambda k: kernels[k])
    flops, byts = kernel_work(w, dom, w.T)
    dom_s = kernels[dom] * 1e-3
    if decode:
        roof = {"bound": "hbm", "achieved": byts / dom_s / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / dom_s / 1e12, "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = read_traffic(w.name, dom)
    roof["kernel"] = dom
    roof["kernel_ms"] = kernels[dom]
    roof["algorithmic_bytes"] = byts
    roof["algorithmic_flops"] = flops

    st = step_stats(per)
    scale = (w.bytes() / 1e9 if decode else (flops_step if backward else w.flops()) / 1e12) * 1e3
    out = {
        "value": value,
        "unit": unit,
        "ms_per_step": ms,
        **st,
        "value_at_median": scale / st["median_ms"],
        "value_at_min": scale / st["min_ms"],
        "pct_of_peak": value / peak * 100.0,
        "dtype": w.dtype,
        "config": {"workload": w.name, "T": w.T, "d": w.d, "f": w.f, "P": w.P, "act": w.act,
                   "ring_order": w.order(), "parallelism": "one TSP rank (shard loop on one GPU)"},
        "kernels_ms": kernels,
        "kernel_sum_ms": sum(kernels.values()),
        "pack_ms": pack_ms,
        "roofline": roof,
    }
    if backward:
        out["config"]["parallelism"] = "one TSP rank's backward (shard loop on one GPU)"
        out["variant"] = variant or "recompute"
        if saved is not None:
            out["saved_bytes"] = saved.numel()
        del grads, dy_dev, saved
    else:
        del y
    mlp.close()
    del x
    torch.cuda.empty_cache()
    if with_cpu:
        log("cpu baseline (fp64 oracle)")
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_budget, dy)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--also", default="long70b,decode70b",
                    help="comma-separated workloads timed after the headline one, in the same process and with "
                         "the same --steps/--warmup, reported under 'also' (empty: none)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the HBM-read and MFMA ceiling probes")
    ap.add_argument("--calibrate-copy", action="store_true", help="only run the copy kernel used to scale counters")
    ap.add_argument("--pass", dest="which", choices=("forward", "backward", "attention"), default="forward",
                    help="forward (the headline metric), the backward (gradients for a seeded dY) or the "
                         "attention block")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU ring transfer is not implemented)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.which == "attention":
        bench_attention(args)
        return

    from sharded_transformer_mlp_amd.inputs import workload

    w = workload(args.workload)
    backward = args.which == "backward"
    res = measure_mlp(w, args, backward=backward)
    decode = is_decode(w) and not backward
    out = {
        "metric": METRIC_BWD if backward else METRIC,
        "value": res["value"],
        "unit": res["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal tokens and weights, bf16-rounded)",
        "config": res["config"],
        "pct_of_peak": res["pct_of_peak"],
        "env": {"gpu": torch.cuda.get_device_name(0),
                "arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", None),
                "torch": torch.__version__, "hip": torch.version.hip},
    }
    for k in ("median_ms", "min_ms", "max_ms", "first_ms", "value_at_median", "value_at_min", "kernels_ms",
              "kernel_sum_ms", "pack_ms", "roofline"):
        out[k] = res[k]
    out["cpu_baseline"] = None
    if backward:
        out["pass"] = "backward"
        # the same backward from saved pre-activations, and whole training
        # steps (forward + backward) both ways, same process and --steps/--warmup
        out["variants"] = {}
        for v in ("saved", "train", "train_saved"):
            rv = measure_mlp(w, args, backward=True, variant=v)
            out["variants"][v] = {k: rv[k] for k in ("value", "unit", "ms_per_step", "median_ms", "min_ms",
                                                     "kernels_ms", "kernel_sum_ms", "saved_bytes") if k in rv}
    also = [a for a in args.also.split(",") if a.strip()] if not backward else []
    if also:
        out["also"] = []
        for name in also:
            wa = workload(name.strip())
            ra = measure_mlp(wa, args)
            ra.pop("dtype")
            out["also"].append(ra)
    if not args.no_ceilings:
        # Measured ceilings of this GPU beside the datasheet peaks, after the
        # timed regions so they do not heat the GPU before them.
        from sharded_transformer_mlp_amd.binding import probe_hbm_read, probe_mfma_bf16
        log("ceiling probes")
        # The read rate depends on the buffer size (measured: ~7.0 TB/s at
        # 1 GiB, 6.8 at 2 GiB, 6.3 at 4 GiB), so the probe reads as many bytes
        # as the headline workload's weights, at least 1 GiB (4x the
        # last-level cache).
        chunk = 64 << 20
        probe_bytes = max(1 << 30, -(-w.bytes() // chunk) * chunk)
        ceil = {"hbm_read_GBs": probe_hbm_read(probe_bytes, 10),
                "mfma_bf16_TFLOPs": probe_mfma_bf16(20000),
                "how": f"library probes: a {probe_bytes >> 20} MiB buffer read 10x with 16-byte nontemporal "
                       "loads; 16 independent 16x16x32 bf16 MFMAs per wave, 2 waves per SIMD, "
                       "pseudo-random operands"}
        out["ceilings"] = ceil
        roof = out["roofline"]
        c = ceil["hbm_read_GBs"] if decode else (ceil["mfma_bf16_TFLOPs"] if w.dtype == "bf16" else None)
        roof["frac_of_measured_ceiling"] = None if c is None else roof["achieved"] / c
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        from sharded_transformer_mlp_amd.inputs import make_inputs, make_output_grad
        out["cpu_baseline"] = cpu_baseline(w, make_inputs(w), args.cpu_budget,
                                           make_output_grad(w) if backward else None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
