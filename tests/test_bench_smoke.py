"""bench.py on every workload with a few steps: one JSON line with the
contract's fields and a roofline object for the dominant kernel."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr


@pytest.mark.gpu
@pytest.mark.parametrize("wl", ["tiny", "gelu", "llama8b", "decode70b", "long70b"])
def test_bench_emits_the_contract_line(wl):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"[gpu] bench {wl}", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", wl, "--steps", "2",
                        "--warmup", "1", "--no-cpu-baseline", "--no-ceilings", "--also", ""],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1 and d["value"] > 0
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert 0 < roof["frac"] < 1


@pytest.mark.gpu
def test_bench_default_line_carries_the_whole_metric():
    """The default run: the Llama-shaped headline, then the 70B long-context
    (TFLOP/s) and decode (GB/s) workloads in the same process, each with its
    per-step median and minimum and its own roofline."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[gpu] bench default line", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--no-cpu-baseline", "--no-ceilings"], capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["config"]["workload"].startswith("llama3-8b") and d["unit"] == "TFLOP/s"
    assert d["min_ms"] <= d["median_ms"] <= d["max_ms"]
    also = {a["config"]["workload"]: a for a in d["also"]}
    long70, dec70 = (also[k] for k in ("70b-long-swiglu-bf16-T16384-d8192-f28672-P8",
                                       "70b-decode-swiglu-bf16-T16-d8192-f28672-P8"))
    assert long70["unit"] == "TFLOP/s" and long70["roofline"]["bound"] == "mfma"
    assert dec70["unit"] == "GB/s" and dec70["roofline"]["bound"] == "hbm"
    for a in (long70, dec70):
        assert a["value"] > 0 and 0 < a["roofline"]["frac"] < 1 and a["min_ms"] <= a["median_ms"]


@pytest.mark.gpu
@pytest.mark.parametrize("wl", ["gelu", "llama8b"])
def test_bench_backward_line(wl):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"[gpu] bench --pass backward {wl}", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", wl, "--pass", "backward",
                        "--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--no-ceilings"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["pass"] == "backward" and d["unit"] == "TFLOP/s" and d["value"] > 0
    assert d["roofline"]["kernel"].startswith("bwd_") and 0 < d["roofline"]["frac"] < 1


@pytest.mark.gpu
def test_bench_attention_line():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[gpu] bench --pass attention", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--pass", "attention",
                        "--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--no-ceilings"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["pass"] == "attention" and d["unit"] == "TFLOP/s" and d["value"] > 0
    assert d["roofline"]["kernel"].startswith("attn_") and 0 < d["roofline"]["frac"] < 1


def test_attention_kernel_work_adds_up_to_the_block():
    """The per-kernel algorithmic flops the attention bench prices each kernel
    with add up to the oracle's flop count of the whole block."""
    sys.path.insert(0, ROOT)
    import bench
    import oracle.attn_oracle as ao
    from sharded_transformer_mlp_amd.inputs import AttnWorkload, attn_workload
    for w in (attn_workload("attn_llama8b"),
              AttnWorkload("x", T=96, d=512, H=16, Hkv=4, dh=128, P=4, rank=3, seed=0, causal=False)):
        total = sum(bench.attn_kernel_work(w, k)[0] for k in ("attn_qkv", "attn_core", "attn_out"))
        assert total == ao.attention_flops(w.T, w.d, w.H, w.Hkv, w.dh, w.P, w.rank, w.causal)


def test_backward_kernel_work_adds_up_to_the_gradients():
    """The algorithmic flops the backward bench prices its two product launches
    with (dH; the weight gradients and dX in one launch) add up to the
    oracle's count of the backward's gradient products, and the dH launch's
    bytes include the transposed copies of X and dY that ride in it."""
    sys.path.insert(0, ROOT)
    import bench
    import oracle
    from sharded_transformer_mlp_amd.inputs import Workload, workload
    for w in (workload("llama8b"), workload("gelu"),
              Workload("x", T=300, d=512, f=2048, P=4, act="swiglu", dtype="bf16", seed=0)):
        total = sum(bench.kernel_work(w, k, w.T)[0] for k in ("bwd_dh", "bwd_dw_dx"))
        assert total == oracle.backward_flops(w.T, w.d, w.f, w.act)
        _, dh_bytes = bench.kernel_work(w, "bwd_dh", w.T)
        es = 2
        assert dh_bytes == w.f * w.d * es + w.T * w.d * es + w.T * w.f * 4 + 4 * w.T * w.d * es
