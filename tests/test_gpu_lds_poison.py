"""Parity on the LDS-poison debug build (libtsp_mlp_lds_poison.so): every
kernel fills its LDS with NaN before first use, so a fragment read that ran
ahead of its data (a missing wait or barrier in a staging ring) shows up as
NaN in Y. Same cases and bars as the main parity tests, fewer of them."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from sharded_transformer_mlp_amd import binding
from sharded_transformer_mlp_amd.inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu

DEBUG_LIB = os.path.join(os.path.dirname(binding.LIB_PATH), "libtsp_mlp_lds_poison.so")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def poison_library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(DEBUG_LIB):
        raise RuntimeError(f"{DEBUG_LIB} is missing: build with `python -m sharded_transformer_mlp_amd.build`")
    saved = (binding._lib, binding.LIB_PATH)
    binding._lib, binding.LIB_PATH = None, DEBUG_LIB
    yield
    binding._lib, binding.LIB_PATH = saved


CASES = [
    ("tiled shape 0 + split", Workload("a", T=300, d=512, f=2048, P=4, act="swiglu", dtype="bf16", seed=11, r0=1),
     "tiled", (0, 0)),
    ("tiled auto shapes + split", Workload("a", T=300, d=512, f=2048, P=4, act="swiglu", dtype="bf16", seed=11,
                                           r0=1), "tiled", None),
    ("tiled shape 0, 4 tiles", Workload("b", T=513, d=1024, f=4096, P=2, act="swiglu", dtype="bf16", seed=12),
     "tiled", (0, 0)),
    ("tiled shape 1", Workload("c", T=290, d=512, f=2048, P=2, act="swiglu", dtype="bf16", seed=21), "tiled", (1, 1)),
    ("tiled shape 2", Workload("c", T=290, d=512, f=2048, P=2, act="swiglu", dtype="bf16", seed=21), "tiled", (2, 2)),
    ("tiled gelu shape 1/3", Workload("g", T=200, d=256, f=1024, P=2, act="gelu_tanh", dtype="bf16", seed=12),
     "tiled", (1, 3)),
    ("skinny", Workload("k", T=17, d=1024, f=2048, P=4, act="swiglu", dtype="bf16", seed=31, r0=2), "skinny", None),
    ("fp32", Workload("f", T=70, d=96, f=200, P=4, act="swiglu", dtype="f32", seed=14, r0=3), "auto", None),
]


@pytest.mark.parametrize("name,w,path,tiles", CASES, ids=[c[0] for c in CASES])
def test_parity_with_poisoned_lds(name, w, path, tiles):
    assert binding.LIB_PATH == DEBUG_LIB
    say(f"[gpu] LDS poison: {name}")
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    mlp = binding.TspMLP(None if inp.w_gate is None else inp.w_gate.to(dev), inp.w_up.to(dev),
                         inp.w_down.to(dev), w.P, order=w.order(), act=w.act, T_max=w.T)
    mlp.set_path(path)
    if tiles is not None:
        mlp.set_tiles(*tiles)
    y = mlp.forward(inp.x.to(dev))
    torch.cuda.synchronize()
    mlp.close()
    y = y.cpu().double().numpy()
    assert np.isfinite(y).all(), f"{name}: NaN in Y (a read ran ahead of its data)"
    f = lambda t: None if t is None else t.float().numpy()
    ref = oracle.mlp_forward(f(inp.x), f(inp.w_gate), f(inp.w_up), f(inp.w_down), w.P, w.order(), w.act)
    dy = y - ref
    if w.dtype == "f32":
        assert np.max(np.abs(dy)) / np.max(np.abs(ref)) <= 1e-4
    else:
        assert np.linalg.norm(dy) / np.linalg.norm(ref) <= 3e-3
        assert np.max(np.abs(dy)) <= 2e-2 * np.max(np.abs(ref))


BWD_CASES = [
    ("backward swiglu", Workload("bs", T=300, d=512, f=2048, P=4, act="swiglu", dtype="bf16", seed=15, r0=1)),
    ("backward gelu", Workload("bg", T=200, d=256, f=1024, P=2, act="gelu_tanh", dtype="bf16", seed=16)),
]


@pytest.mark.parametrize("name,w", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_with_poisoned_lds(name, w):
    """The backward kernels stage operands and results in LDS too: NaN in a
    gradient means a read ran ahead of its data. The backward from saved
    pre-activations (same epilogue, no product) must give the same bits."""
    from sharded_transformer_mlp_amd.inputs import make_output_grad
    assert binding.LIB_PATH == DEBUG_LIB
    say(f"[gpu] LDS poison: {name}")
    inp, dy = make_inputs(w), make_output_grad(w)
    dev = torch.device("cuda:0")
    wg = None if inp.w_gate is None else inp.w_gate.to(dev)
    wu, wd = inp.w_up.to(dev), inp.w_down.to(dev)
    mlp = binding.TspMLP(wg, wu, wd, w.P, order=w.order(), act=w.act, T_max=w.T)
    x, d_y = inp.x.to(dev), dy.to(dev)
    g = mlp.backward(x, d_y)
    _, saved = mlp.forward_train(x)
    gs = mlp.backward(x, d_y, saved=saved)
    torch.cuda.synchronize()
    mlp.close()
    for k in g:
        assert (g[k] is None and gs[k] is None) or torch.equal(g[k], gs[k]), f"{name} {k}: saved != recomputed"
    f = lambda t: None if t is None else t.float().numpy()
    ref = oracle.mlp_backward(f(inp.x), f(inp.w_gate), f(inp.w_up), f(inp.w_down), f(dy), w.P, w.order(), w.act)
    for k, r in ref.items():
        if r is None:
            continue
        got = g[k].cpu().double().numpy()
        assert np.isfinite(got).all(), f"{name} {k}: NaN (a read ran ahead of its data)"
        assert np.linalg.norm(got - r) / np.linalg.norm(r) <= 3e-3, (name, k)
        assert np.max(np.abs(got - r)) <= 2e-2 * np.max(np.abs(r)), (name, k)


ATTN_CASES = [
    ("attention causal g4", dict(T=96, d=512, H=16, Hkv=4, P=4, rank=2, seed=17, causal=True)),
    ("attention full g1", dict(T=64, d=256, H=4, Hkv=4, P=2, rank=1, seed=18, causal=False)),
]


@pytest.mark.parametrize("name,kw", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_attention_with_poisoned_lds(name, kw):
    """The attention kernels stage the projection tile and the K / V^T tiles
    in LDS: NaN in Y means a read ran ahead of its data."""
    import oracle.attn_oracle as ao
    from sharded_transformer_mlp_amd.inputs import AttnWorkload, make_attn_inputs
    assert binding.LIB_PATH == DEBUG_LIB
    say(f"[gpu] LDS poison: {name}")
    w = AttnWorkload("p", dh=128, **kw)
    inp = make_attn_inputs(w)
    dev = torch.device("cuda:0")
    attn = binding.TspAttn(inp.w_q.to(dev), inp.w_k.to(dev), inp.w_v.to(dev), inp.w_o.to(dev), w.H, w.Hkv, w.P,
                           order=w.order(), causal=w.causal, T_max=w.T)
    x_all = inp.x_all.to(dev)
    for rho in range(w.P):
        if rho != w.rank:
            attn.project_kv(x_all[rho * w.T:(rho + 1) * w.T].contiguous(), rho)
    y = attn.forward(x_all[w.rank * w.T:(w.rank + 1) * w.T].contiguous(), w.rank)
    torch.cuda.synchronize()
    attn.close()
    y = y.cpu().double().numpy()
    assert np.isfinite(y).all(), f"{name}: NaN in Y (a read ran ahead of its data)"
    f = lambda t: t.float().numpy()
    ref = ao.tsp_attention(f(inp.x_all), f(inp.w_q), f(inp.w_k), f(inp.w_v), f(inp.w_o), w.H, w.Hkv, w.P, w.rank,
                           order=w.order(), causal=w.causal)
    assert np.linalg.norm(y - ref) / np.linalg.norm(ref) <= 3e-3, name
