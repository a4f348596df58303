"""The library's launches captured into HIP graphs (torch.cuda.CUDAGraph on the
capture stream the binding passes through the C ABI) and replayed.

After a first eager call (which allocates the backward workspace and unpacks
the handle's weights), the forward, the allocation-free forward, the backward
and the training pair launch kernels only, so a caller can capture them into
a graph for a serving or training loop. Every replay here runs on inputs
rewritten between replays by eager work, with synchronisations in between,
and must equal the eager call on the same inputs bit for bit (same kernels).
"""
import sys

import pytest
import torch

from sharded_transformer_mlp_amd.inputs import Workload, make_inputs, make_output_grad

pytestmark = pytest.mark.gpu

KEYS = ("dX", "dW_gate", "dW_up", "dW_down")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sharded_transformer_mlp_amd import binding
    binding.lib()


def _handle(w, inp):
    from sharded_transformer_mlp_amd.binding import TspMLP
    dev = torch.device("cuda:0")
    wg = None if inp.w_gate is None else inp.w_gate.to(dev)
    return TspMLP(wg, inp.w_up.to(dev), inp.w_down.to(dev), w.P, order=w.order(), act=w.act, T_max=w.T)


def _capture(fn):
    """fn() captured into a graph after one eager warm-up on a side stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _inputs_for(w, seed):
    """A fresh token batch (and output gradient) of the workload's shape."""
    ws = w.with_(seed=seed)
    return make_inputs(ws).x, make_output_grad(ws)


FWD_CASES = [
    ("tiled + ring-group split (GeLU)", Workload("g", T=512, d=256, f=2048, P=2, act="gelu_tanh", dtype="bf16",
                                                 seed=71), False),
    ("tiled SwiGLU", Workload("g", T=700, d=512, f=2048, P=4, act="swiglu", dtype="bf16", seed=72, r0=1), False),
    ("skinny", Workload("g", T=16, d=1024, f=4096, P=4, act="swiglu", dtype="bf16", seed=73, r0=2), False),
    ("fp32", Workload("g", T=64, d=256, f=1024, P=2, act="swiglu", dtype="f32", seed=74), False),
    ("allocation-free forward", Workload("g", T=300, d=512, f=2048, P=4, act="swiglu", dtype="bf16", seed=75), True),
]


@pytest.mark.parametrize("name,w,static", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_graph_replays(name, w, static):
    from sharded_transformer_mlp_amd.binding import check, lib
    say(f"[gpu] graph: forward {name}")
    dev = torch.device("cuda:0")
    inp = make_inputs(w)
    mlp = _handle(w, inp)
    x = inp.x.to(dev).contiguous()
    y = torch.empty(w.T, w.d, dtype=torch.float32, device=dev)

    def fwd():
        if static:
            check(lib().tsp_mlp_forward_static(mlp.handle, w.T, x.data_ptr(), y.data_ptr(),
                                               torch.cuda.current_stream().cuda_stream))
        else:
            mlp.forward(x, y)

    g = _capture(fwd)
    for rep in range(3):
        xn, _ = _inputs_for(w, 1000 + rep)
        x.copy_(xn.to(dev))                              # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        y.fill_(float("nan"))
        fwd()                                            # eager, same inputs
        torch.cuda.synchronize()
        assert torch.equal(got, y), f"{name}: replay {rep} differs from the eager forward"
    del g
    mlp.close()


BWD_CASES = [
    ("SwiGLU", Workload("b", T=300, d=512, f=2048, P=4, act="swiglu", dtype="bf16", seed=76, r0=1)),
    ("GeLU", Workload("b", T=200, d=256, f=1024, P=2, act="gelu_tanh", dtype="bf16", seed=77)),
]


@pytest.mark.parametrize("name,w", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_and_training_pair_graph_replays(name, w):
    say(f"[gpu] graph: backward and training pair {name}")
    dev = torch.device("cuda:0")
    inp = make_inputs(w)
    mlp = _handle(w, inp)
    x = inp.x.to(dev).contiguous()
    dy = make_output_grad(w).to(dev).contiguous()
    gated = w.act == "swiglu"

    def grads():
        return {"dX": torch.empty(w.T, w.d, dtype=torch.float32, device=dev),
                "dW_gate": torch.empty(w.d, w.f, dtype=torch.float32, device=dev) if gated else None,
                "dW_up": torch.empty(w.d, w.f, dtype=torch.float32, device=dev),
                "dW_down": torch.empty(w.f, w.d, dtype=torch.float32, device=dev)}

    g_bwd, g_pair = grads(), grads()
    y = torch.empty(w.T, w.d, dtype=torch.float32, device=dev)
    saved = torch.empty(mlp.saved_bytes(w.T), dtype=torch.uint8, device=dev)
    graph_bwd = _capture(lambda: mlp.backward(x, dy, out=g_bwd))

    def pair():
        mlp.forward_train(x, saved=saved, y=y)
        mlp.backward(x, dy, out=g_pair, saved=saved)

    graph_pair = _capture(pair)
    for rep in range(3):
        xn, dyn = _inputs_for(w, 2000 + rep)
        x.copy_(xn.to(dev))
        dy.copy_(dyn.to(dev))
        torch.cuda.synchronize()
        graph_bwd.replay()
        graph_pair.replay()
        torch.cuda.synchronize()
        got_bwd = {k: None if v is None else v.clone() for k, v in g_bwd.items()}
        got_pair = {k: None if v is None else v.clone() for k, v in g_pair.items()}
        got_y = y.clone()
        ref = mlp.backward(x, dy)                        # eager, recomputing
        y_ref, _ = mlp.forward_train(x)                  # eager training forward, its own buffer
        torch.cuda.synchronize()
        for k in KEYS:
            if ref[k] is None:
                assert got_bwd[k] is None and got_pair[k] is None
                continue
            assert torch.equal(got_bwd[k], ref[k]), f"{name} {k}: backward replay {rep} differs"
            assert torch.equal(got_pair[k], ref[k]), f"{name} {k}: training-pair replay {rep} differs"
        assert torch.equal(got_y, y_ref), f"{name}: training forward replay {rep} differs"
    del graph_bwd, graph_pair
    mlp.close()


def test_attention_forward_graph_replays():
    """One rank's attention block (projection, attention over the context the
    other ranks filled, output projection) captured and replayed on new rank
    tokens: every replay bitwise equal to the eager forward."""
    from sharded_transformer_mlp_amd.binding import TspAttn
    from sharded_transformer_mlp_amd.inputs import AttnWorkload, make_attn_inputs
    say("[gpu] graph: attention forward")
    w = AttnWorkload("g", T=96, d=512, H=8, Hkv=4, dh=128, P=4, rank=2, seed=78, causal=True)
    inp = make_attn_inputs(w)
    dev = torch.device("cuda:0")
    attn = TspAttn(inp.w_q.to(dev), inp.w_k.to(dev), inp.w_v.to(dev), inp.w_o.to(dev), w.H, w.Hkv, w.P,
                   order=w.order(), causal=w.causal, T_max=w.T)
    x_all = inp.x_all.to(dev)
    for rho in range(w.P):
        if rho != w.rank:
            attn.project_kv(x_all[rho * w.T:(rho + 1) * w.T].contiguous(), rho)
    x = x_all[w.rank * w.T:(w.rank + 1) * w.T].contiguous()
    y = torch.empty(w.T, w.d, dtype=torch.float32, device=dev)
    g = _capture(lambda: attn.forward(x, w.rank, y=y))
    for rep in range(3):
        xn = make_attn_inputs(w.with_(seed=3000 + rep)).x_all[:w.T].to(dev)
        x.copy_(xn)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        ref = attn.forward(x, w.rank)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"attention replay {rep} differs from the eager forward"
    del g
    attn.close()
