"""GPU tests of the training pair that keeps the gate/up pre-activations
(tsp_mlp_forward_train, tsp_mlp_backward_saved through the C ABI).

The saved pre-activations are the accumulators of the same gate/up product
the backward would recompute, so the pair must reproduce the recomputing
path bit for bit: Y equal to tsp_mlp_forward's on the tiled path with gate/up
tile shape 0, every gradient equal to tsp_mlp_backward's. Y and the gradients
are also held to the oracle at the bf16 bar (as the forward and backward
tests), so that a shared mistake of both paths cannot pass.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from sharded_transformer_mlp_amd.inputs import Workload, make_inputs, make_output_grad, workload

pytestmark = pytest.mark.gpu

EL2, EMAX = 3e-3, 2e-2
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


def _np(t):
    return None if t is None else t.float().numpy()


def _handle(w, inp, T_max=None):
    from sharded_transformer_mlp_amd.binding import TspMLP
    dev = torch.device("cuda:0")
    wg = None if inp.w_gate is None else inp.w_gate.to(dev)
    return TspMLP(wg, inp.w_up.to(dev), inp.w_down.to(dev), w.P, order=w.order(), act=w.act,
                  T_max=T_max or inp.x.shape[0])


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b)), float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


CASES = {
    "swiglu-T300-P2": Workload("s", T=300, d=256, f=1024, P=2, act="swiglu", dtype="bf16", seed=161, r0=1),
    "swiglu-T1-P2": Workload("s", T=1, d=256, f=1024, P=2, act="swiglu", dtype="bf16", seed=162),
    "swiglu-T513-P4": Workload("s", T=513, d=512, f=2048, P=4, act="swiglu", dtype="bf16", seed=163, r0=3),
    "swiglu-T100-P8": Workload("s", T=100, d=256, f=2048, P=8, act="swiglu", dtype="bf16", seed=164, r0=5),
    "gelu-T300-P2": Workload("s", T=300, d=256, f=1024, P=2, act="gelu_tanh", dtype="bf16", seed=165),
    "gelu-T64-P4": Workload("s", T=64, d=512, f=1024, P=4, act="gelu_tanh", dtype="bf16", seed=166, r0=2),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_saved_pair_matches_recompute_and_oracle(name):
    w = CASES[name]
    say(f"[gpu] saved pair {name}")
    inp, dy = make_inputs(w), make_output_grad(w)
    dev = torch.device("cuda:0")
    x, d_y = inp.x.to(dev).contiguous(), dy.to(dev).contiguous()
    mlp = _handle(w, inp)
    assert mlp.saved_bytes(w.T) == w.P * -(-w.T // 256) * (2 if w.act == "swiglu" else 1) * (w.f // w.P // 256) \
        * 256 * 1024
    # stale contents must not leak into the result: Y and the saved buffer start as NaN
    saved = torch.full((mlp.saved_bytes(w.T) // 4,), float("nan"), dtype=torch.float32, device=dev)
    y_t = torch.full((w.T, w.d), float("nan"), dtype=torch.float32, device=dev)
    y_t, saved = mlp.forward_train(x, saved=saved, y=y_t)
    mlp.set_path("tiled")
    mlp.set_tiles(0, -1)
    y_f = mlp.forward(x)
    g_s = mlp.backward(x, d_y, saved=saved)
    g_r = mlp.backward(x, d_y)
    torch.cuda.synchronize()
    assert torch.equal(y_t, y_f), "forward_train's Y differs from the forward's"
    for k in KEYS:
        if g_r[k] is None:
            assert g_s[k] is None
            continue
        assert torch.equal(g_s[k], g_r[k]), f"{k} from saved pre-activations differs from the recomputed one"
    y_ref = oracle.mlp_forward(_np(inp.x), _np(inp.w_gate), _np(inp.w_up), _np(inp.w_down), w.P, w.order(), w.act)
    e2, em = _rel(y_t.cpu().double().numpy(), y_ref)
    say(f"[gpu]   Y e_L2 {e2:.2e} e_max {em:.2e}")
    assert e2 <= EL2 and em <= EMAX
    ref = oracle.mlp_backward(_np(inp.x), _np(inp.w_gate), _np(inp.w_up), _np(inp.w_down), _np(dy), w.P,
                              w.order(), w.act)
    for k in KEYS:
        if ref[k] is None:
            continue
        e2, em = _rel(g_s[k].cpu().double().numpy(), ref[k])
        say(f"[gpu]   {k} e_L2 {e2:.2e} e_max {em:.2e}")
        assert e2 <= EL2 and em <= EMAX, k
    mlp.close()


def test_saved_pair_smaller_T_on_one_handle():
    """Two trips in a row on one handle, the second with fewer tokens and the
    first trip's (larger) buffer: still equal to the recomputing path."""
    w = Workload("s", T=520, d=256, f=2048, P=4, act="swiglu", dtype="bf16", seed=167, r0=1)
    inp, dy = make_inputs(w), make_output_grad(w)
    dev = torch.device("cuda:0")
    mlp = _handle(w, inp)
    saved = None
    for T in (520, 77):
        say(f"[gpu] saved pair T={T} on one handle")
        x, d_y = inp.x[:T].to(dev).contiguous(), dy[:T].to(dev).contiguous()
        y_t, saved = mlp.forward_train(x, saved=saved)
        g_s = mlp.backward(x, d_y, saved=saved)
        g_r = mlp.backward(x, d_y)
        torch.cuda.synchronize()
        for k in KEYS:
            assert torch.equal(g_s[k], g_r[k]), (T, k)
        ref = oracle.mlp_backward(_np(inp.x[:T]), _np(inp.w_gate), _np(inp.w_up), _np(inp.w_down), _np(dy[:T]),
                                  w.P, w.order(), w.act)
        e2, _ = _rel(g_s["dX"].cpu().double().numpy(), ref["dX"])
        assert e2 <= EL2
    mlp.close()


def test_saved_pair_llama_shape():
    """The Llama-3-8B shape at full size: the saved pair against the
    recomputing path, bit for bit (the recomputing path's own oracle checks
    at this size are in test_gpu_backward)."""
    w = workload("llama8b")
    say("[gpu] saved pair llama8b full size")
    inp, dy = make_inputs(w), make_output_grad(w)
    dev = torch.device("cuda:0")
    x, d_y = inp.x.to(dev).contiguous(), dy.to(dev).contiguous()
    mlp = _handle(w, inp)
    y_t, saved = mlp.forward_train(x)
    y_f = mlp.forward(x)                                 # the automatic choice here is gate/up shape 0 too
    g_s = mlp.backward(x, d_y, saved=saved)
    g_r = mlp.backward(x, d_y)
    torch.cuda.synchronize()
    assert torch.equal(y_t, y_f)
    for k in KEYS:
        assert torch.equal(g_s[k], g_r[k]), k
    mlp.close()


def test_saved_pair_beyond_2gib():
    """The 70B shape (d 8192, f 28672, P 8) at a ragged T of 10000 tokens: a
    saved buffer of 40 token tiles x 56 MiB = 2.35 GB, past the 2 GiB that a
    32-bit offset reaches, against the recomputing path bit for bit."""
    w = workload("long70b").with_(T=10000)
    say("[gpu] saved pair 70b shape T=10000 (saved buffer beyond 2 GiB)")
    inp, dy = make_inputs(w), make_output_grad(w)
    dev = torch.device("cuda:0")
    x, d_y = inp.x.to(dev).contiguous(), dy.to(dev).contiguous()
    mlp = _handle(w, inp)
    assert mlp.saved_bytes(w.T) == 40 * 8 * 28 * 256 * 1024 > 2 ** 31
    y_t, saved = mlp.forward_train(x)
    y_f = mlp.forward(x)
    g_s = mlp.backward(x, d_y, saved=saved)
    g_r = mlp.backward(x, d_y)
    torch.cuda.synchronize()
    assert torch.equal(y_t, y_f)
    for k in KEYS:
        assert torch.equal(g_s[k], g_r[k]), k
    assert all(torch.isfinite(g_s[k]).all() for k in KEYS)
    mlp.close()


def test_saved_pair_errors():
    from sharded_transformer_mlp_amd.binding import TSP_ERR_INVALID_ARG, TSP_ERR_UNSUPPORTED, TspError, lib
    dev = torch.device("cuda:0")
    w = Workload("s", T=64, d=256, f=1024, P=2, act="swiglu", dtype="bf16", seed=168)
    inp, dy = make_inputs(w), make_output_grad(w)
    mlp = _handle(w, inp)
    x, d_y = inp.x.to(dev).contiguous(), dy.to(dev).contiguous()
    need = mlp.saved_bytes(64)
    say("[gpu] saved pair error paths")
    small = torch.empty(need - 16, dtype=torch.uint8, device=dev)
    with pytest.raises(TspError) as e:
        mlp.forward_train(x, saved=small)
    assert e.value.status == TSP_ERR_INVALID_ARG
    y = torch.empty(64, 256, dtype=torch.float32, device=dev)
    assert lib().tsp_mlp_forward_train(mlp.handle, 64, x.data_ptr(), y.data_ptr(), None, need, None) \
        == TSP_ERR_INVALID_ARG
    buf = torch.empty(need + 16, dtype=torch.uint8, device=dev)
    assert lib().tsp_mlp_forward_train(mlp.handle, 64, x.data_ptr(), y.data_ptr(), buf.data_ptr() + 4, need,
                                       None) == TSP_ERR_INVALID_ARG                 # misaligned
    _, saved = mlp.forward_train(x)
    with pytest.raises(TspError) as e:
        mlp.backward(x, d_y, saved=saved[:need - 16])
    assert e.value.status == TSP_ERR_INVALID_ARG
    # a gradient output on top of the saved buffer
    dX = torch.empty(64, 256, dtype=torch.float32, device=dev)
    dW = [torch.empty(256, 1024, dtype=torch.float32, device=dev) for _ in range(3)]
    st = lib().tsp_mlp_backward_saved(mlp.handle, 64, x.data_ptr(), d_y.data_ptr(), saved.data_ptr(), need,
                                      saved.data_ptr(), dW[0].data_ptr(), dW[1].data_ptr(), dW[2].data_ptr(), None)
    assert st == TSP_ERR_INVALID_ARG
    st = lib().tsp_mlp_backward_saved(mlp.handle, 64, x.data_ptr(), d_y.data_ptr(), None, need, dX.data_ptr(),
                                      dW[0].data_ptr(), dW[1].data_ptr(), dW[2].data_ptr(), None)
    assert st == TSP_ERR_INVALID_ARG
    mlp.close()
    # fp32 handles and shard widths that are not multiples of 256
    wf = Workload("s", T=16, d=256, f=512, P=2, act="swiglu", dtype="f32", seed=169)
    inpf = make_inputs(wf)
    mf = _handle(wf, inpf)
    with pytest.raises(TspError) as e:
        mf.forward_train(inpf.x.to(dev).contiguous(), saved=torch.empty(1 << 20, dtype=torch.uint8, device=dev))
    assert e.value.status == TSP_ERR_UNSUPPORTED
    mf.close()
    wn = Workload("s", T=16, d=256, f=1024, P=8, act="swiglu", dtype="bf16", seed=170)
    inpn = make_inputs(wn)
    mn = _handle(wn, inpn)
    with pytest.raises(TspError) as e:
        mn.forward_train(inpn.x.to(dev).contiguous(), saved=torch.empty(1 << 20, dtype=torch.uint8, device=dev))
    assert e.value.status == TSP_ERR_UNSUPPORTED
    mn.close()
