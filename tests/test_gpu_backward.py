"""GPU parity of the backward (tsp_mlp_backward through the C ABI) against the
fp64 oracle's mlp_backward on the same seeded bf16 inputs.

Bar, for each of dX, dW_gate, dW_up, dW_down: ||dG||_2 / ||G*||_2 <= 3e-3 and
max|dG| <= 2e-2 * max|G*|, the forward's bf16 bar. Each gradient is one fp32-
accumulated product of bf16 inputs and one bf16-rounded intermediate (dG, dU
or H; dH stays fp32), so the forward's argument for its H rounding applies
(about 1.6e-3). A diagnostic bar against the oracle run with the same
intermediates rounded to bf16 (round_bf16=True) checks that nothing else
is wrong: 5e-4, as for the forward.

Small cases are compared in full (several tiles, ragged token counts, P up
to 8, ring orders); the Llama-shape workload runs at full size and is
compared on sampled token rows of dX and sampled hidden columns of the
weight gradients, which the oracle computes independently.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from sharded_transformer_mlp_amd.inputs import Workload, make_inputs, make_output_grad, sample_rows, workload

pytestmark = pytest.mark.gpu

EL2, EMAX, EL2_ROUNDED = 3e-3, 2e-2, 5e-4
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


def run_bwd(w: Workload, inp, dy, order=None, T_max=None, reuse=None):
    from sharded_transformer_mlp_amd.binding import TspMLP
    dev = torch.device("cuda:0")
    wg = None if inp.w_gate is None else inp.w_gate.to(dev)
    wu, wd = inp.w_up.to(dev), inp.w_down.to(dev)
    mlp = reuse or TspMLP(wg, wu, wd, w.P, order=w.order() if order is None else order, act=w.act,
                          T_max=T_max or inp.x.shape[0])
    # the handle owns its weights: the caller's copies are wiped before the
    # backward, which must not read them
    for t in (wg, wu, wd):
        if t is not None:
            t.fill_(float("nan"))
    g = mlp.backward(inp.x.to(dev).contiguous(), dy.to(dev).contiguous())
    torch.cuda.synchronize()
    return {k: None if v is None else v.cpu().double().numpy() for k, v in g.items()}, mlp


def check(name, got, ref, el2=EL2, emax=EMAX):
    """Every gradient's errors are printed before any is asserted."""
    errs = {}
    for k in KEYS:
        if ref[k] is None:
            assert got[k] is None, (name, k)
            continue
        d = got[k] - ref[k]
        e2 = float(np.linalg.norm(d) / np.linalg.norm(ref[k]))
        em = float(np.max(np.abs(d)) / np.max(np.abs(ref[k])))
        say(f"[gpu]   {name} {k}: e_L2 {e2:.2e} e_max {em:.2e}")
        errs[k] = (e2, em)
    for k, (e2, em) in errs.items():
        assert np.all(np.isfinite(got[k])), (name, k)
        assert e2 <= el2, f"{name} {k}: e_L2 {e2:.3e}"
        if emax is not None:
            assert em <= emax, f"{name} {k}: e_max {em:.3e}"


def oracle_bwd(w, inp, dy, order=None, round_bf16=False):
    return oracle.mlp_backward(_np(inp.x), _np(inp.w_gate), _np(inp.w_up), _np(inp.w_down), _np(dy), w.P,
                               w.order() if order is None else order, w.act, round_bf16=round_bf16)


SMALL = {
    "swiglu-T300-P2": Workload("b", T=300, d=256, f=1024, P=2, act="swiglu", dtype="bf16", seed=61, r0=1),
    "swiglu-T1-P2": Workload("b", T=1, d=256, f=1024, P=2, act="swiglu", dtype="bf16", seed=62),
    "swiglu-T513-P4": Workload("b", T=513, d=512, f=2048, P=4, act="swiglu", dtype="bf16", seed=63, r0=3),
    "swiglu-T100-P8": Workload("b", T=100, d=256, f=2048, P=8, act="swiglu", dtype="bf16", seed=64, r0=5),
    "gelu-T300-P2": Workload("b", T=300, d=256, f=1024, P=2, act="gelu_tanh", dtype="bf16", seed=65),
    "gelu-T64-P4": Workload("b", T=64, d=512, f=1024, P=4, act="gelu_tanh", dtype="bf16", seed=66, r0=2),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_backward_small_full_parity(name):
    w = SMALL[name]
    say(f"[gpu] backward parity {name}")
    inp, dy = make_inputs(w), make_output_grad(w)
    got, _ = run_bwd(w, inp, dy)
    check(name, got, oracle_bwd(w, inp, dy))
    check(name + " (bf16 intermediates)", got, oracle_bwd(w, inp, dy, round_bf16=True), EL2_ROUNDED, None)


def test_backward_ring_orders_and_reuse():
    """Any ring order gives the oracle's gradients; a handle's backward is
    bitwise reproducible and works at a smaller T than T_max."""
    w = Workload("o", T=200, d=256, f=2048, P=4, act="swiglu", dtype="bf16", seed=67)
    inp, dy = make_inputs(w), make_output_grad(w)
    ref = oracle_bwd(w, inp, dy)
    for order in ([0, 1, 2, 3], [2, 3, 0, 1], [3, 2, 1, 0], [1, 3, 0, 2]):
        say(f"[gpu] backward order {order}")
        got, mlp = run_bwd(w, inp, dy, order=order, T_max=300)
        check(f"order {order}", got, oracle_bwd(w, inp, dy, order=order))
        again, _ = run_bwd(w, inp, dy, reuse=mlp)
        for k in KEYS:
            assert np.array_equal(got[k], again[k]), k
        for k in KEYS:                                   # the order does not change the gradients beyond rounding
            d = np.linalg.norm(got[k] - ref[k]) / np.linalg.norm(ref[k])
            assert d <= EL2
        T = 37                                           # the first 37 tokens, same weights
        inpT = make_inputs(w)
        inpT.x = inp.x[:T].contiguous()
        dyT = dy[:T].contiguous()
        gT, _ = run_bwd(w, inpT, dyT, order=order, reuse=mlp)
        check(f"order {order} T={T}", gT, oracle_bwd(w, inpT, dyT, order=order))
        mlp.close()


@pytest.mark.parametrize("name", ["llama8b", "gelu"])
def test_backward_full_size_sampled(name):
    """The Llama-3-8B shape (T 4096, d 4096, f 14336, P 8, ring from 3) and the
    Megatron GeLU block (T 2048, d 4096, f 16384, P 2) at full size: dX on
    sampled token rows, the weight gradients on sampled hidden columns (both
    computed by the oracle on their own)."""
    w = workload(name)
    say(f"[gpu] backward {name} full size")
    inp, dy = make_inputs(w), make_output_grad(w)
    got, mlp = run_bwd(w, inp, dy)
    mlp.close()
    rows = sample_rows(w.T, 8, seed=91).numpy()
    X, dY = _np(inp.x), _np(dy)
    ref_rows = oracle.mlp_backward(X[rows], _np(inp.w_gate), _np(inp.w_up), _np(inp.w_down), dY[rows], w.P,
                                   w.order(), w.act)["dX"]
    cols = np.sort(np.random.default_rng(92).choice(w.f, 12, replace=False))
    refc = oracle.mlp_backward_columns(X, _np(inp.w_gate), _np(inp.w_up), _np(inp.w_down), dY, cols, w.act)
    pairs = {"dX rows": (got["dX"][rows], ref_rows), "dW_up cols": (got["dW_up"][:, cols], refc["dW_up"]),
             "dW_down rows": (got["dW_down"][cols, :], refc["dW_down"])}
    if w.act == "swiglu":
        pairs["dW_gate cols"] = (got["dW_gate"][:, cols], refc["dW_gate"])
    else:
        assert got["dW_gate"] is None and refc["dW_gate"] is None
    for name, (g, r) in pairs.items():
        e2 = float(np.linalg.norm(g - r) / np.linalg.norm(r))
        em = float(np.max(np.abs(g - r)) / np.max(np.abs(r)))
        say(f"[gpu]   {name}: e_L2 {e2:.2e} e_max {em:.2e}")
        assert np.all(np.isfinite(g)) and e2 <= EL2 and em <= EMAX, name


def test_backward_beyond_32bit_offsets():
    """T = 131072 tokens of d = 8192 (X, dY and their transposes 2 GiB each):
    every backward kernel then takes 64-bit addresses instead of 32-bit
    buffer offsets for its operands (dH, the recomputed gate/up product and
    the grouped weight-gradient launch). dX on sampled token rows (the first
    and the last included) and the weight gradients on sampled hidden
    columns, against the oracle."""
    w = Workload("big", T=131072, d=8192, f=1024, P=2, act="swiglu", dtype="bf16", seed=69, r0=1)
    assert w.T * w.d * 2 >= 1 << 31
    say("[gpu] backward T=131072 d=8192: generating inputs")
    inp, dy = make_inputs(w), make_output_grad(w)
    from sharded_transformer_mlp_amd.binding import TspMLP
    dev = torch.device("cuda:0")
    mlp = TspMLP(inp.w_gate.to(dev), inp.w_up.to(dev), inp.w_down.to(dev), w.P, order=w.order(), act=w.act,
                 T_max=w.T)
    say("[gpu] backward T=131072 d=8192 on the GPU")
    g = mlp.backward(inp.x.to(dev), dy.to(dev))
    torch.cuda.synchronize()
    rows = sample_rows(w.T, 16, seed=93, must_include=torch.tensor([0, 65536, w.T - 1])).numpy()
    cols = np.sort(np.random.default_rng(94).choice(w.f, 8, replace=False))
    for k in KEYS:
        assert bool(torch.isfinite(g[k]).all()), k
    got = {"dX rows": g["dX"][torch.from_numpy(rows).to(dev)].cpu().double().numpy(),
           "dW_gate cols": g["dW_gate"][:, cols].cpu().double().numpy(),
           "dW_up cols": g["dW_up"][:, cols].cpu().double().numpy(),
           "dW_down rows": g["dW_down"][cols, :].cpu().double().numpy()}
    mlp.close()
    del g
    say("[gpu] backward T=131072 d=8192: oracle on sampled rows and columns")
    X, dY = _np(inp.x), _np(dy)
    ref_rows = oracle.mlp_backward(X[rows], _np(inp.w_gate), _np(inp.w_up), _np(inp.w_down), dY[rows], w.P,
                                   w.order(), w.act)["dX"]
    refc = oracle.mlp_backward_columns(X, _np(inp.w_gate), _np(inp.w_up), _np(inp.w_down), dY, cols, w.act)
    pairs = {"dX rows": ref_rows, "dW_gate cols": refc["dW_gate"], "dW_up cols": refc["dW_up"],
             "dW_down rows": refc["dW_down"]}
    for name, r in pairs.items():
        gg = got[name]
        e2 = float(np.linalg.norm(gg - r) / np.linalg.norm(r))
        em = float(np.max(np.abs(gg - r)) / np.max(np.abs(r)))
        say(f"[gpu]   {name}: e_L2 {e2:.2e} e_max {em:.2e}")
        assert e2 <= EL2 and em <= EMAX, name


def test_backward_unsupported_and_invalid():
    from sharded_transformer_mlp_amd.binding import TSP_ERR_INVALID_ARG, TSP_ERR_UNSUPPORTED, TspError, TspMLP
    dev = torch.device("cuda:0")
    # F = 128 is not a multiple of 256
    w = Workload("u", T=16, d=256, f=1024, P=8, act="swiglu", dtype="bf16", seed=68)
    inp, dy = make_inputs(w), make_output_grad(w)
    say("[gpu] backward unsupported F=128")
    with pytest.raises(TspError) as e:
        run_bwd(w, inp, dy)
    assert e.value.status == TSP_ERR_UNSUPPORTED
    # fp32 handles have no backward
    wf = Workload("u", T=16, d=256, f=512, P=2, act="swiglu", dtype="f32", seed=69)
    inpf, dyf = make_inputs(wf), make_output_grad(wf)
    say("[gpu] backward fp32 handle")
    with pytest.raises(TspError) as e:
        run_bwd(wf, inpf, dyf)
    assert e.value.status == TSP_ERR_UNSUPPORTED
    # GeLU handle given a gate gradient (C ABI); T above T_max
    from sharded_transformer_mlp_amd.binding import lib
    wg = Workload("u", T=32, d=256, f=1024, P=2, act="gelu_tanh", dtype="bf16", seed=70)
    inpg, dyg = make_inputs(wg), make_output_grad(wg)
    mlp = TspMLP(None, inpg.w_up.to(dev), inpg.w_down.to(dev), wg.P, act=wg.act, T_max=32)
    x, d_y = inpg.x.to(dev), dyg.to(dev)
    dX = torch.empty(32, 256, dtype=torch.float32, device=dev)
    dW = [torch.empty(256, 1024, dtype=torch.float32, device=dev) for _ in range(2)]
    dWd = torch.empty(1024, 256, dtype=torch.float32, device=dev)
    st = lib().tsp_mlp_backward(mlp.handle, 32, x.data_ptr(), d_y.data_ptr(), dX.data_ptr(), dW[0].data_ptr(),
                                dW[1].data_ptr(), dWd.data_ptr(), None)
    assert st == TSP_ERR_INVALID_ARG
    st = lib().tsp_mlp_backward(mlp.handle, 32, x.data_ptr(), d_y.data_ptr(), dX.data_ptr(), None,
                                dW[1].data_ptr(), dW[1].data_ptr(), None)       # dW_down on dW_up
    assert st == TSP_ERR_INVALID_ARG
    big = make_inputs(wg.with_(T=33))
    with pytest.raises(TspError) as e:
        mlp.backward(big.x.to(dev), make_output_grad(wg.with_(T=33)).to(dev))
    assert e.value.status == TSP_ERR_INVALID_ARG
    # the handle still works afterwards
    g = mlp.backward(x, d_y)
    torch.cuda.synchronize()
    assert torch.isfinite(g["dX"]).all()
    mlp.close()
