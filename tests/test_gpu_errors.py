"""Error paths of the C ABI that need a device (forward-time checks,
allocation failure) and run-to-run / create-to-create reproducibility.
Every call here either succeeds or returns a status; none launches a kernel
on bad arguments."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from sharded_transformer_mlp_amd import binding as B
from sharded_transformer_mlp_amd.inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu

OK, INV, UNSUP, OOM = B.TSP_OK, B.TSP_ERR_INVALID_ARG, B.TSP_ERR_UNSUPPORTED, B.TSP_ERR_OOM


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def small():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = Workload("e", T=64, d=256, f=512, P=2, act="swiglu", dtype="bf16", seed=5)
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    mlp = B.TspMLP(inp.w_gate.to(dev), inp.w_up.to(dev), inp.w_down.to(dev), w.P, act=w.act, T_max=w.T)
    yield w, inp, mlp
    mlp.close()


def test_forward_rejects_bad_arguments(small):
    w, inp, mlp = small
    lib = B.lib()
    dev = torch.device("cuda:0")
    x = inp.x.to(dev)
    y = torch.empty(w.T, w.d, dtype=torch.float32, device=dev)
    say("[gpu] forward argument checks")
    h = mlp.handle
    assert lib.tsp_mlp_forward(h, -1, x.data_ptr(), y.data_ptr(), None) == INV
    assert lib.tsp_mlp_forward(h, w.T + 1, x.data_ptr(), y.data_ptr(), None) == INV
    assert lib.tsp_mlp_forward(h, w.T, None, y.data_ptr(), None) == INV
    assert lib.tsp_mlp_forward(h, w.T, x.data_ptr(), None, None) == INV
    assert lib.tsp_mlp_forward(h, w.T, x.data_ptr() + 2, y.data_ptr(), None) == INV     # misaligned X
    assert b"aligned" in lib.tsp_last_error()
    assert lib.tsp_mlp_forward(h, w.T, x.data_ptr(), y.data_ptr() + 4, None) == INV     # misaligned Y
    big = torch.empty(w.T * w.d * 4, dtype=torch.uint8, device=dev)
    assert lib.tsp_mlp_forward(h, 8, big.data_ptr(), big.data_ptr() + 256, None) == INV  # Y overlaps X
    assert b"overlaps" in lib.tsp_last_error()
    assert lib.tsp_mlp_set_tiles(h, 4, -1) == UNSUP
    assert lib.tsp_mlp_set_tiles(h, -2, -1) == INV
    assert lib.tsp_mlp_set_path(h, 9) == INV
    torch.cuda.synchronize()
    # the handle still works after every rejected call
    y2 = mlp.forward(x)
    torch.cuda.synchronize()
    assert torch.isfinite(y2).all()


def test_fp32_handle_rejects_bf16_only_settings():
    w = Workload("f", T=8, d=64, f=128, P=2, act="swiglu", dtype="f32", seed=6)
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    mlp = B.TspMLP(inp.w_gate.to(dev), inp.w_up.to(dev), inp.w_down.to(dev), w.P, act=w.act, T_max=w.T)
    lib = B.lib()
    say("[gpu] fp32 handle: bf16-only settings")
    assert lib.tsp_mlp_set_tiles(mlp.handle, 0, 0) == UNSUP
    mlp.set_path("skinny")
    with pytest.raises(B.TspError) as e:
        mlp.forward(inp.x.to(dev))
    assert e.value.status == UNSUP
    mlp.close()


def test_out_of_device_memory_is_reported_and_leaks_nothing():
    lib = B.lib()
    dev = torch.device("cuda:0")
    d, f, P = 64, 1 << 15, 2
    w = torch.zeros(d, f, dtype=torch.bfloat16, device=dev)
    wd = torch.zeros(f, d, dtype=torch.bfloat16, device=dev)
    free0, _ = torch.cuda.mem_get_info()
    say("[gpu] create with a 512 GiB workspace")
    h = ctypes.c_void_p(1)
    st = lib.tsp_mlp_create(ctypes.byref(h), 1 << 23, d, f, P, 0, 1, None, w.data_ptr(), w.data_ptr(),
                            wd.data_ptr(), None)
    assert st == OOM, (st, lib.tsp_last_error())
    assert h.value is None
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert abs(free1 - free0) < (64 << 20)          # the packed buffer was freed again


def test_two_handles_on_the_same_weights_agree_bitwise():
    w = Workload("r", T=300, d=512, f=2048, P=4, act="swiglu", dtype="bf16", seed=7, r0=2)
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    x = inp.x.to(dev)
    outs = []
    for k in range(2):
        say(f"[gpu] create #{k}")
        mlp = B.TspMLP(inp.w_gate.to(dev), inp.w_up.to(dev), inp.w_down.to(dev), w.P, order=w.order(),
                       act=w.act, T_max=w.T)
        ys = [mlp.forward(x).cpu() for _ in range(5)]
        torch.cuda.synchronize()
        for y in ys[1:]:
            assert torch.equal(y, ys[0])
        outs.append(ys[0])
        mlp.close()
    assert torch.equal(outs[0], outs[1])
