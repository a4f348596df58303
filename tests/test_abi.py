"""Host-side checks of the C ABI (no GPU needed, no compute call).

* the library loads and exports every function include/tsp_mlp.h and
  include/tsp_attn.h declare;
* argument validation returns the documented status before any HIP call.
"""
import ctypes
import os
import re

import pytest

from sharded_transformer_mlp_amd import binding as B

HEADERS = [os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", h) for h in ("tsp_mlp.h", "tsp_attn.h")]


def declared_functions():
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"\b(tsp_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("tsp_mlp_create", "tsp_mlp_forward", "tsp_mlp_destroy", "tsp_mlp_validate", "tsp_attn_create",
              "tsp_attn_project_kv", "tsp_attn_forward", "tsp_attn_destroy"):
        assert n in names
    assert set(names) == set(B.SIGNATURES), "binding and header disagree"


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    for n in declared_functions():
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_status_strings():
    lib = B.lib()
    assert lib.tsp_status_string(0) == b"ok"
    assert lib.tsp_status_string(2) == b"unsupported shape"
    assert lib.tsp_status_string(99) == b"unknown status"


OK, INV, UNS = B.TSP_OK, B.TSP_ERR_INVALID_ARG, B.TSP_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,want", [
    (dict(T_max=4096, d=4096, f=14336, P=8), OK),
    (dict(T_max=16, d=8192, f=28672, P=8, order=[3, 4, 5, 6, 7, 0, 1, 2]), OK),
    (dict(T_max=2048, d=4096, f=16384, P=2, act="gelu_tanh"), OK),
    (dict(T_max=3, d=5, f=12, P=4, dtype="f32"), OK),            # fp32 takes any shape
    (dict(T_max=0, d=64, f=128, P=2), INV),
    (dict(T_max=1, d=0, f=128, P=2), INV),
    (dict(T_max=1, d=64, f=0, P=2), INV),
    (dict(T_max=1, d=64, f=128, P=0), INV),
    (dict(T_max=1, d=64, f=192, P=5), INV),                        # P does not divide f
    (dict(T_max=1, d=64, f=128, P=2, act=7), INV),
    (dict(T_max=1, d=64, f=128, P=2, dtype=9), INV),
    (dict(T_max=1, d=64, f=256, P=4, order=[0, 1, 1, 3]), INV),    # not a permutation
    (dict(T_max=1, d=64, f=256, P=4, order=[0, 1, 2, 4]), INV),
    (dict(T_max=1, d=64, f=256, P=4, order=[0, 1, 2, -1]), INV),
    (dict(T_max=1, d=64, f=128, P=2, has_gate=False), INV),        # SwiGLU without gate
    (dict(T_max=1, d=64, f=128, P=2, act="gelu_tanh", has_gate=True), INV),
    (dict(T_max=1, d=96, f=128, P=2), UNS),                        # bf16 needs d % 64
    (dict(T_max=1, d=64, f=192, P=2), UNS),                        # bf16 needs F % 64
    (dict(T_max=1 << 31, d=64, f=128, P=2), INV),
])
def test_validate(kw, want):
    assert B.validate(**kw) == want


def test_create_rejects_before_touching_the_device():
    lib = B.lib()
    h = ctypes.c_void_p(1234)
    fake = ctypes.c_void_p(0x1000)
    # bad order: rejected by validation, *out cleared
    order = (ctypes.c_int32 * 2)(0, 0)
    st = lib.tsp_mlp_create(ctypes.byref(h), 16, 64, 128, 2, 0, 1,
                            ctypes.cast(order, ctypes.POINTER(ctypes.c_int32)), fake, fake, fake, None)
    assert st == INV and h.value is None
    assert b"permutation" in lib.tsp_last_error()
    # null weights
    st = lib.tsp_mlp_create(ctypes.byref(h), 16, 64, 128, 2, 0, 1, None, fake, None, fake, None)
    assert st == INV
    # misaligned weights
    odd = ctypes.c_void_p(0x1002)
    st = lib.tsp_mlp_create(ctypes.byref(h), 16, 64, 128, 2, 0, 1, None, fake, odd, fake, None)
    assert st == INV and b"aligned" in lib.tsp_last_error()
    # null out pointer
    assert lib.tsp_mlp_create(None, 16, 64, 128, 2, 0, 1, None, fake, fake, fake, None) == INV


def test_null_handle_calls():
    lib = B.lib()
    assert lib.tsp_mlp_destroy(None) == OK
    assert lib.tsp_mlp_forward(None, 1, None, None, None) == INV
    assert lib.tsp_mlp_set_path(None, 0) == INV
    assert lib.tsp_mlp_set_timing(None, 1) == INV
    n = ctypes.c_int32()
    assert lib.tsp_mlp_read_timing(None, 0, None, None, None, ctypes.byref(n)) == INV


def test_probes_reject_bad_arguments_before_any_hip_call():
    lib = B.lib()
    out = ctypes.c_double()
    assert lib.tsp_probe_hbm_read(1 << 30, 5, None, None) == INV
    assert lib.tsp_probe_hbm_read(1 << 20, 5, None, ctypes.byref(out)) == INV       # below 64 MiB
    assert lib.tsp_probe_hbm_read((1 << 30) + 4, 5, None, ctypes.byref(out)) == INV  # not 64 KiB aligned
    assert lib.tsp_probe_hbm_read(1 << 30, 0, None, ctypes.byref(out)) == INV
    assert b"reps" in lib.tsp_last_error()
    assert lib.tsp_probe_mfma_bf16(0, None, ctypes.byref(out)) == INV
    assert lib.tsp_probe_mfma_bf16(100, None, None) == INV


@pytest.mark.parametrize("args,want", [
    # T_max, d, H, Hkv, dh, P
    ((0, 4096, 32, 8, 128, 8), INV),
    ((16, 4096, 32, 6, 128, 8), INV),             # Hkv does not divide H
    ((16, 4096, 32, 8, 128, 3), INV),             # P does not divide Hkv
    ((16, 4096, 32, 8, 64, 8), UNS),              # dh != 128
    ((16, 4096, 24, 8, 128, 8), UNS),             # H/Hkv = 3
    ((16, 4096, 24, 8, 128, 8), UNS),
    ((16, 4096, 8, 8, 128, 8), UNS),              # H/P = 1 is odd
    ((16, 4000, 32, 8, 128, 8), UNS),             # d % 256
    ((1 << 21, 4096, 32, 8, 128, 8), UNS),        # context too long for 32-bit offsets
])
def test_attn_create_rejects_before_touching_the_device(args, want):
    lib = B.lib()
    h = ctypes.c_void_p(1234)
    fake = ctypes.c_void_p(0x1000)
    st = lib.tsp_attn_create(ctypes.byref(h), *args, 1, None, fake, fake, fake, fake, None)
    assert st == want and h.value is None, lib.tsp_last_error()


def test_attn_calls_reject_null_handle():
    lib = B.lib()
    assert lib.tsp_attn_forward(None, 16, 0, ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), None) == INV
    assert lib.tsp_attn_project_kv(None, 16, 0, ctypes.c_void_p(0x1000), None) == INV
    assert lib.tsp_attn_destroy(None) == OK


@pytest.mark.parametrize("case", ["up_cols", "gate_shape", "down_transposed", "gate_missing", "gate_on_gelu", "up_1d"])
def test_binding_rejects_mismatched_weight_shapes(case):
    """The C ABI takes bare pointers, so the binding checks every weight's
    shape against (d, f) before create: a wrong one would be read past its
    end by the packing kernels. CPU tensors suffice, the check comes first."""
    import torch
    d, f = 64, 256
    wg, wu, wd = torch.zeros(d, f), torch.zeros(d, f), torch.zeros(f, d)
    act = "swiglu"
    if case == "up_cols":
        wu = torch.zeros(d, f + 64)
    elif case == "gate_shape":
        wg = torch.zeros(d + 64, f)
    elif case == "down_transposed":
        wd = torch.zeros(d, f)
    elif case == "gate_missing":
        wg = None
    elif case == "gate_on_gelu":
        act = "gelu_tanh"
    elif case == "up_1d":
        wu = torch.zeros(d * f)
    with pytest.raises(ValueError):
        B.TspMLP(wg, wu, wd, 2, act=act, T_max=8)


@pytest.mark.parametrize("case", ["k_heads", "v_width", "o_transposed", "q_not_heads"])
def test_binding_rejects_mismatched_attention_shapes(case):
    import torch
    d, H, Hkv, dh = 256, 4, 2, 128
    wq, wk, wv, wo = (torch.zeros(d, H * dh), torch.zeros(d, Hkv * dh), torch.zeros(d, Hkv * dh),
                      torch.zeros(H * dh, d))
    if case == "k_heads":
        wk = torch.zeros(d, H * dh)
    elif case == "v_width":
        wv = torch.zeros(d, Hkv * dh - 8)
    elif case == "o_transposed":
        wo = torch.zeros(d, H * dh)
    elif case == "q_not_heads":
        wq = torch.zeros(d, H * dh + 8)
    with pytest.raises(ValueError):
        B.TspAttn(wq, wk, wv, wo, H, Hkv, 2, T_max=32)
