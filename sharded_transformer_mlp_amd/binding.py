"""ctypes binding over libtsp_mlp.so (argument marshalling only).

Every step of the forward runs in the library's HIP kernels; this module only
turns torch tensors into device pointers and the current torch stream into a
hipStream_t. It raises if the library is missing: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtsp_mlp.so")

TSP_OK, TSP_ERR_INVALID_ARG, TSP_ERR_UNSUPPORTED, TSP_ERR_OOM, TSP_ERR_HIP = range(5)
ACT = {"swiglu": 0, "gelu_tanh": 1}
DTYPE = {"f32": 0, "bf16": 1}
PATH = {"auto": 0, "tiled": 1, "skinny": 2}

# Every symbol the header declares, with its ctypes signature.
_i64, _i32, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
SIGNATURES = {
    "tsp_mlp_validate": (_i32, [_i64, _i64, _i64, _i32, _i32, _i32, ctypes.POINTER(_i32), _i32]),
    "tsp_mlp_create": (_i32, [ctypes.POINTER(_vp), _i64, _i64, _i64, _i32, _i32, _i32,
                              ctypes.POINTER(_i32), _vp, _vp, _vp, _vp]),
    "tsp_mlp_forward": (_i32, [_vp, _i64, _vp, _vp, _vp]),
    "tsp_mlp_forward_static": (_i32, [_vp, _i64, _vp, _vp, _vp]),
    "tsp_mlp_backward": (_i32, [_vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "tsp_mlp_saved_bytes": (_i32, [_vp, _i64, ctypes.POINTER(_i64)]),
    "tsp_mlp_forward_train": (_i32, [_vp, _i64, _vp, _vp, _vp, _i64, _vp]),
    "tsp_mlp_backward_saved": (_i32, [_vp, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp]),
    "tsp_mlp_destroy": (_i32, [_vp]),
    "tsp_mlp_set_path": (_i32, [_vp, _i32]),
    "tsp_mlp_set_tiles": (_i32, [_vp, _i32, _i32]),
    "tsp_mlp_sizes": (_i32, [_vp, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "tsp_mlp_set_timing": (_i32, [_vp, _i32]),
    "tsp_mlp_read_timing": (_i32, [_vp, _i32, _vp, ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(_i64), ctypes.POINTER(_i32)]),
    "tsp_attn_create": (_i32, [ctypes.POINTER(_vp), _i64, _i64, _i32, _i32, _i32, _i32, _i32,
                               ctypes.POINTER(_i32), _vp, _vp, _vp, _vp, _vp]),
    "tsp_attn_project_kv": (_i32, [_vp, _i64, _i32, _vp, _vp]),
    "tsp_attn_forward": (_i32, [_vp, _i64, _i32, _vp, _vp, _vp]),
    "tsp_attn_destroy": (_i32, [_vp]),
    "tsp_attn_set_timing": (_i32, [_vp, _i32]),
    "tsp_attn_read_timing": (_i32, [_vp, _i32, _vp, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(_i64), ctypes.POINTER(_i32)]),
    "tsp_attn_sizes": (_i32, [_vp, ctypes.POINTER(_i64), ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "tsp_probe_hbm_read": (_i32, [_i64, _i32, _vp, ctypes.POINTER(ctypes.c_double)]),
    "tsp_probe_mfma_bf16": (_i32, [_i32, _vp, ctypes.POINTER(ctypes.c_double)]),
    "tsp_status_string": (ctypes.c_char_p, [_i32]),
    "tsp_last_error": (ctypes.c_char_p, []),
}

_lib = None


class TspError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sharded_transformer_mlp_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != TSP_OK:
        raise TspError(status, lib().tsp_last_error().decode())


def _order_array(order: Optional[Sequence[int]]):
    if order is None:
        return None
    arr = (_i32 * len(order))(*[int(s) for s in order])
    return ctypes.cast(arr, ctypes.POINTER(_i32)), arr


def validate(T_max, d, f, P, act="swiglu", dtype="bf16", order=None, has_gate=None) -> int:
    """Pure host check (no HIP call); returns the status code."""
    a = ACT.get(act, act) if isinstance(act, str) else act
    t = DTYPE.get(dtype, dtype) if isinstance(dtype, str) else dtype
    if has_gate is None:
        has_gate = a == ACT["swiglu"]
    o = _order_array(order)
    return lib().tsp_mlp_validate(T_max, d, f, P, a, t, o[0] if o else None, int(bool(has_gate)))


def _stream_ptr(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check_shape(name, t, shape) -> None:
    if t is None or tuple(int(n) for n in t.shape) != tuple(shape):
        got = None if t is None else tuple(t.shape)
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {got}")


def probe_hbm_read(nbytes: int = 4 << 30, reps: int = 10, stream=None) -> float:
    """Sustained HBM read rate in GB/s (nontemporal 16-byte loads)."""
    out = ctypes.c_double()
    check(lib().tsp_probe_hbm_read(int(nbytes), int(reps), _stream_ptr(stream), ctypes.byref(out)))
    return out.value


def probe_mfma_bf16(iters: int = 4000, stream=None) -> float:
    """Sustained bf16 MFMA rate in TFLOP/s (16x16x32, pseudo-random operands)."""
    out = ctypes.c_double()
    check(lib().tsp_probe_mfma_bf16(int(iters), _stream_ptr(stream), ctypes.byref(out)))
    return out.value


class TspMLP:
    """One rank's sharded gated-MLP block on the GPU.

    w_gate / w_up: d x f, w_down: f x d, CUDA tensors of the storage dtype
    (torch.float32 or torch.bfloat16), row-major contiguous. w_gate is None
    for the GeLU block. ``order`` is the ring order (default 0..P-1).
    """

    def __init__(self, w_gate, w_up, w_down, P: int, order=None, act: str = "swiglu",
                 T_max: int = 1, stream=None):
        import torch
        # The C ABI cannot see buffer sizes: a weight of the wrong shape would
        # make the packing kernels read past its end, so shapes are checked here.
        if w_up.dim() != 2:
            raise ValueError("w_up must be a d x f matrix")
        self.d, self.f = (int(n) for n in w_up.shape)
        _check_shape("w_up", w_up, (self.d, self.f))
        if act == "swiglu":
            if w_gate is None:
                raise ValueError("the SwiGLU block needs w_gate")
            _check_shape("w_gate", w_gate, (self.d, self.f))
        elif w_gate is not None:
            raise ValueError("the GeLU block takes no w_gate")
        _check_shape("w_down", w_down, (self.f, self.d))
        if w_up.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("weights must be float32 or bfloat16")
        self.dtype = {torch.float32: "f32", torch.bfloat16: "bf16"}[w_up.dtype]
        self.tdtype = w_up.dtype
        self.P, self.act = P, act
        self.order = list(range(P)) if order is None else [int(s) for s in order]
        for w in (w_gate, w_up, w_down):
            if w is not None:
                if not (w.is_cuda and w.is_contiguous() and w.dtype == self.tdtype):
                    raise ValueError("weights must be contiguous CUDA tensors of one dtype")
        o = _order_array(self.order)
        h = _vp()
        self._stream = _stream_ptr(stream)
        check(lib().tsp_mlp_create(ctypes.byref(h), int(T_max), int(self.d), int(self.f), int(P),
                                   ACT[act], DTYPE[self.dtype], o[0],
                                   None if w_gate is None else w_gate.data_ptr(),
                                   w_up.data_ptr(), w_down.data_ptr(), self._stream))
        self.handle = h
        self.T_max = int(T_max)

    def set_path(self, path: str) -> None:
        check(lib().tsp_mlp_set_path(self.handle, PATH[path]))

    def set_tiles(self, gateup: int = -1, down: int = -1) -> None:
        check(lib().tsp_mlp_set_tiles(self.handle, int(gateup), int(down)))

    def forward(self, x, y=None, stream=None):
        import torch
        T = x.shape[0]
        if x.dtype != self.tdtype or not x.is_cuda or not x.is_contiguous() or x.shape[1] != self.d:
            raise ValueError("x must be a contiguous CUDA tensor T x d of the handle's dtype")
        if y is None:
            y = torch.empty(T, self.d, dtype=torch.float32, device=x.device)
        elif y.dtype != torch.float32 or not y.is_contiguous() or tuple(y.shape) != (T, self.d):
            raise ValueError("y must be a contiguous fp32 T x d tensor")
        check(lib().tsp_mlp_forward(self.handle, T, x.data_ptr(), y.data_ptr(), _stream_ptr(stream)))
        return y

    __call__ = forward

    def saved_bytes(self, T: int) -> int:
        """Bytes of the saved pre-activations forward_train keeps for T tokens."""
        n = _i64()
        check(lib().tsp_mlp_saved_bytes(self.handle, int(T), ctypes.byref(n)))
        return n.value

    def forward_train(self, x, saved=None, y=None, stream=None):
        """forward() that also keeps the gate/up pre-activations for
        backward(..., saved=...): returns (y, saved), saved a uint8 CUDA
        tensor of saved_bytes(T) bytes (allocated when not given)."""
        import torch
        T = x.shape[0]
        if x.dtype != self.tdtype or not x.is_cuda or not x.is_contiguous() or x.shape[1] != self.d:
            raise ValueError("x must be a contiguous CUDA tensor T x d of the handle's dtype")
        if y is None:
            y = torch.empty(T, self.d, dtype=torch.float32, device=x.device)
        elif y.dtype != torch.float32 or not y.is_contiguous() or tuple(y.shape) != (T, self.d):
            raise ValueError("y must be a contiguous fp32 T x d tensor")
        if saved is None:
            saved = torch.empty(self.saved_bytes(T), dtype=torch.uint8, device=x.device)
        elif not saved.is_cuda or not saved.is_contiguous():
            raise ValueError("saved must be a contiguous CUDA tensor")
        check(lib().tsp_mlp_forward_train(self.handle, T, x.data_ptr(), y.data_ptr(), saved.data_ptr(),
                                          saved.numel() * saved.element_size(), _stream_ptr(stream)))
        return y, saved

    def backward(self, x, dy, out=None, stream=None, saved=None):
        """Gradients for output gradient dy: {"dX", "dW_gate", "dW_up",
        "dW_down"} (fp32 CUDA tensors; dW_gate is None for GeLU) of the
        weights the handle holds. ``out``: a dict of that form to write into
        instead of new tensors. ``saved``: the pre-activations forward_train
        kept for the same x (no recomputation)."""
        import torch
        T = x.shape[0]
        for t in (x, dy):
            if t.dtype != self.tdtype or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != (T, self.d):
                raise ValueError("x and dy must be contiguous CUDA tensors T x d of the handle's dtype")
        dev = x.device
        gated = self.act == "swiglu"
        if out is not None:
            dX, dWg, dWu, dWd = out["dX"], out["dW_gate"], out["dW_up"], out["dW_down"]
            want = {"dX": (T, self.d), "dW_up": (self.d, self.f), "dW_down": (self.f, self.d)}
            if gated:
                want["dW_gate"] = (self.d, self.f)
            for k, shp in want.items():
                t = out[k]
                if t is None or t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != shp:
                    raise ValueError(f"out[{k!r}] must be a contiguous fp32 tensor of shape {shp}")
        else:
            dX = torch.empty(T, self.d, dtype=torch.float32, device=dev)
            dWg = torch.empty(self.d, self.f, dtype=torch.float32, device=dev) if gated else None
            dWu = torch.empty(self.d, self.f, dtype=torch.float32, device=dev)
            dWd = torch.empty(self.f, self.d, dtype=torch.float32, device=dev)
        ptr = lambda t: None if t is None else t.data_ptr()
        if saved is None:
            check(lib().tsp_mlp_backward(self.handle, T, x.data_ptr(), dy.data_ptr(), dX.data_ptr(), ptr(dWg),
                                         dWu.data_ptr(), dWd.data_ptr(), _stream_ptr(stream)))
        else:
            if not saved.is_cuda or not saved.is_contiguous():
                raise ValueError("saved must be a contiguous CUDA tensor")
            check(lib().tsp_mlp_backward_saved(self.handle, T, x.data_ptr(), dy.data_ptr(), saved.data_ptr(),
                                               saved.numel() * saved.element_size(), dX.data_ptr(), ptr(dWg),
                                               dWu.data_ptr(), dWd.data_ptr(), _stream_ptr(stream)))
        return {"dX": dX, "dW_gate": dWg, "dW_up": dWu, "dW_down": dWd}

    def sizes(self):
        p, w = _i64(), _i64()
        check(lib().tsp_mlp_sizes(self.handle, ctypes.byref(p), ctypes.byref(w)))
        return p.value, w.value

    def set_timing(self, enable: bool) -> None:
        check(lib().tsp_mlp_set_timing(self.handle, int(bool(enable))))

    def read_timing(self, max_kernels: int = 8):
        """{kernel name: (total ms, launches)} since the last read."""
        names = (ctypes.c_char * 64 * max_kernels)()
        ms = (ctypes.c_double * max_kernels)()
        n_l = (_i64 * max_kernels)()
        n = _i32()
        check(lib().tsp_mlp_read_timing(self.handle, max_kernels, names, ms, n_l, ctypes.byref(n)))
        return {bytes(names[i]).split(b"\0")[0].decode(): (ms[i], n_l[i]) for i in range(n.value)}

    def close(self) -> None:
        if getattr(self, "handle", None):
            check(lib().tsp_mlp_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class TspAttn:
    """One rank's attention block under TSP on the GPU (bf16).

    w_q: d x (H dh), w_k / w_v: d x (Hkv dh), w_o: (H dh) x d, contiguous
    bf16 CUDA tensors. ``order``: the head groups in the order the rank visits
    them (default 0..P-1). The handle owns the sequence-wide key/value
    context: ``project_kv(x, rank)`` fills rank ``rank``'s rows (what that
    rank computes and sends), ``forward(x, rank)`` computes rank ``rank``'s
    output, writing its own rows first.
    """

    def __init__(self, w_q, w_k, w_v, w_o, H: int, Hkv: int, P: int, order=None, causal: bool = True,
                 T_max: int = 8, stream=None):
        import torch
        # shapes first: the C ABI cannot see buffer sizes (see TspMLP)
        if w_q.dim() != 2 or H < 1 or Hkv < 1 or w_q.shape[1] % H:
            raise ValueError("w_q must be a d x (H dh) matrix")
        self.d = int(w_q.shape[0])
        self.H, self.Hkv, self.P = H, Hkv, P
        self.dh = int(w_q.shape[1]) // H
        _check_shape("w_k", w_k, (self.d, Hkv * self.dh))
        _check_shape("w_v", w_v, (self.d, Hkv * self.dh))
        _check_shape("w_o", w_o, (H * self.dh, self.d))
        for w in (w_q, w_k, w_v, w_o):
            if not (w.is_cuda and w.is_contiguous() and w.dtype == torch.bfloat16):
                raise ValueError("weights must be contiguous bf16 CUDA tensors")
        self.order = list(range(P)) if order is None else [int(s) for s in order]
        o = _order_array(self.order)
        h = _vp()
        self._stream = _stream_ptr(stream)
        check(lib().tsp_attn_create(ctypes.byref(h), int(T_max), int(self.d), int(H), int(Hkv), int(self.dh),
                                    int(P), int(bool(causal)), o[0], w_q.data_ptr(), w_k.data_ptr(),
                                    w_v.data_ptr(), w_o.data_ptr(), self._stream))
        self.handle = h
        self.T_max = int(T_max)

    def _check_x(self, x):
        import torch
        if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous() or x.shape[1] != self.d:
            raise ValueError("x must be a contiguous bf16 CUDA tensor T x d")

    def project_kv(self, x, rank: int, stream=None) -> None:
        self._check_x(x)
        check(lib().tsp_attn_project_kv(self.handle, x.shape[0], int(rank), x.data_ptr(), _stream_ptr(stream)))

    def forward(self, x, rank: int, y=None, stream=None):
        import torch
        self._check_x(x)
        T = x.shape[0]
        if y is None:
            y = torch.empty(T, self.d, dtype=torch.float32, device=x.device)
        elif y.dtype != torch.float32 or not y.is_contiguous() or tuple(y.shape) != (T, self.d):
            raise ValueError("y must be a contiguous fp32 T x d tensor")
        check(lib().tsp_attn_forward(self.handle, T, int(rank), x.data_ptr(), y.data_ptr(), _stream_ptr(stream)))
        return y

    def sizes(self):
        p, w, c = _i64(), _i64(), _i64()
        check(lib().tsp_attn_sizes(self.handle, ctypes.byref(p), ctypes.byref(w), ctypes.byref(c)))
        return p.value, w.value, c.value

    def set_timing(self, enable: bool) -> None:
        check(lib().tsp_attn_set_timing(self.handle, int(bool(enable))))

    def read_timing(self, max_kernels: int = 8):
        """{kernel name: (total ms, launches)} since the last read."""
        names = (ctypes.c_char * 64 * max_kernels)()
        ms = (ctypes.c_double * max_kernels)()
        n_l = (_i64 * max_kernels)()
        n = _i32()
        check(lib().tsp_attn_read_timing(self.handle, max_kernels, names, ms, n_l, ctypes.byref(n)))
        return {bytes(names[i]).split(b"\0")[0].decode(): (ms[i], n_l[i]) for i in range(n.value)}

    def close(self) -> None:
        if getattr(self, "handle", None):
            check(lib().tsp_attn_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
