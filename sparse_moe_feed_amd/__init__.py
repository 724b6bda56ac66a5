"""Sparse Mixture-of-Experts feed-forward layer on AMD MI355X (gfx950).

Thin ctypes binding over ``libmoe.so`` (C ABI in ``include/moe.h``).  This
module only checks and marshals arguments: every step of the layer runs in the
library's HIP kernels.  PyTorch supplies device memory and the stream.  There
is no CPU fallback: if the library is missing, every call raises.

The layer (anatomy page on frontier-model-atlas, "Decoder microscope",
Feed-forward panel): router logits -> softmax -> top-k -> normalised selected
weights; SwiGLU experts; one shared expert scaled by its own sigmoid gate.
Expert weights are bfloat16/binary32 tensors, or MXFP4 tensors packed once by
``mx4_pack`` from row-major ``(codes, scales)`` uint8 pairs (``forward_mx4`` /
``experts_mx4``; both forms are defined in ``include/moe.h``).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_FLAG_ROUTER_EXACT, MOE_FLAG_ROUTER_SHORTLIST = 1, 2
ROUTERS = {None: 0, "auto": 0, "exact": MOE_FLAG_ROUTER_EXACT,
           "shortlist": MOE_FLAG_ROUTER_SHORTLIST}

EXPORTED = ("moe_workspace_size", "moe_workspace_query", "moe_route", "moe_forward",
            "moe_experts", "moe_mx4_packed_bytes", "moe_mx4_pack", "moe_forward_mx4",
            "moe_experts_mx4", "moe_rmsnorm", "moe_forward_prenorm",
            "moe_saved_bytes", "moe_forward_train", "moe_backward_workspace_size",
            "moe_backward", "moe_status_string",
            "moe_last_error", "moe_stage_events", "moe_read_probe", "moe_forward_noalloc")
MOE_WEIGHTS_DTYPE, MOE_WEIGHTS_MX4 = 0, 1


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}" + (f" ({detail})" if detail else ""))


class moe_desc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("d_expert", ctypes.c_int32),
                ("d_shared", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


class moe_workspace_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("logits", "gate", "counts", "offsets", "perm", "h", "h_shared", "y", "xnorm",
                 "total")]


_lib = None


def lib():
    """The loaded libmoe.so.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m sparse_moe_feed_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    dp = ctypes.POINTER(moe_desc)
    L.moe_workspace_size.argtypes = [dp, i64]
    L.moe_workspace_size.restype = sz
    L.moe_workspace_query.argtypes = [dp, i64, ctypes.POINTER(moe_workspace_layout)]
    L.moe_route.argtypes = [dp, i64, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_forward.argtypes = [dp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_experts.argtypes = [dp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_forward_mx4.argtypes = L.moe_forward.argtypes
    L.moe_experts_mx4.argtypes = L.moe_experts.argtypes
    L.moe_mx4_packed_bytes.argtypes = [i64, i64]
    L.moe_mx4_packed_bytes.restype = sz
    L.moe_mx4_pack.argtypes = [vp, vp, i64, i64, vp, vp]
    L.moe_rmsnorm.argtypes = [dp, i64, vp, vp, ctypes.c_float, vp, vp]
    L.moe_forward_prenorm.argtypes = [dp, i64, vp, vp, ctypes.c_float, ctypes.c_int32] + \
        L.moe_forward.argtypes[3:13] + [vp] + L.moe_forward.argtypes[13:]
    L.moe_backward_workspace_size.argtypes = [dp, i64]
    L.moe_backward_workspace_size.restype = sz
    L.moe_backward.argtypes = [dp, i64] + [vp] * 12 + [ctypes.c_float] + [vp] * 8 + [vp, sz, vp]
    L.moe_saved_bytes.argtypes = [dp, i64]
    L.moe_saved_bytes.restype = sz
    L.moe_forward_train.argtypes = [dp, i64] + [vp] * 12 + [sz, vp, sz, vp]
    for f in (L.moe_workspace_query, L.moe_route, L.moe_forward, L.moe_experts,
              L.moe_forward_mx4, L.moe_experts_mx4, L.moe_mx4_pack, L.moe_rmsnorm,
              L.moe_forward_prenorm, L.moe_backward, L.moe_forward_train):
        f.restype = ctypes.c_int
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_stage_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    L.moe_stage_events.restype = ctypes.c_int
    L.moe_read_probe.argtypes = [vp, sz, vp, vp]
    L.moe_read_probe.restype = ctypes.c_int
    L.moe_forward_noalloc.argtypes = [dp, i64] + [vp] * 11 + [vp]
    L.moe_forward_noalloc.restype = ctypes.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


@dataclass(frozen=True)
class Shape:
    d_model: int
    n_experts: int
    top_k: int
    d_expert: int
    d_shared: int
    dtype: torch.dtype
    router: Optional[str] = None   # None/"auto", "exact" or "shortlist"

    def desc(self) -> moe_desc:
        code = {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}.get(self.dtype)
        if code is None:
            raise TypeError(f"unsupported dtype {self.dtype}")
        return moe_desc(self.d_model, self.n_experts, self.top_k, self.d_expert,
                        self.d_shared, code, ROUTERS[self.router])


def workspace_size(shape: Shape, T: int) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(shape.desc()), T))


def workspace_layout(shape: Shape, T: int) -> moe_workspace_layout:
    lay = moe_workspace_layout()
    st = lib().moe_workspace_query(ctypes.byref(shape.desc()), T, ctypes.byref(lay))
    if st != MOE_OK:
        raise MoEError(st, "moe_workspace_query")
    return lay


def alloc_workspace(shape: Shape, T: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(workspace_size(shape, T), 1), dtype=torch.uint8, device=device)


STAGES = ("route", "permute", "gate_up", "down", "combine")

_hip = None


def _hip_rt():
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so")
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                          ctypes.c_void_p]
        h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        for f in (h.hipEventCreateWithFlags, h.hipEventElapsedTime, h.hipEventSynchronize,
                  h.hipEventDestroy):
            f.restype = ctypes.c_int
        _hip = h
    return _hip


class HipEvent:
    """A raw hipEvent_t with timing, for the library's stage marks."""

    def __init__(self):
        self.handle = ctypes.c_void_p()
        if _hip_rt().hipEventCreateWithFlags(ctypes.byref(self.handle), 0) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        _hip_rt().hipEventSynchronize(end.handle)
        if _hip_rt().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle) != 0:
            raise RuntimeError("hipEventElapsedTime failed (event not recorded?)")
        return float(ms.value)

    def __del__(self):
        if self.handle and _hip is not None:
            _hip.hipEventDestroy(self.handle)


def stage_events(events):
    """Have the next forward/experts call on this thread record the given
    HipEvent objects (len <= 8) at its stage boundaries: index 0 at the start,
    then after routing, permutation, gate/up, down and combine."""
    arr = (ctypes.c_void_p * max(1, len(events)))(*[e.handle for e in events])
    st = lib().moe_stage_events(arr, len(events))
    if st != MOE_OK:
        raise MoEError(st, "moe_stage_events")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, shape=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(st: int, where: str):
    if st != MOE_OK:
        raise MoEError(st, where, lib().moe_last_error().decode() if st == MOE_ERR_HIP else "")


def shape_of(x, w_gate_up, k, w_sh_gate_up=None, router=None) -> Shape:
    E, twoF, d = w_gate_up.shape
    Fs = 0 if w_sh_gate_up is None else w_sh_gate_up.shape[0] // 2
    return Shape(d, E, k, twoF // 2, Fs, x.dtype, router)


def route(x, w_router, k, bias=None, sh_gate=None, ws=None, router=None):
    """(topk_idx int32 [T,k], topk_w float32 [T,k], s float32 [T] or None)."""
    T, d = x.shape
    E = w_router.shape[0]
    shape = Shape(d, E, k, 64, 0, x.dtype, router)
    _dev(x, "x"), _dev(w_router, "w_router", x.dtype, (E, d))
    _dev(bias, "router_bias", torch.float32, (E,)), _dev(sh_gate, "sh_gate", x.dtype, (d,))
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    s = torch.empty((T,), dtype=torch.float32, device=x.device) if sh_gate is not None else None
    ws = alloc_workspace(shape, T, x.device) if ws is None else ws
    st = lib().moe_route(ctypes.byref(shape.desc()), T, _ptr(x), _ptr(w_router), _ptr(bias),
                         _ptr(sh_gate), _ptr(idx), _ptr(w), _ptr(s), _ptr(ws), ws.numel(),
                         _stream())
    _check(st, "moe_route")
    return idx, w, s


def forward(x, w_router, w_gate_up, w_down, k, w_sh_gate_up=None, w_sh_down=None,
            sh_gate=None, bias=None, out=None, topk_idx=None, topk_w=None, ws=None, router=None):
    """The whole layer.  Returns (out float32 [T,d], topk_idx, topk_w)."""
    T, d = x.shape
    shape = shape_of(x, w_gate_up, k, w_sh_gate_up, router)
    E, F, Fs = shape.n_experts, shape.d_expert, shape.d_shared
    _dev(x, "x"), _dev(w_router, "w_router", x.dtype, (E, d))
    _dev(w_gate_up, "w_gate_up", x.dtype), _dev(w_down, "w_down", x.dtype, (E, d, F))
    if Fs:
        _dev(w_sh_gate_up, "w_sh_gate_up", x.dtype, (2 * Fs, d))
        _dev(w_sh_down, "w_sh_down", x.dtype, (d, Fs)), _dev(sh_gate, "sh_gate", x.dtype, (d,))
    _dev(bias, "router_bias", torch.float32, (E,))
    out = torch.empty((T, d), dtype=torch.float32, device=x.device) if out is None else out
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=x.device) if topk_idx is None else topk_idx
    topk_w = torch.empty((T, k), dtype=torch.float32, device=x.device) if topk_w is None else topk_w
    _dev(out, "out", torch.float32, (T, d)), _dev(topk_idx, "topk_idx", torch.int32, (T, k))
    _dev(topk_w, "topk_w", torch.float32, (T, k))
    ws = alloc_workspace(shape, T, x.device) if ws is None else ws
    st = lib().moe_forward(ctypes.byref(shape.desc()), T, _ptr(x), _ptr(w_router), _ptr(bias),
                           _ptr(w_gate_up), _ptr(w_down), _ptr(w_sh_gate_up), _ptr(w_sh_down),
                           _ptr(sh_gate), _ptr(out), _ptr(topk_idx), _ptr(topk_w), _ptr(ws),
                           ws.numel(), _stream())
    _check(st, "moe_forward")
    return out, topk_idx, topk_w


NOALLOC_SCRATCH_BYTES = 100 << 20


def forward_noalloc(x, w_router, w_gate_up, w_down, k, w_sh_gate_up=None, w_sh_down=None,
                    sh_gate=None, bias=None, out=None, topk_idx=None, topk_w=None):
    """The whole layer through moe_forward_noalloc: the workspace is the
    library's static device array (100 MiB per GPU), so the call itself
    allocates no device memory.  Calls that may overlap on one GPU race on
    that array.  Returns (out, topk_idx, topk_w); the outputs are allocated
    here when not given."""
    T, d = x.shape
    shape = shape_of(x, w_gate_up, k, w_sh_gate_up)
    E, F, Fs = shape.n_experts, shape.d_expert, shape.d_shared
    _dev(x, "x"), _dev(w_router, "w_router", x.dtype, (E, d))
    _dev(w_gate_up, "w_gate_up", x.dtype), _dev(w_down, "w_down", x.dtype, (E, d, F))
    if Fs:
        _dev(w_sh_gate_up, "w_sh_gate_up", x.dtype, (2 * Fs, d))
        _dev(w_sh_down, "w_sh_down", x.dtype, (d, Fs)), _dev(sh_gate, "sh_gate", x.dtype, (d,))
    _dev(bias, "router_bias", torch.float32, (E,))
    out = torch.empty((T, d), dtype=torch.float32, device=x.device) if out is None else out
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=x.device) if topk_idx is None else topk_idx
    topk_w = torch.empty((T, k), dtype=torch.float32, device=x.device) if topk_w is None else topk_w
    _dev(out, "out", torch.float32, (T, d)), _dev(topk_idx, "topk_idx", torch.int32, (T, k))
    _dev(topk_w, "topk_w", torch.float32, (T, k))
    st = lib().moe_forward_noalloc(ctypes.byref(shape.desc()), T, _ptr(x), _ptr(w_router),
                                   _ptr(bias), _ptr(w_gate_up), _ptr(w_down), _ptr(w_sh_gate_up),
                                   _ptr(w_sh_down), _ptr(sh_gate), _ptr(out), _ptr(topk_idx),
                                   _ptr(topk_w), _stream())
    if st == MOE_ERR_WORKSPACE:
        raise MoEError(st, "moe_forward_noalloc", lib().moe_last_error().decode())
    _check(st, "moe_forward_noalloc")
    return out, topk_idx, topk_w


def experts(x, w_gate_up, w_down, topk_idx, topk_w, w_sh_gate_up=None, w_sh_down=None,
            sh_gate=None, out=None, ws=None):
    """Expert stage with the routing given (topk_idx/topk_w are inputs)."""
    T, d = x.shape
    k = topk_idx.shape[1]
    shape = shape_of(x, w_gate_up, k, w_sh_gate_up)
    E, F, Fs = shape.n_experts, shape.d_expert, shape.d_shared
    _dev(x, "x"), _dev(w_gate_up, "w_gate_up", x.dtype), _dev(w_down, "w_down", x.dtype, (E, d, F))
    _dev(topk_idx, "topk_idx", torch.int32, (T, k)), _dev(topk_w, "topk_w", torch.float32, (T, k))
    if Fs:
        _dev(w_sh_gate_up, "w_sh_gate_up", x.dtype, (2 * Fs, d))
        _dev(w_sh_down, "w_sh_down", x.dtype, (d, Fs)), _dev(sh_gate, "sh_gate", x.dtype, (d,))
    out = torch.empty((T, d), dtype=torch.float32, device=x.device) if out is None else out
    _dev(out, "out", torch.float32, (T, d))
    ws = alloc_workspace(shape, T, x.device) if ws is None else ws
    st = lib().moe_experts(ctypes.byref(shape.desc()), T, _ptr(x), _ptr(w_gate_up), _ptr(w_down),
                           _ptr(w_sh_gate_up), _ptr(w_sh_down), _ptr(sh_gate), _ptr(topk_idx),
                           _ptr(topk_w), _ptr(out), _ptr(ws), ws.numel(), _stream())
    _check(st, "moe_experts")
    return out


BACKWARD_STAGES = ("logits", "gate_up_g", "swiglu_router", "dx_rows", "dw_gate_up", "dw_down",
                   "router_combine")


def backward_workspace_size(shape: Shape, T: int) -> int:
    return int(lib().moe_backward_workspace_size(ctypes.byref(shape.desc()), T))


def saved_bytes(shape: Shape, T: int) -> int:
    return int(lib().moe_saved_bytes(ctypes.byref(shape.desc()), T))


def forward_train(x, w_router, w_gate_up, w_down, k, w_sh_gate_up=None, w_sh_down=None,
                  sh_gate=None, bias=None, out=None, topk_idx=None, topk_w=None, saved=None,
                  ws=None, router=None):
    """The training forward: (out, topk_idx, topk_w, saved), saved being the
    gate/up pre-activations moe_backward can take instead of recomputing them."""
    T, d = x.shape
    shape = shape_of(x, w_gate_up, k, w_sh_gate_up, router)
    E, F, Fs = shape.n_experts, shape.d_expert, shape.d_shared
    _dev(x, "x"), _dev(w_router, "w_router", x.dtype, (E, d))
    _dev(w_gate_up, "w_gate_up", x.dtype), _dev(w_down, "w_down", x.dtype, (E, d, F))
    if Fs:
        _dev(w_sh_gate_up, "w_sh_gate_up", x.dtype, (2 * Fs, d))
        _dev(w_sh_down, "w_sh_down", x.dtype, (d, Fs)), _dev(sh_gate, "sh_gate", x.dtype, (d,))
    _dev(bias, "router_bias", torch.float32, (E,))
    out = torch.empty((T, d), dtype=torch.float32, device=x.device) if out is None else out
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=x.device) if topk_idx is None else topk_idx
    topk_w = torch.empty((T, k), dtype=torch.float32, device=x.device) if topk_w is None else topk_w
    nbytes = saved_bytes(shape, T)
    saved = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device) if saved is None else saved
    _dev(out, "out", torch.float32, (T, d)), _dev(topk_idx, "topk_idx", torch.int32, (T, k))
    _dev(topk_w, "topk_w", torch.float32, (T, k)), _dev(saved, "saved")
    ws = alloc_workspace(shape, T, x.device) if ws is None else ws
    st = lib().moe_forward_train(ctypes.byref(shape.desc()), T, _ptr(x), _ptr(w_router),
                                 _ptr(bias), _ptr(w_gate_up), _ptr(w_down), _ptr(w_sh_gate_up),
                                 _ptr(w_sh_down), _ptr(sh_gate), _ptr(out), _ptr(topk_idx),
                                 _ptr(topk_w), _ptr(saved), saved.numel() * saved.element_size(),
                                 _ptr(ws), ws.numel(), _stream())
    _check(st, "moe_forward_train")
    return out, topk_idx, topk_w, saved


def backward(x, w_router, w_gate_up, w_down, topk_idx, topk_w, dout, w_sh_gate_up=None,
             w_sh_down=None, sh_gate=None, bias=None, aux_coef=0.0, ws=None, grads=None,
             aux_loss=None, saved=None):
    """Gradients of sum(dout * out) + aux_coef * E * sum_e f_e P_e with the
    routing given.  Returns a dict: dx (float32 [T,d]), dw_router,
    dw_gate_up, dw_down, dw_sh_gate_up, dw_sh_down, dsh_gate (x.dtype; the
    shared ones None without a shared expert) and aux_loss (float32 [1]).
    grads may pass preallocated outputs under the same names; saved is the
    buffer forward_train returned for this x and routing (else the gate/up
    pre-activations are recomputed)."""
    T, d = x.shape
    k = topk_idx.shape[1]
    shape = shape_of(x, w_gate_up, k, w_sh_gate_up)
    E, F, Fs = shape.n_experts, shape.d_expert, shape.d_shared
    dt = x.dtype
    _dev(x, "x"), _dev(w_router, "w_router", dt, (E, d))
    _dev(w_gate_up, "w_gate_up", dt, (E, 2 * F, d)), _dev(w_down, "w_down", dt, (E, d, F))
    _dev(topk_idx, "topk_idx", torch.int32, (T, k)), _dev(topk_w, "topk_w", torch.float32, (T, k))
    _dev(dout, "dout", torch.float32, (T, d)), _dev(bias, "router_bias", torch.float32, (E,))
    if Fs:
        _dev(w_sh_gate_up, "w_sh_gate_up", dt, (2 * Fs, d))
        _dev(w_sh_down, "w_sh_down", dt, (d, Fs)), _dev(sh_gate, "sh_gate", dt, (d,))
    shapes = dict(dx=((T, d), torch.float32), dw_router=((E, d), dt),
                  dw_gate_up=((E, 2 * F, d), dt), dw_down=((E, d, F), dt),
                  dw_sh_gate_up=((2 * Fs, d), dt), dw_sh_down=((d, Fs), dt), dsh_gate=((d,), dt))
    g = {} if grads is None else dict(grads)
    for n, (shp, ty) in shapes.items():
        if Fs == 0 and n in ("dw_sh_gate_up", "dw_sh_down", "dsh_gate"):
            g[n] = None
            continue
        if g.get(n) is None:
            g[n] = torch.empty(shp, dtype=ty, device=x.device)
        _dev(g[n], n, ty, shp)
    aux = torch.empty(1, dtype=torch.float32, device=x.device) if aux_loss is None else aux_loss
    _dev(aux, "aux_loss", torch.float32, (1,))
    if ws is None:
        ws = torch.empty(max(backward_workspace_size(shape, T), 1), dtype=torch.uint8,
                         device=x.device)
    st = lib().moe_backward(
        ctypes.byref(shape.desc()), T, _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate_up),
        _ptr(w_down), _ptr(w_sh_gate_up), _ptr(w_sh_down), _ptr(sh_gate), _ptr(topk_idx),
        _ptr(topk_w), _ptr(dout), _ptr(saved), ctypes.c_float(aux_coef), _ptr(g["dx"]),
        _ptr(g["dw_router"]),
        _ptr(g["dw_gate_up"]), _ptr(g["dw_down"]), _ptr(g["dw_sh_gate_up"]),
        _ptr(g["dw_sh_down"]), _ptr(g["dsh_gate"]), _ptr(aux), _ptr(ws), ws.numel(), _stream())
    _check(st, "moe_backward")
    g["aux_loss"] = aux
    return g


@dataclass(frozen=True)
class MX4Tensor:
    """A packed MXFP4 tensor of logical shape [rows, K] in device memory."""
    data: torch.Tensor
    rows: int
    K: int


def mx4_pack(codes: torch.Tensor, scales: torch.Tensor) -> MX4Tensor:
    """Pack a row-major MXFP4 tensor (codes uint8 [..., K/2], scales uint8
    [..., K/32]; leading dimensions are rows) into the layer's tiled form."""
    K = codes.shape[-1] * 2
    rows = codes.numel() // max(1, codes.shape[-1])
    _dev(codes, "codes", torch.uint8), _dev(scales, "scales", torch.uint8,
                                          tuple(codes.shape[:-1]) + (K // 32,))
    nbytes = int(lib().moe_mx4_packed_bytes(rows, K))
    if nbytes == 0:
        raise ValueError(f"MXFP4 packing needs rows % 16 == 0 and K % 128 == 0 (got {rows} x {K})")
    out = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    _check(lib().moe_mx4_pack(_ptr(codes), _ptr(scales), rows, K, _ptr(out), _stream()),
           "moe_mx4_pack")
    return MX4Tensor(out, rows, K)


def _mx4_dims(d, gu, dn, sgu, sdn):
    """(E, F, Fs) of a layer from its packed tensors, shapes checked."""
    for t, n in ((gu, "w_gate_up"), (dn, "w_down"), (sgu, "w_sh_gate_up"), (sdn, "w_sh_down")):
        if t is not None and not isinstance(t, MX4Tensor):
            raise TypeError(f"{n} must be an MX4Tensor (see mx4_pack)")
    F = dn.K
    E = dn.rows // d
    Fs = 0 if sdn is None else sdn.K
    ok = dn.rows == E * d and gu.rows == E * 2 * F and gu.K == d
    if Fs:
        ok = ok and sgu is not None and sgu.rows == 2 * Fs and sgu.K == d and sdn.rows == d
    if not ok:
        raise ValueError("MXFP4 tensor shapes do not form one layer")
    return E, F, Fs


def _mx4_ptrs(*ts):
    return [None if t is None else _ptr(t.data) for t in ts]


def forward_mx4(x, w_router, gu, dn, k, sgu=None, sdn=None, sh_gate=None, bias=None, out=None,
                topk_idx=None, topk_w=None, ws=None, router=None):
    """The whole layer with packed MXFP4 expert weights (MX4Tensor each).
    Returns (out float32 [T,d], topk_idx, topk_w)."""
    T, d = x.shape
    E, F, Fs = _mx4_dims(d, gu, dn, sgu, sdn)
    shape = Shape(d, E, k, F, Fs, x.dtype, router)
    _dev(x, "x", torch.bfloat16), _dev(w_router, "w_router", x.dtype, (E, d))
    if Fs:
        _dev(sh_gate, "sh_gate", x.dtype, (d,))
    _dev(bias, "router_bias", torch.float32, (E,))
    out = torch.empty((T, d), dtype=torch.float32, device=x.device) if out is None else out
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=x.device) if topk_idx is None else topk_idx
    topk_w = torch.empty((T, k), dtype=torch.float32, device=x.device) if topk_w is None else topk_w
    _dev(out, "out", torch.float32, (T, d)), _dev(topk_idx, "topk_idx", torch.int32, (T, k))
    _dev(topk_w, "topk_w", torch.float32, (T, k))
    ws = alloc_workspace(shape, T, x.device) if ws is None else ws
    st = lib().moe_forward_mx4(ctypes.byref(shape.desc()), T, _ptr(x), _ptr(w_router), _ptr(bias),
                               *_mx4_ptrs(gu, dn, sgu, sdn), _ptr(sh_gate), _ptr(out),
                               _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws.numel(), _stream())
    _check(st, "moe_forward_mx4")
    return out, topk_idx, topk_w


def experts_mx4(x, gu, dn, topk_idx, topk_w, sgu=None, sdn=None, sh_gate=None, out=None,
                ws=None):
    """Expert stage with packed MXFP4 expert weights and the routing given."""
    T, d = x.shape
    k = topk_idx.shape[1]
    E, F, Fs = _mx4_dims(d, gu, dn, sgu, sdn)
    shape = Shape(d, E, k, F, Fs, x.dtype)
    _dev(x, "x", torch.bfloat16)
    _dev(topk_idx, "topk_idx", torch.int32, (T, k)), _dev(topk_w, "topk_w", torch.float32, (T, k))
    if Fs:
        _dev(sh_gate, "sh_gate", x.dtype, (d,))
    out = torch.empty((T, d), dtype=torch.float32, device=x.device) if out is None else out
    _dev(out, "out", torch.float32, (T, d))
    ws = alloc_workspace(shape, T, x.device) if ws is None else ws
    st = lib().moe_experts_mx4(ctypes.byref(shape.desc()), T, _ptr(x),
                               *_mx4_ptrs(gu, dn, sgu, sdn), _ptr(sh_gate), _ptr(topk_idx),
                               _ptr(topk_w), _ptr(out), _ptr(ws), ws.numel(), _stream())
    _check(st, "moe_experts_mx4")
    return out


def rmsnorm(h, norm_weight, eps=1e-6, out=None):
    """Pre-FFN RMSNorm of h [T, d] (fixed binary32 order, rounded to h's
    dtype; include/moe.h)."""
    T, d = h.shape
    shape = Shape(d, 1, 1, 64, 0, h.dtype)
    _dev(h, "h"), _dev(norm_weight, "norm_weight", h.dtype, (d,))
    out = torch.empty_like(h) if out is None else out
    _dev(out, "out", h.dtype, (T, d))
    _check(lib().moe_rmsnorm(ctypes.byref(shape.desc()), T, _ptr(h), _ptr(norm_weight),
                             ctypes.c_float(eps), _ptr(out), _stream()), "moe_rmsnorm")
    return out


def forward_prenorm(h, norm_weight, w_router, w_gate_up, w_down, k, w_sh_gate_up=None,
                    w_sh_down=None, sh_gate=None, bias=None, eps=1e-6, out=None, topk_idx=None,
                    topk_w=None, ws=None, router=None, resid=None):
    """The layer on RMSNorm(h), one call.  Expert weights are tensors in h's
    dtype, or MX4Tensor (packed MXFP4).  resid (optional float32 [T, d]) is
    updated in place to resid + out by the same call.  Returns (out,
    topk_idx, topk_w)."""
    T, d = h.shape
    mx4 = isinstance(w_gate_up, MX4Tensor)
    if mx4:
        E, F, Fs = _mx4_dims(d, w_gate_up, w_down, w_sh_gate_up, w_sh_down)
        shape = Shape(d, E, k, F, Fs, h.dtype, router)
        ptrs = _mx4_ptrs(w_gate_up, w_down, w_sh_gate_up, w_sh_down)
    else:
        shape = shape_of(h, w_gate_up, k, w_sh_gate_up, router)
        E, F, Fs = shape.n_experts, shape.d_expert, shape.d_shared
        _dev(w_gate_up, "w_gate_up", h.dtype), _dev(w_down, "w_down", h.dtype, (E, d, F))
        if Fs:
            _dev(w_sh_gate_up, "w_sh_gate_up", h.dtype, (2 * Fs, d))
            _dev(w_sh_down, "w_sh_down", h.dtype, (d, Fs))
        ptrs = [_ptr(w_gate_up), _ptr(w_down), _ptr(w_sh_gate_up), _ptr(w_sh_down)]
    _dev(h, "h"), _dev(norm_weight, "norm_weight", h.dtype, (d,))
    _dev(w_router, "w_router", h.dtype, (E, d)), _dev(bias, "router_bias", torch.float32, (E,))
    if Fs:
        _dev(sh_gate, "sh_gate", h.dtype, (d,))
    out = torch.empty((T, d), dtype=torch.float32, device=h.device) if out is None else out
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=h.device) if topk_idx is None else topk_idx
    topk_w = torch.empty((T, k), dtype=torch.float32, device=h.device) if topk_w is None else topk_w
    _dev(out, "out", torch.float32, (T, d)), _dev(topk_idx, "topk_idx", torch.int32, (T, k))
    _dev(topk_w, "topk_w", torch.float32, (T, k)), _dev(resid, "resid", torch.float32, (T, d))
    ws = alloc_workspace(shape, T, h.device) if ws is None else ws
    st = lib().moe_forward_prenorm(ctypes.byref(shape.desc()), T, _ptr(h), _ptr(norm_weight),
                                   ctypes.c_float(eps), MOE_WEIGHTS_MX4 if mx4 else MOE_WEIGHTS_DTYPE,
                                   _ptr(w_router), _ptr(bias), *ptrs, _ptr(sh_gate), _ptr(out),
                                   _ptr(topk_idx), _ptr(topk_w), _ptr(resid), _ptr(ws), ws.numel(),
                                   _stream())
    _check(st, "moe_forward_prenorm")
    return out, topk_idx, topk_w


class MoELayer:
    """Device-resident weights plus a workspace sized for up to ``max_tokens``
    tokens, so repeated calls allocate nothing but their outputs."""

    def __init__(self, w_router, w_gate_up, w_down, k, w_sh_gate_up=None, w_sh_down=None,
                 sh_gate=None, bias=None, max_tokens=1, router=None, norm_weight=None,
                 eps=1e-6):
        self.w = dict(w_router=w_router, w_gate_up=w_gate_up, w_down=w_down,
                      w_sh_gate_up=w_sh_gate_up, w_sh_down=w_sh_down, sh_gate=sh_gate, bias=bias)
        self.k = k
        self.router = router
        # with norm_weight, calls take the un-normalised rows h (pre-FFN RMSNorm)
        self.norm_weight, self.eps = norm_weight, eps
        # MXFP4 expert weights: MX4Tensor, or row-major (codes, scales) pairs
        # packed here once
        self.mx4 = isinstance(w_gate_up, (tuple, MX4Tensor))
        if self.mx4:
            for n in ("w_gate_up", "w_down", "w_sh_gate_up", "w_sh_down"):
                if isinstance(self.w[n], tuple):
                    self.w[n] = mx4_pack(*self.w[n])
            E, F, Fs = _mx4_dims(w_router.shape[1], self.w["w_gate_up"], self.w["w_down"],
                                 self.w["w_sh_gate_up"], self.w["w_sh_down"])
            self.shape = Shape(w_router.shape[1], E, k, F, Fs, w_router.dtype, router)
        else:
            self.shape = shape_of(w_router, w_gate_up, k, w_sh_gate_up, router)
        self.max_tokens = max_tokens
        self.ws = alloc_workspace(self.shape, max_tokens, w_router.device)

    def __call__(self, x, out=None, topk_idx=None, topk_w=None, resid=None):
        """resid (pre-norm layers only): the binary32 residual stream, updated
        in place to resid + out by the same call."""
        if x.shape[0] > self.max_tokens:
            raise ValueError("more tokens than the workspace was sized for")
        w = self.w
        if self.norm_weight is not None:
            return forward_prenorm(x, self.norm_weight, w["w_router"], w["w_gate_up"], w["w_down"],
                                   self.k, w["w_sh_gate_up"], w["w_sh_down"], w["sh_gate"],
                                   w["bias"], self.eps, out, topk_idx, topk_w, self.ws, self.router,
                                   resid)
        if resid is not None:
            raise ValueError("resid is taken by pre-norm layers (norm_weight given)")
        fwd = forward_mx4 if self.mx4 else forward
        return fwd(x, w["w_router"], w["w_gate_up"], w["w_down"], self.k, w["w_sh_gate_up"],
                   w["w_sh_down"], w["sh_gate"], w["bias"], out, topk_idx, topk_w, self.ws,
                   self.router)


READ_PROBE_SINK_WORDS = 8192


def read_probe(buf: torch.Tensor, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One streaming read of ``buf`` (contiguous device tensor, a multiple of
    16 bytes) by the whole chip (moe_read_probe): the practical HBM read
    ceiling.  Returns the sink of per-wave XOR folds (int32 [8192]); the XOR of
    its words is the XOR of the buffer's 32-bit words."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if sink is None:
        sink = torch.empty(READ_PROBE_SINK_WORDS, dtype=torch.int32, device=buf.device)
    if sink.numel() < READ_PROBE_SINK_WORDS or sink.dtype != torch.int32 or not sink.is_cuda:
        raise ValueError("sink must be a device int32 tensor of 8192 words")
    _check(lib().moe_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                _stream()), "moe_read_probe")
    return sink
