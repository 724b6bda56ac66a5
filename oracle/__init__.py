"""CPU oracle for the sparse Mixture-of-Experts feed-forward layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports, links or calls it, and it
never imports the product: the two share only the seeded inputs.

This module is a thin ctypes wrapper over ``moe_oracle.c`` (plain C, binary64
after the binary32 router logit).  Arrays are numpy: bfloat16 data is passed as
``uint16`` bit patterns, binary32 data as ``float32``.

What each function follows (pages cited by title and section):
  * ``route`` -- router logits, softmax, top-k, selected-weight normalisation:
    the Feed-forward panel of the "Decoder microscope" on the
    Qwen3.8-Flash-Next anatomy page (frontier-model-atlas).
  * ``experts`` / ``forward`` -- gated-MLP experts with SiLU
    (llm-architectures-explained "Qwen3.8-Flash-Next", "Every architecture
    field", ffns.moe.gated; llm-atlas "Qwen3.8-Flash-Next", "Raw config
    fields", hidden_act) plus one shared expert scaled by its own sigmoid gate
    (anatomy page, Feed-forward panel and "Evidence for layer 1").
  * ``rmsnorm`` -- the pre-FFN RMSNorm (eps 1e-6: llm-atlas "Qwen3.8-Flash-Next",
    "Key facts" Norm, "Raw config fields" rms_norm_eps), read as a pre-norm
    whose binary32 evaluation order is fixed so both sides route on the same
    normalised bits.
  * ``backward`` -- the layer's gradients with the routing given, and the
    router's auxiliary load-balancing loss, whose coefficient (0.001) is the
    only thing the pages state about it (llm-atlas "Qwen3.8-Flash-Next",
    "Raw config fields", router_aux_loss_coef); the formula is read as
    coef * E * sum_e f_e P_e (share of assignments times mean probability).
  * ``experts_mx4`` / ``forward_mx4`` / ``mx4_decode`` -- the same layer with
    low-bit expert weights.  The published weights are packed low-bit tensors
    (llm-atlas "Qwen3.8-Flash-Next", "Modelled costs"); the encoding is not
    named there, and the reading taken is MXFP4 of the OCP Microscaling (MX)
    specification v1.0 (E2M1 elements, one E8M0 scale per 32 elements of a
    row, two codes per byte with the even element in the low nibble).  An MX
    tensor is passed as a pair ``(codes uint8 [..., K/2], scales uint8
    [..., K/32])``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32 = 0
BF16 = 1


def build(force: bool = True) -> str:
    """Compile moe_oracle.c into oracle/liboracle.so with gcc (no fast-math,
    no FMA contraction, OpenMP)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    """The oracle library: oracle/liboracle.so (built if missing), or the
    build named by MOE_ORACLE_LIB (the sanitizer test's instrumented copy)."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("MOE_ORACLE_LIB") or _LIB_PATH
    if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_router_logits.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp]
    lib.oracle_route.argtypes = [i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.oracle_experts.argtypes = [i64, i32, i32, i32, i32, i32, i32,
                                   vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_forward.argtypes = [i64, i32, i32, i32, i32, i32, i32,
                                   vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_experts_mx4.argtypes = [i64, i32, i32, i32, i32, i32] + [vp] * 14
    lib.oracle_forward_mx4.argtypes = [i64, i32, i32, i32, i32, i32] + [vp] * 16
    lib.oracle_mx4_decode.argtypes = [i64, i64, vp, vp, vp]
    lib.oracle_rmsnorm.argtypes = [i64, i32, i32, vp, vp, ctypes.c_float, vp]
    lib.oracle_residual.argtypes = [i64, i32, vp, vp, vp]
    lib.oracle_backward.argtypes = ([i64, i32, i32, i32, i32, i32, i32] + [vp] * 11
                                    + [ctypes.c_double, i32, vp, i64, vp] + [vp] * 8)
    for f in (lib.oracle_router_logits, lib.oracle_route, lib.oracle_experts,
              lib.oracle_forward, lib.oracle_threads, lib.oracle_experts_mx4,
              lib.oracle_forward_mx4, lib.oracle_mx4_decode, lib.oracle_rmsnorm,
              lib.oracle_backward, lib.oracle_residual):
        f.restype = ctypes.c_int
    lib.oracle_threads.argtypes = []
    _lib = lib
    return lib


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_threads())


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"oracle arrays are float32 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a):
    if a is None:
        return None
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("oracle arrays must be C-contiguous")
    return a.ctypes.data_as(ctypes.c_void_p)


def _same(dt, *arrays):
    for a in arrays:
        if a is not None and _dtype_code(a) != dt:
            raise TypeError("all weight/activation arrays must share one dtype")


def _bias(bias, E):
    if bias is None:
        return None
    b = np.ascontiguousarray(bias, dtype=np.float32)
    if b.shape != (E,):
        raise ValueError("router bias must have shape [E]")
    return b


def router_logits(x, w_router, bias=None) -> np.ndarray:
    """binary32 router logits [T, E] in the canonical accumulation order."""
    T, d = x.shape
    E = w_router.shape[0]
    dt = _dtype_code(x)
    _same(dt, w_router)
    b = _bias(bias, E)
    out = np.empty((T, E), np.float32)
    rc = _load().oracle_router_logits(T, d, E, dt, _ptr(x), _ptr(w_router),
                                      _ptr(b), _ptr(out))
    if rc:
        raise RuntimeError(f"oracle_router_logits failed ({rc})")
    return out


def route(x, w_router, k, bias=None, return_logits=False):
    """Top-k routing: (topk_idx int32 [T,k], topk_w float64 [T,k][, logits])."""
    T, d = x.shape
    E = w_router.shape[0]
    dt = _dtype_code(x)
    _same(dt, w_router)
    b = _bias(bias, E)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    logits = np.empty((T, E), np.float32) if return_logits else None
    rc = _load().oracle_route(T, d, E, k, dt, _ptr(x), _ptr(w_router), _ptr(b),
                              _ptr(idx), _ptr(w), _ptr(logits))
    if rc:
        raise RuntimeError(f"oracle_route failed ({rc})")
    return (idx, w, logits) if return_logits else (idx, w)


def experts(x, w_gate_up, w_down, topk_idx, topk_w, w_sh_gate_up=None,
            w_sh_down=None, sh_gate=None, return_gate=False):
    """Expert stage with the routing given: float64 out [T, d] (and the
    shared gate s [T] if asked)."""
    T, d = x.shape
    E, twoF, d2 = w_gate_up.shape
    F = twoF // 2
    assert d2 == d and w_down.shape == (E, d, F)
    Fs = 0 if w_sh_gate_up is None else w_sh_gate_up.shape[0] // 2
    k = topk_idx.shape[1]
    dt = _dtype_code(x)
    _same(dt, w_gate_up, w_down, w_sh_gate_up, w_sh_down, sh_gate)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    w = np.ascontiguousarray(topk_w, dtype=np.float64)
    out = np.empty((T, d), np.float64)
    s = np.full((T,), np.nan, np.float64)
    rc = _load().oracle_experts(T, d, E, k, F, Fs, dt, _ptr(x), _ptr(w_gate_up),
                                _ptr(w_down), _ptr(w_sh_gate_up), _ptr(w_sh_down),
                                _ptr(sh_gate), _ptr(idx), _ptr(w), _ptr(out), _ptr(s))
    if rc:
        raise RuntimeError(f"oracle_experts failed ({rc})")
    return (out, s) if return_gate else out


def forward(x, w_router, w_gate_up, w_down, k, w_sh_gate_up=None, w_sh_down=None,
            sh_gate=None, bias=None):
    """The whole layer: (out float64 [T,d], topk_idx [T,k], topk_w float64
    [T,k], s float64 [T] (NaN without a shared expert))."""
    T, d = x.shape
    E, twoF, _ = w_gate_up.shape
    F = twoF // 2
    Fs = 0 if w_sh_gate_up is None else w_sh_gate_up.shape[0] // 2
    dt = _dtype_code(x)
    _same(dt, w_router, w_gate_up, w_down, w_sh_gate_up, w_sh_down, sh_gate)
    b = _bias(bias, E)
    out = np.empty((T, d), np.float64)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    s = np.full((T,), np.nan, np.float64)
    rc = _load().oracle_forward(T, d, E, k, F, Fs, dt, _ptr(x), _ptr(w_router), _ptr(b),
                                _ptr(w_gate_up), _ptr(w_down), _ptr(w_sh_gate_up),
                                _ptr(w_sh_down), _ptr(sh_gate), _ptr(out), _ptr(idx),
                                _ptr(w), _ptr(s))
    if rc:
        raise RuntimeError(f"oracle_forward failed ({rc})")
    return out, idx, w, s


def _mx(t, rows_shape, K):
    """Validate one MXFP4 tensor (codes, scales) of logical shape rows_shape + (K,)."""
    if t is None:
        return None, None
    codes, scales = t
    if codes.dtype != np.uint8 or scales.dtype != np.uint8:
        raise TypeError("MXFP4 codes and scales are uint8 arrays")
    if K % 32:
        raise ValueError("MXFP4 rows must hold a multiple of 32 elements")
    if codes.shape != tuple(rows_shape) + (K // 2,) or scales.shape != tuple(rows_shape) + (K // 32,):
        raise ValueError(f"MXFP4 tensor shapes {codes.shape}/{scales.shape} do not match "
                         f"{tuple(rows_shape)} x {K}")
    return _ptr(codes), _ptr(scales)


def mx4_decode(codes, scales) -> np.ndarray:
    """Every element of an MXFP4 tensor [rows, K] decoded exactly (float64)."""
    rows = int(np.prod(codes.shape[:-1]))
    K = codes.shape[-1] * 2
    c, sc = _mx((codes, scales), codes.shape[:-1], K)
    out = np.empty(codes.shape[:-1] + (K,), np.float64)
    rc = _load().oracle_mx4_decode(rows, K, c, sc, _ptr(out))
    if rc:
        raise RuntimeError(f"oracle_mx4_decode failed ({rc})")
    return out


def _mx4_layer_ptrs(gu, dn, sgu, sdn, E, F, Fs, d):
    ptrs = []
    ptrs += _mx(gu, (E, 2 * F), d)
    ptrs += _mx(dn, (E, d), F)
    ptrs += _mx(sgu, (2 * Fs,), d) if Fs else (None, None)
    ptrs += _mx(sdn, (d,), Fs) if Fs else (None, None)
    return ptrs


def experts_mx4(x, gu, dn, topk_idx, topk_w, sgu=None, sdn=None, sh_gate=None,
                return_gate=False):
    """Expert stage with MXFP4 expert weights and the routing given.  x and
    sh_gate are bfloat16 bits; gu, dn, sgu, sdn are (codes, scales) pairs of
    logical shapes [E,2F,d], [E,d,F], [2Fs,d], [d,Fs]."""
    T, d = x.shape
    if _dtype_code(x) != BF16:
        raise TypeError("MXFP4 layers take bfloat16 activations")
    E, twoF = gu[0].shape[:2]
    F = twoF // 2
    Fs = 0 if sgu is None else sgu[0].shape[0] // 2
    k = topk_idx.shape[1]
    ptrs = _mx4_layer_ptrs(gu, dn, sgu, sdn, E, F, Fs, d)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    w = np.ascontiguousarray(topk_w, dtype=np.float64)
    out = np.empty((T, d), np.float64)
    s = np.full((T,), np.nan, np.float64)
    rc = _load().oracle_experts_mx4(T, d, E, k, F, Fs, _ptr(x), *ptrs, _ptr(sh_gate),
                                    _ptr(idx), _ptr(w), _ptr(out), _ptr(s))
    if rc:
        raise RuntimeError(f"oracle_experts_mx4 failed ({rc})")
    return (out, s) if return_gate else out


def forward_mx4(x, w_router, gu, dn, k, sgu=None, sdn=None, sh_gate=None, bias=None):
    """The whole layer with MXFP4 expert weights: (out float64 [T,d], topk_idx
    [T,k], topk_w float64 [T,k], s float64 [T])."""
    T, d = x.shape
    if _dtype_code(x) != BF16:
        raise TypeError("MXFP4 layers take bfloat16 activations")
    _same(BF16, w_router, sh_gate)
    E, twoF = gu[0].shape[:2]
    F = twoF // 2
    Fs = 0 if sgu is None else sgu[0].shape[0] // 2
    ptrs = _mx4_layer_ptrs(gu, dn, sgu, sdn, E, F, Fs, d)
    b = _bias(bias, E)
    out = np.empty((T, d), np.float64)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    s = np.full((T,), np.nan, np.float64)
    rc = _load().oracle_forward_mx4(T, d, E, k, F, Fs, _ptr(x), _ptr(w_router), _ptr(b),
                                    *ptrs, _ptr(sh_gate), _ptr(out), _ptr(idx), _ptr(w),
                                    _ptr(s))
    if rc:
        raise RuntimeError(f"oracle_forward_mx4 failed ({rc})")
    return out, idx, w, s


def rmsnorm(h, gamma, eps=1e-6):
    """Pre-FFN RMSNorm of h [T, d] with weight gamma [d]: x in h's dtype
    (bfloat16 bits rounded to nearest even, or float32)."""
    T, d = h.shape
    dt = _dtype_code(h)
    _same(dt, gamma)
    if gamma.shape != (d,):
        raise ValueError("gamma must have shape [d]")
    out = np.empty_like(h)
    rc = _load().oracle_rmsnorm(T, d, dt, _ptr(h), _ptr(gamma), ctypes.c_float(eps), _ptr(out))
    if rc:
        raise RuntimeError(f"oracle_rmsnorm failed ({rc})")
    return out


def residual(resid, out):
    """The residual stream after the layer (oracle_residual): resid [T, d]
    float32 plus the layer's out [T, d] (float64), in float64."""
    r = np.ascontiguousarray(resid, dtype=np.float32)
    o = np.ascontiguousarray(out, dtype=np.float64)
    if r.ndim != 2 or r.shape != o.shape:
        raise ValueError("resid and out must both be [T, d]")
    res = np.empty_like(o)
    rc = _load().oracle_residual(r.shape[0], r.shape[1], _ptr(r), _ptr(o), _ptr(res))
    if rc:
        raise RuntimeError(f"oracle_residual failed ({rc})")
    return res


DX, DW_ROUTED, DW_SHARED, DW_ROUTER = 1, 2, 4, 8


def backward(x, w_router, w_gate_up, w_down, topk_idx, topk_w, dout, w_sh_gate_up=None,
             w_sh_down=None, sh_gate=None, bias=None, aux_coef=0.0,
             parts=DX | DW_ROUTED | DW_SHARED | DW_ROUTER, tokens=None, experts=None):
    """Gradients of sum(dout * out) + aux_coef * E * sum_e f_e P_e with the
    routing (topk_idx, topk_w) given, in float64.  Returns a dict with dx
    [T,d], dw_router [E,d], dw_gate_up [E,2F,d], dw_down [E,d,F],
    dw_sh_gate_up [2Fs,d], dw_sh_down [d,Fs], dsh_gate [d] and aux_loss.
    parts / tokens / experts restrict the work: dx of the listed tokens (the
    other rows NaN), the routed weight gradients of the listed experts (then
    dw_gate_up / dw_down hold only those, in the order listed).  Outputs of
    parts not asked for are None."""
    T, d = x.shape
    E, twoF, _ = w_gate_up.shape
    F = twoF // 2
    Fs = 0 if w_sh_gate_up is None else w_sh_gate_up.shape[0] // 2
    k = topk_idx.shape[1]
    dt = _dtype_code(x)
    _same(dt, w_router, w_gate_up, w_down, w_sh_gate_up, w_sh_down, sh_gate)
    b = _bias(bias, E)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    w = np.ascontiguousarray(topk_w, dtype=np.float64)
    g = np.ascontiguousarray(dout, dtype=np.float64)
    if g.shape != (T, d) or idx.shape != (T, k) or w.shape != (T, k):
        raise ValueError("dout must be [T, d], topk_idx / topk_w [T, k]")
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    slot, n_exp = None, E
    if experts is not None:
        experts = np.asarray(experts, dtype=np.int64)
        if len(np.unique(experts)) != len(experts) or (experts < 0).any() or (experts >= E).any():
            raise ValueError("experts must be distinct indices in [0, E)")
        slot = np.full(E, -1, np.int32)
        slot[experts] = np.arange(len(experts), dtype=np.int32)
        n_exp = len(experts)

    def nan(want, *shape):
        return np.full(shape, np.nan, np.float64) if want else None
    r = dict(dx=nan(parts & DX, T, d), dw_router=nan(parts & DW_ROUTER, E, d),
             dw_gate_up=nan(parts & DW_ROUTED, n_exp, 2 * F, d),
             dw_down=nan(parts & DW_ROUTED, n_exp, d, F),
             dw_sh_gate_up=nan(parts & DW_SHARED, 2 * Fs, d),
             dw_sh_down=nan(parts & DW_SHARED, d, Fs), dsh_gate=nan(parts & DW_SHARED, d))
    aux = ctypes.c_double(np.nan)
    rc = _load().oracle_backward(
        T, d, E, k, F, Fs, dt, _ptr(x), _ptr(w_router), _ptr(b), _ptr(w_gate_up),
        _ptr(w_down), _ptr(w_sh_gate_up), _ptr(w_sh_down), _ptr(sh_gate), _ptr(idx), _ptr(w),
        _ptr(g), ctypes.c_double(aux_coef), parts, _ptr(tok), 0 if tok is None else len(tok),
        _ptr(slot), *[_ptr(r[n]) for n in ("dx", "dw_router", "dw_gate_up", "dw_down",
                                           "dw_sh_gate_up", "dw_sh_down", "dsh_gate")],
        ctypes.byref(aux))
    if rc:
        raise RuntimeError(f"oracle_backward failed ({rc})")
    r["aux_loss"] = aux.value
    return r
