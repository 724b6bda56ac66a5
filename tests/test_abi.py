"""The C ABI without a GPU: the library loads, exports what include/moe.h
declares, and rejects bad arguments before any GPU work."""
import ctypes
import os
import re

import pytest

import sparse_moe_feed_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from sparse_moe_feed_amd import build
        build.build()
    return moe.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert names == set(moe.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def desc(d=256, E=16, k=4, F=128, Fs=64, dtype=moe.MOE_BF16, flags=0):
    return moe.moe_desc(d, E, k, F, Fs, dtype, flags)


@pytest.mark.parametrize("bad", [
    dict(d=0), dict(E=0), dict(k=0), dict(k=17), dict(F=0), dict(Fs=-1), dict(dtype=7),
    dict(flags=3), dict(flags=-1)])
def test_invalid_desc(L, bad):
    D = desc(**bad)
    assert L.moe_workspace_size(ctypes.byref(D), 10) == 0
    lay = moe.moe_workspace_layout()
    assert L.moe_workspace_query(ctypes.byref(D), 10, ctypes.byref(lay)) == moe.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", [
    dict(k=33, E=64), dict(E=2048, k=4), dict(d=100), dict(F=96), dict(Fs=32), dict(d=32768),
    dict(dtype=moe.MOE_F32, flags=moe.MOE_FLAG_ROUTER_SHORTLIST)])
def test_unsupported_desc(L, bad):
    D = desc(**bad)
    lay = moe.moe_workspace_layout()
    assert L.moe_workspace_query(ctypes.byref(D), 10, ctypes.byref(lay)) == moe.MOE_ERR_UNSUPPORTED


def test_fp32_accepts_any_width(L):
    D = desc(d=100, F=33, Fs=7, dtype=moe.MOE_F32)
    assert L.moe_workspace_size(ctypes.byref(D), 10) > 0


def test_workspace_grows_with_T_and_layout_is_consistent(L):
    D = desc()
    sizes = [L.moe_workspace_size(ctypes.byref(D), T) for T in (1, 10, 1000)]
    assert sizes[0] < sizes[1] < sizes[2]
    lay = moe.moe_workspace_layout()
    assert L.moe_workspace_query(ctypes.byref(D), 1000, ctypes.byref(lay)) == moe.MOE_OK
    assert lay.total == sizes[2]
    offs = [lay.logits, lay.gate, lay.counts, lay.offsets, lay.perm, lay.h, lay.h_shared]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.h_shared + 1000 * 64 * 2 <= lay.total
    assert lay.perm + 1000 * 4 * 4 <= lay.h


def test_shortlist_router_holds_two_logit_slices(L):
    """The shortlist router keeps the MFMA logits as two partial sums over the
    halves of K when d % 128 == 0 (one slice otherwise): its logits region is
    [S, T, E+1] binary32, the exact router's [T, E+1] (both followed by the
    row norms); nothing else differs."""
    T, E = 300, 16

    def region(d, flags):
        D = desc(d=d, E=E, flags=flags)
        lay = moe.moe_workspace_layout()
        assert L.moe_workspace_query(ctypes.byref(D), T, ctypes.byref(lay)) == moe.MOE_OK
        return lay.gate - lay.logits, lay.total - lay.gate

    def aligned(n):  # regions start on 256-byte boundaries
        return (n + 255) // 256 * 256

    one = T * (E + 1) * 4
    for d, S in ((256, 2), (192, 1)):
        ex_logits, ex_rest = region(d, moe.MOE_FLAG_ROUTER_EXACT)
        sl_logits, sl_rest = region(d, moe.MOE_FLAG_ROUTER_SHORTLIST)
        assert sl_logits - ex_logits == aligned(S * one) - aligned(one)
        assert ex_rest == sl_rest


FAKE = 0x10000  # never dereferenced: every case fails validation first


def call_forward(L, D, T, ptrs=None, ws=FAKE, ws_bytes=1 << 40):
    p = dict(x=FAKE, wr=FAKE, b=None, gu=FAKE, dn=FAKE, sgu=FAKE, sdn=FAKE, g=FAKE, out=FAKE,
             idx=FAKE, w=FAKE)
    p.update(ptrs or {})
    v = lambda a: None if a is None else ctypes.c_void_p(a)
    return L.moe_forward(ctypes.byref(D), T, v(p["x"]), v(p["wr"]), v(p["b"]), v(p["gu"]),
                         v(p["dn"]), v(p["sgu"]), v(p["sdn"]), v(p["g"]), v(p["out"]),
                         v(p["idx"]), v(p["w"]), v(ws), ws_bytes, None)


@pytest.mark.parametrize("missing", ["x", "wr", "gu", "dn", "out", "idx", "w", "sgu", "sdn", "g"])
def test_null_required_pointer(L, missing):
    assert call_forward(L, desc(), 8, {missing: None}) == moe.MOE_ERR_INVALID_ARG


def test_shared_pointers_optional_without_shared_expert(L):
    D = desc(Fs=0)
    # all pointers fine, workspace too small -> reaches the workspace check
    assert call_forward(L, D, 8, {"sgu": None, "sdn": None, "g": None}, ws_bytes=16) == \
        moe.MOE_ERR_WORKSPACE


def test_misaligned_pointer(L):
    assert call_forward(L, desc(), 8, {"x": FAKE + 2}) == moe.MOE_ERR_INVALID_ARG
    assert call_forward(L, desc(), 8, {"b": FAKE + 4}) == moe.MOE_ERR_INVALID_ARG


def test_negative_T_and_workspace(L):
    D = desc()
    assert call_forward(L, D, -1) == moe.MOE_ERR_INVALID_ARG
    assert call_forward(L, D, 8, ws=None) == moe.MOE_ERR_WORKSPACE
    need = L.moe_workspace_size(ctypes.byref(D), 8)
    assert call_forward(L, D, 8, ws_bytes=need - 1) == moe.MOE_ERR_WORKSPACE


def test_zero_tokens_is_noop(L):
    assert call_forward(L, desc(), 0, ws=None, ws_bytes=0) == moe.MOE_OK
    assert call_forward(L, desc(), 0, {"x": None, "out": None}, ws=None, ws_bytes=0) == moe.MOE_OK


def test_route_and_experts_validate(L):
    D = desc()
    v = ctypes.c_void_p
    assert L.moe_route(ctypes.byref(D), 8, None, v(FAKE), None, None, v(FAKE), v(FAKE), None,
                       v(FAKE), 1 << 40, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_route(ctypes.byref(D), 0, v(FAKE), v(FAKE), None, None, v(FAKE), v(FAKE), None,
                       None, 0, None) == moe.MOE_OK
    assert L.moe_experts(ctypes.byref(D), 8, v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE),
                         None, v(FAKE), v(FAKE), v(FAKE), 1 << 40, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_experts(ctypes.byref(D), 8, v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE),
                         v(FAKE), v(FAKE), v(FAKE), v(FAKE), 16, None) == moe.MOE_ERR_WORKSPACE


def call_forward_mx4(L, D, T, ptrs=None, ws=FAKE, ws_bytes=1 << 40):
    p = dict(x=FAKE, wr=FAKE, b=None, gu=FAKE, dn=FAKE, sgu=FAKE, sdn=FAKE, g=FAKE, out=FAKE,
             idx=FAKE, w=FAKE)
    p.update(ptrs or {})
    v = lambda a: None if a is None else ctypes.c_void_p(a)
    return L.moe_forward_mx4(ctypes.byref(D), T, v(p["x"]), v(p["wr"]), v(p["b"]), v(p["gu"]),
                             v(p["dn"]), v(p["sgu"]), v(p["sdn"]), v(p["g"]), v(p["out"]),
                             v(p["idx"]), v(p["w"]), v(ws), ws_bytes, None)


def mx4_desc(**kw):
    base = dict(d=256, E=16, k=4, F=128, Fs=128)
    base.update(kw)
    return desc(**base)


@pytest.mark.parametrize("missing", ["gu", "dn", "sgu", "sdn", "g", "x", "out"])
def test_mx4_null_required_pointer(L, missing):
    assert call_forward_mx4(L, mx4_desc(), 8, {missing: None}) == moe.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", [dict(dtype=moe.MOE_F32), dict(Fs=64), dict(F=192),
                                 dict(d=320)])
def test_mx4_unsupported_shapes(L, bad):
    """MXFP4 layers need bf16 activations and 128-multiples, at any T."""
    assert call_forward_mx4(L, mx4_desc(**bad), 8) == moe.MOE_ERR_UNSUPPORTED
    assert call_forward_mx4(L, mx4_desc(**bad), 0, ws=None, ws_bytes=0) == moe.MOE_ERR_UNSUPPORTED


def test_mx4_offset_limit(L):
    """Batches whose row offsets would not fit 32 bits are refused before
    any GPU work; smaller ones reach the workspace check."""
    D = mx4_desc(d=2560, E=512, k=10, F=640, Fs=640)
    assert call_forward_mx4(L, D, 200000) == moe.MOE_ERR_UNSUPPORTED   # T k d >= 2^32
    assert call_forward_mx4(L, D, 4096, ws_bytes=16) == moe.MOE_ERR_WORKSPACE


def test_mx4_misaligned_and_noop(L):
    assert call_forward_mx4(L, mx4_desc(), 8, {"gu": FAKE + 8}) == moe.MOE_ERR_INVALID_ARG
    assert call_forward_mx4(L, mx4_desc(), 0, ws=None, ws_bytes=0) == moe.MOE_OK
    D = mx4_desc(Fs=0)
    assert call_forward_mx4(L, D, 8, {"sgu": None, "sdn": None, "g": None}, ws_bytes=16) == \
        moe.MOE_ERR_WORKSPACE


def test_mx4_experts_validate(L):
    v = ctypes.c_void_p
    D = mx4_desc()
    assert L.moe_experts_mx4(ctypes.byref(D), 8, v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE),
                             v(FAKE), None, v(FAKE), v(FAKE), v(FAKE), 1 << 40,
                             None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_experts_mx4(ctypes.byref(mx4_desc(dtype=moe.MOE_F32)), 8, v(FAKE), v(FAKE),
                             v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE),
                             v(FAKE), 1 << 40, None) == moe.MOE_ERR_UNSUPPORTED


def test_mx4_packed_bytes_and_pack_validation(L):
    assert L.moe_mx4_packed_bytes(32, 256) == 2 * 2 * 1088
    assert L.moe_mx4_packed_bytes(2 * 1280 * 512, 2560) == 2 * 1280 * 512 * 2560 * 17 // 32
    for rows, K in [(0, 128), (16, 0), (24, 128), (16, 192), (-16, 128)]:
        assert L.moe_mx4_packed_bytes(rows, K) == 0
    v = ctypes.c_void_p
    assert L.moe_mx4_pack(None, v(FAKE), 16, 128, v(FAKE), None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_mx4_pack(v(FAKE), v(FAKE), 16, 128, v(FAKE + 4), None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_mx4_pack(v(FAKE), v(FAKE), 24, 128, v(FAKE), None) == moe.MOE_ERR_INVALID_ARG


def test_rmsnorm_validation(L):
    v = ctypes.c_void_p
    D = desc()
    assert L.moe_rmsnorm(ctypes.byref(D), 8, None, v(FAKE), ctypes.c_float(1e-6), v(FAKE),
                         None) == moe.MOE_ERR_INVALID_ARG
    for eps in (-1.0, float("nan"), float("inf")):
        assert L.moe_rmsnorm(ctypes.byref(D), 8, v(FAKE), v(FAKE), ctypes.c_float(eps), v(FAKE),
                             None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_rmsnorm(ctypes.byref(D), 8, v(FAKE + 2), v(FAKE), ctypes.c_float(1e-6),
                         v(FAKE), None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_rmsnorm(ctypes.byref(D), 0, None, None, ctypes.c_float(1e-6), None,
                         None) == moe.MOE_OK
    assert L.moe_rmsnorm(ctypes.byref(desc(E=0)), 8, v(FAKE), v(FAKE), ctypes.c_float(1e-6),
                         v(FAKE), None) == moe.MOE_ERR_INVALID_ARG


def call_prenorm(L, D, T, fmt=0, eps=1e-6, g=FAKE, ws_bytes=1 << 40, resid=None, out=FAKE + 4096):
    v = lambda a: None if a is None else ctypes.c_void_p(a)
    return L.moe_forward_prenorm(ctypes.byref(D), T, v(FAKE), v(g), ctypes.c_float(eps), fmt,
                                 v(FAKE), None, v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE),
                                 v(out), v(FAKE), v(FAKE), v(resid), v(FAKE), ws_bytes, None)


def test_forward_prenorm_validation(L):
    D = desc()
    assert call_prenorm(L, D, 8, fmt=2) == moe.MOE_ERR_INVALID_ARG
    assert call_prenorm(L, D, 8, g=None) == moe.MOE_ERR_INVALID_ARG
    assert call_prenorm(L, D, 8, eps=-1e-6) == moe.MOE_ERR_INVALID_ARG
    assert call_prenorm(L, desc(k=0), 8, g=None) == moe.MOE_ERR_INVALID_ARG
    assert call_prenorm(L, D, 8, ws_bytes=16) == moe.MOE_ERR_WORKSPACE
    # MXFP4 weights keep their limits
    assert call_prenorm(L, mx4_desc(d=2560, E=512, k=10, F=640, Fs=640), 200000,
                        fmt=1) == moe.MOE_ERR_UNSUPPORTED
    assert call_prenorm(L, mx4_desc(dtype=moe.MOE_F32), 8, fmt=1) == moe.MOE_ERR_UNSUPPORTED
    # the residual stream: 16-byte aligned, aliasing neither out nor h
    assert call_prenorm(L, D, 8, resid=FAKE + 8) == moe.MOE_ERR_INVALID_ARG
    assert call_prenorm(L, D, 8, resid=FAKE + 4096) == moe.MOE_ERR_INVALID_ARG
    assert call_prenorm(L, D, 8, resid=FAKE) == moe.MOE_ERR_INVALID_ARG
    assert call_prenorm(L, D, 8, resid=FAKE + 8192, ws_bytes=16) == moe.MOE_ERR_WORKSPACE


def test_workspace_has_xnorm_region(L):
    D = desc()
    lay = moe.moe_workspace_layout()
    assert L.moe_workspace_query(ctypes.byref(D), 100, ctypes.byref(lay)) == moe.MOE_OK
    assert lay.xnorm % 256 == 0 and lay.xnorm + 100 * 256 * 2 <= lay.total


def test_status_strings(L):
    for st in range(5):
        assert moe.status_string(st).startswith("MOE_")
    assert "unknown" in moe.status_string(99)


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.route(x, torch.zeros(8, 64, dtype=torch.bfloat16), 2)


BWD_PTRS = ("x", "wr", "b", "gu", "dn", "sgu", "sdn", "g", "idx", "w", "dout", "saved", "dx",
            "dwr", "dgu", "ddn", "dsgu", "dsdn", "dg", "aux")


def call_backward(L, D, T, ptrs=None, coef=0.001, ws=FAKE, ws_bytes=1 << 40):
    p = {n: FAKE for n in BWD_PTRS}
    p["b"] = p["aux"] = p["saved"] = None
    p.update(ptrs or {})
    v = lambda a: None if a is None else ctypes.c_void_p(a)
    args = [v(p[n]) for n in BWD_PTRS]
    return L.moe_backward(ctypes.byref(D), T, *args[:12], ctypes.c_float(coef), *args[12:],
                          v(ws), ws_bytes, None)


@pytest.mark.parametrize("missing", ["x", "wr", "gu", "dn", "idx", "w", "dout", "dx", "dwr",
                                     "dgu", "ddn", "sgu", "sdn", "g", "dsgu", "dsdn", "dg"])
def test_backward_null_required_pointer(L, missing):
    assert call_backward(L, desc(), 8, {missing: None}) == moe.MOE_ERR_INVALID_ARG


def test_backward_validation(L):
    D = desc()
    assert call_backward(L, desc(d=0), 8) == moe.MOE_ERR_INVALID_ARG
    assert call_backward(L, desc(F=96), 8) == moe.MOE_ERR_UNSUPPORTED
    assert call_backward(L, D, -1) == moe.MOE_ERR_INVALID_ARG
    assert call_backward(L, D, 8, {"dout": FAKE + 4}) == moe.MOE_ERR_INVALID_ARG
    assert call_backward(L, D, 8, {"aux": FAKE + 2}) == moe.MOE_ERR_INVALID_ARG
    assert call_backward(L, D, 8, {"saved": FAKE + 8}) == moe.MOE_ERR_INVALID_ARG
    assert call_backward(L, D, 8, coef=float("nan")) == moe.MOE_ERR_INVALID_ARG
    assert call_backward(L, D, 8, ws=None) == moe.MOE_ERR_WORKSPACE
    need = L.moe_backward_workspace_size(ctypes.byref(D), 8)
    assert need > 0
    assert call_backward(L, D, 8, ws_bytes=need - 1) == moe.MOE_ERR_WORKSPACE
    # no shared expert: its pointers may be NULL (reaches the workspace check)
    D0 = desc(Fs=0)
    none = {n: None for n in ("sgu", "sdn", "g", "dsgu", "dsdn", "dg")}
    assert call_backward(L, D0, 8, none, ws_bytes=16) == moe.MOE_ERR_WORKSPACE
    # T = 0: nothing is read or written
    assert call_backward(L, D, 0, {n: None for n in BWD_PTRS}, ws=None, ws_bytes=0) == moe.MOE_OK


def test_backward_workspace_grows_with_T(L):
    D = desc()
    sizes = [L.moe_backward_workspace_size(ctypes.byref(D), T) for T in (1, 10, 1000)]
    assert 0 < sizes[0] < sizes[1] < sizes[2]
    assert L.moe_backward_workspace_size(ctypes.byref(desc(E=0)), 10) == 0


def call_forward_train(L, D, T, saved=FAKE, saved_bytes=1 << 40, ws=FAKE, ws_bytes=1 << 40,
                       ptrs=None):
    p = dict(x=FAKE, wr=FAKE, b=None, gu=FAKE, dn=FAKE, sgu=FAKE, sdn=FAKE, g=FAKE, out=FAKE,
             idx=FAKE, w=FAKE)
    p.update(ptrs or {})
    v = lambda a: None if a is None else ctypes.c_void_p(a)
    return L.moe_forward_train(ctypes.byref(D), T, v(p["x"]), v(p["wr"]), v(p["b"]), v(p["gu"]),
                               v(p["dn"]), v(p["sgu"]), v(p["sdn"]), v(p["g"]), v(p["out"]),
                               v(p["idx"]), v(p["w"]), v(saved), saved_bytes, v(ws), ws_bytes,
                               None)


def test_forward_train_validation(L):
    D = desc()
    need = L.moe_saved_bytes(ctypes.byref(D), 8)
    assert need == (8 * 4 * 2 * 128 + 8 * 2 * 64) * 2
    assert L.moe_saved_bytes(ctypes.byref(desc(d=0)), 8) == 0
    assert call_forward_train(L, D, 8, saved=None) == moe.MOE_ERR_INVALID_ARG
    assert call_forward_train(L, D, 8, saved=FAKE + 4) == moe.MOE_ERR_INVALID_ARG
    assert call_forward_train(L, D, 8, saved_bytes=need - 1) == moe.MOE_ERR_INVALID_ARG
    # the rest as moe_forward: a missing x, a small workspace
    assert call_forward_train(L, D, 8, saved_bytes=need, ptrs={"x": None}) == moe.MOE_ERR_INVALID_ARG
    assert call_forward_train(L, D, 8, saved_bytes=need, ws_bytes=16) == moe.MOE_ERR_WORKSPACE
    assert call_forward_train(L, D, 0, saved=None, saved_bytes=0, ws=None, ws_bytes=0) == moe.MOE_OK


def test_read_probe_rejects_bad_arguments(L):
    """moe_read_probe checks its pointers and size before any launch (the
    fake addresses below are never dereferenced)."""
    buf, sink = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21)
    bad = moe.MOE_ERR_INVALID_ARG
    assert L.moe_read_probe(None, 16, sink, None) == bad
    assert L.moe_read_probe(buf, 16, None, None) == bad
    assert L.moe_read_probe(ctypes.c_void_p((1 << 20) + 8), 16, sink, None) == bad
    assert L.moe_read_probe(buf, 24, sink, None) == bad
    assert L.moe_read_probe(buf, 16, ctypes.c_void_p((1 << 21) + 2), None) == bad


def test_noalloc_checks_before_any_gpu_work(L):
    """moe_forward_noalloc validates its arguments and the size of the call
    against its static array before touching the GPU (none is needed here;
    the fake addresses are never dereferenced)."""
    D = desc(d=2560, E=512, k=10, F=640, Fs=640)
    p = [ctypes.c_void_p(1 << 20)] * 10
    # every batch up to 1347 tokens fits the 100 MiB array at the pages' shape
    assert all(L.moe_workspace_size(ctypes.byref(D), T) <= 100 << 20 for T in range(1, 1348))
    assert L.moe_workspace_size(ctypes.byref(D), 1348) > 100 << 20
    assert L.moe_forward_noalloc(ctypes.byref(D), 1348, *p[:3], *p[3:10], p[0], None) == \
        moe.MOE_ERR_WORKSPACE
    assert b"static scratch" in L.moe_last_error()
    assert L.moe_forward_noalloc(ctypes.byref(D), 16, None, *p[1:3], *p[3:10], p[0], None) == \
        moe.MOE_ERR_INVALID_ARG
    assert L.moe_forward_noalloc(ctypes.byref(D), -1, *p[:3], *p[3:10], p[0], None) == \
        moe.MOE_ERR_INVALID_ARG
    assert L.moe_forward_noalloc(ctypes.byref(D), 0, *p[:3], *p[3:10], p[0], None) == moe.MOE_OK
    bad = desc(d=2560, E=512, k=10, F=640, Fs=640, dtype=7)
    assert L.moe_forward_noalloc(ctypes.byref(bad), 16, *p[:3], *p[3:10], p[0], None) == \
        moe.MOE_ERR_INVALID_ARG
