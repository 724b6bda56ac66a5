"""Parity of moe_backward (through the C ABI) with the oracle's backward pass.

The routing (topk_idx, topk_w) and dout are inputs of both sides; the routing
comes from the oracle's router.

Bars, derived from the arithmetic of the bfloat16 path.  On the way to each
gradient the kernels round about four operands to bfloat16 once each (dout,
the pre-activations a and u, h or [da; du], dL; unit roundoff 2^-8, errors
independent from element to element), accumulate in binary32, and bfloat16
gradients are rounded once more when stored.  A rounding-faithful emulation
of that scheme on the CPU gives an RMS error of 0.34% of RMS(oracle) and
worst elements up to ~6% of RMS: an element dominated by one large product
carries that product's rounding error.  The tests therefore bound
  * RMS(g - oracle) <= 2^-7 RMS(oracle)                 (systematic errors);
  * |g - oracle| <= 0.1 RMS(oracle) + 4 * 2^-8 |oracle|  element-wise (local
    errors; the second term is four roundings of a single dominant product,
    which is what an element of an expert with one or two tokens is);
  * expert weight gradients are judged expert by expert (RMS of that expert's
    gradient: its scale follows its own token count);
  * binary32 layers (no bfloat16 rounding anywhere):
    |g - oracle| <= 1e-4 RMS(oracle) element-wise;
  * the auxiliary loss value: relative 1e-4 (binary32 softmax and sums).
Index, sign or missing-term mistakes move elements by O(RMS) and fail the
element-wise bar; a systematically wrong small term (e.g. the load-balancing
gradient) is isolated by the test that drives the router with it alone.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_feed_amd as moe
import workloads as W
from gpu_util import announce, to_dev

pytestmark = pytest.mark.gpu

GRADS = ("dw_router", "dw_gate_up", "dw_down", "dw_sh_gate_up", "dw_sh_down", "dsh_gate")
WEIGHTS = ("x", "w_router", "w_gate_up", "w_down", "w_sh_gate_up", "w_sh_down", "sh_gate")


def as_f64(t):
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def check_grad(name, got, ref, bf16, sel=None, f32_layer=False):
    """got: GPU tensor; ref: oracle float64 (NaN where not computed).  Expert
    weight gradients ([E, ...]) are judged expert by expert: each one's
    scale follows its own token count.  Returns the worst max|err| / RMS."""
    g = as_f64(got)
    if sel is not None:
        g, ref = g[sel], ref[sel]
    assert not np.isnan(ref).any(), name
    groups = [(g, ref)] if ref.ndim < 3 else list(zip(g, ref))
    worst = 0.0
    for gi, ri in groups:
        rms = np.sqrt((ri ** 2).mean())
        err = np.abs(gi - ri)
        if rms == 0:
            assert err.max() == 0, name
            continue
        worst = max(worst, float(err.max() / rms))
        if f32_layer:
            assert np.all(err <= 1e-4 * rms), f"{name}: max|err|/rms = {err.max() / rms:.3e}"
            continue
        rms_err = np.sqrt((err ** 2).mean()) / rms
        assert rms_err <= 2.0 ** -7, f"{name}: RMS err / RMS = {rms_err:.4f}"
        bound = 0.1 * rms + 4 * 2.0 ** -8 * np.abs(ri)
        assert np.all(err <= bound), f"{name}: max|err|/rms = {err.max() / rms:.4f}"
    return worst


def gpu_backward(inp, idx, w, dout, coef, bias=None):
    ins = {n: to_dev(inp[n]) for n in WEIGHTS}
    r = moe.backward(ins["x"], ins["w_router"], ins["w_gate_up"], ins["w_down"], to_dev(idx),
                     to_dev(w.astype(np.float32)), to_dev(dout), ins["w_sh_gate_up"],
                     ins["w_sh_down"], ins["sh_gate"], bias=to_dev(bias), aux_coef=coef)
    torch.cuda.synchronize()
    return r


def oracle_backward(inp, idx, w, dout, coef, bias=None, **kw):
    return oracle.backward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], idx, w,
                           dout.astype(np.float64), inp["w_sh_gate_up"], inp["w_sh_down"],
                           inp["sh_gate"], bias=bias, aux_coef=coef, **kw)


def compare_all(inp, idx, w, dout, coef, bias, name, bf16=True):
    announce(name)
    got = gpu_backward(inp, idx, w, dout, coef, bias)
    ref = oracle_backward(inp, idx, w, dout, coef, bias)
    f32 = not bf16
    worst = {"dx": check_grad("dx", got["dx"], ref["dx"], False, f32_layer=f32)}
    Fs = 0 if inp["w_sh_gate_up"] is None else inp["w_sh_gate_up"].shape[0] // 2
    for n in GRADS:
        if Fs == 0 and n in ("dw_sh_gate_up", "dw_sh_down", "dsh_gate"):
            assert got[n] is None
            continue
        worst[n] = check_grad(n, got[n], ref[n], bf16, f32_layer=f32)
    aux = float(got["aux_loss"].cpu()[0])
    assert aux == pytest.approx(ref["aux_loss"], rel=1e-4, abs=1e-12)
    announce(f"{name}: max|err|/rms " + ", ".join(f"{k} {v:.4f}" for k, v in worst.items()))
    return got, ref


def routed_case(T, d, E, k, F, Fs, dtype, seed, bias):
    inp = W.small_case(T, d, E, k, F, Fs, dtype, seed=seed)
    b = (np.random.default_rng(seed + 3).standard_normal(E) * 0.5).astype(np.float32) \
        if bias else None
    idx, w = oracle.route(inp["x"], inp["w_router"], k, bias=b)
    dout = W.make_dout(T, d, seed + 7)
    return inp, idx, w, dout, b


@pytest.mark.parametrize("T,d,E,k,F,Fs,coef,bias", [
    (300, 256, 16, 4, 128, 128, 0.001, True),   # several tiles per expert
    (200, 128, 24, 3, 64, 0, 0.01, False),      # no shared expert
    (777, 320, 8, 2, 192, 64, 0.5, True),       # ragged tiles, d and F not multiples of 128
    (20, 256, 64, 2, 128, 128, 0.001, False),   # most experts get no token: zero gradients
    (1, 256, 16, 4, 128, 128, 0.001, False),    # one token
    (1200, 256, 32, 4, 128, 128, 0.01, True),   # T >= 1024: router logits in two K slices,
                                                # dW_router over four token chunks
    (1280, 256, 32, 4, 128, 256, 0.01, False),  # T % 64 == 0: the shared expert's weight
                                                # gradients on direct-to-LDS tiles, 3 token chunks
    (512, 384, 16, 4, 128, 128, 0.001, True),   # the same with one chunk
    (160, 256, 256, 2, 128, 128, 0.001, False), # streamed weight-gradient tiles with many
                                                # experts that get no row (zero gradients)
    (600, 256, 64, 4, 256, 128, 0.01, True),    # F = 256: two 128-column slices of H per expert
    (400, 256, 16, 4, 384, 128, 0.01, True),    # G . h in two column tiles for routed rows,
                                                # one for the shared ones
    (264, 256, 16, 4, 128, 384, 0.01, False),   # ... and the other way round
])
def test_backward_bf16_layers(T, d, E, k, F, Fs, coef, bias):
    inp, idx, w, dout, b = routed_case(T, d, E, k, F, Fs, "bf16", T + E, bias)
    got, _ = compare_all(inp, idx, w, dout, coef, b,
                         f"backward bf16 T={T} d={d} E={E} k={k} F={F} Fs={Fs} coef={coef}")
    unused = np.setdiff1d(np.arange(E), idx)
    if len(unused):
        assert not got["dw_gate_up"][unused].abs().max().item()
        assert not got["dw_down"][unused].abs().max().item()


def test_backward_pure_aux_loss():
    """dout = 0: only the load-balancing loss drives the router, so the
    expert weights get exact zeros and dW_router / dx are its gradient."""
    inp, idx, w, _, b = routed_case(64, 256, 16, 4, 128, 128, "bf16", 5, True)
    dout = np.zeros((64, 256), np.float32)
    got, _ = compare_all(inp, idx, w, dout, 1.0, b, "backward: load-balancing loss only")
    for n in ("dw_gate_up", "dw_down", "dw_sh_gate_up", "dw_sh_down", "dsh_gate"):
        assert not got[n].abs().max().item(), n


@pytest.mark.parametrize("T,d,E,k,F,Fs", [
    (32, 128, 16, 4, 32, 32),    # the binary32 layer's shapes
    (9, 100, 5, 2, 33, 7),       # widths that fill no tile
])
def test_backward_f32_layers(T, d, E, k, F, Fs):
    inp, idx, w, dout, b = routed_case(T, d, E, k, F, Fs, "f32", 3, True)
    compare_all(inp, idx, w, dout, 0.01, b, f"backward f32 T={T} d={d} F={F}", bf16=False)


def test_backward_deterministic():
    inp, idx, w, dout, b = routed_case(300, 256, 16, 4, 128, 128, "bf16", 9, True)
    announce("backward determinism")
    r1 = gpu_backward(inp, idx, w, dout, 0.01, b)
    r2 = gpu_backward(inp, idx, w, dout, 0.01, b)
    for n in ("dx",) + GRADS + ("aux_loss",):
        assert torch.equal(r1[n], r2[n]), n


def test_backward_full_shapes_small_batch():
    """The pages' layer shapes (d 2560, 512 experts, top-10, widths 640) on 128
    tokens: dx of every token, every router and shared gradient, and the
    routed gradients of experts with and without tokens."""
    cfg = W.CONFIGS[3]
    lay = W.layer_for(cfg)
    T = 128
    x = W.make_x(T, cfg.d, "bf16", cfg.seed_x)
    inp = dict(lay, x=x)
    idx, w = oracle.route(x, lay["w_router"], cfg.k)
    dout = W.make_dout(T, cfg.d, 17)
    counts = np.bincount(idx.ravel(), minlength=cfg.E)
    experts = list(np.argsort(-counts, kind="stable")[:4]) + list(np.nonzero(counts == 1)[0][:2]) \
        + list(np.nonzero(counts == 0)[0][:2])
    announce(f"backward full shapes T={T}: GPU")
    got = gpu_backward(inp, idx, w, dout, 0.001)
    announce(f"backward full shapes T={T}: oracle")
    ref = oracle_backward(inp, idx, w, dout, 0.001, experts=experts)
    check_grad("dx", got["dx"], ref["dx"], False)
    for n in ("dw_router", "dw_sh_gate_up", "dw_sh_down", "dsh_gate"):
        check_grad(n, got[n], ref[n], True)
    for n in ("dw_gate_up", "dw_down"):
        check_grad(n, got[n][np.array(experts)], ref[n], True)
    assert float(got["aux_loss"].cpu()[0]) == pytest.approx(ref["aux_loss"], rel=1e-4)


@pytest.mark.slow
def test_backward_prefill_full():
    """The timed training workload (backward_T4096: T = 4096 at the pages'
    shapes) against the oracle, both from the training forward's saved
    pre-activations and router logits (the timed launch) and recomputing
    them: dx of every token, the router, shared-expert and shared-gate
    gradients in full, the routed gradients of the four busiest experts,
    three seeded ones and one no token chose, and the loss value; plus the
    softmax invariance sum_e dW_router[e] = 0 (within the bf16 rounding of
    the rows)."""
    cfg = W.CONFIGS[9]
    lay = W.layer_for(cfg)
    x = W.make_x(cfg.T, cfg.d, "bf16", cfg.seed_x)
    inp = dict(lay, x=x)
    announce(f"{cfg.name}: oracle routing")
    idx, w = oracle.route(x, lay["w_router"], cfg.k)
    dout = W.dout_for(cfg)
    announce(f"{cfg.name}: GPU, training forward then backward from its saved buffer")
    ins = {n: to_dev(inp[n]) for n in WEIGHTS}
    _, gidx, gw, saved = moe.forward_train(ins["x"], ins["w_router"], ins["w_gate_up"],
                                           ins["w_down"], cfg.k, ins["w_sh_gate_up"],
                                           ins["w_sh_down"], ins["sh_gate"])
    assert np.array_equal(gidx.cpu().numpy(), idx)
    got_saved = moe.backward(ins["x"], ins["w_router"], ins["w_gate_up"], ins["w_down"], gidx, gw,
                             to_dev(dout), ins["w_sh_gate_up"], ins["w_sh_down"], ins["sh_gate"],
                             aux_coef=cfg.aux_coef, saved=saved)
    torch.cuda.synchronize()
    announce(f"{cfg.name}: GPU, recomputing")
    got = gpu_backward(inp, idx, w, dout, cfg.aux_coef)
    counts = np.bincount(idx.ravel(), minlength=cfg.E)
    experts = list(np.argsort(-counts, kind="stable")[:4])
    experts += [e for e in np.random.default_rng(5).choice(cfg.E, 8, replace=False)
                if e not in experts][:3]
    experts += list(np.nonzero(counts == 0)[0][:1])
    experts = [int(e) for e in experts]
    announce(f"{cfg.name} backward: oracle on every token, experts {experts}")
    ref = oracle_backward(inp, idx, w, dout, cfg.aux_coef, experts=experts)
    for how, g in (("saved", got_saved), ("recomputed", got)):
        worst = {"dx": check_grad("dx", g["dx"], ref["dx"], False)}
        for n in ("dw_router", "dw_sh_gate_up", "dw_sh_down", "dsh_gate"):
            worst[n] = check_grad(n, g[n], ref[n], True)
        for n in ("dw_gate_up", "dw_down"):
            worst[n] = check_grad(n, g[n][np.array(experts)], ref[n], True)
        announce(f"{cfg.name} backward ({how}) max|err|/RMS: "
                 + ", ".join(f"{n} {v:.3e}" for n, v in worst.items()))
        assert float(g["aux_loss"].cpu()[0]) == pytest.approx(ref["aux_loss"], rel=1e-4)
        dwr = as_f64(g["dw_router"])
        assert np.abs(dwr.sum(axis=0)).max() <= 2.0 ** -8 * np.abs(dwr).sum(axis=0).max()


def permuted_rows(idx, E):
    """The pair id of every routed row in the layer's permuted order: the rows
    of expert e (ascending pair id) after those of experts < e."""
    flat = idx.ravel()
    return np.concatenate([np.nonzero(flat == e)[0] for e in range(E)])


@pytest.mark.parametrize("T,d,E,k,F,Fs,dtype", [
    (24, 256, 16, 4, 128, 128, "bf16"),     # weight-streaming path
    (300, 256, 16, 4, 128, 128, "bf16"),    # direct-to-LDS GEMM path
    (300, 256, 16, 4, 192, 64, "bf16"),     # register-staged GEMM (F % 128 != 0)
    (1000, 576, 192, 4, 640, 640, "bf16"),  # direct-to-LDS GEMM at the pages' widths
    (20, 96, 6, 2, 40, 24, "f32"),          # binary32 layer
])
def test_forward_train_saves_preactivations(T, d, E, k, F, Fs, dtype):
    """moe_forward_train gives moe_forward's outputs bit for bit, and its
    saved rows are the gate/up pre-activations x W^T of each (token, expert)
    in the permuted order, within the bf16 rounding of the stored value plus
    the binary32 accumulation."""
    inp, _, _, _, _ = routed_case(T, d, E, k, F, Fs, dtype, 61, False)
    ins = {n: to_dev(inp[n]) for n in WEIGHTS}
    announce(f"forward_train {dtype} T={T} F={F}")
    out, idx, w = moe.forward(ins["x"], ins["w_router"], ins["w_gate_up"], ins["w_down"], k,
                              ins["w_sh_gate_up"], ins["w_sh_down"], ins["sh_gate"])
    out2, idx2, w2, saved = moe.forward_train(ins["x"], ins["w_router"], ins["w_gate_up"],
                                              ins["w_down"], k, ins["w_sh_gate_up"],
                                              ins["w_sh_down"], ins["sh_gate"])
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(idx, idx2) and torch.equal(w, w2)
    es = 2 if dtype == "bf16" else 4
    raw = saved.cpu().numpy()
    au_bytes = (T * k * 2 * F + T * 2 * Fs) * es
    au = raw[:au_bytes]
    vals = (W.bf16_bits_to_f32(au.view(np.uint16)) if es == 2 else au.view(np.float32))
    vals = vals.astype(np.float64)
    routed = vals[:T * k * 2 * F].reshape(T * k, 2 * F)
    shared = vals[T * k * 2 * F:T * k * 2 * F + T * 2 * Fs].reshape(T, 2 * Fs)
    f64 = lambda a: (W.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)
    x, wgu = f64(inp["x"]), f64(inp["w_gate_up"])
    pairs = permuted_rows(idx.cpu().numpy(), E)
    kk = idx.cpu().numpy().ravel()
    ref = np.stack([wgu[kk[p]] @ x[p // k] for p in pairs])
    mag = np.stack([np.abs(wgu[kk[p]]) @ np.abs(x[p // k]) for p in pairs])
    u = 2.0 ** -8 if es == 2 else 0.0
    assert np.all(np.abs(routed - ref) <= u * np.abs(ref) + d * 2.0 ** -23 * mag + 1e-30)
    ref_sh = x @ f64(inp["w_sh_gate_up"]).T
    mag_sh = np.abs(x) @ np.abs(f64(inp["w_sh_gate_up"])).T
    assert np.all(np.abs(shared - ref_sh) <= u * np.abs(ref_sh) + d * 2.0 ** -23 * mag_sh + 1e-30)
    # with the shortlist router (bf16, T >= 128) the router logits follow:
    # K-slice partials of x [W_r; g]^T, binary32, at the next 256 bytes
    if dtype == "bf16" and T >= 128:
        off = (au_bytes + 255) // 256 * 256
        S = 2 if d % 128 == 0 else 1
        end = off + S * T * (E + 1) * 4
        lg = raw[off:end].view(np.float32).reshape(S, T, E + 1).astype(np.float64).sum(axis=0)
        wr = np.concatenate([f64(inp["w_router"]), f64(inp["sh_gate"]).reshape(1, d)])
        ref_l = x @ wr.T
        mag_l = np.abs(x) @ np.abs(wr).T
        assert np.all(np.abs(lg - ref_l) <= d * 2.0 ** -23 * mag_l + 1e-30)
        # with more than one 256-token histogram block the permutation
        # follows: rank and perm [T k] and the counts [E + 1]
        nblk = (T + 255) // 256
        if nblk > 1:
            a256 = lambda v: (v + 255) // 256 * 256
            r_off = a256(end)
            p_off = a256(r_off + T * k * 4)
            c_off = a256(p_off + T * k * 4)
            assert raw.size == c_off + (E + 1) * 4
            rank = raw[r_off:r_off + T * k * 4].view(np.int32)
            perm = raw[p_off:p_off + T * k * 4].view(np.int32)
            counts = raw[c_off:].view(np.int32)
            assert np.array_equal(perm, pairs)
            assert np.array_equal(rank[perm], np.arange(T * k))
            assert np.array_equal(counts[:E], np.bincount(kk, minlength=E)) and counts[E] == T
        else:
            assert raw.size == end
    else:
        assert raw.size == au_bytes


@pytest.mark.parametrize("T,F,dtype", [(300, 128, "bf16"), (24, 128, "bf16"), (20, 40, "f32")])
def test_backward_from_saved_preactivations(T, F, dtype):
    """moe_backward given moe_forward_train's saved pre-activations (no
    recompute) meets the same bars against the oracle."""
    d, E, k, Fs = (256, 16, 4, 128) if dtype == "bf16" else (96, 6, 2, 24)
    inp, idx, w, dout, b = routed_case(T, d, E, k, F, Fs, dtype, 71, True)
    ins = {n: to_dev(inp[n]) for n in WEIGHTS}
    announce(f"backward from saved {dtype} T={T}")
    _, gidx, gw, saved = moe.forward_train(ins["x"], ins["w_router"], ins["w_gate_up"],
                                           ins["w_down"], k, ins["w_sh_gate_up"],
                                           ins["w_sh_down"], ins["sh_gate"], bias=to_dev(b))
    assert np.array_equal(gidx.cpu().numpy(), idx)
    got = moe.backward(ins["x"], ins["w_router"], ins["w_gate_up"], ins["w_down"], gidx, gw,
                       to_dev(dout), ins["w_sh_gate_up"], ins["w_sh_down"], ins["sh_gate"],
                       bias=to_dev(b), aux_coef=0.01, saved=saved)
    torch.cuda.synchronize()
    ref = oracle_backward(inp, idx, gw.cpu().numpy().astype(np.float64), dout, 0.01, b)
    f32 = dtype == "f32"
    check_grad("dx", got["dx"], ref["dx"], False, f32_layer=f32)
    for n in GRADS:
        check_grad(n, got[n], ref[n], not f32, f32_layer=f32)
