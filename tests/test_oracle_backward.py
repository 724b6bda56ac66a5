"""Pins for the oracle's backward pass (oracle.backward).

The backward is the derivative of sum(dout * out) + L_aux with the routing
held fixed, L_aux = coef * E * sum_e f_e P_e (f_e: share of the T*k routed
assignments sent to e; P_e: mean softmax probability of e).  The pages give
only the loss coefficient (llm-atlas "Qwen3.8-Flash-Next", "Raw config
fields", router_aux_loss_coef = 0.001); the formula is the reading stated in
the oracle.  What pins the oracle's hand-written chain rule here:
  * torch's automatic differentiation of the same scalar, written as a plain
    binary64 forward (checked first against the oracle's own, separately
    pinned, forward), on every gradient at once;
  * central finite differences of that forward on sampled coordinates;
  * closed forms: L_aux = coef exactly when every expert gets the same share
    and the router is zero; a single expert reduces the layer to one dense
    gated MLP, whose gradient is textbook;
  * invariants: the router gradient's rows sum to zero over experts (softmax
    is shift invariant), gradients are linear in dout, and zero dout with a
    zero coefficient gives zero gradients.
No test here needs a GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

NAMES = ("x", "w_router", "w_gate_up", "w_down", "w_sh_gate_up", "w_sh_down", "sh_gate")
GRADS = ("dx", "dw_router", "dw_gate_up", "dw_down", "dw_sh_gate_up", "dw_sh_down", "dsh_gate")


def case(T=7, d=32, E=6, k=2, F=16, Fs=8, seed=3, bias=True):
    inp = W.small_case(T, d, E, k, F, Fs, "f32", seed=seed)
    inp["bias"] = (np.random.default_rng(seed + 9).standard_normal(E) * 0.5).astype(np.float32) \
        if bias else None
    idx, _ = oracle.route(inp["x"], inp["w_router"], k, bias=inp["bias"])
    dout = np.random.default_rng(seed + 5).standard_normal((T, d))
    return inp, idx, dout


def torch_loss(params, idx, dout, coef, bias, F, Fs):
    """sum(dout * out) + coef * E * sum_e f_e P_e, binary64, routing fixed."""
    x, wr, wgu, wdn, wsgu, wsdn, g = params
    T, k = idx.shape
    E = wr.shape[0]
    it = torch.from_numpy(idx.astype(np.int64))
    l = x @ wr.T + (0.0 if bias is None else torch.from_numpy(bias.astype(np.float64)))
    p = torch.softmax(l, dim=1)
    w = torch.softmax(torch.gather(l, 1, it), dim=1)
    out = torch.zeros_like(x)
    for j in range(k):
        e = it[:, j]
        a = torch.einsum("td,tfd->tf", x, wgu[e, :F])
        u = torch.einsum("td,tfd->tf", x, wgu[e, F:])
        h = torch.nn.functional.silu(a) * u
        out = out + w[:, j:j + 1] * torch.einsum("tmf,tf->tm", wdn[e], h)
    if Fs:
        s = torch.sigmoid(x @ g)
        hs = torch.nn.functional.silu(x @ wsgu[:Fs].T) * (x @ wsgu[Fs:].T)
        out = out + s[:, None] * (hs @ wsdn.T)
    f = torch.bincount(it.reshape(-1), minlength=E).double() / (T * k)
    aux = coef * E * (f * p.mean(0)).sum()
    return (torch.from_numpy(dout) * out).sum() + aux, out, w, aux


def params64(inp):
    """binary64 leaves of every input (a one-element zero stands in for an
    absent shared expert)."""
    return [torch.tensor(np.zeros(1) if inp[n] is None else inp[n].astype(np.float64),
                         requires_grad=True) for n in NAMES]


def run_oracle(inp, idx, w, dout, coef, **kw):
    return oracle.backward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], idx, w,
                           dout, inp["w_sh_gate_up"], inp["w_sh_down"], inp["sh_gate"],
                           bias=inp["bias"], aux_coef=coef, **kw)


def test_torch_forward_matches_oracle_forward():
    """The binary64 forward used below is the oracle's expert stage (already
    pinned) on the same routing: it differentiates the right function."""
    inp, idx, dout = case()
    P = params64(inp)
    _, out, w, _ = torch_loss(P, idx, dout, 0.0, inp["bias"], 16, 8)
    ref = oracle.experts(inp["x"], inp["w_gate_up"], inp["w_down"], idx, w.detach().numpy(),
                         inp["w_sh_gate_up"], inp["w_sh_down"], inp["sh_gate"])
    assert np.allclose(out.detach().numpy(), ref, rtol=0, atol=1e-12)
    _, w_or = oracle.route(inp["x"], inp["w_router"], idx.shape[1], bias=inp["bias"])
    assert np.allclose(w.detach().numpy(), w_or, atol=1e-6)   # binary32 vs binary64 logits


@pytest.mark.parametrize("coef", [0.0, 0.001, 0.7])
@pytest.mark.parametrize("shape", [dict(), dict(T=9, E=8, k=3, Fs=0, seed=4),
                                   dict(T=4, E=5, k=5, seed=6, bias=False)])
def test_every_gradient_matches_autograd(coef, shape):
    inp, idx, dout = case(**shape)
    F = inp["w_gate_up"].shape[1] // 2
    Fs = 0 if inp["w_sh_gate_up"] is None else inp["w_sh_gate_up"].shape[0] // 2
    P = params64(inp)
    L, _, w, aux = torch_loss(P, idx, dout, coef, inp["bias"], F, Fs)
    L.backward()
    r = run_oracle(inp, idx, w.detach().numpy(), dout, coef)
    assert r["aux_loss"] == pytest.approx(aux.item(), rel=1e-12, abs=1e-15)
    for name, p in zip(GRADS, P):
        if Fs == 0 and name in ("dw_sh_gate_up", "dw_sh_down", "dsh_gate"):
            continue
        ref = p.grad.numpy()
        got = r[name]
        assert got.shape == ref.shape, name
        scale = np.abs(ref).max()
        assert scale > 0, name
        assert np.abs(got - ref).max() <= 1e-11 * scale, name


def test_finite_differences_on_sampled_coordinates():
    """Central differences (step 1e-5, error ~ 1e-10 relative) of the binary64
    scalar at a few coordinates of every input."""
    coef = 0.05
    inp, idx, dout = case(seed=11)
    F, Fs = 16, 8
    P = params64(inp)
    _, _, w, _ = torch_loss(P, idx, dout, coef, inp["bias"], F, Fs)
    r = run_oracle(inp, idx, w.detach().numpy(), dout, coef)
    rng = np.random.default_rng(2)
    for name, gname in zip(NAMES, GRADS):
        base = [q.detach().clone() for q in P]
        i = NAMES.index(name)
        for _ in range(4):
            pos = tuple(int(rng.integers(0, n)) for n in base[i].shape)
            hstep = 1e-5
            vals = []
            for sgn in (1, -1):
                q = [b.clone() for b in base]
                q[i][pos] += sgn * hstep
                vals.append(torch_loss(q, idx, dout, coef, inp["bias"], F, Fs)[0].item())
            fd = (vals[0] - vals[1]) / (2 * hstep)
            assert r[gname][pos] == pytest.approx(fd, rel=1e-6, abs=1e-9), (name, pos)


def test_aux_loss_closed_form_at_balance():
    """Zero router and no bias: p = 1/E for every token.  A routing that gives
    every expert the same share makes L_aux = coef exactly, and its gradient
    p_e (f_e - sum f p) vanishes, so dx and dW_router carry only the routed
    terms (zero here, with dout = 0)."""
    T, d, E, k, F = 6, 16, 6, 2, 8
    inp = W.small_case(T, d, E, k, F, 0, "f32", seed=2)
    inp["w_router"][:] = 0
    inp["bias"] = None
    idx = np.array([[0, 1], [2, 3], [4, 5], [1, 0], [3, 2], [5, 4]], np.int32)
    w = np.full((T, k), 0.5)
    r = run_oracle(inp, idx, w, np.zeros((T, d)), 0.001)
    assert r["aux_loss"] == pytest.approx(0.001, rel=1e-14)
    # zero up to the rounding of f and p (1e-16 relative to terms of size ~1)
    assert np.abs(r["dw_router"]).max() < 1e-17 and np.abs(r["dx"]).max() < 1e-17


def test_single_expert_is_one_dense_gated_mlp():
    """E = k = 1: w = 1 and the router gets no gradient; dx and the weight
    gradients are those of one gated MLP y = W_dn (silu(W_g x) * W_u x),
    written out by hand: with G = W_dn^T dout, dh = G, da = dh u silu'(a),
    du = dh silu(a), dx = W_g^T da + W_u^T du, dW_dn = dout h^T."""
    T, d, F = 5, 24, 12
    inp = W.small_case(T, d, 1, 1, F, 0, "f32", seed=8)
    inp["bias"] = None
    idx = np.zeros((T, 1), np.int32)
    dout = np.random.default_rng(1).standard_normal((T, d))
    r = run_oracle(inp, idx, np.ones((T, 1)), dout, 0.3)
    x = inp["x"].astype(np.float64)
    wg, wu = inp["w_gate_up"][0, :F].astype(np.float64), inp["w_gate_up"][0, F:].astype(np.float64)
    wd = inp["w_down"][0].astype(np.float64)
    a, u = x @ wg.T, x @ wu.T
    sg = 1 / (1 + np.exp(-a))
    h = a * sg * u
    G = dout @ wd
    da, du = G * u * sg * (1 + a * (1 - sg)), G * a * sg
    assert np.allclose(r["dx"], da @ wg + du @ wu, rtol=1e-12, atol=1e-14)
    assert np.allclose(r["dw_down"][0], dout.T @ h, rtol=1e-12, atol=1e-14)
    assert np.allclose(r["dw_gate_up"][0], np.vstack([da.T @ x, du.T @ x]), rtol=1e-12, atol=1e-14)
    assert np.abs(r["dw_router"]).max() == 0
    assert r["aux_loss"] == pytest.approx(0.3)          # f = p = 1


def test_router_gradient_rows_sum_to_zero():
    inp, idx, dout = case(T=10, E=8, k=3, seed=21)
    _, w = oracle.route(inp["x"], inp["w_router"], 3, bias=inp["bias"])
    r = run_oracle(inp, idx, w, dout, 0.2)
    scale = np.abs(r["dw_router"]).max()
    assert scale > 0 and np.abs(r["dw_router"].sum(axis=0)).max() < 1e-13 * scale * 8


def test_linear_in_dout_and_zero_at_zero():
    inp, idx, dout = case(seed=31)
    _, w = oracle.route(inp["x"], inp["w_router"], 2, bias=inp["bias"])
    r1 = run_oracle(inp, idx, w, dout, 0.0)
    r3 = run_oracle(inp, idx, w, 3 * dout, 0.0)
    r0 = run_oracle(inp, idx, w, 0 * dout, 0.0)
    for g in GRADS:
        assert np.allclose(r3[g], 3 * r1[g], rtol=1e-12, atol=1e-15), g
        assert np.abs(r0[g]).max() == 0, g


def test_selected_parts_agree_with_the_full_call():
    """Restricting the work to some tokens and experts gives the same values
    for what is computed (NaN rows for the other tokens, only the listed
    experts' weight gradients, in the order listed)."""
    inp, idx, dout = case(T=9, E=8, k=3, seed=41)
    _, w = oracle.route(inp["x"], inp["w_router"], 3, bias=inp["bias"])
    full = run_oracle(inp, idx, w, dout, 0.01)
    part = run_oracle(inp, idx, w, dout, 0.01, parts=oracle.DX | oracle.DW_ROUTED,
                      tokens=[0, 4, 8], experts=[2, 5])
    assert np.array_equal(part["dx"][[0, 4, 8]], full["dx"][[0, 4, 8]])
    assert np.isnan(part["dx"][1]).all()
    assert np.array_equal(part["dw_gate_up"], full["dw_gate_up"][[2, 5]])
    assert np.array_equal(part["dw_down"], full["dw_down"][[2, 5]])
    assert part["dw_router"] is None and part["dw_sh_down"] is None
    assert part["aux_loss"] == full["aux_loss"]
    rev = run_oracle(inp, idx, w, dout, 0.01, parts=oracle.DW_ROUTED, experts=[5, 2])
    assert np.array_equal(rev["dw_gate_up"], full["dw_gate_up"][[5, 2]])


def test_bfloat16_inputs_are_widened_exactly():
    """bf16 inputs give the gradient of the layer at the widened values."""
    inp32, idx, dout = case(seed=51, bias=False)
    bf = {n: W.f32_to_bf16_bits(inp32[n]) for n in NAMES}
    wid = {n: W.bf16_bits_to_f32(bf[n]) for n in NAMES}
    _, w = oracle.route(bf["x"], bf["w_router"], 2)
    r16 = oracle.backward(bf["x"], bf["w_router"], bf["w_gate_up"], bf["w_down"], idx, w, dout,
                          bf["w_sh_gate_up"], bf["w_sh_down"], bf["sh_gate"], aux_coef=0.01)
    r32 = oracle.backward(wid["x"], wid["w_router"], wid["w_gate_up"], wid["w_down"], idx, w,
                          dout, wid["w_sh_gate_up"], wid["w_sh_down"], wid["sh_gate"],
                          aux_coef=0.01)
    for g in GRADS + ("aux_loss",):
        assert np.array_equal(r16[g], r32[g]), g
