"""Pins for the CPU oracle, checked against what the pages and mathematics fix.

Each test names the mistake it would catch.  No test here needs a GPU.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def widen(a):
    """bf16 bits / float32 -> float64 (exact)."""
    if a.dtype == np.uint16:
        return W.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def to_dtype(a64, dtype):
    a32 = np.ascontiguousarray(a64, dtype=np.float32)
    return W.f32_to_bf16_bits(a32) if dtype == "bf16" else a32


def dense_swiglu(x64, gu64, dn64):
    """Textbook gated MLP in numpy fp64: W_dn (silu(W_g x) * (W_u x))."""
    F = gu64.shape[0] // 2
    a = gu64[:F] @ x64
    u = gu64[F:] @ x64
    return dn64 @ (a * expit(a) * u)


# ---------------------------------------------------------------- router logit

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_canonical_order_fixtures(dtype):
    """Hand-derived fixtures fix the binary32 accumulation order; a wrong lane
    mapping, chunk order or reduction tree gives a different value."""
    cases = json.load(open(os.path.join(GOLDEN, "canonical_order.json")))["cases"]
    for c in cases:
        x = np.zeros((1, c["d"]), np.float64)
        w = np.zeros((1, c["d"]), np.float64)
        for kk, xv, wv in c["nonzero"]:
            x[0, kk], w[0, kk] = xv, wv
        l = oracle.router_logits(to_dtype(x, dtype), to_dtype(w, dtype))
        assert l[0, 0] == np.float32(c["expected_logit"]), c["name"]


@pytest.mark.parametrize("dtype,d", [("f32", 300), ("bf16", 1100), ("f32", 40)])
def test_logit_within_rounding_bound_of_exact(dtype, d):
    """|l - exact| <= (n_seq + 6) u sum|x_k w_k| with the exact dot product in
    rational arithmetic: a dropped term, wrong index or wrong operand blows
    far past this bound."""
    rng = np.random.default_rng(3)
    T, E = 3, 5
    x = to_dtype(rng.standard_normal((T, d)), dtype)
    wr = to_dtype(0.02 * rng.standard_normal((E, d)), dtype)
    b = rng.standard_normal(E).astype(np.float32)
    l = oracle.router_logits(x, wr, b)
    xf, wf = widen(x), widen(wr)
    depth = 8 * math.ceil(d / 512) + 6 + 1
    u = 2.0 ** -24
    for t in range(T):
        for e in range(E):
            exact = sum((Fraction(float(xf[t, i])) * Fraction(float(wf[e, i])) for i in range(d)),
                        Fraction(0)) + Fraction(float(b[e]))
            bound = depth * u * (float(np.abs(xf[t] * wf[e]).sum()) + abs(float(b[e])))
            assert abs(float(Fraction(float(l[t, e])) - exact)) <= bound


# ---------------------------------------------------------------- selection

def test_topk_is_prefix_of_full_sort():
    """Top-k = the first k of a full (value desc, index asc) sort, done here
    by numpy's lexsort; catches ascending selection or wrong tie order."""
    inp = W.small_case(64, 256, 32, 6, 16, 16, "bf16", seed=11)
    idx, _, logits = oracle.route(inp["x"], inp["w_router"], 6, return_logits=True)
    for t in range(64):
        order = np.lexsort((np.arange(32), -logits[t].astype(np.float64)))
        assert np.array_equal(idx[t], order[:6])


def test_topk_set_maximises_selected_sum_brute_force():
    """Brute force over all C(E,k) subsets: with distinct logits the selected
    set is the unique subset with the largest logit sum."""
    inp = W.small_case(16, 64, 8, 3, 8, 0, "f32", seed=5)
    idx, _, logits = oracle.route(inp["x"], inp["w_router"], 3, return_logits=True)
    for t in range(16):
        l = logits[t].astype(np.float64)
        best = max(itertools.combinations(range(8), 3), key=lambda s: sum(l[list(s)]))
        assert set(idx[t]) == set(best)
        assert all(l[idx[t][i]] >= l[idx[t][i + 1]] for i in range(2))


def test_zero_router_ties_go_to_lower_index():
    """All logits equal: topk_idx = [0..k-1] and the weights are 1/k."""
    T, d, E, k = 5, 64, 12, 4
    x = to_dtype(np.random.default_rng(0).standard_normal((T, d)), "bf16")
    wr = np.zeros((E, d), np.uint16)
    idx, w = oracle.route(x, wr, k)
    assert (idx == np.arange(k)).all()
    assert np.allclose(w, 1.0 / k, rtol=0, atol=1e-15)


def test_duplicate_router_rows_lower_index_first():
    """Two identical router rows tie on every token; whenever both are picked
    the lower index comes first, and when one is picked it is the lower."""
    inp = W.small_case(200, 128, 16, 5, 8, 0, "bf16", seed=21)
    wr = inp["w_router"].copy()
    wr[9] = wr[3]
    idx, _ = oracle.route(inp["x"], wr, 5)
    for row in idx:
        s = list(row)
        assert not (9 in s and 3 not in s)
        if 9 in s:
            assert s.index(3) + 1 == s.index(9)


def test_bias_added_after_dot():
    """A large bias on one expert selects it for every token."""
    inp = W.small_case(40, 128, 16, 3, 8, 0, "f32", seed=2)
    b = np.zeros(16, np.float32)
    b[13] = 50.0
    idx, _ = oracle.route(inp["x"], inp["w_router"], 3, bias=b)
    assert (idx[:, 0] == 13).all()


def test_minus_infinity_bias_masks_experts():
    """A -inf bias masks an expert: the finite experts come first in logit
    order, then the masked ones by ascending index (the full sort's order for
    equal keys), with weight exactly 0; the finite weights are the softmax
    over the finite selected logits."""
    inp = W.small_case(30, 128, 16, 6, 8, 0, "bf16", seed=6)
    b = np.full(16, -np.inf, np.float32)
    keep = [2, 7, 11, 12]
    b[keep] = 0.0
    idx, w, logits = oracle.route(inp["x"], inp["w_router"], 6, bias=b, return_logits=True)
    for t in range(30):
        l = logits[t].astype(np.float64)
        order = sorted(keep, key=lambda e: (-l[e], e))
        assert list(idx[t]) == order + [0, 1]
        assert (w[t, 4:] == 0.0).all()
        assert np.allclose(w[t, :4], softmax(l[order]), rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- weights

def test_weights_sum_to_one_and_equal_softmax_of_selected():
    """sum w = 1 and w = softmax over the selected logits alone (a closed
    form different from the oracle's full-softmax-then-renormalise path)."""
    inp = W.small_case(50, 256, 64, 10, 8, 0, "bf16", seed=4)
    idx, w, logits = oracle.route(inp["x"], inp["w_router"], 10, return_logits=True)
    assert np.abs(w.sum(1) - 1.0).max() < 1e-12
    sel = np.take_along_axis(logits.astype(np.float64), idx, 1)
    assert np.allclose(w, softmax(sel, axis=1), rtol=1e-12, atol=1e-15)
    assert (np.diff(w, axis=1) <= 1e-15).all()      # descending logits -> descending weights


def test_k_equals_E_gives_full_softmax_and_k1_gives_one():
    inp = W.small_case(20, 128, 16, 16, 8, 0, "f32", seed=8)
    idx, w, logits = oracle.route(inp["x"], inp["w_router"], 16, return_logits=True)
    p = softmax(logits.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(p, idx, 1), rtol=1e-12, atol=1e-15)
    idx1, w1 = oracle.route(inp["x"], inp["w_router"], 1)
    assert (w1 == 1.0).all()
    assert (idx1[:, 0] == idx[:, 0]).all()


# ---------------------------------------------------------------- experts

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_hot_routing_no_shared_equals_dense_swiglu(dtype):
    """k = 1 and no shared expert: out is one dense gated MLP (numpy matmul).
    Catches swapped gate/up halves, a transposed weight, a missing SiLU."""
    T, d, E, F = 12, 96, 6, 40
    inp = W.small_case(T, d, E, 1, F, 0, dtype, seed=13)
    out, idx, w, _ = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"],
                                    inp["w_down"], 1)
    assert (w == 1.0).all()
    xf, gu, dn = widen(inp["x"]), widen(inp["w_gate_up"]), widen(inp["w_down"])
    for t in range(T):
        ref = dense_swiglu(xf[t], gu[idx[t, 0]], dn[idx[t, 0]])
        assert np.allclose(out[t], ref, rtol=1e-12, atol=1e-14)


def test_all_experts_selected_equals_softmax_mixture():
    """k = E, no shared expert: out = sum_e softmax(l)_e * SwiGLU_e(x), every
    expert computed densely.  Catches weights attached to the wrong expert."""
    T, d, E, F = 6, 64, 8, 24
    inp = W.small_case(T, d, E, E, F, 0, "f32", seed=17)
    out, idx, w, _ = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"],
                                    inp["w_down"], E)
    logits = oracle.router_logits(inp["x"], inp["w_router"]).astype(np.float64)
    p = softmax(logits, axis=1)
    xf, gu, dn = widen(inp["x"]), widen(inp["w_gate_up"]), widen(inp["w_down"])
    for t in range(T):
        ref = sum(p[t, e] * dense_swiglu(xf[t], gu[e], dn[e]) for e in range(E))
        assert np.allclose(out[t], ref, rtol=1e-11, atol=1e-14)


def test_scaling_down_projection_doubles_output_exactly():
    inp = W.small_case(10, 128, 16, 4, 32, 32, "bf16", seed=9)
    args = dict(w_sh_gate_up=inp["w_sh_gate_up"], sh_gate=inp["sh_gate"])
    out1, _, _, _ = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"],
                                   4, w_sh_down=inp["w_sh_down"], **args)
    dbl = lambda a: to_dtype(2.0 * widen(a), "bf16")
    out2, _, _, _ = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"],
                                   dbl(inp["w_down"]), 4, w_sh_down=dbl(inp["w_sh_down"]), **args)
    assert np.array_equal(out2, 2.0 * out1)


def test_zero_gate_vector_gives_half():
    inp = W.small_case(7, 64, 8, 2, 16, 16, "f32", seed=6)
    g0 = np.zeros_like(inp["sh_gate"])
    _, _, _, s = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], 2,
                                inp["w_sh_gate_up"], inp["w_sh_down"], g0)
    assert (s == 0.5).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shared_expert_alone_is_sigmoid_gated_dense_swiglu(dtype):
    """Routed down-projections zeroed: out = sigmoid(g.x) * SwiGLU_shared(x).
    Catches a dropped or unscaled shared term and a gate on the wrong side."""
    T, d, E, F, Fs = 9, 128, 8, 16, 48
    inp = W.small_case(T, d, E, 3, F, Fs, dtype, seed=23)
    zero_dn = np.zeros_like(inp["w_down"])
    out, _, _, s = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], zero_dn, 3,
                                  inp["w_sh_gate_up"], inp["w_sh_down"], inp["sh_gate"])
    xf = widen(inp["x"])
    gate = expit(xf @ widen(inp["sh_gate"]))
    assert np.allclose(s, gate, rtol=1e-13, atol=0)
    for t in range(T):
        ref = gate[t] * dense_swiglu(xf[t], widen(inp["w_sh_gate_up"]), widen(inp["w_sh_down"]))
        assert np.allclose(out[t], ref, rtol=1e-12, atol=1e-14)


def test_experts_entry_matches_forward_with_its_routing():
    inp = W.small_case(15, 128, 16, 4, 32, 32, "bf16", seed=31)
    lay = [inp["w_sh_gate_up"], inp["w_sh_down"], inp["sh_gate"]]
    out, idx, w, s = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"],
                                    4, *lay)
    out2, s2 = oracle.experts(inp["x"], inp["w_gate_up"], inp["w_down"], idx, w, *lay,
                              return_gate=True)
    assert np.array_equal(out, out2) and np.array_equal(s, s2)


# ---------------------------------------------------------------- whole layer

def test_tokens_are_independent_batch_split():
    """Any split of the batch gives bit-identical results per token."""
    inp = W.small_case(37, 128, 16, 4, 32, 32, "bf16", seed=41)
    lay = [inp["w_sh_gate_up"], inp["w_sh_down"], inp["sh_gate"]]
    full = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], 4, *lay)
    for a, b in [(0, 5), (5, 6), (6, 37)]:
        part = oracle.forward(np.ascontiguousarray(inp["x"][a:b]), inp["w_router"],
                              inp["w_gate_up"], inp["w_down"], 4, *lay)
        for f, p in zip(full, part):
            assert np.array_equal(f[a:b], p)


def test_expert_relabelling_equivariance():
    """Permuting the experts permutes topk_idx and leaves out unchanged."""
    inp = W.small_case(20, 128, 16, 4, 16, 16, "bf16", seed=43)
    lay = [inp["w_sh_gate_up"], inp["w_sh_down"], inp["sh_gate"]]
    out, idx, w, _ = oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"],
                                    inp["w_down"], 4, *lay)
    perm = np.random.default_rng(1).permutation(16)          # new expert i = old perm[i]
    inv = np.argsort(perm)
    out2, idx2, w2, _ = oracle.forward(inp["x"], np.ascontiguousarray(inp["w_router"][perm]),
                                       np.ascontiguousarray(inp["w_gate_up"][perm]),
                                       np.ascontiguousarray(inp["w_down"][perm]), 4, *lay)
    assert np.array_equal(inv[idx], idx2)
    # the full-softmax denominator sums in index order: last-bit differences only
    assert np.allclose(w, w2, rtol=1e-14, atol=0)
    assert np.allclose(out, out2, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- pages

def test_layer_shapes_match_pages_and_totals():
    """The configured full-size layer has the pages' shapes, and those shapes
    are consistent with the stated whole-model parameter totals."""
    g = json.load(open(os.path.join(GOLDEN, "layer_shapes.json")))
    for c in (W.CONFIGS[2], W.CONFIGS[3], W.CONFIGS[4], W.CONFIGS[5]):
        assert (c.d, c.E, c.k, c.F, c.Fs) == (g["d_model"]["value"], g["n_experts"]["value"],
                                              g["top_k"]["value"], g["d_expert"]["value"],
                                              g["d_shared"]["value"])
        assert c.dtype == "bf16"
    L, d, E, k, F = (g["n_layers"]["value"], g["d_model"]["value"], g["n_experts"]["value"],
                     g["top_k"]["value"], g["d_expert"]["value"])
    routed = L * E * 3 * d * F
    lo, hi = g["total_params_core"]["value_billions"]
    assert 0.9 * lo * 1e9 < routed < hi * 1e9          # routed experts are most of the core
    active_moe = L * ((k + 1) * 3 * d * F + E * d)
    a_lo, a_hi = g["active_params"]["value_billions"]
    assert active_moe < a_lo * 1e9                     # MoE share fits inside the active count
    assert W.WEIGHT_STD == g["init_std"]["value"]
