"""Pins for the oracle's pre-FFN RMSNorm.

The pages give the norm type (RMSNorm) and eps = 1e-6 (llm-atlas
"Qwen3.8-Flash-Next", "Key facts" Norm and "Raw config fields" rms_norm_eps);
the definition is x = h / sqrt(mean(h^2) + eps) * gamma.  The oracle fixes a
binary32 evaluation order and rounds x to the layer's dtype; these tests tie
that to the definition (rounding bound against binary64, a hand-derived case)
and to exact invariances a wrong formula would break.
"""
import numpy as np
import pytest

import oracle
import workloads as W


def as_f64(a):
    return W.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def definition(h, gamma, eps):
    h64, g64 = as_f64(h), as_f64(gamma)
    return h64 / np.sqrt((h64 ** 2).mean(axis=1, keepdims=True) + eps) * g64


def test_hand_derived_case():
    """d = 64, h = (3, 4, 0, ...), gamma = 1, eps = 0: sum h^2 = 25, mean =
    25/64 = 0.390625 and sqrt = 0.625 are exact, r = 1/0.625 rounds to the
    binary32 1.6000000238 (0x3FCCCCCD).  3 r = 4.8000000715 rounds to
    0x4099999A, whose bf16 rounding (low half 0x999A above the midpoint) is
    0x409A = 4.8125; 4 r = 0x40CCCCCD exactly, bf16 0x40CD = 6.40625."""
    h = np.zeros((1, 64), np.float32)
    h[0, :2] = [3.0, 4.0]
    g = np.ones(64, np.float32)
    x = oracle.rmsnorm(W.f32_to_bf16_bits(h), W.f32_to_bf16_bits(g), eps=0.0)
    assert x[0, 0] == 0x409A and x[0, 1] == 0x40CD and not x[0, 2:].any()
    xf = oracle.rmsnorm(h, g, eps=0.0)                  # binary32 layer: no bf16 rounding
    assert xf[0, 0] == np.float32(3.0) * np.float32(1.6) and xf[0, 1] == np.float32(6.4)


@pytest.mark.parametrize("dtype,d", [("bf16", 2560), ("bf16", 640), ("f32", 100), ("bf16", 64)])
def test_within_rounding_of_the_definition(dtype, d):
    """Against the binary64 definition: within the bf16 rounding (unit
    roundoff 2^-8: 8 significant bits) plus the binary32 evaluation (a few
    2^-24); rows of very different scales, including ones where eps is not
    negligible."""
    rng = np.random.default_rng(d)
    h = rng.standard_normal((24, d)).astype(np.float32)
    h *= np.logspace(-5, 3, 24, dtype=np.float32)[:, None]
    g = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    if dtype == "bf16":
        h, g = W.f32_to_bf16_bits(h), W.f32_to_bf16_bits(g)
    eps = 1e-6
    x = as_f64(oracle.rmsnorm(h, g, eps))
    ref = definition(h, g, float(np.float32(eps)))
    rel = 2.0 ** -8 + 64 * 2.0 ** -24 if dtype == "bf16" else 64 * 2.0 ** -24
    assert np.all(np.abs(x - ref) <= rel * np.abs(ref) + 1e-30)
    # the smallest rows are visibly shrunk by eps (mean(h^2) ~ 1e-10 << eps)
    assert np.abs(x[0]).max() < 0.1 * np.abs(definition(h[:1], g, 0.0)).max()


@pytest.mark.parametrize("k", [-3, 5])
def test_power_of_two_scale_invariance(k):
    """With eps = 0, scaling h by 2^k changes every binary32 step by an exact
    power of two, so x is bit-identical: catches a missing square root, a
    wrong power or a sum where the mean belongs."""
    h = W.make_x(16, 512, "bf16", 3)
    g = W.make_x(1, 512, "bf16", 4)[0]
    hs = W.f32_to_bf16_bits(W.bf16_bits_to_f32(h) * np.float32(2.0 ** k))
    assert np.array_equal(oracle.rmsnorm(hs, g, 0.0), oracle.rmsnorm(h, g, 0.0))


def test_gamma_doubling_doubles_x():
    h = W.make_x(8, 256, "bf16", 5)
    g = W.make_x(1, 256, "bf16", 6)[0]
    g2 = W.f32_to_bf16_bits(W.bf16_bits_to_f32(g) * np.float32(2.0))
    x, x2 = as_f64(oracle.rmsnorm(h, g)), as_f64(oracle.rmsnorm(h, g2))
    assert np.array_equal(x2, 2 * x)


def test_rows_are_independent():
    h = W.make_x(20, 256, "bf16", 7)
    g = W.make_x(1, 256, "bf16", 8)[0]
    full = oracle.rmsnorm(h, g)
    assert np.array_equal(oracle.rmsnorm(np.ascontiguousarray(h[5:9]), g), full[5:9])


def test_prenorm_block_with_residual_equals_textbook():
    """The whole pre-norm block with its residual update, k = 1 and no shared
    expert: resid + SwiGLU_e(RMSNorm(h)) with the definition's binary64 norm
    (no canonical order, no bf16 rounding of the normalised row beyond the
    oracle's own) and a dense numpy gated MLP.  A residual taken from the
    wrong operand, a dropped term or a doubled output fails."""
    from scipy.special import expit

    T, d, E, F = 9, 128, 6, 32
    inp = W.small_case(T, d, E, 1, F, 0, "f32", seed=41)
    h = (2.0 * inp["x"]).astype(np.float32)
    g = W.make_norm_weight(d, "f32", 3)
    resid = np.random.default_rng(4).standard_normal((T, d)).astype(np.float32)
    x = oracle.rmsnorm(h, g, 1e-6)
    out, idx, _, _ = oracle.forward(x, inp["w_router"], inp["w_gate_up"], inp["w_down"], 1)
    res = oracle.residual(resid, out)
    xd = definition(h, g, 1e-6)
    gu, dn = inp["w_gate_up"].astype(np.float64), inp["w_down"].astype(np.float64)
    for t in range(T):
        e = idx[t, 0]
        a, u = gu[e, :F] @ xd[t], gu[e, F:] @ xd[t]
        ref = resid[t].astype(np.float64) + dn[e] @ (a * expit(a) * u)
        # x is binary32 (one rounding per step of the fixed order): 1e-5 relative
        assert np.allclose(res[t], ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())
    assert np.array_equal(oracle.residual(resid, np.zeros_like(out)), resid.astype(np.float64))
    assert np.array_equal(oracle.residual(np.zeros_like(resid), out), out)
