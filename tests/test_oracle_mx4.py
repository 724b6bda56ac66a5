"""Pins for the oracle's MXFP4 expert weights and for the MXFP4 input writer.

The pages say only that the published weights are packed low-bit tensors
(llm-atlas "Qwen3.8-Flash-Next", "Modelled costs"); the encoding read into
that is MXFP4 of the OCP Microscaling (MX) specification v1.0.  The decoder is
pinned to the specification's FP4 E2M1 value set (all 16 codes), to torch's
own E8M0 scale type, and to a one-hot placement of single codes (nibble order,
row and block indexing).  The layer with MXFP4 weights is then pinned to the
already-pinned bfloat16 layer run on the decoded weights.  No test here needs
a GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

# FP4 E2M1 (OCP MX v1.0, FP4 element format): sign bit 3, exponent bits 2..1
# with bias 1, mantissa bit 0.  The representable magnitudes by code 0..7 are
# 0, 0.5, 1, 1.5, 2, 3, 4, 6; codes 8..15 are their negatives.
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _pack(codes4):
    """[..., K] codes 0..15 -> [..., K/2] bytes, element 2i in the low nibble."""
    c = np.asarray(codes4, np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def test_e2m1_all_sixteen_codes():
    """A wrong exponent bias, a missing subnormal case or a wrong sign bit
    changes one of the 16 values."""
    codes4 = np.zeros((1, 32), np.uint8)
    codes4[0, :16] = np.arange(16)
    scales = np.full((1, 1), 127, np.uint8)          # 2^0
    v = oracle.mx4_decode(_pack(codes4), scales)[0, :16]
    expect = E2M1_MAGNITUDES + [-m for m in E2M1_MAGNITUDES]
    assert v.tolist() == expect
    assert np.signbit(v[8]) and not np.signbit(v[0])   # code 8 is -0


def test_e8m0_scales_match_torch():
    """Every scale byte decodes as torch's float8_e8m0fnu does (2^(X-127);
    255 is NaN): catches an off-by-one bias or a clamped exponent."""
    X = np.arange(256, dtype=np.uint8)
    codes4 = np.full((256, 32), 2, np.uint8)          # every element 1.0
    v = oracle.mx4_decode(_pack(codes4), X.reshape(256, 1))[:, 0]
    ref = torch.from_numpy(X.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(v[:255], ref[:255])
    assert np.isnan(v[255]) and np.isnan(ref[255])


@pytest.mark.parametrize("row,kk", [(0, 0), (0, 1), (1, 31), (2, 32), (2, 33), (3, 95)])
def test_one_hot_code_lands_where_placed(row, kk):
    """One non-zero code placed at (row, kk) with its block's scale decodes at
    exactly that element and nowhere else: pins the nibble order (even element
    in the low nibble), the row stride and the block index of the scale."""
    rows, K = 4, 96
    codes4 = np.zeros((rows, K), np.uint8)
    codes4[row, kk] = 13                               # -3.0
    scales = np.full((rows, K // 32), 127, np.uint8)
    scales[row, kk // 32] = 127 - 5                    # 2^-5 on that block only
    v = oracle.mx4_decode(_pack(codes4), scales)
    expect = np.zeros((rows, K))
    expect[row, kk] = -3.0 / 32
    assert np.array_equal(v, expect)


def test_writer_round_trips_representable_values():
    """Values already on the MXFP4 grid (and whose block maximum fixes the
    same scale) come back unchanged from the writer and the decoder."""
    rng = np.random.default_rng(3)
    rows, K = 6, 64
    X = rng.integers(100, 140, size=(rows, K // 32))
    mags = rng.choice(E2M1_MAGNITUDES, size=(rows, K))
    mags[:, ::32] = 6.0                                # each block's maximum is 6
    signs = rng.choice([-1.0, 1.0], size=(rows, K))
    vals = signs * mags * np.ldexp(1.0, np.repeat(X - 127, 32, axis=1))
    codes, scales, wvals = W.mx4_quantize(vals.astype(np.float32), with_values=True)
    assert np.array_equal(scales, X.astype(np.uint8))
    assert np.array_equal(wvals.astype(np.float64), vals)
    assert np.array_equal(oracle.mx4_decode(codes, scales), vals)


def test_writer_rounds_to_nearest_ties_to_even_and_saturates():
    """Midpoints go to the even code; magnitudes between 6 and 8 (scaled)
    saturate to 6; the shared exponent is floor(log2 max) - 2."""
    blk = np.zeros(32, np.float32)
    probes = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.3, 2.6, 7.9, -0.75, -5.0]
    blk[:len(probes)] = probes
    codes, scales, vals = W.mx4_quantize(blk[None], with_values=True)
    assert scales[0, 0] == 127                         # max 7.9: floor(log2) = 2
    assert vals[0, :len(probes)].tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0,
                                              0.5, 3.0, 6.0, -1.0, -4.0]
    assert np.array_equal(oracle.mx4_decode(codes, scales)[0], vals[0].astype(np.float64))


def test_writer_error_bound_and_decoder_agree_on_random_weights():
    """On N(0, 0.02^2) draws, element by element in scaled units u = 2^(X-127):
    |v - q| <= 1 u (half the widest E2M1 gap) where |v| <= 6 u, and
    q = sign(v) 6 u where |v| > 6 u (saturation; |v| < 8 u by the choice of X).
    The decoder reproduces the writer's values exactly (an independent
    encoder/decoder pair)."""
    a = (np.random.default_rng(5).standard_normal((64, 256)) * 0.02).astype(np.float32)
    codes, scales, vals = W.mx4_quantize(a, with_values=True)
    u = np.ldexp(1.0, np.repeat(scales.astype(np.int64) - 127, 32, axis=1))
    v = a.astype(np.float64)
    inner = np.abs(v) <= 6 * u
    assert np.all(np.abs(v - vals)[inner] <= u[inner])
    assert np.all((vals == np.sign(v) * 6 * u)[~inner]) and np.all(np.abs(v) < 8 * u)
    assert inner.mean() < 1.0                        # saturation does occur
    assert np.array_equal(oracle.mx4_decode(codes, scales), vals.astype(np.float64))


def _small_mx4_layer(T=12, d=96, E=6, k=3, F=64, Fs=32, seed=11):
    lay = W.make_layer_mx4(d, E, F, Fs, seed, with_values=True)
    x = W.make_x(T, d, "bf16", seed + 1)
    return lay, x, k


def _values_as_bf16(v):
    b = W.f32_to_bf16_bits(v)
    assert np.array_equal(W.bf16_bits_to_f32(b), v), "decoded weights must be exact in bf16"
    return b


def test_mx4_layer_equals_bf16_layer_on_decoded_weights():
    """The MXFP4 layer is the bf16 layer (pinned elsewhere) run on the decoded
    weights: the same routing bit for bit and the same binary64 output."""
    lay, x, k = _small_mx4_layer()
    out4, idx4, w4, s4 = oracle.forward_mx4(x, lay["w_router"], lay["gu"], lay["dn"], k,
                                            lay["sgu"], lay["sdn"], lay["sh_gate"])
    out2, idx2, w2, s2 = oracle.forward(
        x, lay["w_router"], _values_as_bf16(lay["gu_values"]), _values_as_bf16(lay["dn_values"]),
        k, _values_as_bf16(lay["sgu_values"]), _values_as_bf16(lay["sdn_values"]), lay["sh_gate"])
    assert np.array_equal(idx4, idx2) and np.array_equal(w4, w2) and np.array_equal(s4, s2)
    assert np.array_equal(out4, out2)


def test_mx4_experts_entry_matches_forward():
    """experts_mx4 with forward_mx4's routing reproduces its output."""
    lay, x, k = _small_mx4_layer(seed=12)
    out, idx, w, _ = oracle.forward_mx4(x, lay["w_router"], lay["gu"], lay["dn"], k,
                                        lay["sgu"], lay["sdn"], lay["sh_gate"])
    out2 = oracle.experts_mx4(x, lay["gu"], lay["dn"], idx, w, lay["sgu"], lay["sdn"],
                              lay["sh_gate"])
    assert np.array_equal(out, out2)


def test_mx4_layer_shares_router_with_bf16_layer():
    """The MXFP4 layer draws the same router and gate vector as the bf16 layer
    of the same seed, so both route every token identically."""
    lay4 = W.make_layer_mx4(64, 8, 32, 32, 21)
    lay2 = W.make_layer(64, 8, 32, 32, "bf16", 21)
    assert np.array_equal(lay4["w_router"], lay2["w_router"])
    assert np.array_equal(lay4["sh_gate"], lay2["sh_gate"])
    # and its weights are the bf16 layer's draws, encoded: within 2 scaled
    # units (saturation included) plus the bf16 rounding of the reference
    v = oracle.mx4_decode(*lay4["gu"])
    ref = W.bf16_bits_to_f32(lay2["w_gate_up"]).astype(np.float64)
    u = np.ldexp(1.0, np.repeat(lay4["gu"][1].astype(np.int64) - 127, 32, axis=-1))
    assert np.all(np.abs(v - ref) <= 2 * u + np.abs(ref) * 2.0 ** -8)


def test_mx4_shape_checks():
    lay, x, k = _small_mx4_layer(T=2)
    bad = (lay["gu"][0][:, :, :-1].copy(), lay["gu"][1])
    with pytest.raises(ValueError):
        oracle.forward_mx4(x, lay["w_router"], bad, lay["dn"], k, lay["sgu"], lay["sdn"],
                           lay["sh_gate"])
    with pytest.raises(ValueError):
        W.mx4_quantize(np.zeros((2, 40), np.float32))
