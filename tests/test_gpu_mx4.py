"""Parity of the HIP path with MXFP4 expert weights (moe_mx4_pack, then
moe_forward_mx4 / moe_experts_mx4, through the C ABI) against the CPU oracle's
MXFP4 layer, which reads the row-major MX form directly.

Bars as for the bf16 layer: topk_idx bit for bit, topk_w within 1e-5, out
within 2e-2 x RMS(oracle out).  The decoded weights are exact in bf16, so the
only rounding the GPU adds over the oracle is the bf16 h and y and the
binary32 accumulation.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_feed_amd as moe
import workloads as W
from gpu_util import W_TOL, announce, assert_out, to_dev

pytestmark = pytest.mark.gpu

MX = ("gu", "dn", "sgu", "sdn")


def mx_dev(t):
    """Row-major (codes, scales) -> packed MX4Tensor on the GPU."""
    return None if t is None else moe.mx4_pack(to_dev(t[0]), to_dev(t[1]))


def packed_reference(codes, scales):
    """The packed form, written out from its definition in include/moe.h:
    tile (b, t) of 16 rows x 128 elements at (b K/128 + t) 1088 bytes; byte
    16 (r + 16 c) + j = codes byte 64 t + 16 c + j of row 16 b + r; byte
    1024 + r + 16 c = scales byte 4 t + c of row 16 b + r."""
    R, K = codes.shape[0], codes.shape[1] * 2
    out = np.zeros(R // 16 * (K // 128) * 1088, np.uint8)
    for b in range(R // 16):
        for t in range(K // 128):
            base = (b * (K // 128) + t) * 1088
            for r in range(16):
                for c in range(4):
                    o = base + 16 * (r + 16 * c)
                    out[o:o + 16] = codes[16 * b + r, 64 * t + 16 * c:64 * t + 16 * c + 16]
                    out[base + 1024 + r + 16 * c] = scales[16 * b + r, 4 * t + c]
    return out


@pytest.mark.parametrize("R,K", [(16, 128), (48, 384), (32, 640)])
def test_mx4_pack_matches_layout_definition(R, K):
    """The pack kernel is a pure byte permutation: bit-exact against the
    layout written out element by element."""
    rng = np.random.default_rng(R + K)
    codes = rng.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (R, K // 32), dtype=np.uint8)
    announce(f"mx4_pack {R}x{K}")
    p = moe.mx4_pack(to_dev(codes), to_dev(scales))
    torch.cuda.synchronize()
    assert (p.rows, p.K) == (R, K)
    assert np.array_equal(p.data.cpu().numpy(), packed_reference(codes, scales))


def small_mx4(T, d, E, k, F, Fs, seed):
    inp = W.make_layer_mx4(d, E, F, Fs, seed)
    inp["x"] = W.make_x(T, d, "bf16", seed + 1)
    inp["bias"] = None
    return inp


def gpu_forward_mx4(inp, k):
    out, idx, w = moe.forward_mx4(to_dev(inp["x"]), to_dev(inp["w_router"]),
                                  *[mx_dev(inp[n]) for n in MX[:2]], k,
                                  *[mx_dev(inp[n]) for n in MX[2:]], to_dev(inp["sh_gate"]),
                                  bias=to_dev(inp.get("bias")))
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def oracle_forward_mx4(inp, k):
    return oracle.forward_mx4(inp["x"], inp["w_router"], inp["gu"], inp["dn"], k, inp["sgu"],
                              inp["sdn"], inp["sh_gate"], bias=inp.get("bias"))


def check_mx4(inp, k, name):
    announce(name)
    out, idx, w = gpu_forward_mx4(inp, k)
    ref_out, ref_idx, ref_w, _ = oracle_forward_mx4(inp, k)
    assert np.array_equal(idx, ref_idx), f"{name}: topk_idx differs"
    assert np.abs(w - ref_w).max() <= W_TOL
    return assert_out(out, ref_out)


@pytest.mark.parametrize("T,d,E,k,F,Fs", [
    (8, 256, 16, 4, 128, 128),      # a few rows per expert
    (40, 384, 32, 6, 256, 128),     # d % 256 = 128: odd number of K groups
    (7, 512, 64, 3, 128, 0),        # no shared expert
    (1, 256, 8, 2, 128, 128),       # one token
    (64, 256, 16, 4, 384, 256),     # T k = 16 E (edge of the streaming regime)
])
def test_small_mx4_layers(T, d, E, k, F, Fs):
    inp = small_mx4(T, d, E, k, F, Fs, seed=T + E + 40)
    check_mx4(inp, k, f"mxfp4 T={T} d={d} E={E} k={k} F={F} Fs={Fs}")


def test_mx4_bias_sends_every_token_to_one_expert():
    """60 tokens all pick expert 5 first: a group of two 32-row tiles (the
    two-half MFMA path) beside experts with one row."""
    T, d, E, k, F = 60, 256, 16, 2, 128
    inp = small_mx4(T, d, E, k, F, F, seed=81)
    inp["bias"] = np.zeros(E, np.float32)
    inp["bias"][5] = 100.0
    check_mx4(inp, k, "mxfp4 bias -> expert 5")


def test_mx4_experts_entry_with_given_routing():
    T, d, E, k, F, Fs = 30, 256, 32, 5, 128, 128
    inp = small_mx4(T, d, E, k, F, Fs, seed=12)
    rng = np.random.default_rng(4)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    announce("moe_experts_mx4 given routing")
    out = moe.experts_mx4(to_dev(inp["x"]), mx_dev(inp["gu"]), mx_dev(inp["dn"]), to_dev(idx),
                          to_dev(w), mx_dev(inp["sgu"]), mx_dev(inp["sdn"]), to_dev(inp["sh_gate"]))
    torch.cuda.synchronize()
    ref = oracle.experts_mx4(inp["x"], inp["gu"], inp["dn"], idx, w.astype(np.float64),
                             inp["sgu"], inp["sdn"], inp["sh_gate"])
    assert_out(out.cpu().numpy(), ref)


def test_mx4_decode_without_permutation_matches_permuted_path():
    """MXFP4 weight streaming at T = 24: the forward skips the permutation
    step, the routing-given entry point keeps it; same routing, same bits
    (no shared expert, whose gate each entry point computes in its own
    order)."""
    T, d, E, k, F = 24, 256, 32, 4, 128
    inp = small_mx4(T, d, E, k, F, 0, seed=17)
    announce("mxfp4 decode without permutation T=24")
    out, idx, w = moe.forward_mx4(to_dev(inp["x"]), to_dev(inp["w_router"]), mx_dev(inp["gu"]),
                                  mx_dev(inp["dn"]), k)
    out2 = moe.experts_mx4(to_dev(inp["x"]), mx_dev(inp["gu"]), mx_dev(inp["dn"]), idx, w)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), out2.cpu().numpy())


@pytest.mark.parametrize("T", [24, 300])
def test_mx4_deterministic(T):
    """Both MXFP4 paths (weight streaming at T = 24, the GEMM at T = 300)
    give the same bits twice."""
    d, E, k = 256, 16, 4
    inp = small_mx4(T, d, E, k, 128, 128, seed=55)
    announce(f"mxfp4 determinism T={T}")
    out1, idx1, _ = gpu_forward_mx4(inp, k)
    out2, idx2, _ = gpu_forward_mx4(inp, k)
    assert np.array_equal(idx1, idx2) and np.array_equal(out1, out2)


@pytest.mark.parametrize("T,d,E,k,F,Fs", [
    (65, 256, 16, 4, 128, 128),      # just past the streaming regime: GEMM path
    (300, 256, 16, 4, 128, 128),     # ~75 rows per expert, 3 shared tiles (one ragged)
    (500, 384, 16, 3, 256, 128),     # d % 256 = 128: the last down N-tile is half outside d
    (700, 512, 8, 2, 384, 0),        # experts over 128 rows (two tiles), no shared expert
    (260, 256, 64, 8, 128, 256),     # Fs > F
])
def test_mx4_gemm_layers(T, d, E, k, F, Fs):
    inp = small_mx4(T, d, E, k, F, Fs, seed=T + d)
    check_mx4(inp, k, f"mxfp4 GEMM T={T} d={d} E={E} k={k} F={F} Fs={Fs}")


def test_mx4_gemm_bias_sends_every_token_to_one_expert():
    """All 400 tokens pick expert 5 first: one group of four 128-row tiles."""
    T, d, E, k, F = 400, 256, 16, 2, 128
    inp = small_mx4(T, d, E, k, F, F, seed=82)
    inp["bias"] = np.zeros(E, np.float32)
    inp["bias"][5] = 100.0
    check_mx4(inp, k, "mxfp4 GEMM bias -> expert 5")


def test_mx4_zero_tokens():
    inp = small_mx4(0, 256, 8, 2, 128, 128, seed=2)
    announce("mxfp4 T=0")
    out, idx, _ = gpu_forward_mx4(inp, 2)
    assert out.shape == (0, 256) and idx.shape == (0, 2)


@pytest.mark.slow
def test_full_prefill_mx4():
    """Pages' shapes with MXFP4 weights at T = 4096 (GEMM path), every token:
    topk_idx bit-exact, topk_w within 1e-5 and every element of out against
    the oracle."""
    cfg = W.CONFIGS[8]
    lay = W.layer_for(cfg)
    x = W.make_x(cfg.T, cfg.d, cfg.dtype, cfg.seed_x)
    announce(f"{cfg.name}: GPU forward")
    out, idx, w = gpu_forward_mx4(dict(lay, x=x, bias=None), cfg.k)
    announce(f"{cfg.name}: oracle forward of all {cfg.T} tokens")
    ref, ref_idx, ref_w, _ = oracle.forward_mx4(x, lay["w_router"], lay["gu"], lay["dn"], cfg.k,
                                                lay["sgu"], lay["sdn"], lay["sh_gate"])
    assert np.array_equal(idx, ref_idx)
    assert np.abs(w - ref_w).max() <= W_TOL
    r = assert_out(out, ref)
    announce(f"{cfg.name}: max|err|/rms = {r:.4e}")


def test_full_config_mx4():
    """Pages' shapes with MXFP4 expert weights (decode, T=32): every token's
    topk_idx bit-exact and out of every token against the oracle."""
    cfg = W.CONFIGS[6]
    lay = W.layer_for(cfg)
    x = W.make_x(cfg.T, cfg.d, cfg.dtype, cfg.seed_x)
    inp = dict(lay, x=x, bias=None)
    r = check_mx4(inp, cfg.k, f"{cfg.name}: all {cfg.T} tokens")
    announce(f"{cfg.name}: max|err|/rms = {r:.3e}")
