"""Parity of the pre-FFN RMSNorm on the GPU (moe_rmsnorm, moe_forward_prenorm,
through the C ABI) with the CPU oracle.

The normalised rows are compared bit for bit: both sides follow the same
binary32 order (canonical sum of squares, correctly rounded division and
square root, two rounded products, nearest-even to bf16).  The layer on them
is then held to the usual bars: topk_idx bit-exact, topk_w within 1e-5, out
within 2e-2 x RMS(oracle out).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_feed_amd as moe
import workloads as W
from gpu_util import OUT_TOL, W_TOL, announce, assert_out, to_dev

pytestmark = pytest.mark.gpu


def rows(T, d, dtype, seed):
    """Rows of very different scales, so that eps matters for some."""
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((T, d)).astype(np.float32)
    h *= np.logspace(-5, 3, T, dtype=np.float32)[:, None]
    return W.f32_to_bf16_bits(h) if dtype == "bf16" else h


@pytest.mark.parametrize("T,d,dtype,eps", [
    (37, 2560, "bf16", 1e-6),    # pages' width, five 512-wide chunks
    (64, 640, "bf16", 1e-6),     # ragged last chunk (640 = 512 + 128)
    (9, 64, "bf16", 0.0),
    (50, 100, "f32", 1e-6),      # d % 8 != 0: scalar loads
    (8, 128, "f32", 1e-6),
])
def test_rmsnorm_bit_exact(T, d, dtype, eps):
    h = rows(T, d, dtype, T + d)
    g = W.make_norm_weight(d, dtype, 5)
    announce(f"rmsnorm T={T} d={d} {dtype} eps={eps}")
    x = moe.rmsnorm(to_dev(h), to_dev(g), eps)
    torch.cuda.synchronize()
    if dtype == "bf16":
        xg = x.cpu().view(torch.int16).numpy().view(np.uint16)
    else:
        xg = x.cpu().numpy().view(np.uint32)
    ref = oracle.rmsnorm(h, g, eps)
    ref = ref if dtype == "bf16" else ref.view(np.uint32)
    bad = int((xg != ref).sum())
    assert bad == 0, f"{bad} of {xg.size} normalised elements differ"


def check_prenorm(inp, h, g, k, name, mx4=False):
    announce(name)
    if mx4:
        ws = [moe.mx4_pack(to_dev(inp[n][0]), to_dev(inp[n][1])) if inp[n] is not None else None
              for n in ("gu", "dn", "sgu", "sdn")]
    else:
        ws = [to_dev(inp[n]) for n in ("w_gate_up", "w_down", "w_sh_gate_up", "w_sh_down")]
    out, idx, w = moe.forward_prenorm(to_dev(h), to_dev(g), to_dev(inp["w_router"]), ws[0], ws[1],
                                      k, ws[2], ws[3], to_dev(inp["sh_gate"]),
                                      bias=to_dev(inp.get("bias")))
    torch.cuda.synchronize()
    x = oracle.rmsnorm(h, g, 1e-6)
    if mx4:
        ref, ref_idx, ref_w, _ = oracle.forward_mx4(x, inp["w_router"], inp["gu"], inp["dn"], k,
                                                    inp["sgu"], inp["sdn"], inp["sh_gate"],
                                                    bias=inp.get("bias"))
    else:
        ref, ref_idx, ref_w, _ = oracle.forward(x, inp["w_router"], inp["w_gate_up"],
                                                inp["w_down"], k, inp["w_sh_gate_up"],
                                                inp["w_sh_down"], inp["sh_gate"],
                                                bias=inp.get("bias"))
    assert np.array_equal(idx.cpu().numpy(), ref_idx), f"{name}: topk_idx differs"
    assert np.abs(w.cpu().numpy() - ref_w).max() <= W_TOL
    return assert_out(out.cpu().numpy(), ref)


@pytest.mark.parametrize("T,d,E,k,F,Fs", [
    (24, 256, 32, 4, 128, 128),     # weight-streaming path, exact router
    (300, 256, 16, 4, 128, 64),     # shortlist router, LDS-tiled experts
])
def test_prenorm_layer_bf16(T, d, E, k, F, Fs):
    inp = W.small_case(T, d, E, k, F, Fs, "bf16", seed=T + d)
    h = W.f32_to_bf16_bits(3.0 * W.bf16_bits_to_f32(inp["x"]))
    g = W.make_norm_weight(d, "bf16", 9)
    check_prenorm(inp, h, g, k, f"prenorm bf16 T={T} d={d} E={E} k={k}")


def test_prenorm_layer_mx4():
    T, d, E, k, F, Fs = 16, 256, 32, 4, 128, 128
    inp = W.make_layer_mx4(d, E, F, Fs, 31)
    h = W.f32_to_bf16_bits(2.0 * W.bf16_bits_to_f32(W.make_x(T, d, "bf16", 32)))
    g = W.make_norm_weight(d, "bf16", 10)
    check_prenorm(dict(inp, bias=None), h, g, k, "prenorm mxfp4", mx4=True)


def test_prenorm_full_decode_shape():
    """Pages' shapes at T = 32: normalised rows, routing and output against
    the oracle for every token."""
    cfg = W.CONFIGS[2]
    lay = W.layer_for(cfg)
    h = W.f32_to_bf16_bits(4.0 * W.bf16_bits_to_f32(W.make_x(cfg.T, cfg.d, "bf16", cfg.seed_x)))
    g = W.make_norm_weight(cfg.d, "bf16", 11)
    r = check_prenorm(dict(lay, bias=None), h, g, cfg.k, "prenorm decode_T32")
    announce(f"prenorm decode_T32: max|err|/rms = {r:.3e}")


@pytest.mark.parametrize("T", [24, 300])
def test_prenorm_workspace_rows_bit_exact(T):
    """The normalised rows the experts read (workspace region xnorm) equal
    the oracle's bit for bit, in front of the exact router (T = 24) and of
    the shortlist router (T = 300)."""
    d, E, k, F, Fs = 256, 16, 4, 128, 64
    inp = W.small_case(T, d, E, k, F, Fs, "bf16", seed=T)
    h = rows(T, d, "bf16", T + 1)
    g = W.make_norm_weight(d, "bf16", 12)
    shape = moe.Shape(d, E, k, F, Fs, torch.bfloat16)
    ws = moe.alloc_workspace(shape, T)
    announce(f"prenorm workspace rows T={T}")
    moe.forward_prenorm(to_dev(h), to_dev(g), to_dev(inp["w_router"]), to_dev(inp["w_gate_up"]),
                        to_dev(inp["w_down"]), k, to_dev(inp["w_sh_gate_up"]),
                        to_dev(inp["w_sh_down"]), to_dev(inp["sh_gate"]), ws=ws)
    torch.cuda.synchronize()
    lay = moe.workspace_layout(shape, T)
    got = ws.cpu().numpy()[lay.xnorm:lay.xnorm + 2 * T * d].view(np.uint16).reshape(T, d)
    ref = oracle.rmsnorm(h, g, 1e-6)
    assert int((got != ref).sum()) == 0


@pytest.mark.parametrize("T,d,E,k,F,Fs,dtype", [
    (24, 256, 32, 4, 128, 128, "bf16"),   # weight streaming, no permutation launch
    (300, 256, 16, 4, 128, 64, "bf16"),   # shortlist router, LDS-tiled experts
    (20, 96, 6, 2, 40, 24, "f32"),        # binary32 layer
    (16, 256, 32, 4, 128, 0, "bf16"),     # no shared expert
])
def test_prenorm_residual_stream(T, d, E, k, F, Fs, dtype):
    """moe_forward_prenorm with the residual stream: resid becomes resid + out
    (the binary32 sum of the two, bit for bit, with the out the same call
    returns), within the output tolerance of the oracle's resid + out."""
    inp = W.small_case(T, d, E, k, F, Fs, dtype, seed=T + 3)
    h = rows(T, d, dtype, T + 4)
    g = W.make_norm_weight(d, dtype, 13)
    resid0 = np.random.default_rng(T).standard_normal((T, d)).astype(np.float32)
    resid = to_dev(resid0)
    sh = [to_dev(inp[n]) for n in ("w_sh_gate_up", "w_sh_down", "sh_gate")]
    announce(f"prenorm residual T={T} d={d} {dtype} Fs={Fs}")
    out, idx, _ = moe.forward_prenorm(to_dev(h), to_dev(g), to_dev(inp["w_router"]),
                                      to_dev(inp["w_gate_up"]), to_dev(inp["w_down"]), k, *sh,
                                      resid=resid)
    torch.cuda.synchronize()
    out, got = out.cpu().numpy(), resid.cpu().numpy()
    assert np.array_equal(got, resid0 + out)
    x = oracle.rmsnorm(h, g, 1e-6)
    ref_out, ref_idx, _, _ = oracle.forward(x, inp["w_router"], inp["w_gate_up"], inp["w_down"],
                                            k, *[inp[n] for n in ("w_sh_gate_up", "w_sh_down",
                                                                   "sh_gate")])
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    ref = oracle.residual(resid0, ref_out)
    rms = np.sqrt((ref_out ** 2).mean())
    err = np.abs(got.astype(np.float64) - ref)
    tol = (1e-4 if dtype == "f32" else OUT_TOL) * rms
    assert np.all(err <= tol + 2.0 ** -23 * np.abs(ref)), f"max|err|/rms = {err.max() / rms:.3e}"
