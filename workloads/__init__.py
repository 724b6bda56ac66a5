"""Seeded synthetic inputs for the sparse MoE feed-forward layer.

This module generates data only: it holds none of the layer's arithmetic and
is the one piece of code that both the CPU oracle's tests and the HIP path's
tests/benchmark consume.

Shapes follow the pages: d_model 2,560, 512 routed experts, top-10, expert
width 640, one shared expert of width 640 (llm-architectures-explained
"Qwen3.8-Flash-Next", table "Every architecture field", rows d_model and
ffns.moe.*; anatomy page, "Decoder microscope", Feed-forward panel).  Weights
are drawn N(0, 0.02^2): 0.02 is the checkpoint's initializer range (llm-atlas
"Qwen3.8-Flash-Next", "Raw config fields", initializer_range), read as a
standard deviation.  Data type bfloat16 ("Key facts", Dtype).  No trained
weights exist here; these random weights stand in for them.

Arrays are numpy.  bfloat16 tensors are ``uint16`` arrays of bit patterns
(round-to-nearest-even from float32 draws); the fp32 configuration uses
``float32``.

Low-bit expert weights (configurations of dtype "mxfp4"): the published
checkpoint stores packed low-bit tensors (llm-atlas "Qwen3.8-Flash-Next",
"Modelled costs"), encoding unnamed; these inputs use MXFP4 of the OCP
Microscaling (MX) specification v1.0.  ``mx4_quantize`` plays the part of the
checkpoint writer: it turns the same float32 draws into E2M1 codes with one
E8M0 scale per 32 elements along each weight row, by the specification's
conversion rule (shared exponent floor(log2 max|v|) - 2, elements rounded to
nearest with ties to even and saturated at 6).  Router, shared gate vector and
tokens stay bfloat16.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from statistics import NormalDist
from typing import Optional

import numpy as np

WEIGHT_STD = 0.02

# Independent counter streams per tensor: SeedSequence([seed, TENSOR_ID, i]).
_X, _WR, _WGU, _WDN, _WSGU, _WSDN, _G, _BIAS, _DOUT = range(9)


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d: int
    E: int
    k: int
    F: int
    Fs: int
    dtype: str                      # "f32" | "bf16" | "mxfp4" (bf16, MXFP4 expert weights)
    bias: Optional[str] = None      # None | "zipf" | "hot10"
    seed_w: int = 1
    seed_x: int = 100
    seed_b: int = 1000
    note: str = field(default="", compare=False)
    prenorm: bool = False           # the layer takes un-normalised rows h (pre-FFN RMSNorm)
    backward: bool = False          # the training backward pass (gradients), not the forward
    aux_coef: float = 0.0           # load-balancing loss coefficient of the backward pass


CONFIGS = {
    1: MoEConfig("tiny_fp32_T32", 32, 128, 16, 4, 32, 32, "f32", None, 0, 0, 0,
                 "T=32, d=128, 16 experts top-4, width 32, shared 32, fp32, seed 0"),
    2: MoEConfig("decode_T32", 32, 2560, 512, 10, 640, 640, "bf16", None, 1, 102, 1002,
                 "decode-shaped: T=32, near-uniform routing"),
    3: MoEConfig("prefill_T4096", 4096, 2560, 512, 10, 640, 640, "bf16", None, 1, 103, 1003,
                 "prefill-shaped: T=4096"),
    4: MoEConfig("zipf_T16384", 16384, 2560, 512, 10, 640, 640, "bf16", "zipf", 1, 104, 1004,
                 "router bias with a Zipf(1.2) prior over a seeded expert permutation"),
    5: MoEConfig("hot10_T32768", 32768, 2560, 512, 10, 640, 640, "bf16", "hot10", 1, 105, 1005,
                 "router bias making 10 seeded experts take about half of all assignments"),
    6: MoEConfig("decode_T32_mxfp4", 32, 2560, 512, 10, 640, 640, "mxfp4", None, 1, 102, 1002,
                 "decode_T32 with MXFP4 expert weights quantized from the same draws"),
    8: MoEConfig("prefill_T4096_mxfp4", 4096, 2560, 512, 10, 640, 640, "mxfp4", None, 1, 103, 1003,
                 "prefill_T4096 with MXFP4 expert weights quantized from the same draws"),
    7: MoEConfig("decode_T32_prenorm", 32, 2560, 512, 10, 640, 640, "bf16", None, 1, 102, 1002,
                 "decode_T32 on RMSNorm(h): h = the decode tokens, gamma = 1 + N(0, 0.1^2)",
                 prenorm=True),
    9: MoEConfig("backward_T4096", 4096, 2560, 512, 10, 640, 640, "bf16", None, 1, 103, 1003,
                 "backward pass of prefill_T4096 for its own routing: dx and every weight "
                 "gradient, load-balancing loss coefficient 0.001, dout ~ N(0,1)",
                 backward=True, aux_coef=0.001),
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *key])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return f32_to_bf16_bits(a) if dtype == "bf16" else a


# FP4 E2M1 magnitudes by code 0..7 (code = 2 * exponent field + mantissa bit)
# and the midpoints between neighbours.
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)
_E2M1_MID = (_E2M1_GRID[1:] + _E2M1_GRID[:-1]) / np.float32(2)


def mx4_quantize(a: np.ndarray, with_values: bool = False):
    """MXFP4-encode float32 ``a`` [..., K] along its last axis (K % 32 == 0):
    returns (codes uint8 [..., K/2], scales uint8 [..., K/32]) and, if asked,
    the encoded values as float32 [..., K].

    Per block of 32: X = floor(log2(max |v|)) - 2 + 127 (127 for an all-zero
    block), clamped to 0..254; each v / 2^(X-127) goes to the nearest E2M1
    value, ties to the even code, magnitudes past 6 saturate to 6.  Element 2i
    sits in the low nibble of byte i."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    K = a.shape[-1]
    if K % 32:
        raise ValueError("MXFP4 rows need a multiple of 32 elements")
    blk = a.reshape(a.shape[:-1] + (K // 32, 32))
    amax = np.abs(blk).max(axis=-1)
    _, ex = np.frexp(amax)                       # amax = m 2^ex, m in [0.5, 1)
    X = np.where(amax > 0, ex.astype(np.int32) - 1 - 2 + 127, 127)
    X = np.clip(X, 0, 254)
    scaled = np.ldexp(blk, (127 - X)[..., None].astype(np.int32)).astype(np.float32)
    mag = np.abs(scaled)
    idx = np.searchsorted(_E2M1_MID, mag, side="left")
    at = np.minimum(idx, len(_E2M1_MID) - 1)
    tie = (idx < len(_E2M1_MID)) & (_E2M1_MID[at] == mag) & (idx % 2 == 1)
    idx = (idx + tie).astype(np.uint8)
    code = idx | (np.signbit(scaled).astype(np.uint8) << 3)
    code = code.reshape(a.shape)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    scales = X.astype(np.uint8)
    if not with_values:
        return packed, scales
    vals = np.where(np.signbit(scaled), -1.0, 1.0).astype(np.float32) * _E2M1_GRID[idx]
    vals = np.ldexp(vals, (X - 127)[..., None].astype(np.int32)).astype(np.float32)
    return packed, scales, vals.reshape(a.shape)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_layer(d: int, E: int, F: int, Fs: int, dtype: str, seed: int) -> dict:
    """Layer weights: router [E,d], packed gate/up [E,2F,d] (gate rows first),
    down [E,d,F], shared gate/up [2Fs,d], shared down [d,Fs], shared gate
    vector [d].  Each expert's blocks come from their own seeded stream, so
    they can be drawn in parallel and do not depend on E."""
    npdt = np.uint16 if dtype == "bf16" else np.float32
    w_gu = np.empty((E, 2 * F, d), npdt)
    w_dn = np.empty((E, d, F), npdt)

    def expert(e):
        w_gu[e] = _normal(_rng(seed, _WGU, e), (2 * F, d), WEIGHT_STD, dtype)
        w_dn[e] = _normal(_rng(seed, _WDN, e), (d, F), WEIGHT_STD, dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(expert, range(E)))
    layer = dict(
        w_router=_normal(_rng(seed, _WR), (E, d), WEIGHT_STD, dtype),
        w_gate_up=w_gu,
        w_down=w_dn,
        w_sh_gate_up=None, w_sh_down=None, sh_gate=None,
    )
    if Fs > 0:
        layer["w_sh_gate_up"] = _normal(_rng(seed, _WSGU), (2 * Fs, d), WEIGHT_STD, dtype)
        layer["w_sh_down"] = _normal(_rng(seed, _WSDN), (d, Fs), WEIGHT_STD, dtype)
        layer["sh_gate"] = _normal(_rng(seed, _G), (d,), WEIGHT_STD, dtype)
    return layer


def make_layer_mx4(d: int, E: int, F: int, Fs: int, seed: int, with_values: bool = False) -> dict:
    """The layer of ``make_layer(d, E, F, Fs, "bf16", seed)`` with its expert
    weights (routed and shared) MXFP4-encoded from the same float32 draws:
    keys w_router, sh_gate (bfloat16, identical to the bf16 layer) and gu, dn,
    sgu, sdn, each a (codes, scales) pair of logical shapes [E,2F,d],
    [E,d,F], [2Fs,d], [d,Fs].  with_values adds the encoded values as float32
    arrays gu_values, dn_values, sgu_values, sdn_values."""
    gu_c = np.empty((E, 2 * F, d // 2), np.uint8)
    gu_s = np.empty((E, 2 * F, d // 32), np.uint8)
    dn_c = np.empty((E, d, F // 2), np.uint8)
    dn_s = np.empty((E, d, F // 32), np.uint8)
    vals = {}
    if with_values:
        vals["gu_values"] = np.empty((E, 2 * F, d), np.float32)
        vals["dn_values"] = np.empty((E, d, F), np.float32)

    def expert(e):
        r = mx4_quantize(_normal(_rng(seed, _WGU, e), (2 * F, d), WEIGHT_STD, "f32"), with_values)
        gu_c[e], gu_s[e] = r[0], r[1]
        if with_values:
            vals["gu_values"][e] = r[2]
        r = mx4_quantize(_normal(_rng(seed, _WDN, e), (d, F), WEIGHT_STD, "f32"), with_values)
        dn_c[e], dn_s[e] = r[0], r[1]
        if with_values:
            vals["dn_values"][e] = r[2]

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(expert, range(E)))
    layer = dict(w_router=_normal(_rng(seed, _WR), (E, d), WEIGHT_STD, "bf16"),
                 gu=(gu_c, gu_s), dn=(dn_c, dn_s), sgu=None, sdn=None, sh_gate=None, **vals)
    if Fs > 0:
        r = mx4_quantize(_normal(_rng(seed, _WSGU), (2 * Fs, d), WEIGHT_STD, "f32"), with_values)
        layer["sgu"] = (r[0], r[1])
        if with_values:
            layer["sgu_values"] = r[2]
        r = mx4_quantize(_normal(_rng(seed, _WSDN), (d, Fs), WEIGHT_STD, "f32"), with_values)
        layer["sdn"] = (r[0], r[1])
        if with_values:
            layer["sdn_values"] = r[2]
        layer["sh_gate"] = _normal(_rng(seed, _G), (d,), WEIGHT_STD, "bf16")
    return layer


def make_norm_weight(d: int, dtype: str, seed: int) -> np.ndarray:
    """RMSNorm weight gamma [d] = 1 + N(0, 0.1^2) (a trained-looking spread
    around the usual initial value of ones)."""
    g = (1.0 + 0.1 * _rng(seed, _G, 1).standard_normal(d)).astype(np.float32)
    return f32_to_bf16_bits(g) if dtype in ("bf16", "mxfp4") else g


def make_x(T: int, d: int, dtype: str, seed: int, row0: int = 0) -> np.ndarray:
    """Tokens x ~ N(0,1), [T, d].  Rows are drawn in blocks of 256 tokens from
    per-block streams, so a row's value does not depend on T (a prefix of a
    longer batch equals the shorter batch) and ``row0`` selects a window."""
    if dtype == "mxfp4":
        dtype = "bf16"
    npdt = np.uint16 if dtype == "bf16" else np.float32
    out = np.empty((T, d), npdt)
    B = 256
    b0, b1 = row0 // B, (row0 + T + B - 1) // B

    def block(b):
        rows = _normal(_rng(seed, _X, b), (B, d), 1.0, dtype)
        lo, hi = max(b * B, row0), min((b + 1) * B, row0 + T)
        out[lo - row0:hi - row0] = rows[lo - b * B:hi - b * B]

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(block, range(b0, b1)))
    return out


def make_dout(T: int, d: int, seed: int) -> np.ndarray:
    """Gradient arriving at the layer's output for the backward pass:
    dout ~ N(0,1), binary32 [T, d] (the layer's out is binary32)."""
    return _rng(seed, _DOUT).standard_normal((T, d), dtype=np.float32)


def dout_for(cfg: MoEConfig) -> np.ndarray:
    """dout of a backward configuration (stream seed_b: such configs have no
    router bias)."""
    return make_dout(cfg.T, cfg.d, cfg.seed_b)


def zipf_bias(E: int, s: float, seed: int) -> np.ndarray:
    """Router bias whose softmax prior is exactly Zipf(s) over a seeded
    permutation pi of the experts: b[pi(r)] = -s ln r for ranks r = 1..E."""
    perm = _rng(seed, _BIAS).permutation(E)
    b = np.empty(E, np.float32)
    b[perm] = (-s * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)
    return b


def hot_bias(E: int, k: int, d: int, n_hot: int, share: float, seed: int):
    """Router bias +beta on n_hot seeded experts, 0 elsewhere.  beta is the
    mean-field value at which the hot experts take ``share`` of all
    assignments when logits are N(0, sigma^2) with sigma = 0.02*sqrt(d) (the
    spread of x.w for x ~ N(0,1), w ~ N(0, 0.02^2)): each hot expert must be
    selected with probability k*share/n_hot, so beta sits at the cold
    experts' selection threshold.  Returns (bias, hot expert ids)."""
    sigma = WEIGHT_STD * math.sqrt(d)
    p_hot = k * share / n_hot                     # selection prob. of a hot expert
    cold_slots = k * (1.0 - share)                # expected cold picks per token
    p_cold = cold_slots / (E - n_hot)
    tau = sigma * NormalDist().inv_cdf(1.0 - p_cold)
    beta = tau - sigma * NormalDist().inv_cdf(1.0 - p_hot)
    hot = np.sort(_rng(seed, _BIAS).choice(E, n_hot, replace=False))
    b = np.zeros(E, np.float32)
    b[hot] = np.float32(beta)
    return b, hot


def make_bias(cfg: MoEConfig) -> Optional[np.ndarray]:
    if cfg.bias is None:
        return None
    if cfg.bias == "zipf":
        return zipf_bias(cfg.E, 1.2, cfg.seed_b)
    if cfg.bias == "hot10":
        return hot_bias(cfg.E, cfg.k, cfg.d, 10, 0.5, cfg.seed_b)[0]
    raise ValueError(cfg.bias)


_layer_cache: dict = {}


def layer_for(cfg: MoEConfig) -> dict:
    key = (cfg.d, cfg.E, cfg.F, cfg.Fs, cfg.dtype, cfg.seed_w)
    if key not in _layer_cache:
        _layer_cache.clear()      # keep at most one full-size layer resident
        if cfg.dtype == "mxfp4":
            _layer_cache[key] = make_layer_mx4(cfg.d, cfg.E, cfg.F, cfg.Fs, cfg.seed_w)
        else:
            _layer_cache[key] = make_layer(cfg.d, cfg.E, cfg.F, cfg.Fs, cfg.dtype, cfg.seed_w)
    return _layer_cache[key]


def make_inputs(cfg: MoEConfig, T: Optional[int] = None) -> dict:
    """All inputs of one configuration: the layer (shared across configs with
    the same shapes and weight seed), x and the router bias."""
    T = cfg.T if T is None else T
    inp = dict(layer_for(cfg))
    inp["x"] = make_x(T, cfg.d, cfg.dtype, cfg.seed_x)
    inp["bias"] = make_bias(cfg)
    return inp


def small_case(T, d, E, k, F, Fs, dtype="bf16", seed=7, bias=None) -> dict:
    """Inputs at an arbitrary small shape (weights seed ``seed``, x seed+1)."""
    inp = make_layer(d, E, F, Fs, dtype, seed)
    inp["x"] = make_x(T, d, dtype, seed + 1)
    inp["bias"] = bias
    return inp
