"""Parity of the HIP path (through the C ABI) with the CPU oracle.

topk_idx must match bit for bit; topk_w and the shared gate within 1e-5;
out within 2e-2 x RMS(oracle out) (bfloat16 weights and activations, binary32
accumulation, h rounded to bfloat16 once).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_feed_amd as moe
import workloads as W
from gpu_util import GATE_TOL, OUT_TOL, W_TOL, announce, assert_out, rel_err, to_dev

pytestmark = pytest.mark.gpu

SH = ("w_sh_gate_up", "w_sh_down", "sh_gate")


def gpu_forward(inp, k):
    args = [to_dev(inp[n]) for n in ("x", "w_router", "w_gate_up", "w_down")]
    sh = [to_dev(inp[n]) for n in SH]
    bias = to_dev(inp.get("bias"))
    out, idx, w = moe.forward(*args, k, *sh, bias=bias)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def oracle_forward(inp, k):
    return oracle.forward(inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], k,
                          *[inp[n] for n in SH], bias=inp.get("bias"))


def check_case(inp, k, name):
    announce(name)
    out, idx, w = gpu_forward(inp, k)
    ref_out, ref_idx, ref_w, _ = oracle_forward(inp, k)
    assert np.array_equal(idx, ref_idx), f"{name}: topk_idx differs in {(idx != ref_idx).sum()} entries"
    assert np.abs(w - ref_w).max() <= W_TOL
    return assert_out(out, ref_out)


# ------------------------------------------------------------------ small cases

def test_tiny_fp32_layer():
    """T=32, d=128, 16 experts top-4, width 32, shared 32, binary32, seed 0."""
    cfg = W.CONFIGS[1]
    inp = W.make_inputs(cfg)
    r = check_case(inp, cfg.k, cfg.name)
    assert r < 1e-4     # binary32 end to end: far inside the bound


@pytest.mark.parametrize("T,d,E,k,F,Fs", [
    (300, 256, 16, 4, 128, 64),     # ~75 rows per expert, 3 ragged shared tiles
    (1000, 320, 64, 8, 64, 128),    # some experts > 128 rows (2 tiles); d % 128 = 64
    (1, 512, 32, 3, 64, 0),         # one token, no shared expert
    (77, 128, 8, 8, 64, 64),        # k = E
    (130, 192, 40, 1, 192, 64),     # k = 1
    (513, 64, 1024, 32, 64, 64),    # largest E and k supported
    (40, 256, 64, 4, 128, 128),     # weight-streaming path (few rows per expert)
    (7, 384, 128, 6, 256, 0),       # weight-streaming path, no shared expert
    (100, 256, 16, 2, 128, 128),    # streaming path, experts with 17..32+ rows
    (1000, 256, 16, 4, 128, 128),   # 256-row tiles (partial tiles)
    (1200, 384, 8, 2, 256, 128),    # 256-row tiles, 2 per expert; d % 256 = 128
    (600, 256, 16, 4, 128, 128),    # 128-row LDS-DMA tiles, some experts > 128 rows
    (500, 320, 16, 3, 256, 128),    # 128-row LDS-DMA tiles; d % 256 = 64
    (1000, 576, 192, 4, 640, 640),  # 128-row LDS-DMA tiles at the pages' widths (F == Fs),
                                    # 9 K steps in gate/up, d % 256 = 64
    (2000, 640, 96, 6, 640, 640),   # the same, experts of one and two tiles
    (8192, 1024, 8, 4, 128, 0),     # 256-row tiles, down pipelined across tiles: about two
                                    # tiles per persistent block, no shared expert
    (3000, 384, 32, 4, 640, 640),   # the same with the pages' expert widths (20 K steps per
                                    # tile), ragged last column tile (d % 256 = 128)
])
def test_small_bf16_layers(T, d, E, k, F, Fs):
    inp = W.small_case(T, d, E, k, F, Fs, "bf16", seed=T + E)
    check_case(inp, k, f"bf16 T={T} d={d} E={E} k={k} F={F} Fs={Fs}")


def test_fp32_ragged_width():
    inp = W.small_case(45, 100, 12, 3, 33, 7, "f32", seed=5)
    check_case(inp, 3, "fp32 d=100 F=33 Fs=7")


def test_one_block_permutation_largest():
    # T <= 256: the permutation runs in one block; E = 1024 and k = 32 give
    # it the largest histogram
    inp = W.small_case(256, 64, 1024, 32, 32, 32, "f32", seed=6)
    check_case(inp, 32, "fp32 T=256 E=1024 k=32")


def test_route_entry_matches_oracle():
    inp = W.small_case(200, 256, 64, 10, 64, 64, "bf16", seed=9)
    announce("moe_route T=200 E=64 k=10")
    idx, w, s = moe.route(to_dev(inp["x"]), to_dev(inp["w_router"]), 10,
                          sh_gate=to_dev(inp["sh_gate"]))
    torch.cuda.synchronize()
    ref_idx, ref_w = oracle.route(inp["x"], inp["w_router"], 10)
    _, ref_s = oracle.experts(inp["x"], inp["w_gate_up"], inp["w_down"], ref_idx, ref_w,
                              *[inp[n] for n in SH], return_gate=True)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    assert np.abs(w.cpu().numpy() - ref_w).max() <= W_TOL
    assert np.abs(s.cpu().numpy() - ref_s).max() <= GATE_TOL


def test_experts_entry_with_given_routing():
    """Routing supplied from outside (random distinct experts, random
    weights): exercises the expert stage alone."""
    T, d, E, k, F, Fs = 257, 256, 32, 5, 128, 64
    inp = W.small_case(T, d, E, k, F, Fs, "bf16", seed=12)
    rng = np.random.default_rng(4)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    announce("moe_experts given routing")
    out = moe.experts(to_dev(inp["x"]), to_dev(inp["w_gate_up"]), to_dev(inp["w_down"]),
                      to_dev(idx), to_dev(w), *[to_dev(inp[n]) for n in SH])
    torch.cuda.synchronize()
    ref = oracle.experts(inp["x"], inp["w_gate_up"], inp["w_down"], idx, w.astype(np.float64),
                         *[inp[n] for n in SH])
    assert_out(out.cpu().numpy(), ref)


@pytest.mark.parametrize("T,bias_e", [(1, None), (32, None), (32, 5), (20, 5)])
def test_decode_without_permutation_matches_permuted_path(T, bias_e):
    """At T <= 32 the forward's weight-streaming path skips the permutation
    step (block x serves expert x, h and y rows indexed by pair id); the
    routing-given entry point keeps it.  Fed the forward's own routing, the
    two give the same bits (no shared expert, whose gate each entry point
    computes in its own order).  bias_e sends every token to one expert
    first: at T = 32 its tile is full (32 rows)."""
    d, E, k, F = 256, 64, 4, 128
    inp = W.small_case(T, d, E, k, F, 0, "bf16", seed=70 + T)
    if bias_e is not None:
        inp["bias"] = np.zeros(E, np.float32)
        inp["bias"][bias_e] = 100.0
    announce(f"decode without permutation T={T} bias={bias_e}")
    args = [to_dev(inp[n]) for n in ("x", "w_router", "w_gate_up", "w_down")]
    out, idx, w = moe.forward(*args, k, bias=to_dev(inp.get("bias")))
    out2 = moe.experts(args[0], args[2], args[3], idx, w)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), out2.cpu().numpy())
    ref_out, ref_idx, _, _ = oracle_forward(inp, k)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    assert_out(out.cpu().numpy(), ref_out)


@pytest.mark.parametrize("T,bias_e", [(1, None), (32, 5), (33, None)])
def test_decode_shared_expert_near_permutation_boundary(T, bias_e):
    """The shared expert's block on the path without the permutation (T <= 32)
    and on the permuted path just past it (T = 33), against the oracle."""
    d, E, k, F, Fs = 256, 64, 4, 128, 128
    inp = W.small_case(T, d, E, k, F, Fs, "bf16", seed=90 + T)
    if bias_e is not None:
        inp["bias"] = np.zeros(E, np.float32)
        inp["bias"][bias_e] = 100.0
    check_case(inp, k, f"decode shared expert T={T} bias={bias_e}")


def test_zero_router_ties_to_lower_index():
    T, d, E, k = 70, 128, 32, 6
    inp = W.small_case(T, d, E, k, 64, 64, "bf16", seed=1)
    inp["w_router"] = np.zeros_like(inp["w_router"])
    announce("zero router")
    out, idx, w = gpu_forward(inp, k)
    assert (idx == np.arange(k)).all()
    assert np.abs(w - 1.0 / k).max() <= W_TOL


def test_duplicate_router_rows():
    inp = W.small_case(300, 256, 16, 5, 64, 64, "bf16", seed=21)
    inp["w_router"] = inp["w_router"].copy()
    inp["w_router"][9] = inp["w_router"][3]
    check_case(inp, 5, "duplicate router rows 3 and 9")


def test_cross_tile_pipeline_with_empty_experts():
    """256-row tiles whose down projection runs its K pipeline across tiles,
    with a third of the experts chosen by no token (their tiles absent) and
    one expert taking every token first (many tiles in a row)."""
    T, d, E, k, F = 6144, 512, 12, 3, 256
    inp = W.small_case(T, d, E, k, F, F, "bf16", seed=11)
    inp["bias"] = np.zeros(E, np.float32)
    inp["bias"][[1, 4, 7, 10]] = -100.0
    inp["bias"][2] = 100.0
    check_case(inp, k, "256-row tiles, four empty experts, expert 2 first for every token")


@pytest.mark.parametrize("T,d,E,k,F", [(600, 128, 16, 2, 64), (100, 256, 32, 2, 128)])
def test_bias_sends_every_token_to_one_expert(T, d, E, k, F):
    """All T tokens pick expert 5 first: one group spanning several tiles
    (LDS-tiled GEMM path, then the weight-streaming path)."""
    inp = W.small_case(T, d, E, k, F, F, "bf16", seed=8)
    inp["bias"] = np.zeros(E, np.float32)
    inp["bias"][5] = 100.0
    check_case(inp, k, "bias -> expert 5")


@pytest.mark.parametrize("T", [700, 200])
def test_workspace_grouping_matches_routing(T):
    """counts / offsets / perm in the workspace are exactly the grouping the
    routing implies, rows of one expert in ascending pair id (multi-block
    histogram at T=700, the single-block path at T=200)."""
    d, E, k, F, Fs = 128, 24, 4, 64, 64
    inp = W.small_case(T, d, E, k, F, Fs, "bf16", seed=33)
    shape = moe.Shape(d, E, k, F, Fs, torch.bfloat16)
    ws = moe.alloc_workspace(shape, T)
    announce("workspace grouping")
    args = [to_dev(inp[n]) for n in ("x", "w_router", "w_gate_up", "w_down")]
    _, idx, _ = moe.forward(*args, k, *[to_dev(inp[n]) for n in SH], ws=ws)
    torch.cuda.synchronize()
    lay = moe.workspace_layout(shape, T)
    wsb = ws.cpu().numpy()
    counts = wsb[lay.counts:lay.counts + 4 * (E + 1)].view(np.int32)
    offsets = wsb[lay.offsets:lay.offsets + 4 * (E + 1)].view(np.int32)
    perm = wsb[lay.perm:lay.perm + 4 * T * k].view(np.int32)
    ref_idx, _ = oracle.route(inp["x"], inp["w_router"], k)
    flat = ref_idx.ravel()
    assert counts[E] == T
    for e in range(E):
        pairs = np.nonzero(flat == e)[0]
        assert counts[e] == len(pairs)
        assert np.array_equal(perm[offsets[e]:offsets[e] + counts[e]], pairs)
    assert offsets[E] == T * k


def test_deterministic_and_batch_split():
    T, d, E, k = 400, 256, 32, 6
    inp = W.small_case(T, d, E, k, 128, 64, "bf16", seed=55)
    announce("determinism / batch split")
    out1, idx1, _ = gpu_forward(inp, k)
    out2, idx2, _ = gpu_forward(inp, k)
    assert np.array_equal(idx1, idx2)
    assert np.array_equal(out1, out2)       # fixed-order combine, no atomics
    for a, b in [(0, 1), (1, 150), (150, 400)]:
        part = dict(inp)
        part["x"] = np.ascontiguousarray(inp["x"][a:b])
        o, i, _ = gpu_forward(part, k)
        assert np.array_equal(i, idx1[a:b])
        assert rel_err(o, out1[a:b].astype(np.float64)) < 1e-2


def test_stage_events_are_recorded():
    T, d, E, k = 300, 256, 16, 4
    inp = W.small_case(T, d, E, k, 128, 64, "bf16", seed=3)
    args = [to_dev(inp[n]) for n in ("x", "w_router", "w_gate_up", "w_down")]
    sh = [to_dev(inp[n]) for n in SH]
    evs = [moe.HipEvent() for _ in range(1 + len(moe.STAGES))]
    announce("stage events")
    moe.stage_events(evs)
    moe.forward(*args, k, *sh)
    torch.cuda.synchronize()
    times = [evs[i].elapsed_ms(evs[i + 1]) for i in range(len(moe.STAGES))]
    assert all(t >= 0 for t in times) and sum(times) > 0


def test_zero_tokens():
    inp = W.small_case(0, 128, 8, 2, 64, 64, "bf16", seed=2)
    announce("T=0")
    out, idx, w = gpu_forward(inp, 2)
    assert out.shape == (0, 128) and idx.shape == (0, 2)


# ------------------------------------------------------------------ full-size configs

@pytest.fixture(scope="module")
def full_layer():
    cfg = W.CONFIGS[2]
    lay = W.layer_for(cfg)
    dev = {n: to_dev(lay[n]) for n in ("w_router", "w_gate_up", "w_down") + SH}
    return lay, dev


CHUNK = 4096     # tokens per oracle call: each test case stays well under a minute


def _full_cases():
    cases = []
    for c in (2, 3, 4, 5):
        T = W.CONFIGS[c].T
        marks = [pytest.mark.slow] if c > 2 else []
        cases += [pytest.param(c, i, marks=marks) for i in range((T + CHUNK - 1) // CHUNK)]
    return cases


_gpu_full: dict = {}       # config -> GPU results of the whole batch (one config resident)
_err_full: dict = {}       # config -> {chunk: (max|err|, sum of squares of oracle out, count)}


def gpu_full_forward(full_layer, c):
    if c not in _gpu_full:
        _gpu_full.clear()
        cfg = W.CONFIGS[c]
        _, dev = full_layer
        x = W.make_x(cfg.T, cfg.d, cfg.dtype, cfg.seed_x)
        bias = W.make_bias(cfg)
        announce(f"{cfg.name}: GPU forward of all {cfg.T} tokens")
        out, idx, w = moe.forward(to_dev(x), dev["w_router"], dev["w_gate_up"], dev["w_down"],
                                  cfg.k, *[dev[n] for n in SH], bias=to_dev(bias))
        torch.cuda.synchronize()
        _gpu_full[c] = (x, bias, out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy())
    return _gpu_full[c]


@pytest.mark.parametrize("c,chunk", _full_cases())
def test_full_config(full_layer, c, chunk):
    """Pages' shapes (d 2560, 512 experts top-10, width 640, shared 640), every
    token of every configuration: the GPU runs the whole batch in one call, the
    oracle one chunk of tokens per case (tokens are independent, so a chunk's
    oracle result is that of the whole batch).  topk_idx bit-exact, topk_w
    within 1e-5, every element of out within 2e-2 x RMS; the last chunk also
    checks max|err| over the whole batch against the RMS of the whole oracle
    output."""
    cfg = W.CONFIGS[c]
    lay, _ = full_layer
    x, bias, out, idx, w = gpu_full_forward(full_layer, c)
    lo, hi = chunk * CHUNK, min(cfg.T, (chunk + 1) * CHUNK)
    announce(f"{cfg.name}: oracle forward of tokens {lo}..{hi - 1}")
    ref_out, ref_idx, ref_w, _ = oracle.forward(np.ascontiguousarray(x[lo:hi]), lay["w_router"],
                                                lay["w_gate_up"], lay["w_down"], cfg.k,
                                                *[lay[n] for n in SH], bias=bias)
    bad = (idx[lo:hi] != ref_idx).any(1).sum()
    assert bad == 0, f"{bad} tokens with a different topk_idx"
    assert np.abs(w[lo:hi] - ref_w).max() <= W_TOL
    err = float(np.abs(out[lo:hi].astype(np.float64) - ref_out).max())
    ss = float((ref_out ** 2).sum())
    r = assert_out(out[lo:hi], ref_out)
    _err_full.setdefault(c, {})[chunk] = (err, ss, ref_out.size)
    announce(f"{cfg.name} tokens {lo}..{hi - 1}: max|err|/rms = {r:.4e}")
    n_chunks = (cfg.T + CHUNK - 1) // CHUNK
    if len(_err_full[c]) == n_chunks:
        parts = _err_full[c].values()
        rms = np.sqrt(sum(p[1] for p in parts) / sum(p[2] for p in parts))
        worst = max(p[0] for p in parts) / rms
        announce(f"{cfg.name}: all {cfg.T} tokens, max|err|/RMS(oracle out) = {worst:.4e}")
        assert worst <= OUT_TOL


# ------------------------------------------------------------------ shortlist router

def gpu_route(inp, k, router):
    idx, w, _ = moe.route(to_dev(inp["x"]), to_dev(inp["w_router"]), k, bias=to_dev(inp.get("bias")),
                          router=router)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("T,d,E,k,case", [
    (300, 256, 64, 10, "plain"),
    (260, 2560, 512, 10, "pages' shapes"),
    (129, 640, 96, 7, "ragged chunk (d % 512 != 0)"),
    (150, 128, 64, 6, "zero router: > 32 candidates, exact fallback"),
    (200, 256, 16, 4, "duplicate rows"),
    (180, 512, 128, 12, "large bias on a few experts"),
    (160, 256, 64, 10, "infinite bias: fewer than k finite logits"),
])
def test_shortlist_router_equals_exact(T, d, E, k, case):
    """MFMA shortlist + exact recompute selects exactly what the canonical
    router over all experts selects, and both match the oracle."""
    inp = W.small_case(T, d, E, k, 64, 0, "bf16", seed=T + d)
    if case.startswith("zero"):
        inp["w_router"] = np.zeros_like(inp["w_router"])
    if case == "duplicate rows":
        inp["w_router"] = inp["w_router"].copy()
        inp["w_router"][7] = inp["w_router"][2]
        inp["w_router"][11] = inp["w_router"][2]
    if case.startswith("large bias"):
        b = np.zeros(E, np.float32)
        b[[3, 40, 77]] = [4.0, 2.5, 6.0]
        inp["bias"] = b
    if case.startswith("infinite bias"):
        # six experts keep a finite logit; the other experts' -inf logits
        # tie, so the last four slots go to the lowest such experts, weight 0
        b = np.full(E, -np.inf, np.float32)
        b[[5, 17, 18, 40, 41, 63]] = 0.0
        inp["bias"] = b
    announce(f"shortlist vs exact router: {case}")
    i_ex, w_ex = gpu_route(inp, k, "exact")
    i_sl, w_sl = gpu_route(inp, k, "shortlist")
    ref_idx, ref_w = oracle.route(inp["x"], inp["w_router"], k, bias=inp.get("bias"))
    assert np.array_equal(i_ex, ref_idx)
    assert np.array_equal(i_sl, ref_idx)
    assert np.array_equal(w_ex, w_sl)
    assert np.abs(w_sl - ref_w).max() <= W_TOL


def test_shortlist_bound_is_far_from_tight():
    """Observed |f - l| of the MFMA logits stays well inside the bound the
    shortlist relies on (Delta = coef ||x|| ||w_e||, without the bias term)."""
    T, d, E, k = 256, 2560, 512, 10
    inp = W.small_case(T, d, E, k, 64, 0, "bf16", seed=77)
    shape = moe.Shape(d, E, k, 64, 0, torch.bfloat16, "shortlist")
    ws = moe.alloc_workspace(shape, T)
    announce("shortlist bound")
    moe.route(to_dev(inp["x"]), to_dev(inp["w_router"]), k, ws=ws, router="shortlist")
    torch.cuda.synchronize()
    lay = moe.workspace_layout(shape, T)
    S = 2 if d % 128 == 0 else 1  # K slices of the MFMA logits
    parts = ws.cpu().numpy()[lay.logits:lay.logits + 4 * S * T * (E + 1)].view(np.float32)
    parts = parts.reshape(S, T, E + 1)[:, :, :E]
    f = parts[0]
    for s in range(1, S):
        f = f + parts[s]  # binary32, slice order, as the select step adds them
    l = oracle.router_logits(inp["x"], inp["w_router"]).astype(np.float64)
    xf = W.bf16_bits_to_f32(inp["x"]).astype(np.float64)
    wf = W.bf16_bits_to_f32(inp["w_router"]).astype(np.float64)
    u = 2.0 ** -23
    coef = 2 * (d * u + (8 * ((d + 511) // 512) + 7) * u)
    delta = coef * np.linalg.norm(xf, axis=1)[:, None] * np.linalg.norm(wf, axis=1)[None, :]
    ratio = np.abs(f.astype(np.float64) - l) / delta
    assert ratio.max() < 0.05, ratio.max()


# ------------------------------------------------------------------ MOE_DEBUG_SYNC

@pytest.mark.parametrize("T", [24, 300])
def test_debug_sync_changes_no_result(monkeypatch, T):
    """MOE_DEBUG_SYNC=1 (the host waits after every stage so that a failing
    kernel is named) computes exactly what the asynchronous call computes,
    for the forward (weight-streaming and grouped-GEMM paths) and for the
    routing alone."""
    inp = W.small_case(T, 256, 16, 4, 128, 64, "bf16", seed=T + 9)
    ref = gpu_forward(inp, 4)
    monkeypatch.setenv("MOE_DEBUG_SYNC", "1")
    announce(f"MOE_DEBUG_SYNC forward T={T}")
    got = gpu_forward(inp, 4)
    for r, g in zip(ref, got):
        assert np.array_equal(r, g)
    i_dbg, w_dbg = gpu_route(inp, 4, None)
    monkeypatch.delenv("MOE_DEBUG_SYNC")
    i_ref, w_ref = gpu_route(inp, 4, None)
    assert np.array_equal(i_dbg, i_ref) and np.array_equal(w_dbg, w_ref)


# ------------------------------------------------------------------ direct decode tiles

@pytest.mark.parametrize("T,d,E,k,F,Fs,case", [
    (32, 256, 16, 4, 128, 128, "one expert chosen by every token (two 16-row halves)"),
    (24, 640, 64, 8, 256, 0, "no shared expert; ragged last column block"),
    (32, 2560, 512, 10, 640, 640, "pages' shapes"),
    (1, 384, 32, 6, 128, 256, "one token, Fs > F"),
    (17, 1152, 128, 32, 128, 128, "k = 32, 17 tokens"),
])
def test_direct_decode_shapes(T, d, E, k, F, Fs, case):
    """The weight-streaming path without the permutation step (T <= 32, exact
    router) at odd shapes: routing bit-exact, out within tolerance of the
    oracle, and deterministic run to run."""
    inp = W.small_case(T, d, E, k, F, Fs, "bf16", seed=T * 7 + d)
    if case.startswith("one expert"):
        b = np.zeros(E, np.float32)
        b[5] = 50.0
        inp["bias"] = b
    announce(f"direct decode: {case}")
    r = check_case(inp, k, case)
    out1, _, _ = gpu_forward(inp, k)
    out2, _, _ = gpu_forward(inp, k)
    assert np.array_equal(out1, out2), "not deterministic"


# ------------------------------------------------------------------ direct decode, many experts touched

@pytest.mark.parametrize("T,d,E,k,F,bias_e,case", [
    (32, 256, 1024, 8, 128, None, "227 experts touched, one or two rows each"),
    (32, 256, 1024, 8, 128, 5, "one expert chosen by every token: 32 rows"),
    (20, 384, 512, 16, 256, None, "20 tokens, k = 16"),
    (32, 128, 256, 32, 2048, None, "widest expert held in LDS; d = 128: half the waves "
                                   "have no down columns"),
])
def test_direct_decode_many_experts_matches_permuted_path(T, d, E, k, F, bias_e, case):
    """The direct decode path with 200+ experts touched (the decode
    workload's regime), up to 32 rows on one expert and experts up to 2048
    wide: fed the forward's own routing, the routing-given entry point
    (permuted rows) gives the same bits; both match the oracle."""
    inp = W.small_case(T, d, E, k, F, 0, "bf16", seed=T * 3 + E)
    if bias_e is not None:
        inp["bias"] = np.zeros(E, np.float32)
        inp["bias"][bias_e] = 100.0
    announce(f"direct decode, many experts: {case}")
    args = [to_dev(inp[n]) for n in ("x", "w_router", "w_gate_up", "w_down")]
    out, idx, w = moe.forward(*args, k, bias=to_dev(inp.get("bias")))
    out2 = moe.experts(args[0], args[2], args[3], idx, w)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), out2.cpu().numpy())
    ref_out, ref_idx, _, _ = oracle_forward(inp, k)
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    assert_out(out.cpu().numpy(), ref_out)


@pytest.mark.parametrize("T,d,E,k,F,Fs,case", [
    (32, 512, 1024, 8, 128, 256, "shared expert wider than the routed ones"),
    (32, 256, 1024, 8, 256, 128, "shared expert narrower than the routed ones"),
])
def test_direct_decode_many_experts_with_shared_expert(T, d, E, k, F, Fs, case):
    inp = W.small_case(T, d, E, k, F, Fs, "bf16", seed=T + E + F)
    check_case(inp, k, f"direct decode, many experts: {case}")
