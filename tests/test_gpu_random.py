"""Seeded randomized layer shapes against the oracle (the fixed seed list
below; every case prints its shape before it runs).  Shapes, routing
structure and dtype are drawn from the seed: token counts from 1 to 700,
widths that are multiples of 64 (bfloat16) or anything (binary32), up to 256
experts, top-k up to min(E, 32), with or without a shared expert; some cases
duplicate router rows (exact ties), zero the router, or add a large bias to a
few experts.  topk_idx bit-exact, topk_w within 1e-5, out within 2e-2 x RMS
(binary32 layers: 1e-4 x RMS)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_feed_amd as moe
import workloads as W
from gpu_util import OUT_TOL, W_TOL, announce, rel_err, to_dev

pytestmark = pytest.mark.gpu

SEEDS = list(range(1, 33))
SH = ("w_sh_gate_up", "w_sh_down", "sh_gate")


def draw_case(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    if dtype == "bf16":
        d = 64 * int(rng.integers(1, 17))
        F = 64 * int(rng.integers(1, 9))
        Fs = 0 if rng.random() < 0.3 else 64 * int(rng.integers(1, 9))
    else:
        d = int(rng.integers(8, 200))
        F = int(rng.integers(4, 96))
        Fs = 0 if rng.random() < 0.3 else int(rng.integers(4, 96))
    E = int(rng.choice([1, 2, 5, 16, 33, 64, 128, 200, 256]))
    k = int(rng.integers(1, min(E, 32) + 1))
    T = int(rng.choice([1, 3, 17, 32, 33, 64, 100, 257, 500, 700]))
    structure = rng.choice(["plain", "plain", "ties", "zero router", "bias"])
    return dict(T=T, d=d, E=E, k=k, F=F, Fs=Fs, dtype=dtype, structure=str(structure),
                router=str(rng.choice(["auto", "exact", "shortlist"])) if dtype == "bf16" else "auto")


@pytest.mark.parametrize("seed", SEEDS)
def test_random_layer_against_oracle(seed):
    c = draw_case(seed)
    announce(f"random case seed {seed}: {c}")
    inp = W.small_case(c["T"], c["d"], c["E"], c["k"], c["F"], c["Fs"], c["dtype"], seed=seed)
    E = c["E"]
    if c["structure"] == "ties" and E >= 2:
        wr = inp["w_router"].copy()
        wr[E - 1] = wr[0]
        wr[E // 2] = wr[0]
        inp["w_router"] = wr
    elif c["structure"] == "zero router":
        inp["w_router"] = np.zeros_like(inp["w_router"])
    elif c["structure"] == "bias":
        b = np.zeros(E, np.float32)
        hot = np.random.default_rng(seed).choice(E, min(3, E), replace=False)
        b[hot] = [8.0, 3.0, -5.0][:len(hot)]
        inp["bias"] = b
    args = [to_dev(inp[n]) for n in ("x", "w_router", "w_gate_up", "w_down")]
    sh = [to_dev(inp[n]) for n in SH] if c["Fs"] else [None, None, None]
    out, idx, w = moe.forward(*args, c["k"], *sh, bias=to_dev(inp.get("bias")),
                              router=c["router"])
    torch.cuda.synchronize()
    ref_out, ref_idx, ref_w, _ = oracle.forward(
        inp["x"], inp["w_router"], inp["w_gate_up"], inp["w_down"], c["k"],
        *([inp[n] for n in SH] if c["Fs"] else [None, None, None]), bias=inp.get("bias"))
    assert np.array_equal(idx.cpu().numpy(), ref_idx), "topk_idx differs"
    assert np.abs(w.cpu().numpy() - ref_w).max() <= W_TOL
    r = rel_err(out.cpu().numpy(), ref_out)
    tol = 1e-4 if c["dtype"] == "f32" else OUT_TOL
    assert r <= tol, f"max|err|/rms = {r:.3e}"
