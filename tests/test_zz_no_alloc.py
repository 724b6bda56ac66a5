"""moe_forward_noalloc (workspace in the library's static device array) gives
moe_forward's outputs bit for bit, on two calls in a row, the second with a
smaller batch (the array then holds the first call's contents)."""
import numpy as np
import pytest
import torch

import sparse_moe_feed_amd as moe
import workloads as W
from gpu_util import announce, to_dev

pytestmark = pytest.mark.gpu

SH = ("w_sh_gate_up", "w_sh_down", "sh_gate")


def run_both(inp, k, bias=None):
    args = [to_dev(inp[n]) for n in ("x", "w_router", "w_gate_up", "w_down")]
    sh = [to_dev(inp[n]) for n in SH]
    b = to_dev(bias)
    ref = moe.forward(*args, k, *sh, bias=b)
    got = moe.forward_noalloc(*args, k, *sh, bias=b)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in ref], [t.cpu().numpy() for t in got]


def test_noalloc_equals_forward_two_calls_second_smaller():
    # pages' shape with a batch that takes the grouped-GEMM path and the
    # shortlist router, then a decode-sized batch (weight streaming, exact
    # router, no permutation) on the same layer
    d, E, k, F, Fs = 2560, 512, 10, 640, 640
    lay = W.make_layer(d, E, F, Fs, "bf16", 11)
    bias = W.zipf_bias(E, 1.2, 12)
    for T in (1340, 24):
        inp = dict(lay, x=W.make_x(T, d, "bf16", 13))
        announce(f"noalloc vs forward T={T}")
        ref, got = run_both(inp, k, bias)
        for name, r, g in zip(("out", "topk_idx", "topk_w"), ref, got):
            assert np.array_equal(r, g), f"T={T}: {name} differs"


def test_noalloc_small_layers_and_fp32():
    for T, d, E, k, F, Fs, dt in ((300, 256, 16, 4, 128, 64, "bf16"),
                                  (1000, 320, 64, 8, 64, 128, "bf16"),
                                  (32, 128, 16, 4, 32, 32, "f32"),
                                  (5, 256, 16, 4, 128, 0, "bf16")):
        inp = W.small_case(T, d, E, k, F, Fs, dt, seed=T)
        announce(f"noalloc vs forward T={T} d={d} {dt}")
        ref, got = run_both(inp, k)
        for name, r, g in zip(("out", "topk_idx", "topk_w"), ref, got):
            assert np.array_equal(r, g), f"T={T}: {name} differs"


def test_noalloc_rejects_a_batch_beyond_the_array():
    d, E, k, F, Fs = 2560, 512, 10, 640, 640
    shape = moe.Shape(d, E, k, F, Fs, torch.bfloat16)
    T = 1348
    assert moe.workspace_size(shape, T) > moe.NOALLOC_SCRATCH_BYTES
    # rejected before any GPU work: the tensors are never read
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoEError) as e:
        moe.forward_noalloc(z(T, d), z(E, d), z(E, 2 * F, d), z(E, d, F), k, z(2 * Fs, d),
                            z(d, Fs), z(d))
    assert e.value.status == moe.MOE_ERR_WORKSPACE
