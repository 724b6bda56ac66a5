"""The seeded input generators: data format, determinism and the routing
structure the skewed workloads are meant to have.  CPU only."""
import numpy as np
from scipy.special import softmax

import oracle
import workloads as W


def test_bf16_rounding_is_nearest_even():
    one = np.float32(1.0)
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5],
                    np.float32)
    assert list(W.f32_to_bf16_bits(vals)) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020]
    assert W.bf16_bits_to_f32(np.array([0x3F80, 0xC020], np.uint16)).tolist() == [1.0, -2.5]
    assert one == W.bf16_bits_to_f32(W.f32_to_bf16_bits(np.array([one])))[0]


def test_x_rows_do_not_depend_on_batch_size():
    a = W.make_x(700, 64, "bf16", 5)
    b = W.make_x(300, 64, "bf16", 5)
    c = W.make_x(200, 64, "bf16", 5, row0=250)
    assert np.array_equal(a[:300], b)
    assert np.array_equal(a[250:450], c)


def test_layer_is_deterministic_and_scaled():
    l1 = W.make_layer(128, 8, 32, 32, "bf16", 3)
    l2 = W.make_layer(128, 8, 32, 32, "bf16", 3)
    for key in l1:
        assert np.array_equal(l1[key], l2[key])
    w = W.bf16_bits_to_f32(l1["w_gate_up"]).astype(np.float64)
    assert abs(w.std() - 0.02) < 0.001 and abs(w.mean()) < 0.001


def test_zipf_prior_is_exact():
    b = W.zipf_bias(512, 1.2, 1004)
    p = softmax(b.astype(np.float64))
    perm_rank = np.argsort(-p, kind="stable")
    r = np.arange(1, 513, dtype=np.float64)
    assert np.allclose(p[perm_rank], r ** -1.2 / (r ** -1.2).sum(), rtol=1e-5)


def test_hot_experts_take_about_half_of_assignments():
    cfg = W.CONFIGS[5]
    b, hot = W.hot_bias(cfg.E, cfg.k, cfg.d, 10, 0.5, cfg.seed_b)
    x = W.make_x(512, cfg.d, "bf16", cfg.seed_x)
    router = W._normal(W._rng(cfg.seed_w, W._WR), (cfg.E, cfg.d), W.WEIGHT_STD, "bf16")
    idx, _ = oracle.route(x, router, cfg.k, bias=b)
    share = np.isin(idx, hot).mean()
    assert 0.45 < share < 0.55
