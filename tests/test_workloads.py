"""The seeded input generator: determinism, shapes, the recipe's statistics (CPU only)."""
import math

import numpy as np

import workloads as W


def test_configs_shapes():
    c = W.CONFIGS
    assert (c["tiny_fp32"].N, c["tiny_fp32"].n_qblk, c["tiny_fp32"].n_kvblk) == (1024, 16, 16)
    assert (c["wan13b_480p"].N, c["wan13b_480p"].n_qblk, c["wan13b_480p"].n_kvblk) == (32760, 256, 512)
    assert (c["wan14b_720p"].N, c["wan14b_720p"].n_qblk, c["wan14b_720p"].n_kvblk) == (75600, 591, 1182)
    assert (c["long_245k"].N, c["long_245k"].n_qblk, c["long_245k"].n_kvblk) == (245760, 1920, 3840)
    assert c["sparse_linear"].linear and c["sparse_linear"].N == 32760
    assert [w.N for w in W.long_sweep()] == [32768, 61440, 122880, 245760]


def test_deterministic_and_seed_dependent():
    w = W.small("t", 1, 2, 300, 64, "bf16", 64, 64, 0.1, 0.9, n_sinks=3)
    a = W.make_inputs(w)
    b = W.make_inputs(w, workers=1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    c = W.make_inputs(w.replace(seed=1))
    assert not np.array_equal(a[0], c[0])
    # heads are independent streams: generating one head alone gives the same values
    d = W.make_inputs(w, heads=[(0, 1)])
    assert np.array_equal(d[0][0, 1], a[0][0, 1]) and np.all(d[0][0, 0] == 0)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, 0.0], np.float64)
    bits = W.f64_to_bf16_bits(x)
    back = W.bf16_bits_to_f32(bits).astype(np.float64)
    # ties go to even mantissas; above-tie rounds up
    assert back.tolist() == [1.0, 1.0, 1.0 + 4 * 2 ** -8, 1.0 + 2 * 2 ** -8, -2.5, 0.0]


def test_recipe_statistics():
    w = W.Workload("s", 1, 2, 128, (4, 16, 16), "fp32", 64, 64, 0.25, 0.9, 4)
    q, k, v, alpha = W.make_inputs(w)
    pos = W.positional_term(w, 0, 0)
    rms = math.sqrt(np.mean(pos ** 2))
    assert 2.2 < rms < 3.8      # 8 sinusoids of amplitude 1.5: RMS 1.5*sqrt(8/2) = 3
    # Q and K share the positional term; V does not carry it
    corr = np.mean((q[0, 0] - pos) * (k[0, 0] - pos))
    assert abs(corr) < 0.1
    sinks = W.sink_positions(w, 0)
    assert len(sinks) == 4
    norms = np.linalg.norm(k[0, 0], axis=1)
    assert np.median(norms[sinks]) > 5 * np.median(norms)
    assert alpha.shape == (2, 128) and alpha.dtype == np.float32
    assert alpha.min() >= 0.5 and alpha.max() <= 1.0
    assert abs(v.mean()) < 0.05 and abs(v.std() - 1.0) < 0.05


def test_token_order_on_grid():
    t, y, x = W.grid_coords((3, 4, 5))
    n = (t * 4 + y) * 5 + x
    assert np.array_equal(n, np.arange(60))
