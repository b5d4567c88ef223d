"""Pins of the oracle's ground-truth tile heatmap (Veda page, section 2.1: max pooling of
the full attention matrix over query x key tiles) against facts outside it: brute force
with pure-Python loops, the Q = 0 closed form, unit row mass, and a dominant key."""
import math

import numpy as np
import pytest

from oracle import tile_heatmap


def _brute(q, k, bq, bk):
    """Pure-Python loops: softmax row by row, then the tile max and the tile mean mass."""
    B, H, N, D = q.shape
    nQ, nKV = -(-N // bq), -(-N // bk)
    tmax = np.zeros((B * H * nQ, nKV))
    tmass = np.zeros((B * H * nQ, nKV))
    for b in range(B):
        for h in range(H):
            for I in range(nQ):
                r = (b * H + h) * nQ + I
                qs = range(I * bq, min(N, (I + 1) * bq))
                for i in qs:
                    logits = [sum(float(q[b, h, i, d]) * float(k[b, h, j, d]) for d in range(D)) / math.sqrt(D)
                              for j in range(N)]
                    m = max(logits)
                    ex = [math.exp(x - m) for x in logits]
                    z = sum(ex)
                    for j in range(N):
                        p = ex[j] / z
                        J = j // bk
                        tmax[r, J] = max(tmax[r, J], p)
                        tmass[r, J] += p / len(qs)
    return tmax, tmass


def test_brute_force_ragged():
    rng = np.random.default_rng(3)
    B, H, N, D = 1, 2, 150, 8
    q = rng.normal(size=(B, H, N, D)) * 1.5
    k = rng.normal(size=(B, H, N, D)) * 1.5
    tmax, tmass = tile_heatmap(q, k, 64, 32)
    bmax, bmass = _brute(q, k, 64, 32)
    assert tmax.shape == (B * H * 3, 5)
    np.testing.assert_allclose(tmax, bmax, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(tmass, bmass, rtol=1e-11, atol=1e-15)


def test_zero_queries_closed_form():
    """Q = 0 makes every probability 1/N: the tile max is 1/N, the tile mass |J|/N."""
    rng = np.random.default_rng(0)
    B, H, N, D = 2, 1, 200, 16
    q = np.zeros((B, H, N, D))
    k = rng.normal(size=(B, H, N, D))
    tmax, tmass = tile_heatmap(q, k, 64, 64)
    np.testing.assert_allclose(tmax, 1.0 / N, rtol=1e-12)
    sizes = np.array([64, 64, 64, 8]) / N
    np.testing.assert_allclose(tmass, np.broadcast_to(sizes, tmass.shape), rtol=1e-12)


def test_rows_of_mass_sum_to_one_and_subset_rows():
    rng = np.random.default_rng(1)
    q = rng.normal(size=(1, 3, 300, 32)) * 2.0
    k = rng.normal(size=(1, 3, 300, 32)) * 2.0
    tmax, tmass = tile_heatmap(q, k, 128, 64)
    np.testing.assert_allclose(tmass.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(tmax <= 1.0) and np.all(tmax > 0.0)
    # a tile's mass per query is at most 64 times its largest probability
    assert np.all(tmass <= 64 * tmax + 1e-15)
    sub = [1, 4, 8]
    smax, smass = tile_heatmap(q, k, 128, 64, rows=sub)
    np.testing.assert_array_equal(smax[sub], tmax[sub])
    np.testing.assert_array_equal(smass[sub], tmass[sub])
    assert np.isnan(smax[0]).all()


def test_dominant_key_owns_its_tile():
    """A key aligned with every query at large norm takes nearly all probability."""
    rng = np.random.default_rng(2)
    N, D = 256, 16
    q = np.abs(rng.normal(size=(1, 1, N, D))) + 0.5
    k = rng.normal(size=(1, 1, N, D)) * 0.1
    k[0, 0, 77] = 50.0
    tmax, tmass = tile_heatmap(q, k, 64, 64)
    assert np.all(tmax[:, 1] > 0.999)          # key 77 lies in KV block 1
    assert np.all(tmass[:, 1] > 0.999)
    assert np.all(tmass[:, [0, 2, 3]] < 1e-3)
