"""Pins of the block-mask oracle against facts outside it (CPU only).

The rule under test (SpargeAttention2 page, section 2(1)): per attention row keep the
union of the top-k% entries and the smallest set reaching cumulative probability p.
Pooling (SLA2 page, router item 1): mean pooling of Q and K per block.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import mask as M
from oracle.mask import (exp_sa, pool_blocks, block_scores, tree_sum, select_row, topk_count,
                         oracle_plan, score_scale, plan_stats)

F32 = np.float32
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def ulp_err(got: np.ndarray, x: np.ndarray) -> np.ndarray:
    ref = np.exp(x.astype(np.float64))
    spacing = np.spacing(ref.astype(F32)).astype(np.float64)
    return np.abs(got.astype(np.float64) - ref) / spacing


# ---------------------------------------------------------------- exp_sa
def test_exp_sa_matches_math_exp_within_2_ulp():
    x = np.linspace(-86.0, 0.0, 2_000_001, dtype=np.float64).astype(F32)
    rng = np.random.default_rng(1)
    x = np.concatenate([x, -rng.exponential(3.0, 500_000).astype(F32), -rng.random(200_000, dtype=F32)])
    x = x[x >= -86.0]
    got = exp_sa(x)
    err = ulp_err(got, x)
    assert err.max() <= 2.0, err.max()
    assert np.all(got > 0)


def test_exp_sa_special_values():
    assert exp_sa(np.array([0.0], F32))[0] == F32(1.0)
    assert exp_sa(np.array([-0.0], F32))[0] == F32(1.0)
    assert exp_sa(np.array([-86.5, -1000.0, -np.inf], F32)).tolist() == [0.0, 0.0, 0.0]
    # -86 itself is the smallest argument that is evaluated; the result is normal
    v = exp_sa(np.array([-86.0], F32))[0]
    assert v >= np.finfo(F32).tiny and abs(float(v) / math.exp(-86.0) - 1) < 1e-6
    # exp(-ln2 * j) ~ 2^-j, up to the rounding of the argument to fp32
    j = np.arange(0, 120)
    x = (-j * math.log(2.0)).astype(F32)
    got = exp_sa(x).astype(np.float64)
    assert np.all(np.abs(got * 2.0 ** j - 1.0) <= np.abs(x.astype(np.float64) + j * math.log(2.0)) * 1.01 + 2.5e-7)


def test_exp_sa_reduction_constants_exact():
    # C1 has at most 16 significant bits so n*C1 is exact in fp32 for |n| <= 2^8
    c1 = float(M.LN2_HI)
    assert c1 * 65536 == int(c1 * 65536)
    for n in range(-130, 1):
        assert float(F32(n) * M.LN2_HI) == n * c1
    assert abs((float(M.LN2_HI) + float(M.LN2_LO)) - math.log(2.0)) < 1e-13
    for i, c in enumerate(M.EXP_COEF):
        assert c == F32(1.0 / math.factorial(i))


def test_exp_sa_monotone_on_grid():
    x = np.linspace(-20.0, 0.0, 400_001).astype(F32)
    y = exp_sa(x)
    assert np.all(np.diff(y.astype(np.float64)) >= 0)


# ---------------------------------------------------------------- pooling / scores
def test_pool_mean_closed_form_and_ragged():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((300, 8)).astype(F32)   # 300 = 4*64 + 44: ragged last block
    got = pool_blocks(x, 64)
    assert got.shape == (5, 8)
    for I in range(5):
        ref = x[I * 64:min(300, (I + 1) * 64)].astype(np.float64).mean(axis=0)
        assert np.max(np.abs(got[I] - ref)) < 64 * 1.2e-7 * np.abs(x).max()
    # the ragged block divides by its real token count (44), not by the block size
    y = np.ones((300, 3), F32)
    assert np.all(pool_blocks(y, 64) == 1.0)


def test_pool_sequential_order_bits():
    # values where the summation order changes the fp32 result
    x = np.array([[1.0], [2.0 ** -24], [2.0 ** -24], [-1.0]], F32)
    # sequential: ((0 + 1) + 2^-24) = 1 (tie to even), + 2^-24 = 1, - 1 = 0
    assert pool_blocks(x, 4)[0, 0] == F32(0.0)


def test_scores_are_tile_means_of_true_logits():
    # bilinearity: (mean_i q_i).(mean_j k_j)/sqrt(D) == mean_{i,j} q_i.k_j/sqrt(D)
    rng = np.random.default_rng(3)
    N, D = 200, 16
    q = rng.standard_normal((N, D)).astype(F32)
    k = rng.standard_normal((N + 37, D)).astype(F32)[:N]
    bq, bk = 64, 32
    S = block_scores(pool_blocks(q, bq), pool_blocks(k, bk), score_scale(D))
    assert S.shape == (4, 7)
    logits = (q.astype(np.float64) @ k.astype(np.float64).T) / math.sqrt(D)
    for I in range(4):
        for J in range(7):
            ref = logits[I * bq:(I + 1) * bq, J * bk:(J + 1) * bk].mean()
            assert abs(S[I, J] - ref) < 2e-5, (I, J, S[I, J], ref)


def test_score_hand_example():
    q = np.array([[1.0, 2.0], [3.0, 4.0]], F32)
    k = np.array([[1.0, 0.0], [0.0, 1.0]], F32)
    S = block_scores(pool_blocks(q, 2), pool_blocks(k, 2), score_scale(2))
    assert S.shape == (1, 1)
    assert S[0, 0] == F32(F32(2.0 * 0.5 + 3.0 * 0.5) * F32(1.0 / math.sqrt(2.0)))
    assert score_scale(64) == F32(0.125)


def test_score_no_fma_order():
    # products rounded before the add: (1+2^-12)^2 = 1 + 2^-11 + 2^-24 rounds to 1 + 2^-11,
    # then adding -(1 + 2^-11) gives exactly 0 (an FMA would keep 2^-24)
    a = F32(1.0 + 2.0 ** -12)
    qbar = np.array([[a, F32(1.0)]], F32)
    kbar = np.array([[a, -F32(1.0 + 2.0 ** -11)]], F32)
    assert block_scores(qbar, kbar, F32(1.0))[0, 0] == F32(0.0)


# ---------------------------------------------------------------- tree sum
def test_tree_sum_adjacent_pairs():
    e = np.array([1.0, 2.0 ** -24, -1.0, 2.0 ** -24], F32)
    # adjacent pairing: (1 + 2^-24) -> 1, (-1 + 2^-24) exact -> 2^-24 total
    assert tree_sum(e) == F32(2.0 ** -24)
    e = np.array([1.0, 2.0, 3.0], F32)
    assert tree_sum(e) == F32(6.0)
    x = np.random.default_rng(4).random(1000).astype(F32)
    assert abs(float(tree_sum(x)) - math.fsum(x.astype(np.float64))) < 1e-4


# ---------------------------------------------------------------- selection
def brute_select(S_row, m_k, p):
    """Independent pure-Python reading of the rule: order by (-S, index); the top-p
    prefix from a float32 running sum in that order; union = longer prefix."""
    n = len(S_row)
    order = sorted(range(n), key=lambda j: (-float(S_row[j]), j))
    e = exp_sa(np.asarray(S_row, F32) - F32(S_row[order[0]]))
    Z = tree_sum(e)
    if p >= 1.0:
        mp = n
    else:
        thr = F32(F32(p) * Z)
        acc = F32(0.0)
        mp = n
        for r, j in enumerate(order, start=1):
            acc = F32(acc + e[j])
            if acc >= thr:
                mp = r
                break
    keep = max(m_k, mp)
    return sorted(order[:keep]), mp


def test_select_matches_brute_force_random_rows():
    rng = np.random.default_rng(5)
    for trial in range(300):
        n = int(rng.integers(1, 40))
        S = (rng.standard_normal(n) * rng.choice([0.1, 1.0, 5.0, 30.0])).astype(F32)
        if trial % 5 == 0:
            S = np.round(S).astype(F32)    # many exact ties
        mk = int(rng.integers(1, n + 1))
        p = float(rng.choice([0.0, 0.3, 0.8, 0.9, 0.99, 1.0]))
        kept, mp, keep = select_row(S, mk, p)
        bk, bmp = brute_select(S, mk, p)
        assert kept.tolist() == bk and mp == bmp


def test_golden_topp_boundaries():
    with open(os.path.join(GOLDEN, "topp_golden.json")) as f:
        fixtures = json.load(f)
    for fx in fixtures:
        S = np.asarray(fx["scores"], F32)
        mk = topk_count(fx["k"], len(S))
        assert mk == fx["m_k"], fx["name"]
        for c in fx["cases"]:
            kept, mp, keep = select_row(S, mk, c["p"])
            assert mp == c["m_p"], (fx["name"], c)
            assert kept.tolist() == c["kept"], (fx["name"], c)


def test_topp_boundary_is_inclusive():
    # 10 equal entries, p = 0.5: thr = 5 exactly, C_5 = 5 >= 5 -> 5 blocks (not 6)
    kept, mp, keep = select_row(np.zeros(10, F32), 1, 0.5)
    assert mp == 5 and kept.tolist() == [0, 1, 2, 3, 4]


def test_flat_row_topp_rescues_topk():
    # SpargeAttention2 section 1 / 2(1): on a uniform row, top-k alone keeps too few;
    # the union keeps the top-p set. 16 equal scores, k = 25% (4 blocks), p = 0.9:
    # thr = 0.9*16 = 14.4, so 15 blocks, ties broken by the lower index.
    kept, mp, keep = select_row(np.full(16, 0.7, F32), topk_count(0.25, 16), 0.9)
    assert mp == 15 and keep == 15 and kept.tolist() == list(range(15))


def test_sink_row_topk_rescues_topp():
    # SpargeAttention2 section 1 / 2(1): on a row dominated by one sink block, top-p
    # alone keeps one block; the union keeps the top-k set (sink + lowest-index ties).
    S = np.zeros(16, F32)
    S[5] = 30.0
    kept, mp, keep = select_row(S, topk_count(0.25, 16), 0.9)
    assert mp == 1 and keep == 4 and kept.tolist() == [0, 1, 2, 5]


def test_corner_rules():
    rng = np.random.default_rng(6)
    S = rng.standard_normal(33).astype(F32)
    assert select_row(S, topk_count(1.0, 33), 0.0)[0].tolist() == list(range(33))
    assert select_row(S, topk_count(0.0, 33), 1.0)[0].tolist() == list(range(33))
    kept, mp, keep = select_row(S, topk_count(0.0, 33), 0.0)
    assert kept.tolist() == [int(np.argmax(S))]
    # top-k alone (p = 0) equals the first m_k of a stable descending argsort
    mk = 7
    kept, _, _ = select_row(S, mk, 0.0)
    assert kept.tolist() == sorted(np.argsort(-S, kind="stable")[:mk].tolist())


def test_topk_count_values():
    # the workloads' m_k: 25% of 16, 5% of 512, 3% of 1182, 2% of 3840, 2% of 512
    assert [topk_count(0.25, 16), topk_count(0.05, 512), topk_count(0.03, 1182),
            topk_count(0.02, 3840), topk_count(0.02, 512)] == [4, 26, 36, 77, 11]
    assert topk_count(0.0, 10) == 1 and topk_count(1.0, 10) == 10 and topk_count(0.1, 10) == 1


def test_union_properties_on_random_plan():
    rng = np.random.default_rng(7)
    B, H, N, D = 1, 3, 700, 32
    q = rng.standard_normal((B, H, N, D)).astype(F32)
    k = rng.standard_normal((B, H, N, D)).astype(F32)
    k[:, :, 100] *= 8
    row_ptr, col_idx, mps = oracle_plan(q, k, 64, 32, 0.1, 0.7)
    nkv = -(-N // 32)
    mk = topk_count(0.1, nkv)
    counts = np.diff(row_ptr)
    assert np.all(counts == np.maximum(mk, mps))
    for r in range(len(counts)):
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
        assert np.all(np.diff(cols) > 0) and cols.min() >= 0 and cols.max() < nkv
    # sampled-row interface returns the same lists
    rows = [(0, 1, 3), (0, 2, 10), (0, 0, 0)]
    sub = oracle_plan(q, k, 64, 32, 0.1, 0.7, rows=rows)
    nq = -(-N // 64)
    for (b, h, I) in rows:
        r = (b * H + h) * nq + I
        assert sub[(b, h, I)].tolist() == col_idx[row_ptr[r]:row_ptr[r + 1]].tolist()


def test_duplicate_blocks_tie_to_lower_index():
    rng = np.random.default_rng(8)
    N, D = 256, 16
    q = rng.standard_normal((1, 1, N, D)).astype(F32)
    k = rng.standard_normal((1, 1, N, D)).astype(F32) * 0.1
    k[0, 0, 64:96] = k[0, 0, 192:224] = rng.standard_normal((32, D)).astype(F32) * 3
    # blocks 2 and 6 (bk = 32) are identical, so their pooled scores tie exactly
    _, col_idx, _ = oracle_plan(q, k, 64, 32, 1.0 / 8, 0.0)
    # m_k = 1: exactly one of the tied pair survives per row when it is the maximum
    for I in range(4):
        S = block_scores(pool_blocks(q[0, 0], 64), pool_blocks(k[0, 0], 32), score_scale(D))[I]
        assert S[2] == S[6]
        if S[2] == S.max():
            assert col_idx[I] == 2


def test_mask_agrees_with_float64_selection_away_from_boundaries():
    """The fp32 spec agrees with the same rule in float64 whenever the float64
    cumulative mass is not within a rounding margin of the threshold."""
    rng = np.random.default_rng(9)
    B, H, N, D = 1, 2, 2048, 64
    q = (rng.standard_normal((B, H, N, D)) + 0.5).astype(F32)
    k = (rng.standard_normal((B, H, N, D)) + 0.5).astype(F32)
    bq, bk, kf, p = 64, 64, 0.1, 0.8
    row_ptr, col_idx, _ = oracle_plan(q, k, bq, bk, kf, p)
    nq = nkv = N // 64
    mk = topk_count(kf, nkv)
    checked = 0
    for h in range(H):
        qb = q[0, h].astype(np.float64).reshape(nq, bq, D).mean(1)
        kb = k[0, h].astype(np.float64).reshape(nkv, bk, D).mean(1)
        S = qb @ kb.T / math.sqrt(D)
        for I in range(nq):
            s = S[I]
            order = np.argsort(-s, kind="stable")
            pr = np.exp(s[order] - s[order[0]])
            cum = np.cumsum(pr) / pr.sum()
            mp = int(np.argmax(cum >= p)) + 1
            if np.min(np.abs(cum - p)) < 1e-4 or np.min(np.abs(np.diff(s[order]))) < 1e-5:
                continue
            r = h * nq + I
            assert col_idx[row_ptr[r]:row_ptr[r + 1]].tolist() == sorted(order[:max(mk, mp)].tolist())
            checked += 1
    assert checked > 40


def test_plan_stats_counts_ragged_pairs():
    N = 100   # blocks of 64: sizes 64 and 36
    row_ptr = np.array([0, 1, 3])
    col_idx = np.array([1, 0, 1], np.int32)
    st = plan_stats(row_ptr, col_idx, 1, 1, N, 64, 64)
    assert st["nnz"] == 3
    assert st["kept_pairs"] == 64 * 36 + 36 * 64 + 36 * 36
    assert abs(st["tile_sparsity"] - 0.25) < 1e-12
