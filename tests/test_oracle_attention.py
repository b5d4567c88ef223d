"""Pins of the float64 output oracle (CPU only).

Block-sparse attention skips masked tiles entirely (SpargeAttention2 page, section
2(3)); the linear branch covers the masked-out blocks (SALAD page, section 2.1) and is
blended as O = alpha*Os + (1-alpha)*Ol (SLA2 page, item 2).
"""
import math

import numpy as np
import pytest
import torch

from oracle.attention import (sparse_attention, dense_attention, brute_masked_attention,
                              linear_branch, blend, phi, dense_plan, csr_to_mask)
from oracle.mask import oracle_plan


def rand_qkv(seed, B=1, H=2, N=150, D=16):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, D)) for _ in range(3)]


def random_csr(seed, R, nkv, allow_empty=False):
    rng = np.random.default_rng(seed)
    rows = []
    for r in range(R):
        lo = 0 if allow_empty else 1
        c = int(rng.integers(lo, nkv + 1))
        rows.append(np.sort(rng.choice(nkv, size=c, replace=False)))
    row_ptr = np.zeros(R + 1, np.int64)
    row_ptr[1:] = np.cumsum([len(x) for x in rows])
    col = np.concatenate(rows).astype(np.int32) if rows else np.zeros(0, np.int32)
    return row_ptr, col


def test_dense_matches_torch_sdpa_float64():
    q, k, v = rand_qkv(0, N=97, D=32)
    ours = dense_attention(q, k, v)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    assert np.max(np.abs(ours - ref)) < 1e-12


def test_all_ones_plan_equals_dense():
    q, k, v = rand_qkv(1, N=150)
    rp, ci = dense_plan(1, 2, 150, 64, 32)
    o, lse = sparse_attention(q, k, v, rp, ci, 64, 32, with_lse=True)
    od, lsed = dense_attention(q, k, v, with_lse=True)
    assert np.max(np.abs(o - od)) < 1e-12 and np.max(np.abs(lse - lsed)) < 1e-12


@pytest.mark.parametrize("bq,bk,N", [(64, 64, 150), (32, 16, 77), (16, 32, 64)])
def test_sparse_matches_brute_force_mask(bq, bk, N):
    q, k, v = rand_qkv(2, N=N)
    nq, nkv = -(-N // bq), -(-N // bk)
    rp, ci = random_csr(3, 2 * nq, nkv)
    o = sparse_attention(q, k, v, rp, ci, bq, bk)
    ob = brute_masked_attention(q, k, v, csr_to_mask(rp, ci, 1, 2, N, bq, bk))
    assert np.max(np.abs(o - ob)) < 1e-12


def test_lse_matches_logsumexp_over_kept_tokens():
    q, k, v = rand_qkv(4, N=128, D=8)
    rp, ci = random_csr(5, 2 * 2, 4)
    _, lse = sparse_attention(q, k, v, rp, ci, 64, 32, with_lse=True)
    mask = csr_to_mask(rp, ci, 1, 2, 128, 64, 32)
    s = np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(8)
    ref = np.log(np.where(mask, np.exp(s), 0.0).sum(-1))
    assert np.max(np.abs(lse - ref)) < 1e-12


def test_closed_forms():
    q, k, v = rand_qkv(6, N=130)
    rp, ci = random_csr(7, 2 * 3, 5)
    # V constant -> every output row equals that constant, whatever the mask
    vc = np.broadcast_to(np.arange(16.0), v.shape).copy()
    assert np.max(np.abs(sparse_attention(q, k, vc, rp, ci, 64, 32) - np.arange(16.0))) < 1e-12
    # Q = 0 -> uniform weights: the mean of V over the kept tokens
    o = sparse_attention(np.zeros_like(q), k, v, rp, ci, 64, 32)
    for h in range(2):
        for I in range(3):
            r = h * 3 + I
            tok = np.concatenate([np.arange(J * 32, min(130, J * 32 + 32)) for J in ci[rp[r]:rp[r + 1]]])
            assert np.max(np.abs(o[0, h, I * 64:min(130, I * 64 + 64)] - v[0, h, tok].mean(0))) < 1e-12


def test_masked_tiles_never_read():
    q, k, v = rand_qkv(8, N=192)
    rp, ci = random_csr(9, 2 * 3, 6)
    o = sparse_attention(q, k, v, rp, ci, 64, 32)
    mask = csr_to_mask(rp, ci, 1, 2, 192, 64, 32)
    kp, vp = k.copy(), v.copy()
    for h in range(2):
        for I in range(3):
            r = h * 3 + I
            for J in set(range(6)) - set(ci[rp[r]:rp[r + 1]].tolist()):
                # poison blocks that no query block of this head keeps
                if not mask[0, h, :, J * 32].any():
                    kp[0, h, J * 32:J * 32 + 32] = np.nan
                    vp[0, h, J * 32:J * 32 + 32] = np.nan
    o2 = sparse_attention(q, kp, vp, rp, ci, 64, 32)
    assert np.array_equal(o, o2)


def test_kept_order_irrelevant_and_empty_row():
    q, k, v = rand_qkv(10, N=128)
    rp, ci = random_csr(11, 4, 4, allow_empty=True)
    ci2 = ci.copy()
    for r in range(4):
        ci2[rp[r]:rp[r + 1]] = ci2[rp[r]:rp[r + 1]][::-1]
    o1 = sparse_attention(q, k, v, rp, ci, 64, 32)
    o2 = sparse_attention(q, k, v, rp, ci2, 64, 32)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    rp0 = np.array([0, 0, 1, 1, 2])
    ci0 = np.array([0, 3], np.int32)
    o, lse = sparse_attention(q, k, v, rp0, ci0, 64, 32, with_lse=True)
    assert np.all(o[0, 0, :64] == 0) and np.all(lse[0, 0, :64] == -np.inf)


def test_phi_is_elu_plus_one():
    x = np.array([-3.0, -1.0, -1e-9, 0.0, 1e-9, 0.5, 2.0])
    ref = torch.nn.functional.elu(torch.from_numpy(x)).numpy() + 1.0
    assert np.max(np.abs(phi(x) - ref)) < 1e-15
    assert np.all(phi(np.linspace(-50, 50, 1001)) > 0)


def test_linear_branch_explicit_equals_factorised():
    q, k, v = rand_qkv(12, N=200, D=8)
    nq, nkv = 4, 7
    rp, ci = random_csr(13, 2 * nq, nkv)
    ol = linear_branch(q, k, v, rp, ci, 64, 32)
    # factorised: H_C = phi(K_C)^T V_C and z_C = phi(K_C)^T 1 over the complement
    for h in range(2):
        for I in range(nq):
            r = h * nq + I
            comp = sorted(set(range(nkv)) - set(ci[rp[r]:rp[r + 1]].tolist()))
            qs = slice(I * 64, min(200, I * 64 + 64))
            if not comp:
                assert np.all(ol[0, h, qs] == 0)
                continue
            tok = np.concatenate([np.arange(J * 32, min(200, J * 32 + 32)) for J in comp])
            pk = phi(k[0, h, tok])
            Hc = pk.T @ v[0, h, tok]
            zc = pk.sum(0)
            pq = phi(q[0, h, qs])
            ref = (pq @ Hc) / (pq @ zc)[:, None]
            assert np.max(np.abs(ol[0, h, qs] - ref)) < 1e-12


def test_linear_subtractive_complement_identity():
    # the complement sum equals the total minus the kept blocks' sums
    q, k, v = rand_qkv(14, N=256, D=8, H=1)
    rp, ci = random_csr(15, 4, 8)
    ol = linear_branch(q, k, v, rp, ci, 64, 32)
    pk = phi(k[0, 0])
    Htot, ztot = pk.T @ v[0, 0], pk.sum(0)
    for I in range(4):
        kept = ci[rp[I]:rp[I + 1]]
        if len(kept) == 8:
            continue
        tok = np.concatenate([np.arange(J * 32, J * 32 + 32) for J in kept])
        Hk, zk = pk[tok].T @ v[0, 0, tok], pk[tok].sum(0)
        pq = phi(q[0, 0, I * 64:(I + 1) * 64])
        ref = (pq @ (Htot - Hk)) / (pq @ (ztot - zk))[:, None]
        assert np.max(np.abs(ol[0, 0, I * 64:(I + 1) * 64] - ref)) < 1e-10


def test_blend_limits_and_all_kept():
    q, k, v = rand_qkv(16, N=128)
    rp, ci = random_csr(17, 4, 4)
    os_ = sparse_attention(q, k, v, rp, ci, 64, 32)
    ol = linear_branch(q, k, v, rp, ci, 64, 32)
    assert np.array_equal(blend(os_, ol, np.ones((2, 16))), os_)
    assert np.array_equal(blend(os_, ol, np.zeros((2, 16))), ol)
    a = np.random.default_rng(0).uniform(0.5, 1, (2, 16))
    o = blend(os_, ol, a)
    assert np.allclose(o[0, 1, 5], a[1] * os_[0, 1, 5] + (1 - a[1]) * ol[0, 1, 5], atol=0, rtol=1e-15)
    rpd, cid = dense_plan(1, 2, 128, 64, 32)
    assert np.all(linear_branch(q, k, v, rpd, cid, 64, 32) == 0)


def test_oracle_plan_feeds_output_track():
    rng = np.random.default_rng(18)
    q = rng.standard_normal((1, 2, 256, 16)).astype(np.float32)
    k = rng.standard_normal((1, 2, 256, 16)).astype(np.float32)
    v = rng.standard_normal((1, 2, 256, 16)).astype(np.float32)
    rp, ci, _ = oracle_plan(q, k, 64, 32, 0.25, 0.5)
    o = sparse_attention(q, k, v, rp, ci, 64, 32)
    ob = brute_masked_attention(q, k, v, csr_to_mask(rp, ci, 1, 2, 256, 64, 32))
    assert np.max(np.abs(o - ob)) < 1e-12
    sub = sparse_attention(q, k, v, rp, ci, 64, 32, rows=[(0, 1, 2)])
    assert np.max(np.abs(sub[(0, 1, 2)][0] - o[0, 1, 128:192])) < 1e-15
