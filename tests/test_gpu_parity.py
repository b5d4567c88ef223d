"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Masks (the hybrid top-k / top-p router, SpargeAttention2 page section 2(1), with mean
pooling per block, SLA2 page router item 1) must be bit-identical CSR. Outputs of the
block-sparse forward (SpargeAttention2 page section 2(3)) must be within max |dO| 1e-4
for fp32 inputs, and max |dO| 2e-2 with relative RMS 5e-3 for bf16 inputs, against the
float64 oracle on the same seeded inputs.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_05_amd as sa
import workloads as W
from oracle import (oracle_plan, sparse_attention, dense_attention, dense_plan, exp_sa,
                    topk_count, block_scores, pool_blocks, score_scale)
from tests.gpu_common import drop, check_out, inputs, log, sample_rows, to_dev, to_f64

pytestmark = pytest.mark.gpu


def gpu_plan(w: W.Workload, ent):
    p = sa.plan(ent["dq"], ent["dk"], w.block_q, w.block_kv, w.topk, w.top_p)
    return p, p.csr()


def assert_same_csr(got, ref, what):
    rp, ci = got
    rrp, rci = ref
    assert rp.shape == rrp.shape, what
    bad = np.nonzero(rp != rrp)[0]
    assert bad.size == 0, f"{what}: row_ptr differs first at {bad[:5]}"
    assert np.array_equal(ci, rci), f"{what}: col_idx differs"


# ------------------------------------------------------------------ router exp
def test_router_exp_bitwise():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        np.linspace(-86.0, 0.0, 4_000_001).astype(np.float32),
        -rng.exponential(2.0, 2_000_000).astype(np.float32),
        np.array([0.0, -0.0, -86.0, -86.00001, -1e-30, -1e-45, -np.inf, -1000.0], np.float32),
    ])
    y = sa.router_exp(to_dev(x)).cpu().numpy()
    ref = exp_sa(x)
    bad = np.nonzero(y.view(np.uint32) != ref.view(np.uint32))[0]
    assert bad.size == 0, f"{bad.size} mismatches, e.g. x={x[bad[:4]]} gpu={y[bad[:4]]} cpu={ref[bad[:4]]}"


def test_router_exp_strided_exhaustive():
    """Every 61st fp32 bit pattern in [-86, 0] (the full range, strided)."""
    lo = np.float32(-86.0).view(np.uint32)
    pats = np.arange(0x80000000, int(lo) + 1, 61, dtype=np.uint64).astype(np.uint32)
    pats = np.concatenate([pats, np.arange(0, 1, dtype=np.uint32)])
    x = pats.view(np.float32)
    for s in range(0, x.size, 4_000_000):
        xs = x[s:s + 4_000_000]
        y = sa.router_exp(to_dev(xs)).cpu().numpy()
        assert np.array_equal(y.view(np.uint32), exp_sa(xs).view(np.uint32)), s


# ------------------------------------------------------------------ small cases
SMALL = [
    # name, B, H, N, D, dtype, bq, topk, p
    ("tiny_like", 1, 2, 1024, 64, "fp32", 64, 0.25, 0.9),
    ("ragged_bf16", 1, 2, 1000, 64, "bf16", 64, 0.1, 0.9),
    ("ragged_q128", 2, 3, 3000, 128, "bf16", 128, 0.05, 0.9),
    ("d128_fp32", 1, 2, 700, 128, "fp32", 64, 0.3, 0.5),
    ("argmax_only", 1, 2, 2048, 64, "bf16", 128, 0.0, 0.0),
    ("topk_all", 1, 1, 2048, 64, "bf16", 128, 1.0, 0.0),
    ("topp_all", 1, 1, 2048, 64, "bf16", 128, 0.0, 1.0),
    ("nkv300", 1, 2, 64 * 300 - 5, 128, "bf16", 128, 0.03, 0.95),
    ("nkv1100", 1, 1, 64 * 1100 + 7, 128, "bf16", 128, 0.02, 0.85),
    ("d64_q128_fp32", 1, 3, 1536, 64, "fp32", 128, 0.1, 0.7),
    # fewer tokens than one block: one ragged query block and one ragged KV block
    ("n1", 1, 2, 1, 64, "bf16", 64, 0.5, 0.9),
    ("n37_fp32", 1, 2, 37, 128, "fp32", 128, 0.5, 0.9),
    ("n65_q128", 2, 1, 65, 128, "bf16", 128, 0.3, 0.9),
]


def small_workload(name, B, H, N, D, dtype, bq, topk, p, seed=0):
    T = 1
    return W.Workload(name, B, H, D, (T, 1, N), dtype, bq, 64, topk, p, 4, seed=seed)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_plan_bitexact_small(case):
    w = small_workload(*case)
    log(f"plan {w.name} B={w.B} H={w.H} N={w.N} D={w.D} {w.dtype} bq={w.block_q}")
    ent = inputs(w)
    _, got = gpu_plan(w, ent)
    rp, ci, _ = oracle_plan(ent["q32"], ent["k32"], w.block_q, w.block_kv, w.topk, w.top_p)
    assert_same_csr(got, (rp, ci), w.name)


def visit_reference(S_row, kept, nkv, ragged, every):
    """Host restatement of a row's visit order: its kept blocks by score, descending, ties
    to the lower index (ascending when every block is kept by rule), a kept ragged last
    block moved to the end."""
    kept_set = set(int(J) for J in kept)
    order = range(nkv) if every else np.argsort(-S_row, kind="stable")
    out = [int(J) for J in order if int(J) in kept_set]
    if ragged and nkv - 1 in kept_set:
        out.remove(nkv - 1)
        out.append(nkv - 1)
    return out


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_plan_visit_order(case):
    """The plan's visit lists (the order in which the forward takes a row's kept tiles):
    each row's kept set in the router's score order (descending, ties to the lower block
    index), with a kept ragged last block moved to the end; when every block is kept by
    rule (top_p >= 1 or m_k = nKV) the order is ascending."""
    w = small_workload(*case)
    log(f"visit order {w.name}")
    ent = inputs(w)
    p, (rp, ci) = gpu_plan(w, ent)
    vl = p.visit_lists()
    assert vl is not None
    nq, nkv = w.n_qblk, w.n_kvblk
    every = w.top_p >= 1.0 or topk_count(w.topk, nkv) >= nkv
    ragged = w.N % w.block_kv != 0
    for b in range(w.B):
        for h in range(w.H):
            S = block_scores(pool_blocks(ent["q32"][b, h], w.block_q),
                             pool_blocks(ent["k32"][b, h], w.block_kv), score_scale(w.D))
            for I in range(nq):
                r = (b * w.H + h) * nq + I
                kept = ci[rp[r]:rp[r + 1]]
                assert vl[r].tolist() == visit_reference(S[I], kept, nkv, ragged, every), (w.name, r)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_fwd_small(case):
    w = small_workload(*case)
    log(f"fwd {w.name}")
    ent = inputs(w)
    p, (rp, ci) = gpu_plan(w, ent)
    o, lse = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p, return_lse=True)
    ref, rlse = sparse_attention(ent["q32"], ent["k32"], W.to_f32(ent["v"]), rp, ci, w.block_q,
                                 w.block_kv, with_lse=True)
    check_out(to_f64(o), ref, w.dtype, w.name)
    assert np.max(np.abs(to_f64(lse) - rlse)) < (1e-4 if w.dtype == "fp32" else 2e-3)
    # without the LSE output the bf16 kernel keeps a lazy running max: O to the same bar
    check_out(to_f64(sa.fwd(ent["dq"], ent["dk"], ent["dv"], p)), ref, w.dtype, w.name + " no lse")


def test_fwd_signed_zero_queries():
    """All scores zero: with q = +0 and with q = -0 every kept key gets the same weight, so
    O is the mean of the kept V rows. The tile max is then +0 or -0, which must not change
    any output bit, with or without the LSE output."""
    import torch
    w = small_workload("ragged_q128", 2, 3, 3000, 128, "bf16", 128, 0.05, 0.9)
    log(f"fwd signed-zero queries {w.name}")
    ent = inputs(w)
    p, (rp, ci) = gpu_plan(w, ent)
    qpos = torch.zeros_like(ent["dq"])
    qneg = torch.full(ent["dq"].shape, 0x8000 - 0x10000, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    assert torch.signbit(qneg.float()).all() and not torch.signbit(qpos.float()).any()
    z32 = np.zeros(ent["q32"].shape, np.float32)
    ref, rlse = sparse_attention(z32, ent["k32"], W.to_f32(ent["v"]), rp, ci, w.block_q, w.block_kv,
                                 with_lse=True)
    outs = []
    for q in (qpos, qneg):
        o, lse = sa.fwd(q, ent["dk"], ent["dv"], p, return_lse=True)
        check_out(to_f64(o), ref, w.dtype, "zero q with lse")
        assert np.max(np.abs(to_f64(lse) - rlse)) < 2e-3
        o2 = sa.fwd(q, ent["dk"], ent["dv"], p)
        check_out(to_f64(o2), ref, w.dtype, "zero q")
        outs.append((o, lse, o2))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_plan_nnz_scalar():
    """The plan's device nnz scalar equals row_ptr[R] for the router's plan, the dense
    plan and a caller's CSR."""
    w = small_workload("nnz", 2, 3, 3000, 128, "bf16", 128, 0.05, 0.9)
    ent = inputs(w)
    p, (rp, ci) = gpu_plan(w, ent)
    assert int(p.nnz().item()) == int(rp[-1]) == ci.size
    pd = sa.plan_dense(ent["dq"], 128, 64)
    assert int(pd.nnz().item()) == w.rows * w.n_kvblk
    rows = [np.arange(0, w.n_kvblk, 3)] * w.rows
    crp = np.concatenate([[0], np.cumsum([len(r) for r in rows])])
    pc = sa.plan_from_csr(ent["dq"], crp, np.concatenate(rows).astype(np.int32), 128, 64)
    assert int(pc.nnz().item()) == int(crp[-1])


def test_tie_breaks_to_lower_block():
    w = small_workload("ties", 1, 2, 1024, 64, "bf16", 64, 1.0 / 16, 0.0)
    q, k, v, _ = W.make_inputs(w)
    k[:, :, 5 * 64:6 * 64] = k[:, :, 11 * 64:12 * 64]   # KV blocks 5 and 11 identical
    q32, k32 = W.to_f32(q), W.to_f32(k)
    p = sa.plan(to_dev(q), to_dev(k), 64, 64, w.topk, w.top_p)
    rp, ci, _ = oracle_plan(q32, k32, 64, 64, w.topk, w.top_p)
    assert_same_csr(p.csr(), (rp, ci), "ties")
    assert 11 not in set(ci.tolist()) or 5 in set(ci.tolist())


@pytest.mark.parametrize("scale,nkv,H", [(0.0, 1100, 2), (1e-3, 1100, 2), (0.3, 1100, 2),
                                         (0.0, 2500, 1), (1e-3, 2500, 1)])
def test_plan_flat_and_near_flat_rows(scale, nkv, H):
    """Near-uniform pooled scores over 1,100 KV blocks put more than 512 blocks into the
    top exponent bin, so the router takes its full-sort path; a scale of 0 gives exact
    ties everywhere (lowest block index first). 2,500 blocks take the path with 16 items
    per thread, where e is recomputed from the sort keys."""
    w = small_workload(f"flat{scale}_{nkv}", 1, H, 64 * nkv, 64, "bf16", 128, 0.02, 0.9)
    q, k, v, _ = W.make_inputs(w)
    k32 = W.to_f32(k) * scale
    kb = W.f64_to_bf16_bits(k32.astype(np.float64))
    p = sa.plan(to_dev(q), to_dev(kb), w.block_q, w.block_kv, w.topk, w.top_p)
    rp, ci, mp = oracle_plan(W.to_f32(q), W.to_f32(kb), w.block_q, w.block_kv, w.topk, w.top_p)
    assert_same_csr(p.csr(), (rp, ci), f"flat {scale}")
    if scale == 0.0:
        assert np.all(np.diff(rp) == np.diff(rp)[0])
    # visit lists from the full-sort path: the kept set in score order, ties ascending
    rows = [h * w.n_qblk + I for h in range(w.H) for I in (0, 7, w.n_qblk - 1)]
    vl = p.visit_lists(rows=rows)
    q32, k32 = W.to_f32(q), W.to_f32(kb)
    for h in range(w.H):
        S = block_scores(pool_blocks(q32[0, h], w.block_q), pool_blocks(k32[0, h], w.block_kv),
                         score_scale(w.D))
        for I in (0, 7, w.n_qblk - 1):
            r = h * w.n_qblk + I
            kept = ci[rp[r]:rp[r + 1]]
            assert vl[r].tolist() == visit_reference(S[I], kept, w.n_kvblk, False, False), (scale, r)


def test_dense_plan_matches_dense_oracle():
    w = small_workload("dense", 1, 2, 1000, 128, "bf16", 128, 0.1, 0.9)
    ent = inputs(w)
    p = sa.plan_dense(ent["dq"], 128, 64)
    rp, ci = p.csr()
    drp, dci = dense_plan(1, 2, 1000, 128, 64)
    assert np.array_equal(rp, drp) and np.array_equal(ci, dci)
    o = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p)
    ref = dense_attention(ent["q32"], ent["k32"], W.to_f32(ent["v"]))
    check_out(to_f64(o), ref, "bf16", "dense")


def test_dense_plan_fp32_matches_torch_sdpa():
    w = small_workload("dense32", 1, 2, 1024, 64, "fp32", 64, 0.1, 0.9)
    ent = inputs(w)
    p = sa.plan_dense(ent["dq"], 64, 64)
    o = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(ent["q"]).double(), torch.from_numpy(ent["k"]).double(),
        torch.from_numpy(ent["v"]).double()).numpy()
    check_out(to_f64(o), ref, "fp32", "dense fp32 vs sdpa")


def test_caller_csr_with_empty_rows_and_lse():
    w = small_workload("csr", 1, 2, 640, 64, "bf16", 64, 0.1, 0.9)
    ent = inputs(w)
    nq = nkv = 10
    rng = np.random.default_rng(3)
    rows = []
    for r in range(2 * nq):
        c = 0 if r % 4 == 1 else int(rng.integers(1, nkv + 1))
        rows.append(np.sort(rng.choice(nkv, c, replace=False)))
    rp = np.zeros(2 * nq + 1, np.int64)
    rp[1:] = np.cumsum([len(x) for x in rows])
    ci = np.concatenate(rows).astype(np.int32)
    p = sa.plan_from_csr(ent["dq"], rp, ci, 64, 64)
    grp, gci = p.csr()
    assert np.array_equal(grp, rp) and np.array_equal(gci, ci)
    o, lse = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p, return_lse=True)
    ref, rlse = sparse_attention(ent["q32"], ent["k32"], W.to_f32(ent["v"]), rp, ci, 64, 64,
                                 with_lse=True)
    check_out(to_f64(o), ref, "bf16", "caller csr")
    lg = to_f64(lse)
    assert np.array_equal(np.isinf(lg), np.isinf(rlse))
    fin = np.isfinite(rlse)
    assert np.max(np.abs(lg[fin] - rlse[fin])) < 2e-3
    assert np.all(to_f64(o)[0, 0, 64:128] == 0)      # row 1 is empty


def test_masked_tiles_are_never_read():
    """Poison with NaN every KV block that one target row does not keep: that row's output,
    and that of every row whose kept set lies inside the target's, must not change
    (masked tiles are skipped, SpargeAttention2 page, section 2(3))."""
    w = small_workload("poison", 1, 2, 64 * 40, 128, "bf16", 128, 0.05, 0.5)
    ent = inputs(w)
    p, (rp, ci) = gpu_plan(w, ent)
    o1 = to_f64(sa.fwd(ent["dq"], ent["dk"], ent["dv"], p))
    nq = w.n_qblk
    checked = 0
    for h in range(2):
        target = h * nq + 3
        keep = set(ci[rp[target]:rp[target + 1]].tolist())
        assert len(keep) < w.n_kvblk
        k2, v2 = ent["dk"].clone(), ent["dv"].clone()
        for J in range(w.n_kvblk):
            if J not in keep:
                k2[0, h, J * 64:(J + 1) * 64] = float("nan")
                v2[0, h, J * 64:(J + 1) * 64] = float("nan")
        o2 = to_f64(sa.fwd(ent["dq"], k2, v2, p))
        for I in range(nq):
            r = h * nq + I
            if set(ci[rp[r]:rp[r + 1]].tolist()) <= keep:
                sl = slice(I * 128, (I + 1) * 128)
                assert np.array_equal(o1[0, h, sl], o2[0, h, sl]), (h, I)
                checked += 1
        assert np.array_equal(o1[0, 1 - h], o2[0, 1 - h])
    assert checked >= 2


def test_deterministic_bitwise():
    w = small_workload("det", 1, 3, 4000, 128, "bf16", 128, 0.05, 0.9)
    ent = inputs(w)
    p1, c1 = gpu_plan(w, ent)
    p2, c2 = gpu_plan(w, ent)
    assert np.array_equal(c1[0], c2[0]) and np.array_equal(c1[1], c2[1])
    o1 = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p1)
    o2 = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


# ------------------------------------------------------------------ the workloads
def test_tiny_fp32_config():
    w = W.CONFIGS["tiny_fp32"]
    ent = inputs(w)
    p, got = gpu_plan(w, ent)
    rp, ci, _ = oracle_plan(ent["q32"], ent["k32"], w.block_q, w.block_kv, w.topk, w.top_p)
    assert_same_csr(got, (rp, ci), w.name)
    o = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p)
    ref = sparse_attention(ent["q"], ent["k"], ent["v"], rp, ci, w.block_q, w.block_kv)
    mx, _ = check_out(to_f64(o), ref, "fp32", w.name)
    log(f"{w.name}: max|dO| {mx:.2e}")


@pytest.mark.parametrize("name", ["wan13b_480p", "wan14b_720p"])
def test_workload_plan_bitexact_full(name):
    w = W.CONFIGS[name]
    ent = inputs(w)
    p, got = gpu_plan(w, ent)
    log(f"{name}: gpu plan nnz {got[0][-1]}")
    rp, ci, _ = oracle_plan(ent["q32"], ent["k32"], w.block_q, w.block_kv, w.topk, w.top_p)
    assert_same_csr(got, (rp, ci), name)
    log(f"{name}: tile sparsity {1 - rp[-1] / (w.rows * w.n_kvblk):.4f}")


def test_wan13b_480p_output_full():
    w = W.CONFIGS["wan13b_480p"]
    ent = inputs(w)
    p, (rp, ci) = gpu_plan(w, ent)
    o = to_f64(sa.fwd(ent["dq"], ent["dk"], ent["dv"], p))
    ref = sparse_attention(ent["q32"], ent["k32"], W.to_f32(ent["v"]), rp, ci, w.block_q, w.block_kv)
    mx, rr = check_out(o, ref, "bf16", w.name)
    log(f"{w.name}: max|dO| {mx:.2e} rel-RMS {rr:.2e}")


@pytest.mark.parametrize("name,per_head", [("wan14b_720p", 4), ("long_245k", 12)])
def test_workload_output_sampled(name, per_head):
    w = W.CONFIGS[name]
    ent = inputs(w)
    p, (rp, ci) = gpu_plan(w, ent)
    rows = sample_rows(w, per_head)
    sub = oracle_plan(ent["q32"], ent["k32"], w.block_q, w.block_kv, w.topk, w.top_p, rows=rows)
    nq = w.n_qblk
    mk = topk_count(w.topk, w.n_kvblk)
    counts = np.diff(rp)
    assert counts.min() >= mk
    for (b, h, I), kept in sub.items():
        r = (b * w.H + h) * nq + I
        assert ci[rp[r]:rp[r + 1]].tolist() == kept.tolist(), (b, h, I)
    # the sampled rows' visit lists against the oracle's scores
    vl = p.visit_lists(rows=[(b * w.H + h) * nq + I for (b, h, I) in sub])
    kbars = {}
    for (b, h, I), kept in sub.items():
        if (b, h) not in kbars:
            kbars[(b, h)] = pool_blocks(ent["k32"][b, h], w.block_kv)
        qbar = pool_blocks(ent["q32"][b, h, I * w.block_q:min(w.N, (I + 1) * w.block_q)], w.block_q)
        S_row = block_scores(qbar, kbars[(b, h)], score_scale(w.D))[0]
        r = (b * w.H + h) * nq + I
        assert vl[r].tolist() == visit_reference(S_row, kept, w.n_kvblk, w.N % w.block_kv != 0, False), (b, h, I)
    o = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p)
    ref = sparse_attention(ent["q32"], ent["k32"], W.to_f32(ent["v"]), rp, ci, w.block_q,
                           w.block_kv, rows=rows)
    got, want = [], []
    for (b, h, I), (ob, _) in ref.items():
        sl = slice(I * w.block_q, min(w.N, (I + 1) * w.block_q))
        got.append(to_f64(o[b, h, sl]))
        want.append(ob)
    mx, rr = check_out(np.concatenate(got), np.concatenate(want), "bf16", name)
    log(f"{name}: sampled {len(rows)} rows max|dO| {mx:.2e} rel-RMS {rr:.2e}")


def test_max_kv_blocks_sampled():
    """The largest supported sequence: 4096 KV blocks (N = 262,144) in one head. Sampled
    rows' masks bit-exact and their outputs within the bf16 bound."""
    w = W.Workload("max_kv", 1, 1, 64, (64, 64, 64), "bf16", 128, 64, 0.01, 0.85, 16, seed=2)
    assert w.n_kvblk == 4096
    ent = inputs(w)
    p, (rp, ci) = gpu_plan(w, ent)
    rows = sample_rows(w, 8)
    sub = oracle_plan(ent["q32"], ent["k32"], w.block_q, w.block_kv, w.topk, w.top_p, rows=rows)
    for (b, h, I), kept in sub.items():
        r = (b * w.H + h) * w.n_qblk + I
        assert ci[rp[r]:rp[r + 1]].tolist() == kept.tolist(), (b, h, I)
    o = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p)
    ref = sparse_attention(ent["q32"], ent["k32"], W.to_f32(ent["v"]), rp, ci, w.block_q, w.block_kv,
                           rows=rows)
    got, want = [], []
    for (b, h, I), (ob, _) in ref.items():
        sl = slice(I * w.block_q, min(w.N, (I + 1) * w.block_q))
        got.append(to_f64(o[b, h, sl]))
        want.append(ob)
    mx, rr = check_out(np.concatenate(got), np.concatenate(want), "bf16", w.name)
    log(f"{w.name}: nnz {rp[-1]}, sampled {len(rows)} rows max|dO| {mx:.2e} rel-RMS {rr:.2e}")
    drop(w)


@pytest.mark.parametrize("name,nrows", [("wan14b_720p", 24), ("long_245k", 8)])
def test_workload_dense_sampled(name, nrows):
    w = W.CONFIGS[name]
    ent = inputs(w)
    p = sa.plan_dense(ent["dq"], w.block_q, w.block_kv)
    o = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p)
    rng = np.random.default_rng(7)
    rows = [(0, int(rng.integers(0, w.H)), int(I)) for I in
            np.concatenate([[0, w.n_qblk - 1], rng.integers(0, w.n_qblk, nrows - 2)])]
    drp, dci = dense_plan(w.B, w.H, w.N, w.block_q, w.block_kv)
    ref = sparse_attention(ent["q32"], ent["k32"], W.to_f32(ent["v"]), drp, dci, w.block_q,
                           w.block_kv, rows=rows)
    got, want = [], []
    for (b, h, I), (ob, _) in ref.items():
        sl = slice(I * w.block_q, min(w.N, (I + 1) * w.block_q))
        got.append(to_f64(o[b, h, sl]))
        want.append(ob)
    mx, rr = check_out(np.concatenate(got), np.concatenate(want), "bf16", name + " dense")
    log(f"{name} dense: sampled {len(rows)} rows max|dO| {mx:.2e} rel-RMS {rr:.2e}")


# ------------------------------------------------------------------ work order
def order_chunks(R, nQ):
    """Runs of consecutive rows the work order deals out: whole heads, each head cut into
    k equal runs when there are fewer than 32 heads, or g heads per run beyond 512 runs."""
    M = 8 * (R // 8)
    BH = R // nQ
    k = 1 if BH >= 32 else min(nQ, -(-32 // BH))
    g = -(-BH // 512) if BH > 512 else 1
    out = []
    if g > 1:
        for c in range(-(-BH // g)):
            out.append((c * g * nQ, min(BH, (c + 1) * g) * nQ))
    else:
        for h in range(BH):
            for j in range(k):
                out.append((h * nQ + j * nQ // k, h * nQ + (j + 1) * nQ // k))
    return [(min(s, M), min(e, M) - min(s, M)) for s, e in out]


def balanced_order_reference(rp, nQ):
    """Host restatement of the plan's work order: head-aligned runs of consecutive rows
    dealt to the eight XCD slot ranges, heaviest run first, each to the least-loaded
    range with room (a run that does not fit is split); a range holds its runs in the
    order they were dealt."""
    R = rp.size - 1
    q = R // 8
    order = np.arange(R, dtype=np.int64)
    if q == 0:
        return order
    chunks = order_chunks(R, nQ)
    work = [int(rp[s + n] - rp[s]) for s, n in chunks]
    ranked = sorted(range(len(chunks)), key=lambda c: (-work[c], c))
    load, cap = [0] * 8, [q] * 8
    for c in ranked:
        start, ln = chunks[c]
        len0 = ln
        while ln > 0:
            x = min((y for y in range(8) if cap[y] > 0), key=lambda y: (load[y], y))
            take = min(ln, cap[x])
            off = x * q + (q - cap[x])
            order[off:off + take] = np.arange(start, start + take)
            load[x] += work[c] if take == len0 else (work[c] // len0) * take
            cap[x] -= take
            start += take
            ln -= take
    return order


@pytest.mark.parametrize("name", ["wan14b_720p", "wan13b_480p"])
def test_row_order_balanced(name):
    w = W.CONFIGS[name]
    ent = inputs(w)
    p, (rp, _) = gpu_plan(w, ent)
    got = p.row_order().cpu().numpy().astype(np.int64)
    R = rp.size - 1
    assert np.array_equal(np.sort(got), np.arange(R)), "not a permutation"
    ref = balanced_order_reference(rp, w.n_qblk)
    assert np.array_equal(got, ref)
    q = R // 8
    cnt = np.diff(rp)
    tot = np.array([cnt[got[x * q:(x + 1) * q]].sum() for x in range(8)])
    log(f"{name}: per-XCD kept tiles {tot.tolist()}, max/mean {tot.max() / tot.mean():.4f}")
    heaviest = max(rp[s + n] - rp[s] for s, n in order_chunks(R, w.n_qblk))
    assert tot.max() <= tot.mean() + heaviest


@pytest.mark.parametrize("case", [SMALL[0], SMALL[2], SMALL[7]], ids=["tiny_like", "ragged_q128", "nkv300"])
def test_row_order_small(case):
    w = small_workload(*case)
    ent = inputs(w)
    p, (rp, _) = gpu_plan(w, ent)
    got = p.row_order().cpu().numpy().astype(np.int64)
    assert np.array_equal(got, balanced_order_reference(rp, w.n_qblk))
    pd = sa.plan_dense(ent["dq"], w.block_q, w.block_kv)
    rpd = pd.row_ptr().cpu().numpy().astype(np.int64)
    assert np.array_equal(pd.row_order().cpu().numpy().astype(np.int64),
                          balanced_order_reference(rpd, w.n_qblk))
