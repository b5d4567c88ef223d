"""GPU parity of the linear-attention branch and the blend.

Ol over each query block's masked-out KV blocks with phi = elu + 1 (SALAD page, section
2.1; SLA2 page: dropped blocks feed the linear branch), and O = alpha*Os + (1-alpha)*Ol
(SLA2 page, item 2), against the float64 oracle, which forms every phi(q).phi(k) weight
explicitly.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_05_amd as sa
import workloads as W
from oracle import blend, linear_branch, oracle_plan, sparse_attention
from tests.gpu_common import check_out, inputs, log, sample_rows, to_dev, to_f64

pytestmark = pytest.mark.gpu


def small(name, H, N, D, bq, topk, p, seed=0):
    return W.Workload(name, 1, H, D, (1, 1, N), "bf16", bq, 64, topk, p, 4, linear=True, seed=seed)


def offset_v(ent, shift=1.5):
    """V + shift (re-rounded to bf16) so that the linear average is of order one."""
    v = W.to_f32(ent["v"]).astype(np.float64) + shift
    vb = W.f64_to_bf16_bits(v)
    return vb, to_dev(vb)


CASES = [("lin_d128_q128", 2, 3000, 128, 128, 0.05, 0.8),
         ("lin_d64_q64", 2, 1000, 64, 64, 0.1, 0.7),
         ("lin_d128_q64", 1, 2500, 128, 64, 0.03, 0.6),
         ("lin_d64_q128", 3, 1536, 64, 128, 0.2, 0.9)]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_linear_output_alpha0(case):
    """alpha = 0 makes O equal Ol, compared on its own scale."""
    w = small(*case)
    log(f"linear {w.name}")
    ent = inputs(w)
    vb, dv = offset_v(ent)
    p = sa.plan(ent["dq"], ent["dk"], w.block_q, w.block_kv, w.topk, w.top_p)
    rp, ci = p.csr()
    a0 = torch.zeros((w.H, w.D), dtype=torch.float32, device="cuda")
    o = to_f64(sa.fwd(ent["dq"], ent["dk"], dv, p, alpha=a0))
    ol = linear_branch(ent["q32"], ent["k32"], W.to_f32(vb), rp, ci, w.block_q, w.block_kv)
    mx, rr = check_out(o, ol, "bf16", w.name + " Ol")
    log(f"{w.name}: Ol max|d| {mx:.2e} rel-RMS {rr:.2e}")


def test_linear_all_modes_via_caller_csr():
    """Rows that keep nothing, everything, more than half (complement summed directly)
    and at most half (totals minus kept tiles), with random alpha."""
    w = small("lin_modes", 2, 64 * 24, 128, 128, 0.1, 0.9)
    ent = inputs(w)
    vb, dv = offset_v(ent, 0.7)
    nq, nkv = w.n_qblk, w.n_kvblk
    rng = np.random.default_rng(11)
    rows = []
    for r in range(2 * nq):
        mode = r % 4
        if mode == 0:
            c = 0
        elif mode == 1:
            c = nkv
        elif mode == 2:
            c = int(rng.integers(nkv // 2 + 1, nkv))
        else:
            c = int(rng.integers(1, nkv // 2 + 1))
        rows.append(np.sort(rng.choice(nkv, c, replace=False)))
    rp = np.zeros(2 * nq + 1, np.int64)
    rp[1:] = np.cumsum([len(x) for x in rows])
    ci = np.concatenate(rows).astype(np.int32)
    p = sa.plan_from_csr(ent["dq"], rp, ci, w.block_q, w.block_kv)
    alpha = np.random.default_rng(5).uniform(0.0, 1.0, (w.H, w.D)).astype(np.float32)
    o = to_f64(sa.fwd(ent["dq"], ent["dk"], dv, p, alpha=to_dev(alpha)))
    os_ = sparse_attention(ent["q32"], ent["k32"], W.to_f32(vb), rp, ci, w.block_q, w.block_kv)
    ol = linear_branch(ent["q32"], ent["k32"], W.to_f32(vb), rp, ci, w.block_q, w.block_kv)
    ref = blend(os_, ol, alpha)
    mx, rr = check_out(o, ref, "bf16", "modes")
    log(f"modes: max|d| {mx:.2e} rel-RMS {rr:.2e}")
    # Ol alone in every mode (alpha = 0)
    o0 = to_f64(sa.fwd(ent["dq"], ent["dk"], dv, p, alpha=torch.zeros_like(to_dev(alpha))))
    check_out(o0, ol, "bf16", "modes Ol")
    # a row that keeps every block has Ol = 0, so O = 0 there with alpha = 0
    assert np.all(o0[0, 0, 128:256] == 0)


def test_alpha_one_equals_plain_forward():
    w = small("lin_a1", 2, 3000, 128, 128, 0.05, 0.8)
    ent = inputs(w)
    p = sa.plan(ent["dq"], ent["dk"], w.block_q, w.block_kv, w.topk, w.top_p)
    o_plain = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p)
    a1 = torch.ones((w.H, w.D), dtype=torch.float32, device="cuda")
    o_lin = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p, alpha=a1)
    assert torch.equal(o_plain.view(torch.int16), o_lin.view(torch.int16))


def test_linear_deterministic():
    w = small("lin_det", 2, 3000, 128, 128, 0.05, 0.8)
    ent = inputs(w)
    p = sa.plan(ent["dq"], ent["dk"], w.block_q, w.block_kv, w.topk, w.top_p)
    o1 = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p, alpha=ent["dalpha"])
    o2 = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p, alpha=ent["dalpha"])
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_sparse_linear_workload_sampled():
    """The sparse+linear workload (480p shapes, k = 2%, p = 0.8, alpha ~ U(0.5, 1)):
    the mask in full, O on sampled query blocks against the oracle blend."""
    w = W.CONFIGS["sparse_linear"]
    ent = inputs(w)
    p = sa.plan(ent["dq"], ent["dk"], w.block_q, w.block_kv, w.topk, w.top_p)
    rp, ci = p.csr()
    orp, oci, _ = oracle_plan(ent["q32"], ent["k32"], w.block_q, w.block_kv, w.topk, w.top_p)
    assert np.array_equal(rp, orp) and np.array_equal(ci, oci)
    log(f"sparse_linear: tile sparsity {1 - rp[-1] / (w.rows * w.n_kvblk):.4f}")
    o = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p, alpha=ent["dalpha"])
    rows = sample_rows(w, 3)
    v32 = W.to_f32(ent["v"])
    os_ = sparse_attention(ent["q32"], ent["k32"], v32, rp, ci, w.block_q, w.block_kv, rows=rows)
    ol = linear_branch(ent["q32"], ent["k32"], v32, rp, ci, w.block_q, w.block_kv, rows=rows)
    got, want = [], []
    for (b, h, I) in rows:
        sl = slice(I * w.block_q, min(w.N, (I + 1) * w.block_q))
        got.append(to_f64(o[b, h, sl]))
        want.append(blend(os_[(b, h, I)][0], ol[(b, h, I)], ent["alpha"], h=h))
    mx, rr = check_out(np.concatenate(got), np.concatenate(want), "bf16", w.name)
    log(f"{w.name}: sampled {len(rows)} rows max|dO| {mx:.2e} rel-RMS {rr:.2e}")


@pytest.mark.parametrize("D,tail", [(128, 47), (128, 17), (64, 17)])
def test_linear_tile_counts(D, tail):
    """Rows whose tile lists (kept tiles, or the complement when more than half is kept)
    hold 1 to 5 tiles, with the ragged last KV block (tail tokens: more, or fewer, than
    half a block) inside some of them: every fill level of the apply step's load pipeline,
    and its tail, against the oracle's Ol (alpha = 0)."""
    w = small(f"lin_counts_d{D}_t{tail}", 1, 64 * 19 + tail, D, 128, 0.1, 0.9)
    ent = inputs(w)
    vb, dv = offset_v(ent, 0.9)
    nq, nkv = w.n_qblk, w.n_kvblk
    assert nq == 10 and nkv == 20
    rng = np.random.default_rng(23)
    rows = []
    for r in range(nq):
        n = r % 5 + 1 if r < 5 else r - 4                  # tiles in the row's list
        with_last = r % 2 == 0                               # the ragged block among them
        pool = np.arange(nkv - 1)
        pick = list(rng.choice(pool, n - 1 if with_last else n, replace=False))
        if with_last:
            pick.append(nkv - 1)
        if r < 5:                                            # kept tiles, summed and subtracted
            rows.append(np.sort(np.array(pick)))
        else:                                                # complement summed directly
            rows.append(np.setdiff1d(np.arange(nkv), pick))
    rp = np.zeros(nq + 1, np.int64)
    rp[1:] = np.cumsum([len(x) for x in rows])
    ci = np.concatenate(rows).astype(np.int32)
    p = sa.plan_from_csr(ent["dq"], rp, ci, w.block_q, w.block_kv)
    a0 = torch.zeros((w.H, w.D), dtype=torch.float32, device="cuda")
    o = to_f64(sa.fwd(ent["dq"], ent["dk"], dv, p, alpha=a0))
    ol = linear_branch(ent["q32"], ent["k32"], W.to_f32(vb), rp, ci, w.block_q, w.block_kv)
    mx, rr = check_out(o, ol, "bf16", w.name + " Ol")
    log(f"{w.name}: Ol max|d| {mx:.2e} rel-RMS {rr:.2e}")


def test_linear_at_the_kv_block_limit():
    """4096 KV blocks (N = 262,144, one head): rows whose tile lists reach the apply step's
    capacity of nKV / 2 entries in both modes (2,048 kept tiles subtracted; 2,049 kept, so
    2,047 complement tiles summed), a row that sums 1,096 complement tiles, and rows that
    keep one block; Ol (alpha = 0) on those rows against the oracle's explicit form."""
    w = W.Workload("lin_max_kv", 1, 1, 64, (64, 64, 64), "bf16", 128, 64, 0.01, 0.85, 16, linear=True, seed=4)
    assert w.n_kvblk == 4096 and w.n_qblk == 2048
    ent = inputs(w)
    vb, dv = offset_v(ent, 0.5)
    nq, nkv = w.n_qblk, w.n_kvblk
    rng = np.random.default_rng(31)
    keep_counts = {0: 2048, 1: 2049, 2: 3000}
    rows = []
    for r in range(nq):
        c = keep_counts.get(r, 1)
        rows.append(np.sort(rng.choice(nkv, c, replace=False)))
    rp = np.zeros(nq + 1, np.int64)
    rp[1:] = np.cumsum([len(x) for x in rows])
    ci = np.concatenate(rows).astype(np.int32)
    p = sa.plan_from_csr(ent["dq"], rp, ci, w.block_q, w.block_kv)
    a0 = torch.zeros((w.H, w.D), dtype=torch.float32, device="cuda")
    o = sa.fwd(ent["dq"], ent["dk"], dv, p, alpha=a0)
    check = [(0, 0, 0), (0, 0, 1), (0, 0, 2), (0, 0, 3), (0, 0, nq - 1)]
    ol = linear_branch(ent["q32"], ent["k32"], W.to_f32(vb), rp, ci, w.block_q, w.block_kv, rows=check)
    got = np.concatenate([to_f64(o[0, 0, I * 128:min(w.N, (I + 1) * 128)]) for (_, _, I) in check])
    want = np.concatenate([ol[r] for r in check])
    mx, rr = check_out(got, want, "bf16", w.name + " Ol")
    log(f"{w.name}: Ol on rows with 2,048 / 2,049 / 3,000 / 1 kept blocks max|d| {mx:.2e} rel-RMS {rr:.2e}")
