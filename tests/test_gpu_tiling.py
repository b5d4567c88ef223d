"""GPU parity of head-aware 3-D tiling (Veda page, section 2.2): the cube permutation is
bit-exact against the oracle's order, and attention run on cube-ordered tensors matches
the oracle run on the same host-permuted tensors (masks bit-exact, outputs within the
bf16 tolerance), after the output is moved back to raster order."""
import numpy as np
import pytest
import torch

import block_sparse_attention_05_amd as sa
import workloads as W
from oracle import oracle_plan, permute_heads, sparse_attention, unpermute_heads
from tests.gpu_common import check_out, inputs, log, to_dev, to_f64

pytestmark = pytest.mark.gpu

Q_CUBES = [(2, 4, 16), (1, 8, 16), (4, 4, 8)]
KV_CUBES = [(1, 4, 16), (2, 4, 8), (4, 4, 4)]


def cubes_for(H, table):
    return [table[h % len(table)] for h in range(H)]


def _bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_permute_bitexact_ragged_grid(dtype):
    rng = np.random.default_rng(4)
    grid = (3, 7, 10)
    N, D = 210, 64 if dtype == "bf16" else 32
    x = rng.normal(size=(2, 3, N, D)).astype(np.float32)
    if dtype == "bf16":
        host = W.f64_to_bf16_bits(x)
        dev = to_dev(host)
    else:
        host = x
        dev = to_dev(x)
    cubes = [(2, 3, 4), (3, 7, 1), (1, 2, 10)]
    got = sa.cube_permute(dev, grid, cubes)
    ref = permute_heads(host, grid, cubes)
    assert np.array_equal(_bits(got), ref.view(np.int16 if dtype == "bf16" else np.int32))
    back = sa.cube_permute(got, grid, cubes, inverse=True)
    assert torch.equal(_bits_t(back), _bits_t(dev))


def _bits_t(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_permute_720p_heads():
    w = W.CONFIGS["wan14b_720p"]
    ent = inputs(w)
    cubes = cubes_for(w.H, Q_CUBES)
    got = sa.cube_permute(ent["dq"], w.grid, cubes)
    for h in (0, 1, 2, 39):
        ref = permute_heads(ent["q"][:, h:h + 1], w.grid, [cubes[h]])
        assert np.array_equal(got[:, h].contiguous().view(torch.int16).cpu().numpy(),
                              ref[:, 0].view(np.int16)), f"head {h}"
    back = sa.cube_permute(got, w.grid, cubes, inverse=True)
    assert torch.equal(back.view(torch.int16), ent["dq"].view(torch.int16))


def _tiled_run(w, ent):
    qc, kc = cubes_for(w.H, Q_CUBES), cubes_for(w.H, KV_CUBES)
    qp = sa.cube_permute(ent["dq"], w.grid, qc)
    kp = sa.cube_permute(ent["dk"], w.grid, kc)
    vp = sa.cube_permute(ent["dv"], w.grid, kc)
    p = sa.plan(qp, kp, w.block_q, w.block_kv, w.topk, w.top_p)
    op = sa.fwd(qp, kp, vp, p)
    o = sa.cube_permute(op, w.grid, qc, inverse=True)
    return qc, kc, p.csr(), o


SMALL = [
    # name, H, D, grid, block_q, topk, top_p
    ("cube_d64", 3, 64, (4, 16, 32), 128, 0.1, 0.9),
    ("cube_d128_ragged", 2, 128, (5, 12, 20), 128, 0.1, 0.85),
    ("cube_d128_q64", 3, 128, (4, 8, 32), 64, 0.05, 0.9),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_plan_and_fwd_under_cube_tiling(case):
    name, H, D, grid, bq, topk, p = case
    w = W.Workload(name, 1, H, D, grid, "bf16", bq, 64, topk, p, 4, seed=2)
    ent = inputs(w)
    qc, kc, (rp, ci), o = _tiled_run(w, ent)
    q32p = permute_heads(ent["q32"], w.grid, qc)
    k32p = permute_heads(ent["k32"], w.grid, kc)
    v32p = permute_heads(W.to_f32(ent["v"]), w.grid, kc)
    rrp, rci, _ = oracle_plan(q32p, k32p, bq, 64, topk, p)
    assert np.array_equal(rp, rrp) and np.array_equal(ci, rci), "mask under cube tiling"
    ref = unpermute_heads(sparse_attention(q32p, k32p, v32p, rrp, rci, bq, 64), w.grid, qc)
    mx, rr = check_out(to_f64(o), ref, "bf16", name)
    log(f"{name}: nnz {rp[-1]}, max |dO| {mx:.2e}, rel-RMS {rr:.2e}")


def test_480p_plan_under_cube_tiling():
    w = W.CONFIGS["wan13b_480p"]
    ent = inputs(w)
    qc, kc, (rp, ci), _ = _tiled_run(w, ent)
    rrp, rci, _ = oracle_plan(permute_heads(ent["q32"], w.grid, qc),
                              permute_heads(ent["k32"], w.grid, kc), w.block_q, w.block_kv, w.topk, w.top_p)
    assert np.array_equal(rp, rrp) and np.array_equal(ci, rci)
    log(f"480p cube tiling: nnz {rp[-1]} (tile sparsity {1 - rp[-1] / (w.rows * w.n_kvblk):.4f})")


# ------------------------------------------------------------------ query order table
def test_cube_order_table_bitexact():
    from oracle import cube_order as oracle_cube_order
    grid = (5, 12, 20)
    cubes = [(2, 4, 16), (1, 8, 16), (4, 4, 8)]
    got = sa.cube_order(3, grid, cubes).cpu().numpy()
    for h in range(3):
        assert np.array_equal(got[h], oracle_cube_order(grid, cubes[h]))


ORDERED = [
    # name, H, D, grid, block_q, topk, top_p, linear
    ("ord_d128", 3, 128, (4, 16, 32), 128, 0.1, 0.9, False),
    ("ord_d128_ragged_lin", 2, 128, (5, 12, 20), 128, 0.1, 0.85, True),
    ("ord_d64_q64", 3, 64, (4, 8, 32), 64, 0.05, 0.9, False),
]


@pytest.mark.parametrize("case", ORDERED, ids=[c[0] for c in ORDERED])
def test_ordered_plan_equals_moved_queries(case):
    """Gathering q and scattering o through the table is bitwise the same as moving q,
    running, and moving o back."""
    name, H, D, grid, bq, topk, p, lin = case
    w = W.Workload(name, 1, H, D, grid, "bf16", bq, 64, topk, p, 4, linear=lin, seed=3)
    ent = inputs(w)
    qc, kc = cubes_for(H, Q_CUBES), cubes_for(H, KV_CUBES)
    table = sa.cube_order(H, grid, qc)
    kp = sa.cube_permute(ent["dk"], grid, kc)
    vp = sa.cube_permute(ent["dv"], grid, kc)
    qp = sa.cube_permute(ent["dq"], grid, qc)
    alpha = ent["dalpha"] if lin else None
    p_ord = sa.plan_ordered(ent["dq"], kp, table, bq, 64, topk, p)
    p_mov = sa.plan(qp, kp, bq, 64, topk, p)
    rp1, ci1 = p_ord.csr()
    rp2, ci2 = p_mov.csr()
    assert np.array_equal(rp1, rp2) and np.array_equal(ci1, ci2)
    o1, l1 = sa.fwd(ent["dq"], kp, vp, p_ord, alpha=alpha, return_lse=True)
    o2, l2 = sa.fwd(qp, kp, vp, p_mov, alpha=alpha, return_lse=True)
    o2 = sa.cube_permute(o2, grid, qc, inverse=True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    l2 = unpermute_heads(l2.cpu().numpy()[..., None], grid, qc)[..., 0]
    assert np.array_equal(l1.cpu().numpy(), l2)
    log(f"{name}: ordered path bitwise equal to the moved path (nnz {rp1[-1]})")


@pytest.mark.parametrize("case", ORDERED, ids=[c[0] for c in ORDERED])
def test_ordered_keys_through_table_equal_moved_keys(case):
    """Keys and values read through the plan's key table (no moves at all) are bitwise the
    same as moving k and v into cube order first: the same plan, o and lse. A plan with a
    key table rejects the linear branch."""
    name, H, D, grid, bq, topk, p, lin = case
    w = W.Workload(name, 1, H, D, grid, "bf16", bq, 64, topk, p, 4, linear=lin, seed=3)
    ent = inputs(w)
    qc, kc = cubes_for(H, Q_CUBES), cubes_for(H, KV_CUBES)
    qt = sa.cube_order(H, grid, qc)
    kt = sa.cube_order(H, grid, kc)
    kp = sa.cube_permute(ent["dk"], grid, kc)
    vp = sa.cube_permute(ent["dv"], grid, kc)
    p_tab = sa.plan_ordered(ent["dq"], ent["dk"], qt, bq, 64, topk, p, kv_order=kt)
    p_mov = sa.plan_ordered(ent["dq"], kp, qt, bq, 64, topk, p)
    rp1, ci1 = p_tab.csr()
    rp2, ci2 = p_mov.csr()
    assert np.array_equal(rp1, rp2) and np.array_equal(ci1, ci2)
    o1, l1 = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p_tab, return_lse=True)
    o2, l2 = sa.fwd(ent["dq"], kp, vp, p_mov, return_lse=True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    if lin:
        with pytest.raises(sa.SparseAttnError):
            sa.fwd(ent["dq"], ent["dk"], ent["dv"], p_tab, alpha=ent["dalpha"])
    log(f"{name}: keys through the table bitwise equal to moved keys (nnz {rp1[-1]})")


def test_720p_tables_under_cube_tiling():
    """The 720p shape as the benchmark runs it with cube tiling: queries and keys through
    the plan's tables, nothing moved. On sampled heads the mask is bit-exact against the
    oracle on host-permuted tensors, and sampled query blocks of o (taken to cube order)
    are within the bf16 tolerance."""
    from tests.gpu_common import sample_rows
    w = W.CONFIGS["wan14b_720p"]
    ent = inputs(w)
    qc, kc = cubes_for(w.H, Q_CUBES), cubes_for(w.H, KV_CUBES)
    qt = sa.cube_order(w.H, w.grid, qc)
    kt = sa.cube_order(w.H, w.grid, kc)
    p = sa.plan_ordered(ent["dq"], ent["dk"], qt, w.block_q, w.block_kv, w.topk, w.top_p, kv_order=kt)
    rp, ci = p.csr()
    o = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p)
    op = to_f64(sa.cube_permute(o, w.grid, qc))
    hs = [0, 1, 2, w.H - 1]                       # every query and key cube shape, and the last head
    q32p = permute_heads(ent["q32"][:, hs], w.grid, [qc[h] for h in hs])
    k32p = permute_heads(ent["k32"][:, hs], w.grid, [kc[h] for h in hs])
    v32p = permute_heads(W.to_f32(ent["v"][:, hs]), w.grid, [kc[h] for h in hs])
    rrp, rci, _ = oracle_plan(q32p, k32p, w.block_q, w.block_kv, w.topk, w.top_p)
    nq = w.n_qblk
    for i, h in enumerate(hs):
        for I in range(nq):
            r, rr_ = h * nq + I, i * nq + I
            assert np.array_equal(ci[rp[r]:rp[r + 1]], rci[rrp[rr_]:rrp[rr_ + 1]]), f"head {h} row {I}"
    rows = sample_rows(w, 3, heads=[(0, i) for i in range(len(hs))])
    ref = sparse_attention(q32p, k32p, v32p, rrp, rci, w.block_q, w.block_kv, rows=rows)
    g, r = [], []
    for (b, i, I), (ob, _) in ref.items():
        g.append(op[b, hs[i], I * w.block_q:min(w.N, (I + 1) * w.block_q)])
        r.append(ob)
    mx, rr = check_out(np.concatenate(g), np.concatenate(r), "bf16", "720p cubes")
    log(f"720p cube tiling through tables: masks of heads {hs} bit-exact (nnz {rp[-1]}), "
        f"{len(rows)} sampled query blocks max |dO| {mx:.2e}, rel-RMS {rr:.2e}")
