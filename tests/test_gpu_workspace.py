"""Every workspace is written before it is read. Each call runs once on a workspace
filled with 0xFF bytes (NaN as fp32 and bf16, -1 as int32) and once on a zeroed one,
both longer than required; the results must be equal bit for bit. A kernel that read a
word its call had not written (a stale count, a partial sum, a pooled mean, a visit
entry past a row's kept count, a linear-branch sum of a row that keeps everything)
would see different values in the two runs."""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_attention_05_amd as sa
import workloads as W
from tests.gpu_common import inputs, log

pytestmark = pytest.mark.gpu

PAD = 1 << 16


def _ws(nbytes, fill):
    return torch.full((nbytes + PAD,), fill, dtype=torch.uint8, device="cuda")


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _plan_state(p):
    rp, ci = p.csr()
    return rp, ci, p.row_order().cpu().numpy(), int(p.nnz().item()), p.visit_lists()


CASES = [
    # name, B, H, N, D, dtype, block_q, topk, top_p (ragged N; both select widths)
    ("ws_q128", 1, 3, 64 * 37 + 21, 128, "bf16", 128, 0.05, 0.9),
    ("ws_q64_b2", 2, 2, 64 * 20 - 5, 64, "bf16", 64, 0.1, 0.8),
    ("ws_fp32", 1, 2, 700, 64, "fp32", 64, 0.25, 0.9),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_plan_and_fwd_ignore_workspace_contents(case):
    name, B, H, N, D, dt, bq, topk, p = case
    w = W.Workload(name, B, H, D, (1, 1, N), dt, bq, 64, topk, p, 4, linear=(dt == "bf16"), seed=12)
    ent = inputs(w)
    need = sa.plan_workspace_bytes(B, H, N, D, bq, 64)
    res = []
    for fill in (0xFF, 0x00):
        ws = _ws(need, fill)
        pl = sa.plan(ent["dq"], ent["dk"], bq, 64, topk, p, workspace=ws)
        torch.cuda.synchronize()
        st = _plan_state(pl)
        o = sa.fwd(ent["dq"], ent["dk"], ent["dv"], pl)
        extra = {}
        if w.linear:
            fneed = int(sa.load_library().sparse_attn_fwd_workspace_bytes(ctypes.byref(pl.st), 1))
            fws = _ws(fneed, fill)
            extra["lin"] = sa.fwd(ent["dq"], ent["dk"], ent["dv"], pl, alpha=ent["dalpha"], workspace=fws)
            pws = _ws(sa.pipelined_workspace_bytes(B, H, N, D, bq, 64, 2, linear=True), fill)
            extra["pipe"] = sa.attention(ent["dq"], ent["dk"], ent["dv"], bq, 64, topk, p, chunks=2,
                                         workspace=pws, alpha=ent["dalpha"])
        torch.cuda.synchronize()
        res.append((st, o, extra))
        del ws
    (a, oa, xa), (b, ob, xb) = res
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), "CSR"
    assert np.array_equal(a[2], b[2]), "row order"
    assert a[3] == b[3], "nnz"
    assert all(np.array_equal(x, y) for x, y in zip(a[4], b[4])), "visit lists"
    assert torch.equal(_bits(oa), _bits(ob)), "fwd"
    for key in xa:
        assert torch.equal(_bits(xa[key]), _bits(xb[key])), key
    log(f"{name}: plan, fwd{' and linear' if w.linear else ''} independent of workspace contents")


def test_bwd_ignores_workspace_contents():
    w = W.Workload("ws_bwd", 1, 2, 128, (1, 1, 64 * 23 + 9), "bf16", 128, 64, 0.1, 0.9, 4, seed=13)
    ent = inputs(w)
    pl = sa.plan(ent["dq"], ent["dk"], w.block_q, w.block_kv, w.topk, w.top_p)
    o, lse = sa.fwd(ent["dq"], ent["dk"], ent["dv"], pl, return_lse=True)
    dout = torch.randn_like(o)
    need = sa.bwd_workspace_bytes(w.B, w.H, w.N, w.D, w.block_q, w.block_kv)
    grads = []
    for fill in (0xFF, 0x00):
        ws = _ws(need, fill)
        grads.append(sa.bwd(ent["dq"], ent["dk"], ent["dv"], o, lse, dout, pl, workspace=ws))
        torch.cuda.synchronize()
    for g1, g2, nm in zip(grads[0], grads[1], ("dq", "dk", "dv")):
        assert torch.equal(_bits(g1), _bits(g2)), nm
    log("bwd independent of workspace contents")
