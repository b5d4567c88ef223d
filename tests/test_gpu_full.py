"""GPU parity on whole workloads: every row's mask and every output element.

For the 720p, 245K and sparse+linear workloads and the sequence-length sweep of the long
one, the GPU's CSR is compared with the oracle's mask (the fp32 specification of the
hybrid top-k / top-p router, SpargeAttention2 page, section 2(1)) on every row, and the
GPU's output with the oracle's float64 block-sparse attention (section 2(3)), blended
with the explicit elu+1 linear branch for the sparse+linear workload (SLA2 page, item 2;
SALAD page, section 2.1), on every query. The oracle runs in a pool of worker processes
(tests/oracle_pool.py); the bounds are the usual ones: identical CSR, and for bf16
inputs max |dO| <= 2e-2 with relative RMS <= 5e-3 over the whole tensor.
"""
import time

import numpy as np
import pytest

import block_sparse_attention_05_amd as sa
import workloads as W
from tests.gpu_common import TOL_BF16_MAX, TOL_BF16_RRMS, drop, inputs, log
from tests.oracle_pool import check_workload

pytestmark = pytest.mark.gpu

# (workload, oracle tasks per head): enough tasks to keep 16 workers busy
FULL = [("wan14b_720p", 1), ("long_245k", 4), ("long_T30", 4), ("long_T15", 2),
        ("long_T8", 2), ("sparse_linear", 2)]


def _workload(name):
    return W.CONFIGS[name] if name in W.CONFIGS else W.SWEEP[name]


@pytest.mark.parametrize("name,parts", FULL, ids=[f[0] for f in FULL])
def test_workload_full(name, parts):
    w = _workload(name)
    ent = inputs(w)
    p = sa.plan(ent["dq"], ent["dk"], w.block_q, w.block_kv, w.topk, w.top_p)
    alpha = ent["dalpha"] if w.linear else None
    o = sa.fwd(ent["dq"], ent["dk"], ent["dv"], p, alpha=alpha)
    rp, ci = p.csr()
    o_host = o.view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    del o, p
    drop(w)
    log(f"{name}: gpu nnz {rp[-1]} of {w.rows * w.n_kvblk}; oracle on every row")
    t0 = time.time()
    tot = check_workload(w, rp, ci, o_host, parts_per_head=parts, log=log)
    log(f"{name}: mask identical on {w.rows} rows; output max|dO| {tot['max_err']:.3e} "
        f"rel-RMS {tot['rel_rms']:.3e} over {w.B * w.H * w.N} queries ({time.time() - t0:.0f} s)")
    assert tot["nonfinite"] == 0
    assert tot["max_err"] <= TOL_BF16_MAX, tot
    assert tot["rel_rms"] <= TOL_BF16_RRMS, tot
