"""CPU checks of the whole-workload checker (tests/oracle_pool.py): the oracle's own mask
and its output rounded to bf16 pass; a changed block index or a changed output value is
caught on the row where it sits."""
import numpy as np
import pytest

import workloads as W
from oracle import oracle_plan, sparse_attention, linear_branch, blend
from tests.oracle_pool import check_workload

W_SMALL = W.Workload("pool_small", 1, 2, 64, (2, 32, 40), "bf16", 128, 64, 0.05, 0.8, 4)
W_LIN = W_SMALL.replace(name="pool_lin", linear=True)


def _oracle(w):
    q, k, v, alpha = W.make_inputs(w)
    q32, k32, v32 = W.to_f32(q), W.to_f32(k), W.to_f32(v)
    rp, ci, _ = oracle_plan(q32, k32, w.block_q, w.block_kv, w.topk, w.top_p)
    o = sparse_attention(q32, k32, v32, rp, ci, w.block_q, w.block_kv)
    if w.linear:
        o = blend(o, linear_branch(q32, k32, v32, rp, ci, w.block_q, w.block_kv), alpha)
    return rp, ci, W.f64_to_bf16_bits(o)


@pytest.mark.parametrize("w", [W_SMALL, W_LIN], ids=["sparse", "linear"])
def test_pool_accepts_the_oracle(w):
    rp, ci, ob = _oracle(w)
    tot = check_workload(w, rp, ci, ob, parts_per_head=3, log=lambda m: None)
    assert tot["nnz"] == rp[-1]
    assert tot["nonfinite"] == 0
    # bf16 rounding of the output only: half a unit in the last place, relative
    assert tot["rel_rms"] < 2.0 ** -8
    assert tot["max_err"] > 0


def test_pool_catches_a_changed_block():
    w = W_SMALL
    rp, ci, ob = _oracle(w)
    r = w.n_qblk + 5                      # head 1, query block 5
    ci2 = ci.copy()
    a, z = rp[r], rp[r + 1]
    missing = sorted(set(range(w.n_kvblk)) - set(ci[a:z].tolist()))
    ci2[z - 1] = missing[-1]
    ci2[a:z] = np.sort(ci2[a:z])
    with pytest.raises(AssertionError, match=r"h=1, I=5"):
        check_workload(w, rp, ci2, None, parts_per_head=2, log=lambda m: None)


def test_pool_catches_a_changed_output():
    w = W_SMALL
    rp, ci, ob = _oracle(w)
    ob2 = ob.copy()
    ob2[0, 1, 777, 3] = W.f64_to_bf16_bits(np.array([7.0]))[0]
    tot = check_workload(w, rp, ci, ob2, parts_per_head=2, log=lambda m: None)
    assert tot["max_err"] > 5.0
