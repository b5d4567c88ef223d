"""Whole-workload oracle checks in worker processes.

The float64 output track of a large workload (hundreds of query blocks per head, tens of
heads) is too slow for one process: each query block is a pair of small matrix products,
which a multithreaded BLAS does not speed up. These helpers split a workload into
(head, query-block range) tasks and run the oracle on them in a pool of spawned
processes, one BLAS thread each. A worker regenerates its head's inputs from the seeded
recipe (the generator is deterministic), so only the GPU's results for that head travel
to it, and only error statistics travel back.

Each task checks, for its rows:
  * the mask: the oracle's kept blocks (the fp32 specification of the hybrid top-k /
    top-p router, SpargeAttention2 page, section 2(1)) against the GPU's CSR, bit for bit;
  * optionally the output: the oracle's float64 block-sparse attention (section 2(3)),
    and with a linear branch the explicit elu+1 linear attention over the masked-out
    blocks blended with alpha (SLA2 page, item 2; SALAD page, section 2.1), against the
    GPU's output.

Only numpy, the workload generator and the oracle are imported here: workers never touch
the GPU.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


def pool_size() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _task(args) -> Dict:
    (wl, b, h, lo, hi, rp_rows, ci_rows, o_bits, want_out) = args
    from threadpoolctl import threadpool_limits

    import workloads as W
    from oracle import blend, linear_branch, oracle_plan, sparse_attention

    with threadpool_limits(1):
        q, k, v, alpha = W.make_inputs(wl, heads=[(b, h)], workers=1)
        q32 = W.to_f32(q[b:b + 1, h:h + 1])
        k32 = W.to_f32(k[b:b + 1, h:h + 1])
        v32 = W.to_f32(v[b:b + 1, h:h + 1])
        del q, k, v
        rows = [(0, 0, I) for I in range(lo, hi)]
        kept = oracle_plan(q32, k32, wl.block_q, wl.block_kv, wl.topk, wl.top_p, rows=rows)
        res = {"b": b, "h": h, "lo": lo, "hi": hi, "mask_bad": None, "nnz": 0}
        for i, I in enumerate(range(lo, hi)):
            got = ci_rows[rp_rows[i]:rp_rows[i + 1]]
            ref = kept[(0, 0, I)]
            res["nnz"] += int(ref.size)
            if got.size != ref.size or not np.array_equal(got, ref):
                res["mask_bad"] = (I, got[:8].tolist(), ref[:8].tolist())
                return res
        if not want_out:
            return res
        # the oracle's plan for these rows is the GPU's (checked above); the CSR of the
        # whole head is needed only for the rows' own entries
        nQ = wl.n_qblk
        rp_full = np.zeros(nQ + 1, np.int64)
        rp_full[lo + 1:hi + 1] = rp_rows[1:]
        rp_full[hi + 1:] = rp_rows[-1]
        os_ = sparse_attention(q32, k32, v32, rp_full, ci_rows, wl.block_q, wl.block_kv, rows=rows)
        ol = None
        if wl.linear:
            ol = linear_branch(q32, k32, v32, rp_full, ci_rows, wl.block_q, wl.block_kv, rows=rows)
        n0 = lo * wl.block_q
        got = W.to_f32(o_bits) if o_bits.dtype == np.uint16 else o_bits
        mx, se, sr, nonfin = 0.0, 0.0, 0.0, 0
        for (_, _, I), (ob, _) in os_.items():
            ref = ob if ol is None else blend(ob, ol[(0, 0, I)], alpha, h=h)
            s0 = I * wl.block_q - n0
            g = got[s0:s0 + ref.shape[0]].astype(np.float64)
            nonfin += int(np.count_nonzero(~np.isfinite(g)))
            d = np.abs(g - ref)
            mx = max(mx, float(d.max()))
            se += float(np.sum(d * d))
            sr += float(np.sum(ref * ref))
        res.update(max_err=mx, sq_err=se, sq_ref=sr, nonfinite=nonfin)
        return res


def check_workload(wl, row_ptr: np.ndarray, col_idx: np.ndarray, o: Optional[np.ndarray],
                   parts_per_head: int = 1, log=print) -> Dict:
    """Checks the GPU's whole CSR (and output ``o`` [B, H, N, D] as stored: uint16 bf16
    bits or float32, or None) of workload ``wl`` against the oracle, row by row.

    Returns totals: nnz, max_err, rel_rms, nonfinite; raises AssertionError on the first
    row whose mask differs."""
    nQ = wl.n_qblk
    tasks = []
    bounds = np.linspace(0, nQ, parts_per_head + 1).astype(int)
    for b in range(wl.B):
        for h in range(wl.H):
            for lo, hi in zip(bounds[:-1], bounds[1:]):
                if hi <= lo:
                    continue
                r0 = (b * wl.H + h) * nQ
                a, z = int(row_ptr[r0 + lo]), int(row_ptr[r0 + hi])
                rp = (row_ptr[r0 + lo:r0 + hi + 1] - a).astype(np.int64)
                ci = np.ascontiguousarray(col_idx[a:z])
                ob = None
                if o is not None:
                    ob = np.ascontiguousarray(o[b, h, lo * wl.block_q:min(wl.N, hi * wl.block_q)])
                tasks.append((wl, b, h, int(lo), int(hi), rp, ci, ob, o is not None))
    # the heaviest tasks first, so the pool's tail is short
    tasks.sort(key=lambda t: -int(t[5][-1]))
    tot = {"nnz": 0, "max_err": 0.0, "sq_err": 0.0, "sq_ref": 0.0, "nonfinite": 0}
    ctx = mp.get_context("spawn")
    with ctx.Pool(min(pool_size(), len(tasks))) as pool:
        for i, r in enumerate(pool.imap_unordered(_task, tasks)):
            assert r["mask_bad"] is None, (
                f"{wl.name}: mask differs at (b={r['b']}, h={r['h']}, I={r['mask_bad'][0]}): "
                f"gpu {r['mask_bad'][1]} oracle {r['mask_bad'][2]}")
            tot["nnz"] += r["nnz"]
            if o is not None:
                tot["max_err"] = max(tot["max_err"], r["max_err"])
                tot["sq_err"] += r["sq_err"]
                tot["sq_ref"] += r["sq_ref"]
                tot["nonfinite"] += r["nonfinite"]
            if (i + 1) % max(1, len(tasks) // 8) == 0:
                log(f"{wl.name}: {i + 1}/{len(tasks)} oracle tasks done")
    assert tot["nnz"] == int(row_ptr[-1]), (tot["nnz"], int(row_ptr[-1]))
    if o is not None:
        tot["rel_rms"] = float(np.sqrt(tot["sq_err"] / max(tot["sq_ref"], 1e-300)))
    return tot
