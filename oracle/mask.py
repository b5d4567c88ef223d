"""Block-mask oracle: an fp32 specification of the hybrid top-k / top-p block router.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The method (SpargeAttention2 page, section 2(1)): for every attention row keep the
union of the top-k% entries and of the smallest set whose cumulative probability
reaches p. The router that produces the row (SLA2 page, router item 1) mean-pools Q and
K per block and scores pooled blocks per head; the learnable projection on that page
has no weights here and is the identity. Rows are query blocks and entries are KV
blocks, because the attention kernel that consumes the mask skips whole tiles
(SpargeAttention2 page, section 2(3)).

Every step below is a separately rounded IEEE-754 binary32 operation (round to nearest
even, no fused multiply-add) in one fixed order, so the result is a single, exactly
defined mask:

  R2 pool   acc = 0; acc = acc + x_t over the block's tokens in ascending order;
            mean = acc / count (IEEE division). The ragged last block averages its
            real tokens only.
  R3 score  acc = 0; acc = acc + (qbar[d] * kbar[d]) for d ascending (product rounded
            first); S = acc * c with c = fp32(1/sqrt(D)) rounded once from float64.
  R4 order  pi = KV blocks sorted by S descending, ties by the lower block index
            (-0 and +0 compare equal).
  R5 exp    e_J = exp_sa(S_J - S_max), exp_sa defined below.
  R6 Z      pairwise tree sum of e_J in block-index order, zero-padded to a power of
            two, adjacent pairs at each level.
  R7 top-p  thr = fp32(p) * Z; C_r = C_{r-1} + e_{pi(r)} sequentially;
            m_p = min{r >= 1 : C_r >= thr}, or nKV when no prefix reaches thr or p >= 1.
  R8 union  m_k = min(nKV, max(1, ceil(k * nKV - 1e-9))) in float64. Both rules are
            prefixes of pi, so the union is the first max(m_k, m_p) blocks of pi;
            they are emitted in ascending block order.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

F32 = np.float32

# exp_sa constants. Cody-Waite reduction (Cody & Waite, "Software Manual for the
# Elementary Functions", 1980): ln 2 split into C1, which has 16 significant bits so
# n * C1 is exact for |n| < 2^8, and the fp32 remainder C2.
LOG2E_F32 = F32(math.log2(math.e))
LN2_HI = F32(45426.0 / 65536.0)                 # 0.693145751953125, exact in fp32
LN2_LO = F32(math.log(2.0) - 45426.0 / 65536.0)
EXP_COEF = [F32(1.0 / math.factorial(i)) for i in range(8)]  # Taylor terms 1/i!
EXP_UNDERFLOW = F32(-86.0)


def exp_sa(x: np.ndarray) -> np.ndarray:
    """Deterministic fp32 exp for x <= 0, built only from rounded fp32 + - * and rint.

    x < -86 returns 0, so every nonzero result is a normal fp32 number. Otherwise
    n = rint(x * log2(e)) (half to even), r = (x - n*C1) - n*C2, p = Horner evaluation
    of sum_{i<8} r^i / i!, and the result is p * 2^n (exact scaling).
    """
    x = np.asarray(x, dtype=F32)
    under = ~(x >= EXP_UNDERFLOW)
    x = np.where(under, F32(0.0), x).astype(F32)
    n = np.rint(x * LOG2E_F32).astype(F32)
    r = (x - n * LN2_HI) - n * LN2_LO
    p = np.full_like(x, EXP_COEF[7])
    for i in range(6, -1, -1):
        p = p * r + EXP_COEF[i]
    out = np.ldexp(p, n.astype(np.int32)).astype(F32)
    return np.where(under, F32(0.0), out).astype(F32)


def score_scale(D: int) -> np.float32:
    """c = 1/sqrt(D), computed in float64 and rounded once to fp32."""
    return F32(1.0 / math.sqrt(D))


def topk_count(topk: float, n_kv: int) -> int:
    """m_k: ceil(k * nKV) blocks, at least one, at most nKV (float64 arithmetic)."""
    return int(min(n_kv, max(1, math.ceil(topk * n_kv - 1e-9))))


def pool_blocks(x: np.ndarray, block: int) -> np.ndarray:
    """Per-block mean over tokens, [N, D] fp32 -> [ceil(N/block), D] fp32 (R2)."""
    x = np.asarray(x, dtype=F32)
    N, D = x.shape
    nfull, tail = divmod(N, block)
    nblk = nfull + (1 if tail else 0)
    acc = np.zeros((nblk, D), dtype=F32)
    if nfull:
        xr = x[: nfull * block].reshape(nfull, block, D)
        for t in range(block):
            acc[:nfull] = acc[:nfull] + xr[:, t, :]
        acc[:nfull] = acc[:nfull] / F32(block)
    if tail:
        last = np.zeros(D, dtype=F32)
        for t in range(nfull * block, N):
            last = last + x[t]
        acc[nfull] = last / F32(tail)
    return acc


def block_scores(qbar: np.ndarray, kbar: np.ndarray, c: np.float32) -> np.ndarray:
    """S[I, J] = (sum_d qbar[I,d] * kbar[J,d]) * c in the R3 order, fp32."""
    qbar = np.asarray(qbar, dtype=F32)
    kbar = np.asarray(kbar, dtype=F32)
    S = np.zeros((qbar.shape[0], kbar.shape[0]), dtype=F32)
    for d in range(qbar.shape[1]):
        S = S + np.multiply.outer(qbar[:, d], kbar[:, d])
    return (S * F32(c)).astype(F32)


def tree_sum(e: np.ndarray) -> np.float32:
    """R6: pairwise sum, zero-padded to a power of two, adjacent pairs per level."""
    n = e.shape[0]
    size = 1
    while size < n:
        size *= 2
    a = np.zeros(size, dtype=F32)
    a[:n] = e
    while a.shape[0] > 1:
        a = a[0::2] + a[1::2]
    return F32(a[0])


def select_row(S_row: np.ndarray, m_k: int, top_p: float) -> Tuple[np.ndarray, int, int]:
    """One row of R4-R8. Returns (kept blocks ascending, m_p, kept count)."""
    S_row = np.asarray(S_row, dtype=F32)
    n = S_row.shape[0]
    order = np.argsort(-S_row, kind="stable")
    smax = S_row[order[0]]
    e = exp_sa((S_row - smax).astype(F32))
    Z = tree_sum(e)
    if top_p >= 1.0:
        m_p = n
    else:
        thr = F32(F32(top_p) * Z)
        C = np.cumsum(e[order], dtype=F32)
        hit = np.nonzero(C >= thr)[0]
        m_p = int(hit[0]) + 1 if hit.size else n
    keep = max(m_k, m_p)
    return np.sort(order[:keep]), m_p, keep


def _head_plan(q: np.ndarray, k: np.ndarray, block_q: int, block_kv: int, topk: float,
               top_p: float, q_blocks: Optional[Sequence[int]] = None):
    N, D = q.shape
    qbar = pool_blocks(q, block_q)
    kbar = pool_blocks(k, block_kv)
    if q_blocks is not None:
        qbar = qbar[np.asarray(q_blocks, dtype=np.int64)]
    S = block_scores(qbar, kbar, score_scale(D))
    m_k = topk_count(topk, kbar.shape[0])
    return [select_row(S[i], m_k, top_p) for i in range(S.shape[0])]


def oracle_plan(q: np.ndarray, k: np.ndarray, block_q: int, block_kv: int, topk: float,
                top_p: float, rows: Optional[Iterable[Tuple[int, int, int]]] = None):
    """The block mask of Q, K [B, H, N, D] (stored values, fp32-widened).

    Without ``rows``: returns (row_ptr int64 [R+1], col_idx int32 [nnz], m_p int32 [R])
    with row r = (b*H + h)*nQ + I. With ``rows`` (an iterable of (b, h, I)): returns a
    dict mapping each requested row to its kept block list, for sampled checks.
    """
    B, H, N, D = q.shape
    if rows is not None:
        want: Dict[Tuple[int, int], List[int]] = {}
        for b, h, I in rows:
            want.setdefault((b, h), []).append(I)
        out = {}
        for (b, h), Is in want.items():
            Is = sorted(set(Is))
            res = _head_plan(q[b, h], k[b, h], block_q, block_kv, topk, top_p, Is)
            for I, (kept, _, _) in zip(Is, res):
                out[(b, h, I)] = kept
        return out
    counts, cols, mps = [], [], []
    for b in range(B):
        for h in range(H):
            for kept, m_p, keep in _head_plan(q[b, h], k[b, h], block_q, block_kv, topk, top_p):
                counts.append(keep)
                cols.append(kept.astype(np.int32))
                mps.append(m_p)
    row_ptr = np.zeros(len(counts) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.concatenate(cols) if cols else np.zeros(0, np.int32)
    return row_ptr, col_idx.astype(np.int32), np.asarray(mps, dtype=np.int32)


def plan_stats(row_ptr: np.ndarray, col_idx: np.ndarray, B: int, H: int, N: int,
               block_q: int, block_kv: int) -> Dict[str, float]:
    """Tile sparsity and exact pair sparsity (ragged blocks counted by real tokens)."""
    nQ = -(-N // block_q)
    nKV = -(-N // block_kv)
    R = B * H * nQ
    counts = np.diff(row_ptr)
    qsize = np.minimum(block_q, N - np.arange(nQ) * block_q)
    ksize = np.minimum(block_kv, N - np.arange(nKV) * block_kv)
    rows_q = np.tile(qsize, B * H)
    kept_pairs = int(np.sum(np.repeat(rows_q, counts).astype(np.int64) *
                            ksize[col_idx].astype(np.int64)))
    nnz = int(row_ptr[-1])
    return {
        "nnz": nnz,
        "tile_sparsity": 1.0 - nnz / float(R * nKV),
        "kept_pairs": kept_pairs,
        "pair_sparsity": 1.0 - kept_pairs / float(B * H * N * N),
    }
