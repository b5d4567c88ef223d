"""Output oracle in float64: block-sparse, dense and brute-force attention, and the
elu+1 linear branch blended with the sparse output.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* Block-sparse attention (SpargeAttention2 page, section 2(3)): for query i in query
  block I, softmax attention over the tokens of the KV blocks that the mask keeps for
  I; masked tiles take no part in the matrix products or the softmax. Logits are
  q_i . k_j / sqrt(D) (the pages fix no scale; this is the usual one). Non-causal.
* Linear branch (SALAD page, section 2.1: a linear-attention branch in parallel with
  the sparse one, O(N); SLA2 page: tokens the router drops feed the linear branch):
  Ol_i = sum_{j in C_I} (phi(q_i).phi(k_j)) v_j / sum_{j in C_I} phi(q_i).phi(k_j),
  over the tokens C_I of the KV blocks masked out for I, with phi = elu + 1 on the raw
  q and k. An empty C_I gives Ol_i = 0.
* Blend (SLA2 page, item 2): O = alpha * Os + (1 - alpha) * Ol, alpha per (head,
  channel).

Everything is computed in float64 from the stored input values. Each query block is
formed at once as a matrix product (no online softmax, no tiling beyond the block).
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Tuple

import numpy as np


def _f64(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def phi(x: np.ndarray) -> np.ndarray:
    """elu(x) + 1: x + 1 for x > 0, exp(x) otherwise (strictly positive)."""
    x = _f64(x)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def dense_plan(B: int, H: int, N: int, block_q: int, block_kv: int):
    """All-ones mask in CSR form (every query block keeps every KV block)."""
    nQ = -(-N // block_q)
    nKV = -(-N // block_kv)
    R = B * H * nQ
    row_ptr = np.arange(R + 1, dtype=np.int64) * nKV
    col_idx = np.tile(np.arange(nKV, dtype=np.int32), R)
    return row_ptr, col_idx


def _row_tokens(blocks: np.ndarray, block_kv: int, N: int) -> np.ndarray:
    if len(blocks) == 0:
        return np.zeros(0, dtype=np.int64)
    t = (np.asarray(blocks, np.int64)[:, None] * block_kv + np.arange(block_kv)[None, :]).ravel()
    return t[t < N]


def _softmax_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Exact softmax(q k^T * scale) v for one query block; returns (O, lse)."""
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1])), np.full(q.shape[0], -np.inf)
    s = (q @ k.T) * scale
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    den = p.sum(axis=1, keepdims=True)
    return (p @ v) / den, (m + np.log(den))[:, 0]


def sparse_attention(q, k, v, row_ptr, col_idx, block_q: int, block_kv: int,
                     rows: Optional[Iterable[Tuple[int, int, int]]] = None,
                     with_lse: bool = False):
    """Block-sparse attention of Q, K, V [B, H, N, D] under a CSR block mask.

    Without ``rows``, returns O [B, H, N, D] float64 (and LSE [B, H, N] with
    ``with_lse``). With ``rows`` (an iterable of (b, h, I)), returns a dict mapping each
    row to its (O block, lse block), for sampled checks of large workloads.
    """
    B, H, N, D = q.shape
    nQ = -(-N // block_q)
    scale = 1.0 / math.sqrt(D)
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col_idx = np.asarray(col_idx)

    def one(b, h, I):
        r = (b * H + h) * nQ + I
        blocks = col_idx[row_ptr[r]:row_ptr[r + 1]]
        tok = _row_tokens(blocks, block_kv, N)
        qs = slice(I * block_q, min(N, (I + 1) * block_q))
        return _softmax_rows(_f64(q[b, h, qs]), _f64(k[b, h, tok]), _f64(v[b, h, tok]), scale)

    if rows is not None:
        return {(b, h, I): one(b, h, I) for (b, h, I) in rows}
    out = np.zeros((B, H, N, D), dtype=np.float64)
    lse = np.zeros((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for I in range(nQ):
                qs = slice(I * block_q, min(N, (I + 1) * block_q))
                out[b, h, qs], lse[b, h, qs] = one(b, h, I)
    return (out, lse) if with_lse else out


def dense_attention(q, k, v, with_lse: bool = False):
    """Full softmax attention, float64, one head at a time."""
    B, H, N, D = q.shape
    scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, H, N, D), dtype=np.float64)
    lse = np.zeros((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h], lse[b, h] = _softmax_rows(_f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), scale)
    return (out, lse) if with_lse else out


def csr_to_mask(row_ptr, col_idx, B: int, H: int, N: int, block_q: int, block_kv: int):
    """Token-level boolean mask [B, H, N, N] from the CSR block mask (tiny N only)."""
    nQ = -(-N // block_q)
    mask = np.zeros((B, H, N, N), dtype=bool)
    for b in range(B):
        for h in range(H):
            for I in range(nQ):
                r = (b * H + h) * nQ + I
                for J in np.asarray(col_idx)[row_ptr[r]:row_ptr[r + 1]]:
                    mask[b, h, I * block_q:(I + 1) * block_q, J * block_kv:(J + 1) * block_kv] = True
    return mask


def brute_masked_attention(q, k, v, mask: np.ndarray):
    """Materialise every logit, set -inf where the token mask is False, softmax, x V."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    D = q.shape[-1]
    s = np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(D)
    s = np.where(mask, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.where(mask, np.exp(s - m), 0.0)
    den = p.sum(axis=-1, keepdims=True)
    o = np.einsum("bhij,bhjd->bhid", p, v)
    return np.where(den > 0, o / np.where(den > 0, den, 1.0), 0.0)


def linear_branch(q, k, v, row_ptr, col_idx, block_q: int, block_kv: int,
                  rows: Optional[Iterable[Tuple[int, int, int]]] = None):
    """Ol over the masked-out KV blocks of each query block, computed explicitly
    (every phi(q_i).phi(k_j) weight formed), float64."""
    B, H, N, D = q.shape
    nQ = -(-N // block_q)
    nKV = -(-N // block_kv)
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col_idx = np.asarray(col_idx)

    def one(b, h, I):
        r = (b * H + h) * nQ + I
        kept = set(int(j) for j in col_idx[row_ptr[r]:row_ptr[r + 1]])
        comp = np.array([J for J in range(nKV) if J not in kept], dtype=np.int64)
        qs = slice(I * block_q, min(N, (I + 1) * block_q))
        tok = _row_tokens(comp, block_kv, N)
        if tok.size == 0:
            return np.zeros((qs.stop - qs.start, D))
        w = phi(q[b, h, qs]) @ phi(k[b, h, tok]).T
        return (w @ _f64(v[b, h, tok])) / w.sum(axis=1, keepdims=True)

    if rows is not None:
        return {(b, h, I): one(b, h, I) for (b, h, I) in rows}
    out = np.zeros((B, H, N, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for I in range(nQ):
                out[b, h, I * block_q:min(N, (I + 1) * block_q)] = one(b, h, I)
    return out


def blend(o_sparse: np.ndarray, o_linear: np.ndarray, alpha: np.ndarray, h=None) -> np.ndarray:
    """O = alpha * Os + (1 - alpha) * Ol with alpha [H, D] broadcast over tokens.

    For full tensors [B, H, N, D] pass ``h=None``; for one head's block pass its index.
    """
    a = _f64(alpha)
    if h is None:
        a = a[None, :, None, :]
    else:
        a = a[h][None, :]
    return a * _f64(o_sparse) + (1.0 - a) * _f64(o_linear)
