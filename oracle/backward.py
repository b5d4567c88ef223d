"""Gradients of block-sparse attention, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fine-tune through the sparse kernel (SpargeAttention2 page, section 2; SLA2
page), so the forward of oracle.attention has a backward. For query block I with kept
tokens K_I, scale c = 1/sqrt(D), S = c * q_I k_{K_I}^T, P = softmax(S) row by row and
O = P v_{K_I}. For an upstream gradient dO of O:

    dV[j]  += sum_i P[i, j] dO[i]                 (j in K_I)
    dP      = dO v_{K_I}^T
    Dv[i]   = sum_d dO[i, d] O[i, d]  (= sum_j P[i, j] dP[i, j])
    dS      = P * (dP - Dv[:, None])
    dQ[i]   = c * sum_j dS[i, j] k[j]
    dK[j]  += c * sum_i dS[i, j] q[i]             (j in K_I)

Masked tiles contribute nothing. Each query block is formed at once as matrix products
from the stored input values widened to float64.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np


def _row_tokens(blocks: np.ndarray, block_kv: int, N: int) -> np.ndarray:
    if len(blocks) == 0:
        return np.zeros(0, dtype=np.int64)
    t = (np.asarray(blocks, np.int64)[:, None] * block_kv + np.arange(block_kv)[None, :]).ravel()
    return t[t < N]


def sparse_attention_backward(q, k, v, do, row_ptr, col_idx, block_q: int, block_kv: int,
                              rows=None, o=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(dQ, dK, dV), each [B, H, N, D] float64, for O = block-sparse attention of q, k, v
    [B, H, N, D] under the CSR mask, and the upstream gradient do [B, H, N, D].

    With ``rows`` (row indices r = (b*H + h)*nQ + I), only those query blocks contribute:
    dQ is then complete on those blocks, and dK, dV on every KV block all of whose
    keeping rows are included.

    With ``o`` (the forward output as a caller stored it, for example rounded to bf16),
    Dv is formed from that o instead of the exact one, as a backward that reuses the
    forward's output does."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    o_given = None if o is None else np.asarray(o, dtype=np.float64)
    B, H, N, D = q.shape
    nQ = -(-N // block_q)
    c = 1.0 / math.sqrt(D)
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col_idx = np.asarray(col_idx)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    todo = range(B * H * nQ) if rows is None else sorted(set(int(r) for r in rows))
    for r in todo:
        bh, I = divmod(r, nQ)
        b, h = divmod(bh, H)
        tok = _row_tokens(col_idx[row_ptr[r]:row_ptr[r + 1]], block_kv, N)
        if tok.size == 0:
            continue
        qs = slice(I * block_q, min(N, (I + 1) * block_q))
        qi, gi = q[b, h, qs], do[b, h, qs]
        kj, vj = k[b, h, tok], v[b, h, tok]
        s = c * (qi @ kj.T)
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        oi = p @ vj if o_given is None else o_given[b, h, qs]
        dp = gi @ vj.T
        dvec = (gi * oi).sum(axis=1, keepdims=True)
        ds = p * (dp - dvec)
        dq[b, h, qs] = c * (ds @ kj)
        dk[b, h, tok] += c * (ds.T @ qi)
        dv[b, h, tok] += p.T @ gi
    return dq, dk, dv
