"""Ground-truth tile heatmap of full attention, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The Veda page (section 2.1) builds its reference mask by max pooling the full attention
matrix over each query-tile x key-tile region; max rather than mean, so that sharp peaks
are not washed out by the background (section 2.3 produces this heatmap in two passes).
With A = softmax(q k^T / sqrt(D)) over all N keys, per head, and for query block I and
KV block J:

    tile_max[I, J]  = max over i in I, j in J of A[i, j]
    tile_mass[I, J] = (1 / |I|) * sum over i in I, j in J of A[i, j]

tile_mass is the average over the block's queries of the attention mass that falls on
tile J, so every row of it sums to 1. Ragged blocks use their real tokens only. Each
query block's A is formed at once from a matrix product (no tiling, no online softmax).
"""
from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np


def tile_heatmap(q: np.ndarray, k: np.ndarray, block_q: int, block_kv: int,
                 rows: Optional[Iterable[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """(tile_max, tile_mass), each [R, nKV] float64 with R = B*H*nQ rows in the order
    r = (b*H + h)*nQ + I. With ``rows``, only those rows are computed (the others stay
    NaN). q and k are [B, H, N, D] arrays of the stored input values."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, N, D = q.shape
    nQ = -(-N // block_q)
    nKV = -(-N // block_kv)
    R = B * H * nQ
    scale = 1.0 / np.sqrt(D)
    tmax = np.full((R, nKV), np.nan)
    tmass = np.full((R, nKV), np.nan)
    todo = range(R) if rows is None else rows
    pad = nKV * block_kv - N
    for r in todo:
        bh, I = divmod(int(r), nQ)
        b, h = divmod(bh, H)
        qi = q[b, h, I * block_q:min(N, (I + 1) * block_q)]
        s = (qi @ k[b, h].T) * scale
        s -= s.max(axis=1, keepdims=True)
        a = np.exp(s)
        a /= a.sum(axis=1, keepdims=True)
        # zero probabilities for the key positions past N leave both statistics unchanged
        a = np.pad(a, ((0, 0), (0, pad))).reshape(qi.shape[0], nKV, block_kv)
        tmax[r] = a.max(axis=(0, 2))
        tmass[r] = a.sum(axis=(0, 2)) / qi.shape[0]
    return tmax, tmass
