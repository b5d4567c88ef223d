"""Group-major token order for head-aware 3-D tiling, and the oracle of attention under it.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The Veda page (section 2.2) tiles each head with its own factorisation (p_t, p_h, p_w) of
the hardware tile, so that a block of consecutive tokens is a compact spatio-temporal
cube rather than a strip of raster order. For tokens on a (T, Hg, W) grid with raster
index n = (t*Hg + y)*W + x, the cube order with cube (ct, ch, cw) sorts the tokens by

    (t // ct, y // ch, x // cw, t % ct, y % ch, x % cw)

so the cubes follow each other in raster order of the cube grid, and the tokens of one
cube follow each other in raster order inside it (cubes on the far borders of the grid
are partial). Blocks of block_q (block_kv) consecutive tokens of that order are then the
query (key) blocks. Attention itself does not depend on the order of the keys, and each
query's output does not depend on the order of the queries, so a call on permuted
tensors followed by the inverse permutation of the output is the same attention under a
different block partition.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np


def cube_order(grid: Sequence[int], cube: Sequence[int]) -> np.ndarray:
    """perm[i] = the raster index of the i-th token in cube order (a permutation of N)."""
    T, Hg, W = (int(g) for g in grid)
    ct, ch, cw = (int(c) for c in cube)
    t, y, x = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(W), indexing="ij")
    t, y, x = t.ravel(), y.ravel(), x.ravel()
    # np.lexsort sorts by the last key first
    return np.lexsort((x % cw, y % ch, t % ct, x // cw, y // ch, t // ct)).astype(np.int64)


def permute_heads(x: np.ndarray, grid: Sequence[int], cubes: Sequence[Sequence[int]]) -> np.ndarray:
    """x [B, H, N, ...] with head h's tokens put in the cube order of cubes[h]."""
    out = np.empty_like(x)
    for h in range(x.shape[1]):
        out[:, h] = x[:, h, cube_order(grid, cubes[h])]
    return out


def unpermute_heads(x: np.ndarray, grid: Sequence[int], cubes: Sequence[Sequence[int]]) -> np.ndarray:
    """The inverse of permute_heads."""
    out = np.empty_like(x)
    for h in range(x.shape[1]):
        out[:, h, cube_order(grid, cubes[h])] = x[:, h]
    return out
