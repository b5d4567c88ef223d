"""Pins of the oracle's group-major token order (Veda page, section 2.2: head-aware 3-D
tiling) against enumeration by nested loops, identities and cube membership."""
import numpy as np
import pytest

from oracle import cube_order, permute_heads, unpermute_heads


def _enumerate(grid, cube):
    """Nested loops: cubes in raster order of the cube grid, tokens in raster order inside."""
    T, Hg, W = grid
    ct, ch, cw = cube
    out = []
    for bt in range(0, T, ct):
        for by in range(0, Hg, ch):
            for bx in range(0, W, cw):
                for t in range(bt, min(T, bt + ct)):
                    for y in range(by, min(Hg, by + ch)):
                        for x in range(bx, min(W, bx + cw)):
                            out.append((t * Hg + y) * W + x)
    return np.array(out)


@pytest.mark.parametrize("grid,cube", [((3, 5, 7), (2, 2, 4)), ((4, 4, 8), (2, 2, 2)),
                                       ((5, 9, 16), (1, 4, 16)), ((2, 3, 5), (3, 4, 6))])
def test_matches_enumeration(grid, cube):
    perm = cube_order(grid, cube)
    assert np.array_equal(perm, _enumerate(grid, cube))
    assert np.array_equal(np.sort(perm), np.arange(np.prod(grid)))


def test_identities():
    grid = (3, 6, 10)
    N = 180
    assert np.array_equal(cube_order(grid, (1, 1, 10)), np.arange(N))   # one raster row per cube
    assert np.array_equal(cube_order(grid, (3, 6, 10)), np.arange(N))   # one cube for all
    assert np.array_equal(cube_order(grid, (1, 1, 1)), np.arange(N))


def test_blocks_are_cubes_on_a_divisible_grid():
    grid, cube = (4, 8, 16), (2, 4, 8)
    perm = cube_order(grid, cube)
    for blk in range(perm.size // 64):
        toks = perm[blk * 64:(blk + 1) * 64]
        t, rem = np.divmod(toks, 8 * 16)
        y, x = np.divmod(rem, 16)
        assert np.ptp(t) == 1 and np.ptp(y) == 3 and np.ptp(x) == 7
        assert t.min() % 2 == 0 and y.min() % 4 == 0 and x.min() % 8 == 0


def test_permute_round_trip_per_head():
    rng = np.random.default_rng(0)
    grid = (3, 5, 6)
    x = rng.normal(size=(2, 3, 90, 4))
    cubes = [(1, 2, 3), (3, 5, 2), (2, 2, 2)]
    p = permute_heads(x, grid, cubes)
    assert not np.array_equal(p[:, 0], x[:, 0])
    assert np.array_equal(unpermute_heads(p, grid, cubes), x)
    assert np.array_equal(p[1, 2, 0], x[1, 2, 0])          # the first token stays first
