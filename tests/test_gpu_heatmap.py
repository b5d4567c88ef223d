"""GPU parity of the ground-truth tile heatmap (Veda page, section 2.1: max pooling of the
full attention matrix over query x key tiles; section 2.3: two passes) against the
float64 oracle.

Tolerances, derived from the arithmetic:
* Pass 2 alone (fed the oracle's log-sum-exp rounded to fp32): p = exp2(s*c*log2(e) -
  lse*log2(e)) with s accumulated in fp32 from exact bf16 products. The exponent's error
  is a few fp32 ulps of |s*c| (at most about 1e-3 for the sink-scaled keys here), so p
  is within a relative 2e-3 (plus 1e-6 absolute for tiny values).
* End to end (log-sum-exp from the bf16 forward on the all-ones plan): that forward sums
  the probabilities as rounded to bf16, each within 2^-8 relative (the bf16 unit
  roundoff). When it writes the log-sum-exp its running max is exact, so the largest
  term of every sum is exactly 1 and the others' roundings are independent; the sum's
  relative error stays well below 2^-8, and the bar takes a further relative 3e-3 for
  it: 5e-3 in all.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_05_amd as sa
import workloads as W
from oracle import dense_attention, tile_heatmap
from tests.gpu_common import inputs, log, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, H, N, D, block_q
    ("hm_d64_q64_ragged", 1, 2, 1000, 64, 64),
    ("hm_d128_q128_ragged", 2, 3, 3000, 128, 128),
    ("hm_d128_q64", 1, 2, 2048, 128, 64),
    ("hm_d64_q128_tiny", 1, 1, 100, 64, 128),
]


def _workload(name, B, H, N, D, bq):
    return W.Workload(name, B, H, D, (1, 1, N), "bf16", bq, 64, 0.05, 0.9, 4, seed=5)


def _close(got, ref, rtol, atol, what):
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    assert not bad.any(), (f"{what}: {int(bad.sum())} entries off, worst |d| {float(err.max()):.3e} "
                           f"at ref {float(ref.ravel()[np.argmax(err)]):.3e}")
    return float((err / np.maximum(np.abs(ref), atol)).max())


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pass2_with_oracle_lse(case):
    w = _workload(*case)
    ent = inputs(w)
    _, lse = dense_attention(ent["q32"], ent["k32"], W.to_f32(ent["v"]), with_lse=True)
    tmax, tmass = sa.tile_stats(ent["dq"], ent["dk"], to_dev(lse.astype(np.float32)), w.block_q, w.block_kv)
    rmax, rmass = tile_heatmap(ent["q32"], ent["k32"], w.block_q, w.block_kv)
    e1 = _close(tmax.cpu().numpy(), rmax, 2e-3, 1e-6, "tile_max")
    e2 = _close(tmass.cpu().numpy(), rmass, 2e-3, 1e-6, "tile_mass")
    log(f"{w.name}: worst relative error max {e1:.2e}, mass {e2:.2e}")


@pytest.mark.parametrize("case", CASES[:2], ids=[c[0] for c in CASES[:2]])
def test_two_passes_end_to_end(case):
    w = _workload(*case)
    ent = inputs(w)
    pd = sa.plan_dense(ent["dq"], w.block_q, w.block_kv)
    _, lse = sa.fwd(ent["dq"], ent["dk"], ent["dv"], pd, return_lse=True)
    tmax, tmass = sa.tile_stats(ent["dq"], ent["dk"], lse, w.block_q, w.block_kv)
    rmax, rmass = tile_heatmap(ent["q32"], ent["k32"], w.block_q, w.block_kv)
    _close(tmax.cpu().numpy(), rmax, 5e-3, 1e-6, "tile_max")
    _close(tmass.cpu().numpy(), rmass, 5e-3, 1e-6, "tile_mass")
    # determinism: a second call is bitwise identical
    tmax2, tmass2 = sa.tile_stats(ent["dq"], ent["dk"], lse, w.block_q, w.block_kv)
    assert torch.equal(tmax, tmax2) and torch.equal(tmass, tmass2)


def test_full_480p_sampled_rows():
    """The 480p workload end to end; the oracle on the first, last and 6 random query
    blocks of every head."""
    w = W.CONFIGS["wan13b_480p"]
    ent = inputs(w)
    pd = sa.plan_dense(ent["dq"], w.block_q, w.block_kv)
    _, lse = sa.fwd(ent["dq"], ent["dk"], ent["dv"], pd, return_lse=True)
    tmax, tmass = sa.tile_stats(ent["dq"], ent["dk"], lse, w.block_q, w.block_kv)
    tmax, tmass = tmax.cpu().numpy(), tmass.cpu().numpy()
    rng = np.random.default_rng(11)
    nq = w.n_qblk
    rows = sorted({h * nq + I for h in range(w.H)
                   for I in [0, nq - 1] + list(rng.choice(nq, 6, replace=False))})
    rmax, rmass = tile_heatmap(ent["q32"], ent["k32"], w.block_q, w.block_kv, rows=rows)
    _close(tmax[rows], rmax[rows], 5e-3, 1e-6, "tile_max")
    _close(tmass[rows], rmass[rows], 5e-3, 1e-6, "tile_mass")
    s = tmass.sum(axis=1)
    assert np.all(np.abs(s - 1.0) < 5e-3), f"row mass sums range {s.min():.5f}..{s.max():.5f}"
    log(f"480p: {len(rows)} sampled rows; row mass sums {s.min():.5f}..{s.max():.5f}")


def test_full_720p_row_mass():
    """At 720p every row of tile_mass sums to 1 (to the bf16 log-sum-exp's accuracy) and
    no tile max exceeds 1."""
    w = W.CONFIGS["wan14b_720p"]
    ent = inputs(w)
    pd = sa.plan_dense(ent["dq"], w.block_q, w.block_kv)
    _, lse = sa.fwd(ent["dq"], ent["dk"], ent["dv"], pd, return_lse=True)
    tmax, tmass = sa.tile_stats(ent["dq"], ent["dk"], lse, w.block_q, w.block_kv)
    s = tmass.sum(dim=1).cpu().numpy()
    assert np.all(np.abs(s - 1.0) < 5e-3), f"row mass sums range {s.min():.5f}..{s.max():.5f}"
    assert float(tmax.max()) <= 1.0 + 5e-3
    assert float(tmax.min()) >= 0.0
