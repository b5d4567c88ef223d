"""Shared helpers for the GPU parity tests: tensor transfer, tolerances, cached inputs."""
import sys
import time

import numpy as np

import workloads as W

# Output tolerances: fp32 inputs max |dO| <= 1e-4; bf16 inputs max |dO| <= 2e-2 and
# ||dO||_2 / ||O||_2 <= 5e-3 over the compared outputs. Masks: identical CSR.
TOL_FP32_MAX = 1e-4
TOL_BF16_MAX = 2e-2
TOL_BF16_RRMS = 5e-3


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray):
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def check_out(got: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    if dtype == "fp32":
        assert mx <= TOL_FP32_MAX, f"{what}: max |dO| {mx:.3e} > {TOL_FP32_MAX}"
        return mx, None
    rr = float(np.sqrt(np.sum(err ** 2)) / max(np.sqrt(np.sum(ref ** 2)), 1e-300))
    assert mx <= TOL_BF16_MAX, f"{what}: max |dO| {mx:.3e} > {TOL_BF16_MAX}"
    assert rr <= TOL_BF16_RRMS, f"{what}: rel-RMS {rr:.3e} > {TOL_BF16_RRMS}"
    return mx, rr


_CACHE = {}


def inputs(w: W.Workload):
    """(host q, k, v as stored, fp32-widened q, k, alpha, device q, k, v, alpha)."""
    if w in _CACHE:
        return _CACHE[w]
    t0 = time.time()
    q, k, v, alpha = W.make_inputs(w)
    log(f"generated {w.name} N={w.N} H={w.H} in {time.time() - t0:.1f}s")
    ent = dict(q=q, k=k, v=v, alpha=alpha, q32=W.to_f32(q), k32=W.to_f32(k),
               dq=to_dev(q), dk=to_dev(k), dv=to_dev(v), dalpha=to_dev(alpha))
    _CACHE[w] = ent
    return ent


def drop(w: W.Workload):
    _CACHE.pop(w, None)


def sample_rows(w: W.Workload, per_head: int, seed: int = 1234, heads=None):
    """Seeded sample of (b, h, I): the first and last (ragged) query block of each head
    plus random ones."""
    rng = np.random.default_rng(seed)
    rows = []
    hs = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    for b, h in hs:
        Is = {0, w.n_qblk - 1}
        while len(Is) < min(per_head, w.n_qblk):
            Is.add(int(rng.integers(0, w.n_qblk)))
        rows += [(b, h, I) for I in sorted(Is)]
    return rows
