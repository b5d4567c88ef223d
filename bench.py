"""Benchmark of the block-sparse attention hot path on one MI355X.

One step = sparse_attn_plan (pool, scores, hybrid top-k/top-p select, CSR) followed by
sparse_attn_fwd over the kept tiles, on seeded synthetic video-token Q, K, V already
resident in HBM. By default the step goes through sparse_attn_pipelined, which runs the
two over chunks of heads on two streams (--chunks; by default 4 chunks on steps of at
least 8192 query-block rows, and one chunk below that with the linear branch, whose
prepass then runs beside the plan); the plain plan-then-forward sequence is timed as well
(ms_step_sequential, ms_plan, ms_fwd). Prints one JSON line:

  value        effective TFLOP/s over the exact kept query-key pairs (4*D flops per
               pair) per step, plan included
  roofline     the forward kernel (the dominant one): kept-pair flops / its average
               duration from HIP events on the launch stream, against the bf16 MFMA peak
  cpu_baseline the float64 CPU oracle on a bounded sample of the same workload

plus the dense-mask run of the same kernel (speedup and per-kept-tile utilisation).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan14b_720p]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "sparse-attn ms/call + effective TFLOP/s (kept tiles) vs bf16 MFMA peak @90/95%"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 (vector and matrix)
HBM_PEAK_GBS = 8000.0
# head-aware 3-D tiling (--cubes): (t, h, w) extents, cycled over the heads
Q_CUBES = [(2, 4, 16), (1, 8, 16), (4, 4, 8)]
KV_CUBES = [(1, 4, 16), (2, 4, 8), (4, 4, 4)]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SRC = os.path.join(ROOT, "block_sparse_attention_05_amd", "csrc", "sparse_fwd_bf16.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kept_flops(rp: np.ndarray, ci: np.ndarray, w: W.Workload) -> float:
    """4*D flops per kept (query, key) pair, ragged blocks counted by real tokens."""
    nq = w.n_qblk
    qsize = np.minimum(w.block_q, w.N - np.arange(nq) * w.block_q).astype(np.int64)
    ksize = np.minimum(w.block_kv, w.N - np.arange(w.n_kvblk) * w.block_kv).astype(np.int64)
    counts = np.diff(rp)
    rows_q = np.tile(qsize, w.B * w.H)
    pairs = int(np.sum(np.repeat(rows_q, counts) * ksize[ci]))
    return 4.0 * w.D * pairs, pairs


def mask_quality(tmax: np.ndarray, tmass: np.ndarray, rp: np.ndarray, ci: np.ndarray) -> dict:
    """How well a block mask (CSR rp, ci) matches the ground-truth tile heatmap of full
    attention (tile max and mean mass per row, [R, nKV]). Per row with n kept tiles:
      recall_max   share of the n kept tiles among the n tiles with the largest max
      recall_mass  the same against the n tiles with the largest mass
      retained     attention mass on the kept tiles (of 1 per query)
      efficiency   retained / the largest mass any n tiles of the row hold
    Ties rank the lower block index first. Returns means and a few percentiles."""
    R, nkv = tmax.shape
    counts = np.diff(rp).astype(np.int64)
    kept = np.zeros((R, nkv), dtype=bool)
    kept[np.repeat(np.arange(R), counts), ci] = True
    idx = np.arange(nkv)[None, :]

    def top_n(score):
        order = np.argsort(-score, axis=1, kind="stable")
        rank = np.empty_like(order)
        np.put_along_axis(rank, order, np.broadcast_to(idx, order.shape), axis=1)
        return rank < counts[:, None]

    tmax_top = top_n(tmax)
    tmass_top = top_n(tmass)
    n = np.maximum(counts, 1)
    recall_max = (kept & tmax_top).sum(axis=1) / n
    recall_mass = (kept & tmass_top).sum(axis=1) / n
    retained = np.where(kept, tmass, 0.0).sum(axis=1)
    best = np.where(tmass_top, tmass, 0.0).sum(axis=1)
    eff = retained / np.maximum(best, 1e-30)

    def stats(x):
        return {"mean": round(float(x.mean()), 4), "p10": round(float(np.percentile(x, 10)), 4),
                "min": round(float(x.min()), 4)}

    return {"rows": int(R), "recall_max": stats(recall_max), "recall_mass": stats(recall_mass),
            "retained_mass": stats(retained), "mass_efficiency": stats(eff)}


def source_hash() -> str:
    """sha256 (first 16 hex digits) of the forward kernel's source followed by the compile
    flags the library build gives it: a change to either invalidates recorded counters."""
    from block_sparse_attention_05_amd import build as _build
    flags = _build.COMMON + _build.SOURCES[os.path.basename(KERNEL_SRC)]
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read() + b"\0" + " ".join(flags).encode()).hexdigest()[:16]


def traffic_for(workload: str, launch_bytes_alg: float):
    """HBM bytes per forward launch from committed rocprofv3 counters, when they were
    taken on the current kernel source and compile flags; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    ent = t.get(workload)
    if not ent or ent.get("kernel_source_sha256_16") != source_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w: W.Workload, q, k, v, rp, ci, budget_s: float = 15.0, mask_heads=None):
    """The oracle as it stands, on a bounded sample: the mask track (pooling, scores and
    the hybrid selection) of heads 0 .. mask_heads-1 (all heads by default), then the
    float64 output track over whole heads (0, 1, ...) until the budget is used. q, k, v
    hold the heads the CSR (rp, ci) describes, in order."""
    from oracle import oracle_plan, sparse_attention
    try:
        from threadpoolctl import threadpool_info
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    nq = w.n_qblk
    n_mask = q.shape[1] if mask_heads is None else min(mask_heads, q.shape[1])
    t0 = time.perf_counter()
    for h in range(n_mask):
        oracle_plan(W.to_f32(q[:, h:h + 1]), W.to_f32(k[:, h:h + 1]), w.block_q, w.block_kv, w.topk, w.top_p)
    t_mask = time.perf_counter() - t0
    ksize = np.minimum(w.block_kv, w.N - np.arange(w.n_kvblk) * w.block_kv)
    done_flops, n_rows, n_heads, t_out = 0.0, 0, 0, 0.0
    for h in range(q.shape[1]):
        q32, k32, v32 = (W.to_f32(x[:, h:h + 1]) for x in (q, k, v))
        base = int(rp[h * nq])
        rp_h = rp[h * nq:(h + 1) * nq + 1] - base
        ci_h = ci[base:int(rp[(h + 1) * nq])]
        t1 = time.perf_counter()
        sparse_attention(q32, k32, v32, rp_h, ci_h, w.block_q, w.block_kv)
        t_out += time.perf_counter() - t1
        for I in range(nq):
            qs = min(w.block_q, w.N - I * w.block_q)
            done_flops += 4.0 * w.D * qs * float(ksize[ci_h[rp_h[I]:rp_h[I + 1]]].sum())
        n_rows += nq
        n_heads += 1
        if t_out > budget_s:
            break
    return {
        "value": done_flops / t_out / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "ms_mask_track": round(1e3 * t_mask, 1),
        "mask_track_rows": int(n_mask * nq),
        "ms_output_track": round(1e3 * t_out, 1),
        "output_track_rows": int(n_rows),
        "output_track_gflops": round(done_flops / t_out / 1e9, 2),
        "sample": (f"{w.name}: the mask track of heads 0..{n_mask - 1} ({n_mask * nq} query blocks, "
                   f"{t_mask:.1f} s), then the float64 sparse output track of heads 0..{n_heads - 1} "
                   f"({n_rows} query blocks, {t_out:.1f} s); value = kept-pair flops of the output "
                   f"track per second"),
    }


PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (int8: 5.0 POP/s, the same rate)
# Below this many query-block rows a quarter of the forward no longer fills the chip and
# the pipelined step is slower than the plain sequence (480p: 0.75 against 0.59 ms).
PIPE_MIN_ROWS = 8192


def default_chunks(w) -> int:
    """Chunks of heads for the pipelined step: 4 from PIPE_MIN_ROWS rows up; below that one
    chunk with the linear branch (its prepass, which needs no mask, runs beside the plan on
    the second stream), else none (the plain plan-then-forward sequence)."""
    if w.B * w.H * w.n_qblk >= PIPE_MIN_ROWS:
        return 4
    return 1 if w.linear else 0


def time_fp8(sa, torch, w, dq, dk, dv, p, flops, t_fwd_bf16, args, stream):
    """Times the low-bit forward over the plan p for both q/k formats (E4M3, int8; v is
    E4M3 in both): the quantiser and the attention kernel, each with HIP events on the
    launch stream."""
    out = {"format": "v: OCP FP8 E4M3, power-of-two scale per channel; q, k: E4M3 with a "
                     "power-of-two scale per block (e4m3) or int8 with an fp32 scale per block (int8)"}
    o = torch.empty_like(dq)
    qkv_bytes = 3.0 * w.B * w.H * w.N * w.D * 2
    for qk in ("e4m3", "int8"):
        pack = sa.quantize_fp8(dq, dk, dv, w.block_q, qk=qk)
        for _ in range(max(1, args.warmup)):
            sa.quantize_fp8(dq, dk, dv, w.block_q, out=pack, qk=qk)
            sa.fwd_fp8(pack, p, out=o)
        n = max(3, args.steps)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            ev[i][0].record(stream)
            sa.quantize_fp8(dq, dk, dv, w.block_q, out=pack, qk=qk)
            ev[i][1].record(stream)
            sa.fwd_fp8(pack, p, out=o)
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        tq = [e[0].elapsed_time(e[1]) for e in ev]
        tf = [e[1].elapsed_time(e[2]) for e in ev]
        t = float(np.mean(tf))
        log(f"low-bit ({qk} q, k): quantise {np.mean(tq):.3f} ms, forward {t:.3f} ms "
            f"(bf16 forward {t_fwd_bf16:.3f} ms)")
        out[qk] = {
            "ms_quantize": round(float(np.mean(tq)), 4),
            "ms_fwd": round(t, 4),
            "ms_fwd_median": round(float(np.median(tf)), 4),
            "ms_fwd_min": round(float(np.min(tf)), 4),
            "fwd_tflops": round(flops / t / 1e9, 2),
            "fwd_frac_of_fp8_int8_peak": round(flops / t / 1e9 / PEAK_FP8_TFLOPS, 4),
            "speedup_fwd_vs_bf16": round(t_fwd_bf16 / t, 3),
            "quantize_gbs": round(qkv_bytes * 1.5 / (float(np.mean(tq)) * 1e-3) / 1e9, 1),
        }
        del pack
    return out


def time_backward(sa, torch, w, dq, dk, dv, p, pairs, args, stream):
    """Times sparse_attn_bwd over the plan p. Algorithmic work per kept (query, key) pair:
    the recomputed scores, dP = dO V^T, dV, dK and dQ, 2*D flops each (10*D); the kernels
    form S and dP once per direction (14*D actually issued)."""
    rng = np.random.default_rng([7, w.B, w.H, w.N, w.D])
    ddo = torch.from_numpy(W.f64_to_bf16_bits(rng.normal(size=(w.B, w.H, w.N, w.D))).view(np.int16)
                           ).view(torch.bfloat16).cuda()
    o, lse = sa.fwd(dq, dk, dv, p, return_lse=True)
    ws = torch.empty(sa.bwd_workspace_bytes(w.B, w.H, w.N, w.D, w.block_q, w.block_kv),
                     dtype=torch.uint8, device="cuda")
    grads = tuple(torch.empty_like(dq) for _ in range(3))
    for _ in range(max(1, args.warmup)):
        sa.bwd(dq, dk, dv, o, lse, ddo, p, workspace=ws, out=grads)
    n = max(3, args.steps)
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    e1 = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        e0[i].record(stream)
        sa.bwd(dq, dk, dv, o, lse, ddo, p, workspace=ws, out=grads)
        e1[i].record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in zip(e0, e1)]
    t = float(np.mean(ms))
    log(f"backward {t:.3f} ms (median {float(np.median(ms)):.3f})")
    return {
        "ms_bwd": round(t, 4),
        "ms_bwd_median": round(float(np.median(ms)), 4),
        "ms_bwd_min": round(float(np.min(ms)), 4),
        "bwd_tflops_alg": round(10.0 * w.D * pairs / t / 1e9, 2),
        "bwd_tflops_issued": round(14.0 * w.D * pairs / t / 1e9, 2),
        "flops_per_pair": "10*D algorithmic (S, dP, dV, dK, dQ); 14*D issued",
    }


def other_config(sa, torch, w: W.Workload, steps: int, warmup: int, dense: bool = True) -> dict:
    """One workload besides the headline one: the plan and the forward timed separately
    (HIP events on the launch stream, means over `steps` calls after `warmup`), the
    pipelined step where the headline would use it, the same forward on the all-ones plan,
    and the realised sparsity."""
    t0 = time.time()
    q, k, v, alpha = W.make_inputs(w)

    def dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    dq, dk, dv = dev(q), dev(k), dev(v)
    del q, k, v
    dalpha = dev(alpha) if w.linear else None
    stream = torch.cuda.current_stream()
    ws = torch.empty(sa.plan_workspace_bytes(w.B, w.H, w.N, w.D, w.block_q, w.block_kv),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty_like(dq)
    p = None
    for _ in range(max(1, warmup)):
        p = sa.plan(dq, dk, w.block_q, w.block_kv, w.topk, w.top_p, workspace=ws)
        sa.fwd(dq, dk, dv, p, alpha=dalpha, out=o)
    torch.cuda.synchronize()
    rp, ci = p.csr()
    flops, pairs = kept_flops(rp, ci, w)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record(stream)
        p = sa.plan(dq, dk, w.block_q, w.block_kv, w.topk, w.top_p, workspace=ws)
        e[1].record(stream)
        sa.fwd(dq, dk, dv, p, alpha=dalpha, out=o)
        e[2].record(stream)
    torch.cuda.synchronize()
    t_plan = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    t_fwd = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    t_step = t_plan + t_fwd
    res = {"B": w.B, "H": w.H, "N": w.N, "D": w.D, "dtype": w.dtype, "block_q": w.block_q,
           "block_kv": w.block_kv, "topk": w.topk, "top_p": w.top_p, "linear_branch": bool(w.linear),
           "ms_plan": round(t_plan, 4), "ms_fwd": round(t_fwd, 4), "ms_step_sequential": round(t_step, 4)}
    chunks = default_chunks(w)
    if chunks:
        pws = torch.empty(sa.pipelined_workspace_bytes(w.B, w.H, w.N, w.D, w.block_q, w.block_kv, chunks,
                                                       linear=bool(w.linear)), dtype=torch.uint8, device="cuda")
        for _ in range(max(1, warmup)):
            sa.attention(dq, dk, dv, w.block_q, w.block_kv, w.topk, w.top_p, chunks=chunks, out=o,
                         workspace=pws, alpha=dalpha)
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for a_, b_ in zip(e0, e1):
            a_.record(stream)
            sa.attention(dq, dk, dv, w.block_q, w.block_kv, w.topk, w.top_p, chunks=chunks, out=o,
                         workspace=pws, alpha=dalpha)
            b_.record(stream)
        torch.cuda.synchronize()
        t_step = float(np.mean([a_.elapsed_time(b_) for a_, b_ in zip(e0, e1)]))
        res["ms_step_pipelined"] = round(t_step, 4)
        res["pipeline_chunks"] = chunks
        del pws
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    nnz = int(rp[-1])
    res.update({
        "ms_step": round(t_step, 4),
        "step_tflops": round(flops / t_step / 1e9, 2),
        "fwd_tflops": round(flops / t_fwd / 1e9, 2),
        "fwd_frac_of_peak": round(flops / t_fwd / 1e9 / peak, 4),
        "peak_tflops": peak,
        "kept_pairs": pairs,
        "nnz_tiles": nnz,
        "tile_sparsity": round(1.0 - nnz / float(w.rows * w.n_kvblk), 5),
        "pair_sparsity": round(1.0 - pairs / float(w.B * w.H * w.N * w.N), 5),
    })
    if dense:
        pd = sa.plan_dense(dq, w.block_q, w.block_kv)
        sa.fwd(dq, dk, dv, pd, out=o)
        nd = 3
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(nd)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(nd)]
        for a_, b_ in zip(e0, e1):
            a_.record(stream)
            sa.fwd(dq, dk, dv, pd, out=o)
            b_.record(stream)
        torch.cuda.synchronize()
        t_dense = float(np.mean([a_.elapsed_time(b_) for a_, b_ in zip(e0, e1)]))
        dflops = 4.0 * w.D * w.B * w.H * float(w.N) * w.N
        res.update({
            "ms_dense_fwd": round(t_dense, 4),
            "dense_tflops": round(dflops / t_dense / 1e9, 2),
            "speedup_vs_dense": round(t_dense / t_step, 3),
            "speedup_vs_dense_fwd_only": round(t_dense / t_fwd, 3),
            "per_kept_tile_util_ratio": round((flops / t_fwd) / (dflops / t_dense), 4),
        })
        del pd
    log(f"{w.name}: plan {t_plan:.3f} ms, fwd {t_fwd:.3f} ms ({res['fwd_tflops']} TFLOP/s), step "
        f"{t_step:.3f} ms, tile sparsity {res['tile_sparsity']}" +
        (f", dense {res['ms_dense_fwd']:.2f} ms" if dense else "") + f" [{time.time() - t0:.0f} s]")
    del dq, dk, dv, o, ws, p, dalpha
    torch.cuda.empty_cache()
    return res


def sweep_exponents(points) -> dict:
    """Least-squares slopes of log(time) against log(N) over the length sweep."""
    n = np.log([x["N"] for x in points])
    out = {}
    for key in ("ms_step", "ms_fwd", "ms_dense_fwd"):
        if all(key in x for x in points):
            out["exponent_" + key[3:]] = round(float(np.polyfit(n, np.log([x[key] for x in points]), 1)[0]), 3)
    out["exponent_kept_pairs"] = round(float(np.polyfit(n, np.log([x["kept_pairs"] for x in points]), 1)[0]), 3)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14b_720p", choices=sorted(W.CONFIGS) + sorted(W.SWEEP))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--cubes", action="store_true",
                    help="head-aware 3-D tiling: queries and keys taken per head in a cube "
                         "order (per-head cubes cycled from a fixed list) through the plan's "
                         "tables; nothing is moved")
    ap.add_argument("--quality", action="store_true",
                    help="also build the ground-truth tile heatmap of full attention (two "
                         "passes) and report the router mask's recall and retained mass")
    ap.add_argument("--chunks", type=int, default=None,
                    help="heads per step are split into this many chunks, pipelined over two "
                         "streams (plans of later chunks under the forwards of earlier ones); "
                         "0 times the plain plan-then-forward sequence as the step; default: 4 "
                         "when the step has at least %d query-block rows, else 0" % PIPE_MIN_ROWS)
    ap.add_argument("--backward", action="store_true",
                    help="also time the backward (dq, dk, dv) over the step's plan, from the "
                         "forward's o and lse and a synthetic upstream gradient")
    ap.add_argument("--fp8", action="store_true",
                    help="also time the low-bit forward over the step's plan, q and k in E4M3 and in "
                         "int8: the quantiser and the attention kernel")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--no-configs", action="store_true",
                    help="time the headline workload only (by default the other workloads and "
                         "the long workload's length sweep are timed too, under 'configs')")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards over heads with no exchange between GPUs, so N GPUs each run "
              "this step on their share of the heads)", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_05_amd as sa

    w = W.CONFIGS[args.workload] if args.workload in W.CONFIGS else W.SWEEP[args.workload]
    t0 = time.time()
    q, k, v, alpha = W.make_inputs(w)
    log(f"inputs {w.name}: B={w.B} H={w.H} N={w.N} D={w.D} {w.dtype} in {time.time() - t0:.1f}s")

    def dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    dq, dk, dv = dev(q), dev(k), dev(v)
    dalpha = dev(alpha) if w.linear else None
    stream = torch.cuda.current_stream()
    raw = (dq, dk, dv)
    qc = kc = q_table = kv_table = None
    if args.cubes:
        # fixed per-head cubes (no search): t x h x w extents of 128 (query) and 64 (key).
        # q, k and v stay in raster order; the forward reads them, and writes o, through
        # the plan's query and key tables (built once, like the cube shapes).
        qc = [Q_CUBES[h % len(Q_CUBES)] for h in range(w.H)]
        kc = [KV_CUBES[h % len(KV_CUBES)] for h in range(w.H)]
        q_table = sa.cube_order(w.H, w.grid, qc)
        kv_table = sa.cube_order(w.H, w.grid, kc)

    def make_plan():
        if q_table is not None:
            return sa.plan_ordered(dq, dk, q_table, w.block_q, w.block_kv, w.topk, w.top_p, workspace=ws,
                                   kv_order=kv_table)
        return sa.plan(dq, dk, w.block_q, w.block_kv, w.topk, w.top_p, workspace=ws)
    ws = torch.empty(sa.plan_workspace_bytes(w.B, w.H, w.N, w.D, w.block_q, w.block_kv),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty_like(dq)

    def step():
        p = make_plan()
        sa.fwd(dq, dk, dv, p, alpha=dalpha, out=o)
        return p

    for _ in range(args.warmup):
        p = step()
    torch.cuda.synchronize()
    rp, ci = p.csr()
    flops, pairs = kept_flops(rp, ci, w)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    mids = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        p = make_plan()
        mids[i].record(stream)
        sa.fwd(dq, dk, dv, p, alpha=dalpha, out=o)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms_plan = [s.elapsed_time(m) for s, m in zip(starts, mids)]
    ms_fwd = [m.elapsed_time(e) for m, e in zip(mids, ends)]
    t_step = float(np.mean(ms_step))
    t_fwd = float(np.mean(ms_fwd))
    t_plan = float(np.mean(ms_plan))
    log(f"step {t_step:.3f} ms (plan {t_plan:.3f}, fwd {t_fwd:.3f}); wall {1e3 * wall / args.steps:.3f} ms/step")
    t_seq = t_step
    ms_seq = ms_step
    if args.chunks is None:
        args.chunks = default_chunks(w)
    pipelined = args.chunks > 0 and q_table is None
    if pipelined:
        # the step through the pipelined call: plan + forward over head chunks, two streams
        pws = torch.empty(sa.pipelined_workspace_bytes(w.B, w.H, w.N, w.D, w.block_q, w.block_kv, args.chunks,
                                                       linear=bool(w.linear)),
                          dtype=torch.uint8, device="cuda")

        def pstep():
            sa.attention(dq, dk, dv, w.block_q, w.block_kv, w.topk, w.top_p, chunks=args.chunks, out=o,
                         workspace=pws, alpha=dalpha)
        for _ in range(args.warmup):
            pstep()
        p0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        p1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        torch.cuda.synchronize()
        pw0 = time.perf_counter()
        for i in range(args.steps):
            p0[i].record(stream)
            pstep()
            p1[i].record(stream)
        torch.cuda.synchronize()
        pwall = time.perf_counter() - pw0
        ms_step = [a.elapsed_time(b) for a, b in zip(p0, p1)]
        t_step = float(np.mean(ms_step))
        log(f"pipelined step ({args.chunks} chunks) {t_step:.3f} ms; wall {1e3 * pwall / args.steps:.3f} ms/step")

    res_extra = {}
    if not args.no_dense:
        pd = sa.plan_dense(dq, w.block_q, w.block_kv)
        for _ in range(max(1, args.warmup)):
            sa.fwd(dq, dk, dv, pd, out=o)
        nd = max(3, min(args.steps, 10))
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(nd)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(nd)]
        for i in range(nd):
            e0[i].record(stream)
            sa.fwd(dq, dk, dv, pd, out=o)
            e1[i].record(stream)
        torch.cuda.synchronize()
        t_dense = float(np.mean([a.elapsed_time(b) for a, b in zip(e0, e1)]))
        dflops = 4.0 * w.D * w.B * w.H * float(w.N) * w.N
        res_extra = {
            "ms_dense_fwd": round(t_dense, 4),
            "dense_tflops": round(dflops / t_dense / 1e9, 2),
            "speedup_vs_dense": round(t_dense / t_step, 3),
            "speedup_vs_dense_fwd_only": round(t_dense / t_fwd, 3),
            "per_kept_tile_util_ratio": round((flops / t_fwd) / (dflops / t_dense), 4),
        }
        del pd

    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    achieved = flops / t_fwd / 1e9
    eb = w.elem_bytes
    alg_bytes = 4.0 * w.B * w.H * w.N * w.D * eb + 4.0 * (w.rows + 1 + len(ci))
    traffic = traffic_for(w.name, alg_bytes)
    nnz = int(rp[-1])
    out = {
        "metric": METRIC,
        "value": round(flops / t_step / 1e9, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": w.D, "grid": list(w.grid),
            "block_q": w.block_q, "block_kv": w.block_kv, "topk": w.topk, "top_p": w.top_p,
            "linear_branch": bool(w.linear),
            "pipeline": ({"chunks": args.chunks, "streams": 2, "call": "sparse_attn_pipelined"}
                         if pipelined else None),
            "cube_tiling": ({"query_cubes": Q_CUBES, "key_cubes": KV_CUBES, "per_head": "h mod 3",
                             "moved": "nothing (q, k, v and o through the plan's tables)"}
                            if args.cubes else None),
        },
        "ms_step_sequential": round(t_seq, 4),
        "ms_step_sequential_median": round(float(np.median(ms_seq)), 4),
        "ms_plan": round(t_plan, 4),
        "ms_fwd": round(t_fwd, 4),
        "ms_step_median": round(float(np.median(ms_step)), 4),
        "ms_step_min": round(float(np.min(ms_step)), 4),
        "ms_plan_median": round(float(np.median(ms_plan)), 4),
        "ms_fwd_median": round(float(np.median(ms_fwd)), 4),
        "ms_fwd_min": round(float(np.min(ms_fwd)), 4),
        "fwd_tflops": round(achieved, 2),
        "kept_pairs": pairs,
        "nnz_tiles": nnz,
        "tile_sparsity": round(1.0 - nnz / float(w.rows * w.n_kvblk), 5),
        "pair_sparsity": round(1.0 - pairs / float(w.B * w.H * w.N * w.N), 5),
        **res_extra,
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "kernel": "sparse_fwd_bf16_kernel" if w.dtype == "bf16" else "sparse_fwd_kernel",
        },
    }
    if args.backward:
        if w.dtype != "bf16" or q_table is not None:
            raise SystemExit("--backward needs a bf16 workload in raster order (no --cubes)")
        out["backward"] = time_backward(sa, torch, w, dq, dk, dv, p, pairs, args, stream)
    if args.fp8:
        if w.dtype != "bf16" or q_table is not None:
            raise SystemExit("--fp8 needs a bf16 workload in raster order (no --cubes)")
        out["fp8"] = time_fp8(sa, torch, w, dq, dk, dv, p, flops, t_fwd, args, stream)
    if args.copy_probe_mib > 0:
        # a plain copy of known size: HBM counters of this kernel calibrate the others
        nb = args.copy_probe_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_probe_bytes"] = nb
    if args.quality:
        if w.dtype != "bf16":
            raise SystemExit("--quality needs a bf16 workload")
        # the heatmap's query blocks must be the plan's rows: cube-ordered q under --cubes
        hq = sa.cube_permute(raw[0], w.grid, qc) if qc is not None else dq
        hk = sa.cube_permute(raw[1], w.grid, kc) if qc is not None else dk
        hv = sa.cube_permute(raw[2], w.grid, kc) if qc is not None else dv
        pd = sa.plan_dense(hq, w.block_q, w.block_kv)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        sa.fwd(hq, hk, hv, pd, return_lse=True, out=o, lse=lse)
        tmax, tmass = sa.tile_stats(hq, hk, lse, w.block_q, w.block_kv)
        e[0].record(stream)
        sa.fwd(hq, hk, hv, pd, return_lse=True, out=o, lse=lse)
        e[1].record(stream)
        tmax, tmass = sa.tile_stats(hq, hk, lse, w.block_q, w.block_kv)
        e[2].record(stream)
        torch.cuda.synchronize()
        t2 = e[1].elapsed_time(e[2])
        qual = mask_quality(tmax.cpu().numpy(), tmass.cpu().numpy(), rp, ci)
        qual["ms_pass1_dense_fwd_lse"] = round(e[0].elapsed_time(e[1]), 3)
        qual["ms_pass2_tile_stats"] = round(t2, 3)
        qual["pass2_tflops"] = round(2.0 * w.D * w.B * w.H * float(w.N) * w.N / t2 / 1e9, 1)
        out["quality"] = qual
        del pd, lse, tmax, tmass, hq, hk, hv
    if not args.no_configs:
        # every other workload (plan, forward, dense forward, sparsity), and the length
        # sweep of the long workload with its scaling exponents
        del raw, dq, dk, dv, o, ws
        torch.cuda.empty_cache()
        n_other = max(3, min(args.steps, 10))
        configs = {}
        for name in W.CONFIGS:
            if name != w.name:
                configs[name] = other_config(sa, torch, W.CONFIGS[name], n_other, args.warmup)
        sweep = []
        for sw in W.long_sweep():
            if sw.N == W.LONG_245K.N:
                ent = dict(configs.get(W.LONG_245K.name) or out)
            else:
                ent = other_config(sa, torch, sw, n_other, args.warmup)
            sweep.append({"T": sw.grid[0], "N": sw.N, "ms_step": ent["ms_step"] if "ms_step" in ent
                          else ent["ms_per_step"], "ms_fwd": ent["ms_fwd"], "ms_plan": ent["ms_plan"],
                          "ms_dense_fwd": ent.get("ms_dense_fwd"), "kept_pairs": ent["kept_pairs"],
                          "tile_sparsity": ent["tile_sparsity"],
                          "speedup_vs_dense": ent.get("speedup_vs_dense")})
        configs["long_sweep"] = {"points": sweep, **sweep_exponents(sweep)}
        out["configs"] = configs
    if not args.no_cpu_baseline:
        if qc is not None:
            # the oracle on the same cube-ordered head 0 as the plan's CSR describes
            from oracle import permute_heads
            out["cpu_baseline"] = cpu_baseline(w, permute_heads(q[:, :1], w.grid, qc[:1]),
                                               permute_heads(k[:, :1], w.grid, kc[:1]),
                                               permute_heads(v[:, :1], w.grid, kc[:1]), rp, ci)
        else:
            out["cpu_baseline"] = cpu_baseline(w, q, k, v, rp, ci)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
