"""Block-sparse softmax attention for video DiTs on MI355X (gfx950).

Thin Python face of libsparse_attn.so (C ABI in include/sparse_attn.h):

    plan(q, k, block_q, block_kv, topk, top_p)  the hybrid top-k / top-p block router
    fwd(q, k, v, plan, alpha=None)              attention over the kept tiles, with the
                                                optional elu+1 linear branch blend
    attention(q, k, v, ..., chunks=4)           plan + fwd in one call, pipelined over chunks
                                                of heads on two streams
    attention_noalloc(q, k, v, ..., out=o)      plan + fwd on one stream with the library's
                                                static scratch: allocates nothing
    plan_dense(q, ...), plan_from_csr(q, ...)   all-ones and caller-given masks
    bwd(q, k, v, o, lse, dout, plan)            gradients dq, dk, dv over the same mask
    quantize_fp8(q, k, v, block_q), fwd_fp8     the low-bit forward: FP8 E4M3 codes with
                                                power-of-two group scales, then attention
                                                on fp8 MFMA
    tile_stats(q, k, lse, ...)                  ground-truth tile heatmap (max and mean
                                                mass of full attention per tile)
    cube_permute(x, grid, cubes, inverse)       head-aware 3-D tiling: raster <-> per-head
                                                cube order of the tokens
    cube_order(H, grid, cubes)                  the same order as a table, and
    plan_ordered(q, k, q_order, ...)            a mask whose query blocks follow it
                                                (q and o stay in raster order)

All computation happens in the library's HIP kernels; torch supplies device memory and
streams.
"""
from ._binding import (EXPORTS, SA_BF16, SA_FP32, Fp8Pack, Plan, attention, attention_noalloc, pipelined_workspace_bytes, SaPlan, SparseAttnError, bwd,
                       bwd_workspace_bytes, cube_order, cube_permute, fp8_pack_bytes, fwd_fp8, quantize_fp8, fwd, load_library, plan_ordered,
                       plan, plan_dense, plan_from_csr, plan_workspace_bytes, router_exp, tile_stats,
                       version)

__all__ = [
    "EXPORTS", "SA_BF16", "SA_FP32", "attention", "attention_noalloc", "pipelined_workspace_bytes", "Fp8Pack", "fp8_pack_bytes", "fwd_fp8", "quantize_fp8", "Plan", "SaPlan", "SparseAttnError", "bwd", "bwd_workspace_bytes", "cube_order",
    "cube_permute", "fwd", "load_library", "plan_ordered",
    "plan", "plan_dense", "plan_from_csr", "plan_workspace_bytes", "router_exp", "tile_stats",
    "version",
]
