"""CPU oracle for block-sparse attention with a hybrid top-k / top-p block router.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the bench's CPU
baseline may import this package. The GPU library never calls it, and it shares no
code with the GPU library (the seeded input generator in ``workloads`` is the only
module both sides use, and that module holds none of the method's arithmetic).

Two tracks:

* ``oracle.mask``: the block mask. It is written as an fp32 specification with one
  fixed order for every floating-point operation, so that a GPU router can reproduce
  it bit for bit. Its steps follow the pages: mean pooling of Q and K per block (SLA2
  page, router item 1), a row softmax over pooled block scores, and the union of the
  top-k% set and the smallest top-p cumulative-mass set per row (SpargeAttention2
  page, section 2(1)).
* ``oracle.attention``: the outputs, in float64. Masked softmax attention over the
  kept tiles (SpargeAttention2 page, section 2(3): masked tiles contribute nothing),
  dense attention, a brute-force N x N masked softmax, and the elu+1 linear branch over
  the masked-out blocks blended as O = alpha*Os + (1 - alpha)*Ol (SLA2 page, item 2;
  SALAD page, section 2.1).
* ``oracle.heatmap``: the ground-truth tile heatmap of full attention (Veda page,
  section 2.1: max pooling of the attention matrix over query x key tiles), and the
  mean attention mass per tile, in float64.
* ``oracle.tiling``: the group-major token order of head-aware 3-D tiling (Veda page,
  section 2.2: a per-head factorisation of the tile into a spatio-temporal cube).
* ``oracle.backward``: the gradients dQ, dK, dV of block-sparse attention in float64
  (the pages fine-tune through the sparse kernel).
* ``oracle.fp8``: the low-bit forward (SLA2 page, quantisation-aware fine-tuning):
  Q, K, V quantised to OCP FP8 E4M3 with power-of-two group scales (or Q and K to
  symmetric int8 with fp32 group scales), then attention in float64 on the decoded
  values.

Parity pins (tests marked "not gpu") tie both tracks to facts outside the oracle:
closed forms, library routines, brute force and hand-derived fixtures. Parity of the
realised sparsity against the workloads' targets is unpinned (it depends on the
generator, not on the method).
"""
from .mask import (exp_sa, pool_blocks, block_scores, tree_sum, select_row, topk_count,
                   oracle_plan, plan_stats, score_scale)
from .attention import (sparse_attention, dense_attention, brute_masked_attention,
                        linear_branch, blend, phi, dense_plan, csr_to_mask)
from .heatmap import tile_heatmap
from .tiling import cube_order, permute_heads, unpermute_heads
from .backward import sparse_attention_backward
from .fp8 import (e4m3_decode, e4m3_encode, scale_exponent, quantize_qkv, dequantize,
                  fp8_attention, int8_scales, int8_encode, quantize_qkv_i8qk, dequantize_i8qk,
                  i8qk_attention)

__all__ = [
    "exp_sa", "pool_blocks", "block_scores", "tree_sum", "select_row", "topk_count",
    "oracle_plan", "plan_stats", "score_scale",
    "sparse_attention", "dense_attention", "brute_masked_attention", "linear_branch",
    "blend", "phi", "dense_plan", "csr_to_mask", "tile_heatmap", "cube_order", "permute_heads",
    "unpermute_heads", "sparse_attention_backward", "e4m3_decode", "e4m3_encode",
    "scale_exponent", "quantize_qkv", "dequantize", "fp8_attention", "int8_scales",
    "int8_encode", "quantize_qkv_i8qk", "dequantize_i8qk", "i8qk_attention",
]
