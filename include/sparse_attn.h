/*
 * sparse_attn.h — block-sparse softmax attention for video DiTs on MI355X (gfx950).
 *
 * Two calls make the hot path:
 *
 *   sparse_attn_plan   the per-call block-mask router. Q and K are mean-pooled per block
 *                      and per head (SLA2 page, router item 1; its learnable projection
 *                      is the identity here), pooled blocks are scored, each query-block
 *                      row gets a softmax over its KV-block scores, and the row keeps the
 *                      union of its top-k% blocks and of the smallest set whose cumulative
 *                      probability reaches p (SpargeAttention2 page, section 2(1), applied
 *                      to blocks). The result is a CSR list of kept KV blocks per query
 *                      block.
 *   sparse_attn_fwd    FlashAttention-style attention that visits only the kept Q x KV
 *                      tiles; masked tiles take no part in the products or the softmax
 *                      (SpargeAttention2 page, section 2(3)). With alpha given, an elu+1
 *                      linear-attention branch over each query block's masked-out KV
 *                      blocks (SALAD page, section 2.1; SLA2 page: dropped blocks feed the
 *                      linear branch) is blended as O = alpha*Os + (1-alpha)*Ol (SLA2 page,
 *                      item 2).
 *
 * Conventions for every call:
 *   - Q, K, V, O are contiguous [B, H, N, D] arrays in device memory, D innermost, in
 *     the dtype passed (bf16 or fp32; O has the dtype of Q).
 *   - Block I of a sequence covers tokens [I*bs, min(N, (I+1)*bs)); the last block may
 *     be ragged. Row r = (b*H + h)*n_qblk + I; R = B*H*n_qblk rows.
 *   - Attention is non-causal with logits q.k / sqrt(D).
 *   - The library allocates no memory. The caller owns every buffer, including the
 *     workspaces, whose sizes the *_workspace_bytes calls give; workspaces must be
 *     256-byte aligned device memory.
 *   - Every launch is asynchronous on the given stream; nothing synchronises. Calls on
 *     different streams with different workspaces may run concurrently.
 *   - Arguments are validated on the host before anything is launched; a call that
 *     returns an error has launched nothing (except SA_ERR_HIP, which reports a failed
 *     launch). Device faults surface at the caller's next synchronisation.
 *   - Results are deterministic: the same inputs give bitwise-identical plans and
 *     outputs (no floating-point atomics anywhere).
 *   - Non-finite inputs give unspecified results.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = -1,   /* null pointer, non-positive size, k or p outside [0, 1] */
  SA_ERR_UNSUPPORTED = -2,   /* a valid but unsupported shape (D, block sizes, sizes) */
  SA_ERR_WORKSPACE = -3,     /* workspace null, too small or misaligned */
  SA_ERR_PLAN_MISMATCH = -4, /* plan made for other shapes or another dtype */
  SA_ERR_BAD_CSR = -5,       /* malformed caller CSR (plan_from_csr) */
  SA_ERR_HIP = -6            /* a HIP call or kernel launch failed */
} sa_status;

typedef enum { SA_BF16 = 0, SA_FP32 = 1 } sa_dtype;

/* A block mask in CSR form. Plain data; row_ptr and col_idx point into the workspace
 * the plan was built in and stay valid while that workspace lives. One plan may serve
 * any number of sparse_attn_fwd calls. */
typedef struct sa_plan {
  int32_t B, H, N, D;
  int32_t block_q, block_kv;
  int32_t n_qblk, n_kvblk;   /* ceil(N/block_q), ceil(N/block_kv) */
  int32_t dtype;             /* sa_dtype of the Q and K the plan was built for */
  int32_t reserved;
  int32_t *row_ptr;          /* device, [R + 1], row_ptr[0] = 0, row_ptr[R] = nnz */
  int32_t *col_idx;          /* device, capacity R * n_kvblk; ascending within a row */
  int32_t *row_order;        /* device, [R]: a permutation of the rows, the order in which
                              * the forward kernels visit them (runs of consecutive rows
                              * spread so that each XCD gets an equal kept-tile share);
                              * it changes no result */
  const int32_t *q_order;    /* device [H*N] or NULL (caller-owned, see
                              * sparse_attn_plan_ordered): query position i of head h is
                              * raster token q_order[h*N + i] */
  const int32_t *kv_order;   /* device [H*N] or NULL (caller-owned): key position j of head
                              * h is raster token kv_order[h*N + j]; NULL: k and v are
                              * already in key-position order */
  int32_t *visit;            /* device, capacity R * n_kvblk, or NULL: row r's kept blocks
                              * (the same set as its col_idx range) at visit[r * n_kvblk],
                              * in the order the forward kernels visit them: pooled score
                              * descending, ties to the lower block index, a kept ragged
                              * last block moved to the end. It changes no result beyond
                              * rounding order. NULL (plans from a caller's CSR and the
                              * dense plan): the forward visits col_idx order. */
  int64_t *nnz;              /* device scalar in the workspace: the number of kept blocks,
                              * equal to row_ptr[R]; written by the plan calls on their
                              * stream, so it may be read once that stream has reached the
                              * end of the call (a device-side consumer needs no host
                              * round trip to size its work) */
} sa_plan;

/* Accepted shapes: D in {64, 128}; block_q in {64, 128}; block_kv = 64; B*H <= 65535;
 * n_kvblk <= 4096; B*H*n_qblk*n_kvblk < 2^31. */

/* Workspace bytes that sparse_attn_plan / _plan_dense / _plan_from_csr need; 0 when the
 * shape is invalid or unsupported. */
size_t sparse_attn_plan_workspace_bytes(int B, int H, int N, int D, int block_q, int block_kv);

/* The hybrid top-k / top-p router (SpargeAttention2 page, section 2(1); SLA2 page,
 * router item 1). q, k: device [B, H, N, D] in dtype. topk_frac: the top-k rule keeps
 * m_k = min(nKV, max(1, ceil(topk_frac*nKV - 1e-9))) blocks per row; top_p: the top-p
 * rule keeps the shortest score-ordered prefix whose cumulative softmax mass reaches
 * top_p (all blocks when top_p >= 1). Each row keeps the union, which is the longer of
 * the two prefixes of one order (scores descending, ties to the lower block index).
 * Pooling, scores, softmax and the cumulative sums follow one fixed fp32 order, so the
 * mask is exactly reproducible. On success *out describes the plan. */
sa_status sparse_attn_plan(const void *q, const void *k, sa_dtype dtype,
                           int B, int H, int N, int D, int block_q, int block_kv,
                           double topk_frac, double top_p,
                           void *workspace, size_t ws_bytes, sa_plan *out, hipStream_t stream);

/* The all-ones mask (every query block keeps every KV block): dense attention through the
 * same forward kernel. */
sa_status sparse_attn_plan_dense(sa_dtype dtype, int B, int H, int N, int D, int block_q,
                                 int block_kv, void *workspace, size_t ws_bytes,
                                 sa_plan *out, hipStream_t stream);

/* A caller-given mask. host_row_ptr [R + 1] and host_col_idx [host_row_ptr[R]] are HOST
 * arrays, checked before use (row_ptr starts at 0 and never decreases; columns in
 * [0, n_kvblk) and strictly ascending within a row) and copied into the workspace;
 * the call returns once the host arrays may be reused. Rows may be empty: such a row's
 * outputs are 0 (and its LSE -inf). */
sa_status sparse_attn_plan_from_csr(sa_dtype dtype, int B, int H, int N, int D, int block_q,
                                    int block_kv, const int32_t *host_row_ptr,
                                    const int32_t *host_col_idx, void *workspace,
                                    size_t ws_bytes, sa_plan *out, hipStream_t stream);

/* The mask of sparse_attn_plan for queries taken in a per-head order other than their
 * storage order (head-aware 3-D tiling, Veda page, section 2.2: query blocks that are
 * compact cubes of the token grid). q stays in storage (raster) order; query position i
 * of head h is token q_order[h*N + i], so query block I is positions [I*block_q, ...).
 * Keys likewise: with kv_order, k (and the v later given to sparse_attn_fwd) stay in
 * storage order and key position j of head h is token kv_order[h*N + j], so KV block J
 * is positions [J*block_kv, ...); with kv_order NULL, k and v are given already in
 * key-position order (for example moved by sparse_attn_cube_permute). The plan keeps
 * both pointers: sparse_attn_fwd with this plan reads q, k and v through them and writes
 * o (and lse) back to q's storage rows, so nothing is moved before or after.
 * q_order: device int32 [H*N], a permutation of 0..N-1 per head (sparse_attn_cube_order
 * builds one); kv_order: NULL or the same kind of table. Both must outlive the plan's
 * use. Entries outside [0, N) are clamped (the results are then meaningless, but no
 * access leaves the tensors). bf16 only (fp32: SA_ERR_UNSUPPORTED); sparse_attn_fwd
 * with a kv_order plan has no linear branch (alpha: SA_ERR_UNSUPPORTED). Otherwise as
 * sparse_attn_plan. */
sa_status sparse_attn_plan_ordered(const void *q, const void *k, sa_dtype dtype, int B, int H,
                                   int N, int D, int block_q, int block_kv, double topk_frac,
                                   double top_p, const int32_t *q_order,
                                   const int32_t *kv_order, void *workspace, size_t ws_bytes,
                                   sa_plan *out, hipStream_t stream);

/* Workspace bytes sparse_attn_fwd needs with this plan: 0 without the linear branch
 * (with_linear = 0); 0 as well when plan is NULL or describes an unsupported shape. With
 * it: per head the totals H (fp32 D x D) and z, their per-chunk partials and phi(K) in
 * bf16, and per query block its masked-out sums H_C^T (bf16 D x D) and z_C (fp32). */
size_t sparse_attn_fwd_workspace_bytes(const sa_plan *plan, int with_linear);

/* Block-sparse attention over the plan's kept tiles (SpargeAttention2 page, section 2(3)).
 * q, k, v: device [B, H, N, D] in dtype; the shapes and dtype must equal the plan's.
 * alpha: device float [H, D] or NULL. With alpha, the linear branch (SALAD page, section
 * 2.1) covers each query block's masked-out KV blocks with phi = elu + 1 on the raw q
 * and k, Ol = phi(q).sum_j phi(k_j) v_j^T / phi(q).sum_j phi(k_j) (0 when a query block
 * keeps every KV block), and o = alpha*Os + (1-alpha)*Ol (SLA2 page, item 2).
 * o: device [B, H, N, D] in dtype. lse: device float [B, H, N] or NULL; receives the
 * natural-log sum of exp(logits) over kept tokens (-inf for an empty row).
 * workspace: sparse_attn_fwd_workspace_bytes bytes (may be NULL when that is 0).
 * Rounding: a row's tiles are taken in the plan's visit order (when it has one); for
 * bf16 without lse the running max is lazy (it may trail the true max by up to 16 in
 * the log2 domain, so probabilities reach at most 2^16), with lse it is exact. Both meet the same error bounds, but o may
 * differ in its last bits between a call with lse and one without. */
sa_status sparse_attn_fwd(const void *q, const void *k, const void *v, sa_dtype dtype,
                          int B, int H, int N, int D, const sa_plan *plan,
                          const float *alpha, void *o, float *lse,
                          void *workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes sparse_attn_pipelined needs: one plan workspace per chunk of heads and,
 * with the linear branch (with_linear != 0), one forward workspace for a chunk. */
size_t sparse_attn_pipelined_workspace_bytes(int B, int H, int N, int D, int block_q, int block_kv,
                                             int n_chunks, int with_linear);

/* The two hot-path calls, sparse_attn_plan then sparse_attn_fwd, for all B*H heads,
 * pipelined over chunks of heads: the B*H (batch, head) pairs are split into
 * ceil(B*H / ceil(B*H / n_chunks)) chunks of consecutive pairs.
 * The chunks' plans run back to back on aux_stream and their forwards on `stream`, each
 * forward after its chunk's plan, so every plan but the first (a chain of small,
 * latency-bound kernels) runs under the forwards of earlier chunks. alpha: as for
 * sparse_attn_fwd (device float [H, D], or NULL for no linear branch; bf16 only). With
 * it, each chunk's linear prepass (which reads k and v, not the mask) is enqueued on
 * `stream` before the wait for that chunk's plan, so even with n_chunks = 1 it runs beside
 * the plan. A head's mask depends on that head alone, so o and lse equal those of the
 * two-call path bit for bit.
 * Ordering: the plans on aux_stream start after the work enqueued on `stream` before this
 * call; every forward is on `stream`, so later work there follows them. aux_stream may
 * equal stream (plans and forwards then run in order). The plans live in the workspace and
 * are not returned; a caller that needs the mask (for the backward) uses the two calls.
 * q, k, v, o, lse, dtype, block sizes, topk_frac and top_p as for sparse_attn_plan and
 * sparse_attn_fwd; n_chunks >= 1 (values above B*H act as B*H).
 * workspace: sparse_attn_pipelined_workspace_bytes bytes, 256-byte aligned.
 * With the linear branch and two streams, a chunk's prepass starts once its pooling is
 * done (it then overlaps the score and select kernels) and its apply step waits only for
 * its CSR, not for the work order.
 * With two streams the call orders them with HIP events that it makes on its first use in
 * a thread (per device, n_chunks + 1 of them, 3 * n_chunks + 1 with the linear branch)
 * and reuses on every later call from that thread; it creates and destroys nothing per
 * call. */
sa_status sparse_attn_pipelined(const void *q, const void *k, const void *v, sa_dtype dtype,
                                int B, int H, int N, int D, int block_q, int block_kv,
                                double topk_frac, double top_p, int n_chunks,
                                const float *alpha, void *o, float *lse, void *workspace,
                                size_t ws_bytes, hipStream_t stream, hipStream_t aux_stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): sparse_attn_pipelined with one stream,
 * no workspace argument and no linear branch. The plan workspaces live in a static device array of the
 * library, 128 MiB per device (every device the library runs on holds it until the
 * process ends). Heads are taken in chunks of equal size, as many heads per chunk as fit
 * in that array; each chunk is planned and then attended on `stream` before the next
 * chunk reuses the array. The call allocates nothing (no hipMalloc, hipFree or event);
 * its first call on a device looks up the array's device address once.
 * o and lse equal those of sparse_attn_plan + sparse_attn_fwd (and of
 * sparse_attn_pipelined) bit for bit. Arguments as for sparse_attn_pipelined;
 * SA_ERR_WORKSPACE when one head's plan workspace (sparse_attn_plan_workspace_bytes
 * with B = H = 1) exceeds 128 MiB. Every call on a device shares the one array and
 * leaves its last plan in it: calls on one stream are ordered, but calls on one device
 * that are not ordered with each other (other streams, other threads) race. */
sa_status sparse_attn_pipelined_noalloc(const void *q, const void *k, const void *v, sa_dtype dtype,
                                        int B, int H, int N, int D, int block_q, int block_kv,
                                        double topk_frac, double top_p, void *o, float *lse,
                                        hipStream_t stream);

/* Workspace bytes sparse_attn_bwd needs for this shape. */
size_t sparse_attn_bwd_workspace_bytes(int B, int H, int N, int D, int block_q, int block_kv);

/* Gradients of block-sparse attention over the plan's kept tiles (the pages fine-tune
 * through the sparse kernel: SpargeAttention2 page, section 2; SLA2 page). With
 * c = 1/sqrt(D), P = exp(c*q k^T - lse) on kept tiles and Dv = rowsum(dO * o):
 *   dq = c * (P * (dO v^T - Dv)) k,  dk = c * (P * (dO v^T - Dv))^T q,  dv = P^T dO.
 * q, k, v, o, dout: device [B, H, N, D] bf16 (o and lse as sparse_attn_fwd wrote them
 * with this plan, without the linear branch); lse: device float [B, H, N].
 * dq, dk, dv: device [B, H, N, D] bf16, written in full (zeros where nothing is kept).
 * Deterministic (no atomics on values). bf16 only and plans without a query order;
 * otherwise SA_ERR_UNSUPPORTED. workspace: sparse_attn_bwd_workspace_bytes bytes. */
sa_status sparse_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                          const float *lse, const void *dout, sa_dtype dtype, int B, int H,
                          int N, int D, const sa_plan *plan, void *dq, void *dk, void *dv,
                          void *workspace, size_t ws_bytes, hipStream_t stream);

/* Low-bit forward (SLA2 page, quantisation-aware fine-tuning: the forward pass runs on
 * queries, keys and values quantised to low precision). The page names no format; this
 * library uses OCP FP8 E4M3 (max 448, subnormals down to 2^-9, no infinities) with
 * power-of-two group scales. A group's exponent e is the smallest integer with
 * max|x| <= 448 * 2^e, clamped to [-64, 64] (-64 for an all-zero group), and a value x
 * is stored as the E4M3 code nearest to x * 2^-e, ties to the even code. Groups: q per
 * (batch, head, query block of block_q tokens), k per (batch, head, 64-key block), v per
 * (batch, head, channel) over all tokens.
 *
 * A second format (qk_format = SA_QK_INT8) keeps v as above and stores q and k as
 * symmetric int8 codes, more accurate on the logits at the same MFMA rate: for a group
 * with largest magnitude a, inv = 127 / a and s = a / 127 (correctly rounded fp32
 * divisions; 0 and 0 for an all-zero group), and x is stored as rint(fp32(x * inv)),
 * ties to even, decoding to code * s.
 *
 * The pack is one device buffer of sparse_attn_fp8_pack_bytes bytes holding, each part
 * starting at the next 256-byte boundary after the previous one, in this order:
 *   q8     uint8 [B, H, N, D]       codes of q, row-major (int8 codes with SA_QK_INT8);
 *   k8     uint8 [B, H, N, D]       codes of k (likewise);
 *   vt8    uint8 [B, H, nKV, D, 64] codes of v, each 64-key block transposed to channel
 *                                   rows; byte h*32 + b (h in {0, 1}, b < 32) of a row
 *                                   holds key (b/16)*32 + ((b/4)%4)*8 + h*4 + b%4 of the
 *                                   block; keys past N hold 0;
 *   qe     int32 [B, H, nQ]         exponents of the q groups (nQ = ceil(N/block_q));
 *                                   with SA_QK_INT8 the fp32 scales s, as bit patterns;
 *                                   the part is sized for B*H*ceil(N/64) entries, of
 *                                   which the first B*H*nQ are used;
 *   ke     int32 [B, H, nKV]        exponents of the k groups (nKV = ceil(N/64)); likewise;
 *   ve     int32 [B, H, D]          exponents of the v groups;
 *   vamax  uint32 [B, H, D]         the quantiser's scratch (per-channel max |v|);
 *   tail   4*block_q bytes          unused; it makes the pack's size depend on block_q.
 * Both calls below require pack_bytes to equal sparse_attn_fp8_pack_bytes for their
 * shape and block sizes, and packs for block_q 64 and 128 always differ in size, so a
 * pack quantised for another block_q than the plan's is rejected. */
size_t sparse_attn_fp8_pack_bytes(int B, int H, int N, int D, int block_q, int block_kv);

typedef enum { SA_QK_E4M3 = 0, SA_QK_INT8 = 1 } sa_qk_format;

/* Quantises q, k, v (device [B, H, N, D] bf16, finite) into pack (device, 256-byte
 * aligned, pack_bytes == sparse_attn_fp8_pack_bytes, else SA_ERR_WORKSPACE). block_q
 * must be the block_q of the plans the pack will be used with; block_kv must be 64.
 * fp32 inputs: SA_ERR_UNSUPPORTED. Deterministic. */
sa_status sparse_attn_quantize_fp8(const void *q, const void *k, const void *v, sa_dtype dtype,
                                   int B, int H, int N, int D, int block_q, int block_kv,
                                   int qk_format, void *pack, size_t pack_bytes,
                                   hipStream_t stream);

/* Block-sparse attention over the plan's kept tiles computed from an FP8 pack: the
 * products q k^T and P v run on fp8 MFMA with fp32 accumulation, the softmax in fp32,
 * and P (the probabilities scaled by 2^8 against the running maximum, by 2^4 when the
 * maximum is lazy) is rounded to E4M3 before it multiplies v; the row sums add the same
 * rounded values.
 * pack: as sparse_attn_quantize_fp8 wrote it, with the plan's block_q and the same
 * qk_format (SA_QK_INT8: q k^T on int8 MFMA with exact int32 sums, scaled in fp32);
 * pack_bytes must equal sparse_attn_fp8_pack_bytes for the plan's shape and block_q
 * (SA_ERR_PLAN_MISMATCH otherwise, SA_ERR_WORKSPACE when it is smaller). The format is
 * not recorded in the pack: a pack read with the other qk_format gives meaningless o.
 * plan: a bf16 plan for [B, H, N, D] without a query order (else SA_ERR_UNSUPPORTED).
 * o: device [B, H, N, D] bf16. lse: device float [B, H, N] or NULL, as sparse_attn_fwd;
 * without lse the running max is lazy (trailing by up to 2^4 in the log2 domain), so o
 * may differ in its last bits from a call with lse. */
sa_status sparse_attn_fwd_fp8(const void *pack, size_t pack_bytes, int qk_format, int B, int H,
                              int N, int D, const sa_plan *plan, void *o, float *lse,
                              hipStream_t stream);

/* Ground-truth tile heatmap of full attention (Veda page, section 2.1: the reference mask
 * max-pools the full attention matrix over query x key tiles; section 2.3: two passes).
 * Pass 1 is sparse_attn_fwd on a sparse_attn_plan_dense plan with an lse output; this
 * call is pass 2. With p_ij = exp(q_i.k_j / sqrt(D) - lse_i), for every row
 * r = (b*H + h)*n_qblk + I and KV block J:
 *   tile_max[r*n_kvblk + J]  = max of p_ij over i in query block I, j in KV block J;
 *   tile_mass[r*n_kvblk + J] = the sum of those p_ij divided by the size of block I.
 * q, k: device [B, H, N, D] bf16 (fp32 inputs return SA_ERR_UNSUPPORTED).
 * lse: device float [B, H, N], finite, natural log (as sparse_attn_fwd writes it).
 * tile_max, tile_mass: device float [B*H*n_qblk*n_kvblk]; either may be NULL, not both.
 * Shapes and block sizes are checked as for sparse_attn_plan. Deterministic. */
sa_status sparse_attn_tile_stats(const void *q, const void *k, const float *lse, sa_dtype dtype,
                                 int B, int H, int N, int D, int block_q, int block_kv,
                                 float *tile_max, float *tile_mass, hipStream_t stream);

/* Head-aware 3-D tiling (Veda page, section 2.2: each head tiles the token grid with its
 * own factorisation of the hardware tile, so that a block of consecutive tokens is a
 * compact spatio-temporal cube). Tokens lie on a (T, Hg, W) grid in raster order,
 * n = (t*Hg + y)*W + x, N = T*Hg*W. Head h's cube order with cube (ct, ch, cw) sorts the
 * tokens by (t/ct, y/ch, x/cw, t%ct, y%ch, x%cw); pos_h(n) is token n's place in it.
 * inverse = 0: dst[b, h, pos_h(n), :] = src[b, h, n, :] (raster to cube order);
 * inverse = 1: dst[b, h, n, :] = src[b, h, pos_h(n), :] (back to raster order).
 * Attention on cube-ordered q, k, v (plan and fwd as usual, with the blocks now cubes)
 * followed by the inverse move of o is attention under the cube partition.
 * src, dst: device [B, H, N, D] in dtype, not overlapping; D*element size a multiple of
 * 16 bytes. host_cubes: host int32 [H*3], (ct, ch, cw) per head, each >= 1; H <= 128.
 * Bitwise copy; no arithmetic on the values. */
sa_status sparse_attn_cube_permute(const void *src, void *dst, sa_dtype dtype, int B, int H, int N,
                                   int D, int T, int Hg, int W, const int32_t *host_cubes,
                                   int inverse, hipStream_t stream);

/* The same cube orders as an index table for sparse_attn_plan_ordered: for every head h
 * and position i, order[h*N + pos_h(n)] = n. order: device int32 [H*N]. host_cubes as
 * for sparse_attn_cube_permute (H <= 128). */
sa_status sparse_attn_cube_order(int H, int T, int Hg, int W, const int32_t *host_cubes,
                                 int32_t *order, hipStream_t stream);

/* Diagnostic: y[i] = the router's fp32 exp of x[i] for x[i] <= 0 (0 below -86), evaluated
 * on the device with the router's own code. x, y: device float [n]. */
sa_status sparse_attn_router_exp(const float *x, float *y, int64_t n, hipStream_t stream);

/* A static description of a status code. */
const char *sparse_attn_status_string(sa_status status);

/* Library version, major*10000 + minor*100 + patch. */
int sparse_attn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPARSE_ATTN_H */
