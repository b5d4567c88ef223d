// Internal declarations shared by the library's translation units (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sparse_attn.h"

namespace sa {

constexpr int kMaxKvBlocks = 4096;
constexpr size_t kAlign = 256;
// Word 3 of a raw buffer resource on CDNA: 32-bit data format (field bits 15..18 = 4),
// no swizzle, no thread-id add. Offsets are bytes (stride 0).
constexpr int kRawBufferWord3 = 0x00020000;

// Larger of two scores or probabilities, for the attention kernels' tile max. fmaxf first
// quiets any operand the compiler cannot prove canonical (an MFMA result, a lane swap),
// one VALU instruction each; IEEE maximum (v_maximum3_f32 on gfx950) needs none. The two
// agree on the values these kernels see, which are never NaN (a tile max of +0 against -0
// only changes the sign of a zero that is then subtracted).
__device__ __forceinline__ float score_max(float a, float b) { return __builtin_elementwise_maximum(a, b); }

inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Router launchers (router.hip). All return hipSuccess or the launch error.
// q_order: NULL, or per-head position -> row table; block rows are then read through it
hipError_t launch_pool(const void *x, sa_dtype dt, int BH, int H, int N, int D, int bs,
                       const int32_t *order, float *out, hipStream_t s);
hipError_t launch_scores(const float *qbar, const float *kbar, int BH, int nQ, int nKV, int D,
                         float c, float *scores, hipStream_t s);
// Also overwrites each row's slots of scores with its kept blocks in visit order (int32).
hipError_t launch_select(float *scores, int R, int nKV, int ragged_last, int m_k, float p, int p_all,
                         uint32_t *bitmap, int nwords, int32_t *counts, hipStream_t s);
// also writes the total (row_ptr[R]) to *nnz as int64
hipError_t launch_scan(const int32_t *counts, int R, int32_t *row_ptr, int64_t *nnz, hipStream_t s);
hipError_t launch_fill(const uint32_t *bitmap, int nwords, const int32_t *row_ptr, int R,
                       int32_t *col_idx, hipStream_t s);
hipError_t launch_dense_plan(int R, int nKV, int32_t *row_ptr, int32_t *col_idx, int64_t *nnz, hipStream_t s);
hipError_t launch_row_order(const int32_t *row_ptr, int R, int nQ, int32_t *row_order, hipStream_t s);
hipError_t launch_router_exp(const float *x, float *y, int64_t n, hipStream_t s);

// Attention launchers (attention.hip).
struct FwdArgs {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const int32_t *row_ptr, *col_idx, *row_order;
  const int32_t *visit;    // NULL, or row r's kept blocks in visit order at visit[r * n_kvblk]
  const int32_t *q_order;  // NULL, or per head: query position -> storage row of q, o, lse
  const int32_t *kv_order; // NULL, or per head: key position -> storage row of k, v
  int B, H, N, D, block_q, block_kv, n_qblk, n_kvblk;
  float scale_log2;        // log2(e) / sqrt(D)
  double scale_log2_f64;   // the same in fp64
  // linear branch (null alpha: off)
  const float *alpha;      // [alpha_H, D]: head h of this call uses row (alpha_h0 + h) % alpha_H
  int alpha_h0, alpha_H;
  const uint16_t *hct;     // [R, D, D] bf16 per plan row: H_C^T, row d = value channel
  const float *zc;         // [R, D] fp32 per plan row: z_C
};
hipError_t launch_fwd(const FwdArgs &a, sa_dtype dt, hipStream_t s);
hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t s);  // sparse_fwd_bf16.hip
// Linear branch (linear.hip). The prepass writes, per head, phi(k) in bf16 with zero rows
// padding N up to a multiple of 64 ([B*H, n_pad, D]), H = sum_j phi(k_j) v_j^T (fp32
// [B*H, D, D], row c = key channel, column d = value channel) and z = sum_j phi(k_j) (fp32
// [B*H, D]); the apply step then writes, per query block (plan row) that does not keep
// every KV block, the sums over its masked-out blocks: H_C^T in bf16 and z_C in fp32. The
// forward's epilogue multiplies them by phi(q) and blends.
struct LinearBufs {
  float *partial;          // [B*H, chunks, D*D + D] per-chunk partial H and z
  int chunks;
  uint16_t *phik;          // [B*H, n_pad, D]
  int n_pad;
  float *h;                // [B*H, D, D]
  float *z;                // [B*H, D]
  uint16_t *hct;           // [R, D, D]
  float *zc;               // [R, D]
};
hipError_t launch_linear_prepass(const void *k, const void *v, sa_dtype dt, int BH, int N, int D,
                                 const LinearBufs &lb, hipStream_t s);
hipError_t launch_linear_apply(const FwdArgs &a, const LinearBufs &lb, hipStream_t s);
int linear_prepass_chunks(int N);
// Head-aware 3-D tiling (tiling.hip): raster <-> per-head cube order of [B, H, N, D] rows.
constexpr int kMaxCubeHeads = 128;
struct CubeTable {
  int c[kMaxCubeHeads][3];   // (ct, ch, cw) per head
};
hipError_t launch_cube_permute(const void *src, void *dst, int BH, int H, int N, int row_bytes, int T,
                               int Hg, int W, const CubeTable &cubes, int inverse, hipStream_t s);
hipError_t launch_cube_order(int H, int T, int Hg, int W, const CubeTable &cubes, int32_t *order,
                             hipStream_t s);
// Backward (backward.hip).
struct BwdArgs {
  const uint16_t *q, *k, *v, *o, *dout;   // [B, H, N, D] bf16
  const float *lse;                        // [B, H, N] from the forward
  float *dvec;                             // [B*H, NP] workspace: rowsum(dO * O), 0 past N
  float *lse2;                             // [B*H, NP] workspace: lse * log2(e), +inf past N
  int NP;                                  // n_qblk * block_q (per-head padded length)
  uint16_t *dq, *dk, *dv;                  // [B, H, N, D] bf16
  const int32_t *row_ptr, *col_idx, *row_order;
  int32_t *col_ptr, *row_idx;              // CSC of the mask (workspace)
  int32_t *col_order;                      // dkdv slot -> KV block column, balanced over XCDs (workspace)
  int B, H, N, D, block_q, n_qblk, n_kvblk;
  float scale;                             // 1/sqrt(D)
  float scale_log2;                        // log2(e)/sqrt(D)
};
struct BwdBufs {
  uint32_t *tbits;   // [B*H*n_kvblk, nwq] column-major bitmap of the mask
  int nwq;           // ceil(n_qblk / 32)
  int32_t *ccount;   // [B*H*n_kvblk]
  int64_t *cnnz;     // the CSC's total (written by the scan, not read)
};
hipError_t launch_bwd(const BwdArgs &a, const BwdBufs &w, hipStream_t s);
// Low-bit forward (fp8.hip): OCP FP8 E4M3 codes with power-of-two group exponents.
struct Fp8Pack {
  uint8_t *q8, *k8, *vt8;   // [B,H,N,D], [B,H,N,D], [B,H,nKV,D,64]
  int32_t *qe, *ke, *ve;    // [B,H,nQ], [B,H,nKV], [B,H,D]
  uint32_t *vamax;          // [B,H,D] scratch
};
// i8qk: Q and K as int8 codes with fp32 scales (in qe, ke) instead of E4M3 with exponents
hipError_t launch_quantize_fp8(const uint16_t *q, const uint16_t *k, const uint16_t *v, int BH, int N, int D,
                               int bq, int i8qk, const Fp8Pack &p, hipStream_t s);
struct Fp8FwdArgs {
  const uint8_t *q8, *k8, *vt8;
  const int32_t *qe, *ke, *ve;
  uint16_t *o;              // [B, H, N, D] bf16
  float *lse;               // [B, H, N] or null
  const int32_t *row_ptr, *col_idx, *row_order;
  const int32_t *visit;     // NULL, or row r's kept blocks in visit order at visit[r * n_kvblk]
  int B, H, N, D, block_q, n_qblk, n_kvblk;
  float scale_log2;         // log2(e) / sqrt(D)
};
hipError_t launch_fwd_fp8(const Fp8FwdArgs &a, int i8qk, hipStream_t s);
// Tile heatmap, pass 2 (heatmap.hip): per (row, KV block) max and mean mass of exp(s - lse).
hipError_t launch_tile_stats(const void *q, const void *k, const float *lse, int BH, int H, int N, int D,
                             int bq, int nQ, int nKV, float sl2, float *tmax, float *tmass, hipStream_t s);

}  // namespace sa
