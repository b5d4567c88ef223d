// Block-sparse attention forward, bf16 inputs, for gfx950 (SpargeAttention2 page, section
// 2(3): only the kept Q x KV tiles are visited, so masked tiles cost neither matrix
// products nor softmax work).
//
// One workgroup per query block (CSR row), one wave per 32 queries, 64-key tiles:
//   S^T = K Q^T      bf16 MFMA 32x32x16; each lane holds the 32 scores of one query for
//                    its half of the tile, so max and sum are in-lane plus one exchange
//                    between the two lane halves;
//   softmax          log2 domain, fp32, raw v_exp_f32. The row sums add the bf16-rounded
//                    probabilities that the MFMA multiplies. Without an LSE output the
//                    running max is lazy: it moves only when a tile's max passes it by
//                    more than kLazy (log2 units), so the O rescale (which touches every
//                    accumulator) runs on few tiles, and probabilities stay below
//                    2^kLazy, which bf16 holds at the same relative precision. A dominant
//                    key's probability is then no longer exactly 1, but its rounding
//                    cancels in O = sum(p v) / sum(p). It does not cancel in the sum
//                    itself (up to 2^-8 relative, the bf16 unit roundoff), so when the
//                    LSE is written the max is exact (margin 0) and the largest term of
//                    every row sum is exactly 1;
//   O^T += V^T P^T   bf16 MFMA; P packed with v_cvt_pk_bf16_f32.
// K and V tiles go from HBM straight into LDS (buffer_load_dwordx4 ... lds for whole
// tiles, global_load_lds_dwordx4 for the ragged and gathered ones), row-major with
// one pad granule per row, double-buffered: the next tile's loads are in flight while the
// current tile is computed, with one barrier per tile. The V^T operand is read with the
// transposing LDS read ds_read_b64_tr_b16, so V needs no transposition on the way in. The
// tiles of a row come in the plan's visit order (pooled score descending, so the running
// max settles early) or, without one, in ascending block order. Either way the ragged last
// KV block (if kept) is the last tile of a row; its rows past N reload the last valid
// row, and only that tile carries the key mask.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;
typedef __attribute__((address_space(3))) bf16x4_t lbf16x4_t;

// s_waitcnt immediate that waits for all vector-memory operations (direct LDS loads
// included) and leaves the export and LDS counters unconstrained
constexpr int kVmcnt0 = 0x0F70;

constexpr int kBk = 64;            // keys per tile
constexpr float kLazy = 16.0f;      // lazy-max margin, log2 units

__device__ __forceinline__ int xcd_remap(int b, int G) {
  const int q = G / 8;
  if (b >= q * 8) return b;
  return (b % 8) * q + b / 8;
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  bf16x4_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  v[2] = (__bf16)c;
  v[3] = (__bf16)d;
  return __builtin_bit_cast(uint2, v);
}

// elu + 1 on the raw bf16 value, the linear branch's feature map
__device__ __forceinline__ float phi(float x) { return x > 0.0f ? x + 1.0f : __expf(x); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t phi2(uint32_t w) {
  const bf16x2_t v = {(__bf16)phi(bf_lo(w)), (__bf16)phi(bf_hi(w))};
  return __builtin_bit_cast(uint32_t, v);
}

// Two waves per SIMD with four-wave workgroups (two workgroups per CU by LDS). With
// 64-query workgroups (NW = 2) the double-buffered K/V tiles still take 67.6 KB, so LDS
// allows two workgroups, one wave per SIMD, and the register budget is not the limit.
template <int D, int NW, bool LIN, bool GATHER>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW == 4 ? 2 : 1)))
void sparse_fwd_bf16_kernel(FwdArgs a) {
  constexpr int BQ = 32 * NW;
  constexpr int GR = D / 8 + 1;             // K: 16-byte granules per LDS row (one pad granule)
  constexpr int ROWB = GR * 16;             // K: bytes per LDS row
  constexpr int NI = GR;                    // K: 1 KB direct loads per 64-row tile (64*GR/64)
  constexpr int NIW = (NI + NW - 1) / NW;   // K: direct loads per wave
  constexpr int VROWB = D * 2;              // V: unpadded rows, 64-byte segments XOR-swizzled
  constexpr int VNI = D / 8;                // V: 1 KB direct loads per tile
  constexpr int VNIW = (VNI + NW - 1) / NW;
  constexpr int VSEG = D / 32;              // V: 64-byte segments per row (swizzle range)
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;

  // double-buffered K and V tiles, row-major [key][channel] with padded rows; separate
  // arrays so the compiler can tell the in-flight loads from the tile being read
  __shared__ __align__(16) char k0s[kBk * ROWB];
  __shared__ __align__(16) char v0s[kBk * VROWB];
  __shared__ __align__(16) char k1s[kBk * ROWB];
  __shared__ __align__(16) char v1s[kBk * VROWB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in an SGPR
  __builtin_assume(wid >= 0 && wid < NW);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int rlin = xcd_remap(blockIdx.x, gridDim.x);
  const int row = a.row_order ? a.row_order[rlin] : rlin;
  const int nQ = a.n_qblk;
  const int bh = row / nQ;
  const int I = row - bh * nQ;
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const uint16_t *qg = reinterpret_cast<const uint16_t *>(a.q) + head;
  const uint16_t *kg = reinterpret_cast<const uint16_t *>(a.k) + head;
  const uint16_t *vg = reinterpret_cast<const uint16_t *>(a.v) + head;
  uint16_t *og = reinterpret_cast<uint16_t *>(a.o) + head;

  const int qi = I * BQ + wid * 32 + l32;   // query position
  const bool q_ok = qi < N;
  // storage row of this query's q, o and lse (positions map through the plan's table)
  int qrow = qi;
  if (a.q_order && q_ok) qrow = min(max(a.q_order[(size_t)(bh % a.H) * N + qi], 0), N - 1);
  // loads that depend on the row alone go out before the row's CSR range comes back: the
  // Q fragments and, with visit lists, the first two kept blocks
  bf16x8_t qf[KSTEPS];   // Q fragments: B operand of S^T = K Q^T
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (q_ok) w = *reinterpret_cast<const uint4 *>(qg + (size_t)qrow * D + s * 16 + hf * 8);
    qf[s] = __builtin_bit_cast(bf16x8_t, w);
  }
  int vis0 = 0, vis1 = 0;
  if (a.visit) {
    const int32_t *vr = a.visit + (size_t)row * a.n_kvblk;
    vis0 = vr[0];
    if (a.n_kvblk > 1) vis1 = vr[1];
  }
  const int beg = a.row_ptr[row];
  const int end = a.row_ptr[row + 1];

  if (!LIN && beg == end) {
    // no kept tile: O = 0, LSE = -inf (with the linear branch such a row runs the
    // epilogue below with Os = 0, so O = (1 - alpha) * Ol)
    if (q_ok) {
      for (int d = hf * (D / 2); d < (hf + 1) * (D / 2); d += 4)
        *reinterpret_cast<uint2 *>(og + (size_t)qrow * D + d) = make_uint2(0u, 0u);
      if (a.lse && hf == 0) a.lse[(size_t)bh * N + qrow] = -INFINITY;
    }
    return;
  }

  // Direct HBM -> LDS tile loads. Load i of a matrix fills LDS granules 64i .. 64i+63 of
  // the padded tile; lane p of it carries granule 64i + p = (row r, column granule c).
  // Pad granules (c == D/8) reload granule 0 of their row. Wave w issues loads w, w+NW, ...
  uint32_t goff[NIW]; // K: byte offset of the lane's source granule within a 64-row tile
#pragma unroll
  for (int m = 0; m < NIW; ++m) {
    const int p = 64 * (wid + m * NW) + lane;
    const int c = p % GR;
    goff[m] = ((p / GR) * D + (c < D / 8 ? c : 0) * 8) * 2;
  }
  // V: LDS granule (row r, physical granule pg) holds logical granule
  // pg ^ ((r mod VSEG) << 2), i.e. the 64-byte segments of a row are XOR-permuted by its
  // row index; the four rows a transposing read touches then fall on disjoint bank ranges
  uint32_t vgoff[VNIW];
#pragma unroll
  for (int m = 0; m < VNIW; ++m) {
    const int P = 64 * (wid + m * NW) + lane;
    const int r = P / (D / 8), pg = P % (D / 8);
    vgoff[m] = (r * D + (pg ^ ((r & (VSEG - 1)) << 2)) * 8) * 2;
  }
  const int ragged_blk = (N % kBk) ? (N / kBk) : -1;
  const int32_t *__restrict__ cols = a.visit ? a.visit + (size_t)row * a.n_kvblk : a.col_idx + beg;

  // Key positions through the plan's table (GATHER): key position p of this head is
  // storage row kvo[p]. The tile's 64 rows come one per lane (tabv, lane r = row r); a
  // direct-load lane takes its row's entry by a wave shuffle. Each lane offset above is
  // row * 2D + column bytes, so the row part is swapped for the storage row.
  const int32_t *kvo = GATHER ? a.kv_order + (size_t)(bh % a.H) * N : nullptr;
  constexpr int RSH = D == 128 ? 8 : 7;   // log2(2D)
  auto tab_load = [&](int J) { return min(max(kvo[min(J * kBk + lane, N - 1)], 0), N - 1); };
  auto issue_g = [&](int tabv, char *kdst, char *vdst) {
#pragma unroll
    for (int m = 0; m < NIW; ++m) {
      const int i = wid + m * NW;
      if (i < NI) {
        const int src = __shfl(tabv, (int)(goff[m] >> RSH));
        const uint32_t off = ((uint32_t)src << RSH) + (goff[m] & ((1u << RSH) - 1));
        __builtin_amdgcn_global_load_lds((gvoid_t *)(reinterpret_cast<const char *>(kg) + off),
                                         (lvoid_t *)(kdst + i * 1024), 16, 0, 0);
      }
    }
#pragma unroll
    for (int m = 0; m < VNIW; ++m) {
      const int i = wid + m * NW;
      if (i < VNI) {
        const int src = __shfl(tabv, (int)(vgoff[m] >> RSH));
        const uint32_t off = ((uint32_t)src << RSH) + (vgoff[m] & ((1u << RSH) - 1));
        __builtin_amdgcn_global_load_lds((gvoid_t *)(reinterpret_cast<const char *>(vg) + off),
                                         (lvoid_t *)(vdst + i * 1024), 16, 0, 0);
      }
    }
  };

  // Full tiles load through buffer resources over this head's K and V: the lane offset
  // is the VGPR offset and the tile's byte offset the scalar one, so an issue costs no
  // per-lane address arithmetic. A head holds N * D * 2 bytes (at most 4096 blocks of 64
  // keys: 64 MiB at D = 128); the range check only guards, every full-tile offset is
  // inside it.
  const int head_bytes = N * D * 2;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)kg, (short)0, head_bytes, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)vg, (short)0, head_bytes, kRawBufferWord3);
  auto issue = [&](int J, char *kdst, char *vdst) {
    const int j0 = J * kBk;
    const char *kb = reinterpret_cast<const char *>(kg + (size_t)j0 * D);
    const char *vb = reinterpret_cast<const char *>(vg + (size_t)j0 * D);
    if (J != ragged_blk) {
      const int toff = j0 * D * 2;
#pragma unroll
      for (int m = 0; m < NIW; ++m) {
        const int i = wid + m * NW;
        if (i < NI)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lvoid_t *)(kdst + i * 1024), 16, (int)goff[m], toff, 0, 0);
      }
#pragma unroll
      for (int m = 0; m < VNIW; ++m) {
        const int i = wid + m * NW;
        if (i < VNI)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lvoid_t *)(vdst + i * 1024), 16, (int)vgoff[m], toff, 0, 0);
      }
    } else {
      // the ragged last block: rows past N reload the last valid row (in bounds, finite)
      const int last = N - 1 - j0;
#pragma unroll
      for (int m = 0; m < NIW; ++m) {
        const int i = wid + m * NW;
        if (i < NI) {
          const int p = 64 * i + lane;
          const int c = p % GR;
          const int r = min(p / GR, last);
          const uint32_t off = (r * D + (c < D / 8 ? c : 0) * 8) * 2;
          __builtin_amdgcn_global_load_lds((gvoid_t *)(kb + off), (lvoid_t *)(kdst + i * 1024), 16, 0, 0);
        }
      }
#pragma unroll
      for (int m = 0; m < VNIW; ++m) {
        const int i = wid + m * NW;
        if (i < VNI) {
          const int P = 64 * i + lane;
          const int r = P / (D / 8), pg = P % (D / 8);
          const uint32_t off = (min(r, last) * D + (pg ^ ((r & (VSEG - 1)) << 2)) * 8) * 2;
          __builtin_amdgcn_global_load_lds((gvoid_t *)(vb + off), (lvoid_t *)(vdst + i * 1024), 16, 0, 0);
        }
      }
    }
  };

  floatx16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[t][i] = 0.0f;
  float m_run = -INFINITY;  // running max, scaled logits, log2 domain
  float lsum[2] = {0.0f, 0.0f};  // this lane's part of the running sum (two chains)
  const float sl2 = a.scale_log2;
  const float lazy = a.lse ? 0.0f : kLazy;

  // per-lane LDS byte offsets. K operand: row l32, granule hf. V^T operand source: row
  // hf*4 + u/4 and channel 32t + 16*(group & 1) + 4*(u & 3) (u = lane & 15), whose 64-byte
  // segment t sits at t ^ (u/4 mod VSEG) in the swizzled row
  const int koff = l32 * ROWB + hf * 16;
  const int u = lane & 15;
  int voff[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
    voff[t] = (hf * 4 + (u >> 2)) * VROWB + ((t ^ ((u >> 2) & (VSEG - 1))) * 64) +
              (16 * ((lane >> 4) & 1) + 4 * (u & 3)) * 2;

  auto tile = [&](int J, const char *kt_s, const char *vt_s, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    floatx16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.0f;
    // the two 32-key blocks interleave, so consecutive MFMAs do not share an accumulator
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const uint4 w = *reinterpret_cast<const uint4 *>(kt_s + koff + kt * 32 * ROWB + s * 32);
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), qf[s],
                                                           sacc[kt], 0, 0, 0);
      }
    }
    if constexpr (MASK) {
      const int valid = N - J * kBk;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kt * 32 + (i / 4) * 8 + hf * 4 + (i % 4);
          if (key >= valid) sacc[kt][i] = -INFINITY;
        }
    }
    // the tile max in four independent chains of eight, then the other lane half's max by
    // v_permlane32_swap (each lane gets the pair {own, partner}; no LDS round trip)
    float mc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int kt = c >> 1, i0 = (c & 1) * 8;
      float m = sacc[kt][i0];
#pragma unroll
      for (int i = 1; i < 8; ++i) m = score_max(m, sacc[kt][i0 + i]);
      mc[c] = m;
    }
    float mx = score_max(score_max(mc[0], mc[1]), score_max(mc[2], mc[3]));
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = score_max(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float mt = mx * sl2;
    const bool need = mt > m_run + lazy;
    if (__ballot(need)) {
      const float m_new = need ? mt : m_run;
      const float corr = need ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
      lsum[0] *= corr;
      lsum[1] *= corr;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[t][i] *= corr;
      m_run = m_new;
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kt][i] = __builtin_amdgcn_exp2f(sacc[kt][i] * sl2 - m_run);
    // O^T += V^T P^T. Reduction index hf*8 + e stands for key base + (e/4)*8 + hf*4 + e%4,
    // where the S^T layout left this lane's probabilities; the V^T operand comes from two
    // transposing LDS reads of keys base + hf*4 + 0..3 and base + 8 + hf*4 + 0..3.
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kt = s / 2, i0 = (s % 2) * 8;
      const int base = kt * 32 + (s % 2) * 16;
      bf16x8_t pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sacc[kt][i0 + e];
      // the running sum takes the rounded probabilities that the MFMA multiplies
      const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2_t pp = {pb[2 * e], pb[2 * e + 1]};
        lsum[e & 1] = __builtin_amdgcn_fdot2_f32_bf16(pp, one2, lsum[e & 1], false);
      }
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const char *p0 = vt_s + voff[t] + base * VROWB;
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4_t *)(p0));
        const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4_t *)(p0 + 8 * VROWB));
        const bf16x8_t vw = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vw, pb, oacc[t], 0, 0, 0);
      }
    }
  };

  // Two tiles per trip so the buffer of each tile is fixed at compile time. Only full
  // tiles run in the loop; the ragged block, when kept, is the row's last tile and runs
  // after it with the key mask.
  // The kept-block indices run one tile ahead of the loads that use them: the index of
  // tile it + 2 is fetched while tile it computes, so issuing a tile's loads never waits
  // on a memory round trip. With GATHER the table entries of a tile are fetched one tile
  // ahead of its loads and the indices one further.
  const int n = end - beg;
  // Linear branch: the row's H_C^T (bf16 [D][D], row d = value channel) goes by direct
  // loads into the K/V buffers that the last tile does not use, while that tile computes:
  // rows 0..63 into the V buffer and the rest into the K buffer, 256-byte (2D) rows with
  // the 16-byte granule g of row d at g ^ (d mod D/8). A row that keeps every KV block
  // has an empty complement and Ol = 0.
  const bool lin_on = LIN && n < a.n_kvblk;
  constexpr int HG = D / 8;                   // 16-byte granules per H_C^T row
  constexpr int HLW = (D * D / 512) / NW;     // 1 KB loads per wave
  static_assert((D * D / 512) % NW == 0 && D * D / 512 <= 2 * HG, "H_C^T fits in a K/V buffer pair");
  // With them, one more 1 KB direct load (wave 0) brings the row's z_C and the head's alpha
  // into the K buffer past the H_C^T rows (at EXO: z_C, then alpha), so the epilogue makes
  // no global round trip of its own.
  constexpr int EXO = D == 128 ? 64 * VROWB : 0;
  static_assert(EXO + 1024 <= kBk * ROWB, "z_C and alpha fit in the K buffer");
  auto issue_hct = [&](char *kd, char *vd) {
    const char *hb = reinterpret_cast<const char *>(a.hct + (size_t)row * D * D);
#pragma unroll
    for (int m = 0; m < HLW; ++m) {
      const int i = wid + m * NW;
      const int P = 64 * i + lane;
      const int r = P / HG, pg = P % HG;
      const uint32_t off = (r * D + (pg ^ (r & (HG - 1))) * 8) * 2;
      char *dst = i < HG ? vd + i * 1024 : kd + (i - HG) * 1024;
      __builtin_amdgcn_global_load_lds((gvoid_t *)(hb + off), (lvoid_t *)dst, 16, 0, 0);
    }
    if (wid == 0) {
      // lanes 0 .. D/4-1: z_C, then D/4 lanes of alpha; lanes past 2*(D/4) repeat them
      const int idx = lane % (D / 2);
      const float *src = idx < D / 4 ? a.zc + (size_t)row * D + idx * 4
                                     : a.alpha + (size_t)((a.alpha_h0 + bh) % a.alpha_H) * D + (idx - D / 4) * 4;
      __builtin_amdgcn_global_load_lds((gvoid_t *)src, (lvoid_t *)(kd + EXO), 16, 0, 0);
    }
  };
  if (LIN ? n > 0 : true) {
    const int n_full = n - (cols[n - 1] == ragged_blk ? 1 : 0);
    const int col0 = a.visit ? vis0 : cols[0];
    int c_next = n > 1 ? (a.visit ? vis1 : cols[1]) : 0;
    int tab_next = 0;
    if constexpr (GATHER) {
      issue_g(tab_load(__builtin_amdgcn_readfirstlane(col0)), k0s, v0s);
      if (n > 1) tab_next = tab_load(__builtin_amdgcn_readfirstlane(c_next));
      c_next = n > 2 ? cols[2] : 0;
    } else {
      issue(__builtin_amdgcn_readfirstlane(col0), k0s, v0s);
    }
    // loads of tile t + 1 into (kd, vd), and the look-ahead for later tiles; after the
    // last tile's loads, the linear branch's H_C^T
    auto next = [&](int t, char *kd, char *vd) {
      if constexpr (GATHER) {
        if (t + 1 < n) issue_g(tab_next, kd, vd);
        if (t + 2 < n) tab_next = tab_load(__builtin_amdgcn_readfirstlane(c_next));
        if (t + 3 < n) c_next = cols[t + 3];
      } else {
        if (t + 1 < n) issue(__builtin_amdgcn_readfirstlane(c_next), kd, vd);
        if (t + 2 < n) c_next = cols[t + 2];
      }
      if constexpr (LIN)
        if (lin_on && t + 1 >= n) issue_hct(kd, vd);
    };
    int it = 0;
    for (; it < n_full; it += 2) {
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      __syncthreads();
      next(it, k1s, v1s);
      tile(cols[it], k0s, v0s, std::false_type{});
      if (it + 1 >= n_full) {
        ++it;
        break;
      }
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      __syncthreads();
      next(it + 1, k0s, v0s);
      tile(cols[it + 1], k1s, v1s, std::false_type{});
    }
    if (n_full < n) {
      // tile n - 1 was issued into buffer (n - 1) % 2
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      __syncthreads();
      if ((n - 1) % 2 == 0) {
        if constexpr (LIN)
          if (lin_on) issue_hct(k1s, v1s);
        tile(cols[n - 1], k0s, v0s, std::true_type{});
      } else {
        if constexpr (LIN)
          if (lin_on) issue_hct(k0s, v0s);
        tile(cols[n - 1], k1s, v1s, std::true_type{});
      }
    }
  } else if (lin_on) {
    issue_hct(k0s, v0s);   // no kept tile (LIN only): Os = 0
  }

  // epilogue: normalise (and blend), store bf16
  const float l_run = lsum[0] + lsum[1];
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if constexpr (!LIN) {
    const float inv = 1.0f / l_tot;
    if (a.q_order == nullptr) {
      // Output rows are contiguous: the wave stages its 32 x D bf16 block in the K/V
      // buffer that the row's last tile left free (no loads go there: the last tile issues
      // none), with 16-byte granule c of row r at c ^ (r mod D/8), then writes it out in
      // whole rows, 1 KB per store instruction instead of 16-byte pieces of 32 rows.
      constexpr int GPR = D / 8;               // 16-byte granules per output row
      constexpr int RPI = 64 / GPR;            // rows per store instruction
      char *fb = (n & 1) ? ((wid & 2) ? v1s : k1s) : ((wid & 2) ? v0s : k0s);
      char *ob = fb + (wid & 1) * (32 * D * 2);
      static_assert(2 * 32 * D * 2 <= kBk * VROWB, "two waves' output blocks fit in a V buffer");
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = t * 4 + g;
          *reinterpret_cast<uint2 *>(ob + l32 * (D * 2) + ((c ^ (l32 & (GPR - 1))) * 16) + hf * 8) =
              pack4(oacc[t][g * 4 + 0] * inv, oacc[t][g * 4 + 1] * inv, oacc[t][g * 4 + 2] * inv,
                    oacc[t][g * 4 + 3] * inv);
        }
      const int q0 = I * BQ + wid * 32;        // first query row of this wave
#pragma unroll
      for (int i = 0; i < 32 / RPI; ++i) {
        const int r = i * RPI + lane / GPR, c = lane % GPR;
        const uint4 w = *reinterpret_cast<const uint4 *>(ob + r * (D * 2) + ((c ^ (r & (GPR - 1))) * 16));
        if (q0 + r < N) *reinterpret_cast<uint4 *>(og + (size_t)(q0 + r) * D + c * 8) = w;
      }
      if (q_ok && a.lse && hf == 0) a.lse[(size_t)bh * N + qrow] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
      return;
    }
    if (q_ok) {
      uint16_t *orow = og + (size_t)qrow * D;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = t * 32 + g * 8 + hf * 4;
          *reinterpret_cast<uint2 *>(orow + d) =
              pack4(oacc[t][g * 4 + 0] * inv, oacc[t][g * 4 + 1] * inv, oacc[t][g * 4 + 2] * inv,
                    oacc[t][g * 4 + 3] * inv);
        }
      if (a.lse && hf == 0) a.lse[(size_t)bh * N + qrow] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
    }
    return;
  }
  const float inv = n == 0 ? 0.0f : 1.0f / l_tot;   // a row without kept tiles has Os = 0
  // Linear branch: Ol^T[d][q] = sum_c H_C^T[d][c] phi(q)[c] / (phi(q) . z_C). phi(q)
  // replaces the Q fragments, which are the B operand of this product as they were of
  // S^T = K Q^T; H_C^T rows are the A operand.
  float inv_l = 0.0f;
  if (lin_on) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      uint4 w = __builtin_bit_cast(uint4, qf[s]);
      w.x = phi2(w.x);
      w.y = phi2(w.y);
      w.z = phi2(w.z);
      w.w = phi2(w.w);
      qf[s] = __builtin_bit_cast(bf16x8_t, w);
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    const float *zc = reinterpret_cast<const float *>(((n & 1) ? k1s : k0s) + EXO);   // z_C
    float zdot = 0.0f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const uint4 w = __builtin_bit_cast(uint4, qf[s]);
      const float4 z0 = *reinterpret_cast<const float4 *>(zc + s * 16 + hf * 8);
      const float4 z1 = *reinterpret_cast<const float4 *>(zc + s * 16 + hf * 8 + 4);
      zdot += bf_lo(w.x) * z0.x + bf_hi(w.x) * z0.y + bf_lo(w.y) * z0.z + bf_hi(w.y) * z0.w +
              bf_lo(w.z) * z1.x + bf_hi(w.z) * z1.y + bf_lo(w.w) * z1.z + bf_hi(w.w) * z1.w;
    }
    const float den = zdot + __shfl_xor(zdot, 32);
    inv_l = den > 0.0f ? 1.0f / den : 0.0f;
  }
  const char *hv = (n & 1) ? v1s : v0s;   // H_C^T rows 0..63
  const char *hk = (n & 1) ? k1s : k0s;   // H_C^T rows 64..
  uint16_t *orow = og + (size_t)qrow * D;
  // With contiguous output rows the blended block is staged as in the plain epilogue, in
  // the last tile's K/V buffer: free once every wave has passed the barrier above (with
  // the linear branch) or, without it, the buffer that the last tile left unused.
  constexpr int GPR = D / 8;
  constexpr int RPI = 64 / GPR;
  const bool staged = a.q_order == nullptr;
  const int fbi = lin_on ? ((n - 1) & 1) : (n & 1);
  char *ob = (fbi ? ((wid & 2) ? v1s : k1s) : ((wid & 2) ? v0s : k0s)) + (wid & 1) * (32 * D * 2);
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    floatx16 lacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) lacc[i] = 0.0f;
    if (lin_on) {
      const int d = t * 32 + l32;
      const char *hrow = d < 64 ? hv + d * VROWB : hk + (d - 64) * VROWB;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const uint4 w = *reinterpret_cast<const uint4 *>(hrow + (((2 * s + hf) ^ (d & (HG - 1))) * 16));
        lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), qf[s], lacc, 0, 0, 0);
      }
    }
    if (q_ok) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = t * 32 + g * 8 + hf * 4;
        // O = alpha * Os + (1 - alpha) * Ol, alpha per (head, channel): from LDS when the
        // linear branch's loads brought it, from memory on a row that keeps every block
        const float4 al = lin_on
            ? *reinterpret_cast<const float4 *>(hk + EXO + D * 4 + d * 4)
            : *reinterpret_cast<const float4 *>(a.alpha + (size_t)((a.alpha_h0 + bh) % a.alpha_H) * D + d);
        const float o0 = al.x * (oacc[t][g * 4 + 0] * inv) + (1.f - al.x) * (lacc[g * 4 + 0] * inv_l);
        const float o1 = al.y * (oacc[t][g * 4 + 1] * inv) + (1.f - al.y) * (lacc[g * 4 + 1] * inv_l);
        const float o2 = al.z * (oacc[t][g * 4 + 2] * inv) + (1.f - al.z) * (lacc[g * 4 + 2] * inv_l);
        const float o3 = al.w * (oacc[t][g * 4 + 3] * inv) + (1.f - al.w) * (lacc[g * 4 + 3] * inv_l);
        if (staged) {
          const int c = t * 4 + g;
          *reinterpret_cast<uint2 *>(ob + l32 * (D * 2) + ((c ^ (l32 & (GPR - 1))) * 16) + hf * 8) =
              pack4(o0, o1, o2, o3);
        } else {
          *reinterpret_cast<uint2 *>(orow + d) = pack4(o0, o1, o2, o3);
        }
      }
    }
  }
  if (staged) {
    const int q0 = I * BQ + wid * 32;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + lane / GPR, c = lane % GPR;
      const uint4 w = *reinterpret_cast<const uint4 *>(ob + r * (D * 2) + ((c ^ (r & (GPR - 1))) * 16));
      if (q0 + r < N) *reinterpret_cast<uint4 *>(og + (size_t)(q0 + r) * D + c * 8) = w;
    }
  }
  if (q_ok && a.lse && hf == 0) a.lse[(size_t)bh * N + qrow] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
}

template <int D, bool LIN, bool GATHER>
hipError_t launch_d(const FwdArgs &a, hipStream_t s) {
  const int R = a.B * a.H * a.n_qblk;
  if (a.block_q == 128)
    sparse_fwd_bf16_kernel<D, 4, LIN, GATHER><<<R, 256, 0, s>>>(a);
  else
    sparse_fwd_bf16_kernel<D, 2, LIN, GATHER><<<R, 128, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t s) {
  const bool lin = a.alpha != nullptr;
  if (a.kv_order != nullptr)   // keys through the plan's table (no linear branch)
    return a.D == 128 ? launch_d<128, false, true>(a, s) : launch_d<64, false, true>(a, s);
  if (a.D == 128) return lin ? launch_d<128, true, false>(a, s) : launch_d<128, false, false>(a, s);
  return lin ? launch_d<64, true, false>(a, s) : launch_d<64, false, false>(a, s);
}

}  // namespace sa
