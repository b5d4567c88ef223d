// Backward of block-sparse attention for gfx950 (the pages fine-tune through the sparse
// kernel: SpargeAttention2 page, section 2; SLA2 page). For query block I with kept KV
// tiles K_I, c = 1/sqrt(D), P = exp(c * Q K^T - lse) (the forward's log-sum-exp):
//   Dv  = rowsum(dO * O)        formed by bwd_dq_kernel at row start
//   dS  = P * (dO V^T - Dv)
//   dQ  = c * dS K        over each row's kept tiles          bwd_dq_kernel (CSR)
//   dK  = c * dS^T Q,  dV = P^T dO   over each KV block's query blocks
//                                                             bwd_dkdv_kernel (CSC)
// Both gradient kernels recompute S and P; neither uses atomics, so every gradient is
// summed in one fixed order and the results are deterministic. The CSC copy of the mask
// (query blocks per KV block, ascending) is built from a column-major bitmap, whose
// bits are set in any order, with the plan's row fill kernel. The dK/dV workgroups take
// their columns in the plan's balanced work order, built from the CSC counts: a head's
// columns stay together on one XCD, and the XCDs get near-equal shares of kept tiles.
//
// MFMA layouts follow the forward kernel: 32x32x16 bf16 blocks, one wave per 32 rows of
// the output it owns; a lane holds the 32 scores of one query (dQ kernel) or one key
// (dK/dV kernel) for its half of the tile. The transposed operands (K^T for dQ, Q^T and
// dO^T for dK and dV) come from transposing LDS reads of row-major tiles, with the
// reduction index permuted as in the forward's P V product.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;
typedef __attribute__((address_space(3))) bf16x4_t lbf16x4_t;

constexpr int kVmcnt0 = 0x0F70;   // s_waitcnt: all vector-memory operations (LDS DMA included)
constexpr int kBk = 64;
constexpr float kLog2e = 1.4426950408889634f;

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

__device__ __forceinline__ float bf(uint32_t w, int hi) {
  return __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16));
}

// ---------------------------------------------------------------- Dv = rowsum(dO * O)
// ---------------------------------------------------------------- CSC of the mask
__global__ void zero_words_kernel(uint32_t *__restrict__ p, long n) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) p[i] = 0u;
}

// one thread per CSR row: set bit I of column (bh, J) for each kept J
__global__ void csc_bits_kernel(const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
                                int R, int nQ, int nKV, int nwq, uint32_t *__restrict__ tbits) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  const int bh = r / nQ, I = r - bh * nQ;
  for (int e = row_ptr[r]; e < row_ptr[r + 1]; ++e) {
    const int J = col_idx[e];
    atomicOr(&tbits[((size_t)bh * nKV + J) * nwq + (I >> 5)], 1u << (I & 31));
  }
}

__global__ void csc_count_kernel(const uint32_t *__restrict__ tbits, long C, int nwq,
                                 int32_t *__restrict__ ccount) {
  const long c = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= C) return;
  int n = 0;
  for (int w = 0; w < nwq; ++w) n += __popc(tbits[c * nwq + w]);
  ccount[c] = n;
}

// ---------------------------------------------------------------- dQ (row-major)
// occupancy as in the forward: two waves per SIMD at NW = 4; at NW = 2 LDS allows two
// workgroups per CU, one wave per SIMD
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW == 4 ? 2 : 1)))
void bwd_dq_kernel(BwdArgs a) {
  constexpr int BQ = 32 * NW;
  constexpr int GR = D / 8 + 1;             // padded rows: one extra 16-byte granule
  constexpr int ROWB = GR * 16;
  constexpr int NI = GR;                    // 1 KB direct loads per 64-row tile
  constexpr int NIW = (NI + NW - 1) / NW;
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;

  __shared__ __align__(16) char k0s[kBk * ROWB];
  __shared__ __align__(16) char v0s[kBk * ROWB];
  __shared__ __align__(16) char k1s[kBk * ROWB];
  __shared__ __align__(16) char v1s[kBk * ROWB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int rlin = xcd_remap(blockIdx.x, gridDim.x);
  const int row = a.row_order ? a.row_order[rlin] : rlin;
  const int nQ = a.n_qblk;
  const int bh = row / nQ;
  const int I = row - bh * nQ;
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const uint16_t *qg = a.q + head;
  const uint16_t *kg = a.k + head;
  const uint16_t *vg = a.v + head;
  const uint16_t *dog = a.dout + head;
  uint16_t *dqg = a.dq + head;

  const int qi = I * BQ + wid * 32 + l32;
  const bool q_ok = qi < N;
  const int beg = a.row_ptr[row];
  const int end = a.row_ptr[row + 1];
  // The row's entries of the per-head padded arrays that the dK/dV kernel reads: Dv and
  // lse*log2(e) for n < N, 0 and +inf past N (padded query rows then get P = 0 and dS = 0),
  // and the same for a row with no kept tile, whose queries no KV block visits.
  float *dv_out = a.dvec + (size_t)bh * a.NP + qi;
  float *lse2_out = a.lse2 + (size_t)bh * a.NP + qi;
  if (beg == end) {
    if (q_ok)
      for (int d = hf * (D / 2); d < (hf + 1) * (D / 2); d += 4)
        *reinterpret_cast<uint2 *>(dqg + (size_t)qi * D + d) = make_uint2(0u, 0u);
    if (hf == 0) {
      *dv_out = 0.0f;
      *lse2_out = INFINITY;
    }
    return;
  }

  bf16x8_t qf[KSTEPS], dof[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    uint4 w = make_uint4(0, 0, 0, 0), x = make_uint4(0, 0, 0, 0);
    if (q_ok) {
      w = *reinterpret_cast<const uint4 *>(qg + (size_t)qi * D + s * 16 + hf * 8);
      x = *reinterpret_cast<const uint4 *>(dog + (size_t)qi * D + s * 16 + hf * 8);
    }
    qf[s] = __builtin_bit_cast(bf16x8_t, w);
    dof[s] = __builtin_bit_cast(bf16x8_t, x);
  }
  // Dv = rowsum(dO * O): this lane's 64 channels (those of its dO fragments) in ascending
  // order, then the other half's sum from the partner lane
  float dpart = 0.0f;
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    uint4 ow = make_uint4(0, 0, 0, 0);
    if (q_ok) ow = *reinterpret_cast<const uint4 *>(a.o + head + (size_t)qi * D + s * 16 + hf * 8);
    const uint4 dw = __builtin_bit_cast(uint4, dof[s]);
    const uint32_t oa[4] = {ow.x, ow.y, ow.z, ow.w}, da[4] = {dw.x, dw.y, dw.z, dw.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      dpart = dpart + bf(oa[c], 0) * bf(da[c], 0);
      dpart = dpart + bf(oa[c], 1) * bf(da[c], 1);
    }
  }
  const float dpo = __shfl_xor(dpart, 32);
  const float dv = dpart + dpo;   // the same in both lanes: the sum commutes
  // a query past N gets lse2 = +inf, so its P (and dS) is 0
  const float lse2 = q_ok ? a.lse[(size_t)bh * N + qi] * kLog2e : INFINITY;
  if (hf == 0) {
    *dv_out = dv;
    *lse2_out = lse2;
  }
  const float sl2 = a.scale_log2;

  uint32_t goff[NIW];
#pragma unroll
  for (int m = 0; m < NIW; ++m) {
    const int p = 64 * (wid + m * NW) + lane;
    const int c = p % GR;
    goff[m] = ((p / GR) * D + (c < D / 8 ? c : 0) * 8) * 2;
  }
  const int ragged_blk = (N % kBk) ? (N / kBk) : -1;
  const int32_t *__restrict__ cols = a.col_idx + beg;

  // Full tiles load through buffer resources over this head's K and V (N * D * 2 bytes,
  // at most 64 MiB): the lane offset is the VGPR offset and the tile's byte offset the
  // scalar one, so an issue costs no per-lane address arithmetic. Every offset used is
  // inside the head; the ragged last block keeps its clamped global loads.
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)kg, (short)0, N * D * 2, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)vg, (short)0, N * D * 2, kRawBufferWord3);
  auto issue = [&](int J, char *kdst, char *vdst) {
    const int j0 = J * kBk;
    if (J != ragged_blk) {
      const int toff = j0 * D * 2;
#pragma unroll
      for (int m = 0; m < NIW; ++m) {
        const int i = wid + m * NW;
        if (i < NI) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lvoid_t *)(kdst + i * 1024), 16, (int)goff[m], toff, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lvoid_t *)(vdst + i * 1024), 16, (int)goff[m], toff, 0, 0);
        }
      }
      return;
    }
    const char *kb = reinterpret_cast<const char *>(kg + (size_t)j0 * D);
    const char *vb = reinterpret_cast<const char *>(vg + (size_t)j0 * D);
    const int last = N - 1 - j0;
#pragma unroll
    for (int m = 0; m < NIW; ++m) {
      const int i = wid + m * NW;
      if (i < NI) {
        const int p = 64 * i + lane;
        const int c = p % GR;
        const uint32_t off = (min(p / GR, last) * D + (c < D / 8 ? c : 0) * 8) * 2;
        __builtin_amdgcn_global_load_lds((gvoid_t *)(kb + off), (lvoid_t *)(kdst + i * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((gvoid_t *)(vb + off), (lvoid_t *)(vdst + i * 1024), 16, 0, 0);
      }
    }
  };

  // row reads of K and V (A operands of S^T and dP^T): row l32, granule hf
  const int koff = l32 * ROWB + hf * 16;
  // transposing reads of K for the K^T operand of dQ^T: source lane u of each 16-lane
  // group points at row hf*4 + u/4 and channel 32t + 16*(group & 1) + 4*(u & 3)
  const int u = lane & 15;
  int toff[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
    toff[t] = (hf * 4 + (u >> 2)) * ROWB + (32 * t + 16 * ((lane >> 4) & 1) + 4 * (u & 3)) * 2;

  floatx16 dqacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[t][i] = 0.0f;

  auto tile = [&](int J, const char *ks, const char *vs, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int valid = N - J * kBk;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      floatx16 sacc, dpacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sacc[i] = 0.0f;
        dpacc[i] = 0.0f;
      }
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const uint4 w = *reinterpret_cast<const uint4 *>(ks + koff + kt * 32 * ROWB + s * 32);
        const uint4 x = *reinterpret_cast<const uint4 *>(vs + koff + kt * 32 * ROWB + s * 32);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), qf[s], sacc, 0, 0, 0);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, x), dof[s], dpacc, 0, 0, 0);
      }
      // dS^T = P^T * (dP^T - Dv); lane holds keys kt*32 + (i/4)*8 + hf*4 + i%4 of query l32
      float ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kt * 32 + (i / 4) * 8 + hf * 4 + (i % 4);
        float p = __builtin_amdgcn_exp2f(sacc[i] * sl2 - lse2);
        if (MASK && key >= valid) p = 0.0f;
        ds[i] = p * (dpacc[i] - dv);
      }
      // dQ^T += K^T dS^T, two 16-key steps; reduction index hf*8 + e stands for key
      // base + (e/4)*8 + hf*4 + e%4 (the S^T layout), matched by the transposing reads
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int base = kt * 32 + h2 * 16;
        bf16x8_t pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (__bf16)ds[h2 * 8 + e];
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const char *p0 = ks + toff[t] + base * ROWB;
          const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4_t *)(p0));
          const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4_t *)(p0 + 8 * ROWB));
          const bf16x8_t kw = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          dqacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kw, pb, dqacc[t], 0, 0, 0);
        }
      }
    }
  };

  // the index of tile it + 2 loads while tile it computes (no round trip before a tile's loads)
  const int n = end - beg;
  const int n_full = n - (cols[n - 1] == ragged_blk ? 1 : 0);
  int c_next = n > 1 ? cols[1] : 0;
  issue(cols[0], k0s, v0s);
  int it = 0;
  for (; it < n_full; it += 2) {
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    if (it + 1 < n) issue(__builtin_amdgcn_readfirstlane(c_next), k1s, v1s);
    if (it + 2 < n) c_next = cols[it + 2];
    tile(cols[it], k0s, v0s, std::false_type{});
    if (it + 1 >= n_full) {
      ++it;
      break;
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    if (it + 2 < n) issue(__builtin_amdgcn_readfirstlane(c_next), k0s, v0s);
    if (it + 3 < n) c_next = cols[it + 3];
    tile(cols[it + 1], k1s, v1s, std::false_type{});
  }
  if (n_full < n) {
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    if ((n - 1) % 2 == 0)
      tile(cols[n - 1], k0s, v0s, std::true_type{});
    else
      tile(cols[n - 1], k1s, v1s, std::true_type{});
  }

  // dQ out: each wave stages its 32 x D block in the K/V buffer pair that the row's last
  // tile left free (no loads go there), 16-byte granule c of row r at c ^ (r mod D/8),
  // and writes it in whole rows, 1 KB per store instruction
  {
    constexpr int GPR = D / 8;
    constexpr int RPI = 64 / GPR;
    static_assert(2 * 32 * D * 2 <= kBk * ROWB, "two waves' blocks fit in one buffer");
    const float c = a.scale;
    char *ob = ((n & 1) ? ((wid & 2) ? v1s : k1s) : ((wid & 2) ? v0s : k0s)) + (wid & 1) * (32 * D * 2);
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int gc = t * 4 + g;
        *reinterpret_cast<uint2 *>(ob + l32 * (D * 2) + ((gc ^ (l32 & (GPR - 1))) * 16) + hf * 8) =
            pack4(dqacc[t][g * 4 + 0] * c, dqacc[t][g * 4 + 1] * c, dqacc[t][g * 4 + 2] * c,
                  dqacc[t][g * 4 + 3] * c);
      }
    const int q0 = I * BQ + wid * 32;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + lane / GPR, gc = lane % GPR;
      const uint4 w = *reinterpret_cast<const uint4 *>(ob + r * (D * 2) + ((gc ^ (r & (GPR - 1))) * 16));
      if (q0 + r < N) *reinterpret_cast<uint4 *>(dqg + (size_t)(q0 + r) * D + gc * 8) = w;
    }
  }
}

// ---------------------------------------------------------------- dK, dV (column-major)
// One workgroup of two waves per KV block (64 keys); each wave owns 32 keys. The query
// blocks that keep this KV block (the CSC list, ascending) are walked in stages of 32
// query rows. A stage's Q and dO rows and its lse*log2(e) and Dv values go HBM -> LDS by
// direct loads, double-buffered: stage s + 1 loads while stage s computes. Two stages
// take 38 KB (D = 128), so four workgroups share a CU and each SIMD runs two waves.
// Each stage contributes
//   dV^T += dO^T P,  dK^T += Q^T dS   (then dK is scaled by c).
template <int D, int BQ>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NW = 2;
  constexpr int SR = 32;                     // query rows per stage
  constexpr int SPB = BQ / SR;               // stages per query block
  constexpr int GR = D / 8 + 1;              // 16-byte granules per padded LDS row
  constexpr int ROWB = GR * 16;
  constexpr int NIQ = (SR * GR + 63) / 64;   // 1 KB direct loads per Q (or dO) tile
  constexpr int NIQW = (NIQ + NW - 1) / NW;
  constexpr int TILEB = NIQ * 1024;          // the tile's SR*ROWB bytes, then spare for the last load
  constexpr int STAGE = 2 * TILEB + 1024;    // Q, dO, lse2 (128 B), Dv (128 B), spare
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;

  __shared__ __align__(16) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int col = a.col_order[xcd_remap(blockIdx.x, gridDim.x)];
  const int nKV = a.n_kvblk;
  const int bh = col / nKV;
  const int J = col - bh * nKV;
  const int N = a.N;
  const size_t head = (size_t)bh * N * D;
  const uint16_t *qg = a.q + head;
  const uint16_t *dog = a.dout + head;
  const float *lse2g = a.lse2 + (size_t)bh * a.NP;
  const float *dvg = a.dvec + (size_t)bh * a.NP;
  const int key = J * kBk + wid * 32 + l32;
  const bool k_ok = key < N;

  bf16x8_t kf[KSTEPS], vf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    uint4 w = make_uint4(0, 0, 0, 0), x = make_uint4(0, 0, 0, 0);
    if (k_ok) {
      w = *reinterpret_cast<const uint4 *>(a.k + head + (size_t)key * D + s * 16 + hf * 8);
      x = *reinterpret_cast<const uint4 *>(a.v + head + (size_t)key * D + s * 16 + hf * 8);
    }
    kf[s] = __builtin_bit_cast(bf16x8_t, w);
    vf[s] = __builtin_bit_cast(bf16x8_t, x);
  }
  const float sl2 = a.scale_log2;

  // direct-load sources within a stage: load i fills LDS granules 64i .. 64i+63 of the
  // padded tile; lane p carries granule (row (64i+p)/GR, column (64i+p)%GR), the pad
  // column reloading column 0. Granules past the tile's SR rows land in its spare bytes
  // and read row SR - 1. Wave w issues loads w, w + NW, ... of Q and of dO.
  uint32_t toffs[NIQW];
#pragma unroll
  for (int m = 0; m < NIQW; ++m) {
    const int p = 64 * (wid + m * NW) + lane;
    const int c = p % GR;
    toffs[m] = (min(p / GR, SR - 1) * D + (c < D / 8 ? c : 0) * 8) * 2;
  }
  // the lse2 / Dv load: lanes 0..7 carry lse2, 8..15 Dv, 16..63 repeat them into the spare
  const int lv = lane & 15;
  const float *ldsrc = (lv < 8 ? lse2g : dvg) + 4 * (lv & 7);

  // whole stages load through buffer resources over this head's Q and dO (N * D * 2
  // bytes), with the stage's byte offset as the scalar offset; every offset used is
  // inside the head
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc((void *)qg, (short)0, N * D * 2, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t drs = __builtin_amdgcn_make_buffer_rsrc((void *)dog, (short)0, N * D * 2, kRawBufferWord3);
  auto issue = [&](int q0, char *buf) {
    if (q0 + SR <= N) {
      const int soff = q0 * D * 2;
#pragma unroll
      for (int m = 0; m < NIQW; ++m) {
        const int i = wid + m * NW;
        if (i < NIQ) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (lvoid_t *)(buf + i * 1024), 16, (int)toffs[m], soff, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (lvoid_t *)(buf + TILEB + i * 1024), 16, (int)toffs[m], soff, 0, 0);
        }
      }
    } else {
      // rows past N reload row N - 1 (in bounds; their lse2 is +inf, so they add nothing)
#pragma unroll
      for (int m = 0; m < NIQW; ++m) {
        const int i = wid + m * NW;
        if (i < NIQ) {
          const int p = 64 * i + lane;
          const int c = p % GR;
          const int grow = min(q0 + min(p / GR, SR - 1), N - 1);
          const size_t off = ((size_t)grow * D + (c < D / 8 ? c : 0) * 8) * 2;
          __builtin_amdgcn_global_load_lds((gvoid_t *)(reinterpret_cast<const char *>(qg) + off),
                                           (lvoid_t *)(buf + i * 1024), 16, 0, 0);
          __builtin_amdgcn_global_load_lds((gvoid_t *)(reinterpret_cast<const char *>(dog) + off),
                                           (lvoid_t *)(buf + TILEB + i * 1024), 16, 0, 0);
        }
      }
    }
    if (wid == NW - 1)   // q0 + SR <= NP: the padded arrays cover the whole stage
      __builtin_amdgcn_global_load_lds((gvoid_t *)(ldsrc + q0), (lvoid_t *)(buf + 2 * TILEB), 16, 0, 0);
  };

  const int qoff = l32 * ROWB + hf * 16;     // row reads of Q and dO (A operands of S, dP)
  const int u = lane & 15;
  int toff[DT];                              // transposing reads of Q^T and dO^T
#pragma unroll
  for (int t = 0; t < DT; ++t)
    toff[t] = (hf * 4 + (u >> 2)) * ROWB + (32 * t + 16 * ((lane >> 4) & 1) + 4 * (u & 3)) * 2;

  floatx16 dkacc[DT], dvacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dkacc[t][i] = 0.0f;
      dvacc[t][i] = 0.0f;
    }

  auto compute = [&](const char *cur) {
    const char *qs_ = cur;
    const char *dos_ = cur + TILEB;
    const float *lse_s = reinterpret_cast<const float *>(cur + 2 * TILEB);
    const float *dv_s = lse_s + SR;
#pragma unroll
    for (int qb2 = 0; qb2 < SR / 32; ++qb2) {
      floatx16 sacc, dpacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sacc[i] = 0.0f;
        dpacc[i] = 0.0f;
      }
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const uint4 w = *reinterpret_cast<const uint4 *>(qs_ + qoff + qb2 * 32 * ROWB + s * 32);
        const uint4 y = *reinterpret_cast<const uint4 *>(dos_ + qoff + qb2 * 32 * ROWB + s * 32);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), kf[s], sacc, 0, 0, 0);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, y), vf[s], dpacc, 0, 0, 0);
      }
      // lane holds queries qb2*32 + (i/4)*8 + hf*4 + i%4 of key l32
      float p[16], ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 l4 = *reinterpret_cast<const float4 *>(&lse_s[qb2 * 32 + g * 8 + hf * 4]);
        const float4 d4 = *reinterpret_cast<const float4 *>(&dv_s[qb2 * 32 + g * 8 + hf * 4]);
        const float lv4[4] = {l4.x, l4.y, l4.z, l4.w}, dvv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = g * 4 + r;
          p[i] = __builtin_amdgcn_exp2f(sacc[i] * sl2 - lv4[r]);
          ds[i] = p[i] * (dpacc[i] - dvv[r]);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the slice's two 16-query steps
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int base = qb2 * 32 + h2 * 16;
        bf16x8_t pb, sb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[e] = (__bf16)p[h2 * 8 + e];
          sb[e] = (__bf16)ds[h2 * 8 + e];
        }
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const char *p0 = dos_ + toff[t] + base * ROWB;
          const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4_t *)(p0));
          const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4_t *)(p0 + 8 * ROWB));
          dvacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7),
                                                             pb, dvacc[t], 0, 0, 0);
          const char *p1 = qs_ + toff[t] + base * ROWB;
          const bf16x4_t lo2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4_t *)(p1));
          const bf16x4_t hi2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4_t *)(p1 + 8 * ROWB));
          dkacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_shufflevector(lo2, hi2, 0, 1, 2, 3, 4, 5, 6, 7),
                                                             sb, dkacc[t], 0, 0, 0);
        }
      }
    }
  };

  // stage s covers query rows I*BQ + (s % SPB)*SR .. +SR-1 of I = row_idx[cbeg + s / SPB];
  // the block index of stage s + 2 loads while stage s computes
  const int cbeg = a.col_ptr[col], cend = a.col_ptr[col + 1];
  const int nst = (cend - cbeg) * SPB;
  if (nst > 0) {
    int i_next = nst > 1 ? a.row_idx[cbeg + 1 / SPB] : 0;
    issue(__builtin_amdgcn_readfirstlane(a.row_idx[cbeg]) * BQ, smem);
    for (int st = 0; st < nst; ++st) {
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      __syncthreads();   // stage st has landed; every wave is done with stage st - 1's buffer
      if (st + 1 < nst)
        issue(__builtin_amdgcn_readfirstlane(i_next) * BQ + ((st + 1) % SPB) * SR, smem + ((st + 1) & 1) * STAGE);
      if (st + 2 < nst) i_next = a.row_idx[cbeg + (st + 2) / SPB];
      compute(smem + (st & 1) * STAGE);
    }
  }

  // dK and dV out: once both waves are done with the stage buffers, each wave stages its
  // 32 x D blocks of dK and dV there (16-byte granule c of row r at c ^ (r mod D/8)) and
  // writes them in whole rows, 1 KB per store instruction
  {
    constexpr int GPR = D / 8;
    constexpr int RPI = 64 / GPR;
    constexpr int BLK = 32 * D * 2;            // one wave's 32 x D bf16 block
    static_assert(NW * 2 * BLK <= 2 * STAGE, "both waves' dK and dV blocks fit in the stage buffers");
    const float c = a.scale;
    __syncthreads();
    char *kb = smem + wid * (2 * BLK);
    char *vb = kb + BLK;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int gc = t * 4 + g;
        const int off = l32 * (D * 2) + ((gc ^ (l32 & (GPR - 1))) * 16) + hf * 8;
        *reinterpret_cast<uint2 *>(kb + off) = pack4(dkacc[t][g * 4 + 0] * c, dkacc[t][g * 4 + 1] * c,
                                                     dkacc[t][g * 4 + 2] * c, dkacc[t][g * 4 + 3] * c);
        *reinterpret_cast<uint2 *>(vb + off) = pack4(dvacc[t][g * 4 + 0], dvacc[t][g * 4 + 1],
                                                     dvacc[t][g * 4 + 2], dvacc[t][g * 4 + 3]);
      }
    const int k0 = J * kBk + wid * 32;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + lane / GPR, gc = lane % GPR;
      const int off = r * (D * 2) + ((gc ^ (r & (GPR - 1))) * 16);
      const uint4 wk = *reinterpret_cast<const uint4 *>(kb + off);
      const uint4 wv = *reinterpret_cast<const uint4 *>(vb + off);
      if (k0 + r < N) {
        *reinterpret_cast<uint4 *>(a.dk + head + (size_t)(k0 + r) * D + gc * 8) = wk;
        *reinterpret_cast<uint4 *>(a.dv + head + (size_t)(k0 + r) * D + gc * 8) = wv;
      }
    }
  }
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, const BwdBufs &w, hipStream_t s) {
  const int BH = a.B * a.H;
  hipError_t e;
  // CSC of the mask
  const int R = BH * a.n_qblk;
  const long C = (long)BH * a.n_kvblk;
  const long words = C * w.nwq;
  zero_words_kernel<<<(unsigned)min(65536L, (words + 255) / 256), 256, 0, s>>>(w.tbits, words);
  csc_bits_kernel<<<(unsigned)ceil_div(R, 256), 256, 0, s>>>(a.row_ptr, a.col_idx, R, a.n_qblk, a.n_kvblk,
                                                              w.nwq, w.tbits);
  csc_count_kernel<<<(unsigned)((C + 255) / 256), 256, 0, s>>>(w.tbits, C, w.nwq, w.ccount);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_scan(w.ccount, (int)C, a.col_ptr, w.cnnz, s)) != hipSuccess) return e;
  if ((e = launch_fill(w.tbits, w.nwq, a.col_ptr, (int)C, a.row_idx, s)) != hipSuccess) return e;
  // dkdv's work order: the plan's balance over the XCDs, applied to the columns (heads'
  // column runs dealt heaviest first to the least-loaded XCD, ascending within a run)
  if ((e = launch_row_order(a.col_ptr, (int)C, a.n_kvblk, a.col_order, s)) != hipSuccess) return e;
  // gradients
  if (a.D == 128) {
    if (a.block_q == 128) {
      bwd_dq_kernel<128, 4><<<R, 256, 0, s>>>(a);
      bwd_dkdv_kernel<128, 128><<<(unsigned)C, 128, 0, s>>>(a);
    } else {
      bwd_dq_kernel<128, 2><<<R, 128, 0, s>>>(a);
      bwd_dkdv_kernel<128, 64><<<(unsigned)C, 128, 0, s>>>(a);
    }
  } else {
    if (a.block_q == 128) {
      bwd_dq_kernel<64, 4><<<R, 256, 0, s>>>(a);
      bwd_dkdv_kernel<64, 128><<<(unsigned)C, 128, 0, s>>>(a);
    } else {
      bwd_dq_kernel<64, 2><<<R, 128, 0, s>>>(a);
      bwd_dkdv_kernel<64, 64><<<(unsigned)C, 128, 0, s>>>(a);
    }
  }
  return hipGetLastError();
}

}  // namespace sa
