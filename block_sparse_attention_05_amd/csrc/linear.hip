// Linear-attention branch for gfx950 (SALAD page, section 2.1: a linear-attention branch
// in parallel with the sparse one, O(N) in the sequence length; SLA2 page: the blocks the
// router drops feed the linear branch). phi = elu + 1 on the raw q and k.
//
// For query block I with kept KV blocks K_I and complement C_I:
//   Ol_i = phi(q_i)^T H_C / phi(q_i)^T z_C,  H_C = sum_{j in C_I} phi(k_j) v_j^T,
//                                           z_C = sum_{j in C_I} phi(k_j).
// H_C is a D x D matrix shared by the whole query block, so the apply step forms it once
// per block and multiplies it by the block's phi(Q): the per-tile work is one D x D x 64
// product instead of two BQ x 64 x D ones.
//   linear_kv_kernel     per (head, token chunk): partial H and z with bf16 MFMA and fp32
//                        accumulation; also writes phi(K) in bf16 with zero pad rows;
//   linear_reduce_kernel sums the chunk partials in chunk order (deterministic) into the
//                        per-head totals H and z (fp32);
//   linear_apply_kernel  per query block: when it keeps at most half of the KV blocks,
//                        H_C and z_C are the totals minus the kept tiles' sums (formed in
//                        fp32, then rounded once); otherwise the complement tiles are
//                        summed directly, so no sum is formed as a small difference of
//                        large ones. A query block that keeps every KV block gets Ol = 0.
//                        Ol is written in fp32 for the blend O = alpha*Os + (1 - alpha)*Ol
//                        in the attention epilogue.

#include <hip/hip_runtime.h>
#include <stdint.h>

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

constexpr int kTile = 64;       // tokens per KV tile
constexpr int kChunk = 512;     // tokens per prepass workgroup
constexpr int kVmcnt0 = 0x0F70; // s_waitcnt: all vector-memory operations (LDS DMA included)

__device__ __forceinline__ float bf(uint32_t w, int hi) {
  return __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16));
}
__device__ __forceinline__ float phi(float x) { return x > 0.0f ? x + 1.0f : __expf(x); }
__device__ __forceinline__ uint32_t rne_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack2(float a, float b) { return rne_bf16(a) | (rne_bf16(b) << 16); }

// phi of 8 bf16 values packed in a uint4, re-rounded to bf16
__device__ __forceinline__ uint4 phi8(uint4 w) {
  uint4 r;
  r.x = pack2(phi(bf(w.x, 0)), phi(bf(w.x, 1)));
  r.y = pack2(phi(bf(w.y, 0)), phi(bf(w.y, 1)));
  r.z = pack2(phi(bf(w.z, 0)), phi(bf(w.z, 1)));
  r.w = pack2(phi(bf(w.w, 0)), phi(bf(w.w, 1)));
  return r;
}

// Transposed store of a 4-row x 8-column bf16 chunk: row r of the chunk becomes column r
// of 8 rows of the transposed tile (stride ld elements).
__device__ __forceinline__ void store_t4x8(uint16_t *dst, int ld, const uint4 (&v)[4]) {
  const uint32_t *w0 = reinterpret_cast<const uint32_t *>(&v[0]);
  const uint32_t *w1 = reinterpret_cast<const uint32_t *>(&v[1]);
  const uint32_t *w2 = reinterpret_cast<const uint32_t *>(&v[2]);
  const uint32_t *w3 = reinterpret_cast<const uint32_t *>(&v[3]);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    uint2 lo, hi;
    lo.x = (w0[m] & 0xffffu) | (w1[m] << 16);
    lo.y = (w2[m] & 0xffffu) | (w3[m] << 16);
    hi.x = (w0[m] >> 16) | (w1[m] & 0xffff0000u);
    hi.y = (w2[m] >> 16) | (w3[m] & 0xffff0000u);
    *reinterpret_cast<uint2 *>(dst + (2 * m) * ld) = lo;
    *reinterpret_cast<uint2 *>(dst + (2 * m + 1) * ld) = hi;
  }
}

// ---------------------------------------------------------------- prepass
// grid (chunks, B*H), 256 threads. Wave w owns the (c-block, d-block) pairs
// p = w, w+4, ... of the (D/32)^2 32x32 blocks of H.
template <int D>
__global__ __launch_bounds__(256) void linear_kv_kernel(const uint16_t *__restrict__ k,
                                                        const uint16_t *__restrict__ v, int N,
                                                        float *__restrict__ partial,
                                                        uint16_t *__restrict__ phik, int n_pad) {
  constexpr int ROW = kTile + 8;                 // transposed tile row stride (elements)
  constexpr int NB = (D / 32) * (D / 32);        // 32x32 blocks of H
  constexpr int PER_WAVE = NB / 4 > 0 ? NB / 4 : 1;
  constexpr int CHUNKS_T = (kTile / 4) * (D / 8);  // 4x8 chunks per tile
  __shared__ __align__(16) uint16_t kt[D * ROW];   // phi(K)^T [c][token]
  __shared__ __align__(16) uint16_t vt[D * ROW];   // V^T      [d][token]

  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  const size_t head = (size_t)bh * N * D;
  const uint16_t *kg = k + head;
  const uint16_t *vg = v + head;
  uint16_t *pk = phik + (size_t)bh * n_pad * D;
  const int t_beg = chunk * kChunk;
  const int t_end = min(N, t_beg + kChunk);

  floatx16 acc[PER_WAVE];
#pragma unroll
  for (int p = 0; p < PER_WAVE; ++p)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[p][i] = 0.0f;
  float zacc = 0.0f;  // thread tid < D: sum of phi(k)[tid] over the chunk

  for (int t0 = t_beg; t0 < t_end; t0 += kTile) {
    __syncthreads();
    for (int c = tid; c < CHUNKS_T; c += 256) {
      const int rg = c / (D / 8), col = (c % (D / 8)) * 8;
      uint4 kr[4], vr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = t0 + rg * 4 + r;
        if (tok < t_end) {
          kr[r] = phi8(*reinterpret_cast<const uint4 *>(kg + (size_t)tok * D + col));
          vr[r] = *reinterpret_cast<const uint4 *>(vg + (size_t)tok * D + col);
        } else {
          kr[r] = make_uint4(0, 0, 0, 0);  // tokens past the end contribute nothing
          vr[r] = make_uint4(0, 0, 0, 0);
        }
        // t0 + 64 <= n_pad, so the pad rows past N are written here as zeros
        *reinterpret_cast<uint4 *>(pk + (size_t)tok * D + col) = kr[r];
      }
      store_t4x8(&kt[col * ROW + rg * 4], ROW, kr);
      store_t4x8(&vt[col * ROW + rg * 4], ROW, vr);
    }
    __syncthreads();
    if (tid < D) {
      const uint16_t *row = &kt[tid * ROW];
#pragma unroll 8
      for (int j = 0; j < kTile; ++j) zacc += __uint_as_float(((uint32_t)row[j]) << 16);
    }
#pragma unroll
    for (int p = 0; p < PER_WAVE; ++p) {
      const int blk = wid + 4 * p;
      if (blk < NB) {
        const int cb = blk / (D / 32), db = blk % (D / 32);
#pragma unroll
        for (int s = 0; s < kTile / 16; ++s) {
          const uint4 a = *reinterpret_cast<const uint4 *>(&kt[(cb * 32 + l32) * ROW + s * 16 + hf * 8]);
          const uint4 b = *reinterpret_cast<const uint4 *>(&vt[(db * 32 + l32) * ROW + s * 16 + hf * 8]);
          acc[p] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                           __builtin_bit_cast(bf16x8_t, b), acc[p], 0, 0, 0);
        }
      }
    }
  }
  // partial layout per (bh, chunk): H [c][d] then z [c]
  float *out = partial + ((size_t)bh * gridDim.x + chunk) * (size_t)(D * D + D);
#pragma unroll
  for (int p = 0; p < PER_WAVE; ++p) {
    const int blk = wid + 4 * p;
    if (blk < NB) {
      const int cb = blk / (D / 32), db = blk % (D / 32);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = cb * 32 + (i / 4) * 8 + hf * 4 + (i % 4);
        const int d = db * 32 + l32;
        out[c * D + d] = acc[p][i];
      }
    }
  }
  if (tid < D) out[D * D + tid] = zacc;
}

// Sums the chunk partials in chunk order into H and z (fp32).
__global__ __launch_bounds__(256) void linear_reduce_kernel(const float *__restrict__ partial,
                                                            int chunks, int D,
                                                            float *__restrict__ h,
                                                            float *__restrict__ z) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int per = D * D + D;
  if (e >= per) return;
  const float *p = partial + (size_t)bh * chunks * per + e;
  float s = 0.0f;
  for (int c = 0; c < chunks; ++c) s += p[(size_t)c * per];
  if (e < D * D)
    h[(size_t)bh * D * D + e] = s;
  else
    z[(size_t)bh * D + (e - D * D)] = s;
}

// ---------------------------------------------------------------- apply
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

// One workgroup of four waves per query block (CSR row); QG = block_q / 32 query groups.
// The four waves split the (D/32)^2 blocks of the row's running sum H_S[c][d] in a 2x2
// grid: wave w takes c-blocks of half w >> 1 and d-blocks of half w & 1. phi(K) and V
// tiles go from HBM straight into LDS, both with their 64-byte row segments XOR-swizzled
// by row, and both MFMA operands come from transposing LDS reads (8 keys of one channel
// per lane). At the end the waves stage H_C^T (bf16) in LDS and each wave multiplies it
// by the phi(Q) of its query group.
template <int D, int QG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void linear_apply_kernel(FwdArgs a, LinearBufs lb) {
  constexpr int NW = 4;
  constexpr int BQ = 32 * QG;
  constexpr int VROWB = D * 2;              // bytes per tile row (unpadded)
  constexpr int TB = kTile * VROWB;         // bytes per tile
  constexpr int VNI = D / 8;                // 1 KB direct loads per tile
  constexpr int VNIW = (VNI + NW - 1) / NW;
  constexpr int VSEG = D / 32;              // 64-byte segments per row (swizzle range)
  constexpr int CB = D / 32;                // 32-channel blocks
  constexpr int WC = CB / 2;                // c-blocks per wave
  constexpr int WD = CB / 2;                // d-blocks per wave
  constexpr int KSTEPS = D / 16;
  constexpr int HG = D / 8;                 // 16-byte granules per staged H_C^T row
  constexpr int DBW = CB * QG / NW;         // d-blocks per wave in the final product
  constexpr int kMaxList = kMaxKvBlocks / 2;
  static_assert(WC >= 1 && DBW >= 1, "shape");

  __shared__ __align__(16) char k0s[TB];
  __shared__ __align__(16) char v0s[TB];
  __shared__ __align__(16) char k1s[TB];
  __shared__ __align__(16) char v1s[TB];
  __shared__ int tiles[kMaxList];                    // the tile list of this row
  __shared__ uint32_t keptbits[kMaxKvBlocks / 32];
  __shared__ float zs[2 * D];                        // z partials, then z_C

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wid >= 0 && wid < NW);
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int cp = wid >> 1, dp = wid & 1;

  const int row = xcd_remap(blockIdx.x, gridDim.x);
  const int nQ = a.n_qblk, nKV = a.n_kvblk, N = a.N;
  const int bh = row / nQ;
  const int I = row - bh * nQ;
  const size_t head = (size_t)bh * N * D;
  const uint16_t *qg = reinterpret_cast<const uint16_t *>(a.q) + head;
  const uint16_t *vg = reinterpret_cast<const uint16_t *>(a.v) + head;
  const uint16_t *pk = lb.phik + (size_t)bh * lb.n_pad * D;
  float *olg = lb.ol + head;

  const int beg = a.row_ptr[row], end = a.row_ptr[row + 1];
  const int kept = end - beg;
  if (kept == nKV) {  // empty complement: Ol = 0
    for (int e = tid * 4; e < BQ * D; e += NW * 64 * 4) {
      const int qi = I * BQ + e / D;
      if (qi < N) *reinterpret_cast<float4 *>(olg + (size_t)qi * D + e % D) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  const bool subtract = kept <= nKV / 2;

  // raw q of this wave's final-product query group, loaded early
  const int g = wid % QG;
  const int qi = I * BQ + g * 32 + l32;   // query position (Ol is written by position)
  const bool q_ok = qi < N;
  int qrow = qi;                          // storage row of q
  if (a.q_order && q_ok) qrow = min(max(a.q_order[(size_t)(bh % a.H) * N + qi], 0), N - 1);
  uint4 qraw[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    qraw[s] = make_uint4(0, 0, 0, 0);
    if (q_ok) qraw[s] = *reinterpret_cast<const uint4 *>(qg + (size_t)qrow * D + s * 16 + hf * 8);
  }

  // tile list: the kept tiles (subtract) or the complement (direct sum); both fit in
  // nKV / 2 entries
  int ntiles;
  if (subtract) {
    for (int i = tid; i < kept; i += NW * 64) tiles[i] = a.col_idx[beg + i];
    ntiles = kept;
  } else {
    for (int w = tid; w < (nKV + 31) / 32; w += NW * 64) keptbits[w] = 0u;
    __syncthreads();
    for (int i = tid; i < kept; i += NW * 64) {
      const int J = a.col_idx[beg + i];
      atomicOr(&keptbits[J >> 5], 1u << (J & 31));
    }
    __syncthreads();
    if (wid == 0) {  // compaction in ascending order
      int base = 0;
      for (int J0 = 0; J0 < nKV; J0 += 64) {
        const int J = J0 + lane;
        const bool take = J < nKV && !((keptbits[J >> 5] >> (J & 31)) & 1u);
        const unsigned long long m = __ballot(take);
        const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
        if (take) tiles[pos] = J;
        base += __popcll(m);
      }
    }
    ntiles = nKV - kept;
  }
  __syncthreads();

  // Direct loads: LDS granule (row r, physical granule pg) holds logical granule
  // pg ^ ((r mod VSEG) << 2); load i of a tile fills granules 64i .. 64i+63.
  uint32_t goff[VNIW];
#pragma unroll
  for (int m = 0; m < VNIW; ++m) {
    const int P = 64 * (wid + m * NW) + lane;
    const int r = P / (D / 8), pg = P % (D / 8);
    goff[m] = (r * D + (pg ^ ((r & (VSEG - 1)) << 2)) * 8) * 2;
  }
  const int ragged_blk = (N % kTile) ? (N / kTile) : -1;

  auto issue = [&](int J, char *kdst, char *vdst) {
    const char *kb = reinterpret_cast<const char *>(pk + (size_t)J * kTile * D);
    const char *vb = reinterpret_cast<const char *>(vg + (size_t)J * kTile * D);
    // phi(K) rows past N are zero pad rows of the prepass buffer
#pragma unroll
    for (int m = 0; m < VNIW; ++m) {
      const int i = wid + m * NW;
      if (i < VNI)
        __builtin_amdgcn_global_load_lds((gvoid_t *)(kb + goff[m]), (lvoid_t *)(kdst + i * 1024), 16, 0, 0);
    }
    if (J != ragged_blk) {
#pragma unroll
      for (int m = 0; m < VNIW; ++m) {
        const int i = wid + m * NW;
        if (i < VNI)
          __builtin_amdgcn_global_load_lds((gvoid_t *)(vb + goff[m]), (lvoid_t *)(vdst + i * 1024), 16, 0, 0);
      }
    } else {
      // V rows past N reload the last valid row (finite; their phi(k) is zero)
      const int last = N - 1 - J * kTile;
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

  // Transposing-read offsets: for channel block t the lane reads keys hf*4 + 0..3 (+8 for
  // the second read) of channel 32t + l32; its source row hf*4 + u/4 (u = lane & 15) has
  // segment t at t ^ (u/4 mod VSEG).
  const int u = lane & 15;
  const int rbase = (hf * 4 + (u >> 2)) * VROWB + (16 * ((lane >> 4) & 1) + 4 * (u & 3)) * 2;
  int koff[WC], voff[WD];
#pragma unroll
  for (int x = 0; x < WC; ++x) koff[x] = rbase + (((cp * WC + x) ^ ((u >> 2) & (VSEG - 1))) * 64);
#pragma unroll
  for (int y = 0; y < WD; ++y) voff[y] = rbase + (((dp * WD + y) ^ ((u >> 2) & (VSEG - 1))) * 64);

  floatx16 hacc[WC][WD];
#pragma unroll
  for (int x = 0; x < WC; ++x)
#pragma unroll
    for (int y = 0; y < WD; ++y)
#pragma unroll
      for (int i = 0; i < 16; ++i) hacc[x][y][i] = 0.0f;
  float zacc[WC];
#pragma unroll
  for (int x = 0; x < WC; ++x) zacc[x] = 0.0f;
  const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};

  // H_S[c][d] += sum over the tile's keys of phi(K)[key][c] V[key][d]; the MFMA reduction
  // index hf*8 + e stands for key 16s + hf*4 + e (e < 4) or 16s + 8 + hf*4 + e - 4, the
  // same for both operands.
  auto tile = [&](const char *ks, const char *vs) {
#pragma unroll
    for (int s = 0; s < kTile / 16; ++s) {
      const int base = 16 * s * VROWB;
      bf16x8_t av[WC], bv[WD];
#pragma unroll
      for (int x = 0; x < WC; ++x) {
        const char *p0 = ks + koff[x] + base;
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4_t *)(p0));
        const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4_t *)(p0 + 8 * VROWB));
        av[x] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int y = 0; y < WD; ++y) {
        const char *p0 = vs + voff[y] + base;
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4_t *)(p0));
        const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4_t *)(p0 + 8 * VROWB));
        bv[y] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      // the two waves sharing a c-half split the z sum by k-step parity
      if ((s & 1) == dp) {
#pragma unroll
        for (int x = 0; x < WC; ++x)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2_t pp = {av[x][2 * e], av[x][2 * e + 1]};
            zacc[x] = __builtin_amdgcn_fdot2_f32_bf16(pp, one2, zacc[x], false);
          }
      }
#pragma unroll
      for (int x = 0; x < WC; ++x)
#pragma unroll
        for (int y = 0; y < WD; ++y)
          hacc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[x], bv[y], hacc[x][y], 0, 0, 0);
    }
  };

  if (ntiles > 0) {
    issue(tiles[0], k0s, v0s);
    for (int it = 0; it < ntiles; it += 2) {
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      __syncthreads();
      if (it + 1 < ntiles) issue(tiles[it + 1], k1s, v1s);
      tile(k0s, v0s);
      if (it + 1 >= ntiles) break;
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      __syncthreads();
      if (it + 2 < ntiles) issue(tiles[it + 2], k0s, v0s);
      tile(k1s, v1s);
    }
  }

  // z partials: this wave's k-step half, both lane halves
#pragma unroll
  for (int x = 0; x < WC; ++x) {
    const float zz = zacc[x] + __shfl_xor(zacc[x], 32);
    if (hf == 0) zs[dp * D + (cp * WC + x) * 32 + l32] = zz;
  }
  // H_C = H - H_S (subtract) or H_S, in fp32, then rounded once to bf16
  const float *hg = lb.h + (size_t)bh * D * D;
  float hc[WC][WD][16];
#pragma unroll
  for (int x = 0; x < WC; ++x)
#pragma unroll
    for (int y = 0; y < WD; ++y)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = (cp * WC + x) * 32 + (i / 4) * 8 + hf * 4 + (i % 4);
        const int d = (dp * WD + y) * 32 + l32;
        hc[x][y][i] = subtract ? hg[(size_t)c * D + d] - hacc[x][y][i] : hacc[x][y][i];
      }
  __syncthreads();  // every wave is done with the tile buffers
  // staged H_C^T: row d (64 rows per buffer, k0s then v0s), 16-byte granule c/8 at
  // physical granule (c/8) ^ (d mod HG)
#pragma unroll
  for (int x = 0; x < WC; ++x)
#pragma unroll
    for (int y = 0; y < WD; ++y) {
      const int d = (dp * WD + y) * 32 + l32;
      char *hrow = (d < 64 ? k0s : v0s) + (d & 63) * VROWB;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int gr = (cp * WC + x) * 4 + q4;
        *reinterpret_cast<uint2 *>(hrow + ((gr ^ (d & (HG - 1))) * 16) + hf * 8) =
            pack4(hc[x][y][q4 * 4 + 0], hc[x][y][q4 * 4 + 1], hc[x][y][q4 * 4 + 2], hc[x][y][q4 * 4 + 3]);
      }
    }
  __syncthreads();
  if (tid < D) {
    const float zsum = zs[tid] + zs[D + tid];
    zs[tid] = subtract ? lb.z[(size_t)bh * D + tid] - zsum : zsum;
  }
  __syncthreads();

  // Ol^T[d][q] = sum_c H_C^T[d][c] phi(q)[c] / (phi(q) . z_C)
  bf16x8_t pf[KSTEPS];
  float zdot = 0.0f;
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const uint4 w = q_ok ? phi8(qraw[s]) : make_uint4(0, 0, 0, 0);
    pf[s] = __builtin_bit_cast(bf16x8_t, w);
    const float4 z0 = *reinterpret_cast<const float4 *>(&zs[s * 16 + hf * 8]);
    const float4 z1 = *reinterpret_cast<const float4 *>(&zs[s * 16 + hf * 8 + 4]);
    zdot += bf(w.x, 0) * z0.x + bf(w.x, 1) * z0.y + bf(w.y, 0) * z0.z + bf(w.y, 1) * z0.w +
            bf(w.z, 0) * z1.x + bf(w.z, 1) * z1.y + bf(w.w, 0) * z1.z + bf(w.w, 1) * z1.w;
  }
  const float den = zdot + __shfl_xor(zdot, 32);
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  const int dstart = (wid / QG) * DBW;
#pragma unroll
  for (int t = 0; t < DBW; ++t) {
    const int d = (dstart + t) * 32 + l32;
    const char *hrow = (d < 64 ? k0s : v0s) + (d & 63) * VROWB;
    floatx16 oacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[i] = 0.0f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const uint4 w = *reinterpret_cast<const uint4 *>(hrow + (((2 * s + hf) ^ (d & (HG - 1))) * 16));
      oacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), pf[s], oacc, 0, 0, 0);
    }
    if (q_ok) {
      float *orow = olg + (size_t)qi * D;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dd = (dstart + t) * 32 + g4 * 8 + hf * 4;
        *reinterpret_cast<float4 *>(orow + dd) =
            make_float4(oacc[g4 * 4 + 0] * inv, oacc[g4 * 4 + 1] * inv, oacc[g4 * 4 + 2] * inv,
                        oacc[g4 * 4 + 3] * inv);
      }
    }
  }
}

}  // namespace

int linear_prepass_chunks(int N) { return ceil_div(N, kChunk); }

hipError_t launch_linear_prepass(const void *k, const void *v, sa_dtype dt, int BH, int N, int D,
                                 const LinearBufs &lb, hipStream_t s) {
  if (dt != SA_BF16) return hipErrorNotSupported;
  dim3 grid(lb.chunks, BH);
  if (D == 128)
    linear_kv_kernel<128><<<grid, 256, 0, s>>>((const uint16_t *)k, (const uint16_t *)v, N, lb.partial,
                                              lb.phik, lb.n_pad);
  else
    linear_kv_kernel<64><<<grid, 256, 0, s>>>((const uint16_t *)k, (const uint16_t *)v, N, lb.partial,
                                             lb.phik, lb.n_pad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(ceil_div(D * D + D, 256), BH);
  linear_reduce_kernel<<<g2, 256, 0, s>>>(lb.partial, lb.chunks, D, lb.h, lb.z);
  return hipGetLastError();
}

hipError_t launch_linear_apply(const FwdArgs &a, const LinearBufs &lb, hipStream_t s) {
  const int R = a.B * a.H * a.n_qblk;
  if (a.D == 128) {
    if (a.block_q == 128)
      linear_apply_kernel<128, 4><<<R, 256, 0, s>>>(a, lb);
    else
      linear_apply_kernel<128, 2><<<R, 256, 0, s>>>(a, lb);
  } else {
    if (a.block_q == 128)
      linear_apply_kernel<64, 4><<<R, 256, 0, s>>>(a, lb);
    else
      linear_apply_kernel<64, 2><<<R, 256, 0, s>>>(a, lb);
  }
  return hipGetLastError();
}

}  // namespace sa
