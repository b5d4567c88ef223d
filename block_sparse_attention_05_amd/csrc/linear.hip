// Linear-attention branch for gfx950 (SALAD page, section 2.1: a linear-attention branch
// in parallel with the sparse one, O(N) in the sequence length; SLA2 page: the blocks the
// router drops feed the linear branch). phi = elu + 1 on the raw q and k.
//
// For query block I with kept KV blocks K_I and complement C_I:
//   Ol_i = phi(q_i)^T sum_{j in C_I} phi(k_j) v_j^T / phi(q_i)^T sum_{j in C_I} phi(k_j)
// Two kernels and a reduction:
//   linear_kv_kernel     per (head, token chunk): partial H^T = sum_j v_j phi(k_j)^T and
//                        z = sum_j phi(k_j), with bf16 MFMA and fp32 accumulation;
//   linear_reduce_kernel sums the chunk partials in chunk order (deterministic) into
//                        H^T (bf16, the MFMA operand of the apply step) and z (fp32);
//   linear_apply_kernel  per query block: when it keeps at most half of the KV blocks,
//                        the complement sums are the totals minus the kept tiles'
//                        terms; otherwise the complement tiles are summed directly, so
//                        no sum is formed as a small difference of large ones. A query
//                        block that keeps every KV block gets Ol = 0. The kept-tile or
//                        complement-tile terms use the same 64-key tile loop as the
//                        attention kernel, with A = phi(Q) phi(K)^T in place of the
//                        softmax probabilities. Ol is written in fp32 for the blend
//                        O = alpha*Os + (1 - alpha)*Ol in the attention epilogue.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 64;       // tokens per KV tile
constexpr int kChunk = 512;     // tokens per prepass workgroup

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
// grid (chunks, B*H), 256 threads. Wave w owns the (d-block, c-block) pairs
// p = w, w+4, ... of the (D/32)^2 32x32 blocks of H^T.
template <int D>
__global__ __launch_bounds__(256) void linear_kv_kernel(const uint16_t *__restrict__ k,
                                                        const uint16_t *__restrict__ v, int N,
                                                        float *__restrict__ partial) {
  constexpr int ROW = kTile + 8;                 // transposed tile row stride (elements)
  constexpr int NB = (D / 32) * (D / 32);        // 32x32 blocks of H^T
  constexpr int PER_WAVE = NB / 4 > 0 ? NB / 4 : 1;
  constexpr int CHUNKS_T = (kTile / 4) * (D / 8);  // 4x8 chunks per tile
  __shared__ __align__(16) uint16_t kt[D * ROW];   // phi(K)^T [c][token]
  __shared__ __align__(16) uint16_t vt[D * ROW];   // V^T      [d][token]

  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  const size_t head = (size_t)bh * N * D;
  const uint16_t *kg = k + head;
  const uint16_t *vg = v + head;
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
        const int db = blk / (D / 32), cb = blk % (D / 32);
#pragma unroll
        for (int s = 0; s < kTile / 16; ++s) {
          const uint4 a = *reinterpret_cast<const uint4 *>(&vt[(db * 32 + l32) * ROW + s * 16 + hf * 8]);
          const uint4 b = *reinterpret_cast<const uint4 *>(&kt[(cb * 32 + l32) * ROW + s * 16 + hf * 8]);
          acc[p] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                           __builtin_bit_cast(bf16x8_t, b), acc[p], 0, 0, 0);
        }
      }
    }
  }
  // partial layout per (bh, chunk): H^T [D][D] then z [D]
  float *out = partial + ((size_t)bh * gridDim.x + chunk) * (size_t)(D * D + D);
#pragma unroll
  for (int p = 0; p < PER_WAVE; ++p) {
    const int blk = wid + 4 * p;
    if (blk < NB) {
      const int db = blk / (D / 32), cb = blk % (D / 32);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = db * 32 + (i / 4) * 8 + hf * 4 + (i % 4);
        const int c = cb * 32 + l32;
        out[d * D + c] = acc[p][i];
      }
    }
  }
  if (tid < D) out[D * D + tid] = zacc;
}

// Sums the chunk partials in chunk order; H^T goes out as bf16, z as fp32.
__global__ __launch_bounds__(256) void linear_reduce_kernel(const float *__restrict__ partial,
                                                            int chunks, int D,
                                                            uint16_t *__restrict__ ht,
                                                            float *__restrict__ z) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int per = D * D + D;
  if (e >= per) return;
  const float *p = partial + (size_t)bh * chunks * per + e;
  float s = 0.0f;
  for (int c = 0; c < chunks; ++c) s += p[(size_t)c * per];
  if (e < D * D)
    ht[(size_t)bh * D * D + e] = (uint16_t)rne_bf16(s);
  else
    z[(size_t)bh * D + (e - D * D)] = s;
}

// ---------------------------------------------------------------- apply
__device__ __forceinline__ int xcd_remap(int b, int G) {
  const int q = G / 8;
  if (b >= q * 8) return b;
  return (b % 8) * q + b / 8;
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void linear_apply_kernel(FwdArgs a, const uint16_t *__restrict__ ht,
                                                               const float *__restrict__ zt,
                                                               float *__restrict__ ol) {
  constexpr int NT = 64 * NW;
  constexpr int BQ = 32 * NW;
  constexpr int KROW = D + 8;
  constexpr int VROW = kTile + 4;
  constexpr int KCH = kTile * D / 8;
  constexpr int KPT = (KCH + NT - 1) / NT;
  constexpr int VCH = (kTile / 4) * (D / 8);
  constexpr int VPT = (VCH + NT - 1) / NT;
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;

  __shared__ __align__(16) uint16_t ks[kTile * KROW];   // phi(K) tile, row-major
  __shared__ __align__(16) uint16_t vt[D * VROW];       // V^T tile
  __shared__ int tiles[kMaxKvBlocks];                   // the tile list of this row
  __shared__ uint32_t keptbits[kMaxKvBlocks / 32];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  const int row = xcd_remap(blockIdx.x, gridDim.x);
  const int nQ = a.n_qblk, nKV = a.n_kvblk, N = a.N;
  const int bh = row / nQ;
  const int I = row - bh * nQ;
  const size_t head = (size_t)bh * N * D;
  const uint16_t *qg = reinterpret_cast<const uint16_t *>(a.q) + head;
  const uint16_t *kg = reinterpret_cast<const uint16_t *>(a.k) + head;
  const uint16_t *vg = reinterpret_cast<const uint16_t *>(a.v) + head;
  float *olg = ol + head;
  const int qi = I * BQ + wid * 32 + l32;
  const bool q_ok = qi < N;

  const int beg = a.row_ptr[row], end = a.row_ptr[row + 1];
  const int kept = end - beg;
  if (kept == nKV) {  // empty complement
    if (q_ok)
      for (int d = hf * (D / 2); d < (hf + 1) * (D / 2); d += 4)
        *reinterpret_cast<float4 *>(olg + (size_t)qi * D + d) = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  const bool subtract = kept <= nKV / 2;

  // tile list: the kept tiles (subtract) or the complement (direct sum)
  int ntiles;
  if (subtract) {
    for (int i = tid; i < kept; i += NT) tiles[i] = a.col_idx[beg + i];
    ntiles = kept;
  } else {
    for (int w = tid; w < (nKV + 31) / 32; w += NT) keptbits[w] = 0u;
    __syncthreads();
    for (int i = tid; i < kept; i += NT) {
      const int J = a.col_idx[beg + i];
      atomicOr(&keptbits[J >> 5], 1u << (J & 31));
    }
    __syncthreads();
    // wave 0 compacts the complement in ascending order
    if (wid == 0) {
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

  // phi(Q) operand: lane holds phi(q)[s*16 + hf*8 + 0..7] for each MFMA step
  bf16x8_t qf[KSTEPS];
  float zdot = 0.0f;
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (q_ok) w = phi8(*reinterpret_cast<const uint4 *>(qg + (size_t)qi * D + s * 16 + hf * 8));
    qf[s] = __builtin_bit_cast(bf16x8_t, w);
    const float4 z0 = *reinterpret_cast<const float4 *>(zt + (size_t)bh * D + s * 16 + hf * 8);
    const float4 z1 = *reinterpret_cast<const float4 *>(zt + (size_t)bh * D + s * 16 + hf * 8 + 4);
    zdot += bf(w.x, 0) * z0.x + bf(w.x, 1) * z0.y + bf(w.y, 0) * z0.z + bf(w.y, 1) * z0.w +
            bf(w.z, 0) * z1.x + bf(w.z, 1) * z1.y + bf(w.w, 0) * z1.z + bf(w.w, 1) * z1.w;
  }
  zdot += __shfl_xor(zdot, 32);

  uint4 kr[KPT];
  uint4 vr[VPT][4];
  auto load_tile = [&](int J) {
    const int j0 = J * kTile;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int c = tid + u * NT;
      kr[u] = make_uint4(0, 0, 0, 0);
      if (c < KCH) {
        const int r = c / (D / 8), col = (c % (D / 8)) * 8;
        if (j0 + r < N) kr[u] = *reinterpret_cast<const uint4 *>(kg + (size_t)(j0 + r) * D + col);
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int c = tid + u * NT;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) vr[u][rr] = make_uint4(0, 0, 0, 0);
      if (c < VCH) {
        const int kgp = c / (D / 8), col = (c % (D / 8)) * 8;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int r = j0 + kgp * 4 + rr;
          if (r < N) vr[u][rr] = *reinterpret_cast<const uint4 *>(vg + (size_t)r * D + col);
        }
      }
    }
  };

  floatx16 nacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) nacc[t][i] = 0.0f;
  float dpart = 0.0f;

  if (ntiles > 0) load_tile(tiles[0]);
  for (int it = 0; it < ntiles; ++it) {
    const int J = tiles[it];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int c = tid + u * NT;
      if (c < KCH) {
        const int r = c / (D / 8), col = (c % (D / 8)) * 8;
        *reinterpret_cast<uint4 *>(&ks[r * KROW + col]) = phi8(kr[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int c = tid + u * NT;
      if (c < VCH) {
        const int kgp = c / (D / 8), col = (c % (D / 8)) * 8;
        store_t4x8(&vt[col * VROW + kgp * 4], VROW, vr[u]);
      }
    }
    __syncthreads();
    if (it + 1 < ntiles) load_tile(tiles[it + 1]);

    // A^T = phi(K) phi(Q)^T
    floatx16 sacc[2];
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kt2][i] = 0.0f;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const uint4 w = *reinterpret_cast<const uint4 *>(&ks[(kt2 * 32 + l32) * KROW + s * 16 + hf * 8]);
        sacc[kt2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), qf[s],
                                                            sacc[kt2], 0, 0, 0);
      }
    }
    const int j0 = J * kTile;
#pragma unroll
    for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kt2 * 32 + (i / 4) * 8 + hf * 4 + (i % 4);
        if (j0 + key >= N) sacc[kt2][i] = 0.0f;   // phi(0) = 1 on zero padding: mask it
        dpart += sacc[kt2][i];
      }
    // N^T += V^T A^T (same reduction-index permutation as the attention kernel)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kt2 = s / 2, i0 = (s % 2) * 8;
      const int base = kt2 * 32 + (s % 2) * 16;
      uint4 pw;
      pw.x = pack2(sacc[kt2][i0 + 0], sacc[kt2][i0 + 1]);
      pw.y = pack2(sacc[kt2][i0 + 2], sacc[kt2][i0 + 3]);
      pw.z = pack2(sacc[kt2][i0 + 4], sacc[kt2][i0 + 5]);
      pw.w = pack2(sacc[kt2][i0 + 6], sacc[kt2][i0 + 7]);
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const uint16_t *vrow = &vt[(t * 32 + l32) * VROW + base + hf * 4];
        const uint2 v0 = *reinterpret_cast<const uint2 *>(vrow);
        const uint2 v1 = *reinterpret_cast<const uint2 *>(vrow + 8);
        const uint4 vw = make_uint4(v0.x, v0.y, v1.x, v1.y);
        nacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vw), pb,
                                                          nacc[t], 0, 0, 0);
      }
    }
  }
  float den = dpart + __shfl_xor(dpart, 32);

  if (subtract) {
    // totals: (H^T phi(Q)^T) in the same layout, z . phi(q)
    const uint16_t *hg = ht + (size_t)bh * D * D;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      floatx16 hacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) hacc[i] = 0.0f;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const uint4 w = *reinterpret_cast<const uint4 *>(hg + (size_t)(t * 32 + l32) * D + s * 16 + hf * 8);
        hacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), qf[s], hacc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) nacc[t][i] = hacc[i] - nacc[t][i];
    }
    den = zdot - den;
  }
  if (q_ok) {
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    float *orow = olg + (size_t)qi * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = t * 32 + g * 8 + hf * 4;
        *reinterpret_cast<float4 *>(orow + d) =
            make_float4(nacc[t][g * 4 + 0] * inv, nacc[t][g * 4 + 1] * inv, nacc[t][g * 4 + 2] * inv,
                        nacc[t][g * 4 + 3] * inv);
      }
  }
}

}  // namespace

int linear_prepass_chunks(int N) { return ceil_div(N, kChunk); }

hipError_t launch_linear_prepass(const void *k, const void *v, sa_dtype dt, int BH, int N, int D,
                                 float *partial, int n_chunks, uint16_t *lin_ht, float *lin_z,
                                 hipStream_t s) {
  if (dt != SA_BF16) return hipErrorNotSupported;
  dim3 grid(n_chunks, BH);
  if (D == 128)
    linear_kv_kernel<128><<<grid, 256, 0, s>>>((const uint16_t *)k, (const uint16_t *)v, N, partial);
  else
    linear_kv_kernel<64><<<grid, 256, 0, s>>>((const uint16_t *)k, (const uint16_t *)v, N, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(ceil_div(D * D + D, 256), BH);
  linear_reduce_kernel<<<g2, 256, 0, s>>>(partial, n_chunks, D, lin_ht, lin_z);
  return hipGetLastError();
}

hipError_t launch_linear_apply(const FwdArgs &a, const uint16_t *lin_ht, const float *lin_z, float *ol,
                               hipStream_t s) {
  const int R = a.B * a.H * a.n_qblk;
  if (a.D == 128) {
    if (a.block_q == 128)
      linear_apply_kernel<128, 4><<<R, 256, 0, s>>>(a, lin_ht, lin_z, ol);
    else
      linear_apply_kernel<128, 2><<<R, 128, 0, s>>>(a, lin_ht, lin_z, ol);
  } else {
    if (a.block_q == 128)
      linear_apply_kernel<64, 4><<<R, 256, 0, s>>>(a, lin_ht, lin_z, ol);
    else
      linear_apply_kernel<64, 2><<<R, 128, 0, s>>>(a, lin_ht, lin_z, ol);
  }
  return hipGetLastError();
}

}  // namespace sa
