// Ground-truth tile heatmap for gfx950 (Veda page, section 2.1: the reference mask max-pools
// the full attention matrix over query x key tiles; section 2.3: it is built in two
// passes). Pass 1 is the forward kernel on an all-ones plan, which yields each query's
// log-sum-exp. This kernel is pass 2: for every query block I (one CSR row) and every KV
// block J it forms S = Q K^T / sqrt(D) on the MFMA units again, turns it into
// probabilities p = exp(s - lse_i), and writes
//   tile_max[I, J]  = max over the tile of p,
//   tile_mass[I, J] = (1 / |I|) * sum over the tile of p.
// Queries past N and keys past N contribute p = 0. Every reduction has a fixed order
// (in-lane, lane halves, a 32-lane butterfly, then the waves in index order), so the
// output is deterministic.
//
// One workgroup per row, one wave per 32 queries. K tiles go from HBM straight into LDS
// (buffer_load_dwordx4 ... lds for whole tiles, global_load_lds_dwordx4 for the ragged
// last one), padded by one 16-byte granule per row, double-buffered with
// one barrier per tile, as in the forward kernel. Each wave's per-tile partials go to a
// 128-slot LDS ring; wave 0 folds a group of 64 tiles into the outputs while the next
// group runs.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

constexpr int kVmcnt0 = 0x0F70;   // s_waitcnt: all vector-memory operations (LDS DMA included)
constexpr int kBk = 64;           // keys per tile
constexpr int kRing = 128;        // per-wave partial slots: two groups of 64 tiles

__device__ __forceinline__ int xcd_remap(int b, int G) {
  const int q = G / 8;
  if (b >= q * 8) return b;
  return (b % 8) * q + b / 8;
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void tile_stats_bf16_kernel(const uint16_t *__restrict__ q,
                                                                  const uint16_t *__restrict__ k,
                                                                  const float *__restrict__ lse, int N,
                                                                  int n_qblk, int n_kvblk, float sl2,
                                                                  float *__restrict__ tmax,
                                                                  float *__restrict__ tmass) {
  constexpr int BQ = 32 * NW;
  constexpr int GR = D / 8 + 1;             // 16-byte granules per padded LDS row
  constexpr int ROWB = GR * 16;
  constexpr int NI = GR;                    // 1 KB direct loads per 64-row tile
  constexpr int NIW = (NI + NW - 1) / NW;
  constexpr int KSTEPS = D / 16;

  __shared__ __align__(16) char k0s[kBk * ROWB];
  __shared__ __align__(16) char k1s[kBk * ROWB];
  __shared__ float ring_max[NW][kRing];
  __shared__ float ring_sum[NW][kRing];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int row = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = row / n_qblk;
  const int I = row - bh * n_qblk;
  const size_t head = (size_t)bh * N * D;
  const uint16_t *qg = q + head;
  const uint16_t *kg = k + head;
  const int qi = I * BQ + wid * 32 + l32;
  const bool q_ok = qi < N;
  const int n_i = min(BQ, N - I * BQ);
  const float inv_ni = 1.0f / (float)n_i;
  // p = exp2(s * sl2 - lse * log2(e)); a query past N gets +inf here, so p = 0
  const float lse2 = q_ok ? lse[(size_t)bh * N + qi] * 1.4426950408889634f : INFINITY;

  bf16x8_t qf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (q_ok) w = *reinterpret_cast<const uint4 *>(qg + (size_t)qi * D + s * 16 + hf * 8);
    qf[s] = __builtin_bit_cast(bf16x8_t, w);
  }

  uint32_t goff[NIW];
#pragma unroll
  for (int m = 0; m < NIW; ++m) {
    const int p = 64 * (wid + m * NW) + lane;
    const int c = p % GR;
    goff[m] = ((p / GR) * D + (c < D / 8 ? c : 0) * 8) * 2;
  }
  const int ragged_blk = (N % kBk) ? (N / kBk) : -1;
  // whole tiles load through a buffer resource over this head's K (N * D * 2 bytes, at
  // most 64 MiB) with the tile's byte offset as the scalar offset; every offset used is
  // inside the head
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)kg, (short)0, N * D * 2, kRawBufferWord3);
  auto issue = [&](int J, char *kdst) {
    const char *kb = reinterpret_cast<const char *>(kg + (size_t)J * kBk * D);
    if (J != ragged_blk) {
      const int toff = J * kBk * D * 2;
#pragma unroll
      for (int m = 0; m < NIW; ++m) {
        const int i = wid + m * NW;
        if (i < NI)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lvoid_t *)(kdst + i * 1024), 16, (int)goff[m], toff, 0, 0);
      }
    } else {
      // rows past N reload the last valid row (in bounds, finite; masked below)
      const int last = N - 1 - J * kBk;
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
    }
  };

  const int koff = l32 * ROWB + hf * 16;
  // wave 0 folds the partials of tiles [j0, j0 + n) (ring slots j0 mod 128 ...) into
  // the outputs, waves in index order
  auto fold = [&](int j0, int n) {
    if (wid == 0 && lane < n) {
      const int slot = (j0 + lane) & (kRing - 1);
      float mx = ring_max[0][slot];
      float sm = ring_sum[0][slot];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        mx = score_max(mx, ring_max[w][slot]);
        sm = sm + ring_sum[w][slot];
      }
      const size_t o = (size_t)row * n_kvblk + j0 + lane;
      if (tmax) tmax[o] = mx;
      if (tmass) tmass[o] = sm * inv_ni;
    }
  };

  auto tile = [&](int J, const char *kt_s) {
    floatx16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.0f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const uint4 w = *reinterpret_cast<const uint4 *>(kt_s + koff + kt * 32 * ROWB + s * 32);
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), qf[s],
                                                           sacc[kt], 0, 0, 0);
      }
    }
    // lane (l32, hf) holds the scores of query l32 for keys kt*32 + (i/4)*8 + hf*4 + i%4
    const int valid = N - J * kBk;
    float mx = 0.0f, sm = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kt * 32 + (i / 4) * 8 + hf * 4 + (i % 4);
        const float p = key < valid ? __builtin_amdgcn_exp2f(sacc[kt][i] * sl2 - lse2) : 0.0f;
        mx = score_max(mx, p);
        sm = sm + p;
      }
    mx = score_max(mx, __shfl_xor(mx, 32));
    sm = sm + __shfl_xor(sm, 32);
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      mx = score_max(mx, __shfl_xor(mx, o));
      sm = sm + __shfl_xor(sm, o);
    }
    if (lane == 0) {
      ring_max[wid][J & (kRing - 1)] = mx;
      ring_sum[wid][J & (kRing - 1)] = sm;
    }
  };

  issue(0, k0s);
  for (int J = 0; J < n_kvblk; J += 2) {
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    if (J + 1 < n_kvblk) issue(J + 1, k1s);
    // the group of 64 tiles before this one is complete in the ring
    if (J > 0 && (J & 63) == 0) fold(J - 64, 64);
    tile(J, k0s);
    if (J + 1 >= n_kvblk) break;
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    if (J + 2 < n_kvblk) issue(J + 2, k0s);
    tile(J + 1, k1s);
  }
  __syncthreads();
  const int last_group = (n_kvblk - 1) & ~63;
  fold(last_group, n_kvblk - last_group);
}

template <int D>
hipError_t launch_d(const void *q, const void *k, const float *lse, int BH, int N, int bq,
                    int nQ, int nKV, float sl2, float *tmax, float *tmass, hipStream_t s) {
  const int R = BH * nQ;
  if (bq == 128)
    tile_stats_bf16_kernel<D, 4><<<R, 256, 0, s>>>((const uint16_t *)q, (const uint16_t *)k, lse, N, nQ,
                                                   nKV, sl2, tmax, tmass);
  else
    tile_stats_bf16_kernel<D, 2><<<R, 128, 0, s>>>((const uint16_t *)q, (const uint16_t *)k, lse, N, nQ,
                                                   nKV, sl2, tmax, tmass);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile_stats(const void *q, const void *k, const float *lse, int BH, int H, int N, int D,
                             int bq, int nQ, int nKV, float sl2, float *tmax, float *tmass, hipStream_t s) {
  (void)H;   // rows are (batch, head) major; the kernel needs no head count of its own
  if (D == 128) return launch_d<128>(q, k, lse, BH, N, bq, nQ, nKV, sl2, tmax, tmass, s);
  return launch_d<64>(q, k, lse, BH, N, bq, nQ, nKV, sl2, tmax, tmass, s);
}

}  // namespace sa
