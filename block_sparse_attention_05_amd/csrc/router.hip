// Block-mask router for gfx950: mean pooling, pooled block scores, the hybrid
// top-k / top-p selection and the CSR build.
//
// The mask must be exactly reproducible, so every fp32 operation here is a separately
// rounded IEEE operation in one fixed order (this file is compiled with contraction
// off and the pragma below repeats it):
//   pool    acc = 0, acc += x_t over the block's tokens in ascending order, mean =
//           acc / count (correctly rounded division); a ragged last block averages its
//           real tokens.
//   score   acc = 0, acc += qbar[d]*kbar[d] for d ascending (product rounded first),
//           S = acc * fp32(1/sqrt(D)).
//   order   scores descending, ties to the lower block index (-0 equals +0).
//   softmax e_J = exp_sa(S_J - S_max) with the own exp below; Z = pairwise tree sum of
//           e_J in block order (adjacent pairs, zero padding to a power of two).
//   top-p   thr = fp32(p) * Z; running sum in score order, one add at a time; m_p is
//           the first prefix length whose sum reaches thr (every block when p >= 1 or
//           no prefix reaches thr).
//   union   both rules are prefixes of the same order, so a row keeps the first
//           max(m_k, m_p) blocks of it (SpargeAttention2 page, section 2(1)).
// Pooling per block and per head follows the SLA2 page, router item 1.

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include "sa_internal.h"

#pragma clang fp contract(off)

namespace sa {
namespace {

// ---------------------------------------------------------------- fp32 exp
// exp(x) for x <= 0 from rounded fp32 operations only: Cody-Waite reduction with ln 2 =
// C1 + C2 (C1 has 16 significant bits so n*C1 is exact), a degree-7 Taylor polynomial
// in Horner form on |r| <= ln(2)/2, and exact scaling by 2^n. Arguments below -86
// return 0, so every nonzero result is a normal number.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2Hi = 0.693145751953125f;
constexpr float kLn2Lo = (float)(0.6931471805599453094 - 0.693145751953125);
constexpr float kC0 = 1.0f;
constexpr float kC1 = 1.0f;
constexpr float kC2 = (float)(1.0 / 2.0);
constexpr float kC3 = (float)(1.0 / 6.0);
constexpr float kC4 = (float)(1.0 / 24.0);
constexpr float kC5 = (float)(1.0 / 120.0);
constexpr float kC6 = (float)(1.0 / 720.0);
constexpr float kC7 = (float)(1.0 / 5040.0);

__device__ __forceinline__ float exp_sa(float x) {
  if (!(x >= -86.0f)) return 0.0f;
  const float n = __builtin_rintf(x * kLog2e);
  const float r = (x - n * kLn2Hi) - n * kLn2Lo;
  float p = kC7;
  p = p * r + kC6;
  p = p * r + kC5;
  p = p * r + kC4;
  p = p * r + kC3;
  p = p * r + kC2;
  p = p * r + kC1;
  p = p * r + kC0;
  return __builtin_ldexpf(p, (int)n);
}


// ---------------------------------------------------------------- pooling
// One thread owns 8 channels of one block and walks its tokens in order; D/8 threads
// cover a block row, so each token row is read as contiguous 16-byte pieces.
// With ORD, block positions are mapped to storage rows through a per-head table (clamped
// into [0, N)); the sum still runs over the block's positions in ascending order.
template <typename T, int D, bool ORD>
__global__ __launch_bounds__(256) void pool_kernel(const T *__restrict__ x, int H, int N, int bs,
                                                   int nblk, long total_blocks,
                                                   const int32_t *__restrict__ order,
                                                   float *__restrict__ out) {
  constexpr int kTpb = D / 8;
  constexpr int kBlocksPerWg = 256 / kTpb;
  const int sub = threadIdx.x / kTpb;
  const int lane = threadIdx.x % kTpb;
  const long g = (long)blockIdx.x * kBlocksPerWg + sub;
  // with a table, this workgroup's row indices are staged in LDS first (one coalesced
  // load), so the row loads below do not each wait for their own index
  __shared__ int ordbuf[ORD ? kBlocksPerWg * 128 : 1];
  if constexpr (ORD) {
    for (int e = threadIdx.x; e < kBlocksPerWg * bs; e += 256) {
      const int sb = e / bs, t = e - sb * bs;
      const long g2 = (long)blockIdx.x * kBlocksPerWg + sb;
      if (g2 < total_blocks) {
        const long bh2 = g2 / nblk;
        const int t2 = (int)(g2 % nblk) * bs + t;
        if (t2 < N) ordbuf[e] = min(max(order[(size_t)(bh2 % H) * N + t2], 0), N - 1);
      }
    }
    __syncthreads();
  }
  if (g >= total_blocks) return;
  const long bh = g / nblk;
  const int I = (int)(g % nblk);
  const int t0 = I * bs;
  const int cnt = min(bs, N - t0);
  const T *p = x + ((size_t)bh * N + t0) * D + lane * 8;
  const T *base = x + (size_t)bh * N * D + lane * 8;
  const int *ord = ORD ? ordbuf + sub * bs : nullptr;
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
  // 8 row loads in flight, then their adds in row order (the sum stays sequential)
  auto row = [&](int t) -> const T * {
    if constexpr (ORD) return base + (size_t)ord[t] * D;
    return p + (size_t)t * D;
  };
  auto add_row = [&](const T *rp) {
    if constexpr (sizeof(T) == 2) {
      const uint4 w = *reinterpret_cast<const uint4 *>(rp);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[2 * c] = acc[2 * c] + __uint_as_float(ws[c] << 16);
        acc[2 * c + 1] = acc[2 * c + 1] + __uint_as_float(ws[c] & 0xffff0000u);
      }
    } else {
      const float4 a = *reinterpret_cast<const float4 *>(rp);
      const float4 b = *reinterpret_cast<const float4 *>(rp + 4);
      acc[0] = acc[0] + a.x; acc[1] = acc[1] + a.y; acc[2] = acc[2] + a.z; acc[3] = acc[3] + a.w;
      acc[4] = acc[4] + b.x; acc[5] = acc[5] + b.y; acc[6] = acc[6] + b.z; acc[7] = acc[7] + b.w;
    }
  };
  int t = 0;
  for (; t + 8 <= cnt; t += 8) {
    if constexpr (sizeof(T) == 2) {
      uint4 w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = *reinterpret_cast<const uint4 *>(row(t + u));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[2 * c] = acc[2 * c] + __uint_as_float(ws[c] << 16);
          acc[2 * c + 1] = acc[2 * c + 1] + __uint_as_float(ws[c] & 0xffff0000u);
        }
      }
    } else {
      float4 a[8], b[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        a[u] = *reinterpret_cast<const float4 *>(row(t + u));
        b[u] = *reinterpret_cast<const float4 *>(row(t + u) + 4);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc[0] = acc[0] + a[u].x; acc[1] = acc[1] + a[u].y; acc[2] = acc[2] + a[u].z; acc[3] = acc[3] + a[u].w;
        acc[4] = acc[4] + b[u].x; acc[5] = acc[5] + b[u].y; acc[6] = acc[6] + b[u].z; acc[7] = acc[7] + b[u].w;
      }
    }
  }
  for (; t < cnt; ++t) add_row(row(t));
  const float fc = (float)cnt;
  float *o = out + (size_t)g * D + lane * 8;
  float4 r0 = make_float4(acc[0] / fc, acc[1] / fc, acc[2] / fc, acc[3] / fc);
  float4 r1 = make_float4(acc[4] / fc, acc[5] / fc, acc[6] / fc, acc[7] / fc);
  *reinterpret_cast<float4 *>(o) = r0;
  *reinterpret_cast<float4 *>(o + 4) = r1;
}

// The same sums for bf16 rows in raster order (no table) with a register footprint of at
// most 32: two rows in flight per thread and 32-bit byte offsets from one base (tensors
// under 4 GiB). With enough workgroups it matches the wide kernel's bandwidth with a
// quarter of its registers.
template <int D>
__global__ __launch_bounds__(256) void pool_lean_kernel(const uint16_t *__restrict__ x, int N, int bs,
                                                        int nblk, long total_blocks,
                                                        float *__restrict__ out) {
  constexpr int kTpb = D / 8;
  constexpr int kBlocksPerWg = 256 / kTpb;
  constexpr int kInFlight = 2;
  const int sub = threadIdx.x / kTpb;
  const int lane = threadIdx.x % kTpb;
  const long g = (long)blockIdx.x * kBlocksPerWg + sub;
  if (g >= total_blocks) return;
  const long bh = g / nblk;
  const int I = (int)(g % nblk);
  const int t0 = I * bs;
  const int cnt = min(bs, N - t0);
  const char *base = reinterpret_cast<const char *>(x);
  uint32_t off = (uint32_t)((((size_t)bh * N + t0) * D + lane * 8) * 2);
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
  auto add = [&](const uint4 &w) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      acc[2 * c] = acc[2 * c] + __uint_as_float(ws[c] << 16);
      acc[2 * c + 1] = acc[2 * c + 1] + __uint_as_float(ws[c] & 0xffff0000u);
    }
  };
  int t = 0;
  for (; t + kInFlight <= cnt; t += kInFlight) {
    uint4 w[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) w[u] = *reinterpret_cast<const uint4 *>(base + off + u * D * 2);
    off += kInFlight * D * 2;
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) add(w[u]);
  }
  for (; t < cnt; ++t) {
    add(*reinterpret_cast<const uint4 *>(base + off));
    off += D * 2;
  }
  const float fc = (float)cnt;
  float *o = out + (size_t)g * D + lane * 8;
  *reinterpret_cast<float4 *>(o) = make_float4(acc[0] / fc, acc[1] / fc, acc[2] / fc, acc[3] / fc);
  *reinterpret_cast<float4 *>(o + 4) = make_float4(acc[4] / fc, acc[5] / fc, acc[6] / fc, acc[7] / fc);
}

// ---------------------------------------------------------------- scores
// S[bh, I, J] for a 64 x 64 tile per workgroup; each thread keeps one running sum per
// output of a 4 x 4 patch, adding the rounded products in ascending d. Thread (ti, tj)
// owns query rows 4 ti .. 4 ti + 3 and key columns tj, tj + 16, tj + 32, tj + 48, so a
// wave owns 16 consecutive query rows and skips its products when all of them lie past
// nQ. Chunks of 32 channels are staged row-major in LDS by 16-byte copies; the row pitch
// of 36 floats puts the rows one read touches on distinct banks (4 query rows 4 apart,
// 16 consecutive key rows).
constexpr int kSt = 64;    // tile edge
constexpr int kSd = 32;    // d chunk staged in LDS
constexpr int kSp = 36;    // LDS row pitch (floats)

__global__ __launch_bounds__(256) void scores_kernel(const float *__restrict__ qbar,
                                                     const float *__restrict__ kbar, int nQ,
                                                     int nKV, int D, float c,
                                                     float *__restrict__ S) {
  __shared__ __align__(16) float qs[kSt][kSp];
  __shared__ __align__(16) float ks[kSt][kSp];
  const int bh = blockIdx.z;
  const int i0 = blockIdx.y * kSt;
  const int j0 = blockIdx.x * kSt;
  const int tid = threadIdx.x;
  const int ti = tid / 16, tj = tid % 16;
  const bool live = i0 + 16 * (tid >> 6) < nQ;   // wave-uniform: some row of this wave exists
  const float *qb = qbar + (size_t)bh * nQ * D;
  const float *kb = kbar + (size_t)bh * nKV * D;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;
  for (int d0 = 0; d0 < D; d0 += kSd) {
    // 64 rows x 8 float4 per matrix: two of each per thread
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int e = tid + 256 * m;
      const int r = e / (kSd / 4), c4 = e % (kSd / 4);
      float4 qv = make_float4(0.0f, 0.0f, 0.0f, 0.0f), kv = qv;
      if (i0 + r < nQ) qv = __ldg(reinterpret_cast<const float4 *>(qb + (size_t)(i0 + r) * D + d0 + c4 * 4));
      if (j0 + r < nKV) kv = __ldg(reinterpret_cast<const float4 *>(kb + (size_t)(j0 + r) * D + d0 + c4 * 4));
      *reinterpret_cast<float4 *>(&qs[r][c4 * 4]) = qv;
      *reinterpret_cast<float4 *>(&ks[r][c4 * 4]) = kv;
    }
    __syncthreads();
    if (live) {
#pragma unroll 2
      for (int g = 0; g < kSd / 4; ++g) {
        float qv[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float4 w = *reinterpret_cast<const float4 *>(&qs[ti * 4 + a][g * 4]);
          qv[a][0] = w.x; qv[a][1] = w.y; qv[a][2] = w.z; qv[a][3] = w.w;
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float4 w = *reinterpret_cast<const float4 *>(&ks[tj + 16 * b][g * 4]);
          const float kk[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
              const float prod = qv[a][e] * kk[e];
              acc[a][b] = acc[a][b] + prod;
            }
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int I = i0 + ti * 4 + a;
    if (I >= nQ) continue;
    float *row = S + ((size_t)bh * nQ + I) * nKV;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int J = j0 + tj + 16 * b;
      if (J < nKV) row[J] = acc[a][b] * c;
    }
  }
}

// ---------------------------------------------------------------- selection
__device__ __forceinline__ uint32_t desc_order_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 sorts with +0
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;  // ascending in this value = descending in f
}

// the score a desc_order_bits key was made from (-0 comes back as +0, which exp_sa and
// every comparison here treat alike)
__device__ __forceinline__ float desc_order_value(uint32_t b) {
  const uint32_t asc = ~b;
  return __uint_as_float((asc & 0x80000000u) ? (asc & 0x7fffffffu) : ~asc);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Adjacent-pair tree across the 64 lanes: after the step with stride s, every lane holds
// the sum of its aligned group of 2s chunks, which is the next level of the tree.
__device__ __forceinline__ float wave_tree_sum(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float w = __shfl_xor(v, o);
    v = v + w;
  }
  return v;
}

constexpr int kCandCap = 512;   // largest candidate set ranked without the full sort

// One workgroup per row. Thread t owns blocks [t*ITEMS, (t+1)*ITEMS), so the in-thread
// tree and the lane butterfly together form one adjacent-pair tree over 256*ITEMS
// leaves; leaves past nKV are zero, which leaves the sum of a power-of-two prefix
// unchanged.
//
// Only the first max(m_k, m_p) blocks of the score order matter, so the row is not
// sorted in full when a small candidate set provably contains them: with e_J binned by
// exponent, the bins from the top down to bin b hold the blocks with e >= 2^(b-127),
// which is a top set of the score order (exp_sa is monotone, so equal scores share a
// bin). Each bin also sums its e_J in 2^-40 fixed point (integer adds: exact and
// order-free; truncation keeps it a lower bound). The first such set with at least m_k
// blocks whose mass bound exceeds thr by 2^-10 (more than the relative error of any fp32
// running sum over at most kCandCap terms) contains the top-p crossing. Its blocks are
// ranked by counting, then scanned exactly as the full sort would be. Rows whose set is
// larger than kCandCap take the full bitonic sort.
//
// The kept blocks also leave the kernel in score order (descending, ties to the lower
// index), the order in which the forward kernels visit them: the row's slots of S are
// read once at the start, so their first `count` entries are then overwritten with the
// block indices (int32). A ragged last block, when kept, is moved to the end of the list,
// so only a row's last tile ever carries the key mask. The forward's running max then
// settles on the first tiles, and few later tiles rescale the output.
template <int ITEMS>
__global__ __launch_bounds__(256) void select_kernel(float *S, int nKV, int ragged_last,
                                                     int m_k, float p, int p_all,
                                                     uint32_t *__restrict__ bitmap,
                                                     int nwords, int32_t *__restrict__ counts) {
  constexpr int P = 256 * ITEMS;
  // the full sort's keys and the candidate path's buffers are never live together (the
  // sort starts after the candidate path's last barrier), so they share one LDS region;
  // with that, six rows fit on a CU at ITEMS = 8
  constexpr int kCandBytes = kCandCap * (8 + 8 + 4);
  constexpr int kPool = P * 8 > kCandBytes ? P * 8 : kCandBytes;
  __shared__ __align__(16) char pool[kPool];
  uint64_t *keys = reinterpret_cast<uint64_t *>(pool);
  uint64_t *cand = reinterpret_cast<uint64_t *>(pool);
  uint64_t *csort = cand + kCandCap;
  float *cev = reinterpret_cast<float *>(csort + kCandCap);
  // e_J by block index in LDS up to 8 items per thread; beyond that (more than 2,048
  // blocks) e is recomputed from the sort keys instead, which saves 16 KB and lets four
  // rows share a CU instead of three
  constexpr bool kEvLds = ITEMS <= 8;
  __shared__ float ev[kEvLds ? P : 1];
  __shared__ uint32_t bits[P / 32];   // nwords <= P / 32
  __shared__ int hist[128];
  __shared__ unsigned long long hmass[128];   // per-bin sum of e in 2^-40 fixed point
  __shared__ float red[4];
  __shared__ int sh_count, sh_ncand, sh_bstar, sh_pos, sh_rag;

  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const float *s = S + (size_t)row * nKV;
  float *ord = S + (size_t)row * nKV;   // takes int32 block indices (bit patterns)

  // list[0, count): kept keys in score order -> ord, ragged block last. Called after a
  // barrier that follows the last read of s.
  auto write_order = [&](const uint64_t *list, int count) {
    if (tid == 0) sh_rag = -1;
    __syncthreads();
    if (ragged_last)
      for (int r = tid; r < count; r += 256)
        if ((int)(uint32_t)list[r] == nKV - 1) sh_rag = r;
    __syncthreads();
    const int rag = sh_rag;
    for (int r = tid; r < count; r += 256)
      if (r != rag) ord[r - (rag >= 0 && r > rag ? 1 : 0)] = __int_as_float((int)(uint32_t)list[r]);
    if (rag >= 0 && tid == 0) ord[count - 1] = __int_as_float(nKV - 1);
  };

  float sv[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int J = tid * ITEMS + i;
    sv[i] = (J < nKV) ? s[J] : -INFINITY;
  }
  for (int w = tid; w < nwords; w += 256) bits[w] = 0u;
  if (tid < 128) {
    hist[tid] = 0;
    hmass[tid] = 0ull;
  }

  // row maximum (exact in any order)
  float m = sv[0];
#pragma unroll
  for (int i = 1; i < ITEMS; ++i) m = fmaxf(m, sv[i]);
  m = wave_max(m);
  if (lane == 0) red[wid] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();

  // e_J, the keys, and the in-thread part of the tree
  float tr[ITEMS];
  float ee[ITEMS];   // this thread's e values when they are not kept in LDS
  uint64_t kv[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int J = tid * ITEMS + i;
    const bool ok = J < nKV;
    const float e = ok ? exp_sa(sv[i] - m) : 0.0f;
    tr[i] = e;
    if constexpr (kEvLds) ev[tid * ITEMS + i] = e;
    else ee[i] = e;
    kv[i] = ok ? (((uint64_t)desc_order_bits(sv[i]) << 32) | (uint32_t)J) : ~0ull;
    if (ok) {
      const int b = __float_as_uint(e) >> 23;
      atomicAdd(&hist[b], 1);
      atomicAdd(&hmass[b], (unsigned long long)(e * 0x1p40f));
    }
  }
#pragma unroll
  for (int w = ITEMS; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; ++i) tr[i] = tr[2 * i] + tr[2 * i + 1];
  float z = wave_tree_sum(tr[0]);
  if (lane == 0) red[wid] = z;
  __syncthreads();
  z = (red[0] + red[1]) + (red[2] + red[3]);
  const float thr = p * z;

  if (p_all || m_k >= nKV) {
    // every block is kept (visited in index order; the ragged block is last anyway)
    for (int w = tid; w < nwords; w += 256) {
      const int rem = nKV - 32 * w;
      bitmap[(size_t)row * nwords + w] = rem >= 32 ? 0xffffffffu : ((1u << rem) - 1u);
    }
    for (int J = tid; J < nKV; J += 256) ord[J] = __int_as_float(J);
    if (tid == 0) counts[row] = nKV;
    return;
  }

  // smallest exponent-bin top set that provably holds the answer (wave 0; lane l looks at
  // bins 127-2l and 126-2l, so lane order is descending bin order)
  if (wid == 0) {
    const int bh = 127 - 2 * lane, bl = 126 - 2 * lane;
    const int ch = hist[bh], cl = hist[bl];
    const unsigned long long mh = hmass[bh], ml = hmass[bl];
    int ci = ch + cl;
    unsigned long long mi = mh + ml;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int cy = __shfl_up(ci, o);
      const unsigned long long my = __shfl_up(mi, o);
      if (lane >= o) {
        ci += cy;
        mi += my;
      }
    }
    const int ce = ci - (ch + cl);
    const unsigned long long me = mi - (mh + ml);
    const unsigned long long need =
        (unsigned long long)ceil((double)thr * (1.0 + 1.0 / 1024.0) * 0x1p40);
    const bool ok_h = (ce + ch >= m_k) && (me + mh >= need);
    const bool ok_l = (ci >= m_k) && (mi >= need);
    const unsigned long long bal_h = __ballot(ok_h), bal_l = __ballot(ok_l);
    if (lane == 0) {
      int bstar = 0;
      if (bal_h | bal_l) {
        const int fh = bal_h ? __ffsll((long long)bal_h) - 1 : 64;
        const int fl = bal_l ? __ffsll((long long)bal_l) - 1 : 64;
        if (fh <= fl) {
          bstar = 127 - 2 * fh;
        } else {
          bstar = 126 - 2 * fl;
        }
      }
      sh_bstar = bstar;
      sh_pos = 0;
    }
    if (bal_h | bal_l) {
      const int fh = bal_h ? __ffsll((long long)bal_h) - 1 : 64;
      const int fl = bal_l ? __ffsll((long long)bal_l) - 1 : 64;
      const int src = fh <= fl ? fh : fl;
      const int cnt_h = __shfl(ce + ch, src), cnt_l = __shfl(ci, src);
      if (lane == 0) sh_ncand = fh <= fl ? cnt_h : cnt_l;
    } else if (lane == 0) {
      sh_ncand = nKV;
    }
  }
  __syncthreads();
  const int bstar = sh_bstar;
  const int ncand = sh_ncand;
  int count;

  if (ncand <= kCandCap) {
    // candidates: blocks in bins >= bstar (a top set of the score order)
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int J = tid * ITEMS + i;
      const float eJ = kEvLds ? ev[kEvLds ? J : 0] : ee[i];
      if (J < nKV && (int)(__float_as_uint(eJ) >> 23) >= bstar) {
        const int pos = atomicAdd(&sh_pos, 1);
        cand[pos] = kv[i];
      }
    }
    __syncthreads();
    // rank by counting (keys are distinct), scatter into score order
    for (int c = tid; c < ncand; c += 256) {
      const uint64_t k = cand[c];
      int rank = 0;
      for (int c2 = 0; c2 < ncand; ++c2) rank += cand[c2] < k ? 1 : 0;
      csort[rank] = k;
      cev[rank] = kEvLds ? ev[kEvLds ? (uint32_t)k : 0] : exp_sa(desc_order_value((uint32_t)(k >> 32)) - m);
    }
    __syncthreads();
    if (wid == 0) {
      int mp = -1;
      float acc = 0.0f;
      for (int c0 = 0; c0 < ncand; c0 += 64) {
        const bool in = c0 + lane < ncand;
        const int vbits = __float_as_int(in ? cev[c0 + lane] : 0.0f);
        float pre = 0.0f;
#pragma unroll
        for (int u = 0; u < 64; ++u) {
          acc = acc + __int_as_float(__builtin_amdgcn_readlane(vbits, u));
          pre = (lane == u) ? acc : pre;
        }
        const unsigned long long hit = __ballot(in && pre >= thr);
        if (hit != 0ull) {
          mp = c0 + __ffsll((long long)hit);
          break;
        }
      }
      // no crossing inside a set that holds every block: no prefix reaches thr
      if (mp < 0 && ncand == nKV) mp = nKV;
      if (lane == 0) sh_count = mp < 0 ? -1 : max(m_k, mp);
    }
    __syncthreads();
    count = sh_count;
    if (count >= 0) {
      for (int r = tid; r < count; r += 256) {
        const uint32_t J = (uint32_t)csort[r];
        atomicOr(&bits[J >> 5], 1u << (J & 31));
      }
      __syncthreads();
      for (int w = tid; w < nwords; w += 256) bitmap[(size_t)row * nwords + w] = bits[w];
      if (tid == 0) counts[row] = count;
      write_order(csort, count);
      return;
    }
  }

  // full sort: bitonic sort of all keys, ascending
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) keys[tid * ITEMS + i] = kv[i];
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P / 2; i += 256) {
        const int lo = 2 * i - (i & (j - 1));
        const int hi = lo + j;
        const uint64_t a = keys[lo], b = keys[hi];
        const bool up = (lo & k) == 0;
        if ((a > b) == up) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }

  // e in score order (in LDS, or recomputed from the sorted keys by the scan below)
  if constexpr (kEvLds) {
    float es[ITEMS];
#pragma unroll
    for (int q = 0; q < ITEMS; ++q) {
      const int r = tid + q * 256;
      es[q] = 0.0f;
      if (r < nKV) es[q] = ev[(uint32_t)keys[r]];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < ITEMS; ++q) ev[tid + q * 256] = es[q];
    __syncthreads();
  }

  // sequential top-p scan, one add at a time in score order. Wave 0 walks the sorted
  // values 64 at a time: each value is broadcast from its lane and added to a running
  // sum that every lane holds identically, lane u keeps the sum after position u, and a
  // ballot finds the first position that reaches the threshold. All control flow here
  // is wave-uniform.
  if (wid == 0) {
    int mp = nKV;
    float acc = 0.0f;
    for (int c0 = 0; c0 < nKV; c0 += 64) {
      const bool in = c0 + lane < nKV;
      float val = 0.0f;
      if (in) {
        if constexpr (kEvLds) val = ev[c0 + lane];
        else val = exp_sa(desc_order_value((uint32_t)(keys[c0 + lane] >> 32)) - m);
      }
      const int vbits = __float_as_int(val);
      float pre = 0.0f;
#pragma unroll
      for (int u = 0; u < 64; ++u) {
        acc = acc + __int_as_float(__builtin_amdgcn_readlane(vbits, u));
        pre = (lane == u) ? acc : pre;
      }
      const unsigned long long hit = __ballot(in && pre >= thr);
      if (hit != 0ull) {
        mp = c0 + __ffsll((long long)hit);
        break;
      }
    }
    if (lane == 0) sh_count = max(m_k, mp);
  }
  __syncthreads();
  count = sh_count;
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) {
    const int r = tid + q * 256;
    if (r < count) {
      const uint32_t J = (uint32_t)keys[r];
      atomicOr(&bits[J >> 5], 1u << (J & 31));
    }
  }
  __syncthreads();
  for (int w = tid; w < nwords; w += 256) bitmap[(size_t)row * nwords + w] = bits[w];
  if (tid == 0) counts[row] = count;
  write_order(keys, count);
}

// ---------------------------------------------------------------- CSR
// row_ptr = exclusive prefix sum of counts (one workgroup). Each pass covers 1024 * kScanIt
// rows: a thread loads its kScanIt consecutive counts at once (one memory round trip per
// pass), sums them in order, and the block scans the thread totals.
constexpr int kScanIt = 16;
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t *__restrict__ counts, int R,
                                                    int32_t *__restrict__ row_ptr, int64_t *__restrict__ nnz) {
  __shared__ int wsum[16];
  __shared__ int carry;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid == 0) {
    carry = 0;
    row_ptr[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < R; base += 1024 * kScanIt) {
    const int i0 = base + tid * kScanIt;
    int v[kScanIt];
#pragma unroll
    for (int u = 0; u < kScanIt; ++u) v[u] = i0 + u < R ? counts[i0 + u] : 0;
#pragma unroll
    for (int u = 1; u < kScanIt; ++u) v[u] += v[u - 1];
    int x = v[kScanIt - 1];   // inclusive scan of the thread totals across the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wid] = x;
    __syncthreads();
    if (wid == 0) {
      int w = lane < 16 ? wsum[lane] : 0;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const int y = __shfl_up(w, o);
        if (lane >= o) w += y;
      }
      if (lane < 16) wsum[lane] = w;
    }
    __syncthreads();
    const int before = carry + (wid > 0 ? wsum[wid - 1] : 0) + x - v[kScanIt - 1];
#pragma unroll
    for (int u = 0; u < kScanIt; ++u)
      if (i0 + u < R) row_ptr[i0 + u + 1] = before + v[u];
    __syncthreads();
    if (tid == 1023) carry = before + v[kScanIt - 1];
    __syncthreads();
  }
  if (tid == 0) *nnz = carry;
}

// One wave per row: popcounts, a lane prefix sum, then each lane writes its words' set
// bits in ascending order.
__global__ __launch_bounds__(256) void fill_kernel(const uint32_t *__restrict__ bitmap,
                                                   int nwords, const int32_t *__restrict__ row_ptr,
                                                   int R, int32_t *__restrict__ col_idx) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;
  int running = row_ptr[row];
  for (int w0 = 0; w0 < nwords; w0 += 64) {
    const int w = w0 + lane;
    uint32_t b = w < nwords ? bitmap[(size_t)row * nwords + w] : 0u;
    const int c = __popc(b);
    int x = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    int pos = running + x - c;
    while (b) {
      const int bit = __ffs(b) - 1;
      col_idx[pos++] = w * 32 + bit;
      b &= b - 1;
    }
    running += __shfl(x, 63);
  }
}

__global__ void dense_plan_kernel(int R, int nKV, int32_t *__restrict__ row_ptr,
                                  int32_t *__restrict__ col_idx, int64_t *__restrict__ nnz) {
  const long total = (long)R * nKV;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long)gridDim.x * blockDim.x) {
    col_idx[i] = (int32_t)(i % nKV);
    if (i % nKV == 0) row_ptr[i / nKV] = (int32_t)i;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    row_ptr[R] = (int32_t)total;
    *nnz = total;
  }
}

// Work order for the forward kernels. A forward launch of R workgroups runs workgroup b
// on XCD b mod 8 and gives it slot (b mod 8) * q + b / 8 (q = R / 8; slots from 8q on
// map to themselves), so XCD x works through slots [x q, (x+1) q) in order. Rows are
// dealt to the XCDs in runs of consecutive rows (chunks) aligned to heads: whole heads,
// or each head cut into k equal runs when there are fewer than 32 heads, or g whole
// heads per run when there are more than kOrderMaxChunks. Chunks go by descending
// kept-tile total, each to the XCD with the least work so far that still has free slots,
// split where an XCD fills up; an XCD runs its runs in that order (heaviest first) and
// each run in ascending row order. A head's
// query blocks keep many KV blocks in common, so keeping a head's rows together on one
// XCD keeps its L2 reuse, while the per-XCD totals come out nearly equal.
constexpr int kOrderMaxChunks = 512;

__device__ __forceinline__ void order_chunk(int c, int nQ, int BH, int k, int g, int M, int *start, int *len) {
  int s, e;
  if (g > 1) {
    s = c * g * nQ;
    e = min(BH, (c + 1) * g) * nQ;
  } else {
    const int h = c / k, j = c - (c / k) * k;
    s = h * nQ + (j * nQ) / k;
    e = h * nQ + ((j + 1) * nQ) / k;
  }
  s = min(s, M);
  e = min(e, M);
  *start = s;
  *len = e - s;
}

__global__ __launch_bounds__(256) void balance_order_kernel(const int32_t *__restrict__ row_ptr, int R, int nQ,
                                                            int32_t *__restrict__ row_order) {
  __shared__ int ch_work[kOrderMaxChunks], ch_start[kOrderMaxChunks], ch_len[kOrderMaxChunks];
  __shared__ int4 sorted[kOrderMaxChunks];               // (work, start, len, -)
  __shared__ int pc_start[kOrderMaxChunks + 8], pc_len[kOrderMaxChunks + 8], pc_off[kOrderMaxChunks + 8];
  __shared__ int n_pieces;
  const int tid = threadIdx.x;
  const int q = R / 8;
  const int M = 8 * q;
  for (int s = M + tid; s < R; s += 256) row_order[s] = s;
  if (q == 0) return;
  const int BH = R / nQ;
  const int k = BH >= 32 ? 1 : min(nQ, ceil_div(32, BH));
  const int g = BH > kOrderMaxChunks ? ceil_div(BH, kOrderMaxChunks) : 1;
  const int nch = g > 1 ? ceil_div(BH, g) : BH * k;
  for (int c = tid; c < nch; c += 256) {
    int st, ln;
    order_chunk(c, nQ, BH, k, g, M, &st, &ln);
    ch_start[c] = st;
    ch_len[c] = ln;
    ch_work[c] = row_ptr[st + ln] - row_ptr[st];
  }
  __syncthreads();
  // rank by (work descending, index ascending)
  for (int c = tid; c < nch; c += 256) {
    const int wc = ch_work[c];
    int r = 0;
    for (int c2 = 0; c2 < nch; ++c2) {
      const int w2 = ch_work[c2];
      r += (w2 > wc) || (w2 == wc && c2 < c);
    }
    sorted[r] = make_int4(wc, ch_start[c], ch_len[c], 0);
  }
  __syncthreads();
  if (tid < 64) {
    // wave 0 runs the greedy pass with every value wave-uniform (chunk records read through
    // readfirstlane), so its state lives in scalar registers and its steps run on the
    // scalar unit; lane 0 writes the pieces
    const int lane = tid;
    int load[8], cap[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      load[x] = 0;
      cap[x] = q;
    }
    int np = 0;
    int4 next = sorted[0];
    for (int i = 0; i < nch; ++i) {
      const int4 ch = make_int4(__builtin_amdgcn_readfirstlane(next.x), __builtin_amdgcn_readfirstlane(next.y),
                                __builtin_amdgcn_readfirstlane(next.z), 0);
      if (i + 1 < nch) next = sorted[i + 1];   // the next chunk's LDS read overlaps this one
      int start = ch.y, len = ch.z;
      while (len > 0) {
        int x = 0, best = cap[0] > 0 ? load[0] : INT_MAX;
#pragma unroll
        for (int y = 1; y < 8; ++y) {
          const int ly = cap[y] > 0 ? load[y] : INT_MAX;
          if (ly < best) {
            best = ly;
            x = y;
          }
        }
        const int take = min(len, cap[x]);
        if (lane == 0) {
          pc_off[np] = x * q + (q - cap[x]);  // runs fill an XCD's slots in assignment order
          pc_start[np] = start;
          pc_len[np] = take;
        }
        ++np;
        // a split chunk's work is shared pro rata (rounded down per row)
        load[x] += take == ch.z ? ch.x : (ch.x / ch.z) * take;
        cap[x] -= take;
        start += take;
        len -= take;
      }
    }
    if (lane == 0) n_pieces = np;
  }
  __syncthreads();
  const int np = n_pieces;
  for (int p = tid >> 6; p < np; p += 4) {  // one wave per run
    const int base = pc_off[p], st = pc_start[p], ln = pc_len[p];
    for (int i = tid & 63; i < ln; i += 64) row_order[base + i] = st + i;
  }
}

__global__ void router_exp_kernel(const float *__restrict__ x, float *__restrict__ y, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    y[i] = exp_sa(x[i]);
}

}  // namespace

// ---------------------------------------------------------------- launchers
hipError_t launch_pool(const void *x, sa_dtype dt, int BH, int H, int N, int D, int bs,
                       const int32_t *order, float *out, hipStream_t s) {
  const int nblk = ceil_div(N, bs);
  const long total = (long)BH * nblk;
  const int per_wg = 256 / (D / 8);
  const unsigned grid = (unsigned)((total + per_wg - 1) / per_wg);
#define SA_POOL(T, DD, O)                                                                       \
  pool_kernel<T, DD, O><<<grid, 256, 0, s>>>((const T *)x, H, N, bs, nblk, total, order, out)
  // The lean kernel keeps two rows in flight per thread: with fewer than about three
  // workgroups per CU that leaves too few bytes in flight (on the 12-head 32,760-token
  // shape, 192 and 384 workgroups, it takes 30 us a launch against 19), with more it is
  // as fast as the wide one.
  constexpr unsigned kLeanMinGrid = 3 * 256;
  const bool lean = order == nullptr && (size_t)BH * N * D * 2 < ((size_t)1 << 32) && grid >= kLeanMinGrid;
  if (dt == SA_BF16 && lean) {
    if (D == 128)
      pool_lean_kernel<128><<<grid, 256, 0, s>>>((const uint16_t *)x, N, bs, nblk, total, out);
    else
      pool_lean_kernel<64><<<grid, 256, 0, s>>>((const uint16_t *)x, N, bs, nblk, total, out);
  } else if (dt == SA_BF16) {
    if (D == 128) {
      if (order) SA_POOL(uint16_t, 128, true); else SA_POOL(uint16_t, 128, false);
    } else {
      if (order) SA_POOL(uint16_t, 64, true); else SA_POOL(uint16_t, 64, false);
    }
  } else {
    if (D == 128) SA_POOL(float, 128, false);
    else SA_POOL(float, 64, false);
  }
#undef SA_POOL
  return hipGetLastError();
}

hipError_t launch_scores(const float *qbar, const float *kbar, int BH, int nQ, int nKV, int D,
                         float c, float *scores, hipStream_t s) {
  dim3 grid(ceil_div(nKV, kSt), ceil_div(nQ, kSt), BH);
  scores_kernel<<<grid, 256, 0, s>>>(qbar, kbar, nQ, nKV, D, c, scores);
  return hipGetLastError();
}

hipError_t launch_select(float *scores, int R, int nKV, int ragged_last, int m_k, float p, int p_all,
                         uint32_t *bitmap, int nwords, int32_t *counts, hipStream_t s) {
#define SA_SELECT(IT) \
  select_kernel<IT><<<R, 256, 0, s>>>(scores, nKV, ragged_last, m_k, p, p_all, bitmap, nwords, counts)
  if (nKV <= 256)
    SA_SELECT(1);
  else if (nKV <= 512)
    SA_SELECT(2);
  else if (nKV <= 1024)
    SA_SELECT(4);
  else if (nKV <= 2048)
    SA_SELECT(8);
  else
    SA_SELECT(16);
#undef SA_SELECT
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t *counts, int R, int32_t *row_ptr, int64_t *nnz, hipStream_t s) {
  scan_kernel<<<1, 1024, 0, s>>>(counts, R, row_ptr, nnz);
  return hipGetLastError();
}

hipError_t launch_fill(const uint32_t *bitmap, int nwords, const int32_t *row_ptr, int R,
                       int32_t *col_idx, hipStream_t s) {
  fill_kernel<<<ceil_div(R, 4), 256, 0, s>>>(bitmap, nwords, row_ptr, R, col_idx);
  return hipGetLastError();
}

hipError_t launch_dense_plan(int R, int nKV, int32_t *row_ptr, int32_t *col_idx, int64_t *nnz, hipStream_t s) {
  const long total = (long)R * nKV;
  long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  dense_plan_kernel<<<(unsigned)blocks, 256, 0, s>>>(R, nKV, row_ptr, col_idx, nnz);
  return hipGetLastError();
}

hipError_t launch_row_order(const int32_t *row_ptr, int R, int nQ, int32_t *row_order, hipStream_t s) {
  balance_order_kernel<<<1, 256, 0, s>>>(row_ptr, R, nQ, row_order);
  return hipGetLastError();
}

hipError_t launch_router_exp(const float *x, float *y, int64_t n, hipStream_t s) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  router_exp_kernel<<<(unsigned)blocks, 256, 0, s>>>(x, y, n);
  return hipGetLastError();
}

}  // namespace sa
