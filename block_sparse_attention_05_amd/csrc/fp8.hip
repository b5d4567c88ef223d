// Low-bit forward for gfx950 (SLA2 page, quantisation-aware fine-tuning: the forward pass
// runs on queries, keys and values quantised to low precision).
//
// Format: OCP FP8 E4M3 with power-of-two group scales. A group's exponent e is the
// smallest integer with max|x| <= 448 * 2^e (clamped to [-64, 64]); a value is stored as
// the E4M3 code of x * 2^-e, rounded to nearest even by v_cvt_pk_fp8_f32. Groups: Q per
// (head, query block), K per (head, 64-key block), V per (head, channel).
//
// The pack's layouts are made for the forward kernel:
//   q8, k8   [B, H, N, D] codes, row-major;
//   vt8      [B, H, nKV, D, 64]: each 64-key block of V transposed to channel rows, its
//            keys in the order pi(h, b) = (b/16)*32 + ((b/4)%4)*8 + h*4 + b%4 for byte
//            h*32 + b of a row, zero past N. That is the order in which the S^T MFMA
//            leaves a lane half's probabilities, so P goes into the PV product as it lies;
//   qe, ke, ve  int32 exponents [B, H, nQ], [B, H, nKV], [B, H, D];
//   vamax    uint32 [B, H, D]: per-channel max |v| (fp32 bits), the quantiser's scratch.
//
// Forward: one workgroup per query block, one wave per 32 queries, as the bf16 kernel,
// with the fp8 MFMA v_mfma_f32_32x32x64_f8f6f4 (64 channels or 64 keys per instruction):
//   S^T = K Q^T        D/64 MFMAs per 32-key half; the tile's scale 2^(eq + ek) joins
//                      log2(e)/sqrt(D) in one multiplier per tile;
//   P                  exp2 in fp32, offset by 2^8 so that P * 256 in [0, 256] uses the
//                      E4M3 range, packed to fp8 with v_cvt_pk_fp8_f32. Without an LSE
//                      output the running max is lazy: it moves only when a tile's max
//                      passes it by more than kLazy (log2 units), P is offset by
//                      2^(8 - kLazy) to stay within 256, and the O rescale runs on few
//                      tiles. With the LSE the max is exact, so that the largest term of
//                      each row sum is exactly 2^8 (lazily, it would carry E4M3 rounding);
//   row sums           one MFMA of an all-ones A operand against P: the sums of exactly
//                      the rounded probabilities the PV product multiplies, off the VALU;
//   O^T += V^T P^T     D/32 MFMAs per tile; the per-channel V scale 2^ev is applied once
//                      in the epilogue.
// K and V^T tiles go HBM -> LDS by direct loads. Their 16-byte granules are XOR-permuted
// within a row through the load addresses (no padding): the 16 rows that one pass of a
// 128-bit LDS read touches then fall on distinct banks.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sa_internal.h"

namespace sa {
namespace {

typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx16 __attribute__((ext_vector_type(16)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

constexpr int kVmcnt0 = 0x0F70;   // s_waitcnt: all vector-memory operations done
constexpr int kExpMin = -64, kExpMax = 64;
constexpr float kLazy = 4.0f;     // lazy-max margin (log2 units) without an LSE output

__device__ __forceinline__ int xcd_remap(int b, int G) {
  const int q = G / 8;
  if (b >= q * 8) return b;
  return (b % 8) * q + b / 8;
}

// smallest e with amax <= 448 * 2^e: with amax = m * 2^E (m in [0.5, 1)) and
// 448 = 0.875 * 2^9, that is E - 9 when m <= 0.875 and E - 8 otherwise
__device__ __forceinline__ int fp8_exponent(float amax) {
  if (!(amax > 0.f)) return kExpMin;
  int E;
  const float m = frexpf(amax, &E);
  const int e = (m <= 0.875f) ? E - 9 : E - 8;
  return min(max(e, kExpMin), kExpMax);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// four floats -> four E4M3 codes in one dword (byte u = value u)
__device__ __forceinline__ uint32_t to_fp8x4(float a, float b, float c, float d) {
  // the first conversion fills the low half-word and keeps the high one of its `old`
  // operand, which the second then overwrites: any value will do there, and a's own bits
  // (dead after this use) let the result take a's register with no zeroing move
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// ------------------------------------------------------------------ quantiser
__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t *p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

__device__ __forceinline__ float block_max_256(float v, float *red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// four values -> four int8 codes rint(x * inv) in one dword (byte u = value u)
__device__ __forceinline__ uint32_t to_i8x4(float a, float b, float c, float d, float inv) {
  const int ca = (int)rintf(__fmul_rn(a, inv)), cb = (int)rintf(__fmul_rn(b, inv));
  const int cc = (int)rintf(__fmul_rn(c, inv)), cd = (int)rintf(__fmul_rn(d, inv));
  return (uint32_t)(ca & 0xFF) | ((uint32_t)(cb & 0xFF) << 8) | ((uint32_t)(cc & 0xFF) << 16) |
         ((uint32_t)(cd & 0xFF) << 24);
}

// One workgroup per (block of BLK rows, head): the block's max |x|, its exponent (E4M3)
// or fp32 scale (I8), and the codes of its rows. grid (ceil(N / BLK), B*H), 256 threads.
// I8: inv = 127 / a and s = a / 127 (correctly rounded fp32 divisions), code =
// rint(x * inv); an all-zero block takes inv = s = 0.
template <int D, int BLK, bool I8>
__global__ __launch_bounds__(256) void fp8_quant_rows_kernel(const uint16_t *__restrict__ x, int N, int nblk,
                                                             uint8_t *__restrict__ out, int32_t *__restrict__ exps) {
  constexpr int GPR = D / 8;                 // 16-byte granules per row
  constexpr int PER = BLK * GPR / 256;       // granules per thread
  static_assert(PER * 256 == BLK * GPR, "granules must split evenly");
  __shared__ float red[4];
  const int bh = blockIdx.y, blk = blockIdx.x;
  const int r0 = blk * BLK;
  const int ng = min(BLK, N - r0) * GPR;     // valid granules of the block
  const size_t base = ((size_t)bh * N + r0) * D;
  const uint4 *src = reinterpret_cast<const uint4 *>(x + base);
  uint4 g[PER];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = threadIdx.x + i * 256;
    g[i] = e < ng ? src[e] : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {g[i].x, g[i].y, g[i].z, g[i].w};
#pragma unroll
    for (int u = 0; u < 4; ++u) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[u])), fabsf(bf16_hi(w[u]))));
  }
  const float bmax = block_max_256(amax, red);
  uint2 *dst = reinterpret_cast<uint2 *>(out + base);
  if constexpr (I8) {
    const float inv = bmax > 0.f ? __fdiv_rn(127.0f, bmax) : 0.0f;
    if (threadIdx.x == 0) exps[(size_t)bh * nblk + blk] = __float_as_int(bmax > 0.f ? __fdiv_rn(bmax, 127.0f) : 0.0f);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = threadIdx.x + i * 256;
      if (e < ng) {
        const uint32_t w[4] = {g[i].x, g[i].y, g[i].z, g[i].w};
        uint2 r;
        r.x = to_i8x4(bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1]), inv);
        r.y = to_i8x4(bf16_lo(w[2]), bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3]), inv);
        dst[e] = r;
      }
    }
  } else {
    const int ex = fp8_exponent(bmax);
    if (threadIdx.x == 0) exps[(size_t)bh * nblk + blk] = ex;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = threadIdx.x + i * 256;
      if (e < ng) {
        const uint32_t w[4] = {g[i].x, g[i].y, g[i].z, g[i].w};
        uint2 r;
        r.x = to_fp8x4(ldexpf(bf16_lo(w[0]), -ex), ldexpf(bf16_hi(w[0]), -ex), ldexpf(bf16_lo(w[1]), -ex),
                       ldexpf(bf16_hi(w[1]), -ex));
        r.y = to_fp8x4(ldexpf(bf16_lo(w[2]), -ex), ldexpf(bf16_hi(w[2]), -ex), ldexpf(bf16_lo(w[3]), -ex),
                       ldexpf(bf16_hi(w[3]), -ex));
        dst[e] = r;
      }
    }
  }
}

// Per-channel max |v| over chunks of kVChunk tokens: grid (ceil(N / kVChunk), B*H), 256
// threads; thread t owns granule column t % (D/8) and rows t / (D/8) + RP*i. The result is
// combined across chunks with an integer atomic max on the fp32 bits (order-free: the
// values are non-negative, whose bit patterns order as the values do).
constexpr int kVChunk = 512;
template <int D>
__global__ __launch_bounds__(256) void fp8_vamax_kernel(const uint16_t *__restrict__ v, int N,
                                                        uint32_t *__restrict__ vamax) {
  constexpr int GPR = D / 8;
  constexpr int RP = 256 / GPR;              // row phases
  __shared__ float part[RP][D + 1];
  const int bh = blockIdx.y;
  const int r0 = blockIdx.x * kVChunk;
  const int rows = min(kVChunk, N - r0);
  const int col = threadIdx.x % GPR, ph = threadIdx.x / GPR;
  const uint4 *src = reinterpret_cast<const uint4 *>(v + ((size_t)bh * N + r0) * D) + col;
  float m[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) m[u] = 0.f;
  for (int r = ph; r < rows; r += 8 * RP) {
    uint4 g[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int rr = r + b * RP;
      g[b] = rr < rows ? src[(size_t)rr * GPR] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint32_t w[4] = {g[b].x, g[b].y, g[b].z, g[b].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        m[2 * u] = fmaxf(m[2 * u], fabsf(bf16_lo(w[u])));
        m[2 * u + 1] = fmaxf(m[2 * u + 1], fabsf(bf16_hi(w[u])));
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) part[ph][col * 8 + u] = m[u];
  __syncthreads();
  if (threadIdx.x < D) {
    float r = 0.f;
#pragma unroll 4
    for (int p = 0; p < RP; ++p) r = fmaxf(r, part[p][threadIdx.x]);
    atomicMax(vamax + (size_t)bh * D + threadIdx.x, __float_as_uint(r));
  }
}

// One workgroup per (64-key block, head), 2*D threads: thread (c, h) writes bytes
// h*32 .. h*32+31 of channel row c of the block's V^T, keys in the pi order.
template <int D>
__global__ __launch_bounds__(2 * D) void fp8_quant_vt_kernel(const uint16_t *__restrict__ v, int N, int nKV,
                                                            const uint32_t *__restrict__ vamax,
                                                            uint8_t *__restrict__ vt, int32_t *__restrict__ vexp) {
  constexpr int GPR = D / 8;
  constexpr int NT = 2 * D;
  __shared__ uint16_t vs[64][D + 2];
  const int bh = blockIdx.y, J = blockIdx.x;
  const int j0 = J * 64;
  const int valid = min(64, N - j0);
  const uint4 *src = reinterpret_cast<const uint4 *>(v + ((size_t)bh * N + j0) * D);
  for (int e = threadIdx.x; e < 64 * GPR; e += NT) {
    const int r = e / GPR, c8 = (e % GPR) * 8;
    const uint4 g = r < valid ? src[e] : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      vs[r][c8 + 2 * u] = (uint16_t)(w[u] & 0xFFFF);
      vs[r][c8 + 2 * u + 1] = (uint16_t)(w[u] >> 16);
    }
  }
  __syncthreads();
  const int c = threadIdx.x >> 1, h = threadIdx.x & 1;
  const int ex = fp8_exponent(__uint_as_float(vamax[(size_t)bh * D + c]));
  if (J == 0 && h == 0) vexp[(size_t)bh * D + c] = ex;
  uint32_t w[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int b = 4 * d + u;
      const int key = (b >> 4) * 32 + ((b >> 2) & 3) * 8 + h * 4 + (b & 3);
      x[u] = ldexpf(__uint_as_float((uint32_t)vs[key][c] << 16), -ex);   // zero past N
    }
    w[d] = to_fp8x4(x[0], x[1], x[2], x[3]);
  }
  uint4 *dst = reinterpret_cast<uint4 *>(vt + (((size_t)bh * nKV + J) * D + c) * 64 + h * 32);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

// ------------------------------------------------------------------ forward
constexpr int kBk = 64;

// XOR permutation of the 16-byte granules of a tile row, by row index: rows of 128 bytes
// use (r/2) mod 8, rows of 64 bytes (r/4) mod 4
template <int RB>
__device__ __forceinline__ int swz(int r) {
  return RB == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

template <int D, int NW, bool I8>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
void sparse_fwd_fp8_kernel(Fp8FwdArgs a) {
  constexpr int BQ = 32 * NW;
  constexpr int TB = kBk * D;                // bytes of a K tile and of a V^T tile
  constexpr int NI = TB / 1024;              // 1 KB direct loads per tile
  constexpr int NIW = (NI + NW - 1) / NW;
  constexpr int KG = D / 16;                 // granules per K row
  constexpr int MS = D / 64;                 // S MFMAs per 32-key half
  constexpr int DT = D / 32;                 // PV MFMAs

  __shared__ __align__(16) char k0s[TB];
  __shared__ __align__(16) char v0s[TB];
  __shared__ __align__(16) char k1s[TB];
  __shared__ __align__(16) char v1s[TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const uint8_t *qg = a.q8 + head;
  const uint8_t *kg = a.k8 + head;
  const uint8_t *vtg = a.vt8 + (size_t)bh * a.n_kvblk * TB;
  uint16_t *og = a.o + head;

  const int qi = I * BQ + wid * 32 + l32;
  const bool q_ok = qi < N;
  const int beg = a.row_ptr[row];
  const int end = a.row_ptr[row + 1];

  if (beg == end) {
    if (q_ok) {
      for (int d = hf * (D / 2); d < (hf + 1) * (D / 2); d += 8)
        *reinterpret_cast<uint4 *>(og + (size_t)qi * D + d) = make_uint4(0, 0, 0, 0);
      if (a.lse && hf == 0) a.lse[(size_t)bh * N + qi] = -INFINITY;
    }
    return;
  }

  // Q fragments (B operand of S^T = K Q^T). E4M3: channels m*64 + hf*32 + 0..31 for the
  // 32x32x64 MFMA; I8: channels m*32 + hf*16 + 0..15 for v_mfma_i32_32x32x32_i8.
  intx8 qf[MS];
  intx4 qf4[DT];
  if constexpr (I8) {
#pragma unroll
    for (int m = 0; m < DT; ++m) {
      uint4 w0 = make_uint4(0, 0, 0, 0);
      if (q_ok) w0 = *reinterpret_cast<const uint4 *>(qg + (size_t)qi * D + m * 32 + hf * 16);
      qf4[m] = intx4{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w};
    }
  } else {
#pragma unroll
    for (int m = 0; m < MS; ++m) {
      uint4 w0 = make_uint4(0, 0, 0, 0), w1 = w0;
      if (q_ok) {
        const uint4 *p = reinterpret_cast<const uint4 *>(qg + (size_t)qi * D + m * 64 + hf * 32);
        w0 = p[0];
        w1 = p[1];
      }
      qf[m] = intx8{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
    }
  }
  // E4M3: the block's exponent; I8: its fp32 scale (bits)
  const int eq = a.qe[(size_t)bh * nQ + I];
  const int32_t *__restrict__ keb = a.ke + (size_t)bh * a.n_kvblk;

  // direct-load sources: load i fills LDS granules 64i .. 64i+63 of a tile; lane p of it
  // carries LDS granule P = 64i + p = (row, physical granule), whose logical granule is
  // physical ^ swz(row)
  uint32_t koffs[NIW], voffs[NIW];
#pragma unroll
  for (int m = 0; m < NIW; ++m) {
    const int P = 64 * (wid + m * NW) + lane;
    const int kr = P / KG, kp = P % KG;
    koffs[m] = kr * D + ((kp ^ swz<D>(kr)) * 16);
    const int vr = P / 4, vp = P % 4;
    voffs[m] = vr * 64 + ((vp ^ swz<64>(vr)) * 16);
  }
  const int ragged_blk = (N % kBk) ? (N / kBk) : -1;
  const int32_t *__restrict__ cols = a.visit ? a.visit + (size_t)row * a.n_kvblk : a.col_idx + beg;

  // Buffer resources over this head's K (N * D bytes) and V^T (whole blocks): lane
  // offsets go in the VGPR offset and the tile's byte offset in the scalar one, so an
  // issue costs no per-lane address arithmetic. Both spans are at most 32 MiB (4096 blocks
  // of 64 keys at D = 128), and every offset used is inside them.
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)kg, (short)0, N * D, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void *)vtg, (short)0, a.n_kvblk * TB, kRawBufferWord3);
  auto issue = [&](int J, char *kdst, char *vdst) {
    const uint8_t *kb = kg + (size_t)J * kBk * D;
    const int toff = J * TB;
    if (J != ragged_blk) {
#pragma unroll
      for (int m = 0; m < NIW; ++m) {
        const int i = wid + m * NW;
        if (i < NI)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lvoid_t *)(kdst + i * 1024), 16, (int)koffs[m], toff, 0, 0);
      }
    } else {
      // K rows past N reload the last valid row (in bounds, finite); V^T is stored
      // zero-padded to whole blocks
      const int last = N - 1 - J * kBk;
#pragma unroll
      for (int m = 0; m < NIW; ++m) {
        const int i = wid + m * NW;
        if (i < NI) {
          const int P = 64 * i + lane;
          const int kr = P / KG, kp = P % KG;
          const uint32_t off = min(kr, last) * D + ((kp ^ swz<D>(kr)) * 16);
          __builtin_amdgcn_global_load_lds((gvoid_t *)(kb + off), (lvoid_t *)(kdst + i * 1024), 16, 0, 0);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < NIW; ++m) {
      const int i = wid + m * NW;
      if (i < NI)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lvoid_t *)(vdst + i * 1024), 16, (int)voffs[m], toff, 0, 0);
    }
  };

  // per-lane LDS read offsets. K operand: row l32 (+32 for the second half), logical
  // granules m*4 + hf*2 + {0, 1}; V^T operand: channel row l32 (+32t), granules hf*2 + {0, 1}.
  // The swizzle of rows l32 + 32j equals that of l32.
  int kro[MS][2];
#pragma unroll
  for (int m = 0; m < MS; ++m)
#pragma unroll
    for (int s = 0; s < 2; ++s) kro[m][s] = l32 * D + (((m * 4 + hf * 2 + s) ^ swz<D>(l32)) * 16);
  int kro4[DT];   // I8: granule m*2 + hf
#pragma unroll
  for (int m = 0; m < DT; ++m) kro4[m] = l32 * D + (((m * 2 + hf) ^ swz<D>(l32)) * 16);
  int vro[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) vro[s] = l32 * 64 + (((hf * 2 + s) ^ swz<64>(l32)) * 16);

  floatx16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[t][i] = 0.0f;
  floatx16 lacc;  // running row sum, the same in all 16 entries
#pragma unroll
  for (int i = 0; i < 16; ++i) lacc[i] = 0.0f;
  const intx8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};   // E4M3 1.0
  float m_run = -INFINITY;  // running max of the scaled logits, log2 domain
  const float sl2 = a.scale_log2;
  const float lazy = a.lse ? 0.0f : kLazy;
  const float poff = 8.0f - lazy;   // P is stored times 2^poff: at most 2^8

  auto ld8 = [](const char *p0, int o0, int o1) {
    const uint4 x = *reinterpret_cast<const uint4 *>(p0 + o0);
    const uint4 y = *reinterpret_cast<const uint4 *>(p0 + o1);
    return intx8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
  };

  auto tile = [&](int J, int ek, const char *kt_s, const char *vt_s, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    floatx16 sacc[2];
    float mul;
    if constexpr (I8) {
      // exact int32 dot products of the codes, then one fp32 multiplier: sq * sk * log2(e)/sqrt(D)
      mul = sl2 * __int_as_float(eq) * __int_as_float(ek);
      intx16 iacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) iacc[kt][i] = 0;
#pragma unroll
      for (int m = 0; m < DT; ++m)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const uint4 x = *reinterpret_cast<const uint4 *>(kt_s + kt * 32 * D + kro4[m]);
          iacc[kt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(intx4{(int)x.x, (int)x.y, (int)x.z, (int)x.w}, qf4[m],
                                                           iacc[kt], 0, 0, 0);
        }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kt][i] = (float)iacc[kt][i];
    } else {
      mul = ldexpf(sl2, eq + ek);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.0f;
#pragma unroll
      for (int m = 0; m < MS; ++m)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const intx8 kf = ld8(kt_s + kt * 32 * D, kro[m][0], kro[m][1]);
          sacc[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[m], sacc[kt], 0, 0, 0, 0, 0, 0);
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
    const float mt = mx * mul;
    const bool need = mt > m_run + lazy;
    if (__ballot(need)) {
      const float m_new = need ? mt : m_run;
      const float corr = need ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) lacc[i] *= corr;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[t][i] *= corr;
      m_run = m_new;
    }
    // P * 2^poff = exp2(s * mul - m_run + poff), in [0, 256]
    const float msub = m_run - poff;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kt][i] = __builtin_amdgcn_exp2f(sacc[kt][i] * mul - msub);
    // byte 4w + u of the B operand = entry 4(w mod 4) + u of half w/4: key pi(hf, 4w + u)
    intx8 pb;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kt = w >> 2, i0 = (w & 3) * 4;
      pb[w] = (int)to_fp8x4(sacc[kt][i0], sacc[kt][i0 + 1], sacc[kt][i0 + 2], sacc[kt][i0 + 3]);
    }
    lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pb, lacc, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const intx8 vf = ld8(vt_s + t * 32 * 64, vro[0], vro[1]);
      oacc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pb, oacc[t], 0, 0, 0, 0, 0, 0);
    }
  };

  // Indices and K exponents run ahead of their use: the index of tile it + 2 is fetched
  // while tile it computes, and the exponent of a tile together with its loads, so no
  // tile waits on a memory round trip before its loads or its first multiply.
  const int n = end - beg;
  const int n_full = n - (cols[n - 1] == ragged_blk ? 1 : 0);
  int c_next = n > 1 ? cols[1] : 0;
  int j_cur = __builtin_amdgcn_readfirstlane(cols[0]);
  int e_cur = keb[j_cur], e_next = 0, j_next = 0;
  issue(j_cur, k0s, v0s);
  int it = 0;
  for (; it < n_full; it += 2) {
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    if (it + 1 < n) {
      j_next = __builtin_amdgcn_readfirstlane(c_next);
      issue(j_next, k1s, v1s);
      e_next = keb[j_next];
    }
    if (it + 2 < n) c_next = cols[it + 2];
    tile(j_cur, e_cur, k0s, v0s, std::false_type{});
    j_cur = j_next;
    e_cur = e_next;
    if (it + 1 >= n_full) {
      ++it;
      break;
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    if (it + 2 < n) {
      j_next = __builtin_amdgcn_readfirstlane(c_next);
      issue(j_next, k0s, v0s);
      e_next = keb[j_next];
    }
    if (it + 3 < n) c_next = cols[it + 3];
    tile(j_cur, e_cur, k1s, v1s, std::false_type{});
    j_cur = j_next;
    e_cur = e_next;
  }
  if (n_full < n) {
    // tile n - 1 (the ragged block) was issued into buffer (n - 1) % 2; j_cur and e_cur
    // are its index and exponent
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    if ((n - 1) % 2 == 0)
      tile(j_cur, e_cur, k0s, v0s, std::true_type{});
    else
      tile(j_cur, e_cur, k1s, v1s, std::true_type{});
  }

  // epilogue: O[q][d] = acc * 2^ev[d] / l, stored bf16. Once every wave is past the last
  // tile, each wave stages its 32 x D block in a K/V buffer of its own (16-byte granule c
  // of row r at c ^ (r mod D/8)) and writes it out in whole rows, 1 KB per store
  // instruction instead of 8-byte pieces of 32 rows.
  const float l_tot = lacc[0];
  const float inv = 1.0f / l_tot;
  constexpr int GPR = D / 8;                 // 16-byte granules per output row
  constexpr int RPI = 64 / GPR;              // rows per store instruction
  static_assert(32 * D * 2 <= TB, "a wave's output block fits in one K/V buffer");
  __syncthreads();
  char *ob = wid == 0 ? k0s : wid == 1 ? v0s : wid == 2 ? k1s : v1s;
  const int32_t *veb = a.ve + (size_t)bh * D;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = t * 32 + g * 8 + hf * 4;
      const int4 ev = *reinterpret_cast<const int4 *>(veb + d);
      const __bf16 b0 = (__bf16)ldexpf(oacc[t][g * 4 + 0] * inv, ev.x);
      const __bf16 b1 = (__bf16)ldexpf(oacc[t][g * 4 + 1] * inv, ev.y);
      const __bf16 b2 = (__bf16)ldexpf(oacc[t][g * 4 + 2] * inv, ev.z);
      const __bf16 b3 = (__bf16)ldexpf(oacc[t][g * 4 + 3] * inv, ev.w);
      uint2 pk;
      pk.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
      pk.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
      const int c = t * 4 + g;
      *reinterpret_cast<uint2 *>(ob + l32 * (D * 2) + ((c ^ (l32 & (GPR - 1))) * 16) + hf * 8) = pk;
    }
  const int q0 = I * BQ + wid * 32;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / GPR, c = lane % GPR;
    const uint4 w = *reinterpret_cast<const uint4 *>(ob + r * (D * 2) + ((c ^ (r & (GPR - 1))) * 16));
    if (q0 + r < N) *reinterpret_cast<uint4 *>(og + (size_t)(q0 + r) * D + c * 8) = w;
  }
  if (q_ok && a.lse && hf == 0) a.lse[(size_t)bh * N + qi] = (m_run + __log2f(l_tot) - poff) * 0.69314718055994531f;
}

template <int D, bool I8>
hipError_t launch_fwd_fp8_d(const Fp8FwdArgs &a, hipStream_t s) {
  const int R = a.B * a.H * a.n_qblk;
  if (a.block_q == 128)
    sparse_fwd_fp8_kernel<D, 4, I8><<<R, 256, 0, s>>>(a);
  else
    sparse_fwd_fp8_kernel<D, 2, I8><<<R, 128, 0, s>>>(a);
  return hipGetLastError();
}

template <int D, bool I8>
hipError_t launch_quant_d(const uint16_t *q, const uint16_t *k, const uint16_t *v, int BH, int N, int bq,
                          const Fp8Pack &p, hipStream_t s) {
  const int nQ = ceil_div(N, bq), nKV = ceil_div(N, kBk);
  fill_u32_kernel<<<ceil_div(BH * D, 256), 256, 0, s>>>(p.vamax, BH * D);
  fp8_vamax_kernel<D><<<dim3(ceil_div(N, kVChunk), BH), 256, 0, s>>>(v, N, p.vamax);
  if (bq == 128)
    fp8_quant_rows_kernel<D, 128, I8><<<dim3(nQ, BH), 256, 0, s>>>(q, N, nQ, p.q8, p.qe);
  else
    fp8_quant_rows_kernel<D, 64, I8><<<dim3(nQ, BH), 256, 0, s>>>(q, N, nQ, p.q8, p.qe);
  fp8_quant_rows_kernel<D, 64, I8><<<dim3(nKV, BH), 256, 0, s>>>(k, N, nKV, p.k8, p.ke);
  fp8_quant_vt_kernel<D><<<dim3(nKV, BH), 2 * D, 0, s>>>(v, N, nKV, p.vamax, p.vt8, p.ve);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_fp8(const uint16_t *q, const uint16_t *k, const uint16_t *v, int BH, int N, int D,
                               int bq, int i8qk, const Fp8Pack &p, hipStream_t s) {
  if (i8qk)
    return D == 128 ? launch_quant_d<128, true>(q, k, v, BH, N, bq, p, s) : launch_quant_d<64, true>(q, k, v, BH, N, bq, p, s);
  return D == 128 ? launch_quant_d<128, false>(q, k, v, BH, N, bq, p, s) : launch_quant_d<64, false>(q, k, v, BH, N, bq, p, s);
}

hipError_t launch_fwd_fp8(const Fp8FwdArgs &a, int i8qk, hipStream_t s) {
  if (i8qk) return a.D == 128 ? launch_fwd_fp8_d<128, true>(a, s) : launch_fwd_fp8_d<64, true>(a, s);
  return a.D == 128 ? launch_fwd_fp8_d<128, false>(a, s) : launch_fwd_fp8_d<64, false>(a, s);
}

}  // namespace sa
