// Linear-attention branch for gfx950 (SALAD page, section 2.1: a linear-attention branch
// in parallel with the sparse one, O(N) in the sequence length; SLA2 page: the blocks the
// router drops feed the linear branch). phi = elu + 1 on the raw q and k.
//
// For query block I with kept KV blocks K_I and complement C_I:
//   Ol_i = phi(q_i)^T H_C / phi(q_i)^T z_C,  H_C = sum_{j in C_I} phi(k_j) v_j^T,
//                                           z_C = sum_{j in C_I} phi(k_j).
// H_C is a D x D matrix shared by the whole query block, so the apply step forms it once
// per block: the per-tile work is one D x D x 64 product instead of two BQ x 64 x D ones.
//   linear_kv_kernel     per (head, token chunk): partial H and z with bf16 MFMA and fp32
//                        accumulation; also writes phi(K) in bf16 with zero pad rows;
//   linear_reduce_kernel sums the chunk partials in chunk order (deterministic) into the
//                        per-head totals H and z (fp32);
//   linear_apply_kernel  per query block: when it keeps at most half of the KV blocks,
//                        H_C and z_C are the totals minus the kept tiles' sums (formed in
//                        fp32, then rounded once); otherwise the complement tiles are
//                        summed directly, so no sum is formed as a small difference of
//                        large ones. It writes H_C^T in bf16 and z_C in fp32 per block; a
//                        block that keeps every KV block writes nothing (Ol = 0).
// The forward kernel's epilogue then forms Ol = phi(Q) H_C / phi(Q) z_C on MFMA from the
// Q fragments it already holds and blends O = alpha*Os + (1 - alpha)*Ol, so Ol never goes
// through memory.

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
// two floats to packed bf16, rounded to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

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
// Staging: thread c < 16 * D / 8 owns token group rg = c % 16 (4 tokens) and channels
// 8 * (c / 16) .. +7 of every tile, so a wave's transposed 8-byte stores cover 16 token
// groups and both parities of the channel octet: with 36-dword rows each store lands on
// all 64 banks twice, the least a 512-byte store can take. The thread also keeps its
// channels' phi(k) sums over the chunk; they are added across token groups at the end.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void linear_kv_kernel(const uint16_t *__restrict__ k,
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

  static_assert(CHUNKS_T <= 256, "one staging slot per thread");
  floatx16 acc[PER_WAVE];
#pragma unroll
  for (int p = 0; p < PER_WAVE; ++p)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[p][i] = 0.0f;
  const bool stager = tid < CHUNKS_T;
  const int rg = tid % (kTile / 4), col = (tid / (kTile / 4)) * 8;
  float zp[8];  // this thread's phi(k) sums over its token groups, channels col..col+7
#pragma unroll
  for (int i = 0; i < 8; ++i) zp[i] = 0.0f;

  // The next tile's raw rows are loaded while this tile's MFMAs run (tokens past the end
  // read as zeros: they contribute nothing, and their phi(k) pad rows are written as 0).
  uint4 kn[4], vn[4];
  auto load_rows = [&](int t0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = t0 + rg * 4 + r;
      kn[r] = make_uint4(0, 0, 0, 0);
      vn[r] = make_uint4(0, 0, 0, 0);
      if (stager && tok < t_end) {
        kn[r] = *reinterpret_cast<const uint4 *>(kg + (size_t)tok * D + col);
        vn[r] = *reinterpret_cast<const uint4 *>(vg + (size_t)tok * D + col);
      }
    }
  };
  load_rows(t_beg);
  for (int t0 = t_beg; t0 < t_end; t0 += kTile) {
    uint4 kr[4], vr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      kr[r] = kn[r];
      vr[r] = vn[r];
    }
    if (t0 + kTile < t_end) load_rows(t0 + kTile);
    __syncthreads();
    if (stager) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = t0 + rg * 4 + r;
        if (tok < t_end) kr[r] = phi8(kr[r]);
        // t0 + 64 <= n_pad, so the pad rows past N are written here as zeros
        *reinterpret_cast<uint4 *>(pk + (size_t)tok * D + col) = kr[r];
        zp[0] += bf(kr[r].x, 0); zp[1] += bf(kr[r].x, 1);
        zp[2] += bf(kr[r].y, 0); zp[3] += bf(kr[r].y, 1);
        zp[4] += bf(kr[r].z, 0); zp[5] += bf(kr[r].z, 1);
        zp[6] += bf(kr[r].w, 0); zp[7] += bf(kr[r].w, 1);
      }
      store_t4x8(&kt[col * ROW + rg * 4], ROW, kr);
      store_t4x8(&vt[col * ROW + rg * 4], ROW, vr);
    }
    __syncthreads();
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
  // z: the token groups' sums of each channel, added in token-group order
  __syncthreads();
  float *zs = reinterpret_cast<float *>(kt);  // [kTile / 4][D], 8 KB of the 18 KB tile
  if (stager)
#pragma unroll
    for (int i = 0; i < 8; ++i) zs[rg * D + col + i] = zp[i];
  __syncthreads();
  if (tid < D) {
    float zacc = 0.0f;
#pragma unroll
    for (int g = 0; g < kTile / 4; ++g) zacc += zs[g * D + tid];
    out[D * D + tid] = zacc;
  }
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
  int c = 0;
  for (; c + 8 <= chunks; c += 8) {   // eight loads in flight, added in chunk order
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = p[(size_t)(c + u) * per];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += x[u];
  }
  for (; c < chunks; ++c) s += p[(size_t)c * per];
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

// Workgroup barrier for LDS written by the waves' own waited-for loads: no fence, so no
// wait for the loads still in flight into other buffers; the clobber keeps the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Waits until at most n (<= O) of the stages issued after the one being waited for are
// still in flight; each stage is LPS direct loads per wave, and loads complete in order.
template <int LPS, int O>
__device__ __forceinline__ void wait_stages(int n) {
  static_assert(O * LPS < 16, "vmcnt field");
  if constexpr (O == 0) {
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
  } else {
    if (n >= O)
      __builtin_amdgcn_s_waitcnt(kVmcnt0 | (O * LPS));
    else
      wait_stages<LPS, O - 1>(n);
  }
}

#ifndef LIN_SK
#define LIN_SK 32
#endif
#ifndef LIN_NST
#define LIN_NST 3
#endif

// One workgroup of four waves per query block (CSR row). The four waves split the
// (D/32)^2 blocks of the row's running sum H_S[c][d] in a 2x2 grid: wave w takes c-blocks
// of half w >> 1 and d-blocks of half w & 1. phi(K) and V tiles go from HBM straight into
// LDS, both with their 64-byte row segments XOR-swizzled by row, and both MFMA operands
// come from transposing LDS reads (8 keys of one channel per lane). The tiles stream
// through NST stages of SK keys each, NST - 1 of them in flight while one is multiplied.
// At the end the waves round H_C^T to bf16, stage it in LDS and write it out in row order
// with z_C; the forward's epilogue multiplies it by phi(q).
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(LIN_NST == 3 ? 3 : 2)))
void linear_apply_kernel(FwdArgs a, LinearBufs lb) {
  constexpr int NW = 4;
  constexpr int VROWB = D * 2;              // bytes per tile row (unpadded)
  constexpr int TB = kTile * VROWB;         // bytes per tile
  constexpr int SK = D == 128 ? LIN_SK : 32; // keys per pipeline stage
  constexpr int SPT = kTile / SK;           // stages per tile
  constexpr int NST = LIN_NST;              // stages held in LDS
  constexpr int SB = SK * VROWB;            // bytes per tensor per stage
  constexpr int VNIS = SB / 1024;           // 1 KB direct loads per tensor per stage
  constexpr int VNIWS = VNIS / NW;          // ... per wave
  constexpr int LPS = 2 * VNIWS;            // direct loads per wave per stage
  static_assert(SK % 16 == 0 && kTile % SK == 0 && VNIS % NW == 0 && VNIWS >= 1, "stage shape");
  constexpr int VSEG = D / 32;              // 64-byte segments per row (swizzle range)
  constexpr int CB = D / 32;                // 32-channel blocks
  constexpr int WC = CB / 2;                // c-blocks per wave
  constexpr int WD = CB / 2;                // d-blocks per wave
  constexpr int HG = D / 8;                 // 16-byte granules per staged H_C^T row
  constexpr int kMaxList = kMaxKvBlocks / 2;
  static_assert(WC >= 1, "shape");

  // Stage buffers (phi(K) rows, then V rows), one LDS object each: the compiler then tells
  // a stage's direct loads from the reads of another stage, and the loop's own waits
  // decide how many stages stay in flight.
  __shared__ __align__(16) char sb0[2 * SB], sb1[2 * SB], sb2[2 * SB], sb3[2 * SB];
  __shared__ __align__(16) char sb4[2 * SB], sb5[2 * SB], sb6[2 * SB], sb7[2 * SB];
  auto bufs = [&](int b) -> char * {
    switch (b) {
      case 0: return sb0;
      case 1: return sb1;
      case 2: return sb2;
      case 3: return sb3;
      case 4: return sb4;
      case 5: return sb5;
      case 6: return sb6;
      default: return sb7;
    }
  };
  static_assert(NST <= 8, "stage buffers");
  __shared__ uint16_t tiles[kMaxList];               // the tile list of this row
  __shared__ uint32_t keptbits[kMaxKvBlocks / 32];
  static_assert(kMaxKvBlocks <= 65536, "tile indices in 16 bits");

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
  const size_t head = (size_t)bh * N * D;
  const uint16_t *vg = reinterpret_cast<const uint16_t *>(a.v) + head;
  const uint16_t *pk = lb.phik + (size_t)bh * lb.n_pad * D;

  // The accumulators start from -H when the kept tiles are subtracted, so -H + H_S forms
  // in fp32 inside the MFMA chain and H_C is its negation (exact: round-to-nearest is
  // symmetric in sign, so this is bit for bit H - H_S with every operand negated), taken
  // once at the end. H is read before the row's CSR range is known, so its loads overlap
  // that round trip; rows that sum the complement drop it.
  const float *hg = lb.h + (size_t)bh * D * D;
  floatx16 hacc[WC][WD];
#pragma unroll
  for (int x = 0; x < WC; ++x)
#pragma unroll
    for (int y = 0; y < WD; ++y)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = (cp * WC + x) * 32 + (i / 4) * 8 + hf * 4 + (i % 4);
        const int d = (dp * WD + y) * 32 + l32;
        hacc[x][y][i] = hg[(size_t)c * D + d];
      }

  const int beg = a.row_ptr[row], end = a.row_ptr[row + 1];
  const int kept = end - beg;
  if (kept == nKV) return;  // empty complement: the forward takes Ol = 0 without reading
  const bool subtract = kept <= nKV / 2;

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

  // Direct loads: LDS granule (row r, physical granule pg) of a stage holds logical
  // granule pg ^ ((r mod VSEG) << 2) of key row r0 + r (r0 a multiple of 16, so the
  // swizzle is the same as by the tile row); load i of a stage fills granules 64i .. 64i+63.
  uint32_t goff[VNIWS];
  int grow[VNIWS];
#pragma unroll
  for (int m = 0; m < VNIWS; ++m) {
    const int P = 64 * (wid + m * NW) + lane;
    const int r = P / (D / 8), pg = P % (D / 8);
    grow[m] = r;
    goff[m] = (r * D + (pg ^ ((r & (VSEG - 1)) << 2)) * 8) * 2;
  }
  const int ragged_blk = (N % kTile) ? (N / kTile) : -1;

  // Buffer resources over this head's phi(K) rows (n_pad * D * 2 bytes) and V rows
  // (N * D * 2 bytes), both at most 64 MiB: a stage's byte offset goes in the scalar
  // offset and the lane's offset in the VGPR one, so an issue costs no per-lane address
  // arithmetic. Every offset used is inside the head.
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void *)pk, (short)0, lb.n_pad * D * 2, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)vg, (short)0, N * D * 2, kRawBufferWord3);

  // stage st: keys r0 .. r0 + SK - 1 of tile tiles[st / SPT], r0 = SK * (st % SPT)
  auto issue = [&](int st, char *buf) {
    const int J = tiles[st / SPT];
    const int r0 = SK * (st % SPT);
    char *kdst = buf;
    char *vdst = buf + SB;
    const int soff = (J * kTile + r0) * D * 2;
    // phi(K) rows past N are zero pad rows of the prepass buffer
#pragma unroll
    for (int m = 0; m < VNIWS; ++m)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lvoid_t *)(kdst + (wid + m * NW) * 1024), 16, (int)goff[m], soff, 0, 0);
    if (J != ragged_blk) {
#pragma unroll
      for (int m = 0; m < VNIWS; ++m)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lvoid_t *)(vdst + (wid + m * NW) * 1024), 16, (int)goff[m], soff, 0, 0);
    } else {
      const char *vb = reinterpret_cast<const char *>(vg + ((size_t)J * kTile + r0) * D);
      // V rows past N reload the last valid row (finite; their phi(k) is zero)
      const int last = N - 1 - J * kTile - r0;   // may be negative: the whole stage is past N
#pragma unroll
      for (int m = 0; m < VNIWS; ++m) {
        const int r = grow[m];
        const int rr = r <= last ? r : last;
        const uint32_t off = (uint32_t)(goff[m] + (rr - r) * D * 2);
        __builtin_amdgcn_global_load_lds((gvoid_t *)(vb + (int32_t)off), (lvoid_t *)(vdst + (wid + m * NW) * 1024), 16, 0, 0);
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

#pragma unroll
  for (int x = 0; x < WC; ++x)
#pragma unroll
    for (int y = 0; y < WD; ++y)
#pragma unroll
      for (int i = 0; i < 16; ++i) hacc[x][y][i] = subtract ? -hacc[x][y][i] : 0.0f;
  float zacc[WC];
#pragma unroll
  for (int x = 0; x < WC; ++x) zacc[x] = 0.0f;
  const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};

  // H_S[c][d] += sum over the stage's keys of phi(K)[key][c] V[key][d]; the MFMA reduction
  // index hf*8 + e stands for key 16s + hf*4 + e (e < 4) or 16s + 8 + hf*4 + e - 4, the
  // same for both operands.
  auto stage = [&](int st, const char *buf) {
    const char *ks = buf;
    const char *vs = buf + SB;
#pragma unroll
    for (int s = 0; s < SK / 16; ++s) {
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
      if (((st * (SK / 16) + s) & 1) == dp) {
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

  // Stage st is multiplied from buffer st % NST; after the barrier of step st every wave
  // is done with buffer (st - 1) % NST, which then takes stage st + NST - 1.
  const int nst = ntiles * SPT;
#pragma unroll
  for (int b = 0; b < NST - 1; ++b)
    if (b < nst) issue(b, bufs(b));
  for (int st0 = 0; st0 < nst; st0 += NST) {
#pragma unroll
    for (int b = 0; b < NST; ++b) {
      const int st = st0 + b;
      if (st >= nst) break;
      wait_stages<LPS, NST - 2>(min(nst - 1 - st, NST - 2));
      lds_barrier();
      if (st + NST - 1 < nst) issue(st + NST - 1, bufs((b + NST - 1) % NST));
      stage(st, bufs(b));
    }
  }

  float zz[WC];   // this wave's z partials (its k-step half), both lane halves added
#pragma unroll
  for (int x = 0; x < WC; ++x) zz[x] = zacc[x] + __shfl_xor(zacc[x], 32);
  // H_C (-(-H + H_S) or H_S) in fp32, rounded once to bf16 below
  const float hsign = subtract ? -1.0f : 1.0f;
  __syncthreads();  // every wave is done with the stage buffers
  // z partials, then z_C, in the stage buffer that H_C^T leaves free
  static_assert(NST >= 3 && 2 * D * 4 <= 2 * SB, "z partials fit in a stage buffer");
  float *zs = reinterpret_cast<float *>(bufs(2));
  if (hf == 0)
#pragma unroll
    for (int x = 0; x < WC; ++x) zs[dp * D + (cp * WC + x) * 32 + l32] = zz[x];
  // staged H_C^T: row d in the stage buffers (2 * SK rows each), 16-byte granule c/8 at
  // physical granule (c/8) ^ (d mod HG)
  constexpr int RPB = 2 * SK;
  static_assert(D % RPB == 0 && D / RPB <= 2, "H_C^T fits in stage buffers 0 and 1");
#pragma unroll
  for (int x = 0; x < WC; ++x)
#pragma unroll
    for (int y = 0; y < WD; ++y) {
      const int d = (dp * WD + y) * 32 + l32;
      char *hrow = bufs(d / RPB) + (d % RPB) * VROWB;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int gr = (cp * WC + x) * 4 + q4;
        *reinterpret_cast<uint2 *>(hrow + ((gr ^ (d & (HG - 1))) * 16) + hf * 8) =
            pack4(hsign * hacc[x][y][q4 * 4 + 0], hsign * hacc[x][y][q4 * 4 + 1], hsign * hacc[x][y][q4 * 4 + 2],
                  hsign * hacc[x][y][q4 * 4 + 3]);
      }
    }
  __syncthreads();
  // H_C^T out to the row's slot, 16-byte granules in order (coalesced), and z_C
  uint16_t *hco = lb.hct + (size_t)row * D * D;
  for (int G = tid; G < D * HG; G += NW * 64) {
    const int d = G / HG, gr = G % HG;
    const uint4 w = *reinterpret_cast<const uint4 *>(bufs(d / RPB) + (d % RPB) * VROWB + ((gr ^ (d & (HG - 1))) * 16));
    *reinterpret_cast<uint4 *>(hco + (size_t)d * D + gr * 8) = w;
  }
  if (tid < D) {
    const float zsum = zs[tid] + zs[D + tid];
    lb.zc[(size_t)row * D + tid] = subtract ? lb.z[(size_t)bh * D + tid] - zsum : zsum;
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
  if (a.D == 128)
    linear_apply_kernel<128><<<R, 256, 0, s>>>(a, lb);
  else
    linear_apply_kernel<64><<<R, 256, 0, s>>>(a, lb);
  return hipGetLastError();
}

}  // namespace sa
