// Block-sparse attention forward, bf16 inputs, for gfx950 (SpargeAttention2 page, section
// 2(3): only the kept Q x KV tiles are visited, so masked tiles cost neither matrix
// products nor softmax work).
//
// One workgroup per query block (CSR row), one wave per 32 queries, 64-key tiles:
//   S^T = K Q^T      bf16 MFMA 32x32x16; each lane holds the 32 scores of one query for
//                    its half of the tile, so max and sum are in-lane plus one exchange
//                    between the two lane halves;
//   softmax          log2 domain, fp32, raw v_exp_f32. The O rescale (which touches
//                    every accumulator) runs only when some lane's running max grows; a
//                    lazier max (rescaling only past a margin) is not used, because it
//                    leaves the dominant key's probability off 1.0, and rounding that
//                    probability to bf16 then shows up at full weight in outputs that
//                    one key dominates;
//   O^T += V^T P^T   bf16 MFMA; P packed with v_cvt_pk_bf16_f32.
// K tiles are staged row-major in LDS, V tiles transposed on the way in; the next tile's
// global loads are in flight during the current tile's math. The ragged last KV block (if
// kept) is always the last tile of a row, because kept lists are ascending, so only that
// tile carries the key mask.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBk = 64;            // keys per tile

__device__ __forceinline__ int xcd_remap(int b, int G) {
  const int q = G / 8;
  if (b >= q * 8) return b;
  return (b % 8) * q + b / 8;
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  bf16x4_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  v[2] = (__bf16)c;
  v[3] = (__bf16)d;
  return __builtin_bit_cast(uint2, v);
}

template <int D, int NW, bool LIN>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2)))
void sparse_fwd_bf16_kernel(FwdArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int BQ = 32 * NW;
  constexpr int KROW = D + 8;               // K tile row stride (elements)
  constexpr int VROW = kBk + 4;             // V^T tile row stride (elements)
  constexpr int KCH = kBk * D / 8;          // 16-byte chunks per K tile
  constexpr int KPT = (KCH + NT - 1) / NT;
  constexpr int VCH = (kBk / 4) * (D / 8);  // 4-row x 8-column chunks per V tile
  constexpr int VPT = (VCH + NT - 1) / NT;
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 32;

  __shared__ __align__(16) uint16_t ks[kBk * KROW];
  __shared__ __align__(16) uint16_t vt[D * VROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
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

  const int qi = I * BQ + wid * 32 + l32;
  const bool q_ok = qi < N;
  const int beg = a.row_ptr[row];
  const int end = a.row_ptr[row + 1];

  if (beg == end) {
    // no kept tile: Os = 0 (so O = (1 - alpha) * Ol with the linear branch), LSE = -inf
    if (q_ok) {
      for (int d = hf * (D / 2); d < (hf + 1) * (D / 2); d += 4) {
        float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
        if constexpr (LIN) {
          const int h = bh % a.H;
          const float4 al = *reinterpret_cast<const float4 *>(a.alpha + (size_t)h * D + d);
          const float4 lv = *reinterpret_cast<const float4 *>(a.ol + head + (size_t)qi * D + d);
          o0 = (1.f - al.x) * lv.x;
          o1 = (1.f - al.y) * lv.y;
          o2 = (1.f - al.z) * lv.z;
          o3 = (1.f - al.w) * lv.w;
        }
        *reinterpret_cast<uint2 *>(og + (size_t)qi * D + d) = pack4(o0, o1, o2, o3);
      }
      if (a.lse && hf == 0) a.lse[(size_t)bh * N + qi] = -INFINITY;
    }
    return;
  }

  // Q fragments: B operand of S^T = K Q^T
  bf16x8_t qf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (q_ok) w = *reinterpret_cast<const uint4 *>(qg + (size_t)qi * D + s * 16 + hf * 8);
    qf[s] = __builtin_bit_cast(bf16x8_t, w);
  }

  uint4 kr[KPT];
  uint4 vr[VPT][4];

  auto load_tile = [&](int J) {
    const int j0 = J * kBk;
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

  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int c = tid + u * NT;
      if (c < KCH) {
        const int r = c / (D / 8), col = (c % (D / 8)) * 8;
        *reinterpret_cast<uint4 *>(&ks[r * KROW + col]) = kr[u];
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int c = tid + u * NT;
      if (c < VCH) {
        const int kgp = c / (D / 8), col = (c % (D / 8)) * 8;
        const uint32_t *w0 = reinterpret_cast<const uint32_t *>(&vr[u][0]);
        const uint32_t *w1 = reinterpret_cast<const uint32_t *>(&vr[u][1]);
        const uint32_t *w2 = reinterpret_cast<const uint32_t *>(&vr[u][2]);
        const uint32_t *w3 = reinterpret_cast<const uint32_t *>(&vr[u][3]);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          uint2 lo, hi;
          lo.x = __builtin_amdgcn_perm(w1[m], w0[m], 0x05040100u);
          lo.y = __builtin_amdgcn_perm(w3[m], w2[m], 0x05040100u);
          hi.x = __builtin_amdgcn_perm(w1[m], w0[m], 0x07060302u);
          hi.y = __builtin_amdgcn_perm(w3[m], w2[m], 0x07060302u);
          *reinterpret_cast<uint2 *>(&vt[(col + 2 * m) * VROW + kgp * 4]) = lo;
          *reinterpret_cast<uint2 *>(&vt[(col + 2 * m + 1) * VROW + kgp * 4]) = hi;
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
  float l_run = 0.0f;       // this lane's part of the running sum
  const float sl2 = a.scale_log2;
  const int ragged_blk = (N % kBk) ? (N / kBk) : -1;

  auto tile = [&](int J, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    floatx16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.0f;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const uint4 w = *reinterpret_cast<const uint4 *>(&ks[(kt * 32 + l32) * KROW + s * 16 + hf * 8]);
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
    float mx = sacc[0][0];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt = mx * sl2;
    const bool need = mt > m_run;
    if (__ballot(need)) {
      const float m_new = fmaxf(m_run, mt);
      const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[t][i] *= corr;
      m_run = m_new;
    }
    float psum = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(sacc[kt][i] * sl2 - m_run);
        sacc[kt][i] = pv;
        psum += pv;
      }
    l_run += psum;
    // O^T += V^T P^T; reduction index hf*8 + e stands for key base + (e/4)*8 + hf*4 + e%4,
    // which is where the S^T layout left this lane's probabilities.
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kt = s / 2, i0 = (s % 2) * 8;
      const int base = kt * 32 + (s % 2) * 16;
      bf16x8_t pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sacc[kt][i0 + e];
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const uint16_t *vrow = &vt[(t * 32 + l32) * VROW + base + hf * 4];
        const uint2 v0 = *reinterpret_cast<const uint2 *>(vrow);
        const uint2 v1 = *reinterpret_cast<const uint2 *>(vrow + 8);
        const uint4 vw = make_uint4(v0.x, v0.y, v1.x, v1.y);
        oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vw), pb,
                                                          oacc[t], 0, 0, 0);
      }
    }
  };

  // all tiles but the last: never the ragged block
  load_tile(a.col_idx[beg]);
  for (int it = beg; it < end - 1; ++it) {
    const int J = a.col_idx[it];
    __syncthreads();
    store_tile();
    __syncthreads();
    load_tile(a.col_idx[it + 1]);
    tile(J, std::false_type{});
  }
  {
    const int J = a.col_idx[end - 1];
    __syncthreads();
    store_tile();
    __syncthreads();
    if (J == ragged_blk)
      tile(J, std::true_type{});
    else
      tile(J, std::false_type{});
  }

  // epilogue: normalise (and blend), store bf16
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (q_ok) {
    uint16_t *orow = og + (size_t)qi * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = t * 32 + g * 8 + hf * 4;
        float o0 = oacc[t][g * 4 + 0] * inv, o1 = oacc[t][g * 4 + 1] * inv;
        float o2 = oacc[t][g * 4 + 2] * inv, o3 = oacc[t][g * 4 + 3] * inv;
        if constexpr (LIN) {
          // O = alpha * Os + (1 - alpha) * Ol, alpha per (head, channel)
          const int h = bh % a.H;
          const float4 al = *reinterpret_cast<const float4 *>(a.alpha + (size_t)h * D + d);
          const float4 lv = *reinterpret_cast<const float4 *>(a.ol + head + (size_t)qi * D + d);
          o0 = al.x * o0 + (1.f - al.x) * lv.x;
          o1 = al.y * o1 + (1.f - al.y) * lv.y;
          o2 = al.z * o2 + (1.f - al.z) * lv.z;
          o3 = al.w * o3 + (1.f - al.w) * lv.w;
        }
        *reinterpret_cast<uint2 *>(orow + d) = pack4(o0, o1, o2, o3);
      }
    if (a.lse && hf == 0) a.lse[(size_t)bh * N + qi] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
  }
}

template <int D, bool LIN>
hipError_t launch_d(const FwdArgs &a, hipStream_t s) {
  const int R = a.B * a.H * a.n_qblk;
  if (a.block_q == 128)
    sparse_fwd_bf16_kernel<D, 4, LIN><<<R, 256, 0, s>>>(a);
  else
    sparse_fwd_bf16_kernel<D, 2, LIN><<<R, 128, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t s) {
  const bool lin = a.alpha != nullptr;
  if (a.D == 128) return lin ? launch_d<128, true>(a, s) : launch_d<128, false>(a, s);
  return lin ? launch_d<64, true>(a, s) : launch_d<64, false>(a, s);
}

}  // namespace sa
