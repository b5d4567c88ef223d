// Block-sparse attention forward for gfx950 (SpargeAttention2 page, section 2(3): the
// kernel visits only the kept Q x KV tiles, so masked tiles cost neither matrix products
// nor softmax work; Veda page, section 2.3, likewise fetches non-contiguous K/V tiles
// while the matrix units work).
//
// One workgroup per query block (row of the CSR mask), one wave per 32 queries. Per kept
// 64-key tile:
//   S^T = K Q^T        on MFMA (32x32 output per instruction); with S transposed, each
//                      lane holds the scores of one query, so the online-softmax max and
//                      sum are in-lane plus one exchange between the two lane halves;
//   online softmax     in the log2 domain, fp32;
//   O^T += V^T P^T     on MFMA; the output keeps one query per lane, so the rescale of
//                      the accumulator by exp2(m_old - m_new) is in-lane as well.
// K tiles are staged row-major in LDS; V tiles are transposed on the way into LDS so the
// V^T operand is a pair of 8-byte reads. The next tile's global loads are issued before
// the current tile's math.
// This kernel serves fp32 inputs (fp64 scores and running max on the VALU, fp32 MFMA
// for P V); bf16 inputs use the tuned kernel in sparse_fwd_bf16.hip.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sa_internal.h"

namespace sa {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBk = 64;    // keys per KV tile
constexpr int kVec = 4;    // fp32 elements per 16-byte load
constexpr int kKPad = 4;   // LDS row padding of the K tile (elements)
constexpr int kVPad = 4;   // LDS row padding of the V^T tile (elements)

__device__ __forceinline__ void store4(float *dst, float a, float b, float c, float d) {
  *reinterpret_cast<float4 *>(dst) = make_float4(a, b, c, d);
}

// Workgroup -> row: consecutive workgroup ids go round-robin over the 8 XCDs, so the
// ids are regrouped to give each XCD a contiguous range of rows (neighbouring query
// blocks of one head share most kept K/V tiles, which then stay in that XCD's L2).
__device__ __forceinline__ int xcd_remap(int b, int G) {
  const int q = G / 8;
  if (b >= q * 8) return b;
  return (b % 8) * q + b / 8;
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void sparse_fwd_kernel(FwdArgs a) {
  using T = float;
  constexpr int NT = 64 * NW;             // threads
  constexpr int BQ = 32 * NW;             // queries per workgroup
  constexpr int VEC = kVec;
  constexpr int KROW = D + kKPad;         // K tile row stride (elements)
  constexpr int VROW = kBk + kVPad;       // V^T tile row stride (elements)
  constexpr int KCH = kBk * D / VEC;      // 16-byte chunks per K tile
  constexpr int KPT = (KCH + NT - 1) / NT;
  constexpr int VCH = (kBk / 4) * (D / VEC);  // 4-row chunks per V tile
  constexpr int VPT = (VCH + NT - 1) / NT;
  constexpr int DT = D / 32;              // 32-channel groups of O^T

  __shared__ __align__(16) T ks[kBk * KROW];
  __shared__ __align__(16) T vt[D * VROW];

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
  const T *qg = reinterpret_cast<const T *>(a.q) + head;
  const T *kg = reinterpret_cast<const T *>(a.k) + head;
  const T *vg = reinterpret_cast<const T *>(a.v) + head;
  T *og = reinterpret_cast<T *>(a.o) + head;

  const int q0 = I * BQ + wid * 32;    // first query of this wave
  const int qi = q0 + l32;             // this lane's query
  const bool q_ok = qi < N;

  const int beg = a.row_ptr[row];
  const int end = a.row_ptr[row + 1];

  if (beg == end) {
    // no kept tile: O = 0, LSE = -inf
    if (q_ok) {
      for (int d = hf * (D / 2); d < (hf + 1) * (D / 2); d += 4)
        store4(og + (size_t)qi * D + d, 0.f, 0.f, 0.f, 0.f);
      if (a.lse && hf == 0) a.lse[(size_t)bh * N + qi] = -INFINITY;
    }
    return;
  }

  // the lane's whole query row (scores are formed on the VALU in fp64)
  float qf[D];
#pragma unroll
  for (int s = 0; s < D; ++s) qf[s] = q_ok ? qg[(size_t)qi * D + s] : 0.0f;

  // staging registers for one K/V tile
  uint4 kr[KPT];
  uint4 vr[VPT][4];

  auto load_tile = [&](int J) {
    const int j0 = J * kBk;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int c = tid + u * NT;
      kr[u] = make_uint4(0, 0, 0, 0);
      if (c < KCH) {
        const int r = c / (D / VEC), col = (c % (D / VEC)) * VEC;
        if (j0 + r < N) kr[u] = *reinterpret_cast<const uint4 *>(kg + (size_t)(j0 + r) * D + col);
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int c = tid + u * NT;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) vr[u][rr] = make_uint4(0, 0, 0, 0);
      if (c < VCH) {
        const int kgp = c / (D / VEC), col = (c % (D / VEC)) * VEC;
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
        const int r = c / (D / VEC), col = (c % (D / VEC)) * VEC;
        *reinterpret_cast<uint4 *>(&ks[r * KROW + col]) = kr[u];
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int c = tid + u * NT;
      if (c < VCH) {
        const int kgp = c / (D / VEC), col = (c % (D / VEC)) * VEC;
        const uint32_t *w0 = reinterpret_cast<const uint32_t *>(&vr[u][0]);
        const uint32_t *w1 = reinterpret_cast<const uint32_t *>(&vr[u][1]);
        const uint32_t *w2 = reinterpret_cast<const uint32_t *>(&vr[u][2]);
        const uint32_t *w3 = reinterpret_cast<const uint32_t *>(&vr[u][3]);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          uint4 t4 = make_uint4(w0[m], w1[m], w2[m], w3[m]);
          *reinterpret_cast<uint4 *>(&vt[(col + m) * VROW + kgp * 4]) = t4;
        }
      }
    }
  };

  floatx16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[t][i] = 0.0f;
  double m_run = -INFINITY;  // running max of the raw fp64 scores
  float l_run = 0.0f;       // this lane's part of the running sum
  const double sl2d = (double)a.scale_log2_f64;

  load_tile(a.col_idx[beg]);

  for (int it = beg; it < end; ++it) {
    const int J = a.col_idx[it];
    __syncthreads();
    store_tile();
    __syncthreads();
    if (it + 1 < end) load_tile(a.col_idx[it + 1]);

    // ---- S^T = K Q^T for 64 keys x 32 queries (two 32-key blocks)
    floatx16 sacc[2];
    const int j0 = J * kBk;
    // fp32 inputs: scores in fp64 (exact products, fp64 sums), so large logits keep
    // their small differences; the same (key, query) layout as the MFMA output.
    double sd[2][16];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kt * 32 + (i / 4) * 8 + hf * 4 + (i % 4);
        const float *krow = reinterpret_cast<const float *>(&ks[key * KROW]);
        double acc = 0.0;
#pragma unroll
        for (int d = 0; d < D; d += 4) {
          const float4 kv = *reinterpret_cast<const float4 *>(krow + d);
          acc = fma((double)qf[d], (double)kv.x, acc);
          acc = fma((double)qf[d + 1], (double)kv.y, acc);
          acc = fma((double)qf[d + 2], (double)kv.z, acc);
          acc = fma((double)qf[d + 3], (double)kv.w, acc);
        }
        sd[kt][i] = (j0 + key < N) ? acc : -INFINITY;
      }
    double mx = sd[0][0];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmax(mx, sd[kt][i]);
    mx = fmax(mx, __shfl_xor(mx, 32));
    const double m_new = fmax(m_run, mx);
    const float corr = exp2f((float)((m_run - m_new) * sl2d));
    m_run = m_new;
    float psum = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = exp2f((float)((sd[kt][i] - m_new) * sl2d));
        sacc[kt][i] = pv;
        psum += pv;
      }
    l_run = l_run * corr + psum;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[t][i] *= corr;

    // ---- O^T += V^T P^T. MFMA reduction index kk = hf*8 + e (e < 8) stands for key
    // base + (e/4)*8 + hf*4 + e%4, which is where the S^T layout put this lane's values.
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kt * 32 + (i / 4) * 8 + hf * 4 + (i % 4);
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const float av = vt[(t * 32 + l32) * VROW + key];
          oacc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, sacc[kt][i], oacc[t], 0, 0, 0);
        }
      }
  }

  // ---- epilogue: normalise and store
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (q_ok) {
    T *orow = og + (size_t)qi * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = t * 32 + g * 8 + hf * 4;
        float o0 = oacc[t][g * 4 + 0] * inv, o1 = oacc[t][g * 4 + 1] * inv;
        float o2 = oacc[t][g * 4 + 2] * inv, o3 = oacc[t][g * 4 + 3] * inv;
        store4(orow + d, o0, o1, o2, o3);
      }
    if (a.lse && hf == 0)
      a.lse[(size_t)bh * N + qi] = (float)((m_run * sl2d + (double)log2f(l_tot)) * 0.6931471805599453);
  }
}

template <int D>
hipError_t launch_t(const FwdArgs &a, hipStream_t s) {
  const int R = a.B * a.H * a.n_qblk;
  if (a.block_q == 128)
    sparse_fwd_kernel<D, 4><<<R, 256, 0, s>>>(a);
  else
    sparse_fwd_kernel<D, 2><<<R, 128, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs &a, sa_dtype dt, hipStream_t s) {
  if (dt == SA_BF16) return launch_fwd_bf16(a, s);
  if (a.alpha != nullptr) return hipErrorNotSupported;
  return a.D == 128 ? launch_t<128>(a, s) : launch_t<64>(a, s);
}

}  // namespace sa
