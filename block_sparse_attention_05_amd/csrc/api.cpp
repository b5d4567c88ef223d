// C ABI of the block-sparse attention library: argument validation, workspace layout
// and kernel launches. Every check runs on the host before the first launch.

#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "sa_internal.h"

using namespace sa;

// Scratch of sparse_attn_pipelined_noalloc: the plan workspace of one chunk of heads at a
// time. Every device the library runs on holds its own copy for the life of the process.
// Host code never passes this name to a kernel (on the host it only stands for the
// symbol): it uses the device address that hipGetSymbolAddress returns for the current
// device, kept per device below.
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

struct Shape {
  int B, H, N, D, bq, bk, nQ, nKV;
  long R;
};

sa_status check_shape(int B, int H, int N, int D, int bq, int bk, Shape *sh) {
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || bq <= 0 || bk <= 0) return SA_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return SA_ERR_UNSUPPORTED;
  if (bq != 64 && bq != 128) return SA_ERR_UNSUPPORTED;
  if (bk != 64) return SA_ERR_UNSUPPORTED;
  const int nQ = ceil_div(N, bq), nKV = ceil_div(N, bk);
  if (nKV > kMaxKvBlocks) return SA_ERR_UNSUPPORTED;
  const long R = (long)B * H * nQ;
  if (R * (long)nKV >= (1L << 31)) return SA_ERR_UNSUPPORTED;
  if ((long)B * H > 65535) return SA_ERR_UNSUPPORTED;
  *sh = Shape{B, H, N, D, bq, bk, nQ, nKV, R};
  return SA_OK;
}

bool dtype_ok(int dt) { return dt == SA_BF16 || dt == SA_FP32; }

// Plan workspace layout (each piece 256-byte aligned).
struct PlanLayout {
  size_t row_ptr, col_idx, row_order, counts, bitmap, qbar, kbar, scores, nnz, total;
};

PlanLayout plan_layout(const Shape &s) {
  PlanLayout L;
  const size_t nwords = (size_t)ceil_div(s.nKV, 32);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.row_ptr = take((size_t)(s.R + 1) * 4);
  L.col_idx = take((size_t)s.R * s.nKV * 4);
  L.row_order = take((size_t)s.R * 4);
  L.counts = take((size_t)s.R * 4);
  L.bitmap = take((size_t)s.R * nwords * 4);
  L.qbar = take((size_t)s.B * s.H * s.nQ * s.D * 4);
  L.kbar = take((size_t)s.B * s.H * s.nKV * s.D * 4);
  L.scores = take((size_t)s.B * s.H * s.nQ * s.nKV * 4);
  L.nnz = take(8);
  L.total = off;
  return L;
}

sa_status check_ws(const void *ws, size_t have, size_t need) {
  if (need == 0) return SA_OK;
  if (ws == nullptr || have < need) return SA_ERR_WORKSPACE;
  if (((uintptr_t)ws) % kAlign != 0) return SA_ERR_WORKSPACE;
  return SA_OK;
}

void fill_plan(sa_plan *p, const Shape &s, int dt, char *ws, const PlanLayout &L) {
  p->B = s.B;
  p->H = s.H;
  p->N = s.N;
  p->D = s.D;
  p->block_q = s.bq;
  p->block_kv = s.bk;
  p->n_qblk = s.nQ;
  p->n_kvblk = s.nKV;
  p->dtype = dt;
  p->reserved = 0;
  p->row_ptr = reinterpret_cast<int32_t *>(ws + L.row_ptr);
  p->col_idx = reinterpret_cast<int32_t *>(ws + L.col_idx);
  p->row_order = reinterpret_cast<int32_t *>(ws + L.row_order);
  p->q_order = nullptr;
  p->kv_order = nullptr;
  p->visit = nullptr;
  p->nnz = reinterpret_cast<int64_t *>(ws + L.nnz);
}

sa_status hip_status(hipError_t e) { return e == hipSuccess ? SA_OK : SA_ERR_HIP; }

// Linear-branch workspace: per head H (fp32 [D, D]) and z (fp32 [D]), the per-chunk
// partials of both (fp32), phi(K) (bf16, padded to whole KV blocks), and per plan row the
// masked-out sums H_C^T (bf16 [D, D]) and z_C (fp32 [D]).
struct FwdLayout {
  size_t lin_h, lin_z, partial, hct, zc, phik, total;
  int chunks, n_pad;
};

FwdLayout fwd_layout(const Shape &s, int with_linear) {
  FwdLayout L{0, 0, 0, 0, 0, 0, 0, 0, 0};
  if (!with_linear) return L;
  const size_t BH = (size_t)s.B * s.H;
  L.chunks = linear_prepass_chunks(s.N);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.n_pad = s.nKV * 64;
  L.lin_h = take(BH * s.D * s.D * 4);
  L.lin_z = take(BH * s.D * 4);
  L.partial = take(BH * (size_t)L.chunks * s.D * (s.D + 1) * 4);
  L.hct = take((size_t)s.R * s.D * s.D * 2);
  L.zc = take((size_t)s.R * s.D * 4);
  L.phik = take(BH * (size_t)L.n_pad * s.D * 2);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

size_t sparse_attn_plan_workspace_bytes(int B, int H, int N, int D, int block_q, int block_kv) {
  Shape s;
  if (check_shape(B, H, N, D, block_q, block_kv, &s) != SA_OK) return 0;
  return plan_layout(s).total;
}

namespace {
// pooled, masked: NULL, or events recorded on `stream` once the pooling is done and once
// the CSR is written (before the work order), for work on another stream that should
// start after the pooling or needs the mask but not the order.
sa_status plan_impl(const void *q, const void *k, sa_dtype dtype, int B, int H, int N, int D,
                    int block_q, int block_kv, double topk_frac, double top_p,
                    const int32_t *q_order, const int32_t *kv_order, void *workspace, size_t ws_bytes,
                    sa_plan *out, hipStream_t stream, hipEvent_t pooled = nullptr,
                    hipEvent_t masked = nullptr) {
  if (q == nullptr || k == nullptr || out == nullptr) return SA_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return SA_ERR_INVALID_ARG;
  if (!(topk_frac >= 0.0 && topk_frac <= 1.0)) return SA_ERR_INVALID_ARG;
  if (!(top_p >= 0.0 && top_p <= 1.0)) return SA_ERR_INVALID_ARG;
  Shape s;
  sa_status st = check_shape(B, H, N, D, block_q, block_kv, &s);
  if (st != SA_OK) return st;
  const PlanLayout L = plan_layout(s);
  st = check_ws(workspace, ws_bytes, L.total);
  if (st != SA_OK) return st;

  // top-k count and the fp32 threshold factor, fixed on the host in one place
  double mk = ceil(topk_frac * (double)s.nKV - 1e-9);
  if (mk < 1.0) mk = 1.0;
  if (mk > s.nKV) mk = s.nKV;
  const int m_k = (int)mk;
  const float p32 = (float)top_p;
  const int p_all = top_p >= 1.0 ? 1 : 0;
  const float c = (float)(1.0 / sqrt((double)D));

  char *ws = static_cast<char *>(workspace);
  float *qbar = reinterpret_cast<float *>(ws + L.qbar);
  float *kbar = reinterpret_cast<float *>(ws + L.kbar);
  float *scores = reinterpret_cast<float *>(ws + L.scores);
  uint32_t *bitmap = reinterpret_cast<uint32_t *>(ws + L.bitmap);
  int32_t *counts = reinterpret_cast<int32_t *>(ws + L.counts);
  sa_plan p;
  fill_plan(&p, s, dtype, ws, L);
  const int BH = B * H;
  const int nwords = ceil_div(s.nKV, 32);

  p.q_order = q_order;
  p.kv_order = kv_order;
  p.visit = reinterpret_cast<int32_t *>(scores);   // the select kernel's visit lists
  hipError_t e = launch_pool(q, dtype, BH, H, N, D, block_q, q_order, qbar, stream);
  if (e == hipSuccess) e = launch_pool(k, dtype, BH, H, N, D, block_kv, kv_order, kbar, stream);
  if (e == hipSuccess && pooled != nullptr) e = hipEventRecord(pooled, stream);
  if (e == hipSuccess) e = launch_scores(qbar, kbar, BH, s.nQ, s.nKV, D, c, scores, stream);
  if (e == hipSuccess)
    e = launch_select(scores, (int)s.R, s.nKV, N % block_kv != 0, m_k, p32, p_all, bitmap, nwords, counts,
                      stream);
  if (e == hipSuccess) e = launch_scan(counts, (int)s.R, p.row_ptr, p.nnz, stream);
  if (e == hipSuccess) e = launch_fill(bitmap, nwords, p.row_ptr, (int)s.R, p.col_idx, stream);
  if (e == hipSuccess && masked != nullptr) e = hipEventRecord(masked, stream);
  if (e == hipSuccess)
    e = launch_row_order(p.row_ptr, (int)s.R, s.nQ, p.row_order, stream);
  if (e != hipSuccess) return SA_ERR_HIP;
  *out = p;
  return SA_OK;
}
}  // namespace

sa_status sparse_attn_plan(const void *q, const void *k, sa_dtype dtype, int B, int H, int N,
                           int D, int block_q, int block_kv, double topk_frac, double top_p,
                           void *workspace, size_t ws_bytes, sa_plan *out, hipStream_t stream) {
  return plan_impl(q, k, dtype, B, H, N, D, block_q, block_kv, topk_frac, top_p, nullptr, nullptr,
                   workspace, ws_bytes, out, stream);
}

sa_status sparse_attn_plan_ordered(const void *q, const void *k, sa_dtype dtype, int B, int H,
                                   int N, int D, int block_q, int block_kv, double topk_frac,
                                   double top_p, const int32_t *q_order, const int32_t *kv_order,
                                   void *workspace, size_t ws_bytes, sa_plan *out, hipStream_t stream) {
  if (q_order == nullptr) return SA_ERR_INVALID_ARG;
  if (dtype == SA_FP32) return SA_ERR_UNSUPPORTED;
  return plan_impl(q, k, dtype, B, H, N, D, block_q, block_kv, topk_frac, top_p, q_order, kv_order,
                   workspace, ws_bytes, out, stream);
}

sa_status sparse_attn_plan_dense(sa_dtype dtype, int B, int H, int N, int D, int block_q,
                                 int block_kv, void *workspace, size_t ws_bytes, sa_plan *out,
                                 hipStream_t stream) {
  if (out == nullptr || !dtype_ok(dtype)) return SA_ERR_INVALID_ARG;
  Shape s;
  sa_status st = check_shape(B, H, N, D, block_q, block_kv, &s);
  if (st != SA_OK) return st;
  const PlanLayout L = plan_layout(s);
  st = check_ws(workspace, ws_bytes, L.total);
  if (st != SA_OK) return st;
  sa_plan p;
  fill_plan(&p, s, dtype, static_cast<char *>(workspace), L);
  hipError_t e = launch_dense_plan((int)s.R, s.nKV, p.row_ptr, p.col_idx, p.nnz, stream);
  if (e == hipSuccess)
    e = launch_row_order(p.row_ptr, (int)s.R, s.nQ, p.row_order, stream);
  if (e != hipSuccess) return SA_ERR_HIP;
  *out = p;
  return SA_OK;
}

sa_status sparse_attn_plan_from_csr(sa_dtype dtype, int B, int H, int N, int D, int block_q,
                                    int block_kv, const int32_t *host_row_ptr,
                                    const int32_t *host_col_idx, void *workspace,
                                    size_t ws_bytes, sa_plan *out, hipStream_t stream) {
  if (out == nullptr || host_row_ptr == nullptr || !dtype_ok(dtype)) return SA_ERR_INVALID_ARG;
  Shape s;
  sa_status st = check_shape(B, H, N, D, block_q, block_kv, &s);
  if (st != SA_OK) return st;
  const PlanLayout L = plan_layout(s);
  st = check_ws(workspace, ws_bytes, L.total);
  if (st != SA_OK) return st;
  // validate the caller's CSR
  if (host_row_ptr[0] != 0) return SA_ERR_BAD_CSR;
  for (long r = 0; r < s.R; ++r) {
    const int32_t a = host_row_ptr[r], b = host_row_ptr[r + 1];
    if (b < a || b - a > s.nKV) return SA_ERR_BAD_CSR;
  }
  const long nnz = host_row_ptr[s.R];
  if (nnz > 0 && host_col_idx == nullptr) return SA_ERR_INVALID_ARG;
  for (long r = 0; r < s.R; ++r) {
    for (int32_t i = host_row_ptr[r]; i < host_row_ptr[r + 1]; ++i) {
      const int32_t c = host_col_idx[i];
      if (c < 0 || c >= s.nKV) return SA_ERR_BAD_CSR;
      if (i > host_row_ptr[r] && c <= host_col_idx[i - 1]) return SA_ERR_BAD_CSR;
    }
  }
  sa_plan p;
  char *ws = static_cast<char *>(workspace);
  fill_plan(&p, s, dtype, ws, L);
  hipError_t e = hipMemcpyAsync(p.row_ptr, host_row_ptr, (size_t)(s.R + 1) * 4,
                                hipMemcpyHostToDevice, stream);
  if (e == hipSuccess && nnz > 0)
    e = hipMemcpyAsync(p.col_idx, host_col_idx, (size_t)nnz * 4, hipMemcpyHostToDevice, stream);
  const int64_t nnz64 = nnz;   // read by the copy before the synchronisation below
  if (e == hipSuccess) e = hipMemcpyAsync(p.nnz, &nnz64, 8, hipMemcpyHostToDevice, stream);
  // the host arrays may be pageable and reused as soon as this call returns
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e == hipSuccess)
    e = launch_row_order(p.row_ptr, (int)s.R, s.nQ, p.row_order, stream);
  if (e != hipSuccess) return SA_ERR_HIP;
  *out = p;
  return SA_OK;
}

size_t sparse_attn_fwd_workspace_bytes(const sa_plan *plan, int with_linear) {
  if (plan == nullptr) return 0;
  Shape s;
  if (check_shape(plan->B, plan->H, plan->N, plan->D, plan->block_q, plan->block_kv, &s) != SA_OK) return 0;
  return fwd_layout(s, with_linear).total;
}

}  // extern "C"

namespace {
// The forward in three parts that the pipelined call runs apart: the linear branch's
// prepass (k and v only, no plan needed on the device), its apply step (needs the mask's
// CSR, not the plan's work order) and the attention. sparse_attn_fwd runs all three.
// alpha_h0 / alpha_H: head h of this call takes alpha row (alpha_h0 + h) % alpha_H (0 and
// H for a whole tensor).
enum { kPartPrepass = 1, kPartApply = 2, kPartAttention = 4 };
sa_status fwd_impl(const void *q, const void *k, const void *v, sa_dtype dtype, int B, int H, int N, int D,
                   const sa_plan *plan, const float *alpha, int alpha_h0, int alpha_H, void *o, float *lse,
                   void *workspace, size_t ws_bytes, hipStream_t stream, int parts) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || plan == nullptr)
    return SA_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return SA_ERR_INVALID_ARG;
  Shape s;
  sa_status st = check_shape(B, H, N, D, plan->block_q, plan->block_kv, &s);
  if (st != SA_OK) return st;
  if (plan->B != B || plan->H != H || plan->N != N || plan->D != D || plan->dtype != dtype ||
      plan->n_qblk != s.nQ || plan->n_kvblk != s.nKV)
    return SA_ERR_PLAN_MISMATCH;
  if (plan->row_ptr == nullptr || plan->col_idx == nullptr) return SA_ERR_INVALID_ARG;
  const FwdLayout L = fwd_layout(s, alpha != nullptr);
  st = check_ws(workspace, ws_bytes, L.total);
  if (st != SA_OK) return st;
  if (alpha != nullptr && dtype != SA_BF16) return SA_ERR_UNSUPPORTED;  // linear branch: bf16

  FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.row_ptr = plan->row_ptr;
  a.col_idx = plan->col_idx;
  a.row_order = plan->row_order;
  a.visit = plan->visit;
  a.q_order = plan->q_order;
  a.kv_order = plan->kv_order;
  if ((a.q_order != nullptr || a.kv_order != nullptr) && dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  if (a.kv_order != nullptr && alpha != nullptr) return SA_ERR_UNSUPPORTED;
  a.B = B;
  a.H = H;
  a.N = N;
  a.D = D;
  a.block_q = s.bq;
  a.block_kv = s.bk;
  a.n_qblk = s.nQ;
  a.n_kvblk = s.nKV;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  a.scale_log2_f64 = 1.4426950408889634 / sqrt((double)D);
  a.alpha = nullptr;
  a.alpha_h0 = 0;
  a.alpha_H = 1;
  a.hct = nullptr;
  a.zc = nullptr;
  if (alpha != nullptr) {
    char *ws = static_cast<char *>(workspace);
    LinearBufs lb;
    lb.partial = reinterpret_cast<float *>(ws + L.partial);
    lb.chunks = L.chunks;
    lb.phik = reinterpret_cast<uint16_t *>(ws + L.phik);
    lb.n_pad = L.n_pad;
    lb.h = reinterpret_cast<float *>(ws + L.lin_h);
    lb.z = reinterpret_cast<float *>(ws + L.lin_z);
    lb.hct = reinterpret_cast<uint16_t *>(ws + L.hct);
    lb.zc = reinterpret_cast<float *>(ws + L.zc);
    hipError_t e = hipSuccess;
    if (parts & kPartPrepass) e = launch_linear_prepass(k, v, dtype, B * H, N, D, lb, stream);
    if (e == hipSuccess && (parts & kPartApply)) e = launch_linear_apply(a, lb, stream);
    if (e != hipSuccess) return SA_ERR_HIP;
    a.alpha = alpha;
    a.alpha_h0 = alpha_h0;
    a.alpha_H = alpha_H;
    a.hct = lb.hct;
    a.zc = lb.zc;
  }
  if (!(parts & kPartAttention)) return SA_OK;
  return hip_status(launch_fwd(a, dtype, stream));
}
}  // namespace

extern "C" {

sa_status sparse_attn_fwd(const void *q, const void *k, const void *v, sa_dtype dtype, int B,
                          int H, int N, int D, const sa_plan *plan, const float *alpha, void *o,
                          float *lse, void *workspace, size_t ws_bytes, hipStream_t stream) {
  return fwd_impl(q, k, v, dtype, B, H, N, D, plan, alpha, 0, H, o, lse, workspace, ws_bytes, stream,
                  kPartPrepass | kPartApply | kPartAttention);
}

namespace {
// Events that order the pipelined call's two streams, made once per thread and device and
// reused by every later call. Re-recording an event is safe while earlier waits on it are
// still pending: a wait takes the record that precedes it. Never destroyed (they live as
// long as the thread's HIP context); NULL when an event cannot be made.
hipEvent_t *pipeline_events(int n) {
  struct Pool {
    int device = -1;
    std::vector<hipEvent_t> ev;
  };
  thread_local std::vector<Pool> pools;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  Pool *p = nullptr;
  for (auto &x : pools)
    if (x.device == dev) p = &x;
  if (p == nullptr) {
    pools.push_back(Pool{});
    p = &pools.back();
    p->device = dev;
  }
  while ((int)p->ev.size() < n) {
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return nullptr;
    p->ev.push_back(e);
  }
  return p->ev.data();
}

// The pipelined call splits the B*H heads into chunks of `per` heads, each planned in its
// own plan workspace; with the linear branch one forward workspace for a chunk follows
// (the chunks' forwards run in order on one stream and reuse it).
struct PipeLayout {
  int C, per;
  size_t plan_bytes, lin_off, total;
};
sa_status pipe_layout(int B, int H, int N, int D, int bq, int bk, int n_chunks, int with_linear,
                      PipeLayout *L) {
  Shape s;
  sa_status st = check_shape(B, H, N, D, bq, bk, &s);
  if (st != SA_OK) return st;
  if (n_chunks < 1) return SA_ERR_INVALID_ARG;
  const int BH = B * H;
  L->per = ceil_div(BH, n_chunks < BH ? n_chunks : BH);
  L->C = ceil_div(BH, L->per);
  Shape s1;
  st = check_shape(1, L->per, N, D, bq, bk, &s1);
  if (st != SA_OK) return st;
  L->plan_bytes = plan_layout(s1).total;
  L->lin_off = align_up(L->plan_bytes * L->C);
  L->total = L->lin_off + (with_linear ? fwd_layout(s1, 1).total : 0);
  return SA_OK;
}
}  // namespace

size_t sparse_attn_pipelined_workspace_bytes(int B, int H, int N, int D, int block_q, int block_kv,
                                             int n_chunks, int with_linear) {
  PipeLayout L;
  if (pipe_layout(B, H, N, D, block_q, block_kv, n_chunks, with_linear, &L) != SA_OK) return 0;
  return L.total;
}

sa_status sparse_attn_pipelined(const void *q, const void *k, const void *v, sa_dtype dtype, int B, int H,
                                int N, int D, int block_q, int block_kv, double topk_frac, double top_p,
                                int n_chunks, const float *alpha, void *o, float *lse, void *workspace,
                                size_t ws_bytes, hipStream_t stream, hipStream_t aux_stream) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return SA_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return SA_ERR_INVALID_ARG;
  if (!(topk_frac >= 0.0 && topk_frac <= 1.0) || !(top_p >= 0.0 && top_p <= 1.0)) return SA_ERR_INVALID_ARG;
  if (alpha != nullptr && dtype != SA_BF16) return SA_ERR_UNSUPPORTED;  // linear branch: bf16
  PipeLayout L;
  sa_status st = pipe_layout(B, H, N, D, block_q, block_kv, n_chunks, alpha != nullptr, &L);
  if (st != SA_OK) return st;
  st = check_ws(workspace, ws_bytes, L.total);
  if (st != SA_OK) return st;

  const int BH = B * H;
  const size_t esz = dtype == SA_BF16 ? 2 : 4;
  const size_t head_bytes = (size_t)N * D * esz;
  auto chunk = [&](int c, const char *base) { return base + (size_t)c * L.per * head_bytes; };
  const bool two = aux_stream != stream;
  // Plans go on aux_stream back to back; forwards on `stream`, each after its chunk's plan.
  // Only the first plan is exposed; the others run under the forwards before them.
  // ev[c]: chunk c's plan done; ev[L.C]: the caller's earlier work; with the linear branch
  // ev[L.C + 1 + c]: chunk c's CSR written (its apply step waits only for that) and
  // ev[2 L.C + 1 + c]: chunk c's pooling done (its prepass starts after it, so that it
  // shares the chip with the score and select kernels rather than with the pooling, which
  // heads the critical chain)
  hipEvent_t *ev = nullptr;
  if (two) {
    ev = pipeline_events(alpha ? 3 * L.C + 1 : L.C + 1);
    if (ev == nullptr) return SA_ERR_HIP;
    // the plans start after the caller's earlier work on `stream` (inputs written there)
    if (hipEventRecord(ev[L.C], stream) != hipSuccess || hipStreamWaitEvent(aux_stream, ev[L.C], 0) != hipSuccess)
      return SA_ERR_HIP;
  }
  std::vector<sa_plan> plans(L.C);
  for (int c = 0; c < L.C && st == SA_OK; ++c) {
    const int hc = BH - c * L.per < L.per ? BH - c * L.per : L.per;
    char *ws = static_cast<char *>(workspace) + c * L.plan_bytes;
    st = plan_impl(chunk(c, static_cast<const char *>(q)), chunk(c, static_cast<const char *>(k)), dtype, 1, hc,
                   N, D, block_q, block_kv, topk_frac, top_p, nullptr, nullptr, ws, L.plan_bytes, &plans[c],
                   two ? aux_stream : stream, two && alpha ? ev[2 * L.C + 1 + c] : nullptr,
                   two && alpha ? ev[L.C + 1 + c] : nullptr);
    if (st == SA_OK && two && hipEventRecord(ev[c], aux_stream) != hipSuccess) st = SA_ERR_HIP;
  }
  // With the linear branch, chunk c's prepass (k and v only) goes on `stream` before the
  // wait for its plan, so the first one runs beside the first plan.
  char *lin_ws = alpha ? static_cast<char *>(workspace) + L.lin_off : nullptr;
  const size_t lin_bytes = L.total - L.lin_off;
  for (int c = 0; c < L.C && st == SA_OK; ++c) {
    const int hc = BH - c * L.per < L.per ? BH - c * L.per : L.per;
    const char *qc = chunk(c, static_cast<const char *>(q));
    const char *kc = chunk(c, static_cast<const char *>(k));
    const char *vc = chunk(c, static_cast<const char *>(v));
    char *oc = const_cast<char *>(chunk(c, static_cast<const char *>(o)));
    float *lc = lse ? lse + (size_t)c * L.per * N : nullptr;
    const int h0 = (c * L.per) % H;
    if (alpha) {
      if (two && hipStreamWaitEvent(stream, ev[2 * L.C + 1 + c], 0) != hipSuccess) {
        st = SA_ERR_HIP;
        break;
      }
      st = fwd_impl(qc, kc, vc, dtype, 1, hc, N, D, &plans[c], alpha, h0, H, oc, lc, lin_ws, lin_bytes, stream,
                    kPartPrepass);
      if (st == SA_OK && two && hipStreamWaitEvent(stream, ev[L.C + 1 + c], 0) != hipSuccess) st = SA_ERR_HIP;
      if (st == SA_OK)
        st = fwd_impl(qc, kc, vc, dtype, 1, hc, N, D, &plans[c], alpha, h0, H, oc, lc, lin_ws, lin_bytes,
                      stream, kPartApply);
      if (st != SA_OK) break;
    }
    if (two && hipStreamWaitEvent(stream, ev[c], 0) != hipSuccess) {
      st = SA_ERR_HIP;
      break;
    }
    st = fwd_impl(qc, kc, vc, dtype, 1, hc, N, D, &plans[c], alpha, h0, H, oc, lc, lin_ws, lin_bytes, stream,
                  kPartAttention);
  }
  return st;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
char *scratch_ptr[kMaxDevices];

// The current device's address of `scratch`, looked up once per device.
sa_status device_scratch(char **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SA_ERR_HIP;
    scratch_ptr[dev] = static_cast<char *>(p);
  }
  *out = scratch_ptr[dev];
  return SA_OK;
}
}  // namespace

sa_status sparse_attn_pipelined_noalloc(const void *q, const void *k, const void *v, sa_dtype dtype, int B,
                                        int H, int N, int D, int block_q, int block_kv, double topk_frac,
                                        double top_p, void *o, float *lse, hipStream_t stream) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return SA_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return SA_ERR_INVALID_ARG;
  if (!(topk_frac >= 0.0 && topk_frac <= 1.0) || !(top_p >= 0.0 && top_p <= 1.0)) return SA_ERR_INVALID_ARG;
  Shape s;
  sa_status st = check_shape(B, H, N, D, block_q, block_kv, &s);
  if (st != SA_OK) return st;
  // the largest chunk of heads whose plan workspace fits, then chunks of equal size
  const int BH = B * H;
  auto plan_bytes = [&](int heads) {
    Shape s1;
    return check_shape(1, heads, N, D, block_q, block_kv, &s1) == SA_OK ? plan_layout(s1).total : (size_t)-1;
  };
  if (plan_bytes(1) > kScratchBytes) return SA_ERR_WORKSPACE;   // one head's plan does not fit
  int per = 1;
  while (per < BH && plan_bytes(per + 1) <= kScratchBytes) ++per;
  const int C = ceil_div(BH, per);
  per = ceil_div(BH, C);
  char *ws = nullptr;
  st = device_scratch(&ws);
  if (st != SA_OK) return st;
  const size_t esz = dtype == SA_BF16 ? 2 : 4;
  const size_t head_bytes = (size_t)N * D * esz;
  // one stream: chunk c's plan follows chunk c-1's forward, so the chunks share the scratch
  for (int c = 0; c < C && st == SA_OK; ++c) {
    const int hc = BH - c * per < per ? BH - c * per : per;
    const size_t off = (size_t)c * per * head_bytes;
    sa_plan p;
    st = plan_impl(static_cast<const char *>(q) + off, static_cast<const char *>(k) + off, dtype, 1, hc, N, D,
                   block_q, block_kv, topk_frac, top_p, nullptr, nullptr, ws, kScratchBytes, &p, stream);
    if (st != SA_OK) break;
    st = sparse_attn_fwd(static_cast<const char *>(q) + off, static_cast<const char *>(k) + off,
                         static_cast<const char *>(v) + off, dtype, 1, hc, N, D, &p, nullptr,
                         static_cast<char *>(o) + off, lse ? lse + (size_t)c * per * N : nullptr, nullptr, 0,
                         stream);
  }
  return st;
}

namespace {
// The q exponent part is sized for 64-query blocks whatever block_q is, and the pack ends
// in a tail of 4*block_q bytes, so packs for block_q 64 and 128 never have the same size;
// both calls require the exact size, which rejects a pack made for another block_q.
struct Fp8Layout {
  size_t q8, k8, vt8, qe, ke, ve, vamax, tail, total;
};
Fp8Layout fp8_layout(const Shape &s) {
  Fp8Layout L{};
  const size_t BH = (size_t)s.B * s.H;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.q8 = take(BH * s.N * s.D);
  L.k8 = take(BH * s.N * s.D);
  L.vt8 = take(BH * s.nKV * s.D * 64);
  L.qe = take(BH * ceil_div(s.N, 64) * 4);
  L.ke = take(BH * s.nKV * 4);
  L.ve = take(BH * s.D * 4);
  L.vamax = take(BH * s.D * 4);
  L.tail = take((size_t)s.bq * 4);
  L.total = off;
  return L;
}
}  // namespace

size_t sparse_attn_fp8_pack_bytes(int B, int H, int N, int D, int block_q, int block_kv) {
  Shape s;
  if (check_shape(B, H, N, D, block_q, block_kv, &s) != SA_OK) return 0;
  return fp8_layout(s).total;
}

sa_status sparse_attn_quantize_fp8(const void *q, const void *k, const void *v, sa_dtype dtype, int B, int H,
                                   int N, int D, int block_q, int block_kv, int qk_format, void *pack,
                                   size_t pack_bytes, hipStream_t stream) {
  if (q == nullptr || k == nullptr || v == nullptr) return SA_ERR_INVALID_ARG;
  if (qk_format != SA_QK_E4M3 && qk_format != SA_QK_INT8) return SA_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return SA_ERR_INVALID_ARG;
  Shape s;
  sa_status st = check_shape(B, H, N, D, block_q, block_kv, &s);
  if (st != SA_OK) return st;
  if (dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  const Fp8Layout L = fp8_layout(s);
  st = check_ws(pack, pack_bytes, L.total);
  if (st != SA_OK) return st;
  if (pack_bytes != L.total) return SA_ERR_WORKSPACE;
  char *pk = static_cast<char *>(pack);
  Fp8Pack p{reinterpret_cast<uint8_t *>(pk + L.q8),   reinterpret_cast<uint8_t *>(pk + L.k8),
            reinterpret_cast<uint8_t *>(pk + L.vt8),  reinterpret_cast<int32_t *>(pk + L.qe),
            reinterpret_cast<int32_t *>(pk + L.ke),   reinterpret_cast<int32_t *>(pk + L.ve),
            reinterpret_cast<uint32_t *>(pk + L.vamax)};
  return hip_status(launch_quantize_fp8(static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                                        static_cast<const uint16_t *>(v), B * H, N, D, s.bq,
                                        qk_format == SA_QK_INT8, p, stream));
}

sa_status sparse_attn_fwd_fp8(const void *pack, size_t pack_bytes, int qk_format, int B, int H, int N, int D,
                              const sa_plan *plan, void *o, float *lse, hipStream_t stream) {
  if (pack == nullptr || plan == nullptr || o == nullptr) return SA_ERR_INVALID_ARG;
  if (qk_format != SA_QK_E4M3 && qk_format != SA_QK_INT8) return SA_ERR_INVALID_ARG;
  Shape s;
  sa_status st = check_shape(B, H, N, D, plan->block_q, plan->block_kv, &s);
  if (st != SA_OK) return st;
  if (plan->B != B || plan->H != H || plan->N != N || plan->D != D || plan->n_qblk != s.nQ ||
      plan->n_kvblk != s.nKV)
    return SA_ERR_PLAN_MISMATCH;
  if (plan->row_ptr == nullptr || plan->col_idx == nullptr) return SA_ERR_INVALID_ARG;
  if (plan->dtype != SA_BF16 || (plan->q_order != nullptr || plan->kv_order != nullptr)) return SA_ERR_UNSUPPORTED;
  const Fp8Layout L = fp8_layout(s);
  st = check_ws(pack, pack_bytes, L.total);
  if (st != SA_OK) return st;
  if (pack_bytes != L.total) return SA_ERR_PLAN_MISMATCH;   // a pack made for another block_q
  const char *pk = static_cast<const char *>(pack);
  Fp8FwdArgs a{};
  a.q8 = reinterpret_cast<const uint8_t *>(pk + L.q8);
  a.k8 = reinterpret_cast<const uint8_t *>(pk + L.k8);
  a.vt8 = reinterpret_cast<const uint8_t *>(pk + L.vt8);
  a.qe = reinterpret_cast<const int32_t *>(pk + L.qe);
  a.ke = reinterpret_cast<const int32_t *>(pk + L.ke);
  a.ve = reinterpret_cast<const int32_t *>(pk + L.ve);
  a.o = static_cast<uint16_t *>(o);
  a.lse = lse;
  a.row_ptr = plan->row_ptr;
  a.col_idx = plan->col_idx;
  a.row_order = plan->row_order;
  a.visit = plan->visit;
  a.B = B;
  a.H = H;
  a.N = N;
  a.D = D;
  a.block_q = s.bq;
  a.n_qblk = s.nQ;
  a.n_kvblk = s.nKV;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  return hip_status(launch_fwd_fp8(a, qk_format == SA_QK_INT8, stream));
}

namespace {
struct BwdLayout {
  size_t dvec, lse2, tbits, ccount, col_ptr, row_idx, col_order, cnnz, total;
  int nwq;
};
BwdLayout bwd_layout(const Shape &s) {
  BwdLayout L{};
  const size_t BH = (size_t)s.B * s.H;
  const size_t C = BH * s.nKV;
  L.nwq = ceil_div(s.nQ, 32);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.dvec = take(BH * (size_t)s.nQ * s.bq * 4);
  L.lse2 = take(BH * (size_t)s.nQ * s.bq * 4);
  L.tbits = take(C * L.nwq * 4);
  L.ccount = take(C * 4);
  L.col_ptr = take((C + 1) * 4);
  L.row_idx = take((size_t)s.R * s.nKV * 4);
  L.col_order = take(C * 4);
  L.cnnz = take(8);
  L.total = off;
  return L;
}
}  // namespace

size_t sparse_attn_bwd_workspace_bytes(int B, int H, int N, int D, int block_q, int block_kv) {
  Shape s;
  if (check_shape(B, H, N, D, block_q, block_kv, &s) != SA_OK) return 0;
  return bwd_layout(s).total;
}

sa_status sparse_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                          const float *lse, const void *dout, sa_dtype dtype, int B, int H,
                          int N, int D, const sa_plan *plan, void *dq, void *dk, void *dv,
                          void *workspace, size_t ws_bytes, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !dout || !plan || !dq || !dk || !dv) return SA_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return SA_ERR_INVALID_ARG;
  Shape s;
  sa_status st = check_shape(B, H, N, D, plan->block_q, plan->block_kv, &s);
  if (st != SA_OK) return st;
  if (plan->B != B || plan->H != H || plan->N != N || plan->D != D || plan->dtype != (int)dtype ||
      plan->row_ptr == nullptr || plan->col_idx == nullptr)
    return SA_ERR_PLAN_MISMATCH;
  if (dtype != SA_BF16 || (plan->q_order != nullptr || plan->kv_order != nullptr)) return SA_ERR_UNSUPPORTED;
  const BwdLayout L = bwd_layout(s);
  st = check_ws(workspace, ws_bytes, L.total);
  if (st != SA_OK) return st;
  char *ws = static_cast<char *>(workspace);
  BwdArgs a{};
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.v = (const uint16_t *)v;
  a.o = (const uint16_t *)o;
  a.dout = (const uint16_t *)dout;
  a.lse = lse;
  a.dvec = reinterpret_cast<float *>(ws + L.dvec);
  a.lse2 = reinterpret_cast<float *>(ws + L.lse2);
  a.NP = s.nQ * s.bq;
  a.dq = (uint16_t *)dq;
  a.dk = (uint16_t *)dk;
  a.dv = (uint16_t *)dv;
  a.row_ptr = plan->row_ptr;
  a.col_idx = plan->col_idx;
  a.row_order = plan->row_order;
  a.col_ptr = reinterpret_cast<int32_t *>(ws + L.col_ptr);
  a.row_idx = reinterpret_cast<int32_t *>(ws + L.row_idx);
  a.col_order = reinterpret_cast<int32_t *>(ws + L.col_order);
  a.B = B;
  a.H = H;
  a.N = N;
  a.D = D;
  a.block_q = s.bq;
  a.n_qblk = s.nQ;
  a.n_kvblk = s.nKV;
  a.scale = (float)(1.0 / sqrt((double)D));
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  BwdBufs w;
  w.tbits = reinterpret_cast<uint32_t *>(ws + L.tbits);
  w.nwq = L.nwq;
  w.ccount = reinterpret_cast<int32_t *>(ws + L.ccount);
  w.cnnz = reinterpret_cast<int64_t *>(ws + L.cnnz);
  return hip_status(launch_bwd(a, w, stream));
}

sa_status sparse_attn_tile_stats(const void *q, const void *k, const float *lse, sa_dtype dtype,
                                 int B, int H, int N, int D, int block_q, int block_kv,
                                 float *tile_max, float *tile_mass, hipStream_t stream) {
  if (q == nullptr || k == nullptr || lse == nullptr) return SA_ERR_INVALID_ARG;
  if (tile_max == nullptr && tile_mass == nullptr) return SA_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return SA_ERR_INVALID_ARG;
  Shape s;
  const sa_status st = check_shape(B, H, N, D, block_q, block_kv, &s);
  if (st != SA_OK) return st;
  if (dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  const float sl2 = (float)(1.4426950408889634 / sqrt((double)D));
  return hip_status(launch_tile_stats(q, k, lse, B * H, H, N, D, s.bq, s.nQ, s.nKV, sl2, tile_max,
                                      tile_mass, stream));
}

sa_status sparse_attn_cube_permute(const void *src, void *dst, sa_dtype dtype, int B, int H, int N,
                                   int D, int T, int Hg, int W, const int32_t *host_cubes,
                                   int inverse, hipStream_t stream) {
  if (src == nullptr || dst == nullptr || host_cubes == nullptr) return SA_ERR_INVALID_ARG;
  if (src == dst) return SA_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return SA_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || T <= 0 || Hg <= 0 || W <= 0) return SA_ERR_INVALID_ARG;
  if (inverse != 0 && inverse != 1) return SA_ERR_INVALID_ARG;
  if ((long)T * Hg * W != (long)N) return SA_ERR_INVALID_ARG;
  const int eb = dtype == SA_BF16 ? 2 : 4;
  if ((D * eb) % 16 != 0 || D > 4096) return SA_ERR_UNSUPPORTED;
  if (H > kMaxCubeHeads || (long)B * H > 65535) return SA_ERR_UNSUPPORTED;
  if ((long)N * (D * eb / 16) >= (1L << 31)) return SA_ERR_UNSUPPORTED;
  CubeTable cubes{};
  for (int h = 0; h < H; ++h)
    for (int a = 0; a < 3; ++a) {
      const int c = host_cubes[h * 3 + a];
      if (c < 1) return SA_ERR_INVALID_ARG;
      cubes.c[h][a] = c;
    }
  return hip_status(launch_cube_permute(src, dst, B * H, H, N, D * eb, T, Hg, W, cubes, inverse, stream));
}

sa_status sparse_attn_cube_order(int H, int T, int Hg, int W, const int32_t *host_cubes,
                                 int32_t *order, hipStream_t stream) {
  if (host_cubes == nullptr || order == nullptr) return SA_ERR_INVALID_ARG;
  if (H <= 0 || T <= 0 || Hg <= 0 || W <= 0) return SA_ERR_INVALID_ARG;
  if (H > kMaxCubeHeads) return SA_ERR_UNSUPPORTED;
  if ((long)T * Hg * W * H >= (1L << 31)) return SA_ERR_UNSUPPORTED;
  CubeTable cubes{};
  for (int h = 0; h < H; ++h)
    for (int a = 0; a < 3; ++a) {
      const int c = host_cubes[h * 3 + a];
      if (c < 1) return SA_ERR_INVALID_ARG;
      cubes.c[h][a] = c;
    }
  return hip_status(launch_cube_order(H, T, Hg, W, cubes, order, stream));
}

sa_status sparse_attn_router_exp(const float *x, float *y, int64_t n, hipStream_t stream) {
  if (n < 0 || (n > 0 && (x == nullptr || y == nullptr))) return SA_ERR_INVALID_ARG;
  if (n == 0) return SA_OK;
  return hip_status(launch_router_exp(x, y, n, stream));
}

const char *sparse_attn_status_string(sa_status status) {
  switch (status) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID_ARG: return "invalid argument";
    case SA_ERR_UNSUPPORTED: return "unsupported shape or option";
    case SA_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case SA_ERR_PLAN_MISMATCH: return "plan does not match the inputs";
    case SA_ERR_BAD_CSR: return "malformed CSR mask";
    case SA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

int sparse_attn_version(void) { return 100; }

}  // extern "C"
