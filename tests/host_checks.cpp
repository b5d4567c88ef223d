// Host-side checks of the C ABI, built with AddressSanitizer on the host code (see
// test_host_asan.py). Every call here returns from host validation before anything
// reaches the HIP runtime, so no GPU is needed; host arrays are allocated at their exact
// sizes, so a validation loop that read past them would be reported. Exit code 0 and the
// line "host checks passed" on success.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../include/sparse_attn.h"

static int failures = 0, checks = 0;

#define EXPECT(expr, want)                                                                   \
  do {                                                                                       \
    ++checks;                                                                                \
    const long got_ = (long)(expr);                                                          \
    if (got_ != (long)(want)) {                                                              \
      ++failures;                                                                            \
      fprintf(stderr, "line %d: %s = %ld, expected %ld\n", __LINE__, #expr, got_, (long)(want)); \
    }                                                                                        \
  } while (0)

// A 256-byte aligned address that is never dereferenced on the host.
static void *const FAKE = reinterpret_cast<void *>(static_cast<uintptr_t>(1) << 40);

// Exact-size heap copy of a host array (AddressSanitizer guards its end).
static int32_t *exact(const std::vector<int32_t> &v) {
  int32_t *p = static_cast<int32_t *>(malloc(v.size() * sizeof(int32_t) + (v.empty() ? 1 : 0)));
  if (!v.empty()) memcpy(p, v.data(), v.size() * sizeof(int32_t));
  return p;
}

static void csr_checks() {
  // 2 heads x 3 query blocks of 64 over N = 190 (ragged): 3 KV blocks of 64
  const int B = 1, H = 2, N = 190, D = 64, bq = 64, bk = 64;
  const int R = B * H * 3, nkv = 3;
  const size_t ws = sparse_attn_plan_workspace_bytes(B, H, N, D, bq, bk);
  EXPECT(ws > 0, 1);
  sa_plan out;
  // a valid CSR up to its last entry, which is out of range: the checks read every entry
  std::vector<int32_t> rp = {0}, ci;
  for (int r = 0; r < R; ++r) {
    for (int j = 0; j <= r % nkv; ++j) ci.push_back(j);
    rp.push_back((int32_t)ci.size());
  }
  ci.back() = nkv;
  int32_t *prp = exact(rp), *pci = exact(ci);
  EXPECT(sparse_attn_plan_from_csr(SA_BF16, B, H, N, D, bq, bk, prp, pci, FAKE, ws, &out, nullptr),
         SA_ERR_BAD_CSR);
  // the same with the last row not ascending
  ci.back() = ci[ci.size() - 2];
  free(pci);
  pci = exact(ci);
  EXPECT(sparse_attn_plan_from_csr(SA_BF16, B, H, N, D, bq, bk, prp, pci, FAKE, ws, &out, nullptr),
         SA_ERR_BAD_CSR);
  free(pci);
  free(prp);
  // row_ptr that decreases in its last step, that does not start at 0, and a row with
  // more entries than KV blocks
  std::vector<int32_t> rp2 = {0, 1, 2, 3, 4, 5, 4};
  prp = exact(rp2);
  pci = exact({0, 0, 0, 0, 0});
  EXPECT(sparse_attn_plan_from_csr(SA_BF16, B, H, N, D, bq, bk, prp, pci, FAKE, ws, &out, nullptr),
         SA_ERR_BAD_CSR);
  free(prp);
  rp2 = {1, 1, 2, 3, 4, 5, 6};
  prp = exact(rp2);
  EXPECT(sparse_attn_plan_from_csr(SA_BF16, B, H, N, D, bq, bk, prp, pci, FAKE, ws, &out, nullptr),
         SA_ERR_BAD_CSR);
  free(prp);
  free(pci);
  rp2 = {0, 4, 4, 4, 4, 4, 4};
  prp = exact(rp2);
  pci = exact({0, 1, 2, 2});
  EXPECT(sparse_attn_plan_from_csr(SA_BF16, B, H, N, D, bq, bk, prp, pci, FAKE, ws, &out, nullptr),
         SA_ERR_BAD_CSR);
  free(prp);
  free(pci);
  // arguments checked before the arrays
  EXPECT(sparse_attn_plan_from_csr(SA_BF16, B, H, N, D, bq, bk, nullptr, nullptr, FAKE, ws, &out, nullptr),
         SA_ERR_INVALID_ARG);
  prp = exact(rp);
  EXPECT(sparse_attn_plan_from_csr(SA_BF16, B, H, N, D, bq, bk, prp, nullptr, FAKE, ws - 1, &out, nullptr),
         SA_ERR_WORKSPACE);
  EXPECT(sparse_attn_plan_from_csr(SA_BF16, B, H, N, D, bq, bk, prp, nullptr, FAKE, ws, &out, nullptr),
         SA_ERR_INVALID_ARG);   // entries but no column array
  free(prp);
}

static void cube_checks() {
  for (int H : {1, 5, 128}) {
    std::vector<int32_t> c(3 * H, 2);
    c.back() = 0;   // the last head's last extent is invalid: every entry is read
    int32_t *pc = exact(c);
    EXPECT(sparse_attn_cube_order(H, 4, 4, 4, pc, static_cast<int32_t *>(FAKE), nullptr), SA_ERR_INVALID_ARG);
    EXPECT(sparse_attn_cube_permute(FAKE, static_cast<char *>(FAKE) + 256, SA_BF16, 1, H, 64, 64, 4, 4, 4, pc, 0,
                                    nullptr),
           SA_ERR_INVALID_ARG);
    free(pc);
  }
  std::vector<int32_t> c(3 * 129, 1);
  int32_t *pc = exact(c);
  EXPECT(sparse_attn_cube_order(129, 4, 4, 4, pc, static_cast<int32_t *>(FAKE), nullptr), SA_ERR_UNSUPPORTED);
  free(pc);
}

static void shape_and_argument_checks() {
  // sizes: supported shapes give a size, unsupported ones 0
  EXPECT(sparse_attn_plan_workspace_bytes(1, 40, 75600, 128, 128, 64) > 0, 1);
  EXPECT(sparse_attn_plan_workspace_bytes(1, 1, 64 * 4096, 64, 64, 64) > 0, 1);
  EXPECT(sparse_attn_plan_workspace_bytes(1, 1, 64 * 4097, 64, 64, 64), 0);
  EXPECT(sparse_attn_plan_workspace_bytes(1, 1, 1000, 96, 64, 64), 0);
  EXPECT(sparse_attn_plan_workspace_bytes(0, 1, 1000, 64, 64, 64), 0);
  EXPECT(sparse_attn_bwd_workspace_bytes(1, 40, 75600, 128, 128, 64) > 0, 1);
  EXPECT(sparse_attn_fp8_pack_bytes(1, 40, 75600, 128, 128, 64) != sparse_attn_fp8_pack_bytes(1, 40, 75600, 128, 64, 64), 1);
  EXPECT(sparse_attn_pipelined_workspace_bytes(1, 40, 75600, 128, 128, 64, 4, 0) > 0, 1);
  EXPECT(sparse_attn_pipelined_workspace_bytes(1, 12, 32760, 128, 128, 64, 1, 1) >
             sparse_attn_pipelined_workspace_bytes(1, 12, 32760, 128, 128, 64, 1, 0), 1);
  EXPECT(sparse_attn_pipelined_workspace_bytes(1, 4, 1000, 64, 64, 64, 0, 0), 0);
  EXPECT(sparse_attn_fwd_workspace_bytes(nullptr, 1), 0);

  sa_plan out;
  const size_t ws = sparse_attn_plan_workspace_bytes(1, 2, 1024, 64, 64, 64);
  EXPECT(sparse_attn_plan(nullptr, FAKE, SA_BF16, 1, 2, 1024, 64, 64, 64, 0.1, 0.9, FAKE, ws, &out, nullptr),
         SA_ERR_INVALID_ARG);
  EXPECT(sparse_attn_plan(FAKE, FAKE, (sa_dtype)7, 1, 2, 1024, 64, 64, 64, 0.1, 0.9, FAKE, ws, &out, nullptr),
         SA_ERR_INVALID_ARG);
  EXPECT(sparse_attn_plan(FAKE, FAKE, SA_BF16, 1, 2, 1024, 64, 64, 64, 1.5, 0.9, FAKE, ws, &out, nullptr),
         SA_ERR_INVALID_ARG);
  EXPECT(sparse_attn_plan(FAKE, FAKE, SA_BF16, 1, 2, 1024, 64, 64, 64, 0.1, 0.9, FAKE, ws - 1, &out, nullptr),
         SA_ERR_WORKSPACE);
  EXPECT(sparse_attn_plan(FAKE, FAKE, SA_BF16, 1, 2, 1024, 64, 64, 64, 0.1, 0.9, (char *)FAKE + 8, ws, &out, nullptr),
         SA_ERR_WORKSPACE);
  EXPECT(sparse_attn_plan(FAKE, FAKE, SA_BF16, 1, 2, 1024, 80, 64, 64, 0.1, 0.9, FAKE, ws, &out, nullptr),
         SA_ERR_UNSUPPORTED);
  EXPECT(sparse_attn_plan_dense(SA_BF16, 1, 2, 1024, 64, 64, 64, FAKE, ws - 1, &out, nullptr), SA_ERR_WORKSPACE);

  // a plan struct describing another shape than the forward's arguments
  sa_plan p;
  memset(&p, 0, sizeof(p));
  p.B = 1; p.H = 2; p.N = 1024; p.D = 64; p.block_q = 64; p.block_kv = 64; p.dtype = SA_BF16;
  p.n_qblk = 16; p.n_kvblk = 16;
  p.row_ptr = static_cast<int32_t *>(FAKE); p.col_idx = static_cast<int32_t *>(FAKE);
  EXPECT(sparse_attn_fwd(FAKE, FAKE, FAKE, SA_BF16, 1, 3, 1024, 64, &p, nullptr, FAKE, nullptr, nullptr, 0, nullptr),
         SA_ERR_PLAN_MISMATCH);
  EXPECT(sparse_attn_fwd(FAKE, FAKE, FAKE, SA_FP32, 1, 2, 1024, 64, &p, nullptr, FAKE, nullptr, nullptr, 0, nullptr),
         SA_ERR_PLAN_MISMATCH);
  EXPECT(sparse_attn_fwd(FAKE, FAKE, FAKE, SA_BF16, 1, 2, 1024, 64, &p, static_cast<float *>(FAKE), FAKE, nullptr,
                         nullptr, 0, nullptr),
         SA_ERR_WORKSPACE);   // the linear branch needs its workspace
  EXPECT(sparse_attn_fwd(FAKE, FAKE, FAKE, SA_BF16, 1, 2, 1024, 64, nullptr, nullptr, FAKE, nullptr, nullptr, 0,
                         nullptr),
         SA_ERR_INVALID_ARG);

  const size_t pw = sparse_attn_pipelined_workspace_bytes(1, 2, 1024, 64, 64, 64, 2, 1);
  EXPECT(sparse_attn_pipelined(FAKE, FAKE, FAKE, SA_FP32, 1, 2, 1024, 64, 64, 64, 0.1, 0.9, 2,
                               static_cast<float *>(FAKE), FAKE, nullptr, FAKE, pw, nullptr, nullptr),
         SA_ERR_UNSUPPORTED);
  EXPECT(sparse_attn_pipelined(FAKE, FAKE, FAKE, SA_BF16, 1, 2, 1024, 64, 64, 64, 0.1, 0.9, 0, nullptr, FAKE,
                               nullptr, FAKE, pw, nullptr, nullptr),
         SA_ERR_INVALID_ARG);
  EXPECT(sparse_attn_pipelined_noalloc(FAKE, FAKE, FAKE, SA_BF16, 1, 1, 262144, 64, 64, 64, 0.1, 0.9, FAKE,
                                       nullptr, nullptr),
         SA_ERR_WORKSPACE);
  EXPECT(sparse_attn_router_exp(nullptr, nullptr, -1, nullptr), SA_ERR_INVALID_ARG);
  EXPECT(sparse_attn_router_exp(nullptr, nullptr, 0, nullptr), SA_OK);
  for (int c = -7; c <= 1; ++c) EXPECT(sparse_attn_status_string((sa_status)c) != nullptr, 1);
  EXPECT(sparse_attn_version() > 0, 1);
}

int main() {
  csr_checks();
  cube_checks();
  shape_and_argument_checks();
  if (failures) {
    fprintf(stderr, "%d of %d host checks failed\n", failures, checks);
    return 1;
  }
  printf("host checks passed: %d\n", checks);
  return 0;
}
