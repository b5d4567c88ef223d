"""The C ABI on a machine without a GPU: the library loads, exports every declared
symbol, sizes workspaces, and rejects every invalid argument on the host before any HIP
call (so these checks make no device call)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import block_sparse_attention_05_amd as sa
from block_sparse_attention_05_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000      # 256-aligned non-null "device" address, never dereferenced


@pytest.fixture(scope="module")
def lib():
    return sa.load_library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "sparse_attn.h")).read()
    return sorted(set(re.findall(r"\b(sparse_attn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    decl = declared_functions()
    assert len(decl) == 21
    assert sorted(B.EXPORTS) == decl
    for name in decl:
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    for st in range(-6, 1):
        s = lib.sparse_attn_status_string(st).decode()
        assert s and s != "unknown status"
    assert lib.sparse_attn_status_string(-99).decode() == "unknown status"
    assert sa.version() >= 100


def test_workspace_sizes(lib):
    f = lib.sparse_attn_plan_workspace_bytes
    assert f(1, 40, 75600, 128, 128, 64) > 0
    assert f(1, 8, 245760, 128, 128, 64) > 0
    assert f(1, 2, 1024, 64, 64, 64) > 0
    assert f(1, 1, 1024, 96, 64, 64) == 0         # unsupported D
    assert f(1, 1, 1024, 64, 32, 64) == 0         # unsupported block_q
    assert f(1, 1, 1024, 64, 64, 128) == 0        # unsupported block_kv
    assert f(0, 1, 1024, 64, 64, 64) == 0
    assert f(1, 1, 64 * 4097, 64, 64, 64) == 0    # too many KV blocks per row
    # the workspace holds at least the CSR at full capacity
    R, nkv = 40 * 591, 1182
    assert f(1, 40, 75600, 128, 128, 64) >= 4 * (R + 1 + R * nkv)
    st = B.SaPlan()
    st.B, st.H, st.N, st.D, st.block_q, st.block_kv = 1, 12, 32760, 128, 128, 64
    assert lib.sparse_attn_fwd_workspace_bytes(ctypes.byref(st), 0) == 0
    lin = lib.sparse_attn_fwd_workspace_bytes(ctypes.byref(st), 1)
    # at least H and z per head, phi(K) over whole KV blocks, and per query block the
    # masked-out sums H_C^T (bf16) and z_C (fp32)
    R, n_pad = 12 * 256, 512 * 64
    assert lin >= 12 * (128 * 128 + 128) * 4 + 12 * n_pad * 128 * 2 + R * (128 * 128 * 2 + 128 * 4)
    assert lib.sparse_attn_fwd_workspace_bytes(None, 1) == 0
    st.D = 96
    assert lib.sparse_attn_fwd_workspace_bytes(ctypes.byref(st), 1) == 0


def plan_call(lib, q=FAKE, k=FAKE, dt=0, shape=(1, 2, 1024, 64, 64, 64), topk=0.25, p=0.9,
              ws=FAKE, wsb=1 << 40, out=True):
    st = B.SaPlan()
    return lib.sparse_attn_plan(q, k, dt, *shape, topk, p, ws, wsb,
                                ctypes.byref(st) if out else None, None)


def test_plan_validation(lib):
    E = B
    assert plan_call(lib, q=None) == E.SA_ERR_INVALID_ARG
    assert plan_call(lib, k=None) == E.SA_ERR_INVALID_ARG
    assert plan_call(lib, out=False) == E.SA_ERR_INVALID_ARG
    assert plan_call(lib, dt=7) == E.SA_ERR_INVALID_ARG
    for bad in (-0.01, 1.01, math.nan, math.inf):
        assert plan_call(lib, topk=bad) == E.SA_ERR_INVALID_ARG
        assert plan_call(lib, p=bad) == E.SA_ERR_INVALID_ARG
    assert plan_call(lib, shape=(1, 2, 0, 64, 64, 64)) == E.SA_ERR_INVALID_ARG
    assert plan_call(lib, shape=(1, -2, 1024, 64, 64, 64)) == E.SA_ERR_INVALID_ARG
    assert plan_call(lib, shape=(1, 2, 1024, 80, 64, 64)) == E.SA_ERR_UNSUPPORTED
    assert plan_call(lib, shape=(1, 2, 1024, 64, 256, 64)) == E.SA_ERR_UNSUPPORTED
    assert plan_call(lib, shape=(1, 2, 1024, 64, 64, 32)) == E.SA_ERR_UNSUPPORTED
    assert plan_call(lib, ws=None) == E.SA_ERR_WORKSPACE
    assert plan_call(lib, wsb=1000) == E.SA_ERR_WORKSPACE
    assert plan_call(lib, ws=FAKE + 64) == E.SA_ERR_WORKSPACE


def test_plan_dense_validation(lib):
    E = B

    def dense(dt=0, shape=(1, 2, 1024, 64, 64, 64), ws=FAKE, wsb=1 << 40, out=True):
        st = B.SaPlan()
        return lib.sparse_attn_plan_dense(dt, *shape, ws, wsb, ctypes.byref(st) if out else None, None)

    assert dense(out=False) == E.SA_ERR_INVALID_ARG
    assert dense(dt=7) == E.SA_ERR_INVALID_ARG
    assert dense(shape=(1, 2, 0, 64, 64, 64)) == E.SA_ERR_INVALID_ARG
    assert dense(shape=(1, 2, 1024, 80, 64, 64)) == E.SA_ERR_UNSUPPORTED
    assert dense(shape=(1, 2, 1024, 64, 64, 32)) == E.SA_ERR_UNSUPPORTED
    assert dense(ws=None) == E.SA_ERR_WORKSPACE
    assert dense(wsb=1000) == E.SA_ERR_WORKSPACE
    assert dense(ws=FAKE + 64) == E.SA_ERR_WORKSPACE


def test_plan_struct_matches_header():
    """The ctypes mirror of sa_plan lists the header's fields in the header's order, with
    pointers as pointers and 32-bit integers as c_int32 (a drift here would shift every
    later field)."""
    text = open(os.path.join(ROOT, "include", "sparse_attn.h")).read()
    body = re.search(r"typedef struct sa_plan \{(.*?)\} sa_plan;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        ptr = "*" in decl
        for name in re.sub(r"^(const\s+)?\w+\s*\*?", "", decl).replace("*", "").split(","):
            fields.append((name.strip(), ptr))
    mirror = [(n, t) for n, t in B.SaPlan._fields_]
    assert [n for n, _ in fields] == [n for n, _ in mirror]
    for (n, ptr), (_, t) in zip(fields, mirror):
        assert (t is ctypes.c_void_p) == ptr, n
        if not ptr:
            assert t is ctypes.c_int32, n


def csr_call(lib, rp, ci, shape=(1, 1, 256, 64, 64, 64)):
    st = B.SaPlan()
    rp = np.ascontiguousarray(rp, np.int32)
    ci = np.ascontiguousarray(ci, np.int32)
    return lib.sparse_attn_plan_from_csr(0, *shape, rp.ctypes.data, ci.ctypes.data if ci.size else None,
                                         FAKE, 1 << 40, ctypes.byref(st), None)


def test_plan_from_csr_validation(lib):
    # 256 tokens, 64-blocks: 4 rows, 4 KV blocks each
    assert csr_call(lib, [1, 1, 2, 3, 4], [0, 1, 2, 3]) == B.SA_ERR_BAD_CSR         # row_ptr[0] != 0
    assert csr_call(lib, [0, 2, 1, 3, 4], [0, 1, 2, 3]) == B.SA_ERR_BAD_CSR         # decreasing
    assert csr_call(lib, [0, 1, 2, 3, 4], [0, 1, 4, 3]) == B.SA_ERR_BAD_CSR         # out of range
    assert csr_call(lib, [0, 1, 2, 3, 4], [0, -1, 2, 3]) == B.SA_ERR_BAD_CSR        # negative
    assert csr_call(lib, [0, 2, 2, 2, 2], [1, 0]) == B.SA_ERR_BAD_CSR               # unsorted
    assert csr_call(lib, [0, 2, 2, 2, 2], [1, 1]) == B.SA_ERR_BAD_CSR               # duplicate
    assert csr_call(lib, [0, 5, 5, 5, 5], [0, 1, 2, 3, 3]) == B.SA_ERR_BAD_CSR      # too many
    assert csr_call(lib, [0, 1, 1, 1, 1], []) == B.SA_ERR_INVALID_ARG               # cols missing


def fwd_call(lib, plan_fields, shape=(1, 2, 1024, 64), dt=0, alpha=None, ws=None, wsb=0,
             q=FAKE, o=FAKE):
    st = B.SaPlan(*plan_fields)
    return lib.sparse_attn_fwd(q, FAKE, FAKE, dt, *shape, ctypes.byref(st), alpha, o, None, ws, wsb,
                               None)


def test_fwd_validation(lib):
    good = (1, 2, 1024, 64, 64, 64, 16, 16, 0, 0, FAKE, FAKE, FAKE)
    assert fwd_call(lib, good, q=None) == B.SA_ERR_INVALID_ARG
    assert fwd_call(lib, good, o=None) == B.SA_ERR_INVALID_ARG
    assert fwd_call(lib, good, shape=(1, 2, 1000, 64)) == B.SA_ERR_PLAN_MISMATCH
    assert fwd_call(lib, good, shape=(1, 3, 1024, 64)) == B.SA_ERR_PLAN_MISMATCH
    assert fwd_call(lib, good, dt=1) == B.SA_ERR_PLAN_MISMATCH
    bad_blocks = (1, 2, 1024, 64, 64, 32, 16, 32, 0, 0, FAKE, FAKE, FAKE)
    assert fwd_call(lib, bad_blocks) == B.SA_ERR_UNSUPPORTED
    no_rows = (1, 2, 1024, 64, 64, 64, 16, 16, 0, 0, None, None, None)
    assert fwd_call(lib, no_rows) == B.SA_ERR_INVALID_ARG
    # the linear branch needs its workspace
    need = lib.sparse_attn_fwd_workspace_bytes(ctypes.byref(B.SaPlan(*good)), 1)
    if need > 0:
        assert fwd_call(lib, good, alpha=FAKE) == B.SA_ERR_WORKSPACE
        assert fwd_call(lib, good, alpha=FAKE, ws=FAKE, wsb=need - 1) == B.SA_ERR_WORKSPACE


def test_router_exp_validation(lib):
    assert lib.sparse_attn_router_exp(None, None, -1, None) == B.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_router_exp(None, FAKE, 10, None) == B.SA_ERR_INVALID_ARG
    assert lib.sparse_attn_router_exp(None, None, 0, None) == B.SA_OK


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 64)
    with pytest.raises(ValueError):
        sa.plan(q, q, 64, 64)


def test_tile_stats_validation(lib):
    """Every invalid tile-heatmap call is rejected on the host (nothing is launched)."""
    E = B
    f = lib.sparse_attn_tile_stats

    def call(q=FAKE, k=FAKE, lse=FAKE, dt=0, shape=(1, 2, 1024, 64, 64, 64), tmax=FAKE, tmass=FAKE):
        return f(q, k, lse, dt, *shape, tmax, tmass, None)

    assert call(q=None) == E.SA_ERR_INVALID_ARG
    assert call(k=None) == E.SA_ERR_INVALID_ARG
    assert call(lse=None) == E.SA_ERR_INVALID_ARG
    assert call(tmax=None, tmass=None) == E.SA_ERR_INVALID_ARG
    assert call(dt=5) == E.SA_ERR_INVALID_ARG
    assert call(dt=1) == E.SA_ERR_UNSUPPORTED                     # fp32 inputs
    assert call(shape=(1, 2, 0, 64, 64, 64)) == E.SA_ERR_INVALID_ARG
    assert call(shape=(1, 2, 1024, 96, 64, 64)) == E.SA_ERR_UNSUPPORTED
    assert call(shape=(1, 2, 1024, 64, 64, 128)) == E.SA_ERR_UNSUPPORTED
    assert call(shape=(1, 1, 64 * 4097, 64, 64, 64)) == E.SA_ERR_UNSUPPORTED


def test_cube_permute_validation(lib):
    """Every invalid cube-permutation call is rejected on the host (nothing is launched)."""
    E = B
    f = lib.sparse_attn_cube_permute
    good = np.array([2, 4, 16] * 2, dtype=np.int32)

    def call(src=FAKE, dst=FAKE + 4096, dt=0, shape=(1, 2, 21 * 45 * 80, 128), grid=(21, 45, 80),
             cubes=good, inv=0):
        c = np.ascontiguousarray(cubes, dtype=np.int32)
        return f(src, dst, dt, *shape, *grid, c.ctypes.data if c.size else None, inv, None)

    assert call(src=None) == E.SA_ERR_INVALID_ARG
    assert call(dst=None) == E.SA_ERR_INVALID_ARG
    assert call(dst=FAKE) == E.SA_ERR_INVALID_ARG                    # in place
    assert call(cubes=np.zeros(0)) == E.SA_ERR_INVALID_ARG
    assert call(dt=3) == E.SA_ERR_INVALID_ARG
    assert call(inv=2) == E.SA_ERR_INVALID_ARG
    assert call(grid=(21, 45, 79)) == E.SA_ERR_INVALID_ARG          # T*Hg*W != N
    assert call(cubes=np.array([2, 0, 16, 1, 1, 1])) == E.SA_ERR_INVALID_ARG
    assert call(shape=(1, 2, 21 * 45 * 80, 4)) == E.SA_ERR_UNSUPPORTED   # rows of 8 bytes
    assert call(shape=(1, 129, 21 * 45 * 80, 128), cubes=np.ones(129 * 3)) == E.SA_ERR_UNSUPPORTED


def test_plan_ordered_and_cube_order_validation(lib):
    E = B
    st = B.SaPlan()
    shape = (1, 2, 1024, 64, 64, 64)
    f = lib.sparse_attn_plan_ordered
    for kvo in (None, FAKE):
        assert f(FAKE, FAKE, 0, *shape, 0.1, 0.9, None, kvo, FAKE, 1 << 40, ctypes.byref(st), None) == E.SA_ERR_INVALID_ARG
        assert f(FAKE, FAKE, 1, *shape, 0.1, 0.9, FAKE, kvo, FAKE, 1 << 40, ctypes.byref(st), None) == E.SA_ERR_UNSUPPORTED
        assert f(None, FAKE, 0, *shape, 0.1, 0.9, FAKE, kvo, FAKE, 1 << 40, ctypes.byref(st), None) == E.SA_ERR_INVALID_ARG
        assert f(FAKE, FAKE, 0, *shape, 1.5, 0.9, FAKE, kvo, FAKE, 1 << 40, ctypes.byref(st), None) == E.SA_ERR_INVALID_ARG
    # a plan that reads keys through a table has no linear branch in the forward
    pl = B.SaPlan()
    pl.B, pl.H, pl.N, pl.D, pl.block_q, pl.block_kv = 1, 2, 1024, 64, 64, 64
    pl.n_qblk, pl.n_kvblk, pl.dtype = 16, 16, 0
    pl.row_ptr, pl.col_idx, pl.row_order, pl.q_order, pl.kv_order = FAKE, FAKE, FAKE, FAKE, FAKE
    fw = lib.sparse_attn_fwd
    assert fw(FAKE, FAKE, FAKE, 0, 1, 2, 1024, 64, ctypes.byref(pl), FAKE, FAKE, None, FAKE, 1 << 40,
              None) == E.SA_ERR_UNSUPPORTED
    assert fw(FAKE, FAKE, FAKE, 1, 1, 2, 1024, 64, ctypes.byref(pl), None, FAKE, None, None, 0,
              None) == E.SA_ERR_PLAN_MISMATCH
    g = lib.sparse_attn_cube_order
    c = np.array([1, 4, 16, 2, 2, 2], dtype=np.int32)
    assert g(2, 4, 16, 16, None, FAKE, None) == E.SA_ERR_INVALID_ARG
    assert g(2, 4, 16, 16, c.ctypes.data, None, None) == E.SA_ERR_INVALID_ARG
    assert g(0, 4, 16, 16, c.ctypes.data, FAKE, None) == E.SA_ERR_INVALID_ARG
    bad = np.array([1, 4, 0, 2, 2, 2], dtype=np.int32)
    assert g(2, 4, 16, 16, bad.ctypes.data, FAKE, None) == E.SA_ERR_INVALID_ARG
    big = np.ones(3 * 129, dtype=np.int32)
    assert g(129, 4, 16, 16, big.ctypes.data, FAKE, None) == E.SA_ERR_UNSUPPORTED


def test_bwd_validation(lib):
    E = B
    st = B.SaPlan()
    st.B, st.H, st.N, st.D, st.block_q, st.block_kv = 1, 2, 1024, 64, 64, 64
    st.n_qblk, st.n_kvblk, st.dtype = 16, 16, 0
    st.row_ptr, st.col_idx, st.row_order = FAKE, FAKE, FAKE
    f = lib.sparse_attn_bwd
    good = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dt=0, shape=(1, 2, 1024, 64),
                dq=FAKE, dk=FAKE, dv=FAKE, ws=FAKE, wsb=1 << 40)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dt"], *a["shape"],
                 ctypes.byref(st), a["dq"], a["dk"], a["dv"], a["ws"], a["wsb"], None)

    for name in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv"):
        assert call(**{name: None}) == E.SA_ERR_INVALID_ARG, name
    assert call(shape=(1, 2, 2048, 64)) == E.SA_ERR_PLAN_MISMATCH
    assert call(dt=1) == E.SA_ERR_PLAN_MISMATCH            # the plan was made for bf16
    assert call(wsb=16) == E.SA_ERR_WORKSPACE
    assert call(ws=None) == E.SA_ERR_WORKSPACE
    need = lib.sparse_attn_bwd_workspace_bytes(1, 2, 1024, 64, 64, 64)
    assert need > 0 and lib.sparse_attn_bwd_workspace_bytes(1, 2, 1024, 80, 64, 64) == 0
    st.q_order = FAKE
    assert call() == E.SA_ERR_UNSUPPORTED                   # ordered plans
    st.q_order = None


def _fp8_layout_bytes(B_, H, N, D, bq):
    """The pack size from the layout the header documents, summed independently."""
    BH, nQ, nKV = B_ * H, -(-N // bq), -(-N // 64)
    off = 0
    # q's exponents are reserved for 64-query blocks; a tail of 4 * block_q bytes ends the pack
    for n in (BH * N * D, BH * N * D, BH * nKV * D * 64, 4 * BH * nKV, 4 * BH * nKV, 4 * BH * D, 4 * BH * D,
              4 * bq):
        off = (off + n + 255) // 256 * 256
    return off


def test_fp8_pack_bytes(lib):
    f = lib.sparse_attn_fp8_pack_bytes
    for shape in ((1, 40, 75600, 128, 128), (1, 12, 32760, 128, 64), (2, 3, 1000, 64, 128)):
        assert f(*shape, 64) == _fp8_layout_bytes(*shape)
        p = sa.Fp8Pack(None, shape[:4], shape[4], 64)
        offs = p._parts()
        assert offs["vamax"][0] + offs["vamax"][1] <= f(*shape, 64)
    assert f(1, 1, 1024, 96, 64, 64) == 0
    assert f(1, 1, 1024, 64, 64, 128) == 0


def test_fp8_pack_sizes_differ_by_block_q(lib):
    """The two block_q values never give packs of one size, so the exact-size check in
    both calls tells a pack quantised for 64-query blocks from one for 128."""
    f = lib.sparse_attn_fp8_pack_bytes
    for BH in (1, 2, 3, 5, 8, 12, 40):
        for N in list(range(1, 3000, 37)) + [8192, 32760, 65536, 75600, 245760]:
            a, b = f(1, BH, N, 64, 64, 64), f(1, BH, N, 64, 128, 64)
            assert a > 0 and b > 0 and a != b, (BH, N)


def test_fp8_quantize_and_fwd_validation(lib):
    need = lib.sparse_attn_fp8_pack_bytes(1, 2, 1024, 64, 64, 64)
    q = lib.sparse_attn_quantize_fp8

    def quant(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, dt=0, shape=(1, 2, 1024, 64), bq=64, bk=64, fmt=0, pack=FAKE, pb=need)
        a.update(kw)
        return q(a["q"], a["k"], a["v"], a["dt"], *a["shape"], a["bq"], a["bk"], a["fmt"], a["pack"], a["pb"],
                 None)

    for name in ("q", "k", "v"):
        assert quant(**{name: None}) == B.SA_ERR_INVALID_ARG, name
    assert quant(dt=1) == B.SA_ERR_UNSUPPORTED
    assert quant(dt=7) == B.SA_ERR_INVALID_ARG
    assert quant(pb=need - 1) == B.SA_ERR_WORKSPACE
    assert quant(pack=None) == B.SA_ERR_WORKSPACE
    assert quant(pack=FAKE + 16) == B.SA_ERR_WORKSPACE
    assert quant(bk=128) == B.SA_ERR_UNSUPPORTED
    assert quant(shape=(1, 2, 1024, 80)) == B.SA_ERR_UNSUPPORTED
    assert quant(fmt=2) == B.SA_ERR_INVALID_ARG
    assert quant(fmt=-1) == B.SA_ERR_INVALID_ARG

    st = B.SaPlan()
    st.B, st.H, st.N, st.D, st.block_q, st.block_kv = 1, 2, 1024, 64, 64, 64
    st.n_qblk, st.n_kvblk, st.dtype = 16, 16, 0
    st.row_ptr, st.col_idx, st.row_order = FAKE, FAKE, FAKE
    f = lib.sparse_attn_fwd_fp8

    def fwd(**kw):
        a = dict(pack=FAKE, pb=need, fmt=0, shape=(1, 2, 1024, 64), o=FAKE, lse=None)
        a.update(kw)
        return f(a["pack"], a["pb"], a["fmt"], *a["shape"], ctypes.byref(st), a["o"], a["lse"], None)

    assert fwd(pack=None) == B.SA_ERR_INVALID_ARG
    assert fwd(fmt=3) == B.SA_ERR_INVALID_ARG
    assert fwd(o=None) == B.SA_ERR_INVALID_ARG
    assert fwd(pb=need - 1) == B.SA_ERR_WORKSPACE
    assert fwd(shape=(1, 2, 2048, 64)) == B.SA_ERR_PLAN_MISMATCH
    # a pack sized for another block_q (larger here) is rejected, not read at wrong offsets
    need128 = lib.sparse_attn_fp8_pack_bytes(1, 2, 1024, 64, 128, 64)
    assert need128 > need
    assert fwd(pb=need128) == B.SA_ERR_PLAN_MISMATCH
    assert quant(pb=need128) == B.SA_ERR_WORKSPACE
    st.dtype = 1
    assert fwd() == B.SA_ERR_UNSUPPORTED                    # fp32 plans
    st.dtype = 0
    st.q_order = FAKE
    assert fwd() == B.SA_ERR_UNSUPPORTED                    # ordered plans
    st.q_order = None
    st.row_ptr = None
    assert fwd() == B.SA_ERR_INVALID_ARG


def test_pipelined_noalloc_validation(lib):
    """Host checks of the allocation-free call, before it touches the device: null
    pointers, k or p out of range, unsupported shapes, and a shape whose single-head plan
    exceeds the 128 MiB static scratch."""
    f = lib.sparse_attn_pipelined_noalloc

    def call(q=FAKE, o=FAKE, dt=0, shape=(1, 2, 1024, 64, 64, 64), topk=0.1, p=0.9):
        return f(q, FAKE, FAKE, dt, *shape, topk, p, o, None, None)

    assert call(q=None) == B.SA_ERR_INVALID_ARG
    assert call(o=None) == B.SA_ERR_INVALID_ARG
    assert call(dt=5) == B.SA_ERR_INVALID_ARG
    assert call(topk=1.5) == B.SA_ERR_INVALID_ARG
    assert call(p=-0.1) == B.SA_ERR_INVALID_ARG
    assert call(shape=(1, 2, 1024, 96, 64, 64)) == B.SA_ERR_UNSUPPORTED
    # 262,144 tokens in 64-query blocks: one head's plan needs more than 128 MiB
    one = lib.sparse_attn_plan_workspace_bytes(1, 1, 262144, 64, 64, 64)
    assert one > 128 << 20
    assert call(shape=(1, 1, 262144, 64, 64, 64)) == B.SA_ERR_WORKSPACE
    # the largest workload shapes fit one head (and more) in the scratch
    assert lib.sparse_attn_plan_workspace_bytes(1, 1, 245760, 128, 128, 64) <= 128 << 20
    assert lib.sparse_attn_plan_workspace_bytes(1, 1, 262144, 64, 128, 64) <= 128 << 20


def test_pipelined_validation(lib):
    f = lib.sparse_attn_pipelined_workspace_bytes
    one = lib.sparse_attn_plan_workspace_bytes(1, 5, 75600, 128, 128, 64)
    assert f(1, 40, 75600, 128, 128, 64, 8, 0) == 8 * one          # eight chunks of five heads
    assert f(2, 3, 1000, 64, 64, 64, 4, 0) == 3 * lib.sparse_attn_plan_workspace_bytes(1, 2, 1000, 64, 64, 64)
    assert f(1, 4, 1000, 64, 64, 64, 100, 0) == 4 * lib.sparse_attn_plan_workspace_bytes(1, 1, 1000, 64, 64, 64)
    assert f(1, 4, 1000, 64, 64, 64, 0, 0) == 0
    assert f(1, 4, 1000, 80, 64, 64, 2, 0) == 0
    # with the linear branch: the plan workspaces, then one chunk's forward workspace
    st = B.SaPlan()
    st.B, st.H, st.N, st.D, st.block_q, st.block_kv = 1, 3, 32760, 128, 128, 64
    lin = lib.sparse_attn_fwd_workspace_bytes(ctypes.byref(st), 1)
    plans = f(1, 12, 32760, 128, 128, 64, 4, 0)
    assert plans == 4 * lib.sparse_attn_plan_workspace_bytes(1, 3, 32760, 128, 128, 64)
    assert f(1, 12, 32760, 128, 128, 64, 4, 1) == -(-plans // 256) * 256 + lin
    need = f(1, 2, 1024, 64, 64, 64, 2, 0)
    need_lin = f(1, 2, 1024, 64, 64, 64, 2, 1)
    assert need_lin > need
    g = lib.sparse_attn_pipelined

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, dt=0, shape=(1, 2, 1024, 64), bq=64, bk=64, k_=0.1, p=0.9, C=2,
                 alpha=None, o=FAKE, lse=None, ws=FAKE, wsb=need)
        a.update(kw)
        return g(a["q"], a["k"], a["v"], a["dt"], *a["shape"], a["bq"], a["bk"], a["k_"], a["p"], a["C"],
                 a["alpha"], a["o"], a["lse"], a["ws"], a["wsb"], None, None)

    # the linear branch needs its forward workspace too, and bf16
    assert call(alpha=FAKE, wsb=need) == B.SA_ERR_WORKSPACE
    assert call(alpha=FAKE, dt=1, wsb=need_lin) == B.SA_ERR_UNSUPPORTED

    for name in ("q", "k", "v", "o"):
        assert call(**{name: None}) == B.SA_ERR_INVALID_ARG, name
    assert call(dt=5) == B.SA_ERR_INVALID_ARG
    assert call(k_=1.5) == B.SA_ERR_INVALID_ARG
    assert call(p=-0.1) == B.SA_ERR_INVALID_ARG
    assert call(C=0) == B.SA_ERR_INVALID_ARG
    assert call(wsb=need - 1) == B.SA_ERR_WORKSPACE
    assert call(ws=FAKE + 8) == B.SA_ERR_WORKSPACE
    assert call(bk=128) == B.SA_ERR_UNSUPPORTED
