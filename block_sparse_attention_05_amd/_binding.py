"""ctypes binding of libsparse_attn.so: argument marshalling only.

Every step of the computation runs in the library's HIP kernels; this module checks
tensor shapes, allocates workspaces with torch (device memory and streams are all torch
provides here) and passes raw pointers and sizes across the C ABI declared in
include/sparse_attn.h. When the library is missing, every entry point raises; there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SPARSE_ATTN_LIB", os.path.join(HERE, "libsparse_attn.so"))

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE = 0, -1, -2, -3
SA_ERR_PLAN_MISMATCH, SA_ERR_BAD_CSR, SA_ERR_HIP = -4, -5, -6
SA_BF16, SA_FP32 = 0, 1

EXPORTS = (
    "sparse_attn_plan_workspace_bytes", "sparse_attn_plan", "sparse_attn_plan_dense",
    "sparse_attn_plan_from_csr", "sparse_attn_fwd_workspace_bytes", "sparse_attn_fwd",
    "sparse_attn_bwd_workspace_bytes", "sparse_attn_bwd",
    "sparse_attn_pipelined_workspace_bytes", "sparse_attn_pipelined",
    "sparse_attn_plan_ordered", "sparse_attn_tile_stats", "sparse_attn_cube_permute",
    "sparse_attn_cube_order", "sparse_attn_fp8_pack_bytes", "sparse_attn_quantize_fp8",
    "sparse_attn_fwd_fp8", "sparse_attn_router_exp", "sparse_attn_status_string",
    "sparse_attn_version", "sparse_attn_pipelined_noalloc",
)


class SaPlan(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("D", ctypes.c_int32),
        ("block_q", ctypes.c_int32), ("block_kv", ctypes.c_int32),
        ("n_qblk", ctypes.c_int32), ("n_kvblk", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p), ("row_order", ctypes.c_void_p),
        ("q_order", ctypes.c_void_p), ("kv_order", ctypes.c_void_p), ("visit", ctypes.c_void_p),
        ("nnz", ctypes.c_void_p),
    ]


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_status_string(status)} (status {status})")


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Loads the HIP library once; raises when it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} not found: build it with `python -m block_sparse_attention_05_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, i64, sz, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_double
    pplan = ctypes.POINTER(SaPlan)
    lib.sparse_attn_plan_workspace_bytes.argtypes = [i32] * 6
    lib.sparse_attn_plan_workspace_bytes.restype = sz
    lib.sparse_attn_plan.argtypes = [vp, vp, i32] + [i32] * 6 + [dbl, dbl, vp, sz, pplan, vp]
    lib.sparse_attn_plan.restype = i32
    lib.sparse_attn_plan_ordered.argtypes = [vp, vp, i32] + [i32] * 6 + [dbl, dbl, vp, vp, vp, sz, pplan, vp]
    lib.sparse_attn_plan_ordered.restype = i32
    lib.sparse_attn_plan_dense.argtypes = [i32] * 7 + [vp, sz, pplan, vp]
    lib.sparse_attn_plan_dense.restype = i32
    lib.sparse_attn_plan_from_csr.argtypes = [i32] * 7 + [vp, vp, vp, sz, pplan, vp]
    lib.sparse_attn_plan_from_csr.restype = i32
    lib.sparse_attn_fwd_workspace_bytes.argtypes = [pplan, i32]
    lib.sparse_attn_fwd_workspace_bytes.restype = sz
    lib.sparse_attn_fwd.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, pplan, vp, vp, vp, vp, sz, vp]
    lib.sparse_attn_fwd.restype = i32
    lib.sparse_attn_tile_stats.argtypes = [vp, vp, vp, i32] + [i32] * 6 + [vp, vp, vp]
    lib.sparse_attn_tile_stats.restype = i32
    lib.sparse_attn_cube_permute.argtypes = [vp, vp, i32] + [i32] * 7 + [vp, i32, vp]
    lib.sparse_attn_cube_permute.restype = i32
    lib.sparse_attn_cube_order.argtypes = [i32] * 4 + [vp, vp, vp]
    lib.sparse_attn_cube_order.restype = i32
    lib.sparse_attn_bwd_workspace_bytes.argtypes = [i32] * 6
    lib.sparse_attn_bwd_workspace_bytes.restype = sz
    lib.sparse_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, pplan, vp, vp, vp,
                                    vp, sz, vp]
    lib.sparse_attn_bwd.restype = i32
    lib.sparse_attn_pipelined_workspace_bytes.argtypes = [i32] * 8
    lib.sparse_attn_pipelined_workspace_bytes.restype = sz
    lib.sparse_attn_pipelined.argtypes = [vp, vp, vp, i32] + [i32] * 6 + [dbl, dbl, i32, vp, vp, vp, vp, sz, vp, vp]
    lib.sparse_attn_pipelined.restype = i32
    lib.sparse_attn_pipelined_noalloc.argtypes = [vp, vp, vp, i32] + [i32] * 6 + [dbl, dbl, vp, vp, vp]
    lib.sparse_attn_pipelined_noalloc.restype = i32
    lib.sparse_attn_fp8_pack_bytes.argtypes = [i32] * 6
    lib.sparse_attn_fp8_pack_bytes.restype = sz
    lib.sparse_attn_quantize_fp8.argtypes = [vp, vp, vp, i32] + [i32] * 7 + [vp, sz, vp]
    lib.sparse_attn_quantize_fp8.restype = i32
    lib.sparse_attn_fwd_fp8.argtypes = [vp, sz, i32, i32, i32, i32, i32, pplan, vp, vp, vp]
    lib.sparse_attn_fwd_fp8.restype = i32
    lib.sparse_attn_router_exp.argtypes = [vp, vp, i64, vp]
    lib.sparse_attn_router_exp.restype = i32
    lib.sparse_attn_status_string.argtypes = [i32]
    lib.sparse_attn_status_string.restype = ctypes.c_char_p
    lib.sparse_attn_version.argtypes = []
    lib.sparse_attn_version.restype = i32
    if path is None:
        _lib = lib
    return lib


def _status_string(st: int) -> str:
    try:
        return load_library().sparse_attn_status_string(st).decode()
    except Exception:  # the library itself is missing
        return "unknown"


def _check(st: int, what: str) -> None:
    if st != SA_OK:
        raise SparseAttnError(st, what)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SA_BF16
    if t.dtype == torch.float32:
        return SA_FP32
    raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _stream(stream) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check_qkv(*ts):
    t0 = ts[0]
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, D]")
        if t.dim() != 4 or tuple(t.shape) != tuple(t0.shape) or t.dtype != t0.dtype:
            raise ValueError("q, k, v must share one [B, H, N, D] shape and one dtype")
        if t.device != t0.device:
            raise ValueError("tensors must be on one device")


class Plan:
    """A block mask in CSR form living in a torch-owned workspace on the GPU."""

    def __init__(self, ws, st: SaPlan, keep=None):
        self.ws = ws          # keeps the workspace (and so the CSR arrays) alive
        self.st = st
        self.keep = keep      # keeps a caller table the plan points to (the query order) alive

    @property
    def shape(self) -> Tuple[int, int, int, int]:
        return (self.st.B, self.st.H, self.st.N, self.st.D)

    @property
    def blocks(self) -> Tuple[int, int]:
        return (self.st.block_q, self.st.block_kv)

    @property
    def rows(self) -> int:
        return self.st.B * self.st.H * self.st.n_qblk

    def _view(self, ptr: int, count: int):
        torch = _torch()
        off = ptr - self.ws.data_ptr()
        return self.ws[off:off + 4 * count].view(torch.int32)

    def row_ptr(self):
        return self._view(self.st.row_ptr, self.rows + 1)

    def col_idx(self, nnz: Optional[int] = None):
        if nnz is None:
            nnz = int(self.row_ptr()[-1].item())
        return self._view(self.st.col_idx, nnz)

    def row_order(self):
        return self._view(self.st.row_order, self.rows)

    def nnz(self):
        """The plan's device scalar holding the number of kept blocks (int64, one element)."""
        torch = _torch()
        off = self.st.nnz - self.ws.data_ptr()
        return self.ws[off:off + 8].view(torch.int64)

    def csr(self) -> Tuple[np.ndarray, np.ndarray]:
        """(row_ptr, col_idx) copied to host numpy arrays (synchronises)."""
        rp = self.row_ptr().cpu().numpy().astype(np.int64)
        ci = self.col_idx(int(rp[-1])).cpu().numpy()
        return rp, ci

    def visit_lists(self, rows: Optional[List[int]] = None):
        """Each row's kept blocks in the forward's visit order (host arrays; synchronises),
        or None when the plan has no visit lists. With ``rows``, a dict of those rows only
        (copies just their lists)."""
        if not self.st.visit:
            return None
        rp = self.row_ptr().cpu().numpy().astype(np.int64)
        nkv = self.st.n_kvblk
        full = self._view(self.st.visit, self.rows * nkv).view(self.rows, nkv)
        if rows is not None:
            return {r: full[r, :rp[r + 1] - rp[r]].cpu().numpy() for r in rows}
        full = full.cpu().numpy()
        return [full[r, :rp[r + 1] - rp[r]].copy() for r in range(self.rows)]


def _new_ws(nbytes: int, device):
    torch = _torch()
    # torch's caching allocator returns blocks aligned to at least 512 bytes
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    assert ws.data_ptr() % 256 == 0
    return ws


def plan_workspace_bytes(B, H, N, D, block_q, block_kv) -> int:
    return int(load_library().sparse_attn_plan_workspace_bytes(B, H, N, D, block_q, block_kv))


def bwd_workspace_bytes(B, H, N, D, block_q, block_kv) -> int:
    return int(load_library().sparse_attn_bwd_workspace_bytes(B, H, N, D, block_q, block_kv))


def plan(q, k, block_q: int = 128, block_kv: int = 64, topk: float = 0.05, top_p: float = 0.9,
         stream=None, workspace=None) -> Plan:
    """The hybrid top-k / top-p block mask of q, k [B, H, N, D] (see sparse_attn_plan)."""
    lib = load_library()
    _check_qkv(q, k)
    B, H, N, D = q.shape
    need = lib.sparse_attn_plan_workspace_bytes(B, H, N, D, block_q, block_kv)
    if need == 0:
        raise SparseAttnError(SA_ERR_UNSUPPORTED, "plan shape")
    ws = workspace if workspace is not None else _new_ws(need, q.device)
    st = SaPlan()
    _check(lib.sparse_attn_plan(q.data_ptr(), k.data_ptr(), _dtype_code(q), B, H, N, D, block_q,
                                block_kv, float(topk), float(top_p), ws.data_ptr(), ws.numel(),
                                ctypes.byref(st), _stream(stream)), "sparse_attn_plan")
    return Plan(ws, st)


def plan_ordered(q, k, q_order, block_q: int = 128, block_kv: int = 64, topk: float = 0.05,
                 top_p: float = 0.9, stream=None, workspace=None, kv_order=None) -> Plan:
    """The mask for queries taken per head in the order q_order (int32 [H, N] GPU tensor,
    position -> storage row; see sparse_attn_plan_ordered) and, with kv_order, keys in
    that order too. q (and k, v with kv_order) stay in storage order; without kv_order, k
    and the v later given to fwd are in key-position order. fwd with this plan writes o
    in q's storage order."""
    torch = _torch()
    lib = load_library()
    _check_qkv(q, k)
    B, H, N, D = q.shape
    for t, name in ((q_order, "q_order"), (kv_order, "kv_order")):
        if t is not None and not (t.is_cuda and t.dtype == torch.int32 and t.is_contiguous()
                                  and t.numel() == H * N):
            raise ValueError(f"{name} must be a contiguous int32 [H, N] GPU tensor")
    need = lib.sparse_attn_plan_workspace_bytes(B, H, N, D, block_q, block_kv)
    if need == 0:
        raise SparseAttnError(SA_ERR_UNSUPPORTED, "plan shape")
    ws = workspace if workspace is not None else _new_ws(need, q.device)
    st = SaPlan()
    _check(lib.sparse_attn_plan_ordered(q.data_ptr(), k.data_ptr(), _dtype_code(q), B, H, N, D,
                                        block_q, block_kv, float(topk), float(top_p),
                                        q_order.data_ptr(), kv_order.data_ptr() if kv_order is not None else None,
                                        ws.data_ptr(), ws.numel(), ctypes.byref(st), _stream(stream)),
           "sparse_attn_plan_ordered")
    return Plan(ws, st, keep=(q_order, kv_order))


def cube_order(H: int, grid, cubes, device="cuda", stream=None):
    """Per-head cube orders as a table for plan_ordered: int32 [H, N] with
    order[h, pos_h(n)] = n (see sparse_attn_cube_order)."""
    torch = _torch()
    lib = load_library()
    T, Hg, W = (int(g) for g in grid)
    cub = np.ascontiguousarray(np.asarray(cubes, dtype=np.int32).reshape(-1))
    if cub.size != 3 * H:
        raise ValueError("cubes must give (ct, ch, cw) for every head")
    out = torch.empty((H, T * Hg * W), dtype=torch.int32, device=device)
    _check(lib.sparse_attn_cube_order(H, T, Hg, W, cub.ctypes.data, out.data_ptr(), _stream(stream)),
           "sparse_attn_cube_order")
    return out


def plan_dense(q, block_q: int = 128, block_kv: int = 64, stream=None) -> Plan:
    """The all-ones mask for q's shape (dense attention through the sparse kernel)."""
    lib = load_library()
    B, H, N, D = q.shape
    need = lib.sparse_attn_plan_workspace_bytes(B, H, N, D, block_q, block_kv)
    if need == 0:
        raise SparseAttnError(SA_ERR_UNSUPPORTED, "plan shape")
    ws = _new_ws(need, q.device)
    st = SaPlan()
    _check(lib.sparse_attn_plan_dense(_dtype_code(q), B, H, N, D, block_q, block_kv, ws.data_ptr(),
                                      ws.numel(), ctypes.byref(st), _stream(stream)),
           "sparse_attn_plan_dense")
    return Plan(ws, st)


def plan_from_csr(q, row_ptr: np.ndarray, col_idx: np.ndarray, block_q: int = 128,
                  block_kv: int = 64, stream=None) -> Plan:
    """A caller-given CSR mask (host arrays), validated and copied to the GPU."""
    lib = load_library()
    B, H, N, D = q.shape
    need = lib.sparse_attn_plan_workspace_bytes(B, H, N, D, block_q, block_kv)
    if need == 0:
        raise SparseAttnError(SA_ERR_UNSUPPORTED, "plan shape")
    rp = np.ascontiguousarray(row_ptr, dtype=np.int32)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32)
    ws = _new_ws(need, q.device)
    st = SaPlan()
    _check(lib.sparse_attn_plan_from_csr(_dtype_code(q), B, H, N, D, block_q, block_kv,
                                         rp.ctypes.data, ci.ctypes.data if ci.size else None,
                                         ws.data_ptr(), ws.numel(), ctypes.byref(st),
                                         _stream(stream)), "sparse_attn_plan_from_csr")
    return Plan(ws, st)


def fwd(q, k, v, plan: Plan, alpha=None, return_lse: bool = False, out=None, lse=None,
        workspace=None, stream=None):
    """Block-sparse attention over plan's kept tiles, optionally blended with the linear
    branch (see sparse_attn_fwd). Returns o, or (o, lse) with return_lse."""
    torch = _torch()
    lib = load_library()
    _check_qkv(q, k, v)
    B, H, N, D = q.shape
    if alpha is not None:
        if not (alpha.is_cuda and alpha.dtype == torch.float32 and alpha.is_contiguous()
                and tuple(alpha.shape) == (H, D)):
            raise ValueError("alpha must be a contiguous float32 [H, D] GPU tensor")
    o = out if out is not None else torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    need = lib.sparse_attn_fwd_workspace_bytes(ctypes.byref(plan.st), 1 if alpha is not None else 0)
    ws = workspace
    if need > 0 and ws is None:
        ws = _new_ws(need, q.device)
    _check(lib.sparse_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), B, H, N, D,
                               ctypes.byref(plan.st),
                               alpha.data_ptr() if alpha is not None else None, o.data_ptr(),
                               lse.data_ptr() if lse is not None else None,
                               ws.data_ptr() if ws is not None else None,
                               ws.numel() if ws is not None else 0, _stream(stream)),
           "sparse_attn_fwd")
    return (o, lse) if return_lse else o


def bwd(q, k, v, o, lse, dout, plan: Plan, workspace=None, out=None, stream=None):
    """Gradients (dq, dk, dv) of fwd(q, k, v, plan) for the upstream gradient dout, from
    the forward's o and lse (see sparse_attn_bwd). ``out`` = (dq, dk, dv) tensors shaped
    like q to write into."""
    torch = _torch()
    lib = load_library()
    _check_qkv(q, k, v)
    _check_qkv(q, o, dout)
    B, H, N, D = q.shape
    if not (lse.is_cuda and lse.dtype == torch.float32 and lse.is_contiguous()
            and tuple(lse.shape) == (B, H, N)):
        raise ValueError("lse must be a contiguous float32 [B, H, N] GPU tensor")
    need = lib.sparse_attn_bwd_workspace_bytes(B, H, N, D, plan.st.block_q, plan.st.block_kv)
    if need == 0:
        raise SparseAttnError(SA_ERR_UNSUPPORTED, "bwd shape")
    ws = workspace if workspace is not None else _new_ws(need, q.device)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        _check_qkv(dq, dk, dv)
        if dq.shape != q.shape or dq.dtype != q.dtype:
            raise ValueError("out tensors must match q's shape and dtype")
    _check(lib.sparse_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                               dout.data_ptr(), _dtype_code(q), B, H, N, D, ctypes.byref(plan.st),
                               dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(),
                               _stream(stream)), "sparse_attn_bwd")
    return dq, dk, dv


class Fp8Pack:
    """FP8 E4M3 codes and group exponents of q, k, v in one device buffer (layout as
    documented for sparse_attn_fp8_pack_bytes)."""

    def __init__(self, buf, shape, block_q: int, block_kv: int, qk: str = "e4m3"):
        self.buf = buf
        self.shape = tuple(shape)
        self.block_q = block_q
        self.block_kv = block_kv
        self.qk = qk          # "e4m3" or "int8": the format of the q and k codes

    def _parts(self):
        B, H, N, D = self.shape
        BH = B * H
        nQ, nKV = -(-N // self.block_q), -(-N // 64)
        # (name, bytes used, bytes reserved): q's exponents are reserved for 64-query blocks
        sizes = [("q8", BH * N * D, BH * N * D), ("k8", BH * N * D, BH * N * D),
                 ("vt8", BH * nKV * D * 64, BH * nKV * D * 64), ("qe", BH * nQ * 4, BH * nKV * 4),
                 ("ke", BH * nKV * 4, BH * nKV * 4), ("ve", BH * D * 4, BH * D * 4),
                 ("vamax", BH * D * 4, BH * D * 4), ("tail", 0, 4 * self.block_q)]
        off, out = 0, {}
        for name, n, cap in sizes:
            out[name] = (off, n)
            off = (off + cap + 255) & ~255
        return out

    def part(self, name: str):
        """A torch view of one part: uint8 codes or int32 exponents."""
        torch = _torch()
        off, n = self._parts()[name]
        B, H, N, D = self.shape
        nQ, nKV = -(-N // self.block_q), -(-N // 64)
        raw = self.buf[off:off + n]
        shapes = {"q8": (B, H, N, D), "k8": (B, H, N, D), "vt8": (B, H, nKV, D, 64),
                  "qe": (B, H, nQ), "ke": (B, H, nKV), "ve": (B, H, D), "vamax": (B, H, D)}
        if name in ("q8", "k8", "vt8"):
            t = raw.view(torch.int8) if (self.qk == "int8" and name != "vt8") else raw
        else:
            t = raw.view(torch.float32 if (self.qk == "int8" and name in ("qe", "ke")) else torch.int32)
        return t.view(shapes[name])


def fp8_pack_bytes(B, H, N, D, block_q=128, block_kv=64) -> int:
    return int(load_library().sparse_attn_fp8_pack_bytes(B, H, N, D, block_q, block_kv))


QK_FORMATS = {"e4m3": 0, "int8": 1}


def quantize_fp8(q, k, v, block_q: int = 128, block_kv: int = 64, out: Optional[Fp8Pack] = None,
                 stream=None, qk: str = "e4m3") -> Fp8Pack:
    """Quantises bf16 q, k, v [B, H, N, D] to a low-bit pack (see sparse_attn_quantize_fp8):
    v always E4M3; q and k E4M3 (qk="e4m3") or int8 (qk="int8")."""
    if qk not in QK_FORMATS:
        raise ValueError("qk must be 'e4m3' or 'int8'")
    lib = load_library()
    _check_qkv(q, k, v)
    B, H, N, D = q.shape
    need = lib.sparse_attn_fp8_pack_bytes(B, H, N, D, block_q, block_kv)
    if need == 0:
        raise SparseAttnError(SA_ERR_UNSUPPORTED, "fp8 pack shape")
    pack = out if out is not None else Fp8Pack(_new_ws(need, q.device), q.shape, block_q, block_kv, qk)
    if pack.shape != tuple(q.shape) or pack.block_q != block_q:
        raise ValueError("pack was made for another shape or block_q")
    pack.qk = qk
    _check(lib.sparse_attn_quantize_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), B, H, N, D,
                                        block_q, block_kv, QK_FORMATS[qk], pack.buf.data_ptr(),
                                        pack.buf.numel(), _stream(stream)), "sparse_attn_quantize_fp8")
    return pack


def fwd_fp8(pack: Fp8Pack, plan: Plan, return_lse: bool = False, out=None, lse=None, stream=None):
    """Block-sparse attention over the plan's kept tiles from an FP8 pack (see
    sparse_attn_fwd_fp8). Returns o (bf16 [B, H, N, D]) and, with return_lse, lse."""
    torch = _torch()
    lib = load_library()
    B, H, N, D = pack.shape
    if plan.shape != pack.shape or plan.st.block_q != pack.block_q:
        raise ValueError("plan and pack disagree on shape or block_q")
    dev = pack.buf.device
    o = out if out is not None else torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
    if o.shape != (B, H, N, D) or o.dtype != torch.bfloat16 or not o.is_contiguous():
        raise ValueError("o must be a contiguous bf16 [B, H, N, D] tensor")
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    _check(lib.sparse_attn_fwd_fp8(pack.buf.data_ptr(), pack.buf.numel(), QK_FORMATS[pack.qk], B, H, N, D,
                                   ctypes.byref(plan.st),
                                   o.data_ptr(), lse.data_ptr() if return_lse else None, _stream(stream)),
           "sparse_attn_fwd_fp8")
    return (o, lse) if return_lse else o


_AUX = {}


def _aux_stream(device):
    """One auxiliary stream per device, at the default priority, made once."""
    torch = _torch()
    key = torch.device(device).index
    if key not in _AUX:
        _AUX[key] = torch.cuda.Stream(device=device)
    return _AUX[key]


def pipelined_workspace_bytes(B, H, N, D, block_q=128, block_kv=64, chunks=4, linear=False) -> int:
    return int(load_library().sparse_attn_pipelined_workspace_bytes(B, H, N, D, block_q, block_kv, chunks,
                                                                     1 if linear else 0))


def attention(q, k, v, block_q: int = 128, block_kv: int = 64, topk: float = 0.05, top_p: float = 0.9,
              chunks: int = 4, return_lse: bool = False, out=None, lse=None, workspace=None, stream=None,
              aux_stream=None, alpha=None):
    """Plan and forward for all heads in one call, pipelined over chunks of heads on two
    streams (see sparse_attn_pipelined); alpha [H, D] float32 adds the linear branch as in
    fwd. Returns o (and lse with return_lse)."""
    torch = _torch()
    lib = load_library()
    _check_qkv(q, k, v)
    B, H, N, D = q.shape
    if alpha is not None and not (alpha.is_cuda and alpha.dtype == torch.float32 and alpha.is_contiguous()
                                  and tuple(alpha.shape) == (H, D)):
        raise ValueError("alpha must be a contiguous float32 [H, D] GPU tensor")
    need = lib.sparse_attn_pipelined_workspace_bytes(B, H, N, D, block_q, block_kv, chunks,
                                                     0 if alpha is None else 1)
    if need == 0:
        raise SparseAttnError(SA_ERR_UNSUPPORTED, "pipelined shape")
    ws = workspace if workspace is not None else _new_ws(need, q.device)
    o = out if out is not None else torch.empty_like(q)
    _check_qkv(q, o)
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    s = stream if stream is not None else torch.cuda.current_stream()
    aux = aux_stream if aux_stream is not None else _aux_stream(q.device)
    _check(lib.sparse_attn_pipelined(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), B, H, N, D,
                                     block_q, block_kv, float(topk), float(top_p), int(chunks),
                                     None if alpha is None else alpha.data_ptr(), o.data_ptr(),
                                     lse.data_ptr() if return_lse else None, ws.data_ptr(), ws.numel(),
                                     s.cuda_stream, aux.cuda_stream), "sparse_attn_pipelined")
    return (o, lse) if return_lse else o


def attention_noalloc(q, k, v, block_q: int = 128, block_kv: int = 64, topk: float = 0.05,
                      top_p: float = 0.9, out=None, lse=None, stream=None):
    """Plan and forward for all heads on one stream with the library's static scratch (see
    sparse_attn_pipelined_noalloc): nothing is allocated when ``out`` (and ``lse``, if
    wanted) are given. Returns o, or (o, lse) when lse is given."""
    torch = _torch()
    lib = load_library()
    _check_qkv(q, k, v)
    B, H, N, D = q.shape
    o = out if out is not None else torch.empty_like(q)
    _check_qkv(q, o)
    _check(lib.sparse_attn_pipelined_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), B, H, N,
                                             D, block_q, block_kv, float(topk), float(top_p), o.data_ptr(),
                                             lse.data_ptr() if lse is not None else None, _stream(stream)),
           "sparse_attn_pipelined_noalloc")
    return (o, lse) if lse is not None else o


def tile_stats(q, k, lse, block_q: int = 128, block_kv: int = 64, stream=None):
    """Pass 2 of the ground-truth tile heatmap (see sparse_attn_tile_stats): returns
    (tile_max, tile_mass), float32 [B*H*n_qblk, n_kvblk], from q, k [B, H, N, D] bf16 and
    lse [B, H, N] (fwd on plan_dense with return_lse)."""
    torch = _torch()
    lib = load_library()
    _check_qkv(q, k)
    B, H, N, D = q.shape
    if not (lse.is_cuda and lse.dtype == torch.float32 and lse.is_contiguous()
            and tuple(lse.shape) == (B, H, N)):
        raise ValueError("lse must be a contiguous float32 [B, H, N] GPU tensor")
    nq, nkv = -(-N // block_q), -(-N // block_kv)
    tmax = torch.empty((B * H * nq, nkv), dtype=torch.float32, device=q.device)
    tmass = torch.empty_like(tmax)
    _check(lib.sparse_attn_tile_stats(q.data_ptr(), k.data_ptr(), lse.data_ptr(), _dtype_code(q),
                                      B, H, N, D, block_q, block_kv, tmax.data_ptr(),
                                      tmass.data_ptr(), _stream(stream)), "sparse_attn_tile_stats")
    return tmax, tmass


def cube_permute(x, grid, cubes, inverse: bool = False, out=None, stream=None):
    """Moves each head's tokens of x [B, H, N, D] (raster order on the (T, Hg, W) grid)
    into the cube order of cubes[h] = (ct, ch, cw), or back with inverse=True (see
    sparse_attn_cube_permute). Returns the moved tensor."""
    torch = _torch()
    lib = load_library()
    if not (x.is_cuda and x.is_contiguous() and x.dim() == 4):
        raise ValueError("x must be a contiguous [B, H, N, D] GPU tensor")
    B, H, N, D = x.shape
    cub = np.ascontiguousarray(np.asarray(cubes, dtype=np.int32).reshape(-1))
    if cub.size != 3 * H:
        raise ValueError("cubes must give (ct, ch, cw) for every head")
    o = out if out is not None else torch.empty_like(x)
    T, Hg, W = (int(g) for g in grid)
    _check(lib.sparse_attn_cube_permute(x.data_ptr(), o.data_ptr(), _dtype_code(x), B, H, N, D, T, Hg,
                                        W, cub.ctypes.data, 1 if inverse else 0, _stream(stream)),
           "sparse_attn_cube_permute")
    return o


def router_exp(x, stream=None):
    """The router's device exp over a float32 GPU tensor (diagnostic)."""
    torch = _torch()
    lib = load_library()
    if not (x.is_cuda and x.dtype == torch.float32 and x.is_contiguous()):
        raise ValueError("x must be a contiguous float32 GPU tensor")
    y = torch.empty_like(x)
    _check(lib.sparse_attn_router_exp(x.data_ptr(), y.data_ptr(), x.numel(), _stream(stream)),
           "sparse_attn_router_exp")
    return y


def version() -> int:
    return int(load_library().sparse_attn_version())
