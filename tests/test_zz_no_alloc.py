"""The allocation-free entry point, sparse_attn_pipelined_noalloc, called through the C
ABI, against the existing sparse_attn_pipelined on the same inputs: o and lse must be
equal bit for bit (the same kernels, planning each head from its own q and k). Two calls
in a row share the library's static scratch, the second on a smaller input, so stale
contents left by the first call must not leak into the second."""
import ctypes

import pytest
import torch

import block_sparse_attention_05_amd as sa
import workloads as W
from tests.gpu_common import drop, inputs, log

pytestmark = pytest.mark.gpu


def _noalloc(lib, ent, w, o, lse):
    st = lib.sparse_attn_pipelined_noalloc(
        ent["dq"].data_ptr(), ent["dk"].data_ptr(), ent["dv"].data_ptr(), sa.SA_BF16, w.B, w.H, w.N, w.D,
        w.block_q, w.block_kv, ctypes.c_double(w.topk), ctypes.c_double(w.top_p), o.data_ptr(),
        lse.data_ptr() if lse is not None else None, torch.cuda.current_stream().cuda_stream)
    assert st == 0, sa.SparseAttnError(st, "sparse_attn_pipelined_noalloc")


def test_noalloc_equals_pipelined_twice():
    lib = sa.load_library()
    # the 720p shape (several chunks of heads through the 128 MiB scratch), then the
    # smaller 480p shape (one chunk), each with and without the LSE output
    for name in ("wan14b_720p", "wan13b_480p"):
        w = W.CONFIGS[name]
        ent = inputs(w)
        log(f"noalloc {name}: B={w.B} H={w.H} N={w.N}")
        o_ref, l_ref = sa.attention(ent["dq"], ent["dk"], ent["dv"], w.block_q, w.block_kv, w.topk, w.top_p,
                                    chunks=4, return_lse=True)
        o = torch.full_like(ent["dq"], float("nan"))
        lse = torch.full((w.B, w.H, w.N), float("nan"), dtype=torch.float32, device="cuda")
        _noalloc(lib, ent, w, o, lse)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"{name}: o with lse"
        assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32)), f"{name}: lse"
        # without the LSE output (the lazy running max) against the pipelined call likewise
        o_ref2 = sa.attention(ent["dq"], ent["dk"], ent["dv"], w.block_q, w.block_kv, w.topk, w.top_p, chunks=4)
        o2 = torch.full_like(ent["dq"], float("nan"))
        _noalloc(lib, ent, w, o2, None)
        torch.cuda.synchronize()
        assert torch.equal(o2.view(torch.int16), o_ref2.view(torch.int16)), f"{name}: o"
        log(f"noalloc {name}: bitwise equal to sparse_attn_pipelined")
        del o, lse, o2, o_ref, o_ref2, l_ref
        drop(w)
