"""The pipelined call (plan + forward over chunks of heads on two streams) against the
two-call path: a head's mask and output depend on that head alone, so o and lse must be
equal bit for bit for every chunking, including chunks that cut a batch's heads and a
last chunk shorter than the others."""
import numpy as np
import pytest
import torch

import block_sparse_attention_05_amd as sa
import workloads as W
from tests.gpu_common import inputs, log

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, H, N, D, dtype, block_q, topk, top_p, chunks
    ("pipe_b2h3_c4", 2, 3, 1000, 64, "bf16", 64, 0.1, 0.9, 4),
    ("pipe_h5_c2", 1, 5, 3000, 128, "bf16", 128, 0.05, 0.9, 2),
    ("pipe_h4_c8", 1, 4, 2048, 128, "bf16", 128, 0.1, 0.85, 8),
    ("pipe_fp32_c3", 1, 3, 700, 64, "fp32", 64, 0.25, 0.9, 3),
]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pipelined_equals_two_calls(case):
    name, B, H, N, D, dt, bq, topk, p, C = case
    w = W.Workload(name, B, H, D, (1, 1, N), dt, bq, 64, topk, p, 4, seed=5)
    ent = inputs(w)
    plan = sa.plan(ent["dq"], ent["dk"], bq, 64, topk, p)
    o1, l1 = sa.fwd(ent["dq"], ent["dk"], ent["dv"], plan, return_lse=True)
    o2, l2 = sa.attention(ent["dq"], ent["dk"], ent["dv"], bq, 64, topk, p, chunks=C, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o1), _bits(o2)), "o"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), "lse"
    # one stream for both: the chunks run in order. Without the LSE output the bf16
    # forward keeps a lazy running max, so the reference is the two-call path without it.
    s = torch.cuda.current_stream()
    o3 = sa.attention(ent["dq"], ent["dk"], ent["dv"], bq, 64, topk, p, chunks=C, stream=s, aux_stream=s)
    o4 = sa.fwd(ent["dq"], ent["dk"], ent["dv"], plan)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o4), _bits(o3)), "o, one stream"
    log(f"{name}: pipelined over {C} chunks equals the two-call path bitwise")


def test_pipelined_orders_with_caller_stream():
    """Work the caller enqueues after the call sees the finished output, and the call sees
    the caller's earlier writes (inputs overwritten right before the call)."""
    w = W.Workload("pipe_order", 1, 6, 64, (1, 1, 1500), "bf16", 64, 64, 0.1, 0.9, 4, seed=6)
    ent = inputs(w)
    q = torch.zeros_like(ent["dq"])
    ref = sa.attention(ent["dq"], ent["dk"], ent["dv"], 64, 64, 0.1, 0.9, chunks=6)
    torch.cuda.synchronize()
    for _ in range(3):
        q.zero_()
        q.copy_(ent["dq"])                       # enqueued on the current stream
        o = sa.attention(q, ent["dk"], ent["dv"], 64, 64, 0.1, 0.9, chunks=6)
        snap = o.clone()                         # enqueued after the call
        torch.cuda.synchronize()
        assert torch.equal(snap.view(torch.int16), ref.view(torch.int16))


def test_pipelined_720p_as_benchmarked():
    """The 720p shape in the benchmark's launch configuration: 4 chunks on two streams, no
    LSE output, one caller-owned output and workspace reused by back-to-back calls. Each
    call is bitwise equal to the two-call path, whose output the parity tests check
    against the oracle at this shape."""
    w = W.CONFIGS["wan14b_720p"]
    ent = inputs(w)
    plan = sa.plan(ent["dq"], ent["dk"], w.block_q, w.block_kv, w.topk, w.top_p)
    ref = sa.fwd(ent["dq"], ent["dk"], ent["dv"], plan)
    ws = torch.empty(sa.pipelined_workspace_bytes(w.B, w.H, w.N, w.D, w.block_q, w.block_kv, 4),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(ref)
    for call in range(2):
        out.fill_(float("nan"))
        sa.attention(ent["dq"], ent["dk"], ent["dv"], w.block_q, w.block_kv, w.topk, w.top_p, chunks=4,
                     out=out, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref)), f"call {call}"
    log("720p: pipelined over 4 chunks, workspace reused, bitwise equal to the two-call path")


LIN_CASES = [
    # name, B, H, N, block_q, topk, top_p, chunks: chunks that cut a batch's heads (alpha rows
    # taken modulo H), one chunk, and more chunks than heads
    ("pipe_lin_b2h3_c4", 2, 3, 1000, 64, 0.1, 0.8, 4),
    ("pipe_lin_h4_c1", 1, 4, 2500, 128, 0.05, 0.8, 1),
    ("pipe_lin_h3_c8", 1, 3, 1536, 128, 0.2, 0.9, 8),
]


@pytest.mark.parametrize("case", LIN_CASES, ids=[c[0] for c in LIN_CASES])
def test_pipelined_linear_equals_two_calls(case):
    """With the linear branch each chunk's prepass runs beside the plans; o and lse must
    still equal plan + fwd(alpha) bit for bit, on two streams and on one."""
    name, B, H, N, bq, topk, p, C = case
    w = W.Workload(name, B, H, 128, (1, 1, N), "bf16", bq, 64, topk, p, 4, linear=True, seed=8)
    ent = inputs(w)
    plan = sa.plan(ent["dq"], ent["dk"], bq, 64, topk, p)
    o1, l1 = sa.fwd(ent["dq"], ent["dk"], ent["dv"], plan, alpha=ent["dalpha"], return_lse=True)
    o2, l2 = sa.attention(ent["dq"], ent["dk"], ent["dv"], bq, 64, topk, p, chunks=C, return_lse=True,
                          alpha=ent["dalpha"])
    torch.cuda.synchronize()
    assert torch.equal(_bits(o1), _bits(o2)), "o"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), "lse"
    s = torch.cuda.current_stream()
    o3 = sa.attention(ent["dq"], ent["dk"], ent["dv"], bq, 64, topk, p, chunks=C, stream=s, aux_stream=s,
                      alpha=ent["dalpha"])
    o4 = sa.fwd(ent["dq"], ent["dk"], ent["dv"], plan, alpha=ent["dalpha"])
    torch.cuda.synchronize()
    assert torch.equal(_bits(o4), _bits(o3)), "o, one stream"
    log(f"{name}: pipelined linear over {C} chunks equals the two-call path bitwise")


def test_pipelined_sparse_linear_as_benchmarked():
    """The sparse+linear workload in the benchmark's launch configuration (one chunk, two
    streams, the prepass beside the plan), workspace reused by back-to-back calls."""
    w = W.CONFIGS["sparse_linear"]
    ent = inputs(w)
    plan = sa.plan(ent["dq"], ent["dk"], w.block_q, w.block_kv, w.topk, w.top_p)
    ref = sa.fwd(ent["dq"], ent["dk"], ent["dv"], plan, alpha=ent["dalpha"])
    ws = torch.empty(sa.pipelined_workspace_bytes(w.B, w.H, w.N, w.D, w.block_q, w.block_kv, 1, linear=True),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(ref)
    for call in range(2):
        out.fill_(float("nan"))
        sa.attention(ent["dq"], ent["dk"], ent["dv"], w.block_q, w.block_kv, w.topk, w.top_p, chunks=1,
                     out=out, workspace=ws, alpha=ent["dalpha"])
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref)), f"call {call}"
    log("sparse_linear: pipelined (one chunk, prepass beside the plan) bitwise equal to the two-call path")
