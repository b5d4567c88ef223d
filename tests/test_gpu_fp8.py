"""GPU parity of the low-bit forward (SLA2 page, quantisation-aware fine-tuning: Q, K, V
quantised for the forward pass), through the C ABI.

* Quantisation: the pack's codes and exponents equal the oracle's bit for bit (the
  rounding decision is the same on both sides: x * 2^-e is exact, then one
  round-to-nearest-even to E4M3).
* Attention: the kernel against the oracle's low-bit forward (float64 attention on the
  decoded values). The kernel's one deliberate rounding is P * 2^8 to E4M3 before the PV
  product (row sums add the same rounded values); modelled on the CPU with the oracle's
  encoder on these inputs, it moves O by rel-RMS 5.4e-3 to 5.8e-3 and at most 1.35% of
  max |v| (tests/test_oracle_fp8.py pins that model below these bounds). fp32 softmax,
  the MFMA's accumulation and the bf16 store add far less. Bounds: rel-RMS 1e-2, max
  |dO| 3% of max |v|. lse: each rounded P lies within 2^-4 of P (relative) in the normal
  range, so the row sum, and lse, move by at most about 2^-4: bound 0.07.
* Without the LSE output the kernel's running max is lazy (it trails the true max by up
  to 2^4) and P is rounded as P * 2^4: the same relative rounding in the E4M3 normal
  range, and the row sums still add the rounded values, so O is held to the same bars.
* The distance to exact attention on the bf16 inputs is the format's own error (3
  mantissa bits on the logits) and is logged, not bounded tightly.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_05_amd as sa
import workloads as W
from oracle import sparse_attention
from oracle.fp8 import dequantize, dequantize_i8qk, quantize_qkv, quantize_qkv_i8qk
from tests.gpu_common import inputs, log, to_f64

pytestmark = pytest.mark.gpu

TOL_RRMS = 1e-2
TOL_MAX_FRAC_V = 0.03
TOL_LSE = 0.07

CASES = [
    # name, B, H, N, D, block_q, topk, top_p
    ("fp8_d64_q64_ragged", 1, 2, 1000, 64, 64, 0.1, 0.9),
    ("fp8_d128_q128_ragged", 2, 2, 3000, 128, 128, 0.05, 0.9),
    ("fp8_d128_q64", 1, 2, 2048, 128, 64, 0.1, 0.85),
    ("fp8_d64_q128", 1, 3, 1536, 64, 128, 0.1, 0.7),
    ("fp8_n37", 1, 2, 37, 128, 128, 0.5, 0.9),
]


def pi_keys():
    """Key of byte h*32 + b of a V^T row, as the pack's layout documents it."""
    return np.array([(b // 16) * 32 + ((b // 4) % 4) * 8 + h * 4 + b % 4 for h in range(2) for b in range(32)])


def unpack_vt(vt8: np.ndarray, N: int) -> np.ndarray:
    """[B, H, nKV, D, 64] -> [B, H, N, D] codes, checking the bytes past N are zero."""
    B, H, nKV, D, _ = vt8.shape
    out = np.zeros((B, H, nKV * 64, D), np.uint8)
    keys = pi_keys()
    for J in range(nKV):
        out[:, :, J * 64 + keys, :] = np.transpose(vt8[:, :, J], (0, 1, 3, 2))
    assert not out[:, :, N:].any(), "V^T bytes past N must be zero"
    return out[:, :, :N]


def _case(case):
    name, B, H, N, D, bq, topk, p = case
    w = W.Workload(name, B, H, D, (1, 1, N), "bf16", bq, 64, topk, p, 4, seed=1)
    return w, inputs(w)


def _oracle_codes(ent, w, qk):
    v32 = W.to_f32(ent["v"])
    if qk == "int8":
        return quantize_qkv_i8qk(ent["q32"], ent["k32"], v32, w.block_q, 64)
    return quantize_qkv(ent["q32"], ent["k32"], v32, w.block_q, 64)


def _oracle_decoded(ent, w, qk):
    parts = _oracle_codes(ent, w, qk)
    return (dequantize_i8qk if qk == "int8" else dequantize)(*parts, w.block_q, 64)


QK = ["e4m3", "int8"]


@pytest.mark.parametrize("qk", QK)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_quantize_bitexact(case, qk):
    w, ent = _case(case)
    pack = sa.quantize_fp8(ent["dq"], ent["dk"], ent["dv"], w.block_q, qk=qk)
    torch.cuda.synchronize()
    qc, qe, kc, ke, vc, ve = _oracle_codes(ent, w, qk)
    bits = (lambda t: t.cpu().numpy().view(np.int32)) if qk == "int8" else (lambda t: t.cpu().numpy())
    ref_bits = (lambda a: np.asarray(a, np.float32).view(np.int32)) if qk == "int8" else (lambda a: a)
    assert np.array_equal(bits(pack.part("qe")), ref_bits(qe))
    assert np.array_equal(bits(pack.part("ke")), ref_bits(ke))
    assert np.array_equal(pack.part("ve").cpu().numpy(), ve)
    assert np.array_equal(pack.part("q8").cpu().numpy(), qc)
    assert np.array_equal(pack.part("k8").cpu().numpy(), kc)
    assert np.array_equal(unpack_vt(pack.part("vt8").cpu().numpy(), w.N), vc)
    log(f"{case[0]} {qk}: codes and scales bit-exact (v exps {ve.min()}..{ve.max()})")


def _check(o, ref, vmax, what):
    assert np.all(np.isfinite(o)), f"{what}: non-finite"
    err = np.abs(o - ref)
    rr = float(np.sqrt((err ** 2).sum()) / np.sqrt((ref ** 2).sum()))
    mx = float(err.max())
    assert rr <= TOL_RRMS, f"{what}: rel-RMS {rr:.3e}"
    assert mx <= TOL_MAX_FRAC_V * vmax, f"{what}: max |dO| {mx:.3e} vs max |v| {vmax:.3f}"
    return rr, mx


@pytest.mark.parametrize("qk", QK)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fwd_fp8_parity(case, qk):
    w, ent = _case(case)
    plan = sa.plan(ent["dq"], ent["dk"], w.block_q, 64, w.topk, w.top_p)
    pack = sa.quantize_fp8(ent["dq"], ent["dk"], ent["dv"], w.block_q, qk=qk)
    o, lse = sa.fwd_fp8(pack, plan, return_lse=True)
    rp, ci = plan.csr()
    v32 = W.to_f32(ent["v"])
    qd, kd, vd = _oracle_decoded(ent, w, qk)
    ref, ref_lse = sparse_attention(qd, kd, vd, rp, ci, w.block_q, 64, with_lse=True)
    rr, mx = _check(to_f64(o), ref, float(np.abs(vd).max()), case[0])
    rr2, mx2 = _check(to_f64(sa.fwd_fp8(pack, plan)), ref, float(np.abs(vd).max()), case[0] + " no lse")
    dl = np.abs(lse.cpu().numpy() - ref_lse)
    assert float(dl.max()) <= TOL_LSE, f"lse: max {dl.max():.3e}"
    exact = sparse_attention(ent["q32"], ent["k32"], v32, rp, ci, w.block_q, 64)
    e = to_f64(o) - exact
    log(f"{case[0]} {qk}: nnz {rp[-1]}; vs the low-bit oracle rel-RMS {rr:.2e}, max {mx:.2e} "
        f"(without lse {rr2:.2e}, {mx2:.2e}), lse max {dl.max():.2e}; "
        f"vs exact attention on the bf16 inputs rel-RMS {np.sqrt((e ** 2).sum() / (exact ** 2).sum()):.2e}")


def test_fwd_fp8_empty_rows_and_ragged_only_row():
    """Caller mask: row 1 keeps nothing (o = 0, lse = -inf); row 4 keeps only the ragged
    last KV block."""
    w = W.Workload("fp8_edges", 1, 1, 64, (1, 1, 300), "bf16", 64, 64, 0.5, 0.9, 2, seed=3)
    ent = inputs(w)
    rp = np.array([0, 2, 2, 4, 5, 6], dtype=np.int32)
    ci = np.array([0, 1, 0, 3, 4, 4], dtype=np.int32)
    plan = sa.plan_from_csr(ent["dq"], rp, ci, 64, 64)
    pack = sa.quantize_fp8(ent["dq"], ent["dk"], ent["dv"], 64)
    o, lse = sa.fwd_fp8(pack, plan, return_lse=True)
    got = to_f64(o)
    assert not got[0, 0, 64:128].any()
    assert np.all(np.isneginf(lse.cpu().numpy()[0, 0, 64:128]))
    qd, kd, vd = dequantize(*quantize_qkv(ent["q32"], ent["k32"], W.to_f32(ent["v"]), 64, 64), 64, 64)
    ref = sparse_attention(qd, kd, vd, rp, ci, 64, 64)
    _check(got, ref, float(np.abs(vd).max()), "edges")
    o2 = to_f64(sa.fwd_fp8(pack, plan))
    assert not o2[0, 0, 64:128].any()
    _check(o2, ref, float(np.abs(vd).max()), "edges, no lse")


def test_fwd_fp8_deterministic():
    w, ent = _case(CASES[1])
    plan = sa.plan(ent["dq"], ent["dk"], w.block_q, 64, w.topk, w.top_p)
    p1 = sa.quantize_fp8(ent["dq"], ent["dk"], ent["dv"], w.block_q)
    p2 = sa.quantize_fp8(ent["dq"], ent["dk"], ent["dv"], w.block_q)
    for part in ("q8", "k8", "vt8", "qe", "ke", "ve"):      # the padding between parts is never written
        assert torch.equal(p1.part(part), p2.part(part)), part
    a = sa.fwd_fp8(p1, plan)
    b = sa.fwd_fp8(p1, plan)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("qk", QK)
@pytest.mark.parametrize("workload", ["wan13b_480p", "wan14b_720p"])
def test_fp8_workload_sampled(workload, qk):
    """Full-size workloads (720p is the shape the benchmark times): codes of sampled heads
    bit-exact, outputs of sampled query blocks against the oracle."""
    from tests.gpu_common import sample_rows
    w = W.CONFIGS[workload]
    ent = inputs(w)
    plan = sa.plan(ent["dq"], ent["dk"], w.block_q, w.block_kv, w.topk, w.top_p)
    pack = sa.quantize_fp8(ent["dq"], ent["dk"], ent["dv"], w.block_q, qk=qk)
    o = sa.fwd_fp8(pack, plan)
    rp, ci = plan.csr()
    heads = [(0, 0), (0, w.H - 1)]
    hs = [h for _, h in heads]
    v32 = W.to_f32(ent["v"])
    sub = lambda x: x[:, hs]
    quant = quantize_qkv_i8qk if qk == "int8" else quantize_qkv
    qc, qe, kc, ke, vc, ve = quant(sub(ent["q32"]), sub(ent["k32"]), sub(v32), w.block_q, 64)
    assert np.array_equal(pack.part("q8")[:, hs].cpu().numpy(), qc)
    assert np.array_equal(pack.part("k8")[:, hs].cpu().numpy(), kc)
    assert np.array_equal(unpack_vt(pack.part("vt8")[:, hs].cpu().numpy(), w.N), vc)
    assert np.array_equal(pack.part("ve")[:, hs].cpu().numpy(), ve)
    qd, kd, vd = (dequantize_i8qk if qk == "int8" else dequantize)(qc, qe, kc, ke, vc, ve, w.block_q, 64)
    rows = [r for r in sample_rows(w, 6, heads=heads)]
    # the oracle on the two heads: rows re-indexed to the two-head sub-problem
    nq = w.n_qblk
    sub_rp = [0]
    sub_ci = []
    for h in hs:
        for I in range(nq):
            r = h * nq + I
            sub_ci += list(ci[rp[r]:rp[r + 1]])
            sub_rp.append(len(sub_ci))
    sub_rows = [(0, hs.index(h), I) for _, h, I in rows]
    ref = sparse_attention(qd, kd, vd, np.array(sub_rp), np.array(sub_ci), w.block_q, 64, rows=sub_rows)
    got = to_f64(o[:, hs])
    g, r = [], []
    for (b, hi, I), (ob, _) in ref.items():
        g.append(got[b, hi, I * w.block_q:min(w.N, (I + 1) * w.block_q)])
        r.append(ob)
    rr, mx = _check(np.concatenate(g), np.concatenate(r), float(np.abs(vd).max()), workload)
    log(f"{workload} {qk} sampled ({len(rows)} query blocks): rel-RMS {rr:.2e}, max {mx:.2e}")
