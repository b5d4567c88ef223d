"""Pins of the low-bit (FP8 E4M3) forward oracle against facts outside it: the OCP E4M3
format's stated values, torch's own float8_e4m3fn conversions (a library routine), ties
worked by hand, brute-force minimality of the scale exponent, the rounding bound, and
special cases where quantisation is the identity."""
import numpy as np
import pytest
import torch

from oracle import dense_plan, sparse_attention
from oracle.fp8 import (dequantize, e4m3_decode, e4m3_encode, fp8_attention, quantize_qkv,
                        scale_exponent)


def test_decode_format_facts():
    # OCP 8-bit floating point specification, E4M3: max normal S.1111.110 = 448, min
    # normal 2^-6, max subnormal 0.875 * 2^-6, min subnormal 2^-9, NaN S.1111.111,
    # no infinities; 1.0 = 0.0111.000
    v = e4m3_decode(np.array([0x7E, 0xFE, 0x08, 0x07, 0x01, 0x38, 0xB8, 0x00], np.uint8))
    assert list(v) == [448.0, -448.0, 2.0 ** -6, 0.875 * 2.0 ** -6, 2.0 ** -9, 1.0, -1.0, 0.0]
    assert np.isnan(e4m3_decode(np.array([0x7F, 0xFF]))).all()
    assert np.signbit(e4m3_decode(np.array([0x80])))[0]
    assert np.isfinite(e4m3_decode(np.arange(256))).sum() == 254


def test_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def _bf16_values_in_range():
    bits = np.arange(65536, dtype=np.uint32) << 16
    finite = ((bits >> 23) & 0xFF) != 0xFF          # exponent field not all ones
    return bits[finite].view(np.float32).astype(np.float64)


@pytest.mark.parametrize("shift", [0, -4, 6])
def test_encode_matches_torch_on_every_bf16(shift):
    x = np.ldexp(_bf16_values_in_range(), shift)
    x = x[np.abs(x) <= 448.0]
    got = e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_encode_ties_by_hand():
    # 1 + 1/16 lies halfway between 1.0 (mantissa 0, even) and 1.125 (mantissa 1)
    # 1 + 3/16 lies halfway between 1.125 (odd) and 1.25 (mantissa 2, even)
    # 3 * 2^-10 lies halfway between the subnormals 2^-9 (odd) and 2^-8 (even)
    # 2^-10 lies halfway between 0 (even) and 2^-9
    # 432 lies halfway between 416 (mantissa 5) and 448 (mantissa 6)
    x = np.array([1 + 1 / 16, 1 + 3 / 16, 3 * 2.0 ** -10, 2.0 ** -10, 432.0, -432.0])
    assert list(e4m3_encode(x)) == [0x38, 0x3A, 0x02, 0x00, 0x7E, 0xFE]


def test_encode_decode_round_trip():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        e4m3_encode(np.array([449.0]))


def test_scale_exponent_minimal_by_brute_force():
    rng = np.random.default_rng(0)
    amax = np.concatenate([np.exp(rng.uniform(-30, 30, 2000)), [448.0, 449.0, 224.0, 896.0, 1.0]])
    e = scale_exponent(amax)
    for a, ei in zip(amax, e):
        best = next(t for t in range(-64, 65) if a <= 448.0 * 2.0 ** t)
        assert ei == best, (a, ei, best)
    assert list(scale_exponent(np.array([0.0, 1e-40, 1e40]))) == [-64, -64, 64]


def test_quantize_error_bound():
    rng = np.random.default_rng(1)
    B, H, N, D = 1, 2, 200, 64
    q, k, v = (rng.normal(size=(B, H, N, D)) * s for s in (1.0, 3.0, 0.5))
    qc, qe, kc, ke, vc, ve = quantize_qkv(q, k, v, 64, 64)
    qd, kd, vd = dequantize(qc, qe, kc, ke, vc, ve, 64, 64)
    for x, xd, e in ((q, qd, np.repeat(qe, 64, axis=2)[:, :, :N, None]),
                     (k, kd, np.repeat(ke, 64, axis=2)[:, :, :N, None]),
                     (v, vd, ve[:, :, None, :])):
        # relative 2^-4 in the normal range, half a subnormal step (2^-10 * 2^e) below it
        bound = np.maximum(np.abs(x) * 2.0 ** -4, np.ldexp(1.0, (e - 10).astype(int)))
        assert np.all(np.abs(xd - x) <= bound)
    # the largest magnitude of each group is scaled into (224, 448], so its code decodes
    # to at least 224 (ragged last block included)
    dq = np.abs(e4m3_decode(qc))
    for blk in range(-(-N // 64)):
        assert np.all(dq[:, :, blk * 64:(blk + 1) * 64].max(axis=(2, 3)) >= 224)
    assert np.all(np.abs(e4m3_decode(vc)).max(axis=2) >= 224)


def _on_grid(rng, shape, e):
    codes = rng.integers(0, 256, size=shape).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    x = e4m3_decode(codes)
    return x, codes


def test_identity_quantisation_and_attention():
    """Inputs already on the E4M3 grid, each group holding 448 * 2^e: the codes come back
    unchanged and the low-bit forward equals float64 attention on the same values."""
    rng = np.random.default_rng(2)
    B, H, N, D, bq, bk = 1, 1, 192, 64, 64, 64
    q, qcode = _on_grid(rng, (B, H, N, D), 0)
    k, kcode = _on_grid(rng, (B, H, N, D), 0)
    v, vcode = _on_grid(rng, (B, H, N, D), 0)
    # scale to the inputs' ranges and pin each group's max to 448 * 2^e
    q, k = q / 64.0, k / 64.0
    for blk in range(N // bq):
        q[0, 0, blk * bq, 0] = 448.0 / 64.0
    for blk in range(N // bk):
        k[0, 0, blk * bk, 0] = -448.0 / 64.0
    v[0, 0, 0, :] = 448.0
    qc, qe, kc, ke, vc, ve = quantize_qkv(q, k, v, bq, bk)
    assert (qe == -6).all() and (ke == -6).all() and (ve == 0).all()
    qd, kd, vd = dequantize(qc, qe, kc, ke, vc, ve, bq, bk)
    assert np.array_equal(qd, q) and np.array_equal(kd, k) and np.array_equal(vd, v)
    rp, ci = dense_plan(B, H, N, bq, bk)
    assert np.array_equal(fp8_attention(q, k, v, rp, ci, bq, bk), sparse_attention(q, k, v, rp, ci, bq, bk))


def test_power_of_two_scaling_commutes():
    rng = np.random.default_rng(3)
    B, H, N, D = 1, 2, 130, 64
    q, k, v = (rng.normal(size=(B, H, N, D)) for _ in range(3))
    rp, ci = dense_plan(B, H, N, 64, 64)
    o1 = fp8_attention(q, k, v, rp, ci, 64, 64)
    o2 = fp8_attention(q, k, v * 8.0, rp, ci, 64, 64)
    assert np.array_equal(o2, o1 * 8.0)
    _, qe, _, ke, _, ve = quantize_qkv(q * 0.25, k, v * 8.0, 64, 64)
    _, qe0, _, _, _, ve0 = quantize_qkv(q, k, v, 64, 64)
    assert np.array_equal(qe, qe0 - 2) and np.array_equal(ve, ve0 + 3)


def test_p_rounding_model_below_gpu_bounds():
    """The model behind the GPU bounds for the low-bit forward: rounding P * 2^8 to E4M3
    (the kernel's one deliberate rounding after quantisation) moves O, on a seeded case
    like the GPU tests', by less than half the bounds those tests use (rel-RMS 1e-2, max
    3% of max |v|)."""
    import math
    rng = np.random.default_rng(7)
    N, D = 512, 64
    q, k, v = (rng.normal(size=(N, D)) + s for s in (1.0, 1.0, 0.0))
    k[::97] *= 8.0                                    # sink keys, as the generator's
    qd, kd, vd = (dequantize(*quantize_qkv(x[None, None], x[None, None], x[None, None], 64, 64), 64, 64)[i][0, 0]
                  for i, x in enumerate((q, k, v)))
    s_ = qd @ kd.T / math.sqrt(D)
    p = np.exp(s_ - s_.max(axis=1, keepdims=True)) * 256.0
    ph = e4m3_decode(e4m3_encode(p))
    o = (p @ vd) / p.sum(axis=1, keepdims=True)
    oh = (ph @ vd) / ph.sum(axis=1, keepdims=True)
    rr = np.sqrt(((oh - o) ** 2).sum() / (o ** 2).sum())
    mx = np.abs(oh - o).max() / np.abs(vd).max()
    assert rr < 0.5e-2 and mx < 0.015, (rr, mx)
    assert rr > 1e-4                                  # the rounding does act


# ------------------------------------------------------------------ int8 Q and K
from oracle.fp8 import (dequantize_i8qk, i8qk_attention, int8_encode, int8_scales,  # noqa: E402
                        quantize_qkv_i8qk)


def test_int8_scales_are_correctly_rounded_divisions():
    """fp32 a / 127 and 127 / a: a quotient of two fp32 values computed in fp64 and rounded
    once to fp32 is the correctly rounded fp32 quotient (53 >= 2*24 + 2)."""
    rng = np.random.default_rng(11)
    a = np.concatenate([np.exp(rng.uniform(-20, 20, 5000)), [1.0, 127.0, 254.0, 3.0e-30]]).astype(np.float32)
    inv, sc = int8_scales(a)
    assert np.array_equal(sc, (a.astype(np.float64) / 127.0).astype(np.float32))
    assert np.array_equal(inv, (127.0 / a.astype(np.float64)).astype(np.float32))
    z_inv, z_sc = int8_scales(np.zeros(3, np.float32))
    assert not z_inv.any() and not z_sc.any()


def test_int8_encode_is_nearest_with_ties_to_even():
    rng = np.random.default_rng(12)
    y = np.concatenate([rng.uniform(-127, 127, 4000), np.arange(-127, 127) + 0.5]).astype(np.float32)
    got = int8_encode(y, np.float32(1)).astype(np.int64)
    cand = np.arange(-127, 128)
    d = np.abs(y.astype(np.float64)[:, None] - cand[None, :])
    best = d.min(axis=1, keepdims=True)
    ties = (d == best)
    # nearest; on a tie the even candidate
    want = np.array([c[t][np.argmax(c[t] % 2 == 0)] if t.sum() > 1 else c[t][0]
                     for c, t in zip(np.broadcast_to(cand, d.shape), ties)])
    assert np.array_equal(got, want)


def test_int8_qk_bounds_and_group_max():
    rng = np.random.default_rng(13)
    B, H, N, D = 1, 2, 200, 64
    q, k, v = (rng.normal(size=(B, H, N, D)).astype(np.float32) * s for s in (1.0, 3.0, 0.5))
    qc, qs, kc, ks, vc, ve = quantize_qkv_i8qk(q, k, v, 64, 64)
    assert qc.dtype == np.int8 and np.abs(qc.astype(int)).max() <= 127
    qd, kd, _ = dequantize_i8qk(qc, qs, kc, ks, vc, ve, 64, 64)
    for x, xd, sc in ((q, qd, np.repeat(qs, 64, axis=2)[:, :, :N, None]),
                      (k, kd, np.repeat(ks, 64, axis=2)[:, :, :N, None])):
        bound = sc.astype(np.float64) / 2 + np.abs(x) * 2.0 ** -22
        assert np.all(np.abs(xd - x) <= bound)
    for blk in range(-(-N // 64)):
        assert np.all(np.abs(qc[:, :, blk * 64:(blk + 1) * 64].astype(int)).max(axis=(2, 3)) == 127)


def test_int8_qk_identity_case():
    """Integer-valued q and k whose groups reach 127 quantise to themselves (scale 1), and
    the forward equals float64 attention on them."""
    rng = np.random.default_rng(14)
    B, H, N, D, bq, bk = 1, 1, 192, 64, 64, 64
    q = rng.integers(-127, 128, size=(B, H, N, D)).astype(np.float32)
    k = rng.integers(-127, 128, size=(B, H, N, D)).astype(np.float32)
    q[:, :, ::64, 0] = 127
    k[:, :, ::64, 0] = -127
    v = rng.normal(size=(B, H, N, D))
    qc, qs, kc, ks, vc, ve = quantize_qkv_i8qk(q, k, v, bq, bk)
    assert (qs == 1).all() and (ks == 1).all()
    assert np.array_equal(qc.astype(np.float32), q) and np.array_equal(kc.astype(np.float32), k)
    rp, ci = dense_plan(B, H, N, bq, bk)
    _, _, vd = dequantize_i8qk(qc, qs, kc, ks, vc, ve, bq, bk)
    ref = sparse_attention(q.astype(np.float64) / 16, k.astype(np.float64) / 16, vd, rp, ci, bq, bk)
    got = i8qk_attention(q / 16, k / 16, v, rp, ci, bq, bk)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
