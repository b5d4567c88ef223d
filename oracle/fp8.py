"""Low-bit forward: Q, K, V quantised to 8-bit floats, then attention over the kept tiles.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The SLA2 page (quantisation-aware fine-tuning, component 3) runs the forward pass on
queries, keys and values quantised to low precision and keeps the backward at full
precision. The page names no format. The reading taken here:

* Format: OCP FP8 E4M3 (the "e4m3fn" variant): sign, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6; the all-ones
  exponent with all-ones mantissa is NaN; there is no infinity, so the largest finite
  magnitude is 1.75 * 2^8 = 448.
* Scaling: each group of values shares a power-of-two scale 2^e, with e the smallest
  integer such that the group's largest magnitude is at most 448 * 2^e, clamped to
  [-64, 64] (an all-zero group takes -64). A value x is stored as the code of
  x * 2^-e rounded to the nearest E4M3 value, ties to the even code. Multiplying by
  a power of two is exact, so the only rounding is that one.
* Groups: Q per (batch, head, query block), K per (batch, head, KV block), V per
  (batch, head, channel) over all tokens.
* Attention then runs in float64 on the decoded values code * 2^e
  (``oracle.attention.sparse_attention``): the quantisation is the definition of the
  low-bit forward, and everything after it is exact here.

A second format keeps V as above and stores Q and K as symmetric 8-bit integers (the
same groups), a more accurate choice for the logits on gfx950 at the same peak rate:
for a group with largest magnitude a (an fp32 value), the inverse scale
inv = fp32(127 / a) and the scale s = fp32(a / 127) are single fp32 divisions, a value
x is stored as rint(fp32(x * inv)) (round half to even; it lies in [-127, 127]) and
decodes to code * s. An all-zero group takes inv = s = 0. Every step is one IEEE fp32
operation, so the codes are reproducible exactly.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .attention import sparse_attention

E4M3_MAX = 448.0
EXP_MIN, EXP_MAX = -64, 64


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each E4M3 code (uint8); NaN for the two NaN codes."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = (c & 7).astype(np.float64)
    normal = np.ldexp(1.0 + mf / 8.0, (ef - 7).astype(np.int64))
    sub = np.ldexp(mf / 8.0, -6)
    mag = np.where(ef == 0, sub, normal)
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """Code (uint8) of the E4M3 value nearest to each x, ties to the even code. Every
    |x| must be at most 448 (the caller scales first); NaN is not accepted."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN input")
    a = np.abs(x)
    if (a > E4M3_MAX).any():
        raise ValueError("|x| > 448: scale the group first")
    # binade of a: a = f * 2^p with f in [0.5, 1), so 2^(p-1) <= a < 2^p; values below
    # 2^-6 share the subnormal spacing 2^-9
    _, p = np.frexp(a)
    E = np.maximum(p - 1, -6)
    step = np.ldexp(1.0, E - 3)            # spacing of E4M3 values at that binade
    n = np.rint(a / step).astype(np.int64)  # exact quotient; rint rounds half to even
    # n = 8..16 inside a normal binade (16 carries into the next one), 0..8 below 2^-6.
    # Code = (biased exponent << 3) | mantissa; with n steps of 2^(E-3) above zero:
    #   normal, E >= -6: code = ((E + 7) << 3) + (n - 8), which also covers the carry n = 16;
    #   subnormal range (a < 2^-6): code = n (n = 8 is 2^-6, the smallest normal).
    sub = a < np.ldexp(1.0, -6)
    code = np.where(sub, n, ((E + 7) << 3) + (n - 8))
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


def scale_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e, clamped to [-64, 64]; -64 for 0."""
    a = np.asarray(amax, dtype=np.float64)
    out = np.full(a.shape, EXP_MIN, dtype=np.int64)
    nz = a > 0
    e = np.ceil(np.log2(np.where(nz, a, 1.0) / E4M3_MAX)).astype(np.int64)
    # correct the rare off-by-one of the floating log
    e = np.where(nz & (np.ldexp(E4M3_MAX, e - 1) >= a), e - 1, e)
    e = np.where(nz & (np.ldexp(E4M3_MAX, e) < a), e + 1, e)
    out = np.where(nz, e, out)
    return np.clip(out, EXP_MIN, EXP_MAX)


def _quantize_groups(x: np.ndarray, e: np.ndarray) -> np.ndarray:
    """Codes of x * 2^-e, e broadcast against x."""
    return e4m3_encode(np.ldexp(np.asarray(x, np.float64), -e))


def quantize_qkv(q, k, v, block_q: int, block_kv: int):
    """(qc, qe, kc, ke, vc, ve) for q, k, v [B, H, N, D]:
    qc, kc, vc uint8 [B, H, N, D] codes; qe int [B, H, nQ]; ke [B, H, nKV]; ve [B, H, D]."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, H, N, D = q.shape
    nQ, nKV = -(-N // block_q), -(-N // block_kv)

    def per_block(x, bs, nb):
        pad = nb * bs - N
        ax = np.abs(x)
        if pad:
            ax = np.concatenate([ax, np.zeros((B, H, pad, D))], axis=2)
        amax = ax.reshape(B, H, nb, bs * D).max(axis=3)
        e = scale_exponent(amax)
        et = np.repeat(e, bs, axis=2)[:, :, :N, None]
        return _quantize_groups(x, et), e

    qc, qe = per_block(q, block_q, nQ)
    kc, ke = per_block(k, block_kv, nKV)
    ve = scale_exponent(np.abs(v).max(axis=2))
    vc = _quantize_groups(v, ve[:, :, None, :])
    return qc, qe, kc, ke, vc, ve


def dequantize(qc, qe, kc, ke, vc, ve, block_q: int, block_kv: int):
    """float64 q, k, v from codes and exponents (exact)."""
    N = qc.shape[2]
    q = np.ldexp(e4m3_decode(qc), np.repeat(qe, block_q, axis=2)[:, :, :N, None])
    k = np.ldexp(e4m3_decode(kc), np.repeat(ke, block_kv, axis=2)[:, :, :N, None])
    v = np.ldexp(e4m3_decode(vc), ve[:, :, None, :])
    return q, k, v


def fp8_attention(q, k, v, row_ptr, col_idx, block_q: int, block_kv: int,
                  rows=None) -> np.ndarray:
    """The low-bit forward: quantise q, k, v as above, then block-sparse attention in
    float64 on the decoded values. Returns O [B, H, N, D] float64."""
    qc, qe, kc, ke, vc, ve = quantize_qkv(q, k, v, block_q, block_kv)
    qd, kd, vd = dequantize(qc, qe, kc, ke, vc, ve, block_q, block_kv)
    return sparse_attention(qd, kd, vd, row_ptr, col_idx, block_q, block_kv, rows=rows)


def int8_scales(amax):
    """(inv, s) float32 for group maxima amax: inv = fp32(127 / a), s = fp32(a / 127);
    0 and 0 for a zero group."""
    a = np.asarray(amax, dtype=np.float32)
    nz = a > 0
    safe = np.where(nz, a, np.float32(1))
    inv = np.where(nz, np.float32(127) / safe, np.float32(0)).astype(np.float32)
    sc = np.where(nz, safe / np.float32(127), np.float32(0)).astype(np.float32)
    return inv, sc


def int8_encode(x, inv):
    """rint(fp32(x * inv)) as int8, x and inv float32 (broadcast)."""
    y = np.asarray(x, dtype=np.float32) * np.asarray(inv, dtype=np.float32)
    return np.rint(y).astype(np.int8)


def quantize_qkv_i8qk(q, k, v, block_q: int, block_kv: int):
    """(qc, qs, kc, ks, vc, ve): Q and K as int8 codes [B, H, N, D] with fp32 scales per
    query block [B, H, nQ] and per KV block [B, H, nKV]; V as quantize_qkv."""
    q32, k32 = (np.asarray(t, dtype=np.float32) for t in (q, k))
    B, H, N, D = q32.shape

    def per_block(x, bs):
        nb = -(-N // bs)
        pad = nb * bs - N
        ax = np.abs(x)
        if pad:
            ax = np.concatenate([ax, np.zeros((B, H, pad, D), np.float32)], axis=2)
        amax = ax.reshape(B, H, nb, bs * D).max(axis=3)
        inv, sc = int8_scales(amax)
        codes = int8_encode(x, np.repeat(inv, bs, axis=2)[:, :, :N, None])
        return codes, sc

    qc, qs = per_block(q32, block_q)
    kc, ks = per_block(k32, block_kv)
    ve = scale_exponent(np.abs(np.asarray(v, np.float64)).max(axis=2))
    vc = _quantize_groups(v, ve[:, :, None, :])
    return qc, qs, kc, ks, vc, ve


def dequantize_i8qk(qc, qs, kc, ks, vc, ve, block_q: int, block_kv: int):
    """float64 q, k, v from the int8-QK format (exact)."""
    N = qc.shape[2]
    q = qc.astype(np.float64) * np.repeat(qs.astype(np.float64), block_q, axis=2)[:, :, :N, None]
    k = kc.astype(np.float64) * np.repeat(ks.astype(np.float64), block_kv, axis=2)[:, :, :N, None]
    v = np.ldexp(e4m3_decode(vc), ve[:, :, None, :])
    return q, k, v


def i8qk_attention(q, k, v, row_ptr, col_idx, block_q: int, block_kv: int, rows=None):
    """The low-bit forward with int8 Q and K: quantise as above, then block-sparse
    attention in float64 on the decoded values."""
    parts = quantize_qkv_i8qk(q, k, v, block_q, block_kv)
    qd, kd, vd = dequantize_i8qk(*parts, block_q, block_kv)
    return sparse_attention(qd, kd, vd, row_ptr, col_idx, block_q, block_kv, rows=rows)
