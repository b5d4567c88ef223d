"""Pins of the oracle's block-sparse attention gradients against facts outside it: central
finite differences of the oracle's own forward (a different code path: no gradient
formula), torch autograd on the dense mask, and zero gradients for masked-out tokens."""
import numpy as np
import pytest
import torch

from oracle import dense_plan, sparse_attention, sparse_attention_backward


def _case(seed=0, B=1, H=2, N=40, D=8):
    rng = np.random.default_rng(seed)
    q, k, v, g = (rng.normal(size=(B, H, N, D)) for _ in range(4))
    # a mask with a ragged last block, an empty row and varied kept sets (blocks of 16)
    nQ = nKV = -(-N // 16)
    rows = []
    for r in range(B * H * nQ):
        rows.append(sorted(rng.choice(nKV, size=1 + (r % nKV), replace=False)) if r % 5 != 3 else [])
    rp = np.concatenate([[0], np.cumsum([len(x) for x in rows])])
    ci = np.concatenate([np.array(x, dtype=np.int32) for x in rows])
    return q, k, v, g, rp, ci


def test_finite_differences():
    """dL/dx for L = sum(O * G) against central differences of the forward."""
    q, k, v, g, rp, ci = _case()
    dq, dk, dv = sparse_attention_backward(q, k, v, g, rp, ci, 16, 16)
    rng = np.random.default_rng(1)
    eps = 1e-6

    def loss(q_, k_, v_):
        return float((sparse_attention(q_, k_, v_, rp, ci, 16, 16) * g).sum())

    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(rng.integers(0, s) for s in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if n == name else y for n, y in (("q", q), ("k", k), ("v", v))]
            args_m = [xm if n == name else y for n, y in (("q", q), ("k", k), ("v", v))]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 + 1e-6 * abs(fd), (name, idx, fd, grad[idx])


def test_dense_matches_torch_autograd():
    rng = np.random.default_rng(2)
    B, H, N, D = 1, 2, 50, 16
    q, k, v, g = (rng.normal(size=(B, H, N, D)) for _ in range(4))
    rp, ci = dense_plan(B, H, N, 16, 16)
    dq, dk, dv = sparse_attention_backward(q, k, v, g, rp, ci, 16, 16)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    (o * torch.tensor(g)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_unkept_tokens_get_no_gradient_and_empty_rows_no_dq():
    """Rows keep {0}, {} and {0, 2}: block 1 is kept by no row, row 1 is empty."""
    rng = np.random.default_rng(3)
    q, k, v, g = (rng.normal(size=(1, 1, 40, 8)) for _ in range(4))
    rp = np.array([0, 1, 1, 3])
    ci = np.array([0, 0, 2], dtype=np.int32)
    dq, dk, dv = sparse_attention_backward(q, k, v, g, rp, ci, 16, 16)
    assert not dk[0, 0, 16:32].any() and not dv[0, 0, 16:32].any()
    assert dk[0, 0, 32:40].any() and dv[0, 0, 0:16].any()
    assert not dq[0, 0, 16:32].any()
    assert dq[0, 0, 0:16].any() and dq[0, 0, 32:40].any()


def test_given_output_changes_only_dv_term():
    """With o given as the exact output, the result is unchanged; with o perturbed, dV is
    unchanged (it does not use Dv) while dQ and dK move."""
    q, k, v, g, rp, ci = _case(seed=5)
    ref = sparse_attention_backward(q, k, v, g, rp, ci, 16, 16)
    o = sparse_attention(q, k, v, rp, ci, 16, 16)
    same = sparse_attention_backward(q, k, v, g, rp, ci, 16, 16, o=o)
    for a, b in zip(ref, same):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    moved = sparse_attention_backward(q, k, v, g, rp, ci, 16, 16, o=o * 1.01)
    np.testing.assert_array_equal(moved[2], ref[2])
    assert not np.allclose(moved[0], ref[0])
