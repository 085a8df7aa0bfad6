"""Pins for the oracle's attention backward (CPU only).

The gradient is pinned to things other than its own formula: central finite
differences of the (separately pinned) forward oracle, the two conservation
laws of softmax attention (every row of dS sums to zero, so the key
gradients of a head sum to zero and the value gradients sum to the output
gradients), exact zeros where a row sees a single key or identical keys, and
PyTorch's autograd of causal scaled-dot-product attention in float64, which
the text rows reduce to when every summary has left the window of no row.
"""
import numpy as np
import pytest
import torch

from oracle import ksa_oracle as O


def _inputs(n, k, hq, hkv, d, seed):
    r = np.random.default_rng(seed)
    L = O.augmented_len(n, k)
    return (r.standard_normal((L, hq, d)), r.standard_normal((L, hkv, d)),
            r.standard_normal((L, hkv, d)), r.standard_normal((L, hq, d)))


def _loss(q, kx, v, g, n, k, scale, mode, C, W):
    o, _ = O.baseline_attention(q, kx, v, n, k, mode, scale, C=C, W=W)
    return float((o * g).sum())


@pytest.mark.parametrize("mode,C,W", [(O.MODE_KSA, 1, 0), (O.MODE_KSA, 0, 0), (O.MODE_SCA, 1, 0),
                                      (O.MODE_SWA, 0, 3)])
def test_finite_differences(mode, C, W):
    n, k, scale = 10, 3, 0.7
    q, kx, v, g = _inputs(n, k, 4, 2, 3, seed=11 + mode)
    dq, dk, dv = O.attention_backward(q, kx, v, g, n, k, scale, mode=mode, C=C, W=W)
    eps = 1e-6
    for x, dx in ((q, dq), (kx, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            fp = _loss(q, kx, v, g, n, k, scale, mode, C, W)
            x[idx] = old - eps
            fm = _loss(q, kx, v, g, n, k, scale, mode, C, W)
            x[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(dx, num, atol=2e-7, rtol=1e-6)


@pytest.mark.parametrize("n,k,C,hq,hkv", [(37, 4, 2, 4, 2), (64, 8, 1, 2, 2), (25, 5, 0, 3, 1)])
def test_conservation(n, k, C, hq, hkv):
    q, kx, v, g = _inputs(n, k, hq, hkv, 6, seed=n)
    dq, dk, dv = O.attention_backward(q, kx, v, g, n, k, 0.4, C=C)
    grp = hq // hkv
    for h in range(hkv):
        np.testing.assert_allclose(dk[:, h].sum(0), 0.0, atol=1e-12)
        np.testing.assert_allclose(dv[:, h].sum(0), g[:, h * grp:(h + 1) * grp].sum((0, 1)), atol=1e-11)


def test_single_key_and_identical_keys():
    n, k = 20, 4
    q, kx, v, g = _inputs(n, k, 2, 1, 5, seed=3)
    dq, dk, dv = O.attention_backward(q, kx, v, g, n, k, 0.5, C=1)
    # t_0 sees only itself: its softmax is the constant 1
    assert np.all(dq[O.text_row(0, k)] == 0.0)
    kx[:] = kx[0]
    dq, _, _ = O.attention_backward(q, kx, v, g, n, k, 0.5, C=1)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)


@pytest.mark.parametrize("n,k,hq,hkv", [(40, 4, 4, 2), (33, 8, 2, 1)])
def test_reduces_to_causal_autograd(n, k, hq, hkv):
    """With C >= M - 1 no text row reads a summary; with zero output gradient
    on the summary rows, the text rows' gradients are those of causal
    attention over the text alone and summaries get none."""
    M = n // k
    q, kx, v, g = _inputs(n, k, hq, hkv, 8, seed=5)
    is_s, idx = O.augmented_rows(n, k)
    g[is_s] = 0.0
    scale = 0.3
    dq, dk, dv = O.attention_backward(q, kx, v, g, n, k, scale, C=M)
    txt = np.nonzero(~is_s)[0]
    grp = hq // hkv
    tq = torch.tensor(q[txt].transpose(1, 0, 2), requires_grad=True)
    tk = torch.tensor(kx[txt].transpose(1, 0, 2), requires_grad=True)
    tv = torch.tensor(v[txt].transpose(1, 0, 2), requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(grp, 0), tv.repeat_interleave(grp, 0), is_causal=True, scale=scale)
    (o * torch.tensor(g[txt].transpose(1, 0, 2))).sum().backward()
    np.testing.assert_allclose(dq[txt], tq.grad.numpy().transpose(1, 0, 2), atol=1e-12)
    np.testing.assert_allclose(dk[txt], tk.grad.numpy().transpose(1, 0, 2), atol=1e-12)
    np.testing.assert_allclose(dv[txt], tv.grad.numpy().transpose(1, 0, 2), atol=1e-12)
    assert np.all(dk[is_s] == 0.0) and np.all(dv[is_s] == 0.0)


def test_rows_split_sums_to_full_backward():
    """The per-row terms over a partition of the rows add up to the full
    backward (each key's gradient is a sum over the queries that see it)."""
    n, k, C = 30, 4, 1
    q, kx, v, g = _inputs(n, k, 4, 2, 5, seed=21)
    dq, dk, dv = O.attention_backward(q, kx, v, g, n, k, 0.6, C=C)
    L = O.augmented_len(n, k)
    parts = [np.arange(0, 11), np.arange(11, 20), np.arange(20, L)]
    sk, sv = np.zeros_like(dk), np.zeros_like(dv)
    for rows in parts:
        a, b, c = O.attention_backward_rows(q, kx, v, g, n, k, 0.6, rows, C=C)
        np.testing.assert_allclose(a, dq[rows], atol=1e-13)
        sk += b
        sv += c
    np.testing.assert_allclose(sk, dk, atol=1e-12)
    np.testing.assert_allclose(sv, dv, atol=1e-12)
    a, _, _ = O.attention_backward_rows(q, kx, v, g, n, k, 0.6, [3, 7], C=C, heads=[1, 2])
    np.testing.assert_allclose(a, dq[[3, 7]][:, [1, 2]], atol=1e-13)
