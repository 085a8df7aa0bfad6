"""Pins for the oracle's attention, RoPE and decode arithmetic (CPU only).

References used here are independent of the oracle's own code paths: plain
Python loops with ``math.exp`` on tiny inputs, torch's causal
scaled-dot-product attention (the full-window reduction to Eq. (9)), closed
forms (constant V, the first text row, uniform weights at zero scale), the
log-sum-exp merge identity and hand-worked RoPE values.
"""
import math

import numpy as np
import pytest
import torch

from oracle import ksa_oracle as O


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _loop_attention(q, kx, v, n, k, C, scale, g):
    """Per-element Python softmax over the visible set, from Eq. (3)."""
    L, Hq, _ = q.shape
    Dv = v.shape[-1]
    out = np.zeros((L, Hq, Dv))
    for a in range(L):
        vis = sorted(O.visible_set_eq3(n, k, C, a))
        for h in range(Hq):
            kv = h // g
            sc = [scale * sum(q[a, h, d] * kx[b, kv, d] for d in range(q.shape[2])) for b in vis]
            mx = max(sc)
            w = [math.exp(s - mx) for s in sc]
            den = sum(w)
            for d in range(Dv):
                out[a, h, d] = sum(w[t] * v[vis[t], kv, d] for t in range(len(vis))) / den
    return out


def test_brute_force_tiny():
    rng = np.random.default_rng(7)
    n, k, C, Hq, Hkv, D = 13, 3, 1, 4, 2, 5
    L = O.augmented_len(n, k)
    q, kx, v = _rand(rng, L, Hq, D), _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    scale = 0.37
    got, _ = O.ksa_attention(q, kx, v, n, k, C, scale, row_block=4)
    want = _loop_attention(q, kx, v, n, k, C, scale, Hq // Hkv)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_full_window_reduces_to_causal_sdpa():
    rng = np.random.default_rng(1)
    n, k, Hq, Hkv, D = 48, 4, 4, 2, 8
    M = n // k
    L = O.augmented_len(n, k)
    q, kx, v = _rand(rng, L, Hq, D), _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    scale = 1 / math.sqrt(D)
    got, _ = O.ksa_attention(q, kx, v, n, k, M - 1, scale)
    is_s, _ = O.augmented_rows(n, k)
    t = ~is_s
    g = Hq // Hkv
    qt = torch.from_numpy(q[t]).permute(1, 0, 2)                   # [Hq, n, D]
    kt = torch.from_numpy(kx[t]).permute(1, 0, 2).repeat_interleave(g, 0)
    vt = torch.from_numpy(v[t]).permute(1, 0, 2).repeat_interleave(g, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    np.testing.assert_allclose(got[t], ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


def test_first_row_and_constant_v_and_zero_scale():
    rng = np.random.default_rng(2)
    n, k, C, Hq, Hkv, D = 40, 4, 2, 2, 1, 6
    L = O.augmented_len(n, k)
    q, kx, v = _rand(rng, L, Hq, D), _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    out, lse = O.ksa_attention(q, kx, v, n, k, C, 0.5)
    # t_0 sees only itself: p = 1
    np.testing.assert_array_equal(out[0, 0], v[0, 0])
    # LSE of t_0 is its single score
    assert abs(lse[0, 0] - 0.5 * q[0, 0] @ kx[0, 0]) < 1e-12
    # all V rows equal u => every output equals u
    u = rng.standard_normal(D)
    vc = np.broadcast_to(u, v.shape).copy()
    oc, _ = O.ksa_attention(q, kx, vc, n, k, C, 0.5)
    np.testing.assert_allclose(oc, np.broadcast_to(u, oc.shape), rtol=0, atol=1e-13)
    # scale 0: uniform weights, output = mean of visible V rows
    oz, lz = O.ksa_attention(q, kx, v, n, k, C, 0.0)
    for a in [0, 5, 17, L - 1]:
        vis = sorted(O.visible_set_eq3(n, k, C, a))
        np.testing.assert_allclose(oz[a, 1], v[vis, 0].mean(axis=0), rtol=1e-12, atol=1e-14)
        assert abs(lz[1, a] - math.log(len(vis))) < 1e-12


def test_summary_row_hand_softmax():
    rng = np.random.default_rng(3)
    n, k, C, D = 32, 8, 1, 4
    L = O.augmented_len(n, k)
    q, kx, v = _rand(rng, L, 1, D), _rand(rng, L, 1, D), _rand(rng, L, 1, D)
    out, _ = O.ksa_attention(q, kx, v, n, k, C, 0.25)
    j = 2
    a = O.summary_row(j, k)
    keys = [O.text_row(i, k) for i in range(j * k, j * k + k)] + [a]
    w = [math.exp(0.25 * float(np.dot(q[a, 0], kx[b, 0]))) for b in keys]
    want = sum(w[t] * v[keys[t], 0] for t in range(k + 1)) / sum(w)
    np.testing.assert_allclose(out[a, 0], want, rtol=1e-12)


def test_gqa_head_mapping_is_grouped():
    rng = np.random.default_rng(4)
    n, k, C, Hq, Hkv, D = 24, 4, 1, 4, 2, 4
    L = O.augmented_len(n, k)
    q1 = _rand(rng, L, 1, D)
    q = np.repeat(q1, Hq, axis=1)
    kx, v = _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    out, _ = O.ksa_attention(q, kx, v, n, k, C, 0.5)
    np.testing.assert_array_equal(out[:, 0], out[:, 1])   # heads 0,1 -> kv 0
    np.testing.assert_array_equal(out[:, 2], out[:, 3])   # heads 2,3 -> kv 1
    assert np.abs(out[:, 0] - out[:, 2]).max() > 1e-3


def test_absorbed_v_is_k_prefix():
    rng = np.random.default_rng(5)
    n, k, C, Hq, D, Dv = 20, 4, 1, 3, 9, 6
    L = O.augmented_len(n, k)
    q, kx = _rand(rng, L, Hq, D), _rand(rng, L, 1, D)
    a, la = O.ksa_attention(q, kx, None, n, k, C, 0.3, dv=Dv)
    b, lb = O.ksa_attention(q, kx, kx[..., :Dv].copy(), n, k, C, 0.3)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


def test_lse_merge_identity():
    # attention over (distant summaries) and over (window text), merged by
    # their log-sum-exps, equals attention over the union
    rng = np.random.default_rng(6)
    n, k, C, D = 64, 4, 2, 5
    L = O.augmented_len(n, k)
    q, kx, v = _rand(rng, L, 1, D), _rand(rng, L, 1, D), _rand(rng, L, 1, D)
    out, lse = O.ksa_attention(q, kx, v, n, k, C, 0.4)
    is_s, _ = O.augmented_rows(n, k)
    a = O.text_row(57, k)
    m = O.visibility_mask_fast(n, k, C, rows=[a])
    ms, mt = m & is_s[None, :], m & ~is_s[None, :]
    o1, l1 = O.attention_masked(q[[a], 0], kx[:, 0], v[:, 0], ms, 0.4)
    o2, l2 = O.attention_masked(q[[a], 0], kx[:, 0], v[:, 0], mt, 0.4)
    mx = max(l1[0], l2[0])
    w1, w2 = math.exp(l1[0] - mx), math.exp(l2[0] - mx)
    merged = (w1 * o1[0] + w2 * o2[0]) / (w1 + w2)
    np.testing.assert_allclose(merged, out[a, 0], rtol=1e-12)
    assert abs(mx + math.log(w1 + w2) - lse[0, a]) < 1e-12


# ---------------------------------------------------------------- RoPE ----


def test_rope_hand_values():
    # D = 4, theta = 1e6: pair (0,2) turns at 1 rad/position, pair (1,3) at
    # 1e6**(-1/2) = 1e-3 rad/position
    x = np.zeros((2, 1, 4))
    x[:, 0] = [1.0, 2.0, 3.0, 4.0]
    y = O.rope_rotate(x, np.array([0, 5]), 1e6)
    np.testing.assert_array_equal(y[0], x[0])
    c1, s1 = math.cos(5.0), math.sin(5.0)
    c2, s2 = math.cos(5e-3), math.sin(5e-3)
    want = [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 3 * c1 + 1 * s1, 4 * c2 + 2 * s2]
    np.testing.assert_allclose(y[1, 0], want, rtol=1e-13, atol=1e-15)


def test_rope_relative_and_norm():
    rng = np.random.default_rng(8)
    D = 16
    qv, kv = rng.standard_normal(D), rng.standard_normal(D)
    x = np.stack([qv, kv])[:, None, :]
    def dot(m, nn):
        a = O.rope_rotate(x[:1], np.array([m]), 1e4)[0, 0]
        b = O.rope_rotate(x[1:], np.array([nn]), 1e4)[0, 0]
        return a @ b
    assert abs(dot(7, 3) - dot(107, 103)) < 1e-11
    assert abs(dot(130000, 5) - dot(129995, 0)) < 1e-9
    y = O.rope_rotate(x, np.array([123456, 99]), 1e6)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_rope_partial_block():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((3, 2, 10))
    y = O.rope_rotate(x, np.array([1, 2, 3]), 1e4, rot_off=6, rot_dim=4)
    np.testing.assert_array_equal(y[..., :6], x[..., :6])
    z = O.rope_rotate(x[..., 6:], np.array([1, 2, 3]), 1e4)
    np.testing.assert_array_equal(y[..., 6:], z)


# -------------------------------------------------------------- decode ----


@pytest.mark.parametrize("k,C,n_text", [(4, 2, 23), (4, 2, 24), (8, 1, 9), (4, 0, 30), (3, 5, 17)])
def test_decode_text_equals_prefill_row(k, C, n_text):
    rng = np.random.default_rng(10)
    Hq, Hkv, D = 4, 2, 6
    L = O.augmented_len(n_text, k)
    q, kx, v = _rand(rng, L, Hq, D), _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    full, flse = O.ksa_attention(q, kx, v, n_text, k, C, 0.3)
    a = O.text_row(n_text - 1, k)
    o, l_ = O.decode_attention(q[a], kx, v, n_text, k, C, 0.3, "t")
    np.testing.assert_allclose(o, full[a], rtol=1e-12)
    np.testing.assert_allclose(l_, flse[:, a], rtol=1e-12)


@pytest.mark.parametrize("k,C,n_text", [(4, 2, 24), (8, 1, 16), (4, 0, 8)])
def test_decode_summary_equals_prefill_row(k, C, n_text):
    rng = np.random.default_rng(11)
    Hq, Hkv, D = 2, 1, 5
    L = O.augmented_len(n_text, k)
    q, kx, v = _rand(rng, L, Hq, D), _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    full, _ = O.ksa_attention(q, kx, v, n_text, k, C, 0.3)
    a = O.summary_row(n_text // k - 1, k)
    o, _ = O.decode_attention(q[a], kx, v, n_text, k, C, 0.3, "s")
    np.testing.assert_allclose(o, full[a], rtol=1e-12)
