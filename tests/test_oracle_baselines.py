"""Pins for the summary-free baseline modes of the oracle (CPU only).

The report measures KSA against sliding chunk attention (SCA, Fig. 3 right
without summaries) and token sliding windows (SWA); the oracle lays both
over the Eq. 1 sequence.  The pins: hand-written visible sets for a 12-row
case, per-row window counts, the reductions to causal attention and to
KSA, and a per-element softmax on a tiny input.
"""
import math

import numpy as np
import pytest

from oracle import ksa_oracle as O


def _sets(mask, n, k):
    is_s, idx = O.augmented_rows(n, k)
    name = lambda r: ("s" if is_s[r] else "t") + str(idx[r])
    return {name(a): sorted(name(b) for b in np.nonzero(mask[a])[0]) for a in range(mask.shape[0])}


def _key(lbl):
    return (lbl[0], int(lbl[1:]))


# n = 10, k = 4: rows t0 t1 t2 t3 s0 t4 t5 t6 t7 s1 t8 t9, written out by hand.
SWA_W3 = {
    "t0": "t0", "t1": "t0 t1", "t2": "t0 t1 t2", "t3": "t1 t2 t3", "s0": "t0 t1 t2 t3 s0",
    "t4": "t2 t3 t4", "t5": "t3 t4 t5", "t6": "t4 t5 t6", "t7": "t5 t6 t7", "s1": "t4 t5 t6 t7 s1",
    "t8": "t6 t7 t8", "t9": "t7 t8 t9",
}
SCA_C1 = {
    "t0": "t0", "t1": "t0 t1", "t2": "t0 t1 t2", "t3": "t0 t1 t2 t3", "s0": "t0 t1 t2 t3 s0",
    "t4": "t0 t1 t2 t3 t4", "t5": "t0 t1 t2 t3 t4 t5", "t6": "t0 t1 t2 t3 t4 t5 t6",
    "t7": "t0 t1 t2 t3 t4 t5 t6 t7", "s1": "t4 t5 t6 t7 s1",
    "t8": "t4 t5 t6 t7 t8", "t9": "t4 t5 t6 t7 t8 t9",
}


@pytest.mark.parametrize("mode,kw,expect", [(O.MODE_SWA, {"W": 3}, SWA_W3), (O.MODE_SCA, {"C": 1}, SCA_C1)])
def test_hand_written_sets(mode, kw, expect):
    got = _sets(O.baseline_mask(10, 4, mode, **kw), 10, 4)
    want = {q: sorted(v.split()) for q, v in expect.items()}
    assert {q: sorted(v, key=_key) for q, v in got.items()} == {q: sorted(v, key=_key) for q, v in want.items()}


@pytest.mark.parametrize("n,k,C,W", [(64, 8, 2, 5), (77, 5, 3, 1), (100, 4, 0, 17), (33, 1, 4, 33), (9, 3, 9, 2)])
def test_counts_closed_form(n, k, C, W):
    assert O.baseline_mask(n, k, O.MODE_SCA, C=C).sum() == O.baseline_pairs_closed_form(n, k, O.MODE_SCA, C=C)
    assert O.baseline_mask(n, k, O.MODE_SWA, W=W).sum() == O.baseline_pairs_closed_form(n, k, O.MODE_SWA, W=W)


@pytest.mark.parametrize("n,k", [(50, 4), (31, 7), (24, 1)])
def test_wide_windows_reduce_to_causal(n, k):
    is_s, idx = O.augmented_rows(n, k)
    txt = np.nonzero(~is_s)[0]
    causal = idx[txt][:, None] >= idx[txt][None, :]
    M = n // k
    sca = O.baseline_mask(n, k, O.MODE_SCA, C=M + 1)
    swa = O.baseline_mask(n, k, O.MODE_SWA, W=n)
    for m in (sca, swa):
        assert np.array_equal(m[np.ix_(txt, txt)], causal)
        assert not m[np.ix_(txt, np.nonzero(is_s)[0])].any()
    # with the window past every chunk KSA sees no summary either
    assert np.array_equal(sca, O.visibility_mask_fast(n, k, M + 1))


@pytest.mark.parametrize("n,k,C", [(96, 8, 3), (70, 5, 2), (40, 4, 0)])
def test_ksa_is_sca_plus_summary_strip(n, k, C):
    is_s, idx = O.augmented_rows(n, k)
    ksa = O.visibility_mask_fast(n, k, C)
    sca = O.baseline_mask(n, k, O.MODE_SCA, C=C)
    assert not (sca & ~ksa).any()
    extra = ksa & ~sca
    for a in np.nonzero(extra.any(axis=1))[0]:
        assert not is_s[a]
        c = idx[a] // k
        got = set(np.nonzero(extra[a])[0])
        assert got == {O.summary_row(j, k) for j in range(0, c - C)}


def test_swa_softmax_by_hand():
    rng = np.random.default_rng(7)
    n, k, W = 6, 3, 2
    L = O.augmented_len(n, k)
    q = rng.standard_normal((L, 1, 4))
    kx = rng.standard_normal((L, 1, 4))
    v = rng.standard_normal((L, 1, 3))
    out, lse = O.baseline_attention(q, kx, v, n, k, O.MODE_SWA, 0.5, W=W)
    is_s, idx = O.augmented_rows(n, k)
    for a in range(L):
        if is_s[a]:
            keys = [b for b in range(L) if (not is_s[b] and idx[b] // k == idx[a]) or b == a]
        else:
            keys = [b for b in range(L) if not is_s[b] and idx[a] - W < idx[b] <= idx[a]]
        sc = [0.5 * sum(q[a, 0, d] * kx[b, 0, d] for d in range(4)) for b in keys]
        mx = max(sc)
        e = [math.exp(x - mx) for x in sc]
        z = sum(e)
        for d in range(3):
            assert out[a, 0, d] == pytest.approx(sum(e[i] * v[b, 0, d] for i, b in enumerate(keys)) / z, rel=1e-12)
        assert lse[0, a] == pytest.approx(mx + math.log(z), rel=1e-12)


def test_bad_modes():
    with pytest.raises(ValueError):
        O.baseline_mask(8, 4, O.MODE_SWA, W=0)
    with pytest.raises(ValueError):
        O.baseline_mask(8, 4, 7)
