"""Pins for the oracle's index map and visibility rule (CPU only).

Each test checks the oracle against something other than itself: a literal
written out by hand from Eq. (3) for the Fig. 3 configuration, closed-form
counts, the coverage guarantee stated with Fig. 3/Fig. 4, a second encoding
of the same sets, and a negative control built from the rejected token-level
window of Fig. 3 (left).
"""
import os

import numpy as np
import pytest

from oracle import ksa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fig3_sca_k4_c1_n16.txt")
GOLDEN_SWA = os.path.join(os.path.dirname(__file__), "golden", "fig3_token_swa_k4_w4_n16.txt")


def _label_to_row(lbl, k):
    kind, idx = lbl[0], int(lbl[1:])
    return O.text_row(idx, k) if kind == "t" else O.summary_row(idx, k)


def _read_golden(path=GOLDEN):
    rows = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            q, keys = line.split(":")
            rows[q.strip()] = keys.split()
    return rows


def test_fig3_literal_matches_both_encodings():
    k, C, n = 4, 1, 16
    gold = _read_golden()
    assert len(gold) == 20
    L = O.augmented_len(n, k)
    want = np.zeros((L, L), dtype=bool)
    for q, keys in gold.items():
        a = _label_to_row(q, k)
        for key in keys:
            want[a, _label_to_row(key, k)] = True
    assert want.sum() == 120
    np.testing.assert_array_equal(O.visibility_mask(n, k, C), want)
    np.testing.assert_array_equal(O.visibility_mask_fast(n, k, C), want)
    for a in range(L):
        assert O.visible_set_eq3(n, k, C, a) == set(np.nonzero(want[a])[0])


def _golden_mask(path, n, k):
    gold = _read_golden(path)
    L = O.augmented_len(n, k)
    assert len(gold) == L
    want = np.zeros((L, L), dtype=bool)
    for q, keys in gold.items():
        a = _label_to_row(q, k)
        for key in keys:
            want[a, _label_to_row(key, k)] = True
    return want


def test_token_window_literal():
    """The negative control itself is pinned: a hand-written literal of the
    token-level window of Fig. 3 (left) with W = 4 over four chunks of 4."""
    want = _golden_mask(GOLDEN_SWA, 16, 4)
    assert want.sum() == 93
    np.testing.assert_array_equal(O.token_swa_mask(16, 4, W=4), want)


def test_index_map_eq1():
    for n, k in [(16, 4), (37, 8), (7, 8), (64, 1), (100, 3)]:
        is_s, idx = O.augmented_rows(n, k)
        L = O.augmented_len(n, k)
        assert len(is_s) == L == n + n // k
        for a in range(L):
            kind, q = O.decode_row(a, n, k)
            assert (kind == "s") == bool(is_s[a]) and q == idx[a]
            assert (O.summary_row(q, k) if kind == "s" else O.text_row(q, k)) == a
        # text rows in order, each summary right after its chunk's last text
        assert list(idx[~is_s]) == list(range(n))
        for j in range(n // k):
            assert O.summary_row(j, k) == O.text_row(j * k + k - 1, k) + 1


def test_position_rule():
    n, k = 37, 8
    pos = O.position_ids(n, k)
    is_s, idx = O.augmented_rows(n, k)
    # text positions are the text indices: no jump where a summary sits
    assert list(pos[~is_s]) == list(range(n))
    # summary j takes the id of its chunk's last text token
    for j in range(n // k):
        assert pos[O.summary_row(j, k)] == pos[O.text_row(j * k + k - 1, k)]


@pytest.mark.parametrize("n,k,C", [(16, 4, 1), (37, 8, 2), (64, 8, 0), (45, 4, 3),
                                   (30, 1, 5), (12, 5, 10), (96, 8, 4)])
def test_predicate_equals_set_enumeration_and_loop(n, k, C):
    fast = O.visibility_mask_fast(n, k, C)
    loop = O.visibility_mask(n, k, C)
    np.testing.assert_array_equal(fast, loop)
    for a in range(O.augmented_len(n, k)):
        assert O.visible_set_eq3(n, k, C, a) == set(np.nonzero(fast[a])[0])


@pytest.mark.parametrize("n,k,C", [(37, 8, 2), (64, 8, 0), (45, 4, 3), (30, 1, 5), (96, 8, 4)])
def test_per_row_counts(n, k, C):
    m = O.visibility_mask_fast(n, k, C)
    is_s, idx = O.augmented_rows(n, k)
    for a in range(len(is_s)):
        if is_s[a]:
            assert m[a].sum() == k + 1
        else:
            c, p = divmod(int(idx[a]), k)
            assert m[a].sum() == min(c, C) * k + p + 1 + max(0, c - C)


@pytest.mark.parametrize("n,k,C,want", [(16, 4, 1, 120), (512, 8, 4, 32784),
                                        (64, 8, 0, 584), (64, 8, 100, 2152)])
def test_total_pairs_brute_force_and_closed_form(n, k, C, want):
    assert O.visible_pairs_bruteforce(n, k, C) == want
    assert O.visible_pairs_closed_form(n // k, k, C) == want
    assert O.visible_pairs_general(n, k, C) == want


def test_closed_form_general_n():
    for n, k, C in [(37, 8, 2), (45, 4, 3), (101, 8, 3), (9, 8, 0)]:
        assert O.visible_pairs_general(n, k, C) == O.visible_pairs_bruteforce(n, k, C)


def test_large_config_pair_counts():
    # per-head visible pairs of the benchmark workloads (closed form, checked
    # against brute force above on small sizes)
    assert O.visible_pairs_closed_form(32768 // 8, 8, 64) == 81840384
    assert O.visible_pairs_closed_form(131072 // 8, 8, 64) == 1133017344
    assert O.visible_pairs_closed_form(131072 // 8, 8, 16) == 1089086016


def _coverage_ok(mask, n, k):
    """Every text row covers each earlier complete chunk by text XOR summary."""
    for i in range(n):
        a = O.text_row(i, k)
        c = i // k
        for cc in range(c):
            if (cc + 1) * k > n:
                continue
            text = [mask[a, O.text_row(t, k)] for t in range(cc * k, cc * k + k)]
            summ = mask[a, O.summary_row(cc, k)] if cc < n // k else False
            full = all(text)
            none = not any(text)
            if not ((full and not summ) or (none and summ)):
                return False
        # own chunk: causal text only, never its (not yet existing) summary
        for t in range(c * k, min(n, c * k + k)):
            if mask[a, O.text_row(t, k)] != (t <= i):
                return False
    return True


@pytest.mark.parametrize("n,k,C", [(64, 8, 2), (37, 8, 2), (45, 4, 3), (40, 4, 0), (60, 5, 20)])
def test_coverage_text_xor_summary(n, k, C):
    assert _coverage_ok(O.visibility_mask_fast(n, k, C), n, k)


def test_token_window_cutting_a_chunk_breaks_coverage():
    # Fig. 3 left: a token-level window that cuts a chunk loses that chunk
    n, k = 16, 4
    assert not _coverage_ok(O.token_swa_mask(n, k, W=4), n, k)
    # a chunk-aligned window of the same width (C = 1) keeps it
    assert _coverage_ok(O.visibility_mask_fast(n, k, 1), n, k)


@pytest.mark.parametrize("n,k,C", [(64, 8, 2), (45, 4, 3)])
def test_summary_locality(n, k, C):
    m = O.visibility_mask_fast(n, k, C)
    for j in range(n // k):
        a = O.summary_row(j, k)
        allowed = {O.text_row(i, k) for i in range(j * k, j * k + k)} | {a}
        assert set(np.nonzero(m[a])[0]) == allowed
    # reading A (summary does not see itself) removes exactly the diagonal
    mA = O.visibility_mask_fast(n, k, C, summary_sees_self=False)
    for j in range(n // k):
        a = O.summary_row(j, k)
        assert not mA[a, a] and mA[a].sum() == k


def test_full_window_is_causal_over_text():
    n, k = 40, 4
    M = n // k
    m = O.visibility_mask_fast(n, k, M - 1)
    is_s, idx = O.augmented_rows(n, k)
    t = ~is_s
    sub = m[np.ix_(t, t)]
    np.testing.assert_array_equal(sub, np.tril(np.ones((n, n), dtype=bool)))
    assert not m[np.ix_(t, is_s)].any()
