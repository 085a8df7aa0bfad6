"""Pins for the oracle's cache model (CPU only).

The cache model steps through the Fig. 4 lifecycle; these tests check it
against the attention rule itself (what each decode slice must contain is a
mask row of Eq. (3)), the held-token count n/k + w*k + current chunk stated
for the layout, contiguity of every read, and Table 1's printed ratios.
"""
import pytest

from oracle import ksa_oracle as O


def _run(k, C, n_total, cap):
    """Feed n_total text tokens (with summaries) through the model; yield states."""
    cm = O.CacheModel(k, C, cap)
    for i in range(n_total):
        cm.append_text(O.text_row(i, k))
        yield "t", i + 1, cm
        if (i + 1) % k == 0:
            cm.append_summary(O.summary_row((i + 1) // k - 1, k))
            yield "s", i + 1, cm


@pytest.mark.parametrize("k,C", [(4, 2), (4, 0), (8, 1), (3, 5), (1, 3), (2, 1)])
def test_slices_equal_mask_rows_every_step(k, C):
    for kind, n_text, cm in _run(k, C, 80, 80):
        if kind == "t":
            s, ln = cm.text_slice()
        else:
            s, ln = cm.summary_slice()
        got = sorted(cm.slots[s:s + ln])
        want = list(O.decode_visible_rows(n_text, k, C, kind))
        assert got == want, (kind, n_text)
        assert None not in cm.slots[s:s + ln]


@pytest.mark.parametrize("k,C", [(4, 2), (4, 0), (8, 3), (1, 2)])
def test_held_set_and_count(k, C):
    for kind, n_text, cm in _run(k, C, 70, 70):
        # after a text append the chunk may be full with its summary still
        # to come; after a summary append the chunk is committed
        m = n_text // k if kind == "s" else (n_text - 1) // k
        r = n_text - m * k
        assert (m, r) == (cm.m, cm.r)
        held = sorted(cm.held())
        assert held == O.cache_held_rows(m, r, k, C)
        assert len(held) == m + min(m, C) * k + r
        if m >= C:
            assert len(held) == m + C * k + r   # n/k + w*k + current chunk


def test_misuse_raises():
    cm = O.CacheModel(4, 1, 2)
    with pytest.raises(RuntimeError):
        cm.append_summary("s")
    for t in range(4):
        cm.append_text(t)
    with pytest.raises(RuntimeError):
        cm.append_text(9)


def test_table1_ratios():
    k, h, d, g, dc, dr = 8, 128, 128, 8, 512, 64
    r = {m: O.per_token_cache_ratio(m, k, h, d, g, dc, dr)
         for m in ["gqa", "mla", "ksa", "ksa+gqa", "ksa+mla"]}
    # values printed in Table 1 (rounded there to 3 significant digits)
    assert round(100 * r["gqa"], 2) == 6.25
    assert round(100 * r["mla"], 2) == 1.76
    assert round(100 * r["ksa"], 1) == 12.5
    assert round(100 * r["ksa+gqa"], 2) == 0.78
    assert round(100 * r["ksa+mla"], 2) == 0.22


def test_cache_slots_per_token_tend_to_table1():
    # slots of a cache sized for n tokens, per token, over MHA's per-token cost
    k, C, h, d, g, dc, dr = 8, 64, 128, 128, 8, 512, 64
    n = 1 << 26
    slots = O.CacheModel.num_slots(k, C, n // k)
    gqa = slots * 2 * g * d / n / (2 * h * d)
    mla = slots * (dc + dr) / n / (2 * h * d)
    assert abs(gqa - 1 / k * g / h) < 1e-5
    assert abs(mla - 1 / k * (dc + dr) / (2 * h * d)) < 1e-5


@pytest.mark.parametrize("k,C", [(4, 2), (8, 3), (3, 1), (1, 2), (4, 0)])
def test_slot_of_row_matches_model(k, C):
    for kind, n_text, cm in _run(k, C, 60, 60):
        for slot_payload in cm.held():
            a = slot_payload
            s = O.slot_of_row(a, cm.m, cm.r, k, C)
            assert cm.slots[s] == a
