"""Bit-exact row coverage of the split-K decode reads (GQA and absorbed MLA).

Every decode read is one contiguous cache slice ("Kwai Summary Attention
Technical Report", Sec. 2.3.1 and Fig. 4); the split-K kernels cut that
slice into pieces (GQA: up to 64 splits per (sequence, kv head); MLA: row
ranges of about total/CUs rows across the whole batch) and merge the partial
softmax results.  An absolute tolerance cannot see one dropped or doubled
row among thousands, so these tests count rows exactly:

* q = 0, so every visible score is 0 and every visible row has weight 1:
  out[d] = (sum of V[row, d] over the slice) / len and LSE = ln(len);
* V of augmented row a is one-hot (or two-hot) on a code of a, so
  out[d] * len = the number of visible rows whose code is d.

Exactness: the weights are exactly 1 and the sums exact integers in fp32;
the output is count / len rounded to bf16 (8 significand bits, relative
error <= 2^-8), so round(out * len) == count whenever count < 128, which
the codes and sizes below keep (asserted per step).
len itself is recovered from the fp32 LSE.  Recovered counts and lengths
must equal, bit for bit, the histograms of the oracle's decode mask row
(the rows of the logical history the query reads, Eq. 3) on ragged
batches long enough for many splits.
"""
import math

import numpy as np
import pytest
import torch

from oracle import ksa_oracle as O

pytestmark = pytest.mark.gpu

ksa = pytest.importorskip("kv_cache_compression_amd")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _np(t):
    return t.detach().float().cpu().double().numpy()


def _recover(out_row, lse_val):
    """(len, counts) from one head's output row and normaliser."""
    n = int(round(math.exp(float(lse_val))))
    return n, np.rint(out_row * n).astype(np.int64)


# --------------------------------------------------------------- GQA d128 --

GQA_D = 128


def _gqa_codes(rows, kvh):
    """Codes per kv head: head 0 is two-hot, (a mod 64) and 64 + (a / 64 mod 64);
    head 1 is one-hot on a mod 128."""
    if kvh == 0:
        return [rows % 64, 64 + (rows // 64) % 64]
    return [rows % GQA_D]


def _gqa_values(L, hkv):
    a = np.arange(L)
    v = np.zeros((L, hkv, GQA_D), dtype=np.float32)
    for h in range(hkv):
        for code in _gqa_codes(a, h):
            v[a, h, code] = 1.0
    return torch.from_numpy(v).to(torch.bfloat16)


def _expected(rows, codes, width):
    cnt = np.zeros(width, dtype=np.int64)
    for c in codes:
        cnt += np.bincount(c, minlength=width)
    return cnt


def _gqa_splits(batch, hkv, k, C, max_s):
    """Splits per slice under the launch's documented policy: about 2048
    workgroups in all, at least 256 capacity rows per split, at most 64."""
    cap = k + C * k + max_s + 1
    ns = (2048 + batch * hkv - 1) // (batch * hkv)
    return max(1, min(ns, (cap + 255) // 256, 64))


@pytest.mark.parametrize("max_s", [4096, 16000])
def test_gqa_decode_rows_exact_multi_split(max_s):
    dev = _dev()
    k, C, hq, hkv = 8, 4, 8, 2
    ns_text = [29003, 26005, 31007]           # ragged histories (text tokens incl. the query)
    B = len(ns_text)
    nsplit = _gqa_splits(B, hkv, k, C, max_s)
    assert nsplit >= 8
    L_max = O.augmented_len(max(ns_text) + k + 1, k)
    g = torch.Generator().manual_seed(7)
    kx = torch.randn((L_max, hkv, GQA_D), generator=g).to(torch.bfloat16)
    vx = _gqa_values(L_max, hkv)
    p = ksa.Params(k, C, hq, hkv, GQA_D, GQA_D, torch.bfloat16)
    cache = ksa.Cache(p, B, max_s, device=dev)
    # ragged fill through the row-wise append: each sequence gets its own prefix
    Ls = [O.augmented_len(n - 1, k) for n in ns_text]   # history before the query token
    seg = torch.tensor(np.concatenate([[0], np.cumsum(Ls)]), dtype=torch.int64, device=dev)
    ksa.ksa_cache_append_rows(cache, seg, max(Ls), torch.cat([kx[:l] for l in Ls]).contiguous().to(dev),
                              torch.cat([vx[:l] for l in Ls]).contiguous().to(dev))
    q = torch.zeros((B, hq, GQA_D), dtype=torch.bfloat16, device=dev)
    ws = ksa.decode_workspace(cache)
    n_now = [n - 1 for n in ns_text]
    a_next = list(Ls)                                    # next augmented row of each sequence
    # k + 2 decode steps per sequence: text appends through the end of a chunk,
    # its summary, and text again; every step is checked
    for step in range(k + 2):
        kinds = [1 if (a % (k + 1)) == k else 0 for a in a_next]
        kt = torch.tensor(kinds, dtype=torch.int32, device=dev)
        ksa.ksa_cache_append(cache, kx[a_next].contiguous().to(dev), vx[a_next].contiguous().to(dev), kt)
        for b in range(B):
            a_next[b] += 1
            if not kinds[b]:
                n_now[b] += 1
        lse = torch.empty((B, hq), dtype=torch.float32, device=dev)
        print(f"GQA split coverage: step {step} kinds {kinds} splits {nsplit}", flush=True)
        out = ksa.ksa_decode_attn(cache, q, kt, lse=lse, workspace=ws)
        torch.cuda.synchronize()
        o, ls = _np(out), _np(lse)
        for b in range(B):
            rows = O.decode_visible_rows(n_now[b], k, C, "s" if kinds[b] else "t")
            for h in range(hq):
                kvh = h // (hq // hkv)
                n_rows, cnt = _recover(o[b, h], ls[b, h])
                assert n_rows == len(rows), (step, b, h, n_rows, len(rows))
                want = _expected(rows, _gqa_codes(rows, kvh), GQA_D)
                assert want.max() < 128
                np.testing.assert_array_equal(cnt, want, err_msg=f"step {step} seq {b} head {h}")
    assert ksa.ksa_cache_read_errors(cache) == [0] * B


# ------------------------------------------------------ absorbed MLA ------

MLA_HQ, MLA_DQK, MLA_DV = 128, 576, 512


def _mla_codes(rows):
    """Two-hot latent code: (a mod 256) and 256 + (a / 128 mod 256)."""
    return [rows % 256, 256 + (rows // 128) % 256]


@pytest.mark.parametrize("ns_text,C,min_ranges", [
    ([45003, 38005, 52007], 4, 4), ([3003, 2505], 2, 4), ([700, 1900, 130, 2600], 64, 4),
    # more sequences than a wave has lanes: the cut is formed 64 sequences at a time
    ([int(x) for x in np.random.default_rng(11).integers(40, 6000, 100)], 8, 2),
])
def test_mla_decode_rows_exact_multi_range(ns_text, C, min_ranges):
    """Ranges cut across a ragged batch: long slices (rows per range above
    64), short ones (64-row ranges), a wide window and a batch of 100."""
    dev = _dev()
    k = 8
    B = len(ns_text)
    L_max = O.augmented_len(max(ns_text) + k + 1, k)
    a = np.arange(L_max)
    kx = np.zeros((L_max, 1, MLA_DQK), dtype=np.float32)
    for c in _mla_codes(a):
        kx[a, 0, c] = 1.0
    kx[:, 0, MLA_DV:] = np.random.default_rng(3).standard_normal((L_max, MLA_DQK - MLA_DV))
    kx = torch.from_numpy(kx).to(torch.bfloat16)
    p = ksa.Params(k, C, MLA_HQ, 1, MLA_DQK, MLA_DV, torch.bfloat16, v_is_k_prefix=True)
    cache = ksa.Cache(p, B, max(ns_text) // k + 2, device=dev)
    Ls = [O.augmented_len(n - 1, k) for n in ns_text]
    seg = torch.tensor(np.concatenate([[0], np.cumsum(Ls)]), dtype=torch.int64, device=dev)
    ksa.ksa_cache_append_rows(cache, seg, max(Ls), torch.cat([kx[:l] for l in Ls]).contiguous().to(dev), None)
    q = torch.zeros((B, MLA_HQ, MLA_DQK), dtype=torch.bfloat16, device=dev)
    ws = ksa.decode_workspace(cache)
    n_now = [n - 1 for n in ns_text]
    a_next = list(Ls)
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    most_ranges = 0
    for step in range(k + 2):
        kinds = [1 if (a % (k + 1)) == k else 0 for a in a_next]
        kt = torch.tensor(kinds, dtype=torch.int32, device=dev)
        ksa.ksa_cache_append(cache, kx[a_next].contiguous().to(dev), None, kt)
        for b in range(B):
            a_next[b] += 1
            if not kinds[b]:
                n_now[b] += 1
        lse = torch.empty((B, MLA_HQ), dtype=torch.float32, device=dev)
        print(f"MLA range coverage: step {step} kinds {kinds}", flush=True)
        out = ksa.ksa_decode_attn(cache, q, kt, lse=lse, workspace=ws)
        torch.cuda.synchronize()
        o, ls = _np(out), _np(lse)
        lens = [len(O.decode_visible_rows(n_now[b], k, C, "s" if kinds[b] else "t")) for b in range(B)]
        # the launch's cut: about total / (CUs - batch) rows per range, at
        # least 64, a whole number of 32-row tiles
        per = max(64, -(-sum(lens) // max(n_cu - B, n_cu // 2)))
        per = -(-per // 32) * 32
        most_ranges = max(most_ranges, max(-(-n // per) for n in lens))
        for b in range(B):
            rows = O.decode_visible_rows(n_now[b], k, C, "s" if kinds[b] else "t")
            want = _expected(rows, _mla_codes(rows), MLA_DV)
            assert want.max() < 128
            for h in (0, 45, 127):
                n_rows, cnt = _recover(o[b, h], ls[b, h])
                assert n_rows == len(rows), (step, b, h, n_rows, len(rows))
                np.testing.assert_array_equal(cnt, want, err_msg=f"step {step} seq {b} head {h}")
            # every head reads the same rows
            np.testing.assert_array_equal(o[b], np.broadcast_to(o[b, 0], o[b].shape))
    assert most_ranges >= min_ranges
    assert ksa.ksa_cache_read_errors(cache) == [0] * B
