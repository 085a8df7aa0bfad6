"""GPU parity of the chunked / variable-length prefill against the cache and
of the row-wise cache append that follows it (all through the C ABI).

* ksa_cache_append_rows: after every step the whole cache equals, slot for
  slot, the oracle's Fig. 4 slot model stepped through the same rows one
  append at a time (bit-exact; rows tagged in element 0).
* ksa_prefill_chunk: each segment's rows equal the rows of the oracle's
  one-shot prefill over the whole sequence (Eq. 10 under the Eq. 3 rule),
  whatever the split: segments that start mid-chunk, right before a summary
  row, on chunk boundaries, one row long or the whole sequence, and
  sequences of different lengths packed in one call.  bf16: max |err| <=
  2e-2, mean <= 2e-3; fp32 <= 1e-4.
"""
import numpy as np
import pytest
import torch

import ksa_synth
from oracle import ksa_oracle as O

pytestmark = pytest.mark.gpu

ksa = pytest.importorskip("kv_cache_compression_amd")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _np(t):
    return t.detach().float().cpu().double().numpy()


def _pack(splits, step):
    """Row counts of every sequence at this step -> seg_rows, max_rows."""
    counts = [s[step] if step < len(s) else 0 for s in splits]
    seg = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return counts, seg, max(max(counts), 1)


def _starts(splits, step):
    return [int(sum(s[:step])) for s in splits]


@pytest.mark.parametrize("k,C,dtype,D", [(4, 2, torch.float32, 8), (3, 1, torch.float32, 8),
                                         (4, 0, torch.float32, 8), (8, 3, torch.bfloat16, 128)])
def test_append_rows_matches_slot_model(k, C, dtype, D):
    dev = _dev()
    n = 61
    L = O.augmented_len(n, k)
    is_s, _ = O.augmented_rows(n, k)
    # three sequences, each its own split of the same L rows (bf16 tags stay exact below 256)
    splits = [[L], [1, k, k + 1, 2, L - 2 * k - 4], [k, 1, 5, 3 * (k + 1), L - 4 * k - 9]]
    hkv = 2
    rows_k = torch.zeros((L, hkv, D), dtype=torch.float32)
    rows_v = torch.zeros((L, hkv, D), dtype=torch.float32)
    rows_k[:, :, 0] = torch.arange(L, dtype=torch.float32)[:, None] + 1
    rows_v[:, :, 0] = -(torch.arange(L, dtype=torch.float32)[:, None] + 1)
    rows_k[:, 1, 1] = 0.5
    p = ksa.Params(k, C, 2 * hkv, hkv, D, D, dtype)
    max_s = n // k + 1
    cache = ksa.Cache(p, 3, max_s, device=dev)
    models = [O.CacheModel(k, C, max_s) for _ in range(3)]
    for step in range(max(len(s) for s in splits)):
        counts, seg, max_rows = _pack(splits, step)
        starts = _starts(splits, step)
        idx = np.concatenate([np.arange(st, st + c) for st, c in zip(starts, counts)]).astype(np.int64)
        kr = rows_k[idx].to(dtype).to(dev)
        vr = rows_v[idx].to(dtype).to(dev)
        print(f"step {step}: rows {counts}", flush=True)
        ksa.ksa_cache_append_rows(cache, torch.tensor(seg, device=dev), max_rows, kr, vr)
        for b in range(3):
            for a in range(starts[b], starts[b] + counts[b]):
                (models[b].append_summary if is_s[a] else models[b].append_text)(a + 1)
        torch.cuda.synchronize()
        ck, cv, st = cache.k.float().cpu(), cache.v.float().cpu(), cache.state.cpu()
        for b in range(3):
            mdl = models[b]
            assert st[b, 0].item() == mdl.m and st[b, 1].item() == mdl.r and st[b, 3].item() == 0
            assert st[b, 2].item() == 0   # reserved word untouched
            want = torch.tensor([0.0 if t is None else float(t) for t in mdl.slots])
            assert torch.equal(ck[b, :, :, 0], want[None].expand(hkv, -1))
            assert torch.equal(cv[b, :, :, 0], -want[None].expand(hkv, -1))
            assert torch.equal(ck[b, 1, :, 1], torch.where(want > 0, 0.5, 0.0))


def test_append_rows_overflow_sets_error():
    dev = _dev()
    k, C = 4, 1
    p = ksa.Params(k, C, 2, 1, 8, 8, torch.float32)
    cache = ksa.Cache(p, 1, 2, device=dev)
    rows = torch.ones((3 * (k + 1), 1, 8), device=dev)
    ksa.ksa_cache_append_rows(cache, torch.tensor([0, 3 * (k + 1)], device=dev), 3 * (k + 1), rows, rows)
    torch.cuda.synchronize()
    st = cache.state.cpu()
    assert st[0, 3].item() == ksa.KSA_CACHE_ERR_SUMMARY_FULL and st[0, 0].item() == 0
    assert torch.count_nonzero(cache.k).item() == 0


def _chunk_case(dtype, D, n, k, C, hq, hkv, splits, seed):
    dev = _dev()
    L = O.augmented_len(n, k)
    B = len(splits)
    w = ksa_synth.PrefillWorkload("case", B, n, k, C, hq, hkv, D, D, dtype, 1e6, seed)
    q, kx, v = ksa_synth.prefill_qkv(w, L)
    p = ksa.Params(k, C, hq, hkv, D, D, dtype)
    cache = ksa.Cache(p, B, n // k + 1, device=dev)
    refs = []
    for b in range(B):
        o, l_ = O.ksa_attention(q[b].double().numpy(), kx[b].double().numpy(), v[b].double().numpy(), n, k, C,
                                p.scale)
        refs.append((o, l_))
    bf = dtype == torch.bfloat16
    for step in range(max(len(s) for s in splits)):
        counts, seg, max_rows = _pack(splits, step)
        starts = _starts(splits, step)
        sel = [(b, np.arange(st, st + c)) for b, (st, c) in enumerate(zip(starts, counts))]
        cat = lambda t: torch.cat([t[b, rows] for b, rows in sel]).to(dev)
        qs, ks, vs = cat(q), cat(kx), cat(v)
        segd = torch.tensor(seg, device=dev)
        lse = torch.full((hq, int(seg[-1])), float("nan"), device=dev)
        print(f"step {step}: rows {counts} from {starts}", flush=True)
        out = ksa.ksa_prefill_chunk(cache, segd, max_rows, qs, ks, vs, lse=lse)
        ksa.ksa_cache_append_rows(cache, segd, max_rows, ks, vs)
        torch.cuda.synchronize()
        o = _np(out)
        ls = _np(lse)
        for b, rows in sel:
            if len(rows) == 0:
                continue
            got = o[seg[b]:seg[b + 1]]
            ref = refs[b][0][rows]
            e = np.abs(got - ref)
            if bf:
                assert e.max() <= 2e-2 and e.mean() <= 2e-3, (b, step, e.max())
            else:
                assert e.max() <= 1e-4, (b, step, e.max())
            el = np.abs(ls[:, seg[b]:seg[b + 1]] - refs[b][1][:, rows])
            assert el.max() <= (2e-2 if bf else 1e-4), (b, step, el.max())
    st = cache.state.cpu()
    for b in range(B):
        assert st[b, 0].item() == n // k and st[b, 1].item() == n % k and st[b, 3].item() == 0


@pytest.mark.parametrize("dtype,D,n,k,C,hq,hkv", [
    (torch.bfloat16, 128, 700, 8, 4, 8, 2),   # MFMA path
    (torch.bfloat16, 128, 530, 5, 3, 4, 4),   # MFMA path, g = 1, k = 5
    (torch.bfloat16, 128, 400, 8, 0, 4, 2),   # MFMA path, no ring
    (torch.bfloat16, 128, 600, 8, 3, 16, 2),  # MFMA path, g = 8: two head groups per summary
    (torch.bfloat16, 128, 500, 12, 2, 8, 2),  # MFMA path, k = 12: summary rows in two passes
    (torch.float32, 64, 300, 8, 2, 4, 2),     # generic path
])
def test_chunked_prefill_matches_one_shot(dtype, D, n, k, C, hq, hkv):
    L = O.augmented_len(n, k)
    splits = [
        [L],                                          # one-shot through the chunk path
        [1, k - 1, 1, 2 * (k + 1), 64, 200, L - 3 * k - 267],   # ends right before a summary, then on it
        [130, 1, 1, 1, 127, L - 260],
        [k + 1, L - k - 1],
    ]
    _chunk_case(dtype, D, n, k, C, hq, hkv, splits, seed=n + k)


def test_chunked_prefill_long_history():
    """A short segment after a long history: most keys come from the cache's
    summary buffer and ring (MFMA path, several tiles of cached summaries)."""
    n, k, C = 3000, 8, 8
    L = O.augmented_len(n, k)
    _chunk_case(torch.bfloat16, 128, n, k, C, 8, 2, [[L - 150, 150], [L - 1, 1]], seed=99)


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 32)])
def test_chunk_skips_sequences_with_bad_state(dtype, D):
    """A cache state out of range (m beyond the summary capacity, r > k)
    leaves that sequence's rows unwritten; the other sequence is computed."""
    dev = _dev()
    k, C, n = 8, 2, 40
    L = O.augmented_len(n, k)
    p = ksa.Params(k, C, 4, 2, D, D, dtype)
    cache = ksa.Cache(p, 2, 8, device=dev)
    g = ksa_synth.gen(3)
    q = ksa_synth.normal((2 * L, 4, D), dtype, g).to(dev)
    kx = ksa_synth.normal((2 * L, 2, D), dtype, g).to(dev)
    v = ksa_synth.normal((2 * L, 2, D), dtype, g).to(dev)
    seg = torch.tensor([0, L, 2 * L], dtype=torch.int64, device=dev)
    for bad in ([9, 0], [0, k + 1], [-1, 0]):
        cache.state.zero_()
        cache.state[1, :2] = torch.tensor(bad, dtype=torch.int32)
        out = torch.full((2 * L, 4, D), float("nan"), dtype=dtype, device=dev)
        ksa.ksa_prefill_chunk(cache, seg, L, q, kx, v, out=out)
        torch.cuda.synchronize()
        assert torch.isnan(out[L:].float()).all(), bad
        assert not torch.isnan(out[:L].float()).any(), bad
        st = cache.state.cpu()
        assert st[1, 3].item() & 16 and st[0, 3].item() == 0, (bad, st)  # KSA_CACHE_ERR_BAD_SEGMENT


def test_chunked_prefill_absorbed_latent_generic():
    """V as the first Dv columns of K (absorbed latent form), fp32 generic path:
    chunked prefill through the cache equals the one-shot oracle."""
    dev = _dev()
    n, k, C, hq, dqk, dv = 150, 4, 3, 4, 48, 32
    L = O.augmented_len(n, k)
    g = ksa_synth.gen(31)
    q = ksa_synth.normal((L, hq, dqk), torch.float32, g)
    kx = ksa_synth.normal((L, 1, dqk), torch.float32, g)
    p = ksa.Params(k, C, hq, 1, dqk, dv, torch.float32, v_is_k_prefix=True)
    ref, rl = O.ksa_attention(q.double().numpy(), kx.double().numpy(), None, n, k, C, p.scale, dv=dv)
    cache = ksa.Cache(p, 1, n // k + 1, device=dev)
    start = 0
    for cnt in (7, 1, k, 40, L - 52):
        seg = torch.tensor([0, cnt], dtype=torch.int64, device=dev)
        qs, ks_ = q[start:start + cnt].to(dev), kx[start:start + cnt].to(dev)
        lse = torch.empty((hq, cnt), dtype=torch.float32, device=dev)
        out = ksa.ksa_prefill_chunk(cache, seg, cnt, qs, ks_, None, lse=lse)
        ksa.ksa_cache_append_rows(cache, seg, cnt, ks_, None)
        torch.cuda.synchronize()
        assert np.abs(_np(out) - ref[start:start + cnt]).max() <= 1e-4
        assert np.abs(_np(lse) - rl[:, start:start + cnt]).max() <= 1e-4
        start += cnt
    assert cache.state[0, 0].item() == n // k and cache.state[0, 1].item() == n % k
