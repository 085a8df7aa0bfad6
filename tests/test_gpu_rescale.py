"""GPU parity on inputs that force the kernels' deferred rescale.

The MFMA prefill kernels (one-shot and chunked, d = 128) and the absorbed-MLA
decode and prefill keep one exponent reference per query row and move it only when a
later key tile's maximum exceeds it by more than 8 (log2 units); O and the
row sum are then multiplied by 2^(old - new).  With N(0,1) inputs a later
tile practically never beats the first by that much, so these tests build
inputs where it must:

* every query is close to one direction u (all heads), every key is small
  noise, so every score is about 0;
* a few keys get + J w, w = u / (|u|^2 scale log2(e)), which lifts their
  score by about J log2 units;
* values of the lifted keys are offset by -0.5, the others by +0.5, so the
  output measures how much weight the keys before the jump keep.

J = 9.5 moves the reference once while the keys before the jump still hold
a large share of the softmax mass (asserted below: doubling their weight
would move outputs far beyond the tolerance); J = 150 would overflow the
exponentials (2^150 > fp32 max) without the rescale.  Outputs and LSE are
compared element by element with the fp64 oracle (Eq. 10 under the Eq. 3
rule): bf16 max |err| <= 2e-2, mean <= 2e-3; LSE <= 2e-2.
"""
import math

import numpy as np
import pytest
import torch

import ksa_synth
from oracle import ksa_oracle as O

pytestmark = pytest.mark.gpu

ksa = pytest.importorskip("kv_cache_compression_amd")

LOG2E = 1.0 / math.log(2.0)


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _np(t):
    return t.detach().float().cpu().double().numpy()


def _lift_direction(u, scale):
    """w with (u . w) scale log2(e) = 1: adding J w to a key lifts the score
    of a query equal to u by J log2 units."""
    return u / (u.dot(u) * scale * LOG2E)


def _gqa_inputs(n, k, hq, hkv, D, J, lifted_rows, seed):
    L = O.augmented_len(n, k)
    g = ksa_synth.gen(seed)
    scale = 1.0 / math.sqrt(D)
    u = ksa_synth.normal((D,), torch.float32, g)
    w = _lift_direction(u, scale)
    q = (u + 0.3 * ksa_synth.normal((1, L, hq, D), torch.float32, g)).to(torch.bfloat16)
    kx = 0.1 * ksa_synth.normal((1, L, hkv, D), torch.float32, g)
    v = 0.3 * ksa_synth.normal((1, L, hkv, D), torch.float32, g) + 0.5
    for a in lifted_rows:
        kx[0, a] += J * w
        v[0, a] -= 1.0
    return q, kx.to(torch.bfloat16), v.to(torch.bfloat16), scale


def _check_sensitive(qn, kn, vn, n, k, C, scale, rows, lifted, hq, hkv):
    """The case is informative: for the rows that see a lifted key, the keys
    that are not lifted keep a share of the mass such that doubling their
    weight moves the output by > 4e-2 (twice the tolerance)."""
    mask = O.visibility_mask_fast(n, k, C, rows=rows)
    g = hq // hkv
    moved = []
    for ri, a in enumerate(rows):
        if not mask[ri, lifted].any():
            continue
        for h in range(0, hq, g + 1):
            kv = h // g
            s = (kn[:, kv] @ qn[a, h]) * scale
            s = np.where(mask[ri], s, -np.inf)
            wt = np.exp(s - s.max())
            # the jump the kernel must take: lifted score above every other visible one by > 8 log2
            others = np.delete(s, lifted)
            assert (s[lifted][mask[ri, lifted]].max() - others.max()) * LOG2E > 8.0
            o1 = (wt[:, None] * vn[:, kv]).sum(0) / wt.sum()
            w2 = wt * 2.0
            w2[lifted] = wt[lifted]
            o2 = (w2[:, None] * vn[:, kv]).sum(0) / w2.sum()
            moved.append(np.abs(o2 - o1).max())
    assert len(moved) > 20 and np.median(moved) > 4e-2, (len(moved), np.median(moved) if moved else None)


def _compare(out, lse, ref, rl, what):
    e = np.abs(out - ref)
    el = np.abs(lse - rl)
    assert np.isfinite(out).all() and np.isfinite(lse).all(), what
    print(f"{what}: max {e.max():.3e} mean {e.mean():.3e} lse {el.max():.3e}", flush=True)
    assert e.max() <= 2e-2 and e.mean() <= 2e-3 and el.max() <= 2e-2, what


N, K, C, HQ, HKV, D = 4101, 8, 4, 8, 2, 128


def _lifted_rows():
    # s_64 lifts the summary run of every query in chunk >= 69; t_320 (chunk
    # 40) lifts the text run of chunks 40..44, which see no lifted summary
    return [O.summary_row(64, K), O.text_row(320, K)]


@pytest.mark.parametrize("J", [9.5, 150.0])
def test_prefill_d128_forced_rescale(J):
    dev = _dev()
    lifted = _lifted_rows()
    q, kx, v, scale = _gqa_inputs(N, K, HQ, HKV, D, J, lifted, 41)
    L = O.augmented_len(N, K)
    qn, kn, vn = q[0].double().numpy(), kx[0].double().numpy(), v[0].double().numpy()
    if J < 20:
        _check_sensitive(qn, kn, vn, N, K, C, scale, np.arange(0, L, 7), lifted, HQ, HKV)
    p = ksa.Params(K, C, HQ, HKV, D, D, torch.bfloat16)
    lse = torch.empty((1, HQ, L), dtype=torch.float32, device=dev)
    print(f"one-shot prefill, lift {J}", flush=True)
    out = ksa.ksa_prefill_attn(p, q.to(dev), kx.to(dev), v.to(dev), N, lse=lse)
    torch.cuda.synchronize()
    ref, rl = O.ksa_attention(qn, kn, vn, N, K, C, scale)
    _compare(_np(out[0]), _np(lse[0]), ref, rl, f"one-shot J={J}")


@pytest.mark.parametrize("J", [9.5, 150.0])
def test_prefill_chunk_d128_forced_rescale(J):
    """The same inputs fed in three segments through the cache: s_64 lies in
    the second segment's own summary run and in the third segment's cache
    summary run; t_320 in the second segment's text run."""
    dev = _dev()
    lifted = _lifted_rows()
    q, kx, v, scale = _gqa_inputs(N, K, HQ, HKV, D, J, lifted, 43)
    L = O.augmented_len(N, K)
    qn, kn, vn = q[0].double().numpy(), kx[0].double().numpy(), v[0].double().numpy()
    ref, rl = O.ksa_attention(qn, kn, vn, N, K, C, scale)
    p = ksa.Params(K, C, HQ, HKV, D, D, torch.bfloat16)
    cache = ksa.Cache(p, 1, N // K + 1, device=dev)
    bounds = [0, 301, 2900, L]
    for s in range(3):
        a0, a1 = bounds[s], bounds[s + 1]
        R = a1 - a0
        seg = torch.tensor([0, R], dtype=torch.int64, device=dev)
        qs, ks_, vs = (t[0, a0:a1].contiguous().to(dev) for t in (q, kx, v))
        lse = torch.empty((HQ, R), dtype=torch.float32, device=dev)
        print(f"chunked prefill, lift {J}, rows {a0}..{a1}", flush=True)
        out = ksa.ksa_prefill_chunk(cache, seg, R, qs, ks_, vs, lse=lse)
        ksa.ksa_cache_append_rows(cache, seg, R, ks_, vs)
        torch.cuda.synchronize()
        _compare(_np(out), _np(lse), ref[a0:a1], rl[:, a0:a1], f"chunk J={J} rows {a0}..{a1}")
    assert ksa.ksa_cache_read_errors(cache) == [0]


# ------------------------------------------------------------ MLA decode --

MLA_HQ, MLA_DQK, MLA_DV = 128, 576, 512


def _mla_inputs(n, k, J, lifted_rows, seed):
    """Latent rows K [1, L, 1, 576] (V = the first 512 columns) and queries
    close to u.  The lift lives in the 64 rotary columns, which are not part
    of V, so lifted rows keep values of the same size as the others; their
    values are offset along a latent direction orthogonal to u (so the
    offset does not move scores)."""
    L = O.augmented_len(n, k)
    g = ksa_synth.gen(seed)
    scale = 1.0 / math.sqrt(MLA_DQK)
    u = ksa_synth.normal((MLA_DQK,), torch.float32, g)
    ur = u.clone()
    ur[:MLA_DV] = 0.0
    w = _lift_direction(ur, scale)
    off = ksa_synth.normal((MLA_DQK,), torch.float32, g)
    off[MLA_DV:] = 0.0
    ul = u.clone()
    ul[MLA_DV:] = 0.0
    off = off - off.dot(ul) / ul.dot(ul) * ul
    off = 0.5 * off / off.abs().mean()
    kx = 0.05 * ksa_synth.normal((1, L, 1, MLA_DQK), torch.float32, g) + 0.5 * off
    for a in lifted_rows:
        kx[0, a, 0] += J * w - off
    return kx.to(torch.bfloat16), u, scale


@pytest.mark.parametrize("J", [10.0, 150.0])
def test_decode_mla_forced_rescale(J):
    """One sequence whose text slice is 128 rows: the split launch cuts it
    into two 64-row ranges of two 32-key tiles each.  The lifted summary sits
    at slice offset 40, in the second tile of the first range, so that range
    moves its reference after a tile of 32 keys at the old level."""
    dev = _dev()
    k, C = 8, 2
    r = 3
    m = 111                      # slice: r + C k + (m - C) = 3 + 16 + 109 = 128 rows
    n = m * k + r
    start = 1 + k - r
    # summary j sits at slice offset r + C k + j
    j_lift = 40 - r - C * k
    a_lift = O.summary_row(j_lift, k)
    assert O.slot_of_row(a_lift, m, r, k, C) - start == 40
    kx, u, scale = _mla_inputs(n, k, J, [a_lift], 51)
    g = ksa_synth.gen(52)
    q = (u + 0.3 * ksa_synth.normal((1, MLA_HQ, MLA_DQK), torch.float32, g)).to(torch.bfloat16)
    kn = kx[0].double().numpy()
    qn = q[0].double().numpy()
    rows = O.decode_visible_rows(n, k, C, "t")
    assert len(rows) == 128
    s = (kn[rows, 0] @ qn.T) * scale * LOG2E                 # [rows, heads], log2 units
    li = int(np.nonzero(rows == a_lift)[0][0])
    assert (s[li] - np.delete(s, li, axis=0).max(0)).min() > 8.0
    if J < 20:
        # the 32 keys of the first tile keep enough weight to show a wrong rescale
        v = kn[rows, 0, :MLA_DV]
        order = np.array([O.slot_of_row(int(a), m, r, k, C) - start for a in rows])
        first_tile = order < 32
        wt = np.exp((s - s.max(0)) / LOG2E)
        o1 = (wt.T @ v) / wt.sum(0)[:, None]
        w2 = wt.copy()
        w2[first_tile] *= 2.0
        o2 = (w2.T @ v) / w2.sum(0)[:, None]
        assert np.median(np.abs(o2 - o1).max(1)) > 4e-2
    p = ksa.Params(k, C, MLA_HQ, 1, MLA_DQK, MLA_DV, torch.bfloat16, v_is_k_prefix=True)
    cache = ksa.Cache(p, 1, m + 1, device=dev)
    print(f"MLA decode, lift {J}", flush=True)
    ksa.ksa_cache_fill(cache, kx.to(dev), None, n)
    kind = torch.zeros((1,), dtype=torch.int32, device=dev)
    lse = torch.empty((1, MLA_HQ), dtype=torch.float32, device=dev)
    out = ksa.ksa_decode_attn(cache, q.to(dev), kind, lse=lse)
    torch.cuda.synchronize()
    ref, rl = O.decode_attention(qn, kn, None, n, k, C, scale, "t", dv=MLA_DV)
    _compare(_np(out[0]), _np(lse[0]), ref, rl, f"MLA decode J={J}")
    assert ksa.ksa_cache_read_errors(cache) == [0]


@pytest.mark.parametrize("J", [10.0, 150.0])
def test_decode_mla_forced_rescale_ragged_batch(J):
    """Three ragged sequences (many ranges each), filled through the
    row-wise append with packed rows; lifted summaries at spread positions,
    some in the second tile of their range."""
    dev = _dev()
    k, C = 8, 4
    ns = [5003, 6101, 7007]
    B = len(ns)
    Ls = [O.augmented_len(n, k) for n in ns]
    lifted = [O.summary_row(j, k) for j in (40, 97, 161, 230, 300, 371, 433, 500)]
    kx, u, scale = _mla_inputs(max(ns), k, J, lifted, 61)
    g = ksa_synth.gen(62)
    q = (u + 0.3 * ksa_synth.normal((B, MLA_HQ, MLA_DQK), torch.float32, g)).to(torch.bfloat16)
    p = ksa.Params(k, C, MLA_HQ, 1, MLA_DQK, MLA_DV, torch.bfloat16, v_is_k_prefix=True)
    cache = ksa.Cache(p, B, max(ns) // k + 1, device=dev)
    rows = torch.cat([kx[0, :Lb] for Lb in Ls]).contiguous().to(dev)
    seg = torch.tensor(np.concatenate([[0], np.cumsum(Ls)]), dtype=torch.int64, device=dev)
    ksa.ksa_cache_append_rows(cache, seg, max(Ls), rows, None)
    kind = torch.zeros((B,), dtype=torch.int32, device=dev)
    lse = torch.empty((B, MLA_HQ), dtype=torch.float32, device=dev)
    print(f"MLA decode ragged, lift {J}", flush=True)
    out = ksa.ksa_decode_attn(cache, q.to(dev), kind, lse=lse)
    torch.cuda.synchronize()
    kn = kx[0].double().numpy()
    for b, n in enumerate(ns):
        ref, rl = O.decode_attention(q[b].double().numpy(), kn, None, n, k, C, scale, "t", dv=MLA_DV)
        _compare(_np(out[b]), _np(lse[b]), ref, rl, f"MLA ragged b={b} J={J}")
    assert ksa.ksa_cache_read_errors(cache) == [0] * B


# ------------------------------------------------------------ MLA prefill --


@pytest.mark.parametrize("J", [10.0, 150.0])
def test_prefill_mla_forced_rescale(J):
    """Absorbed-MLA prefill: summaries s_40 and s_70 are lifted, so every
    text row of chunk >= 45 meets a lifted key in the second (or a later)
    32-key tile of its summary run, after a whole tile at the old level, and
    must move its reference and rescale what it holds.  All rows against the
    oracle."""
    dev = _dev()
    n, k, C = 803, 8, 4
    L = O.augmented_len(n, k)
    lifted = [O.summary_row(40, k), O.summary_row(70, k)]
    kx, u, scale = _mla_inputs(n, k, J, lifted, 71)
    g = ksa_synth.gen(72)
    q = (u + 0.3 * ksa_synth.normal((1, L, MLA_HQ, MLA_DQK), torch.float32, g)).to(torch.bfloat16)
    kn = kx[0].double().numpy()
    # the lifted keys beat every other key by more than 2^8 for a text row
    # late in the sequence
    row = L - 2
    s = (kn[:, 0] @ q[0, row].double().numpy().T) * scale * LOG2E   # [keys, heads]
    others = np.delete(s, lifted, axis=0).max(0)
    assert (s[lifted[0]] - others).min() > 8.0
    p = ksa.Params(k, C, MLA_HQ, 1, MLA_DQK, MLA_DV, torch.bfloat16, v_is_k_prefix=True)
    lse = torch.empty((1, MLA_HQ, L), dtype=torch.float32, device=dev)
    print(f"MLA prefill, lift {J}", flush=True)
    out = ksa.ksa_prefill_attn(p, q.to(dev), kx.to(dev), None, n, lse=lse)
    torch.cuda.synchronize()
    ref, rl = O.ksa_attention(q[0].double().numpy(), kn, None, n, k, C, scale, dv=MLA_DV)
    _compare(_np(out[0]), _np(lse[0]), ref, rl, f"MLA prefill J={J}")
