"""Plain fp64 CPU oracle for Kwai Summary Attention (KSA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the package's ``smoke()`` entry and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
and imports nothing from it.

Everything is written straight from "Kwai Summary Attention Technical Report"
(arXiv:2604.24432) and the close reading of it, with no blocking, fusion or
reordering beyond what the definitions state:

* augmented sequence ............ Sec. 2.2.1, Eq. (1)
* summary visibility and the summary position id ... Sec. 2.2.1 (the two
  bullet rules that follow Eq. (1))
* sliding-chunk text window ..... Sec. 2.2.2, Eq. (2)
* full text-token visible set ... Sec. 2.2.2, Eq. (3) and the note that
  in-window summaries are not read
* masked softmax attention ...... Sec. 4.1.4, Eq. (9) and Eq. (10)
* KV-cache layout and lifecycle . Sec. 2.3.1 and Fig. 4 (a)-(e)
* per-token cache accounting .... Sec. 3, Table 1, Eq. (4)-(6)
* attention backward ............ chain rule through Eq. (10) (the report
  trains with this kernel, Sec. 2.3); the softmax Jacobian written out

Readings taken where the pages are silent or ambiguous:

* a summary token sees the k text tokens of its own chunk and itself
  (``summary_sees_self=True``, the default); the other reading (k keys) is
  kept behind the switch;
* ``C`` counts complete past chunks; the query's own (possibly partial) chunk
  is always in the window; chunks with negative index do not exist;
* ``n`` need not be a multiple of ``k``: the trailing partial chunk has no
  summary yet;
* text position ids are text indices; a summary's position id is that of its
  chunk's last text token, ``j*k + k - 1``;
* RoPE is the half-split ("rotate-half") form with frequencies
  ``theta ** (-2 f / rot_dim)``;
* query head ``h`` uses key/value head ``h // (Hq // Hkv)``.

Parity status of every function is pinned by ``tests/test_oracle_*.py``
(closed forms, a hand-enumerated literal for the Fig. 3 configuration,
invariants, reductions to a library routine, brute force).  No function here
is "parity unpinned".
"""

from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence, Set, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# Augmented sequence, Eq. (1)
# ---------------------------------------------------------------------------


def num_chunks(n: int, k: int) -> int:
    """Number of complete chunks M = floor(n / k); each one carries a summary."""
    return n // k


def augmented_len(n: int, k: int) -> int:
    """L = n + floor(n/k): one summary token after every k text tokens (Eq. 1)."""
    return n + n // k


def text_row(i: int, k: int) -> int:
    """Augmented row of text token t_i.

    Eq. (1) lays chunk j out as [t_jk .. t_jk+k-1, s_j], so every complete
    chunk before t_i adds one summary row ahead of it.
    """
    return i + i // k


def summary_row(j: int, k: int) -> int:
    """Augmented row of summary s_j: the last row of chunk j in Eq. (1)."""
    return j * (k + 1) + k


def decode_row(a: int, n: int, k: int) -> Tuple[str, int]:
    """Inverse of the Eq. (1) map: augmented row -> ('t', i) or ('s', j)."""
    M = n // k
    if a < 0 or a >= augmented_len(n, k):
        raise IndexError(a)
    if a < M * (k + 1):
        c, o = divmod(a, k + 1)
        return ("s", c) if o == k else ("t", c * k + o)
    return ("t", M * k + (a - M * (k + 1)))


def augmented_rows(n: int, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per augmented row: (is_summary bool[L], index int64[L]).

    ``index`` is the text index i for a text row and the chunk index j for a
    summary row.  Built by walking Eq. (1) chunk by chunk.
    """
    kinds: List[bool] = []
    idx: List[int] = []
    M = n // k
    for j in range(M):
        for o in range(k):
            kinds.append(False)
            idx.append(j * k + o)
        kinds.append(True)
        idx.append(j)
    for i in range(M * k, n):  # trailing partial chunk: no summary yet
        kinds.append(False)
        idx.append(i)
    return np.array(kinds, dtype=bool), np.array(idx, dtype=np.int64)


def position_ids(n: int, k: int) -> np.ndarray:
    """Position id per augmented row (Sec. 2.2.1).

    Text tokens keep their text index (summaries consume no position); the
    summary of chunk j takes the id of the chunk's last text token, jk+k-1.
    """
    is_s, idx = augmented_rows(n, k)
    pos = np.where(is_s, idx * k + (k - 1), idx)
    return pos.astype(np.int64)


# ---------------------------------------------------------------------------
# Rotary position embedding (half-split), applied to Q and K before attention
# ---------------------------------------------------------------------------


def rope_rotate(x: np.ndarray, pos: np.ndarray, theta: float,
                rot_off: int = 0, rot_dim: Optional[int] = None) -> np.ndarray:
    """Rotate dims [rot_off, rot_off+rot_dim) of ``x`` (shape [..., R, H, D]).

    ``pos`` has shape [R] (one id per row).  Pair (f, f + rot_dim/2) of the
    rotated block turns by angle pos * theta**(-2f/rot_dim).  fp64 throughout.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    D = x.shape[-1]
    if rot_dim is None:
        rot_dim = D - rot_off
    if rot_dim % 2 or rot_off + rot_dim > D:
        raise ValueError("bad rotary block")
    half = rot_dim // 2
    f = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * f / rot_dim)                  # [half]
    ang = pos.astype(np.float64)[:, None] * inv_freq[None, :]  # [R, half]
    c = np.cos(ang)[:, None, :]                                # [R, 1, half]
    s = np.sin(ang)[:, None, :]
    lo = x[..., rot_off:rot_off + half].copy()
    hi = x[..., rot_off + half:rot_off + rot_dim].copy()
    x[..., rot_off:rot_off + half] = lo * c - hi * s
    x[..., rot_off + half:rot_off + rot_dim] = hi * c + lo * s
    return x


# ---------------------------------------------------------------------------
# Visibility (Sec. 2.2.1 rules, Eq. (2)-(3))
# ---------------------------------------------------------------------------


def _visible(kind_q: str, iq: int, kind_k: str, ik: int, k: int, C: int,
             summary_sees_self: bool) -> bool:
    """Predicate form of the KSA visibility rule for one (query, key) pair."""
    if kind_q == "s":
        # A summary reads only its own chunk's text (and, by the reading
        # taken here, itself).
        if kind_k == "t":
            return ik // k == iq
        return summary_sees_self and ik == iq
    c = iq // k
    if kind_k == "t":
        # Eq. (2): text from the first token of chunk c-C up to t_i itself.
        return ik // k >= c - C and ik <= iq
    # Eq. (3): distant summaries s_0 .. s_{c-C-1}; in-window summaries unseen.
    return ik <= c - C - 1


def visibility_mask(n: int, k: int, C: int, summary_sees_self: bool = True,
                    rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Dense bool mask V[a, b] over the augmented sequence (rows subset optional)."""
    is_s, idx = augmented_rows(n, k)
    L = len(is_s)
    rows = range(L) if rows is None else rows
    out = np.zeros((len(rows), L), dtype=bool)
    kk = np.where(is_s, "s", "t")
    for r, a in enumerate(rows):
        for b in range(L):
            out[r, b] = _visible(kk[a], int(idx[a]), kk[b], int(idx[b]), k, C,
                                 summary_sees_self)
    return out


def visibility_mask_fast(n: int, k: int, C: int, summary_sees_self: bool = True,
                         rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Same predicate as :func:`visibility_mask`, evaluated with array compares.

    Used for sizes where the per-pair loop is too slow; a test checks that the
    two agree element for element.
    """
    is_s, idx = augmented_rows(n, k)
    rows = np.arange(len(is_s)) if rows is None else np.asarray(rows, dtype=np.int64)
    qs = is_s[rows][:, None]
    qi = idx[rows][:, None]
    ks = is_s[None, :]
    ki = idx[None, :]
    c = qi // k
    text_q = (~ks & (ki // k >= c - C) & (ki <= qi)) | (ks & (ki <= c - C - 1))
    summ_q = (~ks & (ki // k == qi))
    if summary_sees_self:
        summ_q = summ_q | (ks & (ki == qi))
    return np.where(qs, summ_q, text_q)


def visible_set_eq3(n: int, k: int, C: int, a: int,
                    summary_sees_self: bool = True) -> Set[int]:
    """Visible augmented rows of row ``a``, enumerated directly from the sets.

    Text t_i: {s_0 .. s_{floor(i/k)-C-1}} U {t_{(floor(i/k)-C)k} .. t_i}
    (Eq. 3), clamped at index 0.  Summary s_j: {t_jk .. t_jk+k-1} (and s_j).
    This is a second, independent encoding of the same rule.
    """
    kind, q = decode_row(a, n, k)
    out: Set[int] = set()
    if kind == "s":
        for i in range(q * k, q * k + k):
            out.add(text_row(i, k))
        if summary_sees_self:
            out.add(summary_row(q, k))
        return out
    c = q // k
    for j in range(0, c - C):            # s_0 .. s_{c-C-1}
        out.add(summary_row(j, k))
    for i in range(max(0, (c - C) * k), q + 1):
        out.add(text_row(i, k))
    return out


def token_swa_mask(n: int, k: int, W: int) -> np.ndarray:
    """The rejected token-level window of Fig. 3 (left), for negative tests.

    Text t_i sees text t_{i-W+1} .. t_i and every summary whose whole chunk
    has left that window; summaries see their own chunk and themselves.
    """
    is_s, idx = augmented_rows(n, k)
    L = len(is_s)
    out = np.zeros((L, L), dtype=bool)
    for a in range(L):
        for b in range(L):
            if is_s[a]:
                out[a, b] = (not is_s[b] and idx[b] // k == idx[a]) or (is_s[b] and b == a)
            else:
                i = idx[a]
                if not is_s[b]:
                    out[a, b] = i - W + 1 <= idx[b] <= i
                else:
                    out[a, b] = idx[b] * k + k - 1 < i - W + 1
    return out


MODE_KSA, MODE_SCA, MODE_SWA = 0, 1, 2


def baseline_mask(n: int, k: int, mode: int, C: int = 0, W: int = 0,
                  rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Visibility of the summary-free baselines the report compares KSA with
    (Fig. 3; the Hybrid-SCA / Hybrid-SWA rows of its comparisons), laid over
    the same Eq. 1 sequence so that inputs and outputs keep one layout.

    ``MODE_SCA`` (sliding chunk attention): text t_i, c = floor(i/k), sees
    the text t_{(c-C)k} .. t_i (clamped at 0) and no summary.
    ``MODE_SWA`` (token sliding window of W tokens): text t_i sees the text
    t_{i-W+1} .. t_i (clamped at 0) and no summary.
    ``MODE_KSA`` is :func:`visibility_mask_fast`.
    Summary rows keep the KSA rule in every mode: s_j sees its chunk and
    itself.  These modes are a reading of the baselines (the report gives
    no kernel for them); the window sizes are parameters.
    """
    if mode == MODE_KSA:
        return visibility_mask_fast(n, k, C, rows=rows)
    is_s, idx = augmented_rows(n, k)
    rows = np.arange(len(is_s)) if rows is None else np.asarray(rows, dtype=np.int64)
    qs = is_s[rows][:, None]
    qi = idx[rows][:, None]
    ks = is_s[None, :]
    ki = idx[None, :]
    if mode == MODE_SCA:
        text_q = ~ks & (ki // k >= qi // k - C) & (ki <= qi)
    elif mode == MODE_SWA:
        if W < 1:
            raise ValueError("token window must hold at least the query")
        text_q = ~ks & (ki >= qi - W + 1) & (ki <= qi)
    else:
        raise ValueError(f"unknown mode {mode}")
    summ_q = (~ks & (ki // k == qi)) | (ks & (ki == qi))
    return np.where(qs, summ_q, text_q)


def baseline_pairs_closed_form(n: int, k: int, mode: int, C: int = 0, W: int = 0) -> int:
    """Visible pairs of one head under :func:`baseline_mask`, counted row by
    row from the window sizes: text t_i sees min(floor(i/k), C) k + i mod k + 1
    keys (SCA) or min(i + 1, W) keys (SWA); each summary sees k + 1."""
    M = n // k
    tot = M * (k + 1)
    for i in range(n):
        if mode == MODE_SCA:
            tot += min(i // k, C) * k + i % k + 1
        else:
            tot += min(i + 1, W)
    return tot


def baseline_attention(q: np.ndarray, kx: np.ndarray, v: Optional[np.ndarray], n: int, k: int,
                       mode: int, scale: float, C: int = 0, W: int = 0,
                       rows: Optional[Sequence[int]] = None, dv: Optional[int] = None,
                       row_block: int = 512) -> Tuple[np.ndarray, np.ndarray]:
    """Eq. 10 (masked softmax attention) under :func:`baseline_mask`, in fp64;
    same shapes and conventions as :func:`ksa_attention`."""
    L = augmented_len(n, k)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    if v is None:
        v = kx[..., :dv]
    Hq, Hkv = q.shape[1], kx.shape[1]
    g = Hq // Hkv
    out = np.zeros((len(rows), Hq, v.shape[-1]))
    lse = np.zeros((Hq, len(rows)))
    for b0 in range(0, len(rows), row_block):
        rb = rows[b0:b0 + row_block]
        mask = baseline_mask(n, k, mode, C, W, rows=rb)
        for h in range(Hq):
            o, l_ = attention_masked(q[rb, h], kx[:, h // g], v[:, h // g], mask, scale)
            out[b0:b0 + len(rb), h] = o
            lse[h, b0:b0 + len(rb)] = l_
    return out, lse


def attention_masked_backward(q: np.ndarray, kx: np.ndarray, v: np.ndarray, mask: np.ndarray,
                              scale: float, dout: np.ndarray
                              ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of O = softmax(scale * q k^T + M) v (one head, Eq. 10) with
    respect to q, k and v, given dL/dO = ``dout``, in fp64.

    Straight chain rule: with P the masked softmax, dV = P^T dO and
    dP = dO v^T; each row of P goes through the softmax Jacobian
    diag(p) - p p^T, so dS_i = p_i * dP_i - p_i (p_i . dP_i); then
    dq = scale dS k and dk = scale dS^T q.  Hidden pairs have p = 0 and get
    no gradient.  Returns (dq [R, Dqk], dk [L, Dqk], dv [L, Dv]).
    """
    q = q.astype(np.float64)
    kx = kx.astype(np.float64)
    v = v.astype(np.float64)
    g = dout.astype(np.float64)
    s = np.where(mask, (q @ kx.T) * scale, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    if not np.all(np.isfinite(mx)):
        raise ValueError("a query row sees no key")
    p = np.exp(s - mx)
    p /= p.sum(axis=1, keepdims=True)
    dv = p.T @ g
    dp = g @ v.T
    ds = p * dp - p * (p * dp).sum(axis=1, keepdims=True)
    return scale * (ds @ kx), scale * (ds.T @ q), dv


def attention_backward(q: np.ndarray, kx: np.ndarray, v: np.ndarray, dout: np.ndarray,
                       n: int, k: int, scale: float, mode: int = MODE_KSA, C: int = 0,
                       W: int = 0, row_block: int = 512
                       ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Backward of the prefill attention over the whole augmented sequence
    (Eq. 10 under the KSA mask of Sec. 2.2, or a baseline mask).

    q [L, Hq, Dqk], kx [L, Hkv, Dqk], v [L, Hkv, Dv], dout [L, Hq, Dv].
    Query head h reads kv head h // (Hq/Hkv), so dk and dv of a kv head sum
    the contributions of every query head in its group.  Returns
    (dq [L, Hq, Dqk], dk [L, Hkv, Dqk], dv [L, Hkv, Dv]) in fp64.
    """
    L, Hq, _ = q.shape
    Hkv = kx.shape[1]
    g = Hq // Hkv
    dq = np.zeros(q.shape)
    dk = np.zeros(kx.shape)
    dvv = np.zeros(v.shape)
    for b0 in range(0, L, row_block):
        rb = np.arange(b0, min(L, b0 + row_block))
        mask = baseline_mask(n, k, mode, C, W, rows=rb)
        for h in range(Hq):
            a, b, c = attention_masked_backward(q[rb, h], kx[:, h // g], v[:, h // g], mask,
                                                scale, dout[rb, h])
            dq[rb, h] = a
            dk[:, h // g] += b
            dvv[:, h // g] += c
    return dq, dk, dvv


def attention_backward_rows(q: np.ndarray, kx: np.ndarray, v: np.ndarray, dout: np.ndarray,
                            n: int, k: int, scale: float, rows: Sequence[int], mode: int = MODE_KSA,
                            C: int = 0, W: int = 0, heads: Optional[Sequence[int]] = None
                            ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The terms of :func:`attention_backward` that come from the query rows
    ``rows`` (query heads ``heads``, default all): dq of those rows
    [R, Hq', Dqk] and their contributions to dk, dv of every key
    [L, Hkv, D].  Summed over all rows and heads it is the full backward;
    restricted to the rows that see a key, it is that key's exact gradient.
    """
    rows = np.asarray(rows, dtype=np.int64)
    Hq = q.shape[1]
    Hkv = kx.shape[1]
    g = Hq // Hkv
    heads = list(range(Hq)) if heads is None else list(heads)
    mask = baseline_mask(n, k, mode, C, W, rows=rows)
    dq = np.zeros((len(rows), len(heads), q.shape[2]))
    dk = np.zeros(kx.shape)
    dvv = np.zeros(v.shape)
    for hi, h in enumerate(heads):
        a, b, c = attention_masked_backward(q[rows, h], kx[:, h // g], v[:, h // g], mask, scale,
                                            dout[rows, h])
        dq[:, hi] = a
        dk[:, h // g] += b
        dvv[:, h // g] += c
    return dq, dk, dvv


def visible_pairs_bruteforce(n: int, k: int, C: int,
                             summary_sees_self: bool = True) -> int:
    return int(visibility_mask_fast(n, k, C, summary_sees_self).sum())


# ---------------------------------------------------------------------------
# Masked softmax attention, Eq. (10) (Eq. (9) when the mask is causal)
# ---------------------------------------------------------------------------


def attention_masked(q: np.ndarray, kx: np.ndarray, v: np.ndarray,
                     mask: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """softmax(scale * q k^T + M) v for one head; M = 0 visible, -inf hidden.

    q [R, Dqk], kx [L, Dqk], v [L, Dv], mask bool [R, L].  Returns (O [R, Dv],
    LSE [R]) in fp64; LSE is the natural-log normaliser of the masked scores.
    """
    s = (q.astype(np.float64) @ kx.astype(np.float64).T) * scale
    s = np.where(mask, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    if not np.all(np.isfinite(mx)):
        raise ValueError("a query row sees no key")
    p = np.exp(s - mx)
    den = p.sum(axis=1, keepdims=True)
    o = (p @ v.astype(np.float64)) / den
    return o, (mx[:, 0] + np.log(den[:, 0]))


def ksa_attention(q: np.ndarray, kx: np.ndarray, v: Optional[np.ndarray],
                  n: int, k: int, C: int, scale: float,
                  rows: Optional[Sequence[int]] = None,
                  summary_sees_self: bool = True, dv: Optional[int] = None,
                  row_block: int = 512) -> Tuple[np.ndarray, np.ndarray]:
    """KSA prefill attention over the augmented sequence (Eq. 10).

    q [L, Hq, Dqk], kx [L, Hkv, Dqk], v [L, Hkv, Dv] (or None: V is the first
    ``dv`` columns of K, the absorbed latent form).  Returns O [R, Hq, Dv] and
    LSE [Hq, R] for the requested augmented rows (all rows by default).  The
    dense mask is built a block of rows at a time; each block is a plain
    masked softmax.
    """
    L, Hq, _ = q.shape
    Hkv = kx.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    if v is None:
        v = kx[..., :dv]
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    Dv = v.shape[-1]
    out = np.zeros((len(rows), Hq, Dv))
    lse = np.zeros((Hq, len(rows)))
    for b0 in range(0, len(rows), row_block):
        rr = rows[b0:b0 + row_block]
        m = visibility_mask_fast(n, k, C, summary_sees_self, rows=rr)
        for h in range(Hq):
            o, l_ = attention_masked(q[rr, h], kx[:, h // g], v[:, h // g], m, scale)
            out[b0:b0 + len(rr), h] = o
            lse[h, b0:b0 + len(rr)] = l_
    return out, lse


# ---------------------------------------------------------------------------
# Decode: the same mask row, over the logical augmented history
# ---------------------------------------------------------------------------


def decode_attention(q: np.ndarray, hist_k: np.ndarray, hist_v: Optional[np.ndarray],
                     n_text: int, k: int, C: int, scale: float, kind: str,
                     summary_sees_self: bool = True,
                     dv: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """One decode query against its logical history (never the cache layout).

    ``kind='t'``: the query is text token t_{n_text-1}; the history holds the
    augmented rows 0 .. text_row(n_text-1) (its own K/V last).
    ``kind='s'``: the query is the summary of chunk j = n_text//k - 1 (its
    chunk is complete); the history ends with that summary's row.
    q [Hq, Dqk]; hist_k [A, Hkv, Dqk]; hist_v [A, Hkv, Dv] or None.
    Returns (O [Hq, Dv], LSE [Hq]).
    """
    if kind == "t":
        a = text_row(n_text - 1, k)
        n_log = n_text
    elif kind == "s":
        j = n_text // k - 1
        if j < 0 or n_text % k:
            raise ValueError("summary query needs a just-completed chunk")
        a = summary_row(j, k)
        n_log = n_text + k  # any length that keeps row a inside the sequence
    else:
        raise ValueError(kind)
    A = a + 1
    if hist_k.shape[0] < A:
        raise ValueError("history too short")
    mrow = visibility_mask_fast(n_log, k, C, summary_sees_self, rows=[a])[:, :A]
    Hq = q.shape[0]
    Hkv = hist_k.shape[1]
    g = Hq // Hkv
    if hist_v is None:
        hist_v = hist_k[..., :dv]
    out = np.zeros((Hq, hist_v.shape[-1]))
    lse = np.zeros(Hq)
    for h in range(Hq):
        o, l_ = attention_masked(q[None, h], hist_k[:A, h // g], hist_v[:A, h // g],
                                 mrow, scale)
        out[h] = o[0]
        lse[h] = l_[0]
    return out, lse


def decode_visible_rows(n_text: int, k: int, C: int, kind: str,
                        summary_sees_self: bool = True) -> np.ndarray:
    """Augmented rows a decode query reads (its mask row), sorted."""
    if kind == "t":
        a = text_row(n_text - 1, k)
        n_log = n_text
    else:
        a = summary_row(n_text // k - 1, k)
        n_log = n_text + k
    mrow = visibility_mask_fast(n_log, k, C, summary_sees_self, rows=[a])[0, :a + 1]
    return np.nonzero(mrow)[0]


# ---------------------------------------------------------------------------
# The three-region cache, Sec. 2.3.1 / Fig. 4
# ---------------------------------------------------------------------------


class CacheModel:
    """Physical KSA KV cache of one sequence, one KV head, stepped as in Fig. 4.

    Slot order, left to right: [scratch | current chunk (k) | ring (C*k) |
    summary buffer].  The current chunk fills right to left with its right
    edge against the ring (Fig. 4a/4b); the summary's self-KV goes to the
    scratch slot on the current chunk's left (4c); the finished chunk is
    copied block-wise into ring chunk-slot (m mod C), overwriting the oldest
    (4d); the summary is appended at the right end of the buffer (4e).

    Each slot stores a payload (any Python object: a tag or a row of values);
    ``None`` marks a slot never written.  ``m`` counts committed chunks, ``r``
    the tokens in the current chunk.
    """

    def __init__(self, k: int, C: int, max_summaries: int):
        self.k, self.C, self.cap = k, C, max_summaries
        self.slots: List[object] = [None] * self.num_slots(k, C, max_summaries)
        self.m = 0
        self.r = 0

    @staticmethod
    def num_slots(k: int, C: int, max_summaries: int) -> int:
        return 1 + k + C * k + max_summaries

    # region offsets
    @property
    def cur0(self) -> int:
        return 1

    @property
    def ring0(self) -> int:
        return 1 + self.k

    @property
    def sum0(self) -> int:
        return 1 + self.k + self.C * self.k

    def append_text(self, payload: object) -> None:
        """Fig. 4b: the next free current-chunk slot, right to left."""
        if self.r >= self.k:
            raise RuntimeError("current chunk full: a summary must come first")
        self.slots[self.cur0 + self.k - 1 - self.r] = payload
        self.r += 1

    def append_summary(self, payload: object) -> None:
        """Fig. 4c-4e for the summary of the chunk just completed."""
        if self.r != self.k:
            raise RuntimeError("summary before the chunk is complete")
        if self.m >= self.cap:
            raise RuntimeError("summary buffer full")
        self.slots[0] = payload                                   # 4c
        if self.C > 0:                                            # 4d
            dst = self.ring0 + (self.m % self.C) * self.k
            self.slots[dst:dst + self.k] = self.slots[self.cur0:self.cur0 + self.k]
        self.slots[self.sum0 + self.m] = payload                  # 4e
        self.m += 1
        self.r = 0

    def text_slice(self) -> Tuple[int, int]:
        """(start, length) read by a text query: current fill + ring + distant summaries."""
        start = self.cur0 + self.k - self.r
        length = self.r + min(self.m, self.C) * self.k + max(0, self.m - self.C)
        return start, length

    def summary_slice(self) -> Tuple[int, int]:
        """(start, length) read by the summary query: scratch + the full chunk."""
        return 0, self.k + 1

    def held(self) -> List[object]:
        """Payloads the cache holds for future reads (Fig. 4 regions)."""
        out = list(self.slots[self.cur0 + self.k - self.r:self.cur0 + self.k])
        nring = min(self.m, self.C) * self.k
        out += self.slots[self.ring0:self.ring0 + nring]
        out += self.slots[self.sum0:self.sum0 + self.m]
        return out


def slot_of_row(a: int, m: int, r: int, k: int, C: int) -> int:
    """Physical slot that holds augmented row ``a`` in cache state (m, r).

    Follows the placement rules of :class:`CacheModel` (Fig. 4): summary s_j
    at buffer position j; text token p of a committed chunk c in the window
    at ring chunk-slot (c mod C), position k-1-p (the current chunk is copied
    block-wise and fills right to left); token p of the current chunk at
    current-chunk slot k-1-p.  Raises if the row is not held.
    """
    n_guess = a + 1
    kind, idx = decode_row(a, n_guess + k * 2, k)
    cur0, ring0, sum0 = 1, 1 + k, 1 + k + C * k
    if kind == "s":
        if idx >= m:
            raise KeyError(a)
        return sum0 + idx
    c, p = divmod(idx, k)
    if c == m and p < r:
        return cur0 + k - 1 - p
    if max(0, m - C) <= c < m and C > 0:
        return ring0 + (c % C) * k + (k - 1 - p)
    raise KeyError(a)


def cache_held_rows(m: int, r: int, k: int, C: int) -> List[int]:
    """Augmented rows a cache must hold in state (m committed chunks, r tokens
    in the current chunk): every committed summary, the text of the last
    min(m, C) committed chunks and the current chunk's r tokens."""
    rows = [summary_row(j, k) for j in range(m)]
    for c in range(max(0, m - C), m):
        rows += [text_row(i, k) for i in range(c * k, c * k + k)]
    rows += [text_row(i, k) for i in range(m * k, m * k + r)]
    return sorted(rows)


# ---------------------------------------------------------------------------
# Table 1 accounting
# ---------------------------------------------------------------------------


def per_token_cache_ratio(kind: str, k: int, h: int, d: int, g: int,
                          dc: int, dr: int) -> float:
    """Per-token cache size of a mechanism over MHA's 2*h*d, as n -> inf.

    KSA keeps n/k summaries (the window's w*k text is O(1) in n), so its
    per-token cost is the per-summary cost divided by k (Table 1, Eq. 5-6).
    """
    mha = 2 * h * d
    per = {
        "mha": 2 * h * d,
        "gqa": 2 * g * d,
        "mla": dc + dr,
        "ksa": 2 * h * d / k,
        "ksa+gqa": 2 * g * d / k,
        "ksa+mla": (dc + dr) / k,
    }[kind]
    return per / mha


def visible_pairs_closed_form(M: int, k: int, C: int) -> int:
    """Visible (query, key) pairs for n = M*k, summary seeing itself.

    Summaries: M(k+1).  Text in chunk c at offset p sees min(c, C)*k + p + 1
    text keys and max(0, c-C) summaries.
    """
    if M <= C:
        s1 = M * (M - 1) // 2
        s2 = 0
    else:
        s1 = C * (C - 1) // 2 + (M - C) * C
        s2 = (M - C) * (M - C - 1) // 2
    return M * (k + 1) + M * k * (k + 1) // 2 + k * k * s1 + k * s2


def visible_pairs_general(n: int, k: int, C: int) -> int:
    """Visible pairs for any n (trailing partial chunk allowed), by per-row sums."""
    M = n // k
    tot = M * (k + 1)
    for i in range(n):
        c = i // k
        tot += min(c, C) * k + (i - c * k) + 1 + max(0, c - C)
    return tot
