"""The prefill backward at full size: the 32K-token, 32/8-head, d = 128
workload the benchmark times, in the same launch configuration.

The oracle cannot form the whole gradient at this size, so it checks what it
can compute exactly: dq of sampled query rows (each row's own softmax), and
dk, dv of sampled keys from every query row that sees them (text keys early,
late and mid-sequence; summary keys whose readers span two of the kernel's
query segments and the last one).  Every summary key, including those read
by tens of thousands of queries, is covered by the conservation laws of
softmax attention: the key gradients of a kv head sum to zero and the value
gradients sum to the output gradients of its query heads."""
import numpy as np
import pytest
import torch

import ksa_synth
from oracle import ksa_oracle as O

pytestmark = pytest.mark.gpu

ksa = pytest.importorskip("kv_cache_compression_amd")


def _np(t):
    return t.detach().float().cpu().double().numpy()


def _close(name, got, ref):
    e = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    print(f"  {name}: max {e.max():.3e} mean {e.mean():.3e} rel-l2 {rel:.3e} |ref|mean {np.abs(ref).mean():.3e}",
          flush=True)
    assert np.all(e <= 2e-2 * (1 + np.abs(ref))), name
    assert e.mean() <= 2e-3 * (1 + np.abs(ref).mean()), name
    assert rel <= 1.5e-2, name


@pytest.fixture(scope="module")
def full_case():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = ksa_synth.PREFILL_32K
    dev = torch.device("cuda:0")
    L = O.augmented_len(w.n_text, w.chunk)
    q, kx, v = ksa_synth.prefill_qkv(w, L)
    g = ksa_synth.normal((1, L, w.hq, w.dv), w.dtype, ksa_synth.gen(w.seed + 7))
    p = ksa.Params(w.chunk, w.window, w.hq, w.hkv, w.dqk, w.dv, w.dtype)
    qd, kd, vd, gd = q.to(dev), kx.to(dev), v.to(dev), g.to(dev)
    lse = torch.empty((1, w.hq, L), dtype=torch.float32, device=dev)
    print(f"32K backward: L={L}", flush=True)
    out = ksa.ksa_prefill_attn(p, qd, kd, vd, w.n_text, lse=lse)
    dq, dk, dv = ksa.ksa_prefill_attn_bwd(p, ksa.MODE_KSA, 0, qd, kd, vd, out, gd, lse, w.n_text)
    torch.cuda.synchronize()
    arrs = [x[0].double().numpy() for x in (q, kx, v, g)]
    return w, p, L, arrs, (_np(dq[0]), _np(dk[0]), _np(dv[0]))


def test_full_dq_sampled_rows(full_case):
    w, p, L, (q, kx, v, g), (dq, _, _) = full_case
    n, k = w.n_text, w.chunk
    rows = [O.text_row(i, k) for i in (0, 7, 8, 520, 12345, n - 1)] + [O.summary_row(0, k),
                                                                       O.summary_row(n // k - 1, k)]
    ref, _, _ = O.attention_backward_rows(q, kx, v, g, n, k, p.scale, rows, C=w.window)
    _close("dq rows", dq[rows], ref)


@pytest.mark.parametrize("kind,idx", [("t", 5000), ("t", 32768 - 600), ("t", 32767),
                                      ("s", 3770), ("s", 4096 - 64 - 2)])
def test_full_dkdv_sampled_keys(full_case, kind, idx):
    w, p, L, (q, kx, v, g), (_, dk, dv) = full_case
    n, k, C = w.n_text, w.chunk, w.window
    if kind == "t":
        r = O.text_row(idx, k)
        # readers: text rows up to (c+C+1)k - 1 and the summary of chunk c,
        # which follows its chunk's text rows
        last = min(L - 1, O.text_row(min(n - 1, idx + (C + 2) * k), k) + k + 1)
        rows = np.arange(r, last + 1)
    else:
        r = O.summary_row(idx, k)
        rows = np.arange(r, L)
    for kvh in (0, w.hkv - 1):
        heads = range(kvh * (w.hq // w.hkv), (kvh + 1) * (w.hq // w.hkv))
        _, rk, rv = O.attention_backward_rows(q, kx, v, g, n, k, p.scale, rows, C=C, heads=heads)
        print(f"{kind}{idx} kv head {kvh}: {len(rows)} query rows", flush=True)
        _close(f"dk {kind}{idx}", dk[r, kvh], rk[r, kvh])
        _close(f"dv {kind}{idx}", dv[r, kvh], rv[r, kvh])


def test_full_conservation(full_case):
    w, p, L, (_, _, _, g), (_, dk, dv) = full_case
    grp = w.hq // w.hkv
    for kvh in range(w.hkv):
        sk = dk[:, kvh].sum(0)
        sv = dv[:, kvh].sum(0)
        gv = g[:, kvh * grp:(kvh + 1) * grp].sum((0, 1))
        # bf16 outputs: each row's rounding is at most 2^-9 of it, and the
        # errors of 36864 rows add up like a random walk
        tol_k = 6 * np.sqrt(L) * 2.0 ** -9 * np.sqrt((dk[:, kvh] ** 2).mean(0)) + 1e-3
        tol_v = 6 * np.sqrt(L) * 2.0 ** -9 * np.sqrt((dv[:, kvh] ** 2).mean(0)) + 1e-3
        print(f"kv head {kvh}: |sum dk| max {np.abs(sk).max():.3e}  |sum dv - sum dout| max "
              f"{np.abs(sv - gv).max():.3e}  (|sum dout| max {np.abs(gv).max():.1f})", flush=True)
        assert np.all(np.abs(sk) <= tol_k)
        assert np.all(np.abs(sv - gv) <= tol_v)
