"""Prefill with the query's rotary embedding applied as the kernel loads
each query row (ksa_prefill_attn_qrope), against the oracle: O.rope_rotate
of queries and keys by the report's Sec. 2.2.1 position ids
(O.position_ids: text index for text, the chunk's last text token for a
summary), then O.ksa_attention.  The keys are rotated beforehand by the
library's own pass (the cache keeps post-RoPE keys); the oracle rotates the
un-rounded keys in fp64.

  - tiny fp32 configuration (generic kernel): max abs <= 1e-4 on outputs
    and LSE;
  - bf16 MFMA shapes with ragged tails and g = 1, 2, 4, 8: max abs <= 2e-2,
    mean abs <= 2e-3 (the bf16 prefill bounds);
  - the 32768-token workload (positions up to 32767) on sampled rows;
  - q is not written.
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
    return t.float().cpu().double().numpy()


def _run(w, p, q, k, v, lse=True):
    """Un-rotated q to the fused call; k rotated by the library's pass."""
    dev = _dev()
    L = O.augmented_len(w.n_text, w.chunk)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    q_before = qd.clone()
    ksa.ksa_rope_augmented(p, kd, w.n_text, w.rope_theta)
    ls = torch.empty((q.shape[0], w.hq, L), dtype=torch.float32, device=dev) if lse else None
    out = ksa.ksa_prefill_attn_qrope(p, qd, kd, vd, w.n_text, w.rope_theta, lse=ls)
    torch.cuda.synchronize()
    assert torch.equal(qd, q_before), "q was written"
    return out, ls


def test_tiny_config_fp32_fused_rope():
    """batch 1, 512 text tokens, k=8, w=4, 4/2 heads, d=64, fp32, theta 1e6."""
    w = ksa_synth.TINY_PREFILL
    L = O.augmented_len(w.n_text, w.chunk)
    q, k, v = ksa_synth.prefill_qkv(w, L)
    p = ksa.Params(w.chunk, w.window, w.hq, w.hkv, w.dqk, w.dv, w.dtype)
    out, lse = _run(w, p, q, k, v)
    pos = O.position_ids(w.n_text, w.chunk)
    qr = O.rope_rotate(q[0].double().numpy(), pos, w.rope_theta)
    kr = O.rope_rotate(k[0].double().numpy(), pos, w.rope_theta)
    ref, rl = O.ksa_attention(qr, kr, v[0].double().numpy(), w.n_text, w.chunk, w.window, p.scale)
    assert np.abs(_np(out[0]) - ref).max() <= 1e-4
    assert np.abs(_np(lse[0]) - rl).max() <= 1e-4


# (n, k, C, Hq, Hkv, theta): ragged tails, g = 1, 2, 4, 8, two bases
CASES = [
    (1000, 8, 4, 8, 2, 1e6),
    (777, 5, 3, 4, 4, 1e4),
    (2100, 8, 16, 16, 4, 1e6),
    (301, 3, 0, 2, 1, 5e5),
    (33, 8, 1, 4, 1, 1e4),
    (600, 16, 3, 8, 2, 1e6),   # k > 8: the summary rows' rotation on the one-summary-per-wave path
]


@pytest.mark.parametrize("n,k,C,hq,hkv,theta", CASES)
def test_bf16_mfma_fused_rope_parity(n, k, C, hq, hkv, theta):
    D = 128
    w = ksa_synth.PrefillWorkload("qrope", 2, n, k, C, hq, hkv, D, D, torch.bfloat16, theta, 300 + n)
    L = O.augmented_len(n, k)
    q, kx, v = ksa_synth.prefill_qkv(w, L)
    p = ksa.Params(k, C, hq, hkv, D, D, torch.bfloat16)
    print(f"qrope case n={n} k={k} C={C} hq={hq} hkv={hkv} theta={theta}", flush=True)
    out, lse = _run(w, p, q, kx, v)
    pos = O.position_ids(n, k)
    for b in range(2):
        qr = O.rope_rotate(q[b].double().numpy(), pos, theta)
        kr = O.rope_rotate(kx[b].double().numpy(), pos, theta)
        ref, rl = O.ksa_attention(qr, kr, v[b].double().numpy(), n, k, C, p.scale)
        e = np.abs(_np(out[b]) - ref)
        assert e.max() <= 2e-2 and e.mean() <= 2e-3, (b, e.max(), e.mean())
        assert np.abs(_np(lse[b]) - rl).max() <= 2e-2


def test_fused_rope_32k_sampled_rows():
    """The 32768-token, 32/8-head workload in the launch configuration the
    benchmark times; rows at both ends, around summaries, and random."""
    dev = _dev()
    w = ksa_synth.PREFILL_32K
    L = O.augmented_len(w.n_text, w.chunk)
    q, k, v = ksa_synth.prefill_qkv(w, L)
    p = ksa.Params(w.chunk, w.window, w.hq, w.hkv, w.dqk, w.dv, w.dtype)
    out, _ = _run(w, p, q, k, v, lse=False)
    rng = np.random.default_rng(21)
    rows = sorted(set([0, 1, 8, 9, 585, 17999, L - 10, L - 2, L - 1] + list(rng.integers(0, L, 24))))
    pos = O.position_ids(w.n_text, w.chunk)
    kr = O.rope_rotate(k[0].double().numpy(), pos, w.rope_theta)
    qfull = np.zeros((L,) + tuple(q.shape[2:]))
    qfull[rows] = O.rope_rotate(q[0, rows].double().numpy(), pos[rows], w.rope_theta)
    ref, _ = O.ksa_attention(qfull, kr, v[0].double().numpy(), w.n_text, w.chunk, w.window, p.scale, rows=rows)
    e = np.abs(_np(out[0, rows]) - ref)
    print(f"fused rope 32K: max {e.max():.3e} mean {e.mean():.3e}", flush=True)
    assert e.max() <= 2e-2 and e.mean() <= 2e-3, (e.max(), e.mean())
    del out
    torch.cuda.empty_cache()
