"""GPU parity of the summary-free baseline modes of the prefill (sliding
chunk attention and token sliding window over the Eq. 1 layout) against the
oracle's baseline masks.  Same tolerances as the KSA prefill: bf16 max abs
<= 2e-2, mean abs <= 2e-3; fp32 max abs <= 1e-4; visibility bit-exact."""
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


def _run(p, mode, W, q, k, v, n, lse=True):
    dev = _dev()
    L = O.augmented_len(n, p.chunk_size)
    ls = torch.empty((q.shape[0], p.num_q_heads, L), dtype=torch.float32, device=dev) if lse else None
    out = ksa.ksa_prefill_attn_mode(p, mode, W, q.to(dev), k.to(dev), v.to(dev), n, lse=ls)
    torch.cuda.synchronize()
    return out, ls


@pytest.mark.parametrize("mode,W", [(O.MODE_SCA, 0), (O.MODE_SWA, 37), (O.MODE_SWA, 1), (O.MODE_SWA, 100000)])
@pytest.mark.parametrize("dtype,D,n,k,C,hq,hkv", [
    (torch.bfloat16, 128, 300, 8, 3, 8, 2),   # MFMA path
    (torch.bfloat16, 128, 333, 4, 5, 4, 4),   # MFMA path, g = 1, ragged tail
    (torch.float32, 64, 200, 8, 2, 4, 2),     # generic path
])
def test_mode_visibility_bit_exact(mode, W, dtype, D, n, k, C, hq, hkv):
    """Q = 0: every visible weight is exactly 1, every hidden one exactly 0;
    V one-hot on the augmented row makes output column d of row a non-zero
    exactly when row (base + d) is visible."""
    L = O.augmented_len(n, k)
    nb = (L + D - 1) // D
    q = torch.zeros((nb, L, hq, D), dtype=dtype)
    kx = ksa_synth.normal((nb, L, hkv, D), dtype, ksa_synth.gen(19))
    v = torch.zeros((nb, L, hkv, D), dtype=dtype)
    for b in range(nb):
        for d in range(D):
            if b * D + d < L:
                v[b, b * D + d, :, d] = 1.0
    p = ksa.Params(k, C, hq, hkv, D, D, dtype)
    print(f"mode {mode} W {W} {dtype} D={D} n={n} k={k} C={C} {hq}/{hkv}", flush=True)
    out, _ = _run(p, mode, W, q, kx, v, n, lse=False)
    o = _np(out)
    got = np.zeros((hq, L, L), dtype=bool)
    for b in range(nb):
        cols = min(D, L - b * D)
        for h in range(hq):
            got[h, :, b * D:b * D + cols] = o[b, :, h, :cols] > 0
    want = O.baseline_mask(n, k, mode, C=C, W=W)
    for h in range(hq):
        np.testing.assert_array_equal(got[h], want)


@pytest.mark.parametrize("mode,W,n,k,C,hq,hkv", [
    (O.MODE_SCA, 0, 1000, 8, 4, 8, 2),
    (O.MODE_SWA, 129, 1000, 8, 4, 8, 2),
    (O.MODE_SWA, 64, 777, 5, 3, 4, 4),
    (O.MODE_SCA, 0, 2100, 8, 16, 16, 4),
])
def test_mode_bf16_values(mode, W, n, k, C, hq, hkv):
    D = 128
    w = ksa_synth.PrefillWorkload("case", 2, n, k, C, hq, hkv, D, D, torch.bfloat16, 1e6, 300 + n)
    L = O.augmented_len(n, k)
    q, kx, v = ksa_synth.prefill_qkv(w, L)
    p = ksa.Params(k, C, hq, hkv, D, D, torch.bfloat16)
    print(f"mode {mode} W {W} n={n} k={k} C={C} {hq}/{hkv}", flush=True)
    out, lse = _run(p, mode, W, q, kx, v, n)
    for b in range(2):
        ref, rl = O.baseline_attention(q[b].double().numpy(), kx[b].double().numpy(), v[b].double().numpy(),
                                       n, k, mode, p.scale, C=C, W=W)
        e = np.abs(_np(out[b]) - ref)
        print(f"  b{b}: max {e.max():.3e} mean {e.mean():.3e}", flush=True)
        assert e.max() <= 2e-2 and e.mean() <= 2e-3
        assert np.abs(_np(lse[b]) - rl).max() <= 2e-2


def test_mode_fp32_values_generic():
    n, k, C, hq, hkv, D, W = 300, 8, 2, 4, 2, 64, 50
    w = ksa_synth.PrefillWorkload("case", 1, n, k, C, hq, hkv, D, D, torch.float32, 1e6, 77)
    L = O.augmented_len(n, k)
    q, kx, v = ksa_synth.prefill_qkv(w, L)
    p = ksa.Params(k, C, hq, hkv, D, D, torch.float32)
    for mode in (O.MODE_SCA, O.MODE_SWA):
        out, lse = _run(p, mode, W, q, kx, v, n)
        ref, rl = O.baseline_attention(q[0].double().numpy(), kx[0].double().numpy(), v[0].double().numpy(),
                                       n, k, mode, p.scale, C=C, W=W)
        assert np.abs(_np(out[0]) - ref).max() <= 1e-4
        assert np.abs(_np(lse[0]) - rl).max() <= 1e-4


def test_ksa_mode_equals_plain_prefill():
    n, k, C, hq, hkv, D = 900, 8, 6, 8, 2, 128
    w = ksa_synth.PrefillWorkload("case", 1, n, k, C, hq, hkv, D, D, torch.bfloat16, 1e6, 5)
    L = O.augmented_len(n, k)
    q, kx, v = ksa_synth.prefill_qkv(w, L)
    p = ksa.Params(k, C, hq, hkv, D, D, torch.bfloat16)
    dev = _dev()
    a = ksa.ksa_prefill_attn(p, q.to(dev), kx.to(dev), v.to(dev), n)
    b, _ = _run(p, O.MODE_KSA, 0, q, kx, v, n, lse=False)
    assert torch.equal(a, b)
