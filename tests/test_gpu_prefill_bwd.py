"""GPU parity of the prefill backward (dq, dk, dv through the C ABI)
against the oracle's fp64 gradient of Eq. 10 under the same masks.

The GPU backward consumes its own forward's output and normaliser, as a
training step would.  Tolerances: fp32 |err| <= 1e-4 (1 + |ref|); bf16
|err| <= 2e-2 (1 + |ref|) element-wise, mean |err| <= 2e-3 (1 + mean |ref|)
(fp32: 1e-5) and relative L2 <= 1.5e-2 per tensor
(bf16 inputs and outputs, fp32 accumulation, P and dS rounded to bf16 before
their products on the MFMA path)."""
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


def _gpu_bwd(p, mode, W, q, kx, v, g, n):
    dev = _dev()
    L = O.augmented_len(n, p.chunk_size)
    qd, kd, vd, gd = q.to(dev), kx.to(dev), v.to(dev), g.to(dev)
    lse = torch.empty((q.shape[0], p.num_q_heads, L), dtype=torch.float32, device=dev)
    out = ksa.ksa_prefill_attn_mode(p, mode, W, qd, kd, vd, n, lse=lse)
    dq, dk, dv = ksa.ksa_prefill_attn_bwd(p, mode, W, qd, kd, vd, out, gd, lse, n)
    torch.cuda.synchronize()
    return dq, dk, dv


def _compare(name, got, ref, bf16):
    e = np.abs(got - ref)
    tol = 2e-2 if bf16 else 1e-4
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    print(f"  {name}: max {e.max():.3e} mean {e.mean():.3e} rel-l2 {rel:.3e} |ref|max {np.abs(ref).max():.2f} "
          f"|ref|mean {np.abs(ref).mean():.3e}", flush=True)
    assert np.all(e <= tol * (1 + np.abs(ref))), name
    # the mean error, on the same relative footing (the output bound's 2e-3
    # for bf16; fp32 stays 10x under its own element bound)
    assert e.mean() <= (2e-3 if bf16 else 1e-5) * (1 + np.abs(ref).mean()), name
    # a relative error needs a reference away from zero: rows that see a
    # single key have dS = P (dP - Delta) = 0 exactly, so dq and dk vanish
    if bf16 and np.linalg.norm(ref) > 1e-3:
        assert rel <= 1.5e-2, name


def _case(dtype, D, n, k, C, hq, hkv, mode, W, batch, seed):
    w = ksa_synth.PrefillWorkload("case", batch, n, k, C, hq, hkv, D, D, dtype, 1e6, seed)
    L = O.augmented_len(n, k)
    q, kx, v = ksa_synth.prefill_qkv(w, L)
    g = ksa_synth.normal((batch, L, hq, D), dtype, ksa_synth.gen(seed + 1))
    p = ksa.Params(k, C, hq, hkv, D, D, dtype)
    print(f"bwd mode {mode} W {W} {dtype} D={D} n={n} k={k} C={C} {hq}/{hkv} B={batch}", flush=True)
    dq, dk, dv = _gpu_bwd(p, mode, W, q, kx, v, g, n)
    for b in range(batch):
        rq, rk, rv = O.attention_backward(q[b].double().numpy(), kx[b].double().numpy(), v[b].double().numpy(),
                                          g[b].double().numpy(), n, k, p.scale, mode=mode, C=C, W=W)
        bf = dtype == torch.bfloat16
        _compare(f"b{b} dq", _np(dq[b]), rq, bf)
        _compare(f"b{b} dk", _np(dk[b]), rk, bf)
        _compare(f"b{b} dv", _np(dv[b]), rv, bf)


@pytest.mark.parametrize("mode,W", [(O.MODE_KSA, 0), (O.MODE_SCA, 0), (O.MODE_SWA, 29)])
def test_bwd_fp32_generic(mode, W):
    _case(torch.float32, 64, 203, 8, 2, 4, 2, mode, W, 2, 41 + mode)


def test_bwd_fp32_generic_k1_wide_window():
    _case(torch.float32, 32, 70, 1, 100, 2, 1, O.MODE_KSA, 0, 1, 7)


def test_bwd_bf16_generic_d64():
    _case(torch.bfloat16, 64, 260, 4, 3, 4, 4, O.MODE_KSA, 0, 1, 9)


# bf16, Dqk = Dv = 128: the MFMA dq / dkdv / summary-key kernels.  Cases span
# several 64-row tiles and 128-key workgroups, ragged tails (n % k, n % 64),
# the group sizes 1, 2, 4, chunk sizes 1, 5, 8, every mode, and a sequence
# long enough that the summary keys are cut into several query segments.
@pytest.mark.parametrize("n,k,C,hq,hkv,mode,W,batch", [
    (300, 8, 3, 8, 2, O.MODE_KSA, 0, 1),
    (333, 4, 5, 4, 4, O.MODE_KSA, 0, 2),
    (700, 5, 2, 4, 2, O.MODE_KSA, 0, 1),
    (400, 1, 20, 4, 4, O.MODE_KSA, 0, 1),
    (1000, 8, 4, 8, 2, O.MODE_SCA, 0, 1),
    (1000, 8, 4, 8, 2, O.MODE_SWA, 129, 1),
    (2100, 8, 16, 16, 4, O.MODE_KSA, 0, 1),
    (5000, 8, 4, 8, 2, O.MODE_KSA, 0, 1),
    (1, 8, 4, 4, 1, O.MODE_KSA, 0, 1),      # one text token
    (1, 1, 0, 4, 1, O.MODE_KSA, 0, 1),      # one token completing a chunk (text row + summary)
    (8, 8, 0, 4, 2, O.MODE_KSA, 0, 1),      # exactly one chunk
    (65, 64, 1, 4, 2, O.MODE_KSA, 0, 1),    # chunk wider than a key tile
])
def test_bwd_bf16_mfma(n, k, C, hq, hkv, mode, W, batch):
    _case(torch.bfloat16, 128, n, k, C, hq, hkv, mode, W, batch, 1000 + n + mode)
