"""Full-size parity of the paths the benchmark times beside the one-shot
prefill, in the launch configuration it times them, on sampled rows the
oracle computes one by one:

  - the RoPE pre-pass of the 32768-token workload;
  - the 32768-token, 32/8-head workload fed through the cache in 8 segments
    (ksa_prefill_chunk + ksa_cache_append_rows per segment);
  - the same workload under the two summary-free baselines (sliding chunks,
    and a token window of w k = 512 tokens);
  - the absorbed-MLA prefill, 8192 tokens, 128 heads over one 576/512 latent
    head.

Tolerances are those of the bf16 prefill: max abs <= 2e-2, mean abs <= 2e-3.
"""
import math

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


def _check(got, ref, what):
    e = np.abs(got - ref)
    print(f"{what}: max {e.max():.3e} mean {e.mean():.3e}", flush=True)
    assert e.max() <= 2e-2 and e.mean() <= 2e-3, (what, e.max(), e.mean())


@pytest.fixture(scope="module")
def w32k():
    """The 32K workload after the RoPE pre-pass, on the GPU, with the
    oracle's rotated keys and the sampled rows' rotated queries."""
    dev = _dev()
    w = ksa_synth.PREFILL_32K
    L = O.augmented_len(w.n_text, w.chunk)
    q, k, v = ksa_synth.prefill_qkv(w, L)
    p = ksa.Params(w.chunk, w.window, w.hq, w.hkv, w.dqk, w.dv, w.dtype)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    ksa.ksa_rope_augmented(p, qd, w.n_text, w.rope_theta)
    ksa.ksa_rope_augmented(p, kd, w.n_text, w.rope_theta)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    # both ends, the first summary, segment boundaries of the 8-way split, random
    bounds = [L * i // 8 for i in range(9)]
    edge = [b + d for b in bounds[1:-1] for d in (-1, 0, 1)]
    rows = sorted(set([0, 1, 8, 9, 585, L - 2, L - 1] + edge + list(rng.integers(0, L, 24))))
    pos = O.position_ids(w.n_text, w.chunk)
    kr = O.rope_rotate(k[0].double().numpy(), pos, w.rope_theta)
    qfull = np.zeros((L,) + tuple(q.shape[2:]))
    qfull[rows] = O.rope_rotate(q[0, rows].double().numpy(), pos[rows], w.rope_theta)
    yield dict(w=w, L=L, p=p, qd=qd, kd=kd, vd=vd, rows=rows, q=qfull, k=kr, v=v[0].double().numpy(),
               bounds=bounds)
    del qd, kd, vd
    torch.cuda.empty_cache()


def test_rope_pre_pass_32k_sampled_rows(w32k):
    """The RoPE pre-pass over the 32K augmented Q and K (position ids of the
    summary rows included) against the oracle's rotation, on sampled rows."""
    rows = w32k["rows"]
    for name, got, ref in (("q", w32k["qd"], w32k["q"]), ("k", w32k["kd"], w32k["k"])):
        e = np.abs(got[0, rows].float().cpu().double().numpy() - ref[rows])
        print(f"rope {name}: max {e.max():.3e} mean {e.mean():.3e}", flush=True)
        assert e.max() <= 2e-2 and e.mean() <= 2e-3, (name, e.max(), e.mean())


def test_chunked_32k_in_8_segments_sampled_rows(w32k):
    w, L, p, rows = w32k["w"], w32k["L"], w32k["p"], w32k["rows"]
    dev = w32k["qd"].device
    cache = ksa.Cache(p, 1, w.n_text // w.chunk + 1, device=dev)
    ksa.ksa_cache_reset(cache)
    out = torch.empty((L, w.hq, w.dv), dtype=w.dtype, device=dev)
    bounds = w32k["bounds"]
    for i in range(8):
        a, b = bounds[i], bounds[i + 1]
        seg = torch.tensor([0, b - a], dtype=torch.int64, device=dev)
        k_ = w32k["kd"][0, a:b].contiguous()
        v_ = w32k["vd"][0, a:b].contiguous()
        ksa.ksa_prefill_chunk(cache, seg, b - a, w32k["qd"][0, a:b].contiguous(), k_, v_, out=out[a:b])
        ksa.ksa_cache_append_rows(cache, seg, b - a, k_, v_)
    torch.cuda.synchronize()
    assert ksa.ksa_cache_read_errors(cache) == [0]
    st = cache.state.cpu()
    assert st[0, 0].item() == L // (w.chunk + 1) and st[0, 1].item() == L % (w.chunk + 1)
    ref, _ = O.ksa_attention(w32k["q"], w32k["k"], w32k["v"], w.n_text, w.chunk, w.window, p.scale, rows=rows)
    _check(out[rows].float().cpu().double().numpy(), ref, "chunked 32K, 8 segments")


@pytest.mark.parametrize("mode,W", [(O.MODE_SCA, 0), (O.MODE_SWA, 512)], ids=["sliding_chunks", "window_512"])
def test_baselines_32k_sampled_rows(w32k, mode, W):
    w, p, rows = w32k["w"], w32k["p"], w32k["rows"]
    kmode = ksa.MODE_SCA if mode == O.MODE_SCA else ksa.MODE_SWA
    out = ksa.ksa_prefill_attn_mode(p, kmode, W, w32k["qd"], w32k["kd"], w32k["vd"], w.n_text)
    torch.cuda.synchronize()
    ref, _ = O.baseline_attention(w32k["q"], w32k["k"], w32k["v"], w.n_text, w.chunk, mode, p.scale,
                                  C=w.window, W=W, rows=rows)
    _check(out[0, rows].float().cpu().double().numpy(), ref, f"baseline mode {mode} W {W}, 32K")


def test_mla_prefill_8k_128_heads_sampled_rows():
    dev = _dev()
    w = ksa_synth.PREFILL_MLA_8K
    L = O.augmented_len(w.n_text, w.chunk)
    # keys drawn as the benchmark draws them; queries drawn on the device
    # (seeded torch generator) and the sampled rows copied back for the oracle
    k = ksa_synth.normal((w.batch, L, w.hkv, w.dqk), w.dtype, ksa_synth.gen(w.seed + 1))
    gd = torch.Generator(device=dev)
    gd.manual_seed(w.seed)
    qd = torch.randn((w.batch, L, w.hq, w.dqk), generator=gd, device=dev, dtype=torch.float32).to(w.dtype)
    p = ksa.Params(w.chunk, w.window, w.hq, w.hkv, w.dqk, w.dv, w.dtype, v_is_k_prefix=True)
    lse = torch.empty((w.batch, w.hq, L), dtype=torch.float32, device=dev)
    out = ksa.ksa_prefill_attn(p, qd, k.to(dev), None, w.n_text, lse=lse)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = sorted(set([0, 8, 9, 584, 585, L - 1] + list(rng.integers(0, L, 6))))
    qn = np.zeros((L, w.hq, w.dqk))
    qn[rows] = qd[0, rows].float().cpu().double().numpy()
    ref, ref_lse = O.ksa_attention(qn, k[0].double().numpy(), None, w.n_text, w.chunk, w.window,
                                   1.0 / math.sqrt(w.dqk), rows=rows, dv=w.dv)
    _check(out[0, rows].float().cpu().double().numpy(), ref, "absorbed-MLA prefill 8K x 128 heads")
    lerr = np.abs(lse[0][:, rows].cpu().double().numpy() - ref_lse)   # both [Hq, rows]
    assert lerr.max() <= 2e-2, lerr.max()
