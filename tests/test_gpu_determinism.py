"""Two launches of the same call on the same inputs are bit-identical.

No kernel of the path accumulates through atomics or depends on the order
in which workgroups finish: tile schedules are functions of the shapes, the
split-K and range cuts are functions of the cache states, and every merge
reads its partials in a fixed order.  Checked for the one-shot prefill
(MFMA and generic), the chunked prefill, both split-K decodes, the
allocation-free decode and the backward, at sizes that launch many
workgroups.
"""
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


def _twice(fn):
    a = [t.clone() for t in fn()]
    b = [t.clone() for t in fn()]
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    return a


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_prefill_forward_and_backward_repeat_bit_exactly(dtype, D):
    dev = _dev()
    n, k, C, hq, hkv = 3001, 8, 16, 8, 2
    L = O.augmented_len(n, k)
    w = ksa_synth.PrefillWorkload("det", 1, n, k, C, hq, hkv, D, D, dtype, 1e6, 71)
    q, kx, v = (t.to(dev) for t in ksa_synth.prefill_qkv(w, L))
    g = ksa_synth.normal((1, L, hq, D), dtype, ksa_synth.gen(72)).to(dev)
    p = ksa.Params(k, C, hq, hkv, D, D, dtype)
    print(f"determinism prefill {dtype} D={D}", flush=True)

    def fwd():
        lse = torch.empty((1, hq, L), dtype=torch.float32, device=dev)
        out = ksa.ksa_prefill_attn(p, q, kx, v, n, lse=lse)
        return out, lse

    out, lse = _twice(fwd)
    _twice(lambda: ksa.ksa_prefill_attn_bwd(p, ksa.MODE_KSA, 0, q, kx, v, out, g, lse, n))


def test_chunked_prefill_repeats_bit_exactly():
    dev = _dev()
    n, k, C, hq, hkv, D = 2500, 8, 8, 8, 2, 128
    L = O.augmented_len(n, k)
    w = ksa_synth.PrefillWorkload("detc", 1, n, k, C, hq, hkv, D, D, torch.bfloat16, 1e6, 73)
    q, kx, v = (t[0].to(dev) for t in ksa_synth.prefill_qkv(w, L))
    p = ksa.Params(k, C, hq, hkv, D, D, torch.bfloat16)

    def run():
        cache = ksa.Cache(p, 1, n // k + 1, device=dev)
        outs = []
        for a0, a1 in ((0, 900), (900, 1700), (1700, L)):
            seg = torch.tensor([0, a1 - a0], dtype=torch.int64, device=dev)
            outs.append(ksa.ksa_prefill_chunk(cache, seg, a1 - a0, q[a0:a1], kx[a0:a1], v[a0:a1]))
            ksa.ksa_cache_append_rows(cache, seg, a1 - a0, kx[a0:a1], v[a0:a1])
        return outs + [cache.k, cache.v, cache.state]

    _twice(run)


@pytest.mark.parametrize("shape", ["gqa", "mla"])
def test_split_k_decodes_repeat_bit_exactly(shape):
    dev = _dev()
    w = ksa_synth.DECODE_GQA if shape == "gqa" else ksa_synth.DECODE_MLA
    B = 16
    hist = ksa_synth.decode_histories(w)[:B]
    hist = [min(n, 40001) for n in hist]
    p = ksa.Params(w.chunk, w.window, w.hq, w.hkv, w.dqk, w.dv, w.dtype, v_is_k_prefix=w.v_is_k_prefix)
    cache = ksa.Cache(p, B, max(hist) // w.chunk + 1, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(74)
    cache.k.normal_(generator=gen)
    if cache.v is not None:
        cache.v.normal_(generator=gen)
    st = torch.zeros((B, 4), dtype=torch.int32)
    for b, n in enumerate(hist):
        m = (n - 1) // w.chunk
        st[b, 0], st[b, 1] = m, n - m * w.chunk
    cache.state.copy_(st.to(dev))
    q = ksa_synth.decode_query(w)[:B].contiguous().to(dev)
    kind = torch.zeros((B,), dtype=torch.int32, device=dev)
    print(f"determinism decode {shape}", flush=True)

    def run():
        lse = torch.empty((B, w.hq), dtype=torch.float32, device=dev)
        return ksa.ksa_decode_attn(cache, q, kind, lse=lse), lse

    a = _twice(run)
    # the allocation-free entry point: the same kernels, the same bits
    lse2 = torch.empty((B, w.hq), dtype=torch.float32, device=dev)
    out2 = ksa.ksa_decode_attn_noalloc(cache, q, kind, lse=lse2)
    torch.cuda.synchronize()
    assert torch.equal(a[0], out2) and torch.equal(a[1], lse2)
