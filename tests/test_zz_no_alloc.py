"""ksa_decode_attn_noalloc (the allocation-free decode) against
ksa_decode_attn with a caller workspace, through the C ABI.

Both run the same kernels with the same split layout, so outputs and
normalisers must be bit-identical.  Two calls in a row on each split-K path
(GQA d = 128 and absorbed MLA), the second with a smaller batch and shorter
histories, so that the second call reads a scratch array that still holds
the first call's partials.  A shape whose partials exceed the scratch array
is refused before anything is launched.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

ksa = pytest.importorskip("kv_cache_compression_amd")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _cache(p, hist, seed, dev):
    """A cache whose sequence b holds hist[b] text tokens (query included):
    m complete chunks, r = hist - m k in the current chunk."""
    k = p.chunk_size
    B = len(hist)
    c = ksa.Cache(p, B, max(hist) // k + 1, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    c.k.normal_(generator=g)
    if c.v is not None:
        c.v.normal_(generator=g)
    st = torch.zeros((B, 4), dtype=torch.int32)
    for b, n in enumerate(hist):
        m = (n - 1) // k
        st[b, 0] = m
        st[b, 1] = n - m * k
    c.state.copy_(st.to(dev))
    return c


def _both(c, q, kind):
    B, hq = q.shape[0], q.shape[1]
    dev = q.device
    l1 = torch.empty((B, hq), dtype=torch.float32, device=dev)
    l2 = torch.full((B, hq), 5.0, dtype=torch.float32, device=dev)
    o1 = ksa.ksa_decode_attn(c, q, kind, lse=l1)
    o2 = torch.full_like(o1, 3.0)
    ksa.ksa_decode_attn_noalloc(c, q, kind, out=o2, lse=l2)
    torch.cuda.synchronize()
    return o1, l1, o2, l2


@pytest.mark.parametrize("shape", ["gqa", "mla"])
def test_noalloc_matches_workspace_path(shape):
    dev = _dev()
    if shape == "gqa":
        p = ksa.Params(8, 64, 32, 8, 128, 128, torch.bfloat16)
        calls = [[20001, 19003, 20007, 18005, 20000, 17777, 20008, 19999], [3001, 2505, 4099]]
    else:
        p = ksa.Params(8, 64, 128, 1, 576, 512, torch.bfloat16, v_is_k_prefix=True)
        calls = [[40003, 16385, 29001, 33333, 17000, 38005], [9001, 12003]]
    for i, hist in enumerate(calls):
        c = _cache(p, hist, 40 + i, dev)
        B = len(hist)
        g = torch.Generator().manual_seed(50 + i)
        q = torch.randn((B, p.num_q_heads, p.head_dim_qk), generator=g).to(torch.bfloat16).to(dev)
        kind = torch.zeros((B,), dtype=torch.int32, device=dev)
        if B > 2:
            kind[1] = -1       # a skipped sequence: its output rows stay as they were
        print(f"no-alloc {shape} call {i}: batch {B}", flush=True)
        o1, l1, o2, l2 = _both(c, q, kind)
        run = kind.cpu().numpy() >= 0
        assert torch.equal(o1[run], o2[run]) and torch.equal(l1[run], l2[run])
        assert bool((o2[~run] == 3.0).all()) and bool((l2[~run] == 5.0).all())
        assert torch.isfinite(o2[run].float()).all()
        assert ksa.ksa_cache_read_errors(c) == [0] * B


def test_noalloc_refuses_partials_beyond_the_scratch():
    dev = _dev()
    # absorbed MLA: one partial record per (work item, head); 1024 sequences
    # need about (CUs + 1024) x 128 x 1 KB, above the 128 MiB array
    p = ksa.Params(8, 0, 128, 1, 576, 512, torch.bfloat16, v_is_k_prefix=True)
    c = ksa.Cache(p, 1024, 1, device=dev)
    q = torch.zeros((1024, 128, 576), dtype=torch.bfloat16, device=dev)
    kind = torch.zeros((1024,), dtype=torch.int32, device=dev)
    with pytest.raises(ksa.KsaError) as ei:
        ksa.ksa_decode_attn_noalloc(c, q, kind)
    assert ei.value.status == 4  # KSA_STATUS_WORKSPACE_TOO_SMALL
    # a small call afterwards still works
    p2 = ksa.Params(8, 4, 8, 2, 128, 128, torch.bfloat16)
    c2 = _cache(p2, [700, 333], 61, dev)
    q2 = torch.randn((2, 8, 128), generator=torch.Generator().manual_seed(62)).to(torch.bfloat16).to(dev)
    kind2 = torch.zeros((2,), dtype=torch.int32, device=dev)
    o1, l1, o2, l2 = _both(c2, q2, kind2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
