"""Host-side checks of the C ABI library (no GPU needed).

The library must load, export every function ``include/ksa.h`` declares, and
reject bad arguments on the host, before anything is launched.
"""
import ctypes
import os
import re

import pytest
import torch

import kv_cache_compression_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(K.LIB_PATH):
        from kv_cache_compression_amd import _build
        _build.build()
    return K.lib()


def _declared():
    txt = open(os.path.join(ROOT, "include", "ksa.h")).read()
    return sorted(set(re.findall(r"KSA_API[^;(]*?\b(ksa_\w+)\s*\(", txt)))


def test_exports_every_declared_symbol(L):
    decl = _declared()
    assert len(decl) == 20
    assert sorted(K.EXPORTS) == decl
    for name in decl:
        assert hasattr(L, name), name


def test_probe_library_exports_every_declared_symbol():
    """The machine-peak probes (include/ksa_probe.h) live in their own library."""
    from kv_cache_compression_amd import probe
    if not os.path.exists(probe.PROBE_LIB_PATH):
        from kv_cache_compression_amd import _build
        _build.build()
    txt = open(os.path.join(ROOT, "include", "ksa_probe.h")).read()
    decl = sorted(set(re.findall(r"^\w[\w ]*?\b(ksa_probe_\w+)\s*\(", txt, re.M)))
    assert decl == sorted(probe.EXPORTS)
    PL = probe.lib()
    for name in decl:
        assert hasattr(PL, name), name
    # host-side argument checks: nothing is launched
    assert PL.ksa_probe_mfma_bf16(0, 2, None, None, None) == -1
    assert PL.ksa_probe_mfma_bf16(1, 3, None, None, None) == -1
    assert PL.ksa_probe_mfma_bf16_operand_bytes(2) == 2 * 256 * 16 * 16
    assert PL.ksa_probe_hbm_read(None, 16, 1, None, None) == -1
    assert PL.ksa_probe_hbm_copy(None, None, 16, 1, None) == -1
    assert PL.ksa_probe_mfma_bf16_flops(2, 3) == 2 * 4 * 3 * 4 * 2 * 32 * 32 * 16
    # the attention library holds none of them
    K_syms = open(K.LIB_PATH, "rb").read()
    assert b"ksa_probe_mfma_bf16" not in K_syms


def _params(**kw):
    d = dict(chunk_size=8, window_chunks=4, num_q_heads=4, num_kv_heads=2, head_dim_qk=64,
             head_dim_v=64, v_is_k_prefix=0, softmax_scale=0.125, dtype=K.KSA_DTYPE_FP32)
    d.update(kw)
    return K.ksa_params(**d)


def test_sizes(L):
    assert L.ksa_augmented_len(512, 8) == 576
    assert L.ksa_augmented_len(517, 8) == 581
    assert L.ksa_augmented_len(-1, 8) == -1
    assert L.ksa_augmented_len(5, 0) == -1
    p = _params()
    assert L.ksa_cache_slots(ctypes.byref(p), 100) == 1 + 8 + 32 + 100
    assert L.ksa_cache_slots(ctypes.byref(p), -1) == -1
    assert L.ksa_decode_workspace_bytes(ctypes.byref(p), 64, 16384) > 0


def _status(L, rc):
    return rc, L.ksa_last_error_message().decode()


def test_invalid_arguments_rejected_before_launch(L):
    p = _params()
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    rc, msg = _status(L, L.ksa_prefill_attn(None, 1, 512, fake, fake, fake, fake, None, None))
    assert rc == 1 and "NULL" in msg
    bad = _params(num_q_heads=3)
    rc, msg = _status(L, L.ksa_prefill_attn(ctypes.byref(bad), 1, 512, fake, fake, fake, fake, None, None))
    assert rc == 1 and "multiple" in msg
    bad = _params(dtype=7)
    rc, _ = _status(L, L.ksa_prefill_attn(ctypes.byref(bad), 1, 512, fake, fake, fake, fake, None, None))
    assert rc == 2
    bad = _params(chunk_size=0)
    rc, _ = _status(L, L.ksa_prefill_attn(ctypes.byref(bad), 1, 512, fake, fake, fake, fake, None, None))
    assert rc == 1
    bad = _params(softmax_scale=0.0)
    rc, _ = _status(L, L.ksa_prefill_attn(ctypes.byref(bad), 1, 512, fake, fake, fake, fake, None, None))
    assert rc == 1
    rc, _ = _status(L, L.ksa_prefill_attn(ctypes.byref(p), 1, 512, fake, fake, None, fake, None, None))
    assert rc == 1  # v missing without v_is_k_prefix
    bad = _params(head_dim_qk=64, head_dim_v=128, v_is_k_prefix=1)
    rc, _ = _status(L, L.ksa_prefill_attn(ctypes.byref(bad), 1, 512, fake, fake, None, fake, None, None))
    assert rc == 1
    assert L.ksa_prefill_attn(ctypes.byref(p), 0, 512, None, None, None, None, None, None) == 0


def test_prefill_mode_arguments(L):
    p = _params()
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    rc, msg = _status(L, L.ksa_prefill_attn_mode(ctypes.byref(p), 3, 0, 1, 512, fake, fake, fake, fake, None, None))
    assert rc == 1 and "mode" in msg
    rc, msg = _status(L, L.ksa_prefill_attn_mode(ctypes.byref(p), 2, 0, 1, 512, fake, fake, fake, fake, None, None))
    assert rc == 1 and "window" in msg
    rc, _ = _status(L, L.ksa_prefill_attn_mode(ctypes.byref(p), 1, 0, 1, 512, fake, fake, None, fake, None, None))
    assert rc == 1  # v missing
    for mode in (0, 1, 2):
        assert L.ksa_prefill_attn_mode(ctypes.byref(p), mode, 5, 0, 512, None, None, None, None, None, None) == 0


def test_prefill_qrope_arguments(L):
    p = _params()
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    for theta in (0.0, -1.0, float("inf"), float("nan")):
        rc, msg = _status(L, L.ksa_prefill_attn_qrope(ctypes.byref(p), 1, 512, fake, fake, fake, fake, None, theta,
                                                      None))
        assert rc == 1 and "rope_theta" in msg
    odd = _params(head_dim_qk=63, head_dim_v=64)
    rc, msg = _status(L, L.ksa_prefill_attn_qrope(ctypes.byref(odd), 1, 512, fake, fake, fake, fake, None, 1e4, None))
    assert rc == 1 and "even" in msg
    mla = _params(num_q_heads=128, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, v_is_k_prefix=1)
    rc, msg = _status(L, L.ksa_prefill_attn_qrope(ctypes.byref(mla), 1, 512, fake, fake, None, fake, None, 1e4, None))
    assert rc == 2 and "absorbed" in msg
    rc, _ = _status(L, L.ksa_prefill_attn_qrope(ctypes.byref(p), 1, 512, fake, fake, None, fake, None, 1e4, None))
    assert rc == 1  # v missing
    assert L.ksa_prefill_attn_qrope(ctypes.byref(p), 0, 512, None, None, None, None, None, 1e4, None) == 0


def test_prefill_bwd_arguments(L):
    p = _params()
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    need = L.ksa_prefill_bwd_workspace_bytes(ctypes.byref(p), 2, 512)
    assert need >= 2 * 4 * 576 * 4
    assert L.ksa_prefill_bwd_workspace_bytes(None, 2, 512) == 0

    def call(params, mode=0, W=0, ptrs=(fake,) * 9, ws=fake, wsb=need, batch=2):
        return _status(L, L.ksa_prefill_attn_bwd(ctypes.byref(params), mode, W, batch, 512, *ptrs, ws, wsb, None))

    assert call(p, mode=5)[0] == 1
    assert call(p, mode=2, W=0)[0] == 1
    rc, msg = call(p, ptrs=(fake,) * 5 + (None,) + (fake,) * 3)
    assert rc == 1 and "NULL" in msg  # lse is required
    rc, msg = call(p, wsb=need - 1)
    assert rc == 4 and "workspace" in msg
    assert call(p, ws=None)[0] == 4
    mla = _params(head_dim_qk=64, head_dim_v=32, v_is_k_prefix=1)
    assert call(mla)[0] == 2
    assert call(p, batch=0, ptrs=(None,) * 9, ws=None, wsb=0)[0] == 0


def test_chunk_and_append_rows_arguments(L):
    p = _params()
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    c = K.ksa_cache(16, 16, 16, 10)
    rc, msg = _status(L, L.ksa_prefill_chunk(ctypes.byref(p), ctypes.byref(c), 2, None, 10, 20, fake, fake, fake,
                                             fake, None, None))
    assert rc == 1 and "NULL" in msg
    rc, _ = _status(L, L.ksa_prefill_chunk(ctypes.byref(p), None, 2, fake, 10, 20, fake, fake, fake, fake, None,
                                           None))
    assert rc == 1
    rc, _ = _status(L, L.ksa_prefill_chunk(ctypes.byref(p), ctypes.byref(c), 2, fake, -1, 20, fake, fake, fake,
                                           fake, None, None))
    assert rc == 1
    assert L.ksa_prefill_chunk(ctypes.byref(p), ctypes.byref(c), 2, fake, 0, 0, None, None, None, None, None,
                               None) == 0
    rc, _ = _status(L, L.ksa_cache_append_rows(ctypes.byref(p), ctypes.byref(c), 2, None, 10, fake, fake, None))
    assert rc == 1
    nov = K.ksa_cache(16, None, 16, 10)
    rc, _ = _status(L, L.ksa_cache_append_rows(ctypes.byref(p), ctypes.byref(nov), 2, fake, 10, fake, fake, None))
    assert rc == 1
    assert L.ksa_cache_append_rows(ctypes.byref(p), ctypes.byref(c), 0, None, 10, None, None, None) == 0


def test_rope_empty_inputs_are_no_ops(L):
    p = _params()
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    assert L.ksa_rope_augmented(ctypes.byref(p), 1, 0, None, 4, 64, 0, 64, ctypes.c_double(1e6), None) == 0
    assert L.ksa_rope_augmented(ctypes.byref(p), 0, 100, None, 4, 64, 0, 64, ctypes.c_double(1e6), None) == 0
    rc, msg = _status(L, L.ksa_rope_augmented(ctypes.byref(p), 1, 10, None, 4, 64, 0, 64, ctypes.c_double(1e6),
                                              None))
    assert rc == 1 and "NULL" in msg
    # argument errors are still reported for an empty input
    rc, _ = _status(L, L.ksa_rope_augmented(ctypes.byref(p), 1, 0, None, 4, 64, 0, 63, ctypes.c_double(1e6), None))
    assert rc == 1
    assert L.ksa_rope_positions(ctypes.byref(p), 0, None, None, 4, 64, 0, 64, ctypes.c_double(1e6), None) == 0
    rc, msg = _status(L, L.ksa_rope_positions(ctypes.byref(p), 3, None, fake, 4, 64, 0, 64, ctypes.c_double(1e6),
                                              None))
    assert rc == 1 and "positions" in msg


def test_cache_argument_checks(L):
    p = _params()
    fake = ctypes.c_void_p(16)
    c = K.ksa_cache(16, 16, 16, 10)
    # 11 complete chunks do not fit in a 10-summary buffer
    rc, msg = _status(L, L.ksa_cache_fill(ctypes.byref(p), ctypes.byref(c), 1, 88, fake, fake, None))
    assert rc == 3 and "max_summaries" in msg
    rc, _ = _status(L, L.ksa_cache_append(ctypes.byref(p), None, 1, fake, fake, fake, None))
    assert rc == 1
    rc, _ = _status(L, L.ksa_decode_attn(ctypes.byref(p), ctypes.byref(c), 2, fake, fake, fake, None,
                                         fake, 8, None))
    assert rc == 4
    nov = K.ksa_cache(16, None, 16, 10)
    rc, _ = _status(L, L.ksa_cache_append(ctypes.byref(p), ctypes.byref(nov), 1, fake, fake, fake, None))
    assert rc == 1
    # the allocation-free decode validates the same way, before any launch
    rc, msg = _status(L, L.ksa_decode_attn_noalloc(ctypes.byref(p), ctypes.byref(c), 2, None, fake, fake, None,
                                                   None))
    assert rc == 1 and "NULL" in msg
    rc, _ = _status(L, L.ksa_decode_attn_noalloc(ctypes.byref(p), ctypes.byref(nov), 2, fake, fake, fake, None,
                                                 None))
    assert rc == 1
    assert L.ksa_decode_attn_noalloc(ctypes.byref(p), ctypes.byref(c), 0, None, None, None, None, None) == 0


def test_status_strings(L):
    assert L.ksa_status_string(0) == b"ok"
    assert L.ksa_status_string(4) == b"workspace too small"
    assert L.ksa_status_string(99) == b"unknown status"


def test_python_binding_requires_gpu_tensors(L):
    p = K.Params(8, 4, 4, 2, 64, 64, torch.float32)
    q = torch.zeros(1, 576, 4, 64)
    with pytest.raises(ValueError):
        K.ksa_prefill_attn(p, q, torch.zeros(1, 576, 2, 64), torch.zeros(1, 576, 2, 64), 512)


def test_table1_ratios_from_library_accounting(L):
    """Per-token cache of the library's own layout (ksa_cache_slots x bytes
    per slot) as the history grows, against the ratios the report prints in
    Table 1 for k = 8, h = 128 heads, d = 128, g = 8 KV heads, d_c = 512,
    d_r = 64: KSA alone 12.5%, KSA + GQA 0.78%, KSA + MLA 0.22% of
    multi-head attention's 2 h d values per token (Sec. 3, Table 1)."""
    k, C, n = 8, 64, 8 * 2 ** 22                 # 33.5M tokens: the fixed regions vanish
    mha = 2 * 128 * 128                          # K and V of 128 heads of 128 per token

    def per_token(hq, hkv, dqk, dv, absorbed):
        p = K.Params(k, C, hq, hkv, dqk, dv, torch.bfloat16, v_is_k_prefix=absorbed).c()
        slots = L.ksa_cache_slots(ctypes.byref(p), n // k)
        assert slots == 1 + k + C * k + n // k
        width = dqk if absorbed else dqk + dv    # values per slot and kv head
        return slots * hkv * width / n

    assert per_token(128, 128, 128, 128, False) / mha == pytest.approx(0.125, rel=1e-3)
    assert round(100 * per_token(128, 8, 128, 128, False) / mha, 2) == 0.78
    assert round(100 * per_token(128, 1, 576, 512, True) / mha, 2) == 0.22
