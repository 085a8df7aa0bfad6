"""Python binding of the KSA C ABI (``include/ksa.h``).

Argument marshalling only: every step of the attention path runs in the HIP
kernels of ``libksa.so``.  PyTorch supplies device memory and the stream.
There is no CPU fallback: if the library is missing the import still works,
but every call raises ``KsaLibraryMissing``.

Function names match the C entry points.  Tensors must be contiguous, on the
GPU, in the layouts the header documents; the binding checks shapes, dtypes
and devices before it calls into the library.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# KSA_LIB_PATH selects another build of the same library (for instance the
# host-sanitized one the CPU tests build); the default is the in-tree build
LIB_PATH = os.environ.get("KSA_LIB_PATH") or os.path.join(_PKG, "libksa.so")

KSA_DTYPE_BF16 = 0
KSA_DTYPE_FP32 = 1

KSA_CACHE_ERR_CHUNK_FULL = 1
KSA_CACHE_ERR_CHUNK_NOT_FULL = 2
KSA_CACHE_ERR_SUMMARY_FULL = 4
KSA_CACHE_ERR_BAD_SUMMARY_READ = 8
KSA_CACHE_ERR_BAD_SEGMENT = 16

# Every symbol the header declares.
EXPORTS = (
    "ksa_status_string", "ksa_last_error_message", "ksa_augmented_len", "ksa_rope_augmented",
    "ksa_rope_positions", "ksa_prefill_attn", "ksa_prefill_attn_qrope", "ksa_prefill_attn_mode",
    "ksa_prefill_bwd_workspace_bytes", "ksa_prefill_attn_bwd", "ksa_cache_slots", "ksa_cache_reset",
    "ksa_cache_append", "ksa_cache_fill", "ksa_cache_append_rows", "ksa_prefill_chunk", "ksa_decode_workspace_bytes",
    "ksa_decode_attn", "ksa_decode_attn_noalloc", "ksa_cache_read_errors",
)


class KsaLibraryMissing(RuntimeError):
    pass


class KsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"KSA status {status}: {message}")
        self.status = status


class ksa_params(ctypes.Structure):
    _fields_ = [
        ("chunk_size", ctypes.c_int32),
        ("window_chunks", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("v_is_k_prefix", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


class ksa_cache(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("state", ctypes.c_void_p),
        ("max_summaries", ctypes.c_int32),
    ]


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.POINTER(ksa_params)
_C = ctypes.POINTER(ksa_cache)
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64

_SIGS = {
    "ksa_status_string": (ctypes.c_char_p, [_i32]),
    "ksa_last_error_message": (ctypes.c_char_p, []),
    "ksa_augmented_len": (_i64, [_i64, _i32]),
    "ksa_rope_augmented": (_i32, [_P, _i32, _i64, _vp, _i32, _i32, _i32, _i32, ctypes.c_double, _vp]),
    "ksa_rope_positions": (_i32, [_P, _i64, _vp, _vp, _i32, _i32, _i32, _i32, ctypes.c_double, _vp]),
    "ksa_prefill_attn": (_i32, [_P, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "ksa_prefill_attn_qrope": (_i32, [_P, _i32, _i64, _vp, _vp, _vp, _vp, _vp, ctypes.c_double, _vp]),
    "ksa_prefill_attn_mode": (_i32, [_P, _i32, _i64, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "ksa_prefill_bwd_workspace_bytes": (ctypes.c_size_t, [_P, _i32, _i64]),
    "ksa_prefill_attn_bwd": (_i32, [_P, _i32, _i64, _i32, _i64] + [_vp] * 10 + [ctypes.c_size_t, _vp]),
    "ksa_cache_slots": (_i64, [_P, _i32]),
    "ksa_cache_reset": (_i32, [_P, _C, _i32, _vp]),
    "ksa_cache_append": (_i32, [_P, _C, _i32, _vp, _vp, _vp, _vp]),
    "ksa_cache_fill": (_i32, [_P, _C, _i32, _i64, _vp, _vp, _vp]),
    "ksa_cache_append_rows": (_i32, [_P, _C, _i32, _vp, _i64, _vp, _vp, _vp]),
    "ksa_prefill_chunk": (_i32, [_P, _C, _i32, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "ksa_decode_workspace_bytes": (ctypes.c_size_t, [_P, _i32, _i32]),
    "ksa_decode_attn": (_i32, [_P, _C, _i32, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "ksa_decode_attn_noalloc": (_i32, [_P, _C, _i32, _vp, _vp, _vp, _vp, _vp]),
    "ksa_cache_read_errors": (_i32, [_P, _C, _i32, _vp, _vp]),
}


def lib() -> ctypes.CDLL:
    """Load ``libksa.so`` (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise KsaLibraryMissing(
                f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        msg = lib().ksa_last_error_message().decode(errors="replace")
        name = lib().ksa_status_string(status).decode()
        raise KsaError(status, f"{name}: {msg}")


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return KSA_DTYPE_BF16
    if t == torch.float32:
        return KSA_DTYPE_FP32
    raise TypeError(f"unsupported dtype {t}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, shape: Sequence[int], dtype: torch.dtype, name: str) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype} != {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")


@dataclass(frozen=True)
class Params:
    """Python mirror of ``ksa_params``."""
    chunk_size: int
    window_chunks: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    dtype: torch.dtype
    softmax_scale: Optional[float] = None
    v_is_k_prefix: bool = False

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale is not None else 1.0 / math.sqrt(self.head_dim_qk)

    def c(self) -> ksa_params:
        return ksa_params(self.chunk_size, self.window_chunks, self.num_q_heads, self.num_kv_heads,
                          self.head_dim_qk, self.head_dim_v, int(self.v_is_k_prefix), self.scale,
                          _dtype_code(self.dtype))


def ksa_augmented_len(n_text: int, chunk_size: int) -> int:
    return int(lib().ksa_augmented_len(n_text, chunk_size))


def ksa_rope_augmented(p: Params, x: torch.Tensor, n_text: int, theta: float,
                       rot_off: int = 0, rot_dim: Optional[int] = None, stream=None) -> None:
    """In-place RoPE over the augmented sequence; x [B, L, H, D]."""
    B, L, H, D = x.shape
    _need(x, (B, ksa_augmented_len(n_text, p.chunk_size), H, D), p.dtype, "x")
    rot_dim = D - rot_off if rot_dim is None else rot_dim
    pc = p.c()
    _check(lib().ksa_rope_augmented(ctypes.byref(pc), B, n_text, _ptr(x), H, D, rot_off, rot_dim,
                                    float(theta), _stream(stream)))


def ksa_rope_positions(p: Params, x: torch.Tensor, positions: torch.Tensor, theta: float,
                       rot_off: int = 0, rot_dim: Optional[int] = None, stream=None) -> None:
    """In-place RoPE with explicit positions; x [R, H, D], positions [R] int64."""
    R, H, D = x.shape
    _need(x, (R, H, D), p.dtype, "x")
    _need(positions, (R,), torch.int64, "positions")
    rot_dim = D - rot_off if rot_dim is None else rot_dim
    pc = p.c()
    _check(lib().ksa_rope_positions(ctypes.byref(pc), R, _ptr(positions), _ptr(x), H, D, rot_off,
                                    rot_dim, float(theta), _stream(stream)))


MODE_KSA, MODE_SCA, MODE_SWA = 0, 1, 2


def _prefill_buffers(p: Params, q, k, v, n_text: int, out, lse):
    B = q.shape[0]
    L = ksa_augmented_len(n_text, p.chunk_size)
    _need(q, (B, L, p.num_q_heads, p.head_dim_qk), p.dtype, "q")
    _need(k, (B, L, p.num_kv_heads, p.head_dim_qk), p.dtype, "k")
    if not p.v_is_k_prefix:
        _need(v, (B, L, p.num_kv_heads, p.head_dim_v), p.dtype, "v")
    if out is None:
        out = torch.empty((B, L, p.num_q_heads, p.head_dim_v), dtype=p.dtype, device=q.device)
    _need(out, (B, L, p.num_q_heads, p.head_dim_v), p.dtype, "out")
    if lse is not None:
        _need(lse, (B, p.num_q_heads, L), torch.float32, "lse")
    return B, out


def ksa_prefill_attn(p: Params, q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor],
                     n_text: int, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """KSA prefill over the augmented sequence.  Returns ``out`` [B, L, Hq, Dv]."""
    B, out = _prefill_buffers(p, q, k, v, n_text, out, lse)
    pc = p.c()
    _check(lib().ksa_prefill_attn(ctypes.byref(pc), B, n_text, _ptr(q), _ptr(k),
                                  None if p.v_is_k_prefix else _ptr(v), _ptr(out), _ptr(lse),
                                  _stream(stream)))
    return out


def ksa_prefill_attn_qrope(p: Params, q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor], n_text: int,
                           rope_theta: float, out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """:func:`ksa_prefill_attn` on un-rotated queries: each query row is
    rotated (half-split over all Dqk columns, report Sec. 2.2.1 positions) as
    the kernel loads it; ``q`` is not written, ``k`` must be rotated already."""
    B, out = _prefill_buffers(p, q, k, v, n_text, out, lse)
    pc = p.c()
    _check(lib().ksa_prefill_attn_qrope(ctypes.byref(pc), B, n_text, _ptr(q), _ptr(k),
                                        None if p.v_is_k_prefix else _ptr(v), _ptr(out), _ptr(lse),
                                        float(rope_theta), _stream(stream)))
    return out


def ksa_prefill_attn_mode(p: Params, mode: int, window_tokens: int, q: torch.Tensor, k: torch.Tensor,
                          v: Optional[torch.Tensor], n_text: int, out: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Prefill with a visibility mode (MODE_KSA, MODE_SCA, MODE_SWA with a
    window of ``window_tokens``).  Returns ``out`` [B, L, Hq, Dv]."""
    B, out = _prefill_buffers(p, q, k, v, n_text, out, lse)
    pc = p.c()
    _check(lib().ksa_prefill_attn_mode(ctypes.byref(pc), mode, window_tokens, B, n_text, _ptr(q), _ptr(k),
                                       None if p.v_is_k_prefix else _ptr(v), _ptr(out), _ptr(lse),
                                       _stream(stream)))
    return out


def ksa_prefill_bwd_workspace_bytes(p: Params, batch: int, n_text: int) -> int:
    pc = p.c()
    return int(lib().ksa_prefill_bwd_workspace_bytes(ctypes.byref(pc), batch, n_text))


def ksa_prefill_attn_bwd(p: Params, mode: int, window_tokens: int, q: torch.Tensor, k: torch.Tensor,
                         v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor,
                         n_text: int, dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                         dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                         stream=None):
    """Backward of :func:`ksa_prefill_attn_mode`.  ``lse`` is the forward's
    [B, Hq, L] fp32 normaliser.  Returns (dq, dk, dv)."""
    B, _ = _prefill_buffers(p, q, k, v, n_text, out, lse)
    L = ksa_augmented_len(n_text, p.chunk_size)
    _need(dout, (B, L, p.num_q_heads, p.head_dim_v), p.dtype, "dout")
    if lse is None:
        raise ValueError("the backward needs the forward's lse")
    mk = lambda shape: torch.empty(shape, dtype=p.dtype, device=q.device)
    dq = mk(q.shape) if dq is None else dq
    dk = mk(k.shape) if dk is None else dk
    dv = mk(v.shape) if dv is None else dv
    _need(dq, tuple(q.shape), p.dtype, "dq")
    _need(dk, tuple(k.shape), p.dtype, "dk")
    _need(dv, tuple(v.shape), p.dtype, "dv")
    need = ksa_prefill_bwd_workspace_bytes(p, B, n_text)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    pc = p.c()
    _check(lib().ksa_prefill_attn_bwd(ctypes.byref(pc), mode, window_tokens, B, n_text, _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)))
    return dq, dk, dv


def ksa_cache_slots(p: Params, max_summaries: int) -> int:
    pc = p.c()
    return int(lib().ksa_cache_slots(ctypes.byref(pc), max_summaries))


class Cache:
    """Caller-owned cache buffers (allocated here with torch, owned by Python)."""

    def __init__(self, p: Params, batch: int, max_summaries: int, device="cuda"):
        self.p = p
        self.batch = batch
        self.max_summaries = max_summaries
        self.slots = ksa_cache_slots(p, max_summaries)
        if self.slots < 0:
            raise ValueError("bad cache parameters")
        self.k = torch.zeros((batch, p.num_kv_heads, self.slots, p.head_dim_qk), dtype=p.dtype, device=device)
        self.v = None if p.v_is_k_prefix else torch.zeros(
            (batch, p.num_kv_heads, self.slots, p.head_dim_v), dtype=p.dtype, device=device)
        self.state = torch.zeros((batch, 4), dtype=torch.int32, device=device)

    def c(self) -> ksa_cache:
        return ksa_cache(_ptr(self.k), _ptr(self.v), _ptr(self.state), self.max_summaries)


def ksa_cache_reset(c: Cache, stream=None) -> None:
    pc, cc = c.p.c(), c.c()
    _check(lib().ksa_cache_reset(ctypes.byref(pc), ctypes.byref(cc), c.batch, _stream(stream)))


def ksa_cache_append(c: Cache, k_new: torch.Tensor, v_new: Optional[torch.Tensor], kind: torch.Tensor,
                     stream=None) -> None:
    p = c.p
    _need(k_new, (c.batch, p.num_kv_heads, p.head_dim_qk), p.dtype, "k_new")
    if not p.v_is_k_prefix:
        _need(v_new, (c.batch, p.num_kv_heads, p.head_dim_v), p.dtype, "v_new")
    _need(kind, (c.batch,), torch.int32, "kind")
    pc, cc = p.c(), c.c()
    _check(lib().ksa_cache_append(ctypes.byref(pc), ctypes.byref(cc), c.batch, _ptr(k_new),
                                  None if p.v_is_k_prefix else _ptr(v_new), _ptr(kind), _stream(stream)))


def ksa_cache_fill(c: Cache, k_aug: torch.Tensor, v_aug: Optional[torch.Tensor], n_text: int,
                   stream=None) -> None:
    p = c.p
    L = ksa_augmented_len(n_text, p.chunk_size)
    _need(k_aug, (c.batch, L, p.num_kv_heads, p.head_dim_qk), p.dtype, "k_aug")
    if not p.v_is_k_prefix:
        _need(v_aug, (c.batch, L, p.num_kv_heads, p.head_dim_v), p.dtype, "v_aug")
    pc, cc = p.c(), c.c()
    _check(lib().ksa_cache_fill(ctypes.byref(pc), ctypes.byref(cc), c.batch, n_text, _ptr(k_aug),
                                None if p.v_is_k_prefix else _ptr(v_aug), _stream(stream)))


def _seg_rows(c: Cache, seg_rows: torch.Tensor, rows: torch.Tensor):
    _need(seg_rows, (c.batch + 1,), torch.int64, "seg_rows")
    total = rows.shape[0]
    return total


def ksa_cache_append_rows(c: Cache, seg_rows: torch.Tensor, max_rows: int, k_rows: torch.Tensor,
                          v_rows: Optional[torch.Tensor], stream=None) -> None:
    """Append each sequence's next augmented rows (packed at ``seg_rows``)."""
    p = c.p
    total = _seg_rows(c, seg_rows, k_rows)
    _need(k_rows, (total, p.num_kv_heads, p.head_dim_qk), p.dtype, "k_rows")
    if not p.v_is_k_prefix:
        _need(v_rows, (total, p.num_kv_heads, p.head_dim_v), p.dtype, "v_rows")
    pc, cc = p.c(), c.c()
    _check(lib().ksa_cache_append_rows(ctypes.byref(pc), ctypes.byref(cc), c.batch, _ptr(seg_rows), max_rows,
                                       _ptr(k_rows), None if p.v_is_k_prefix else _ptr(v_rows),
                                       _stream(stream)))


def ksa_prefill_chunk(c: Cache, seg_rows: torch.Tensor, max_rows: int, q: torch.Tensor, k: torch.Tensor,
                      v: Optional[torch.Tensor], out: Optional[torch.Tensor] = None,
                      lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Chunked / varlen prefill of each sequence's next rows against its
    cache.  Returns ``out`` [total_rows, Hq, Dv]."""
    p = c.p
    total = _seg_rows(c, seg_rows, q)
    _need(q, (total, p.num_q_heads, p.head_dim_qk), p.dtype, "q")
    _need(k, (total, p.num_kv_heads, p.head_dim_qk), p.dtype, "k")
    if not p.v_is_k_prefix:
        _need(v, (total, p.num_kv_heads, p.head_dim_v), p.dtype, "v")
    if out is None:
        out = torch.empty((total, p.num_q_heads, p.head_dim_v), dtype=p.dtype, device=q.device)
    _need(out, (total, p.num_q_heads, p.head_dim_v), p.dtype, "out")
    if lse is not None:
        _need(lse, (p.num_q_heads, total), torch.float32, "lse")
    pc, cc = p.c(), c.c()
    _check(lib().ksa_prefill_chunk(ctypes.byref(pc), ctypes.byref(cc), c.batch, _ptr(seg_rows), max_rows, total,
                                   _ptr(q), _ptr(k), None if p.v_is_k_prefix else _ptr(v), _ptr(out), _ptr(lse),
                                   _stream(stream)))
    return out


def ksa_decode_workspace_bytes(p: Params, batch: int, max_summaries: int) -> int:
    pc = p.c()
    return int(lib().ksa_decode_workspace_bytes(ctypes.byref(pc), batch, max_summaries))


def decode_workspace(c: Cache) -> torch.Tensor:
    n = ksa_decode_workspace_bytes(c.p, c.batch, c.max_summaries)
    return torch.empty((max(n, 1),), dtype=torch.uint8, device=c.k.device)


def ksa_decode_attn(c: Cache, q: torch.Tensor, kind: torch.Tensor, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    p = c.p
    _need(q, (c.batch, p.num_q_heads, p.head_dim_qk), p.dtype, "q")
    _need(kind, (c.batch,), torch.int32, "kind")
    if out is None:
        out = torch.empty((c.batch, p.num_q_heads, p.head_dim_v), dtype=p.dtype, device=q.device)
    _need(out, (c.batch, p.num_q_heads, p.head_dim_v), p.dtype, "out")
    if lse is not None:
        _need(lse, (c.batch, p.num_q_heads), torch.float32, "lse")
    if workspace is None:
        workspace = decode_workspace(c)
    pc, cc = p.c(), c.c()
    _check(lib().ksa_decode_attn(ctypes.byref(pc), ctypes.byref(cc), c.batch, _ptr(q), _ptr(kind),
                                 _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def ksa_decode_attn_noalloc(c: Cache, q: torch.Tensor, kind: torch.Tensor, out: Optional[torch.Tensor] = None,
                            lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """ksa_decode_attn with the library's own scratch (no workspace)."""
    p = c.p
    _need(q, (c.batch, p.num_q_heads, p.head_dim_qk), p.dtype, "q")
    _need(kind, (c.batch,), torch.int32, "kind")
    if out is None:
        out = torch.empty((c.batch, p.num_q_heads, p.head_dim_v), dtype=p.dtype, device=q.device)
    _need(out, (c.batch, p.num_q_heads, p.head_dim_v), p.dtype, "out")
    if lse is not None:
        _need(lse, (c.batch, p.num_q_heads), torch.float32, "lse")
    pc, cc = p.c(), c.c()
    _check(lib().ksa_decode_attn_noalloc(ctypes.byref(pc), ctypes.byref(cc), c.batch, _ptr(q), _ptr(kind),
                                         _ptr(out), _ptr(lse), _stream(stream)))
    return out


def ksa_cache_read_errors(c: Cache, stream=None) -> list:
    host = (ctypes.c_int32 * c.batch)()
    pc, cc = c.p.c(), c.c()
    _check(lib().ksa_cache_read_errors(ctypes.byref(pc), ctypes.byref(cc), c.batch, ctypes.cast(host, ctypes.c_void_p),
                                       _stream(stream)))
    return list(host)
