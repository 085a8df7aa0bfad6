"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and names workload sizes; it contains
none of the attention method's arithmetic (no index maps, masks, rotations or
softmax), so both the HIP path and the CPU oracle can consume what it returns
without sharing any computation.

All tensors are produced on the CPU with a seeded ``torch.Generator`` so the
same bytes reach both sides.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import torch


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    batch: int
    n_text: int
    chunk: int
    window: int
    hq: int
    hkv: int
    dqk: int
    dv: int
    dtype: torch.dtype
    rope_theta: float
    seed: int


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    batch: int
    chunk: int
    window: int
    hq: int
    hkv: int
    dqk: int
    dv: int
    v_is_k_prefix: bool
    dtype: torch.dtype
    seed: int
    # history sizes: fixed (m, f) per sequence or ragged text lengths
    fixed_chunks: Optional[int] = None
    ragged_lo: Optional[int] = None
    ragged_hi: Optional[int] = None


# Workloads of the benchmark suite (sizes as named there).
TINY_PREFILL = PrefillWorkload("tiny_prefill_n512_k8_w4_h4x2_d64_fp32", 1, 512, 8, 4, 4, 2, 64, 64,
                               torch.float32, 1e6, 0)
PREFILL_32K = PrefillWorkload("prefill_n32768_k8_w64_h32x8_d128_bf16", 1, 32768, 8, 64, 32, 8, 128, 128,
                              torch.bfloat16, 1e6, 1)
PREFILL_128K_W64 = PrefillWorkload("prefill_n131072_k8_w64_h32x8_d128_bf16", 1, 131072, 8, 64, 32, 8,
                                   128, 128, torch.bfloat16, 1e6, 2)
PREFILL_128K_W16 = PrefillWorkload("prefill_n131072_k8_w16_h32x8_d128_bf16", 1, 131072, 8, 16, 32, 8,
                                   128, 128, torch.bfloat16, 1e6, 2)
DECODE_GQA = DecodeWorkload("decode_b64_n131072_k8_w64_h32x8_d128_bf16", 64, 8, 64, 32, 8, 128, 128,
                            False, torch.bfloat16, 3, fixed_chunks=16384)
# absorbed-MLA prefill: 128 query heads over one 576/512 latent head (V = K prefix)
PREFILL_MLA_8K = PrefillWorkload("prefill_mla_n8192_k8_w64_h128x1_d576x512_bf16", 1, 8192, 8, 64, 128, 1, 576, 512,
                                 torch.bfloat16, 1e6, 5)
DECODE_MLA = DecodeWorkload("decode_mla_b32_n16k-128k_k8_w64_h128x1_d576x512_bf16", 32, 8, 64, 128, 1,
                            576, 512, True, torch.bfloat16, 4, ragged_lo=16384, ragged_hi=131072)


def gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def normal(shape, dtype: torch.dtype, g: torch.Generator) -> torch.Tensor:
    """N(0, 1) samples drawn in fp32 and rounded once to ``dtype``."""
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(dtype)


def prefill_qkv(w: PrefillWorkload, L: int, n_text: Optional[int] = None, batch: Optional[int] = None):
    """Q [B, L, Hq, Dqk], K [B, L, Hkv, Dqk], V [B, L, Hkv, Dv] (augmented row order).

    ``L`` is the augmented length for ``n_text`` text tokens; the caller
    supplies it so that this module needs no knowledge of the layout.
    """
    B = w.batch if batch is None else batch
    g = gen(w.seed)
    q = normal((B, L, w.hq, w.dqk), w.dtype, g)
    k = normal((B, L, w.hkv, w.dqk), w.dtype, g)
    v = normal((B, L, w.hkv, w.dv), w.dtype, g)
    return q, k, v


def decode_histories(w: DecodeWorkload) -> List[int]:
    """Text-token count of each sequence *including* the query token.

    Fixed workload: m complete chunks plus a current-chunk fill f ~ U{0..k-1}
    already present, so the query is token number m*k + f + 1.
    Ragged workload: a history length uniform in [lo, hi], plus the query.
    """
    g = gen(w.seed)
    if w.fixed_chunks is not None:
        f = torch.randint(0, w.chunk, (w.batch,), generator=g)
        return [w.fixed_chunks * w.chunk + int(x) + 1 for x in f]
    n = torch.randint(w.ragged_lo, w.ragged_hi + 1, (w.batch,), generator=g)
    return [int(x) + 1 for x in n]


def decode_query(w: DecodeWorkload, seed_offset: int = 100) -> torch.Tensor:
    """One query token per sequence: [B, Hq, Dqk]."""
    g = gen(w.seed + seed_offset)
    return normal((w.batch, w.hq, w.dqk), w.dtype, g)
