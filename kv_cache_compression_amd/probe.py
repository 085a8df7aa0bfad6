"""Binding of the machine-peak probes (``include/ksa_probe.h``,
``libksa_probe.so``): argument marshalling only.  The benchmark times these
to report its rooflines against measured ceilings as well as published ones.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

PROBE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libksa_probe.so")
EXPORTS = ("ksa_probe_mfma_bf16", "ksa_probe_mfma_bf16_flops", "ksa_probe_mfma_bf16_operand_bytes",
           "ksa_probe_hbm_read", "ksa_probe_hbm_copy")

_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"{PROBE_LIB_PATH} is not built")
        L = ctypes.CDLL(PROBE_LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.ksa_probe_mfma_bf16.argtypes = [i32, i32, vp, vp, vp]
        L.ksa_probe_mfma_bf16.restype = i32
        L.ksa_probe_mfma_bf16_flops.argtypes = [i32, i32]
        L.ksa_probe_mfma_bf16_flops.restype = ctypes.c_double
        L.ksa_probe_mfma_bf16_operand_bytes.argtypes = [i32]
        L.ksa_probe_mfma_bf16_operand_bytes.restype = sz
        L.ksa_probe_hbm_read.argtypes = [vp, sz, i32, vp, vp]
        L.ksa_probe_hbm_read.restype = i32
        L.ksa_probe_hbm_copy.argtypes = [vp, vp, sz, i32, vp]
        L.ksa_probe_hbm_copy.restype = i32
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed with status {rc}")


def _stream(stream) -> int:
    return (stream or torch.cuda.current_stream()).cuda_stream


def ksa_probe_mfma_bf16(blocks: int, iters: int, sink: torch.Tensor, operands: Optional[torch.Tensor] = None,
                       stream=None) -> float:
    """Launch the MFMA loop (operands from ``operands`` when given, else
    from the lane index); returns the FLOP count of the launch."""
    if sink.dtype != torch.float32 or not sink.is_cuda or sink.numel() < blocks * 256:
        raise ValueError("sink must be a CUDA float32 tensor of blocks * 256 elements")
    optr = None
    if operands is not None:
        need = lib().ksa_probe_mfma_bf16_operand_bytes(blocks)
        if (not operands.is_cuda or not operands.is_contiguous()
                or operands.numel() * operands.element_size() < need):
            raise ValueError(f"operands must be a contiguous CUDA tensor of at least {need} bytes")
        optr = operands.data_ptr()
    _check(lib().ksa_probe_mfma_bf16(blocks, iters, optr, sink.data_ptr(), _stream(stream)), "ksa_probe_mfma_bf16")
    return lib().ksa_probe_mfma_bf16_flops(blocks, iters)


def ksa_probe_hbm_read(src: torch.Tensor, blocks: int, sink: torch.Tensor, stream=None) -> int:
    """Launch the streaming read over all of ``src``; returns the bytes read."""
    nbytes = src.numel() * src.element_size()
    if not src.is_cuda or not src.is_contiguous() or sink.dtype != torch.int32 or sink.numel() < blocks * 256:
        raise ValueError("src must be contiguous on the GPU; sink an int32 tensor of blocks * 256 elements")
    _check(lib().ksa_probe_hbm_read(src.data_ptr(), nbytes, blocks, sink.data_ptr(), _stream(stream)),
           "ksa_probe_hbm_read")
    return nbytes


def ksa_probe_hbm_copy(src: torch.Tensor, dst: torch.Tensor, blocks: int, stream=None) -> int:
    """Launch the streaming copy src -> dst; returns the bytes read plus written."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous and of equal size")
    _check(lib().ksa_probe_hbm_copy(src.data_ptr(), dst.data_ptr(), nbytes, blocks, _stream(stream)),
           "ksa_probe_hbm_copy")
    return 2 * nbytes
