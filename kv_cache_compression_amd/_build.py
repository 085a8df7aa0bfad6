"""Build libksa.so (HIP kernels + C ABI) and libksa_probe.so (machine-peak
probes used by the benchmark) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libksa.so")
PROBE_LIB = os.path.join(PKG, "libksa_probe.so")
PROBE_SOURCES = ["ksa_probe.hip"]

SOURCES = [
    "ksa_api.cpp",
    "ksa_rope.hip",
    "ksa_prefill_generic.hip",
    "ksa_prefill_mfma.hip",
    "ksa_prefill_bwd_generic.hip",
    "ksa_prefill_bwd_mfma.hip",
    "ksa_prefill_chunk_generic.hip",
    "ksa_prefill_chunk_mfma.hip",
    "ksa_prefill_mla.hip",
    "ksa_cache.hip",
    "ksa_decode.hip",
    "ksa_decode_mla.hip",
]

# Packed fp32 ops stay disabled for every kernel.
COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# Per-file extra flags.  The one-shot prefill and both absorbed-MLA kernels
# are scheduled for instruction-level parallelism (same code and results;
# prefill 0.5-1.7% faster at 32K and 128K).
EXTRA = {
    "ksa_prefill_mfma.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    # with the LDS operand reads issued ahead: 115.6 -> 108.5 us on the
    # 32-sequence decode, bit-identical
    "ksa_decode_mla.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    # 8K absorbed-MLA prefill: 2874 -> 2798 us in one same-run A/B
    "ksa_prefill_mla.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + COMMON + EXTRA.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


HOSTSAN_LIB = os.path.join(BUILD, "libksa_hostsan.so")


def build_host_sanitized(verbose: bool = False) -> str:
    """The same library with its host code (the C ABI's argument checks and
    dispatch, ksa_api.cpp) built by g++ under AddressSanitizer and
    UndefinedBehaviorSanitizer, linked with the kernel objects of the last
    build().  Loaded with the sanitizer runtimes preloaded; used by the CPU
    tests of the ABI."""
    if not all(os.path.exists(os.path.join(BUILD, os.path.splitext(s)[0] + ".o")) for s in SOURCES):
        build(verbose)
    api_obj = os.path.join(BUILD, "ksa_api_hostsan.o")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    inc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
    libdir = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    cmds = [
        ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer"] + san +
        ["-D__HIP_PLATFORM_AMD__", "-I" + inc, "-c", os.path.join(CSRC, "ksa_api.cpp"), "-o", api_obj],
        ["g++", "-shared"] + san + ["-o", HOSTSAN_LIB + ".tmp", api_obj] +
        [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "ksa_api.cpp"] +
        ["-L" + libdir, "-lamdhip64", "-Wl,-rpath," + libdir],
    ]
    for cmd in cmds:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"host-sanitized build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(HOSTSAN_LIB + ".tmp", HOSTSAN_LIB)
    if verbose:
        print("built", HOSTSAN_LIB)
    return HOSTSAN_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
