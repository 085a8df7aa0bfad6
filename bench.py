"""Benchmark of the KSA hot path on one MI355X.

One step = one pass of the whole path on synthetic inputs already resident
in HBM:
  1. RoPE pass (KSA position rule) over K of the 32K-token prefill (the
     cache keeps post-RoPE keys),
  2. KSA prefill attention (32K text tokens, k=8, w=64, 32/8 heads, d=128,
     bf16) with Q's rotation applied as the kernel loads each query row,
  3. hand-off of that prefill's K/V into its decode cache (bulk fill),
  4. one decode step of the 64-sequence, 131072-token-history batch
     (text-token cache append, then split-K decode over the contiguous slice),
  5. one decode step of the 32-sequence absorbed-MLA batch (ragged 16K-128K
     histories, 128 heads on one 576/512 latent head), rotating over three
     cache copies so that reads come from HBM.
The 131072-token prefill (w = 64 and w = 16) is timed separately after the
steps and reported beside them.

``value`` is the prefill throughput in TFLOP/s counted over visible
(query, key) pairs only, 2 (Dqk + Dv) Hq per pair; the decode step's HBM
throughput is reported beside it.  Kernel times come from HIP events on the
stream every launch goes to.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KSA prefill TFLOP/s (visible pairs) + decode HBM GB/s, 1 MI355X, % roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def visible_pairs(n: int, k: int, C: int) -> int:
    """Visible (query, key) pairs of one head: every summary sees k+1 keys;
    text token i in chunk c sees min(c, C) k + (i mod k) + 1 text keys and
    max(0, c - C) summaries.  Summed in closed form over whole chunks."""
    M = n // k
    tot = M * (k + 1)

    def text_rows(c0: int, c1: int, rows_per_chunk: int) -> int:
        # sum over chunks c in [c0, c1) of sum_{p<rows} (min(c,C) k + p + 1 + max(0, c-C))
        s = 0
        for lo, hi in ((c0, min(c1, C)), (max(c0, C), c1)):
            if hi <= lo:
                continue
            cnt = hi - lo
            csum = (lo + hi - 1) * cnt // 2
            if lo >= C:   # min(c,C) = C, max(0,c-C) = c - C
                per = C * k * cnt + (csum - C * cnt)
            else:         # min(c,C) = c, max = 0
                per = k * csum
            s += per * rows_per_chunk + cnt * rows_per_chunk * (rows_per_chunk + 1) // 2
        return s

    tot += text_rows(0, M, k)
    rem = n - M * k
    if rem:
        tot += text_rows(M, M + 1, rem)
    return tot


def baseline_pairs(n: int, k: int, mode: int, C: int, W: int) -> int:
    """Visible (query, key) pairs of one head for the summary-free baselines:
    text t_i sees min(floor(i/k), C) k + i mod k + 1 keys (sliding chunks) or
    min(i + 1, W) keys (token window); every summary row sees k + 1."""
    import numpy as np

    i = np.arange(n, dtype=np.int64)
    text = np.minimum(i // k, C) * k + i % k + 1 if mode == 1 else np.minimum(i + 1, W)
    return int(text.sum()) + (n // k) * (k + 1)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long", action="store_true", help="skip the 131072-token prefill lines")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the backward, chunked, MLA-prefill and baseline-mode lines")
    ap.add_argument("--cpu-rows", type=int, default=0, help="oracle sample rows (0 = auto)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 256 MiB device copy three times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only; runs on several GPUs are not supported",
                          "n_gpus": args.gpus}))
        return 2
    if args.copy_probe:
        return copy_probe()

    import torch

    import kv_cache_compression_amd as ksa
    import ksa_synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # ---- prefill workload: 32K text tokens ----
    w = ksa_synth.PREFILL_32K
    L = ksa.ksa_augmented_len(w.n_text, w.chunk)
    q, kx, v = ksa_synth.prefill_qkv(w, L)
    p = ksa.Params(w.chunk, w.window, w.hq, w.hkv, w.dqk, w.dv, w.dtype)
    qd, kd, vd = q.to(dev), kx.to(dev), v.to(dev)
    del q, kx, v
    out = torch.empty((1, L, w.hq, w.dv), dtype=w.dtype, device=dev)
    pcache = ksa.Cache(p, 1, w.n_text // w.chunk, device=dev)
    pairs = visible_pairs(w.n_text, w.chunk, w.window)
    flops = 2 * (w.dqk + w.dv) * w.hq * pairs * w.batch
    rope_bytes = 2 * 2 * L * w.hkv * w.dqk                      # read + write K
    fill_rows = 1 + w.chunk + w.window * w.chunk + w.n_text // w.chunk

    # ---- decode workload: 64 sequences x 131072-token history ----
    dw = ksa_synth.DECODE_GQA
    dp = ksa.Params(dw.chunk, dw.window, dw.hq, dw.hkv, dw.dqk, dw.dv, dw.dtype)
    hist = ksa_synth.decode_histories(dw)      # text tokens incl. the query
    max_s = max(n // dw.chunk for n in hist) + 1
    dcache = ksa.Cache(dp, dw.batch, max_s, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(dw.seed)
    dcache.k.normal_(generator=gen)
    dcache.v.normal_(generator=gen)
    st0 = torch.zeros((dw.batch, 4), dtype=torch.int32)
    for b, n in enumerate(hist):
        m = (n - 1) // dw.chunk
        st0[b, 0] = m
        st0[b, 1] = n - 1 - m * dw.chunk            # fill before the query token arrives
    st0 = st0.to(dev)
    g2 = ksa_synth.gen(dw.seed + 7)
    k_new = ksa_synth.normal((dw.batch, dw.hkv, dw.dqk), dw.dtype, g2).to(dev)
    v_new = ksa_synth.normal((dw.batch, dw.hkv, dw.dv), dw.dtype, g2).to(dev)
    dq = ksa_synth.decode_query(dw).to(dev)
    kind = torch.zeros((dw.batch,), dtype=torch.int32, device=dev)
    dout = torch.empty((dw.batch, dw.hq, dw.dv), dtype=dw.dtype, device=dev)
    ws = ksa.decode_workspace(dcache)
    dec_rows = 0
    for n in hist:
        m = (n - 1) // dw.chunk
        r = n - m * dw.chunk
        dec_rows += r + min(m, dw.window) * dw.chunk + max(0, m - dw.window)
    dec_bytes = (dec_rows * dw.hkv * (dw.dqk + dw.dv) * 2
                 + dw.batch * dw.hq * (dw.dqk + dw.dv) * 2)  # cache slice + q + out
    # ---- absorbed-MLA decode workload: 32 sequences, ragged histories ----
    mw = ksa_synth.DECODE_MLA
    mp = ksa.Params(mw.chunk, mw.window, mw.hq, mw.hkv, mw.dqk, mw.dv, mw.dtype, v_is_k_prefix=True)
    mhist = ksa_synth.decode_histories(mw)
    mmax = max(n // mw.chunk for n in mhist) + 1
    mcaches = []
    for c in range(3):   # > 3 x the 256 MB last-level cache in total
        mc = ksa.Cache(mp, mw.batch, mmax, device=dev)
        gm = torch.Generator(device=dev)
        gm.manual_seed(mw.seed + c)
        mc.k.normal_(generator=gm)
        mst = torch.zeros((mw.batch, 4), dtype=torch.int32)
        for b, n in enumerate(mhist):
            m = (n - 1) // mw.chunk
            mst[b, 0] = m
            mst[b, 1] = n - m * mw.chunk
        mc.state.copy_(mst.to(dev))
        mcaches.append(mc)
    mq = ksa_synth.decode_query(mw).to(dev)
    mkind = torch.zeros((mw.batch,), dtype=torch.int32, device=dev)
    mout = torch.empty((mw.batch, mw.hq, mw.dv), dtype=mw.dtype, device=dev)
    mws = ksa.decode_workspace(mcaches[0])
    mla_rows = 0
    for n in mhist:
        m = (n - 1) // mw.chunk
        r = n - m * mw.chunk
        mla_rows += r + min(m, mw.window) * mw.chunk + max(0, m - mw.window)
    mla_bytes = mla_rows * mw.dqk * 2 + mw.batch * mw.hq * (mw.dqk + mw.dv) * 2
    mla_flops = 2 * mw.hq * (mw.dqk + mw.dv) * mla_rows
    torch.cuda.synchronize()

    segs = ["rope", "prefill", "fill", "append", "decode", "decode_mla"]
    counter = [0]

    # every step rotates K in place: restore the pristine keys first, outside
    # the timed segments, so that every timed prefill sees the inputs the
    # parity tests check (RoPE applied once); Q is never written
    k0 = kd.clone()

    def step(ev):
        kd.copy_(k0)
        ev[0].record(stream)
        ksa.ksa_rope_augmented(p, kd, w.n_text, w.rope_theta, stream=stream)
        ev[1].record(stream)
        ksa.ksa_prefill_attn_qrope(p, qd, kd, vd, w.n_text, w.rope_theta, out=out, stream=stream)
        ev[2].record(stream)
        ksa.ksa_cache_fill(pcache, kd, vd, w.n_text, stream=stream)
        ev[3].record(stream)
        dcache.state.copy_(st0)
        ksa.ksa_cache_append(dcache, k_new, v_new, kind, stream=stream)
        ev[4].record(stream)
        ksa.ksa_decode_attn(dcache, dq, kind, out=dout, workspace=ws, stream=stream)
        ev[5].record(stream)
        mc = mcaches[counter[0] % len(mcaches)]
        counter[0] += 1
        ksa.ksa_decode_attn(mc, mq, mkind, out=mout, workspace=mws, stream=stream)
        ev[6].record(stream)

    # the GPU's own ceilings, measured before the timed work so that they are
    # not taken on a chip already heated by it
    peaks = machine_peaks(torch, dev, stream)

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(7)]
    for _ in range(args.warmup):
        step(mk())
    torch.cuda.synchronize()
    evs = [mk() for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    seg_all = {s: sorted(e[i].elapsed_time(e[i + 1]) for e in evs) for i, s in enumerate(segs)}
    seg_ms = {s: sum(v) / args.steps for s, v in seg_all.items()}
    for c in [dcache] + mcaches:
        errs = ksa.ksa_cache_read_errors(c)
        if any(errs):
            raise RuntimeError(f"decode cache error bits {errs}")
    kd.copy_(k0)
    rope_fusion = rope_fusion_line(ksa, torch, w, p, qd, kd, vd, out, stream)
    long_runs = [] if args.no_long else prefill_long(ksa, ksa_synth, torch, dev, stream)
    bwd, chunked, mla_pre, modes = None, None, None, []
    if not args.no_extra:
        bwd, chunked, mla_pre, modes = extra_lines(ksa, ksa_synth, torch, dev, stream, w, p, qd, kd, vd, out,
                                                   seg_ms["prefill"])

    pre_tflops = flops / (seg_ms["prefill"] * 1e-3) / 1e12
    dec_gbps = dec_bytes / (seg_ms["decode"] * 1e-3) / 1e9
    rope_gbps = rope_bytes / (seg_ms["rope"] * 1e-3) / 1e9
    mla_gbps = mla_bytes / (seg_ms["decode_mla"] * 1e-3) / 1e9

    res = {
        "metric": METRIC,
        "value": round(pre_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V and cache)",
        "config": {
            "workload": w.name + " + " + dw.name,
            "prefill": {"batch": w.batch, "n_text": w.n_text, "augmented_len": L, "chunk": w.chunk,
                        "window_chunks": w.window, "q_heads": w.hq, "kv_heads": w.hkv, "head_dim": w.dqk,
                        "rope_theta": w.rope_theta, "q_rope": "applied in the prefill kernel's query load",
                        "visible_pairs_per_head": pairs, "flops": flops},
            "decode": {"batch": dw.batch, "history_text_tokens": hist[0] - hist[0] % dw.chunk,
                       "chunk": dw.chunk, "window_chunks": dw.window, "q_heads": dw.hq,
                       "kv_heads": dw.hkv, "head_dim": dw.dqk, "slice_rows_total": dec_rows,
                       "bytes": dec_bytes},
        },
        "decode": {"value": round(dec_gbps, 1), "unit": "GB/s", "frac_of_peak": round(dec_gbps / PEAK_HBM_GBPS, 4),
                   "ms": round(seg_ms["decode"], 4)},
        "decode_mla": {"value": round(mla_gbps, 1), "unit": "GB/s",
                       "frac_of_peak": round(mla_gbps / PEAK_HBM_GBPS, 4),
                       "tflops": round(mla_flops / (seg_ms["decode_mla"] * 1e-3) / 1e12, 1),
                       "ms": round(seg_ms["decode_mla"], 4), "workload": mw.name,
                       "slice_rows_total": mla_rows, "bytes": mla_bytes},
        "prefill_long": long_runs,
        "prefill_baselines": modes,
        "prefill_backward": bwd,
        "prefill_chunked": chunked,
        "prefill_mla": mla_pre,
        "rope": {"value": round(rope_gbps, 1), "unit": "GB/s", "ms": round(seg_ms["rope"], 4), "rotates": "K"},
        "rope_fusion": rope_fusion,
        "breakdown_ms": {s: round(v, 4) for s, v in seg_ms.items()},
        "breakdown_ms_min": {s: round(v[0], 4) for s, v in seg_all.items()},
        "breakdown_ms_median": {s: round(v[len(v) // 2], 4) for s, v in seg_all.items()},
        "roofline": {"kernel": "prefill_mfma_d128_kernel", "bound": "mfma", "achieved": round(pre_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
    }
    if peaks:
        res["machine_peaks"] = peaks
        res["roofline"]["frac_of_measured_peak"] = round(pre_tflops / peaks["mfma_bf16_tflops"], 4)
        res["decode"]["frac_of_measured_read"] = round(dec_gbps / peaks["hbm_read_gbps"], 4)
    traffic = prefill_traffic()
    if traffic is not None:
        res["roofline"]["traffic"] = traffic["total_bytes"]
        res["roofline"]["traffic_detail"] = traffic
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
        if not args.no_extra:
            extra_oracle_rates(res, w)
        long_oracle_rates(res)
    print(json.dumps(res), flush=True)
    return 0


COPY_PROBE_BYTES = 256 << 20
PMC_SUMMARY = os.path.join(ROOT, "profiles", "prefill_mfma_d128_32k_pmc.txt")
PREFILL_SOURCE = os.path.join(ROOT, "kv_cache_compression_amd", "csrc", "ksa_prefill_mfma.hip")


def machine_peaks(torch, dev, stream) -> dict:
    """Measured ceilings of this GPU: the bf16 MFMA issue loop and the
    streaming HBM read and copy of libksa_probe.so, best of three launches
    each, timed with HIP events on the benchmark stream."""
    try:
        from kv_cache_compression_amd import probe
        probe.lib()
    except Exception as e:  # the attention numbers stand without it
        print(f"machine-peak probes unavailable: {e}", file=sys.stderr)
        return {}

    def best_ms(fn, reps=3):
        fn()
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        return min(out)

    blocks, iters = 2048, 2048
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    flops = probe.lib().ksa_probe_mfma_bf16_flops(blocks, iters)
    ms = best_ms(lambda: probe.ksa_probe_mfma_bf16(blocks, iters, sink, None, stream))
    mfma = flops / (ms * 1e-3) / 1e12
    # the same loop on N(0,1) bf16 operands, as the attention kernels see them
    nel = probe.lib().ksa_probe_mfma_bf16_operand_bytes(blocks) // 2
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    opnd = torch.randn(nel, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    ms = best_ms(lambda: probe.ksa_probe_mfma_bf16(blocks, iters, sink, opnd, stream))
    mfma_data = flops / (ms * 1e-3) / 1e12
    del opnd
    nbytes = 4 << 30        # 16 x the 256 MB last-level cache
    src = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    rd = {}
    for nb in (512, 2048, 8192):
        isink = torch.empty(nb * 256, dtype=torch.int32, device=dev)
        rd[nb] = nbytes / (best_ms(lambda: probe.ksa_probe_hbm_read(src, nb, isink, stream)) * 1e-3) / 1e9
    half = src[: nbytes // 2]
    dst = torch.empty(nbytes // 2, dtype=torch.uint8, device=dev)
    cp = max(nbytes / (best_ms(lambda: probe.ksa_probe_hbm_copy(half, dst, nb, stream)) * 1e-3) / 1e9
             for nb in (512, 2048, 8192))
    del src, dst, half
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(mfma_data, 1), "mfma_bf16_tflops_constant_operands": round(mfma, 1),
            "hbm_read_gbps": round(max(rd.values()), 1),
            "hbm_copy_gbps": round(cp, 1),
            "source": "libksa_probe.so: 32x32x16 bf16 MFMA loop (2048 x 256 threads, 2048 iterations) on "
                      "N(0,1) operands (and on lane-index constants), "
                      "4 GiB non-temporal read and 2 GiB copy (read + write counted) at 512/2048/8192 "
                      "workgroups; best of 3 launches each"}


def copy_probe() -> int:
    """A plain device-to-device copy of known size, used to scale the
    FETCH_SIZE / WRITE_SIZE hardware counters to bytes."""
    import torch

    a = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "copies": 3}), flush=True)
    return 0


def prefill_traffic():
    """HBM bytes per prefill launch from the committed counter summary, or
    None when the summary is missing or the kernel source (or its extra
    compile flags) has changed since the counters were taken."""
    import hashlib

    try:
        kv = {}
        with open(PMC_SUMMARY) as f:
            for line in f:
                if "=" in line and not line.lstrip().startswith("#"):
                    key, val = line.split("=", 1)
                    kv[key.strip()] = val.strip()
        from kv_cache_compression_amd import _build as kb

        flags = " ".join(kb.EXTRA.get(os.path.basename(PREFILL_SOURCE), [])).encode()
        with open(PREFILL_SOURCE, "rb") as f:   # the source and its extra compile flags
            digest = hashlib.sha256(f.read() + flags).hexdigest()
        if kv.get("kernel_source_sha256") != digest:
            return None
        fetch = float(kv["fetch_kib_per_dispatch"]) * float(kv["fetch_scale"]) * 1024
        write = float(kv["write_kib_per_dispatch"]) * float(kv["write_scale"]) * 1024
        return {"read_bytes": int(fetch), "write_bytes": int(write), "total_bytes": int(fetch + write),
                "algorithmic_bytes": int(kv["algorithmic_bytes"]), "source": os.path.relpath(PMC_SUMMARY, ROOT)}
    except (OSError, KeyError, ValueError):
        return None


def prefill_long(ksa, ksa_synth, torch, dev, stream, reps: int = 5) -> list:
    """The 131072-token prefill at w = 64 and w = 16 (RoPE pre-pass applied
    once, outside the timing)."""
    res = []
    for w in (ksa_synth.PREFILL_128K_W64, ksa_synth.PREFILL_128K_W16):
        L = ksa.ksa_augmented_len(w.n_text, w.chunk)
        g = ksa_synth.gen(w.seed)
        qd = ksa_synth.normal((w.batch, L, w.hq, w.dqk), w.dtype, g).to(dev)
        kd = ksa_synth.normal((w.batch, L, w.hkv, w.dqk), w.dtype, g).to(dev)
        vd = ksa_synth.normal((w.batch, L, w.hkv, w.dv), w.dtype, g).to(dev)
        p = ksa.Params(w.chunk, w.window, w.hq, w.hkv, w.dqk, w.dv, w.dtype)
        ksa.ksa_rope_augmented(p, qd, w.n_text, w.rope_theta, stream=stream)
        ksa.ksa_rope_augmented(p, kd, w.n_text, w.rope_theta, stream=stream)
        out = torch.empty((w.batch, L, w.hq, w.dv), dtype=w.dtype, device=dev)
        ksa.ksa_prefill_attn(p, qd, kd, vd, w.n_text, out=out, stream=stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            ksa.ksa_prefill_attn(p, qd, kd, vd, w.n_text, out=out, stream=stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / reps
        fl = 2 * (w.dqk + w.dv) * w.hq * visible_pairs(w.n_text, w.chunk, w.window) * w.batch
        tf = fl / (ms * 1e-3) / 1e12
        res.append({"workload": w.name, "ms": round(ms, 4), "tflops": round(tf, 2),
                    "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "flops": fl})
        del qd, kd, vd, out
        torch.cuda.empty_cache()
    return res


def rope_fusion_line(ksa, torch, w, p, qd, kd, vd, out, stream, reps: int = 10) -> dict:
    """RoPE + prefill both ways on the same inputs: a separate rotation pass
    over Q and K, then ksa_prefill_attn, against a pass over K only, then
    ksa_prefill_attn_qrope.  Copies are rotated, so the inputs stay as
    they are; the copies' refresh is inside both timings alike."""
    qs, ks = qd.clone(), kd.clone()

    def two_pass():
        qs.copy_(qd)
        ks.copy_(kd)
        ksa.ksa_rope_augmented(p, qs, w.n_text, w.rope_theta, stream=stream)
        ksa.ksa_rope_augmented(p, ks, w.n_text, w.rope_theta, stream=stream)
        ksa.ksa_prefill_attn(p, qs, ks, vd, w.n_text, out=out, stream=stream)

    def fused():
        qs.copy_(qd)
        ks.copy_(kd)
        ksa.ksa_rope_augmented(p, ks, w.n_text, w.rope_theta, stream=stream)
        ksa.ksa_prefill_attn_qrope(p, qs, ks, vd, w.n_text, w.rope_theta, out=out, stream=stream)

    res = {}
    for name, fn in (("two_pass_ms", two_pass), ("fused_ms", fused)):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        res[name] = round(ev[0].elapsed_time(ev[1]) / reps, 4)
    res["saved_ms"] = round(res["two_pass_ms"] - res["fused_ms"], 4)
    del qs, ks
    return res


def extra_lines(ksa, ksa_synth, torch, dev, stream, w, p, qd, kd, vd, out, ksa_ms):
    """The backward, the chunked prefill, the MLA prefill and the report's
    summary-free baselines on the same inputs (A/B timing)."""
    bwd = prefill_backward(ksa, ksa_synth, torch, w, p, qd, kd, vd, stream)
    chunked = prefill_chunked(ksa, torch, w, p, qd, kd, vd, stream)
    mla_pre = prefill_mla(ksa, ksa_synth, torch, dev, stream)
    modes = []
    for mode, name, W in ((ksa.MODE_SCA, "sliding chunks (no summaries)", 0),
                          (ksa.MODE_SWA, f"token window of {w.window * w.chunk}", w.window * w.chunk)):
        ksa.ksa_prefill_attn_mode(p, mode, W, qd, kd, vd, w.n_text, out=out, stream=stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(5):
            ksa.ksa_prefill_attn_mode(p, mode, W, qd, kd, vd, w.n_text, out=out, stream=stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / 5
        fl = 2 * (w.dqk + w.dv) * w.hq * baseline_pairs(w.n_text, w.chunk, mode, w.window, W) * w.batch
        modes.append({"mode": name, "ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                      "ksa_ms": round(ksa_ms, 4)})
    return bwd, chunked, mla_pre, modes


def prefill_backward(ksa, ksa_synth, torch, w, p, qd, kd, vd, stream, reps: int = 5) -> dict:
    """Backward of the prefill on the same workload and inputs: dq, dk, dv
    from a seeded output gradient, the forward's output and normaliser."""
    L = ksa.ksa_augmented_len(w.n_text, w.chunk)
    g = ksa_synth.normal((w.batch, L, w.hq, w.dv), w.dtype, ksa_synth.gen(w.seed + 7)).to(qd.device)
    lse = torch.empty((w.batch, w.hq, L), dtype=torch.float32, device=qd.device)
    out = ksa.ksa_prefill_attn(p, qd, kd, vd, w.n_text, lse=lse, stream=stream)
    ws = torch.empty(ksa.ksa_prefill_bwd_workspace_bytes(p, w.batch, w.n_text), dtype=torch.uint8,
                     device=qd.device)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    run = lambda: ksa.ksa_prefill_attn_bwd(p, ksa.MODE_KSA, 0, qd, kd, vd, out, g, lse, w.n_text,
                                           dq, dk, dv, ws, stream=stream)
    run()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        run()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    # recompute S, dP, then dV, dK, dQ: five products over every visible pair
    fl = 2 * (3 * w.dqk + 2 * w.dv) * w.hq * visible_pairs(w.n_text, w.chunk, w.window) * w.batch
    tf = fl / (ms * 1e-3) / 1e12
    del g, lse, out, ws, dq, dk, dv
    torch.cuda.empty_cache()
    return {"workload": w.name, "ms": round(ms, 4), "tflops": round(tf, 2),
            "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "flops": fl,
            "workspace_mb": round(ksa.ksa_prefill_bwd_workspace_bytes(p, w.batch, w.n_text) / 1e6, 1)}


def prefill_chunked(ksa, torch, w, p, qd, kd, vd, stream, n_chunks: int = 8, reps: int = 10) -> dict:
    """The same workload fed in n_chunks segments through the cache: each
    segment is prefilled against the cache (ksa_prefill_chunk) and then
    appended (ksa_cache_append_rows); one pass = the whole sequence."""
    L = ksa.ksa_augmented_len(w.n_text, w.chunk)
    bounds = [L * i // n_chunks for i in range(n_chunks + 1)]
    cache = ksa.Cache(p, w.batch, w.n_text // w.chunk + 1, device=qd.device)
    segs = []
    for i in range(n_chunks):
        a, b = bounds[i], bounds[i + 1]
        segs.append((torch.tensor([0, b - a], dtype=torch.int64, device=qd.device), b - a,
                     qd[0, a:b].contiguous(), kd[0, a:b].contiguous(), vd[0, a:b].contiguous()))
    out = torch.empty((max(s[1] for s in segs), w.hq, w.dv), dtype=w.dtype, device=qd.device)

    def one_pass():
        ksa.ksa_cache_reset(cache, stream=stream)
        for seg, rows, q_, k_, v_ in segs:
            ksa.ksa_prefill_chunk(cache, seg, rows, q_, k_, v_, out=out[:rows], stream=stream)
            ksa.ksa_cache_append_rows(cache, seg, rows, k_, v_, stream=stream)

    one_pass()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        one_pass()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    fl = 2 * (w.dqk + w.dv) * w.hq * visible_pairs(w.n_text, w.chunk, w.window) * w.batch
    del cache, segs, out
    torch.cuda.empty_cache()
    return {"workload": w.name, "segments": n_chunks, "ms": round(ms, 4),
            "tflops": round(fl / (ms * 1e-3) / 1e12, 2)}


def prefill_mla(ksa, ksa_synth, torch, dev, stream, reps: int = 5) -> dict:
    """Absorbed-MLA prefill: 128 heads over one 576/512 latent head."""
    w = ksa_synth.PREFILL_MLA_8K
    L = ksa.ksa_augmented_len(w.n_text, w.chunk)
    g = ksa_synth.gen(w.seed)
    qd = ksa_synth.normal((w.batch, L, w.hq, w.dqk), w.dtype, g).to(dev)
    kd = ksa_synth.normal((w.batch, L, w.hkv, w.dqk), w.dtype, g).to(dev)
    p = ksa.Params(w.chunk, w.window, w.hq, w.hkv, w.dqk, w.dv, w.dtype, v_is_k_prefix=True)
    out = torch.empty((w.batch, L, w.hq, w.dv), dtype=w.dtype, device=dev)
    ksa.ksa_prefill_attn(p, qd, kd, None, w.n_text, out=out, stream=stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        ksa.ksa_prefill_attn(p, qd, kd, None, w.n_text, out=out, stream=stream)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    fl = 2 * (w.dqk + w.dv) * w.hq * visible_pairs(w.n_text, w.chunk, w.window) * w.batch
    tf = fl / (ms * 1e-3) / 1e12
    del qd, kd, out
    torch.cuda.empty_cache()
    return {"workload": w.name, "ms": round(ms, 4), "tflops": round(tf, 2),
            "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "flops": fl}


_ORACLE_INPUTS: dict = {}   # the oracle's fp64 keys and values, kept for the extra lines


def cpu_baseline(w, rows_req: int) -> dict:
    """The fp64 oracle on a bounded sample of the same prefill workload."""
    import numpy as np
    import torch

    import ksa_synth
    from oracle import ksa_oracle as O

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    L = O.augmented_len(w.n_text, w.chunk)
    q, kx, v = ksa_synth.prefill_qkv(w, L)
    pos = O.position_ids(w.n_text, w.chunk)
    kr = O.rope_rotate(kx[0].double().numpy(), pos, w.rope_theta)
    vv = v[0].double().numpy()
    _ORACLE_INPUTS.update(q=q[0], k=kr, v=vv, L=L)
    scale = 1.0 / math.sqrt(w.dqk)
    mask_count = lambda rows: int(O.visibility_mask_fast(w.n_text, w.chunk, w.window, rows=rows).sum())

    def run(nrows):
        rows = np.linspace(0, L - 1, nrows).astype(np.int64)
        qs = np.zeros((L, w.hq, w.dqk))
        qs[rows] = O.rope_rotate(q[0, rows].double().numpy(), pos[rows], w.rope_theta)
        t0 = time.perf_counter()
        O.ksa_attention(qs, kr, vv, w.n_text, w.chunk, w.window, scale, rows=rows, row_block=64)
        dt = time.perf_counter() - t0
        return rows, dt

    nrows = rows_req or 16
    rows, dt = run(nrows)
    for _ in range(3 if not rows_req else 0):   # scale the sample to about 15 s of oracle work
        if dt >= 10.0 or nrows >= 4096:
            break
        nrows = int(min(4096, max(16, nrows * 15.0 / max(dt, 1e-3))))
        rows, dt = run(nrows)
    fl = 2 * (w.dqk + w.dv) * w.hq * mask_count(rows)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(rows)} evenly spaced augmented rows x {w.hq} heads of {w.name} "
                      f"(fp64, dense masked rows), {dt:.1f} s"}


def long_oracle_rates(res: dict, nrows: int = 24) -> None:
    """The fp64 oracle beside each 131072-token line: evenly spaced augmented
    rows x all heads (dense masked rows over the whole sequence), timed, with
    the full workload's time extrapolated from the rate on the sampled rows'
    visible pairs."""
    import numpy as np

    import ksa_synth
    from oracle import ksa_oracle as O

    for line in res.get("prefill_long", []):
        w = {x.name: x for x in (ksa_synth.PREFILL_128K_W64, ksa_synth.PREFILL_128K_W16)}[line["workload"]]
        L = O.augmented_len(w.n_text, w.chunk)
        g = ksa_synth.gen(w.seed)
        # the workload's keys and values (same draws as the GPU line), rotated once
        qb = ksa_synth.normal((L, w.hq, w.dqk), w.dtype, g)
        kb = ksa_synth.normal((L, w.hkv, w.dqk), w.dtype, g).double().numpy()
        vb = ksa_synth.normal((L, w.hkv, w.dv), w.dtype, g).double().numpy()
        pos = O.position_ids(w.n_text, w.chunk)
        kr = O.rope_rotate(kb, pos, w.rope_theta)
        rows = np.linspace(0, L - 1, nrows).astype(np.int64)
        qs = np.zeros((L, w.hq, w.dqk))          # only the sampled rows are touched
        qs[rows] = O.rope_rotate(qb[rows].double().numpy(), pos[rows], w.rope_theta)
        del qb, kb
        t0 = time.perf_counter()
        O.ksa_attention(qs, kr, vb, w.n_text, w.chunk, w.window, 1.0 / math.sqrt(w.dqk), rows=rows, row_block=8)
        dt = time.perf_counter() - t0
        pairs = int(O.visibility_mask_fast(w.n_text, w.chunk, w.window, rows=rows).sum())
        rate = 2 * (w.dqk + w.dv) * w.hq * pairs / dt
        line["cpu_oracle"] = {"tflops": rate / 1e12, "extrapolated_full_s": round(line["flops"] / rate, 1),
                              "sample": f"{nrows} evenly spaced augmented rows x {w.hq} heads (fp64, dense masked "
                                        f"rows over all {L} rows), {dt:.1f} s; full-workload time extrapolated "
                                        f"from the rate"}
        del qs, kr, vb


def extra_oracle_rates(res: dict, w) -> None:
    """The fp64 oracle beside each extra line, on a few seconds of sampled
    rows: backward terms of sampled query rows, MLA prefill rows, baseline
    rows.  Same units as the GPU lines (FLOP over the sampled rows' pairs)."""
    import numpy as np

    import ksa_synth
    from oracle import ksa_oracle as O

    L, kn, vn = _ORACLE_INPUTS["L"], _ORACLE_INPUTS["k"], _ORACLE_INPUTS["v"]
    scale = 1.0 / math.sqrt(w.dqk)
    rows = np.linspace(0, L - 1, 24).astype(np.int64)
    pairs = int(O.visibility_mask_fast(w.n_text, w.chunk, w.window, rows=rows).sum())
    # only the sampled rows' queries and output gradients are read
    qn = np.zeros((L, w.hq, w.dqk))
    qn[rows] = _ORACLE_INPUTS["q"][rows].double().numpy()
    g = np.zeros((L, w.hq, w.dv))
    g[rows] = ksa_synth.normal((len(rows), w.hq, w.dv), w.dtype, ksa_synth.gen(w.seed + 7)).double().numpy()
    t0 = time.perf_counter()
    O.attention_backward_rows(qn, kn, vn, g, w.n_text, w.chunk, scale, rows, C=w.window)
    dt = time.perf_counter() - t0
    fl = 2 * (3 * w.dqk + 2 * w.dv) * w.hq * pairs
    if res.get("prefill_backward"):
        res["prefill_backward"]["cpu_oracle"] = {
            "tflops": fl / dt / 1e12, "sample": f"backward terms of {len(rows)} rows x {w.hq} heads, {dt:.1f} s"}

    for line in res.get("prefill_baselines", []):
        mode = O.MODE_SCA if line["mode"].startswith("sliding") else O.MODE_SWA
        W = w.window * w.chunk
        t0 = time.perf_counter()
        O.baseline_attention(qn, kn, vn, w.n_text, w.chunk, mode, scale, C=w.window, W=W, rows=rows)
        dt = time.perf_counter() - t0
        bp = int(O.baseline_mask(w.n_text, w.chunk, mode, C=w.window, W=W, rows=rows).sum())
        line["cpu_oracle"] = {"tflops": 2 * (w.dqk + w.dv) * w.hq * bp / dt / 1e12,
                              "sample": f"{len(rows)} rows x {w.hq} heads, {dt:.1f} s"}

    # chunked: the segments' rows are the one-shot rows (same rule, keys from
    # the cache regions); rows sampled on both sides of every segment boundary
    if res.get("prefill_chunked"):
        segs = res["prefill_chunked"]["segments"]
        bnd = [L * i // segs for i in range(1, segs)]
        crows = np.unique(np.clip(np.concatenate([[b - 2, b - 1, b, b + 1] for b in bnd]), 0, L - 1))
        qc = np.zeros((L, w.hq, w.dqk))
        qc[crows] = _ORACLE_INPUTS["q"][crows].double().numpy()
        t0 = time.perf_counter()
        O.ksa_attention(qc, kn, vn, w.n_text, w.chunk, w.window, scale, rows=crows, row_block=64)
        dt = time.perf_counter() - t0
        cp = int(O.visibility_mask_fast(w.n_text, w.chunk, w.window, rows=crows).sum())
        rate = 2 * (w.dqk + w.dv) * w.hq * cp / dt
        fl = 2 * (w.dqk + w.dv) * w.hq * visible_pairs(w.n_text, w.chunk, w.window) * w.batch
        res["prefill_chunked"]["cpu_oracle"] = {
            "tflops": rate / 1e12, "extrapolated_full_s": round(fl / rate, 1),
            "sample": f"{len(crows)} rows at the {segs - 1} segment boundaries x {w.hq} heads (fp64, the "
                      f"one-shot rows the segments must equal), {dt:.1f} s; full pass extrapolated from the rate"}
        del qc

    mw = ksa_synth.PREFILL_MLA_8K
    ml = O.augmented_len(mw.n_text, mw.chunk)
    gm = ksa_synth.gen(mw.seed)
    mrows = np.linspace(0, ml - 1, 6).astype(np.int64)
    mq = np.zeros((ml, mw.hq, mw.dqk))
    mq[mrows] = ksa_synth.normal((len(mrows), mw.hq, mw.dqk), mw.dtype, gm).double().numpy()
    mk = ksa_synth.normal((ml, mw.hkv, mw.dqk), mw.dtype, gm).double().numpy()
    t0 = time.perf_counter()
    O.ksa_attention(mq, mk, None, mw.n_text, mw.chunk, mw.window, 1.0 / math.sqrt(mw.dqk), rows=mrows,
                    dv=mw.dv)
    dt = time.perf_counter() - t0
    mp = int(O.visibility_mask_fast(mw.n_text, mw.chunk, mw.window, rows=mrows).sum())
    if res.get("prefill_mla"):
        res["prefill_mla"]["cpu_oracle"] = {
            "tflops": 2 * (mw.dqk + mw.dv) * mw.hq * mp / dt / 1e12,
            "sample": f"{len(mrows)} rows x {mw.hq} heads of {mw.name}, {dt:.1f} s"}

    # one decode query per workload, against its whole logical history
    for key, dw in (("decode", ksa_synth.DECODE_GQA), ("decode_mla", ksa_synth.DECODE_MLA)):
        if key not in res:
            continue
        n = ksa_synth.decode_histories(dw)[0]
        A = O.text_row(n - 1, dw.chunk) + 1
        gd = ksa_synth.gen(dw.seed + 11)
        hk = ksa_synth.normal((A, dw.hkv, dw.dqk), dw.dtype, gd).double().numpy()
        hv = None if dw.v_is_k_prefix else ksa_synth.normal((A, dw.hkv, dw.dv), dw.dtype, gd).double().numpy()
        # the oracle's time is linear in the query heads: time at most 16 and scale
        nh = min(dw.hq, 16 if dw.hkv == 1 else dw.hq)
        dq1 = ksa_synth.decode_query(dw)[0, :nh].double().numpy()
        t0 = time.perf_counter()
        O.decode_attention(dq1, hk, hv, n, dw.chunk, dw.window, 1.0 / math.sqrt(dw.dqk), "t", dv=dw.dv)
        dt = (time.perf_counter() - t0) * dw.hq / nh
        m = (n - 1) // dw.chunk
        rows1 = n - m * dw.chunk + min(m, dw.window) * dw.chunk + max(0, m - dw.window)
        width = dw.dqk if dw.v_is_k_prefix else dw.dqk + dw.dv
        nbytes = rows1 * dw.hkv * width * 2 + dw.hq * (dw.dqk + dw.dv) * 2
        res[key]["cpu_oracle"] = {"gbps": nbytes / dt / 1e9,
                                  "sample": f"one {n}-token sequence of {dw.name}, {nh} of {dw.hq} "
                                            f"query heads timed, {dt:.2f} s scaled"}
        del hk, hv


if __name__ == "__main__":
    sys.exit(main())
