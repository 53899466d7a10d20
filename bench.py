#!/usr/bin/env python3
"""Throughput of exact tiled attention on one MI355X, as one JSON line.

A step is one pass of the whole hot path over one batch of synthetic input: the
forward (O and the per-row log-sum-exp) followed by the recomputing backward
(dQ, dK, dV) of a LLaMA-7B-shaped causal attention layer, B=2, H=32, L=4096,
d=128, bf16 inputs with fp32 accumulation.  Inputs are seeded Gaussians already
resident in HBM when the timed region starts.

FLOPs are counted algorithmically: forward 4*B*Hq*L^2*d, halved for causal
(the allowed band for a sliding window); backward 2.5x the forward (five
matrix products, the recomputation of Q K^T included).

Besides the headline step, the line carries a "configs" object with forward (and,
where the workload has one, backward) time, TFLOP/s and fraction of peak for every
workload of the method's configuration list (fp32 tiny, the LLaMA-7B layer, GQA 16k,
sliding window 32k, 128k forward, 8k backward), plus the extra device memory each
call allocates beyond its inputs and outputs.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-configs]
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0              # MI355X HBM3E, published
PEAK_FP32_VECTOR_TFLOPS = 157.3    # MI355X fp32 vector ALU, published
# The published bf16 figure assumes 2.4 GHz; under sustained MFMA load the shader
# clock measured about 2.1 GHz (s_memtime against the 100 MHz s_memrealtime
# across an MFMA loop), so the peak at the measured clock is 2.5 PF * 2.1 / 2.4.
MEASURED_MFMA_CLOCK_GHZ = 2.1
PEAK_BF16_AT_MEASURED_CLOCK_TFLOPS = PEAK_BF16_TFLOPS * MEASURED_MFMA_CLOCK_GHZ / 2.4
METRIC = "attention fwd/bwd TFLOP/s + % bf16 MFMA peak, B2 H32 L4096 d128 causal"


def window_pairs(L, w, causal):
    """Allowed (query, key) pairs of one L x L head under a window w >= 1: one-sided
    (keys i-w+1..i) with causal, |i - j| < w without."""
    w = min(int(w), int(L))
    one_sided = w * L - w * (w - 1) // 2
    return one_sided if causal else 2 * one_sided - L


def fwd_flops(B, Hq, L, d, causal, window):
    """4*d flops per allowed (query, key) pair: the two products S = QK^T and P.V."""
    if window and window > 0:
        return 4.0 * B * Hq * d * window_pairs(L, window, causal)
    full = 4.0 * B * Hq * L * L * d
    return full / 2 if causal else full


def bwd_flops(B, Hq, L, d, causal, window):
    return 2.5 * fwd_flops(B, Hq, L, d, causal, window)


def score_matrix_bytes(B, H, L, elt=2):
    """Bytes of the full L x L score matrix of one layer (what the tiled method never stores)."""
    return elt * B * H * L * L


def fwd_bytes(B, Hq, Hkv, L, d, elt=2):
    """Algorithmic HBM bytes of one forward: Q, K, V read once; O and LSE written."""
    return (B * Hq * L * d + 2 * B * Hkv * L * d) * elt + B * Hq * L * d * elt + B * Hq * L * 4


def allowed_pairs(L, causal=False, window=0, global_tokens=(), block_mask=None, block=64):
    """Number of allowed (query, key) pairs of the general mask over one sequence of
    length L (the same rule as ``MaskPlan``): the algorithmic work of one head is
    4 * d * allowed_pairs flops forward.  Counted on the host: per row in interval form
    without a block mask, else over row chunks of the boolean mask."""
    import torch
    L = int(L)
    glob = sorted({(p + L if p < 0 else p) for p in global_tokens if -L <= p < L})
    if block_mask is None:
        # interval form: row i's local keys are one interval [lo, hi]; the global
        # keys outside it (and visible under the causal mask) are added, and a
        # global row sees every visible key
        i = torch.arange(L, dtype=torch.int64)
        hi = i.clone() if causal else torch.full((L,), L - 1, dtype=torch.int64)
        lo = torch.zeros(L, dtype=torch.int64)
        if window > 0:
            lo = (i - window + 1).clamp_min(0)
            if not causal:
                hi = (i + window - 1).clamp_max(L - 1)
        g = torch.tensor(glob, dtype=torch.int64)
        inside = torch.searchsorted(g, hi, right=True) - torch.searchsorted(g, lo, right=False)
        visible = torch.searchsorted(g, i, right=True) if causal else torch.full((L,), len(glob), dtype=torch.int64)
        count = hi - lo + 1 + visible - inside
        if glob:
            count[g] = (g + 1) if causal else L
        return int(count.sum())
    is_g = torch.zeros(L, dtype=torch.bool)
    if glob:
        is_g[torch.tensor(glob)] = True
    bm = torch.as_tensor(block_mask).bool().cpu()
    total = 0
    chunk = max(1, (1 << 24) // L)
    j = torch.arange(L)
    for r0 in range(0, L, chunk):
        i = torch.arange(r0, min(L, r0 + chunk))[:, None]
        local = torch.ones(i.shape[0], L, dtype=torch.bool)
        if window > 0:
            local &= (i - j[None, :]).abs() < window
        local &= bm[(i // block), (j // block)[None, :]]
        ok = local | is_g[i] | is_g[None, :]
        if causal:
            ok &= j[None, :] <= i
        total += int(ok.sum())
    return total


# The sources each timed kernel is compiled from: a counter reading stays valid
# while these files are unchanged.
KERNEL_SOURCES = {
    "fwd_bf16_kernel<128,causal>": ("fa_fwd_bf16.hip", "fa_fwd_tile.hpp", "fa_common.hpp", "fa_kernels.h"),
    "bwd_dkdv_kernel<128,causal>": ("fa_bwd_bf16.hip", "fa_bwd_tile.hpp", "fa_common.hpp", "fa_kernels.h"),
    "bwd_dq_kernel<128,causal>": ("fa_bwd_bf16.hip", "fa_bwd_tile.hpp", "fa_common.hpp", "fa_kernels.h"),
    "bwd_delta_kernel<128>": ("fa_bwd_bf16.hip", "fa_bwd_tile.hpp", "fa_common.hpp", "fa_kernels.h"),
}


def kernel_source_digest(kernel_key=None):
    """Digest of the kernel sources: those of one timed kernel, or all of them."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_tiled_attention_flash_amd", "csrc")
    names = KERNEL_SOURCES[kernel_key] if kernel_key else sorted(
        f for f in os.listdir(csrc) if f.endswith((".hip", ".hpp", ".h")))
    for f in names:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key):
    """HBM traffic per launch from committed rocprofv3 counter runs, or None if stale/absent."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        data = json.load(open(p))
        ent = data.get(kernel_key)
        if not ent or ent.get("source_digest") != kernel_source_digest(kernel_key):
            return None
        return float(ent["bytes_per_launch"])
    except Exception:
        return None


def host_cores():
    """Host CPU counts and the BLAS threads the oracle runs with."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    try:
        affinity = len(os.sched_getaffinity(0))
    except Exception:
        affinity = None
    return {"blas_threads": threads, "os_cpu_count": os.cpu_count(), "affinity": affinity}


def cpu_baseline(budget_s=20.0):
    """Time the fp64 oracle on a bounded sample of the headline workload (rank 0 only)."""
    import numpy as np
    import oracle
    import workloads as W
    cores = host_cores()
    w = W.LLAMA7B_CAUSAL
    q, k, v, do = W.make_inputs(w, with_dout=True)
    qn, kn, vn, don = (t.float().numpy() for t in (q, k, v, do))
    flops = 0.0
    heads = 0
    t0 = time.perf_counter()
    # forward, one (batch, head) at a time, until about half the budget is spent
    for h in range(w.Hq):
        oracle.forward(qn[:1, h:h + 1], kn[:1, h:h + 1], vn[:1, h:h + 1], w.scale, True, 0)
        flops += fwd_flops(1, 1, w.L, w.d, True, 0)
        heads += 1
        if time.perf_counter() - t0 > budget_s / 2:
            break
    t_f = time.perf_counter() - t0
    t1 = time.perf_counter()
    bheads = 0
    for h in range(w.Hq):
        oracle.backward(qn[:1, h:h + 1], kn[:1, h:h + 1], vn[:1, h:h + 1], don[:1, h:h + 1], w.scale, True, 0)
        flops += bwd_flops(1, 1, w.L, w.d, True, 0)
        bheads += 1
        if time.perf_counter() - t1 > budget_s / 2:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores["blas_threads"], "kind": "oracle",
            "host": cores,
            "sample": f"fp64 NumPy oracle on {heads} head(s) forward + {bheads} head(s) backward "
                      f"of B2 H32 L4096 d128 causal (each one full 4096x4096 head); "
                      f"{dt:.1f} s wall, {t_f:.1f} s of it forward"}


def _sample_rows(L, window, n_random=256, seed=0):
    """Rows timed for the long workloads: 0, 1, the 64-row tile edges near the
    start and end, w - 1 and w for a window, L - 1, and seeded random rows."""
    import numpy as np
    fixed = {0, 1, 63, 64, 127, 128, L // 2, L - 65, L - 64, L - 2, L - 1}
    if window:
        fixed |= {window - 1, window, window + 1}
    rng = np.random.default_rng(seed)
    rows = sorted(fixed | set(int(x) for x in rng.integers(0, L, n_random)))
    return np.array([r for r in rows if 0 <= r < L])


def cpu_baseline_configs():
    """The oracle timed on every workload of the configuration list (a baseline only).

    Whole (batch, head) slices where one fits in a few seconds (tiny fp32: every head;
    the 4k layer: one head forward and backward; the 8k backward: one head), sampled
    query rows elsewhere (exact for those rows).  Each entry gives the timed sample,
    its algorithmic TFLOP/s and the time of the full workload extrapolated from it,
    labelled as such."""
    import numpy as np
    import oracle
    import workloads as W
    out = {"host": host_cores(), "note": "fp64 NumPy oracle, untuned; extrapolated_full_s is "
                                         "sample time x (full work / sampled work), not a measurement"}

    def entry(name, sample, secs, flops_sample, flops_full):
        out[name] = {"sample": sample, "seconds": round(secs, 3),
                     "algorithmic_tflops": round(flops_sample / secs / 1e12, 5),
                     "extrapolated_full_s": round(secs * flops_full / flops_sample, 1)}

    def head_inputs(w, h=0):
        q, k, v, do = W.make_inputs(w, with_dout=w.backward)
        hk = h // (w.Hq // w.Hkv)
        sl = lambda t, hh: t[:1, hh:hh + 1].float().numpy()
        return sl(q, h), sl(k, hk), sl(v, hk), (sl(do, h) if do is not None else None)

    # tiny fp32: the whole workload
    w = W.TINY_FP32
    q, k, v, _ = (t.float().numpy() if t is not None else None for t in W.make_inputs(w))
    t0, n = time.perf_counter(), 0
    while n < 3 or time.perf_counter() - t0 < 0.5:
        oracle.forward(q, k, v, w.scale, w.causal, w.window)
        n += 1
    ff = fwd_flops(w.B, w.Hq, w.L, w.d, w.causal, w.window)
    entry(w.name + " fwd", "every head (whole workload), mean of %d calls" % n, (time.perf_counter() - t0) / n, ff, ff)
    # the 4k layer and the 8k backward: one whole head, forward and backward
    for w in (W.LLAMA7B_CAUSAL, W.LONG_BWD_8K):
        q, k, v, do = head_inputs(w)
        one_f = fwd_flops(1, 1, w.L, w.d, w.causal, w.window)
        full_f = fwd_flops(w.B, w.Hq, w.L, w.d, w.causal, w.window)
        if w is W.LLAMA7B_CAUSAL:
            t0 = time.perf_counter()
            oracle.forward(q, k, v, w.scale, w.causal, w.window)
            entry(w.name + " fwd", "1 of %d (batch, head) slices" % (w.B * w.Hq), time.perf_counter() - t0,
                  one_f, full_f)
        t0 = time.perf_counter()
        oracle.backward(q, k, v, do, w.scale, w.causal, w.window)
        entry(w.name + " bwd", "1 of %d (batch, head) slices" % (w.B * w.Hq), time.perf_counter() - t0,
              2.5 * one_f, 2.5 * full_f)
    # long rows: sampled query rows of one head
    for w in (W.GQA_16K, W.WINDOW_32K, W.LONG_FWD_128K, W.LONG_BWD_8K):
        q, k, v, _ = head_inputs(w)
        rows = _sample_rows(w.L, w.window)
        ok = oracle.allowed_mask(rows, w.L, w.causal, w.window)
        t0 = time.perf_counter()
        oracle.forward_rows(q, k, v, rows, w.scale, w.causal, w.window)
        secs = time.perf_counter() - t0
        pairs = float(ok.sum())
        full_f = fwd_flops(w.B, w.Hq, w.L, w.d, w.causal, w.window)
        entry(w.name + " fwd", "%d sampled query rows of 1 of %d heads" % (rows.size, w.B * w.Hq), secs,
              4.0 * w.d * pairs, full_f)
    return out


# The pages' own figures, reported beside the measurement as context (other hardware;
# none is a target): claspmoon.cn "14 · 缩放定律与高效注意力" §3.1 (A100 bandwidths), §2.1
# (the full score matrix of the LLaMA-7B-shaped layer); book.anysome.cn "高效注意力" §2
# (speed-up claimed over naive attention).
PAGES_CONTEXT = {
    "a100_hbm_tb_s": 2.0,
    "a100_on_chip_sram_tb_s": 19.0,
    "claimed_speedup_vs_naive_attention": "2-4x",
    "score_matrix_gb_per_layer_fp16_B2_H32_L4096": 2.15,
    "mi355x_hbm_tb_s": PEAK_HBM_GBS / 1000.0,
}


def time_calls(fn, iters, warmup, warm_ms=150.0):
    """Median and mean of `iters` calls, each bracketed by HIP events on the current stream.

    Warm-up runs at least `warmup` calls and at least `warm_ms` of them: after a light
    phase the clocks take on the order of 100 ms to ramp back up."""
    import time
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < warmup or (time.perf_counter() - t0) * 1e3 < warm_ms:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[len(t) // 2], sum(t) / len(t)


def measure_config(w, iters=10, warmup=3):
    """Forward (and backward) timing of one workload, with its extra device memory."""
    import torch
    import exact_tiled_attention_flash_amd as fa
    import workloads as W
    dev = torch.device("cuda:0")
    q, k, v, do = W.make_inputs(w, with_dout=w.backward)
    q, k, v = (t.to(dev) for t in (q, k, v))
    do = do.to(dev) if do is not None else None
    o = torch.empty_like(q)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    _, lse = fa.fwd(q, k, v, causal=w.causal, window=w.window, scale=w.scale, out=o)
    torch.cuda.synchronize()
    fwd_extra = torch.cuda.max_memory_allocated() - base
    ff = fwd_flops(w.B, w.Hq, w.L, w.d, w.causal, w.window)
    fp32 = w.dtype == torch.float32
    peak = PEAK_FP32_VECTOR_TFLOPS if fp32 else PEAK_BF16_TFLOPS
    med, mean = time_calls(lambda: fa.fwd(q, k, v, causal=w.causal, window=w.window, scale=w.scale, out=o, lse=lse),
                           iters, warmup)
    tf = ff / (med * 1e-3) / 1e12
    dname = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}[w.dtype]
    r = {"shape": f"B{w.B} Hq{w.Hq} Hkv{w.Hkv} L{w.L} d{w.d}", "dtype": dname,
         "causal": w.causal, "window": w.window,
         "fwd": {"ms_median": round(med, 4), "ms_mean": round(mean, 4), "tflop": ff / 1e12,
                 "tflops": round(tf, 2), "peak_tflops": peak, "frac_peak": round(tf / peak, 4),
                 "extra_mem_bytes": int(fwd_extra)}}
    if w.backward:
        nbytes = fa.bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.L, w.d, w.dtype)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        run = lambda: fa.bwd(q, k, v, o, lse, do, causal=w.causal, window=w.window, scale=w.scale,
                             workspace=ws, dq=dq, dk=dk, dv=dv)
        bmed, bmean = time_calls(run, iters, warmup)
        bf = bwd_flops(w.B, w.Hq, w.L, w.d, w.causal, w.window)
        btf = bf / (bmed * 1e-3) / 1e12
        r["bwd"] = {"ms_median": round(bmed, 4), "ms_mean": round(bmean, 4), "tflop": bf / 1e12,
                    "tflops": round(btf, 2), "peak_tflops": peak, "frac_peak": round(btf / peak, 4),
                    "extra_mem_bytes": int(nbytes)}
    del q, k, v, do, o, lse
    torch.cuda.empty_cache()
    return r


def measure_bwd_fused(iters=10, warmup=3):
    """The single-kernel backward (dQ accumulated with float32 atomics) against the
    staged one (dQ recomputing S and dP) on the LLaMA-7B-shaped layer and the 8k
    backward workload: both compute the same five products' worth of gradient."""
    import torch
    import exact_tiled_attention_flash_amd as fa
    import workloads as W
    out = {}
    dev = torch.device("cuda:0")
    for w in (W.LLAMA7B_CAUSAL, W.LONG_BWD_8K):
        q, k, v, do = (t.to(dev) for t in W.make_inputs(w, with_dout=True))
        o, lse = fa.fwd(q, k, v, causal=True, scale=w.scale)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(fa.bwd_fused_workspace_bytes(w.B, w.Hq, w.Hkv, w.L, w.d), dtype=torch.uint8, device=dev)
        fmed, _ = time_calls(lambda: fa.bwd_fused(q, k, v, o, lse, do, causal=True, scale=w.scale, workspace=ws,
                                                  dq=dq, dk=dk, dv=dv), iters, warmup)
        smed, _ = time_calls(lambda: fa.bwd(q, k, v, o, lse, do, causal=True, scale=w.scale, workspace=ws,
                                            dq=dq, dk=dk, dv=dv), iters, warmup)
        bf = bwd_flops(w.B, w.Hq, w.L, w.d, True, 0)
        out[w.name] = {"fused_ms": round(fmed, 4), "staged_ms": round(smed, 4),
                       "fused_tflops": round(bf / (fmed * 1e-3) / 1e12, 2),
                       "staged_tflops": round(bf / (smed * 1e-3) / 1e12, 2),
                       "fused_workspace_bytes": int(ws.numel())}
        del q, k, v, do, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    return out


def decode_cache_reads(Hq, Hkv, Lq):
    """How often a decode call reads each K/V head: once per work-group, which
    serves up to four groups of 32 rows (query heads x new tokens)."""
    groups = (Hq // Hkv * Lq + 31) // 32
    per_wg = 1 if groups == 1 else 2 if groups == 2 else 4
    return (groups + per_wg - 1) // per_wg


def measure_decode(B=8, Hq=32, Hkv=8, Lq=1, Lk=32768, d=128, iters=20, warmup=5):
    """KV-cache decode: Lq new tokens per sequence (1, or a chunk as in speculative
    decoding) against a 32k-entry GQA cache.

    The call reads the whole cache once (HBM-bound), so it is reported as bytes of
    K and V read per second against the HBM peak."""
    import torch
    import exact_tiled_attention_flash_amd as fa
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(9)
    q = torch.randn(B, Hq, Lq, d, generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn(B, Hkv, Lk, d, generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn(B, Hkv, Lk, d, generator=g, device=dev).to(torch.bfloat16)
    ws = torch.empty(fa.decode_workspace_bytes(B, Hq, Hkv, Lq, Lk, d), dtype=torch.uint8, device=dev)
    o, lse = torch.empty_like(q), torch.empty(B, Hq, Lq, device=dev)
    med, mean = time_calls(lambda: fa.decode(q, k, v, None, causal=True, workspace=ws, out=o, lse=lse), iters, warmup)
    cache_bytes = 2 * B * Hkv * Lk * d * 2
    gbs = cache_bytes / (med * 1e-3) / 1e9
    return {"shape": f"B{B} Hq{Hq} Hkv{Hkv} new tokens {Lq} cache {Lk} d{d} bf16 causal",
            "ms_median": round(med, 4), "ms_mean": round(mean, 4), "cache_bytes": cache_bytes,
            "cache_reads": decode_cache_reads(Hq, Hkv, Lq),
            "hbm_gbs": round(gbs, 1), "peak_gbs": PEAK_HBM_GBS, "frac_peak": round(gbs / PEAK_HBM_GBS, 4),
            "workspace_bytes": int(ws.numel()), "data": "synthetic N(0,1), generated on the device"}


def measure_decode_rolling(B=8, Hq=32, Hkv=8, W=4096, d=128, iters=20, warmup=5):
    """Decode over a full rolling window buffer of W slots (the sequences have seen
    far more than W tokens, so the buffer has wrapped), for 1 and 16 new tokens per
    sequence.  HBM-bound like the plain decode: reported as bytes of the buffer and
    the new tokens' K/V read per second against the HBM peak."""
    import torch
    import exact_tiled_attention_flash_amd as fa
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(10)
    kr = torch.randn(B, Hkv, W, d, generator=g, device=dev).to(torch.bfloat16)
    vr = torch.randn(B, Hkv, W, d, generator=g, device=dev).to(torch.bfloat16)
    seen = torch.tensor([5 * W + 123 * b for b in range(B)], dtype=torch.int32, device=dev)
    out = {}
    for Lq in (1, 16):
        q = torch.randn(B, Hq, Lq, d, generator=g, device=dev).to(torch.bfloat16)
        kn = torch.randn(B, Hkv, Lq, d, generator=g, device=dev).to(torch.bfloat16)
        vn = torch.randn(B, Hkv, Lq, d, generator=g, device=dev).to(torch.bfloat16)
        ws = torch.empty(fa.decode_rolling_workspace_bytes(B, Hq, Hkv, Lq, W, d), dtype=torch.uint8, device=dev)
        o, lse = torch.empty_like(q), torch.empty(B, Hq, Lq, device=dev)
        med, mean = time_calls(lambda: fa.decode_rolling(q, kr, vr, kn, vn, seen, workspace=ws, out=o, lse=lse),
                               iters, warmup)
        nbytes = 2 * B * Hkv * (W + Lq) * d * 2
        gbs = nbytes / (med * 1e-3) / 1e9
        out[f"new tokens {Lq}"] = {
            "ms_median": round(med, 4), "ms_mean": round(mean, 4), "kv_bytes": nbytes,
            "buffer_reads": decode_cache_reads(Hq, Hkv, Lq),
            "hbm_gbs": round(gbs, 1), "peak_gbs": PEAK_HBM_GBS, "frac_peak": round(gbs / PEAK_HBM_GBS, 4),
            "workspace_bytes": int(ws.numel())}
    return {"shape": f"B{B} Hq{Hq} Hkv{Hkv} rolling buffer W={W} (wrapped) d{d} bf16", **out,
            "data": "synthetic N(0,1), generated on the device"}


def measure_autograd(iters=10, warmup=3):
    """The differentiable drop-in on the headline shape: scaled_dot_product_attention
    (forward, then backward through autograd) against the same two calls made directly,
    so the difference is what the autograd route adds."""
    import torch
    import exact_tiled_attention_flash_amd as fa
    import workloads as W
    w = W.LLAMA7B_CAUSAL
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in W.make_inputs(w, with_dout=True))
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))

    def through_autograd():
        o = fa.scaled_dot_product_attention(qa, ka, va, is_causal=True)
        o.backward(do)
        qa.grad = ka.grad = va.grad = None

    def direct():
        o, lse = fa.fwd(q, k, v, causal=True)
        fa.bwd(q, k, v, o, lse, do, causal=True)

    # A training loop issues step after step: time back-to-back calls between two
    # events, the two routes alternated three times, and report the host's issue
    # time per call beside it.
    import time

    def loop_ms(fn, n):
        time_calls(fn, 1, warmup)                 # warm-up (clocks, allocator)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        t1 = time.perf_counter()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n, (t1 - t0) * 1e3 / n

    n = max(iters, 20)
    runs = {"autograd": [], "direct": []}
    for _ in range(3):
        runs["autograd"].append(loop_ms(through_autograd, n))
        runs["direct"].append(loop_ms(direct, n))
    amed = sorted(r[0] for r in runs["autograd"])[1]
    dmed = sorted(r[0] for r in runs["direct"])[1]
    ahost = sorted(r[1] for r in runs["autograd"])[1]
    dhost = sorted(r[1] for r in runs["direct"])[1]
    flops = fwd_flops(w.B, w.Hq, w.L, w.d, True, 0) * 3.5
    return {"shape": "B2 H32 L4096 d128 causal bf16 (forward + backward)",
            "timing": "%d back-to-back calls between two HIP events, median of 3 alternated runs" % n,
            "autograd_ms": round(amed, 4), "direct_ms": round(dmed, 4),
            "autograd_tflops": round(flops / (amed * 1e-3) / 1e12, 2),
            "overhead_frac": round(amed / dmed - 1.0, 4),
            "host_issue_ms": {"autograd": round(ahost, 4), "direct": round(dhost, 4)}}


def measure_ring(iters=10, warmup=3):
    """One GPU's share of ring attention: a 131072-token causal sequence on 8 GPUs gives
    each GPU a 16384-token query chunk that meets every key/value chunk in turn.  Times
    the chunk-pair forward and backward on an off-diagonal block (queries after all keys:
    no mask, 16384 x 16384) and on the diagonal block (causal inside the chunk), and the
    exact merge of two partials (HBM-bound: reads two O and LSE, writes one)."""
    import torch
    import exact_tiled_attention_flash_amd as fa
    B, H, C, d = 1, 32, 16384, 128
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(11)
    q, k, v, do = (torch.randn(B, H, C, d, generator=g, device=dev).to(torch.bfloat16) for _ in range(4))
    s = 1.0 / math.sqrt(d)
    out = {"shape": f"B{B} H{H} chunk {C} d{d} bf16 causal (131072 tokens / 8)",
           "data": "synthetic N(0,1), generated on the device"}
    o, lse = torch.empty_like(q), torch.empty(B, H, C, dtype=torch.float32, device=dev)
    ws = torch.empty(fa.bwd_workspace_bytes(B, H, H, C, d), dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    for name, qo, ko, flops in (("off_diagonal", C, 0, 4.0 * B * H * C * C * d),
                                ("diagonal", 0, 0, 2.0 * B * H * C * C * d)):
        fmed, _ = time_calls(lambda: fa.fwd_block(q, k, v, causal=True, q_offset=qo, k_offset=ko, scale=s,
                                                  out=o, lse=lse), iters, warmup)
        bmed, _ = time_calls(lambda: fa.bwd_block(q, k, v, o, lse, do, causal=True, q_offset=qo, k_offset=ko,
                                                  scale=s, workspace=ws, dq=dq, dk=dk, dv=dv), iters, warmup)
        ftf, btf = flops / (fmed * 1e-3) / 1e12, 2.5 * flops / (bmed * 1e-3) / 1e12
        out[name] = {"fwd_ms": round(fmed, 4), "fwd_tflops": round(ftf, 2),
                     "fwd_frac_peak": round(ftf / PEAK_BF16_TFLOPS, 4),
                     "bwd_ms": round(bmed, 4), "bwd_tflops": round(btf, 2),
                     "bwd_frac_peak": round(btf / PEAK_BF16_TFLOPS, 4)}
    ob, lb = torch.empty_like(q), torch.empty_like(lse)
    fa.fwd_block(q, k, v, causal=True, q_offset=C, k_offset=0, scale=s, out=ob, lse=lb)
    mo, ml = torch.empty_like(q), torch.empty_like(lse)
    mmed, _ = time_calls(lambda: fa.merge(o, lse, ob, lb, out=mo, lse_out=ml), iters, warmup)
    mbytes = 3 * B * H * C * d * 2 + 3 * B * H * C * 4
    mgbs = mbytes / (mmed * 1e-3) / 1e9
    out["merge"] = {"ms": round(mmed, 4), "bytes": mbytes, "hbm_gbs": round(mgbs, 1),
                    "frac_peak": round(mgbs / PEAK_HBM_GBS, 4)}
    del q, k, v, do, o, lse, ws, dq, dk, dv, ob, lb, mo, ml
    torch.cuda.empty_cache()
    return out


def measure_sparse(iters=5, warmup=2, block_band=False):
    """General sparse mask, forward and backward under one mask plan: by default the
    hybrid configuration (window reaching 512 positions both ways, first and last
    token global, 131072 tokens, batch 2) on 32 heads of 128; with `block_band` the
    banded block-sparse mask (blocks of 128, radius 1) at the same size.

    Reported as effective TFLOP/s over the allowed pairs only (4 d flops per pair
    forward, 2.5x that backward): the work the mask leaves is the algorithmic work."""
    import torch
    import exact_tiled_attention_flash_amd as fa
    import workloads as W
    w = W.BLOCK_BAND_128K if block_band else W.HYBRID_SPARSE_128K
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(w.seed)
    q, k, v, do = (torch.randn(w.B, h, w.L, w.d, generator=g, device=dev).to(w.dtype)
                   for h in (w.Hq, w.Hkv, w.Hkv, w.Hq))
    bm = W.block_band_mask(w.L, W.BLOCK_BAND_BLOCK, W.BLOCK_BAND_RADIUS) if block_band else None
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s0.record()
    plan = fa.MaskPlan(w.L, causal=w.causal, window=w.window, global_tokens=w.global_tokens, block_mask=bm,
                       block=W.BLOCK_BAND_BLOCK, device=dev)
    s1.record()
    torch.cuda.synchronize()
    plan_ms = s0.elapsed_time(s1)
    pairs = allowed_pairs(w.L, w.causal, w.window, w.global_tokens, bm, W.BLOCK_BAND_BLOCK)
    o, lse = torch.empty_like(q), torch.empty(w.B, w.Hq, w.L, dtype=torch.float32, device=dev)
    fws = fa.masked_workspace_bytes(w.B, w.Hq, w.Hkv, w.L, w.d, plan, False)
    bws = fa.masked_workspace_bytes(w.B, w.Hq, w.Hkv, w.L, w.d, plan, True)
    fw = torch.empty(max(fws, 256), dtype=torch.uint8, device=dev)
    bw = torch.empty(bws, dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fmed, fmean = time_calls(lambda: fa.fwd_masked(q, k, v, plan, scale=w.scale, out=o, lse=lse, workspace=fw),
                             iters, warmup)
    bmed, bmean = time_calls(lambda: fa.bwd_masked(q, k, v, o, lse, do, plan, scale=w.scale, workspace=bw,
                                                   dq=dq, dk=dk, dv=dv), iters, warmup)
    ff = 4.0 * w.d * pairs * w.B * w.Hq
    bf = 2.5 * ff
    ftf, btf = ff / (fmed * 1e-3) / 1e12, bf / (bmed * 1e-3) / 1e12
    mask_desc = (f"band of radius {W.BLOCK_BAND_RADIUS} over {W.BLOCK_BAND_BLOCK}-token blocks" if block_band
                 else None)
    out = {"workload": w.name, "mask": {"causal": w.causal, "window": w.window,
                                        "global_tokens": list(w.global_tokens), "block_mask": mask_desc},
           "allowed_pairs": pairs, "pairs_per_row": round(pairs / w.L, 2), "density": pairs / float(w.L) ** 2,
           "plan_ms": round(plan_ms, 3), "plan_bytes": int(plan.plan.numel()),
           "fwd": {"ms_median": round(fmed, 4), "ms_mean": round(fmean, 4), "tflop": ff / 1e12,
                   "tflops": round(ftf, 2), "frac_peak": round(ftf / PEAK_BF16_TFLOPS, 4),
                   "workspace_bytes": int(fws)},
           "bwd": {"ms_median": round(bmed, 4), "ms_mean": round(bmean, 4), "tflop": bf / 1e12,
                   "tflops": round(btf, 2), "frac_peak": round(btf / PEAK_BF16_TFLOPS, 4),
                   "workspace_bytes": int(bws)},
           "data": "synthetic N(0,1), generated on the device"}
    del q, k, v, do, o, lse, dq, dk, dv, fw, bw, plan
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload table")
    ap.add_argument("--sparse-only", action="store_true",
                    help="only the general-mask workload (for profiling its kernels); prints its JSON")
    ap.add_argument("--ring-only", action="store_true",
                    help="only the ring-attention chunk-pair workload; prints its JSON")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the KV-cache decode workload; prints its JSON")
    ap.add_argument("--bwd-fused-only", action="store_true",
                    help="only the fused (atomic dQ) against the staged backward; prints its JSON")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (3x), so that HBM counters "
                         "(FETCH_SIZE/WRITE_SIZE) can be scaled against a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads and batches would shard with no communication).", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_tiled_attention_flash_amd as fa
    import workloads as W

    fa.library()
    dev = torch.device("cuda:0")
    if args.sparse_only:
        print(json.dumps({"sparse": measure_sparse(iters=args.steps, warmup=args.warmup),
                          "sparse_block": measure_sparse(iters=args.steps, warmup=args.warmup, block_band=True)}),
              flush=True)
        return
    if args.ring_only:
        print(json.dumps({"ring": measure_ring(iters=args.steps, warmup=args.warmup)}), flush=True)
        return
    if args.decode_only:
        print(json.dumps({"decode": measure_decode(iters=args.steps, warmup=args.warmup),
                          "decode_16": measure_decode(Lq=16, iters=args.steps, warmup=args.warmup),
                          "decode_rolling": measure_decode_rolling(iters=args.steps, warmup=args.warmup)}),
              flush=True)
        return
    if args.bwd_fused_only:
        print(json.dumps({"bwd_fused": measure_bwd_fused(iters=args.steps, warmup=args.warmup)}), flush=True)
        return
    if args.calibrate_copy:
        src = torch.ones(64 * 2**20, dtype=torch.float32, device=dev)    # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = W.LLAMA7B_CAUSAL
    q, k, v, do = W.make_inputs(w, with_dout=True)
    q, k, v, do = (t.to(dev) for t in (q, k, v, do))
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.Hq, w.L, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.L, w.d), dtype=torch.uint8, device=dev)

    def run_fwd():
        fa.fwd(q, k, v, causal=True, scale=w.scale, out=o, lse=lse)

    def run_bwd():
        fa.bwd(q, k, v, o, lse, do, causal=True, scale=w.scale, workspace=ws, dq=dq, dk=dk, dv=dv)

    def run_bwd_stages(between=None):
        fa.bwd_stages(q, k, v, o, lse, do, causal=True, scale=w.scale, workspace=ws, dq=dq, dk=dk, dv=dv,
                      between=between)

    run_fwd()
    run_bwd()
    torch.cuda.synchronize()
    # Warm-up: the W steps asked for, and more untimed steps until 300 ms have
    # passed -- from idle the clocks take on the order of 100 ms to ramp up (the
    # kernel trace shows dK/dV at 0.64 ms in the first steps and 0.57 ms once
    # settled), so the timed steps measure the sustained rate.
    t_warm = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - t_warm < 0.3:
        run_fwd()
        run_bwd()
        n_warm += 1
        if n_warm % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    # The timed region: exactly K steps (forward + backward), nothing else on
    # the stream, bracketed by synchronisations and two HIP events.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        run_fwd()
        run_bwd()
    t_end.record()
    torch.cuda.synchronize()

    # Per-kernel times: K more steps with the forward and the backward's three
    # stages (the same kernels flash_attn_bwd runs) each bracketed by HIP events
    # on the stream they run on (torch's current stream).
    names = ("fwd", "preprocess", "dkdv", "dq")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    for i in range(args.steps):
        e = ev[i]
        e[0].record()
        run_fwd()
        e[1].record()
        marks = iter(e[2:])
        run_bwd_stages(between=lambda _name: next(marks).record())
    torch.cuda.synchronize()

    total_ms = t_start.elapsed_time(t_end)
    per = {n: [e[j].elapsed_time(e[j + 1]) for e in ev] for j, n in enumerate(names)}
    avg = {n: sum(x) / len(x) for n, x in per.items()}
    med = {n: sorted(x)[len(x) // 2] for n, x in per.items()}
    ms_step = total_ms / args.steps
    ff = fwd_flops(w.B, w.Hq, w.L, w.d, True, 0)
    bf = bwd_flops(w.B, w.Hq, w.L, w.d, True, 0)
    value = (ff + bf) / (ms_step * 1e-3) / 1e12
    f_ms = avg["fwd"]
    b_ms = avg["preprocess"] + avg["dkdv"] + avg["dq"]     # the instrumented pass
    fwd_tf = ff / (f_ms * 1e-3) / 1e12
    bwd_tf = bf / (b_ms * 1e-3) / 1e12
    # Algorithmic work per launch.  The backward's five L x L x d products
    # (2.5x the forward) split as: dK/dV kernel -- S recomputation, dV, dP, dK
    # (4 products); dQ kernel -- dQ (1 product; it also recomputes S and dP,
    # which are not counted again).  The preprocess is HBM-bound: it reads O
    # and dO and writes two floats per row.
    one = ff / 2
    alg = {"fwd": ("mfma", 2 * one), "dkdv": ("mfma", 4 * one), "dq": ("mfma", 1 * one),
           "preprocess": ("hbm", 2 * w.B * w.Hq * w.L * w.d * 2 + 3 * w.B * w.Hq * w.L * 4)}
    dom = max(avg, key=avg.get)
    kernel_names = {"fwd": "fwd_bf16_kernel<128,causal>", "preprocess": "bwd_delta_kernel<128>",
                    "dkdv": "bwd_dkdv_kernel<128,causal>", "dq": "bwd_dq_kernel<128,causal>"}
    bound, work = alg[dom]
    if bound == "mfma":
        achieved, peak, unit = work / (avg[dom] * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = work / (avg[dom] * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": n_warm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama7b-shaped attention layer fwd+bwd",
                   "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "L": w.L, "d": w.d, "causal": True,
                   "window": 0, "inputs": "seeded N(0,1) bf16, resident in HBM"},
        "fwd": {"ms_mean": round(f_ms, 4), "ms_median": round(med["fwd"], 4),
                "tflops": round(fwd_tf, 2), "frac_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
                "frac_peak_at_measured_clock": round(fwd_tf / PEAK_BF16_AT_MEASURED_CLOCK_TFLOPS, 4)},
        "bwd": {"ms_mean": round(b_ms, 4), "tflops": round(bwd_tf, 2),
                "frac_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
                "frac_peak_at_measured_clock": round(bwd_tf / PEAK_BF16_AT_MEASURED_CLOCK_TFLOPS, 4)},
        "peak_at_measured_clock": {"tflops": PEAK_BF16_AT_MEASURED_CLOCK_TFLOPS,
                                   "clock_ghz": MEASURED_MFMA_CLOCK_GHZ},
        "kernels_ms_mean": {n: round(avg[n], 4) for n in names},
        "roofline": {"kernel": kernel_names[dom], "bound": bound, "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": load_traffic(kernel_names[dom]),
                     "algorithmic_per_launch": work,
                     "ms_per_launch": round(avg[dom], 4),
                     "time_base": "mean over K instrumented steps (run after the timed region) of the "
                                  "interval between HIP events recorded on the launch stream right before "
                                  "and right after the kernel's launch; compare with the kernel-trace "
                                  "average of the same launches in profiles/kernel_time_llama7b_fwd_bwd.txt"},
    }
    if not args.no_configs:
        out["configs"] = {wl.name: measure_config(wl) for wl in W.ALL}
        f16 = W.LLAMA7B_CAUSAL.with_(name="llama7b-layer B2 H32 L4096 d128 causal fp16", dtype=torch.float16)
        out["configs"][f16.name] = measure_config(f16)
        out["autograd"] = measure_autograd()
        out["bwd_fused"] = measure_bwd_fused()
        out["decode"] = measure_decode()
        out["decode_16"] = measure_decode(Lq=16)
        out["decode_rolling"] = measure_decode_rolling()
        out["ring"] = measure_ring()
        out["sparse"] = measure_sparse()
        out["sparse_block"] = measure_sparse(block_band=True)
    ctx = dict(PAGES_CONTEXT)
    ctx["this_layer"] = {"score_matrix_bytes_fp16": score_matrix_bytes(w.B, w.Hq, w.L),
                         "extra_bytes_fwd_lse": int(lse.numel() * 4),
                         "extra_bytes_bwd_workspace": int(ws.numel())}
    out["context"] = ctx
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
        out["cpu_baseline_configs"] = cpu_baseline_configs()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
