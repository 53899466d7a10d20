"""GPU backward parity: dQ, dK, dV from the HIP kernels against the fp64 oracle.

The backward always consumes O and LSE from a separate forward call of the
library (the forward -> backward contract: only O and the log-sum-exp are
kept).  Tolerance: relative L2 error ||x - x*|| / ||x*|| <= 2e-2 per tensor.
Small shapes are compared on every element; the full-size workloads run the
kernels at full size and compare whole (batch, head) slices, which the oracle
computes independently of the other heads.  The exact identities
sum_j dK_j = 0 and sum_j dV_j = sum over the group's heads of sum_i dO_i are
checked on the GPU outputs of every head.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

REL_TOL = 2e-2


def fa():
    import exact_tiled_attention_flash_amd as m
    m.library()
    return m


def f64(t):
    return t.double().numpy()


def gpu_fwd_bwd(w, q, k, v, do):
    dev = "cuda:0"
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa().fwd(qd, kd, vd, causal=w.causal, window=w.window, scale=w.scale)
    dq, dk, dv = fa().bwd(qd, kd, vd, o, lse, dod, causal=w.causal, window=w.window, scale=w.scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def rel(x, ref):
    """||x - ref|| / ||ref||, with ||ref|| floored at 1e-2 * sqrt(numel): a gradient
    that vanishes exactly (L = 1: a softmax over one key has zero gradient) is
    then held to an absolute bound instead of a relative one."""
    den = max(float(np.linalg.norm(ref)), 1e-2 * math.sqrt(ref.size))
    return float(np.linalg.norm(f64(x) - ref)) / den


def check_identities(w, dk, dv, do):
    """sum_j dK_j = 0 and sum_j dV_j = sum_{group heads} sum_i dO_i, per (batch, K/V head)."""
    G = w.Hq // w.Hkv
    sdk = dk.double().sum(2)                                  # [B, Hkv, d]
    sdv = dv.double().sum(2)
    sdo = do.double().sum(2).reshape(w.B, w.Hkv, G, w.d).sum(2)
    # floor the scale at 1e-2 per row: dK vanishes exactly when every query
    # sees a single key (L = 1, window = 1), and noise over noise means nothing
    scale_dk = dk.double().abs().sum(2).clamp_min(1e-2 * w.L)
    err_dk = float((sdk.abs() / scale_dk).max())
    err_dv = float(((sdv - sdo).abs() / (dv.double().abs().sum(2) + sdo.abs()).clamp_min(1e-30)).max())
    print(f"[parity] identities: max |sum dK|/sum|dK| = {err_dk:.2e}, sum dV vs sum dO rel = {err_dv:.2e}", flush=True)
    # bf16 output rounding of each element bounds the residual of the sums
    assert err_dk < 2e-2 and err_dv < 2e-2


def check_full(w):
    print(f"[parity] bwd case {w.name} B{w.B} Hq{w.Hq} Hkv{w.Hkv} L{w.L} d{w.d} causal={w.causal} "
          f"window={w.window} seed={w.seed}", flush=True)
    q, k, v, do = W.make_inputs(w, with_dout=True)
    dq, dk, dv = gpu_fwd_bwd(w, q, k, v, do)
    ref = oracle.backward(f64(q), f64(k), f64(v), f64(do), w.scale, w.causal, w.window)
    errs = [rel(x, r) for x, r in zip((dq, dk, dv), ref)]
    print(f"[parity] {w.name}: relL2 dQ={errs[0]:.3e} dK={errs[1]:.3e} dV={errs[2]:.3e}", flush=True)
    for x in (dq, dk, dv):
        assert torch.isfinite(x.float()).all()
    assert max(errs) <= REL_TOL
    check_identities(w, dk, dv, do)


SMALL = [
    W.small("bwd L1", 1, 2, 2, 1, 64),
    W.small("bwd L7 noncausal d64", 1, 2, 1, 7, 64, causal=False, seed=201),
    W.small("bwd L100 causal d128", 2, 2, 2, 100, 128, seed=202),
    W.small("bwd L257 causal d64 gqa3", 1, 6, 2, 257, 64, seed=203),
    W.small("bwd L300 noncausal d128", 1, 3, 3, 300, 128, causal=False, seed=204),
    W.small("bwd L1000 causal gqa4", 1, 8, 2, 1000, 128, seed=205),
    W.small("bwd L777 window1", 1, 2, 2, 777, 128, window=1, seed=206),
    W.small("bwd L777 window3 d64", 1, 2, 1, 777, 64, window=3, seed=207),
    W.small("bwd L1500 window200", 1, 2, 2, 1500, 128, window=200, seed=208, std=0.5),
    W.small("bwd L640 window64 gqa4", 2, 4, 1, 640, 128, window=64, seed=209),
    W.small("bwd L2048 window5000", 1, 2, 2, 2048, 128, window=5000, seed=210),
    W.small("bwd MQA L513", 1, 8, 1, 513, 128, seed=211),
    W.small("bwd fp16 L300 causal gqa2", 1, 4, 2, 300, 128, dtype=torch.float16, seed=212),
    W.small("bwd fp16 L640 window64 d64", 1, 2, 2, 640, 64, dtype=torch.float16, window=64, seed=213),
    W.small("bwd fp16 L200 noncausal", 2, 2, 2, 200, 128, dtype=torch.float16, causal=False, seed=214),
    W.small("bwd sym window1", 1, 2, 2, 300, 128, causal=False, window=1, seed=215),
    W.small("bwd sym window7 d64 gqa2", 1, 4, 2, 777, 64, causal=False, window=7, seed=216),
    W.small("bwd sym window200 L1500", 1, 2, 2, 1500, 128, causal=False, window=200, seed=217, std=0.5),
    W.small("bwd sym window513 L2100", 1, 2, 1, 2100, 128, causal=False, window=513, seed=218),
    W.small("bwd fp16 sym window64 L640", 1, 2, 2, 640, 64, dtype=torch.float16, causal=False, window=64, seed=219),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_shapes(w):
    check_full(w)


def check_heads_at_full_size(w, heads):
    print(f"[parity] bwd full-size case {w.name} seed={w.seed}", flush=True)
    assert w.Hq == w.Hkv
    q, k, v, do = W.make_inputs(w, with_dout=True)
    dq, dk, dv = gpu_fwd_bwd(w, q, k, v, do)
    for x in (dq, dk, dv):
        assert torch.isfinite(x.float()).all()
    check_identities(w, dk, dv, do)
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.backward(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(do[sl]), w.scale, w.causal, w.window)
        errs = [rel(x[sl], r) for x, r in zip((dq, dk, dv), ref)]
        print(f"[parity] {w.name} head ({b},{h}): relL2 dQ={errs[0]:.3e} dK={errs[1]:.3e} dV={errs[2]:.3e}",
              flush=True)
        assert max(errs) <= REL_TOL


def test_llama7b_layer_backward():
    check_heads_at_full_size(W.LLAMA7B_CAUSAL, [(0, 0), (1, 17)])


def test_llama7b_layer_backward_fp16():
    check_heads_at_full_size(W.LLAMA7B_CAUSAL.with_(name="llama7b-layer fp16", dtype=torch.float16), [(1, 3)])


def test_long_context_backward():
    check_heads_at_full_size(W.LONG_BWD_8K, [(1, 5)])


def same_gradients(a, b, what):
    """dK and dV bit for bit; dQ -- summed with float32 atomics in the fused
    backward, so in an order that varies from run to run -- to float32
    rounding before the final 16-bit rounding: each element within one unit in
    the last place of the 16-bit result plus 1e-3 of the tensor's largest
    element (an element that is a small difference of large terms carries the
    float32 error of the terms), and relative L2 <= 1e-4."""
    dq_a, dq_b = a[0].float(), b[0].float()
    bound = dq_b.abs() * 2.0 ** -7 + 1e-3 * float(dq_b.abs().max())
    assert bool(((dq_a - dq_b).abs() <= bound).all()), what
    assert float((dq_a - dq_b).norm() / dq_b.norm().clamp_min(1e-30)) <= 1e-4, what
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2]), what


def test_backward_stages_equal_bwd_call():
    """The three exported stages (preprocess, dK/dV, dQ) reproduce flash_attn_bwd bit for bit."""
    for w in (W.small("stages", 1, 4, 2, 513, 128, seed=230, backward=True),
              W.small("stages d64 window", 1, 2, 2, 300, 64, window=50, seed=231, backward=True),
              W.LLAMA7B_CAUSAL):
        q, k, v, do = W.make_inputs(w, with_dout=True)
        dev = "cuda:0"
        qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
        o, lse = fa().fwd(qd, kd, vd, causal=w.causal, window=w.window, scale=w.scale)
        a = fa().bwd(qd, kd, vd, o, lse, dod, causal=w.causal, window=w.window, scale=w.scale)
        seen = []
        b = fa().bwd_stages(qd, kd, vd, o, lse, dod, causal=w.causal, window=w.window, scale=w.scale,
                            between=seen.append)
        torch.cuda.synchronize()
        assert seen == ["preprocess", "dkdv", "dq"]
        for x, y in zip(a, b):
            assert torch.equal(x, y)


FUSED = [
    W.small("fused L513 gqa2", 1, 4, 2, 513, 128, seed=230, backward=True),
    W.small("fused d64 window50", 1, 2, 2, 300, 64, window=50, seed=231, backward=True),
    W.small("fused fp16 noncausal mqa", 1, 2, 1, 257, 128, dtype=torch.float16, causal=False, seed=232,
            backward=True),
    W.small("fused L7 noncausal d64", 1, 2, 1, 7, 64, causal=False, seed=233, backward=True),
    W.small("fused L1", 1, 2, 2, 1, 128, seed=234, backward=True),
    W.small("fused sym window40 L700", 2, 2, 2, 700, 128, causal=False, window=40, seed=235, backward=True),
    W.small("fused d64 gqa4 L1000", 1, 8, 2, 1000, 64, seed=236, backward=True),
]


@pytest.mark.parametrize("w", FUSED, ids=[w.name for w in FUSED])
def test_fused_backward(w):
    """flash_attn_bwd_fused (one K/V-stationary kernel, dQ by float32 atomics)
    against the oracle, and against flash_attn_bwd: dK and dV bit for bit, dQ to
    float32 rounding."""
    print(f"[parity] fused bwd case {w.name} B{w.B} Hq{w.Hq} Hkv{w.Hkv} L{w.L} d{w.d} causal={w.causal} "
          f"window={w.window} seed={w.seed}", flush=True)
    q, k, v, do = W.make_inputs(w, with_dout=True)
    dev = "cuda:0"
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa().fwd(qd, kd, vd, causal=w.causal, window=w.window, scale=w.scale)
    a = fa().bwd_fused(qd, kd, vd, o, lse, dod, causal=w.causal, window=w.window, scale=w.scale)
    b = fa().bwd(qd, kd, vd, o, lse, dod, causal=w.causal, window=w.window, scale=w.scale)
    torch.cuda.synchronize()
    a = [x.cpu() for x in a]
    ref = oracle.backward(f64(q), f64(k), f64(v), f64(do), w.scale, w.causal, w.window)
    errs = [rel(x, r) for x, r in zip(a, ref)]
    print(f"[parity] {w.name}: relL2 dQ={errs[0]:.3e} dK={errs[1]:.3e} dV={errs[2]:.3e}", flush=True)
    assert max(errs) <= REL_TOL
    same_gradients(a, [x.cpu() for x in b], w.name)


def test_fused_backward_full_size():
    """The fused backward at the LLaMA-7B-shaped layer: whole heads against the oracle."""
    w = W.LLAMA7B_CAUSAL
    q, k, v, do = W.make_inputs(w, with_dout=True)
    dev = "cuda:0"
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa().fwd(qd, kd, vd, causal=True, scale=w.scale)
    a = fa().bwd_fused(qd, kd, vd, o, lse, dod, causal=True, scale=w.scale)
    b = fa().bwd(qd, kd, vd, o, lse, dod, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    same_gradients([x.cpu() for x in a], [x.cpu() for x in b], w.name)
    for bb, h in ((0, 0), (1, 31)):
        sl = (slice(bb, bb + 1), slice(h, h + 1))
        ref = oracle.backward(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(do[sl]), w.scale, True, 0)
        errs = [rel(x.cpu()[sl], r) for x, r in zip(a, ref)]
        print(f"[parity] fused {w.name} head ({bb},{h}): relL2 dQ={errs[0]:.3e} dK={errs[1]:.3e} dV={errs[2]:.3e}",
              flush=True)
        assert max(errs) <= REL_TOL


def test_backward_is_deterministic():
    """flash_attn_bwd is deterministic bit for bit; the fused backward repeats dK
    and dV bit for bit and dQ to float32 rounding (the order of its atomics)."""
    w = W.small("det", 1, 4, 2, 700, 128, seed=220, backward=True)
    q, k, v, do = W.make_inputs(w, with_dout=True)
    a = gpu_fwd_bwd(w, q, k, v, do)
    b = gpu_fwd_bwd(w, q, k, v, do)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    dev = "cuda:0"
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa().fwd(qd, kd, vd, causal=w.causal, window=w.window, scale=w.scale)
    f1 = [x.cpu() for x in fa().bwd_fused(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale)]
    f2 = [x.cpu() for x in fa().bwd_fused(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale)]
    same_gradients(f1, f2, "fused, two runs")


def test_huge_window_backward_equals_no_window():
    # a window >= 2^30 admits every pair: gradients equal the no-window call's
    w = W.small("huge-window-bwd", 1, 2, 2, 300, 64, seed=221, backward=True)
    q, k, v, do = W.make_inputs(w, with_dout=True)
    for causal in (False, True):
        a = gpu_fwd_bwd(w.with_(causal=causal, window=0), q, k, v, do)
        b = gpu_fwd_bwd(w.with_(causal=causal, window=2**31 - 1), q, k, v, do)
        for x, y in zip(a, b):
            assert torch.equal(x, y), causal
