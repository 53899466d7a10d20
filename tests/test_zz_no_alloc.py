"""flash_attn_bwd_noalloc (the backward without a workspace argument, for callers
that cannot allocate) against flash_attn_bwd and the fp64 oracle, through the C
ABI.

Two calls in a row on one GPU, the second with a smaller input: the library's
static per-row statistics then hold the first call's values where the second
does not overwrite them, and the second call must not read them.  The bar is
the backward's: relative L2 error <= 2e-2 per tensor against flash_attn_bwd on
the same inputs and against the oracle; no device memory may be allocated by
the call itself.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

REL_TOL = 2e-2
DEV = "cuda:0"


def fa():
    import exact_tiled_attention_flash_amd as m
    m.library()
    return m


def rel(x, ref):
    ref = np.asarray(ref, dtype=np.float64)
    den = max(float(np.linalg.norm(ref)), 1e-2 * math.sqrt(ref.size))
    return float(np.linalg.norm(x.double().cpu().numpy() - ref)) / den


def run_case(w):
    print(f"[noalloc] case {w.name} B{w.B} Hq{w.Hq} Hkv{w.Hkv} L{w.L} d{w.d} causal={w.causal} "
          f"window={w.window} seed={w.seed}", flush=True)
    q, k, v, do = W.make_inputs(w, with_dout=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa().fwd(qd, kd, vd, causal=w.causal, window=w.window, scale=w.scale)
    ref_dev = fa().bwd(qd, kd, vd, o, lse, dod, causal=w.causal, window=w.window, scale=w.scale)
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (qd, kd, vd))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    fa().bwd_noalloc(qd, kd, vd, o, lse, dod, dq, dk, dv, causal=w.causal, window=w.window, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    ref = oracle.backward(q.double().numpy(), k.double().numpy(), v.double().numpy(), do.double().numpy(),
                          w.scale, w.causal, w.window)
    for name, x, xr, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref_dev, ref):
        assert torch.isfinite(x.float()).all(), name
        e_dev = rel(x, xr.double().cpu().numpy())
        e_ref = rel(x, r)
        print(f"[noalloc]   {name}: relL2 vs flash_attn_bwd {e_dev:.3e}, vs oracle {e_ref:.3e}", flush=True)
        assert e_dev <= REL_TOL and e_ref <= REL_TOL, name


def test_noalloc_two_calls_second_smaller():
    big = W.small("noalloc first B2 Hq4 Hkv2 L700 d128 causal", 2, 4, 2, 700, 128, causal=True, seed=41,
                  backward=True)
    small = W.small("noalloc second B1 Hq2 Hkv1 L130 d64 window 37", 1, 2, 1, 130, 64, causal=True, window=37,
                    seed=42, backward=True)
    run_case(big)
    run_case(small)


def test_noalloc_fp16_non_causal_then_smaller_bf16():
    a = W.small("noalloc fp16 B1 Hq2 Hkv2 L333 d128 non-causal", 1, 2, 2, 333, 128, dtype=torch.float16,
                causal=False, seed=43, backward=True)
    b = W.small("noalloc bf16 B1 Hq1 Hkv1 L1 d128 causal", 1, 1, 1, 1, 128, causal=True, seed=44, backward=True)
    run_case(a)
    run_case(b)


def test_noalloc_too_large_is_rejected_on_the_gpu():
    """The row limit holds on the device path too, before any launch."""
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device=DEV)
    lib = fa().library()
    rc = lib.flash_attn_bwd_noalloc(*([x.data_ptr()] * 9), 1, 1 << 11, 1, 1 << 10 | 1, 64, 0.125, 1, 0,
                                    fa().FA_DTYPE_BF16, None)
    assert rc == -6
