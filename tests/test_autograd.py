"""The autograd drop-in -- FlashAttentionFunction and scaled_dot_product_attention --
against the fp64 oracle, through the library's C ABI.

A training-style call: leaf tensors with requires_grad, o = attention(q, k, v),
loss = sum(o * w) for a seeded w, loss.backward().  The gradient reaching o is
exactly w, so o must match the oracle forward and q.grad, k.grad, v.grad the
oracle backward with dO = w, to the parity tolerances (O max-abs 2e-2, gradients
relative L2 2e-2).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def f64(t):
    return t.detach().double().cpu().numpy()


def rel(x, ref):
    den = max(float(np.linalg.norm(ref)), 1e-2 * math.sqrt(ref.size))
    return float(np.linalg.norm(f64(x) - ref)) / den


CASES = [
    W.small("autograd bf16 causal gqa2", 1, 4, 2, 384, 128, seed=401, backward=True),
    W.small("autograd fp16 window100 d64", 1, 2, 2, 500, 64, dtype=torch.float16, window=100, seed=402,
            backward=True),
    W.small("autograd bf16 noncausal", 2, 2, 2, 130, 128, causal=False, seed=403, backward=True),
]


@pytest.mark.gpu
@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_drop_in_matches_oracle(w):
    import exact_tiled_attention_flash_amd as fa
    print(f"[autograd] {w.name} B{w.B} Hq{w.Hq} Hkv{w.Hkv} L{w.L} d{w.d} seed={w.seed}", flush=True)
    q, k, v, wgt = W.make_inputs(w, with_dout=True)
    dev = "cuda:0"
    qd, kd, vd = (t.to(dev).requires_grad_() for t in (q, k, v))
    o = fa.scaled_dot_product_attention(qd, kd, vd, is_causal=w.causal, window=w.window)
    (o * wgt.to(dev)).sum().backward()
    torch.cuda.synchronize()
    O_ref, _ = oracle.forward(f64(q), f64(k), f64(v), w.scale, w.causal, w.window)
    err_o = float(np.abs(f64(o) - O_ref).max())
    ref = oracle.backward(f64(q), f64(k), f64(v), f64(wgt), w.scale, w.causal, w.window)
    errs = [rel(x.grad, r) for x, r in zip((qd, kd, vd), ref)]
    print(f"[autograd] {w.name}: max|dO|={err_o:.3e} relL2 dQ={errs[0]:.3e} dK={errs[1]:.3e} dV={errs[2]:.3e}",
          flush=True)
    assert o.dtype == w.dtype and qd.grad.dtype == w.dtype
    assert err_o <= 2e-2 and max(errs) <= 2e-2


@pytest.mark.gpu
def test_explicit_scale_and_noncontiguous_inputs():
    import exact_tiled_attention_flash_amd as fa
    w = W.small("autograd scale", 1, 2, 2, 200, 64, seed=404, backward=True)
    q, k, v, wgt = W.make_inputs(w, with_dout=True)
    dev = "cuda:0"
    # a transposed-then-transposed-back view is non-contiguous with the same values
    qd = q.to(dev).transpose(1, 2).contiguous().transpose(1, 2).requires_grad_()
    kd, vd = (t.to(dev).requires_grad_() for t in (k, v))
    assert not qd.is_contiguous()
    o = fa.scaled_dot_product_attention(qd, kd, vd, is_causal=True, scale=0.3)
    (o * wgt.to(dev)).sum().backward()
    torch.cuda.synchronize()
    O_ref, _ = oracle.forward(f64(q), f64(k), f64(v), 0.3, True, 0)
    ref = oracle.backward(f64(q), f64(k), f64(v), f64(wgt), 0.3, True, 0)
    assert float(np.abs(f64(o) - O_ref).max()) <= 2e-2
    assert max(rel(x.grad, r) for x, r in zip((qd, kd, vd), ref)) <= 2e-2


@pytest.mark.gpu
def test_float32_has_forward_only():
    import exact_tiled_attention_flash_amd as fa
    w = W.small("autograd fp32", 1, 2, 2, 64, 64, dtype=torch.float32, seed=405)
    q, k, v, _ = W.make_inputs(w, with_dout=False)
    qd, kd, vd = (t.to("cuda:0").requires_grad_() for t in (q, k, v))
    o = fa.scaled_dot_product_attention(qd, kd, vd, is_causal=True)
    with pytest.raises(RuntimeError, match="unsupported"):
        o.sum().backward()


def test_drop_in_rejects_host_tensors():
    # argument checks happen in the binding before the library is called
    import exact_tiled_attention_flash_amd as fa
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.scaled_dot_product_attention(q, q, q, is_causal=True)
