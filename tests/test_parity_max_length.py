"""GPU parity at the largest supported sequence length, L = 2^23.

At d = 128 one head of K or V then spans 2 GiB, so the kernels' per-head
buffer ranges and the byte offsets of the last tiles come within 16 KiB of
2^31.  A sliding window of 200 keys keeps the work small.  Forward and
backward run over the whole tensors; the oracle checks 32-row blocks at the
start, the middle and the very end.  Because of the window, a block of rows
sees only the keys of a short slice (and a block of keys is seen only by the
queries of a short slice), so the chunk-pair oracle (block_forward /
block_backward with the slices' positions as offsets) gives those rows'
exact O, LSE and dQ, and those keys' exact dK and dV.  Inputs are drawn on the
device from a fixed seed and the sliced rows are copied to the host for the
oracle.  Tolerances as everywhere for bf16: O max-abs 2e-2, LSE max-abs
1e-3, gradients relative L2 2e-2.
"""

import math

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def fa():
    import exact_tiled_attention_flash_amd as m
    m.library()
    return m


def rel(x, ref):
    den = max(float(np.linalg.norm(ref)), 1e-2 * math.sqrt(ref.size))
    return float(np.linalg.norm(x - ref)) / den


def test_maximum_length_sliding_window():
    L, d, Hq, Hkv, w = 1 << 23, 128, 2, 1, 200
    s = 1.0 / math.sqrt(d)
    g = torch.Generator(device=DEV).manual_seed(4242)

    def draw(h):
        return torch.randn(1, h, L, d, generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)

    q, k, v, do = draw(Hq), draw(Hkv), draw(Hkv), draw(Hq)
    print(f"[maxlen] L={L} d={d} Hq={Hq} Hkv={Hkv} causal window={w}", flush=True)
    o, lse = fa().fwd(q, k, v, causal=True, window=w, scale=s)
    dq, dk, dv = fa().bwd(q, k, v, o, lse, do, causal=True, window=w, scale=s)
    torch.cuda.synchronize()

    def rows(t, lo, hi):
        return t[:, :, lo:hi].float().cpu().numpy()

    starts = [0, 1, 190, 4095, L // 2 - 17, (1 << 22) + 12345, L - 300, L - 64, L - 33, L - 1]
    rng = np.random.default_rng(4242)
    starts += [int(x) for x in rng.integers(0, L, size=6)]
    worst = [0.0, 0.0, 0.0]
    for p in starts:
        # queries [p, p + 32) see keys [p - w + 1, p + 32) only
        q_lo, q_hi = p, min(L, p + 32)
        k_lo = max(0, q_lo - w + 1)
        qs, ks, vs, dos = rows(q, q_lo, q_hi), rows(k, k_lo, q_hi), rows(v, k_lo, q_hi), rows(do, q_lo, q_hi)
        O_ref, l_ref = oracle.block_forward(qs, ks, vs, s, True, w, q_lo, k_lo)
        err_o = float(np.abs(rows(o, q_lo, q_hi) - O_ref).max())
        err_l = float(np.abs(lse[:, :, q_lo:q_hi].cpu().numpy().astype(np.float64) - l_ref).max())
        dq_ref, _, _ = oracle.block_backward(qs, ks, vs, dos, O_ref, l_ref, s, True, w, q_lo, k_lo)
        err_dq = rel(rows(dq, q_lo, q_hi), dq_ref)
        # keys [p, p + 32) are seen by queries [p, p + 32 + w - 1) only; those
        # queries' O and LSE come from the keys [p - w + 1, p + 32 + w - 1)
        kk_lo, kk_hi = p, min(L, p + 32)
        qq_lo, qq_hi = p, min(L, p + 32 + w - 1)
        kr_lo = max(0, qq_lo - w + 1)
        qs2, dos2 = rows(q, qq_lo, qq_hi), rows(do, qq_lo, qq_hi)
        O2, l2 = oracle.block_forward(qs2, rows(k, kr_lo, qq_hi), rows(v, kr_lo, qq_hi), s, True, w, qq_lo, kr_lo)
        _, dk_ref, dv_ref = oracle.block_backward(qs2, rows(k, kk_lo, kk_hi), rows(v, kk_lo, kk_hi), dos2, O2, l2,
                                                  s, True, w, qq_lo, kk_lo)
        err_dkv = max(rel(rows(dk, kk_lo, kk_hi), dk_ref), rel(rows(dv, kk_lo, kk_hi), dv_ref))
        print(f"[maxlen] rows/keys from {p}: max|dO|={err_o:.2e} max|dLSE|={err_l:.2e} "
              f"dQ relL2={err_dq:.2e} dK/dV relL2={err_dkv:.2e}", flush=True)
        assert err_o <= 2e-2 and err_l <= 1e-3 and err_dq <= 2e-2 and err_dkv <= 2e-2, p
        worst = [max(worst[0], err_o), max(worst[1], err_l), max(worst[2], err_dq, err_dkv)]
    assert bool(torch.isfinite(lse).all()) and bool(torch.isfinite(o.float()).all())
    print(f"[maxlen] worst: O {worst[0]:.2e} LSE {worst[1]:.2e} grads {worst[2]:.2e}", flush=True)
