"""GPU forward parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Small shapes are compared element by element on every output; the full-size
workloads are compared on sampled query rows (all heads), which the oracle
computes exactly row by row.  Tolerances: bf16 inputs with fp32 accumulation
-- O max abs <= 2e-2, LSE max abs <= 1e-3; fp32 -- both <= 1e-4.  fp16 runs the
same MFMA kernels (fp16 opcode and conversions) and is held to the bf16 bounds,
which its finer rounding meets with room to spare.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: (2e-2, 1e-3), torch.float16: (2e-2, 1e-3), torch.float32: (1e-4, 1e-4)}


def fa():
    import exact_tiled_attention_flash_amd as m
    m.library()
    return m


# Unit roundoff of the 16-bit types (round to nearest even): 8 significant bits
# for bfloat16, 11 for float16.
UNIT_ROUNDOFF = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}


def o_error_bound(w, q, k, v, O_ref):
    """Per-element bound on |O_gpu - O| for inputs whose spread exceeds the unit
    variance the stated tolerance assumes (std > 1).

    O_ic = sum_j A_ij V_jc with A the softmax weights.  The kernels round each
    probability P_j to the 16-bit type before P.V (relative error <= u) but sum the
    row total l in fp32 from the unrounded P_j, so the numerator's rounding moves
    O_ic by at most u * sum_j A_ij |V_jc|; the output rounding adds at most
    u * |O_ic|.  fp32 accumulation and exp2 errors are below 1e-4 relative and
    are covered by a 1e-4 term.  sum_j A_ij |V_jc| is the oracle's attention
    output for |V|, so the bound is computed, not assumed:
        |O_gpu - O|_ic <= (u + 1e-4) * (A |V|)_ic + u * |O_ic|.
    """
    u = UNIT_ROUNDOFF[w.dtype]
    O_abs, _ = oracle.forward(np32(q), np32(k), np.abs(np32(v)), w.scale, w.causal, w.window)
    return (u + 1e-4) * O_abs + u * np.abs(O_ref)


def np32(t):
    return t.numpy() if t.dtype == torch.float32 else t.float().numpy()


def gpu_fwd(w, q, k, v):
    dev = "cuda:0"
    o, lse = fa().fwd(q.to(dev), k.to(dev), v.to(dev), causal=w.causal, window=w.window, scale=w.scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def sample_rows(L, window, n_random=48, seed=0):
    fixed = {0, 1, 2, 31, 32, 63, 64, 65, 127, 128, 129, 255, 256, L // 2, L - 129, L - 128, L - 65,
             L - 64, L - 2, L - 1}
    if window > 0:
        fixed |= {window - 2, window - 1, window, window + 1, window + 63, window + 64}
    rng = np.random.default_rng(seed)
    fixed |= set(rng.integers(0, L, size=n_random).tolist())
    return np.array(sorted(r for r in fixed if 0 <= r < L))


def report(name, err_o, err_l, tol):
    print(f"[parity] {name}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e} (tol {tol[0]:g}, {tol[1]:g})", flush=True)


def check_full(w):
    print(f"[parity] case {w.name} B{w.B} Hq{w.Hq} Hkv{w.Hkv} L{w.L} d{w.d} causal={w.causal} "
          f"window={w.window} seed={w.seed}", flush=True)
    q, k, v, _ = W.make_inputs(w, with_dout=False)
    o, lse = gpu_fwd(w, q, k, v)
    O_ref, lse_ref = oracle.forward(np32(q), np32(k), np32(v), w.scale, w.causal, w.window)
    tol = TOL[w.dtype]
    diff = np.abs(np32(o) - O_ref)
    err_o = float(diff.max())
    err_l = float(np.abs(lse.numpy() - lse_ref).max())
    report(w.name, err_o, err_l, tol)
    assert np.isfinite(np32(o)).all() and np.isfinite(lse.numpy()).all()
    assert err_l <= tol[1]
    if w.std > 1.0:
        # values beyond the unit-variance scale the stated O bound assumes:
        # held to the derived per-element bound instead
        bound = o_error_bound(w, q, k, v, O_ref)
        ratio = float((diff / bound).max())
        print(f"[parity] {w.name}: max |dO| / derived bound = {ratio:.3f} "
              f"(largest bound {float(bound.max()):.3e})", flush=True)
        assert ratio <= 1.0
    else:
        assert err_o <= tol[0]


def check_sampled(w, n_random=48):
    print(f"[parity] sampled case {w.name} seed={w.seed}", flush=True)
    q, k, v, _ = W.make_inputs(w, with_dout=False)
    o, lse = gpu_fwd(w, q, k, v)
    rows = sample_rows(w.L, w.window, n_random)
    O_ref, lse_ref = oracle.forward_rows(np32(q), np32(k), np32(v), rows, w.scale, w.causal, w.window)
    tol = TOL[w.dtype]
    err_o = float(np.abs(np32(o[:, :, rows]) - O_ref).max())
    err_l = float(np.abs(lse[:, :, rows].numpy() - lse_ref).max())
    report(w.name + f" ({rows.size} rows x all heads)", err_o, err_l, tol)
    assert np.isfinite(np32(o)).all() and np.isfinite(lse.numpy()).all()
    assert err_o <= tol[0] and err_l <= tol[1]


SMALL = [
    W.small("L1", 1, 2, 2, 1, 64),
    W.small("L7 noncausal d64", 1, 2, 1, 7, 64, causal=False),
    W.small("L100 causal d128", 2, 2, 2, 100, 128),
    W.small("L257 causal d64 gqa3", 1, 6, 2, 257, 64, seed=101),
    W.small("L300 noncausal d128", 1, 3, 3, 300, 128, causal=False, seed=102),
    W.small("L1000 causal d128 gqa4", 1, 8, 2, 1000, 128, seed=103),
    W.small("L777 window1", 1, 2, 2, 777, 128, window=1, seed=104),
    W.small("L777 window3 d64", 1, 2, 1, 777, 64, window=3, seed=105),
    W.small("L1500 window200", 1, 2, 2, 1500, 128, window=200, seed=106, std=0.5),
    W.small("L640 window64 gqa", 2, 4, 1, 640, 128, window=64, seed=107),
    W.small("L2048 window5000", 1, 2, 2, 2048, 128, window=5000, seed=108),
    W.small("MQA L513 causal", 1, 8, 1, 513, 128, seed=109),
    W.small("large scores", 1, 2, 2, 384, 128, seed=110, std=3.0),
    W.small("fp32 L200 causal d128", 1, 2, 2, 200, 128, dtype=torch.float32, seed=111),
    W.small("fp32 L150 window7 d64 gqa", 1, 4, 2, 150, 64, dtype=torch.float32, window=7, seed=112),
    W.small("fp32 L70 noncausal", 2, 1, 1, 70, 64, dtype=torch.float32, causal=False, seed=113),
    W.small("fp16 L300 causal d128 gqa2", 1, 4, 2, 300, 128, dtype=torch.float16, seed=114),
    W.small("fp16 L1000 window200 d64", 1, 2, 2, 1000, 64, dtype=torch.float16, window=200, seed=115),
    W.small("fp16 L257 noncausal d128 mqa", 1, 2, 1, 257, 128, dtype=torch.float16, causal=False, seed=116),
    W.small("fp16 large scores", 1, 2, 2, 384, 128, dtype=torch.float16, seed=117, std=3.0),
    # windows reaching both ways (no causal mask): |i - j| < w
    W.small("sym window1", 1, 2, 2, 300, 128, causal=False, window=1, seed=118),
    W.small("sym window5 d64 gqa2", 1, 4, 2, 777, 64, causal=False, window=5, seed=119),
    W.small("sym window200 L1500", 1, 2, 2, 1500, 128, causal=False, window=200, seed=123, std=0.5),
    W.small("sym window513 L2100", 1, 2, 1, 2100, 128, causal=False, window=513, seed=124),
    W.small("sym window5000 L2048", 1, 2, 2, 2048, 64, causal=False, window=5000, seed=125),
    W.small("fp32 sym window9 L150", 1, 2, 2, 150, 64, dtype=torch.float32, causal=False, window=9, seed=126),
    W.small("fp16 sym window64 L640", 1, 2, 2, 640, 128, dtype=torch.float16, causal=False, window=64, seed=127),
    # fp32 edge cases of the 16-rows-per-work-group kernel: one row, a partial
    # 16-row group and a partial 64-key tile, a window wider than the sequence
    W.small("fp32 L1", 1, 2, 2, 1, 64, dtype=torch.float32, seed=128),
    W.small("fp32 L17 noncausal d128 gqa2", 2, 4, 2, 17, 128, dtype=torch.float32, causal=False, seed=129),
    W.small("fp32 L129 window300", 1, 2, 1, 129, 64, dtype=torch.float32, window=300, seed=130),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_shapes(w):
    check_full(w)


def test_tiny_fp32_workload():
    check_full(W.TINY_FP32)


def test_llama7b_layer_sampled():
    check_sampled(W.LLAMA7B_CAUSAL)


def test_llama7b_layer_heads_full():
    # every row of two heads of the bench workload (same launch configuration)
    w = W.LLAMA7B_CAUSAL
    q, k, v, _ = W.make_inputs(w, with_dout=False)
    o, lse = gpu_fwd(w, q, k, v)
    sel = [(0, 0), (1, 31)]
    for b, h in sel:
        O_ref, lse_ref = oracle.forward(np32(q[b:b + 1, h:h + 1]), np32(k[b:b + 1, h:h + 1]),
                                        np32(v[b:b + 1, h:h + 1]), w.scale, True, 0)
        err_o = float(np.abs(np32(o[b:b + 1, h:h + 1]) - O_ref).max())
        err_l = float(np.abs(lse[b:b + 1, h:h + 1].numpy() - lse_ref).max())
        report(f"{w.name} head ({b},{h}) all rows", err_o, err_l, TOL[w.dtype])
        assert err_o <= 2e-2 and err_l <= 1e-3


def test_llama7b_layer_fp16_sampled():
    check_sampled(W.LLAMA7B_CAUSAL.with_(name="llama7b-layer fp16", dtype=torch.float16))


def test_gqa_16k_sampled():
    check_sampled(W.GQA_16K)


def test_window_32k_sampled():
    check_sampled(W.WINDOW_32K)


def test_long_128k_sampled():
    check_sampled(W.LONG_FWD_128K, n_random=24)


def test_forward_is_deterministic():
    w = W.small("det", 1, 4, 2, 1024, 128, seed=120)
    q, k, v, _ = W.make_inputs(w, with_dout=False)
    o1, l1 = gpu_fwd(w, q, k, v)
    o2, l2 = gpu_fwd(w, q, k, v)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_window_at_least_L_equals_causal():
    w = W.small("wL", 1, 2, 2, 700, 128, seed=121)
    q, k, v, _ = W.make_inputs(w, with_dout=False)
    o1, l1 = gpu_fwd(w, q, k, v)
    o2, l2 = gpu_fwd(w.with_(window=700), q, k, v)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_rows_of_probabilities_sum_to_one_via_lse():
    # exp(s q_i.k_j - LSE_i) over allowed keys sums to 1 (rows of A sum to 1)
    w = W.small("lse-sum", 1, 2, 2, 300, 64, seed=122)
    q, k, v, _ = W.make_inputs(w, with_dout=False)
    _, lse = gpu_fwd(w, q, k, v)
    S = w.scale * (q.double() @ k.double().transpose(-1, -2))
    mask = torch.ones(300, 300, dtype=torch.bool).tril()
    P = torch.exp(S - lse.double()[..., None]).masked_fill(~mask, 0.0)
    assert torch.allclose(P.sum(-1), torch.ones(1, 2, 300, dtype=torch.float64), atol=1e-3)


def test_huge_window_admits_every_pair():
    # every window >= 2^30 admits all pairs (no two positions are that far apart),
    # so it must give exactly the no-window result -- also for windows near
    # INT_MAX, where i + w would not fit an int
    w = W.small("huge-window", 1, 2, 2, 400, 64, seed=123)
    q, k, v, _ = W.make_inputs(w, with_dout=False)
    for causal in (False, True):
        o0, l0 = gpu_fwd(w.with_(causal=causal, window=0), q, k, v)
        for win in (1 << 30, 2**31 - 1):
            o1, l1 = gpu_fwd(w.with_(causal=causal, window=win), q, k, v)
            assert torch.equal(o0, o1) and torch.equal(l0, l1), (causal, win)
