"""GPU parity of the ring-attention pieces -- chunk-pair forward, partial merge and
chunk-pair backward -- against the fp64 oracle, through the C ABI.

A query chunk holds the queries at positions q_offset + i, a key/value chunk the
keys at k_offset + j; masks are decided on those positions (claspmoon.cn "14 ·
缩放定律与高效注意力" §5.1, ring attention).  Tolerances as everywhere: O max-abs
2e-2, LSE max-abs 1e-3 (rows with no allowed key must be exactly O = 0,
LSE = -inf), gradients relative L2 2e-2.  A simulated ring on one GPU (P chunks,
each query chunk visiting every key chunk, partials merged in place) must
reproduce whole-sequence attention and its gradient.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def fa():
    import exact_tiled_attention_flash_amd as m
    m.library()
    return m


def f64(t):
    return t.detach().double().cpu().numpy()


def rel(x, ref):
    den = max(float(np.linalg.norm(ref)), 1e-2 * math.sqrt(ref.size))
    return float(np.linalg.norm(f64(x) - ref)) / den


def draw(shape, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(dtype)


def check_partial(o, lse, O_ref, lse_ref, name):
    """O and LSE against the oracle; rows without allowed keys must be exactly 0 / -inf."""
    lse_n = lse.cpu().numpy().astype(np.float64)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_n), empty), name
    assert np.all(f64(o)[empty] == 0.0), name
    err_o = float(np.abs(f64(o) - O_ref).max())
    err_l = float(np.abs(lse_n[~empty] - lse_ref[~empty]).max()) if (~empty).any() else 0.0
    print(f"[chunks] {name}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e} empty rows={int(empty.sum())}", flush=True)
    assert err_o <= 2e-2 and err_l <= 1e-3


# (B, Hq, Hkv, Lq, Lk, d, causal, window, q_offset, k_offset, dtype)
PAIRS = [
    (1, 2, 2, 256, 256, 128, True, 0, 256, 0, torch.bfloat16),       # later queries see a whole earlier chunk
    (1, 4, 2, 300, 200, 64, True, 0, 250, 200, torch.bfloat16),      # overlapping positions, ragged, GQA
    (1, 2, 1, 130, 520, 128, True, 0, 0, 0, torch.float16),          # Lq < Lk, same start (top-left aligned)
    (2, 2, 2, 64, 192, 128, True, 0, 128, 0, torch.bfloat16),        # decode-like bottom-right alignment
    (1, 2, 2, 200, 300, 128, True, 64, 500, 300, torch.bfloat16),    # window across the chunk edge
    (1, 2, 2, 100, 100, 64, True, 0, 0, 400, torch.bfloat16),        # keys after all queries: every row empty
    (1, 2, 2, 150, 333, 128, False, 0, 1000, 7, torch.float16),      # non-causal: offsets irrelevant
    (1, 2, 2, 96, 64, 128, True, 16, 1000, 0, torch.bfloat16),       # window far past the chunk: all empty
    (1, 2, 2, 200, 300, 128, False, 64, 300, 200, torch.bfloat16),   # symmetric window across both chunk edges
    (1, 4, 2, 130, 250, 64, False, 100, 0, 180, torch.float16),      # symmetric window, keys partly after queries
    (1, 2, 2, 64, 64, 128, False, 8, 0, 500, torch.bfloat16),        # symmetric window far away: all empty
]


@pytest.mark.parametrize("case", PAIRS, ids=[f"pair{i}" for i in range(len(PAIRS))])
def test_chunk_pair_forward(case):
    B, Hq, Hkv, Lq, Lk, d, causal, window, qo, ko, dt = case
    print(f"[chunks] pair {case}", flush=True)
    seed = 500 + Lq + Lk + qo
    q, k, v = draw((B, Hq, Lq, d), seed, dt), draw((B, Hkv, Lk, d), seed + 1, dt), draw((B, Hkv, Lk, d), seed + 2, dt)
    s = 1.0 / math.sqrt(d)
    o, lse = fa().fwd_block(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window=window, q_offset=qo,
                            k_offset=ko, scale=s)
    torch.cuda.synchronize()
    O_ref, l_ref = oracle.block_forward(f64(q), f64(k), f64(v), s, causal, window, qo, ko)
    check_partial(o, lse, O_ref, l_ref, f"pair {case}")


def test_merge_matches_oracle_and_is_in_place_safe():
    B, Hq, L, d = 2, 3, 77, 128
    for dt in (torch.bfloat16, torch.float16, torch.float32):
        oa, ob = draw((B, Hq, L, d), 600, dt), draw((B, Hq, L, d), 601, dt)
        la, lb = draw((B, Hq, L), 602, torch.float32) * 3, draw((B, Hq, L), 603, torch.float32) * 3
        la[0, 0, :5] = -math.inf             # empty side a
        lb[0, 1, 3:9] = -math.inf            # empty side b
        la[1, 2, 10:12] = -math.inf
        lb[1, 2, 10:12] = -math.inf          # both empty
        O_ref, l_ref = oracle.merge_partials(f64(oa), f64(la), f64(ob), f64(lb))
        o, lse = fa().merge(oa.to(DEV), la.to(DEV), ob.to(DEV), lb.to(DEV))
        tol = 1e-5 if dt == torch.float32 else 1e-2
        assert float(np.abs(f64(o) - O_ref).max()) <= tol
        fin = ~np.isneginf(l_ref)
        assert np.array_equal(np.isneginf(lse.cpu().numpy()), ~fin)
        assert float(np.abs(lse.cpu().numpy()[fin] - l_ref[fin]).max()) <= 1e-5
        # in place: out is o_a, lse_out is lse_a
        oad, lad = oa.to(DEV), la.to(DEV)
        fa().merge(oad, lad, ob.to(DEV), lb.to(DEV), out=oad, lse_out=lad)
        torch.cuda.synchronize()
        assert torch.equal(oad.cpu(), o.cpu()) and torch.equal(lad.cpu(), lse.cpu())


def ring(w, P):
    """Whole-sequence attention of workload `w` computed as P x P chunk pairs on one GPU:
    forward by merging partials in place, backward by summing chunk-pair gradients."""
    q, k, v, do = (t.to(DEV) for t in W.make_inputs(w, with_dout=True))
    n = w.L // P
    cuts = [i * n for i in range(P)] + [w.L]
    O, LSE = torch.empty_like(q), torch.empty(w.B, w.Hq, w.L, dtype=torch.float32, device=DEV)
    for i in range(P):
        r0, r1 = cuts[i], cuts[i + 1]
        qi = q[:, :, r0:r1].contiguous()
        acc_o, acc_l = None, None
        for j in range(P):
            c0, c1 = cuts[j], cuts[j + 1]
            po, pl = fa().fwd_block(qi, k[:, :, c0:c1].contiguous(), v[:, :, c0:c1].contiguous(), causal=w.causal,
                                    window=w.window, q_offset=r0, k_offset=c0, scale=w.scale)
            if acc_o is None:
                acc_o, acc_l = po, pl
            else:
                fa().merge(acc_o, acc_l, po, pl, out=acc_o, lse_out=acc_l)
        O[:, :, r0:r1], LSE[:, :, r0:r1] = acc_o, acc_l
    dq = torch.zeros(q.shape, dtype=torch.float32, device=DEV)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=DEV)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=DEV)
    for i in range(P):
        r0, r1 = cuts[i], cuts[i + 1]
        args = [t[:, :, r0:r1].contiguous() for t in (q, O)]
        for j in range(P):
            c0, c1 = cuts[j], cuts[j + 1]
            pq, pk, pv = fa().bwd_block(args[0], k[:, :, c0:c1].contiguous(), v[:, :, c0:c1].contiguous(), args[1],
                                        LSE[:, :, r0:r1].contiguous(), do[:, :, r0:r1].contiguous(), causal=w.causal,
                                        window=w.window, q_offset=r0, k_offset=c0, scale=w.scale)
            dq[:, :, r0:r1] += pq.float()
            dk[:, :, c0:c1] += pk.float()
            dv[:, :, c0:c1] += pv.float()
    torch.cuda.synchronize()
    return (q, k, v, do), (O, LSE), (dq, dk, dv)


RINGS = [
    (W.small("ring causal gqa2 P4", 1, 4, 2, 1000, 128, seed=610, backward=True), 4),
    (W.small("ring window100 fp16 P3", 1, 2, 2, 768, 64, dtype=torch.float16, window=100, seed=611,
             backward=True), 3),
    (W.small("ring noncausal P2", 2, 2, 2, 300, 128, causal=False, seed=612, backward=True), 2),
    (W.small("ring sym window150 P3", 1, 2, 2, 900, 128, causal=False, window=150, seed=613, backward=True), 3),
]


@pytest.mark.parametrize("w,P", RINGS, ids=[w.name for w, _ in RINGS])
def test_simulated_ring_matches_oracle(w, P):
    print(f"[chunks] {w.name} B{w.B} Hq{w.Hq} Hkv{w.Hkv} L{w.L} d{w.d} seed={w.seed}", flush=True)
    (q, k, v, do), (O, LSE), grads = ring(w, P)
    O_ref, l_ref = oracle.forward(f64(q), f64(k), f64(v), w.scale, w.causal, w.window)
    err_o = float(np.abs(f64(O) - O_ref).max())
    err_l = float(np.abs(LSE.cpu().numpy() - l_ref).max())
    ref = oracle.backward(f64(q), f64(k), f64(v), f64(do), w.scale, w.causal, w.window)
    errs = [rel(x, r) for x, r in zip(grads, ref)]
    print(f"[chunks] {w.name}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e} relL2 dQ={errs[0]:.3e} dK={errs[1]:.3e} "
          f"dV={errs[2]:.3e}", flush=True)
    assert err_o <= 2e-2 and err_l <= 1e-3 and max(errs) <= 2e-2


def test_ring_at_the_llama7b_shape_matches_whole_sequence_call():
    # the bench layer shape split into 4 chunks: compare with the single-call kernels
    w = W.LLAMA7B_CAUSAL
    print(f"[chunks] ring P4 of {w.name}", flush=True)
    (q, k, v, do), (O, LSE), (dq, dk, dv) = ring(w, 4)
    o1, l1 = fa().fwd(q, k, v, causal=True, scale=w.scale)
    g1 = fa().bwd(q, k, v, o1, l1, do, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    d_o = float((O.float() - o1.float()).abs().max())
    d_l = float((LSE - l1).abs().max())
    rels = [float((x - y.float()).norm() / y.float().norm()) for x, y in zip((dq, dk, dv), g1)]
    print(f"[chunks] ring vs whole: max|dO|={d_o:.3e} max|dLSE|={d_l:.3e} rel dQ,dK,dV={rels}", flush=True)
    assert d_o <= 2e-2 and d_l <= 1e-3 and max(rels) <= 2e-2
    # and one head against the oracle
    sl = (slice(1, 2), slice(7, 8))
    ref = oracle.backward(*(f64(t[sl]) for t in (q, k, v, do)), w.scale, True, 0)
    errs = [rel(x[sl], r) for x, r in zip((dq, dk, dv), ref)]
    assert max(errs) <= 2e-2


def test_chunk_pair_at_the_largest_offsets():
    # only q_offset - k_offset enters the masks: a pair placed at the top of the
    # offset range (2^29) gives the bits of the same pair near position 0, for the
    # forward and the backward, with a window that reaches across the pair (every
    # query row keeps at least one allowed key)
    B, Hq, Hkv, Lq, Lk, d = 1, 4, 2, 128, 160, 64
    dev = "cuda:0"
    q = draw((B, Hq, Lq, d), 301, torch.bfloat16).to(dev)
    k = draw((B, Hkv, Lk, d), 302, torch.bfloat16).to(dev)
    v = draw((B, Hkv, Lk, d), 303, torch.bfloat16).to(dev)
    do = draw((B, Hq, Lq, d), 304, torch.bfloat16).to(dev)
    top = 1 << 29
    for causal, window in ((True, 100), (False, 90), (True, 0)):
        res = []
        for qo, ko in ((100, 0), (top, top - 100)):
            o, lse = fa().fwd_block(q, k, v, causal=causal, window=window, q_offset=qo, k_offset=ko)
            g = fa().bwd_block(q, k, v, o, lse, do, causal=causal, window=window, q_offset=qo, k_offset=ko)
            torch.cuda.synchronize()
            res.append([o.cpu(), lse.cpu()] + [x.cpu() for x in g])
        for x, y in zip(*res):
            assert torch.equal(x, y), (causal, window)
