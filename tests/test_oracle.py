"""Pins for the fp64 CPU oracle (no GPU).

The oracle must be anchored to something other than itself before GPU results
are compared with it.  Each pin below is a fact fixed by the pages or by the
mathematics: closed forms, invariants, exact zeros, a library routine
(PyTorch's float64 CPU ``scaled_dot_product_attention`` and autograd,
``scipy.special.logsumexp``), central finite differences, and the equivalence
of the tiled online-softmax recurrence with the direct definition.  The
``test_planted_*`` cases plant plausible mistakes in the oracle (on the CPU)
and check that at least one pin catches each of them.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
import oracle.attention as oa

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def allowed_range(i, L, causal, window):
    """Allowed keys of query i as a Python range (written independently of the mask code)."""
    hi = i if causal else L - 1
    lo = 0
    if window > 0:
        lo = max(0, i - window + 1)
        if not causal:
            hi = min(L - 1, i + window - 1)
    return range(lo, hi + 1)


MASKS = [(False, 0), (True, 0), (True, 1), (True, 3), (True, 7), (False, 1), (False, 3), (False, 5)]


# ----------------------------------------------------------------------------- pins

def pin_rows_stochastic(o):
    for causal, window in MASKS:
        q, k = rnd((2, 3, 9, 4), 1), rnd((2, 3, 9, 4), 2)
        A = o.probabilities(q, k, 0.5, causal, window)
        assert np.allclose(A.sum(-1), 1.0, atol=1e-14, rtol=0), "rows of A must sum to 1"
        for i in range(9):
            allowed = set(allowed_range(i, 9, causal, window))
            for j in range(9):
                if j in allowed:
                    assert (A[:, :, i, j] > 0).all()
                else:
                    assert (A[:, :, i, j] == 0.0).all(), "masked keys carry exactly zero weight"


def pin_two_key_worked_example(o):
    # scores 0 and ln 3 -> weights 1/4 and 3/4 -> O = 1/4*1 + 3/4*5 = 4, LSE = ln 4
    q = np.array([1.0, 1.0]).reshape(1, 1, 2, 1)
    k = np.array([0.0, math.log(3.0)]).reshape(1, 1, 2, 1)
    v = np.array([1.0, 5.0]).reshape(1, 1, 2, 1)
    O, lse = o.forward(q, k, v, 1.0, causal=False)
    assert abs(O[0, 0, 0, 0] - 4.0) < 1e-14 and abs(O[0, 0, 1, 0] - 4.0) < 1e-14
    assert abs(lse[0, 0, 0] - math.log(4.0)) < 1e-14
    # causal: query 0 sees only key 0 -> O = 1, LSE = 0
    O, lse = o.forward(q, k, v, 1.0, causal=True)
    assert O[0, 0, 0, 0] == 1.0 and lse[0, 0, 0] == 0.0
    assert abs(O[0, 0, 1, 0] - 4.0) < 1e-14


def pin_length_one(o):
    q, k, v = rnd((2, 4, 1, 8), 3), rnd((2, 2, 1, 8), 4), rnd((2, 2, 1, 8), 5)
    for causal, window in [(False, 0), (True, 0), (True, 1)]:
        O, lse = o.forward(q, k, v, 0.3, causal, window)
        for h in range(4):
            assert np.allclose(O[:, h], v[:, h // 2], atol=1e-15, rtol=0)
            assert np.allclose(lse[:, h, 0], 0.3 * (q[:, h, 0] * k[:, h // 2, 0]).sum(-1), atol=1e-14, rtol=0)


def pin_zero_query_is_mean(o):
    L = 11
    for causal, window in MASKS:
        q = np.zeros((1, 2, L, 5))
        k, v = rnd((1, 2, L, 5), 6), rnd((1, 2, L, 5), 7)
        O, lse = o.forward(q, k, v, 0.7, causal, window)
        for h in range(2):
            for i in range(L):
                r = allowed_range(i, L, causal, window)
                assert np.allclose(O[0, h, i], v[0, h, r.start:r.stop].mean(0), atol=1e-14, rtol=0)
                assert abs(lse[0, h, i] - math.log(len(r))) < 1e-14


def pin_identical_keys(o):
    L = 10
    for causal, window in MASKS:
        q, v = rnd((1, 2, L, 4), 8), rnd((1, 1, L, 4), 9)
        k0 = rnd((4,), 10)
        k = np.broadcast_to(k0, (1, 1, L, 4)).copy()
        O, lse = o.forward(q, k, v, 0.9, causal, window)
        for h in range(2):
            for i in range(L):
                r = allowed_range(i, L, causal, window)
                assert np.allclose(O[0, h, i], v[0, 0, r.start:r.stop].mean(0), atol=1e-13, rtol=0)
                expect = 0.9 * float(q[0, h, i] @ k0) + math.log(len(r))
                assert abs(lse[0, h, i] - expect) < 1e-13


def pin_convexity(o):
    L = 13
    for causal, window in MASKS:
        q, k, v = rnd((2, 2, L, 6), 11, 3.0), rnd((2, 2, L, 6), 12, 3.0), rnd((2, 2, L, 6), 13)
        O, _ = o.forward(q, k, v, 1.0, causal, window)
        for i in range(L):
            r = allowed_range(i, L, causal, window)
            lo = v[:, :, r.start:r.stop].min(2)
            hi = v[:, :, r.start:r.stop].max(2)
            assert (O[:, :, i] >= lo - 1e-14).all() and (O[:, :, i] <= hi + 1e-14).all()


def pin_shift_invariance(o):
    L = 12
    q, k, v = rnd((1, 3, L, 5), 14), rnd((1, 3, L, 5), 15), rnd((1, 3, L, 5), 16)
    c = rnd((5,), 17)
    for causal, window in MASKS:
        O1, l1 = o.forward(q, k, v, 0.6, causal, window)
        O2, l2 = o.forward(q, k + c, v, 0.6, causal, window)
        assert np.allclose(O1, O2, atol=1e-13, rtol=0)
        assert np.allclose(l2 - l1, 0.6 * (q @ c), atol=1e-12, rtol=0)


def pin_permutation_noncausal(o):
    L = 9
    q, k, v = rnd((2, 2, L, 4), 18), rnd((2, 2, L, 4), 19), rnd((2, 2, L, 4), 20)
    perm = np.random.default_rng(21).permutation(L)
    O1, l1 = o.forward(q, k, v, 0.5)
    O2, l2 = o.forward(q, k[:, :, perm], v[:, :, perm], 0.5)
    assert np.allclose(O1, O2, atol=1e-14, rtol=0) and np.allclose(l1, l2, atol=1e-14, rtol=0)


def pin_gqa_is_repeated_mha(o):
    B, Hq, Hkv, L, d = 2, 6, 2, 10, 4
    q, k, v, do = rnd((B, Hq, L, d), 22), rnd((B, Hkv, L, d), 23), rnd((B, Hkv, L, d), 24), rnd((B, Hq, L, d), 25)
    G = Hq // Hkv
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    for causal, window in MASKS:
        O1, l1 = o.forward(q, k, v, 0.5, causal, window)
        O2, l2 = o.forward(q, kr, vr, 0.5, causal, window)
        assert np.allclose(O1, O2, atol=1e-14, rtol=0) and np.allclose(l1, l2, atol=1e-14, rtol=0)
        dq1, dk1, dv1 = o.backward(q, k, v, do, 0.5, causal, window)
        dq2, dk2, dv2 = o.backward(q, kr, vr, do, 0.5, causal, window)
        assert np.allclose(dq1, dq2, atol=1e-13, rtol=0)
        assert np.allclose(dk1, dk2.reshape(B, Hkv, G, L, d).sum(2), atol=1e-13, rtol=0)
        assert np.allclose(dv1, dv2.reshape(B, Hkv, G, L, d).sum(2), atol=1e-13, rtol=0)


def pin_window_at_least_L_is_causal(o):
    L = 8
    q, k, v = rnd((1, 2, L, 3), 26), rnd((1, 2, L, 3), 27), rnd((1, 2, L, 3), 28)
    for causal in (True, False):
        O1, l1 = o.forward(q, k, v, 1.0, causal, 0)
        for w in (L, L + 5):
            O2, l2 = o.forward(q, k, v, 1.0, causal, w)
            assert np.array_equal(O1, O2) and np.array_equal(l1, l2)


def _torch_mask(L, causal, window):
    m = torch.zeros(L, L, dtype=torch.bool)
    for i in range(L):
        for j in allowed_range(i, L, causal, window):
            m[i, j] = True
    return m


def pin_torch_sdpa_and_logsumexp(o):
    B, Hq, Hkv, L, d = 2, 4, 2, 17, 8
    q, k, v = rnd((B, Hq, L, d), 29), rnd((B, Hkv, L, d), 30), rnd((B, Hkv, L, d), 31)
    scale = 1.0 / math.sqrt(d)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    for causal, window in MASKS:
        mask = _torch_mask(L, causal, window)
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale, enable_gqa=True).numpy()
        O, lse = o.forward(q, k, v, scale, causal, window)
        assert np.allclose(O, ref, atol=1e-13, rtol=0), "oracle O disagrees with torch float64 SDPA"
        kr = torch.repeat_interleave(tk, Hq // Hkv, dim=1)
        S = (tq @ kr.transpose(-1, -2)).numpy() * scale
        S = np.where(mask.numpy(), S, -np.inf)
        assert np.allclose(lse, scipy.special.logsumexp(S, axis=-1), atol=1e-13, rtol=0)


def pin_backward_vs_torch_autograd(o):
    B, Hq, Hkv, L, d = 1, 4, 2, 13, 6
    q, k, v, do = rnd((B, Hq, L, d), 32), rnd((B, Hkv, L, d), 33), rnd((B, Hkv, L, d), 34), rnd((B, Hq, L, d), 35)
    for causal, window in MASKS:
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
        out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=_torch_mask(L, causal, window),
                                             scale=0.4, enable_gqa=True)
        out.backward(torch.from_numpy(do))
        dq, dk, dv = o.backward(q, k, v, do, 0.4, causal, window)
        assert np.allclose(dq, tq.grad.numpy(), atol=1e-12, rtol=0)
        assert np.allclose(dk, tk.grad.numpy(), atol=1e-12, rtol=0)
        assert np.allclose(dv, tv.grad.numpy(), atol=1e-12, rtol=0)


def pin_backward_finite_differences(o):
    B, Hq, Hkv, L, d = 1, 2, 1, 5, 3
    q, k, v, do = rnd((B, Hq, L, d), 36), rnd((B, Hkv, L, d), 37), rnd((B, Hkv, L, d), 38), rnd((B, Hq, L, d), 39)
    h = 1e-6
    for causal, window in [(False, 0), (True, 0), (True, 2), (False, 2)]:
        grads = o.backward(q, k, v, do, 0.8, causal, window)

        def f(q_, k_, v_):
            return float((o.forward(q_, k_, v_, 0.8, causal, window)[0] * do).sum())

        for which, x in enumerate((q, k, v)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [q, k, v]
                args_m = [q, k, v]
                args_p[which], args_m[which] = xp, xm
                num[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
            g = grads[which]
            rel = np.linalg.norm(num - g) / np.linalg.norm(num)
            assert rel <= 1e-6, f"finite-difference mismatch on input {which}: rel {rel:.2e}"


def pin_backward_identities(o):
    B, Hq, Hkv, L, d = 2, 4, 2, 15, 5
    q, k, v, do = rnd((B, Hq, L, d), 40), rnd((B, Hkv, L, d), 41), rnd((B, Hkv, L, d), 42), rnd((B, Hq, L, d), 43)
    for causal, window in MASKS:
        dq, dk, dv = o.backward(q, k, v, do, 0.5, causal, window)
        assert np.allclose(dk.sum(2), 0.0, atol=1e-12), "sum_j dK_j must vanish"
        assert np.allclose(dv.sum(2), do.reshape(B, Hkv, Hq // Hkv, L, d).sum((2, 3)), atol=1e-12)


def pin_tiled_recurrence_equals_direct(o):
    B, Hq, Hkv, L, d = 1, 4, 2, 37, 6
    q, k, v = rnd((B, Hq, L, d), 44, 2.0), rnd((B, Hkv, L, d), 45, 2.0), rnd((B, Hkv, L, d), 46)
    rng = np.random.default_rng(47)
    for causal, window in MASKS:
        for _ in range(3):
            re = [0] + sorted(rng.choice(np.arange(1, L), size=4, replace=False).tolist()) + [L]
            ce = [0] + sorted(rng.choice(np.arange(1, L), size=5, replace=False).tolist()) + [L]
            O1, l1 = o.forward(q, k, v, 0.45, causal, window)
            O2, l2 = o.tiled_online_forward(q, k, v, 0.45, causal, window, re, ce)
            assert np.allclose(O1, O2, atol=1e-12, rtol=0) and np.allclose(l1, l2, atol=1e-12, rtol=0)


def pin_rows_subset(o):
    L = 20
    q, k, v = rnd((1, 2, L, 4), 48), rnd((1, 2, L, 4), 49), rnd((1, 2, L, 4), 50)
    rows = np.array([0, 3, 7, 19])
    for causal, window in MASKS:
        O, l = o.forward(q, k, v, 0.5, causal, window)
        Or, lr = o.forward_rows(q, k, v, rows, 0.5, causal, window)
        assert np.array_equal(O[:, :, rows], Or) and np.array_equal(l[:, :, rows], lr)


# ---------------------------------------------------- chunked (ring-attention) pins

def pin_block_whole_sequence_equals_full(o):
    # one chunk holding every query and key is the full definition, and moving
    # both chunks by the same offset changes nothing
    for causal, window in MASKS:
        q, k, v = rnd((1, 4, 10, 5), 60), rnd((1, 2, 10, 5), 61), rnd((1, 2, 10, 5), 62)
        O, l = o.forward(q, k, v, 0.4, causal, window)
        for off in (0, 1000):
            Ob, lb = o.block_forward(q, k, v, 0.4, causal, window, off, off)
            assert np.allclose(Ob, O, atol=1e-13, rtol=0) and np.allclose(lb, l, atol=1e-13, rtol=0)


def pin_block_brute_force(o):
    # tiny chunks at offsets, by explicit loops over the definition (empty rows: O = 0, LSE = -inf)
    q, k, v = rnd((1, 2, 3, 2), 70), rnd((1, 1, 5, 2), 71), rnd((1, 1, 5, 2), 72)
    for causal, window, qo, ko in [(True, 0, 4, 2), (True, 2, 4, 2), (False, 0, 0, 7), (True, 0, 0, 3),
                                   (True, 3, 9, 3), (False, 2, 4, 2), (False, 3, 1, 4)]:
        O, l = o.block_forward(q, k, v, 0.7, causal, window, qo, ko)
        for h in range(2):
            for i in range(3):
                keys = [j for j in range(5)
                        if (not causal or ko + j <= qo + i) and (window <= 0 or ko + j >= qo + i - window + 1)
                        and (causal or window <= 0 or ko + j <= qo + i + window - 1)]
                if not keys:
                    assert np.isneginf(l[0, h, i]) and np.all(O[0, h, i] == 0.0)
                    continue
                e = [math.exp(0.7 * sum(q[0, h, i, c] * k[0, 0, j, c] for c in range(2))) for j in keys]
                assert abs(l[0, h, i] - math.log(sum(e))) < 1e-12
                for c in range(2):
                    ref = sum(w * v[0, 0, j, c] for w, j in zip(e, keys)) / sum(e)
                    assert abs(O[0, h, i, c] - ref) < 1e-12


def pin_merged_partials_equal_full(o):
    # partial results over any partition of the keys merge to the full result
    L = 23
    for causal, window in MASKS:
        q, k, v = rnd((2, 4, L, 6), 80), rnd((2, 2, L, 6), 81), rnd((2, 2, L, 6), 82)
        O, l = o.forward(q, k, v, 0.3, causal, window)
        for cuts in ([0, 7, 23], [0, 1, 12, 20, 23]):
            for r0, r1 in [(0, 23), (5, 16)]:
                acc = None
                for c0, c1 in zip(cuts[:-1], cuts[1:]):
                    part = o.block_forward(q[:, :, r0:r1], k[:, :, c0:c1], v[:, :, c0:c1], 0.3, causal, window,
                                           r0, c0)
                    acc = part if acc is None else o.merge_partials(*acc, *part)
                assert np.allclose(acc[0], O[:, :, r0:r1], atol=1e-12, rtol=0)
                assert np.allclose(acc[1], l[:, :, r0:r1], atol=1e-12, rtol=0)
        a = o.block_forward(q, k[:, :, :9], v[:, :, :9], 0.3, causal, window, 0, 0)
        b = o.block_forward(q, k[:, :, 9:], v[:, :, 9:], 0.3, causal, window, 0, 9)
        m1, m2 = o.merge_partials(*a, *b), o.merge_partials(*b, *a)
        assert np.allclose(m1[0], m2[0], atol=1e-14, rtol=0) and np.allclose(m1[1], m2[1], atol=1e-14, rtol=0)


def pin_merge_edge_cases(o):
    oa_, la = rnd((1, 1, 3, 2), 90), np.array([[[0.3, -np.inf, 2.0]]])
    ob_, lb = rnd((1, 1, 3, 2), 91), np.array([[[-np.inf, -np.inf, -1.0]]])
    O, l = o.merge_partials(oa_, la, ob_, lb)
    assert np.array_equal(O[0, 0, 0], oa_[0, 0, 0]) and l[0, 0, 0] == 0.3      # an empty side is neutral
    assert np.array_equal(O[0, 0, 1], [0.0, 0.0]) and np.isneginf(l[0, 0, 1])   # both sides empty
    assert abs(l[0, 0, 2] - np.logaddexp(2.0, -1.0)) < 1e-14
    w = 1.0 / (1.0 + math.exp(-3.0))
    assert np.allclose(O[0, 0, 2], w * oa_[0, 0, 2] + (1 - w) * ob_[0, 0, 2], atol=1e-14, rtol=0)


def pin_block_backward_sums_to_full(o):
    L = 17
    for causal, window in MASKS:
        q, k, v, do = rnd((1, 4, L, 5), 100), rnd((1, 2, L, 5), 101), rnd((1, 2, L, 5), 102), rnd((1, 4, L, 5), 103)
        dq, dk, dv = o.backward(q, k, v, do, 0.6, causal, window)
        O, l = o.forward(q, k, v, 0.6, causal, window)
        gq, gk, gv = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
        qc, kc = [0, 6, 17], [0, 4, 11, 17]
        for r0, r1 in zip(qc[:-1], qc[1:]):
            for c0, c1 in zip(kc[:-1], kc[1:]):
                pq, pk, pv = o.block_backward(q[:, :, r0:r1], k[:, :, c0:c1], v[:, :, c0:c1], do[:, :, r0:r1],
                                              O[:, :, r0:r1], l[:, :, r0:r1], 0.6, causal, window, r0, c0)
                gq[:, :, r0:r1] += pq
                gk[:, :, c0:c1] += pk
                gv[:, :, c0:c1] += pv
        for g, ref in ((gq, dq), (gk, dk), (gv, dv)):
            assert np.allclose(g, ref, atol=1e-12, rtol=0)


def pin_decode_new_tokens_only_is_full_causal(o):
    # a cache holding exactly the Lq new tokens: bottom-right alignment is the plain causal forward
    q, k, v = rnd((2, 4, 6, 5), 110), rnd((2, 2, 6, 5), 111), rnd((2, 2, 6, 5), 112)
    for window in (0, 2):
        O, l = o.decode_forward(q, k, v, [6, 6], 0.5, True, window)
        Of, lf = o.forward(q, k, v, 0.5, True, window)
        assert np.allclose(O, Of, atol=1e-13, rtol=0) and np.allclose(l, lf, atol=1e-13, rtol=0)


def pin_decode_rows_match_whole_sequence(o):
    # new token t of a sequence of length n is row n - Lq + t of the whole-sequence forward;
    # sequences of different lengths share one padded cache
    L, Lq = 19, 3
    q_all, k, v = rnd((2, 4, L, 6), 120), rnd((2, 2, L, 6), 121), rnd((2, 2, L, 6), 122)
    lens = [L, 11]
    for causal, window in [(True, 0), (True, 4), (False, 0)]:
        q = np.stack([q_all[b, :, n - Lq:n] for b, n in enumerate(lens)])
        kc = k.copy()
        kc[1, :, lens[1]:] = 1e3          # entries past a sequence's length must be ignored
        O, l = o.decode_forward(q, kc, v, lens, 0.45, causal, window)
        for b, n in enumerate(lens):
            Of, lf = o.forward(q_all[b:b + 1, :, :n], k[b:b + 1, :, :n], v[b:b + 1, :, :n], 0.45, causal, window)
            assert np.allclose(O[b], Of[0, :, n - Lq:n], atol=1e-12, rtol=0)
            assert np.allclose(l[b], lf[0, :, n - Lq:n], atol=1e-12, rtol=0)


def pin_decode_rolling_window_buffer(o):
    # a single new token with a rolling buffer of the last W keys (slots in any order) needs no
    # mask: the non-causal decode over the W valid slots equals the windowed causal row
    L, W = 23, 6
    q_all, k, v = rnd((1, 2, L, 4), 130), rnd((1, 1, L, 4), 131), rnd((1, 1, L, 4), 132)
    Of, lf = o.forward(q_all, k, v, 0.6, True, W)
    pos = np.arange(L - W, L)
    slots = pos % W                                   # position p lives in slot p mod W
    kb, vb = np.empty((1, 1, W, 4)), np.empty((1, 1, W, 4))
    kb[:, :, slots], vb[:, :, slots] = k[:, :, pos], v[:, :, pos]
    O, l = o.decode_forward(q_all[:, :, L - 1:], kb, vb, [W], 0.6, False, 0)
    assert np.allclose(O[0, :, 0], Of[0, :, L - 1], atol=1e-12, rtol=0)
    assert np.allclose(l[0, :, 0], lf[0, :, L - 1], atol=1e-12, rtol=0)


def pin_rolling_buffer_rows_match_whole_sequence(o):
    # A rolling buffer of W slots, filled token by token (position p overwrites slot p mod W),
    # plus the Lq new tokens' own K/V: new token t must equal row n + t of the whole-sequence
    # causal forward with window w <= W -- before the buffer is full, exactly full, and wrapped
    # (n not a multiple of W), for Lq = 1, several tokens, and more tokens than slots.
    W, d = 5, 4
    N = 17
    q_all, k, v = rnd((2, 4, N, d), 140), rnd((2, 2, N, d), 141), rnd((2, 2, N, d), 142)
    for n, Lq, w in [(0, 3, 0), (3, 2, 0), (5, 1, 0), (7, 3, 0), (11, 4, 2), (9, 1, 5), (6, 8, 0), (12, 5, 3)]:
        kb, vb = np.full((2, 2, W, d), 1e3), np.full((2, 2, W, d), -1e3)   # never-written slots are junk
        for p in range(n):
            kb[:, :, p % W], vb[:, :, p % W] = k[:, :, p], v[:, :, p]
        seen = [n, n]
        O, l = o.rolling_decode_forward(q_all[:, :, n:n + Lq], kb, vb, k[:, :, n:n + Lq], v[:, :, n:n + Lq],
                                        seen, 0.55, w)
        Of, lf = o.forward(q_all[:, :, :n + Lq], k[:, :, :n + Lq], v[:, :, :n + Lq], 0.55, True, w or W)
        assert np.allclose(O, Of[:, :, n:n + Lq], atol=1e-12, rtol=0), (n, Lq, w)
        assert np.allclose(l, lf[:, :, n:n + Lq], atol=1e-12, rtol=0), (n, Lq, w)


def pin_general_mask_reduces_to_causal_window(o):
    L = 13
    pos = np.arange(L)
    for causal, window in MASKS:
        assert np.array_equal(o.general_mask(pos, pos, causal, window), o.allowed_mask(pos, L, causal, window))
    ones = np.ones((1, 1), dtype=bool)
    assert np.array_equal(o.general_mask(pos, pos, True, 0, ones, 64), o.allowed_mask(pos, L, True, 0))


def pin_general_mask_brute_force(o):
    L, blk = 11, 3
    rng = np.random.default_rng(140)
    bm = rng.integers(0, 2, size=(4, 4)).astype(bool)
    for causal, window, glob in [(False, 3, ()), (False, 0, (0, 10)), (True, 2, (5,)), (False, 4, (0, 10)),
                                 (True, 0, (3, 7))]:
        for use_bm in (False, True):
            ok = o.general_mask(np.arange(L), np.arange(L), causal, window, bm if use_bm else None, blk, glob)
            for i in range(L):
                for j in range(L):
                    local = (window <= 0 or abs(i - j) < window) and (not use_bm or bm[i // blk][j // blk])
                    want = (local or i in glob or j in glob) and (not causal or j <= i)
                    assert ok[i, j] == want, (causal, window, glob, use_bm, i, j)


def pin_masked_forward_backward_reduce_to_plain(o):
    L = 12
    for causal, window in MASKS:
        q, k, v, do = rnd((1, 4, L, 5), 150), rnd((1, 2, L, 5), 151), rnd((1, 2, L, 5), 152), rnd((1, 4, L, 5), 153)
        ok = o.allowed_mask(np.arange(L), L, causal, window)
        O, l = o.forward_with_mask(q, k, v, 0.4, ok)
        Of, lf = o.forward(q, k, v, 0.4, causal, window)
        assert np.allclose(O, Of, atol=1e-13, rtol=0) and np.allclose(l, lf, atol=1e-13, rtol=0)
        g = o.backward_with_mask(q, k, v, do, 0.4, ok)
        gf = o.backward(q, k, v, do, 0.4, causal, window)
        for a, b in zip(g, gf):
            assert np.allclose(a, b, atol=1e-12, rtol=0)


def pin_global_rows_are_unmasked(o):
    # a global query attends to every key: its row equals the unmasked row; a local row with a
    # symmetric window sees the global keys in addition to its window
    L = 16
    q, k, v = rnd((1, 2, L, 4), 160), rnd((1, 2, L, 4), 161), rnd((1, 2, L, 4), 162)
    ok = o.general_mask(np.arange(L), np.arange(L), False, 3, None, 64, (0, L - 1))
    O, l = o.forward_with_mask(q, k, v, 0.5, ok)
    Of, lf = o.forward(q, k, v, 0.5, False, 0)
    for r in (0, L - 1):
        assert np.allclose(O[:, :, r], Of[:, :, r], atol=1e-13, rtol=0)
    i = 7
    keys = sorted({0, L - 1} | set(range(i - 2, i + 3)))
    s = 0.5 * q[0, 1, i] @ k[0, 1, keys].T
    assert abs(l[0, 1, i] - scipy.special.logsumexp(s)) < 1e-12


def pin_masked_backward_finite_differences(o):
    L, d = 6, 3
    q, k, v, do = rnd((1, 1, L, d), 170), rnd((1, 1, L, d), 171), rnd((1, 1, L, d), 172), rnd((1, 1, L, d), 173)
    ok = o.general_mask(np.arange(L), np.arange(L), False, 2, [[1, 0], [1, 1]], 3, (2,))
    dq, dk, dv = o.backward_with_mask(q, k, v, do, 0.7, ok)
    f = lambda q_, k_, v_: float((o.forward_with_mask(q_, k_, v_, 0.7, ok)[0] * do).sum())
    eps = 1e-6
    for x, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * eps)
        assert np.allclose(num, g, rtol=1e-6, atol=1e-8)


def pin_masked_rows_equal_whole_sequence(o):
    L = 40
    q, k, v, do = rnd((2, 4, L, 6), 180), rnd((2, 2, L, 6), 181), rnd((2, 2, L, 6), 182), rnd((2, 4, L, 6), 183)
    bm = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 1]], dtype=bool)
    for causal, window, glob, blk in [(False, 5, (0, -1), None), (True, 7, (13,), None), (False, 0, (), bm),
                                      (True, 4, (2, 30), bm)]:
        gl = tuple(p + L if p < 0 else p for p in glob)
        ok = o.general_mask(np.arange(L), np.arange(L), causal, window, blk, 16, gl)
        O, l = o.forward_with_mask(q, k, v, 0.45, ok)
        dq = o.backward_with_mask(q, k, v, do, 0.45, ok)[0]
        rows = np.array([0, 3, 17, 39])
        Or, lr = o.forward_rows_with_mask(q, k, v, rows, 0.45, ok[rows])
        assert np.allclose(Or, O[:, :, rows], atol=1e-13, rtol=0) and np.allclose(lr, l[:, :, rows], atol=1e-13, rtol=0)
        dqr = o.dq_rows_with_mask(q, k, v, do, rows, 0.45, ok[rows])
        assert np.allclose(dqr, dq[:, :, rows], atol=1e-12, rtol=0)


MASK_PINS = [pin_general_mask_reduces_to_causal_window, pin_general_mask_brute_force, pin_masked_rows_equal_whole_sequence,
             pin_masked_forward_backward_reduce_to_plain, pin_global_rows_are_unmasked,
             pin_masked_backward_finite_differences]


BLOCK_PINS = [pin_block_whole_sequence_equals_full, pin_block_brute_force, pin_merged_partials_equal_full,
              pin_merge_edge_cases, pin_block_backward_sums_to_full]
DECODE_PINS = [pin_decode_new_tokens_only_is_full_causal, pin_decode_rows_match_whole_sequence,
               pin_decode_rolling_window_buffer, pin_rolling_buffer_rows_match_whole_sequence]


PINS = [pin_rows_stochastic, pin_two_key_worked_example, pin_length_one, pin_zero_query_is_mean,
        pin_identical_keys, pin_convexity, pin_shift_invariance, pin_permutation_noncausal,
        pin_gqa_is_repeated_mha, pin_window_at_least_L_is_causal, pin_torch_sdpa_and_logsumexp,
        pin_backward_vs_torch_autograd, pin_backward_finite_differences, pin_backward_identities,
        pin_tiled_recurrence_equals_direct, pin_rows_subset] + BLOCK_PINS + DECODE_PINS + MASK_PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle)


# ----------------------------------------------------------------- planted mistakes

def _some_pin_fails(pins):
    for p in pins:
        try:
            p(oracle)
        except AssertionError:
            return True
    return False


FWD_PINS = [pin_zero_query_is_mean, pin_torch_sdpa_and_logsumexp, pin_length_one,
            pin_shift_invariance, pin_gqa_is_repeated_mha, pin_rows_stochastic]
BWD_PINS = [pin_backward_finite_differences, pin_backward_vs_torch_autograd, pin_backward_identities]


def test_planted_causal_off_by_one(monkeypatch):
    good = oa.allowed_mask

    def bad(rows, L, causal, window):
        ok = good(rows, L, False, 0)
        i = np.asarray(rows)[:, None]
        j = np.arange(L)[None, :]
        if causal:
            ok &= j < i                      # diagonal wrongly excluded
        if window > 0:
            ok &= j >= i - window + 1
        return ok

    monkeypatch.setattr(oa, "allowed_mask", bad)
    assert _some_pin_fails(FWD_PINS)


def test_planted_window_off_by_one(monkeypatch):
    good = oa.allowed_mask

    def bad(rows, L, causal, window):
        ok = good(rows, L, causal, 0)
        if window > 0:
            ok &= np.arange(L)[None, :] >= np.asarray(rows)[:, None] - window   # one key too many
        return ok

    monkeypatch.setattr(oa, "allowed_mask", bad)
    assert _some_pin_fails(FWD_PINS)


def test_planted_gqa_head_mapping(monkeypatch):
    monkeypatch.setattr(oa, "kv_head_of", lambda h, hq, hkv: h % hkv)   # interleaved instead of grouped
    assert _some_pin_fails(FWD_PINS)


def test_planted_lse_without_max(monkeypatch):
    good = oa._masked_softmax_rows

    def bad(S, ok):
        A, lse = good(S, ok)
        Sm = np.where(ok, S, -np.inf)
        return A, lse - Sm.max(axis=-1)       # drops the max term from the log-sum-exp
    monkeypatch.setattr(oa, "_masked_softmax_rows", bad)
    assert _some_pin_fails(FWD_PINS)


def test_planted_softmax_backward_without_D(monkeypatch):
    monkeypatch.setattr(oa, "_softmax_backward", lambda A, dA: A * dA)
    assert _some_pin_fails(BWD_PINS)


def test_planted_softmax_backward_sign(monkeypatch):
    monkeypatch.setattr(oa, "_softmax_backward",
                        lambda A, dA: A * ((A * dA).sum(-1, keepdims=True) - dA))
    assert _some_pin_fails(BWD_PINS)


def test_symmetric_window_mask_and_bad_gqa():
    # w = 2 without causal: each position sees itself and one neighbour on each side
    want = np.array([[1, 1, 0, 0], [1, 1, 1, 0], [0, 1, 1, 1], [0, 0, 1, 1]], dtype=bool)
    assert np.array_equal(oracle.allowed_mask(np.arange(4), 4, False, 2), want)
    with pytest.raises(ValueError):
        oracle.kv_head_of(0, 6, 4)


def test_planted_block_offset_sign(monkeypatch):
    good = oa.position_mask
    # queries and keys swapped in the causal comparison
    monkeypatch.setattr(oa, "position_mask", lambda qp, kp, causal, window: good(kp, qp, causal, window).T)
    assert _some_pin_fails(BLOCK_PINS)


def test_planted_merge_unnormalised(monkeypatch):
    def bad(o_a, lse_a, o_b, lse_b):
        lse = np.logaddexp(lse_a, lse_b)
        return np.exp(lse_a)[..., None] * o_a + np.exp(lse_b)[..., None] * o_b, lse   # weights not divided
    monkeypatch.setattr(oa, "merge_partials", bad)
    monkeypatch.setattr(oracle, "merge_partials", bad)
    assert _some_pin_fails(BLOCK_PINS)


def test_planted_block_backward_D_over_chunk(monkeypatch):
    # each chunk treated as if it held the whole row (its own softmax and its own D)
    monkeypatch.setattr(oracle, "block_backward",
                        lambda q, k, v, dout, o, lse, scale, causal=False, window=0, q_offset=0, k_offset=0:
                        _chunk_local_backward(q, k, v, dout, scale, causal, window, q_offset, k_offset))
    assert _some_pin_fails([pin_block_backward_sums_to_full])


def _chunk_local_backward(q, k, v, dout, scale, causal, window, q_offset, k_offset):
    """A wrong chunk gradient: the chunk treated as if it were the whole row (own softmax)."""
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    ok = oa.position_mask(q_offset + np.arange(Lq), k_offset + np.arange(Lk), causal, window)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kh = oa.kv_head_of(h, Hq, Hkv)
            A, _ = oa._masked_softmax_rows(scale * (q[b, h] @ k[b, kh].T), ok)
            dv[b, kh] += A.T @ dout[b, h]
            dS = oa._softmax_backward(A, dout[b, h] @ v[b, kh].T)
            dq[b, h] = scale * (dS @ k[b, kh])
            dk[b, kh] += scale * (dS.T @ q[b, h])
    return dq, dk, dv


def test_planted_decode_top_left_alignment(monkeypatch):
    # new tokens placed at the start of the cache instead of its end
    good = oa.block_forward
    monkeypatch.setattr(oa, "block_forward", lambda q, k, v, scale, causal=False, window=0, q_offset=0, k_offset=0:
                        good(q, k, v, scale, causal, window, 0, k_offset))
    assert _some_pin_fails(DECODE_PINS)


def test_planted_rolling_buffer_read_in_slot_order(monkeypatch):
    # the buffer read back in slot order 0..W-1 instead of position order
    def bad(q, k_ring, v_ring, k_new, v_new, seen, scale, window=0):
        q, k_ring, v_ring, k_new, v_new = (np.asarray(x, dtype=np.float64) for x in (q, k_ring, v_ring, k_new, v_new))
        B, W = q.shape[0], k_ring.shape[2]
        outs = []
        for b in range(B):
            n = int(seen[b])
            m = min(n, W)
            ks = np.concatenate([k_ring[b:b + 1, :, :m], k_new[b:b + 1]], axis=2)
            vs = np.concatenate([v_ring[b:b + 1, :, :m], v_new[b:b + 1]], axis=2)
            outs.append(oa.block_forward(q[b:b + 1], ks, vs, scale, True, window or W, n, n - m))
        return np.concatenate([x[0] for x in outs]), np.concatenate([x[1] for x in outs])
    monkeypatch.setattr(oracle, "rolling_decode_forward", bad)
    assert _some_pin_fails([pin_rolling_buffer_rows_match_whole_sequence])


def test_planted_rolling_buffer_window_off_by_one(monkeypatch):
    good = oa.rolling_decode_forward
    monkeypatch.setattr(oracle, "rolling_decode_forward",
                        lambda q, kr, vr, kn, vn, seen, scale, window=0:
                        good(q, kr, vr, kn, vn, seen, scale, (window or kr.shape[2]) - 1 or 1))
    assert _some_pin_fails([pin_rolling_buffer_rows_match_whole_sequence])


def test_planted_general_mask_window_off_by_one(monkeypatch):
    good = oa.general_mask

    def bad(q_pos, k_pos, causal=False, window=0, block_mask=None, block=64, global_pos=()):
        return good(q_pos, k_pos, causal, window + 1 if window > 0 else 0, block_mask, block, global_pos)
    monkeypatch.setattr(oa, "general_mask", bad)
    monkeypatch.setattr(oracle, "general_mask", bad)
    assert _some_pin_fails(MASK_PINS)


def test_planted_global_keys_ignored(monkeypatch):
    good = oa.general_mask

    def bad(q_pos, k_pos, causal=False, window=0, block_mask=None, block=64, global_pos=()):
        ok = good(q_pos, k_pos, causal, window, block_mask, block, ())
        return ok | good(q_pos, k_pos, causal, window, block_mask, block, global_pos) & np.isin(
            np.asarray(q_pos)[:, None], list(global_pos))       # global queries kept, global keys dropped
    monkeypatch.setattr(oa, "general_mask", bad)
    monkeypatch.setattr(oracle, "general_mask", bad)
    assert _some_pin_fails(MASK_PINS)


def test_planted_symmetric_window_one_sided(monkeypatch):
    good = oa.position_mask

    def bad(q_pos, k_pos, causal, window):
        # the window's upper edge dropped: a non-causal window reaching back only
        if window > 0 and not causal:
            i = np.asarray(q_pos)[:, None]
            j = np.asarray(k_pos)[None, :]
            return j >= i - window + 1
        return good(q_pos, k_pos, causal, window)
    monkeypatch.setattr(oa, "position_mask", bad)
    assert _some_pin_fails(PINS)
