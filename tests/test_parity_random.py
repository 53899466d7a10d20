"""Seeded random parity cases across the GPU paths -- whole-sequence forward and
backward, ring chunk pairs, general masks, decode -- against the fp64 oracle.

Each case draws its sizes from a fixed seed (ragged lengths, offsets up to 2^29,
windows up to INT_MAX, GQA ratios, dtypes, block patterns, global positions), so the set is the same
on every run and a failing case is named by its index and parameters.
Tolerances as everywhere: O max-abs 2e-2, LSE max-abs 1e-3 (rows with no allowed
key exactly O = 0, LSE = -inf), gradients relative L2 2e-2.
"""

import math
import random

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KINDS = ("range", "chunk", "mask", "decode")
N_CASES = 60


def fa():
    import exact_tiled_attention_flash_amd as m
    m.library()
    return m


def f64(t):
    return t.detach().double().cpu().numpy()


def rel(x, ref):
    den = max(float(np.linalg.norm(ref)), 1e-2 * math.sqrt(ref.size))
    return float(np.linalg.norm(f64(x) - ref)) / den


def draw(shape, seed, dt):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(dt)


def case_params(i):
    rng = random.Random(9000 + i)
    p = dict(kind=KINDS[i % len(KINDS)], seed=rng.randrange(1 << 20),
             dt=rng.choice([torch.bfloat16, torch.float16]), d=rng.choice([64, 128]),
             G=rng.choice([1, 2, 4]), Hkv=rng.choice([1, 2]), B=rng.choice([1, 2]),
             causal=rng.random() < 0.6, window=rng.choice([0, 0, 1, 7, 65, 300, 1 << 30, 2**31 - 1]))
    p["Hq"] = p["G"] * p["Hkv"]
    if p["kind"] == "range":
        p["L"] = rng.randrange(1, 900)
    elif p["kind"] == "chunk":
        p["Lq"], p["Lk"] = rng.randrange(1, 500), rng.randrange(1, 500)
        p["ko"] = rng.randrange(0, 900)
        p["qo"] = max(0, p["ko"] + rng.randrange(-300, 600))
        if rng.random() < 0.3:             # near the top of the offset range (2^29)
            p["ko"] += (1 << 29) - 2000
            p["qo"] += (1 << 29) - 2000
    elif p["kind"] == "mask":
        p["L"] = rng.randrange(2, 1400)
        p["blk"] = rng.choice([64, 128, 192])
        p["use_bm"] = rng.random() >= 0.4
        p["density"] = rng.choice([0.2, 0.5, 0.9])
        p["glob"] = tuple(rng.randrange(-p["L"], p["L"]) for _ in range(rng.choice([0, 0, 1, 2, 5])))
    else:
        Lq = rng.choice([1, 1, 2, 3])
        while p["G"] * Lq > 32:
            Lq -= 1
        p["Lq"] = Lq
        p["Lk"] = rng.randrange(Lq, 20000)
        p["lens"] = [rng.randrange(Lq, p["Lk"] + 1) for _ in range(p["B"])]
    return p


def check_out(o, lse, O_ref, l_ref):
    empty = np.isneginf(l_ref)
    ln = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(ln), empty), "rows with no allowed key must be exactly those with LSE = -inf"
    on = f64(o)
    assert np.all(on[empty] == 0.0)
    err_o = float(np.abs(on - O_ref).max())
    err_l = float(np.abs(ln[~empty] - l_ref[~empty]).max()) if (~empty).any() else 0.0
    return err_o, err_l


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    p = case_params(i)
    print(f"[random] case {i}: {p}", flush=True)
    B, Hq, Hkv, d, dt, seed = p["B"], p["Hq"], p["Hkv"], p["d"], p["dt"], p["seed"]
    causal, window = p["causal"], p["window"]
    s = 1.0 / math.sqrt(d)
    err_g = 0.0
    if p["kind"] == "range":
        L = p["L"]
        q, k, v, do = (draw((B, h, L, d), seed + n, dt) for n, h in enumerate((Hq, Hkv, Hkv, Hq)))
        qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
        o, lse = fa().fwd(qd, kd, vd, causal=causal, window=window, scale=s)
        grads = fa().bwd(qd, kd, vd, o, lse, dod, causal=causal, window=window, scale=s)
        torch.cuda.synchronize()
        err_o, err_l = check_out(o, lse, *oracle.forward(f64(q), f64(k), f64(v), s, causal, window))
        ref = oracle.backward(f64(q), f64(k), f64(v), f64(do), s, causal, window)
        err_g = max(rel(x, r) for x, r in zip(grads, ref))
    elif p["kind"] == "chunk":
        Lq, Lk, qo, ko = p["Lq"], p["Lk"], p["qo"], p["ko"]
        q, k, v = draw((B, Hq, Lq, d), seed, dt), draw((B, Hkv, Lk, d), seed + 1, dt), draw((B, Hkv, Lk, d), seed + 2, dt)
        o, lse = fa().fwd_block(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window=window, q_offset=qo,
                                k_offset=ko, scale=s)
        torch.cuda.synchronize()
        err_o, err_l = check_out(o, lse, *oracle.block_forward(f64(q), f64(k), f64(v), s, causal, window, qo, ko))
    elif p["kind"] == "mask":
        L, blk = p["L"], p["blk"]
        nbm = (L + blk - 1) // blk
        bm = (np.random.default_rng(seed).random((nbm, nbm)) < p["density"]) if p["use_bm"] else None
        q, k, v, do = (draw((B, h, L, d), seed + n, dt) for n, h in enumerate((Hq, Hkv, Hkv, Hq)))
        plan = fa().MaskPlan(L, causal=causal, window=window, global_tokens=p["glob"],
                             block_mask=None if bm is None else torch.from_numpy(bm), block=blk, device=DEV)
        qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
        o, lse = fa().fwd_masked(qd, kd, vd, plan, scale=s)
        grads = fa().bwd_masked(qd, kd, vd, o, lse, dod, plan, scale=s)
        torch.cuda.synchronize()
        gl = tuple(x + L if x < 0 else x for x in p["glob"])
        ok = oracle.general_mask(np.arange(L), np.arange(L), causal, window, bm, blk, gl)
        err_o, err_l = check_out(o, lse, *oracle.forward_with_mask(f64(q), f64(k), f64(v), s, ok))
        ref = oracle.backward_with_mask(f64(q), f64(k), f64(v), f64(do), s, ok)
        err_g = max(rel(x, r) for x, r in zip(grads, ref))
    else:
        Lq, Lk, lens = p["Lq"], p["Lk"], p["lens"]
        cw = window if causal else 0
        q, k, v = draw((B, Hq, Lq, d), seed, dt), draw((B, Hkv, Lk, d), seed + 1, dt), draw((B, Hkv, Lk, d), seed + 2, dt)
        cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
        o, lse = fa().decode(q.to(DEV), k.to(DEV), v.to(DEV), cl, causal=causal, window=cw, scale=s)
        torch.cuda.synchronize()
        err_o, err_l = check_out(o, lse, *oracle.decode_forward(f64(q), f64(k), f64(v), np.array(lens), s, causal, cw))
    print(f"[random] case {i}: max|dO|={err_o:.2e} max|dLSE|={err_l:.2e} grad relL2={err_g:.2e}", flush=True)
    assert err_o <= 2e-2 and err_l <= 1e-3 and err_g <= 2e-2
