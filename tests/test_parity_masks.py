"""GPU parity of the general-mask path -- mask plan, masked forward, masked
backward -- against the fp64 oracle, through the C ABI.

The mask: allowed(i, j) = causal_ok and ((|i - j| < w and block_ok) or i global
or j global) (claspmoon.cn "14 · 缩放定律与高效注意力" §4.3, local window plus
global tokens; kler.cn §4.1.2 block-sparse masks, §3.2.1 / §5.1.2 a window
before and after with the first and last token global).  Tolerances as for the
plain path: O max-abs 2e-2, LSE max-abs 1e-3 (rows with no allowed key exactly
O = 0, LSE = -inf), gradients relative L2 2e-2.  The plan itself is checked
block by block against the oracle's boolean mask: a block it calls empty holds
no allowed pair, a full one only allowed pairs, and every block with an
allowed pair is listed.
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


def band(nbm, radius=1):
    i = np.arange(nbm)
    return np.abs(i[:, None] - i[None, :]) <= radius


def random_blocks(nbm, seed, p=0.35):
    m = np.random.default_rng(seed).random((nbm, nbm)) < p
    np.fill_diagonal(m, True)
    return m


def empty_row_blocks(nbm):
    m = band(nbm, 1)
    m[1, :] = False                 # query block 1 sees nothing
    return m


# name, B, Hq, Hkv, L, d, dtype, causal, window, global tokens, block, block-mask builder, seed
CASES = [
    ("sym w5 globals 0,-1 L1000", 1, 2, 2, 1000, 128, torch.bfloat16, False, 5, (0, -1), 64, None, 700),
    ("causal w64 globals L777 d64 gqa2", 1, 4, 2, 777, 64, torch.bfloat16, True, 64, (5, 700), 64, None, 701),
    ("band r1 b64 L1024", 1, 2, 2, 1024, 128, torch.bfloat16, False, 0, (), 64, lambda n: band(n, 1), 702),
    ("band r1 b128 causal L900 gqa4", 1, 4, 1, 900, 128, torch.bfloat16, True, 0, (), 128, lambda n: band(n, 1), 703),
    ("random b64 w200 globals fp16 L1300", 1, 2, 2, 1300, 128, torch.float16, False, 200, (0, 640, -1), 64,
     lambda n: random_blocks(n, 11), 704),
    ("random b192 causal globals L1100 d64", 2, 2, 2, 1100, 64, torch.bfloat16, True, 0, (3, 1000), 192,
     lambda n: random_blocks(n, 12, 0.5), 705),
    ("empty block row L500", 1, 2, 2, 500, 128, torch.bfloat16, False, 0, (), 64, empty_row_blocks, 706),
    ("no blocks, one global key L300", 1, 2, 2, 300, 128, torch.bfloat16, False, 0, (150,), 64,
     lambda n: np.zeros((n, n), dtype=bool), 707),
    ("globals only, many L700 fp16", 1, 2, 1, 700, 64, torch.float16, True, 1, tuple(range(0, 700, 37)), 64, None, 708),
    ("plain non-causal L300", 1, 2, 2, 300, 128, torch.bfloat16, False, 0, (), 64, None, 709),
    ("window 1 only L257", 1, 2, 2, 257, 128, torch.bfloat16, False, 1, (), 64, None, 710),
    # global keys inside wide windows: their band tiles would be full, but the folded keys
    # (at most 8 global positions) must be masked out of them and counted once
    ("sym w300 globals in band L1000", 1, 2, 2, 1000, 128, torch.bfloat16, False, 300, (300, 301, 700), 64,
     None, 711),
    ("causal w400 globals in band L900 d64", 1, 2, 1, 900, 64, torch.bfloat16, True, 400, (100, 450, -1), 64,
     None, 712),
    ("nine globals, tile path L800", 1, 2, 2, 800, 128, torch.bfloat16, False, 100, tuple(range(40, 800, 90)), 64,
     None, 713),
]


def case_inputs(case):
    name, B, Hq, Hkv, L, d, dt, causal, window, glob, block, bm_fn, seed = case
    w = W.small(name, B, Hq, Hkv, L, d, dtype=dt, causal=causal, window=window, seed=seed, backward=True)
    nbm = (L + block - 1) // block
    bm = None if bm_fn is None else bm_fn(nbm)
    gl = tuple(p + L if p < 0 else p for p in glob)
    ok = oracle.general_mask(np.arange(L), np.arange(L), causal, window, bm, block, gl)
    return w, bm, ok


def make_plan(case, bm):
    name, B, Hq, Hkv, L, d, dt, causal, window, glob, block, bm_fn, seed = case
    return fa().MaskPlan(L, causal=causal, window=window, global_tokens=glob,
                         block_mask=None if bm is None else torch.from_numpy(bm), block=block, device=DEV)


def check_out(o, lse, O_ref, l_ref, name):
    lse_n = lse.cpu().numpy().astype(np.float64)
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lse_n), empty), "empty rows must be exactly those with LSE = -inf"
    on = f64(o)
    assert np.all(on[empty] == 0.0)
    err_o = float(np.abs(on - O_ref).max())
    err_l = float(np.abs(lse_n[~empty] - l_ref[~empty]).max()) if (~empty).any() else 0.0
    print(f"[masks] {name}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e} empty rows={int(empty.sum())}", flush=True)
    assert err_o <= 2e-2 and err_l <= 1e-3


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_masked_forward_and_backward(case):
    print(f"[masks] case {case[0]} seed={case[-1]}", flush=True)
    w, bm, ok = case_inputs(case)
    q, k, v, do = W.make_inputs(w, with_dout=True)
    plan = make_plan(case, bm)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa().fwd_masked(qd, kd, vd, plan, scale=w.scale)
    dq, dk, dv = fa().bwd_masked(qd, kd, vd, o, lse, dod, plan, scale=w.scale)
    torch.cuda.synchronize()
    O_ref, l_ref = oracle.forward_with_mask(f64(q), f64(k), f64(v), w.scale, ok)
    check_out(o, lse, O_ref, l_ref, case[0])
    ref = oracle.backward_with_mask(f64(q), f64(k), f64(v), f64(do), w.scale, ok)
    errs = [rel(x, r) for x, r in zip((dq, dk, dv), ref)]
    print(f"[masks] {case[0]}: relL2 dQ={errs[0]:.3e} dK={errs[1]:.3e} dV={errs[2]:.3e}", flush=True)
    for x in (dq, dk, dv):
        assert torch.isfinite(x.float()).all()
    assert max(errs) <= 2e-2


# ---- the plan against the oracle mask, block by block (white box: the layout of
# flash_attn_mask_plan's buffer -- 256-byte aligned sections in the order
# gbits, row counts, row order, column counts, column order, meta, global
# positions, row entries, column entries).  The row lists leave global query
# rows to the global-row pass and the column lists leave global keys to the
# global-key pass, so each list is checked against the mask without them.

def plan_sections(L):
    nb, nw = (L + 63) // 64, (L + 127) // 128
    off, out = 0, {}
    for name, nbytes in (("gbits", 8 * nb), ("row_cnt", 4 * nw), ("row_ord", 4 * nw), ("col_cnt", 4 * nw),
                         ("col_ord", 4 * nw), ("meta", 16), ("gpos", 4 * L), ("row_ent", 4 * nw * nb),
                         ("col_ent", 4 * nw * nb)):
        out[name] = (off, nbytes)
        off = (off + nbytes + 255) & ~255
    return nb, nw, out


def check_lists(cnt, ent, ordr, heavy, nb, nw, ok, L, cols, no_full=None):
    assert sorted(ordr.tolist()) == list(range(nw))
    counts = cnt[ordr]
    assert np.all(counts[:-1] >= counts[1:]), "work-group order must be by descending count"
    assert 0 <= heavy <= nw // 2
    for wg in range(nw):
        e = ent[wg, :cnt[wg]]
        tiles = (e & 0xFFFF).astype(np.int64)
        assert np.all(np.diff(tiles) > 0), "entries ascending, no repeats"
        listed = {int(t): int(x) for t, x in zip(tiles, e)}
        for t in range(nb):
            for half in range(2):
                a = 2 * wg + half                      # the work-group's own 64-block
                blk = ok[64 * t:64 * t + 64, 64 * a:64 * a + 64] if cols else ok[64 * a:64 * a + 64, 64 * t:64 * t + 64]
                inside = 64 * a + 64 <= L and 64 * t + 64 <= L
                cls = (listed[t] >> (16 + 2 * half)) & 3 if t in listed else 0
                if blk.size == 0:
                    assert cls == 0, (wg, t, half, "a block past the sequence end must be empty")
                elif not blk.any():
                    assert cls in (0, 1), (wg, t, half, cls)
                else:
                    assert cls in (1, 2), (wg, t, half, "a block with an allowed pair must be listed")
                if cls == 2:
                    assert inside and blk.all(), (wg, t, half, "a full block must hold only allowed pairs")
                    if no_full is not None:
                        assert not no_full[64 * t:64 * t + 64].any(), (wg, t, half, "a folded global key in a full block")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_plan_blocks_match_oracle_mask(case):
    w, bm, ok = case_inputs(case)
    plan = make_plan(case, bm)
    torch.cuda.synchronize()
    raw = plan.plan.cpu().numpy()
    nb, nw, sec = plan_sections(w.L)

    def arr(name, dtype):
        o, n = sec[name]
        return raw[o:o + n].view(dtype)
    gbits = arr("gbits", np.uint64)
    gl = {p + w.L if p < 0 else p for p in case[9]}
    for p in range(w.L):
        assert bool((int(gbits[p // 64]) >> (p % 64)) & 1) == (p in gl)
    meta = arr("meta", np.int32)
    assert int(meta[2]) == len(gl) and arr("gpos", np.int32)[:len(gl)].tolist() == sorted(gl)
    # the mask without global rows (for the row lists) and without global keys (column lists).
    # With at most 8 global positions the row kernels fold the global keys into each row's
    # initial state: the row lists then hold only the window / block pairs, and no full
    # block of theirs may hold a global key (its tile must mask the key out).
    L = w.L
    i, j = np.arange(L)[:, None], np.arange(L)[None, :]
    causal_ok = (j <= i) if case[7] else np.ones((L, L), dtype=bool)
    base = oracle.general_mask(np.arange(L), np.arange(L), case[7], case[8], bm, case[10], ())
    isg = np.isin(np.arange(L), sorted(gl))
    fold = 0 < len(gl) <= 8
    ok_gk = isg[None, :] & causal_ok
    ok_rows = base if fold else base | ok_gk
    ok_cols = base | (isg[:, None] & causal_ok)
    assert np.array_equal(ok_rows | ok_cols | ok_gk, ok)
    check_lists(arr("row_cnt", np.int32), arr("row_ent", np.uint32).reshape(nw, nb), arr("row_ord", np.int32),
                int(meta[0]), nb, nw, ok_rows, w.L, cols=False, no_full=isg if fold else None)
    check_lists(arr("col_cnt", np.int32), arr("col_ent", np.uint32).reshape(nw, nb), arr("col_ord", np.int32),
                int(meta[1]), nb, nw, ok_cols, w.L, cols=True)


def test_plan_of_plain_masks_reproduces_range_kernels_bitwise():
    """A plan holding only causal / window masks visits the same tiles in the same
    order with the same tile steps as the range-tiled kernels: identical bits."""
    # (the last case: a window near INT_MAX admits every pair on both paths)
    for causal, window, L, d in ((True, 0, 1000, 128), (True, 100, 777, 64), (False, 33, 900, 128),
                                 (False, 2**31 - 1, 640, 64)):
        w = W.small("plain plan", 1, 4, 2, L, d, causal=causal, window=window, seed=720, backward=True)
        q, k, v, do = (t.to(DEV) for t in W.make_inputs(w, with_dout=True))
        plan = fa().MaskPlan(L, causal=causal, window=window, device=DEV)
        a = fa().fwd_masked(q, k, v, plan, scale=w.scale)
        b = fa().fwd(q, k, v, causal=causal, window=window, scale=w.scale)
        ga = fa().bwd_masked(q, k, v, a[0], a[1], do, plan, scale=w.scale)
        gb = fa().bwd(q, k, v, b[0], b[1], do, causal=causal, window=window, scale=w.scale)
        torch.cuda.synchronize()
        print(f"[masks] plain plan causal={causal} window={window} L={L}", flush=True)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
        for x, y in zip(ga, gb):
            assert torch.equal(x, y)


def test_autograd_with_mask_plan():
    case = CASES[0]
    w, bm, ok = case_inputs(case)
    q, k, v, do = W.make_inputs(w, with_dout=True)
    plan = make_plan(case, bm)
    qd, kd, vd = (t.to(DEV).requires_grad_(True) for t in (q, k, v))
    o = fa().scaled_dot_product_attention(qd, kd, vd, mask_plan=plan)
    o.backward(do.to(DEV))
    torch.cuda.synchronize()
    O_ref, _ = oracle.forward_with_mask(f64(q), f64(k), f64(v), w.scale, ok)
    assert float(np.abs(f64(o) - O_ref).max()) <= 2e-2
    ref = oracle.backward_with_mask(f64(q), f64(k), f64(v), f64(do), w.scale, ok)
    for x, r in zip((qd.grad, kd.grad, vd.grad), ref):
        assert rel(x, r) <= 2e-2


def check_identities(dk, dv, do, Hq, Hkv, name):
    G = Hq // Hkv
    B, _, L, d = dk.shape
    sdk, sdv = dk.double().sum(2), dv.double().sum(2)
    sdo = do.double().sum(2).reshape(B, Hkv, G, d).sum(2)
    err_dk = float((sdk.abs() / dk.double().abs().sum(2).clamp_min(1e-2 * L)).max())
    err_dv = float(((sdv - sdo).abs() / (dv.double().abs().sum(2) + sdo.abs()).clamp_min(1e-30)).max())
    print(f"[masks] {name} identities: |sum dK|/sum|dK| = {err_dk:.2e}, sum dV vs sum dO = {err_dv:.2e}", flush=True)
    assert err_dk < 2e-2 and err_dv < 2e-2


def test_hybrid_mask_mid_size_whole_heads():
    """The hybrid configuration's mask (window 513 both ways, first and last token
    global) at L = 4096, every output against the oracle."""
    w = W.HYBRID_SPARSE_128K.with_(name="hybrid L4096", B=1, Hq=4, Hkv=4, L=4096, seed=730)
    print(f"[masks] {w.name}", flush=True)
    q, k, v, do = W.make_inputs(w, with_dout=True)
    gl = tuple(p + w.L if p < 0 else p for p in w.global_tokens)
    ok = oracle.general_mask(np.arange(w.L), np.arange(w.L), w.causal, w.window, None, 64, gl)
    plan = fa().MaskPlan(w.L, causal=w.causal, window=w.window, global_tokens=w.global_tokens, device=DEV)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa().fwd_masked(qd, kd, vd, plan, scale=w.scale)
    grads = fa().bwd_masked(qd, kd, vd, o, lse, dod, plan, scale=w.scale)
    torch.cuda.synchronize()
    O_ref, l_ref = oracle.forward_with_mask(f64(q), f64(k), f64(v), w.scale, ok)
    check_out(o, lse, O_ref, l_ref, w.name)
    ref = oracle.backward_with_mask(f64(q), f64(k), f64(v), f64(do), w.scale, ok)
    errs = [rel(x, r) for x, r in zip(grads, ref)]
    print(f"[masks] {w.name}: relL2 dQ={errs[0]:.3e} dK={errs[1]:.3e} dV={errs[2]:.3e}", flush=True)
    assert max(errs) <= 2e-2


def test_hybrid_mask_full_size_sampled():
    """The timed hybrid workload at full size (B2 H32 L131072 d128, window 513 both
    ways, tokens 0 and -1 global): sampled rows of O, LSE and dQ against the oracle
    (each row depends on its own query only), the gradient identities on every head."""
    w = W.HYBRID_SPARSE_128K
    print(f"[masks] full size {w.name} seed={w.seed}", flush=True)
    q, k, v, do = W.make_inputs(w, with_dout=True)
    plan = fa().MaskPlan(w.L, causal=w.causal, window=w.window, global_tokens=w.global_tokens, device=DEV)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa().fwd_masked(qd, kd, vd, plan, scale=w.scale)
    dq, dk, dv = fa().bwd_masked(qd, kd, vd, o, lse, dod, plan, scale=w.scale)
    torch.cuda.synchronize()
    for x in (o, dq, dk, dv):
        assert torch.isfinite(x.float()).all()
    check_identities(dk, dv, dod, w.Hq, w.Hkv, w.name)
    L = w.L
    rows = np.array([0, 1, 63, 64, 700, L // 2, L - 513, L - 2, L - 1])
    gl = tuple(p + L if p < 0 else p for p in w.global_tokens)
    ok_rows = oracle.general_mask(rows, np.arange(L), w.causal, w.window, None, 64, gl)
    ri = torch.as_tensor(rows)
    for b, h in ((0, 0), (1, 21)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        O_ref, l_ref = oracle.forward_rows_with_mask(f64(q[sl]), f64(k[sl]), f64(v[sl]), rows, w.scale, ok_rows)
        err_o = float(np.abs(f64(o[sl].cpu()[:, :, ri]) - O_ref).max())
        err_l = float(np.abs(lse[sl].cpu()[:, :, ri].numpy() - l_ref).max())
        dq_ref = oracle.dq_rows_with_mask(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(do[sl]), rows, w.scale, ok_rows)
        err_dq = rel(dq[sl].cpu()[:, :, ri], dq_ref)
        print(f"[masks] {w.name} head ({b},{h}) rows {rows.tolist()}: max|dO|={err_o:.3e} "
              f"max|dLSE|={err_l:.3e} relL2 dQ={err_dq:.3e}", flush=True)
        assert err_o <= 2e-2 and err_l <= 1e-3 and err_dq <= 2e-2


def test_block_band_mask_full_size_sampled():
    """The timed block-sparse workload at full size (B2 H32 L131072 d128, blocks of 128,
    each query block with its own and both neighbouring key blocks): sampled rows of O,
    LSE and dQ against the oracle, the dK/dV identities on every head."""
    w = W.BLOCK_BAND_128K
    print(f"[masks] full size {w.name} seed={w.seed}", flush=True)
    q, k, v, do = W.make_inputs(w, with_dout=True)
    blk = W.BLOCK_BAND_BLOCK
    bm = W.block_band_mask(w.L, blk, W.BLOCK_BAND_RADIUS)
    plan = fa().MaskPlan(w.L, causal=w.causal, block_mask=bm, block=blk, device=DEV)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa().fwd_masked(qd, kd, vd, plan, scale=w.scale)
    dq, dk, dv = fa().bwd_masked(qd, kd, vd, o, lse, dod, plan, scale=w.scale)
    torch.cuda.synchronize()
    for x in (o, dq, dk, dv):
        assert torch.isfinite(x.float()).all()
    check_identities(dk, dv, dod, w.Hq, w.Hkv, w.name)
    L = w.L
    rows = np.array([0, 127, 128, 255, 4000, L // 2, L - 129, L - 128, L - 1])
    ok_rows = oracle.general_mask(rows, np.arange(L), w.causal, 0, bm.numpy(), blk, ())
    ri = torch.as_tensor(rows)
    for b, h in ((0, 3), (1, 30)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        O_ref, l_ref = oracle.forward_rows_with_mask(f64(q[sl]), f64(k[sl]), f64(v[sl]), rows, w.scale, ok_rows)
        err_o = float(np.abs(f64(o[sl].cpu()[:, :, ri]) - O_ref).max())
        err_l = float(np.abs(lse[sl].cpu()[:, :, ri].numpy() - l_ref).max())
        dq_ref = oracle.dq_rows_with_mask(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(do[sl]), rows, w.scale, ok_rows)
        err_dq = rel(dq[sl].cpu()[:, :, ri], dq_ref)
        print(f"[masks] {w.name} head ({b},{h}): max|dO|={err_o:.3e} max|dLSE|={err_l:.3e} relL2 dQ={err_dq:.3e}",
              flush=True)
        assert err_o <= 2e-2 and err_l <= 1e-3 and err_dq <= 2e-2
