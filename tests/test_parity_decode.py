"""GPU parity of the KV-cache decode path against the fp64 oracle, through the C ABI.

The Lq newest tokens of each sequence attend to its first cache_len[b] cache
entries, the new tokens sitting at the end (bottom-right alignment;
book.anysome.cn "高效注意力" §1 KV cache, §3 GQA).  Tolerances: O max-abs 2e-2,
LSE max-abs 1e-3.  Also checked: a decode of the last token equals the last
row of the whole-sequence forward, and a single token over a rolling window
buffer in ring-slot order equals the windowed forward's row.  The rolling-
buffer call (flash_attn_decode_rolling: W slots, position p in slot p mod W,
the new tokens' own K/V passed separately) is checked against the oracle's
rolling_decode_forward before and after the buffer wraps, with more rows per
K/V head than one group of 32, and with more new tokens than slots.
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


def f64(t):
    return t.detach().double().cpu().numpy()


def draw(shape, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(dtype)


# (B, Hq, Hkv, Lq, Lk, d, causal, window, cache_len or None, dtype)
CASES = [
    (2, 32, 8, 1, 4096, 128, True, 0, [4096, 1500], torch.bfloat16),      # GQA-4 single token, ragged batch
    (1, 8, 1, 4, 1000, 64, True, 100, [1000], torch.float16),            # MQA, 4 new tokens, window
    (3, 4, 4, 2, 777, 128, False, 0, [777, 5, 300], torch.bfloat16),     # MHA, non-causal, tiny sequence
    (2, 16, 2, 2, 2048, 128, True, 0, None, torch.bfloat16),            # 32 rows per K/V head, no lengths
    (1, 4, 4, 8, 8, 128, True, 0, [8], torch.bfloat16),                  # cache = the new tokens only
    (1, 32, 8, 1, 131072, 128, True, 0, [131072], torch.bfloat16),       # a 128k cache
    (1, 32, 8, 1, 32768, 128, True, 4096, [30000], torch.bfloat16),      # sliding window over a long cache
    (1, 4, 1, 1, 70000, 128, True, 0, [70000], torch.bfloat16),          # one K/V head, ~220 key splits merged
    (1, 2, 1, 3, 50000, 64, False, 0, [49999], torch.float16),           # many splits, non-causal, ragged tile
    (1, 32, 8, 20, 5000, 128, True, 0, [4321], torch.bfloat16),          # 80 rows per K/V head: 3 row groups
    (2, 4, 2, 40, 300, 64, True, 17, [300, 123], torch.float16),         # 80 rows, window, ragged batch
    (1, 16, 2, 20, 3000, 64, True, 0, [2999], torch.bfloat16),           # 160 rows: 5 groups, 2 work-groups
    (2, 8, 4, 32, 1500, 64, False, 0, [1500, 900], torch.float16),       # 64 rows (2 groups), non-causal
]


@pytest.mark.parametrize("case", CASES, ids=[f"decode{i}" for i in range(len(CASES))])
def test_decode_matches_oracle(case):
    B, Hq, Hkv, Lq, Lk, d, causal, window, lens, dt = case
    print(f"[decode] case {case[:8]} lens={lens}", flush=True)
    seed = 700 + Lk + Lq
    q, k, v = draw((B, Hq, Lq, d), seed, dt), draw((B, Hkv, Lk, d), seed + 1, dt), draw((B, Hkv, Lk, d), seed + 2, dt)
    s = 1.0 / math.sqrt(d)
    cl = torch.tensor(lens, dtype=torch.int32, device=DEV) if lens is not None else None
    o, lse = fa().decode(q.to(DEV), k.to(DEV), v.to(DEV), cl, causal=causal, window=window, scale=s)
    torch.cuda.synchronize()
    O_ref, l_ref = oracle.decode_forward(f64(q), f64(k), f64(v), lens if lens is not None else [Lk] * B, s,
                                         causal, window)
    err_o = float(np.abs(f64(o) - O_ref).max())
    err_l = float(np.abs(lse.cpu().numpy() - l_ref).max())
    print(f"[decode] {case[:8]}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= 2e-2 and err_l <= 1e-3


def test_decode_of_last_token_matches_whole_sequence_forward():
    B, Hq, Hkv, L, d = 1, 8, 2, 1500, 128
    q, k, v = (draw(sh, 720 + i, torch.bfloat16).to(DEV) for i, sh in
               enumerate(((B, Hq, L, d), (B, Hkv, L, d), (B, Hkv, L, d))))
    o_full, l_full = fa().fwd(q, k, v, causal=True)
    o, lse = fa().decode(q[:, :, L - 1:].contiguous(), k, v, None, causal=True)
    torch.cuda.synchronize()
    assert float((o.float() - o_full[:, :, L - 1:].float()).abs().max()) <= 2e-2
    assert float((lse - l_full[:, :, L - 1:]).abs().max()) <= 1e-3


def test_rolling_window_buffer():
    # positions p of the last W tokens live in slot p mod W; one new token, no mask
    L, W, d = 3000, 1024, 128
    q, k, v = (draw(sh, 730 + i, torch.bfloat16) for i, sh in
               enumerate(((1, 4, L, d), (1, 2, L, d), (1, 2, L, d))))
    pos = torch.arange(L - W, L)
    kb, vb = torch.empty(1, 2, W, d, dtype=torch.bfloat16), torch.empty(1, 2, W, d, dtype=torch.bfloat16)
    kb[:, :, pos % W], vb[:, :, pos % W] = k[:, :, pos], v[:, :, pos]
    cl = torch.tensor([W], dtype=torch.int32, device=DEV)
    o, lse = fa().decode(q[:, :, L - 1:].contiguous().to(DEV), kb.to(DEV), vb.to(DEV), cl, causal=False)
    torch.cuda.synchronize()
    O_ref, l_ref = oracle.forward_rows(f64(q), f64(k), f64(v), np.array([L - 1]), 1.0 / math.sqrt(d), True, W)
    assert float(np.abs(f64(o) - O_ref).max()) <= 2e-2
    assert float(np.abs(lse.cpu().numpy() - l_ref).max()) <= 1e-3


def ring_of(k, v, n, W):
    """The buffer after tokens 0 .. n-1 were written one by one, position p into slot p mod W
    (slots never written hold junk, which the call must not read as keys)."""
    B, H, _, d = k.shape
    kb = torch.full((B, H, W, d), 30.0, dtype=k.dtype)
    vb = torch.full((B, H, W, d), -30.0, dtype=v.dtype)
    for p in range(n):
        kb[:, :, p % W], vb[:, :, p % W] = k[:, :, p], v[:, :, p]
    return kb, vb


# (B, Hq, Hkv, Lq, W, d, seen per sequence, window, dtype)
ROLLING = [
    (2, 8, 2, 4, 1024, 128, [3000, 700], 0, torch.bfloat16),      # wrapped and not yet full
    (1, 32, 8, 16, 512, 64, [512 * 3 + 17], 200, torch.float16),  # 64 rows per K/V head, window < W
    (1, 2, 1, 100, 64, 128, [100], 0, torch.bfloat16),            # more new tokens than slots
    (1, 4, 4, 5, 256, 128, [0], 0, torch.bfloat16),               # empty buffer: the new tokens only
    (3, 4, 1, 1, 300, 64, [299, 300, 301], 0, torch.bfloat16),    # one token at the fill boundary
    (1, 4, 2, 3, 1, 128, [7], 0, torch.bfloat16),                 # one slot: every token sees only itself
    (2, 2, 2, 5, 3, 64, [2, 10], 2, torch.float16),               # tiny buffer, window < W, Lq > W
]


@pytest.mark.parametrize("case", ROLLING, ids=[f"rolling{i}" for i in range(len(ROLLING))])
def test_rolling_buffer_decode_matches_oracle(case):
    B, Hq, Hkv, Lq, W, d, seen, window, dt = case
    print(f"[decode] rolling case {case}", flush=True)
    seed = 760 + W + Lq
    per_seq = [(draw((1, Hkv, n + Lq, d), seed + 10 * b, dt), draw((1, Hkv, n + Lq, d), seed + 10 * b + 1, dt))
               for b, n in enumerate(seen)]
    rings = [ring_of(k, v, n, W) for (k, v), n in zip(per_seq, seen)]
    kb = torch.cat([r[0] for r in rings])
    vb = torch.cat([r[1] for r in rings])
    kn = torch.cat([k[:, :, n:] for (k, _), n in zip(per_seq, seen)])
    vn = torch.cat([v[:, :, n:] for (_, v), n in zip(per_seq, seen)])
    q = draw((B, Hq, Lq, d), seed + 5, dt)
    s = 1.0 / math.sqrt(d)
    sd = torch.tensor(seen, dtype=torch.int32, device=DEV)
    o, lse = fa().decode_rolling(q.to(DEV), kb.to(DEV), vb.to(DEV), kn.to(DEV), vn.to(DEV), sd, window=window, scale=s)
    torch.cuda.synchronize()
    O_ref, l_ref = oracle.rolling_decode_forward(f64(q), f64(kb), f64(vb), f64(kn), f64(vn), seen, s, window)
    err_o = float(np.abs(f64(o) - O_ref).max())
    err_l = float(np.abs(lse.cpu().numpy() - l_ref).max())
    print(f"[decode] rolling {case[:7]}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= 2e-2 and err_l <= 1e-3


def test_rolling_buffer_decode_equals_whole_sequence_rows():
    # the rolling call gives the rows of the windowed causal forward over the whole sequence
    Hq, Hkv, W, d, n, Lq = 8, 2, 256, 128, 1000, 6
    q, k, v = (draw(sh, 790 + i, torch.bfloat16) for i, sh in
               enumerate(((1, Hq, n + Lq, d), (1, Hkv, n + Lq, d), (1, Hkv, n + Lq, d))))
    kb, vb = ring_of(k, v, n, W)
    sd = torch.tensor([n], dtype=torch.int32, device=DEV)
    o, lse = fa().decode_rolling(q[:, :, n:].contiguous().to(DEV), kb.to(DEV), vb.to(DEV),
                                 k[:, :, n:].contiguous().to(DEV), v[:, :, n:].contiguous().to(DEV), sd)
    o_full, l_full = fa().fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=True, window=W)
    torch.cuda.synchronize()
    assert float((o.float() - o_full[:, :, n:].float()).abs().max()) <= 2e-2
    assert float((lse - l_full[:, :, n:]).abs().max()) <= 1e-3
