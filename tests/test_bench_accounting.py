"""The bench's host-side work accounting, checked against brute-force counts.

bench.py reports TFLOP/s as 4*d flops per allowed (query, key) pair forward
(claspmoon.cn "14 · 缩放定律与高效注意力" §2.1: the score matrix has one entry
per pair; mdooai.com "Ch.04": a masked entry carries no weight).  These tests
count the allowed pairs by brute force over the oracle's boolean mask.
"""

import numpy as np

import bench
import oracle
import workloads as W


def brute_pairs(L, causal, window, block_mask=None, block=64, glob=()):
    ok = oracle.general_mask(np.arange(L), np.arange(L), causal, window, block_mask, block, glob)
    return int(ok.sum())


def test_window_pairs_one_and_two_sided():
    for L in (1, 5, 64, 300):
        for w in (1, 2, 7, 64, 299, 300, 1000):
            for causal in (True, False):
                assert bench.window_pairs(L, w, causal) == brute_pairs(L, causal, w), (L, w, causal)


def test_fwd_flops_counts_allowed_pairs():
    """Windows and the full matrix count their allowed pairs exactly; plain causal
    masks follow the stated convention of half the full matrix (L^2 / 2 pairs
    instead of L (L + 1) / 2)."""
    d, B, H = 64, 2, 3
    for L, causal, window in ((300, False, 0), (300, True, 0), (300, True, 17), (300, False, 17), (257, False, 400)):
        pairs = L * L / 2 if causal and not window else brute_pairs(L, causal, window)
        assert bench.fwd_flops(B, H, L, d, causal, window) == 4.0 * d * pairs * B * H, (L, causal, window)
        assert bench.bwd_flops(B, H, L, d, causal, window) == 2.5 * 4.0 * d * pairs * B * H


def test_allowed_pairs_counts_the_oracle_mask():
    """The host pair count of the general masks against the oracle's mask."""
    bmask = W.block_band_mask(300, 64, 1).numpy()
    assert bmask.shape == (5, 5) and bmask[0, 1] and not bmask[0, 2]
    for L, causal, window, glob, bm, blk in [(300, False, 0, (), None, 64), (300, True, 0, (), None, 64),
                                           (300, False, 7, (0, -1), None, 64), (300, True, 20, (5, 299), bmask, 64),
                                           (257, False, 0, (3,), W.block_band_mask(257, 128, 0).numpy(), 128),
                                           (300, True, 9, (0, 150, -1), None, 64), (257, False, 0, (5, 5, -3), None, 64),
                                           (200, False, 300, (7,), None, 64), (64, True, 1, tuple(range(0, 64, 5)), None, 64)]:
        gl = tuple(p + L if p < 0 else p for p in glob)
        assert bench.allowed_pairs(L, causal, window, glob, bm, blk) == brute_pairs(L, causal, window, bm, blk, gl)


def test_decode_cache_reads_counts_work_groups():
    """The decode reads each K/V head once per work-group, and a work-group serves up to
    four groups of 32 rows (query heads per K/V head x new tokens): 1 row group -> one
    1-wave work-group, 2 -> one 2-wave work-group, more -> 4-wave work-groups."""
    cases = [  # (Hq, Hkv, Lq) -> reads
        ((32, 8, 1), 1),      # 4 rows
        ((32, 8, 8), 1),      # 32 rows: one group
        ((32, 8, 16), 1),     # 64 rows: two groups, one 2-wave work-group
        ((32, 8, 32), 1),     # 128 rows: four groups
        ((32, 8, 40), 2),     # 160 rows: five groups, two 4-wave work-groups
        ((40, 2, 4), 1),      # 80 rows: three groups
        ((8, 1, 100), 7),     # 800 rows: 25 groups
    ]
    for (hq, hkv, lq), reads in cases:
        assert bench.decode_cache_reads(hq, hkv, lq) == reads, (hq, hkv, lq)
