"""Stored values printed by the sources, checked against the bench's accounting.

score_matrix_memory_fp16_B2_H32.txt: the full score matrix's size per layer, from the measured-output
table of claspmoon.cn "14 · 缩放定律与高效注意力" section 3.4; the bench reports the L = 4096 row as
context beside its result and counts the score matrix the tiled path avoids with the same rule.
"""
import os

import bench

HERE = os.path.dirname(os.path.abspath(__file__))


def _rows(name):
    out = []
    for line in open(os.path.join(HERE, "golden", name)):
        line = line.strip()
        if line and not line.startswith("#"):
            a, b = line.split()
            out.append((int(a), float(b)))
    return out


def test_score_matrix_memory_table():
    rows = _rows("score_matrix_memory_fp16_B2_H32.txt")
    assert [L for L, _ in rows] == [2048, 4096, 8192, 32768, 131072]
    for L, gb in rows[:-1]:
        assert round(bench.score_matrix_bytes(2, 32, L) / 1e9, 2) == gb, L
    # the page prints its last row at half of what its own code computes (garbled row)
    L, gb = rows[-1]
    assert round(bench.score_matrix_bytes(2, 32, L) / 2 / 1e9, 2) == gb


def test_context_figure_matches_table():
    gb = dict(_rows("score_matrix_memory_fp16_B2_H32.txt"))[4096]
    assert bench.PAGES_CONTEXT["score_matrix_gb_per_layer_fp16_B2_H32_L4096"] == gb
