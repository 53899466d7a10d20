"""The Python binding rejects bad tensors and out-of-range integers before any
library call (CPU only).

The C ABI sees device pointers and sizes but not the buffers behind them, so a
mis-shaped, mistyped, strided or host-side tensor must never reach it.  Every
case here runs with the library loader replaced by one that fails the test if
it is reached.
"""

import pytest
import torch

import exact_tiled_attention_flash_amd as fa


@pytest.fixture
def no_library(monkeypatch):
    def forbidden():
        raise AssertionError("the library was reached")
    monkeypatch.setattr(fa, "library", forbidden)


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


def test_expect_checks_shape_dtype_layout_and_device():
    cpu = torch.device("cpu")
    x = t(2, 3)
    with pytest.raises(ValueError, match="shape"):
        fa._expect(x, "x", (3, 2), torch.bfloat16, cpu)
    with pytest.raises(ValueError, match="float32"):
        fa._expect(x, "x", (2, 3), torch.float32, cpu)
    with pytest.raises(ValueError, match="must be on"):
        fa._expect(x, "x", (2, 3), torch.bfloat16, torch.device("cuda:0"))
    with pytest.raises(ValueError, match="must be a tensor"):
        fa._expect([1, 2], "x", (2,), torch.bfloat16, cpu)


def test_workspace_checks():
    dev = torch.device("cuda:0")
    with pytest.raises(ValueError, match="uint8"):
        fa._workspace(t(256, dtype=torch.float32), 256, dev)
    with pytest.raises(ValueError, match="contiguous tensor on"):
        fa._workspace(t(256, dtype=torch.uint8), 256, dev)
    with pytest.raises(ValueError, match="1-D"):
        fa._workspace(t(16, 16, dtype=torch.uint8), 256, dev)


def test_window_and_offsets():
    assert fa._window(0) == 0 and fa._window(4096) == 4096 and fa._window(2**30 - 1) == 2**30 - 1
    # every window of 2^30 or more admits all pairs: passed as "none", never truncated
    assert fa._window(2**30) == 0 and fa._window(2**32 + 5) == 0 and fa._window(2**63) == 0
    with pytest.raises(ValueError):
        fa._window(-1)
    assert fa._offset(0, "q") == 0 and fa._offset(2**29, "q") == 2**29
    for bad in (-1, 2**29 + 1, 2**32, 2**32 + 7):
        with pytest.raises(ValueError):
            fa._offset(bad, "q_offset")


def test_scale_checks():
    assert fa._scale(None, 64) == 0.125
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            fa._scale(bad, 64)


def test_entry_points_reject_host_tensors(no_library):
    q, k, v = t(1, 2, 8, 64), t(1, 1, 8, 64), t(1, 1, 8, 64)
    lse = t(1, 2, 8, dtype=torch.float32)
    with pytest.raises(ValueError):
        fa.fwd(q, k, v)
    with pytest.raises(ValueError):
        fa.bwd(q, k, v, q, lse, q)
    with pytest.raises(ValueError):
        fa.bwd_stages(q, k, v, q, lse, q)
    with pytest.raises(ValueError):
        fa.fwd_block(q, k, v)
    with pytest.raises(ValueError):
        fa.bwd_block(q, k, v, q, lse, q)
    with pytest.raises(ValueError):
        fa.merge(q, lse, q, lse)
    with pytest.raises(ValueError):
        fa.decode(q, k, v)


def test_mismatched_inputs_rejected(no_library):
    q = t(1, 2, 8, 64)
    with pytest.raises(ValueError):
        fa.fwd(q, t(1, 1, 9, 64), t(1, 1, 9, 64))          # key length differs
    with pytest.raises(ValueError):
        fa.fwd(q, t(1, 1, 8, 64), t(1, 1, 8, 32))          # k and v differ
    with pytest.raises(ValueError):
        fa.fwd(q, t(1, 1, 8, 64, dtype=torch.float16), t(1, 1, 8, 64))   # dtypes differ
    with pytest.raises(ValueError):
        fa.fwd(q.transpose(2, 3), t(1, 1, 64, 8), t(1, 1, 64, 8))       # not contiguous
    with pytest.raises(ValueError):
        fa.merge(q, t(1, 2, 7, dtype=torch.float32), q, t(1, 2, 8, dtype=torch.float32))
