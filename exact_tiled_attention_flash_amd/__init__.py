"""Exact tiled attention for AMD MI355X (gfx950): thin Python binding.

The work is done entirely by the HIP kernels in ``libflashattn.so`` behind the
C ABI declared in ``include/flash_attn.h``; this module only marshals torch
tensors into device pointers, sizes and the current HIP stream.  There is no
fallback: if the library is missing or a call fails, a RuntimeError is raised.

    o, lse = fwd(q, k, v, causal=True)                 # q [B,Hq,L,d], k/v [B,Hkv,L,d]
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=True)
    o = scaled_dot_product_attention(q, k, v, is_causal=True)   # autograd drop-in

The interface mirrors the pages' ``scaled_dot_product_attention(q, k, v,
is_causal=...)`` usage (claspmoon.cn "14 · 缩放定律与高效注意力" §3.5) plus the
grouped-query and sliding-window options (kler.cn, §3.2.1 configuration keys).
"""

import ctypes
import math
import os

import torch

__all__ = ["fwd", "bwd", "bwd_stages", "bwd_workspace_bytes", "bwd_fused", "bwd_fused_workspace_bytes",
           "bwd_noalloc", "NOALLOC_MAX_ROWS", "fwd_block", "bwd_block", "merge",
           "decode", "decode_workspace_bytes", "decode_rolling", "decode_rolling_workspace_bytes",
           "MaskPlan", "fwd_masked", "bwd_masked", "masked_workspace_bytes",
           "strerror", "library", "library_path",
           "FlashAttentionFunction", "scaled_dot_product_attention",
           "FA_DTYPE_F32", "FA_DTYPE_BF16", "FA_DTYPE_F16", "EXPORTED_SYMBOLS"]

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_F16 = 2
_DTYPES = {torch.float32: FA_DTYPE_F32, torch.bfloat16: FA_DTYPE_BF16, torch.float16: FA_DTYPE_F16}

EXPORTED_SYMBOLS = ("flash_attn_fwd", "flash_attn_bwd", "flash_attn_bwd_workspace_bytes",
                    "flash_attn_bwd_fused", "flash_attn_bwd_fused_workspace_bytes",
                    "flash_attn_bwd_preprocess", "flash_attn_bwd_dkdv", "flash_attn_bwd_dq",
                    "flash_attn_fwd_block", "flash_attn_merge", "flash_attn_bwd_block",
                    "flash_attn_decode", "flash_attn_decode_workspace_bytes",
                    "flash_attn_decode_rolling", "flash_attn_decode_rolling_workspace_bytes",
                    "flash_attn_mask_plan_bytes", "flash_attn_mask_plan", "flash_attn_masked_workspace_bytes",
                    "flash_attn_fwd_masked", "flash_attn_bwd_masked",
                    "flash_attn_bwd_noalloc", "flash_attn_strerror", "flash_attn_version")

# B * Hq * L limit of flash_attn_bwd_noalloc (its static scratch holds two float32 per row)
NOALLOC_MAX_ROWS = 1 << 21

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class FaMask(ctypes.Structure):
    """``fa_mask`` of ``include/flash_attn.h``."""
    _fields_ = [("causal", ctypes.c_int), ("window", ctypes.c_int), ("global_pos", ctypes.c_void_p),
                ("n_global", ctypes.c_int), ("block_mask", ctypes.c_void_p), ("block", ctypes.c_int)]


def library_path():
    return os.path.join(_HERE, "libflashattn.so")


def library():
    """Load ``libflashattn.so`` (once).  Raises RuntimeError if it is not built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            "libflashattn.so is not built (expected at %s); run "
            "`python -m exact_tiled_attention_flash_amd.build`" % path)
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.flash_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp]
    lib.flash_attn_fwd.restype = i
    lib.flash_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                   i, i, i, i, i, f, i, i, i, vp]
    lib.flash_attn_bwd.restype = i
    lib.flash_attn_bwd_fused.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                         i, i, i, i, i, f, i, i, i, vp]
    lib.flash_attn_bwd_fused.restype = i
    lib.flash_attn_bwd_fused_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.flash_attn_bwd_fused_workspace_bytes.restype = sz
    lib.flash_attn_bwd_preprocess.argtypes = [vp, vp, vp, vp, sz, i, i, i, i, i, i, vp]
    lib.flash_attn_bwd_preprocess.restype = i
    lib.flash_attn_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, sz, vp, vp, i, i, i, i, i, f, i, i, i, vp]
    lib.flash_attn_bwd_dkdv.restype = i
    lib.flash_attn_bwd_dq.argtypes = [vp, vp, vp, vp, vp, sz, vp, i, i, i, i, i, f, i, i, i, vp]
    lib.flash_attn_bwd_dq.restype = i
    lib.flash_attn_fwd_block.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, i, i, vp]
    lib.flash_attn_fwd_block.restype = i
    lib.flash_attn_merge.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.flash_attn_merge.restype = i
    lib.flash_attn_bwd_block.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                         i, i, i, i, i, i, f, i, i, i, i, i, vp]
    lib.flash_attn_bwd_block.restype = i
    lib.flash_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, i, i, i, vp]
    lib.flash_attn_decode.restype = i
    lib.flash_attn_decode_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.flash_attn_decode_workspace_bytes.restype = sz
    lib.flash_attn_decode_rolling.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, i, i, vp]
    lib.flash_attn_decode_rolling.restype = i
    lib.flash_attn_decode_rolling_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.flash_attn_decode_rolling_workspace_bytes.restype = sz
    lib.flash_attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.flash_attn_bwd_workspace_bytes.restype = sz
    mp = ctypes.POINTER(FaMask)
    lib.flash_attn_mask_plan_bytes.argtypes = [i]
    lib.flash_attn_mask_plan_bytes.restype = sz
    lib.flash_attn_mask_plan.argtypes = [mp, i, vp, sz, vp]
    lib.flash_attn_mask_plan.restype = i
    lib.flash_attn_masked_workspace_bytes.argtypes = [i, i, i, i, i, mp, i]
    lib.flash_attn_masked_workspace_bytes.restype = sz
    lib.flash_attn_fwd_masked.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, mp, vp, sz, i, vp]
    lib.flash_attn_fwd_masked.restype = i
    lib.flash_attn_bwd_masked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                          i, i, i, i, i, f, mp, vp, sz, i, vp]
    lib.flash_attn_bwd_masked.restype = i
    lib.flash_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp]
    lib.flash_attn_bwd_noalloc.restype = i
    lib.flash_attn_strerror.argtypes = [i]
    lib.flash_attn_strerror.restype = ctypes.c_char_p
    lib.flash_attn_version.argtypes = []
    lib.flash_attn_version.restype = i
    _LIB = lib
    return lib


def strerror(code):
    return library().flash_attn_strerror(int(code)).decode()


def _check(rc, what):
    if rc != 0:
        raise RuntimeError("%s failed: %s (code %d)" % (what, strerror(rc), rc))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _expect(t, name, shape, dtype, device):
    """Check a caller-supplied tensor before its pointer crosses the C ABI, which
    cannot see sizes: a wrong shape, dtype, device or layout raises ValueError."""
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda or t.device != device:
        raise ValueError("%s must be on %s" % (name, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _workspace(ws, nbytes, device, name="workspace"):
    """A caller's workspace: a contiguous uint8 tensor on the device holding at least nbytes."""
    if ws is None:
        return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.dim() != 1:
        raise ValueError("%s must be a 1-D uint8 tensor" % name)
    if not ws.is_cuda or ws.device != device or not ws.is_contiguous():
        raise ValueError("%s must be a contiguous tensor on %s" % (name, device))
    if ws.numel() < nbytes:
        raise ValueError("%s holds %d bytes, %d needed" % (name, ws.numel(), nbytes))
    return ws


_INT_MAX = 2**31 - 1
_MAX_OFFSET = 2**29


def _window(window):
    """The window as the C int the boundary takes (0 = none).  Windows of 2^30 and
    more admit every pair of positions the boundary accepts, so they are passed as 0."""
    w = int(window)
    if w < 0:
        raise ValueError("window must be >= 0, got %d" % w)
    return 0 if w >= 2**30 else w


def _offset(x, name):
    x = int(x)
    if not 0 <= x <= _MAX_OFFSET:
        raise ValueError("%s must be in [0, 2^29], got %d" % (name, x))
    return x


def _shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, Hq, L, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != L or k.shape[3] != d:
        raise ValueError("k and v must be [B, Hkv, L, d] matching q")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must be contiguous tensors of one dtype on one GPU")
    if q.dtype not in _DTYPES:
        raise ValueError("dtype must be float32, bfloat16 or float16")
    return B, Hq, k.shape[1], L, d


def _out(t, name, shape, dtype, device):
    """An output buffer: allocated when not given, else checked."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return _expect(t, name, shape, dtype, device)


def _scale(scale, d):
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if not (scale > 0.0 and math.isfinite(scale)):
        raise ValueError("scale must be positive and finite")
    return scale


def fwd(q, k, v, causal=False, window=0, scale=None, out=None, lse=None):
    """Exact attention forward.  Returns ``(o, lse)``; ``lse`` is float32 ``[B,Hq,L]``.

    ``window`` (>= 1) limits query i to keys i-window+1..i with ``causal`` and to
    keys j with |i - j| < window without it (a window reaching both ways).
    ``scale`` defaults to 1/sqrt(d).
    """
    B, Hq, Hkv, L, d = _shapes(q, k, v)
    scale, window = _scale(scale, d), _window(window)
    out = _out(out, "out", q.shape, q.dtype, q.device)
    lse = _out(lse, "lse", (B, Hq, L), torch.float32, q.device)
    rc = library().flash_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                  B, Hq, Hkv, L, d, scale, int(bool(causal)), window,
                                  _DTYPES[q.dtype], _stream(q))
    _check(rc, "flash_attn_fwd")
    return out, lse


def bwd_workspace_bytes(B, Hq, Hkv, L, d, dtype=torch.bfloat16):
    return int(library().flash_attn_bwd_workspace_bytes(B, Hq, Hkv, L, d, _DTYPES[dtype]))


def _bwd_buffers(q, k, v, o, lse, dout, Lq, workspace, dq, dk, dv):
    """Checks the backward's tensors (Lq query rows) and allocates the missing outputs."""
    B, Hq = q.shape[0], q.shape[1]
    _expect(o, "o", q.shape, q.dtype, q.device)
    _expect(dout, "dout", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (B, Hq, Lq), torch.float32, q.device)
    nbytes = bwd_workspace_bytes(B, Hq, k.shape[1], Lq, q.shape[3], q.dtype)
    if nbytes == 0:
        raise RuntimeError("flash_attn_bwd: unsupported sizes")
    workspace = _workspace(workspace, nbytes, q.device)
    dq = _out(dq, "dq", q.shape, q.dtype, q.device)
    dk = _out(dk, "dk", k.shape, k.dtype, k.device)
    dv = _out(dv, "dv", v.shape, v.dtype, v.device)
    return workspace, dq, dk, dv


def bwd(q, k, v, o, lse, dout, causal=False, window=0, scale=None, workspace=None,
        dq=None, dk=None, dv=None):
    """Gradient of sum(o * dout) w.r.t. q, k, v, recomputing P from ``lse``.

    Returns ``(dq, dk, dv)`` in the input dtype.  ``workspace`` (optional) is a
    device uint8 tensor of at least ``bwd_workspace_bytes(...)`` bytes.
    """
    B, Hq, Hkv, L, d = _shapes(q, k, v)
    scale, window = _scale(scale, d), _window(window)
    workspace, dq, dk, dv = _bwd_buffers(q, k, v, o, lse, dout, L, workspace, dq, dk, dv)
    rc = library().flash_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                  _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                                  B, Hq, Hkv, L, d, scale, int(bool(causal)), window,
                                  _DTYPES[q.dtype], _stream(q))
    _check(rc, "flash_attn_bwd")
    return dq, dk, dv


def bwd_fused_workspace_bytes(B, Hq, Hkv, L, d, dtype=torch.bfloat16):
    return int(library().flash_attn_bwd_fused_workspace_bytes(B, Hq, Hkv, L, d, _DTYPES[dtype]))


def bwd_fused(q, k, v, o, lse, dout, causal=False, window=0, scale=None, workspace=None,
              dq=None, dk=None, dv=None):
    """``bwd`` by the single K/V-stationary kernel that accumulates dQ with float32
    atomics (``flash_attn_bwd_fused``): dK and dV bit for bit as ``bwd``, dQ to
    float32 rounding.  ``workspace`` needs ``bwd_fused_workspace_bytes(...)`` bytes."""
    B, Hq, Hkv, L, d = _shapes(q, k, v)
    scale, window = _scale(scale, d), _window(window)
    nbytes = bwd_fused_workspace_bytes(B, Hq, Hkv, L, d, q.dtype)
    if nbytes == 0:
        raise RuntimeError("flash_attn_bwd_fused: unsupported sizes")
    _expect(o, "o", q.shape, q.dtype, q.device)
    _expect(dout, "dout", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (B, Hq, L), torch.float32, q.device)
    workspace = _workspace(workspace, nbytes, q.device)
    dq = _out(dq, "dq", q.shape, q.dtype, q.device)
    dk = _out(dk, "dk", k.shape, k.dtype, k.device)
    dv = _out(dv, "dv", v.shape, v.dtype, v.device)
    rc = library().flash_attn_bwd_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(),
                                        B, Hq, Hkv, L, d, scale, int(bool(causal)), window,
                                        _DTYPES[q.dtype], _stream(q))
    _check(rc, "flash_attn_bwd_fused")
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, causal=False, window=0, scale=None):
    """``bwd`` for callers that cannot allocate: the outputs ``dq, dk, dv`` are given, and
    the library keeps the per-row statistics in its own static device array (at most
    ``NOALLOC_MAX_ROWS`` query rows, B * Hq * L).  Calls that overlap in time on one GPU
    share that array and race.  Nothing is allocated on this path."""
    B, Hq, Hkv, L, d = _shapes(q, k, v)
    scale, window = _scale(scale, d), _window(window)
    _expect(o, "o", q.shape, q.dtype, q.device)
    _expect(dout, "dout", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (B, Hq, L), torch.float32, q.device)
    _expect(dq, "dq", q.shape, q.dtype, q.device)
    _expect(dk, "dk", k.shape, k.dtype, k.device)
    _expect(dv, "dv", v.shape, v.dtype, v.device)
    rc = library().flash_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                          _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, L, d, scale,
                                          int(bool(causal)), window, _DTYPES[q.dtype], _stream(q))
    _check(rc, "flash_attn_bwd_noalloc")
    return dq, dk, dv


def bwd_stages(q, k, v, o, lse, dout, causal=False, window=0, scale=None, workspace=None,
               dq=None, dk=None, dv=None, between=None):
    """The backward as its three exported stages (preprocess, dK/dV, dQ) on the
    current stream; same results as ``bwd``.  ``between(stage_name)`` is called
    after each launch (for example to record timing events)."""
    B, Hq, Hkv, L, d = _shapes(q, k, v)
    scale, window = _scale(scale, d), _window(window)
    workspace, dq, dk, dv = _bwd_buffers(q, k, v, o, lse, dout, L, workspace, dq, dk, dv)
    lib, dt, st, c = library(), _DTYPES[q.dtype], _stream(q), int(bool(causal))
    _check(lib.flash_attn_bwd_preprocess(_ptr(o), _ptr(lse), _ptr(dout), _ptr(workspace), workspace.numel(),
                                         B, Hq, Hkv, L, d, dt, st), "flash_attn_bwd_preprocess")
    if between:
        between("preprocess")
    _check(lib.flash_attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(workspace), workspace.numel(),
                                   _ptr(dk), _ptr(dv), B, Hq, Hkv, L, d, scale, c, window, dt, st),
           "flash_attn_bwd_dkdv")
    if between:
        between("dkdv")
    _check(lib.flash_attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(workspace), workspace.numel(),
                                 _ptr(dq), B, Hq, Hkv, L, d, scale, c, window, dt, st),
           "flash_attn_bwd_dq")
    if between:
        between("dq")
    return dq, dk, dv


def _chunk_shapes(q, k, v):
    """Shapes of a (query chunk, key/value chunk) pair: q [B,Hq,Lq,d], k/v [B,Hkv,Lk,d]."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, Hq, Lq, d] and k, v [B, Hkv, Lk, d]")
    B, Hq, Lq, d = q.shape
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k and v must share B and d with q")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must be contiguous tensors of one dtype on one GPU")
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("chunk pairs take bfloat16 or float16")
    return B, Hq, k.shape[1], Lq, k.shape[2], d


def fwd_block(q, k, v, causal=False, window=0, q_offset=0, k_offset=0, scale=None, out=None, lse=None):
    """One ring-attention step: the queries at positions ``q_offset + i`` attend to the keys at
    ``k_offset + j`` only.  Returns the partial ``(o, lse)`` over this key chunk (rows with no
    allowed key: o = 0, lse = -inf); combine partials with ``merge``."""
    B, Hq, Hkv, Lq, Lk, d = _chunk_shapes(q, k, v)
    scale, window = _scale(scale, d), _window(window)
    q_offset, k_offset = _offset(q_offset, "q_offset"), _offset(k_offset, "k_offset")
    out = _out(out, "out", q.shape, q.dtype, q.device)
    lse = _out(lse, "lse", (B, Hq, Lq), torch.float32, q.device)
    rc = library().flash_attn_fwd_block(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Lq, Lk, d,
                                        scale, int(bool(causal)), window, q_offset, k_offset,
                                        _DTYPES[q.dtype], _stream(q))
    _check(rc, "flash_attn_fwd_block")
    return out, lse


def merge(o_a, lse_a, o_b, lse_b, out=None, lse_out=None):
    """Exact combination of two partial results over disjoint key sets.  ``out``/``lse_out``
    may be ``o_a``/``lse_a`` (in-place accumulation)."""
    if o_a.shape != o_b.shape or o_a.dtype != o_b.dtype or o_a.dim() != 4:
        raise ValueError("partials must be [B, Hq, L, d] of one dtype")
    if o_a.dtype not in _DTYPES:
        raise ValueError("dtype must be float32, bfloat16 or float16")
    B, Hq, L, d = o_a.shape
    dev = o_a.device
    _expect(o_a, "o_a", o_a.shape, o_a.dtype, dev)
    _expect(o_b, "o_b", o_a.shape, o_a.dtype, dev)
    _expect(lse_a, "lse_a", (B, Hq, L), torch.float32, dev)
    _expect(lse_b, "lse_b", (B, Hq, L), torch.float32, dev)
    out = _out(out, "out", o_a.shape, o_a.dtype, dev)
    lse_out = _out(lse_out, "lse_out", (B, Hq, L), torch.float32, dev)
    rc = library().flash_attn_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(out), _ptr(lse_out),
                                    B, Hq, L, d, _DTYPES[o_a.dtype], _stream(o_a))
    _check(rc, "flash_attn_merge")
    return out, lse_out


def bwd_block(q, k, v, o, lse, dout, causal=False, window=0, q_offset=0, k_offset=0, scale=None,
              workspace=None, dq=None, dk=None, dv=None):
    """One ring-attention backward step: this chunk pair's contributions ``(dq, dk, dv)`` to the
    gradient, given the query rows' full ``o`` and ``lse`` (over all key chunks)."""
    B, Hq, Hkv, Lq, Lk, d = _chunk_shapes(q, k, v)
    scale, window = _scale(scale, d), _window(window)
    q_offset, k_offset = _offset(q_offset, "q_offset"), _offset(k_offset, "k_offset")
    workspace, dq, dk, dv = _bwd_buffers(q, k, v, o, lse, dout, Lq, workspace, dq, dk, dv)
    rc = library().flash_attn_bwd_block(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                        _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), B, Hq, Hkv, Lq, Lk,
                                        d, scale, int(bool(causal)), window, q_offset, k_offset,
                                        _DTYPES[q.dtype], _stream(q))
    _check(rc, "flash_attn_bwd_block")
    return dq, dk, dv


def decode_workspace_bytes(B, Hq, Hkv, Lq, Lk, d, dtype=torch.bfloat16):
    return int(library().flash_attn_decode_workspace_bytes(B, Hq, Hkv, Lq, Lk, d, _DTYPES[dtype]))


def decode(q, k_cache, v_cache, cache_len=None, causal=True, window=0, scale=None, workspace=None,
           out=None, lse=None):
    """The ``Lq`` newest tokens ``q [B,Hq,Lq,d]`` attend to a KV cache ``[B,Hkv,Lk,d]``.

    ``cache_len`` (int32 CUDA tensor ``[B]``, optional) holds each sequence's valid
    entries, the new tokens' K/V being the last ``Lq`` of them.  Returns ``(o, lse)``.
    """
    if q.dim() != 4 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B, Hq, Lq, d] and the caches [B, Hkv, Lk, d]")
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError("the caches must share B and d with q")
    for t in (q, k_cache, v_cache):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q and the caches must be contiguous tensors of one dtype on one GPU")
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("decode takes bfloat16 or float16")
    if cache_len is not None:
        _expect(cache_len, "cache_len", (B,), torch.int32, q.device)
    scale, window = _scale(scale, d), _window(window)
    nbytes = decode_workspace_bytes(B, Hq, Hkv, Lq, Lk, d, q.dtype)
    if nbytes == 0:
        raise RuntimeError("flash_attn_decode: unsupported sizes")
    workspace = _workspace(workspace, nbytes, q.device)
    out = _out(out, "out", q.shape, q.dtype, q.device)
    lse = _out(lse, "lse", (B, Hq, Lq), torch.float32, q.device)
    rc = library().flash_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len), _ptr(out), _ptr(lse),
                                     _ptr(workspace), workspace.numel(), B, Hq, Hkv, Lq, Lk, d, scale,
                                     int(bool(causal)), window, _DTYPES[q.dtype], _stream(q))
    _check(rc, "flash_attn_decode")
    return out, lse


def decode_rolling_workspace_bytes(B, Hq, Hkv, Lq, W, d, dtype=torch.bfloat16):
    return int(library().flash_attn_decode_rolling_workspace_bytes(B, Hq, Hkv, Lq, W, d, _DTYPES[dtype]))


def decode_rolling(q, k_ring, v_ring, k_new, v_new, seen, window=0, scale=None, workspace=None, out=None,
                   lse=None):
    """The ``Lq`` new tokens ``q [B,Hq,Lq,d]`` over a rolling buffer ``[B,Hkv,W,d]``.

    Position ``p`` of sequence ``b`` lives in slot ``p % W``; ``seen`` (int32 CUDA
    tensor ``[B]``) holds the tokens before this call, and ``k_new``/``v_new``
    ``[B,Hkv,Lq,d]`` the new tokens' own K/V (not yet in the buffer).  New token
    ``t`` sees positions ``seen[b] + t - w + 1 .. seen[b] + t`` with ``w = window``
    (0: ``W``).  Returns ``(o, lse)``.
    """
    if q.dim() != 4 or k_ring.dim() != 4:
        raise ValueError("q must be [B, Hq, Lq, d] and the buffers [B, Hkv, W, d]")
    B, Hq, Lq, d = q.shape
    Hkv, W = k_ring.shape[1], k_ring.shape[2]
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("decode_rolling takes bfloat16 or float16")
    _expect(q, "q", (B, Hq, Lq, d), q.dtype, q.device)
    _expect(k_ring, "k_ring", (B, Hkv, W, d), q.dtype, q.device)
    _expect(v_ring, "v_ring", (B, Hkv, W, d), q.dtype, q.device)
    _expect(k_new, "k_new", (B, Hkv, Lq, d), q.dtype, q.device)
    _expect(v_new, "v_new", (B, Hkv, Lq, d), q.dtype, q.device)
    _expect(seen, "seen", (B,), torch.int32, q.device)
    scale, window = _scale(scale, d), int(window)
    if window < 0 or window > W:
        raise ValueError("window must be 0 (the whole buffer) or 1 .. W")
    nbytes = decode_rolling_workspace_bytes(B, Hq, Hkv, Lq, W, d, q.dtype)
    if nbytes == 0:
        raise RuntimeError("flash_attn_decode_rolling: unsupported sizes")
    workspace = _workspace(workspace, nbytes, q.device)
    out = _out(out, "out", q.shape, q.dtype, q.device)
    lse = _out(lse, "lse", (B, Hq, Lq), torch.float32, q.device)
    rc = library().flash_attn_decode_rolling(_ptr(q), _ptr(k_ring), _ptr(v_ring), _ptr(k_new), _ptr(v_new),
                                             _ptr(seen), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                             B, Hq, Hkv, Lq, W, d, scale, window, _DTYPES[q.dtype], _stream(q))
    _check(rc, "flash_attn_decode_rolling")
    return out, lse


class MaskPlan:
    """A general sparse mask over sequences of length ``L`` and its device plan.

    allowed(i, j) = causal_ok and ((|i - j| < window and block_mask[i // block, j // block])
                                   or i global or j global)
    (claspmoon.cn "14 · 缩放定律与高效注意力" §4.3: local window plus global tokens;
    kler.cn §4.1.2: block-sparse masks; §3.2.1 / §5.1.2: a window before and after,
    first and last token global).  ``global_tokens`` are positions (negative ones count
    from the end); ``block_mask`` is a ``[nbm, nbm]`` bool tensor with nbm = ceil(L / block)
    and ``block`` a multiple of 64.  The plan is built once on the device and serves every
    masked call of that length (all heads and layers, forward and backward).
    """

    def __init__(self, L, causal=False, window=0, global_tokens=(), block_mask=None, block=64, device="cuda"):
        self.L, self.causal, self.window, self.block = int(L), bool(causal), _window(window), int(block)
        self.global_tokens = tuple(int(p) for p in global_tokens)
        dev = torch.device(device)
        self._gpos = (torch.tensor(self.global_tokens, dtype=torch.int32, device=dev)
                      if self.global_tokens else None)
        self._bmask = None
        if block_mask is not None:
            nbm = (self.L + self.block - 1) // self.block
            bm = torch.as_tensor(block_mask)
            if bm.shape != (nbm, nbm):
                raise ValueError("block_mask must be [ceil(L / block)] * 2 = [%d, %d]" % (nbm, nbm))
            self._bmask = bm.to(dtype=torch.uint8, device=dev).contiguous()
        self.block_mask = None if block_mask is None else torch.as_tensor(block_mask).bool().cpu()
        nbytes = int(library().flash_attn_mask_plan_bytes(self.L))
        if nbytes == 0:
            raise RuntimeError("MaskPlan: unsupported length %d (1 <= L <= 2^18)" % self.L)
        self.plan = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.desc = FaMask(int(self.causal), self.window, _ptr(self._gpos), len(self.global_tokens),
                           _ptr(self._bmask), self.block)
        rc = library().flash_attn_mask_plan(ctypes.byref(self.desc), self.L, _ptr(self.plan), nbytes,
                                            _stream(self.plan))
        _check(rc, "flash_attn_mask_plan")
        # The plan is built asynchronously on the stream current now; a masked call
        # on any other stream first waits for this event.
        self.ready = torch.cuda.Event()
        self.ready.record(torch.cuda.current_stream(dev))

    def wait(self, device):
        """Make the current stream of ``device`` wait until the plan is built."""
        if self.plan.device != device:
            raise ValueError("the plan lives on %s" % self.plan.device)
        torch.cuda.current_stream(device).wait_event(self.ready)


def masked_workspace_bytes(B, Hq, Hkv, L, d, plan, backward):
    return int(library().flash_attn_masked_workspace_bytes(B, Hq, Hkv, L, d, ctypes.byref(plan.desc),
                                                           int(bool(backward))))


def fwd_masked(q, k, v, plan, scale=None, out=None, lse=None, workspace=None):
    """Exact attention under a ``MaskPlan`` (16-bit dtypes).  Returns ``(o, lse)``; rows
    with no allowed key get o = 0, lse = -inf."""
    B, Hq, Hkv, L, d = _shapes(q, k, v)
    if L != plan.L:
        raise ValueError("the plan was built for L = %d" % plan.L)
    scale = _scale(scale, d)
    out = _out(out, "out", q.shape, q.dtype, q.device)
    lse = _out(lse, "lse", (B, Hq, L), torch.float32, q.device)
    nbytes = masked_workspace_bytes(B, Hq, Hkv, L, d, plan, False)
    if workspace is not None or nbytes > 0:
        workspace = _workspace(workspace, nbytes, q.device)
    plan.wait(q.device)
    rc = library().flash_attn_fwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(workspace),
                                         0 if workspace is None else workspace.numel(), B, Hq, Hkv, L, d, scale,
                                         ctypes.byref(plan.desc), _ptr(plan.plan), plan.plan.numel(),
                                         _DTYPES[q.dtype], _stream(q))
    _check(rc, "flash_attn_fwd_masked")
    return out, lse


def bwd_masked(q, k, v, o, lse, dout, plan, scale=None, workspace=None, dq=None, dk=None, dv=None):
    """Gradient of sum(o * dout) under a ``MaskPlan``; returns ``(dq, dk, dv)``."""
    B, Hq, Hkv, L, d = _shapes(q, k, v)
    if L != plan.L:
        raise ValueError("the plan was built for L = %d" % plan.L)
    scale = _scale(scale, d)
    _expect(o, "o", q.shape, q.dtype, q.device)
    _expect(dout, "dout", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (B, Hq, L), torch.float32, q.device)
    nbytes = masked_workspace_bytes(B, Hq, Hkv, L, d, plan, True)
    workspace = _workspace(workspace, nbytes, q.device)
    dq = _out(dq, "dq", q.shape, q.dtype, q.device)
    dk = _out(dk, "dk", k.shape, k.dtype, k.device)
    dv = _out(dv, "dv", v.shape, v.dtype, v.device)
    plan.wait(q.device)
    rc = library().flash_attn_bwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                         _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), B, Hq, Hkv, L, d,
                                         scale, ctypes.byref(plan.desc), _ptr(plan.plan), plan.plan.numel(),
                                         _DTYPES[q.dtype], _stream(q))
    _check(rc, "flash_attn_bwd_masked")
    return dq, dk, dv


class FlashAttentionFunction(torch.autograd.Function):
    """Exact attention as a ``torch.autograd.Function``.

    The forward keeps only O and the per-row log-sum-exp for the backward, which
    recomputes the probabilities (claspmoon.cn "14 · 缩放定律与高效注意力" §3.3).
    Inputs are ``[B, H, L, d]`` CUDA tensors of one dtype (bfloat16 or float16 for
    training; float32 has a forward only).
    """

    @staticmethod
    def forward(ctx, q, k, v, causal=False, window=0, scale=None, plan=None):
        q, k, v = (t.contiguous() for t in (q, k, v))
        if plan is None:
            o, lse = fwd(q, k, v, causal=causal, window=window, scale=scale)
        else:
            o, lse = fwd_masked(q, k, v, plan, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.window, ctx.scale, ctx.plan = causal, window, scale, plan
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        if ctx.plan is None:
            dq, dk, dv = bwd(q, k, v, o, lse, do.contiguous(), causal=ctx.causal, window=ctx.window,
                             scale=ctx.scale)
        else:
            dq, dk, dv = bwd_masked(q, k, v, o, lse, do.contiguous(), ctx.plan, scale=ctx.scale)
        return dq, dk, dv, None, None, None, None


def scaled_dot_product_attention(q, k, v, is_causal=False, scale=None, window=0, mask_plan=None):
    """Drop-in for ``scaled_dot_product_attention(q, k, v, is_causal=...)`` on ``[B, H, L, d]``
    tensors (claspmoon.cn "14 · 缩放定律与高效注意力" §3.5), with grouped-query K/V
    (``k.shape[1]`` dividing ``q.shape[1]``) and an optional sliding ``window`` (one-sided
    with ``is_causal``, symmetric without)
    (kler.cn, §3.2.1 configuration keys).  A ``mask_plan`` (``MaskPlan``) replaces
    ``is_causal`` and ``window`` by its general sparse mask.  Differentiable through
    ``FlashAttentionFunction``.
    """
    if mask_plan is not None:
        return FlashAttentionFunction.apply(q, k, v, False, 0, scale, mask_plan)
    return FlashAttentionFunction.apply(q, k, v, bool(is_causal), int(window), scale, None)
