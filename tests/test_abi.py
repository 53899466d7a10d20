"""C-ABI checks that need no GPU: the library loads, exports every symbol the
public header declares, and rejects invalid arguments before any HIP call."""

import ctypes
import os
import re

import pytest

import exact_tiled_attention_flash_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flash_attn.h")

FAKE = 0x10000      # 16-byte aligned, never dereferenced: validation must fail first
MISALIGNED = 0x10008


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flash_attn_\w+)\s*\(", text)))


def header_constants():
    text = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"#define\s+(FA_\w+)\s+\(?(-?\d+)\)?", text)}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.library_path()):
        pytest.skip("libflashattn.so not built")
    return fa.library()


def test_header_declares_the_boundary():
    assert header_functions() == sorted(fa.EXPORTED_SYMBOLS)


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_binding_constants_match_header():
    c = header_constants()
    assert c["FA_DTYPE_F32"] == fa.FA_DTYPE_F32 and c["FA_DTYPE_BF16"] == fa.FA_DTYPE_BF16
    assert c["FA_DTYPE_F16"] == fa.FA_DTYPE_F16
    assert c["FA_OK"] == 0


def test_strerror_and_version(lib):
    c = header_constants()
    for name in ("FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_GQA",
                 "FA_ERR_WORKSPACE", "FA_ERR_HIP", "FA_ERR_TOO_LARGE"):
        s = fa.strerror(c[name])
        assert s and s != "unknown error code"
    assert fa.strerror(12345) == "unknown error code"
    assert lib.flash_attn_version() >= 100


def call_fwd(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=2, Hkv=2, L=16, d=64,
             scale=0.125, causal=1, window=0, dtype=fa.FA_DTYPE_BF16):
    return lib.flash_attn_fwd(q, k, v, o, lse, B, Hq, Hkv, L, d, scale, causal, window, dtype, None)


def call_bwd(lib, ws=FAKE * 16, ws_bytes=1 << 20, B=1, Hq=2, Hkv=2, L=16, d=64, scale=0.125,
             causal=1, window=0, dtype=fa.FA_DTYPE_BF16, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE)
    p.update(ptrs)
    return lib.flash_attn_bwd(p["q"], p["k"], p["v"], p["o"], p["lse"], p["do"], p["dq"], p["dk"], p["dv"],
                              ws, ws_bytes, B, Hq, Hkv, L, d, scale, causal, window, dtype, None)


def test_fwd_rejects_invalid_arguments(lib):
    c = header_constants()
    INV, UNS, GQA = c["FA_ERR_INVALID_ARG"], c["FA_ERR_UNSUPPORTED"], c["FA_ERR_GQA"]
    assert call_fwd(lib, q=None) == INV
    assert call_fwd(lib, o=None) == INV
    assert call_fwd(lib, k=MISALIGNED) == INV
    assert call_fwd(lib, lse=MISALIGNED) == INV
    for bad in (dict(B=0), dict(Hq=0), dict(Hkv=0), dict(L=0), dict(L=-3), dict(L=(1 << 23) + 1),
                dict(B=128, Hq=1, Hkv=1, L=1 << 23), dict(B=1 << 10, Hq=1 << 10, Hkv=1 << 10, L=1 << 10),
                dict(scale=0.0), dict(scale=-1.0), dict(scale=float("inf")), dict(scale=float("nan")),
                dict(causal=2), dict(window=-1)):
        assert call_fwd(lib, **bad) == INV, bad
    assert call_fwd(lib, d=96) == UNS
    assert call_fwd(lib, d=256) == UNS
    assert call_fwd(lib, dtype=7) == UNS
    assert call_fwd(lib, dtype=3) == UNS
    assert call_fwd(lib, dtype=fa.FA_DTYPE_F16, q=None) == INV    # fp16 passes the dtype check
    assert call_fwd(lib, causal=0, window=4, q=None) == INV     # a symmetric window passes the mask check
    assert call_fwd(lib, Hq=6, Hkv=4) == GQA


def test_bwd_rejects_invalid_arguments(lib):
    c = header_constants()
    INV, UNS, WS = c["FA_ERR_INVALID_ARG"], c["FA_ERR_UNSUPPORTED"], c["FA_ERR_WORKSPACE"]
    need = lib.flash_attn_bwd_workspace_bytes(1, 2, 2, 16, 64, fa.FA_DTYPE_BF16)
    assert need == 256                                   # 2*2*16 floats rounded up to 256 bytes
    assert call_bwd(lib, ws=None) == WS
    assert call_bwd(lib, ws_bytes=need - 1) == WS
    assert call_bwd(lib, ws=FAKE * 16 + 16) == WS        # must be 256-byte aligned
    assert call_bwd(lib, dq=None) == INV
    assert call_bwd(lib, lse=MISALIGNED) == INV
    assert call_bwd(lib, dtype=fa.FA_DTYPE_F32) == UNS
    assert call_bwd(lib, dtype=3) == UNS
    assert call_bwd(lib, dtype=fa.FA_DTYPE_F16, dq=None) == INV   # fp16 passes the dtype check
    assert call_bwd(lib, causal=0, window=3, dq=None) == INV    # a symmetric window passes the mask check
    assert call_bwd(lib, Hq=3, Hkv=2) == c["FA_ERR_GQA"]


def test_stage_entry_points_reject_invalid_arguments(lib):
    c = header_constants()
    INV, UNS, WS, GQA = c["FA_ERR_INVALID_ARG"], c["FA_ERR_UNSUPPORTED"], c["FA_ERR_WORKSPACE"], c["FA_ERR_GQA"]
    ws, nb = FAKE * 16, 1 << 20
    pre = lambda o=FAKE, lse=FAKE, do=FAKE, ws=ws, nb=nb, B=1, Hq=2, Hkv=2, L=16, d=64, dt=fa.FA_DTYPE_BF16: \
        lib.flash_attn_bwd_preprocess(o, lse, do, ws, nb, B, Hq, Hkv, L, d, dt, None)
    assert pre(o=None) == INV and pre(lse=MISALIGNED) == INV
    assert pre(ws=None) == WS and pre(nb=255) == WS
    assert pre(d=80) == UNS and pre(dt=fa.FA_DTYPE_F32) == UNS and pre(Hq=3) == GQA and pre(L=0) == INV
    kv = lambda q=FAKE, dk=FAKE, ws=ws, nb=nb, L=16, causal=1, window=0, Hkv=2: \
        lib.flash_attn_bwd_dkdv(q, FAKE, FAKE, FAKE, ws, nb, dk, FAKE, 1, 2, Hkv, L, 64, 0.125, causal, window,
                                fa.FA_DTYPE_BF16, None)
    assert kv(q=None) == INV and kv(dk=MISALIGNED) == INV and kv(ws=FAKE * 16 + 64) == WS
    assert kv(causal=0, window=2, q=None) == INV and kv(Hkv=3) == GQA and kv(L=-1) == INV
    dqf = lambda dq=FAKE, ws=ws, nb=nb, scale=0.125: \
        lib.flash_attn_bwd_dq(FAKE, FAKE, FAKE, FAKE, ws, nb, dq, 1, 2, 2, 16, 64, scale, 1, 0,
                              fa.FA_DTYPE_BF16, None)
    assert dqf(dq=None) == INV and dqf(nb=0) == WS and dqf(scale=-2.0) == INV


def test_workspace_size_formula(lib):
    """flash_attn_bwd's workspace: two float32 per query row (D and LSE*log2 e)
    rounded up to 256 bytes.  flash_attn_bwd_fused's adds its float32 dQ
    accumulator [B, Hq, L, d] after them."""
    f = lib.flash_attn_bwd_workspace_bytes
    assert f(2, 32, 32, 4096, 128, fa.FA_DTYPE_BF16) == 2 * 32 * 4096 * 8
    assert f(1, 3, 1, 5, 64, fa.FA_DTYPE_BF16) == 256
    assert f(1, 1, 1, 40, 64, fa.FA_DTYPE_BF16) == 512
    assert f(1, 3, 2, 5, 64, fa.FA_DTYPE_BF16) == 0       # invalid sizes -> 0
    assert f(1, 2, 2, 5, 80, fa.FA_DTYPE_BF16) == 0
    assert f(2, 32, 32, 4096, 128, fa.FA_DTYPE_F16) == 2 * 32 * 4096 * 8
    assert f(2, 32, 32, 4096, 128, 3) == 0
    ff = lib.flash_attn_bwd_fused_workspace_bytes
    assert ff(2, 32, 32, 4096, 128, fa.FA_DTYPE_BF16) == 2 * 32 * 4096 * 8 + 2 * 32 * 4096 * 128 * 4
    assert ff(1, 3, 1, 5, 64, fa.FA_DTYPE_BF16) == 256 + 3 * 5 * 64 * 4
    assert ff(1, 3, 2, 5, 64, fa.FA_DTYPE_BF16) == 0
    # one head of the accumulator must stay below 4 GiB (L * d * 4 < 2^32)
    assert ff(1, 1, 1, 1 << 23, 128, fa.FA_DTYPE_BF16) == 0
    assert ff(1, 1, 1, (1 << 23) - 1, 128, fa.FA_DTYPE_BF16) == -(-((1 << 23) - 1) * 8 // 256) * 256 + ((1 << 23) - 1) * 512


def test_bwd_fused_rejects_invalid_arguments(lib):
    c = header_constants()
    ff = lib.flash_attn_bwd_fused_workspace_bytes
    need = ff(1, 2, 2, 16, 64, fa.FA_DTYPE_BF16)

    def call(ws=FAKE * 16, nb=need, L=16, d=64, dq=FAKE, dtype=fa.FA_DTYPE_BF16):
        return lib.flash_attn_bwd_fused(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dq, FAKE, FAKE, ws, nb, 1, 2, 2, L, d,
                                        0.125, 1, 0, dtype, None)
    assert call(nb=need - 1) == c["FA_ERR_WORKSPACE"]
    assert call(nb=lib.flash_attn_bwd_workspace_bytes(1, 2, 2, 16, 64, fa.FA_DTYPE_BF16)) == c["FA_ERR_WORKSPACE"]
    assert call(ws=None) == c["FA_ERR_WORKSPACE"]
    assert call(dq=None) == c["FA_ERR_INVALID_ARG"]
    assert call(dtype=fa.FA_DTYPE_F32) == c["FA_ERR_UNSUPPORTED"]
    assert call(L=1 << 23, d=128, nb=1 << 40) == c["FA_ERR_UNSUPPORTED"]   # one head's accumulator: 4 GiB


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "_LIB", None)
    monkeypatch.setattr(fa, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        fa.library()


def test_chunk_and_merge_entry_points_reject_invalid_arguments(lib):
    c = header_constants()
    INV, UNS, WS, GQA = c["FA_ERR_INVALID_ARG"], c["FA_ERR_UNSUPPORTED"], c["FA_ERR_WORKSPACE"], c["FA_ERR_GQA"]

    def fb(q=FAKE, Lq=16, Lk=32, d=64, causal=1, window=0, qo=0, ko=0, dt=fa.FA_DTYPE_BF16, Hkv=2):
        return lib.flash_attn_fwd_block(q, FAKE, FAKE, FAKE, FAKE, 1, 2, Hkv, Lq, Lk, d, 0.125, causal, window,
                                        qo, ko, dt, None)
    assert fb(q=None) == INV and fb(Lk=0) == INV and fb(Lq=0) == INV
    assert fb(qo=-1) == INV and fb(ko=(1 << 29) + 1) == INV and fb(qo=(1 << 29) + 1) == INV
    assert fb(Lk=(1 << 23) + 1) == INV
    assert fb(dt=fa.FA_DTYPE_F32) == UNS and fb(dt=3) == UNS and fb(d=96) == UNS
    assert fb(causal=0, window=2, q=None) == INV and fb(Hkv=3) == GQA
    assert fb(dt=fa.FA_DTYPE_F16, q=None) == INV                     # fp16 passes the dtype check

    def mg(oa=FAKE, la=FAKE, o=FAKE, L=16, d=64, dt=fa.FA_DTYPE_BF16):
        return lib.flash_attn_merge(oa, la, FAKE, FAKE, o, FAKE, 1, 2, L, d, dt, None)
    assert mg(oa=None) == INV and mg(la=MISALIGNED) == INV and mg(o=None) == INV and mg(L=0) == INV
    assert mg(d=80) == UNS and mg(dt=3) == UNS
    assert mg(dt=fa.FA_DTYPE_F32, oa=None) == INV                    # fp32 partials are accepted

    def bb(ws=FAKE * 16, nb=1 << 20, Lk=32, qo=0, dt=fa.FA_DTYPE_BF16, dq=FAKE):
        return lib.flash_attn_bwd_block(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dq, FAKE, FAKE, ws, nb, 1, 2, 2, 16, Lk,
                                        64, 0.125, 1, 0, qo, 0, dt, None)
    assert bb(ws=None) == WS and bb(nb=16) == WS and bb(Lk=-1) == INV and bb(qo=-5) == INV
    assert bb(dt=fa.FA_DTYPE_F32) == UNS and bb(dq=None) == INV


def test_decode_entry_points_reject_invalid_arguments(lib):
    c = header_constants()
    INV, UNS, WS, GQA = c["FA_ERR_INVALID_ARG"], c["FA_ERR_UNSUPPORTED"], c["FA_ERR_WORKSPACE"], c["FA_ERR_GQA"]
    wsb = lib.flash_attn_decode_workspace_bytes
    assert wsb(1, 8, 2, 1, 4096, 128, fa.FA_DTYPE_BF16) > 0
    assert wsb(1, 8, 2, 9, 4096, 128, fa.FA_DTYPE_BF16) > 0         # 4 heads x 9 tokens: two row groups
    assert wsb(1, 1 << 16, 1, 33, 4096, 64, fa.FA_DTYPE_BF16) == 0  # more than 65535 row groups
    assert wsb(1, 8, 2, 1, 4096, 128, fa.FA_DTYPE_F32) == 0
    assert wsb(1, 8, 3, 1, 4096, 128, fa.FA_DTYPE_BF16) == 0
    assert wsb(1, 8, 2, 5, 4, 128, fa.FA_DTYPE_BF16) == 0           # cache shorter than the new tokens

    def dec(q=FAKE, cl=None, ws=FAKE * 16, nb=1 << 30, Hq=8, Hkv=2, Lq=1, Lk=4096, d=128, scale=0.1, causal=1,
            window=0, dt=fa.FA_DTYPE_BF16):
        return lib.flash_attn_decode(q, FAKE, FAKE, cl, FAKE, FAKE, ws, nb, 1, Hq, Hkv, Lq, Lk, d, scale, causal,
                                     window, dt, None)
    assert dec(q=None) == INV and dec(cl=FAKE + 2) == INV and dec(scale=0.0) == INV and dec(causal=3) == INV
    assert dec(ws=None) == WS and dec(nb=16) == WS and dec(ws=FAKE * 16 + 128) == WS
    assert dec(Lq=40, q=None) == INV                 # 160 rows per K/V head pass the size checks
    assert dec(dt=fa.FA_DTYPE_F32) == UNS and dec(d=96) == UNS
    assert dec(causal=0, window=8) == UNS and dec(Hkv=3) == GQA and dec(Lk=0) == INV


def test_rolling_decode_rejects_invalid_arguments(lib):
    c = header_constants()
    INV, UNS, WS, GQA = c["FA_ERR_INVALID_ARG"], c["FA_ERR_UNSUPPORTED"], c["FA_ERR_WORKSPACE"], c["FA_ERR_GQA"]
    wsb = lib.flash_attn_decode_rolling_workspace_bytes
    assert wsb(1, 8, 2, 4, 1024, 128, fa.FA_DTYPE_BF16) > 0
    assert wsb(1, 8, 2, 4, 1024, 128, fa.FA_DTYPE_BF16) >= lib.flash_attn_decode_workspace_bytes(
        1, 8, 2, 4, 1024, 128, fa.FA_DTYPE_BF16)                  # the buffer's splits and the new tokens'
    assert wsb(1, 8, 2, 2000, 1024, 128, fa.FA_DTYPE_BF16) > 0      # more new tokens than slots
    assert wsb(1, 8, 2, 4, 1024, 128, fa.FA_DTYPE_F32) == 0
    assert wsb(1, 8, 3, 4, 1024, 128, fa.FA_DTYPE_BF16) == 0
    assert wsb(1, 8, 2, 0, 1024, 128, fa.FA_DTYPE_BF16) == 0
    assert wsb(1, 8, 2, 4, 0, 128, fa.FA_DTYPE_BF16) == 0

    def roll(q=FAKE, seen=FAKE, ws=FAKE * 16, nb=1 << 30, Hq=8, Hkv=2, Lq=4, W=1024, d=128, scale=0.1, window=0,
             dt=fa.FA_DTYPE_BF16, kn=FAKE):
        return lib.flash_attn_decode_rolling(q, FAKE, FAKE, kn, FAKE, seen, FAKE, FAKE, ws, nb, 1, Hq, Hkv, Lq, W, d,
                                             scale, window, dt, None)
    assert roll(q=None) == INV and roll(kn=None) == INV and roll(kn=MISALIGNED) == INV
    assert roll(seen=None) == INV and roll(seen=FAKE + 2) == INV
    assert roll(scale=0.0) == INV and roll(window=-1) == INV and roll(window=1025) == INV
    assert roll(ws=None) == WS and roll(nb=16) == WS and roll(ws=FAKE * 16 + 128) == WS
    assert roll(dt=fa.FA_DTYPE_F32) == UNS and roll(d=96) == UNS and roll(Hkv=3) == GQA
    assert roll(W=0) == INV and roll(Lq=0) == INV


def test_mask_entry_points_reject_invalid_arguments(lib):
    c = header_constants()
    INV, UNS, WS, GQA = c["FA_ERR_INVALID_ARG"], c["FA_ERR_UNSUPPORTED"], c["FA_ERR_WORKSPACE"], c["FA_ERR_GQA"]
    pb = lib.flash_attn_mask_plan_bytes
    assert pb(1) == 9 * 256                      # nine 256-byte aligned sections
    assert pb(0) == 0 and pb((1 << 18) + 1) == 0
    assert pb(1 << 18) > pb(4096) > 0
    need = pb(1000)

    def mask(causal=0, window=0, gpos=None, ng=0, bmask=None, block=64):
        return ctypes.byref(fa.FaMask(causal, window, gpos, ng, bmask, block))

    def plan(m=None, L=1000, p=FAKE * 256, nb=need):
        return lib.flash_attn_mask_plan(mask() if m is None else m, L, p, nb, None)
    assert lib.flash_attn_mask_plan(None, 1000, FAKE * 256, need, None) == INV
    assert plan(m=mask(causal=2)) == INV and plan(m=mask(window=-1)) == INV
    assert plan(m=mask(ng=3)) == INV and plan(m=mask(gpos=FAKE, ng=-1)) == INV
    assert plan(m=mask(gpos=FAKE, ng=(1 << 16) + 1)) == INV
    assert plan(m=mask(bmask=FAKE, block=96)) == UNS and plan(m=mask(bmask=FAKE, block=32)) == UNS
    assert plan(L=(1 << 18) + 1) == UNS and plan(L=0) == INV
    assert plan(p=None) == WS and plan(p=FAKE * 256 + 64) == WS and plan(nb=need - 1) == WS

    def fm(q=FAKE, m=None, p=FAKE * 256, nb=need, L=1000, dt=fa.FA_DTYPE_BF16, Hkv=2, d=128, ws=None, wn=0):
        return lib.flash_attn_fwd_masked(q, FAKE, FAKE, FAKE, None, ws, wn, 1, 2, Hkv, L, d, 0.125,
                                         mask() if m is None else m, p, nb, dt, None)
    assert lib.flash_attn_fwd_masked(FAKE, FAKE, FAKE, FAKE, None, None, 0, 1, 2, 2, 1000, 128, 0.125, None,
                                     FAKE * 256, need, fa.FA_DTYPE_BF16, None) == INV
    # the forward needs a workspace only with global positions
    wsb_f = lib.flash_attn_masked_workspace_bytes
    assert wsb_f(1, 2, 2, 1000, 128, mask(), 0) == 0
    gneed = wsb_f(1, 2, 2, 1000, 128, mask(gpos=FAKE, ng=2), 0)
    assert gneed > 0 and gneed % 256 == 0
    assert fm(m=mask(gpos=FAKE, ng=2)) == WS and fm(m=mask(gpos=FAKE, ng=2), ws=FAKE * 256, wn=gneed - 1) == WS
    assert fm(m=mask(gpos=FAKE, ng=2), ws=FAKE * 256 + 16, wn=gneed) == WS
    assert fm(m=mask(gpos=FAKE, ng=2), ws=FAKE * 256, wn=gneed, q=None) == INV
    assert wsb_f(1, 2, 2, 1000, 128, None, 0) == 0 and wsb_f(1, 2, 2, (1 << 18) + 1, 128, mask(), 0) == 0
    assert fm(q=None) == INV and fm(dt=fa.FA_DTYPE_F32) == UNS and fm(d=80) == UNS and fm(Hkv=3) == GQA
    assert fm(p=None) == WS and fm(nb=need - 1) == WS and fm(m=mask(bmask=FAKE, block=100)) == UNS
    assert fm(m=mask(causal=1, window=-2)) == INV and fm(L=(1 << 18) + 2, nb=1 << 40) == UNS

    wsb = lib.flash_attn_bwd_workspace_bytes(1, 2, 2, 1000, 128, fa.FA_DTYPE_BF16)
    assert wsb_f(1, 2, 2, 1000, 128, mask(), 1) == wsb
    assert wsb_f(1, 2, 2, 1000, 128, mask(gpos=FAKE, ng=40), 1) > wsb

    def bm(dq=FAKE, ws=FAKE * 256, wn=wsb, p=FAKE * 256, nb=need, m=None):
        return lib.flash_attn_bwd_masked(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dq, FAKE, FAKE, ws, wn, 1, 2, 2, 1000,
                                         128, 0.125, mask() if m is None else m, p, nb, fa.FA_DTYPE_BF16, None)
    assert bm(dq=None) == INV and bm(ws=None) == WS and bm(wn=wsb - 1) == WS
    assert bm(p=None) == WS and bm(nb=16) == WS and bm(m=mask(ng=1)) == INV


def test_bwd_noalloc_rejects_before_any_hip_call(lib):
    """Sizes beyond the static scratch, and the usual invalid arguments, return an
    error code before the scratch is looked up or any kernel launched."""
    c = header_constants()
    assert c["FA_NOALLOC_MAX_ROWS"] == fa.NOALLOC_MAX_ROWS == 1 << 21

    def call(B=1, Hq=2, Hkv=2, L=16, d=64, scale=0.125, causal=1, window=0, dtype=fa.FA_DTYPE_BF16, dq=FAKE):
        return lib.flash_attn_bwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dq, FAKE, FAKE,
                                          B, Hq, Hkv, L, d, scale, causal, window, dtype, None)
    assert call(B=1, Hq=32, L=(1 << 16) + 1) == c["FA_ERR_TOO_LARGE"]
    assert call(B=2, Hq=32, L=(1 << 15) + 1, Hkv=8) == c["FA_ERR_TOO_LARGE"]
    assert call(dtype=fa.FA_DTYPE_F32) == c["FA_ERR_UNSUPPORTED"]
    assert call(d=96) == c["FA_ERR_UNSUPPORTED"]
    assert call(Hkv=3) == c["FA_ERR_GQA"]
    assert call(dq=None) == c["FA_ERR_INVALID_ARG"]
    assert call(dq=MISALIGNED) == c["FA_ERR_INVALID_ARG"]
    assert call(scale=0.0) == c["FA_ERR_INVALID_ARG"]
    assert fa.strerror(c["FA_ERR_TOO_LARGE"]).startswith("sizes exceed")
