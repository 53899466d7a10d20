"""fp64 oracle: exact attention by its plain definition, and its gradient.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Nothing here is
tuned; every function forms the quantities the pages define explicitly.

Tensor layout: Q and O are ``[B, Hq, L, d]``; K and V are ``[B, Hkv, L, d]``;
the per-row log-sum-exp is ``[B, Hq, L]``.  Any float input is first
converted to float64 (bf16 values are exactly representable in float64).

Readings of the pages that this file encodes:

* Attention is ``softmax(s * Q K^T) V`` with the softmax over keys (mdooai.com
  "Ch.04 注意力优化", core formula); ``s`` is passed in (default 1/sqrt(d)).
* A masked logit is minus infinity, so a masked key carries exactly zero
  weight (same page, the sparse-attention formula in "公式速览").
* Causal: key j is allowed for query i iff j <= i, the diagonal included
  (claspmoon.cn "14 · 缩放定律与高效注意力" §3.5, ``is_causal=True``).
* Sliding window of width w >= 1 (only together with causal): key j is
  allowed iff i - w + 1 <= j <= i, i.e. the w most recent keys including
  the query's own (book.anysome.cn "高效注意力" §4; window width as in the
  Mistral-style configuration key of kler.cn §3.2.1).
* GQA: query head h reads key/value head h // (Hq // Hkv) (book.anysome.cn
  "高效注意力" §3: groups of query heads share one K/V head).
* The log-sum-exp saved for the backward is the natural log over the scaled,
  masked scores (claspmoon.cn §3.3: keep O and the per-row logsumexp).
* A row with no allowed key (impossible for w >= 1 with causal masking, or
  without masking) is defined as O = 0, LSE = -inf.
"""

import numpy as np


def kv_head_of(h, hq, hkv):
    """K/V head read by query head ``h``: contiguous groups of G = Hq/Hkv heads.

    book.anysome.cn "高效注意力" §3 (MQA/GQA: several query heads share one
    K/V head).  Requires Hq % Hkv == 0.
    """
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (hq // hkv)


def position_mask(q_pos, k_pos, causal, window):
    """Boolean ``[len(q_pos), len(k_pos)]``: may the query at sequence position
    ``q_pos[r]`` attend to the key at position ``k_pos[c]``?

    Causal per claspmoon.cn §3.5 (``is_causal``: keys at or before the query);
    window per book.anysome.cn §4 (each token attends only to the w nearby
    tokens, itself included): with causal masking the w - 1 preceding ones;
    without it the window reaches both ways (kler.cn §3.2.1, positions before
    and after), |i - j| < w.
    """
    i = np.asarray(q_pos, dtype=np.int64)[:, None]
    j = np.asarray(k_pos, dtype=np.int64)[None, :]
    ok = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if causal:
        ok &= j <= i
    if window > 0:
        ok &= j >= i - window + 1
        if not causal:
            ok &= j <= i + window - 1
    return ok


def allowed_mask(rows, L, causal, window):
    """Boolean ``[len(rows), L]``: may query ``rows[r]`` attend to key ``j``?
    Queries and keys of one sequence: positions are the indices."""
    return position_mask(rows, np.arange(L), causal, window)


def _masked_softmax_rows(S, ok):
    """Row softmax of S with masked logits set to -inf (mdooai.com core formula).

    Returns (A, lse) where A is row-stochastic over the allowed keys and
    lse = log sum_j exp(S_ij) over allowed j.  The row maximum is subtracted
    before exponentiating (safe softmax, kler.cn §3.1.1); in exact arithmetic
    this changes nothing.
    """
    S = np.where(ok, S, -np.inf)
    m = S.max(axis=-1, keepdims=True)
    empty = ~ok.any(axis=-1, keepdims=True)
    m_safe = np.where(empty, 0.0, m)
    E = np.exp(S - m_safe)                       # exp(-inf) == 0 exactly
    ell = E.sum(axis=-1, keepdims=True)
    A = np.where(empty, 0.0, E / np.where(empty, 1.0, ell))
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, ell)))
    return A, lse[..., 0]


def _as64(x):
    x = np.asarray(x)
    return x.astype(np.float64, copy=False)


def probabilities(q, k, scale, causal=False, window=0):
    """The full attention matrix A = softmax(s Q K^T) per (b, hq): ``[B,Hq,L,L]``.

    mdooai.com "Ch.04" core formula (A = softmax(S), rows sum to 1).  Only for
    small L: it materialises L x L per head on purpose.
    """
    q, k = _as64(q), _as64(k)
    B, Hq, L, _ = q.shape
    Hkv = k.shape[1]
    ok = allowed_mask(np.arange(L), L, causal, window)
    A = np.empty((B, Hq, L, L))
    for b in range(B):
        for h in range(Hq):
            S = scale * (q[b, h] @ k[b, kv_head_of(h, Hq, Hkv)].T)
            A[b, h], _ = _masked_softmax_rows(S, ok)
    return A


def forward_rows(q, k, v, rows, scale, causal=False, window=0):
    """O and LSE for the query rows ``rows`` only (exact for those rows).

    For each row i: S_i = s * q_i K^T over all keys, masked logits -> -inf,
    A_i = softmax(S_i), O_i = A_i V, LSE_i = log sum_j exp(S_ij)
    (mdooai.com "Ch.04" core formula; claspmoon.cn §3.3 for the saved LSE).
    Rows are independent in the definition, so any subset is exact.
    Returns float64 ``O [B,Hq,len(rows),d]`` and ``LSE [B,Hq,len(rows)]``.
    """
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    rows = np.asarray(rows, dtype=np.int64)
    ok = allowed_mask(rows, L, causal, window)
    O = np.empty((B, Hq, rows.size, d))
    lse = np.empty((B, Hq, rows.size))
    for b in range(B):
        for h in range(Hq):
            kh = kv_head_of(h, Hq, Hkv)
            # float64 copies are made one head at a time (memory only)
            qh, kk, vv = _as64(q[b, h])[rows], _as64(k[b, kh]), _as64(v[b, kh])
            S = scale * (qh @ kk.T)
            A, lse[b, h] = _masked_softmax_rows(S, ok)
            O[b, h] = A @ vv
    return O, lse


def forward(q, k, v, scale, causal=False, window=0, rows_per_chunk=4096):
    """Exact attention forward: float64 ``(O [B,Hq,L,d], LSE [B,Hq,L])``.

    The definition of ``forward_rows`` applied to every query row; rows are
    visited in chunks only to bound the memory of the explicit S (each row's
    arithmetic is unchanged by the chunking).
    """
    L = np.asarray(q).shape[2]
    Os, ls = [], []
    for r0 in range(0, L, rows_per_chunk):
        O, lse = forward_rows(q, k, v, np.arange(r0, min(L, r0 + rows_per_chunk)),
                              scale, causal, window)
        Os.append(O)
        ls.append(lse)
    return np.concatenate(Os, axis=2), np.concatenate(ls, axis=2)


def backward(q, k, v, dout, scale, causal=False, window=0):
    """Analytic gradient of sum(O * dO) w.r.t. Q, K, V, in float64.

    The pages only say that the backward recomputes the attention matrix from
    Q, K, V instead of storing it (claspmoon.cn §3.3;
    transformer.xph.ink "原理与机制").  The gradient itself is the softmax
    Jacobian applied row by row, with A formed explicitly from its definition:
        dV  = A^T dO
        dA  = dO V^T
        D_i = sum_j A_ij dA_ij
        dS  = A * (dA - D)            (softmax Jacobian)
        dQ  = s dS K,   dK = s dS^T Q
    For GQA the K/V gradients of a group's query heads are summed into the
    shared head.  Returns float64 ``(dQ, dK, dV)``.
    """
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    ok = allowed_mask(np.arange(L), L, causal, window)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kh = kv_head_of(h, Hq, Hkv)
            S = scale * (q[b, h] @ k[b, kh].T)
            A, _ = _masked_softmax_rows(S, ok)
            dv[b, kh] += A.T @ dout[b, h]
            dA = dout[b, h] @ v[b, kh].T
            dS = _softmax_backward(A, dA)
            dq[b, h] = scale * (dS @ k[b, kh])
            dk[b, kh] += scale * (dS.T @ q[b, h])
    return dq, dk, dv


def _softmax_backward(A, dA):
    """dS = A * (dA - rowsum(A * dA)): the Jacobian of a row softmax."""
    D = (A * dA).sum(axis=-1, keepdims=True)
    return A * (dA - D)


def tiled_online_forward(q, k, v, scale, causal=False, window=0,
                         row_edges=None, col_edges=None):
    """The pages' tiled algorithm with the online-softmax recurrence, in fp64.

    claspmoon.cn §3.2 (loop over query tiles Q_i, then key tiles K_j; only
    the final O is written) with the running statistics of
    transformer.xph.ink "原理与机制": per row a running max m and running sum
    l; for each key tile
        m_new = max(m, rowmax(S_tile))
        P     = exp(S_tile - m_new)
        l     = exp(m - m_new) * l + rowsum(P)
        O     = exp(m - m_new) * O + P V_tile
    and at the end O / l, LSE = m + log l.  (The printed recurrence on
    claspmoon.cn swaps the names of the max and the sum; the reading used
    here is the one the other pages state.)  ``row_edges``/``col_edges`` are
    increasing tile boundaries from 0 to L; tiles may have any sizes.
    This is an independent second path, used only to pin that the recurrence
    equals the direct definition.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    row_edges = list(row_edges) if row_edges is not None else [0, L]
    col_edges = list(col_edges) if col_edges is not None else [0, L]
    O = np.zeros((B, Hq, L, d))
    lse = np.zeros((B, Hq, L))
    for b in range(B):
        for h in range(Hq):
            kh = kv_head_of(h, Hq, Hkv)
            for r0, r1 in zip(row_edges[:-1], row_edges[1:]):
                rows = np.arange(r0, r1)
                m = np.full(rows.size, -np.inf)
                ell = np.zeros(rows.size)
                acc = np.zeros((rows.size, d))
                for c0, c1 in zip(col_edges[:-1], col_edges[1:]):
                    ok = allowed_mask(rows, L, causal, window)[:, c0:c1]
                    S = scale * (q[b, h, rows] @ k[b, kh, c0:c1].T)
                    S = np.where(ok, S, -np.inf)
                    m_new = np.maximum(m, S.max(axis=1))
                    # rows with nothing allowed so far keep m = -inf; use 0 as
                    # the shift there so that exp(-inf - 0) = 0 and no NaN arises
                    shift = np.where(np.isneginf(m_new), 0.0, m_new)
                    P = np.exp(S - shift[:, None])
                    alpha = np.exp(np.where(np.isneginf(m), -np.inf, m - shift))
                    ell = alpha * ell + P.sum(axis=1)
                    acc = alpha[:, None] * acc + P @ v[b, kh, c0:c1]
                    m = m_new
                empty = ell == 0.0
                O[b, h, rows] = np.where(empty[:, None], 0.0,
                                         acc / np.where(empty, 1.0, ell)[:, None])
                with np.errstate(divide="ignore"):
                    lse[b, h, rows] = np.where(empty, -np.inf,
                                               m + np.log(np.where(empty, 1.0, ell)))
    return O, lse


# ---------------------------------------------------------------- blocks
#
# Sequence parallelism (claspmoon.cn "14 · 缩放定律与高效注意力" §5.1: ring
# attention extends exact tiled attention across devices) splits the
# sequence into chunks.  A query chunk holds the queries at positions
# q_offset .. q_offset + Lq - 1, a key/value chunk the keys at k_offset ..
# k_offset + Lk - 1, and masks are decided on those global positions.  One
# step attends a query chunk to one key/value chunk and yields a partial
# (O, LSE) normalised over that chunk's keys; partials over disjoint key sets
# combine exactly (the online-softmax rescaling of transformer.xph.ink
# "原理与机制" applied to whole chunks).


def block_forward(q, k, v, scale, causal=False, window=0, q_offset=0, k_offset=0):
    """Attention of a query chunk against one key/value chunk: float64
    ``(O [B,Hq,Lq,d], LSE [B,Hq,Lq])``.

    Per row: S = s q K_chunk^T, masked logits (on global positions) -> -inf,
    A = softmax over the chunk's keys, O = A V_chunk, LSE = log sum exp S over
    the allowed keys of the chunk.  A row with no allowed key in the chunk has
    O = 0 and LSE = -inf (it contributes nothing to a merge).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    ok = position_mask(q_offset + np.arange(Lq), k_offset + np.arange(Lk), causal, window)
    O = np.empty((B, Hq, Lq, d))
    lse = np.empty((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            kh = kv_head_of(h, Hq, Hkv)
            S = scale * (q[b, h] @ k[b, kh].T)
            A, lse[b, h] = _masked_softmax_rows(S, ok)
            O[b, h] = A @ v[b, kh]
    return O, lse


def merge_partials(o_a, lse_a, o_b, lse_b):
    """Exact combination of two partial results over disjoint key sets.

    With LSE = log(e^{LSE_a} + e^{LSE_b}) the combined softmax weights are the
    partial ones times e^{LSE_a - LSE} and e^{LSE_b - LSE}, so
    O = e^{LSE_a - LSE} O_a + e^{LSE_b - LSE} O_b.  A side with LSE = -inf
    has no keys and weight 0; both -inf gives O = 0, LSE = -inf.
    """
    o_a, o_b = _as64(o_a), _as64(o_b)
    lse_a, lse_b = _as64(lse_a), _as64(lse_b)
    m = np.maximum(lse_a, lse_b)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    ea = np.exp(lse_a - m_safe)                 # exp(-inf) == 0
    eb = np.exp(lse_b - m_safe)
    tot = ea + eb
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, tot)))
    wa = np.where(empty, 0.0, ea / np.where(empty, 1.0, tot))
    wb = np.where(empty, 0.0, eb / np.where(empty, 1.0, tot))
    return wa[..., None] * o_a + wb[..., None] * o_b, lse


def block_backward(q, k, v, dout, o, lse, scale, causal=False, window=0, q_offset=0, k_offset=0):
    """One chunk pair's share of the gradient of sum(O * dO): float64
    ``(dQ part [B,Hq,Lq,d], dK part [B,Hkv,Lk,d], dV part [B,Hkv,Lk,d])``.

    ``o`` and ``lse`` are the query rows' results over ALL keys (every chunk),
    so the chunk's slice of the attention matrix is A_blk = exp(S - LSE) on the
    allowed keys (the recomputation of claspmoon.cn §3.3, restricted to the
    chunk).  The softmax Jacobian row term D_i = sum over all keys of A_ij dA_ij
    equals sum_c dO_ic O_ic, which only needs the row's O:
        dV_blk = A_blk^T dO,   dA_blk = dO V_blk^T,
        dS     = A_blk * (dA_blk - D),
        dQ     = s dS K_blk,   dK_blk = s dS^T Q.
    Summing dQ over the key chunks, and taking dK/dV per key chunk summed over
    the query chunks, gives the full gradient.
    """
    q, k, v, dout, o, lse = (_as64(x) for x in (q, k, v, dout, o, lse))
    B, Hq, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    ok = position_mask(q_offset + np.arange(Lq), k_offset + np.arange(Lk), causal, window)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kh = kv_head_of(h, Hq, Hkv)
            S = scale * (q[b, h] @ k[b, kh].T)
            finite = ~np.isneginf(lse[b, h])[:, None]
            A = np.where(ok & finite, np.exp(S - np.where(finite, lse[b, h][:, None], 0.0)), 0.0)
            dv[b, kh] += A.T @ dout[b, h]
            dA = dout[b, h] @ v[b, kh].T
            D = (dout[b, h] * o[b, h]).sum(axis=-1, keepdims=True)
            dS = A * (dA - D)
            dq[b, h] = scale * (dS @ k[b, kh])
            dk[b, kh] += scale * (dS.T @ q[b, h])
    return dq, dk, dv


# ---------------------------------------------------------------- decode
#
# Autoregressive generation keeps the keys and values of every earlier token
# in a cache and attends only the newest tokens' queries to it (book.anysome.cn
# "高效注意力" §1: the KV cache is one of the two large costs; §3: GQA shrinks
# it by sharing K/V heads).


def decode_forward(q, k_cache, v_cache, cache_len, scale, causal=True, window=0):
    """Attention of the Lq newest tokens to a KV cache: float64 ``(O [B,Hq,Lq,d], LSE [B,Hq,Lq])``.

    ``k_cache``/``v_cache`` are ``[B,Hkv,Lk_max,d]``; sequence b uses its first
    ``cache_len[b]`` entries, which already include the Lq new tokens at the
    end.  New token t of sequence b sits at position cache_len[b] - Lq + t
    (bottom-right alignment), so with ``causal`` it sees cache entries 0 ..
    that position (and with a window the last ``window`` of them); without
    ``causal`` it sees all cache_len[b] entries.  This is the chunk-pair
    forward with the query chunk at offset cache_len[b] - Lq and the key chunk
    at 0.
    """
    q, k_cache, v_cache = _as64(q), _as64(k_cache), _as64(v_cache)
    B, Hq, Lq, d = q.shape
    O = np.empty((B, Hq, Lq, d))
    lse = np.empty((B, Hq, Lq))
    for b in range(B):
        n = int(cache_len[b])
        if not Lq <= n <= k_cache.shape[2]:
            raise ValueError("each cache length must hold the new tokens and fit the cache")
        O[b:b + 1], lse[b:b + 1] = block_forward(q[b:b + 1], k_cache[b:b + 1, :, :n], v_cache[b:b + 1, :, :n],
                                                 scale, causal, window, n - Lq, 0)
    return O, lse


def rolling_decode_forward(q, k_ring, v_ring, k_new, v_new, seen, scale, window=0):
    """New tokens over a rolling window buffer: float64 ``(O [B,Hq,Lq,d], LSE [B,Hq,Lq])``.

    The buffer (transformer.xph.ink "高效注意力：FlashAttention 与线性注意力",
    实例或案例: Mistral keeps only the last W keys, in W slots) is ``[B,Hkv,W,d]``:
    the K/V of position p of sequence b sits in slot p mod W, and after
    ``seen[b] = n`` tokens the buffer holds positions max(0, n - W) .. n - 1.
    ``k_new``/``v_new`` ``[B,Hkv,Lq,d]`` are the new tokens' own K/V, positions
    n .. n + Lq - 1.  New token t (position n + t) attends causally to the
    ``window`` most recent positions (0 means W).

    By definition: read the buffer back into position order, append the new
    keys, and attend the query chunk at offset n to that key chunk at offset
    max(0, n - W) with the causal window -- the chunk-pair forward.
    """
    q, k_ring, v_ring = _as64(q), _as64(k_ring), _as64(v_ring)
    k_new, v_new = _as64(k_new), _as64(v_new)
    B, Hq, Lq, d = q.shape
    W = k_ring.shape[2]
    w = W if window == 0 else int(window)
    if not 1 <= w <= W:
        raise ValueError("the window must fit the buffer")
    O = np.empty((B, Hq, Lq, d))
    lse = np.empty((B, Hq, Lq))
    for b in range(B):
        n = int(seen[b])
        if n < 0:
            raise ValueError("seen counts must be >= 0")
        positions = np.arange(max(0, n - W), n)
        slots = positions % W
        k_seq = np.concatenate([k_ring[b:b + 1, :, slots], k_new[b:b + 1]], axis=2)
        v_seq = np.concatenate([v_ring[b:b + 1, :, slots], v_new[b:b + 1]], axis=2)
        O[b:b + 1], lse[b:b + 1] = block_forward(q[b:b + 1], k_seq, v_seq, scale, True, w, n, max(0, n - W))
    return O, lse


# ---------------------------------------------------------------- general masks
#
# Sparse patterns that keep attention exact on the positions they allow
# (claspmoon.cn "14 · 缩放定律与高效注意力" §4.3, Longformer / BigBird: a
# sliding window plus a few global tokens; kler.cn §3.2.1: a sliding window
# looks at positions before and after; kler.cn §4.1.2: block-sparse masks in
# which a query block attends to nearby key blocks; kler.cn's hybrid
# configuration: window 512 with the first and last token global).


def general_mask(q_pos, k_pos, causal=False, window=0, block_mask=None, block=64, global_pos=()):
    """Boolean ``[len(q_pos), len(k_pos)]`` of the general mask family:

        allowed(i, j) = causal_ok(i, j) and ((window_ok(i, j) and block_ok(i, j))
                                            or i is global or j is global)

    causal_ok: j <= i when ``causal``; window_ok: |i - j| < window when
    window > 0 (with causal this is the usual i - w < j <= i; without it the
    window is symmetric); block_ok: ``block_mask[i // block][j // block]``
    when a block mask is given; global: the position is in ``global_pos``.
    """
    i = np.asarray(q_pos, dtype=np.int64)[:, None]
    j = np.asarray(k_pos, dtype=np.int64)[None, :]
    local = np.ones((i.shape[0], j.shape[1]), dtype=bool)
    if window > 0:
        local &= np.abs(i - j) < window
    if block_mask is not None:
        bm = np.asarray(block_mask, dtype=bool)
        local &= bm[i // block, j // block]
    g = np.asarray(sorted(set(int(x) for x in global_pos)), dtype=np.int64)
    ok = local | np.isin(i, g) | np.isin(j, g)
    if causal:
        ok &= j <= i
    return ok


def forward_with_mask(q, k, v, scale, ok):
    """Exact attention under an explicit boolean mask ``ok [L, L]`` (same for every head):
    the definition of ``forward_rows`` with ``ok`` in place of the causal/window mask."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    O = np.empty((B, Hq, L, d))
    lse = np.empty((B, Hq, L))
    for b in range(B):
        for h in range(Hq):
            kh = kv_head_of(h, Hq, Hkv)
            S = scale * (q[b, h] @ k[b, kh].T)
            A, lse[b, h] = _masked_softmax_rows(S, ok)
            O[b, h] = A @ v[b, kh]
    return O, lse


def backward_with_mask(q, k, v, dout, scale, ok):
    """Gradient of sum(O * dO) under an explicit boolean mask: ``backward`` with ``ok``."""
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kh = kv_head_of(h, Hq, Hkv)
            A, _ = _masked_softmax_rows(scale * (q[b, h] @ k[b, kh].T), ok)
            dv[b, kh] += A.T @ dout[b, h]
            dS = _softmax_backward(A, dout[b, h] @ v[b, kh].T)
            dq[b, h] = scale * (dS @ k[b, kh])
            dk[b, kh] += scale * (dS.T @ q[b, h])
    return dq, dk, dv


def forward_rows_with_mask(q, k, v, rows, scale, ok_rows):
    """Rows ``rows`` of ``forward_with_mask``: ``ok_rows [len(rows), L]`` is the mask of those
    query rows (for example ``general_mask(rows, arange(L), ...)``).  Each row of the
    definition depends on its own query only, so sampled rows of a long sequence are exact."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    rows = np.asarray(rows)
    O = np.empty((B, Hq, len(rows), d))
    lse = np.empty((B, Hq, len(rows)))
    for b in range(B):
        for h in range(Hq):
            kh = kv_head_of(h, Hq, Hkv)
            S = scale * (q[b, h, rows] @ k[b, kh].T)
            A, lse[b, h] = _masked_softmax_rows(S, ok_rows)
            O[b, h] = A @ v[b, kh]
    return O, lse


def dq_rows_with_mask(q, k, v, dout, rows, scale, ok_rows):
    """Rows ``rows`` of dQ from ``backward_with_mask``.  dQ_i needs only row i: its
    probabilities P_i, dP_i = dO_i V^T and D_i = sum_j P_ij dP_ij (claspmoon.cn §3.3)."""
    q, k, v, dout = _as64(q), _as64(k), _as64(v), _as64(dout)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    rows = np.asarray(rows)
    dq = np.empty((B, Hq, len(rows), d))
    for b in range(B):
        for h in range(Hq):
            kh = kv_head_of(h, Hq, Hkv)
            A, _ = _masked_softmax_rows(scale * (q[b, h, rows] @ k[b, kh].T), ok_rows)
            dS = _softmax_backward(A, dout[b, h, rows] @ v[b, kh].T)
            dq[b, h] = scale * (dS @ k[b, kh])
    return dq
