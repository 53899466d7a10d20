/*
 * flash_attn.h -- C ABI of the MI355X (gfx950) exact tiled attention library.
 *
 * What is computed (forward): for every batch b and query head h,
 *     O = softmax(s * Q K^T) V
 * with the softmax taken over keys (mdooai.com, "Ch.04 注意力优化：
 * FlashAttention 与稀疏注意力", core formula), computed tile by tile with the
 * online-softmax recurrence -- a running row maximum and running row sum,
 * and a rescale of the partial output whenever the maximum grows
 * (claspmoon.cn, "14 · 缩放定律与高效注意力", §3.2 Tiling;
 * transformer.xph.ink, "高效注意力：FlashAttention 与线性注意力", 原理与机制).
 * The L x L score matrix is never stored.  The forward also returns the
 * per-row natural log-sum-exp of the scaled, masked scores, which is all the
 * backward needs besides O (claspmoon.cn §3.3, backward recomputation).
 *
 * Backward: given dO, returns dQ, dK, dV of sum(O * dO), recomputing the
 * attention probabilities from Q, K and the saved log-sum-exp instead of
 * reading a stored matrix (claspmoon.cn §3.3).
 *
 * Masks (a masked score is -inf and carries exactly zero weight,
 * mdooai.com "Ch.04", sparse-attention formula):
 *   causal  -- key j is allowed for query i iff j <= i (claspmoon.cn §3.5,
 *              is_causal);
 *   window  -- w >= 1 with causal: allowed iff i-w+1 <= j <= i, the w most
 *              recent keys including the query itself (book.anysome.cn,
 *              "高效注意力", §4 sliding window); w >= 1 without causal: the
 *              window reaches both ways, allowed iff |i - j| < w (kler.cn
 *              §3.2.1: positions before and after the query).
 * Grouped-query attention (book.anysome.cn "高效注意力" §3): Hkv divides Hq
 * and query head h reads K/V head h / (Hq / Hkv).
 *
 * Layout (all tensors dense, row-major, the head dimension fastest):
 *   Q, O, dO, dQ : [B, Hq,  L, d]
 *   K, V, dK, dV : [B, Hkv, L, d]
 *   LSE          : [B, Hq,  L]     float32, natural logarithm
 * Element type of Q/K/V/O/dO/dQ/dK/dV is given by `dtype` (FA_DTYPE_*).
 *
 * Conventions shared by every entry point:
 *   - Pointers are device pointers (hipMalloc'd or equivalent), 16-byte
 *     aligned.  The caller allocates and owns every buffer; the library
 *     allocates nothing and keeps no per-call state.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *     asynchronous on that stream and never synchronise the host.
 *   - Every argument is validated on the host before any HIP call; a
 *     rejected call launches nothing and returns a negative FA_ERR_* code.
 *     A HIP launch failure returns FA_ERR_HIP.  flash_attn_strerror() names
 *     every code.
 *   - Outputs must not alias inputs.
 */
#ifndef FLASH_ATTN_MI355_H
#define FLASH_ATTN_MI355_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types: 32-bit float, bfloat16, IEEE half (fp16).  The 16-bit
 * types take the MFMA path with float32 accumulation and round-to-nearest-even
 * outputs; float32 takes a vector-ALU path (forward only). */
#define FA_DTYPE_F32  0
#define FA_DTYPE_BF16 1
#define FA_DTYPE_F16  2

/* return codes */
#define FA_OK                0
#define FA_ERR_INVALID_ARG  (-1)  /* null/misaligned pointer, non-positive size, bad scale */
#define FA_ERR_UNSUPPORTED  (-2)  /* head dim, dtype, or an unsupported mask combination */
#define FA_ERR_GQA          (-3)  /* Hq is not a multiple of Hkv */
#define FA_ERR_WORKSPACE    (-4)  /* backward workspace missing or too small */
#define FA_ERR_HIP          (-5)  /* a HIP launch or runtime call failed */
#define FA_ERR_TOO_LARGE    (-6)  /* sizes beyond flash_attn_bwd_noalloc's static scratch */

/*
 * Forward pass.
 *   q [B,Hq,L,d], k/v [B,Hkv,L,d]  : inputs (dtype)
 *   o [B,Hq,L,d]                    : output (dtype, rounded to nearest even)
 *   lse [B,Hq,L] float32            : output log-sum-exp; may be NULL if not wanted
 *   softmax_scale                   : s > 0 and finite (usually 1/sqrt(d))
 *   causal                          : 0 or 1
 *   window                          : 0 = none; w >= 1 (one-sided with causal,
 *                                     symmetric without); every w >= 2^30
 *                                     admits all pairs and acts as none
 *   dtype                           : FA_DTYPE_BF16, FA_DTYPE_F16 or
 *                                     FA_DTYPE_F32, each with d in {64,128}
 * Sizes: 1 <= L <= 2^23 (one head must stay below 4 GiB), B, Hq, Hkv >= 1,
 *        B*Hq*L < 2^30 (launch sizes; beyond 128 GiB per bf16 tensor at d=64).
 * Extra device memory: none.  Returns FA_OK or a negative FA_ERR_* code.
 */
int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int L, int d,
                   float softmax_scale, int causal, int window, int dtype, void* stream);

/*
 * Bytes of device workspace flash_attn_bwd needs for these sizes: two
 * float32 per query row (the row dot product D_i = sum_c dO_ic * O_ic, stored
 * negated, and the log-sum-exp in base 2), i.e. 8*B*Hq*L rounded up to 256 bytes.
 * Returns 0 for invalid sizes.
 */
size_t flash_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int dtype);

/*
 * Backward pass (recomputation from Q, K, V, O and the forward's LSE).
 *   q, k, v, o, lse                 : exactly the forward's inputs and outputs
 *   dout [B,Hq,L,d]                 : upstream gradient dO (dtype)
 *   dq [B,Hq,L,d], dk/dv [B,Hkv,L,d]: outputs (dtype); for GQA the K/V
 *                                     gradients of a group's query heads are
 *                                     summed into the shared head
 *   workspace, workspace_bytes      : caller-owned device scratch of at least
 *                                     flash_attn_bwd_workspace_bytes() bytes,
 *                                     256-byte aligned; its contents on entry
 *                                     are ignored
 *   dtype                           : FA_DTYPE_BF16 or FA_DTYPE_F16, d in
 *                                     {64,128} (FA_DTYPE_F32: unsupported)
 * Returns FA_OK or a negative FA_ERR_* code.
 */
int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes,
                   int B, int Hq, int Hkv, int L, int d,
                   float softmax_scale, int causal, int window, int dtype, void* stream);

/*
 * flash_attn_bwd_fused: the same gradient from one K/V-stationary kernel that
 * also produces dQ -- every work-group adds its 128 keys' share s * dS K into
 * a float32 accumulator [B, Hq, L, d] in the workspace with atomics, and a
 * last kernel rounds the accumulator to dQ -- so S and dP are formed once
 * instead of twice (claspmoon.cn "14 · 缩放定律与高效注意力" §3.3: the
 * backward recomputes the attention matrix once).  dK and dV equal
 * flash_attn_bwd's bit for bit; dQ is summed in an order that varies from run
 * to run, so it matches to float32 rounding, not bitwise.  On MI355X the
 * float32 atomics make it slower than flash_attn_bwd; it is kept for callers
 * that want the single-kernel form and for the comparison.
 *   workspace, workspace_bytes : at least flash_attn_bwd_fused_workspace_bytes()
 *                                bytes, 256-byte aligned: the row statistics,
 *                                then the accumulator (4*B*Hq*L*d bytes)
 * Requires L * d * 4 < 2^32 (one query head of the accumulator is addressed
 * with 32-bit offsets), else FA_ERR_UNSUPPORTED; the workspace size function
 * then returns 0.  Other arguments and return codes as flash_attn_bwd.
 */
size_t flash_attn_bwd_fused_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int dtype);
int flash_attn_bwd_fused(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes,
                         int B, int Hq, int Hkv, int L, int d,
                         float softmax_scale, int causal, int window, int dtype, void* stream);

/*
 * The backward in three stages, for callers that schedule them (for example
 * dK/dV and dQ on two streams).  flash_attn_bwd runs exactly these three in
 * order on one stream.  Arguments mean what they mean for flash_attn_bwd.
 *
 * Stage 1, flash_attn_bwd_preprocess: from O, the forward's LSE and dO, writes
 * into the workspace the per-row -D_i = -sum_c dO_ic * O_ic and LSE_i * log2(e)
 * (the statistics the recomputation needs, claspmoon.cn §3.3).  Stages 2 and
 * 3 read only those from the workspace and may run in either order or
 * concurrently once stage 1 has completed:
 *   flash_attn_bwd_dkdv -- dK and dV (K/V-stationary; GQA groups summed)
 *   flash_attn_bwd_dq   -- dQ (Q-stationary)
 * Same validation and return codes as flash_attn_bwd.
 */
int flash_attn_bwd_preprocess(const void* o, const float* lse, const void* dout,
                              void* workspace, size_t workspace_bytes,
                              int B, int Hq, int Hkv, int L, int d, int dtype, void* stream);
int flash_attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                        const void* workspace, size_t workspace_bytes, void* dk, void* dv,
                        int B, int Hq, int Hkv, int L, int d,
                        float softmax_scale, int causal, int window, int dtype, void* stream);
int flash_attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                      const void* workspace, size_t workspace_bytes, void* dq,
                      int B, int Hq, int Hkv, int L, int d,
                      float softmax_scale, int causal, int window, int dtype, void* stream);

/*
 * Chunk pairs for sequence parallelism (ring attention, claspmoon.cn "14 ·
 * 缩放定律与高效注意力" §5.1: exact tiled attention extended across devices by
 * splitting the sequence).  A query chunk holds the Lq queries at sequence
 * positions q_offset .. q_offset + Lq - 1, a key/value chunk the Lk keys at
 * k_offset .. k_offset + Lk - 1; causal and window masks are decided on those
 * positions.  Layouts are the ones above with L replaced by Lq for Q, O, dO,
 * dQ, LSE and by Lk for K, V, dK, dV.  16-bit dtypes only (FA_DTYPE_F32
 * returns FA_ERR_UNSUPPORTED); 0 <= q_offset, k_offset <= 2^29 and
 * 1 <= Lq, Lk <= 2^23, else FA_ERR_INVALID_ARG.
 *
 * flash_attn_fwd_block: attention of the query chunk to this key/value chunk
 * only -- O normalised over the chunk's allowed keys and LSE their natural
 * log-sum-exp (the partial result of one ring step).  A row with no allowed
 * key in the chunk gets O = 0 and LSE = -inf.  With Lq = Lk and equal offsets
 * it is flash_attn_fwd.
 */
int flash_attn_fwd_block(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int Lq, int Lk, int d, float softmax_scale,
                         int causal, int window, int q_offset, int k_offset, int dtype, void* stream);

/*
 * flash_attn_merge: exact combination of two partial results over disjoint
 * key sets (the online-softmax rescaling of transformer.xph.ink "高效注意力：
 * FlashAttention 与线性注意力", 原理与机制, applied to whole chunks):
 *   LSE = log(exp(LSE_a) + exp(LSE_b)),
 *   O   = exp(LSE_a - LSE) * O_a + exp(LSE_b - LSE) * O_b;
 * a side with LSE = -inf has weight 0, both -inf give O = 0, LSE = -inf.
 *   o_a, o_b, o [B,Hq,L,d] (dtype: any of the three), lse_a, lse_b, lse
 *   [B,Hq,L] float32.  o may be o_a and lse may be lse_a (accumulation in
 *   place); no other aliasing.  HBM-bound elementwise kernel, no workspace.
 */
int flash_attn_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                     void* o, float* lse, int B, int Hq, int L, int d, int dtype, void* stream);

/*
 * flash_attn_bwd_block: this chunk pair's share of the gradient.  o and lse
 * are the query rows' results over ALL key chunks (after every merge), dout
 * their upstream gradient; the chunk's probabilities are recomputed as
 * exp(s*q.k - LSE) on its allowed keys.  Writes (does not accumulate) dq
 * [B,Hq,Lq,d] = this key chunk's contribution to dQ, and dk, dv [B,Hkv,Lk,d]
 * = this query chunk's contribution to dK, dV; summing over the chunk pairs
 * gives the full gradient.  The workspace is the one flash_attn_bwd needs for
 * Lq query rows (flash_attn_bwd_workspace_bytes(B, Hq, Hkv, Lq, d, dtype)).
 */
int flash_attn_bwd_block(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes,
                         int B, int Hq, int Hkv, int Lq, int Lk, int d, float softmax_scale,
                         int causal, int window, int q_offset, int k_offset, int dtype, void* stream);

/*
 * KV-cache decode (book.anysome.cn "高效注意力" §1: autoregressive generation
 * caches every earlier token's K and V; §3: the G = Hq/Hkv query heads of a
 * group share one K/V head).  The Lq newest tokens of each sequence attend to
 * its cache:
 *   q [B,Hq,Lq,d]                    : the new tokens' queries (dtype)
 *   k_cache, v_cache [B,Hkv,Lk,d]    : the cache (dtype), the new tokens' K/V
 *                                      already written at its end
 *   cache_len [B] int32 (device)     : valid entries per sequence, Lq <= n <=
 *                                      Lk; NULL means every sequence has Lk.
 *                                      Entries past n are never read.  An
 *                                      out-of-range entry is clamped into
 *                                      [Lq, Lk] (results then are meaningless
 *                                      but every access stays in bounds).
 *   o [B,Hq,Lq,d] (dtype), lse [B,Hq,Lq] float32 (may be NULL)
 * New token t of sequence b sits at position n_b - Lq + t (bottom-right
 * alignment): causal = 1 lets it see entries 0 .. that position (window w:
 * the last w of them); causal = 0 lets every new token see all n_b entries.
 * (A rolling window buffer has its own call, flash_attn_decode_rolling; for a
 * single new token it can also be served here with causal = 0 and cache_len =
 * the number of filled slots, since the slot order then does not matter.)
 * The keys are split across work-groups and the partials merged exactly; the
 * cache is read once per K/V head for every 128 rows of R = (Hq/Hkv) * Lq
 * (query heads times new tokens), so R <= 128 reads it once.  For long chunks
 * of new tokens flash_attn_fwd_block is the faster call.
 * A window needs causal = 1 here (FA_ERR_UNSUPPORTED otherwise).
 * Requires 1 <= Lq <= Lk <= 2^23, d in {64,128}, bf16 or fp16, B * Hkv <=
 * 65535, ceil(R / 32) <= 65535 (else FA_ERR_UNSUPPORTED) and B * Hq * Lq <
 * 2^30.  workspace: at least flash_attn_decode_workspace_bytes() bytes,
 * 256-byte aligned (float32 partials of every key split).
 */
size_t flash_attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lk, int d, int dtype);
int flash_attn_decode(const void* q, const void* k_cache, const void* v_cache, const int* cache_len,
                      void* o, float* lse, void* workspace, size_t workspace_bytes,
                      int B, int Hq, int Hkv, int Lq, int Lk, int d, float softmax_scale,
                      int causal, int window, int dtype, void* stream);

/*
 * Decode over a rolling window buffer (transformer.xph.ink "高效注意力：
 * FlashAttention 与线性注意力", 实例或案例: Mistral's sliding window keeps only
 * the last W keys, in a ring of W slots, so the cache stays a fixed size).
 *   q [B,Hq,Lq,d]                    : the new tokens' queries (dtype)
 *   k_ring, v_ring [B,Hkv,W,d]       : the buffer: the K/V of position p of
 *                                      sequence b is in slot p mod W; it holds
 *                                      positions max(0, n_b - W) .. n_b - 1
 *   k_new, v_new [B,Hkv,Lq,d]        : the new tokens' own K/V (positions
 *                                      n_b .. n_b + Lq - 1), not yet written
 *                                      to the buffer (the caller writes them to
 *                                      slots (n_b + t) mod W after the call)
 *   seen [B] int32 (device, not NULL): n_b, the tokens of sequence b before
 *                                      this call; clamped into [0, 2^30]
 *   o [B,Hq,Lq,d] (dtype), lse [B,Hq,Lq] float32 (may be NULL)
 *   window                           : w, 1 <= w <= W; 0 means w = W
 * New token t sits at position n_b + t and attends to positions
 * max(0, n_b + t - w + 1) .. n_b + t: the older ones from the buffer (slot
 * order does not matter: each slot's position is known from n_b), the newer
 * ones from k_new / v_new, causally.  The partials of both are merged exactly
 * (log-sum-exp weights), so any Lq and G = Hq/Hkv are exact; the buffer is
 * read once per K/V head for every 128 rows of R = G * Lq.
 * Sizes as for flash_attn_decode with W in place of Lk (Lq may exceed W);
 * window > W is FA_ERR_INVALID_ARG (those keys are gone from the buffer).
 * workspace: at least flash_attn_decode_rolling_workspace_bytes() bytes,
 * 256-byte aligned.
 */
size_t flash_attn_decode_rolling_workspace_bytes(int B, int Hq, int Hkv, int Lq, int W, int d, int dtype);
int flash_attn_decode_rolling(const void* q, const void* k_ring, const void* v_ring, const void* k_new,
                              const void* v_new, const int* seen, void* o, float* lse,
                              void* workspace, size_t workspace_bytes,
                              int B, int Hq, int Hkv, int Lq, int W, int d, float softmax_scale,
                              int window, int dtype, void* stream);

/*
 * General sparse masks over one sequence of L positions (queries and keys are
 * the same positions: self-attention, layouts as for flash_attn_fwd).  Key j
 * is allowed for query i iff
 *   causal_ok(i, j) && ((window_ok(i, j) && block_ok(i, j)) || global(i) || global(j))
 * where
 *   causal_ok  -- j <= i when causal = 1, else always;
 *   window_ok  -- |i - j| < window when window >= 1 (with causal: the w most
 *                 recent keys, book.anysome.cn "高效注意力" §4; without: w - 1
 *                 positions before and after, kler.cn §3.2.1), else always;
 *   block_ok   -- block_mask[i / block][j / block] != 0: block-sparse
 *                 attention over block x block tiles (kler.cn §4.1.2), or
 *                 always when block_mask is NULL;
 *   global(p)  -- p is one of global_pos: a global position attends to and is
 *                 attended by every position, Longformer / BigBird style
 *                 (claspmoon.cn "14 · 缩放定律与高效注意力" §4.3; kler.cn
 *                 §5.1.2: first and last token global, entries 0 and -1).
 * A row with no allowed key gets O = 0 and LSE = -inf (its gradients are 0).
 *
 *   global_pos  : device int32[n_global]; an entry p < 0 means L + p; entries
 *                 outside [-L, L) are ignored; 0 <= n_global <= 65536.
 *   block_mask  : device uint8[nbm * nbm], row-major, nbm = ceil(L / block);
 *                 block a multiple of 64 (else FA_ERR_UNSUPPORTED).  Its
 *                 size is the caller's promise.
 */
typedef struct fa_mask {
  int causal;
  int window;
  const int* global_pos;
  int n_global;
  const unsigned char* block_mask;
  int block;
} fa_mask;

/*
 * flash_attn_mask_plan: classifies every 64 x 64 block of the mask (empty,
 * partial or full) and writes, into the caller's device buffer `plan`, the
 * tile lists, the global positions and the work-group order the masked
 * kernels follow.  Runs four small kernels on `stream`; reads the mask's
 * device arrays there.  Plan contents are clamped when used, so a buffer that
 * never held a plan gives wrong results but no out-of-bounds access.  A plan
 * depends on the mask and L only: build it once and pass it to every masked
 * call (every head, layer, forward and backward) with that same mask and L.
 * 1 <= L <= 2^18 (FA_ERR_UNSUPPORTED above).  plan: at least
 * flash_attn_mask_plan_bytes(L) bytes, 256-byte aligned (else
 * FA_ERR_WORKSPACE).  flash_attn_mask_plan_bytes returns 0 for an
 * unsupported L.
 */
size_t flash_attn_mask_plan_bytes(int L);
int flash_attn_mask_plan(const fa_mask* mask, int L, void* plan, size_t plan_bytes, void* stream);

/*
 * flash_attn_fwd_masked / flash_attn_bwd_masked: flash_attn_fwd and
 * flash_attn_bwd under the mask (16-bit dtypes; FA_DTYPE_F32 returns
 * FA_ERR_UNSUPPORTED).  `mask` supplies causal, window and the number of
 * global entries to the call; the global positions themselves and the block
 * mask are read from the plan, which must have been built from this mask and
 * this L (a plan for another mask gives that mask's result).  Tiles the mask
 * leaves empty are never loaded, so the work scales with the allowed pairs.
 * Global positions are whole rows and columns of the mask: split passes over
 * the sequence compute them, with float32 partials in the workspace.
 *
 * workspace: at least flash_attn_masked_workspace_bytes(..., backward) bytes,
 * 256-byte aligned (else FA_ERR_WORKSPACE).  The forward needs none (NULL is
 * accepted) when n_global is 0; the backward always needs flash_attn_bwd's
 * per-row statistics and this size includes them.  With global positions,
 * B * Hq must be at most 65535 (else FA_ERR_UNSUPPORTED).
 */
size_t flash_attn_masked_workspace_bytes(int B, int Hq, int Hkv, int L, int d, const fa_mask* mask,
                                         int backward);
int flash_attn_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                          void* workspace, size_t workspace_bytes,
                          int B, int Hq, int Hkv, int L, int d, float softmax_scale,
                          const fa_mask* mask, const void* plan, size_t plan_bytes, int dtype, void* stream);
int flash_attn_bwd_masked(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv,
                          void* workspace, size_t workspace_bytes,
                          int B, int Hq, int Hkv, int L, int d, float softmax_scale,
                          const fa_mask* mask, const void* plan, size_t plan_bytes, int dtype, void* stream);

/*
 * flash_attn_bwd_noalloc: flash_attn_bwd without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  It runs the three
 * staged kernels of flash_attn_bwd_preprocess / _dkdv / _dq, with the per-row
 * statistics (-D_i and LSE_i * log2 e, two float32 per query row) in a static
 * device array of 16 MiB that the library owns: B * Hq * L must be at most
 * FA_NOALLOC_MAX_ROWS (2^21), else FA_ERR_TOO_LARGE.  The call allocates
 * nothing and calls no allocating routine.  Each GPU has its own copy of the
 * array, looked up on the first call on that device; `stream` must belong to
 * the current device (else FA_ERR_INVALID_ARG).  Every call on one GPU shares
 * that GPU's array, which keeps the last call's contents (every row used is
 * rewritten before it is read, so nothing needs clearing): calls that overlap
 * in time on one GPU (on different streams, or from different threads) race
 * and give wrong results -- serialise them.  Other arguments and return codes
 * as flash_attn_bwd.
 */
#define FA_NOALLOC_MAX_ROWS 2097152  /* 2^21 query rows */
int flash_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv,
                           int B, int Hq, int Hkv, int L, int d,
                           float softmax_scale, int causal, int window, int dtype, void* stream);

/* Static, never-NULL description of a return code. */
const char* flash_attn_strerror(int code);

/* Library ABI version (major*10000 + minor*100 + patch). */
int flash_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASH_ATTN_MI355_H */
