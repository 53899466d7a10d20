// fa_masked.hip -- exact attention under general sparse masks, driven by a
// mask plan (gfx950).
//
// The mask family: a sliding window (one-sided with causal masking, else
// reaching both ways), a block-sparse pattern over b x b blocks, and global
// positions that see and are seen by every position, all under an optional
// causal mask (claspmoon.cn "14 · 缩放定律与高效注意力" §4.3: Longformer /
// BigBird combine a local window with a few global tokens; kler.cn
// "大模型高效注意力机制全解析" §4.1.2: block-sparse attention over b x b blocks,
// §3.2.1 and §5.1.2: a window of positions before and after, the first and
// last token global).  The masked positions are exactly excluded, so the
// result is exact attention over the allowed pairs.
//
// 1. Plan (four small kernels, once per mask and length; reused by every
//    head, layer and by the backward): the global positions become a bitmap
//    and a sorted list, every 64 x 64 block of the L x L mask is classified as
//    empty, partial or full from interval arithmetic on its corners, and
//    every work-group row (128 queries) and column (128 keys) gets the
//    compact, ascending list of the 64-wide tiles it must visit, ordered
//    heaviest first.
// 2. Attention: the range-tiled kernels' tile steps, unchanged, iterate over
//    the lists instead of an index range.  Full tiles run unmasked; partial
//    tiles evaluate the mask per element (window, causal, block bit and the
//    global bits of the tile); empty tiles are never loaded.
// 3. Global positions are whole rows and columns of the mask.  The row lists
//    leave global query rows out and the column lists leave global keys out;
//    split passes over the whole sequence compute those rows and keys
//    (section 3 below), so no work-group has to walk a whole row.  With few
//    global positions the row kernels also take the global keys themselves,
//    from LDS after their tiles, instead of visiting the tiles holding them
//    (kFoldGlobals).
#include "fa_bwd_tile.hpp"
#include "fa_fwd_tile.hpp"

namespace fa {

PlanLayout plan_layout(int L) {
  PlanLayout y{};
  y.L = L;
  y.nb = (L + 63) / 64;
  y.nw = (L + 127) / 128;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = (off + bytes + 255) & ~(size_t)255;
    return at;
  };
  y.gbits = take(8 * (size_t)y.nb);
  y.row_cnt = take(4 * (size_t)y.nw);
  y.row_ord = take(4 * (size_t)y.nw);
  y.col_cnt = take(4 * (size_t)y.nw);
  y.col_ord = take(4 * (size_t)y.nw);
  y.meta = take(16);
  y.gpos = take(4 * (size_t)L);
  y.row_ent = take(4 * (size_t)y.nw * y.nb);
  y.col_ent = take(4 * (size_t)y.nw * y.nb);
  y.total = off;
  return y;
}

PlanPtrs plan_ptrs(const void* plan, int L) {
  const PlanLayout y = plan_layout(L);
  const char* b = static_cast<const char*>(plan);
  PlanPtrs p{};
  p.gbits = reinterpret_cast<const unsigned long long*>(b + y.gbits);
  p.row_cnt = reinterpret_cast<const int*>(b + y.row_cnt);
  p.row_ord = reinterpret_cast<const int*>(b + y.row_ord);
  p.row_ent = reinterpret_cast<const unsigned*>(b + y.row_ent);
  p.col_cnt = reinterpret_cast<const int*>(b + y.col_cnt);
  p.col_ord = reinterpret_cast<const int*>(b + y.col_ord);
  p.col_ent = reinterpret_cast<const unsigned*>(b + y.col_ent);
  p.meta = reinterpret_cast<const int*>(b + y.meta);
  p.gpos = reinterpret_cast<const int*>(b + y.gpos);
  p.nb = y.nb;
  p.nw = y.nw;
  return p;
}

namespace {

// ------------------------------------------------------------ 1. plan

// Global keys folded into the row kernels: with at most kFoldGlobals global
// positions, the forward and dQ kernels take every row's global keys before
// their first tile, straight from the keys' rows in HBM (fold_keys_fwd,
// fold_keys_dq), instead of visiting the key tiles that hold them (a whole
// tile for one key, on every work-group row).  The row lists then leave those
// tiles out unless the window or the blocks reach them, and such tiles mask
// the global keys out.  The count comes from the plan (meta[2], the distinct
// global positions), so the plan and the kernels always agree.
constexpr int kFoldGlobals = 8;
__device__ __forceinline__ int fold_count(const int* meta, int L) {
  const int n = min(max(meta[2], 0), L);
  return n <= kFoldGlobals ? n : 0;
}

struct PlanBuild {
  MaskDesc m;
  int L, nb, nw, nbm;
  unsigned long long* gbits;
  int* row_cnt;
  int* row_ord;
  unsigned* row_ent;
  int* col_cnt;
  int* col_ord;
  unsigned* col_ent;
  int* meta;
  int* gpos;
};

// One thread per 64-block: the bitmap word of the global positions in it.
__global__ __launch_bounds__(256) void plan_gbits_kernel(PlanBuild p) {
  const int blk = blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= p.nb) return;
  unsigned long long w = 0;
  for (int n = 0; n < p.m.n_global; ++n) {
    int pos = p.m.global_pos[n];
    if (pos < 0) pos += p.L;
    if (pos >= 0 && pos < p.L && (pos >> 6) == blk) w |= 1ull << (pos & 63);
  }
  p.gbits[blk] = w;
}

// One work-group: the global positions in ascending order (from the bitmap,
// so each appears once) and their count in meta[2].
__global__ __launch_bounds__(1024) void plan_gpos_kernel(PlanBuild p) {
  __shared__ int wave_tot[16];
  int base = 0;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int x0 = 0; x0 < p.nb; x0 += 1024) {
    const int x = x0 + tid;
    const unsigned long long w = x < p.nb ? p.gbits[x] : 0ull;
    const int n = __popcll(w);
    // exclusive prefix of n over the work-group: within the wave, then across waves
    int incl = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    if (lane == 63) wave_tot[wv] = incl;
    __syncthreads();
    int at = base + incl - n;
    for (int k = 0; k < wv; ++k) at += wave_tot[k];
    unsigned long long rest = w;
    while (rest != 0ull) {
      const int b = __builtin_ctzll(rest);
      p.gpos[at++] = 64 * x + b;
      rest &= rest - 1ull;
    }
    for (int k = 0; k < 16; ++k) base += wave_tot[k];
    __syncthreads();
  }
  if (tid == 0) p.meta[2] = base;
}

// Class of the 64 x 64 block (query block qb, key block kb): 0 when no pair
// is allowed, 2 when every pair is (and the block lies inside the sequence),
// else 1.  Empty and full are decided exactly from the block's extreme
// positions; anything undecided is partial, which only costs the per-element
// mask.  block_ok is the block-sparse bit of the block.  Global queries (keys)
// count only when use_gq (use_gk) is set: a global query row sees every key,
// so the row lists leave it to the global-row pass instead of visiting every
// tile; likewise the column lists leave global keys to the global-key pass.
// excl_gk: global keys are folded into the row kernels (fold_count), so a
// block holding one is never full (the tile masks it out).
__device__ int block_class(const PlanBuild& p, int qb, int kb, bool use_gq, bool use_gk, bool excl_gk,
                           int& block_ok) {
  block_ok = 0;
  if (qb >= p.nb || kb >= p.nb) return 0;
  const int i0 = 64 * qb, i1 = min(i0 + 63, p.L - 1);
  const int j0 = 64 * kb, j1 = min(j0 + 63, p.L - 1);
  const bool inside = i0 + 63 < p.L && j0 + 63 < p.L;
  const bool c_all = !p.m.causal || j1 <= i0;
  const bool c_none = p.m.causal && j0 > i1;
  bool w_all = true, w_none = false;
  if (p.m.window > 0) {
    const int far = max(i1 - j0, j1 - i0);                              // largest |i - j|
    const int near = j0 > i1 ? j0 - i1 : (i0 > j1 ? i0 - j1 : 0);        // smallest |i - j|
    w_all = far < p.m.window;
    w_none = near >= p.m.window;
  }
  const bool bm = p.m.block_mask == nullptr ||
                  p.m.block_mask[(size_t)(i0 / p.m.block) * p.nbm + j0 / p.m.block] != 0;
  block_ok = bm ? 1 : 0;
  const bool glob = (use_gq && p.gbits[qb] != 0) || (use_gk && p.gbits[kb] != 0);
  if (c_none || ((w_none || !bm) && !glob)) return 0;
  return (inside && c_all && w_all && bm && !(excl_gk && p.gbits[kb] != 0)) ? 2 : 1;
}

// One work-group per work-group row (blockIdx.y == 0: 128 queries against
// every 64-key tile) or column (blockIdx.y == 1: 128 keys against every
// 64-query tile); the non-empty tiles are compacted in ascending order.
__global__ __launch_bounds__(256) void plan_lists_kernel(PlanBuild p) {
  __shared__ int wave_tot[4];
  const int w = blockIdx.x;
  const bool cols = blockIdx.y == 1;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  unsigned* ent = (cols ? p.col_ent : p.row_ent) + (size_t)w * p.nb;
  const bool fold = fold_count(p.meta, p.L) > 0;
  int base = 0;
  for (int x0 = 0; x0 < p.nb; x0 += 256) {
    const int x = x0 + tid;
    unsigned e = 0;
    bool keep = false;
    if (x < p.nb) {
      int bm0, bm1;
      const int c0 = cols ? block_class(p, x, 2 * w, true, false, false, bm0)
                          : block_class(p, 2 * w, x, false, !fold, fold, bm0);
      const int c1 = cols ? block_class(p, x, 2 * w + 1, true, false, false, bm1)
                          : block_class(p, 2 * w + 1, x, false, !fold, fold, bm1);
      keep = (c0 | c1) != 0;
      e = (unsigned)x | ((unsigned)c0 << 16) | ((unsigned)c1 << 18) | ((unsigned)bm0 << 20) | ((unsigned)bm1 << 21) |
          ((unsigned)(p.gbits[x] != 0ull) << 22);
    }
    const unsigned long long bal = __ballot(keep);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wv] = __popcll(bal);
    __syncthreads();
    int at = base;
    for (int k = 0; k < wv; ++k) at += wave_tot[k];
    if (keep) ent[at + before] = e;
    base += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    __syncthreads();
  }
  if (tid == 0) (cols ? p.col_cnt : p.row_cnt)[w] = base;
}

constexpr int kMaxOrder = 2048;   // work-group rows a plan can order (L <= 2^18)

// One work-group: work-group rows (then columns) sorted by descending entry
// count (ties by index), bitonic sort in LDS; the leading ranks whose count
// exceeds twice the median (plus a margin) are marked heavy.
__global__ __launch_bounds__(1024) void plan_order_kernel(PlanBuild p) {
  __shared__ unsigned key[kMaxOrder];
  for (int which = 0; which < 2; ++which) {
    const int* cnt = which ? p.col_cnt : p.row_cnt;
    int* ord = which ? p.col_ord : p.row_ord;
    for (int i = threadIdx.x; i < kMaxOrder; i += blockDim.x)
      key[i] = i < p.nw ? (((unsigned)cnt[i] << 12) | (4095u - (unsigned)i)) : 0u;
    __syncthreads();
    for (int k = 2; k <= kMaxOrder; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = threadIdx.x; i < kMaxOrder; i += blockDim.x) {
          const int l = i ^ j;
          if (l > i) {
            const unsigned a = key[i], b = key[l];
            const bool desc = (i & k) == 0;
            if (desc ? a < b : a > b) {
              key[i] = b;
              key[l] = a;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int r = threadIdx.x; r < p.nw; r += blockDim.x) ord[r] = 4095 - (int)(key[r] & 4095u);
    if (threadIdx.x == 0) {
      const unsigned med = key[p.nw / 2] >> 12;
      int h = 0;
      while (h < p.nw && (key[h] >> 12) > 2 * med + 8) ++h;
      p.meta[which] = h;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------ 2. attention

// Logical work-group -> (head, work-group row or column): the heavy ranks of
// every head first (rank-major), then the rest head by head in rank order.
// Values read from the plan are clamped into range, so that even a buffer that
// never held a plan keeps every access inside its arrays.
__device__ __forceinline__ void plan_wg(int r, int n_heads, int nw, int n_heavy_raw, const int* ord, int& head,
                                        int& tile) {
  const int n_heavy = min(max(n_heavy_raw, 0), nw / 2);
  const int heavy = n_heavy * n_heads;
  int rank;
  if (r < heavy) {
    rank = r / n_heads;
    head = r - rank * n_heads;
  } else {
    const int rr = r - heavy, per = nw - n_heavy;
    head = rr / per;
    rank = n_heavy + (rr - head * per);
  }
  tile = min(max(__builtin_amdgcn_readfirstlane(ord[rank]), 0), nw - 1);
}

// Query-major element mask: the lane's query i is fixed; k0 is the tile's
// first key, gk the global bits of its 64 keys, gq whether i is global, bm
// the block-sparse bit of the lane's 64 x 64 block.  excl: the global keys
// are folded into the row's initial state (fold_keys_*), so the tile leaves
// them out instead.
template <bool CAUSAL>
struct GeneralMaskQ {
  int L, window, i, k0;
  bool gq, bm;
  unsigned long long gk;
  bool excl;
  // bitwise, not short-circuit, so that no divergent branch is formed
  __device__ __forceinline__ bool operator()(int j) const {
    const bool gbit = ((gk >> (j - k0)) & 1ull) != 0;
    const bool local = bm & ((window <= 0) | ((j > i - window) & (j < i + window))) & !(excl & gbit);
    const bool glob = gq | (!excl & gbit);
    return (j < L) & (!CAUSAL | (j <= i)) & (local | glob);
  }
};

// Key-major element mask: the lane's key j is fixed; q0 is the tile's first
// query, gq the global bits of its 64 queries, gk whether j is global.
template <bool CAUSAL>
struct GeneralMaskK {
  int L, window, j, q0;
  bool gk, bm;
  unsigned long long gq;
  __device__ __forceinline__ bool operator()(int q) const {
    const bool local = bm & ((window <= 0) | ((j > q - window) & (j < q + window)));
    const bool glob = gk | (((gq >> (q - q0)) & 1ull) != 0);
    return (q < L) & (!CAUSAL | (j <= q)) & (local | glob);
  }
};

__device__ __forceinline__ bool is_global(const unsigned long long* gbits, int pos, int L) {
  return pos < L && ((gbits[pos >> 6] >> (pos & 63)) & 1ull) != 0;
}

// ---- global keys folded into the row kernels (fold_count > 0)
// With the work-group's first tile copies, its waves copy the n_g global
// keys' K and V rows into an LDS area of their own (kGlobalRowsBytes) with
// the direct buffer -> LDS copies, so the first tile's wait covers them: row
// t of K at t * 2D bytes, row t of V at (kFoldGlobals + t) * 2D, 16 bytes per
// lane, thread i = 64 wave + lane taking row i / (D/8), chunk i % (D/8); a
// wave's rows are all K or all V, so its resource is uniform.  Rows past n_g
// repeat the first global position (never read).  The global positions come
// through the scalar path (plan memory is read-only here).
template <int D>
constexpr int kGlobalRowsBytes = 2 * kFoldGlobals * 2 * D;
template <int D>
__device__ __forceinline__ void stage_global_rows(char* lds, __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                                  const int* gpos, int n_g, int L, int wave, int lane) {
  constexpr int CH = D / 8;                          // 16-byte chunks per row
  constexpr int kWavesUsed = (2 * kFoldGlobals * CH) / 64;
  static_assert((2 * kFoldGlobals * CH) % 64 == 0 && kWavesUsed <= 4, "rows of one wave must be all K or all V");
  if (wave >= kWavesUsed) return;
  typedef const __attribute__((address_space(4))) int* cptr;
  const int t = wave * 64 + lane;
  const int r = t / CH, chunk = t % CH;
  const int row = r % kFoldGlobals;
  int pos = ((cptr)gpos)[0];
#pragma unroll
  for (int i = 1; i < kFoldGlobals; ++i)
    if (i < n_g) pos = row == i ? ((cptr)gpos)[i] : pos;
  pos = min(max(pos, 0), L - 1);
  const bool is_v = wave * 64 >= kFoldGlobals * CH;
  buf2lds16(is_v ? vrs : krs, pos * (2 * D) + 16 * chunk, 0, lds + wave * 1024);
}

// The lane holds its query's head dims 16k + 8g .. +7 (the MFMA B-operand
// layout of the Q and dO registers): half a dot product with an LDS row,
// completed with the partner lane (lane ^ 32), which holds the other half.
template <int D, bool F16>
__device__ __forceinline__ float row_dot(const bf16x8 (&x)[D / 16], const char* row, int g) {
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < D / 16; ++k) {
    const bf16x8 y = lds_load16(row, 32 * k + 16 * g);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(unpack1<F16>(x[k][e]), unpack1<F16>(y[e]), acc);
  }
  return pair_sum(acc);
}

// acc += f * an LDS row, over the lane's elements of an accumulator in the
// MFMA C layout with lane = query (block db, register i: head dim 32db +
// 8(i/4) + 4g + i%4).
template <int D, bool F16>
__device__ __forceinline__ void row_axpy(f32x16 (&acc)[D / 32], float f, const char* row, int g) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const bf16x4 y = *(const FA_LDS bf16x4*)((const FA_LDS char*)row + 64 * db + 16 * i4 + 8 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[db][4 * i4 + e] = fmaf(f, unpack1<F16>(y[e]), acc[db][4 * i4 + e]);
    }
}

// Forward: the row's global keys (all n_g of them, or those at or before the
// row when causal) taken into the online-softmax state after its tiles, one
// key at a time like a tile of one key (the order does not change the
// softmax); P stays in float32 here.  lds: the staged rows (read after the
// tiles, when the tile loop's registers are free).
template <int D, bool CAUSAL, bool F16>
__device__ __forceinline__ void fold_keys_fwd(fwdtile::FwdState<D>& st, const char* lds, const int* gpos, int n_g,
                                              int L, int my_q, float c, int g) {
  typedef const __attribute__((address_space(4))) int* cptr;
#pragma unroll 1
  for (int t = 0; t < n_g; ++t) {
    const int pg = ((cptr)gpos)[t];
    const float x = row_dot<D, F16>(st.qr, lds + t * (2 * D), g) * c;
    if (!CAUSAL || pg <= my_q) {
      if (x > st.m_run) {
        const float alpha = fast_exp2(st.m_run - x);
        st.l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) st.o[db] *= alpha;
        st.m_run = x;
      }
      const float pt = fast_exp2(x - st.m_run);
      if (g == 0) st.l_run += pt;   // the row sum is the two lanes' sum
      row_axpy<D, F16>(st.o, pt, lds + (kFoldGlobals + t) * (2 * D), g);
    }
  }
}

// dQ: the row's global keys' terms of dQ = sum_j dS_ij K_j (scaled at the
// end like the rest), dS_ij = P_ij (dP_ij - D_i), P_ij = exp2(S_ij c - LSE_i
// log2 e), dP_ij = dO_i . V_j (the chain from -D_i); dS stays in float32.
// After the row's tiles, from the staged rows, as in the forward.
template <int D, bool CAUSAL, bool F16>
__device__ __forceinline__ void fold_keys_dq(bwdtile::QState<D>& st, const char* lds, const int* gpos, int n_g,
                                             int L, int my_q, float c, int g) {
  typedef const __attribute__((address_space(4))) int* cptr;
#pragma unroll 1
  for (int t = 0; t < n_g; ++t) {
    const int pg = ((cptr)gpos)[t];
    const char* krow = lds + t * (2 * D);
    const float sc = row_dot<D, F16>(st.qr, krow, g);
    const float dp = row_dot<D, F16>(st.dor, lds + (kFoldGlobals + t) * (2 * D), g) + st.negd[0];
    const float pt = fast_exp2(fmaf(sc, c, -st.lse2));
    const float ds = (!CAUSAL || pg <= my_q) ? pt * dp : 0.f;
    row_axpy<D, F16>(st.dq, ds, krow, g);
  }
}

// entry fields (the tile index is clamped by the caller's list length)
__device__ __forceinline__ int ent_tile(unsigned e, int nb) { return min((int)(e & 0xffffu), nb - 1); }
__device__ __forceinline__ int ent_class(unsigned e, int half) { return (int)((e >> (16 + 2 * half)) & 3u); }
__device__ __forceinline__ bool ent_block(unsigned e, int half) { return ((e >> (20 + half)) & 1u) != 0; }
// Does the listed tile hold a global position?  Only then do the kernels read
// the tile's global bits (plan_word).
__device__ __forceinline__ bool ent_glob(unsigned e) { return ((e >> 22) & 1u) != 0; }

// A word of the plan at a wave-uniform index, read through the constant
// address space (the attention kernels never write the plan), i.e. a scalar
// load into scalar registers.  A vector load would be waited for with the
// vector-memory counter, which also counts the next tile's copies issued just
// before: where its register is reused after a branch, the wait is for all of
// them, on every tile.
__device__ __forceinline__ unsigned long long plan_word(const unsigned long long* a, int i) {
  typedef const __attribute__((address_space(4))) unsigned long long* cptr;
  return ((cptr)a)[i];
}

// A zero the compiler cannot see through.
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// A work-group's list, read two tiles ahead through the vector memory path:
// the load is issued with the tile copies, so the copies' own wait covers it,
// and readfirstlane returns the (uniform) entry to scalar registers.  A scalar
// load of the next entry would instead hold up the next tile's copies by its
// latency on every tile.  Entries past the list read as 0.
struct EntryStream {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ unsigned fetch(int e) const {
    return __builtin_amdgcn_raw_buffer_load_b32(r, opaque_zero(), 4 * e, 0);
  }
};
__device__ __forceinline__ unsigned uniform(unsigned v) { return __builtin_amdgcn_readfirstlane(v); }

// Forward: one work-group of 4 waves per (batch, query head, 128 queries), as
// the range-tiled forward; waves 0-1 hold the first 64 rows, 2-3 the second.
template <int D, bool CAUSAL, bool F16>
__global__ __launch_bounds__(256, 2) void fwd_masked_kernel(FwdArgs a, PlanPtrs p) {
  using namespace fwdtile;
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) char k_st0[C::KT];
  __shared__ __attribute__((aligned(1024))) char v_st0[C::VT];
  __shared__ __attribute__((aligned(1024))) char k_st1[C::KT];
  __shared__ __attribute__((aligned(1024))) char v_st1[C::VT];
  __shared__ __attribute__((aligned(1024))) char g_rows[kGlobalRowsBytes<D>];

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int g = lane >> 5, ln = lane & 31;
  const int half = wave >> 1;
  const int L = a.L, window = a.window;

  int bh, qt;
  plan_wg(xcd_remap(blockIdx.x, gridDim.x), a.B * a.Hq, p.nw, p.meta[0], p.row_ord, bh, qt);
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const bf16* __restrict__ Qh = reinterpret_cast<const bf16*>(a.q) + ((size_t)(b * a.Hq + h) * L) * D;
  const size_t kv_off = ((size_t)(b * a.Hkv + hk) * L) * D;
  const unsigned head_bytes = (unsigned)L * (2 * D);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(reinterpret_cast<const bf16*>(a.k) + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(reinterpret_cast<const bf16*>(a.v) + kv_off, head_bytes);

  const int q_wg0 = qt * C::BR;
  const int q_w0 = q_wg0 + 32 * wave;
  const int my_q = q_w0 + ln;
  const int n_ent = min(max(__builtin_amdgcn_readfirstlane(p.row_cnt[qt]), 0), p.nb);
  const unsigned* ents = p.row_ent + (size_t)qt * p.nb;
  const bool gq = is_global(p.gbits, my_q, L);

  const EntryStream es{make_rsrc(ents, 4u * (unsigned)n_ent)};
  unsigned cur = n_ent > 0 ? ents[0] : 0u, nxt = n_ent > 1 ? ents[1] : 0u;
  CopyPlan<D> cp;
  make_copy_plan<D>(cp, wave, lane);
  if (n_ent > 0) issue_kv<D>(cp, krs, vrs, ent_tile(cur, p.nb) * C::BC, k_st0, v_st0, wave);
  const int n_fold = fold_count(p.meta, L);
  if (n_fold > 0) stage_global_rows<D>(g_rows, krs, vrs, p.gpos, n_fold, L, wave, lane);

  FwdState<D> st;
#pragma unroll
  for (int k = 0; k < C::NSTEP; ++k) {
    if (my_q < L) st.qr[k] = *reinterpret_cast<const bf16x8*>(Qh + (size_t)my_q * D + 16 * k + 8 * g);
    else st.qr[k] = bf16x8{};
  }
  st.m_run = kNegBig;
  st.l_run = 0.f;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) st.o[db] = f32x16{};
  const float c = a.scale_log2;

  auto step = [&](unsigned ent, const char* kb, const char* vb) {
    const int cls = ent_class(ent, half);
    if (cls != 0 && q_w0 < L) {
      const int kt = ent_tile(ent, p.nb);
      const bool tg = (cls == 1) & ent_glob(ent);
      const unsigned long long gk = tg ? plan_word(p.gbits, kt) : 0ull;
      const bool bm = ent_block(ent, half);
      // without a global key in the tile and with the block allowed, the
      // window and causal range alone decide (a global row's own output is
      // not stored here): the range kernels' cheaper element test
      const EitherMask<RangeMaskQ<CAUSAL>, GeneralMaskQ<CAUSAL>> ok{
          (bool)(!tg & bm), RangeMaskQ<CAUSAL>{L, window, my_q},
          GeneralMaskQ<CAUSAL>{L, window, my_q, kt * C::BC, gq, bm, gk, n_fold > 0}};
      fwd_tile<D, F16>(st, kb, vb, kt * C::BC, cls == 1, ok, c, lane);
    }
  };

  // stage 0 holds tile e (entry cur), stage 1 receives tile e + 1 (entry nxt)
  wait_copies_and_barrier();
  for (int e = 0; e < n_ent; e += 2) {
    const unsigned far0 = es.fetch(e + 2);
    if (e + 1 < n_ent) issue_kv<D>(cp, krs, vrs, ent_tile(nxt, p.nb) * C::BC, k_st1, v_st1, wave);
    step(cur, k_st0, v_st0);
    wait_copies_and_barrier();
    if (e + 1 >= n_ent) break;
    cur = nxt;
    nxt = uniform(far0);
    const unsigned far1 = es.fetch(e + 3);
    if (e + 2 < n_ent) issue_kv<D>(cp, krs, vrs, ent_tile(nxt, p.nb) * C::BC, k_st0, v_st0, wave);
    step(cur, k_st1, v_st1);
    wait_copies_and_barrier();
    cur = nxt;
    nxt = uniform(far1);
  }

  if (n_fold > 0 && q_w0 < L) fold_keys_fwd<D, CAUSAL, F16>(st, g_rows, p.gpos, n_fold, L, my_q, c, g);

  // epilogue: a row with no allowed key gets O = 0, LSE = -inf; a global row
  // is left to the global-row pass
  const float l_tot = pair_sum(st.l_run);
  if (my_q < L && !gq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    bf16* Oq = reinterpret_cast<bf16*>(a.o) + ((size_t)(b * a.Hq + h) * L + my_q) * D;
    store_row_c<F16, C::NDB>(Oq, st.o, inv, g);
    if (a.lse != nullptr && g == 0)
      a.lse[(size_t)(b * a.Hq + h) * L + my_q] = l_tot > 0.f ? (st.m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// dK/dV: one work-group of 8 waves per (batch, K/V head, 128 keys), as the
// range-tiled kernel, streaming the query tiles of its column list for every
// query head of the group.
template <int D, bool CAUSAL, bool F16>
__global__ __launch_bounds__(512, 1) void dkdv_masked_kernel(BwdArgs a, PlanPtrs p) {
  using namespace bwdtile;
  using C = KVCfg<D>;
  __shared__ __attribute__((aligned(C::QT))) char q_st0[C::QT];
  __shared__ __attribute__((aligned(C::QT))) char do_st0[C::QT];
  __shared__ __attribute__((aligned(C::QT))) char q_st1[C::QT];
  __shared__ __attribute__((aligned(C::QT))) char do_st1[C::QT];
  __shared__ __attribute__((aligned(1024))) char k_blk[C::KB];
  __shared__ __attribute__((aligned(1024))) char v_blk[C::KB];
  __shared__ __attribute__((aligned(16))) float stat_st0[2 * C::BQ];   // LSE*log2e, then -D
  __shared__ __attribute__((aligned(16))) float stat_st1[2 * C::BQ];

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int g = lane >> 5, ln = lane & 31;
  const int kb = wave & 3, qh = wave >> 2;
  const int half = kb >> 1;                        // which 64-key block of the 128
  const int L = a.L, window = a.window;
  const int G = a.Hq / a.Hkv;

  int bhk, kt;
  plan_wg(xcd_remap(blockIdx.x, gridDim.x), a.B * a.Hkv, p.nw, p.meta[1], p.col_ord, bhk, kt);
  const int b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const int key_wg0 = kt * C::BK;
  const int key_w0 = key_wg0 + 32 * kb;
  const int my_key = key_w0 + ln;

  const size_t kv_off = ((size_t)(b * a.Hkv + hk) * L) * D;
  const unsigned head_bytes = (unsigned)L * (2 * D);

  const int n_ent = min(max(__builtin_amdgcn_readfirstlane(p.col_cnt[kt]), 0), p.nb);
  const unsigned* ents = p.col_ent + (size_t)kt * p.nb;
  const int n_it = G * n_ent;
  const bool gk = is_global(p.gbits, my_key, L);

  KVAddr<D> ad;
#pragma unroll
  for (int i = 0; i < C::QPER; ++i) ad.qcopy[i] = dual_slot_src<D>((wave + C::kWaves * i) * 64 + lane);
#pragma unroll
  for (int k = 0; k < C::NSTEP; ++k) ad.row[k] = row_offset_dual<D>(32 * qh + ln, k, g);
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    ad.tr[db][0] = tr_offset_dual<D>(2 * qh, db, 0, lane);
    ad.tr[db][1] = tr_offset_dual<D>(2 * qh, db, 1, lane);
  }
  ad.kv = row_offset_kpad<D>(32 * kb + ln, 0, g);

  // iteration it visits entry it % n_ent for query head hk*G + it / n_ent
  auto issue = [&](unsigned ent, int hoff, char* qs, char* dos, float* ss) {
    const int hq = hk * G + hoff, q0 = ent_tile(ent, p.nb) * C::BQ;
    const size_t qoff = ((size_t)(b * a.Hq + hq) * L) * D;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(reinterpret_cast<const bf16*>(a.q) + qoff, head_bytes);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(reinterpret_cast<const bf16*>(a.dout) + qoff, head_bytes);
    const int soff = q0 * (2 * D);
#pragma unroll
    for (int i = 0; i < C::QPER; ++i) {
      buf2lds16(qrs, ad.qcopy[i], soff, qs + (wave + C::kWaves * i) * 1024);
      buf2lds16(drs, ad.qcopy[i], soff, dos + (wave + C::kWaves * i) * 1024);
    }
    if (wave == 0) {
      const size_t srow = (size_t)(b * a.Hq + hq) * L;
      const __amdgpu_buffer_rsrc_t lrs = make_rsrc(a.lse2 + srow, (unsigned)L * 4);
      const __amdgpu_buffer_rsrc_t ers = make_rsrc(a.delta + srow, (unsigned)L * 4);
      buf2lds4(lrs, 4 * lane, 4 * q0, reinterpret_cast<char*>(ss));
      buf2lds4(ers, 4 * lane, 4 * q0, reinterpret_cast<char*>(ss) + 4 * C::BQ);
    }
  };

  {
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(reinterpret_cast<const bf16*>(a.k) + kv_off, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(reinterpret_cast<const bf16*>(a.v) + kv_off, head_bytes);
    const int soff = key_wg0 * (2 * D);
#pragma unroll
    for (int n = wave; n < C::KBCOPIES; n += C::kWaves) {
      const int src = pad_slot_src<D, Pad<D>::KSTR>(n * 64 + lane);
      buf2lds16(krs, src, soff, k_blk + n * 1024);
      buf2lds16(vrs, src, soff, v_blk + n * 1024);
    }
  }
  // cursors: entry and head offset of iterations it and it + 1, list position of it + 2
  const EntryStream es{make_rsrc(ents, 4u * (unsigned)n_ent)};
  unsigned cur = n_ent > 0 ? ents[0] : 0u, nxt = n_ent > 1 ? ents[1] : cur;
  int cur_h = 0, nxt_h = n_ent > 1 ? 0 : 1;
  int fe = 2, fh = 0;
  if (n_ent > 0)
    while (fe >= n_ent) {
      fe -= n_ent;
      ++fh;
    }
  auto advance = [&]() {
    if (++fe == n_ent) {
      fe = 0;
      ++fh;
    }
  };
  if (n_it > 0) issue(cur, cur_h, q_st0, do_st0, stat_st0);

  KVState<D> st;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    st.dv[db] = f32x16{};
    st.dk[db] = f32x16{};
  }
  const float c = a.scale_log2;

  auto step = [&](unsigned ent, const char* qs, const char* dos, const float* ss) {
    const int cls = ent_class(ent, half);
    const int q0 = ent_tile(ent, p.nb) * C::BQ;
    if (cls != 0 && key_w0 < L && q0 + 32 * qh < L) {
      const bool tg = (cls == 1) & ent_glob(ent);
      const unsigned long long gqb = tg ? plan_word(p.gbits, ent_tile(ent, p.nb)) : 0ull;
      const bool bm = ent_block(ent, half);
      // without a global query in the tile and with the block allowed, the
      // window and causal range alone decide (a global key's own dK, dV are
      // not stored here)
      const EitherMask<RangeMaskK<CAUSAL>, GeneralMaskK<CAUSAL>> ok{
          (bool)(!tg & bm), RangeMaskK<CAUSAL>{L, 0, window, my_key},
          GeneralMaskK<CAUSAL>{L, window, my_key, q0, gk, bm, gqb}};
      kv_tile<D, F16>(st, ad, k_blk, v_blk, qs, dos, ss, q0, cls == 1, ok, qh, c, lane);
    }
  };

  fwdtile::wait_copies_and_barrier();
  for (int it = 0; it < n_it; it += 2) {
    const unsigned far0 = es.fetch(fe);
    const int far0_h = fh;
    advance();
    if (it + 1 < n_it) issue(nxt, nxt_h, q_st1, do_st1, stat_st1);
    step(cur, q_st0, do_st0, stat_st0);
    fwdtile::wait_copies_and_barrier();
    if (it + 1 >= n_it) break;
    cur = nxt;
    cur_h = nxt_h;
    nxt = uniform(far0);
    nxt_h = far0_h;
    const unsigned far1 = es.fetch(fe);
    const int far1_h = fh;
    advance();
    if (it + 2 < n_it) issue(nxt, nxt_h, q_st0, do_st0, stat_st0);
    step(cur, q_st1, do_st1, stat_st1);
    fwdtile::wait_copies_and_barrier();
    cur = nxt;
    cur_h = nxt_h;
    nxt = uniform(far1);
    nxt_h = far1_h;
  }

  // sum the two query halves and store as the range-tiled kernel; global keys
  // are left to the global-key pass
  const size_t row0 = (size_t)key_wg0 * (2 * D);
  const int b0 = min(2 * kt, p.nb - 1), b1 = min(2 * kt + 1, p.nb - 1);
  const unsigned long long gw0 = p.gbits[b0], gw1 = p.gbits[b1];
  kv_store<D, F16>(st, q_st0, do_st0, q_st1, do_st1, reinterpret_cast<char*>(reinterpret_cast<bf16*>(a.dk) + kv_off) + row0,
                   reinterpret_cast<char*>(reinterpret_cast<bf16*>(a.dv) + kv_off) + row0, a.scale, kb, qh, wave,
                   lane, [&](int r) {
                     const int key = key_wg0 + r;
                     const bool kglob = (((key >> 6) == b0 ? gw0 : gw1) >> (key & 63)) & 1ull;
                     return (key >= L) | kglob;
                   });
}

// dQ: one work-group of 4 waves per (batch, query head, 128 queries), as the
// range-tiled kernel, streaming the key tiles of its row list.
template <int D, bool CAUSAL, bool F16>
__global__ __launch_bounds__(256, 2) void dq_masked_kernel(BwdArgs a, PlanPtrs p) {
  using namespace bwdtile;
  using C = QCfg<D>;
  __shared__ __attribute__((aligned(1024))) char k_st0[C::KT];
  __shared__ __attribute__((aligned(1024))) char v_st0[C::VT];
  __shared__ __attribute__((aligned(1024))) char k_st1[C::KT];
  __shared__ __attribute__((aligned(1024))) char v_st1[C::VT];
  __shared__ __attribute__((aligned(1024))) char g_rows[kGlobalRowsBytes<D>];

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int g = lane >> 5, ln = lane & 31;
  const int half = wave >> 1;
  const int L = a.L, window = a.window;

  int bh, qt;
  plan_wg(xcd_remap(blockIdx.x, gridDim.x), a.B * a.Hq, p.nw, p.meta[0], p.row_ord, bh, qt);
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const size_t q_off = ((size_t)(b * a.Hq + h) * L) * D;
  const size_t kv_off = ((size_t)(b * a.Hkv + hk) * L) * D;
  const unsigned head_bytes = (unsigned)L * (2 * D);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(reinterpret_cast<const bf16*>(a.k) + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(reinterpret_cast<const bf16*>(a.v) + kv_off, head_bytes);

  const int q_w0 = qt * C::BQ + 32 * wave;
  const int my_q = q_w0 + ln;
  const int n_ent = min(max(__builtin_amdgcn_readfirstlane(p.row_cnt[qt]), 0), p.nb);
  const unsigned* ents = p.row_ent + (size_t)qt * p.nb;
  const bool gq = is_global(p.gbits, my_q, L);

  QAddr<D> ad;
#pragma unroll
  for (int i = 0; i < C::KPER; ++i) ad.kcopy[i] = dual_slot_src<D>((wave + C::kWaves * i) * 64 + lane);
#pragma unroll
  for (int i = 0; i < C::VPER; ++i) ad.vcopy[i] = pad_slot_src<D, Pad<D>::KSTR>((wave + C::kWaves * i) * 64 + lane);
#pragma unroll
  for (int k = 0; k < C::NSTEP; ++k) ad.krow[k] = row_offset_dual<D>(ln, k, g);
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    ad.ktr[db][0] = tr_offset_dual<D>(0, db, 0, lane);
    ad.ktr[db][1] = tr_offset_dual<D>(0, db, 1, lane);
  }
  ad.vrow = row_offset_kpad<D>(ln, 0, g);

  auto issue = [&](unsigned ent, char* kb, char* vb) {
    const int soff = ent_tile(ent, p.nb) * C::BC * (2 * D);
#pragma unroll
    for (int i = 0; i < C::KPER; ++i) buf2lds16(krs, ad.kcopy[i], soff, kb + (wave + C::kWaves * i) * 1024);
#pragma unroll
    for (int i = 0; i < C::VPER; ++i)
      if (owns_copy<C::kWaves, C::VCOPIES>(wave, i)) buf2lds16(vrs, ad.vcopy[i], soff, vb + (wave + C::kWaves * i) * 1024);
  };
  const EntryStream es{make_rsrc(ents, 4u * (unsigned)n_ent)};
  unsigned cur = n_ent > 0 ? ents[0] : 0u, nxt = n_ent > 1 ? ents[1] : 0u;
  if (n_ent > 0) issue(cur, k_st0, v_st0);
  const int n_fold = fold_count(p.meta, L);
  if (n_fold > 0) stage_global_rows<D>(g_rows, krs, vrs, p.gpos, n_fold, L, wave, lane);

  QState<D> st;
  {
    const int qr = min(my_q, L - 1);
    const bf16* Qr = reinterpret_cast<const bf16*>(a.q) + q_off + (size_t)qr * D;
    const bf16* dOr = reinterpret_cast<const bf16*>(a.dout) + q_off + (size_t)qr * D;
#pragma unroll
    for (int k = 0; k < C::NSTEP; ++k) {
      st.qr[k] = *reinterpret_cast<const bf16x8*>(Qr + 16 * k + 8 * g);
      st.dor[k] = *reinterpret_cast<const bf16x8*>(dOr + 16 * k + 8 * g);
    }
    const size_t srow = (size_t)(b * a.Hq + h) * L + qr;
    st.set_stats(a.lse2[srow], a.delta[srow]);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) st.dq[db] = f32x16{};
  }
  const float c = a.scale_log2;
  const bool excl_gk = n_fold > 0;

  auto step = [&](unsigned ent, const char* kb, const char* vb) {
    const int cls = ent_class(ent, half);
    if (cls != 0 && q_w0 < L) {
      const int kt = ent_tile(ent, p.nb);
      // (the forward's choice of a cheaper element test costs this kernel
      // spills: it keeps the general one)
      const GeneralMaskQ<CAUSAL> ok{L, window, my_q, kt * C::BC, gq, ent_block(ent, half),
                                    ((cls == 1) & ent_glob(ent)) ? plan_word(p.gbits, kt) : 0ull, excl_gk};
      q_tile<D, F16>(st, ad, kb, vb, kt * C::BC, cls == 1, ok, c, lane);
    }
  };

  fwdtile::wait_copies_and_barrier();
  for (int e = 0; e < n_ent; e += 2) {
    const unsigned far0 = es.fetch(e + 2);
    if (e + 1 < n_ent) issue(nxt, k_st1, v_st1);
    step(cur, k_st0, v_st0);
    fwdtile::wait_copies_and_barrier();
    if (e + 1 >= n_ent) break;
    cur = nxt;
    nxt = uniform(far0);
    const unsigned far1 = es.fetch(e + 3);
    if (e + 2 < n_ent) issue(nxt, k_st0, v_st0);
    step(cur, k_st1, v_st1);
    fwdtile::wait_copies_and_barrier();
    cur = nxt;
    nxt = uniform(far1);
  }

  if (n_fold > 0 && q_w0 < L) fold_keys_dq<D, CAUSAL, F16>(st, g_rows, p.gpos, n_fold, L, my_q, c, g);

  if (my_q < L && !gq) {         // global rows: the global-row pass
    bf16* dQr = reinterpret_cast<bf16*>(a.dq) + q_off + (size_t)my_q * D;
    const float s = a.scale;
    store_row_c<F16, C::NDB>(dQr, st.dq, s, g);
  }
}

// ------------------------------------------------------------ 3. global positions
//
// A global query row attends to every key and a global key is attended by
// every query, so each is a whole row (column) of the mask: the lists leave
// them out and these passes compute them, split over the sequence so that a
// handful of long rows still spread over the chip ("split-K"), each split
// writing a float32 partial to the workspace and a last kernel combining the
// splits exactly (forward: LSE = log sum_s e^{LSE_s}, O = sum_s e^{LSE_s - LSE}
// O_s; gradients: plain sums).  One work-group holds 32 global positions of
// one head as the 32 MFMA columns of the tile steps.  A global position sees
// every position (subject to the causal mask): the element mask is j <= i.

template <bool CAUSAL>
struct DenseMask {                 // the lane's position `self` against position x
  int L, self;
  bool key_side;                   // self is a key (x a query) or a query (x a key)
  __device__ __forceinline__ bool operator()(int x) const {
    return (x < L) & (!CAUSAL | (key_side ? self <= x : x <= self));
  }
};

// Forward of the global query rows over key tiles [split*per, split*per + per):
// one wave per (split, batch*query head, 32 rows).
template <int D, bool CAUSAL, bool F16>
__global__ __launch_bounds__(64) void grows_fwd_kernel(FwdArgs a, PlanPtrs p, GlobalArgs ga) {
  using namespace fwdtile;
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) char k_st0[C::KT];
  __shared__ __attribute__((aligned(1024))) char v_st0[C::VT];
  __shared__ __attribute__((aligned(1024))) char k_st1[C::KT];
  __shared__ __attribute__((aligned(1024))) char v_st1[C::VT];

  const int lane = threadIdx.x, g = lane >> 5, ln = lane & 31;
  const int split = blockIdx.x, bh = blockIdx.y, r0 = 32 * blockIdx.z;
  const int L = a.L;
  const int n_g = min(max(p.meta[2], 0), ga.ngp);
  if (r0 >= n_g) return;
  const int r = r0 + ln;
  const bool valid = r < n_g;
  const int pos = min(max(p.gpos[valid ? r : r0], 0), L - 1);
  const int lo_pos = min(max(p.gpos[r0], 0), L - 1);                        // ascending: the wave's first
  const int hi_pos = min(max(p.gpos[min(n_g, r0 + 32) - 1], 0), L - 1);     // and last row
  const int b = bh / a.Hq, h = bh % a.Hq, hk = h / (a.Hq / a.Hkv);

  const size_t kv_off = ((size_t)(b * a.Hkv + hk) * L) * D;
  const unsigned head_bytes = (unsigned)L * (2 * D);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(reinterpret_cast<const bf16*>(a.k) + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(reinterpret_cast<const bf16*>(a.v) + kv_off, head_bytes);

  const int t_lo = split * ga.per;
  int t_hi = min(p.nb, t_lo + ga.per) - 1;
  if (CAUSAL) t_hi = min(t_hi, hi_pos / C::BC);

  int koff[C::KCOPIES], voff[C::VCOPIES];
#pragma unroll
  for (int i = 0; i < C::KCOPIES; ++i) koff[i] = pad_slot_src<D, Pad<D>::KSTR>(i * 64 + lane);
#pragma unroll
  for (int i = 0; i < C::VCOPIES; ++i) voff[i] = pad_slot_src<D, Pad<D>::VSTR>(i * 64 + lane);
  auto issue = [&](int j, char* kbuf, char* vbuf) {
    const int soff = j * C::BC * (2 * D);
#pragma unroll
    for (int i = 0; i < C::KCOPIES; ++i) buf2lds16(krs, koff[i], soff, kbuf + i * 1024);
#pragma unroll
    for (int i = 0; i < C::VCOPIES; ++i) buf2lds16(vrs, voff[i], soff, vbuf + i * 1024);
  };
  if (t_lo <= t_hi) issue(t_lo, k_st0, v_st0);

  FwdState<D> st;
  const bf16* Qr = reinterpret_cast<const bf16*>(a.q) + ((size_t)(b * a.Hq + h) * L + pos) * D;
#pragma unroll
  for (int k = 0; k < C::NSTEP; ++k) st.qr[k] = valid ? *reinterpret_cast<const bf16x8*>(Qr + 16 * k + 8 * g) : bf16x8{};
  st.m_run = kNegBig;
  st.l_run = 0.f;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) st.o[db] = f32x16{};
  const float c = a.scale_log2;
  const DenseMask<CAUSAL> ok{L, pos, false};
  auto tile_mask = [&](int k0) { return k0 + C::BC > L || (CAUSAL && k0 + C::BC - 1 > lo_pos); };

  wait_copies_and_barrier();
  for (int j = t_lo; j <= t_hi; j += 2) {
    if (j < t_hi) issue(j + 1, k_st1, v_st1);
    fwd_tile<D, F16>(st, k_st0, v_st0, j * C::BC, tile_mask(j * C::BC), ok, c, lane);
    wait_copies_and_barrier();
    if (j + 1 > t_hi) break;
    if (j + 1 < t_hi) issue(j + 2, k_st0, v_st0);
    fwd_tile<D, F16>(st, k_st1, v_st1, (j + 1) * C::BC, tile_mask((j + 1) * C::BC), ok, c, lane);
    wait_copies_and_barrier();
  }

  const float l_tot = pair_sum(st.l_run);
  if (valid) {
    const size_t prow = ((size_t)split * a.B * a.Hq + bh) * ga.ngp + r;
    float* po = ga.part + prow * D;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<f32x4*>(po + 32 * db + 8 * i4 + 4 * g) =
            f32x4{st.o[db][4 * i4] * inv, st.o[db][4 * i4 + 1] * inv, st.o[db][4 * i4 + 2] * inv,
                  st.o[db][4 * i4 + 3] * inv};
    if (g == 0)
      ga.part_lse[prow] = l_tot > 0.f ? (st.m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// Merge the splits of every (head, global row) into O and LSE at the row's position.
template <int D, bool F16>
__global__ __launch_bounds__(256) void grows_combine_kernel(FwdArgs a, PlanPtrs p, GlobalArgs ga) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerBlock = 256 / kLanesPerRow;
  const long long rows = (long long)a.B * a.Hq * ga.ngp;
  const long long row = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const int part = threadIdx.x % kLanesPerRow;
  if (row >= rows) return;
  const int bh = (int)(row / ga.ngp), r = (int)(row % ga.ngp);
  const int n_g = min(max(p.meta[2], 0), ga.ngp);
  if (r >= n_g) return;
  const int pos = min(max(p.gpos[r], 0), a.L - 1);
  float m = -INFINITY;
  for (int s = 0; s < ga.n_splits; ++s) m = fmaxf(m, ga.part_lse[(size_t)s * rows + row]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < ga.n_splits; ++s) {
      const float w = __expf(ga.part_lse[(size_t)s * rows + row] - m);
      if (w == 0.f) continue;
      const f32x4* x = reinterpret_cast<const f32x4*>(ga.part + ((size_t)s * rows + row) * D + 8 * part);
      const f32x4 x0 = x[0], x1 = x[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += w * x0[i];
        acc[4 + i] += w * x1[i];
      }
      tot += w;
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const size_t orow = (size_t)bh * a.L + pos;
  bf16* out = static_cast<bf16*>(a.o) + orow * D + 8 * part;
  *reinterpret_cast<bf16x8*>(out) = pack8<F16>(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv,
                                                acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  if (part == 0 && a.lse != nullptr) a.lse[orow] = tot > 0.f ? m + __logf(tot) : -INFINITY;
}

// dQ of the global query rows over key tiles [split*per, split*per + per):
// one wave per (split, batch*query head, 32 rows); float32 partial sums.
template <int D, bool CAUSAL, bool F16>
__global__ __launch_bounds__(64) void grows_dq_kernel(BwdArgs a, PlanPtrs p, GlobalArgs ga) {
  using namespace bwdtile;
  using C = QCfg<D>;
  __shared__ __attribute__((aligned(1024))) char k_st0[C::KT];
  __shared__ __attribute__((aligned(1024))) char v_st0[C::VT];
  __shared__ __attribute__((aligned(1024))) char k_st1[C::KT];
  __shared__ __attribute__((aligned(1024))) char v_st1[C::VT];

  const int lane = threadIdx.x, g = lane >> 5, ln = lane & 31;
  const int split = blockIdx.x, bh = blockIdx.y, r0 = 32 * blockIdx.z;
  const int L = a.L;
  const int n_g = min(max(p.meta[2], 0), ga.ngp);
  if (r0 >= n_g) return;
  const int r = r0 + ln;
  const bool valid = r < n_g;
  const int pos = min(max(p.gpos[valid ? r : r0], 0), L - 1);
  const int lo_pos = min(max(p.gpos[r0], 0), L - 1);
  const int hi_pos = min(max(p.gpos[min(n_g, r0 + 32) - 1], 0), L - 1);
  const int b = bh / a.Hq, h = bh % a.Hq, hk = h / (a.Hq / a.Hkv);

  const size_t q_off = ((size_t)(b * a.Hq + h) * L) * D;
  const size_t kv_off = ((size_t)(b * a.Hkv + hk) * L) * D;
  const unsigned head_bytes = (unsigned)L * (2 * D);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(reinterpret_cast<const bf16*>(a.k) + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(reinterpret_cast<const bf16*>(a.v) + kv_off, head_bytes);

  const int t_lo = split * ga.per;
  int t_hi = min(p.nb, t_lo + ga.per) - 1;
  if (CAUSAL) t_hi = min(t_hi, hi_pos / C::BC);

  QAddr<D> ad;
#pragma unroll
  for (int k = 0; k < C::NSTEP; ++k) ad.krow[k] = row_offset_dual<D>(ln, k, g);
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    ad.ktr[db][0] = tr_offset_dual<D>(0, db, 0, lane);
    ad.ktr[db][1] = tr_offset_dual<D>(0, db, 1, lane);
  }
  ad.vrow = row_offset_kpad<D>(ln, 0, g);
  int koff[C::KCOPIES], voff[C::VCOPIES];
#pragma unroll
  for (int i = 0; i < C::KCOPIES; ++i) koff[i] = dual_slot_src<D>(i * 64 + lane);
#pragma unroll
  for (int i = 0; i < C::VCOPIES; ++i) voff[i] = pad_slot_src<D, Pad<D>::KSTR>(i * 64 + lane);
  auto issue = [&](int j, char* kb, char* vb) {
    const int soff = j * C::BC * (2 * D);
#pragma unroll
    for (int i = 0; i < C::KCOPIES; ++i) buf2lds16(krs, koff[i], soff, kb + i * 1024);
#pragma unroll
    for (int i = 0; i < C::VCOPIES; ++i) buf2lds16(vrs, voff[i], soff, vb + i * 1024);
  };
  if (t_lo <= t_hi) issue(t_lo, k_st0, v_st0);

  QState<D> st;
  {
    const bf16* Qr = reinterpret_cast<const bf16*>(a.q) + q_off + (size_t)pos * D;
    const bf16* dOr = reinterpret_cast<const bf16*>(a.dout) + q_off + (size_t)pos * D;
#pragma unroll
    for (int k = 0; k < C::NSTEP; ++k) {
      st.qr[k] = *reinterpret_cast<const bf16x8*>(Qr + 16 * k + 8 * g);
      st.dor[k] = *reinterpret_cast<const bf16x8*>(dOr + 16 * k + 8 * g);
    }
    const size_t srow = (size_t)(b * a.Hq + h) * L + pos;
    st.set_stats(a.lse2[srow], a.delta[srow]);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) st.dq[db] = f32x16{};
  }
  const float c = a.scale_log2;
  const DenseMask<CAUSAL> ok{L, pos, false};
  auto tile_mask = [&](int k0) { return k0 + C::BC > L || (CAUSAL && k0 + C::BC - 1 > lo_pos); };

  fwdtile::wait_copies_and_barrier();
  for (int j = t_lo; j <= t_hi; j += 2) {
    if (j < t_hi) issue(j + 1, k_st1, v_st1);
    q_tile<D, F16>(st, ad, k_st0, v_st0, j * C::BC, tile_mask(j * C::BC), ok, c, lane);
    fwdtile::wait_copies_and_barrier();
    if (j + 1 > t_hi) break;
    if (j + 1 < t_hi) issue(j + 2, k_st0, v_st0);
    q_tile<D, F16>(st, ad, k_st1, v_st1, (j + 1) * C::BC, tile_mask((j + 1) * C::BC), ok, c, lane);
    fwdtile::wait_copies_and_barrier();
  }

  if (valid) {
    float* po = ga.part + (((size_t)split * a.B * a.Hq + bh) * ga.ngp + r) * D;
    const float s = a.scale;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<f32x4*>(po + 32 * db + 8 * i4 + 4 * g) =
            f32x4{st.dq[db][4 * i4] * s, st.dq[db][4 * i4 + 1] * s, st.dq[db][4 * i4 + 2] * s,
                  st.dq[db][4 * i4 + 3] * s};
  }
}

// Sum the float32 partials of every (head, global position) into the rows of
// out0 (and out1): the partial of split s holds n_tensors rows of D floats
// per (head, position); tensor 0 is multiplied by scale0.
template <int D, bool F16>
__global__ __launch_bounds__(256) void gsum_kernel(const float* __restrict__ part, int n_parts, long long rows,
                                                   int ngp, int L, const int* meta, const int* gpos,
                                                   bf16* __restrict__ out0, bf16* __restrict__ out1, int n_tensors,
                                                   float scale0) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerBlock = 256 / kLanesPerRow;
  const long long row = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const int part_i = threadIdx.x % kLanesPerRow;
  if (row >= rows) return;
  const int head = (int)(row / ngp), r = (int)(row % ngp);
  const int n_g = min(max(meta[2], 0), ngp);
  if (r >= n_g) return;
  const int pos = min(max(gpos[r], 0), L - 1);
  for (int t = 0; t < n_tensors; ++t) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < n_parts; ++s) {
      const f32x4* x = reinterpret_cast<const f32x4*>(part + (((size_t)s * rows + row) * n_tensors + t) * D +
                                                      8 * part_i);
      const f32x4 x0 = x[0], x1 = x[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += x0[i];
        acc[4 + i] += x1[i];
      }
    }
    const float f = t == 0 ? scale0 : 1.f;
    bf16* o = (t == 0 ? out0 : out1) + ((size_t)head * L + pos) * D + 8 * part_i;
    *reinterpret_cast<bf16x8*>(o) = pack8<F16>(acc[0] * f, acc[1] * f, acc[2] * f, acc[3] * f, acc[4] * f,
                                               acc[5] * f, acc[6] * f, acc[7] * f);
  }
}

// dK and dV of the global keys over query tiles [split*per, split*per + per) of
// every query head of the group: two waves (the halves of a 64-query tile) per
// (split, batch*K/V head, 32 keys); float32 partials, one per (split, half).
template <int D, bool CAUSAL, bool F16>
__global__ __launch_bounds__(128) void gcols_dkdv_kernel(BwdArgs a, PlanPtrs p, GlobalArgs ga) {
  using namespace bwdtile;
  using C = KVCfg<D>;
  constexpr int KB32 = 32 * Pad<D>::KSTR;           // a padded block of 32 keys
  __shared__ __attribute__((aligned(C::QT))) char q_st0[C::QT];
  __shared__ __attribute__((aligned(C::QT))) char do_st0[C::QT];
  __shared__ __attribute__((aligned(C::QT))) char q_st1[C::QT];
  __shared__ __attribute__((aligned(C::QT))) char do_st1[C::QT];
  __shared__ __attribute__((aligned(1024))) char k_blk[KB32];
  __shared__ __attribute__((aligned(1024))) char v_blk[KB32];
  __shared__ __attribute__((aligned(16))) float stat_st0[2 * C::BQ];
  __shared__ __attribute__((aligned(16))) float stat_st1[2 * C::BQ];

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int g = lane >> 5, ln = lane & 31;
  const int qh = wave;
  const int split = blockIdx.x, bhk = blockIdx.y, r0 = 32 * blockIdx.z;
  const int L = a.L, G = a.Hq / a.Hkv;
  const int n_g = min(max(p.meta[2], 0), ga.ngp);
  if (r0 >= n_g) return;
  const int r = r0 + ln;
  const bool valid = r < n_g;
  const int pos = min(max(p.gpos[valid ? r : r0], 0), L - 1);
  const int lo_pos = min(max(p.gpos[r0], 0), L - 1);
  const int hi_pos = min(max(p.gpos[min(n_g, r0 + 32) - 1], 0), L - 1);
  const int b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const size_t kv_off = ((size_t)(b * a.Hkv + hk) * L) * D;
  const unsigned head_bytes = (unsigned)L * (2 * D);

  // query tiles of this split; with causal masking a key sees queries at or after it
  int t_lo = split * ga.per;
  const int t_hi = min(p.nb, t_lo + ga.per) - 1;
  if (CAUSAL) t_lo = max(t_lo, lo_pos / C::BQ);
  const int nq = max(0, t_hi - t_lo + 1);
  const int n_it = G * nq;

  // the 32 gathered K and V rows, padded (plain loads: 32 padded rows are not a whole number of 1 KiB copies)
  {
    const bf16* Kh = reinterpret_cast<const bf16*>(a.k) + kv_off;
    const bf16* Vh = reinterpret_cast<const bf16*>(a.v) + kv_off;
    constexpr int kChunks = D / 8;
    for (int e = threadIdx.x; e < 32 * kChunks; e += 128) {
      const int row = e / kChunks, ch = e % kChunks;
      const int rr = min(r0 + row, n_g - 1);
      const int kpos = min(max(p.gpos[rr], 0), L - 1);
      const bf16x8 kx = *reinterpret_cast<const bf16x8*>(Kh + (size_t)kpos * D + 8 * ch);
      const bf16x8 vx = *reinterpret_cast<const bf16x8*>(Vh + (size_t)kpos * D + 8 * ch);
      *reinterpret_cast<bf16x8*>(k_blk + row * Pad<D>::KSTR + 16 * ch) = kx;
      *reinterpret_cast<bf16x8*>(v_blk + row * Pad<D>::KSTR + 16 * ch) = vx;
    }
  }

  KVAddr<D> ad;
#pragma unroll
  for (int k = 0; k < C::NSTEP; ++k) ad.row[k] = row_offset_dual<D>(32 * qh + ln, k, g);
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    ad.tr[db][0] = tr_offset_dual<D>(2 * qh, db, 0, lane);
    ad.tr[db][1] = tr_offset_dual<D>(2 * qh, db, 1, lane);
  }
  ad.kv = row_offset_kpad<D>(ln, 0, g);
  constexpr int kCopies = C::QT / 1024 / 2;          // per wave, per tensor
  int qcopy[kCopies];
#pragma unroll
  for (int i = 0; i < kCopies; ++i) qcopy[i] = dual_slot_src<D>((wave + 2 * i) * 64 + lane);

  auto issue = [&](int it, char* qs, char* dos, float* ss) {
    const int hq = hk * G + it / nq, q0 = (t_lo + it % nq) * C::BQ;
    const size_t qoff = ((size_t)(b * a.Hq + hq) * L) * D;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(reinterpret_cast<const bf16*>(a.q) + qoff, head_bytes);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(reinterpret_cast<const bf16*>(a.dout) + qoff, head_bytes);
    const int soff = q0 * (2 * D);
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      buf2lds16(qrs, qcopy[i], soff, qs + (wave + 2 * i) * 1024);
      buf2lds16(drs, qcopy[i], soff, dos + (wave + 2 * i) * 1024);
    }
    if (wave == 0) {
      const size_t srow = (size_t)(b * a.Hq + hq) * L;
      const __amdgpu_buffer_rsrc_t lrs = make_rsrc(a.lse2 + srow, (unsigned)L * 4);
      const __amdgpu_buffer_rsrc_t ers = make_rsrc(a.delta + srow, (unsigned)L * 4);
      buf2lds4(lrs, 4 * lane, 4 * q0, reinterpret_cast<char*>(ss));
      buf2lds4(ers, 4 * lane, 4 * q0, reinterpret_cast<char*>(ss) + 4 * C::BQ);
    }
  };
  if (n_it > 0) issue(0, q_st0, do_st0, stat_st0);

  KVState<D> st;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    st.dv[db] = f32x16{};
    st.dk[db] = f32x16{};
  }
  const float c = a.scale_log2;
  const DenseMask<CAUSAL> ok{L, pos, true};
  auto block_mask = [&](int q0) {
    const int qw0 = q0 + 32 * qh;
    return qw0 + 32 > L || (CAUSAL && qw0 < hi_pos);
  };

  fwdtile::wait_copies_and_barrier();
  for (int it = 0; it < n_it; it += 2) {
    if (it + 1 < n_it) issue(it + 1, q_st1, do_st1, stat_st1);
    {
      const int q0 = (t_lo + it % nq) * C::BQ;
      if (q0 + 32 * qh < L) kv_tile<D, F16>(st, ad, k_blk, v_blk, q_st0, do_st0, stat_st0, q0, block_mask(q0), ok, qh, c, lane);
    }
    fwdtile::wait_copies_and_barrier();
    if (it + 1 >= n_it) break;
    if (it + 2 < n_it) issue(it + 2, q_st0, do_st0, stat_st0);
    {
      const int q0 = (t_lo + (it + 1) % nq) * C::BQ;
      if (q0 + 32 * qh < L) kv_tile<D, F16>(st, ad, k_blk, v_blk, q_st1, do_st1, stat_st1, q0, block_mask(q0), ok, qh, c, lane);
    }
    fwdtile::wait_copies_and_barrier();
  }

  // partial (split, half): dK (unscaled) then dV; lane holds head-dim column
  // 32db + ln of keys 8(i/4) + 4g + i%4 of the block
  const long long rows = (long long)a.B * a.Hkv * ga.ngp;
  const size_t pidx = (size_t)(2 * split + qh) * rows + (size_t)bhk * ga.ngp;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int kr = r0 + 8 * (i >> 2) + 4 * g + (i & 3);
    if (kr < n_g) {
      float* pk = ga.part + ((pidx + kr) * 2) * D;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        pk[32 * db + ln] = st.dk[db][i];
        pk[D + 32 * db + ln] = st.dv[db][i];
      }
    }
  }
}

template <int D, bool CAUSAL, bool F16>
hipError_t fwd_masked_launch(const FwdArgs& a, const PlanPtrs& p, const GlobalArgs& ga, hipStream_t stream) {
  const long long nblk = (long long)a.B * a.Hq * p.nw;
  hipLaunchKernelGGL((fwd_masked_kernel<D, CAUSAL, F16>), dim3((unsigned)nblk), dim3(256), 0, stream, a, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ga.ngp == 0) return e;
  hipLaunchKernelGGL((grows_fwd_kernel<D, CAUSAL, F16>), dim3(ga.n_splits, a.B * a.Hq, ga.ngp / 32), dim3(64), 0,
                     stream, a, p, ga);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int kRowsPerBlock = 256 / (D / 8);
  const long long rows = (long long)a.B * a.Hq * ga.ngp;
  hipLaunchKernelGGL((grows_combine_kernel<D, F16>), dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)),
                     dim3(256), 0, stream, a, p, ga);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool F16>
hipError_t bwd_masked_launch(const BwdArgs& a, const PlanPtrs& p, const GlobalArgs& gr, const GlobalArgs& gc,
                             hipStream_t stream) {
  constexpr int kRowsPerBlock = 256 / (D / 8);
  hipError_t e = launch_bwd_preprocess_bf16(a, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dkdv_masked_kernel<D, CAUSAL, F16>), dim3((unsigned)((long long)a.B * a.Hkv * p.nw)),
                     dim3(512), 0, stream, a, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (gc.ngp > 0) {
    hipLaunchKernelGGL((gcols_dkdv_kernel<D, CAUSAL, F16>), dim3(gc.n_splits, a.B * a.Hkv, gc.ngp / 32), dim3(128),
                       0, stream, a, p, gc);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long rows = (long long)a.B * a.Hkv * gc.ngp;
    hipLaunchKernelGGL((gsum_kernel<D, F16>), dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), dim3(256),
                       0, stream, gc.part, 2 * gc.n_splits, rows, gc.ngp, a.L, p.meta, p.gpos,
                       static_cast<bf16*>(a.dk), static_cast<bf16*>(a.dv), 2, a.scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((dq_masked_kernel<D, CAUSAL, F16>), dim3((unsigned)((long long)a.B * a.Hq * p.nw)), dim3(256),
                     0, stream, a, p);
  e = hipGetLastError();
  if (e != hipSuccess || gr.ngp == 0) return e;
  hipLaunchKernelGGL((grows_dq_kernel<D, CAUSAL, F16>), dim3(gr.n_splits, a.B * a.Hq, gr.ngp / 32), dim3(64), 0,
                     stream, a, p, gr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long rows = (long long)a.B * a.Hq * gr.ngp;
  hipLaunchKernelGGL((gsum_kernel<D, F16>), dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), dim3(256),
                     0, stream, gr.part, gr.n_splits, rows, gr.ngp, a.L, p.meta, p.gpos, static_cast<bf16*>(a.dq),
                     static_cast<bf16*>(nullptr), 1, 1.f);
  return hipGetLastError();
}

template <bool F16>
hipError_t fwd_masked_typed(const FwdArgs& a, const PlanPtrs& p, const GlobalArgs& ga, bool causal, hipStream_t s) {
  if (a.d == 128)
    return causal ? fwd_masked_launch<128, true, F16>(a, p, ga, s) : fwd_masked_launch<128, false, F16>(a, p, ga, s);
  return causal ? fwd_masked_launch<64, true, F16>(a, p, ga, s) : fwd_masked_launch<64, false, F16>(a, p, ga, s);
}

template <bool F16>
hipError_t bwd_masked_typed(const BwdArgs& a, const PlanPtrs& p, const GlobalArgs& gr, const GlobalArgs& gc,
                            bool causal, hipStream_t s) {
  if (a.d == 128)
    return causal ? bwd_masked_launch<128, true, F16>(a, p, gr, gc, s)
                  : bwd_masked_launch<128, false, F16>(a, p, gr, gc, s);
  return causal ? bwd_masked_launch<64, true, F16>(a, p, gr, gc, s) : bwd_masked_launch<64, false, F16>(a, p, gr, gc, s);
}

}  // namespace

hipError_t launch_mask_plan(const MaskDesc& m, int L, void* plan, hipStream_t stream) {
  const PlanLayout y = plan_layout(L);
  if (y.nw > kMaxOrder) return hipErrorInvalidValue;
  char* base = static_cast<char*>(plan);
  PlanBuild p{};
  p.m = m;
  p.L = L;
  p.nb = y.nb;
  p.nw = y.nw;
  p.nbm = m.block_mask != nullptr ? (L + m.block - 1) / m.block : 0;
  p.gbits = reinterpret_cast<unsigned long long*>(base + y.gbits);
  p.row_cnt = reinterpret_cast<int*>(base + y.row_cnt);
  p.row_ord = reinterpret_cast<int*>(base + y.row_ord);
  p.row_ent = reinterpret_cast<unsigned*>(base + y.row_ent);
  p.col_cnt = reinterpret_cast<int*>(base + y.col_cnt);
  p.col_ord = reinterpret_cast<int*>(base + y.col_ord);
  p.col_ent = reinterpret_cast<unsigned*>(base + y.col_ent);
  p.meta = reinterpret_cast<int*>(base + y.meta);
  p.gpos = reinterpret_cast<int*>(base + y.gpos);
  hipLaunchKernelGGL(plan_gbits_kernel, dim3((unsigned)((y.nb + 255) / 256)), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(plan_gpos_kernel, dim3(1), dim3(1024), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(plan_lists_kernel, dim3((unsigned)y.nw, 2), dim3(256), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(plan_order_kernel, dim3(1), dim3(1024), 0, stream, p);
  return hipGetLastError();
}

// Splits of a global-position pass: about 1024 work-groups in all, at least
// four tiles per split.
GlobalArgs global_plan(int L, int n_global, int n_heads) {
  GlobalArgs g{};
  if (n_global <= 0) return g;
  g.ngp = (n_global + 31) / 32 * 32;
  const int nb = (L + 63) / 64;
  const int groups = n_heads * (g.ngp / 32);
  int want = (1024 + groups - 1) / groups;
  want = max(1, min(min(want, max(1, nb / 4)), 64));
  g.per = (nb + want - 1) / want;
  g.n_splits = (nb + g.per - 1) / g.per;
  return g;
}

size_t global_fwd_bytes(const GlobalArgs& g, int n_heads, int d) {
  const size_t rows = (size_t)g.n_splits * n_heads * g.ngp;
  return (rows * (size_t)(d + 1) * sizeof(float) + 255) & ~(size_t)255;
}

size_t global_dq_bytes(const GlobalArgs& g, int n_heads, int d) {
  return ((size_t)g.n_splits * n_heads * g.ngp * (size_t)d * sizeof(float) + 255) & ~(size_t)255;
}

size_t global_dkdv_bytes(const GlobalArgs& g, int n_kv_heads, int d) {
  return ((size_t)2 * g.n_splits * n_kv_heads * g.ngp * (size_t)(2 * d) * sizeof(float) + 255) & ~(size_t)255;
}

hipError_t launch_fwd_masked(const FwdArgs& a, const PlanPtrs& p, const GlobalArgs& ga, bool causal,
                             hipStream_t stream) {
  return a.f16 ? fwd_masked_typed<true>(a, p, ga, causal, stream) : fwd_masked_typed<false>(a, p, ga, causal, stream);
}

hipError_t launch_bwd_masked(const BwdArgs& a, const PlanPtrs& p, const GlobalArgs& gr, const GlobalArgs& gc,
                             bool causal, hipStream_t stream) {
  return a.f16 ? bwd_masked_typed<true>(a, p, gr, gc, causal, stream)
               : bwd_masked_typed<false>(a, p, gr, gc, causal, stream);
}

}  // namespace fa
