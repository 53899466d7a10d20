// fa_decode.hip -- attention of the newest tokens to a KV cache (gfx950).
//
// Autoregressive generation keeps every earlier token's K and V in a cache and
// attends only the Lq newest queries to it (book.anysome.cn "高效注意力" §1:
// the KV cache is one of the two large costs; §3: with GQA the G = Hq/Hkv
// query heads of a group share one K/V head).  New token t of sequence b sits
// at position cache_len[b] - Lq + t (bottom-right alignment).
//
// The work is bound by reading the cache from HBM, so the kernel reads each
// K/V head once for up to 128 of its rows -- the R = G*Lq rows (G query heads
// times Lq new tokens) form groups of 32, the query columns of the forward's
// per-tile MFMA step, and up to four groups (one wave each) share a work-group
// and its staged tiles; beyond 128 rows every further work-group reads the
// head again -- and splits the keys across work-groups so that short batches
// still fill the chip ("split-K").  Each split writes a partial (O, LSE) normalised over
// its keys to the workspace; the combine kernel merges a row's partials
// exactly: LSE = log sum_s e^{LSE_s}, O = sum_s e^{LSE_s - LSE} O_s.
// A work-group stages one tile at a time (37 KiB of LDS), so four of them fit
// on a CU: the bytes in flight that keep HBM busy come from four work-groups
// per CU copying at once, more than two double-buffered ones would have.
// (Work-groups of 2 or 4 waves run at two waves per SIMD, so four resp. two
// of them share a CU.)
//
// A rolling buffer of W slots (position p in slot p mod W) is read the same way
// with a slot -> position map: the new tokens' window over the buffer comes
// from its splits, their own keys (passed separately, not yet in the buffer)
// from one plain causal pass over them, and the combine merges both kinds of
// partial.
#include "fa_fwd_tile.hpp"

namespace fa {

namespace {

using namespace fwdtile;

// Key positions of a rolling buffer (transformer.xph.ink "高效注意力：FlashAttention
// 与线性注意力", 实例或案例: Mistral keeps the last W keys in W slots, position p
// in slot p mod W).  With n tokens seen the slots hold positions
// max(0, n - W) .. n - 1; h = n mod W is the slot the next token goes to, so
// slots h .. W-1 hold the oldest positions (n - W ..) and slots 0 .. h-1 the
// newest (.. n - 1).  Before the buffer is full (n < W) h = n and slot j holds
// position j.
struct RingPos {
  int n, h, W;
  __device__ __forceinline__ int operator()(int j) const { return j < h ? n - h + j : n - W - h + j; }
};

// Query-major mask over ring slots: the slot is filled and its position is in
// the row's window (positions lo .. the row's own; every filled slot precedes it).
struct RingMaskQ {
  int filled, lo;
  RingPos pos;
  __device__ __forceinline__ bool operator()(int j) const { return j < filled && pos(j) >= lo; }
};

constexpr int kMaxSeen = 1 << 30;   // tokens seen before a rolling-buffer call (clamped)

// One split of the keys for one (sequence, K/V head, group of 32 rows) -- the
// part of a work-group of NW waves that one wave computes.  The rows of a K/V
// head are its G query heads times the Lq new tokens, row r = head * Lq +
// token; wave w takes rows 32(NW z + w) .. 32(NW z + w) + 31, z = blockIdx.z.
//   RING = false: the cache holds positions 0 .. n-1 in order (n = cache_len[b]
//                 or Lk), the new tokens at positions n - Lq .. n - 1;
//   RING = true:  the cache is a rolling buffer of Lk = W slots (RingPos) after
//                 n = cache_len[b] tokens; the new tokens sit at positions
//                 n .. n + Lq - 1 and see the window of a.window positions
//                 ending at their own (their own keys come from another pass).
template <int D, bool CAUSAL, bool F16, bool RING, int NW>
__device__ __forceinline__ void split_body(const DecodeArgs& a, int split, char* k_st0, char* v_st0) {
  using C = FwdCfg<D>;
  const int lane = threadIdx.x & 63;
  const int wave = NW == 1 ? 0 : wave_id();
  const int g = lane >> 5, ln = lane & 31;
  const int bhk = blockIdx.y;
  const int b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const int G = a.Hq / a.Hkv, Lq = a.Lq;
  const long long R = (long long)G * Lq;
  // cache length / tokens seen of this sequence, clamped so that every access
  // stays inside the cache even for an out-of-range entry
  int n = a.cache_len != nullptr ? a.cache_len[b] : a.Lk;
  n = RING ? min(max(n, 0), kMaxSeen) : min(max(n, Lq), a.Lk);
  n = __builtin_amdgcn_readfirstlane(n);
  const int filled = RING ? min(n, a.Lk) : n;   // keys of the cache that hold tokens

  // this lane's row: query head hk*G + r/Lq, new token r%Lq (rows >= R are
  // padding); wave w of the work-group takes row group NW * blockIdx.z + w
  const long long r = 32LL * (NW * (long long)blockIdx.z + wave) + ln;
  const bool valid = r < R;
  const int hq = hk * G + (valid ? (int)(r / Lq) : 0);
  const int t = valid ? (int)(r % Lq) : Lq - 1;
  const int first = RING ? n : n - Lq;          // position of new token 0
  const int my_pos = first + t;
  const int min_pos = first, max_pos = first + Lq - 1;

  // keys of this split that any row may see
  const int s_lo = split * a.split_keys;
  const int k_hi = min(filled, s_lo + a.split_keys);   // causal: every row sees up to its own position
  const int k_lo = RING ? s_lo : max(s_lo, (a.window > 0) ? max(0, min_pos - a.window + 1) : 0);
  const bool empty = k_hi <= k_lo;
  const int j_lo = empty ? 0 : k_lo / C::BC, j_hi = empty ? -1 : (k_hi - 1) / C::BC;

  const size_t kv_off = ((size_t)(b * a.Hkv + hk) * a.Lk) * D;
  const unsigned head_bytes = (unsigned)a.Lk * (2 * D);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(reinterpret_cast<const bf16*>(a.k) + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(reinterpret_cast<const bf16*>(a.v) + kv_off, head_bytes);

  // The NW waves share the 1 KiB copies of a tile (copy n belongs to wave
  // n % NW); the per-lane source offsets are loop-invariant
  constexpr int KPER = (C::KCOPIES + NW - 1) / NW, VPER = (C::VCOPIES + NW - 1) / NW;
  int koff[KPER], voff[VPER];
#pragma unroll
  for (int i = 0; i < KPER; ++i) koff[i] = pad_slot_src<D, Pad<D>::KSTR>((wave + NW * i) * 64 + lane);
#pragma unroll
  for (int i = 0; i < VPER; ++i) voff[i] = pad_slot_src<D, Pad<D>::VSTR>((wave + NW * i) * 64 + lane);
  auto issue = [&](int j, char* kbuf, char* vbuf) {
    const int soff = j * C::BC * (2 * D);
#pragma unroll
    for (int i = 0; i < KPER; ++i)
      if (owns_copy<NW, C::KCOPIES>(wave, i)) buf2lds16(krs, koff[i], soff, kbuf + (wave + NW * i) * 1024);
#pragma unroll
    for (int i = 0; i < VPER; ++i)
      if (owns_copy<NW, C::VCOPIES>(wave, i)) buf2lds16(vrs, voff[i], soff, vbuf + (wave + NW * i) * 1024);
  };

  FwdState<D> st;
  const bf16* Qr = reinterpret_cast<const bf16*>(a.q) + ((size_t)((b * a.Hq + hq) * Lq + t)) * D;
#pragma unroll
  for (int k = 0; k < C::NSTEP; ++k) st.qr[k] = valid ? *reinterpret_cast<const bf16x8*>(Qr + 16 * k + 8 * g) : bf16x8{};
  st.m_run = kNegBig;
  st.l_run = 0.f;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) st.o[db] = f32x16{};
  const float c = a.scale_log2;

  // one stage: the work-group copies a tile, waits, computes; several such
  // work-groups per CU keep tiles in flight.  A single wave only has to see its
  // own reads of the previous tile finish before the stage is overwritten;
  // several waves wait for each other.
  auto run = [&](const auto& tile_mask, const auto& ok) {
    for (int j = j_lo; j <= j_hi; ++j) {
      if (NW == 1) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      else __syncthreads();
      issue(j, k_st0, v_st0);
      wait_copies_and_barrier();
      fwd_tile<D, F16>(st, k_st0, v_st0, j * C::BC, tile_mask(j * C::BC), ok, c, lane);
    }
  };
  if constexpr (RING) {
    // a tile needs the mask if it holds an empty slot or a position that the
    // last new token's window (the narrowest) no longer covers; its oldest
    // position is at slot h when the tile holds it, else at its first slot
    const RingPos pos{n, n % a.Lk, a.Lk};
    const int all_lo = max_pos - a.window + 1;
    auto tile_mask = [&](int k0) {
      const int oldest = (pos.h >= k0 && pos.h < k0 + C::BC && pos.h < filled) ? pos(pos.h) : pos(k0);
      return k0 + C::BC > filled || oldest < all_lo;
    };
    run(tile_mask, RingMaskQ{filled, my_pos - a.window + 1, pos});
  } else {
    // the window of a plain decode call is one-sided (causal): the key range
    // above already ends at the newest entry
    auto tile_mask = [&](int k0) { return range_tile_needs_mask<CAUSAL, C::BC>(k0, n, a.window, min_pos, max_pos); };
    run(tile_mask, RangeMaskQ<CAUSAL>{n, a.window, my_pos});
  }

  // partial for this split: O normalised over its keys (fp32), LSE in ln units
  // (-inf and O = 0 when the split holds no key the row may see)
  const float l_tot = pair_sum(st.l_run);
  if (valid) {
    const size_t row = (size_t)(b * a.Hq + hq) * Lq + t;
    const size_t prow = (size_t)(a.split_base + split) * a.rows + row;
    float* po = a.part_o + prow * D;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<f32x4*>(po + 32 * db + 8 * i4 + 4 * g) =
            f32x4{st.o[db][4 * i4] * inv, st.o[db][4 * i4 + 1] * inv, st.o[db][4 * i4 + 2] * inv,
                  st.o[db][4 * i4 + 3] * inv};
    if (g == 0) a.part_lse[prow] = l_tot > 0.f ? (st.m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// NW waves per work-group, one group of 32 rows each, share every K/V tile:
// NW = 1 for up to 32 rows per K/V head (four work-groups per CU, one wave per
// SIMD), 2 or 4 when there are more (two waves per SIMD; the tile is read once
// for all the work-group's row groups).
template <int NW>
struct DecodeOcc {
  static constexpr int kThreads = 64 * NW;
  static constexpr int kWavesPerEU = NW == 1 ? 1 : 2;
};

template <int D, bool CAUSAL, bool F16, int NW>
__global__ __launch_bounds__(DecodeOcc<NW>::kThreads) __attribute__((amdgpu_waves_per_eu(DecodeOcc<NW>::kWavesPerEU)))
void decode_split_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) char k_st0[FwdCfg<D>::KT];
  __shared__ __attribute__((aligned(1024))) char v_st0[FwdCfg<D>::VT];
  split_body<D, CAUSAL, F16, false, NW>(a, blockIdx.x, k_st0, v_st0);
}

// The rolling-buffer decode in one launch: splits 0 .. ring.n_splits - 1 read
// the buffer, the rest the new tokens' own keys (a plain causal decode whose
// cache is exactly those tokens); both write partials for the one combine.
template <int D, bool F16, int NW>
__global__ __launch_bounds__(DecodeOcc<NW>::kThreads) __attribute__((amdgpu_waves_per_eu(DecodeOcc<NW>::kWavesPerEU)))
void decode_rolling_kernel(DecodeArgs ring, DecodeArgs fresh) {
  __shared__ __attribute__((aligned(1024))) char k_st0[FwdCfg<D>::KT];
  __shared__ __attribute__((aligned(1024))) char v_st0[FwdCfg<D>::VT];
  if ((int)blockIdx.x < ring.n_splits) split_body<D, true, F16, true, NW>(ring, blockIdx.x, k_st0, v_st0);
  else split_body<D, true, F16, false, NW>(fresh, blockIdx.x - ring.n_splits, k_st0, v_st0);
}

// Merge one row's split partials: one work-group per row.  The splits are
// dealt to groups of d/8 adjacent lanes (8 elements each), so that a row with
// many splits -- a long cache with few sequences and K/V heads -- is merged by
// the whole work-group rather than by one group of lanes walking every split;
// the groups' weighted sums then meet in LDS.
template <int D, bool F16>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kGroups = 256 / kLanesPerRow;
  __shared__ float red[kGroups][D];
  __shared__ float gtot[kGroups];
  __shared__ float wmax[4];
  const long long row = blockIdx.x;
  const int t = threadIdx.x, grp = t / kLanesPerRow, part = t % kLanesPerRow;
  // 1. the largest split LSE of the row
  float m = -INFINITY;
  for (int s = t; s < a.n_splits_total; s += 256) m = fmaxf(m, a.part_lse[(size_t)s * a.rows + row]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((t & 63) == 0) wmax[t >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  // 2. this group's splits, weighted by e^{LSE_s - m}
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (m != -INFINITY) {
    for (int s = grp; s < a.n_splits_total; s += kGroups) {
      const float w = __expf(a.part_lse[(size_t)s * a.rows + row] - m);   // exp(-inf) = 0
      if (w == 0.f) continue;
      const f32x4* p = reinterpret_cast<const f32x4*>(a.part_o + ((size_t)s * a.rows + row) * D + 8 * part);
      const f32x4 x0 = p[0], x1 = p[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += w * x0[i];
        acc[4 + i] += w * x1[i];
      }
      tot += w;
    }
  }
  // 3. across the groups
#pragma unroll
  for (int i = 0; i < 8; ++i) red[grp][8 * part + i] = acc[i];
  if (part == 0) gtot[grp] = tot;
  __syncthreads();
  if (grp != 0) return;
  float sum = 0.f;
  for (int gi = 0; gi < kGroups; ++gi) sum += gtot[gi];
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float x = 0.f;
    for (int gi = 0; gi < kGroups; ++gi) x += red[gi][8 * part + i];
    o[i] = x;
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  bf16* out = static_cast<bf16*>(a.o) + (size_t)row * D + 8 * part;
  *reinterpret_cast<bf16x8*>(out) = pack8<F16>(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv, o[4] * inv,
                                                o[5] * inv, o[6] * inv, o[7] * inv);
  if (part == 0 && a.lse != nullptr) a.lse[row] = sum > 0.f ? m + __logf(sum) : -INFINITY;
}

// groups of 32 rows (query heads x new tokens) of one K/V head
inline long long row_groups(const DecodeArgs& a) { return ((long long)(a.Hq / a.Hkv) * a.Lq + 31) / 32; }

// waves per work-group for this many row groups
inline int waves_for(long long groups) { return groups == 1 ? 1 : groups == 2 ? 2 : 4; }

template <int D, bool CAUSAL, bool F16, int NW>
hipError_t launch_split_nw(const DecodeArgs& a, hipStream_t stream) {
  const unsigned gz = (unsigned)((row_groups(a) + NW - 1) / NW);
  hipLaunchKernelGGL((decode_split_kernel<D, CAUSAL, F16, NW>), dim3(a.n_splits, a.B * a.Hkv, gz),
                     dim3(64 * NW), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool F16>
hipError_t launch_split(const DecodeArgs& a, hipStream_t stream) {
  switch (waves_for(row_groups(a))) {
    case 1: return launch_split_nw<D, CAUSAL, F16, 1>(a, stream);
    case 2: return launch_split_nw<D, CAUSAL, F16, 2>(a, stream);
    default: return launch_split_nw<D, CAUSAL, F16, 4>(a, stream);
  }
}

template <int D, bool F16>
hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_combine_kernel<D, F16>), dim3((unsigned)a.rows), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool F16>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  hipError_t e = launch_split<D, CAUSAL, F16>(a, stream);
  if (e != hipSuccess) return e;
  return launch_combine<D, F16>(a, stream);
}

template <int D, bool F16, int NW>
hipError_t launch_rolling_nw(const DecodeArgs& ring, const DecodeArgs& fresh, hipStream_t stream) {
  const unsigned gz = (unsigned)((row_groups(ring) + NW - 1) / NW);
  hipLaunchKernelGGL((decode_rolling_kernel<D, F16, NW>), dim3(ring.n_splits + fresh.n_splits, ring.B * ring.Hkv, gz),
                     dim3(64 * NW), 0, stream, ring, fresh);
  return hipGetLastError();
}

template <int D, bool F16>
hipError_t launch_rolling(const DecodeArgs& ring, const DecodeArgs& fresh, hipStream_t stream) {
  hipError_t e;
  switch (waves_for(row_groups(ring))) {
    case 1: e = launch_rolling_nw<D, F16, 1>(ring, fresh, stream); break;
    case 2: e = launch_rolling_nw<D, F16, 2>(ring, fresh, stream); break;
    default: e = launch_rolling_nw<D, F16, 4>(ring, fresh, stream); break;
  }
  if (e != hipSuccess) return e;
  return launch_combine<D, F16>(ring, stream);
}

}  // namespace

namespace {
constexpr int DECODE_TARGET = 1024;   // work-groups a decode call aims for (four per CU)
constexpr int DECODE_CAP = 256;       // most key splits per sequence and K/V head
}  // namespace

void decode_plan(int B, int Hkv, int Lk, int& n_splits, int& split_keys) {
  constexpr int kBC = 64;
  const int tiles = (Lk + kBC - 1) / kBC;
  // about four work-groups per CU across the 256 CUs (a single-stage
  // work-group holds 37 KiB of LDS, so four fit on a CU), at least four tiles
  // per split
  int want = (DECODE_TARGET + B * Hkv - 1) / (B * Hkv);
  want = min(want, max(1, tiles / 4));
  want = max(1, min(want, DECODE_CAP));
  const int per = (tiles + want - 1) / want;
  split_keys = per * kBC;
  n_splits = (tiles + per - 1) / per;
}

hipError_t launch_decode_rolling(const DecodeArgs& ring, const DecodeArgs& fresh, hipStream_t stream) {
  if (ring.d == 128) return ring.f16 ? launch_rolling<128, true>(ring, fresh, stream) : launch_rolling<128, false>(ring, fresh, stream);
  return ring.f16 ? launch_rolling<64, true>(ring, fresh, stream) : launch_rolling<64, false>(ring, fresh, stream);
}

hipError_t launch_decode(const DecodeArgs& a, bool causal, hipStream_t stream) {
  if (a.d == 128) {
    if (a.f16) return causal ? launch_typed<128, true, true>(a, stream) : launch_typed<128, false, true>(a, stream);
    return causal ? launch_typed<128, true, false>(a, stream) : launch_typed<128, false, false>(a, stream);
  }
  if (a.f16) return causal ? launch_typed<64, true, true>(a, stream) : launch_typed<64, false, true>(a, stream);
  return causal ? launch_typed<64, true, false>(a, stream) : launch_typed<64, false, false>(a, stream);
}

}  // namespace fa
