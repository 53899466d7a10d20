// fa_decode.hip -- attention of the newest tokens to a KV cache (gfx950).
//
// Autoregressive generation keeps every earlier token's K and V in a cache and
// attends only the Lq newest queries to it (book.anysome.cn "高效注意力" §1:
// the KV cache is one of the two large costs; §3: with GQA the G = Hq/Hkv
// query heads of a group share one K/V head).  New token t of sequence b sits
// at position cache_len[b] - Lq + t (bottom-right alignment).
//
// The work is bound by reading the cache from HBM, so the kernel reads each
// K/V head once for all G query heads and all Lq new tokens -- the R = G*Lq
// rows become the 32 query columns of the forward's per-tile MFMA step (R <= 32)
// -- and splits the keys across work-groups so that short batches still fill
// the chip ("split-K").  Each split writes a partial (O, LSE) normalised over
// its keys to the workspace; the combine kernel merges a row's partials
// exactly: LSE = log sum_s e^{LSE_s}, O = sum_s e^{LSE_s - LSE} O_s.
// A work-group stages one tile at a time (37 KiB of LDS), so four of them fit
// on a CU: the bytes in flight that keep HBM busy come from four work-groups
// per CU copying at once, more than two double-buffered ones would have.
#include "fa_fwd_tile.hpp"

namespace fa {

namespace {

using namespace fwdtile;

template <int D, bool CAUSAL, bool F16>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) char k_st0[C::KT];
  __shared__ __attribute__((aligned(1024))) char v_st0[C::VT];

  const int lane = threadIdx.x;
  const int g = lane >> 5, ln = lane & 31;
  const int split = blockIdx.x;
  const int bhk = blockIdx.y;
  const int b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const int G = a.Hq / a.Hkv, Lq = a.Lq;
  const int R = G * Lq;
  // valid cache length of this sequence, clamped so that every access stays
  // inside the cache even for an out-of-range entry
  int n = a.cache_len != nullptr ? a.cache_len[b] : a.Lk;
  n = __builtin_amdgcn_readfirstlane(min(max(n, Lq), a.Lk));

  // this lane's row: query head hk*G + r/Lq, new token r%Lq (rows >= R are padding)
  const int r = ln;
  const bool valid = r < R;
  const int hq = hk * G + (valid ? r / Lq : 0);
  const int t = valid ? r % Lq : Lq - 1;
  const int my_pos = n - Lq + t;
  const int min_pos = n - Lq, max_pos = n - 1;

  // keys of this split that any row may see
  const int s_lo = split * a.split_keys;
  const int k_hi = min(n, s_lo + a.split_keys);   // causal: every row sees up to n - 1
  const int k_lo = max(s_lo, (a.window > 0) ? max(0, min_pos - a.window + 1) : 0);
  const bool empty = k_hi <= k_lo;
  const int j_lo = empty ? 0 : k_lo / C::BC, j_hi = empty ? -1 : (k_hi - 1) / C::BC;

  const size_t kv_off = ((size_t)(b * a.Hkv + hk) * a.Lk) * D;
  const unsigned head_bytes = (unsigned)a.Lk * (2 * D);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(reinterpret_cast<const bf16*>(a.k) + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(reinterpret_cast<const bf16*>(a.v) + kv_off, head_bytes);

  // one wave issues every 1 KiB copy of a tile; the per-lane source offsets are loop-invariant
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

  FwdState<D> st;
  const bf16* Qr = reinterpret_cast<const bf16*>(a.q) + ((size_t)((b * a.Hq + hq) * Lq + t)) * D;
#pragma unroll
  for (int k = 0; k < C::NSTEP; ++k) st.qr[k] = valid ? *reinterpret_cast<const bf16x8*>(Qr + 16 * k + 8 * g) : bf16x8{};
  st.m_run = kNegBig;
  st.l_run = 0.f;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) st.o[db] = f32x16{};
  const float c = a.scale_log2;

  // the window of a decode call is one-sided (causal): the key range above
  // already ends at the newest entry
  auto tile_mask = [&](int k0) { return range_tile_needs_mask<CAUSAL, C::BC>(k0, n, a.window, min_pos, max_pos); };
  const RangeMaskQ<CAUSAL> ok{n, a.window, my_pos};

  // one stage: the work-group copies a tile, waits, computes; four such
  // work-groups per CU keep several tiles in flight
  for (int j = j_lo; j <= j_hi; ++j) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue(j, k_st0, v_st0);
    wait_copies_and_barrier();
    fwd_tile<D, F16>(st, k_st0, v_st0, j * C::BC, tile_mask(j * C::BC), ok, c, lane);
  }

  // partial for this split: O normalised over its keys (fp32), LSE in ln units
  // (-inf and O = 0 when the split holds no key the row may see)
  const float l_tot = pair_sum(st.l_run);
  if (valid) {
    const size_t row = (size_t)(b * a.Hq + hq) * Lq + t;
    const size_t prow = (size_t)split * a.rows + row;
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
  for (int s = t; s < a.n_splits; s += 256) m = fmaxf(m, a.part_lse[(size_t)s * a.rows + row]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((t & 63) == 0) wmax[t >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  // 2. this group's splits, weighted by e^{LSE_s - m}
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (m != -INFINITY) {
    for (int s = grp; s < a.n_splits; s += kGroups) {
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

template <int D, bool CAUSAL, bool F16>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<D, CAUSAL, F16>), dim3(a.n_splits, a.B * a.Hkv), dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D, F16>), dim3((unsigned)a.rows), dim3(256), 0, stream, a);
  return hipGetLastError();
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

hipError_t launch_decode(const DecodeArgs& a, bool causal, hipStream_t stream) {
  if (a.d == 128) {
    if (a.f16) return causal ? launch_typed<128, true, true>(a, stream) : launch_typed<128, false, true>(a, stream);
    return causal ? launch_typed<128, true, false>(a, stream) : launch_typed<128, false, false>(a, stream);
  }
  if (a.f16) return causal ? launch_typed<64, true, true>(a, stream) : launch_typed<64, false, true>(a, stream);
  return causal ? launch_typed<64, true, false>(a, stream) : launch_typed<64, false, false>(a, stream);
}

}  // namespace fa
