// fa_fwd_bf16.hip -- tiled exact attention forward, bf16 in, fp32 accumulate (gfx950).
//
// One work-group of 4 waves owns 128 query rows of one (batch, query head);
// each wave owns 32 of them.  The work-group streams the allowed 64-key tiles
// of K and V through LDS (double-buffered, filled by direct buffer->LDS copies
// while the previous tile is being used), and for every tile each wave
//   1. S^T = K Q^T on MFMA (keys as rows, the wave's 32 queries as columns:
//      every lane then holds 32 scores of ONE query),
//   2. masks the scores (only on tiles that straddle the causal diagonal, an
//      edge of the window or the end of the sequence),
//   3. runs the online-softmax update in registers -- running maximum m and
//      running sum l per query, rescale of the partial output by
//      exp(m_old - m_new) (transformer.xph.ink "高效注意力：FlashAttention 与
//      线性注意力", 原理与机制; claspmoon.cn "14 · 缩放定律与高效注意力" §3.2),
//   4. O^T += V^T P^T on MFMA, with P^T fed straight from step 1's result
//      registers and V^T read with the gfx950 transposing LDS read.
// The work is done in base 2: scores are multiplied by s*log2(e) and exp2 is
// the hardware v_exp_f32; the saved log-sum-exp is converted back to ln.
// Only O and the per-row log-sum-exp are written (claspmoon.cn §3.3).
//
// The vector ALU work of a tile adds to its matrix-core time more than it
// hides under it (the products and the softmax depend on each other within a
// wave, and the second wave of a SIMD covers only part of it), so the kernel
// keeps the per-tile VALU instruction count close to the softmax itself: padded LDS rows make every operand address a per-lane base
// plus an immediate, the copies use buffer loads with loop-invariant lane
// offsets (past-the-end rows read as zeros, no clamping), the pair of lanes
// holding one query exchange values with v_permlane32_swap, and the running
// maximum is only raised (and O rescaled) when a tile's maximum exceeds it by
// a wide margin.  (Summing the bf16-rounded probabilities with v_dot2 would
// halve the row-sum instructions, but moves the log-sum-exp of short rows by
// up to 2^-9 relative, beyond its tolerance; the sum stays fp32.)
#include "fa_fwd_tile.hpp"

namespace fa {

namespace {

using namespace fwdtile;

template <int D, bool CAUSAL, bool F16>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  // Four distinct LDS objects (K and V of two stages): distinct objects carry
  // distinct alias scopes, which lets the compiler see that reading one stage
  // does not have to wait for the direct copies into the other.
  __shared__ __attribute__((aligned(1024))) char k_st0[C::KT];
  __shared__ __attribute__((aligned(1024))) char v_st0[C::VT];
  __shared__ __attribute__((aligned(1024))) char k_st1[C::KT];
  __shared__ __attribute__((aligned(1024))) char v_st1[C::VT];

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int g = lane >> 5, ln = lane & 31;

  // ---- work decomposition: heads in pairs, heaviest query tiles first
  const int r = xcd_remap(blockIdx.x, gridDim.x);
  int bh, qt_rank;
  head_tile_of(r, a.B * a.Hq, a.n_qtiles, bh, qt_rank);
  const int qt = CAUSAL ? a.n_qtiles - 1 - qt_rank : qt_rank;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  // L query rows; Lk keys; query row i sits at key position i + shift (the
  // chunks of a ring step), so every mask compares key j with i + shift
  const int L = a.L, Lk = a.Lk, shift = a.shift;

  const bf16* __restrict__ Qh = reinterpret_cast<const bf16*>(a.q) + ((size_t)(b * a.Hq + h) * L) * D;
  const size_t kv_off = ((size_t)(b * a.Hkv + hk) * Lk) * D;
  const unsigned head_bytes = (unsigned)Lk * (2 * D);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(reinterpret_cast<const bf16*>(a.k) + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(reinterpret_cast<const bf16*>(a.v) + kv_off, head_bytes);

  const int q_wg0 = qt * C::BR;
  const int q_w0 = q_wg0 + 32 * wave;
  const int my_q = q_w0 + ln;
  const int wq_hi = min(q_w0 + 31, L - 1);
  // the same three in key coordinates
  const int dq_w0 = q_w0 + shift, dmy_q = my_q + shift, dwq_hi = wq_hi + shift;
  const int window = a.window;

  // ---- key-tile range of the work-group
  const int kv_end = range_key_end<CAUSAL>(Lk, window, min(L, q_wg0 + C::BR) - 1 + shift);
  const int kv_begin = (window > 0) ? max(0, q_wg0 + shift - window + 1) : 0;
  const bool empty = kv_end <= kv_begin;     // possible between chunks of a ring step
  const int j_lo = empty ? 0 : kv_begin / C::BC, j_hi = empty ? -1 : (kv_end - 1) / C::BC;

  CopyPlan<D> cp;
  make_copy_plan<D>(cp, wave, lane);
  if (!empty) issue_kv<D>(cp, krs, vrs, j_lo * C::BC, k_st0, v_st0, wave);

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

  auto wave_needs = [&](int k0) { return (q_w0 < L) && range_tile_any<CAUSAL, C::BC>(k0, window, dq_w0, dwq_hi); };
  auto tile_mask = [&](int k0) { return range_tile_needs_mask<CAUSAL, C::BC>(k0, Lk, window, dq_w0, dwq_hi); };
  const RangeMaskQ<CAUSAL> ok{Lk, window, dmy_q};

  wait_copies_and_barrier();
  // Tiles alternate between the two stages; the loop is unrolled by two so
  // that every LDS access names its stage statically.
  for (int j = j_lo; j <= j_hi; j += 2) {
    if (j < j_hi) issue_kv<D>(cp, krs, vrs, (j + 1) * C::BC, k_st1, v_st1, wave);
    if (wave_needs(j * C::BC))
      fwd_tile<D, F16>(st, k_st0, v_st0, j * C::BC, tile_mask(j * C::BC), ok, c, lane);
    wait_copies_and_barrier();
    if (j + 1 > j_hi) break;
    if (j + 1 < j_hi) issue_kv<D>(cp, krs, vrs, (j + 2) * C::BC, k_st0, v_st0, wave);
    if (wave_needs((j + 1) * C::BC))
      fwd_tile<D, F16>(st, k_st1, v_st1, (j + 1) * C::BC, tile_mask((j + 1) * C::BC), ok, c, lane);
    wait_copies_and_barrier();
  }

  // ---- epilogue: O = O_acc / l, LSE = (m + log2 l) * ln 2; a row that saw no
  // allowed key (only between chunks of a ring step) gets O = 0, LSE = -inf
  const float l_tot = pair_sum(st.l_run);
  if (my_q < L) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    bf16* Oq = reinterpret_cast<bf16*>(a.o) + ((size_t)(b * a.Hq + h) * L + my_q) * D;
    store_row_c<F16, C::NDB>(Oq, st.o, inv, g);
    if (a.lse != nullptr && g == 0)
      a.lse[(size_t)(b * a.Hq + h) * L + my_q] = l_tot > 0.f ? (st.m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL, bool F16>
hipError_t launch(const FwdArgs& args, hipStream_t stream) {
  using C = FwdCfg<D>;
  FwdArgs a = args;
  a.n_qtiles = (a.L + C::BR - 1) / C::BR;
  const long long nblk = (long long)a.B * a.Hq * a.n_qtiles;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, F16>), dim3((unsigned)nblk), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <bool F16>
hipError_t launch_typed(const FwdArgs& a, bool causal, hipStream_t stream) {
  if (a.d == 128) return causal ? launch<128, true, F16>(a, stream) : launch<128, false, F16>(a, stream);
  return causal ? launch<64, true, F16>(a, stream) : launch<64, false, F16>(a, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, bool causal, hipStream_t stream) {
  return a.f16 ? launch_typed<true>(a, causal, stream) : launch_typed<false>(a, causal, stream);
}

}  // namespace fa
