// fa_fwd_bf16.hip -- tiled exact attention forward, bf16 in, fp32 accumulate (gfx950).
//
// One work-group of 4 waves owns 128 query rows of one (batch, query head);
// each wave owns 32 of them.  The work-group streams the allowed 64-key tiles
// of K and V through LDS (double-buffered, filled by direct buffer->LDS copies
// while the previous tile is being used), and for every tile each wave
//   1. S^T = K Q^T on MFMA (keys as rows, the wave's 32 queries as columns:
//      every lane then holds 32 scores of ONE query),
//   2. masks the scores (only on tiles that straddle the causal diagonal, the
//      window's left edge or the end of the sequence),
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
// On gfx950 the vector ALU work of a wave does not hide behind its matrix-core
// work, so the kernel keeps the per-tile VALU instruction count close to the
// softmax itself: padded LDS rows make every operand address a per-lane base
// plus an immediate, the copies use buffer loads with loop-invariant lane
// offsets (past-the-end rows read as zeros, no clamping), the pair of lanes
// holding one query exchange values with v_permlane32_swap, and the running
// maximum is only raised (and O rescaled) when a tile's maximum exceeds it by
// a wide margin.  (Summing the bf16-rounded probabilities with v_dot2 would
// halve the row-sum instructions, but moves the log-sum-exp of short rows by
// up to 2^-9 relative, beyond its tolerance; the sum stays fp32.)
#include "fa_common.hpp"
#include "fa_kernels.h"

namespace fa {

namespace {

// Slack (log2 units) before the running maximum is raised: tile terms stay
// below 2^8 = 256, far from fp32 (and bf16) overflow.
constexpr float kRescaleSlack = 8.0f;

template <int D>
struct FwdCfg {
  static constexpr int kWaves = 4;
  static constexpr int BR = 32 * kWaves;          // query rows per work-group
  static constexpr int BC = 64;                   // keys per K/V tile
  static constexpr int KT = BC * Pad<D>::KSTR;    // bytes of a padded K tile
  static constexpr int VT = BC * Pad<D>::VSTR;    // bytes of a padded V tile
  static constexpr int KCOPIES = KT / 1024;       // wave-wide 1 KiB copies per K tile
  static constexpr int VCOPIES = VT / 1024;
  static constexpr int KPER = (KCOPIES + kWaves - 1) / kWaves;   // copies per wave (at most)
  static constexpr int VPER = (VCOPIES + kWaves - 1) / kWaves;
  static constexpr int NSTEP = D / 16;            // MFMA K-steps over the head dim
  static constexpr int NDB = D / 32;              // 32-wide blocks of the head dim
  static_assert(KT % 1024 == 0 && VT % 1024 == 0, "padded tiles must split into 1 KiB copies");
};

// Loop-invariant per-lane source offsets of this wave's share of a tile copy.
// Copy n (0 <= n < COPIES) belongs to wave n % 4 and fills tile bytes
// [1024n, 1024n + 1024).
template <int D>
struct CopyPlan {
  int koff[FwdCfg<D>::KPER];
  int voff[FwdCfg<D>::VPER];
};

template <int D>
__device__ __forceinline__ void make_copy_plan(CopyPlan<D>& cp, int wave, int lane) {
  using C = FwdCfg<D>;
#pragma unroll
  for (int i = 0; i < C::KPER; ++i) cp.koff[i] = pad_slot_src<D, Pad<D>::KSTR>((wave + 4 * i) * 64 + lane);
#pragma unroll
  for (int i = 0; i < C::VPER; ++i) cp.voff[i] = pad_slot_src<D, Pad<D>::VSTR>((wave + 4 * i) * 64 + lane);
}

// Copy K and V rows [k0, k0 + 64) into one LDS stage (rows past L read zeros).
template <int D>
__device__ __forceinline__ void issue_kv(const CopyPlan<D>& cp, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                         int k0, char* kbuf, char* vbuf, int wave) {
  using C = FwdCfg<D>;
  const int soff = k0 * (2 * D);
#pragma unroll
  for (int i = 0; i < C::KPER; ++i)
    if (wave + 4 * i < C::KCOPIES) buf2lds16(kr, cp.koff[i], soff, kbuf + (wave + 4 * i) * 1024);
#pragma unroll
  for (int i = 0; i < C::VPER; ++i)
    if (wave + 4 * i < C::VCOPIES) buf2lds16(vr, cp.voff[i], soff, vbuf + (wave + 4 * i) * 1024);
}

__device__ __forceinline__ void wait_copies_and_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// Per-wave state carried across key tiles.
template <int D>
struct FwdState {
  bf16x8 qr[FwdCfg<D>::NSTEP];   // the wave's 32 queries (B operand of S^T = K Q^T)
  f32x16 o[FwdCfg<D>::NDB];      // O^T accumulator: lane = query, registers = head dims
  float m_run, l_run;            // running max (log2 units) and this lane's partial sum
};

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// One key tile for one wave: S^T, mask, online softmax, O^T += V^T P^T.
template <int D, bool CAUSAL, bool F16>
__device__ __forceinline__ void fwd_tile(FwdState<D>& st, const char* kbuf, const char* vbuf, int k0,
                                         int Lk, int window, int my_q, int q_w0, int wq_hi, float c,
                                         int lane) {
  using C = FwdCfg<D>;
  const int g = lane >> 5, ln = lane & 31;
  // 1. S^T (64 keys x 32 queries) as two 32x32 blocks
  f32x16 s0, s1;
  {
    const bf16x8 a0 = lds_load16(kbuf, row_offset_kpad<D>(ln, 0, g));
    const bf16x8 a1 = lds_load16(kbuf, row_offset_kpad<D>(32 + ln, 0, g));
    s0 = mfma32x<F16>(a0, st.qr[0], f32x16{});
    s1 = mfma32x<F16>(a1, st.qr[0], f32x16{});
  }
#pragma unroll
  for (int k = 1; k < C::NSTEP; ++k) {
    const bf16x8 a0 = lds_load16(kbuf, row_offset_kpad<D>(ln, k, g));
    const bf16x8 a1 = lds_load16(kbuf, row_offset_kpad<D>(32 + ln, k, g));
    s0 = mfma32x<F16>(a0, st.qr[k], s0);
    s1 = mfma32x<F16>(a1, st.qr[k], s1);
  }

  // 2. mask, only on tiles that straddle a boundary (wave-uniform decision)
  const bool need_mask = (k0 + C::BC > Lk) || (CAUSAL && k0 + C::BC - 1 > q_w0) ||
                         (window > 0 && k0 < wq_hi - window + 1);
  if (need_mask) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk0 = k0 + 8 * (i >> 2) + 4 * g + (i & 3);
      const int kk1 = kk0 + 32;
      const bool ok0 = kk0 < Lk && (!CAUSAL || kk0 <= my_q) && (window <= 0 || kk0 > my_q - window);
      const bool ok1 = kk1 < Lk && (!CAUSAL || kk1 <= my_q) && (window <= 0 || kk1 > my_q - window);
      if (!ok0) s0[i] = -INFINITY;
      if (!ok1) s1[i] = -INFINITY;
    }
  }

  // 3. online softmax: the two lanes holding one query share the tile maximum.
  // The running maximum m is only raised when the tile's maximum exceeds it by
  // more than kRescaleSlack (log2 units); otherwise the tile is exponentiated
  // against the old m, so its terms are at most 2^kRescaleSlack.  O and l share
  // that m, which cancels in O / l and is folded into the log-sum-exp, so the
  // result is the same softmax; the rescale of O (and l) by exp2(m_old - m_new)
  // then runs only when some lane raised its maximum.
  float mA = max3(s0[0], s1[0], s0[1]), mB = max3(s1[1], s0[2], s1[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) {
    mA = max3(mA, s0[i], s1[i]);
    mB = max3(mB, s0[i + 1], s1[i + 1]);
  }
  const float mx = pair_max(max3(mA, mB, fmaxf(s0[15], s1[15])));
  const bool raise = mx * c > st.m_run + kRescaleSlack;
  const float m_new = raise ? mx * c : st.m_run;
  if (__ballot(raise) != 0) {
    const float alpha = fast_exp2(st.m_run - m_new);
    st.l_run *= alpha;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) st.o[db] *= alpha;
    st.m_run = m_new;
  }
  // P = exp2(s*c - m); the row sum is accumulated in fp32 from the unrounded
  // values (two chains), and P is rounded to bf16 for the P.V product.
  float rA = 0.f, rB = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    s0[i] = fast_exp2(fmaf(s0[i], c, -m_new));
    s1[i] = fast_exp2(fmaf(s1[i], c, -m_new));
    rA += s0[i];
    rB += s1[i];
  }
  st.l_run += rA + rB;
  bf16x8 pb[4];
  pb[0] = pack8<F16>(s0[0], s0[1], s0[2], s0[3], s0[4], s0[5], s0[6], s0[7]);
  pb[1] = pack8<F16>(s0[8], s0[9], s0[10], s0[11], s0[12], s0[13], s0[14], s0[15]);
  pb[2] = pack8<F16>(s1[0], s1[1], s1[2], s1[3], s1[4], s1[5], s1[6], s1[7]);
  pb[3] = pack8<F16>(s1[8], s1[9], s1[10], s1[11], s1[12], s1[13], s1[14], s1[15]);

  // 4. O^T += V^T P^T, 16 keys per MFMA step.  P^T's K slots (from the C
  // layout of step 1) are keys 16t + 8*(slot/4) + 4g + slot%4; the transposing
  // read gives V^T the same keys.
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const bf16x4 lo = lds_load_tr(vbuf, tr_offset_vpad<D>(t, db, 0, lane));
      const bf16x4 hi = lds_load_tr(vbuf, tr_offset_vpad<D>(t, db, 1, lane));
      st.o[db] = mfma32x<F16>(concat4(lo, hi), pb[t], st.o[db]);
    }
  }
}

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
  const int kv_end = CAUSAL ? min(Lk, min(L, q_wg0 + C::BR) + shift) : Lk;
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

  auto wave_needs = [&](int k0) {
    return (q_w0 < L) && (!CAUSAL || k0 <= dwq_hi) && (window <= 0 || k0 + C::BC - 1 >= dq_w0 - window + 1);
  };

  wait_copies_and_barrier();
  // Tiles alternate between the two stages; the loop is unrolled by two so
  // that every LDS access names its stage statically.
  for (int j = j_lo; j <= j_hi; j += 2) {
    if (j < j_hi) issue_kv<D>(cp, krs, vrs, (j + 1) * C::BC, k_st1, v_st1, wave);
    if (wave_needs(j * C::BC))
      fwd_tile<D, CAUSAL, F16>(st, k_st0, v_st0, j * C::BC, Lk, window, dmy_q, dq_w0, dwq_hi, c, lane);
    wait_copies_and_barrier();
    if (j + 1 > j_hi) break;
    if (j + 1 < j_hi) issue_kv<D>(cp, krs, vrs, (j + 2) * C::BC, k_st0, v_st0, wave);
    if (wave_needs((j + 1) * C::BC))
      fwd_tile<D, CAUSAL, F16>(st, k_st1, v_st1, (j + 1) * C::BC, Lk, window, dmy_q, dq_w0, dwq_hi, c, lane);
    wait_copies_and_barrier();
  }

  // ---- epilogue: O = O_acc / l, LSE = (m + log2 l) * ln 2; a row that saw no
  // allowed key (only between chunks of a ring step) gets O = 0, LSE = -inf
  const float l_tot = pair_sum(st.l_run);
  if (my_q < L) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    bf16* Oq = reinterpret_cast<bf16*>(a.o) + ((size_t)(b * a.Hq + h) * L + my_q) * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 w;
        w[0] = pack1<F16>(st.o[db][4 * i4 + 0] * inv);
        w[1] = pack1<F16>(st.o[db][4 * i4 + 1] * inv);
        w[2] = pack1<F16>(st.o[db][4 * i4 + 2] * inv);
        w[3] = pack1<F16>(st.o[db][4 * i4 + 3] * inv);
        *reinterpret_cast<bf16x4*>(Oq + 32 * db + 8 * i4 + 4 * g) = w;
      }
    }
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
