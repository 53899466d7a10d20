// fa_fwd_tile.hpp -- the forward's per-tile machinery, shared by the
// whole-sequence / chunk-pair forward kernel, the decode kernel and the
// mask-plan forward kernels.
//
// For one 64-key tile staged in LDS (padded rows, filled by direct
// buffer->LDS copies) and one wave's 32 query columns:
//   1. S^T = K Q^T on MFMA (keys as rows, queries as columns: every lane then
//      holds 32 scores of ONE query),
//   2. masks the scores (only on tiles that straddle a boundary),
//   3. runs the online-softmax update in registers -- running maximum m and
//      running sum l per query, rescale of the partial output by
//      exp(m_old - m_new) (transformer.xph.ink "高效注意力：FlashAttention 与
//      线性注意力", 原理与机制; claspmoon.cn "14 · 缩放定律与高效注意力" §3.2),
//   4. O^T += V^T P^T on MFMA, with P^T fed straight from step 1's result
//      registers and V^T read with the gfx950 transposing LDS read.
// The work is done in base 2: scores are multiplied by s*log2(e) and exp2 is
// the hardware v_exp_f32.
#pragma once

#include "fa_common.hpp"
#include "fa_kernels.h"

namespace fa {
namespace fwdtile {

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
  static constexpr int NSTEP = D / 16;            // MFMA K-steps over the head dim
  static constexpr int NDB = D / 32;              // 32-wide blocks of the head dim
  static_assert(KT % 1024 == 0 && VT % 1024 == 0, "padded tiles must split into 1 KiB copies");
};

// Loop-invariant per-lane source offsets of this wave's share of a tile copy,
// for a work-group of NW waves.  Copy n (0 <= n < COPIES) belongs to wave
// n % NW and fills tile bytes [1024n, 1024n + 1024).
template <int D, int NW = 4>
struct CopyPlan {
  static constexpr int KPER = (FwdCfg<D>::KCOPIES + NW - 1) / NW;   // copies per wave (at most)
  static constexpr int VPER = (FwdCfg<D>::VCOPIES + NW - 1) / NW;
  int koff[KPER];
  int voff[VPER];
};

template <int D, int NW = 4>
__device__ __forceinline__ void make_copy_plan(CopyPlan<D, NW>& cp, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < CopyPlan<D, NW>::KPER; ++i) cp.koff[i] = pad_slot_src<D, Pad<D>::KSTR>((wave + NW * i) * 64 + lane);
#pragma unroll
  for (int i = 0; i < CopyPlan<D, NW>::VPER; ++i) cp.voff[i] = pad_slot_src<D, Pad<D>::VSTR>((wave + NW * i) * 64 + lane);
}

// This wave's share of the copy of K rows [k0, k0 + 64) into one LDS stage
// (rows past the end of the buffer resource read zeros); V likewise.
template <int D, int NW = 4>
__device__ __forceinline__ void issue_k(const CopyPlan<D, NW>& cp, __amdgpu_buffer_rsrc_t kr, int k0, char* kbuf, int wave) {
  constexpr int COPIES = FwdCfg<D>::KCOPIES;
  const int soff = k0 * (2 * D);
#pragma unroll
  for (int i = 0; i < CopyPlan<D, NW>::KPER; ++i)
    if (owns_copy<NW, COPIES>(wave, i)) buf2lds16(kr, cp.koff[i], soff, kbuf + (wave + NW * i) * 1024);
}

template <int D, int NW = 4>
__device__ __forceinline__ void issue_v(const CopyPlan<D, NW>& cp, __amdgpu_buffer_rsrc_t vr, int k0, char* vbuf, int wave) {
  constexpr int COPIES = FwdCfg<D>::VCOPIES;
  const int soff = k0 * (2 * D);
#pragma unroll
  for (int i = 0; i < CopyPlan<D, NW>::VPER; ++i)
    if (owns_copy<NW, COPIES>(wave, i)) buf2lds16(vr, cp.voff[i], soff, vbuf + (wave + NW * i) * 1024);
}

// Copy K and V rows [k0, k0 + 64) into one LDS stage.
template <int D, int NW = 4>
__device__ __forceinline__ void issue_kv(const CopyPlan<D, NW>& cp, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                         int k0, char* kbuf, char* vbuf, int wave) {
  issue_k<D, NW>(cp, kr, k0, kbuf, wave);
  issue_v<D, NW>(cp, vr, k0, vbuf, wave);
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

// 1. S^T (64 keys x 32 queries) for one key tile staged in LDS, as two 32x32
// blocks: s0 keys 0..31, s1 keys 32..63 of the tile.
template <int D, bool F16>
__device__ __forceinline__ void tile_scores(const FwdState<D>& st, const char* kbuf, int lane, f32x16& s0, f32x16& s1) {
  using C = FwdCfg<D>;
  const int g = lane >> 5, ln = lane & 31;
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
}

// 2.-3. Mask (only when need_mask, wave-uniform: the tile straddles a mask
// boundary; ok(j) then says whether key j is visible to the lane's query) and
// online-softmax update; the probabilities leave as the 16-bit B operand pb of
// the P.V product.
//
// The two lanes holding one query share the tile maximum.  The running maximum
// m is only raised when the tile's maximum exceeds it by more than
// kRescaleSlack (log2 units); otherwise the tile is exponentiated against the
// old m, so its terms are at most 2^kRescaleSlack.  O and l share that m, which
// cancels in O / l and is folded into the log-sum-exp, so the result is the
// same softmax; the rescale of O (and l) by exp2(m_old - m_new) then runs only
// when some lane raised its maximum.
template <int D, bool F16, class Mask>
__device__ __forceinline__ void tile_softmax(FwdState<D>& st, f32x16& s0, f32x16& s1, int k0, bool need_mask,
                                             const Mask& ok, float c, int lane, bf16x8 (&pb)[4]) {
  using C = FwdCfg<D>;
  const int g = lane >> 5;
  if (need_mask) {
    with_mask(ok, k0 + 4 * g, [&](const auto& m) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = 8 * (i >> 2) + (i & 3);
        s0[i] = keep_or(s0[i], m(c), -INFINITY);
        s1[i] = keep_or(s1[i], m(c + 32), -INFINITY);
      }
    });
  }
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
  pb[0] = pack8<F16>(s0[0], s0[1], s0[2], s0[3], s0[4], s0[5], s0[6], s0[7]);
  pb[1] = pack8<F16>(s0[8], s0[9], s0[10], s0[11], s0[12], s0[13], s0[14], s0[15]);
  pb[2] = pack8<F16>(s1[0], s1[1], s1[2], s1[3], s1[4], s1[5], s1[6], s1[7]);
  pb[3] = pack8<F16>(s1[8], s1[9], s1[10], s1[11], s1[12], s1[13], s1[14], s1[15]);
}

// 4. O^T += V^T P^T, 16 keys per MFMA step.  P^T's K slots (from the C layout
// of step 1) are keys 16t + 8*(slot/4) + 4g + slot%4; the transposing read
// gives V^T the same keys.
template <int D, bool F16>
__device__ __forceinline__ void tile_pv(FwdState<D>& st, const char* vbuf, const bf16x8 (&pb)[4], int lane) {
  using C = FwdCfg<D>;
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

// One key tile for one wave: S^T, mask, online softmax, O^T += V^T P^T.
template <int D, bool F16, class Mask>
__device__ __forceinline__ void fwd_tile(FwdState<D>& st, const char* kbuf, const char* vbuf, int k0,
                                         bool need_mask, const Mask& ok, float c, int lane) {
  f32x16 s0, s1;
  tile_scores<D, F16>(st, kbuf, lane, s0, s1);
  bf16x8 pb[4];
  tile_softmax<D, F16>(st, s0, s1, k0, need_mask, ok, c, lane, pb);
  tile_pv<D, F16>(st, vbuf, pb, lane);
}

}  // namespace fwdtile
}  // namespace fa
