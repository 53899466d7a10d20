// fa_bwd_tile.hpp -- the backward's per-tile machinery, shared by the
// range-tiled kernels (whole sequence, chunk pairs) and the kernels driven by
// a mask plan.
//
// dK/dV: a work-group of 8 waves owns 128 keys; wave w owns the 32 keys of
// block w % 4 and the 32-query half w / 4 of every streamed 64-query tile.  K
// and V of the work-group's keys sit in LDS in padded rows (read row-wise
// only); the streamed Q and dO tiles are read both row-wise and by the
// transposing read, so they use the swz_dual layout.
// dQ: a work-group of 4 waves owns 128 queries (32 per wave) and streams
// 64-key tiles; the K tile is read row-wise and transposed (swz_dual), the V
// tile row-wise only (padded).
// Every LDS address is a loop-invariant per-lane offset plus an immediate.
#pragma once

#include "fa_common.hpp"
#include "fa_kernels.h"

namespace fa {
namespace bwdtile {

template <int D>
struct KVCfg {
  static constexpr int kWaves = 8;
  static constexpr int BK = 128;                 // keys per work-group
  static constexpr int BQ = 64;                  // queries per streamed tile
  static constexpr int QT = BQ * D * 2;          // bytes of a Q (or dO) tile (swz_dual)
  static constexpr int KB = BK * Pad<D>::KSTR;   // bytes of the padded K (or V) block
  static constexpr int QCOPIES = QT / 1024;
  static constexpr int QPER = QCOPIES / kWaves;  // copies per wave per tensor
  static constexpr int KBCOPIES = KB / 1024;
  static constexpr int NSTEP = D / 16;
  static constexpr int NDB = D / 32;
  static_assert(QCOPIES % kWaves == 0 && KB % 1024 == 0, "tiles must split into whole wave copies");
};

template <int D>
struct KVState {
  f32x16 dv[KVCfg<D>::NDB];     // dV accumulator: lane = head-dim column, registers = keys
  f32x16 dk[KVCfg<D>::NDB];     // dK accumulator (scale applied at the end)
};

// Loop-invariant per-lane offsets of one wave.
template <int D>
struct KVAddr {
  int qcopy[KVCfg<D>::QPER];           // source offsets of this wave's Q / dO tile copies
  int row[KVCfg<D>::NSTEP];            // row reads of the wave's 32 queries, per K-step
  int tr[KVCfg<D>::NDB][2];            // transposing reads (t = 2*qh), per column block and half
  int kv;                              // row reads of the wave's 32 keys in the padded K/V block
};

// Key-major element mask of the range-tiled kernels: the lane's key j is
// fixed; query row q sits at key position q + shift (visibility as range_ok).
template <bool CAUSAL>
struct RangeMaskK {
  int L, shift, window, j;
  __device__ __forceinline__ bool operator()(int q) const {
    const int i = q + shift;
    return q < L && (!CAUSAL || j <= i) && (window <= 0 || (i - j < window && (CAUSAL || j - i < window)));
  }
};

// One streamed 64-query tile for one wave of the dK/dV kernel.  need_mask
// (wave-uniform) says whether the wave's 32 x 32 block straddles a mask
// boundary; ok(q) then says whether query row q sees the lane's key.
template <int D, bool F16, class Mask>
__device__ __forceinline__ void kv_tile(KVState<D>& st, const KVAddr<D>& ad, const char* kblk, const char* vblk,
                                        const char* qbuf, const char* dobuf, const float* stats, int q0,
                                        bool need_mask, const Mask& ok, int qh, float c, int lane) {
  using C = KVCfg<D>;
  const int g = lane >> 5;

  // S = Q K^T (32 queries x 32 keys): lane = key, registers = queries
  f32x16 p = mfma32x<F16>(lds_load16(qbuf, ad.row[0]), lds_load16(kblk, ad.kv), f32x16{});
#pragma unroll
  for (int k = 1; k < C::NSTEP; ++k)
    p = mfma32x<F16>(lds_load16(qbuf, ad.row[k]), lds_load16(kblk, ad.kv + 32 * k), p);

  // P = exp2(S*s*log2e - LSE*log2e), zero where masked
  const int qw0 = q0 + 32 * qh;           // first query of this wave's half
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const f32x4 l4 = *(const FA_LDS f32x4*)((const FA_LDS char*)(stats) + 4 * (32 * qh + 8 * i4 + 4 * g));
#pragma unroll
    for (int j = 0; j < 4; ++j) p[4 * i4 + j] = fast_exp2(fmaf(p[4 * i4 + j], c, -l4[j]));
  }
  // the mask as a separate pass, so that the common unmasked tile stays one
  // straight-line block
  if (need_mask) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = qw0 + 8 * (i >> 2) + 4 * g + (i & 3);
      p[i] = ok(q) ? p[i] : 0.f;
    }
  }
  // dV += P^T dO: A = P (lane = key, K slots = queries), B = dO via the transposing read
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int o8 = 8 * u;
    const bf16x8 pa = pack8<F16>(p[o8 + 0], p[o8 + 1], p[o8 + 2], p[o8 + 3], p[o8 + 4], p[o8 + 5], p[o8 + 6], p[o8 + 7]);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const bf16x8 bo = concat4(lds_load_tr(dobuf, ad.tr[db][0] + u * 16 * (2 * D)),
                                lds_load_tr(dobuf, ad.tr[db][1] + u * 16 * (2 * D)));
      st.dv[db] = mfma32x<F16>(pa, bo, st.dv[db]);
    }
  }
  // dP = dO V^T, then dS = P * (dP - D) in place
  f32x16 dp = mfma32x<F16>(lds_load16(dobuf, ad.row[0]), lds_load16(vblk, ad.kv), f32x16{});
#pragma unroll
  for (int k = 1; k < C::NSTEP; ++k)
    dp = mfma32x<F16>(lds_load16(dobuf, ad.row[k]), lds_load16(vblk, ad.kv + 32 * k), dp);
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const f32x4 d4 = *(const FA_LDS f32x4*)((const FA_LDS char*)(stats) + 4 * (C::BQ + 32 * qh + 8 * i4 + 4 * g));
#pragma unroll
    for (int j = 0; j < 4; ++j) p[4 * i4 + j] *= dp[4 * i4 + j] - d4[j];
  }
  // dK += dS^T Q: A = dS (lane = key), B = Q via the transposing read
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int o8 = 8 * u;
    const bf16x8 da = pack8<F16>(p[o8 + 0], p[o8 + 1], p[o8 + 2], p[o8 + 3], p[o8 + 4], p[o8 + 5], p[o8 + 6], p[o8 + 7]);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const bf16x8 bq = concat4(lds_load_tr(qbuf, ad.tr[db][0] + u * 16 * (2 * D)),
                                lds_load_tr(qbuf, ad.tr[db][1] + u * 16 * (2 * D)));
      st.dk[db] = mfma32x<F16>(da, bq, st.dk[db]);
    }
  }
}

template <int D>
struct QCfg {
  static constexpr int kWaves = 4;
  static constexpr int BQ = 32 * kWaves;         // queries per work-group
  static constexpr int BC = 64;                  // keys per streamed tile
  static constexpr int KT = BC * D * 2;          // bytes of a K tile (swz_dual)
  static constexpr int VT = BC * Pad<D>::KSTR;   // bytes of a padded V tile
  static constexpr int KCOPIES = KT / 1024;
  static constexpr int VCOPIES = VT / 1024;
  static constexpr int KPER = KCOPIES / kWaves;
  static constexpr int VPER = (VCOPIES + kWaves - 1) / kWaves;
  static constexpr int NSTEP = D / 16;
  static constexpr int NDB = D / 32;
  static_assert(KCOPIES % kWaves == 0 && VT % 1024 == 0, "tiles must split into whole wave copies");
};

template <int D>
struct QState {
  bf16x8 qr[QCfg<D>::NSTEP];    // this wave's 32 Q rows (B operand of S^T = K Q^T)
  bf16x8 dor[QCfg<D>::NSTEP];   // this wave's 32 dO rows (B operand of dP^T = V dO^T)
  f32x16 dq[QCfg<D>::NDB];      // dQ^T accumulator: lane = query, registers = head dims
  float lse2, dlt;              // this lane's query statistics
};

template <int D>
struct QAddr {
  int kcopy[QCfg<D>::KPER];     // source offsets of this wave's K tile copies (swz_dual)
  int vcopy[QCfg<D>::VPER];     // source offsets of this wave's V tile copies (padded)
  int krow[QCfg<D>::NSTEP];     // row reads of K rows ln (+32 per key half), per K-step
  int ktr[QCfg<D>::NDB][2];     // transposing reads of K (t = 0), per column block and half
  int vrow;                     // row reads of padded V rows ln (+32 per key half)
};

// One streamed 64-key tile for one wave of the dQ kernel; need_mask and ok as
// in the forward's tile step.
template <int D, bool F16, class Mask>
__device__ __forceinline__ void q_tile(QState<D>& st, const QAddr<D>& ad, const char* kbuf, const char* vbuf, int k0,
                                       bool need_mask, const Mask& ok, float c, int lane) {
  using C = QCfg<D>;
  const int g = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    // S^T = K Q^T for keys 32kb..32kb+31: lane = query, registers = keys
    f32x16 p = mfma32x<F16>(lds_load16(kbuf, ad.krow[0] + kb * 32 * (2 * D)), st.qr[0], f32x16{});
#pragma unroll
    for (int k = 1; k < C::NSTEP; ++k)
      p = mfma32x<F16>(lds_load16(kbuf, ad.krow[k] + kb * 32 * (2 * D)), st.qr[k], p);
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = fast_exp2(fmaf(p[i], c, -st.lse2));
    if (need_mask) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = k0 + 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
        p[i] = ok(kk) ? p[i] : 0.f;
      }
    }
    // dP^T = V dO^T, dS^T = P^T * (dP^T - D)
    f32x16 dp = mfma32x<F16>(lds_load16(vbuf, ad.vrow + kb * 32 * Pad<D>::KSTR), st.dor[0], f32x16{});
#pragma unroll
    for (int k = 1; k < C::NSTEP; ++k)
      dp = mfma32x<F16>(lds_load16(vbuf, ad.vrow + kb * 32 * Pad<D>::KSTR + 32 * k), st.dor[k], dp);
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] *= dp[i] - st.dlt;
    // dQ^T += K^T dS^T: A = K^T via the transposing read, B = dS^T (lane = query)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int o8 = 8 * u;
      const int t = 2 * kb + u;
      const bf16x8 db8 = pack8<F16>(p[o8 + 0], p[o8 + 1], p[o8 + 2], p[o8 + 3], p[o8 + 4], p[o8 + 5],
                                   p[o8 + 6], p[o8 + 7]);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const bf16x8 ka = concat4(lds_load_tr(kbuf, ad.ktr[db][0] + t * 16 * (2 * D)),
                                  lds_load_tr(kbuf, ad.ktr[db][1] + t * 16 * (2 * D)));
        st.dq[db] = mfma32x<F16>(ka, db8, st.dq[db]);
      }
    }
  }
}

}  // namespace bwdtile
}  // namespace fa
