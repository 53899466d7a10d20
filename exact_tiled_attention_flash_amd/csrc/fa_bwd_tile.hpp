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

// Compact addressing of swz_dual tiles (the fused backward, whose larger
// register state leaves no room for one offset per read): every offset is a
// per-lane base plus (a loop-invariant multiple of the step) XOR a per-lane
// swizzle term, one v_xad_u32 per read.
//   row read, head dims 16k + 8g .. +7 of row r:
//     r * 2D + ((2k + g) ^ swz) * 16 = [r * 2D + ((g ^ swz0) << 4)] + ((32k) ^ ((swz & ~1) << 4))
//   transposing read, column block db (16-byte chunk 4db + c, c < 4):
//     [row * 2D + ((c ^ (swz & 3)) << 4) + 8 * (col bit 2)] + ((64 db) ^ ((swz & ~3) << 4))
template <int D>
struct DualRow {
  int base, swz;
  __device__ __forceinline__ void init(int r, int g) {
    const int sw = swz_dual<D>(r);
    base = r * (2 * D) + ((g ^ (sw & 1)) << 4);
    swz = (sw & ~1) << 4;
  }
  __device__ __forceinline__ int at(int k) const { return base + ((32 * k) ^ swz); }
};
template <int D>
struct DualTr {
  int base, swz;
  // the lanes' 8-byte pieces for key step t, half h (tr_offset_dual with db = 0)
  __device__ __forceinline__ void init(int t, int h, int lane) {
    const int s16 = lane & 15, jg = lane >> 4;
    const int row = 16 * t + 8 * h + 4 * (lane >> 5) + (s16 >> 2);
    const int col = 16 * (jg & 1) + 4 * (s16 & 3);
    const int sw = swz_dual<D>(row);
    base = row * (2 * D) + (((col >> 3) ^ (sw & 3)) << 4) + ((col & 4) << 1);
    swz = (sw & ~3) << 4;
  }
  __device__ __forceinline__ int at(int db) const { return base + ((64 * db) ^ swz); }
};

// Addresses of the fused backward's dK/dV tile: Q / dO rows and transposed
// pieces (swz_dual tiles), the K block's rows (swz_dual), V's rows (padded).
template <int D>
struct KVAddrDual {
  DualRow<D> qrow;        // the wave's 32 queries, row reads
  DualTr<D> qtr[2];       // transposing reads (t = 2*qh), halves 0 and 1
  DualRow<D> krow;        // the wave's 32 keys in the K block
  int kv;                 // the same keys' rows in the padded V block
};

// A work-group barrier that waits for this wave's LDS accesses only (its
// copies in flight keep going: __syncthreads would also wait for those).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// End of a dK/dV work-group: sum the two query halves through LDS and store dV,
// then dK (times the softmax scale s), for the work-group's 128 keys, using
// only the four stage buffers st0..st3 (key block kb uses st<kb>), so that
// the K and V blocks are free for the next copies meanwhile.  Waves 4..7
// deposit their float32 partials (16 bytes per lane and access); waves 0..3
// add them, round, and overwrite their own stage with the block's rows,
// row-major; then all eight waves store the rows to dv_rows / dk_rows (the
// work-group's first row in memory) 16 bytes per lane.  skip(r) says local
// row r is not stored (past the end of the sequence, or written by another
// pass).  Its barriers wait for LDS accesses only; the caller must see every
// wave's reads of the stage buffers done (lds_barrier) before refilling them.
template <int D, bool F16, class Skip>
__device__ __forceinline__ void kv_store(KVState<D>& st, char* st0, char* st1, char* st2, char* st3, char* dk_rows,
                                         char* dv_rows, float s, int kb, int qh, int wave, int lane,
                                         const Skip& skip) {
  using C = KVCfg<D>;
  constexpr int kPart = C::NDB * 16 * 64 * 4;     // bytes per wave per tensor
  constexpr int kRowBytes = 2 * D;
  constexpr int kKbBytes = 32 * kRowBytes;        // one key block's rows
  constexpr int kKbChunks = kKbBytes / 1024;
  static_assert(kPart <= C::QT && kKbBytes <= C::QT && kKbBytes % 1024 == 0, "stage buffers too small");
  // the lane index laundered, so that the per-lane offsets below are formed
  // here and not hoisted out of a caller's loop (and kept or spilled there)
  asm volatile("" : "+v"(lane));
  const int g = lane >> 5, ln = lane & 31;
  char* mine = kb == 0 ? st0 : kb == 1 ? st1 : kb == 2 ? st2 : st3;
  f32x4* part = reinterpret_cast<f32x4*>(mine);
  bf16* rows16 = reinterpret_cast<bf16*>(mine);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if (qh == 1) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x16& acc = pass == 0 ? st.dv[db] : st.dk[db];
          part[(db * 4 + i4) * 64 + lane] = f32x4{acc[4 * i4], acc[4 * i4 + 1], acc[4 * i4 + 2], acc[4 * i4 + 3]};
        }
    }
    lds_barrier();
    if (qh == 0) {
      const float f = pass == 0 ? 1.f : s;
      // The rows overwrite the first kKbBytes of the stage, which hold the
      // partials of column blocks db < kFirst: those are read before any row
      // is written, the others one block at a time.
      constexpr int kFirst = kKbBytes / (16 * 64 * 4);
      auto sum_block = [&](int db, const f32x4 (&o)[4]) __attribute__((always_inline)) {
        // lane holds head-dim column 32*db + ln of keys 8*(i/4) + 4g + i%4 of the block
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x = ((pass == 0 ? st.dv[db][4 * i4 + j] : st.dk[db][4 * i4 + j]) + o[i4][j]) * f;
            rows16[(8 * i4 + 4 * g + j) * D + 32 * db + ln] = pack1<F16>(x);
          }
      };
      f32x4 first[kFirst][4];
#pragma unroll
      for (int db = 0; db < kFirst; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) first[db][i4] = part[(db * 4 + i4) * 64 + lane];
#pragma unroll
      for (int db = 0; db < kFirst; ++db) sum_block(db, first[db]);
#pragma unroll
      for (int db = kFirst; db < C::NDB; ++db) {
        f32x4 o[4];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) o[i4] = part[(db * 4 + i4) * 64 + lane];
        sum_block(db, o);
      }
    }
    lds_barrier();
    char* dst = pass == 0 ? dv_rows : dk_rows;
#pragma unroll
    for (int c = wave; c < 4 * kKbChunks; c += C::kWaves) {
      const int kbc = c / kKbChunks;
      const char* src = kbc == 0 ? st0 : kbc == 1 ? st1 : kbc == 2 ? st2 : st3;
      const int in_kb = (c % kKbChunks) * 1024 + 16 * lane;
      const int off = kbc * kKbBytes + in_kb;
      if (!skip(off / kRowBytes))
        *reinterpret_cast<bf16x8*>(dst + off) = *reinterpret_cast<const bf16x8*>(src + in_kb);
    }
    if (pass == 0) lds_barrier();   // the rows are read before the second pass overwrites the stages
  }
}

// Key-major element mask of the range-tiled kernels: the lane's key j is
// fixed; query row q (of L) sits at key position q + shift and sees j as
// range_ok says, which for rows q >= 0 holds on one run of rows (fresh(): as
// RangeMaskQ's).
template <bool CAUSAL>
struct RangeMaskK {
  int L, shift, window, j;
  __host__ __device__ __forceinline__ PosRun run() const {
    const int p = j - shift;   // the row at the key's own position
    return pos_run(CAUSAL ? max(0, p) : (window > 0 ? max(0, p - window + 1) : 0), window > 0 ? min(L, p + window) : L);
  }
  __host__ __device__ __forceinline__ bool operator()(int q) const { return run()(q); }
  __device__ __forceinline__ PosRun fresh() const {
    RangeMaskK m = *this;
    asm volatile("" : "+v"(m.j));
    return m.run();
  }
};

// One streamed 64-query tile for one wave of the dK/dV kernel.  need_mask
// (wave-uniform) says whether the wave's 32 x 32 block straddles a mask
// boundary; ok(q) then says whether query row q sees the lane's key.
//
// KDUAL: the K block is stored with swz_dual (the fused backward also reads it
// transposed) instead of padded rows.  DS_OUT: also write this wave's dS
// (16-bit) into the dS exchange buffer at dsbuf, for dQ = dS K.
// A copy of the compact addresses that the compiler cannot hoist out of the
// tile loop: offsets derived from it are formed next to their reads instead of
// being precomputed once and kept (or spilled) for the whole kernel.
template <int D>
__device__ __forceinline__ KVAddrDual<D> fresh(const KVAddrDual<D>& ad) {
  KVAddrDual<D> r = ad;
  asm volatile("" : "+v"(r.qrow.base), "+v"(r.qrow.swz), "+v"(r.qtr[0].base), "+v"(r.qtr[0].swz),
               "+v"(r.qtr[1].base), "+v"(r.qtr[1].swz), "+v"(r.krow.base), "+v"(r.krow.swz));
  return r;
}
template <int D>
__device__ __forceinline__ const KVAddr<D>& fresh(const KVAddr<D>& ad) { return ad; }

template <int D>
__device__ __forceinline__ int kv_qrow(const KVAddr<D>& ad, int k) { return ad.row[k]; }
template <int D>
__device__ __forceinline__ int kv_qrow(const KVAddrDual<D>& ad, int k) { return ad.qrow.at(k); }
template <int D>
__device__ __forceinline__ int kv_qtr(const KVAddr<D>& ad, int db, int h) { return ad.tr[db][h]; }
template <int D>
__device__ __forceinline__ int kv_qtr(const KVAddrDual<D>& ad, int db, int h) { return ad.qtr[h].at(db); }
template <int D>
__device__ __forceinline__ int kv_krow(const KVAddr<D>& ad, int k) { return ad.kv + 32 * k; }
template <int D>
__device__ __forceinline__ int kv_krow(const KVAddrDual<D>& ad, int k) { return ad.krow.at(k); }

template <int D, bool F16, bool DS_OUT = false, class Addr, class Mask>
__device__ __forceinline__ void kv_tile(KVState<D>& st, const Addr& ad_in, const char* kblk, const char* vblk,
                                        const char* qbuf, const char* dobuf, const float* stats, int q0,
                                        bool need_mask, const Mask& ok, int qh, float c, int lane,
                                        char* dsbuf = nullptr, int ds_row = 0) {
  using C = KVCfg<D>;
  const auto& ad = fresh<D>(ad_in);
  const int g = lane >> 5;
  auto krow = [&](int k) { return kv_krow<D>(ad, k); };

  // With DS_OUT (the fused backward, short of registers) the operand reads of
  // each MFMA chain run at most two steps ahead of their MFMAs.
  auto chain_order = [&]() {
    if constexpr (DS_OUT) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int k = 0; k < C::NSTEP - 2; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
  };

  // S = Q K^T (32 queries x 32 keys): lane = key, registers = queries
  f32x16 p = mfma32x<F16>(lds_load16(qbuf, kv_qrow<D>(ad, 0)), lds_load16(kblk, krow(0)), f32x16{});
#pragma unroll
  for (int k = 1; k < C::NSTEP; ++k)
    p = mfma32x<F16>(lds_load16(qbuf, kv_qrow<D>(ad, k)), lds_load16(kblk, krow(k)), p);
  chain_order();

  // dP - D = dO V^T - D: the chain starts from the stored -D of each query
  // row (C-layout register i is query row 8(i/4) + 4g + i%4 of the half).
  // It is independent of P, so it is issued before the exponentials below and
  // its products run beside them (one basic block up to the mask branch).
  // (Interleaving the S and dP chains step by step measured 0.4% slower, and
  // S as two chains over the even and odd K-steps 2.5% slower.)
  f32x16 dp;
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const f32x4 d4 = *(const FA_LDS f32x4*)((const FA_LDS char*)(stats) + 4 * (C::BQ + 32 * qh + 8 * i4 + 4 * g));
#pragma unroll
    for (int j = 0; j < 4; ++j) dp[4 * i4 + j] = d4[j];
  }
#pragma unroll
  for (int k = 0; k < C::NSTEP; ++k)
    dp = mfma32x<F16>(lds_load16(dobuf, kv_qrow<D>(ad, k)), lds_load16(vblk, ad.kv + 32 * k), dp);
  chain_order();
  // P = exp2(S*s*log2e - LSE*log2e), zero where masked
  const int qw0 = q0 + 32 * qh;           // first query of this wave's half
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const f32x4 l4 = *(const FA_LDS f32x4*)((const FA_LDS char*)(stats) + 4 * (32 * qh + 8 * i4 + 4 * g));
#pragma unroll
    for (int j = 0; j < 4; ++j) p[4 * i4 + j] = fast_exp2(fmaf(p[4 * i4 + j], c, -l4[j]));
  }
  // the mask as a separate pass, so that the common unmasked tile stays one
  // straight-line block.  Each select is done in place (tied asm operand): a
  // plain select writes new registers, and the join of the two versions of P
  // then costs 16 register copies on the unmasked path.
  if (need_mask) {
    with_mask(ok, qw0 + 4 * g, [&](const auto& m) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = keep_or_zero(p[i], m(8 * (i >> 2) + (i & 3)));
    });
  }
  // dV += P^T dO: A = P (lane = key, K slots = queries), B = dO via the transposing read
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int o8 = 8 * u;
    const bf16x8 pa = pack8<F16>(p[o8 + 0], p[o8 + 1], p[o8 + 2], p[o8 + 3], p[o8 + 4], p[o8 + 5], p[o8 + 6], p[o8 + 7]);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const bf16x8 bo = concat4(lds_load_tr(dobuf, kv_qtr<D>(ad, db, 0) + u * 16 * (2 * D)),
                                lds_load_tr(dobuf, kv_qtr<D>(ad, db, 1) + u * 16 * (2 * D)));
      st.dv[db] = mfma32x<F16>(pa, bo, st.dv[db]);
    }
  }
  // dS = P * (dP - D) in place
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i] *= dp[i];
  // dK += dS^T Q: A = dS (lane = key), B = Q via the transposing read
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int o8 = 8 * u;
    const bf16x8 da = pack8<F16>(p[o8 + 0], p[o8 + 1], p[o8 + 2], p[o8 + 3], p[o8 + 4], p[o8 + 5], p[o8 + 6], p[o8 + 7]);
    if constexpr (DS_OUT) {
      // registers 4*i4 .. 4*i4 + 3 are queries 8*i4 + 4g .. +3 of the half:
      // chunk 8qh + 2*i4 + g of the key's row
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      const i16x8 w = __builtin_bit_cast(i16x8, da);
      *(FA_LDS i16x4*)((FA_LDS char*)dsbuf + ds_offset(ds_row, 8 * qh + 4 * u + g)) =
          __builtin_shufflevector(w, w, 0, 1, 2, 3);
      *(FA_LDS i16x4*)((FA_LDS char*)dsbuf + ds_offset(ds_row, 8 * qh + 4 * u + 2 + g)) =
          __builtin_shufflevector(w, w, 4, 5, 6, 7);
    }
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const bf16x8 bq = concat4(lds_load_tr(qbuf, kv_qtr<D>(ad, db, 0) + u * 16 * (2 * D)),
                                lds_load_tr(qbuf, kv_qtr<D>(ad, db, 1) + u * 16 * (2 * D)));
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
  float lse2;                   // this lane's LSE * log2(e)
  f32x16 negd;                  // this lane's -D in every register: the start of the dP^T chains
  __device__ __forceinline__ void set_stats(float lse2_row, float negd_row) {
    lse2 = lse2_row;
#pragma unroll
    for (int i = 0; i < 16; ++i) negd[i] = negd_row;
  }
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
    // dP^T - D = V dO^T - D (the chain starts from -D); independent of P, so
    // its products can run beside the exponentials
    f32x16 dp = mfma32x<F16>(lds_load16(vbuf, ad.vrow + kb * 32 * Pad<D>::KSTR), st.dor[0], st.negd);
#pragma unroll
    for (int k = 1; k < C::NSTEP; ++k)
      dp = mfma32x<F16>(lds_load16(vbuf, ad.vrow + kb * 32 * Pad<D>::KSTR + 32 * k), st.dor[k], dp);
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = fast_exp2(fmaf(p[i], c, -st.lse2));
    if (need_mask) {
      with_mask(ok, k0 + 32 * kb + 4 * g, [&](const auto& m) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) p[i] = keep_or_zero(p[i], m(8 * (i >> 2) + (i & 3)));
      });
    }
    // dS^T = P^T * (dP^T - D)
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] *= dp[i];
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
