// fa_bwd_bf16.hip -- recomputing attention backward, bf16 in, fp32 accumulate (gfx950).
//
// Only O and the per-row log-sum-exp survive the forward; the probabilities
// are recomputed here as P = exp(s*Q K^T - LSE) from Q, K and that statistic
// (claspmoon.cn "14 · 缩放定律与高效注意力" §3.3, backward by recomputation;
// transformer.xph.ink "高效注意力：FlashAttention 与线性注意力", 原理与机制).
// The gradient is the softmax Jacobian applied row by row:
//     dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,  dS = P * (dP - D),
//     dQ = s dS K,  dK = s dS^T Q.
// Three kernels, all on the caller's stream, none using atomics:
//   1. delta:  -D_i and LSE_i*log2(e) per query row into the workspace;
//   2. dK/dV:  one work-group per (batch, K/V head, 128 keys) with its K and
//              V rows staged once in LDS; each of its 8 waves owns 32 keys and
//              one 32-query half of every allowed 64-query tile of Q and dO
//              (every query head of the GQA group) streamed through LDS, and
//              accumulates dK and dV in registers (the two halves are summed
//              through LDS at the end);
//   3. dQ:     one work-group per (batch, query head, 128 queries), each wave
//              holding 32 queries' Q and dO rows in registers, streams the
//              allowed 64-key tiles of K and V through LDS and accumulates dQ.
// The two tile kernels reuse the forward's MFMA layouts: a product whose C
// registers hold one column per lane feeds the next product's A or B operand
// directly, and the operand that needs the other orientation comes from the
// gfx950 transposing LDS read.  As in the forward, every LDS address is a
// loop-invariant per-lane offset plus an immediate and all tile copies are
// buffer->LDS loads, which keeps the VALU work per tile small.
#include "fa_bwd_tile.hpp"

namespace fa {

namespace {

using namespace bwdtile;

__device__ __forceinline__ void wait_copies_and_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// ------------------------------------------------------------ 1. delta

template <int D, bool F16>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const bf16* __restrict__ o, const bf16* __restrict__ dout,
                                                        const float* __restrict__ lse, float* __restrict__ delta,
                                                        float* __restrict__ lse2, float* __restrict__ dq_acc,
                                                        long long rows) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerBlock = 256 / kLanesPerRow;
  const long long row = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const int part = threadIdx.x % kLanesPerRow;
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(o + row * D + part * 8);
    const bf16x8 y = *reinterpret_cast<const bf16x8*>(dout + row * D + part * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(unpack1<F16>(x[i]), unpack1<F16>(y[i]), acc);
    if (dq_acc != nullptr) {
      f32x4* z = reinterpret_cast<f32x4*>(dq_acc + row * D + part * 8);
      z[0] = f32x4{};
      z[1] = f32x4{};
    }
  }
#pragma unroll
  for (int off = kLanesPerRow / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && part == 0) {
    delta[row] = -acc;               // stored negated: the dP chains start from it
    lse2[row] = lse[row] * kLog2e;
  }
}

// ------------------------------------------------------------ 2. dK / dV

// One work-group of 8 waves per (batch, K/V head, 128 keys).  Wave w owns the
// 32 keys of block w % 4 and the 32-query half w / 4 of every streamed 64-query
// tile, so two waves share each SIMD; the halves' partial dK and dV are summed
// through LDS at the end.  K and V of the work-group's keys sit in LDS for the
// whole kernel, in padded rows (they are only read row-wise); the streamed Q
// and dO tiles are read both row-wise and by the transposing read, so they use
// the swz_dual layout.  Every LDS address is a loop-invariant per-lane offset
// plus an immediate, and all copies are buffer->LDS loads (rows past the end
// of the sequence read as zeros).

template <int D, bool CAUSAL, bool F16>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using C = KVCfg<D>;
  // distinct LDS objects per stage so reads of one stage need not wait for the
  // direct copies into the other (alias scopes).  The stage buffers carry the
  // larger alignment so that they are laid out first, in the low 64 KiB: their
  // swizzled per-lane offsets then take the buffer base in the 16-bit
  // immediate of the LDS read instead of a VALU add per read.
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
  // L query rows, Lk keys; query row i sits at key position i + shift
  const int L = a.L, Lk = a.Lk, shift = a.shift, window = a.window;
  const int G = a.Hq / a.Hkv;

  // (batch, K/V head) pairs, key tiles rank by rank within a pair; with
  // causal masking the first key tile sees the most queries, so the heaviest
  // work-groups go first
  const int r = xcd_remap(blockIdx.x, gridDim.x);
  int bhk, kt;
  head_tile_of(r, a.B * a.Hkv, a.n_tiles, bhk, kt);
  const int b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const int key_wg0 = kt * C::BK;
  const int key_w0 = key_wg0 + 32 * kb;

  const size_t kv_off = ((size_t)(b * a.Hkv + hk) * Lk) * D;
  const unsigned head_bytes = (unsigned)Lk * (2 * D);      // one K/V head
  const unsigned qhead_bytes = (unsigned)L * (2 * D);      // one Q/dO head

  // queries that can see this work-group's keys (none: only between chunks)
  const int q_begin = CAUSAL ? max(0, key_wg0 - shift) : (window > 0 ? max(0, key_wg0 - shift - window + 1) : 0);
  const int q_end = (window > 0) ? min(L, key_wg0 + C::BK - 1 + window - shift) : L;
  const bool empty = q_end <= q_begin;
  const int qt_lo = empty ? 0 : q_begin / C::BQ, qt_hi = empty ? -1 : (q_end - 1) / C::BQ;
  const int nq = qt_hi - qt_lo + 1;
  const int n_it = G * nq;

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

  // Iteration it visits query tile qt_lo + it % nq of query head hk*G + it / nq.
  // Both are stepped incrementally (no integer division in the loop): (i_h,
  // i_q) for the next tile to copy, c_q for the tile being computed.
  int i_h = 0, i_q = 0, c_q = 0;
  const bf16* q_head = reinterpret_cast<const bf16*>(a.q) + ((size_t)(b * a.Hq + hk * G) * L) * D;
  const bf16* do_head = reinterpret_cast<const bf16*>(a.dout) + ((size_t)(b * a.Hq + hk * G) * L) * D;
  const float* l_head = a.lse2 + (size_t)(b * a.Hq + hk * G) * L;
  const float* e_head = a.delta + (size_t)(b * a.Hq + hk * G) * L;
  auto issue = [&](char* qs, char* dos, float* ss) {
    const size_t qoff = (size_t)i_h * L * D;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(q_head + qoff, qhead_bytes);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(do_head + qoff, qhead_bytes);
    const int q0 = (qt_lo + i_q) * C::BQ;
    const int soff = q0 * (2 * D);
#pragma unroll
    for (int i = 0; i < C::QPER; ++i) {
      buf2lds16(qrs, ad.qcopy[i], soff, qs + (wave + C::kWaves * i) * 1024);
      buf2lds16(drs, ad.qcopy[i], soff, dos + (wave + C::kWaves * i) * 1024);
    }
    if (wave == 0) {
      const size_t srow = (size_t)i_h * L;
      const __amdgpu_buffer_rsrc_t lrs = make_rsrc(l_head + srow, (unsigned)L * 4);
      const __amdgpu_buffer_rsrc_t ers = make_rsrc(e_head + srow, (unsigned)L * 4);
      buf2lds4(lrs, 4 * lane, 4 * q0, reinterpret_cast<char*>(ss));
      buf2lds4(ers, 4 * lane, 4 * q0, reinterpret_cast<char*>(ss) + 4 * C::BQ);
    }
    if (++i_q == nq) {
      i_q = 0;
      ++i_h;
    }
  };
  auto next_q0 = [&]() {
    const int q0 = (qt_lo + c_q) * C::BQ;
    if (++c_q == nq) c_q = 0;
    return q0;
  };

  // the work-group's K and V rows, once (padded layout; rows past L read zeros)
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
  if (n_it > 0) issue(q_st0, do_st0, stat_st0);

  KVState<D> st;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    st.dv[db] = f32x16{};
    st.dk[db] = f32x16{};
  }
  const float c = a.scale_log2;
  auto wave_needs = [&](int q0) {
    const int qw0 = q0 + 32 * qh;
    return key_w0 < Lk && qw0 < L && (!CAUSAL || qw0 + 31 + shift >= key_w0) &&
           (window <= 0 || qw0 + shift <= key_w0 + 31 + window - 1) &&
           (CAUSAL || window <= 0 || qw0 + 31 + shift >= key_w0 - window + 1);
  };
  // the wave's 32 x 32 block straddles a mask boundary
  auto block_mask = [&](int q0) {
    const int qw0 = q0 + 32 * qh;
    return (qw0 + 32 > L) || (CAUSAL && qw0 + shift < key_w0 + 31) ||
           (window > 0 && qw0 + 31 + shift > key_w0 + window - 1) ||
           (!CAUSAL && window > 0 && qw0 + shift < key_w0 + 31 - window + 1);
  };
  const RangeMaskK<CAUSAL> ok{L, shift, window, key_w0 + ln};

  wait_copies_and_barrier();
  for (int it = 0; it < n_it; it += 2) {
    if (it + 1 < n_it) issue(q_st1, do_st1, stat_st1);
    const int q0a = next_q0();
    if (wave_needs(q0a))
      kv_tile<D, F16>(st, ad, k_blk, v_blk, q_st0, do_st0, stat_st0, q0a, block_mask(q0a), ok, qh, c, lane);
    wait_copies_and_barrier();
    if (it + 1 >= n_it) break;
    if (it + 2 < n_it) issue(q_st0, do_st0, stat_st0);
    const int q0b = next_q0();
    if (wave_needs(q0b))
      kv_tile<D, F16>(st, ad, k_blk, v_blk, q_st1, do_st1, stat_st1, q0b, block_mask(q0b), ok, qh, c, lane);
    wait_copies_and_barrier();
  }

  // Sum the two query halves and store, in the stage buffers (free now):
  // rows 16 bytes per lane rather than 2-byte pieces of the MFMA layout, which
  // made the kernel 1.4% slower.
  const size_t row0 = (size_t)key_wg0 * (2 * D);
  const int n_rows = min(C::BK, Lk - key_wg0);    // rows of this block inside the sequence
  kv_store<D, F16>(st, q_st0, do_st0, q_st1, do_st1,
                   reinterpret_cast<char*>(reinterpret_cast<bf16*>(a.dk) + kv_off) + row0,
                   reinterpret_cast<char*>(reinterpret_cast<bf16*>(a.dv) + kv_off) + row0, a.scale, kb, qh, wave,
                   lane, [&](int r) { return r >= n_rows; });
}

// ------------------------------------------------------------ 2'. fused dK / dV / dQ

// The dK/dV kernel above plus dQ: after each streamed 64-query tile every wave
// writes its 32 x 32 block of dS (16-bit) into an LDS exchange buffer; after a
// barrier, wave 4 + kb computes the two 32 queries x 32 head dims blocks
// (both query halves, head-dim block kb) of dQ = s dS K over all 128 keys of
// the work-group -- 16 MFMAs, dS by the transposing read of the exchange
// buffer, K by the transposing read of the K block (stored with swz_dual for
// this) -- and adds them into the float32 accumulator with atomics.  The
// copies of the streamed tiles are issued by waves 0-3 only, so only those
// wait for their vector-memory counter before the tile barrier; the atomics of
// waves 4-7 drain in the background.  The accumulator is zeroed by the
// preprocess and converted to dQ by bwd_dq_convert_kernel.  This removes the
// dQ kernel's recomputation of S and dP: five products instead of seven.
template <int D, bool CAUSAL, bool F16>
__global__ __launch_bounds__(512, 1) void bwd_fused_kernel(BwdArgs a) {
  using C = KVCfg<D>;
  constexpr int KBD = C::BK * D * 2;                 // K block, swz_dual
  __shared__ __attribute__((aligned(C::QT))) char q_st0[C::QT];
  __shared__ __attribute__((aligned(C::QT))) char do_st0[C::QT];
  __shared__ __attribute__((aligned(C::QT))) char q_st1[C::QT];
  __shared__ __attribute__((aligned(C::QT))) char do_st1[C::QT];
  __shared__ __attribute__((aligned(1024))) char k_blk[KBD];
  __shared__ __attribute__((aligned(1024))) char v_blk[C::KB];
  __shared__ __attribute__((aligned(1024))) char ds_buf[C::BK * C::BQ * 2];
  __shared__ __attribute__((aligned(16))) float stat_st0[2 * C::BQ];   // LSE*log2e, then -D
  __shared__ __attribute__((aligned(16))) float stat_st1[2 * C::BQ];

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int g = lane >> 5, ln = lane & 31;
  const int kb = wave & 3, qh = wave >> 2;
  const int L = a.L, Lk = a.Lk, shift = a.shift, window = a.window;
  const int G = a.Hq / a.Hkv;

  const int r = xcd_remap(blockIdx.x, gridDim.x);
  const int bhk = r / a.n_tiles;
  const int kt = r % a.n_tiles;
  const int b = bhk / a.Hkv, hk = bhk % a.Hkv;
  const int key_wg0 = kt * C::BK;
  const int key_w0 = key_wg0 + 32 * kb;

  const size_t kv_off = ((size_t)(b * a.Hkv + hk) * Lk) * D;
  const unsigned head_bytes = (unsigned)Lk * (2 * D);
  const unsigned qhead_bytes = (unsigned)L * (2 * D);

  const int q_begin = CAUSAL ? max(0, key_wg0 - shift) : (window > 0 ? max(0, key_wg0 - shift - window + 1) : 0);
  const int q_end = (window > 0) ? min(L, key_wg0 + C::BK - 1 + window - shift) : L;
  const bool empty = q_end <= q_begin;
  const int qt_lo = empty ? 0 : q_begin / C::BQ, qt_hi = empty ? -1 : (q_end - 1) / C::BQ;
  const int nq = qt_hi - qt_lo + 1;
  const int n_it = G * nq;

  constexpr int kCopyWaves = 4;                         // waves 0-3 stream the Q / dO tiles
  constexpr int kCopies = C::QCOPIES / kCopyWaves;      // copies per copy wave per tensor
  const bool copier = wave < kCopyWaves;
  int qcopy[kCopies];
#pragma unroll
  for (int i = 0; i < kCopies; ++i) qcopy[i] = dual_slot_src<D>(((wave & 3) + kCopyWaves * i) * 64 + lane);
  KVAddrDual<D> ad;
  ad.qrow.init(32 * qh + ln, g);
  ad.qtr[0].init(2 * qh, 0, lane);
  ad.qtr[1].init(2 * qh, 1, lane);
  ad.krow.init(32 * kb + ln, g);
  ad.kv = row_offset_kpad<D>(32 * kb + ln, 0, g);

  auto q0_of = [&](int it) { return (qt_lo + it % nq) * C::BQ; };
  auto issue = [&](int it, char* qs, char* dos, float* ss) {
    const int hq = hk * G + it / nq, q0 = q0_of(it);
    const size_t qoff = ((size_t)(b * a.Hq + hq) * L) * D;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(reinterpret_cast<const bf16*>(a.q) + qoff, qhead_bytes);
    const __amdgpu_buffer_rsrc_t drs = make_rsrc(reinterpret_cast<const bf16*>(a.dout) + qoff, qhead_bytes);
    const int soff = q0 * (2 * D);
    if (copier) {
#pragma unroll
      for (int i = 0; i < kCopies; ++i) {
        buf2lds16(qrs, qcopy[i], soff, qs + (wave + kCopyWaves * i) * 1024);
        buf2lds16(drs, qcopy[i], soff, dos + (wave + kCopyWaves * i) * 1024);
      }
    }
    if (wave == 0) {
      const size_t srow = (size_t)(b * a.Hq + hq) * L;
      const __amdgpu_buffer_rsrc_t lrs = make_rsrc(a.lse2 + srow, (unsigned)L * 4);
      const __amdgpu_buffer_rsrc_t ers = make_rsrc(a.delta + srow, (unsigned)L * 4);
      buf2lds4(lrs, 4 * lane, 4 * q0, reinterpret_cast<char*>(ss));
      buf2lds4(ers, 4 * lane, 4 * q0, reinterpret_cast<char*>(ss) + 4 * C::BQ);
    }
  };

  // the work-group's K (swz_dual) and V (padded) rows, once; rows past Lk read zeros
  {
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(reinterpret_cast<const bf16*>(a.k) + kv_off, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(reinterpret_cast<const bf16*>(a.v) + kv_off, head_bytes);
    const int soff = key_wg0 * (2 * D);
#pragma unroll
    for (int n = wave; n < KBD / 1024; n += C::kWaves)
      buf2lds16(krs, dual_slot_src<D>(n * 64 + lane), soff, k_blk + n * 1024);
#pragma unroll
    for (int n = wave; n < C::KBCOPIES; n += C::kWaves)
      buf2lds16(vrs, pad_slot_src<D, Pad<D>::KSTR>(n * 64 + lane), soff, v_blk + n * 1024);
  }
  if (n_it > 0) issue(0, q_st0, do_st0, stat_st0);

  KVState<D> st;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    st.dv[db] = f32x16{};
    st.dk[db] = f32x16{};
  }
  const float c = a.scale_log2;
  auto block_mask = [&](int q0) {
    const int qw0 = q0 + 32 * qh;
    return (qw0 + 32 > L) || (CAUSAL && qw0 + shift < key_w0 + 31) ||
           (window > 0 && qw0 + 31 + shift > key_w0 + window - 1) ||
           (!CAUSAL && window > 0 && qw0 + shift < key_w0 + 31 - window + 1);
  };
  const RangeMaskK<CAUSAL> ok{L, shift, window, key_w0 + ln};
  const int ds_row = 32 * kb + ln;

  // one tile: dK/dV work and the dS exchange, then dQ of the tile into registers
  auto tile = [&](int it, const char* qs, const char* dos, const float* ss) {
    const int q0 = q0_of(it);
    // every wave runs the tile, also one whose 32 x 32 block no query sees:
    // its mask then zeroes all of P and dS (skipping it would need a branch
    // around the tile that costs the kernel more registers than the ~2% of
    // work it saves on causal masks)
    kv_tile<D, F16, true>(st, ad, k_blk, v_blk, qs, dos, ss, q0, block_mask(q0), ok, qh, c, lane, ds_buf, ds_row);
    __syncthreads();     // every wave's dS block is in the exchange buffer
    if (!copier && kb < C::NDB) {
      // dQ blocks (0, kb) and (1, kb): A = dS of either query half by the
      // transposing read of the exchange buffer, B = K columns 32kb .. 32kb + 31
      // by the transposing read of the K block (shared by both blocks).  The
      // offsets are recomputed here (from a lane index the compiler cannot
      // hoist) rather than kept live through the tile.
      int ll = lane;
      asm volatile("" : "+v"(ll));
      const int kt0 = tr_offset_dual<D>(0, kb, 0, ll), kt1 = tr_offset_dual<D>(0, kb, 1, ll);
      const int hq = hk * G + it / nq;
      const __amdgpu_buffer_rsrc_t dq_rs =
          make_rsrc(a.dq_acc + (size_t)(b * a.Hq + hq) * L * D, (unsigned)L * D * 4);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int qw0 = q0 + 32 * half;
        const bool any = key_wg0 < Lk && qw0 < L && (!CAUSAL || qw0 + 31 + shift >= key_wg0) &&
                         (window <= 0 || qw0 + shift <= key_wg0 + C::BK - 1 + window - 1) &&
                         (CAUSAL || window <= 0 || qw0 + 31 + shift >= key_wg0 - window + 1);
        if (!any) continue;
        const int dsa0 = ds_tr_offset(0, 0, half, ll), dsa1 = ds_tr_offset(0, 1, half, ll);
        const int dsb0 = ds_tr_offset(1, 0, half, ll), dsb1 = ds_tr_offset(1, 1, half, ll);
        f32x16 acc = f32x16{};
#pragma unroll
        for (int t = 0; t < C::BK / 16; ++t) {
          const int da0 = (t & 1) ? dsb0 : dsa0, da1 = (t & 1) ? dsb1 : dsa1;
          const int base = (t >> 1) * 32 * 128;        // the swizzle repeats every 32 rows
          const bf16x8 av = concat4(lds_load_tr(ds_buf, da0 + base), lds_load_tr(ds_buf, da1 + base));
          const bf16x8 bv = concat4(lds_load_tr(k_blk, kt0 + t * 16 * (2 * D)),
                                    lds_load_tr(k_blk, kt1 + t * 16 * (2 * D)));
          acc = mfma32x<F16>(av, bv, acc);
        }
        // lane holds head dim 32kb + ln of queries qw0 + 8(i/4) + 4g + i%4; rows
        // past the sequence fall outside the resource and are dropped
        const int voff = ((qw0 + 4 * g) * D + 32 * kb + ln) * 4;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[i] * a.scale, dq_rs,
                                                          voff + (8 * (i >> 2) + (i & 3)) * D * 4, 0, 0);
      }
    }
  };

  // Only the copy waves wait for their copies; the atomics of the other waves
  // stay in flight across the barrier.
  auto wait_and_barrier = [&]() {
    if (copier) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  wait_copies_and_barrier();    // the K / V block and the first tile, all waves
  for (int it = 0; it < n_it; it += 2) {
    if (it + 1 < n_it) issue(it + 1, q_st1, do_st1, stat_st1);
    tile(it, q_st0, do_st0, stat_st0);
    wait_and_barrier();
    if (it + 1 >= n_it) break;
    if (it + 2 < n_it) issue(it + 2, q_st0, do_st0, stat_st0);
    tile(it + 1, q_st1, do_st1, stat_st1);
    wait_and_barrier();
  }

  // Sum the two query halves' dK and dV through LDS (as bwd_dkdv_kernel)
  constexpr int kPart = C::NDB * 16 * 64 * 4;
  static_assert(kPart <= C::QT, "a partial must fit in one stage buffer");
  bf16* dKh = reinterpret_cast<bf16*>(a.dk) + kv_off;
  bf16* dVh = reinterpret_cast<bf16*>(a.dv) + kv_off;
  const float s = a.scale;
  float* part = reinterpret_cast<float*>(kb == 0 ? q_st0 : kb == 1 ? do_st0 : kb == 2 ? q_st1 : do_st1);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if (qh == 1) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          part[(db * 16 + i) * 64 + lane] = pass == 0 ? st.dv[db][i] : st.dk[db][i];
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (pass == 0) st.dv[db][i] += part[(db * 16 + i) * 64 + lane];
          else st.dk[db][i] += part[(db * 16 + i) * 64 + lane];
        }
    }
    __syncthreads();
  }
  if (qh == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key_w0 + 8 * (i >> 2) + 4 * g + (i & 3);
      if (key < Lk) {
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          dKh[(size_t)key * D + 32 * db + ln] = pack1<F16>(st.dk[db][i] * s);
          dVh[(size_t)key * D + 32 * db + ln] = pack1<F16>(st.dv[db][i]);
        }
      }
    }
  }
}

// dQ = the float32 accumulator rounded to the 16-bit type (the scale was
// applied before the atomics).  8 elements per thread.
template <bool F16>
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(const float* __restrict__ acc, bf16* __restrict__ dq,
                                                             long long n8) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n8) {
    const f32x4 x0 = reinterpret_cast<const f32x4*>(acc)[2 * i];
    const f32x4 x1 = reinterpret_cast<const f32x4*>(acc)[2 * i + 1];
    reinterpret_cast<bf16x8*>(dq)[i] = pack8<F16>(x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]);
  }
}

// ------------------------------------------------------------ 3. dQ

// One work-group of 4 waves per (batch, query head, 128 queries), mirroring the
// forward.  The streamed K tile is read row-wise (S^T = K Q^T) and by the
// transposing read (dQ^T = K^T dS^T), so it uses the swz_dual layout; the V
// tile is only read row-wise (dP^T = V dO^T) and is padded.  The two 32-key
// halves of a tile are processed one after the other to keep registers low.

template <int D, bool CAUSAL, bool F16>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  using C = QCfg<D>;
  __shared__ __attribute__((aligned(1024))) char k_st0[C::KT];
  __shared__ __attribute__((aligned(1024))) char v_st0[C::VT];
  __shared__ __attribute__((aligned(1024))) char k_st1[C::KT];
  __shared__ __attribute__((aligned(1024))) char v_st1[C::VT];

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int g = lane >> 5, ln = lane & 31;
  // L query rows, Lk keys; query row i sits at key position i + shift
  const int L = a.L, Lk = a.Lk, shift = a.shift, window = a.window;

  const int r = xcd_remap(blockIdx.x, gridDim.x);
  int bh, qt_rank;
  head_tile_of(r, a.B * a.Hq, a.n_tiles, bh, qt_rank);
  const int qt = CAUSAL ? a.n_tiles - 1 - qt_rank : qt_rank;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int hk = h / (a.Hq / a.Hkv);

  const size_t q_off = ((size_t)(b * a.Hq + h) * L) * D;
  const size_t kv_off = ((size_t)(b * a.Hkv + hk) * Lk) * D;
  const unsigned head_bytes = (unsigned)Lk * (2 * D);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(reinterpret_cast<const bf16*>(a.k) + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(reinterpret_cast<const bf16*>(a.v) + kv_off, head_bytes);

  const int q_wg0 = qt * C::BQ;
  const int q_w0 = q_wg0 + 32 * wave;
  const int my_q = q_w0 + ln;
  const int wq_hi = min(q_w0 + 31, L - 1);
  // the same three in key coordinates
  const int dq_w0 = q_w0 + shift, dmy_q = my_q + shift, dwq_hi = wq_hi + shift;

  const int kv_end = range_key_end<CAUSAL>(Lk, window, min(L, q_wg0 + C::BQ) - 1 + shift);
  const int kv_begin = (window > 0) ? max(0, q_wg0 + shift - window + 1) : 0;
  const bool empty = kv_end <= kv_begin;     // only between chunks of a ring step
  const int j_lo = empty ? 0 : kv_begin / C::BC, j_hi = empty ? -1 : (kv_end - 1) / C::BC;

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

  auto issue = [&](int j, char* kb, char* vb) {
    const int soff = j * C::BC * (2 * D);
#pragma unroll
    for (int i = 0; i < C::KPER; ++i) buf2lds16(krs, ad.kcopy[i], soff, kb + (wave + C::kWaves * i) * 1024);
#pragma unroll
    for (int i = 0; i < C::VPER; ++i)
      if (owns_copy<C::kWaves, C::VCOPIES>(wave, i)) buf2lds16(vrs, ad.vcopy[i], soff, vb + (wave + C::kWaves * i) * 1024);
  };
  if (!empty) issue(j_lo, k_st0, v_st0);

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
  auto wave_needs = [&](int k0) { return (q_w0 < L) && range_tile_any<CAUSAL, C::BC>(k0, window, dq_w0, dwq_hi); };
  auto tile_mask = [&](int k0) { return range_tile_needs_mask<CAUSAL, C::BC>(k0, Lk, window, dq_w0, dwq_hi); };
  const RangeMaskQ<CAUSAL> ok{Lk, window, dmy_q};

  wait_copies_and_barrier();
  for (int j = j_lo; j <= j_hi; j += 2) {
    if (j < j_hi) issue(j + 1, k_st1, v_st1);
    if (wave_needs(j * C::BC))
      q_tile<D, F16>(st, ad, k_st0, v_st0, j * C::BC, tile_mask(j * C::BC), ok, c, lane);
    wait_copies_and_barrier();
    if (j + 1 > j_hi) break;
    if (j + 1 < j_hi) issue(j + 2, k_st0, v_st0);
    if (wave_needs((j + 1) * C::BC))
      q_tile<D, F16>(st, ad, k_st1, v_st1, (j + 1) * C::BC, tile_mask((j + 1) * C::BC), ok, c, lane);
    wait_copies_and_barrier();
  }

  // epilogue: dQ = s * dQ^T; lane = query, registers = head dims 32db + 8*(i/4) + 4g + i%4
  if (my_q < L) {
    bf16* dQr = reinterpret_cast<bf16*>(a.dq) + q_off + (size_t)my_q * D;
    const float s = a.scale;
    store_row_c<F16, C::NDB>(dQr, st.dq, s, g);
  }
}

template <int D, bool F16>
hipError_t launch_delta(const BwdArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.Hq * a.L;
  constexpr int kRowsPerBlock = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_delta_kernel<D, F16>), dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)),
                     dim3(256), 0, stream, reinterpret_cast<const bf16*>(a.o),
                     reinterpret_cast<const bf16*>(a.dout), a.lse, a.delta, a.lse2, a.dq_acc, rows);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool F16>
hipError_t launch_dkdv(const BwdArgs& args, hipStream_t stream) {
  BwdArgs a = args;
  a.n_tiles = (a.Lk + KVCfg<D>::BK - 1) / KVCfg<D>::BK;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, F16>), dim3((unsigned)((long long)a.B * a.Hkv * a.n_tiles)),
                     dim3(64 * KVCfg<D>::kWaves), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool F16>
hipError_t launch_dq(const BwdArgs& args, hipStream_t stream) {
  BwdArgs a = args;
  a.n_tiles = (a.L + QCfg<D>::BQ - 1) / QCfg<D>::BQ;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, F16>), dim3((unsigned)((long long)a.B * a.Hq * a.n_tiles)),
                     dim3(64 * QCfg<D>::kWaves), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool F16>
hipError_t launch_fused(const BwdArgs& args, hipStream_t stream) {
  BwdArgs a = args;
  a.n_tiles = (a.Lk + KVCfg<D>::BK - 1) / KVCfg<D>::BK;
  hipLaunchKernelGGL((bwd_fused_kernel<D, CAUSAL, F16>), dim3((unsigned)((long long)a.B * a.Hkv * a.n_tiles)),
                     dim3(64 * KVCfg<D>::kWaves), 0, stream, a);
  return hipGetLastError();
}

template <bool F16>
hipError_t launch_convert(const BwdArgs& a, hipStream_t stream) {
  const long long n8 = (long long)a.B * a.Hq * a.L * a.d / 8;
  hipLaunchKernelGGL((bwd_dq_convert_kernel<F16>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                     a.dq_acc, reinterpret_cast<bf16*>(a.dq), n8);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_preprocess_bf16(const BwdArgs& a, hipStream_t stream) {
  if (a.f16) return a.d == 128 ? launch_delta<128, true>(a, stream) : launch_delta<64, true>(a, stream);
  return a.d == 128 ? launch_delta<128, false>(a, stream) : launch_delta<64, false>(a, stream);
}

namespace {
template <bool F16>
hipError_t dkdv_typed(const BwdArgs& a, bool causal, hipStream_t stream) {
  if (a.d == 128) return causal ? launch_dkdv<128, true, F16>(a, stream) : launch_dkdv<128, false, F16>(a, stream);
  return causal ? launch_dkdv<64, true, F16>(a, stream) : launch_dkdv<64, false, F16>(a, stream);
}
template <bool F16>
hipError_t dq_typed(const BwdArgs& a, bool causal, hipStream_t stream) {
  if (a.d == 128) return causal ? launch_dq<128, true, F16>(a, stream) : launch_dq<128, false, F16>(a, stream);
  return causal ? launch_dq<64, true, F16>(a, stream) : launch_dq<64, false, F16>(a, stream);
}
}  // namespace

hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a, bool causal, hipStream_t stream) {
  return a.f16 ? dkdv_typed<true>(a, causal, stream) : dkdv_typed<false>(a, causal, stream);
}

hipError_t launch_bwd_dq_bf16(const BwdArgs& a, bool causal, hipStream_t stream) {
  return a.f16 ? dq_typed<true>(a, causal, stream) : dq_typed<false>(a, causal, stream);
}

hipError_t launch_bwd_bf16(const BwdArgs& a, bool causal, hipStream_t stream) {
  hipError_t e = launch_bwd_preprocess_bf16(a, stream);
  if (e != hipSuccess) return e;
  e = launch_bwd_dkdv_bf16(a, causal, stream);
  if (e != hipSuccess) return e;
  return launch_bwd_dq_bf16(a, causal, stream);
}

namespace {
template <bool F16>
hipError_t fused_typed(const BwdArgs& a, bool causal, hipStream_t stream) {
  if (a.d == 128) return causal ? launch_fused<128, true, F16>(a, stream) : launch_fused<128, false, F16>(a, stream);
  return causal ? launch_fused<64, true, F16>(a, stream) : launch_fused<64, false, F16>(a, stream);
}
}  // namespace

hipError_t launch_bwd_fused_bf16(const BwdArgs& a, bool causal, hipStream_t stream) {
  hipError_t e = launch_bwd_preprocess_bf16(a, stream);
  if (e != hipSuccess) return e;
  e = a.f16 ? fused_typed<true>(a, causal, stream) : fused_typed<false>(a, causal, stream);
  if (e != hipSuccess) return e;
  return a.f16 ? launch_convert<true>(a, stream) : launch_convert<false>(a, stream);
}

}  // namespace fa
