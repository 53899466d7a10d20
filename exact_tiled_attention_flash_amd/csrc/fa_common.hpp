// fa_common.hpp -- device-side building blocks shared by the gfx950 kernels.
//
// MFMA register layouts used throughout (v_mfma_f32_32x32x16_bf16, one wave):
//   A operand (32 x 16, M x K): lane l holds row m = l % 32 and 8 consecutive
//     K slots of slice g = l / 32.
//   B operand (16 x 32, K x N): lane l holds column n = l % 32, same K slots.
//   C/D (32 x 32 fp32):         lane l, register i holds
//     row m = 8*(i/4) + 4*(l/32) + (i%4), column n = l % 32.
// A and B label their K slots identically, so any bijection between
// (slice, slot) and the contraction index gives the same product; the kernels
// choose the bijection that lets one MFMA's C registers feed the next MFMA's
// B operand directly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running-max sentinel: finite, so that exp2(m_old - m_new) never sees
// (-inf) - (-inf).  Any real scaled score is far above it.
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The 16-bit kernels serve bf16 and fp16 alike: bf16x8 / bf16x4 / bf16 are
// then plain containers of 16-bit values, and the F16 template parameter
// decides how the arithmetic reads and writes them (the MFMA opcode and the
// fp32 <-> 16-bit conversions, both round-to-nearest-even).
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <bool F16>
__device__ __forceinline__ f32x16 mfma32x(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <bool F16>
__device__ __forceinline__ bf16 pack1(float x) {
  if constexpr (F16) return __builtin_bit_cast(bf16, (f16)x);
  else return (bf16)x;
}

template <bool F16>
__device__ __forceinline__ float unpack1(bf16 x) {
  if constexpr (F16) return (float)__builtin_bit_cast(f16, x);
  else return (float)x;
}

template <bool F16>
__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                        float a7) {
  if constexpr (F16) {
    f16x8 r;
    r[0] = (f16)a0; r[1] = (f16)a1; r[2] = (f16)a2; r[3] = (f16)a3;
    r[4] = (f16)a4; r[5] = (f16)a5; r[6] = (f16)a6; r[7] = (f16)a7;
    return __builtin_bit_cast(bf16x8, r);
  } else {
    bf16x8 r;
    r[0] = (bf16)a0; r[1] = (bf16)a1; r[2] = (bf16)a2; r[3] = (bf16)a3;
    r[4] = (bf16)a4; r[5] = (bf16)a5; r[6] = (bf16)a6; r[7] = (bf16)a7;
    return r;
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte LDS load at a byte offset.
__device__ __forceinline__ bf16x8 lds_load16(const char* base, int byte_off) {
  return *(const FA_LDS bf16x8*)((const FA_LDS char*)(base) + byte_off);
}

// gfx950 transposing LDS read.  Within each group of 16 lanes, result lane i,
// element r is element (i % 4) of the 8 bytes addressed by lane 4*r + i/4.
__device__ __forceinline__ bf16x4 lds_load_tr(const char* base, int byte_off) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)((FA_LDS char*)(base) + byte_off));
  return __builtin_bit_cast(bf16x4, r);
}

// Buffer resource over `bytes` bytes at `base` (raw, no stride): loads past
// the end return zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Direct 16-byte buffer -> LDS copy for a whole wave: lane l's 16 bytes from
// byte voff + soff of the resource land at lds_wave_base + 16*l.
// `lds_wave_base` and `soff` must be wave-uniform.
__device__ __forceinline__ void buf2lds16(__amdgpu_buffer_rsrc_t r, int voff, int soff, char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void*)(lds_wave_base), 16, voff, soff, 0, 0);
}

// Same with 4 bytes per lane: lane l's dword lands at lds_wave_base + 4*l.
__device__ __forceinline__ void buf2lds4(__amdgpu_buffer_rsrc_t r, int voff, int soff, char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void*)(lds_wave_base), 4, voff, soff, 0, 0);
}

// Value of x in lane l XOR 32 combined with x by op -- both halves of the wave
// end up with op(x[l % 32], x[l % 32 + 32]).  One v_permlane32_swap.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// acc + a + b for two bf16 values (v_dot2 with (1, 1)), exact products.
__device__ __forceinline__ float dot2_ones(bf16 a, bf16 b, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {a, b};
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(v, one, acc, false);
}

// Store one row held in the MFMA C layout with lane = row: in block db, the
// lane's register i is element 32db + 8(i/4) + 4g + i%4 (g = lane / 32), so a
// lane alone holds runs of 4.  For each pair of 8-element groups two
// v_permlane32_swap between the lanes g = 0 and g = 1 of the row give lane g
// elements 32db + 16p + 8g .. +7 (p = the pair), and every lane stores 16
// contiguous bytes: 2 * NDB stores of 16 bytes instead of 4 * NDB of 8.  Both
// lanes of a row must take part (they do when the caller's condition depends
// on the row only).  The values are multiplied by f and rounded to 16 bits.
template <bool F16, int NDB>
__device__ __forceinline__ void store_row_c(bf16* row, const f32x16 (&acc)[NDB], float f, int g) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = pack1<F16>(acc[db][8 * p + e] * f);
      u32x4 u = __builtin_bit_cast(u32x4, v);
      const auto s0 = __builtin_amdgcn_permlane32_swap(u[0], u[2], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(u[1], u[3], false, false);
      u[0] = s0[0];
      u[2] = s0[1];
      u[1] = s1[0];
      u[3] = s1[1];
      *reinterpret_cast<u32x4*>(row + 32 * db + 16 * p + 8 * g) = u;
    }
  }
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Direct 16-byte global -> LDS copy for a whole wave: lane l's 16 bytes from
// `src` land at lds_wave_base + 16*l.  `lds_wave_base` must be wave-uniform.
__device__ __forceinline__ void g2lds16(const void* src, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (FA_LDS void*)(lds_wave_base), 16, 0, 0);
}

__device__ __forceinline__ bf16x8 concat4(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Round-to-nearest-even fp32 -> bf16 of 8 values (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3,
                                            float a4, float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (bf16)a0; r[1] = (bf16)a1; r[2] = (bf16)a2; r[3] = (bf16)a3;
  r[4] = (bf16)a4; r[5] = (bf16)a5; r[6] = (bf16)a6; r[7] = (bf16)a7;
  return r;
}

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

// Index of the calling wave in its work-group, as a value the compiler knows to
// be uniform across the wave: branches on quantities derived from it then
// stay scalar branches instead of becoming exec-masked code that runs both
// sides.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Does wave `wave` (< NW) of a work-group of NW waves own copy i of a tile of
// COPIES 1 KiB copies (copy wave + NW*i)?  Every wave owns one copy in each of
// the first COPIES / NW rounds, so those resolve at compile time and only the
// last, partial round costs a (wave-uniform) branch.
template <int NW, int COPIES>
__device__ __forceinline__ bool owns_copy(int wave, int i) {
  return i < COPIES / NW || wave + NW * i < COPIES;
}

// Forward LDS swizzles (XOR on the 16-byte chunk index of row r of a tile).
// K is only read 16 rows at a time at one chunk: spread those rows over all
// banks.  V is only read by the transposing read (4 rows x 4 chunks per
// half-wave), and rows r and r+8 share a swizzle.
template <int D> __host__ __device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D> __host__ __device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// Offsets into the forward's K tile (16-byte row read) and V tile (8 bytes
// supplied to the transposing read; h selects K slots 0..3 or 4..7).
template <int D>
__host__ __device__ __forceinline__ int row_offset_k(int r, int k, int g) {
  return r * (2 * D) + (((2 * k + g) ^ swz_k<D>(r)) << 4);
}
template <int D>
__host__ __device__ __forceinline__ int tr_offset_v(int t, int db, int h, int lane) {
  const int s16 = lane & 15, jg = lane >> 4;
  const int row = 16 * t + 8 * h + 4 * (lane >> 5) + (s16 >> 2);
  const int col = 32 * db + 16 * (jg & 1) + 4 * (s16 & 3);
  return row * (2 * D) + (((col >> 3) ^ swz_v<D>(row)) << 4) + ((col & 4) << 1);
}

// Padded LDS tiles.  A row of D bf16 values (2D bytes) is stored with a stride
// of KSTR = 2D + 16 bytes in a tile read only by 16-byte row reads, and of
// VSTR = 2D + 64 bytes in a tile read only by the transposing read.  Either
// stride spreads the rows a read touches over all 64 banks, and, unlike an
// XOR swizzle, keeps every operand address "one per-lane base + an immediate",
// so the loop needs no address arithmetic.
template <int D> struct Pad {
  static constexpr int KSTR = 2 * D + 16;
  static constexpr int VSTR = 2 * D + 64;
};

// Byte offset in a K-padded tile of head dims 16k + 8g .. +7 of row r.
template <int D>
__host__ __device__ __forceinline__ int row_offset_kpad(int r, int k, int g) {
  return r * Pad<D>::KSTR + (2 * k + g) * 16;
}

// Byte offset in a V-padded tile of the 8 bytes lane `lane` supplies to the
// transposing read for MFMA K-step t (16 rows), 32-wide column block db and
// half h (K slots 0..3 or 4..7, 8 rows further down); the slots then hold rows
// 16t + 8*(slot/4) + 4*(lane/32) + slot%4 and column 32db + lane%32.
template <int D>
__host__ __device__ __forceinline__ int tr_offset_vpad(int t, int db, int h, int lane) {
  const int s16 = lane & 15, jg = lane >> 4;
  const int row = 16 * t + 8 * h + 4 * (lane >> 5) + (s16 >> 2);
  const int col = 32 * db + 16 * (jg & 1) + 4 * (s16 & 3);
  return row * Pad<D>::VSTR + col * 2;
}

// Source of 16-byte slot p of a padded tile with STRIDE-byte rows: byte offset,
// relative to the tile's first row in the [rows x D] bf16 tensor, of the data
// that belongs there.  Padding slots repeat the row's first chunk.
template <int D, int STRIDE>
__host__ __device__ __forceinline__ int pad_slot_src(int p) {
  constexpr int kSlots = STRIDE / 16, kChunks = D / 8;
  const int r = p / kSlots, slot = p % kSlots;
  return r * (2 * D) + (slot < kChunks ? slot : 0) * 16;
}

// LDS row swizzle (XOR on the 16-byte chunk index of row r) that keeps two read
// patterns free of bank conflicts: 16 consecutive rows read at one chunk
// (16-byte reads), and 4 consecutive rows x 4 chunks (the transposing read).
template <int D>
__host__ __device__ __forceinline__ int swz_dual(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Byte offset, inside a [rows x D] bf16 tile stored with swz_dual, of the 8
// bytes lane `lane` supplies to the transposing read for MFMA K-step t (16
// rows), 32-wide column block db and half h: h = 0 gives K slots 0..3, h = 1
// slots 4..7 (8 rows further down, with that row's own swizzle).  The rows
// then line up with the C-layout rows 16t + 8*(slot/4) + 4*(lane/32) + slot%4
// of an MFMA result.
template <int D>
__host__ __device__ __forceinline__ int tr_offset_dual(int t, int db, int h, int lane) {
  const int s16 = lane & 15, jg = lane >> 4;
  const int row = 16 * t + 8 * h + 4 * (lane >> 5) + (s16 >> 2);
  const int col = 32 * db + 16 * (jg & 1) + 4 * (s16 & 3);
  return row * (2 * D) + (((col >> 3) ^ swz_dual<D>(row)) << 4) + ((col & 4) << 1);
}

// Source of 16-byte slot p of a [rows x D] tile stored with swz_dual: byte
// offset, relative to the tile's first row, of the chunk that belongs there.
template <int D>
__host__ __device__ __forceinline__ int dual_slot_src(int p) {
  constexpr int kChunks = D / 8;
  const int r = p / kChunks, slot = p % kChunks;
  return r * (2 * D) + (slot ^ swz_dual<D>(r)) * 16;
}

// Byte offset of the 16 bytes (head dims 16k + 8g .. +7) of row r in a tile
// stored with swz_dual.
template <int D>
__host__ __device__ __forceinline__ int row_offset_dual(int r, int k, int g) {
  return r * (2 * D) + (((2 * k + g) ^ swz_dual<D>(r)) << 4);
}

// dS exchange buffer of the fused backward: [128 keys][64 queries] of 16-bit
// values, rows of 128 bytes.  The 8-byte chunk c of row r (queries 4c ..
// 4c + 3) is stored at chunk c ^ ds_swz(r).  The swizzle is a bijection over
// the 16 rows of one parity in any aligned 32-row window, and rows 4n and
// 4n + 2 (likewise 4n + 1 and 4n + 3) differ in its bit 3, so both access
// patterns are free of bank conflicts: the writes from an MFMA C layout (32
// consecutive rows, one chunk each) and the transposing reads (4 consecutive
// rows x 8 consecutive chunks per half-wave).  Its period is 32 rows.
__host__ __device__ __forceinline__ int ds_swz(int r) {
  const int u = (r >> 1) & 15;
  return ((u & 1) << 3) | (u >> 1);
}
__host__ __device__ __forceinline__ int ds_offset(int r, int c) { return r * 128 + 8 * (c ^ ds_swz(r)); }

// Byte offset of the 8 bytes lane `lane` supplies to the transposing read of
// the dS buffer for key step t (keys 16t .. 16t + 15), half h and query half
// qh: result lane l then holds query 32qh + l % 32 and its slots the keys
// 16t + 8h + 4*(l/32) + slot % 4 -- the A operand of dQ = dS K in the key
// labelling of an MFMA C layout.
__host__ __device__ __forceinline__ int ds_tr_offset(int t, int h, int qh, int lane) {
  const int s16 = lane & 15, jg = lane >> 4;
  const int row = 16 * t + 8 * h + 4 * (lane >> 5) + (s16 >> 2);
  return ds_offset(row, 8 * qh + 4 * (jg & 1) + (s16 & 3));
}

// Work-group -> (head, query-tile) remap.  Work-groups are dealt round-robin to
// the 8 XCDs (each with its own L2), so when the grid is a multiple of 8 the
// index is permuted such that consecutive logical indices run on one XCD:
// the query tiles of one (batch, K/V head) then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int id, int n) {
  constexpr int kXcds = 8;
  if (n % kXcds != 0) return id;
  return (id % kXcds) * (n / kXcds) + id / kXcds;
}

// Logical work-group index -> (head, tile rank) for a grid of n_heads x
// n_tiles work-groups in which tile rank 0 is the heaviest (causal masking
// makes the tiles' work range from 1 to n_tiles units).  Heads go in pairs,
// and inside a pair rank by rank (rank 0 of both heads, then rank 1, ...):
// the heaviest work-groups of a pair are dispatched first, which evens out
// when the work-group slots of a CU run dry, while only two heads' streamed
// operands are live in an XCD's L2 at a time.  With an odd head count the
// last head goes alone.
__device__ __forceinline__ void head_tile_of(int r, int n_heads, int n_tiles, int& head, int& rank) {
  const int paired = (n_heads >> 1) * 2 * n_tiles;
  if (r < paired) {
    const int pair = r / (2 * n_tiles), rest = r - pair * 2 * n_tiles;
    head = 2 * pair + (rest & 1);
    rank = rest >> 1;
  } else {
    head = n_heads - 1;
    rank = r - paired;
  }
}

// ---- applying an element mask
// Two element masks and a wave-uniform choice between them: the tile steps
// evaluate only the chosen one (with_mask branches once per tile, outside the
// element loop), so a cheap mask can stand in for an expensive one on the
// tiles where both agree.
template <class A, class B>
struct EitherMask {
  bool use_a;
  A a;
  B b;
};

// The tile steps evaluate a mask at base + c, base per lane and tile, c a
// compile-time offset.  A mask with a fresh() member (one run of positions,
// PosRun) is shifted by base once per tile, so that each element costs a
// subtraction from an immediate, a compare and a select, with nothing held in
// registers across tiles; fresh() forms the run from a copy of the lane's
// position that the compiler must take as new on every tile (otherwise it
// keeps the run, or per-element offsets, in registers for the whole kernel).
// Other masks are called at base + c.
template <class M>
struct AtBase {
  const M& m;
  int base;
  __device__ __forceinline__ bool operator()(int c) const { return m(base + c); }
};
template <class M>
__device__ __forceinline__ auto mask_at(const M& m, int base, int) -> decltype(m.fresh()) {
  auto r = m.fresh();
  r.lo -= base;
  return r;
}
template <class M>
__device__ __forceinline__ AtBase<M> mask_at(const M& m, int base, long) { return AtBase<M>{m, base}; }

template <class M, class F>
__device__ __forceinline__ void with_mask(const M& m, int base, const F& f) { f(mask_at(m, base, 0)); }
template <class A, class B, class F>
__device__ __forceinline__ void with_mask(const EitherMask<A, B>& m, int base, const F& f) {
  if (m.use_a) f(mask_at(m.a, base, 0));
  else f(mask_at(m.b, base, 0));
}

// x = keep ? x : y in place (a tied operand writes no new register, so the
// masked and unmasked versions of a tile's values join without copies).  All
// lanes must be active.
__device__ __forceinline__ float keep_or(float x, bool keep, float y) {
  const unsigned long long k = __builtin_amdgcn_ballot_w64(keep);
  asm("v_cndmask_b32_e64 %0, %2, %0, %1" : "+v"(x) : "s"(k), "v"(y));
  return x;
}
__device__ __forceinline__ float keep_or_zero(float x, bool keep) {
  const unsigned long long k = __builtin_amdgcn_ballot_w64(keep);
  asm("v_cndmask_b32_e64 %0, 0, %0, %1" : "+v"(x) : "s"(k));
  return x;
}

// ---- masks of the range-tiled kernels (positions in key coordinates)
// Key j is visible to the query at position i iff j < Lk, j <= i when causal,
// and, for a window w > 0, i - w < j -- plus j < i + w when not causal: the
// window then reaches both ways, |i - j| < w (kler.cn "大模型高效注意力机制全
// 解析" §3.2.1; book.anysome.cn "高效注意力" §4 for the one-sided form).
template <bool CAUSAL>
__host__ __device__ __forceinline__ bool range_ok(int j, int i, int Lk, int window) {
  // bitwise, not short-circuit, so that no divergent branch is formed
  return (j < Lk) & (!CAUSAL | (j <= i)) & ((window <= 0) | ((j > i - window) & (CAUSAL | (j < i + window))));
}

// One run of positions, lo .. lo+span-1 (span 0: none): one subtraction and
// one unsigned compare per position.
struct PosRun {
  int lo;
  unsigned span;
  __host__ __device__ __forceinline__ bool operator()(int x) const { return unsigned(x - lo) < span; }
};
__host__ __device__ __forceinline__ PosRun pos_run(int lo, int hi) { return PosRun{lo, hi > lo ? unsigned(hi - lo) : 0u}; }

// Query-major element mask: the lane's query position i is fixed.  For keys
// j >= 0, range_ok(j, i, ..) holds on one run of keys, which the tile steps
// evaluate (fresh(): from a copy of i that the compiler must take as new on
// every tile, so the run is formed per masked tile and not kept in registers
// for the whole kernel).
template <bool CAUSAL>
struct RangeMaskQ {
  int Lk, window, i;
  __host__ __device__ __forceinline__ PosRun run() const {
    const int hi = CAUSAL ? min(Lk, i + 1) : (window > 0 ? min(Lk, i + window) : Lk);
    return pos_run(window > 0 ? max(0, i - window + 1) : 0, hi);
  }
  __host__ __device__ __forceinline__ bool operator()(int j) const { return run()(j); }
  __device__ __forceinline__ PosRun fresh() const {
    RangeMaskQ m = *this;
    asm volatile("" : "+v"(m.i));
    return m.run();
  }
};

// Do the keys [k0, k0 + BC) need the elementwise mask for queries [i_lo, i_hi]?
template <bool CAUSAL, int BC>
__device__ __forceinline__ bool range_tile_needs_mask(int k0, int Lk, int window, int i_lo, int i_hi) {
  return (k0 + BC > Lk) || (CAUSAL && k0 + BC - 1 > i_lo) || (window > 0 && k0 < i_hi - window + 1) ||
         (!CAUSAL && window > 0 && k0 + BC - 1 > i_lo + window - 1);
}

// Does any query in [i_lo, i_hi] see any key in [k0, k0 + BC)?
template <bool CAUSAL, int BC>
__device__ __forceinline__ bool range_tile_any(int k0, int window, int i_lo, int i_hi) {
  return (!CAUSAL || k0 <= i_hi) && (window <= 0 || k0 + BC - 1 >= i_lo - window + 1) &&
         (CAUSAL || window <= 0 || k0 <= i_hi + window - 1);
}

// One past the last key any query in [.., i_hi] may see (i_hi = the last query
// row of a work-group, in key coordinates).
template <bool CAUSAL>
__device__ __forceinline__ int range_key_end(int Lk, int window, int i_hi) {
  return CAUSAL ? min(Lk, i_hi + 1) : (window > 0 ? min(Lk, i_hi + window) : Lk);
}

}  // namespace fa
