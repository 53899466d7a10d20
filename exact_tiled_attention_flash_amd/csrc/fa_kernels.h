// fa_kernels.h -- internal launcher interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;        // may be null
  int B, Hq, Hkv, L, d;  // L = query rows
  int Lk;            // keys (= L except for chunk pairs)
  int shift;         // query row i sits at key position i + shift (0 except for chunk pairs)
  int window;        // 0 = none
  float scale_log2;  // softmax scale * log2(e)
  int n_qtiles;      // filled in by the launcher
  bool f16;          // 16-bit inputs are fp16 (else bf16)
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;      // workspace: -D_i = -sum_c dO_ic * O_ic, [B, Hq, L] (negated: dP - D starts from it)
  float* lse2;       // workspace: LSE_i * log2(e), [B, Hq, L]
  float* dq_acc;     // workspace of the fused backward: float32 dQ accumulator [B, Hq, L, d], or null
  int B, Hq, Hkv, L, d;  // L = query rows
  int Lk;            // keys (= L except for chunk pairs)
  int shift;         // query row i sits at key position i + shift (0 except for chunk pairs)
  int window;
  float scale;       // softmax scale
  float scale_log2;  // softmax scale * log2(e)
  int n_tiles;       // filled in by the launchers
  bool f16;          // 16-bit inputs are fp16 (else bf16)
};

struct MergeArgs {
  const void* o_a;
  const float* lse_a;
  const void* o_b;
  const float* lse_b;
  void* o;           // may be o_a (in-place accumulation)
  float* lse;        // may be lse_a
  long long rows;    // B * Hq * L
};

// 16-bit (bf16 or fp16, by a.f16) kernels
hipError_t launch_fwd_bf16(const FwdArgs& a, bool causal, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, bool causal, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs& a, bool causal, hipStream_t stream);
// the three stages of launch_bwd_bf16, in order (stage 2 and 3 are independent)
hipError_t launch_bwd_preprocess_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a, bool causal, hipStream_t stream);
hipError_t launch_bwd_dq_bf16(const BwdArgs& a, bool causal, hipStream_t stream);
// the fused backward: preprocess (also zeroing a.dq_acc), one K/V-stationary
// kernel producing dK, dV and accumulating dQ into a.dq_acc with float32
// atomics, and a conversion of a.dq_acc into dQ
hipError_t launch_bwd_fused_bf16(const BwdArgs& a, bool causal, hipStream_t stream);
// exact combination of two partial results; dtype 0 fp32, 1 bf16, 2 fp16
hipError_t launch_merge(const MergeArgs& a, int d, int dtype, hipStream_t stream);

struct DecodeArgs {
  const void* q;          // [B, Hq, Lq, d] newest tokens' queries
  const void* k;          // [B, Hkv, Lk, d] cache
  const void* v;
  const int* cache_len;   // [B] valid cache entries per sequence, or null (= Lk)
  void* o;                // [B, Hq, Lq, d]
  float* lse;             // [B, Hq, Lq] or null
  float* part_o;          // workspace: [n_splits, rows, d] float32
  float* part_lse;        // workspace: [n_splits, rows] float32
  int B, Hq, Hkv, Lq, Lk, d;
  int window;
  float scale_log2;
  bool f16;
  int n_splits, split_keys;
  long long rows;         // B * Hq * Lq
  int split_base;         // index of this launch's first split among the partials
  int n_splits_total;     // partials the combine merges per row
};
// key splits for a decode call (deterministic in its sizes)
void decode_plan(int B, int Hkv, int Lk, int& n_splits, int& split_keys);
hipError_t launch_decode(const DecodeArgs& a, bool causal, hipStream_t stream);
// Rolling (ring) cache of Lk = W slots, position p of sequence b in slot p mod W,
// cache_len = tokens seen before the call; `fresh` holds the new tokens' own
// K/V ([B, Hkv, Lq, d], k and v of it) with their splits after the ring's.
hipError_t launch_decode_rolling(const DecodeArgs& ring, const DecodeArgs& fresh, hipStream_t stream);

// ---- general masks through a mask plan
// A mask over one sequence of L positions (queries and keys alike):
//   allowed(i, j) = causal_ok && ((window_ok && block_ok) || global(i) || global(j))
// with causal_ok: j <= i (when causal); window_ok: |i - j| < window (when
// window > 0); block_ok: block_mask[i / block][j / block] != 0 (when given);
// global: the position is one of global_pos (negative entries count from L).
struct MaskDesc {
  int causal, window;
  const int* global_pos;             // device, n_global entries (may be null when n_global == 0)
  int n_global;
  const unsigned char* block_mask;   // device, [nbm][nbm] with nbm = ceil(L / block), or null
  int block;                         // multiple of 64
};

// A plan classifies every 64 x 64 block of the L x L mask as empty, partial or
// full and lists, for every 128-row work-group of the forward and dQ kernels,
// the 64-key tiles it must visit (and, for every 128-key work-group of the
// dK/dV kernel, the 64-query tiles), plus a heaviest-first work-group order.
// Global query rows (for the forward and dQ) and global keys (for dK/dV) see
// the whole sequence; the lists leave them out and separate split passes over
// every key (every query) compute them, so no work-group has to walk a whole
// row.
// List entry: tile index | class(first 64 rows or keys) << 16 | class(second)
// << 18 | block_ok(first) << 20 | block_ok(second) << 21; class 0 empty,
// 1 partial (elementwise mask), 2 full.
struct PlanLayout {
  int L, nb, nw;                     // nb 64-blocks, nw 128-wide work-group rows (= columns)
  size_t gbits, row_cnt, row_ord, col_cnt, col_ord, meta, gpos, row_ent, col_ent, total;   // byte offsets
};
PlanLayout plan_layout(int L);

struct PlanPtrs {
  const unsigned long long* gbits;   // [nb] bit t of word b: position 64b + t is global
  const int* row_cnt;                // [nw] entries per work-group row
  const int* row_ord;                // [nw] work-group rows by descending entry count
  const unsigned* row_ent;           // [nw][nb] entries (key tiles), ascending
  const int* col_cnt;
  const int* col_ord;
  const unsigned* col_ent;           // [nw][nb] entries (query tiles), ascending
  const int* meta;                   // [0], [1]: leading heavy ranks of row_ord, col_ord; [2]: global count
  const int* gpos;                   // [meta[2]] global positions, ascending
  int nb, nw;
};
PlanPtrs plan_ptrs(const void* plan, int L);

hipError_t launch_mask_plan(const MaskDesc& m, int L, void* plan, hipStream_t stream);

// Split passes for the global positions (rows for the forward and dQ, keys for
// dK/dV): ngp = the global count rounded up to 32 (0: no pass), n_splits
// splits of `per` tiles, float32 partials in `part` (and `part_lse`).
struct GlobalArgs {
  int n_splits, per, ngp;
  float* part;
  float* part_lse;
};
GlobalArgs global_plan(int L, int n_global, int n_heads);
size_t global_fwd_bytes(const GlobalArgs& g, int n_heads, int d);
size_t global_dq_bytes(const GlobalArgs& g, int n_heads, int d);
size_t global_dkdv_bytes(const GlobalArgs& g, int n_kv_heads, int d);

// forward / backward (preprocess, dK/dV, dQ) under a plan; a.L is the sequence
// length the plan was built for, a.window its window
hipError_t launch_fwd_masked(const FwdArgs& a, const PlanPtrs& p, const GlobalArgs& ga, bool causal,
                             hipStream_t stream);
hipError_t launch_bwd_masked(const BwdArgs& a, const PlanPtrs& p, const GlobalArgs& gr, const GlobalArgs& gc,
                             bool causal, hipStream_t stream);

}  // namespace fa
