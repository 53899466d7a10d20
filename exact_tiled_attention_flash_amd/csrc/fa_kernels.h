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
  float* delta;      // workspace: D_i = sum_c dO_ic * O_ic, [B, Hq, L]
  float* lse2;       // workspace: LSE_i * log2(e), [B, Hq, L]
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
};
// key splits for a decode call (deterministic in its sizes)
void decode_plan(int B, int Hkv, int Lk, int& n_splits, int& split_keys);
hipError_t launch_decode(const DecodeArgs& a, bool causal, hipStream_t stream);

}  // namespace fa
