// flash_attn_api.hip -- the extern "C" boundary: validation, then dispatch.
//
// Every argument is checked on the host before any HIP call, so a rejected
// call has no side effect.  The library allocates nothing; all buffers and the
// stream belong to the caller.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>

#include "../../include/flash_attn.h"
#include "fa_kernels.h"

namespace {

// keeps the byte size of one head (L * 2d, d <= 128) in 32 bits: the kernels
// address each head through a buffer resource with a 32-bit range
constexpr int kMaxL = 1 << 23;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(int B, int Hq, int Hkv, int L, int d, float scale, int causal, int window, int dtype) {
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || L > kMaxL) return FA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (window < 0) return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_F32) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (Hq % Hkv != 0) return FA_ERR_GQA;
  // launch sizes: a 1-D launch covers at most 2^32 - 1 work-items, and the
  // kernels use up to 4 per query row (or key row), so B*Hq*L stays below 2^30
  if ((long long)B * Hq * L >= (1LL << 30)) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// Backward row statistics: two float32 per query row -- -D_i and LSE_i*log2(e).
// The staged (deterministic) backward needs only these.
size_t workspace_bytes(int B, int Hq, int L) {
  const size_t raw = 2 * (size_t)B * (size_t)Hq * (size_t)L * sizeof(float);
  return (raw + 255) & ~(size_t)255;
}

// The fused backward adds its float32 dQ accumulator [B, Hq, L, d] after them.
size_t fused_workspace_bytes(int B, int Hq, int L, int d) {
  return workspace_bytes(B, Hq, L) + (size_t)B * Hq * L * d * sizeof(float);
}

// The fused kernel adds into one query head of the accumulator through a
// buffer resource whose byte range is 32 bits.
bool fused_fits(int L, int d) { return (size_t)L * d * sizeof(float) < ((size_t)1 << 32); }

// Chunk positions: offsets are non-negative and at most 2^29, so every
// position (offset + index < 2^29 + 2^23) and every distance between a query
// and a key position stays below 2^30.
constexpr int kMaxOffset = 1 << 29;

// A window of 2^30 or more admits every pair (all distances are below 2^30)
// and is passed to the kernels as "no window"; smaller windows keep every
// position +- window expression of the kernels inside an int.
constexpr int kWindowNone = 1 << 30;
int norm_window(int w) { return w >= kWindowNone ? 0 : w; }

int fwd_common(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Lq,
               int Lk, int d, float softmax_scale, int causal, int window, int q_offset, int k_offset, int dtype,
               void* stream) {
  int rc = check_common(B, Hq, Hkv, Lq, d, softmax_scale, causal, window, dtype);
  if (rc != FA_OK) return rc;
  if (Lk < 1 || Lk > kMaxL || q_offset < 0 || k_offset < 0 || q_offset > kMaxOffset || k_offset > kMaxOffset)
    return FA_ERR_INVALID_ARG;
  // the float32 path covers whole sequences only
  if (dtype == FA_DTYPE_F32 && (Lk != Lq || q_offset != k_offset)) return FA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return FA_ERR_INVALID_ARG;

  fa::FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.L = Lq; a.d = d;
  a.Lk = Lk;
  a.shift = q_offset - k_offset;
  a.window = norm_window(window);
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.f16 = dtype == FA_DTYPE_F16;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = (dtype == FA_DTYPE_F32) ? fa::launch_fwd_f32(a, causal != 0, s)
                                         : fa::launch_fwd_bf16(a, causal != 0, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int Hq, int Hkv, int L, int d,
                              float softmax_scale, int causal, int window, int dtype, void* stream) {
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, L, L, d, softmax_scale, causal, window, 0, 0, dtype, stream);
}

extern "C" int flash_attn_fwd_block(const void* q, const void* k, const void* v, void* o, float* lse,
                                    int B, int Hq, int Hkv, int Lq, int Lk, int d, float softmax_scale,
                                    int causal, int window, int q_offset, int k_offset, int dtype, void* stream) {
  if (dtype == FA_DTYPE_F32) return FA_ERR_UNSUPPORTED;
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, d, softmax_scale, causal, window, q_offset, k_offset,
                    dtype, stream);
}

extern "C" size_t flash_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int dtype) {
  if (check_common(B, Hq, Hkv, L, d, 1.f, 0, 0, dtype) != FA_OK) return 0;
  return workspace_bytes(B, Hq, L);
}

extern "C" size_t flash_attn_bwd_fused_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int dtype) {
  if (check_common(B, Hq, Hkv, L, d, 1.f, 0, 0, dtype) != FA_OK || !fused_fits(L, d)) return 0;
  return fused_workspace_bytes(B, Hq, L, d);
}

namespace {

// Common validation of the backward entry points; fills the kernel arguments.
int bwd_setup(fa::BwdArgs& a, const void* workspace, size_t ws_bytes, int B, int Hq, int Hkv, int L, int d,
              float scale, int causal, int window, int dtype) {
  int rc = check_common(B, Hq, Hkv, L, d, scale, causal, window, dtype);
  if (rc != FA_OK) return rc;
  if (dtype == FA_DTYPE_F32) return FA_ERR_UNSUPPORTED;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || ws_bytes < workspace_bytes(B, Hq, L))
    return FA_ERR_WORKSPACE;
  a.delta = static_cast<float*>(const_cast<void*>(workspace));
  a.lse2 = a.delta + (size_t)B * Hq * L;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.L = L; a.d = d;
  a.Lk = L;
  a.shift = 0;
  a.window = norm_window(window);
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.f16 = dtype == FA_DTYPE_F16;
  return FA_OK;
}

bool all_aligned(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return false;
  return true;
}

}  // namespace

extern "C" int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, void* dq, void* dk, void* dv,
                              void* workspace, size_t workspace_bytes,
                              int B, int Hq, int Hkv, int L, int d,
                              float softmax_scale, int causal, int window, int dtype, void* stream) {
  fa::BwdArgs a{};
  int rc = bwd_setup(a, workspace, workspace_bytes, B, Hq, Hkv, L, d, softmax_scale, causal, window, dtype);
  if (rc != FA_OK) return rc;
  if (!all_aligned({q, k, v, o, lse, dout, dq, dk, dv})) return FA_ERR_INVALID_ARG;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv;
  hipError_t e = fa::launch_bwd_bf16(a, causal != 0, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int flash_attn_bwd_fused(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                    const void* dout, void* dq, void* dk, void* dv,
                                    void* workspace, size_t workspace_bytes,
                                    int B, int Hq, int Hkv, int L, int d,
                                    float softmax_scale, int causal, int window, int dtype, void* stream) {
  fa::BwdArgs a{};
  int rc = bwd_setup(a, workspace, workspace_bytes, B, Hq, Hkv, L, d, softmax_scale, causal, window, dtype);
  if (rc != FA_OK) return rc;
  if (!fused_fits(L, d)) return FA_ERR_UNSUPPORTED;
  if (workspace_bytes < fused_workspace_bytes(B, Hq, L, d)) return FA_ERR_WORKSPACE;
  if (!all_aligned({q, k, v, o, lse, dout, dq, dk, dv})) return FA_ERR_INVALID_ARG;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.dq_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + ::workspace_bytes(B, Hq, L));
  hipError_t e = fa::launch_bwd_fused_bf16(a, causal != 0, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int flash_attn_bwd_preprocess(const void* o, const float* lse, const void* dout,
                                         void* workspace, size_t workspace_bytes,
                                         int B, int Hq, int Hkv, int L, int d, int dtype, void* stream) {
  fa::BwdArgs a{};
  int rc = bwd_setup(a, workspace, workspace_bytes, B, Hq, Hkv, L, d, 1.f, 0, 0, dtype);
  if (rc != FA_OK) return rc;
  if (!all_aligned({o, lse, dout})) return FA_ERR_INVALID_ARG;
  a.o = o; a.lse = lse; a.dout = dout;
  hipError_t e = fa::launch_bwd_preprocess_bf16(a, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int flash_attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                                   const void* workspace, size_t workspace_bytes, void* dk, void* dv,
                                   int B, int Hq, int Hkv, int L, int d,
                                   float softmax_scale, int causal, int window, int dtype, void* stream) {
  fa::BwdArgs a{};
  int rc = bwd_setup(a, workspace, workspace_bytes, B, Hq, Hkv, L, d, softmax_scale, causal, window, dtype);
  if (rc != FA_OK) return rc;
  if (!all_aligned({q, k, v, dout, dk, dv})) return FA_ERR_INVALID_ARG;
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.dk = dk; a.dv = dv;
  hipError_t e = fa::launch_bwd_dkdv_bf16(a, causal != 0, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int flash_attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                                 const void* workspace, size_t workspace_bytes, void* dq,
                                 int B, int Hq, int Hkv, int L, int d,
                                 float softmax_scale, int causal, int window, int dtype, void* stream) {
  fa::BwdArgs a{};
  int rc = bwd_setup(a, workspace, workspace_bytes, B, Hq, Hkv, L, d, softmax_scale, causal, window, dtype);
  if (rc != FA_OK) return rc;
  if (!all_aligned({q, k, v, dout, dq})) return FA_ERR_INVALID_ARG;
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.dq = dq;
  hipError_t e = fa::launch_bwd_dq_bf16(a, causal != 0, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int flash_attn_bwd_block(const void* q, const void* k, const void* v, const void* o,
                                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                    void* workspace, size_t workspace_bytes,
                                    int B, int Hq, int Hkv, int Lq, int Lk, int d, float softmax_scale,
                                    int causal, int window, int q_offset, int k_offset, int dtype, void* stream) {
  fa::BwdArgs a{};
  int rc = bwd_setup(a, workspace, workspace_bytes, B, Hq, Hkv, Lq, d, softmax_scale, causal, window, dtype);
  if (rc != FA_OK) return rc;
  if (Lk < 1 || Lk > kMaxL || q_offset < 0 || k_offset < 0 || q_offset > kMaxOffset || k_offset > kMaxOffset)
    return FA_ERR_INVALID_ARG;
  if (!all_aligned({q, k, v, o, lse, dout, dq, dk, dv})) return FA_ERR_INVALID_ARG;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.Lk = Lk;
  a.shift = q_offset - k_offset;
  hipError_t e = fa::launch_bwd_bf16(a, causal != 0, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// ---- backward without allocation: the per-row statistics live in a static
// device array instead of a caller-provided workspace.
namespace {

// 16 MiB: two float32 per query row, so B * Hq * L <= 2^21 rows.  Each GPU the
// library runs on holds its own copy until the process ends.
constexpr size_t kNoAllocScratchBytes = (size_t)FA_NOALLOC_MAX_ROWS * 2 * sizeof(float);
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// The array's device address, looked up once per device.  In host code the
// name `scratch` is only a host-side handle; kernels receive this address.
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return FA_ERR_HIP;
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" int flash_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                      const void* dout, void* dq, void* dk, void* dv,
                                      int B, int Hq, int Hkv, int L, int d,
                                      float softmax_scale, int causal, int window, int dtype, void* stream) {
  int rc = check_common(B, Hq, Hkv, L, d, softmax_scale, causal, window, dtype);
  if (rc != FA_OK) return rc;
  if (dtype == FA_DTYPE_F32) return FA_ERR_UNSUPPORTED;
  if ((long long)B * Hq * L > FA_NOALLOC_MAX_ROWS) return FA_ERR_TOO_LARGE;
  if (!all_aligned({q, k, v, o, lse, dout, dq, dk, dv})) return FA_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (s != nullptr) {
    // the scratch is looked up on the current device: the stream must be one of its streams
    int sdev = -1, cdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess || hipGetDevice(&cdev) != hipSuccess) return FA_ERR_HIP;
    if (sdev != cdev) return FA_ERR_INVALID_ARG;
  }
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != FA_OK) return rc;
  fa::BwdArgs a{};
  rc = bwd_setup(a, ws, kNoAllocScratchBytes, B, Hq, Hkv, L, d, softmax_scale, causal, window, dtype);
  if (rc != FA_OK) return rc;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv;
  // the three staged kernels: the preprocess overwrites every row's statistics
  // in the scratch before the dK/dV and dQ kernels read them
  hipError_t e = fa::launch_bwd_preprocess_bf16(a, s);
  if (e == hipSuccess) e = fa::launch_bwd_dkdv_bf16(a, causal != 0, s);
  if (e == hipSuccess) e = fa::launch_bwd_dq_bf16(a, causal != 0, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int flash_attn_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                                void* o, float* lse, int B, int Hq, int L, int d, int dtype, void* stream) {
  if (B < 1 || Hq < 1 || L < 1 || L > kMaxL) return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_F32) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!all_aligned({o_a, lse_a, o_b, lse_b, o, lse})) return FA_ERR_INVALID_ARG;
  fa::MergeArgs a{};
  a.o_a = o_a; a.lse_a = lse_a; a.o_b = o_b; a.lse_b = lse_b; a.o = o; a.lse = lse;
  a.rows = (long long)B * Hq * L;
  hipError_t e = fa::launch_merge(a, d, dtype, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

namespace {

// Validation shared by the decode entry points; fills the plan.
// sizes shared by the decode calls: Lq new tokens per sequence against a
// cache (or rolling buffer) of Lk entries
int decode_sizes(int B, int Hq, int Hkv, int Lq, int Lk, int d, int dtype) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Lq < 1 || Lq > kMaxL || Lk < 1 || Lk > kMaxL) return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (Hq % Hkv != 0) return FA_ERR_GQA;
  if ((long long)B * Hkv > 65535) return FA_ERR_INVALID_ARG;               // grid rows
  if (((long long)(Hq / Hkv) * Lq + 31) / 32 > 65535) return FA_ERR_UNSUPPORTED;   // row groups of 32
  if ((long long)B * Hq * Lq >= (1LL << 30)) return FA_ERR_INVALID_ARG;   // combine grid
  return FA_OK;
}

int decode_check(int B, int Hq, int Hkv, int Lq, int Lk, int d, int dtype, int& n_splits, int& split_keys) {
  const int rc = decode_sizes(B, Hq, Hkv, Lq, Lk, d, dtype);
  if (rc != FA_OK) return rc;
  if (Lk < Lq) return FA_ERR_INVALID_ARG;
  fa::decode_plan(B, Hkv, Lk, n_splits, split_keys);
  return FA_OK;
}

// the rolling-buffer decode: key splits of the W-slot buffer, then of the Lq new tokens' own keys
int rolling_check(int B, int Hq, int Hkv, int Lq, int W, int d, int dtype, int& ns_ring, int& sk_ring, int& ns_new,
                  int& sk_new) {
  const int rc = decode_sizes(B, Hq, Hkv, Lq, W, d, dtype);
  if (rc != FA_OK) return rc;
  fa::decode_plan(B, Hkv, W, ns_ring, sk_ring);
  fa::decode_plan(B, Hkv, Lq, ns_new, sk_new);
  return FA_OK;
}

size_t decode_bytes(int B, int Hq, int Lq, int d, int n_splits) {
  const size_t rows = (size_t)B * Hq * Lq;
  const size_t raw = (size_t)n_splits * rows * (size_t)(d + 1) * sizeof(float);
  return (raw + 255) & ~(size_t)255;
}

}  // namespace

extern "C" size_t flash_attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lk, int d, int dtype) {
  int ns = 0, sk = 0;
  if (decode_check(B, Hq, Hkv, Lq, Lk, d, dtype, ns, sk) != FA_OK) return 0;
  return decode_bytes(B, Hq, Lq, d, ns);
}

extern "C" int flash_attn_decode(const void* q, const void* k_cache, const void* v_cache, const int* cache_len,
                                 void* o, float* lse, void* workspace, size_t workspace_bytes,
                                 int B, int Hq, int Hkv, int Lq, int Lk, int d, float softmax_scale,
                                 int causal, int window, int dtype, void* stream) {
  int ns = 0, sk = 0;
  int rc = decode_check(B, Hq, Hkv, Lq, Lk, d, dtype, ns, sk);
  if (rc != FA_OK) return rc;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return FA_ERR_INVALID_ARG;
  if ((causal != 0 && causal != 1) || window < 0) return FA_ERR_INVALID_ARG;
  if (norm_window(window) > 0 && !causal) return FA_ERR_UNSUPPORTED;
  if (!all_aligned({q, k_cache, v_cache, o})) return FA_ERR_INVALID_ARG;
  if ((lse && !aligned16(lse)) || (reinterpret_cast<uintptr_t>(cache_len) & 3u) != 0) return FA_ERR_INVALID_ARG;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
      workspace_bytes < decode_bytes(B, Hq, Lq, d, ns))
    return FA_ERR_WORKSPACE;
  fa::DecodeArgs a{};
  a.q = q; a.k = k_cache; a.v = v_cache; a.cache_len = cache_len; a.o = o; a.lse = lse;
  a.rows = (long long)B * Hq * Lq;
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = a.part_o + (size_t)ns * (size_t)a.rows * d;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lk = Lk; a.d = d;
  a.window = norm_window(window);
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.f16 = dtype == FA_DTYPE_F16;
  a.n_splits = ns;
  a.split_keys = sk;
  a.split_base = 0;
  a.n_splits_total = ns;
  hipError_t e = fa::launch_decode(a, causal != 0, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" size_t flash_attn_decode_rolling_workspace_bytes(int B, int Hq, int Hkv, int Lq, int W, int d, int dtype) {
  int nr = 0, sr = 0, nn = 0, sn = 0;
  if (rolling_check(B, Hq, Hkv, Lq, W, d, dtype, nr, sr, nn, sn) != FA_OK) return 0;
  return decode_bytes(B, Hq, Lq, d, nr + nn);
}

extern "C" int flash_attn_decode_rolling(const void* q, const void* k_ring, const void* v_ring, const void* k_new,
                                         const void* v_new, const int* seen, void* o, float* lse, void* workspace,
                                         size_t workspace_bytes, int B, int Hq, int Hkv, int Lq, int W, int d,
                                         float softmax_scale, int window, int dtype, void* stream) {
  int nr = 0, sr = 0, nn = 0, sn = 0;
  int rc = rolling_check(B, Hq, Hkv, Lq, W, d, dtype, nr, sr, nn, sn);
  if (rc != FA_OK) return rc;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return FA_ERR_INVALID_ARG;
  if (window < 0 || window > W) return FA_ERR_INVALID_ARG;   // older keys are gone from the buffer
  if (!all_aligned({q, k_ring, v_ring, k_new, v_new, o})) return FA_ERR_INVALID_ARG;
  if (seen == nullptr || (reinterpret_cast<uintptr_t>(seen) & 3u) != 0) return FA_ERR_INVALID_ARG;
  if (lse && !aligned16(lse)) return FA_ERR_INVALID_ARG;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
      workspace_bytes < decode_bytes(B, Hq, Lq, d, nr + nn))
    return FA_ERR_WORKSPACE;
  fa::DecodeArgs ring{};
  ring.q = q; ring.k = k_ring; ring.v = v_ring; ring.cache_len = seen; ring.o = o; ring.lse = lse;
  ring.rows = (long long)B * Hq * Lq;
  ring.part_o = static_cast<float*>(workspace);
  ring.part_lse = ring.part_o + (size_t)(nr + nn) * (size_t)ring.rows * d;
  ring.B = B; ring.Hq = Hq; ring.Hkv = Hkv; ring.Lq = Lq; ring.Lk = W; ring.d = d;
  ring.window = window == 0 ? W : window;
  ring.scale_log2 = softmax_scale * 1.4426950408889634f;
  ring.f16 = dtype == FA_DTYPE_F16;
  ring.n_splits = nr;
  ring.split_keys = sr;
  ring.split_base = 0;
  ring.n_splits_total = nr + nn;
  // the new tokens against their own keys: a plain causal decode whose cache is exactly them
  fa::DecodeArgs fresh = ring;
  fresh.k = k_new; fresh.v = v_new; fresh.cache_len = nullptr; fresh.Lk = Lq;
  fresh.n_splits = nn;
  fresh.split_keys = sn;
  fresh.split_base = nr;
  hipError_t e = fa::launch_decode_rolling(ring, fresh, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

namespace {

// General masks: the plan's per-row lists hold at most 2^18 / 64 tiles and its
// work-group order covers at most 2048 work-group rows.
constexpr int kMaxMaskL = 1 << 18;
constexpr int kMaxGlobal = 1 << 16;

int check_mask(const fa_mask* m, int L) {
  if (m == nullptr || L < 1) return FA_ERR_INVALID_ARG;
  if ((m->causal != 0 && m->causal != 1) || m->window < 0) return FA_ERR_INVALID_ARG;
  if (m->n_global < 0 || m->n_global > kMaxGlobal || (m->n_global > 0 && m->global_pos == nullptr))
    return FA_ERR_INVALID_ARG;
  if (m->block_mask != nullptr && (m->block < 64 || m->block % 64 != 0)) return FA_ERR_UNSUPPORTED;
  if (L > kMaxMaskL) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int check_plan(const void* plan, size_t plan_bytes, int L) {
  if (plan == nullptr || (reinterpret_cast<uintptr_t>(plan) & 255u) != 0 || plan_bytes < fa::plan_layout(L).total)
    return FA_ERR_WORKSPACE;
  return FA_OK;
}

}  // namespace

extern "C" size_t flash_attn_mask_plan_bytes(int L) {
  if (L < 1 || L > kMaxMaskL) return 0;
  return fa::plan_layout(L).total;
}

extern "C" int flash_attn_mask_plan(const fa_mask* mask, int L, void* plan, size_t plan_bytes, void* stream) {
  int rc = check_mask(mask, L);
  if (rc != FA_OK) return rc;
  rc = check_plan(plan, plan_bytes, L);
  if (rc != FA_OK) return rc;
  fa::MaskDesc m{};
  m.causal = mask->causal;
  m.window = norm_window(mask->window);
  m.global_pos = mask->n_global > 0 ? mask->global_pos : nullptr;
  m.n_global = mask->n_global;
  m.block_mask = mask->block_mask;
  m.block = mask->block_mask != nullptr ? mask->block : 64;
  hipError_t e = fa::launch_mask_plan(m, L, plan, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

namespace {

// Workspace of the masked calls: the backward's -D_i and LSE_i*log2(e) rows
// (backward only), then the float32 partials of the global-position passes
// (the dK/dV and dQ passes run one after the other and share one region).
struct MaskedWs {
  fa::GlobalArgs rows, cols;
  size_t base, partial, total;
};

MaskedWs masked_ws(int B, int Hq, int Hkv, int L, int d, const fa_mask* m, bool backward) {
  MaskedWs w{};
  w.rows = fa::global_plan(L, m->n_global, B * Hq);
  w.cols = fa::global_plan(L, m->n_global, B * Hkv);
  w.base = backward ? workspace_bytes(B, Hq, L) : 0;
  w.partial = backward ? std::max(fa::global_dq_bytes(w.rows, B * Hq, d), fa::global_dkdv_bytes(w.cols, B * Hkv, d))
                       : fa::global_fwd_bytes(w.rows, B * Hq, d);
  if (w.rows.ngp == 0) w.partial = 0;
  w.total = w.base + w.partial;
  return w;
}

}  // namespace

extern "C" size_t flash_attn_masked_workspace_bytes(int B, int Hq, int Hkv, int L, int d, const fa_mask* mask,
                                                    int backward) {
  if (check_common(B, Hq, Hkv, L, d, 1.f, 0, 0, FA_DTYPE_BF16) != FA_OK || check_mask(mask, L) != FA_OK) return 0;
  return masked_ws(B, Hq, Hkv, L, d, mask, backward != 0).total;
}

extern "C" int flash_attn_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                                     void* workspace, size_t workspace_bytes,
                                     int B, int Hq, int Hkv, int L, int d, float softmax_scale,
                                     const fa_mask* mask, const void* plan, size_t plan_bytes, int dtype,
                                     void* stream) {
  if (mask == nullptr) return FA_ERR_INVALID_ARG;
  int rc = check_common(B, Hq, Hkv, L, d, softmax_scale, mask->causal, mask->window, dtype);
  if (rc != FA_OK) return rc;
  if (dtype == FA_DTYPE_F32) return FA_ERR_UNSUPPORTED;
  rc = check_mask(mask, L);
  if (rc != FA_OK) return rc;
  rc = check_plan(plan, plan_bytes, L);
  if (rc != FA_OK) return rc;
  MaskedWs w = masked_ws(B, Hq, Hkv, L, d, mask, false);
  if (w.rows.ngp > 0 && (long long)B * Hq > 65535) return FA_ERR_UNSUPPORTED;   // grid rows of the global pass
  if (w.total > 0 && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
                      workspace_bytes < w.total))
    return FA_ERR_WORKSPACE;
  if (!all_aligned({q, k, v, o}) || (lse && !aligned16(lse))) return FA_ERR_INVALID_ARG;
  fa::FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.L = L; a.d = d;
  a.Lk = L;
  a.shift = 0;
  a.window = norm_window(mask->window);
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.f16 = dtype == FA_DTYPE_F16;
  if (w.rows.ngp > 0) {
    w.rows.part = static_cast<float*>(workspace);
    w.rows.part_lse = w.rows.part + (size_t)w.rows.n_splits * B * Hq * w.rows.ngp * d;
  }
  hipError_t e = fa::launch_fwd_masked(a, fa::plan_ptrs(plan, L), w.rows, mask->causal != 0,
                                       reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" int flash_attn_bwd_masked(const void* q, const void* k, const void* v, const void* o,
                                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                     void* workspace, size_t workspace_bytes,
                                     int B, int Hq, int Hkv, int L, int d, float softmax_scale,
                                     const fa_mask* mask, const void* plan, size_t plan_bytes, int dtype,
                                     void* stream) {
  if (mask == nullptr) return FA_ERR_INVALID_ARG;
  int rc = check_mask(mask, L);
  if (rc != FA_OK) return rc;
  fa::BwdArgs a{};
  rc = bwd_setup(a, workspace, workspace_bytes, B, Hq, Hkv, L, d, softmax_scale, mask->causal, mask->window, dtype);
  if (rc != FA_OK) return rc;
  rc = check_plan(plan, plan_bytes, L);
  if (rc != FA_OK) return rc;
  MaskedWs w = masked_ws(B, Hq, Hkv, L, d, mask, true);
  if (w.rows.ngp > 0 && (long long)B * Hq > 65535) return FA_ERR_UNSUPPORTED;   // grid rows of the global passes
  if (workspace_bytes < w.total) return FA_ERR_WORKSPACE;
  if (!all_aligned({q, k, v, o, lse, dout, dq, dk, dv})) return FA_ERR_INVALID_ARG;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
  a.dq = dq; a.dk = dk; a.dv = dv;
  float* partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.base);
  w.rows.part = partials;
  w.cols.part = partials;
  hipError_t e = fa::launch_bwd_masked(a, fa::plan_ptrs(plan, L), w.rows, w.cols, mask->causal != 0,
                                       reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

extern "C" const char* flash_attn_strerror(int code) {
  switch (code) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, non-positive size, or bad scale)";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration (head dim, dtype, or a decode window without causal)";
    case FA_ERR_GQA: return "number of query heads is not a multiple of the number of key/value heads";
    case FA_ERR_WORKSPACE: return "backward workspace missing, misaligned or too small";
    case FA_ERR_HIP: return "HIP launch or runtime error";
    case FA_ERR_TOO_LARGE: return "sizes exceed the static scratch of flash_attn_bwd_noalloc (B * Hq * L > 2^21)";
    default: return "unknown error code";
  }
}

extern "C" int flash_attn_version(void) { return 100; }
