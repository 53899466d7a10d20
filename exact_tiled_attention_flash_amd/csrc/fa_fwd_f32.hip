// fa_fwd_f32.hip -- tiled exact attention forward in fp32 throughout (gfx950).
//
// The fp32 path serves small, accuracy-first problems.  One wave owns 64 query
// rows (one per lane); 32-key tiles of K and V are staged in LDS and every lane
// applies the online-softmax recurrence to its own row: running maximum,
// running sum, and a rescale of the partial output when the maximum grows
// (transformer.xph.ink "高效注意力：FlashAttention 与线性注意力", 原理与机制;
// claspmoon.cn "14 · 缩放定律与高效注意力" §3.2).  Scores and products are
// plain fp32 FMAs; LDS reads are wave-wide broadcasts.
#include "fa_common.hpp"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kRows = 64;   // query rows per work-group (one wave)
constexpr int kKeys = 32;   // keys per LDS tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void fwd_f32_kernel(FwdArgs a) {
  __shared__ float ks[kKeys][D];
  __shared__ float vs[kKeys][D];
  const int lane = threadIdx.x;
  const int bh = blockIdx.x / a.n_qtiles;
  const int qt = blockIdx.x % a.n_qtiles;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int L = a.L;
  const float* Qh = reinterpret_cast<const float*>(a.q) + ((size_t)(b * a.Hq + h) * L) * D;
  const float* Kh = reinterpret_cast<const float*>(a.k) + ((size_t)(b * a.Hkv + hk) * L) * D;
  const float* Vh = reinterpret_cast<const float*>(a.v) + ((size_t)(b * a.Hkv + hk) * L) * D;

  const int q0 = qt * kRows;
  const int my_q = q0 + lane;
  const int qmax = min(L, q0 + kRows) - 1;
  const int window = a.window;

  float qv[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qv[c] = (my_q < L) ? Qh[(size_t)my_q * D + c] : 0.f;
    acc[c] = 0.f;
  }
  const float cs = a.scale_log2;
  float m_run = kNegBig, l_run = 0.f;

  const int kv_end = range_key_end<CAUSAL>(L, window, qmax);
  const int kv_begin = (window > 0) ? max(0, q0 - window + 1) : 0;
  for (int k0 = (kv_begin / kKeys) * kKeys; k0 < kv_end; k0 += kKeys) {
    __syncthreads();
    for (int e = lane; e < kKeys * D; e += 64) {
      const int r = e / D, c = e % D;
      const int row = min(k0 + r, L - 1);
      ks[r][c] = Kh[(size_t)row * D + c];
      vs[r][c] = Vh[(size_t)row * D + c];
    }
    __syncthreads();
    float s[kKeys];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = fmaf(qv[c], ks[j][c], dot);
      const int kk = k0 + j;
      s[j] = range_ok<CAUSAL>(kk, my_q, L, window) ? dot : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx * cs);
    const float alpha = fast_exp2(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      s[j] = fast_exp2(fmaf(s[j], cs, -m_new));
      rs += s[j];
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      float t = acc[c] * alpha;
#pragma unroll
      for (int j = 0; j < kKeys; ++j) t = fmaf(s[j], vs[j][c], t);
      acc[c] = t;
    }
  }
  if (my_q < L) {
    const float inv = 1.f / l_run;
    float* Oq = reinterpret_cast<float*>(a.o) + ((size_t)(b * a.Hq + h) * L + my_q) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) Oq[c] = acc[c] * inv;
    if (a.lse != nullptr) a.lse[(size_t)(b * a.Hq + h) * L + my_q] = (m_run + __log2f(l_run)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& args, hipStream_t stream) {
  FwdArgs a = args;
  a.n_qtiles = (a.L + kRows - 1) / kRows;
  const long long nblk = (long long)a.B * a.Hq * a.n_qtiles;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)nblk), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, bool causal, hipStream_t stream) {
  if (a.d == 128) return causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  return causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace fa
