// fa_fwd_f32.hip -- tiled exact attention forward in fp32 throughout (gfx950).
//
// The fp32 path serves small, accuracy-first problems, where the whole job is a
// few dozen work-groups: latency, not throughput, decides its time.  So the
// work of one query row is spread over 16 lanes.  A work-group of 4 waves owns
// 16 query rows; lane l of wave w holds query row l % 16 and key subset
// s = 4w + l / 16.  64-key tiles of K and V are staged in LDS (rows padded so
// that the 4 subsets a wave reads at once sit in different banks), and subset
// s takes keys 4s .. 4s + 3 of every tile.  Every lane runs the online-softmax
// recurrence over its own keys -- running maximum, running sum, rescale of the
// partial output when the maximum grows (transformer.xph.ink "高效注意力：
// FlashAttention 与线性注意力", 原理与机制; claspmoon.cn "14 · 缩放定律与高效
// 注意力" §3.2) -- and the 16 partial (m, l, O) of a row are then merged
// exactly, each scaled by exp(m_s - max m): first the 4 lanes of a wave that
// share the row (cross-lane reads), then the 4 waves in a fixed order through
// LDS, so the result does not depend on timing.  Scores and products are plain
// fp32 FMAs.
#include "fa_common.hpp"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kRows = 16;   // query rows per work-group
constexpr int kTile = 64;   // keys per LDS tile (16 subsets x 4 keys)

template <int D>
struct F32Cfg {
  static constexpr int KSTR = D + 4;                  // padded row, floats
  static constexpr int TILE = kTile * KSTR;           // floats per staged tile
  static constexpr int NV = kTile * D / 4 / 256;      // 16-byte pieces per thread per tensor
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fwd_f32_kernel(FwdArgs a) {
  using C = F32Cfg<D>;
  __shared__ __attribute__((aligned(16))) float ks[C::TILE];
  __shared__ __attribute__((aligned(16))) float vs[C::TILE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, sub = 4 * wave + (lane >> 4);
  const int bh = blockIdx.y;
  const int qt = blockIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int L = a.L;
  const float* Qh = reinterpret_cast<const float*>(a.q) + ((size_t)(b * a.Hq + h) * L) * D;
  const float* Kh = reinterpret_cast<const float*>(a.k) + ((size_t)(b * a.Hkv + hk) * L) * D;
  const float* Vh = reinterpret_cast<const float*>(a.v) + ((size_t)(b * a.Hkv + hk) * L) * D;

  const int q0 = qt * kRows;
  const int my_q = q0 + row;
  const int qmax = min(L, q0 + kRows) - 1;
  const int window = a.window;

  float qv[D], acc[D];
  {
    const float* Qr = Qh + (size_t)min(my_q, L - 1) * D;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(Qr + c);
      qv[c] = x[0]; qv[c + 1] = x[1]; qv[c + 2] = x[2]; qv[c + 3] = x[3];
    }
  }
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;
  const float cs = a.scale_log2;
  float m_run = kNegBig, l_run = 0.f;

  const int kv_end = range_key_end<CAUSAL>(L, window, qmax);
  const int kv_begin = (window > 0) ? max(0, q0 - window + 1) : 0;
  const int t_lo = kv_begin / kTile, t_hi = (kv_end - 1) / kTile;   // kv_end >= 1 for a real row

  // tile copies: thread tid moves 16-byte piece tid + 256 n of the tile; the
  // next tile's loads are in flight while the current one is used
  f32x4 kr[C::NV], vr[C::NV];
  int src[C::NV], dst[C::NV];
#pragma unroll
  for (int n = 0; n < C::NV; ++n) {
    const int e = tid + 256 * n, r = e / (D / 4), c4 = e % (D / 4);
    src[n] = r * D + 4 * c4;
    dst[n] = r * C::KSTR + 4 * c4;
  }
  const int last_row = (L - 1) * D;
  if (t_lo <= t_hi) {
#pragma unroll
    for (int n = 0; n < C::NV; ++n) {
      const int o = min(t_lo * kTile * D + src[n], last_row + src[n] % D);
      kr[n] = *reinterpret_cast<const f32x4*>(Kh + o);
      vr[n] = *reinterpret_cast<const f32x4*>(Vh + o);
    }
  }
  for (int t = t_lo; t <= t_hi; ++t) {
    __syncthreads();                 // every lane is done with the previous tile
#pragma unroll
    for (int n = 0; n < C::NV; ++n) {
      *reinterpret_cast<f32x4*>(ks + dst[n]) = kr[n];
      *reinterpret_cast<f32x4*>(vs + dst[n]) = vr[n];
    }
    __syncthreads();
    if (t < t_hi) {
#pragma unroll
      for (int n = 0; n < C::NV; ++n) {
        const int o = min((t + 1) * kTile * D + src[n], last_row + src[n] % D);
        kr[n] = *reinterpret_cast<const f32x4*>(Kh + o);
        vr[n] = *reinterpret_cast<const f32x4*>(Vh + o);
      }
    }
    float s[4];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float* kp = ks + (4 * sub + j) * C::KSTR;
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D; c += 4) {
        const f32x4 k4 = *reinterpret_cast<const f32x4*>(kp + c);
        dot = fmaf(qv[c], k4[0], dot);
        dot = fmaf(qv[c + 1], k4[1], dot);
        dot = fmaf(qv[c + 2], k4[2], dot);
        dot = fmaf(qv[c + 3], k4[3], dot);
      }
      s[j] = range_ok<CAUSAL>(t * kTile + 4 * sub + j, my_q, L, window) ? dot : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx * cs);
    const float alpha = fast_exp2(m_run - m_new);
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] = fast_exp2(fmaf(s[j], cs, -m_new));
    l_run = fmaf(l_run, alpha, (s[0] + s[1]) + (s[2] + s[3]));
    m_run = m_new;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      float t0 = acc[c] * alpha, t1 = acc[c + 1] * alpha, t2 = acc[c + 2] * alpha, t3 = acc[c + 3] * alpha;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(vs + (4 * sub + j) * C::KSTR + c);
        t0 = fmaf(s[j], v4[0], t0);
        t1 = fmaf(s[j], v4[1], t1);
        t2 = fmaf(s[j], v4[2], t2);
        t3 = fmaf(s[j], v4[3], t3);
      }
      acc[c] = t0; acc[c + 1] = t1; acc[c + 2] = t2; acc[c + 3] = t3;
    }
  }

  // ---- merge the 4 lanes of this wave that share the row (lanes row + 16 u)
  float m_w = fmaxf(m_run, __shfl_xor(m_run, 16));
  m_w = fmaxf(m_w, __shfl_xor(m_w, 32));
  const float sc = fast_exp2(m_run - m_w);
  float l_w = l_run * sc;
  l_w += __shfl_xor(l_w, 16);
  l_w += __shfl_xor(l_w, 32);
#pragma unroll
  for (int c = 0; c < D; ++c) {
    float x = acc[c] * sc;
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    acc[c] = x;
  }

  // ---- merge the 4 waves: waves 1..3 leave (m, l, O) in LDS, wave 0 adds
  // them in wave order.  Layout (reusing the K tile): per wave w >= 1 and row r,
  // D partial outputs at ((w-1)*16 + r) * KSTR, then m and l after all of them.
  __syncthreads();                   // the last tile is no longer read
  float* part = ks;
  float* stats = ks + 3 * kRows * C::KSTR;
  if (wave > 0 && lane < 16) {
    float* dst = part + ((wave - 1) * kRows + row) * C::KSTR;
#pragma unroll
    for (int c = 0; c < D; c += 4)
      *reinterpret_cast<f32x4*>(dst + c) = f32x4{acc[c], acc[c + 1], acc[c + 2], acc[c + 3]};
    stats[2 * ((wave - 1) * kRows + row)] = m_w;
    stats[2 * ((wave - 1) * kRows + row) + 1] = l_w;
  }
  __syncthreads();
  if (wave != 0 || lane >= 16 || my_q >= L) return;
  float mw[4], lw[4];
  mw[0] = m_w;
  lw[0] = l_w;
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    mw[w] = stats[2 * ((w - 1) * kRows + row)];
    lw[w] = stats[2 * ((w - 1) * kRows + row) + 1];
  }
  const float m_tot = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
  float scw[4], l_tot = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    scw[w] = fast_exp2(mw[w] - m_tot);
    l_tot = fmaf(lw[w], scw[w], l_tot);
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  float* Oq = reinterpret_cast<float*>(a.o) + ((size_t)(b * a.Hq + h) * L + my_q) * D;
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    float o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = acc[c + u] * scw[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4 p4 = *reinterpret_cast<const f32x4*>(part + ((w - 1) * kRows + row) * C::KSTR + c);
      o[0] = fmaf(p4[0], scw[w], o[0]);
      o[1] = fmaf(p4[1], scw[w], o[1]);
      o[2] = fmaf(p4[2], scw[w], o[2]);
      o[3] = fmaf(p4[3], scw[w], o[3]);
    }
    *reinterpret_cast<f32x4*>(Oq + c) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
  }
  if (a.lse != nullptr)
    a.lse[(size_t)(b * a.Hq + h) * L + my_q] = l_tot > 0.f ? (m_tot + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& args, hipStream_t stream) {
  FwdArgs a = args;
  a.n_qtiles = (a.L + kRows - 1) / kRows;
  // 2-D grid: query tiles x (batch, head), each dimension far below its limit
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)a.n_qtiles, (unsigned)(a.B * a.Hq)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, bool causal, hipStream_t stream) {
  if (a.d == 128) return causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
  return causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

}  // namespace fa
