// fa_merge.hip -- exact combination of two partial attention results.
//
// Ring attention (claspmoon.cn "14 · 缩放定律与高效注意力" §5.1: sequence
// parallelism on top of exact tiled attention) attends a query chunk to one
// key/value chunk per step and gets a partial (O_p, LSE_p) normalised over that
// chunk's keys.  Two partials over disjoint key sets combine exactly -- the
// online-softmax rescaling (transformer.xph.ink "高效注意力：FlashAttention 与
// 线性注意力", 原理与机制) applied to whole chunks:
//     LSE = log(e^{LSE_a} + e^{LSE_b}),
//     O   = e^{LSE_a - LSE} O_a + e^{LSE_b - LSE} O_b,
// where a side with LSE = -inf has no keys and weight 0 (both: O = 0, LSE = -inf).
// HBM-bound and elementwise: each thread owns 8 consecutive elements of one row,
// and a row's d/8 threads are consecutive lanes of one wave, so the row's
// log-sum-exp values are read by all of them before any of them writes.
#include "fa_common.hpp"
#include "fa_kernels.h"

namespace fa {

namespace {

template <int D, int DT>   // DT: 0 fp32, 1 bf16, 2 fp16
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerBlock = 256 / kLanesPerRow;
  const long long row = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const int part = threadIdx.x % kLanesPerRow;
  if (row >= a.rows) return;
  const float la = a.lse_a[row], lb = a.lse_b[row];
  const float m = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, lse = -INFINITY;
  if (m != -INFINITY) {
    const float ea = __expf(la - m), eb = __expf(lb - m);   // exp(-inf) = 0
    const float tot = ea + eb;
    wa = ea / tot;
    wb = eb / tot;
    lse = m + __logf(tot);
  }
  const size_t off = (size_t)row * D + 8 * part;
  float r[8];
  if constexpr (DT == 0) {
    const f32x4* pa = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.o_a) + off);
    const f32x4* pb = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.o_b) + off);
    const f32x4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = wa * a0[i] + wb * b0[i];
      r[4 + i] = wa * a1[i] + wb * b1[i];
    }
    f32x4* po = reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + off);
    po[0] = f32x4{r[0], r[1], r[2], r[3]};
    po[1] = f32x4{r[4], r[5], r[6], r[7]};
  } else {
    constexpr bool F16 = DT == 2;
    const bf16x8 xa = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(a.o_a) + off);
    const bf16x8 xb = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(a.o_b) + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = wa * unpack1<F16>(xa[i]) + wb * unpack1<F16>(xb[i]);
    *reinterpret_cast<bf16x8*>(static_cast<bf16*>(a.o) + off) = pack8<F16>(r[0], r[1], r[2], r[3], r[4], r[5], r[6], r[7]);
  }
  if (part == 0) a.lse[row] = lse;
}

template <int D>
hipError_t launch_d(const MergeArgs& a, int dtype, hipStream_t stream) {
  constexpr int kRowsPerBlock = 256 / (D / 8);
  const unsigned grid = (unsigned)((a.rows + kRowsPerBlock - 1) / kRowsPerBlock);
  if (dtype == 0) hipLaunchKernelGGL((merge_kernel<D, 0>), dim3(grid), dim3(256), 0, stream, a);
  else if (dtype == 1) hipLaunchKernelGGL((merge_kernel<D, 1>), dim3(grid), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((merge_kernel<D, 2>), dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int d, int dtype, hipStream_t stream) {
  return d == 128 ? launch_d<128>(a, dtype, stream) : launch_d<64>(a, dtype, stream);
}

}  // namespace fa
