// coissue.hip -- microbenchmark of the gfx950 SIMD facts the attention
// kernels' schedules rest on.  Not part of the library.
//
// One work-group of 8 waves per CU (96 KiB of LDS keeps a second one out), so
// waves w and w + 4 share SIMD w % 4.  Every wave runs the same number of loop
// iterations; in each one a "matrix" wave issues 8 v_mfma_f32_32x32x16_bf16
// on four independent accumulators and a "vector" wave does 16 lanes-values
// of softmax-like work (fma, exp2, add: 48 VALU instructions, the exp2 at half
// rate).  The modes place the two kinds of work:
//   mfma 1/SIMD, mfma 2/SIMD  -- sustained MFMA rate with one or two waves;
//   valu 1/SIMD, valu 2/SIMD  -- the vector work alone;
//   split                    -- waves 0-3 matrix, waves 4-7 vector (does one
//                               wave's VALU issue under the other's MFMA?);
//   split+prio               -- the same with the matrix waves at s_setprio 3;
//   same-wave 1/SIMD, 2/SIMD -- each wave does both, MFMA and VALU interleaved
//                               one MFMA then six VALU (does a wave's own VALU
//                               issue under its MFMA?);
//   ... acc in AGPRs         -- mfma 2/SIMD, split and same-wave 2/SIMD again
//                               with the accumulators (MFMA source C and
//                               result) in AGPRs rather than VGPRs.  The
//                               compiler picks that form for a function whose
//                               inline asm names an AGPR operand, so these
//                               modes carry an empty asm statement with one.
// If two kinds of work overlap, the mixed time approaches the larger of the
// two times alone; if they serialise, it approaches their sum.  The shader
// clock is read with s_memtime against the 100 MHz s_memrealtime.
//
// Build and run: python -m exact_tiled_attention_flash_amd.probes coissue
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum { M1 = 0, M2, V1, V2, SPLIT, SPLIT_PRIO, SAME1, SAME2, M2_ACC, SPLIT_ACC, SAME2_ACC, NMODES };
static const char* kNames[NMODES] = {"mfma 1/SIMD", "mfma 2/SIMD", "valu 1/SIMD", "valu 2/SIMD",
                                     "split (mfma | valu)", "split, mfma waves prio 3",
                                     "same-wave 1/SIMD", "same-wave 2/SIMD",
                                     "mfma 2/SIMD, acc in AGPRs", "split, acc in AGPRs",
                                     "same-wave 2/SIMD, acc AGPRs"};
constexpr bool acc_in_agprs(int mode) { return mode == M2_ACC || mode == SPLIT_ACC || mode == SAME2_ACC; }

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));         \
      std::exit(1);                                                               \
    }                                                                             \
  } while (0)

template <int MODE>
__global__ __launch_bounds__(512, 1) void probe(float* out, unsigned long long* clk, int iters, float c) {
  __shared__ float pad[24 * 1024];   // 96 KiB: one work-group per CU
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const bool hi = wave >= 4;
  bool mat = false, vec = false;
  switch (MODE) {
    case M1: mat = !hi; break;
    case M2: case M2_ACC: mat = true; break;
    case V1: vec = !hi; break;
    case V2: vec = true; break;
    case SPLIT:
    case SPLIT_PRIO: case SPLIT_ACC: mat = !hi; vec = hi; break;
    case SAME1: mat = vec = !hi; break;
    case SAME2: case SAME2_ACC: mat = vec = true; break;
  }
  pad[threadIdx.x] = c;
  __syncthreads();
  const float seed = pad[(threadIdx.x + 1) & 511];
  if constexpr (acc_in_agprs(MODE)) asm volatile("; AGPR operand: %0" ::"a"(seed));
  unsigned long long t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  bf16x8 a0, a1, b;
  for (int i = 0; i < 8; ++i) {
    a0[i] = (__bf16)(seed * (lane + i));
    a1[i] = (__bf16)(seed * (lane - i));
    b[i] = (__bf16)(seed * 0.5f);
  }
  f32x16 acc[4] = {};
  float v[16], sum[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < 16; ++i) v[i] = seed * (float)(i + lane) * 0.01f;
  if (MODE == SPLIT_PRIO && mat) __builtin_amdgcn_s_setprio(3);
  // three separate loops, so that no wave carries the other kind's registers
  // through its loop (a shared loop had the vector waves copy the AGPR
  // accumulators every iteration)
  if (mat && vec) {
    for (int it = 0; it < iters; ++it) {
      // one MFMA, then six VALU instructions (two elements), eight times
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((m & 1) ? a1 : a0, b, acc[m & 3], 0, 0, 0);
#pragma unroll
        for (int e = 2 * m; e < 2 * m + 2; ++e) {
          v[e] = __builtin_amdgcn_exp2f(fmaf(v[e], c, -1.0f));
          sum[e & 3] += v[e];
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // six VALU
      }
    }
  } else if (mat) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int m = 0; m < 8; ++m)
        acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((m & 1) ? a1 : a0, b, acc[m & 3], 0, 0, 0);
    }
  } else if (vec) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        v[e] = __builtin_amdgcn_exp2f(fmaf(v[e], c, -1.0f));
        sum[e & 3] += v[e];
      }
    }
  }
  if (MODE == SPLIT_PRIO && mat) __builtin_amdgcn_s_setprio(0);
  float r = sum[0] + sum[1] + sum[2] + sum[3];
  for (int q = 0; q < 4; ++q)
    for (int i = 0; i < 16; ++i) r += acc[q][i];
  for (int i = 0; i < 16; ++i) r += v[i];
  out[blockIdx.x * 512 + threadIdx.x] = r;
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

template <int MODE>
static void run(int cus, int iters, float* out, unsigned long long* clk, unsigned long long* hclk) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  for (int rep = 0; rep < 2; ++rep)   // first launch warms the clocks
    hipLaunchKernelGGL(probe<MODE>, dim3(cus), dim3(512), 0, 0, out, clk, iters, 0.5f);
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e0, 0));
  hipLaunchKernelGGL(probe<MODE>, dim3(cus), dim3(512), 0, 0, out, clk, iters, 0.5f);
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipMemcpy(hclk, clk, sizeof(unsigned long long) * 2 * cus, hipMemcpyDeviceToHost));
  double cyc = 0, real = 0;
  for (int i = 0; i < cus; ++i) {
    cyc += (double)hclk[2 * i];
    real += (double)hclk[2 * i + 1];
  }
  cyc /= cus;
  real /= cus;
  const double ghz = cyc / (real * 10.0);   // s_memrealtime ticks at 100 MHz
  int mat_waves = 0, vec_waves = 0;
  switch (MODE) {
    case M1: mat_waves = 4; break;
    case M2: case M2_ACC: mat_waves = 8; break;
    case V1: vec_waves = 4; break;
    case V2: vec_waves = 8; break;
    case SPLIT: case SPLIT_PRIO: case SPLIT_ACC: mat_waves = 4; vec_waves = 4; break;
    case SAME1: mat_waves = vec_waves = 4; break;
    case SAME2: case SAME2_ACC: mat_waves = vec_waves = 8; break;
  }
  const double flop = (double)cus * mat_waves * iters * 8 * (2.0 * 32 * 32 * 16);
  const double mfma_per_simd = (double)mat_waves / 4 * iters * 8;
  const double valu_per_simd = (double)vec_waves / 4 * iters * 48;
  std::printf("%-26s %8.3f ms  %6.3f GHz  %9.1f cyc/iter/SIMD  MFMA %7.1f TFLOP/s  cyc/MFMA %6.2f  cyc/VALU %5.2f\n",
              kNames[MODE], ms, ghz, cyc / iters, flop / (ms * 1e-3) / 1e12,
              mfma_per_simd > 0 ? cyc / mfma_per_simd : 0.0, valu_per_simd > 0 ? cyc / valu_per_simd : 0.0);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
}

int main(int argc, char** argv) {
  int dev = 0;
  hipDeviceProp_t p;
  CHECK(hipGetDeviceProperties(&p, dev));
  const int cus = p.multiProcessorCount;
  const int iters = argc > 1 ? std::atoi(argv[1]) : 4000;
  std::printf("device %s, %d CUs, %d iterations per wave; per iteration a matrix wave issues 8 MFMA "
              "32x32x16 bf16, a vector wave 48 VALU (16 x fma, exp2, add)\n", p.gcnArchName, cus, iters);
  float* out;
  unsigned long long* clk;
  CHECK(hipMalloc(&out, sizeof(float) * 512 * cus));
  CHECK(hipMalloc(&clk, sizeof(unsigned long long) * 2 * cus));
  unsigned long long* hclk = (unsigned long long*)std::malloc(sizeof(unsigned long long) * 2 * cus);
  run<M1>(cus, iters, out, clk, hclk);
  run<M2>(cus, iters, out, clk, hclk);
  run<V1>(cus, iters, out, clk, hclk);
  run<V2>(cus, iters, out, clk, hclk);
  run<SPLIT>(cus, iters, out, clk, hclk);
  run<SPLIT_PRIO>(cus, iters, out, clk, hclk);
  run<SAME1>(cus, iters, out, clk, hclk);
  run<SAME2>(cus, iters, out, clk, hclk);
  run<M2_ACC>(cus, iters, out, clk, hclk);
  run<SPLIT_ACC>(cus, iters, out, clk, hclk);
  run<SAME2_ACC>(cus, iters, out, clk, hclk);
  // the two accumulator forms once more, alternated, so that a clock
  // difference between them is not an effect of the order
  run<M2>(cus, iters, out, clk, hclk);
  run<M2_ACC>(cus, iters, out, clk, hclk);
  run<M2>(cus, iters, out, clk, hclk);
  run<M2_ACC>(cus, iters, out, clk, hclk);
  run<SPLIT>(cus, iters, out, clk, hclk);
  run<SPLIT_ACC>(cus, iters, out, clk, hclk);
  CHECK(hipFree(out));
  CHECK(hipFree(clk));
  std::free(hclk);
  return 0;
}
