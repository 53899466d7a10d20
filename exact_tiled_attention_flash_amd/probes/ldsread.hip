// LDS read throughput per CU on gfx950 for the three read forms the tile
// kernels use to feed MFMA operands: 16-byte row reads (ds_read_b128), 8-byte
// row reads (ds_read_b64) and 8-byte transposing reads (ds_read_b64_tr_b16).
//
// One work-group per CU (96 KiB of LDS each), 4 to 16 waves.  The LDS is
// filled first (so that no read is of undefined memory), then every wave reads
// 1 KiB-spaced blocks of it, each lane at a distinct bank-aligned address, and
// folds what it read into a value that is stored, so no read can be removed.
// Shader cycles come from s_memtime, the clock from s_memtime against the
// 100 MHz s_memrealtime.  All reads stay inside the 96 KiB block.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));              \
      exit(1);                                                                    \
    }                                                                             \
  } while (0)

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kLdsBytes = 96 * 1024;   // more than half of the CU's 160 KiB: one work-group per CU
constexpr int kUnroll = 8;             // reads in flight per wave between waits

enum Mode { kB128 = 0, kB64 = 1, kTr16 = 2 };

template <int MODE>
__global__ void lds_read_kernel(int iters, unsigned* out, long long* clocks) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int i = t; i < kLdsBytes / 4; i += blockDim.x) reinterpret_cast<unsigned*>(lds)[i] = i * 2654435761u;
  __syncthreads();
  const long long c0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  u32x4 acc = {0, 0, 0, 0};
  constexpr int kBlocks = kLdsBytes / 1024 - 1;   // 1 KiB blocks a wave may start at
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      // block index below kBlocks (it <= 10^6, so no overflow): the wave's 1 KiB stays inside the array
      const int off = ((8 * wave + it * kUnroll + u) % kBlocks) * 1024;
      if constexpr (MODE == kB128) {
        acc ^= *(const LDS_AS u32x4*)((const LDS_AS char*)lds + off + 16 * lane);
      } else {
        i16x4 v;
        if constexpr (MODE == kB64)
          v = *(const LDS_AS i16x4*)((const LDS_AS char*)lds + off + 8 * lane);
        else
          v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)((LDS_AS char*)lds + off + 8 * lane));
        acc[0] ^= (unsigned)(unsigned short)v[0] | ((unsigned)(unsigned short)v[1] << 16);
        acc[1] ^= (unsigned)(unsigned short)v[2] | ((unsigned)(unsigned short)v[3] << 16);
      }
    }
  }
  __syncthreads();
  const long long c1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  out[(size_t)blockIdx.x * blockDim.x + t] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (t == 0) {
    clocks[2 * blockIdx.x] = c1 - c0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

template <int MODE>
void run(const char* name, int waves, int grid, int iters) {
  const int block = 64 * waves;
  unsigned* out = nullptr;
  long long* clocks = nullptr;
  CHECK(hipMalloc(&out, sizeof(unsigned) * (size_t)grid * block));
  CHECK(hipMalloc(&clocks, sizeof(long long) * 2 * grid));
  for (int rep = 0; rep < 3; ++rep) {   // the last launch's clocks are kept
    hipLaunchKernelGGL((lds_read_kernel<MODE>), dim3(grid), dim3(block), 0, 0, iters, out, clocks);
    CHECK(hipGetLastError());
  }
  CHECK(hipDeviceSynchronize());
  std::vector<long long> c(2 * grid);
  CHECK(hipMemcpy(c.data(), clocks, sizeof(long long) * 2 * grid, hipMemcpyDeviceToHost));
  double cyc = 0, rt = 0;
  for (int i = 0; i < grid; ++i) {
    cyc += c[2 * i];
    rt += c[2 * i + 1];
  }
  cyc /= grid;
  rt /= grid;
  const double bytes_per_read = MODE == kB128 ? 1024.0 : 512.0;   // per wave
  const double reads = (double)iters * kUnroll * waves;            // per work-group (= per CU)
  printf("%-20s waves/CU %2d  %9.0f cycles  %.2f GHz  %6.1f B/clk/CU  %.3f reads/clk/CU  %5.1f clk/read\n", name, waves,
         cyc, cyc / (rt * 10.0), reads * bytes_per_read / cyc, reads / cyc, cyc / reads);
  CHECK(hipFree(out));
  CHECK(hipFree(clocks));
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 2000;
  if (iters <= 0 || iters > 1000000) {
    fprintf(stderr, "iterations must be in 1..1000000\n");
    return 2;
  }
  hipDeviceProp_t p;
  CHECK(hipGetDeviceProperties(&p, 0));
  const int grid = p.multiProcessorCount;   // one work-group per CU
  printf("device %s, %d CUs, %d iterations of %d reads per wave\n", p.gcnArchName, grid, iters, kUnroll);
  for (int w : {4, 8, 16}) run<kB128>("ds_read_b128", w, grid, iters);
  for (int w : {4, 8, 16}) run<kB64>("ds_read_b64", w, grid, iters);
  for (int w : {4, 8, 16}) run<kTr16>("ds_read_b64_tr_b16", w, grid, iters);
  return 0;
}
