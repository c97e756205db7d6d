// Calibration of the matrix-core throughput the products can reach on this
// GPU (not a step of the method).  Under a sustained MFMA load the clock
// settles below the 2.4 GHz at which the published 2.5 PFLOP/s bf16 peak is
// quoted, so the products are also reported against the rate an MFMA-only
// loop reaches here.
//
// k_calib_mfma: every wave keeps 16 independent v_mfma_f32_16x16x32_bf16
// accumulators (the instruction of the products and of attention) busy for
// `iters` rounds (with 8 the loop reaches only about 70% of the rate 16
// reach: a wave needs that many independent products in flight), on operands taken from random bf16 data (random operands
// draw the power of real products; zero operands would not).  The sums are
// written only if they equal a value they cannot reach, so the work is kept
// and nothing is stored.
#include "common.h"
#include "internal.h"

namespace h3 {

namespace {

__global__ __launch_bounds__(256) void k_calib_mfma(const u32x4_t* __restrict__ src, long n_vec,
                                                    float* __restrict__ sink, int iters) {
  f32x4_t acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bf16x8_t f[8];
  const long base = ((long)blockIdx.x * 256 + threadIdx.x) * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = as_bf16x8(src[(base + i) % n_vec]);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f[i & 7], f[(i + 1) & 7], acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += (acc[i][0] + acc[i][1]) + (acc[i][2] + acc[i][3]);
  if (s == 1234.5f) sink[threadIdx.x] = s;
}

}  // namespace

hipError_t launch_calib_mfma(const void* operands, size_t bytes, int n_blocks, int iters,
                             float* sink, hipStream_t s) {
  hipLaunchKernelGGL(k_calib_mfma, dim3(n_blocks), dim3(256), 0, s,
                     static_cast<const u32x4_t*>(operands), (long)(bytes / 16), sink, iters);
  return hipGetLastError();
}

}  // namespace h3
