// Modulated RMS norm (AdaLN) and the narrow output heads.
//
// Norm: h3.c README (fused gated AdaLN: one row kept on chip, per-row RMS,
// rounded bf16 output) and TensorFold PR #949, "What it adds" (modulated
// norm, final norm, rows out).  The row is read once with 16-byte loads held
// in registers, the fp32 sum of squares is reduced across the wave, and the
// output is written once: 2 x H x 2 bytes of HBM traffic per row.
//
//   out[r][c] = bf( x[r][c] * (sum_c x[r][c]^2 / H + eps)^-1/2 * (1 + scale[seg][c]) + shift[seg][c] )
#include "common.h"
#include "internal.h"

namespace h3 {

namespace {

constexpr int kMaxVec = 16;  // 8 bf16 per vector, so H <= 64 lanes * 16 * 8 = 8192

__global__ __launch_bounds__(256) void k_modnorm(const bf16_t* __restrict__ x,
                                                 bf16_t* __restrict__ out, int out_row0,
                                                 const float* __restrict__ shift,
                                                 const float* __restrict__ scale,
                                                 int seg_stride, int row0, int row1, int H,
                                                 int n_text, int n_prefix, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = row0 + blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= row1) return;
  const int nvec = H >> 3;
  const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(x + (size_t)row * H);
  u32x4_t v[kMaxVec];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int c = lane + 64 * i;
    if (c < nvec) {
      v[i] = xr[c];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float a = bflo(v[i][t]), b = bfhi(v[i][t]);
        ss = fmaf(a, a, ss);
        ss = fmaf(b, b, ss);
      }
    }
  }
  ss = wave_sum(ss);
  const float rinv = rsqrtf(ss / (float)H + eps);
  const int sg = row < n_text ? 0 : (row < n_prefix ? 1 : 2);
  const float* sh = shift + (size_t)sg * seg_stride;
  const float* sc = scale + (size_t)sg * seg_stride;
  u32x4_t* orow = reinterpret_cast<u32x4_t*>(out + (size_t)(row - out_row0) * H);
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int c = lane + 64 * i;
    if (c < nvec) {
      const f32x4_t s0 = *reinterpret_cast<const f32x4_t*>(sh + 8 * c);
      const f32x4_t s1 = *reinterpret_cast<const f32x4_t*>(sh + 8 * c + 4);
      const f32x4_t k0 = *reinterpret_cast<const f32x4_t*>(sc + 8 * c);
      const f32x4_t k1 = *reinterpret_cast<const f32x4_t*>(sc + 8 * c + 4);
      const float shv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
      const float scv[8] = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
      u32x4_t o;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float a = bflo(v[i][t]) * rinv, b = bfhi(v[i][t]) * rinv;
        o[t] = pack2(fmaf(a, 1.0f + scv[2 * t], shv[2 * t]),
                     fmaf(b, 1.0f + scv[2 * t + 1], shv[2 * t + 1]));
      }
      orow[c] = o;
    }
  }
}

// vel[r][c] = sum_k z[r][k] * w[c][k] + b[c], fp32 with no rounding (h3.c
// README: bf16 heads, F32 rows).  One wave per (row, group of 4 outputs): the
// lanes split k, products are summed in fp32 and reduced across the wave.
__global__ __launch_bounds__(256) void k_out_head(const bf16_t* __restrict__ z, int rows, int H,
                                                  const bf16_t* __restrict__ w,
                                                  const bf16_t* __restrict__ b, int C,
                                                  float* __restrict__ vel) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int cg = (C + 3) >> 2;
  const int row = gw / cg, c0 = (gw % cg) * 4;
  if (row >= rows) return;
  const u32x4_t* zr = reinterpret_cast<const u32x4_t*>(z + (size_t)row * H);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int kv = lane; kv < (H >> 3); kv += 64) {
    const u32x4_t zv = zr[kv];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = min(c0 + j, C - 1);
      const u32x4_t wv = reinterpret_cast<const u32x4_t*>(w + (size_t)c * H)[kv];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc[j] = fmaf(bflo(zv[t]), bflo(wv[t]), acc[j]);
        acc[j] = fmaf(bfhi(zv[t]), bfhi(wv[t]), acc[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float s = wave_sum(acc[j]);
    if (lane == 0 && c0 + j < C) vel[(size_t)row * C + c0 + j] = s + bf2f(b[c0 + j]);
  }
}

struct PokePayload {
  int v[480];
};

__global__ void k_poke(int* __restrict__ dst, int n, PokePayload p) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = p.v[i];
}

}  // namespace

hipError_t launch_modnorm(const bf16_t* x, bf16_t* out, int out_row0, const float* shift,
                          const float* scale, int seg_stride, int row0, int row1, int H,
                          int n_text, int n_prefix, float eps, hipStream_t s) {
  const int n = row1 - row0;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_modnorm, dim3((n + 3) / 4), dim3(256), 0, s, x, out, out_row0, shift,
                     scale, seg_stride, row0, row1, H, n_text, n_prefix, eps);
  return hipGetLastError();
}

hipError_t launch_out_head(const bf16_t* z, int rows, int H, const bf16_t* w, const bf16_t* b,
                           int C, float* vel, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const long waves = (long)rows * ((C + 3) / 4);
  hipLaunchKernelGGL(k_out_head, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, z, rows, H,
                     w, b, C, vel);
  return hipGetLastError();
}

hipError_t launch_poke(int* dst, const int* src, int n, hipStream_t s) {
  for (int off = 0; off < n; off += 480) {
    PokePayload p;
    const int m = n - off < 480 ? n - off : 480;
    for (int i = 0; i < m; ++i) p.v[i] = src[off + i];
    hipLaunchKernelGGL(k_poke, dim3(1), dim3(256), 0, s, dst + off, m, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace h3
