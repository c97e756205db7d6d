// int8 quantization of the products' inputs (h3.c README, implementation
// notes: the int8 path quantizes activations dynamically, keeps one scale per
// weight output channel, gives the FC2 input one scale per 1,024 channels,
// and folds the QKV / MLP input quantization into the gated AdaLN kernel).
//
// Codes are symmetric: for a row (or a group of consecutive columns) with
// m = max |x| over the bf16 values,
//   code = clamp(rint(x * (127 / m)), -127, 127),  scale = m / 127
// in fp32 (IEEE division, round-half-even rint); a zero group has codes 0
// and scale 0.  The integer product of two code rows times their two scales
// is the int8 product of the block.
//
// k_modnorm_q: the modulated RMS norm of k_modnorm (same arithmetic, the
//   output rounded to bf16 first), then the row's codes: one wave per row,
//   the row held in registers, so the norm output never goes to memory (it
//   can be written as well, for diagnostics).
// k_quant_rows: codes of a bf16 matrix, per row or per group; one workgroup
//   per row, each group's values held in registers between the max and the
//   codes.  k_quant_groups: groups of at most 2,048 values, one wave each.
#include "common.h"
#include "internal.h"

namespace h3 {

namespace {

constexpr int kMaxVec = 16;  // 16-byte vectors per lane: H <= 64 * 16 * 8 = 8192

__device__ __forceinline__ uint32_t codes4(float a, float b, float c, float d, float inv) {
  auto one = [&](float v) -> uint32_t {
    const float r = fminf(fmaxf(rintf(v * inv), -127.f), 127.f);
    return (uint32_t)(uint8_t)(int8_t)(int)r;
  };
  return one(a) | (one(b) << 8) | (one(c) << 16) | (one(d) << 24);
}

__global__ __launch_bounds__(256) void k_modnorm_q(const bf16_t* __restrict__ x,
                                                   const float* __restrict__ shift,
                                                   const float* __restrict__ scale,
                                                   int seg_stride, int rows, int H, int n_text,
                                                   int n_prefix, float eps,
                                                   int8_t* __restrict__ q,
                                                   float* __restrict__ qscale,
                                                   bf16_t* __restrict__ n_out) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
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
  float m = 0.f;
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
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float a = bflo(v[i][t]) * rinv, b = bfhi(v[i][t]) * rinv;
        v[i][t] = pack2(fmaf(a, 1.0f + scv[2 * t], shv[2 * t]),
                        fmaf(b, 1.0f + scv[2 * t + 1], shv[2 * t + 1]));
        m = fmaxf(m, fmaxf(fabsf(bflo(v[i][t])), fabsf(bfhi(v[i][t]))));
      }
    }
  }
  m = wave_max(m);
  const float inv = m > 0.f ? 127.0f / m : 0.f;
  uint32_t* qr = reinterpret_cast<uint32_t*>(q + (size_t)row * H);
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int c = lane + 64 * i;
    if (c < nvec) {
      u32x2_t w;
      w[0] = codes4(bflo(v[i][0]), bfhi(v[i][0]), bflo(v[i][1]), bfhi(v[i][1]), inv);
      w[1] = codes4(bflo(v[i][2]), bfhi(v[i][2]), bflo(v[i][3]), bfhi(v[i][3]), inv);
      *reinterpret_cast<u32x2_t*>(qr + 2 * c) = w;
      if (n_out) reinterpret_cast<u32x4_t*>(n_out + (size_t)row * H)[c] = v[i];
    }
  }
  if (lane == 0) qscale[row] = m / 127.0f;
}

constexpr int kQrMax = 16;  // 16-byte vectors per thread and group: groups of <= 32768

__global__ __launch_bounds__(256) void k_quant_rows(const bf16_t* __restrict__ x, int K, int G,
                                                    int8_t* __restrict__ q,
                                                    float* __restrict__ qscale) {
  __shared__ float sMax[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  const int ng = K / G, nu = G / 8;
  for (int gi = 0; gi < ng; ++gi) {
    const bf16_t* src = x + (size_t)row * K + (size_t)gi * G;
    u32x4_t v[kQrMax];
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < kQrMax; ++j) {
      const int u = tid + 256 * j;
      if (u < nu) {
        v[j] = reinterpret_cast<const u32x4_t*>(src)[u];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          m = fmaxf(m, fmaxf(fabsf(bflo(v[j][t])), fabsf(bfhi(v[j][t]))));
      }
    }
    m = wave_max(m);
    if (lane == 0) sMax[gi & 1][wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(sMax[gi & 1][0], sMax[gi & 1][1]), fmaxf(sMax[gi & 1][2], sMax[gi & 1][3]));
    const float inv = m > 0.f ? 127.0f / m : 0.f;
    uint32_t* dst = reinterpret_cast<uint32_t*>(q + (size_t)row * K + (size_t)gi * G);
#pragma unroll
    for (int j = 0; j < kQrMax; ++j) {
      const int u = tid + 256 * j;
      if (u < nu) {
        u32x2_t w;
        w[0] = codes4(bflo(v[j][0]), bfhi(v[j][0]), bflo(v[j][1]), bfhi(v[j][1]), inv);
        w[1] = codes4(bflo(v[j][2]), bfhi(v[j][2]), bflo(v[j][3]), bfhi(v[j][3]), inv);
        *reinterpret_cast<u32x2_t*>(dst + 2 * u) = w;
      }
    }
    if (tid == 0) qscale[(size_t)row * ng + gi] = m / 127.0f;
  }
}

// one wave per (row, group) of G <= 2048 values: lanes hold G/512 16-byte vectors
template <int NV>
__global__ __launch_bounds__(256) void k_quant_groups(const bf16_t* __restrict__ x, int rows,
                                                      int K, int G, int8_t* __restrict__ q,
                                                      float* __restrict__ qscale) {
  const int lane = threadIdx.x & 63;
  const int ng = K / G;
  const long wid = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= (long)rows * ng) return;
  const int row = (int)(wid / ng), gi = (int)(wid % ng);
  const size_t base = (size_t)row * K + (size_t)gi * G;
  const int nu = G / 8;
  u32x4_t v[NV];
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int u = lane + 64 * j;
    if (u < nu) {
      v[j] = reinterpret_cast<const u32x4_t*>(x + base)[u];
#pragma unroll
      for (int t = 0; t < 4; ++t) m = fmaxf(m, fmaxf(fabsf(bflo(v[j][t])), fabsf(bfhi(v[j][t]))));
    }
  }
  m = wave_max(m);
  const float inv = m > 0.f ? 127.0f / m : 0.f;
  uint32_t* dst = reinterpret_cast<uint32_t*>(q + base);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int u = lane + 64 * j;
    if (u < nu) {
      u32x2_t w;
      w[0] = codes4(bflo(v[j][0]), bfhi(v[j][0]), bflo(v[j][1]), bfhi(v[j][1]), inv);
      w[1] = codes4(bflo(v[j][2]), bfhi(v[j][2]), bflo(v[j][3]), bfhi(v[j][3]), inv);
      *reinterpret_cast<u32x2_t*>(dst + 2 * u) = w;
    }
  }
  if (lane == 0) qscale[(size_t)row * ng + gi] = m / 127.0f;
}

}  // namespace

hipError_t launch_modnorm_q(const bf16_t* x, const float* shift, const float* scale,
                            int seg_stride, int rows, int H, int n_text, int n_prefix, float eps,
                            int8_t* q, float* qscale, bf16_t* n_out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_modnorm_q, dim3((rows + 3) / 4), dim3(256), 0, s, x, shift, scale,
                     seg_stride, rows, H, n_text, n_prefix, eps, q, qscale, n_out);
  return hipGetLastError();
}

bool quant_shape_ok(int K, int G) {
  return K >= 8 && K % 8 == 0 && G >= 8 && G % 8 == 0 && K % G == 0 && G <= 256 * 8 * kQrMax;
}

hipError_t launch_quant_rows(const bf16_t* x, int rows, int K, int G, int8_t* q, float* qscale,
                             hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (G < K && G <= 2048) {  // small groups: a wave each
    const long waves = (long)rows * (K / G);
    const dim3 grid((unsigned)((waves + 3) / 4));
    if (G <= 512) hipLaunchKernelGGL(k_quant_groups<1>, grid, dim3(256), 0, s, x, rows, K, G, q, qscale);
    else if (G <= 1024) hipLaunchKernelGGL(k_quant_groups<2>, grid, dim3(256), 0, s, x, rows, K, G, q, qscale);
    else hipLaunchKernelGGL(k_quant_groups<4>, grid, dim3(256), 0, s, x, rows, K, G, q, qscale);
  } else {
    hipLaunchKernelGGL(k_quant_rows, dim3(rows), dim3(256), 0, s, x, K, G, q, qscale);
  }
  return hipGetLastError();
}

}  // namespace h3
