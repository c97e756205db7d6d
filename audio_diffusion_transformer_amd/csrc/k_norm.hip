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

// One wave per RW consecutive rows: each lane holds its NV 16-byte vectors
// (columns 8c .. 8c+7, c = lane + 64 i) of every row in registers, so the
// row is read once; the fp32 shift and scale of a column (64 bytes per 16
// bytes of x) are read once for all RW rows, which share their segment except
// where a segment ends inside the group (then a row reads its own).  Per
// element the arithmetic is that of one row at a time: the lane's sum of
// squares in column order, the wave sum, then the modulated value.  Two rows
// per wave: 4 rows (half the occupancy) and the parameters staged in LDS per
// workgroup (a 40 KB load before the first row) were both slower.
template <int NV, int RW>
__global__ __launch_bounds__(256) void k_modnorm(const bf16_t* __restrict__ x,
                                                 bf16_t* __restrict__ out, int out_row0,
                                                 const float* __restrict__ shift,
                                                 const float* __restrict__ scale,
                                                 int seg_stride, int row0, int row1, int H,
                                                 int n_text, int n_prefix, float eps) {
  const int lane = threadIdx.x & 63;
  const int rbase = row0 + (blockIdx.x * 4 + (threadIdx.x >> 6)) * RW;
  if (rbase >= row1) return;
  const int nvec = H >> 3;
  u32x4_t v[RW][NV];
  float rinv[RW];
  int sg[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int row = rbase + r;
    float ss = 0.f;
    if (row < row1) {
      const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(x + (size_t)row * H);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c = lane + 64 * i;
        if (c < nvec) {
          v[r][i] = xr[c];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float a = bflo(v[r][i][t]), b = bfhi(v[r][i][t]);
            ss = fmaf(a, a, ss);
            ss = fmaf(b, b, ss);
          }
        }
      }
    }
    ss = wave_sum(ss);
    rinv[r] = rsqrtf(ss / (float)H + eps);
    sg[r] = row < n_text ? 0 : (row < n_prefix ? 1 : 2);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c >= nvec) continue;
    float shv[8], scv[8];
    auto params = [&](int seg) {
      const float* sh = shift + (size_t)seg * seg_stride + 8 * c;
      const float* sc = scale + (size_t)seg * seg_stride + 8 * c;
      const f32x4_t s0 = *reinterpret_cast<const f32x4_t*>(sh);
      const f32x4_t s1 = *reinterpret_cast<const f32x4_t*>(sh + 4);
      const f32x4_t k0 = *reinterpret_cast<const f32x4_t*>(sc);
      const f32x4_t k1 = *reinterpret_cast<const f32x4_t*>(sc + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        shv[e] = s0[e];
        shv[4 + e] = s1[e];
        scv[e] = k0[e];
        scv[4 + e] = k1[e];
      }
    };
    params(sg[0]);
    int cur = sg[0];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int row = rbase + r;
      if (row >= row1) break;
      if (sg[r] != cur) {  // a segment ends inside this wave's rows
        params(sg[r]);
        cur = sg[r];
      }
      u32x4_t o;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float a = bflo(v[r][i][t]) * rinv[r], b = bfhi(v[r][i][t]) * rinv[r];
        o[t] = pack2(fmaf(a, 1.0f + scv[2 * t], shv[2 * t]),
                     fmaf(b, 1.0f + scv[2 * t + 1], shv[2 * t + 1]));
      }
      reinterpret_cast<u32x4_t*>(out + (size_t)(row - out_row0) * H)[c] = o;
    }
  }
}

// vel[r][c] = sum_k z[r][k] * w[c][k] + b[c], fp32 with no rounding (h3.c
// README: bf16 heads, F32 rows), on the matrix cores: a workgroup takes 32
// rows and all C outputs (CB blocks of 16, the last clamped); its 4 waves
// split k into quarters, each summing its quarter with
// v_mfma_f32_16x16x32_bf16 (fp32 sums), and the 4 partial sums of an output
// are added in wave order through LDS before the bias.  z and w are read with
// 16-byte loads straight into the operand registers (w, at most 256 rows, is
// served from the caches).
template <int CB>
__global__ __launch_bounds__(256) void k_out_head(const bf16_t* __restrict__ z, int rows, int H,
                                                  const bf16_t* __restrict__ w,
                                                  const bf16_t* __restrict__ b, int C,
                                                  float* __restrict__ vel) {
  extern __shared__ __attribute__((aligned(16))) float sPart[];  // [4][32][CB * 16]
  constexpr int NC = CB * 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, q4 = lane >> 4;
  const int r0 = blockIdx.x * 32;
  const int kq = H / 4, k0 = wave * kq;  // this wave's quarter of k (a multiple of 64)
  const bf16_t* zr[2];
  const bf16_t* wr[CB];
#pragma unroll
  for (int i = 0; i < 2; ++i) zr[i] = z + (size_t)min(r0 + 16 * i + l16, rows - 1) * H + k0 + 8 * q4;
#pragma unroll
  for (int j = 0; j < CB; ++j) wr[j] = w + (size_t)min(16 * j + l16, C - 1) * H + k0 + 8 * q4;
  // lane l of block (i, j): z row 16 i + 4 (l / 16) + e, output 16 j + l % 16
  f32x4_t acc[2][CB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int ks = 0; ks < kq; ks += 32) {
    u32x4_t a[2], bw[CB];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = *reinterpret_cast<const u32x4_t*>(zr[i] + ks);
#pragma unroll
    for (int j = 0; j < CB; ++j) bw[j] = *reinterpret_cast<const u32x4_t*>(wr[j] + ks);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[i]), as_bf16x8(bw[j]),
                                                            acc[i][j], 0, 0, 0);
  }
  float* const mine = sPart + wave * 32 * NC;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) mine[(16 * i + 4 * q4 + e) * NC + 16 * j + l16] = acc[i][j][e];
  __syncthreads();
  for (int idx = tid; idx < 32 * C; idx += 256) {
    const int r = idx / C, c = idx % C;
    if (r0 + r >= rows) break;  // idx grows with r
    float s = sPart[r * NC + c];
#pragma unroll
    for (int q = 1; q < 4; ++q) s += sPart[q * 32 * NC + r * NC + c];
    vel[(size_t)(r0 + r) * C + c] = s + bf2f(b[c]);
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
  // vectors per lane: the row's H / 8 16-byte vectors over 64 lanes (H <= 8192)
  const int nv = (H / 8 + 63) / 64;
  auto go = [&](auto kern, int rw) {
    const int waves = (n + rw - 1) / rw;
    hipLaunchKernelGGL(kern, dim3((waves + 3) / 4), dim3(256), 0, s, x, out, out_row0, shift,
                       scale, seg_stride, row0, row1, H, n_text, n_prefix, eps);
  };
  if (nv <= 2) go(k_modnorm<2, 2>, 2);
  else if (nv <= 4) go(k_modnorm<4, 2>, 2);
  else if (nv <= 8) go(k_modnorm<8, 2>, 2);
  else if (nv <= 11) go(k_modnorm<11, 2>, 2);
  else go(k_modnorm<16, 2>, 2);
  return hipGetLastError();
}

hipError_t launch_out_head(const bf16_t* z, int rows, int H, const bf16_t* w, const bf16_t* b,
                           int C, float* vel, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (C < 1 || C > 256 || H % 256 != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((rows + 31) / 32)), block(256);
  auto go = [&](auto kern, int cb) {
    hipLaunchKernelGGL(kern, grid, block, (size_t)4 * 32 * cb * 16 * sizeof(float), s, z, rows,
                       H, w, b, C, vel);
  };
  const int cb = (C + 15) / 16;
  if (cb <= 2) go(k_out_head<2>, 2);
  else if (cb <= 4) go(k_out_head<4>, 4);
  else if (cb <= 6) go(k_out_head<6>, 6);
  else if (cb <= 8) go(k_out_head<8>, 8);
  else if (cb <= 12) go(k_out_head<12>, 12);
  else go(k_out_head<16>, 16);
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
