// Modulated RMS norm (AdaLN) and the narrow output heads.
//
// Norm: h3.c README (fused gated AdaLN: one row kept on chip, per-row RMS,
// rounded bf16 output) and TensorFold PR #949, "What it adds" (modulated
// norm, final norm, rows out).  The row is read once with 16-byte loads held
// in registers, the fp32 sum of squares is reduced across the workgroup, and
// the output is written once: 2 x H x 2 bytes of HBM traffic per row.
//
//   out[r][c] = bf( x[r][c] * (sum_c x[r][c]^2 / H + eps)^-1/2 * (1 + scale[seg][c]) + shift[seg][c] )
#include "common.h"
#include "internal.h"

namespace h3 {

namespace {

// Column-split form: a workgroup of ceil(H / 512) waves takes a run of
// consecutive rows; wave w owns columns 512 w .. 512 w + 511 (8 a lane) and
// keeps their shift and scale (fp32) in registers for all of its rows,
// reloading them only where a segment ends inside the run, so the parameters
// are read once per workgroup instead of once per row.  Rows go kMnBatch at
// a time: a lane's sum of squares of its 8 values (column order), the wave's
// xor tree, then the waves' partial sums added in wave order through LDS.
constexpr int kMnBatch = 4;   // rows per batch (8 held twice the registers: 4 waves per SIMD)
constexpr int kMnRows = 32;  // rows per workgroup

__global__ __launch_bounds__(1024) void k_modnorm_cols(const bf16_t* __restrict__ x,
                                                       bf16_t* __restrict__ out, int out_row0,
                                                       const float* __restrict__ shift,
                                                       const float* __restrict__ scale,
                                                       int seg_stride, int row0, int row1, int H,
                                                       int n_text, int n_prefix, float eps,
                                                       int rows_per_wg) {
  __shared__ float part[2][kMnBatch][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int c8 = 512 * wave + 8 * lane;  // this lane's first column
  const bool cok = c8 < H;
  const int rb = row0 + blockIdx.x * rows_per_wg;
  if (rb >= row1) return;  // uniform over the workgroup
  const int re = min(rb + rows_per_wg, row1);
  float shv[8], scv[8];
  int cur = -1;
  auto params = [&](int seg) {
    const float* sh = shift + (size_t)seg * seg_stride + c8;
    const float* sc = scale + (size_t)seg * seg_stride + c8;
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, k0 = s0, k1 = s0;
    if (cok) {
      s0 = *reinterpret_cast<const f32x4_t*>(sh);
      s1 = *reinterpret_cast<const f32x4_t*>(sh + 4);
      k0 = *reinterpret_cast<const f32x4_t*>(sc);
      k1 = *reinterpret_cast<const f32x4_t*>(sc + 4);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      shv[e] = s0[e];
      shv[4 + e] = s1[e];
      scv[e] = k0[e];
      scv[4 + e] = k1[e];
    }
  };
  int buf = 0;
  for (int r = rb; r < re; r += kMnBatch, buf ^= 1) {
    u32x4_t v[kMnBatch];
    float ss[kMnBatch];
#pragma unroll
    for (int k = 0; k < kMnBatch; ++k) {
      v[k] = (u32x4_t){0u, 0u, 0u, 0u};
      if (r + k < re && cok) v[k] = *reinterpret_cast<const u32x4_t*>(x + (size_t)(r + k) * H + c8);
    }
#pragma unroll
    for (int k = 0; k < kMnBatch; ++k) {
      float q = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float a = bflo(v[k][t]), b = bfhi(v[k][t]);
        q = fmaf(a, a, q);
        q = fmaf(b, b, q);
      }
      ss[k] = q;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
      for (int k = 0; k < kMnBatch; ++k) ss[k] += __shfl_xor(ss[k], o, kWave);
    if (lane == 0)
#pragma unroll
      for (int k = 0; k < kMnBatch; ++k) part[buf][k][wave] = ss[k];
    __syncthreads();  // (two buffers: the next batch's partial sums go to the other one)
#pragma unroll
    for (int k = 0; k < kMnBatch; ++k) {
      const int row = r + k;
      if (row >= re) break;
      float tot = 0.f;
      for (int q = 0; q < nw; ++q) tot += part[buf][k][q];
      const float rinv = rsqrtf(tot / (float)H + eps);
      const int seg = row < n_text ? 0 : (row < n_prefix ? 1 : 2);
      if (seg != cur) {
        params(seg);
        cur = seg;
      }
      if (!cok) continue;
      u32x4_t o;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float a = bflo(v[k][t]) * rinv, b = bfhi(v[k][t]) * rinv;
        o[t] = pack2(fmaf(a, 1.0f + scv[2 * t], shv[2 * t]),
                     fmaf(b, 1.0f + scv[2 * t + 1], shv[2 * t + 1]));
      }
      *reinterpret_cast<u32x4_t*>(out + (size_t)(row - out_row0) * H + c8) = o;
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
  if (H % 8 != 0 || H > 8192) return hipErrorInvalidValue;  // at most 16 waves of 512 columns
  const int nw = (H + 511) / 512;
  hipLaunchKernelGGL(k_modnorm_cols, dim3((n + kMnRows - 1) / kMnRows), dim3(64 * nw), 0, s, x,
                     out, out_row0, shift, scale, seg_stride, row0, row1, H, n_text, n_prefix, eps,
                     kMnRows);
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
