// The pieces of a denoising pass around the forward: the rows in (F32 patch
// projections into the packed bf16 stream), the time embedder and the
// modulation tables, and the Euler transition of the latents.
//
// Rows in: h3.c README, implementation notes (the 96 -> 5376 video and
// 32 -> 5376 audio patch projections keep F32 weights, inputs and
// accumulation and round each result straight into the packed hidden
// stream); TensorFold PR #949, "What it adds" (the rows in).
//   x[row][c] = bf( sum_k patch[row][k] W[c][k] + b[c] )   fp32, k ascending
// One workgroup per 32 rows x 256 columns of one segment: 32-wide k slices
// of W (transposed) and of the patches are staged in LDS; each thread owns
// 4 rows x 8 consecutive columns and writes them as 16-byte bf16 runs.  Text
// rows (the text encoder's output) are copied as they are.
//
// Time conditioning: TensorFold PR #949, "What comes next" (the time embedder
// and the modulation tables).  For each segment s (text, audio, video) with
// timestep sigma_s and t_s = 1000 sigma_s:
//   e_s  = [cos(t_s w_i)] ++ [sin(t_s w_i)], w_i = 10000^(-i/128), i < 128
//   h_s  = silu(W1 e_s + b1);  c_s = W2 h_s + b2
//   mod[l][s] = W_mod silu(c_s) + b_mod + table[l];  final[s] = W_final silu(c_s) + b_final
// as four matrix-vector products over the three segments at once: a
// workgroup stages the three input vectors (fp32) in LDS, each wave takes 4
// output rows and reads its weight rows once with 16-byte loads (the
// products are bound by reading the bf16 weights from HBM).
//
// Euler: h3.c README (Euler transitions; video and audio on independent
// schedules, a terminal zero after the last pass):
//   latent <- latent + (sigma_to - sigma_from) vel     (fp64 arithmetic, one fp32 rounding)
#include "common.h"
#include "internal.h"

namespace h3 {

namespace {

// ---- rows in ---------------------------------------------------------------

constexpr int kRiRows = 32, kRiCols = 256, kRiK = 32;

__global__ __launch_bounds__(256) void k_rows_in(RowsInArgs a) {
  const int seg = blockIdx.z;  // 0 text, 1 audio, 2 video
  const int nrows = seg == 0 ? a.n_text : (seg == 1 ? a.n_audio : a.n_video);
  const int m0 = blockIdx.y * kRiRows, n0 = blockIdx.x * kRiCols;
  if (m0 >= nrows) return;  // uniform over the workgroup
  const int tid = threadIdx.x;
  const int row0 = seg == 0 ? 0 : (seg == 1 ? a.n_text : a.n_text + a.n_audio);
  const int H = a.H;
  if (seg == 0) {  // text rows: a 16-byte copy
    for (int idx = tid; idx < kRiRows * (kRiCols / 8); idx += 256) {
      const int r = idx / (kRiCols / 8), c8 = (idx % (kRiCols / 8)) * 8;
      if (m0 + r < nrows) {
        const size_t o = (size_t)(m0 + r) * H + n0 + c8;
        *reinterpret_cast<u32x4_t*>(a.x + o) = *reinterpret_cast<const u32x4_t*>(a.text + o);
      }
    }
    return;
  }
  const float* __restrict__ patch = seg == 1 ? a.audio : a.video;
  const float* __restrict__ W = seg == 1 ? a.w_audio : a.w_video;
  const float* __restrict__ bias = seg == 1 ? a.b_audio : a.b_video;
  const int C = seg == 1 ? a.c_audio : a.c_video;

  __shared__ __attribute__((aligned(16))) float sW[kRiK][kRiCols + 4];  // [k][column]
  __shared__ float sP[kRiRows][kRiK + 1];                               // [row][k]
  const int cg = tid & 31, rg = tid >> 5;  // columns 8 cg .. 8 cg + 7; rows rg + 8 i
  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < C; k0 += kRiK) {
    __syncthreads();
    for (int idx = tid; idx < kRiCols * kRiK; idx += 256) {
      const int c = idx / kRiK, k = idx % kRiK;
      sW[k][c] = k0 + k < C ? W[(size_t)(n0 + c) * C + k0 + k] : 0.f;
    }
    for (int idx = tid; idx < kRiRows * kRiK; idx += 256) {
      const int r = idx / kRiK, k = idx % kRiK;
      sP[r][k] = (m0 + r < nrows && k0 + k < C) ? patch[(size_t)(m0 + r) * C + k0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < kRiK; ++k) {
      const f32x4_t w0 = *reinterpret_cast<const f32x4_t*>(&sW[k][8 * cg]);
      const f32x4_t w1 = *reinterpret_cast<const f32x4_t*>(&sW[k][8 * cg + 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = sP[rg + 8 * i][k];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(p, w0[j], acc[i][j]);
          acc[i][4 + j] = fmaf(p, w1[j], acc[i][4 + j]);
        }
      }
    }
  }
  const f32x4_t b0 = *reinterpret_cast<const f32x4_t*>(bias + n0 + 8 * cg);
  const f32x4_t b1 = *reinterpret_cast<const f32x4_t*>(bias + n0 + 8 * cg + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = rg + 8 * i;
    if (m0 + r >= nrows) continue;
    u32x4_t w;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      w[t] = pack2(acc[i][2 * t] + b0[2 * t], acc[i][2 * t + 1] + b0[2 * t + 1]);
      w[2 + t] = pack2(acc[i][4 + 2 * t] + b1[2 * t], acc[i][4 + 2 * t + 1] + b1[2 * t + 1]);
    }
    *reinterpret_cast<u32x4_t*>(a.x + (size_t)(row0 + m0 + r) * H + n0 + 8 * cg) = w;
  }
}

// ---- time conditioning: out[s][o] = W[o] . act(in[s]) + b[o], s < 3 --------

constexpr int kTvRowsPerWave = 4;

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

__global__ __launch_bounds__(256) void k_time_gemv(TimeGemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) float sIn[];  // [3][K]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K;
  if (a.in == nullptr) {
    // the frequency embedding of t_s = 1000 sigma_s (fp64 arguments, so the
    // large angles keep their accuracy)
    for (int idx = tid; idx < 3 * K; idx += 256) {
      const int s = idx / K, i = idx % K, half = K / 2;
      const int f = i < half ? i : i - half;
      const double om = exp(-9.210340371976184 * (double)f / (double)half);  // 10000^(-f/half)
      const double ang = 1000.0 * (double)a.sigma[s] * om;
      sIn[idx] = (float)(i < half ? cos(ang) : sin(ang));
    }
  } else {
    for (int idx = tid; idx < 3 * K; idx += 256) {
      const float v = a.in[idx];
      sIn[idx] = a.in_silu ? silu_f(v) : v;
    }
  }
  __syncthreads();
  const int o0 = (blockIdx.x * 4 + wave) * kTvRowsPerWave;
#pragma unroll
  for (int rr = 0; rr < kTvRowsPerWave; ++rr) {
    const int o = o0 + rr;
    if (o >= a.N) break;  // uniform over the wave
    const bf16_t* wr = a.w + (size_t)o * K;
    float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f;
    for (int k8 = lane * 8; k8 < K; k8 += 512) {
      const u32x4_t wv = *reinterpret_cast<const u32x4_t*>(wr + k8);
      float wf[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        wf[2 * t] = bflo(wv[t]);
        wf[2 * t + 1] = bfhi(wv[t]);
      }
      float* accs[3] = {&acc0, &acc1, &acc2};
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        const f32x4_t i0 = *reinterpret_cast<const f32x4_t*>(&sIn[s * K + k8]);
        const f32x4_t i1 = *reinterpret_cast<const f32x4_t*>(&sIn[s * K + k8 + 4]);
        float acc = *accs[s];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc = fmaf(wf[t], i0[t], acc);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc = fmaf(wf[4 + t], i1[t], acc);
        *accs[s] = acc;
      }
    }
    acc0 = wave_sum(acc0);
    acc1 = wave_sum(acc1);
    acc2 = wave_sum(acc2);
    if (lane < 3) {
      const float b = bf2f(a.b[o]);
      float v = (lane == 0 ? acc0 : (lane == 1 ? acc1 : acc2)) + b;
      if (a.out_silu) v = silu_f(v);
      if (a.table == nullptr) {
        a.out[(size_t)lane * a.N + o] = v;
      } else {  // modulation tables: mod[l][s][o] = v + table[l][o]
        for (int l = 0; l < a.n_blocks; ++l)
          a.out[((size_t)l * 3 + lane) * a.N + o] = v + bf2f(a.table[(size_t)l * a.N + o]);
      }
    }
  }
}

// ---- Euler -------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_euler(float* __restrict__ x, const float* __restrict__ v,
                                               size_t n, double dsigma) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = (float)((double)x[i] + dsigma * (double)v[i]);
}

}  // namespace

hipError_t launch_rows_in(const RowsInArgs& a, hipStream_t s) {
  const int nmax = a.n_text > a.n_audio ? (a.n_text > a.n_video ? a.n_text : a.n_video)
                                        : (a.n_audio > a.n_video ? a.n_audio : a.n_video);
  if (nmax == 0) return hipSuccess;
  dim3 grid(a.H / kRiCols, (nmax + kRiRows - 1) / kRiRows, 3);
  hipLaunchKernelGGL(k_rows_in, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_time_gemv(const TimeGemvArgs& a, hipStream_t s) {
  const int rows_per_wg = 4 * kTvRowsPerWave;
  dim3 grid((a.N + rows_per_wg - 1) / rows_per_wg);
  hipLaunchKernelGGL(k_time_gemv, grid, dim3(256), (size_t)3 * a.K * sizeof(float), s, a);
  return hipGetLastError();
}

hipError_t launch_euler(float* x, const float* v, size_t n, double dsigma, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_euler, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, v, n, dsigma);
  return hipGetLastError();
}

}  // namespace h3
