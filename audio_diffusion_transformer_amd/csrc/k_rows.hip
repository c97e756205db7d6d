// The pieces of a denoising pass around the forward: the rows in (F32 patch
// projections into the packed bf16 stream), the time embedder and the
// modulation tables, and the Euler transition of the latents.
//
// Rows in: h3.c README, implementation notes (the 96 -> 5376 video and
// 32 -> 5376 audio patch projections keep F32 weights, inputs and
// accumulation and round each result straight into the packed hidden
// stream); TensorFold PR #949, "What it adds" (the rows in).
//   x[row][c] = bf( sum_k patch[row][k] W[c][k] + b[c] )   fp32 products and sums
// One workgroup (4 waves) per 64 rows x 256 columns of one segment: 32-wide k
// slices of W and of the patches are staged in LDS (row-major, k contiguous);
// wave w computes the 64 x 64 block of columns 64w .. 64w+63 with fp32 matrix
// products (v_mfma_f32_16x16x4_f32, fp32 accumulation; lane group g feeds the
// products' k slot g with k = 4g .. 4g+3 of each 16-wide half slice, so one
// 16-byte LDS read serves four products); the sums plus bias are rounded to
// bf16, staged in LDS and written as 16-byte runs.  Text rows (the text
// encoder's output) are copied as they are.
//
// Time conditioning: TensorFold PR #949, "What comes next" (the time embedder
// and the modulation tables).  For each segment s (text, audio, video) with
// timestep sigma_s and t_s = 1000 sigma_s:
//   e_s  = [cos(t_s w_i)] ++ [sin(t_s w_i)], w_i = 10000^(-i/128), i < 128
//   h_s  = silu(W1 e_s + b1);  c_s = W2 h_s + b2
//   mod[l][s] = W_mod silu(c_s) + b_mod + table[l];  final[s] = W_final silu(c_s) + b_final
// as four matrix-vector products over the three segments at once: a
// workgroup (8 waves) stages the three input vectors (fp32) in LDS, each wave
// takes a few output rows at once (eight for the wide modulation products, two
// for the narrow ones) and reads its weight rows once with 16-byte loads (the
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

constexpr int kRiRows = 64, kRiCols = 256, kRiK = 32;

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

  constexpr int SK = kRiK + 4;  // padded row of a staged k slice (16-byte reads free of conflicts)
  constexpr int SO = kRiCols + 8;  // padded bf16 row of the output staging
  __shared__ __attribute__((aligned(16))) float sW[kRiCols * SK];  // [column][k]
  __shared__ __attribute__((aligned(16))) float sP[kRiRows * SK];  // [row][k]
  static_assert(kRiRows * SO * 2 <= kRiCols * SK * 4, "output staging fits sW");
  const int lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
  f32x4_t acc[4][4];  // blocks (row block i, column block j) of the wave's 64 x 64
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // a thread's share of a k slice: 32 W values and 8 patch values, all
  // loaded before any is stored, so that their latencies overlap
  constexpr int NW = kRiCols * kRiK / 256, NP = kRiRows * kRiK / 256;
  const int kt = tid % kRiK, ct = tid / kRiK;  // k of this thread; its first column (row)
  for (int k0 = 0; k0 < C; k0 += kRiK) {
    float wv[NW], pv[NP];
    const bool kin = k0 + kt < C;
#pragma unroll
    for (int u = 0; u < NW; ++u) {
      const int c = ct + u * (256 / kRiK);
      wv[u] = kin ? W[(size_t)(n0 + c) * C + k0 + kt] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int r = ct + u * (256 / kRiK);
      pv[u] = (kin && m0 + r < nrows) ? patch[(size_t)(m0 + r) * C + k0 + kt] : 0.f;
    }
    __syncthreads();  // every wave is done with the previous slice
#pragma unroll
    for (int u = 0; u < NW; ++u) sW[(ct + u * (256 / kRiK)) * SK + kt] = wv[u];
#pragma unroll
    for (int u = 0; u < NP; ++u) sP[(ct + u * (256 / kRiK)) * SK + kt] = pv[u];
    __syncthreads();
#pragma unroll
    for (int hk = 0; hk < kRiK; hk += 16) {  // two 16-wide halves of the slice
      const int kk = hk + 4 * g;
      f32x4_t pa[4], wb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pa[i] = *reinterpret_cast<const f32x4_t*>(&sP[(16 * i + l16) * SK + kk]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wb[j] = *reinterpret_cast<const f32x4_t*>(&sW[(64 * wave + 16 * j + l16) * SK + kk]);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[i][t], wb[j][t], acc[i][j], 0, 0, 0);
    }
  }
  // bias, bf16, staged row-major (lane: rows 16i + 4g + e, column 64 wave + 16j + l16)
  __syncthreads();  // every wave is done with the k slices
  bf16_t* const sO = reinterpret_cast<bf16_t*>(sW);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = 64 * wave + 16 * j + l16;
    const float bv = bias[n0 + col];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) sO[(16 * i + 4 * g + e) * SO + col] = f2bf(acc[i][j][e] + bv);
  }
  __syncthreads();
  for (int idx = tid; idx < kRiRows * (kRiCols / 8); idx += 256) {
    const int r = idx / (kRiCols / 8), c8 = (idx % (kRiCols / 8)) * 8;
    if (m0 + r < nrows)
      *reinterpret_cast<u32x4_t*>(a.x + (size_t)(row0 + m0 + r) * H + n0 + c8) =
          *reinterpret_cast<const u32x4_t*>(&sO[r * SO + c8]);
  }
}

// ---- time conditioning: out[s][o] = W[o] . act(in[s]) + b[o], s < 3 --------

constexpr int kTvWaves = 8;

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// One wave: RW weight rows against the three staged inputs at once (eight for
// the large products, two for the small ones so that they still give every CU
// work), so that each lane keeps RW 16-byte weight loads in flight and reads
// each staged input value once for all of its rows.  The lane takes the
// 16-byte units lane, lane + 64, ... of a row and sums them in that order; the
// 64 lane sums are then added by wave_sum.
template <int RW>
__global__ __launch_bounds__(64 * kTvWaves) void k_time_gemv(TimeGemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) float sIn[];  // [3][K], then the outputs [3][ROWS]
  constexpr int ROWS = kTvWaves * RW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K;
  if (a.in == nullptr) {
    // the frequency embedding of t_s = 1000 sigma_s (fp64 arguments, so the
    // large angles keep their accuracy): cos in [0, K/2), sin in [K/2, K)
    const int half = K / 2;
    for (int f = tid; f < half; f += 64 * kTvWaves) {
      const double om = exp(-9.210340371976184 * (double)f / (double)half);  // 10000^(-f/half)
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        double sn, cs;
        sincos(1000.0 * (double)a.sigma[s] * om, &sn, &cs);
        sIn[s * K + f] = (float)cs;
        sIn[s * K + half + f] = (float)sn;
      }
    }
  } else {
    for (int idx = 4 * tid; idx < 3 * K; idx += 4 * 64 * kTvWaves) {
      f32x4_t v = *reinterpret_cast<const f32x4_t*>(a.in + idx);
      if (a.in_silu)
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = silu_f(v[t]);
      *reinterpret_cast<f32x4_t*>(&sIn[idx]) = v;
    }
  }
  __syncthreads();
  const int ob = blockIdx.x * ROWS;            // the workgroup's first output
  const int o0 = ob + wave * RW;               // this wave's first row
  float acc[RW][3];
#pragma unroll
  for (int r = 0; r < RW; ++r) acc[r][0] = acc[r][1] = acc[r][2] = 0.f;
  // The next 8 columns' weights are loaded before the current ones are used,
  // so a load's latency passes under the previous step's products (addresses
  // clamped into the row, so every load is a valid one; rows past N: a valid
  // row, result dropped).
  const bf16_t* wrow[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) wrow[r] = a.w + (size_t)min(o0 + r, a.N - 1) * K;
  u32x4_t wv[RW];
  auto load_w = [&](u32x4_t* dst, int k8) {
    const int kc = min(k8, K - 8);
#pragma unroll
    for (int r = 0; r < RW; ++r) dst[r] = *reinterpret_cast<const u32x4_t*>(wrow[r] + kc);
  };
  load_w(wv, lane * 8);
  for (int k8 = lane * 8; k8 < K; k8 += 512) {
    u32x4_t wn[RW];
    load_w(wn, k8 + 512);
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const f32x4_t i0 = *reinterpret_cast<const f32x4_t*>(&sIn[s * K + k8]);
      const f32x4_t i1 = *reinterpret_cast<const f32x4_t*>(&sIn[s * K + k8 + 4]);
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        float v = acc[r][s];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          v = fmaf(bflo(wv[r][t]), i0[2 * t], v);
          v = fmaf(bfhi(wv[r][t]), i0[2 * t + 1], v);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          v = fmaf(bflo(wv[r][2 + t]), i1[2 * t], v);
          v = fmaf(bfhi(wv[r][2 + t]), i1[2 * t + 1], v);
        }
        acc[r][s] = v;
      }
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) wv[r] = wn[r];
  }
  // the 3 RW lane sums reduced across the wave together (each the xor tree of
  // wave_sum, in the same order), so their lane exchanges overlap
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int s = 0; s < 3; ++s) acc[r][s] += __shfl_xor(acc[r][s], o, kWave);
  __syncthreads();  // every wave is done with the staged inputs
  float* const sOut = sIn;  // [3][ROWS]
  if (lane == 0)
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
      for (int s = 0; s < 3; ++s) sOut[s * ROWS + wave * RW + r] = acc[r][s];
  __syncthreads();
  // bias, activation and the stores, one output per lane (coalesced rows of
  // ROWS outputs): out[s][o], or the modulation tables out[l][s][o] = v + table[l][o].
  // A thread's outputs all share the column j = tid % ROWS (the stride is a
  // multiple of ROWS), so it reads its bias and three sums once; the table
  // reads of a group are issued unconditionally (clamped) before its stores.
  const int nl = a.table == nullptr ? 1 : a.n_blocks;
  const int total = nl * 3 * ROWS;
  constexpr int NB = 8, STRIDE = 64 * kTvWaves;
  static_assert(STRIDE % ROWS == 0, "a thread keeps one output column");
  const int j = tid % ROWS, o = ob + j;
  const bool col_ok = o < a.N;
  const float bias = bf2f(a.b[min(o, a.N - 1)]);
  const float sv[3] = {sOut[j], sOut[ROWS + j], sOut[2 * ROWS + j]};
  auto put = [&](int idx, float tv) {
    const int ls = idx / ROWS, s = ls % 3, l = ls / 3;
    float v = sv[s] + bias;
    if (a.out_silu) v = silu_f(v);
    a.out[((size_t)l * 3 + s) * a.N + o] = v + tv;
  };
  if (a.table == nullptr) {
    for (int idx = tid; idx < total; idx += STRIDE)
      if (col_ok) put(idx, 0.f);
    return;
  }
  const bf16_t* const tcol = a.table + min(o, a.N - 1);
  for (int base = tid; base < total; base += NB * STRIDE) {
    float tv[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u)
      tv[u] = bf2f(tcol[(size_t)min((base + u * STRIDE) / (3 * ROWS), nl - 1) * a.N]);
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int idx = base + u * STRIDE;
      if (idx < total && col_ok) put(idx, tv[u]);
    }
  }
}

// ---- Euler -------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_euler(float* __restrict__ x, const float* __restrict__ v,
                                               size_t n, double dsigma) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = (float)((double)x[i] + dsigma * (double)v[i]);
}

// ---- token reduction ---------------------------------------------------------
//
// h3.c README, implementation notes (--token-reduction): after a given block
// horizontally adjacent video tokens are pooled into one, text and audio rows
// pass as they are, the full-resolution state is kept; at the restore block
// each token returns as its kept value plus its pair's update.
//   pool:    red[r] = bf((x[a] + x[b]) / 2), or x[a] for a single token; orig = x (video rows)
//   restore: out[i] = bf(orig[i] + (cur[r] - base[r])) for both tokens of pair r,
//            cur[r] for a single token; prefix rows take cur
// The sums are formed in fp64 (exact for bf16 operands) and rounded once to
// bf16 through a round-to-odd step to fp32 (exact round-to-nearest-even).
// One wave per reduced row, 16-byte vectors; pair indices outside [0, V) are
// skipped.

__device__ __forceinline__ uint32_t pack2_f64(double a, double b) {
  float ta = __double2float_rz(a), tb = __double2float_rz(b);
  if ((double)ta != a) ta = __uint_as_float(__float_as_uint(ta) | 1u);  // round to odd
  if ((double)tb != b) tb = __uint_as_float(__float_as_uint(tb) | 1u);
  return pack2(ta, tb);
}

__global__ __launch_bounds__(256) void k_token_pool(TokenArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);  // reduced-stream row
  if (r >= a.P + a.Vr) return;
  const int nv = a.H / 8;
  if (r < a.P) {  // prefix row: as it is
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.x + (size_t)r * a.H);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(a.red + (size_t)r * a.H);
    for (int c = lane; c < nv; c += 64) dst[c] = src[c];
    return;
  }
  const int ia = a.pairs[2 * (r - a.P)], ib = a.pairs[2 * (r - a.P) + 1];
  if (ia < 0 || ia >= a.V || ib >= a.V) return;
  const u32x4_t* xa = reinterpret_cast<const u32x4_t*>(a.x + (size_t)(a.P + ia) * a.H);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(a.red + (size_t)r * a.H);
  u32x4_t* oa = reinterpret_cast<u32x4_t*>(a.orig + (size_t)ia * a.H);
  if (ib < 0) {
    for (int c = lane; c < nv; c += 64) {
      const u32x4_t v = xa[c];
      dst[c] = v;
      oa[c] = v;
    }
    return;
  }
  const u32x4_t* xb = reinterpret_cast<const u32x4_t*>(a.x + (size_t)(a.P + ib) * a.H);
  u32x4_t* ob = reinterpret_cast<u32x4_t*>(a.orig + (size_t)ib * a.H);
  for (int c = lane; c < nv; c += 64) {
    const u32x4_t u = xa[c], v = xb[c];
    u32x4_t w;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      w[t] = pack2_f64(((double)bflo(u[t]) + (double)bflo(v[t])) * 0.5,
                       ((double)bfhi(u[t]) + (double)bfhi(v[t])) * 0.5);
    dst[c] = w;
    oa[c] = u;
    ob[c] = v;
  }
}

__global__ __launch_bounds__(256) void k_token_restore(TokenArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.P + a.Vr) return;
  const int nv = a.H / 8;
  const u32x4_t* cur = reinterpret_cast<const u32x4_t*>(a.cur + (size_t)r * a.H);
  if (r < a.P) {
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(a.out + (size_t)r * a.H);
    for (int c = lane; c < nv; c += 64) dst[c] = cur[c];
    return;
  }
  const int ia = a.pairs[2 * (r - a.P)], ib = a.pairs[2 * (r - a.P) + 1];
  if (ia < 0 || ia >= a.V || ib >= a.V) return;
  u32x4_t* da = reinterpret_cast<u32x4_t*>(a.out + (size_t)(a.P + ia) * a.H);
  if (ib < 0) {
    for (int c = lane; c < nv; c += 64) da[c] = cur[c];
    return;
  }
  const u32x4_t* base = reinterpret_cast<const u32x4_t*>(a.red + (size_t)r * a.H);
  const u32x4_t* oa = reinterpret_cast<const u32x4_t*>(a.orig + (size_t)ia * a.H);
  const u32x4_t* ob = reinterpret_cast<const u32x4_t*>(a.orig + (size_t)ib * a.H);
  u32x4_t* db = reinterpret_cast<u32x4_t*>(a.out + (size_t)(a.P + ib) * a.H);
  for (int c = lane; c < nv; c += 64) {
    const u32x4_t cu = cur[c], ba = base[c], u = oa[c], v = ob[c];
    u32x4_t wa, wb;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const double d0 = (double)bflo(cu[t]) - (double)bflo(ba[t]);
      const double d1 = (double)bfhi(cu[t]) - (double)bfhi(ba[t]);
      wa[t] = pack2_f64((double)bflo(u[t]) + d0, (double)bfhi(u[t]) + d1);
      wb[t] = pack2_f64((double)bflo(v[t]) + d0, (double)bfhi(v[t]) + d1);
    }
    da[c] = wa;
    db[c] = wb;
  }
}

}  // namespace

hipError_t launch_token_pool(const TokenArgs& a, hipStream_t s) {
  const int rows = a.P + a.Vr;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_token_pool, dim3((rows + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_token_restore(const TokenArgs& a, hipStream_t s) {
  const int rows = a.P + a.Vr;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_token_restore, dim3((rows + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rows_in(const RowsInArgs& a, hipStream_t s) {
  const int nmax = a.n_text > a.n_audio ? (a.n_text > a.n_video ? a.n_text : a.n_video)
                                        : (a.n_audio > a.n_video ? a.n_audio : a.n_video);
  if (nmax == 0) return hipSuccess;
  dim3 grid(a.H / kRiCols, (nmax + kRiRows - 1) / kRiRows, 3);
  hipLaunchKernelGGL(k_rows_in, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_time_gemv(const TimeGemvArgs& a, hipStream_t s) {
  // eight rows a wave from N = 8,192 on (at least 128 workgroups); below, two
  const bool big = a.N >= 8192;
  const int rows_per_wg = kTvWaves * (big ? 8 : 2);
  dim3 grid((a.N + rows_per_wg - 1) / rows_per_wg);
  const size_t lds = (size_t)3 * (a.K > rows_per_wg ? a.K : rows_per_wg) * sizeof(float);
  if (big) hipLaunchKernelGGL(k_time_gemv<8>, grid, dim3(64 * kTvWaves), lds, s, a);
  else hipLaunchKernelGGL(k_time_gemv<2>, grid, dim3(64 * kTvWaves), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_euler(float* x, const float* v, size_t n, double dsigma, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_euler, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, v, n, dsigma);
  return hipGetLastError();
}

}  // namespace h3
