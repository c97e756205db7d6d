// bf16 GEMM with fused epilogues for gfx950:  C[M][N] = A[M][K] * B[N][K]^T.
//
// These are the block's four products (TensorFold PR #949, "What it adds":
// q/k/v products, out projection, MLP in / out; "Precision": bf16 operands,
// fp32 sums).  Both operands are K-contiguous ([row][K] activations, [out][in]
// weights), which is exactly the per-lane operand order of the CDNA4 MFMA:
// v_mfma_f32_32x32x16_bf16 takes 8 consecutive K elements of one A row and of
// one B row per lane.
//
// Tiling: a 256-thread workgroup (4 wave64) owns a 256x256 C tile; each wave
// owns a 128x128 quadrant as 4x4 MFMA blocks of 32x32 (256 fp32 accumulators
// per lane).  K advances 64 at a time through two LDS stages (rows padded to
// 72 bf16 = 144 B so the 16-byte fragment reads of 8 consecutive rows hit
// distinct banks); the next stage's global loads are issued before the MFMAs
// of the current one.  Workgroup ids are remapped so that each XCD (ids are
// dealt round-robin over the 8 XCDs) works on a contiguous band of tiles, and
// within a band tiles are walked in groups of 8 tile-rows for L2 reuse.
//
// Epilogues (rounding points of the block, h3.c README on rounded bf16
// residuals):
//   EPI_BIAS:         C = bf(acc + bias)
//   EPI_BIAS_GELU:    C = bf(gelu(acc + bias)),  gelu(z) = z/2 (1 + erf(z/sqrt2))
//   EPI_BIAS_RESGATE: C = bf(res + gate[seg(row)] * bf(acc + bias))
#include "common.h"
#include "internal.h"

namespace h3 {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per LDS row

__device__ __forceinline__ int seg_of(int row, int n_text, int n_prefix) {
  return row < n_text ? 0 : (row < n_prefix ? 1 : 2);
}

__device__ __forceinline__ void gload8(u32x4_t (&ra)[8], u32x4_t (&rb)[8], const bf16_t* A,
                                       const bf16_t* B, const int (&oa)[8], const int (&ob)[8],
                                       int k0) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ra[i] = *reinterpret_cast<const u32x4_t*>(A + oa[i] + k0);
    rb[i] = *reinterpret_cast<const u32x4_t*>(B + ob[i] + k0);
  }
}

__device__ __forceinline__ void lstore8(bf16_t* sa, bf16_t* sb, const u32x4_t (&ra)[8],
                                        const u32x4_t (&rb)[8], int lrow, int lseg) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    *reinterpret_cast<u32x4_t*>(&sa[(lrow + 32 * i) * LDS_STRIDE + lseg * 8]) = ra[i];
    *reinterpret_cast<u32x4_t*>(&sb[(lrow + 32 * i) * LDS_STRIDE + lseg * 8]) = rb[i];
  }
}

template <int EPI>
__global__ __launch_bounds__(256, 1) void k_gemm_bf16(const bf16_t* __restrict__ A,
                                                      const bf16_t* __restrict__ B, int M,
                                                      int N, int K, GemmEpi ep) {
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * LDS_STRIDE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = N / BN;

  // XCD-aware id: XCD x receives ids x, x+8, ...; give it a contiguous range.
  const int nb = gridDim.x, bid = blockIdx.x;
  const int q8 = nb >> 3, r8 = nb & 7, xcd = bid & 7, idx = bid >> 3;
  const int lin = (xcd < r8) ? xcd * (q8 + 1) + idx : r8 * (q8 + 1) + (xcd - r8) * q8 + idx;
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int g = lin / per_group;
  const int first_m = g * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (lin % per_group) % gsize;
  const int tn = (lin % per_group) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

  // Global -> LDS copy: thread t moves rows t/8 + 32 i (i < 8), 16 bytes at
  // column (t % 8) * 8 of the current 64-wide K slab, for A and for B.
  const int lrow = tid >> 3, lseg = tid & 7;
  int oa[8], ob[8];  // element offsets (M*K and N*K stay below 2^31)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ra = min(m0 + lrow + 32 * i, M - 1);  // ragged M: clamp, result rows dropped
    oa[i] = ra * K + lseg * 8;
    ob[i] = (n0 + lrow + 32 * i) * K + lseg * 8;
  }
  const int wm = wave >> 1, wn = wave & 1;
  const int frow = lane & 31, fk = (lane >> 5) * 8;

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int KT = K / BK;
  {
    u32x4_t ra[8], rb[8];
    gload8(ra, rb, A, B, oa, ob, 0);
    lstore8(sA[0], sB[0], ra, rb, lrow, lseg);
  }
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < KT;
    u32x4_t ra[8], rb[8];
    if (more) gload8(ra, rb, A, B, oa, ob, (kt + 1) * BK);
    const bf16_t* a_base = &sA[buf][(wm * 128 + frow) * LDS_STRIDE + fk];
    const bf16_t* b_base = &sB[buf][(wn * 128 + frow) * LDS_STRIDE + fk];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(a_base + i * 32 * LDS_STRIDE + kk * 16));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(b_base + j * 32 * LDS_STRIDE + kk * 16));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) lstore8(sA[buf ^ 1], sB[buf ^ 1], ra, rb, lrow, lseg);
    __syncthreads();
  }

  // Epilogue.  Accumulator element e of block (i, j) in lane l sits at
  // row 8(e/4) + 4(l/32) + e%4, column l%32 of that 32x32 block.
  const int col_l = lane & 31, row_l = (lane >> 5) * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = n0 + wn * 128 + j * 32 + col_l;
    const float bias = bf2f(ep.bias[col]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + row_l + (e & 3);
        if (row >= M) continue;
        const float v = acc[i][j][e] + bias;
        const size_t o = (size_t)row * N + col;
        if constexpr (EPI == EPI_BIAS) {
          ep.out[o] = f2bf(v);
        } else if constexpr (EPI == EPI_BIAS_GELU) {
          ep.out[o] = f2bf(0.5f * v * (1.0f + erff(v * 0.70710678118654752f)));
        } else {
          const float ob = bf2f(f2bf(v));
          const int sg = seg_of(row, ep.n_text, ep.n_prefix);
          const float gv = ep.gate[(size_t)sg * ep.gate_seg_stride + col];
          ep.out[o] = f2bf(fmaf(gv, ob, bf2f(ep.res[o])));
        }
      }
    }
  }
}

}  // namespace

bool gemm_shape_ok(int M, int N, int K) {
  return M >= 1 && N >= BN && N % BN == 0 && K >= BK && K % BK == 0;
}

hipError_t launch_gemm(int epi, const bf16_t* A, const bf16_t* B, int M, int N, int K,
                       const GemmEpi& ep, hipStream_t s) {
  const int tiles = ((M + BM - 1) / BM) * (N / BN);
  dim3 grid(tiles), block(256);
  switch (epi) {
    case EPI_BIAS:
      hipLaunchKernelGGL(k_gemm_bf16<EPI_BIAS>, grid, block, 0, s, A, B, M, N, K, ep);
      break;
    case EPI_BIAS_GELU:
      hipLaunchKernelGGL(k_gemm_bf16<EPI_BIAS_GELU>, grid, block, 0, s, A, B, M, N, K, ep);
      break;
    default:
      hipLaunchKernelGGL(k_gemm_bf16<EPI_BIAS_RESGATE>, grid, block, 0, s, A, B, M, N, K, ep);
      break;
  }
  return hipGetLastError();
}

}  // namespace h3
