// Head layout: per-head Q/K RMS norm with gain + rotary embedding, the
// attention operands in a padded head-major layout, and fp32 tile means.
//
// TensorFold PR #949, "What it adds" (h3_routing: head layout with q/k norm
// and rotary, tile means) and "Precision" (fp32 tile means); h3.c README
// (QKV rows interleaved per attention head, consumed directly by the fused
// Q/K norm + RoPE kernel).
//
// One workgroup (4 waves) per (head, tile); heads vary fastest over the grid
// so the 40 workgroups of a tile share its rows of y and of the rotary table
// in L2.  The tile is processed 32 padded rows at a time.  A q or k row is
// D/8 lanes x 16 bytes (8 elements per lane), so a wave handles 64/(D/8) row
// vectors at once:
//   u~ = bf( rope( u * (sum u^2 / D + eps)^-1/2 * gain ) )
//   rope: (a, b) -> (a cos - b sin, b cos + a sin) on the pairs (i, i + D/2),
//   cos/sin from the caller's table; the partner element sits D/16 lanes away.
// v rows are staged in LDS and written transposed, one 32-row chunk at a
// time (v^T [nh][Rp/32][D][32]: the D x 32 block of a chunk is 8 KB of
// contiguous memory), in 16-byte runs of 8 positions; within each chunk the
// 4-row blocks are interleaved (see below).  Padded rows (beyond a tile's
// length, up to the next multiple of 32) are written as zeros.  Tile sums of
// q~, k~ and v are kept in fp32 per lane, combined across lanes and waves in
// a fixed order, and divided by the tile's true row count.
#include "common.h"
#include "internal.h"

namespace h3 {

namespace {

template <int D, int MODE>
__global__ __launch_bounds__(256) void k_heads(HeadsArgs a) {
  constexpr int LPR = D / 8;        // lanes per row vector (16 bytes each)
  constexpr int RPW = 64 / LPR;     // row vectors per wave per iteration
  constexpr int NIT = 64 / (4 * RPW);  // iterations for the 32 q + 32 k rows of a group
  constexpr int SV = D + 8;         // LDS row stride (bf16) of the v staging tile
  __shared__ __attribute__((aligned(16))) bf16_t sV[32 * SV];
  __shared__ float sSum[4][3][D];

  const int h = blockIdx.x, t = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r_beg = a.tstart[t], len = a.tstart[t + 1] - r_beg;
  const int ps = a.tpstart[t], plen = a.tpstart[t + 1] - ps;
  const int u = lane % LPR, slot = lane / LPR;  // 16-byte unit within the row, row slot
  const bool hi_half = u >= LPR / 2;            // holds elements i + D/2 of the rotary pairs

  float g8[2][8];  // q and k gains of this lane's 8 columns
  if constexpr (MODE == HEADS_QKV) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      g8[0][e] = bf2f(a.q_gain[8 * u + e]);
      g8[1][e] = bf2f(a.k_gain[8 * u + e]);
    }
  }
  float sum[3][8];  // q, k, v column sums of this lane (columns 8u .. 8u+7)
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[w][e] = 0.f;

  auto src_of = [&](int which, int row) -> const bf16_t* {
    if constexpr (MODE == HEADS_QKV)
      return a.y + (size_t)row * a.ystride + h * a.parts * D + which * D + 8 * u;
    else
      return (which == 0 ? a.q_in : which == 1 ? a.k_in : a.v_in) + ((size_t)h * a.R + row) * D +
             8 * u;
  };
  const float inv_d = 1.0f / (float)D;

  // The q / k row vectors (vector v = (it * 4 + wave) * RPW + slot, v < 32 is
  // q) and the v rows of the group of 32 rows at c0.  The next group's are
  // loaded before this group's v sums and transpose, so that their latency
  // passes under them.
  constexpr int NVL = 32 * LPR / 256;  // 16-byte units of the group's v rows per thread
  u32x4_t raw[NIT], vraw[NVL];
  auto load_rows = [&](int c0) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int v = (it * 4 + wave) * RPW + slot;
      const int rl = c0 + (v & 31);
      raw[it] = (u32x4_t){0u, 0u, 0u, 0u};
      if (rl < len) raw[it] = *reinterpret_cast<const u32x4_t*>(src_of(v >> 5, r_beg + rl));
    }
    // v: unit k2 * 256 + tid is row unit / LPR, 16-byte unit unit % LPR
#pragma unroll
    for (int k2 = 0; k2 < NVL; ++k2) {
      const int unit = k2 * 256 + tid;
      const int rl = c0 + unit / LPR, uu = unit % LPR;
      vraw[k2] = (u32x4_t){0u, 0u, 0u, 0u};
      if (rl < len) {
        if constexpr (MODE == HEADS_QKV)
          vraw[k2] = *reinterpret_cast<const u32x4_t*>(a.y + (size_t)(r_beg + rl) * a.ystride +
                                                        h * a.parts * D + 2 * D + 8 * uu);
        else
          vraw[k2] = *reinterpret_cast<const u32x4_t*>(
              a.v_in + ((size_t)h * a.R + r_beg + rl) * D + 8 * uu);
      }
    }
  };
  load_rows(0);

  for (int c0 = 0; c0 < plen; c0 += 32) {
    // ---- q / k ----
    // A lane's k row in iteration it + NIT/2 is its q row of iteration it (v + 32),
    // so the rotary cos/sin loaded for the q row serve the k row as well.
    f32x4_t rope_cs[NIT / 2][4];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int v = (it * 4 + wave) * RPW + slot;
      constexpr int kStride = 4 * RPW;             // row vectors per iteration (all waves)
      const int which = (it * kStride) >> 5;       // = v >> 5, known at compile time
      const int rl = c0 + (v & 31);
      const bool real = rl < len;
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bflo(raw[it][e]);
        x[2 * e + 1] = bfhi(raw[it][e]);
      }
      if constexpr (MODE == HEADS_QKV) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
        for (int o = 1; o < LPR; o <<= 1) ss += __shfl_xor(ss, o, kWave);
        const float rinv = rsqrtf(ss * inv_d + a.eps);
        const float* gg = g8[which];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = x[e] * rinv * gg[e];
        if (a.rope) {
          // cos/sin of pairs i = 8 (u mod LPR/2) + e of this row (loaded with the q row)
          if (which == 0) {
            const float* cs = a.rope + ((size_t)(r_beg + (real ? rl : 0)) * (D / 2) +
                                        8 * (u % (LPR / 2))) * 2;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
              rope_cs[it % (NIT / 2)][q4] = *reinterpret_cast<const f32x4_t*>(cs + 4 * q4);
          }
          const f32x4_t* c4 = rope_cs[it % (NIT / 2)];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float c = c4[e >> 1][(e & 1) * 2], sn = c4[e >> 1][(e & 1) * 2 + 1];
            const float other = __shfl_xor(x[e], LPR / 2, kWave);
            // lo lane: a = x, b = other -> a c - b s; hi lane: b = x, a = other -> b c + a s
            x[e] = hi_half ? fmaf(x[e], c, other * sn) : fmaf(x[e], c, -(other * sn));
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = bf2f(f2bf(x[e]));
      }
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (real) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[which][e] += x[e];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack2(x[2 * e], x[2 * e + 1]);
      }
      bf16_t* dst = (which == 0 ? a.q : a.k) + ((size_t)h * a.Rp + ps + rl) * D + 8 * u;
      *reinterpret_cast<u32x4_t*>(dst) = w;
    }
    // ---- v: 32 rows x LPR units, staged row-major in LDS ----
#pragma unroll
    for (int k2 = 0; k2 < NVL; ++k2) {
      const int unit = k2 * 256 + tid;
      *reinterpret_cast<u32x4_t*>(&sV[(unit / LPR) * SV + 8 * (unit % LPR)]) = vraw[k2];
    }
    if (c0 + 32 < plen) load_rows(c0 + 32);
    __syncthreads();
    // v sums: this lane's columns 8u..8u+7 over rows slot, slot + RPW, ... of the
    // wave's share (rows wave * 8 .. wave * 8 + 7)
    for (int r = wave * 8 + slot; r < wave * 8 + 8; r += RPW) {
      if (c0 + r < len) {
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(&sV[r * SV + 8 * u]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sum[2][2 * e] += bflo(w[e]);
          sum[2][2 * e + 1] += bfhi(w[e]);
        }
      }
    }
    // v^T: thread -> (dimension d, 8 positions).  Within every aligned group of
    // 32 rows the 4-row blocks are stored in the order 0, 4, 1, 5, 2, 6, 3, 7,
    // so that the 8 keys one lane feeds to the value-product MFMA (rows
    // 4g..4g+3 and 16+4g..16+4g+3 of a 32-row chunk) are 16 contiguous bytes:
    // positions 8p8 .. 8p8+7 hold rows 4p8..4p8+3 and 16+4p8..16+4p8+3.
#pragma unroll
    for (int k2 = 0; k2 < D * 4 / 256; ++k2) {
      const int idx = k2 * 256 + tid;
      const int d = idx % D, p8 = idx / D;  // p8: 8-position run 0..3 of the 32-row group
      const int r0 = 4 * p8, r1 = r0 + 16;
      u32x4_t w;
      w[0] = (uint32_t)sV[(r0 + 0) * SV + d] | ((uint32_t)sV[(r0 + 1) * SV + d] << 16);
      w[1] = (uint32_t)sV[(r0 + 2) * SV + d] | ((uint32_t)sV[(r0 + 3) * SV + d] << 16);
      w[2] = (uint32_t)sV[(r1 + 0) * SV + d] | ((uint32_t)sV[(r1 + 1) * SV + d] << 16);
      w[3] = (uint32_t)sV[(r1 + 2) * SV + d] | ((uint32_t)sV[(r1 + 3) * SV + d] << 16);
      const size_t chunk = ((size_t)h * a.Rp + ps + c0) >> 5;  // ps + c0: a multiple of 32
      *reinterpret_cast<u32x4_t*>(a.vt + (chunk * D + d) * 32 + 8 * p8) = w;
    }
    __syncthreads();
  }

  // ---- tile means: lanes with the same columns (slots), then waves, fixed order ----
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1) sum[w][e] += __shfl_xor(sum[w][e], o, kWave);
  if (slot == 0) {
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
      for (int e = 0; e < 8; ++e) sSum[wave][w][8 * u + e] = sum[w][e];
  }
  __syncthreads();
  const float inv_len = 1.0f / (float)len;
  for (int idx = tid; idx < 3 * D; idx += 256) {
    const int which = idx / D, c = idx % D;
    const float sm = ((sSum[0][which][c] + sSum[1][which][c]) + sSum[2][which][c]) + sSum[3][which][c];
    const float m = sm * inv_len;
    if (which == 0) {
      if (t >= a.npt) a.qbar[((size_t)h * (a.nT - a.npt) + (t - a.npt)) * D + c] = m;
    } else if (which == 1) {
      a.kbar[((size_t)h * a.nT + t) * D + c] = m;
    } else {
      a.vbar[((size_t)h * a.nT + t) * D + c] = m;
    }
  }
}

}  // namespace

hipError_t launch_heads(int mode, int head_dim, const HeadsArgs& a, hipStream_t s) {
  dim3 grid(a.nh, a.nT), block(256);
  if (head_dim == 128) {
    if (mode == HEADS_QKV) hipLaunchKernelGGL((k_heads<128, HEADS_QKV>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_heads<128, HEADS_SPLIT>), grid, block, 0, s, a);
  } else {
    if (mode == HEADS_QKV) hipLaunchKernelGGL((k_heads<64, HEADS_QKV>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_heads<64, HEADS_SPLIT>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace h3
