// Head layout: per-head Q/K RMS norm with gain + rotary embedding, the
// attention operands in a padded head-major layout, and fp32 tile means.
//
// TensorFold PR #949, "What it adds" (h3_routing: head layout with q/k norm
// and rotary, tile means) and "Precision" (fp32 tile means); h3.c README
// (QKV rows interleaved per attention head, consumed directly by the fused
// Q/K norm + RoPE kernel).
//
// One workgroup per (tile, head).  The tile's rows are processed 32 padded
// rows at a time (4 waves x 8 rows).  For a row, lanes 0-31 handle q and
// lanes 32-63 handle k; each lane owns D/64 rotary pairs (i, i + D/2):
//   u~ = bf( rope( u * (sum u^2 / D + eps)^-1/2 * gain ) )
//   rope: (a, b) -> (a cos - b sin, b cos + a sin),  cos/sin from the caller's table
// v is copied unchanged and written transposed (v^T [nh][D][Rp]) through LDS, so
// that the attention kernel reads runs of keys per head dimension; within each
// aligned 16-row group the middle two 4-row blocks are swapped (see below).
// Padded rows (beyond a tile's length, up to the next multiple of 32) are
// written as zeros.  Tile sums of q~, k~ and v are kept in fp32 per lane, then
// combined across the waves in a fixed order and divided by the tile's true
// row count.
#include "common.h"
#include "internal.h"

namespace h3 {

namespace {

template <int D, int MODE>
__global__ __launch_bounds__(256) void k_heads(HeadsArgs a) {
  constexpr int PPL = D / 64;       // rotary pairs per lane (32 lanes per q or k row)
  constexpr int VPL = D / 64;       // v elements per lane (64 lanes per v row)
  constexpr int SV = D + 2;         // LDS row stride (bf16) of the v staging tile
  __shared__ bf16_t sV[32 * SV];
  __shared__ float sSum[4][3][D];

  const int t = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r_beg = a.tstart[t], len = a.tstart[t + 1] - r_beg;
  const int ps = a.tpstart[t], plen = a.tpstart[t + 1] - ps;
  const int hl = lane & 31;         // lane within the q (or k) half-wave
  const bool is_k = lane >= 32;

  const float* gainp = nullptr;
  float gain[2 * PPL];
  if constexpr (MODE == HEADS_QKV) {
    const bf16_t* g = is_k ? a.k_gain : a.q_gain;
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      gain[p] = bf2f(g[PPL * hl + p]);
      gain[PPL + p] = bf2f(g[D / 2 + PPL * hl + p]);
    }
  }
  (void)gainp;

  float qk_sum[2 * PPL];
  float v_sum[VPL];
#pragma unroll
  for (int p = 0; p < 2 * PPL; ++p) qk_sum[p] = 0.f;
#pragma unroll
  for (int p = 0; p < VPL; ++p) v_sum[p] = 0.f;

  bf16_t* qk_out = is_k ? a.k : a.q;
  const float inv_d = 1.0f / (float)D;

  for (int c0 = 0; c0 < plen; c0 += 32) {
    for (int j = 0; j < 8; ++j) {
      const int rl = c0 + wave * 8 + j;       // row within the padded tile
      const bool real = rl < len;
      const int row = r_beg + rl;
      // ---- q / k ----
      float lo[PPL], hi[PPL];
      if (real) {
        const bf16_t* src;
        if constexpr (MODE == HEADS_QKV)
          src = a.y + (size_t)row * (3 * a.H) + h * 3 * D + (is_k ? D : 0);
        else
          src = (is_k ? a.k_in : a.q_in) + ((size_t)h * a.R + row) * D;
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
          lo[p] = bf2f(src[PPL * hl + p]);
          hi[p] = bf2f(src[D / 2 + PPL * hl + p]);
        }
        if constexpr (MODE == HEADS_QKV) {
          float ss = 0.f;
#pragma unroll
          for (int p = 0; p < PPL; ++p) {
            ss = fmaf(lo[p], lo[p], ss);
            ss = fmaf(hi[p], hi[p], ss);
          }
          ss = half_sum(ss);
          const float rinv = rsqrtf(ss * inv_d + a.eps);
#pragma unroll
          for (int p = 0; p < PPL; ++p) {
            const float x0 = lo[p] * rinv * gain[p];
            const float x1 = hi[p] * rinv * gain[PPL + p];
            if (a.rope) {
              const float* cs = a.rope + ((size_t)row * (D / 2) + PPL * hl + p) * 2;
              const float c = cs[0], s = cs[1];
              lo[p] = bf2f(f2bf(x0 * c - x1 * s));
              hi[p] = bf2f(f2bf(x1 * c + x0 * s));
            } else {
              lo[p] = bf2f(f2bf(x0));
              hi[p] = bf2f(f2bf(x1));
            }
          }
        }
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
          qk_sum[p] += lo[p];
          qk_sum[PPL + p] += hi[p];
        }
      } else {
#pragma unroll
        for (int p = 0; p < PPL; ++p) lo[p] = hi[p] = 0.f;
      }
      bf16_t* dst = qk_out + ((size_t)h * a.Rp + ps + rl) * D;
#pragma unroll
      for (int p = 0; p < PPL; ++p) {
        dst[PPL * hl + p] = f2bf(lo[p]);
        dst[D / 2 + PPL * hl + p] = f2bf(hi[p]);
      }
      // ---- v (all 64 lanes) ----
      const int rr = wave * 8 + j;
#pragma unroll
      for (int p = 0; p < VPL; ++p) {
        bf16_t vb = 0;
        if (real) {
          if constexpr (MODE == HEADS_QKV)
            vb = a.y[(size_t)row * (3 * a.H) + h * 3 * D + 2 * D + VPL * lane + p];
          else
            vb = a.v_in[((size_t)h * a.R + row) * D + VPL * lane + p];
          v_sum[p] += bf2f(vb);
        }
        sV[rr * SV + VPL * lane + p] = vb;
      }
    }
    __syncthreads();
    // v^T: thread -> (dimension c, 4 consecutive rows).  Within every aligned
    // group of 16 rows the 4-row blocks are stored in the order 0, 2, 1, 3, so
    // that the 8 keys one lane feeds to the value-product MFMA (rows 4g..4g+3
    // and 8+4g..8+4g+3 of a 16-row group) are 16 contiguous bytes.
    for (int idx = tid; idx < D * 8; idx += 256) {
      const int c = idx >> 3, r4 = (idx & 7) * 4;
      u32x2_t w;
      w[0] = (uint32_t)sV[(r4 + 0) * SV + c] | ((uint32_t)sV[(r4 + 1) * SV + c] << 16);
      w[1] = (uint32_t)sV[(r4 + 2) * SV + c] | ((uint32_t)sV[(r4 + 3) * SV + c] << 16);
      const int blk = (r4 >> 2) & 3;
      const int pos = (r4 & ~12) | (((blk == 1) ? 2 : (blk == 2) ? 1 : blk) << 2);
      *reinterpret_cast<u32x2_t*>(a.vt + ((size_t)h * D + c) * a.Rp + ps + c0 + pos) = w;
    }
    __syncthreads();
  }

  // ---- tile means ----
#pragma unroll
  for (int p = 0; p < PPL; ++p) {
    sSum[wave][is_k ? 1 : 0][PPL * hl + p] = qk_sum[p];
    sSum[wave][is_k ? 1 : 0][D / 2 + PPL * hl + p] = qk_sum[PPL + p];
  }
#pragma unroll
  for (int p = 0; p < VPL; ++p) sSum[wave][2][VPL * lane + p] = v_sum[p];
  __syncthreads();
  const float inv_len = 1.0f / (float)len;
  for (int idx = tid; idx < 3 * D; idx += 256) {
    const int which = idx / D, c = idx % D;
    const float s = ((sSum[0][which][c] + sSum[1][which][c]) + sSum[2][which][c]) + sSum[3][which][c];
    const float m = s * inv_len;
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
  dim3 grid(a.nT, a.nh), block(256);
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
