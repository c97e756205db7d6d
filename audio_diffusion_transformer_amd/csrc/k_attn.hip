// Tile-routed attention (video rows) and dense attention (text and audio
// rows) in one kernel, on bf16 MFMA with an fp32 online softmax.
//
// TensorFold PR #949: "What it adds" (h3_attention: tile-routed attention
// with fp32 scores and an online softmax), "Precision" (softmax weights
// rounded to bf16 before the value product) and the parity notes (the audio
// rows attend densely).  A video row of query tile i attends the prefix rows,
// then the rows of the selected tiles sel[h][i] in ascending order, and gets
// the fp32 pooled branch pooled[h][i] added before the bf16 rounding; a text
// or audio row attends every row.
//
// Operands (written by the head-layout kernel): q, k [nh][Rp][D] and v^T
// [nh][D][Rp] in a padded row space where every tile starts on a multiple of
// 32 rows; a 32-row "chunk" therefore never straddles two tiles, and
// chunk_valid[c] gives its number of real rows.
//
// One workgroup (4 wave64) per (64-row query block, head).  Every wave takes
// all 64 queries and every 4th key chunk of the block's key list:
//   S^T (32 keys x 32 queries) = K (32 x D) * Q^T (D x 32)   v_mfma_f32_32x32x16_bf16
// The MFMA result holds, in lane l, query l%32 and keys 8(e/4) + 4(l/32) + e%4
// (e < 16).  That is also the B-operand layout the value product needs:
//   O^T (D x 32 queries) += V^T (D x 16 keys) * P^T (16 keys x 32 queries)
// with the 8 key slots of lane l taken as elements e = 8m..8m+7 of S^T, so
// the probabilities never leave their lanes; V^T supplies the matching keys
// as two runs of 4 consecutive keys.  Each lane thus owns one query per
// 32-query half: the running max / sum need one exchange with lane l^32.
// Scores are scaled into the log2 domain (exp2).  At the end the four waves'
// (max, sum, O) are combined in LDS in a fixed wave order.
#include "common.h"
#include "internal.h"

namespace h3 {

namespace {

constexpr int kMaxChunks = 8192;
constexpr int kMaxSelAttn = 1024;

__device__ __forceinline__ bf16x8_t pack8(const float* p) {
  u32x4_t w;
#pragma unroll
  for (int t = 0; t < 4; ++t) w[t] = pack2(p[2 * t], p[2 * t + 1]);
  return as_bf16x8(w);
}

template <int D>
__global__ __launch_bounds__(256, 1) void k_attn(AttnArgs a) {
  constexpr int NDC = D / 16;  // 16-wide d slices of the score product
  constexpr int NDB = D / 32;  // 32-row d blocks of the value product
  __shared__ int sChunk[kMaxChunks];
  __shared__ int sOff[kMaxSelAttn + 1];
  __shared__ float sM[4][64], sL[4][64], sLt[64];
  __shared__ float sO[64][D + 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Dense query blocks of every head come first (they are the long ones).
  int qbi, h;
  {
    const int id = blockIdx.x, nd = a.nqb_dense * a.nh;
    if (id < nd) {
      qbi = id % a.nqb_dense;
      h = id / a.nqb_dense;
    } else {
      const int nv = a.nqb - a.nqb_dense;
      qbi = a.nqb_dense + (id - nd) % nv;
      h = (id - nd) / nv;
    }
  }
  const int4 qb = a.qblocks[qbi];
  const int tile = qb.x, prow0 = qb.y, nrows = qb.z, row0 = qb.w;
  const bool dense = tile < a.npt;

  int nchunk;
  if (dense) {
    nchunk = a.n_chunks;
  } else {
    const int vi = tile - a.npt;
    const int* sel = a.sel + ((size_t)h * a.nQ + vi) * a.nsel;
    if (tid == 0) {
      int off = a.n_prefix_chunks;
      for (int e = 0; e < a.nsel; ++e) {
        sOff[e] = off;
        const int s = sel[e];
        off += (a.tpstart[s + 1] - a.tpstart[s]) >> 5;
      }
      sOff[a.nsel] = off;
    }
    __syncthreads();
    for (int c = tid; c < a.n_prefix_chunks; c += 256) sChunk[c] = c;
    for (int e = tid; e < a.nsel; e += 256) {
      const int c0 = a.tpstart[sel[e]] >> 5;
      for (int c = sOff[e]; c < sOff[e + 1]; ++c) sChunk[c] = c0 + (c - sOff[e]);
    }
    __syncthreads();
    nchunk = sOff[a.nsel];
  }

  const size_t Rp = (size_t)a.Rp;
  const int l32 = lane & 31, g = lane >> 5;

  // Q^T fragments (B operand): query l%32 of each half, d = 16c + 8g .. +7.
  bf16x8_t qf[2][NDC];
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const int r = qh * 32 + l32;
    const bf16_t* qp = a.q + ((size_t)h * Rp + prow0 + r) * D + 8 * g;
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (r < nrows) w = *reinterpret_cast<const u32x4_t*>(qp + 16 * c);
      qf[qh][c] = as_bf16x8(w);
    }
  }

  const float sl2 = rsqrtf((float)D) * 1.4426950408889634f;  // d^-1/2 * log2(e)
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  f32x16_t o[NDB][2];
#pragma unroll
  for (int b = 0; b < NDB; ++b)
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[b][qh][e] = 0.f;

  const bf16_t* kbase = a.k + ((size_t)h * Rp + l32) * D + 8 * g;
  const bf16_t* vbase = a.vt + ((size_t)h * D + l32) * Rp + 4 * g;

  for (int ci = wave; ci < nchunk; ci += 4) {
    const int chunk = dense ? ci : sChunk[ci];
    const int krow0 = chunk * 32;
    const int valid = a.chunk_valid[chunk];

    // K fragments (A operand): key l%32 of the chunk, d = 16c + 8g .. +7.
    bf16x8_t kf[NDC];
#pragma unroll
    for (int c = 0; c < NDC; ++c)
      kf[c] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(kbase + (size_t)krow0 * D + 16 * c));
    // V^T fragments (A operand): d row 32b + l%32, keys 16mm + 4g + {0..3, 8..11}.
    bf16x8_t vf[NDB][2];
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const bf16_t* vp = vbase + (size_t)b * 32 * Rp + krow0 + 16 * mm;
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vp);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vp + 8);
        u32x4_t w = {lo[0], lo[1], hi[0], hi[1]};
        vf[b][mm] = as_bf16x8(w);
      }

#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      f32x16_t st;
#pragma unroll
      for (int e = 0; e < 16; ++e) st[e] = 0.f;
#pragma unroll
      for (int c = 0; c < NDC; ++c)
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c], qf[qh][c], st, 0, 0, 0);

      float p[16];
      float mloc = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = 8 * (e >> 2) + 4 * g + (e & 3);
        const float s = key < valid ? st[e] * sl2 : -INFINITY;
        p[e] = s;
        mloc = fmaxf(mloc, s);
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
      const float m_new = fmaxf(m[qh], mloc);
      const float alpha = exp2f(m[qh] - m_new);
      float lsum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = exp2f(p[e] - m_new);
        lsum += p[e];
      }
      lsum += __shfl_xor(lsum, 32, kWave);
      l[qh] = l[qh] * alpha + lsum;
      m[qh] = m_new;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int b = 0; b < NDB; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[b][qh][e] *= alpha;
      }
      const bf16x8_t p0 = pack8(p), p1 = pack8(p + 8);
#pragma unroll
      for (int b = 0; b < NDB; ++b) {
        o[b][qh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[b][0], p0, o[b][qh], 0, 0, 0);
        o[b][qh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[b][1], p1, o[b][qh], 0, 0, 0);
      }
    }
  }

  // ---- combine the four waves: fixed order 0, 1, 2, 3 ----
  if (lane < 32) {
    sM[wave][lane] = m[0];
    sM[wave][32 + lane] = m[1];
    sL[wave][lane] = l[0];
    sL[wave][32 + lane] = l[1];
  }
  __syncthreads();
  float f[2];
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const int q = qh * 32 + l32;
    const float M = fmaxf(fmaxf(sM[0][q], sM[1][q]), fmaxf(sM[2][q], sM[3][q]));
    f[qh] = m[qh] == -INFINITY ? 0.f : exp2f(m[qh] - M);
    if (wave == 0 && g == 0) {
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        L += sM[w][q] == -INFINITY ? 0.f : sL[w][q] * exp2f(sM[w][q] - M);
      sLt[q] = L;
    }
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int qh = 0; qh < 2; ++qh)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int d = 32 * b + 8 * (e >> 2) + 4 * g + (e & 3);
            const int q = qh * 32 + l32;
            const float val = o[b][qh][e] * f[qh];
            sO[q][d] = (w == 0) ? val : sO[q][d] + val;
          }
    }
    __syncthreads();
  }

  // ---- normalise, add the pooled branch, round, store row-major ----
  const float* pooled = (!dense && a.pooled)
                            ? a.pooled + ((size_t)h * a.nQ + (tile - a.npt)) * D
                            : nullptr;
  for (int idx = tid; idx < 64 * (D / 8); idx += 256) {
    const int q = idx / (D / 8), d8 = (idx % (D / 8)) * 8;
    if (q >= nrows) continue;
    const float inv = 1.0f / sLt[q];
    u32x4_t w;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float x0 = sO[q][d8 + 2 * t] * inv, x1 = sO[q][d8 + 2 * t + 1] * inv;
      if (pooled) {
        x0 += pooled[d8 + 2 * t];
        x1 += pooled[d8 + 2 * t + 1];
      }
      w[t] = pack2(x0, x1);
    }
    *reinterpret_cast<u32x4_t*>(a.out + (size_t)(row0 + q) * a.H + h * D + d8) = w;
  }
}

}  // namespace

bool attn_shape_ok(int n_chunks, int nsel) { return n_chunks <= kMaxChunks && nsel <= kMaxSelAttn; }

hipError_t launch_attn(int head_dim, const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.nqb * a.nh), block(256);
  if (head_dim == 128) hipLaunchKernelGGL(k_attn<128>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(k_attn<64>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace h3
