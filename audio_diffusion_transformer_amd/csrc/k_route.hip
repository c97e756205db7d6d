// Routing for video query tiles: tile scores, top-k key tiles and the pooled
// branch, all in fp32.
//
// TensorFold PR #949: "What it adds" (h3_routing: tile scores, top-k, pooled
// branch), "Precision" (fp32 tile means, scores, top-k and pooled branch) and
// "Kernel contract" (top-k rule: a NaN score ranks as -inf, ties go to the
// lower tile).
//
// One wave per (head, video query tile), four per workgroup.
//   S[j]   = (qbar . kbar_j) * D^-1/2          for every key tile j (fp32)
//   sel    = the top_k video tiles by (S, lower j first), written ascending
//   pooled = sum_j exp(S_j - max S) vbar_j / sum_j exp(S_j - max S)   over all key tiles
// Top-k is a repeated wave-wide argmax over 64-bit keys: the high word is the
// score mapped to an order-preserving unsigned integer (NaN -> -inf, -0 -> +0),
// the low word is the inverted tile id, so the larger key is the larger score
// and, between equal scores, the lower tile.  The k winners are then placed in
// ascending order by counting.
#include "common.h"
#include "internal.h"

namespace h3 {

namespace {

constexpr int kMaxTiles = 2048;  // key tiles per head (LDS bound)
constexpr int kMaxSel = 1024;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) u = 0xff800000u;  // NaN ranks as -inf
  if ((u & 0x7fffffffu) == 0u) u = 0u;                   // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, kWave);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
    const uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void k_route(RouteArgs a) {
  __shared__ float sS[4][kMaxTiles];
  __shared__ int sSel[4][kMaxSel];
  __shared__ float sQ[4][D];
  __shared__ uint8_t sTaken[4][kMaxTiles];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int item = blockIdx.x * 4 + wave;
  if (item >= a.nh * a.nQ) return;  // whole wave exits together; no block barrier below
  const int h = item / a.nQ, i = item % a.nQ;
  const int nT = a.nT, npt = a.npt, nQ = a.nQ;

  const float* qb = a.qbar + ((size_t)h * nQ + i) * D;
  for (int c = lane; c < D; c += 64) sQ[wave][c] = qb[c];
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // ---- scores: lane per key tile, fp32 dot product in ascending c ----
  const float scale = rsqrtf((float)D);
  float* S = sS[wave];
  bool any_nan = false;
  for (int j = lane; j < nT; j += 64) {
    const f32x4_t* kb = reinterpret_cast<const f32x4_t*>(a.kbar + ((size_t)h * nT + j) * D);
    float s = 0.f;
#pragma unroll 8
    for (int c4 = 0; c4 < D / 4; ++c4) {
      const f32x4_t kv = kb[c4];
      s = fmaf(sQ[wave][4 * c4 + 0], kv[0], s);
      s = fmaf(sQ[wave][4 * c4 + 1], kv[1], s);
      s = fmaf(sQ[wave][4 * c4 + 2], kv[2], s);
      s = fmaf(sQ[wave][4 * c4 + 3], kv[3], s);
    }
    s *= scale;
    S[j] = s;
    any_nan |= (s != s);
    a.scores[((size_t)h * nQ + i) * nT + j] = s;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // ---- top-k over the video key tiles [npt, nT) ----
  int* sel_out = a.sel + ((size_t)h * nQ + i) * a.nsel;
  if (a.top_k >= nQ) {
    for (int j = lane; j < nQ; j += 64) sel_out[j] = npt + j;
  } else {
    int* sl = sSel[wave];
    uint8_t* taken = sTaken[wave];
    for (int j = lane; j < nT; j += 64) taken[j] = 0;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    for (int it = 0; it < a.top_k; ++it) {
      uint64_t best = 0;
      for (int j = npt + lane; j < nT; j += 64) {
        if (taken[j]) continue;
        const uint64_t key = ((uint64_t)order_key(S[j]) << 32) | (uint32_t)(~j);
        best = key > best ? key : best;
      }
      best = wave_max_u64(best);
      const int win = (int)(~(uint32_t)best);
      if (lane == 0) {
        sl[it] = win;
        taken[win] = 1;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
    // ascending order by counting
    for (int it = lane; it < a.top_k; it += 64) {
      const int j = sl[it];
      int rank = 0;
      for (int u = 0; u < a.top_k; ++u) rank += sl[u] < j;
      sel_out[rank] = j;
    }
  }

  // ---- pooled branch over all key tiles ----
  if (!a.use_pooled) return;
  any_nan = __any(any_nan);
  float m = -INFINITY;
  for (int j = lane; j < nT; j += 64) m = fmaxf(m, S[j]);
  m = wave_max(m);
  float l = 0.f;
  for (int j = lane; j < nT; j += 64) {
    const float w = __expf(S[j] - m);
    S[j] = w;
    l += w;
  }
  l = wave_sum(l);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const float inv_l = 1.0f / l;
  float* po = a.pooled + ((size_t)h * nQ + i) * D;
  for (int c = lane; c < D; c += 64) {
    float acc = 0.f;
    const float* vb = a.vbar + (size_t)h * nT * D + c;
    for (int j = 0; j < nT; ++j) acc = fmaf(S[j], vb[(size_t)j * D], acc);
    po[c] = any_nan ? __uint_as_float(0x7fc00000u) : acc * inv_l;
  }
}

}  // namespace

bool route_shape_ok(int nT, int top_k) { return nT <= kMaxTiles && top_k <= kMaxSel; }

hipError_t launch_route(int head_dim, const RouteArgs& a, hipStream_t s) {
  const int items = a.nh * a.nQ;
  dim3 grid((items + 3) / 4), block(256);
  if (head_dim == 128) hipLaunchKernelGGL(k_route<128>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(k_route<64>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace h3
