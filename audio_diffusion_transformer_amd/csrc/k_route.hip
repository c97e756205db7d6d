// Routing for video query tiles: tile scores, top-k key tiles and the pooled
// branch, all in fp32.
//
// TensorFold PR #949: "What it adds" (h3_routing: tile scores, top-k, pooled
// branch), "Precision" (fp32 tile means, scores, top-k and pooled branch) and
// "Kernel contract" (top-k rule: a NaN score ranks as -inf, ties go to the
// lower tile).
//
// One wave per (head, video query tile); a workgroup takes 8 query tiles of one
// head, so the head's key-tile means are staged through LDS once for 8 waves.
//   S[j]   = (qbar . kbar_j) * D^-1/2          for every key tile j (fp32, c ascending)
//   sel    = the top_k video tiles by (S, lower j first), written ascending
//   pooled = sum_j exp(S_j - max S) vbar_j / sum_j exp(S_j - max S)   over all key tiles
// Lane l holds the scores of tiles l, l + 64, ...  Top-k is a radix select
// over 64-bit keys: the high word is the score mapped to an order-preserving
// unsigned integer (NaN -> -inf, -0 -> +0), the low word the inverted tile id,
// so the larger key is the larger score and, between equal scores, the lower
// tile; keys are distinct.  The k-th largest key T is found bit by bit from
// the top (a candidate bit stays set when at least k keys are >= the
// candidate, counted with wave ballots; the low word's bits above the tile
// ids, set in every real key, are set without counting), and the selected
// tiles are exactly the keys >= T, written in ascending tile order from the
// ballot masks.
#include "common.h"
#include "internal.h"

namespace h3 {

namespace {

constexpr int kMaxTiles = 2048;            // key tiles per head (64 lanes x 32 scores)
constexpr int kMaxSel = 1024;
constexpr int kQT = 8;                     // query tiles (waves) per workgroup

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) u = 0xff800000u;  // NaN ranks as -inf
  if ((u & 0x7fffffffu) == 0u) u = 0u;                   // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// PL: scores held per lane (tiles <= 64 PL)
// (up to 8 scores per lane: at most 80 VGPRs, six waves per SIMD, so three
// 8-wave workgroups share a CU)
template <int D, int PL>
__global__ __launch_bounds__(64 * kQT, PL <= 8 ? 6 : 1) void k_route(RouteArgs a) {
  constexpr int SR = D + 4;  // LDS row stride (floats): 16-byte row reads of 16 lanes hit distinct banks
  __shared__ __attribute__((aligned(16))) float sRow[64 * SR];
  __shared__ __attribute__((aligned(16))) float sQ[kQT][D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, i = blockIdx.x * kQT + wave;
  const int nT = a.nT, npt = a.npt, nQ = a.nQ;
  const bool active = i < nQ;  // an idle wave still takes part in the staging and barriers
  const int ntl = (nT + 63) >> 6;

  if (active)
    for (int c = lane; c < D; c += 64) sQ[wave][c] = a.qbar[((size_t)h * nQ + i) * D + c];

  // Rows j0 .. j0+63 of a [nT][D] table (rows >= nT as zeros) pass through
  // registers into sRow: the next group's loads are issued before the current
  // group is used, so their latency passes under the work on it.
  constexpr int NSL = 64 * (D / 4) / (64 * kQT);  // 16-byte units per thread and group
  f32x4_t sreg[NSL];
  auto load_stage = [&](const float* src, int j0) {
    const int rows = min(64, nT - j0);
#pragma unroll
    for (int k = 0; k < NSL; ++k) {
      const int idx = k * 64 * kQT + tid;
      const int r = idx / (D / 4), c4 = idx % (D / 4);
      sreg[k] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      if (r < rows) sreg[k] = *reinterpret_cast<const f32x4_t*>(src + (size_t)(j0 + r) * D + 4 * c4);
    }
  };
  auto store_stage = [&]() {
#pragma unroll
    for (int k = 0; k < NSL; ++k) {
      const int idx = k * 64 * kQT + tid;
      *reinterpret_cast<f32x4_t*>(&sRow[(idx / (D / 4)) * SR + 4 * (idx % (D / 4))]) = sreg[k];
    }
  };

  // ---- scores: lane l scores tile 64 t + l ----
  const float scale = rsqrtf((float)D);
  const float* kb = a.kbar + (size_t)h * nT * D;
  const float* vb = a.vbar + (size_t)h * nT * D;
  float* srow_out = a.scores + ((size_t)h * nQ + i) * nT;
  float sc[PL];
  bool any_nan = false;
  load_stage(kb, 0);
#pragma unroll
  for (int t = 0; t < PL; ++t) {
    sc[t] = 0.f;
    if (t < ntl) {
      __syncthreads();
      store_stage();
      __syncthreads();
      if (t + 1 < ntl) load_stage(kb, 64 * (t + 1));
      else if (a.use_pooled) load_stage(vb, 0);  // first v-bar rows, under the top-k
      const int j = 64 * t + lane;
      if (active && j < nT) {
        const float* kr = &sRow[lane * SR];
        float s = 0.f;
        // (deeper unrolling holds more loads in flight but costs registers: by 2
        // up to 4 scores per lane, not at all with 8, for the 80-register bound)
        constexpr int kScoreUnroll = PL <= 4 ? 2 : 1;
#pragma unroll kScoreUnroll
        for (int c4 = 0; c4 < D / 4; ++c4) {
          const f32x4_t kv = *reinterpret_cast<const f32x4_t*>(kr + 4 * c4);
          const f32x4_t qv = *reinterpret_cast<const f32x4_t*>(&sQ[wave][4 * c4]);
          s = fmaf(qv[0], kv[0], s);
          s = fmaf(qv[1], kv[1], s);
          s = fmaf(qv[2], kv[2], s);
          s = fmaf(qv[3], kv[3], s);
        }
        s *= scale;
        sc[t] = s;
        any_nan |= (s != s);
        srow_out[j] = s;
      }
    }
  }

  // ---- top-k over the video key tiles [npt, nT) ----
  if (active) {
    int* sel_out = a.sel + ((size_t)h * nQ + i) * a.nsel;
    if (a.top_k >= nQ) {
      for (int j = lane; j < nQ; j += 64) sel_out[j] = npt + j;
    } else {
      uint64_t key[PL];
#pragma unroll
      for (int t = 0; t < PL; ++t) {
        const int j = 64 * t + lane;
        key[t] = (t < ntl && j >= npt && j < nT)
                     ? (((uint64_t)order_key(sc[t]) << 32) | (uint32_t)(~j))
                     : 0ull;  // below every real key
      }
      // T, the top_k-th largest key, built from the top bit down.  It is a
      // real key (top_k < nQ real keys), and every real key's low word ~j has
      // all bits from log2(nT) up set (j < nT): those bits of T are set
      // without counting.
      int idb = 0;  // bits of a tile id
      while ((1 << idb) < nT) ++idb;
      uint64_t T = 0;
      for (int b = 63; b >= 0; --b) {
        if (b < 32 && b >= idb) {
          T |= 1ull << b;
          continue;
        }
        const uint64_t cand = T | (1ull << b);
        int cnt = 0;
#pragma unroll
        for (int t = 0; t < PL; ++t)
          if (t < ntl) cnt += __popcll(__ballot(key[t] >= cand));
        if (cnt >= a.top_k) T = cand;
      }
      int off = 0;
#pragma unroll
      for (int t = 0; t < PL; ++t) {
        if (t < ntl) {
          const bool mine = key[t] >= T;
          const uint64_t msk = __ballot(mine);
          if (mine) sel_out[off + __popcll(msk & ((1ull << lane) - 1ull))] = 64 * t + lane;
          off += __popcll(msk);
        }
      }
    }
  }

  // ---- pooled branch over all key tiles ----
  if (!a.use_pooled) return;  // uniform over the grid
  any_nan = __any(any_nan);
  float m = -INFINITY;
#pragma unroll
  for (int t = 0; t < PL; ++t)
    if (t < ntl && 64 * t + lane < nT) m = fmaxf(m, sc[t]);
  m = wave_max(m);
  float l = 0.f;
#pragma unroll
  for (int t = 0; t < PL; ++t) {
    const bool ok = t < ntl && 64 * t + lane < nT;
    sc[t] = ok ? __expf(sc[t] - m) : 0.f;
    l += sc[t];
  }
  l = wave_sum(l);
  float acc[D / 64];
#pragma unroll
  for (int u = 0; u < D / 64; ++u) acc[u] = 0.f;
#pragma unroll
  for (int t = 0; t < PL; ++t) {
    if (t < ntl) {
      __syncthreads();
      store_stage();
      __syncthreads();
      if (t + 1 < ntl) load_stage(vb, 64 * (t + 1));
      // rows past nT are staged as zeros and their weights are 0: adding
      // 0 * 0 leaves the sum unchanged, so all 64 rows run unconditionally
#pragma unroll 16
      for (int r = 0; r < 64; ++r) {
        const float w = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc[t]), r));
#pragma unroll
        for (int u = 0; u < D / 64; ++u) acc[u] = fmaf(w, sRow[r * SR + lane + 64 * u], acc[u]);
      }
    }
  }
  if (active) {
    const float inv_l = 1.0f / l;
    float* po = a.pooled + ((size_t)h * nQ + i) * D;
#pragma unroll
    for (int u = 0; u < D / 64; ++u)
      po[lane + 64 * u] = any_nan ? __uint_as_float(0x7fc00000u) : acc[u] * inv_l;
  }
}

}  // namespace

bool route_shape_ok(int nT, int top_k) { return nT <= kMaxTiles && top_k <= kMaxSel; }

template <int D>
static void launch_d(int ntl, dim3 grid, dim3 block, const RouteArgs& a, hipStream_t s) {
  if (ntl <= 4) hipLaunchKernelGGL((k_route<D, 4>), grid, block, 0, s, a);
  else if (ntl <= 8) hipLaunchKernelGGL((k_route<D, 8>), grid, block, 0, s, a);
  else if (ntl <= 16) hipLaunchKernelGGL((k_route<D, 16>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((k_route<D, 32>), grid, block, 0, s, a);
}

hipError_t launch_route(int head_dim, const RouteArgs& a, hipStream_t s) {
  dim3 grid((a.nQ + kQT - 1) / kQT, a.nh), block(64 * kQT);
  const int ntl = (a.nT + 63) / 64;
  if (head_dim == 128) launch_d<128>(ntl, grid, block, a, s);
  else launch_d<64>(ntl, grid, block, a, s);
  return hipGetLastError();
}

}  // namespace h3
