// Tile-routed attention (video rows) and dense attention (text and audio
// rows) in one kernel, on bf16 MFMA with an fp32 online softmax.
//
// TensorFold PR #949: "What it adds" (h3_attention: tile-routed attention
// with fp32 scores and an online softmax), "Precision" (softmax weights
// rounded to bf16 before the value product) and the parity notes (the audio
// rows attend densely).  A video row of query tile i attends the prefix rows
// and the rows of the selected tiles sel[h][i], and gets the fp32 pooled
// branch pooled[h][i] (times the routing gate g of the row, when one is
// given: "What it adds", q/k/v and the routing gate) added before the bf16
// rounding; a text or audio row attends every row.  (The kernel's visiting
// order of the keys, below, changes only where the online softmax rounds.)
//
// Operands (written by the head-layout kernel): q, k [nh][Rp][D] and v^T
// blocked per 32-row chunk, [nh][Rp/32][D][32], in a padded row space where
// every tile starts on a multiple of 32 rows; a 32-row "chunk" therefore never
// straddles two tiles, its K rows and its v^T block are each 32 x D contiguous
// bf16, and chunk_valid[c] gives its number of real rows.
//
// One workgroup (4 wave64) per (64-row query block, head); wave w owns the 16
// queries 16w .. 16w+15 of the block, and all four waves walk the block's key
// list one 32-key chunk at a time.  Each chunk (K rows and the matching v^T
// columns, 2 x 32 x D bf16) is streamed into a two-stage LDS ring with
// global_load_lds_dwordx4 (waves 0-1 move K, waves 2-3 move v^T), one chunk
// ahead of the one computed; the ring is XOR-swizzled so that the 16-byte
// fragment reads below are free of bank conflicts.  With 16 queries per wave
// a workgroup needs about 35 KB of LDS and few registers, so four workgroups
// share a CU and every SIMD holds four waves: one wave's softmax runs while
// another's products occupy the matrix core.
//   S^T (32 keys x 16 queries) = K (32 x D) Q^T (D x 16)      v_mfma_f32_16x16x32_bf16
// computed as two 16-key blocks kb; lane l holds query l%16 and keys
// 16 kb + 4(l/16) + e (e < 4).  Those 8 scores, rounded to bf16, are exactly
// the lane's B operand of the value product
//   O^T (D x 16 queries) += V^T (D x 32 keys) P^T (32 keys x 16 queries)
// when the contraction slot 8(l/16) + j stands for key 4(l/16) + j (j < 4) or
// 16 + 4(l/16) + j - 4 (j >= 4): v^T stores the eight 4-key blocks of every
// 32-key chunk in the order 0, 4, 1, 5, 2, 6, 3, 7, so the matching keys of a
// V^T row are one 16-byte run.  The probabilities never leave their lanes;
// the four lanes that share a query exchange the running max with two
// shuffles.  Scores are scaled into the log2 domain (exp2).
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace h3 {

namespace {

constexpr int kMaxChunks = 4096;
constexpr int kMaxSelAttn = 512;

__device__ __forceinline__ bf16x8_t pack8(const float* p) {
  u32x4_t w;
#pragma unroll
  for (int t = 0; t < 4; ++t) w[t] = pack2(p[2 * t], p[2 * t + 1]);
  return as_bf16x8(w);
}

// max(a, b), NaN if either is NaN (IEEE 754-2019 maximum): gfx950 has it as
// one instruction (v_maximum3_f32), where fmaxf needs each operand quieted
// first.  A NaN score makes its query's output NaN either way.
__device__ __forceinline__ float fmax_nan(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// The value of lanes l ^ 16 (and l ^ 32) through the gfx950 lane-swap
// instructions: with both operands equal, v_permlane16_swap returns rows
// (r0, r0, r2, r2) and (r1, r1, r3, r3) of 16 lanes, v_permlane32_swap
// (lo, lo) and (hi, hi), so max / sum of the pair is the xor-16 (xor-32)
// reduction, computed in the same operand order in every lane.
__device__ __forceinline__ float max_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t lds_addr(const bf16_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) bf16_t*)p;
}

// 16 bytes per lane from (sbase + voff) into LDS at (m0 + 16 * lane): sbase a
// wave-uniform address in SGPRs, voff a per-lane byte offset, with the one
// wait state the ISA asks for between the M0 write and the load.  M0 is a
// reserved register the compiler allocates no value to (a build test checks
// that the kernels' assembly writes it only here).  The compiler does not
// track this load; the kernel waits for it on vmcnt itself.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff),
               "s"(sbase), "s"(lds)
               : "memory");
}

// XOR swizzle of the 16-byte units of a K row (D/8 units) and of a v^T row (4
// units).  ds_read_b128 is served 8 lanes at a time over 128 bytes (8 units):
// the 8 consecutive K rows of such a group read one unit each, so their
// swizzles must differ mod 8.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (row & 15) : (row & 7);
}
// (ds_read_b128 is served 8 lanes at a time over 128 bytes: the 8 v^T rows d
// of one such group, 64 bytes apart, need distinct (d & 1, unit) pairs)
__device__ __forceinline__ int swz_v(int d) { return (d >> 1) & 3; }

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_attn(AttnArgs a) {
  constexpr int NDS = D / 32;  // 32-wide d steps of the score product
  constexpr int NDB = D / 16;  // 16-row d blocks of the value product
  constexpr int U = D / 8;     // 16-byte units per K row
  constexpr int CH = 32 * D;   // bf16 elements of a K chunk (and of a v^T chunk)
  constexpr int STG = 2 * CH;  // one stage: K chunk then v^T chunk
  constexpr int NDMA = D / 32; // 1 KB loads per lane and chunk
  constexpr int SO = D + 4;    // fp32 row stride of the output staging
  constexpr int RING = 2 * STG * 2, OSTG = 64 * SO * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[RING > OSTG ? RING : OSTG];
  // dynamic: the selected tiles' scores, chunk starts and key-list offsets (in
  // visiting order), the key list of a video block as chunk ids, then the
  // valid-row counts of every chunk
  extern __shared__ __attribute__((aligned(16))) int dyn[];
  float* const sKey = reinterpret_cast<float*>(dyn);          // [nsel]
  int* const sC0 = dyn + a.nsel;                              // [nsel]
  int* const sOff = dyn + 2 * a.nsel;                         // [nsel + 1]
  uint16_t* const sList = reinterpret_cast<uint16_t*>(dyn + 3 * a.nsel + 1);  // [max_list]
  uint8_t* const sValid = reinterpret_cast<uint8_t*>(sList + a.max_list);     // [n_chunks]
  bf16_t* const ring = reinterpret_cast<bf16_t*>(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: kept in SGPRs
  // Work order.  Dense query blocks first (they are the long ones), then video
  // blocks.  Workgroup ids are dealt round-robin over the 8 XCDs; when the head
  // count is a multiple of 8, head h is given to XCD h % 8 (XCD x runs the
  // dense blocks of its heads, then their video blocks head by head), so each
  // head's K / v^T chunks stay in one XCD's L2 and the XCDs get equal work.
  int qbi, h;
  {
    const int bid = blockIdx.x, nqv = a.nqb - a.nqb_dense;
    if ((a.nh & 7) == 0) {
      const int xcd = bid & 7, idx = bid >> 3, nhx = a.nh >> 3;
      const int nd = nhx * a.nqb_dense;
      if (idx < nd) {
        h = xcd + 8 * (idx / a.nqb_dense);
        qbi = idx % a.nqb_dense;
      } else {
        h = xcd + 8 * ((idx - nd) / nqv);
        qbi = a.nqb_dense + (idx - nd) % nqv;
      }
    } else {
      const int nd = a.nqb_dense * a.nh;
      if (bid < nd) {
        qbi = bid % a.nqb_dense;
        h = bid / a.nqb_dense;
      } else {
        qbi = a.nqb_dense + (bid - nd) % nqv;
        h = (bid - nd) / nqv;
      }
    }
  }
  const int4 qb = a.qblocks[qbi];
  const int tile = qb.x, prow0 = qb.y, nrows = qb.z, row0 = qb.w;
  const bool q_live = wave * 16 < nrows;  // this wave's 16 queries hold real rows
  const bool dense = tile < a.npt;

  for (int c = tid; c < a.n_chunks; c += 256) sValid[c] = (uint8_t)a.chunk_valid[c];

  // Key list: every chunk in order (dense rows); for video rows the chunks of
  // the selected tiles, the best-scoring tile first, then the prefix chunks.
  // The attention output does not depend on the order (each weight is taken
  // against the running max and rescaled with it); visiting the tiles the
  // routing ranks highest first settles the running max early, so later
  // chunks rarely rescale the accumulators.  When every video tile is
  // selected the list is the dense one, in the same ascending order, so a
  // routed call with all tiles gives the dense call's bytes.
  int nchunk;
  if (dense) {
    nchunk = a.n_chunks;
    __syncthreads();
  } else {
    const int qt = tile - a.npt;
    const int* sel = a.sel + ((size_t)h * a.nQ + qt) * a.nsel;
    const bool ranked = a.nsel < a.nQ;
    if (ranked) {
      const float* srow = a.scores + ((size_t)h * a.nQ + qt) * a.nT;
      for (int e = tid; e < a.nsel; e += 256) {
        const float v = srow[sel[e]];
        sKey[e] = v != v ? -INFINITY : v;  // NaN ranks as -inf
      }
      __syncthreads();
    }
    // entry e goes to position r: by descending score, ties in selection order
    // (ascending tile); with every tile selected, r = e
    for (int e = tid; e < a.nsel; e += 256) {
      int r = e;
      if (ranked) {
        const float v = sKey[e];
        r = 0;
        for (int j = 0; j < a.nsel; ++j) {
          const float w = sKey[j];
          r += (w > v) || (w == v && j < e);
        }
      }
      const int t = sel[e];
      const int p0 = a.tpstart[t], p1 = a.tpstart[t + 1];
      sC0[r] = p0 >> 5;
      sOff[r] = (p1 - p0) >> 5;
    }
    __syncthreads();
    if (wave == 0) {  // exclusive scan of the chunk counts (wave 0, shuffles)
      const int per = (a.nsel + 63) >> 6;  // entries per lane
      int lsum = 0;
      for (int j = 0; j < per; ++j) {
        const int e = lane * per + j;
        if (e < a.nsel) lsum += sOff[e];
      }
      int incl = lsum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
      }
      int run = incl - lsum;
      for (int j = 0; j < per; ++j) {
        const int e = lane * per + j;
        if (e < a.nsel) {
          const int c = sOff[e];
          sOff[e] = run;
          run += c;
        }
      }
      if (lane == 63) sOff[a.nsel] = run;
    }
    __syncthreads();
    // flat list of chunk ids: ranked tiles' chunks, then the prefix chunks
    // (ascending order with every tile selected: prefix first, like dense)
    const int nsc = sOff[a.nsel];
    const int base_sel = ranked ? 0 : a.n_prefix_chunks;
    const int base_pre = ranked ? nsc : 0;
    for (int e = tid; e < a.nsel; e += 256)
      for (int c = 0; c < sOff[e + 1] - sOff[e]; ++c)
        sList[base_sel + sOff[e] + c] = (uint16_t)(sC0[e] + c);
    for (int c = tid; c < a.n_prefix_chunks; c += 256) sList[base_pre + c] = (uint16_t)c;
    nchunk = nsc + a.n_prefix_chunks;
    __syncthreads();
  }
  auto chunk_at = [&](int ci) -> int { return dense ? ci : (int)sList[ci]; };

  const size_t Rp = (size_t)a.Rp;
  const int l16 = lane & 15, g = lane >> 4;

  // Q^T fragments (B operand): query 16 wave + l%16, d = 32 s + 8g .. +7.
  bf16x8_t qf[NDS];
  {
    const int r = wave * 16 + l16;
    const bf16_t* qp = a.q + ((size_t)h * Rp + prow0 + r) * D + 8 * g;
#pragma unroll
    for (int c = 0; c < NDS; ++c) {
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (r < nrows) w = *reinterpret_cast<const u32x4_t*>(qp + 32 * c);
      qf[c] = as_bf16x8(w);
    }
  }

  const float sl2 = rsqrtf((float)D) * 1.4426950408889634f;  // c = d^-1/2 * log2(e)
  float m = -INFINITY, l = 0.f;
  f32x4_t o[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) o[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Chunk loads: waves 0-1 move the 32 K rows (16 U units each), waves 2-3
  // the D v^T rows of 32 keys (2 D units each); lane-linear LDS slots, so the
  // swizzle is applied to the global side.
  const int part = wave >> 1, sub = wave & 1;
  const bf16_t* const gsrc = part == 0 ? a.k + (size_t)h * Rp * D : a.vt + (size_t)h * D * Rp;
  const size_t cstride = (size_t)32 * D;  // a K chunk and a v^T chunk are both 32 x D, contiguous
  uint32_t goff[NDMA];  // byte offsets of this lane's 16-byte units within a chunk
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int p = sub * (NDMA * 64) + i * 64 + lane;  // LDS slot within the K (or v^T) chunk
    if (part == 0) {
      const int row = p / U;
      goff[i] = 2u * (uint32_t)(row * D + (((p % U) ^ swz_k<D>(row)) * 8));
    } else {
      const int d = p >> 2;
      goff[i] = 2u * ((uint32_t)d * 32u + (uint32_t)(((p & 3) ^ swz_v(d)) * 8));
    }
  }
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane(
      lds_addr(ring + part * CH + sub * (NDMA * 64 * 8)));
  auto issue = [&](int stage, int chunk) {
    // (the chunk id is wave-uniform: the address is formed in SGPRs)
    const int cs = __builtin_amdgcn_readfirstlane(chunk);
    const void* src = gsrc + (size_t)(uint32_t)cs * cstride;
    const uint32_t dst = lds0 + (uint32_t)(stage * STG * 2);
#pragma unroll
    for (int i = 0; i < NDMA; ++i) dma16(src, goff[i], dst + i * 1024);
  };

  // Step j: wait for this wave's loads of chunk j, barrier (every wave's part
  // has landed, and every wave is done with the other stage), start the loads
  // of chunk j + 1 into the other stage, compute chunk j.
  __builtin_amdgcn_s_waitcnt(0);  // q fragments in registers before the chunk stream starts
  int chunk = nchunk > 0 ? chunk_at(0) : 0;
  if (nchunk > 0) issue(0, chunk);
  // (the step is written once for each ring stage, so that the stage's LDS
  // addresses are constants of the unrolled loop)
  auto step = [&](const int ci, auto stage) {
    constexpr int cur = decltype(stage)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int this_chunk = chunk;
    if (ci + 1 < nchunk) {
      chunk = chunk_at(ci + 1);
      issue(cur ^ 1, chunk);
    }
    if (!q_live) return;  // no real query in this wave: loads and barriers only
    const int valid = sValid[this_chunk];
    const bf16_t* kb = ring + cur * STG;
    const bf16_t* vb = kb + CH;

    // S^T, two 16-key blocks: K fragment (A operand, key 16 kk + l%16, d = 32 s + 8g .. +7).
    f32x4_t st[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      st[kk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int row = 16 * kk + l16;
#pragma unroll
      for (int c = 0; c < NDS; ++c) {
        const bf16x8_t kf = as_bf16x8(*reinterpret_cast<const u32x4_t*>(
            kb + row * D + (((4 * c + g) ^ swz_k<D>(row)) * 8)));
        st[kk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[c], st[kk], 0, 0, 0);
      }
    }

    // Online softmax in the log2 domain: with c = d^-1/2 log2(e) and the
    // running max m of the raw scores, p = 2^(s c - m c); when some query's
    // max rises, its sum and accumulators are rescaled by 2^(m_old c - m c).
    float sv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv[e] = st[0][e];
      sv[4 + e] = st[1][e];
    }
    if (valid < 32) {  // ragged chunk: rows at or beyond `valid` do not exist
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = 16 * (e >> 2) + 4 * g + (e & 3);
        sv[e] = key < valid ? sv[e] : -INFINITY;
      }
    }
    float mloc = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mloc = fmax_nan(mloc, sv[e]);
    mloc = max_x32(max_x16(mloc));
    const float m_new = fmax_nan(m, mloc);
    if (__any(m_new > m)) {
      const float alpha = __builtin_amdgcn_exp2f((m - m_new) * sl2);  // 0 on the first chunk
      l *= alpha;
#pragma unroll
      for (int b = 0; b < NDB; ++b) o[b] *= alpha;
      m = m_new;
    }
    const float mc = m * sl2;
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], sl2, -mc));
    l += ((sv[0] + sv[1]) + (sv[2] + sv[3])) + ((sv[4] + sv[5]) + (sv[6] + sv[7]));
    const bf16x8_t p8 = pack8(sv);

    // O^T += V^T P^T: V^T fragment (A operand, d row 16b + l%16, key slots 8g .. 8g+7).
#pragma unroll
    for (int b = 0; b < NDB; ++b) {
      const int d = 16 * b + l16;
      const bf16x8_t vf = as_bf16x8(
          *reinterpret_cast<const u32x4_t*>(vb + d * 32 + ((g ^ swz_v(d)) * 8)));
      o[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, p8, o[b], 0, 0, 0);
    }
  };
  int ci = 0;
  for (; ci + 1 < nchunk; ci += 2) {
    step(ci, std::integral_constant<int, 0>{});
    step(ci + 1, std::integral_constant<int, 1>{});
  }
  if (ci < nchunk) step(ci, std::integral_constant<int, 0>{});
  // each lane summed its own 8 keys of a chunk; the query's other keys are in
  // lanes l ^ 16, l ^ 32 and l ^ 48 (the same sum in every one of the four)
  l = sum_x32(sum_x16(l));

  // ---- stage O / l (fp32) in LDS, row-major ----
  __syncthreads();  // every wave is done with the ring (the staging reuses it)
  float* const sO = reinterpret_cast<float*>(smem);
  const int q = wave * 16 + l16;
  if (q_live) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
      *reinterpret_cast<f32x4_t*>(&sO[q * SO + 16 * b + 4 * g]) = o[b] * inv;
  }
  __syncthreads();

  // ---- add the pooled branch, round, store row-major ----
  const float* pooled = (!dense && a.pooled)
                            ? a.pooled + ((size_t)h * a.nQ + (tile - a.npt)) * D
                            : nullptr;
  const bool gated = pooled && a.gate;  // routed + g * pooled
  for (int idx = tid; idx < 64 * (D / 8); idx += 256) {
    const int qq = idx / (D / 8), d8 = (idx % (D / 8)) * 8;
    if (qq >= nrows) continue;
    u32x4_t gw = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 pairs
    if (gated)
      gw = *reinterpret_cast<const u32x4_t*>(
          a.gate + (size_t)(row0 + qq) * a.gate_stride + h * a.gate_hstride + d8);
    u32x4_t w;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float x0 = sO[qq * SO + d8 + 2 * t], x1 = sO[qq * SO + d8 + 2 * t + 1];
      if (pooled) {
        x0 = fmaf(bflo(gw[t]), pooled[d8 + 2 * t], x0);
        x1 = fmaf(bfhi(gw[t]), pooled[d8 + 2 * t + 1], x1);
      }
      w[t] = pack2(x0, x1);
    }
    *reinterpret_cast<u32x4_t*>(a.out + (size_t)(row0 + qq) * a.A + h * D + d8) = w;
  }
}

}  // namespace

bool attn_shape_ok(int n_chunks, int nsel) { return n_chunks <= kMaxChunks && nsel <= kMaxSelAttn; }

hipError_t launch_attn(int head_dim, const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.nqb * a.nh), block(256);
  const size_t dyn = sizeof(int) * (3 * (size_t)a.nsel + 1) + 2 * (size_t)a.max_list +
                     (size_t)a.n_chunks;
  if (head_dim == 128) hipLaunchKernelGGL(k_attn<128>, grid, block, dyn, s, a);
  else hipLaunchKernelGGL(k_attn<64>, grid, block, dyn, s, a);
  return hipGetLastError();
}

}  // namespace h3
