// Tile-routed attention (video rows) and dense attention (text and audio
// rows) in one kernel, on bf16 MFMA with an fp32 online softmax.
//
// TensorFold PR #949: "What it adds" (h3_attention: tile-routed attention
// with fp32 scores and an online softmax), "Precision" (softmax weights
// rounded to bf16 before the value product) and the parity notes (the audio
// rows attend densely).  A video row of query tile i attends the prefix rows,
// then the rows of the selected tiles sel[h][i] in ascending order, and gets
// the fp32 pooled branch pooled[h][i] (times the routing gate g of the row,
// when one is given: "What it adds", q/k/v and the routing gate) added before
// the bf16 rounding; a text or audio row attends every row.
//
// Operands (written by the head-layout kernel): q, k [nh][Rp][D] and v^T
// [nh][D][Rp] in a padded row space where every tile starts on a multiple of
// 32 rows; a 32-row "chunk" therefore never straddles two tiles, and
// chunk_valid[c] gives its number of real rows.
//
// One workgroup (4 wave64) per (64-row query block, head).  Every wave takes
// all 64 queries and every 4th key chunk of the block's key list.  Each wave
// streams its chunks (K rows and the matching v^T columns, 2 x 32 x D bf16)
// into its own two LDS buffers with global_load_lds_dwordx4, one chunk ahead
// of the one it computes; the buffers are XOR-swizzled so that the 16-byte
// fragment reads below are free of bank conflicts.  No workgroup barrier is
// needed inside the loop: each wave waits only for its own loads.
//   S^T (32 keys x 32 queries) = K (32 x D) * Q^T (D x 32)   v_mfma_f32_32x32x16_bf16
// The MFMA result holds, in lane l, query l%32 and keys 8(e/4) + 4(l/32) + e%4
// (e < 16).  That is also the B-operand layout the value product needs:
//   O^T (D x 32 queries) += V^T (D x 16 keys) * P^T (16 keys x 32 queries)
// with the 8 key slots of lane l taken as elements e = 8m..8m+7 of S^T, so
// the probabilities never leave their lanes; v^T is stored with the middle two
// 4-key blocks of every 16-key group swapped, so the matching 8 keys of V^T
// (16m + 4(l/32) + {0..3, 8..11}) are one 16-byte run.  Each lane thus owns one query per
// 32-query half: the running max / sum need one exchange with lane l^32.
// Scores are scaled into the log2 domain (exp2).  At the end the four waves'
// (max, sum, O) are combined in LDS in a fixed wave order.
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

__device__ __forceinline__ uint32_t lds_addr(const bf16_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) bf16_t*)p;
}

// 16 bytes per lane from (sbase + voff) into LDS at (m0 + 16 * lane): sbase a
// wave-uniform address in SGPRs, voff a per-lane byte offset.  The compiler
// does not track this load; the kernel waits for it on vmcnt itself.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(lds)
               : "memory");
}

// XOR swizzle of the 16-byte units of a K row (D/8 units) and of a v^T row (4 units).
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
__device__ __forceinline__ int swz_v(int d) { return (d >> 2) & 3; }

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_attn(AttnArgs a) {
  constexpr int NDC = D / 16;  // 16-wide d slices of the score product
  constexpr int NDB = D / 32;  // 32-row d blocks of the value product
  constexpr int U = D / 8;     // 16-byte units per K row
  constexpr int CH = 32 * D;   // bf16 elements of a K chunk (and of a v^T chunk)
  constexpr int STG = 2 * CH;  // one stage: K chunk then v^T chunk
  constexpr int NDMA = D / 16; // 1 KB loads per lane for a K (or a v^T) chunk
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * 2 * STG];  // [stream][stage]
  __shared__ int sOff[kMaxSelAttn + 1];
  __shared__ int sC0[kMaxSelAttn];
  __shared__ uint8_t sValid[kMaxChunks];  // real rows of every 32-row key chunk
  __shared__ float sM[2][64], sL[2][64], sLt[64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qh = wave & 1;   // query half (rows 32 qh .. 32 qh + 31 of the block)
  const int str = wave >> 1; // key stream: chunks str, str + 2, str + 4, ...
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
  const bool q_live = qh * 32 < nrows;  // this wave's query half holds real rows
  const bool dense = tile < a.npt;

  for (int c = tid; c < a.n_chunks; c += 256) sValid[c] = (uint8_t)a.chunk_valid[c];

  // Key list: every chunk (dense rows), or the prefix chunks followed by the
  // chunks of the selected tiles in ascending tile order (video rows).
  int nchunk;
  if (dense) {
    nchunk = a.n_chunks;
    __syncthreads();
  } else {
    // Selected tiles -> chunk starts and chunk counts, all entries in
    // parallel; then an exclusive scan of the counts (wave 0, shuffles).
    const int* sel = a.sel + ((size_t)h * a.nQ + (tile - a.npt)) * a.nsel;
    for (int e = tid; e < a.nsel; e += 256) {
      const int t = sel[e];
      const int p0 = a.tpstart[t], p1 = a.tpstart[t + 1];
      sC0[e] = p0 >> 5;
      sOff[e] = (p1 - p0) >> 5;
    }
    __syncthreads();
    if (wave == 0) {
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
      int run = a.n_prefix_chunks + incl - lsum;
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
    nchunk = sOff[a.nsel];
  }
  // Position ci of the key list -> chunk id.  ci only grows, so the selected
  // entry holding it is tracked forward.
  int ent = 0;
  auto chunk_at = [&](int ci) -> int {
    if (dense || ci < a.n_prefix_chunks) return ci;
    while (sOff[ent + 1] <= ci) ++ent;
    return sC0[ent] + (ci - sOff[ent]);
  };

  const size_t Rp = (size_t)a.Rp;
  const int l32 = lane & 31, g = lane >> 5;

  // Q^T fragments (B operand): query l%32 of this wave's half, d = 16c + 8g .. +7.
  bf16x8_t qf[NDC];
  {
    const int r = qh * 32 + l32;
    const bf16_t* qp = a.q + ((size_t)h * Rp + prow0 + r) * D + 8 * g;
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (r < nrows) w = *reinterpret_cast<const u32x4_t*>(qp + 16 * c);
      qf[c] = as_bf16x8(w);
    }
  }

  const float sl2 = rsqrtf((float)D) * 1.4426950408889634f;  // c = d^-1/2 * log2(e)
  float m = -INFINITY, l = 0.f;
  f32x16_t o[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[b][e] = 0.f;

  // Chunk loads: the stream's two waves split each chunk, the first half-wave
  // pair loading the K rows and the second the v^T columns.
  bf16_t* const sbuf = smem + str * 2 * STG;
  const bf16_t* const gsrc =
      qh == 0 ? a.k + (size_t)h * Rp * D : a.vt + (size_t)h * D * Rp;
  const size_t cstride = qh == 0 ? (size_t)32 * D : (size_t)32;
  uint32_t goff[NDMA];  // byte offsets of this lane's 16-byte units within a chunk
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int p = i * 64 + lane;
    if (qh == 0) {
      const int row = p / U;
      goff[i] = 2u * (uint32_t)(row * D + (((p % U) ^ swz_k<D>(row)) * 8));
    } else {
      const int d = p >> 2;
      goff[i] = 2u * ((uint32_t)d * (uint32_t)a.Rp + (uint32_t)(((p & 3) ^ swz_v(d)) * 8));
    }
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(sbuf + qh * CH));
  auto issue = [&](int stage, int chunk) {
    const uint64_t sa = (uint64_t)(uintptr_t)(gsrc + (size_t)chunk * cstride);
    // (the builtin returns int: widen through uint32_t, never by sign extension)
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sa);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(sa >> 32));
    const void* src = (const void*)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
    const uint32_t dst = lds0 + (uint32_t)(stage * STG * 2);
#pragma unroll
    for (int i = 0; i < NDMA; ++i) dma16(src, goff[i], dst + i * 1024);
  };

  // Both streams run the same number of steps (a stream past the end of the
  // list only takes part in the barriers).  Step j: wait for this wave's loads
  // of chunk 2j + str, barrier (the partner wave's half has landed, and every
  // wave is done with the other stage), start the loads of chunk 2j + 2 + str
  // into the other stage, compute chunk 2j + str.
  const int nstep = (nchunk + 1) >> 1;
  __builtin_amdgcn_s_waitcnt(0);  // q fragments in registers before the chunk stream starts
  int chunk = str < nchunk ? chunk_at(str) : 0;
  if (str < nchunk) issue(0, chunk);
  for (int j = 0; j < nstep; ++j) {
    const int ci = 2 * j + str, cur = j & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int this_chunk = chunk;
    if (ci + 2 < nchunk) {
      chunk = chunk_at(ci + 2);
      issue(cur ^ 1, chunk);
    }
    // past the end of this stream's list, or no real query in this half (a
    // block of at most 32 rows): only the loads and barriers above
    if (ci >= nchunk || !q_live) continue;
    const int valid = sValid[this_chunk];
    const bf16_t* kb = sbuf + cur * STG;
    const bf16_t* vb = kb + CH;

    // S^T: K fragment (A operand, key l%32, d = 16c + 8g .. +7).
    f32x16_t st;
#pragma unroll
    for (int e = 0; e < 16; ++e) st[e] = 0.f;
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      const bf16x8_t kf = as_bf16x8(*reinterpret_cast<const u32x4_t*>(
          kb + l32 * D + (((2 * c + g) ^ swz_k<D>(l32)) * 8)));
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], st, 0, 0, 0);
    }

    // Online softmax in the log2 domain: with c = d^-1/2 log2(e) and the
    // running max m of the raw scores, p = 2^(s c - m c); when some query's
    // max rises, its sum and accumulators are rescaled by 2^(m_old c - m c).
    float sv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) sv[e] = st[e];
    if (valid < 32) {  // ragged chunk: rows at or beyond `valid` do not exist
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = 8 * (e >> 2) + 4 * g + (e & 3);
        sv[e] = key < valid ? sv[e] : -INFINITY;
      }
    }
    float mloc = sv[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mloc = fmaxf(mloc, sv[e]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
    const float m_new = fmaxf(m, mloc);
    if (__any(m_new > m)) {
      const float alpha = __builtin_amdgcn_exp2f((m - m_new) * sl2);  // 0 on the first chunk
      l *= alpha;
#pragma unroll
      for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[b][e] *= alpha;
      m = m_new;
    }
    const float mc = m * sl2;
    float lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      sv[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], sl2, -mc));
      lsum += sv[e];
    }
    l += lsum;
    const bf16x8_t p0 = pack8(sv), p1 = pack8(sv + 8);

    // O^T += V^T P^T: V^T fragment (A operand, d row 32b + l%32, keys 16mm + 4g
    // + {0..3, 8..11}).
#pragma unroll
    for (int b = 0; b < NDB; ++b) {
      const int d = 32 * b + l32;
      const bf16x8_t v0 = as_bf16x8(*reinterpret_cast<const u32x4_t*>(
          vb + d * 32 + (((0 + g) ^ swz_v(d)) * 8)));
      const bf16x8_t v1 = as_bf16x8(*reinterpret_cast<const u32x4_t*>(
          vb + d * 32 + (((2 + g) ^ swz_v(d)) * 8)));
      o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, p0, o[b], 0, 0, 0);
      o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, p1, o[b], 0, 0, 0);
    }
  }
  // each lane summed its own 16 keys of a chunk; the query's other 16 are in lane l ^ 32
  l += __shfl_xor(l, 32, kWave);

  // ---- combine the two streams: fixed order 0, 1 ----
  __syncthreads();  // every wave is done with its chunk buffers (sO reuses them)
  float (*sO)[D + 1] = reinterpret_cast<float (*)[D + 1]>(smem);
  const int q = qh * 32 + l32;
  if (g == 0) {
    sM[str][q] = m;
    sL[str][q] = l;
  }
  __syncthreads();
  const float M = fmaxf(sM[0][q], sM[1][q]);
  const float f = m == -INFINITY ? 0.f : exp2f((m - M) * sl2);
  if (str == 0 && g == 0) {
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 2; ++w)
      L += sM[w][q] == -INFINITY ? 0.f : sL[w][q] * exp2f((sM[w][q] - M) * sl2);
    sLt[q] = L;
  }
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    if (str == w) {
#pragma unroll
      for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int d = 32 * b + 8 * (e >> 2) + 4 * g + (e & 3);
          const float val = o[b][e] * f;
          sO[q][d] = (w == 0) ? val : sO[q][d] + val;
        }
    }
    __syncthreads();
  }

  // ---- normalise, add the pooled branch, round, store row-major ----
  const float* pooled = (!dense && a.pooled)
                            ? a.pooled + ((size_t)h * a.nQ + (tile - a.npt)) * D
                            : nullptr;
  const bool gated = pooled && a.gate;  // routed + g * pooled
  for (int idx = tid; idx < 64 * (D / 8); idx += 256) {
    const int qq = idx / (D / 8), d8 = (idx % (D / 8)) * 8;
    if (qq >= nrows) continue;
    const float inv = 1.0f / sLt[qq];
    u32x4_t gw = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 pairs
    if (gated)
      gw = *reinterpret_cast<const u32x4_t*>(
          a.gate + (size_t)(row0 + qq) * a.gate_stride + h * a.gate_hstride + d8);
    u32x4_t w;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float x0 = sO[qq][d8 + 2 * t] * inv, x1 = sO[qq][d8 + 2 * t + 1] * inv;
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
  if (head_dim == 128) hipLaunchKernelGGL(k_attn<128>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(k_attn<64>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace h3
