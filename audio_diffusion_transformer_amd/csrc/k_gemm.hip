// bf16 GEMM with fused epilogues for gfx950:  C[M][N] = A[M][K] * B[N][K]^T.
//
// These are the block's four products (TensorFold PR #949, "What it adds":
// q/k/v products, out projection, MLP in / out; "Precision": bf16 operands,
// fp32 sums).  Both operands are K-contiguous ([row][K] activations, [out][in]
// weights), which is the per-lane operand order of the CDNA4 MFMA:
// v_mfma_f32_16x16x32_bf16 takes 8 consecutive K elements of one A row and of
// one B row per lane.
//
// Tiling: a 512-thread workgroup (8 wave64, two per SIMD) owns a 256x256 C
// tile; wave w owns the 128x64 sub-tile (w/4, w%4) as 8x4 blocks of 16x16
// computed with v_mfma_f32_16x16x32_bf16 (128 fp32 accumulators per lane).  K advances 64 at a time through a
// two-stage LDS ring filled by global_load_lds_dwordx4: each lane's 16 bytes
// go straight to LDS, so no registers hold staged tiles.  A stage row is one
// full 128-byte line of A or B; its eight 16-byte chunks are stored XOR-
// swizzled by (row / 2) % 8, which makes the fragment reads (16 consecutive
// rows, same chunk) hit 16 distinct bank groups.
//
// Schedule (ping-pong): waves w and w + 4 share a SIMD.  Waves 0-3 (group 0)
// and 4-7 (group 1) run the same sequence of phases one phase apart: in its
// memory phase a wave reads the fragments of a whole stage (24 LDS reads), in
// its MFMA phase it issues the stage's 64 products (2 k-steps of 8x4 blocks);
// while one wave of a SIMD computes, the other reads.  All eight waves meet at
// a barrier between phases.  Each group loads half of every stage: group 0
// issues its half of stage s+1 at the start of its memory phase of stage s
// (the buffer's last readers finished a phase earlier); group 1 issues its
// half of stage s+2 at the end of its memory phase of stage s, right after its
// own reads of that buffer.  The other waves of group 1 may still be reading
// that buffer then, so group 1's half is made of rows no other wave of the
// group reads: the A rows of group 0's sub-tiles (read a phase earlier) and,
// per wave, half of the B rows that the wave itself reads.  Both groups thus
// have two phases to land their loads before the barrier that precedes the
// first read, and each phase carries half of the stage's loads.  The loads are issued as
// inline assembly (scalar base address, per-lane 32-bit offsets) so that the
// compiler does not insert its own conservative waits for them; this kernel
// waits on vmcnt itself.
//
// Workgroup ids are remapped so that each XCD (ids are dealt round-robin over
// the 8 XCDs) works on a contiguous band of tiles; within a band tiles are
// walked in groups of 8 tile-rows so that concurrent tiles share A and B
// panels in that XCD's L2.
//
// Epilogues (rounding points of the block; h3.c README on rounded bf16
// residuals).  The bf16 tile is staged through LDS so that residual loads and
// output stores are 16-byte coalesced.  The outputs are written with
// nontemporal stores: this kernel never reads them back, and streaming them
// leaves L2 to the operand panels that the running tiles share.
//   EPI_BIAS:         C = bf(acc + bias)
//   EPI_BIAS_GELU:    C = bf(gelu(acc + bias)),  gelu(z) = z/2 (1 + erf(z/sqrt2)) (gelu_erf below)
//   EPI_BIAS_RESGATE: C = bf(res + gate[seg(row)] * bf(acc + bias))
//   EPI_BIAS_SWIGLU:  C[., f] = bf(silu(bf(acc_g + bias_g)) bf(acc_u + bias_u)), the gate and
//                     up columns of feature f interleaved in blocks of 16 (C is N/2 wide)
#include "common.h"
#include "internal.h"

namespace h3 {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int STAGE = BM * BK;  // bf16 elements of one operand in one stage (32 KB)
constexpr int STAGE_BYTES = 128;  // bytes of K per stage and row: 64 bf16 or 128 int8

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// s_waitcnt immediate that waits for vmcnt <= n and leaves expcnt and lgkmcnt
// unchecked (gfx9 encoding: vmcnt in [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
#define H3_VMCNT(n) ((((n) & 15) | (((n) >> 4) << 14)) | 0x0F70)
// s_waitcnt immediate that waits for lgkmcnt == 0 only
#define H3_LGKMCNT0 0xC07F

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ uint32_t lds_addr(const bf16_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) bf16_t*)p;
}

// 16 bytes per lane from (sbase + voff) into LDS at (m0 + 16 * lane): sbase a
// wave-uniform address in SGPRs, voff a per-lane byte offset.  The ISA asks
// for one wait state between a write of M0 and a global load into LDS that
// reads it (the s_nop).  M0 is a reserved register: the compiler rejects it as
// a clobber and allocates no value to it; a build test checks that the
// kernels' assembly writes M0 only here and reads it only in these loads.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff),
               "s"(sbase), "s"(lds)
               : "memory");
}

// A wave-uniform pointer moved into SGPRs (the builtin returns int: widen
// through uint32_t, never by sign extension).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
}

__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// GELU z * Phi(z), Phi(z) = (1 + erf(z / sqrt2)) / 2, with erfc(x), x = |z| / sqrt2,
// from Abramowitz & Stegun 7.1.26: erfc(x) = (a1 t + ... + a5 t^5) e^(-x^2),
// t = 1 / (1 + p x), |error| <= 1.5e-7.  With q = erfc(x) / 2 (the
// coefficients halved), z Phi(z) = max(z, 0) - |z| q for either sign of z
// (z >= 0: z (1 - q); z < 0: z q): one fused multiply-add at the end, and the
// negative tail is computed without cancellation.  Straight-line code: one
// reciprocal, one exp2.
__device__ __forceinline__ float gelu_erf(float z) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.23164190f, az, 1.0f));  // p / sqrt2
  float q = fmaf(0.5307027145f, t, -0.7265760135f);                   // a5 / 2, a4 / 2
  q = fmaf(q, t, 0.7107068705f);                                       // a3 / 2
  q = fmaf(q, t, -0.142248368f);                                       // a2 / 2
  q = fmaf(q, t, 0.127414796f);                                        // a1 / 2
  q = q * t * __builtin_amdgcn_exp2f((z * -0.72134752044448170f) * z);  // e^(-z^2 / 2)
  return fmaf(-az, q, __builtin_elementwise_maximum(z, 0.0f));
}

__device__ __forceinline__ int seg_of(int row, int n_text, int n_prefix) {
  return row < n_text ? 0 : (row < n_prefix ? 1 : 2);
}

// I8: int8 operands (v_mfma_i32_16x16x64_i8, 64 k-values per product, 128
// per stage) with exact int32 sums, scaled in the epilogue by the row scale
// of A and the column scale of B: acc_f = (float)acc * a_scale[row] * b_scale[col].
//
// Split-K tail (MODE).  The tiles of the last, partly filled round would
// leave most CUs idle; instead the first ep.n_main workgroups of the launch
// (MODE_MAIN) cover the full rounds, and the remaining `tail` tiles are each
// split into S ranges of K, one workgroup per range, which writes its raw sums
// (fp32, or int32 for int8) to a workspace slot in the thread layout of the
// accumulators (a thread's 128 sums are one column of 16-byte vectors).  A
// second launch (MODE_REDUCE) adds a tile's S slots in a fixed order and runs
// the epilogue, one workgroup per tile and block row i of the accumulators
// (16 rows of each wave's 128), so that eight workgroups share a tile's reads.
enum { MODE_MAIN = 0, MODE_REDUCE = 1 };

template <int EPI, bool I8, int MODE>
__global__ __launch_bounds__(512, 1) void k_gemm_bf16(const void* __restrict__ A,
                                                      const void* __restrict__ B, int M,
                                                      int N, int K, GemmEpi ep) {
  // two stages of (A, B); reused whole (128 KB) by the epilogue
  __shared__ __attribute__((aligned(16))) bf16_t smem[4 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = N / BN;
  const int bid = blockIdx.x;
  int lin, slot = 0, part = 0, ib = 0;
  bool is_part = false;
  if constexpr (MODE == MODE_MAIN) {
    if (bid < ep.n_main) {  // XCD-aware: consecutive tiles on one XCD
      const int nm = ep.n_main;
      const int q8 = nm >> 3, r8 = nm & 7, xcd = bid & 7, idx = bid >> 3;
      lin = (xcd < r8) ? xcd * (q8 + 1) + idx : r8 * (q8 + 1) + (xcd - r8) * q8 + idx;
    } else {  // tail tile t = slot / S, K range slot % S
      is_part = true;
      slot = bid - ep.n_main;
      part = slot % ep.split;
      lin = ep.n_main + slot / ep.split;
    }
  } else {
    slot = (bid >> 3) * ep.split;  // the tile's first slot
    ib = bid & 7;                  // block row of the accumulators
    lin = ep.n_main + (bid >> 3);
  }
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int g = lin / per_group;
  const int first_m = g * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (lin % per_group) % gsize;
  const int tn = (lin % per_group) / gsize;
  const int m0 = tm * BM, n0 = tn * BN;
  const int grp = wave >> 2, wm = wave >> 2, wn = wave & 3;

  // Loads: a stage is 256 rows x 8 chunks per operand, moved in row groups of
  // 8 rows (64 chunks, 1 KB of LDS: one load instruction of a wave, lane l
  // taking chunk l).  Wave w of a group loads 4 row groups of each operand:
  // group 1 those of A rows 0-127 (read only by group 0) and the first half
  // of its own B rows, group 0 those of A rows 128-255 and the second half of
  // the B rows of its SIMD partner (see the schedule).  Byte offsets from the
  // stage's column.
  constexpr int ES = I8 ? 1 : 2;  // bytes per element
  const int rowb = K * ES;         // bytes per operand row
  const int ra0 = 16 * (1 - grp) + 4 * wn, rb0 = 8 * wn + 4 * (1 - grp);  // first row groups
  uint32_t ga[4], gb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane & 7;
    const int r = (ra0 + i) * 8 + (lane >> 3), rb = (rb0 + i) * 8 + (lane >> 3);
    // byte offsets below 2^32 (M K and N K are below 2^31); ragged M: clamp, rows >= M are dropped
    ga[i] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)rowb + (uint32_t)((c ^ swz(r)) * 16);
    gb[i] = (uint32_t)(n0 + rb) * (uint32_t)rowb + (uint32_t)((c ^ swz(rb)) * 16);
  }
  const uint32_t lda = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(smem) + ra0 * 1024);
  const uint32_t ldb =
      (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(smem) + STAGE * 2 + rb0 * 1024);
  auto issue = [&](int s) {
    const void* pa = uniform_ptr(static_cast<const char*>(A) + s * STAGE_BYTES);
    const void* pb = uniform_ptr(static_cast<const char*>(B) + s * STAGE_BYTES);
    const uint32_t so = (uint32_t)((s & 1) * 2 * STAGE * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dma16(pa, ga[i], lda + so + i * 1024);
      dma16(pb, gb[i], ldb + so + i * 1024);
    }
  };

  // v_mfma_f32_16x16x32_bf16: lane l supplies row l%16 of a 16-row block and
  // the 8 k-values 8 (l/16) .. +7 of a 32-wide k-step (A and B alike); the
  // result block holds, in lane l, column l%16 and rows 4 (l/16) .. +3.
  const int l16 = lane & 15, q4 = lane >> 4;
  f32x4_t acc[8][4];   // bf16 products (and the scaled int8 sums in the epilogue)
  i32x4_t acci[8][4];  // int8 products: exact int32 sums
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[i][j][e] = 0.f;
        acci[i][j][e] = 0;
      }

  // fragments of a stage (k-steps kk = 0, 1 of 32): A rows wm*128 + 16i + l%16,
  // B rows wn*64 + 16j + l%16, k-chunk 4 kk + l/16 (8 values each)
  u32x4_t fa[2][8], fb[2][4];
  auto read_frags = [&](int s) {
    const bf16_t* sa = smem + (s & 1) * 2 * STAGE;
    const bf16_t* sb = sa + STAGE;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int gc = kk * 4 + q4;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = wm * 128 + i * 16 + l16;
        fa[kk][i] = *reinterpret_cast<const u32x4_t*>(sa + r * BK + (gc ^ swz(r)) * 8);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 64 + j * 16 + l16;
        fb[kk][j] = *reinterpret_cast<const u32x4_t*>(sb + r * BK + (gc ^ swz(r)) * 8);
      }
    }
  };
  auto products = [&]() {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (I8)
            acci[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                __builtin_bit_cast(i32x4_t, fa[kk][i]), __builtin_bit_cast(i32x4_t, fb[kk][j]),
                acci[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                as_bf16x8(fa[kk][i]), as_bf16x8(fb[kk][j]), acc[i][j], 0, 0, 0);
        }
  };

  const int KT = rowb / STAGE_BYTES;  // >= 2
  // stages [k0, k1): all of K, or one of the S ranges of a split tile (>= 2 stages)
  const int k0 = is_part ? part * KT / ep.split : 0;
  const int k1 = is_part ? (part + 1) * KT / ep.split : KT;
  if constexpr (MODE == MODE_MAIN) {
    issue(k0);
    if (grp == 1) {
      issue(k0 + 1);
      __builtin_amdgcn_s_waitcnt(H3_VMCNT(8));  // stage k0 landed; stage k0+1 may be in flight
    } else {
      __builtin_amdgcn_s_waitcnt(H3_VMCNT(0));
    }
    phase_barrier();
    if (grp == 1) phase_barrier();  // the second group runs one phase behind
    for (int s = k0; s < k1; ++s) {
      // memory phase
      if (grp == 0 && s + 1 < k1) issue(s + 1);
      read_frags(s);
      __builtin_amdgcn_s_waitcnt(H3_LGKMCNT0);
      if (grp == 1) {
        if (s + 2 < k1) {
          issue(s + 2);
          __builtin_amdgcn_s_waitcnt(H3_VMCNT(8));  // this wave's half of stage s+1 has landed
        } else {
          __builtin_amdgcn_s_waitcnt(H3_VMCNT(0));
        }
      }
      phase_barrier();
      // MFMA phase
      products();
      if (grp == 0 && s + 1 < k1) __builtin_amdgcn_s_waitcnt(H3_VMCNT(0));
      phase_barrier();
    }
    if (grp == 0) phase_barrier();
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (MODE == MODE_MAIN && is_part) {  // raw sums of this K range to slot `slot`
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(ep.partial) + (size_t)slot * 32 * 512 + tid;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dst[(i * 4 + j) * 512] = I8 ? __builtin_bit_cast(u32x4_t, acci[i][j])
                                    : __builtin_bit_cast(u32x4_t, acc[i][j]);
    return;
  }
  if constexpr (MODE == MODE_REDUCE) {  // block row ib of the tile's S slots, in order
    const u32x4_t* src =
        reinterpret_cast<const u32x4_t*>(ep.partial) + ((size_t)slot * 32 + ib * 4) * 512 + tid;
#pragma unroll 4
    for (int p = 0; p < ep.split; ++p) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4_t v = src[((size_t)p * 32 + j) * 512];
        if constexpr (I8) acci[0][j] += __builtin_bit_cast(i32x4_t, v);
        else acc[0][j] += __builtin_bit_cast(f32x4_t, v);
      }
    }
  }
  // block rows in the epilogue: all 8, or row ib (held in acc[0]) when reducing
  constexpr int NI = MODE == MODE_REDUCE ? 1 : 8;

  // ---- epilogue ----
  // Accumulator element e of block (i, j) in lane l sits at row 4(l/16) + e,
  // column l%16 of that 16x16 block.  Each wave rounds its 128x64 sub-tile into
  // its own 16 KB of LDS, then writes it back in 16-byte chunks.
  if constexpr (I8) {  // int32 sums -> fp32 with the row and column scales
    float sa[NI][4], sb[4];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sa[i][e] = ep.a_scale[min(m0 + wm * 128 + (i + ib) * 16 + 4 * q4 + e, M - 1)];
#pragma unroll
    for (int j = 0; j < 4; ++j) sb[j] = ep.b_scale[n0 + wn * 64 + j * 16 + l16];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[i][j][e] = (float)acci[i][j][e] * sa[i][e] * sb[j];
  }
  bf16_t* st = smem + wave * (128 * 64);
  if constexpr (EPI == EPI_BIAS_SWIGLU) {
    // GEMM columns 32b .. 32b+15 are the gate values of features 16b .. 16b+15
    // and 32b+16 .. 32b+31 their up values, so blocks j = 2jj (gate) and
    // 2jj + 1 (up) of a lane hold the same feature: h = bf(silu(bf g) bf u).
    // The wave's 64 GEMM columns give 32 output columns (128 x 32 in LDS).
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int ncol = n0 + wn * 64 + jj * 32 + l16;
      const float bg = bf2f(ep.bias[ncol]), bu = bf2f(ep.bias[ncol + 16]);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = (i + ib) * 16 + 4 * q4 + e;
          const float g = bf2f(f2bf(acc[i][2 * jj][e] + bg));
          const float u = bf2f(f2bf(acc[i][2 * jj + 1][e] + bu));
          const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
          st[r * 32 + jj * 16 + l16] = f2bf(g * sig * u);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    const int NO = N / 2;  // output width
#pragma unroll 4
    for (int t = 0; t < NI; ++t) {  // 16 rows per t
      const int q = (t + ib) * 64 + lane;
      const int r = q >> 2, c8 = (q & 3) * 8;
      const int row = m0 + wm * 128 + r;
      if (row >= M) continue;
      const int col = (n0 + wn * 64) / 2 + c8;
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(st + r * 32 + c8),
                                  reinterpret_cast<u32x4_t*>(ep.out + (size_t)row * NO + col));
    }
    return;
  }
  // Gated residual: this lane's residual chunks (the output chunks it writes
  // below) are loaded before the staging, so that their latency passes under it.
  // The int8 form holds the int32 sums and their scales too and would spill
  // with these 64 registers live, so it loads each chunk where it is used.
  constexpr bool kResEarly = EPI == EPI_BIAS_RESGATE && !I8;
  u32x4_t xres[kResEarly ? 2 * NI : 1];
  if constexpr (kResEarly) {
#pragma unroll
    for (int t = 0; t < 2 * NI; ++t) {
      const int q = (t + 2 * ib) * 64 + lane;
      const int row = m0 + wm * 128 + (q >> 3);
      xres[t] = (u32x4_t){0u, 0u, 0u, 0u};
      if (row < M)
        xres[t] = *reinterpret_cast<const u32x4_t*>(ep.res + (size_t)row * N + n0 + wn * 64 +
                                                    (q & 7) * 8);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float bias = bf2f(ep.bias[n0 + wn * 64 + j * 16 + l16]);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = (i + ib) * 16 + 4 * q4 + e;
        float v = acc[i][j][e] + bias;
        if constexpr (EPI == EPI_BIAS_GELU) v = gelu_erf(v);
        st[r * 64 + j * 16 + l16] = f2bf(v);
      }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int t = 0; t < 2 * NI; ++t) {  // 8 rows per t
    const int q = (t + 2 * ib) * 64 + lane;
    const int r = q >> 3, c8 = (q & 7) * 8;
    const int row = m0 + wm * 128 + r;
    if (row >= M) continue;
    const int col = n0 + wn * 64 + c8;
    u32x4_t v = *reinterpret_cast<const u32x4_t*>(st + r * 64 + c8);
    const size_t o = (size_t)row * N + col;
    if constexpr (EPI == EPI_BIAS_RESGATE) {
      u32x4_t x;
      if constexpr (kResEarly) x = xres[t];
      else x = *reinterpret_cast<const u32x4_t*>(ep.res + o);
      const float* gp =
          ep.gate + (size_t)seg_of(row, ep.n_text, ep.n_prefix) * ep.gate_seg_stride + col;
      const f32x4_t g0 = *reinterpret_cast<const f32x4_t*>(gp);
      const f32x4_t g1 = *reinterpret_cast<const f32x4_t*>(gp + 4);
      const float gv[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2)
        v[t2] = pack2(fmaf(gv[2 * t2], bflo(v[t2]), bflo(x[t2])),
                      fmaf(gv[2 * t2 + 1], bfhi(v[t2]), bfhi(x[t2])));
    }
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(ep.out + o));
  }
}

// int8 product whose A rows carry one scale per group of G consecutive k
// (the FC2 input: one scale per 1,024 channels), with the gated-residual
// epilogue.  The int32 sums of each group are scaled by their row's group
// scale and added to fp32 sums, so every lane holds two sets of accumulators;
// to keep them within the registers of two waves per SIMD the workgroup tile
// is 128 x 256 (wave tile 64 x 64 as 4 x 4 blocks).  Loads, LDS layout and the
// ping-pong schedule are those of k_gemm_bf16 (A half the rows: 6 loads per
// wave and stage instead of 8).
constexpr int BMG = 128;

template <int G>
__global__ __launch_bounds__(512, 1) void k_gemm_i8g(const int8_t* __restrict__ A,
                                                     const int8_t* __restrict__ B, int M, int N,
                                                     int K, GemmEpi ep) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * (BMG + BN) * 64];  // 2 x 48 KB
  constexpr int SA = BMG * 64, SB = BN * 64, SST = SA + SB;  // bf16-element sizes (128 B rows)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles_m = (M + BMG - 1) / BMG, tiles_n = N / BN;
  const int nb = gridDim.x, bid = blockIdx.x;
  const int q8 = nb >> 3, r8 = nb & 7, xcd = bid & 7, idx = bid >> 3;
  const int lin = (xcd < r8) ? xcd * (q8 + 1) + idx : r8 * (q8 + 1) + (xcd - r8) * q8 + idx;
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int gq = lin / per_group;
  const int first_m = gq * GROUP;
  const int gsize = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (lin % per_group) % gsize;
  const int tn = (lin % per_group) / gsize;
  const int m0 = tm * BMG, n0 = tn * BN;
  const int grp = wave >> 2, wm = wave >> 2, wn = wave & 3;

  // row groups of 8 rows as in k_gemm_bf16: group 1 loads A rows 0-63 (read
  // only by group 0) and the first half of its own B rows, group 0 the rest
  const uint32_t rowb = (uint32_t)K;
  const int ra0 = 8 * (1 - grp) + 2 * wn, rb0 = 8 * wn + 4 * (1 - grp);
  uint32_t ga[2], gb[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (ra0 + i) * 8 + (lane >> 3);
    ga[i] = (uint32_t)min(m0 + r, M - 1) * rowb + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (rb0 + i) * 8 + (lane >> 3);
    gb[i] = (uint32_t)(n0 + r) * rowb + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
  }
  const uint32_t lda = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(smem) + ra0 * 1024);
  const uint32_t ldb =
      (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(smem) + SA * 2 + rb0 * 1024);
  auto issue = [&](int s) {
    const void* pa = uniform_ptr(A + s * STAGE_BYTES);
    const void* pb = uniform_ptr(B + s * STAGE_BYTES);
    const uint32_t so = (uint32_t)((s & 1) * SST * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(pa, ga[i], lda + so + i * 1024);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(pb, gb[i], ldb + so + i * 1024);
  };

  const int l16 = lane & 15, q4 = lane >> 4;
  i32x4_t acci[4][4];
  f32x4_t accf[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acci[i][j][e] = 0;
        accf[i][j][e] = 0.f;
      }
  u32x4_t fa[2][4], fb[2][4];
  auto read_frags = [&](int s) {
    const bf16_t* sa = smem + (s & 1) * SST;
    const bf16_t* sb = sa + SA;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int gc = kk * 4 + q4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + i * 16 + l16;
        fa[kk][i] = *reinterpret_cast<const u32x4_t*>(sa + r * BK + (gc ^ swz(r)) * 8);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 64 + j * 16 + l16;
        fb[kk][j] = *reinterpret_cast<const u32x4_t*>(sb + r * BK + (gc ^ swz(r)) * 8);
      }
    }
  };
  auto products = [&]() {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acci[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
              __builtin_bit_cast(i32x4_t, fa[kk][i]), __builtin_bit_cast(i32x4_t, fb[kk][j]),
              acci[i][j], 0, 0, 0);
  };
  const int ng = K / G;  // groups per row
  // the end of a group: fp32 sums += int32 sums * the rows' group scales
  auto flush = [&](int gi) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = min(m0 + wm * 64 + i * 16 + 4 * q4 + e, M - 1);
        const float sc = ep.a_scale[(size_t)row * ng + gi];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          accf[i][j][e] = fmaf((float)acci[i][j][e], sc, accf[i][j][e]);
          acci[i][j][e] = 0;
        }
      }
  };

  const int KT = K / STAGE_BYTES;  // >= 2
  constexpr int SPG = G / STAGE_BYTES;  // stages per group
  issue(0);
  if (grp == 1) {
    issue(1);
    __builtin_amdgcn_s_waitcnt(H3_VMCNT(6));
  } else {
    __builtin_amdgcn_s_waitcnt(H3_VMCNT(0));
  }
  phase_barrier();
  if (grp == 1) phase_barrier();
  for (int s = 0; s < KT; ++s) {
    if (grp == 0 && s + 1 < KT) issue(s + 1);
    read_frags(s);
    __builtin_amdgcn_s_waitcnt(H3_LGKMCNT0);
    if (grp == 1) {
      if (s + 2 < KT) {
        issue(s + 2);
        __builtin_amdgcn_s_waitcnt(H3_VMCNT(6));
      } else {
        __builtin_amdgcn_s_waitcnt(H3_VMCNT(0));
      }
    }
    phase_barrier();
    products();
    if ((s + 1) % SPG == 0) flush(s / SPG);
    if (grp == 0 && s + 1 < KT) __builtin_amdgcn_s_waitcnt(H3_VMCNT(0));
    phase_barrier();
  }
  if (grp == 0) phase_barrier();
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // ---- epilogue: bias, bf16, gated residual (as EPI_BIAS_RESGATE) ----
  // the residual chunks this lane writes, loaded before the staging
  u32x4_t xres[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int q = t * 64 + lane;
    const int row = m0 + wm * 64 + (q >> 3);
    xres[t] = (u32x4_t){0u, 0u, 0u, 0u};
    if (row < M)
      xres[t] = *reinterpret_cast<const u32x4_t*>(ep.res + (size_t)row * N + n0 + wn * 64 +
                                                  (q & 7) * 8);
  }
  bf16_t* st = smem + wave * (64 * 64);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = n0 + wn * 64 + j * 16 + l16;
    const float sbv = ep.b_scale[col], bias = bf2f(ep.bias[col]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = i * 16 + 4 * q4 + e;
        st[r * 64 + j * 16 + l16] = f2bf(accf[i][j][e] * sbv + bias);
      }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int q = t * 64 + lane;
    const int r = q >> 3, c8 = (q & 7) * 8;
    const int row = m0 + wm * 64 + r;
    if (row >= M) continue;
    const int col = n0 + wn * 64 + c8;
    u32x4_t v = *reinterpret_cast<const u32x4_t*>(st + r * 64 + c8);
    const size_t o = (size_t)row * N + col;
    const u32x4_t x = xres[t];
    const float* gp =
        ep.gate + (size_t)seg_of(row, ep.n_text, ep.n_prefix) * ep.gate_seg_stride + col;
    const f32x4_t g0 = *reinterpret_cast<const f32x4_t*>(gp);
    const f32x4_t g1 = *reinterpret_cast<const f32x4_t*>(gp + 4);
    const float gv[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
#pragma unroll
    for (int t2 = 0; t2 < 4; ++t2)
      v[t2] = pack2(fmaf(gv[2 * t2], bflo(v[t2]), bflo(x[t2])),
                    fmaf(gv[2 * t2 + 1], bfhi(v[t2]), bfhi(x[t2])));
    *reinterpret_cast<u32x4_t*>(ep.out + o) = v;
  }
}

}  // namespace

bool gemm_shape_ok(int M, int N, int K) {
  return M >= 1 && N >= BN && N % BN == 0 && K >= 2 * BK && K % (2 * BK) == 0 &&
         (long long)M * K < (1ll << 31) && (long long)N * K < (1ll << 31);
}

bool gemm_i8_shape_ok(int M, int N, int K) {
  return M >= 1 && N >= BN && N % BN == 0 && K >= 4 * BK && K % (4 * BK) == 0 &&
         (long long)M * K < (1ll << 31) && (long long)N * K < (1ll << 31);
}

template <bool I8, int MODE>
static void launch_epi(int epi, dim3 grid, dim3 block, const void* A, const void* B, int M, int N,
                       int K, const GemmEpi& ep, hipStream_t s) {
  switch (epi) {
    case EPI_BIAS:
      hipLaunchKernelGGL((k_gemm_bf16<EPI_BIAS, I8, MODE>), grid, block, 0, s, A, B, M, N, K, ep);
      break;
    case EPI_BIAS_GELU:
      hipLaunchKernelGGL((k_gemm_bf16<EPI_BIAS_GELU, I8, MODE>), grid, block, 0, s, A, B, M, N, K,
                         ep);
      break;
    case EPI_BIAS_SWIGLU:
      hipLaunchKernelGGL((k_gemm_bf16<EPI_BIAS_SWIGLU, I8, MODE>), grid, block, 0, s, A, B, M, N,
                         K, ep);
      break;
    default:
      hipLaunchKernelGGL((k_gemm_bf16<EPI_BIAS_RESGATE, I8, MODE>), grid, block, 0, s, A, B, M, N,
                         K, ep);
      break;
  }
}

// Ways the tiles of the last round are split along K: 0 (no split) unless
// that round is at most half filled; each range keeps >= 2 stages.  The split
// costs about 50 us whatever its size (the partial sums' round trip through
// HBM and the reduction launch), some 36 stages of a tile's K loop, so it is
// taken only when it shortens the last round by at least that much.
static int tail_split(int M, int N, int K, int es) {
  const int tiles = ((M + BM - 1) / BM) * (N / BN);
  const int KT = K * es / STAGE_BYTES;
  const int tail = tiles % kGemmRound;
  if (tail == 0 || 2 * tail > kGemmRound) return 0;
  int S = kGemmRound / tail;
  if (S > kGemmMaxSplit) S = kGemmMaxSplit;
  if (S > KT / 2) S = KT / 2;
  if (S < 2 || KT - (KT + S - 1) / S < kGemmSplitMinStages) return 0;
  return S;
}

size_t gemm_partial_bytes(int M, int N, int K, bool i8) {
  const int S = tail_split(M, N, K, i8 ? 1 : 2);
  const int tail = (((M + BM - 1) / BM) * (N / BN)) % kGemmRound;
  return (size_t)S * tail * BM * BN * 4;
}

// The full rounds of tiles and, when the last round is at most half filled
// and the workspace holds its partial sums, that round split along K, in one
// launch; then the reduction of the split tiles.
template <bool I8>
static hipError_t launch_split(int epi, const void* A, const void* B, int M, int N, int K,
                               const GemmEpi& ep_in, hipStream_t s) {
  const int tiles = ((M + BM - 1) / BM) * (N / BN);
  const int tail = tiles % kGemmRound;
  int S = tail_split(M, N, K, I8 ? 1 : 2);
  if (!ep_in.partial || gemm_partial_bytes(M, N, K, I8) > ep_in.partial_bytes) S = 0;
  GemmEpi ep = ep_in;
  if (S < 2) {
    ep.n_main = tiles;
    ep.split = 1;
    launch_epi<I8, MODE_MAIN>(epi, dim3(tiles), dim3(512), A, B, M, N, K, ep, s);
    return hipGetLastError();
  }
  ep.n_main = tiles - tail;
  ep.split = S;
  launch_epi<I8, MODE_MAIN>(epi, dim3(ep.n_main + tail * S), dim3(512), A, B, M, N, K, ep, s);
  launch_epi<I8, MODE_REDUCE>(epi, dim3(tail * 8), dim3(512), A, B, M, N, K, ep, s);
  return hipGetLastError();
}

hipError_t launch_gemm(int epi, const bf16_t* A, const bf16_t* B, int M, int N, int K,
                       const GemmEpi& ep, hipStream_t s) {
  return launch_split<false>(epi, A, B, M, N, K, ep, s);
}

hipError_t launch_gemm_i8(int epi, const int8_t* A, const int8_t* B, int M, int N, int K,
                          const GemmEpi& ep, hipStream_t s) {
  return launch_split<true>(epi, A, B, M, N, K, ep, s);
}

bool gemm_i8g_shape_ok(int M, int N, int K, int G) {
  return G == kFc2Group && K % G == 0 && gemm_i8_shape_ok(M, N, K);
}

hipError_t launch_gemm_i8g_resgate(const int8_t* A, const int8_t* B, int M, int N, int K, int G,
                                   const GemmEpi& ep, hipStream_t s) {
  if (G != kFc2Group) return hipErrorInvalidValue;
  const int tiles = ((M + BMG - 1) / BMG) * (N / BN);
  hipLaunchKernelGGL((k_gemm_i8g<kFc2Group>), dim3(tiles), dim3(512), 0, s, A, B, M, N, K, ep);
  return hipGetLastError();
}

}  // namespace h3
