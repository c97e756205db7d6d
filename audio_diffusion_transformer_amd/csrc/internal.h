// Host-side declarations shared by the kernel files and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3.h"

namespace h3 {

typedef uint16_t bf16_t;

// Per-kernel-class event bracketing (enabled by h3_prof_enable).
void prof_begin(int cls, hipStream_t s);
void prof_end(int cls, hipStream_t s);

// ---- modulated RMS norm ----------------------------------------------------
// out[r] = bf(x[r] * (mean(x[r]^2) + eps)^-1/2 * (1 + scale[seg]) + shift[seg])
// for rows r in [row0, row1); shift/scale of segment s at base + s*seg_stride.
// out row index is (r - out_row0).
hipError_t launch_modnorm(const bf16_t* x, bf16_t* out, int out_row0, const float* shift,
                          const float* scale, int seg_stride, int row0, int row1, int H,
                          int n_text, int n_prefix, float eps, hipStream_t s);

// ---- GEMM: C[M][N] = A[M][K] * B[N][K]^T with a fused epilogue -------------
enum { EPI_BIAS = 0, EPI_BIAS_GELU = 1, EPI_BIAS_RESGATE = 2, EPI_BIAS_SWIGLU = 3 };
struct GemmEpi {
  const bf16_t* bias;   // [N]
  bf16_t* out;          // [M][N]; EPI_BIAS_SWIGLU: [M][N/2]
  const bf16_t* res;    // [M][N] residual input (EPI_BIAS_RESGATE)
  const float* gate;    // gate of segment s, column n at gate[s * gate_seg_stride + n]
  int gate_seg_stride;
  int n_text, n_prefix; // row segment boundaries
  const float* a_scale; // int8 products: [M] row scales of A
  const float* b_scale; // int8 products: [N] row scales of B (output columns)
  void* partial;         // null, or workspace for the split-K tail's partial sums
  size_t partial_bytes;  // its size
  int n_main, split;     // set by the launcher: whole tiles, ways of the split tail
};
// a launch round: one 256x256 tile per CU; a tail tile is split at most 16 ways
constexpr int kGemmRound = 256, kGemmMaxSplit = 16, kGemmSplitMinStages = 36;
// bytes of partial sums the split-K tail of this product uses (<= 64 MB; 0: no split)
size_t gemm_partial_bytes(int M, int N, int K, bool i8);
bool gemm_shape_ok(int M, int N, int K);
bool gemm_i8_shape_ok(int M, int N, int K);
hipError_t launch_gemm(int epi, const bf16_t* A, const bf16_t* B, int M, int N, int K,
                       const GemmEpi& ep, hipStream_t s);
// int8 operands (codes), exact int32 sums scaled by a_scale[row] * b_scale[col]
hipError_t launch_gemm_i8(int epi, const int8_t* A, const int8_t* B, int M, int N, int K,
                          const GemmEpi& ep, hipStream_t s);
// int8 product with one A scale per row and group of G = kFc2Group k-values
// (a_scale [M][K/G]), gated-residual epilogue
constexpr int kFc2Group = 1024;
bool gemm_i8g_shape_ok(int M, int N, int K, int G);
hipError_t launch_gemm_i8g_resgate(const int8_t* A, const int8_t* B, int M, int N, int K, int G,
                                   const GemmEpi& ep, hipStream_t s);

// ---- head layout: q/k RMS norm + RoPE, padded head-major q, k, v^T, tile means
struct HeadsArgs {
  // source: MODE_QKV: y [R][3H] (per-head [q|k|v] interleaved);
  //         MODE_SPLIT: q, k, v [nh][R][d]
  const bf16_t* y;
  const bf16_t* q_in;
  const bf16_t* k_in;
  const bf16_t* v_in;
  const bf16_t* q_gain;  // [d] (MODE_QKV)
  const bf16_t* k_gain;
  const float* rope;     // [R][d/2][2] or null (MODE_QKV)
  bf16_t* q;             // [nh][Rp][d]
  bf16_t* k;             // [nh][Rp][d]
  bf16_t* vt;            // [nh][Rp/32][d][32]
  float* qbar;           // [nh][nQ][d]
  float* kbar;           // [nh][nT][d]
  float* vbar;           // [nh][nT][d]
  const int* tstart;     // [nT+1] real rows
  const int* tpstart;    // [nT+1] padded rows
  int R, Rp, nh, nT, npt;
  int parts;             // MODE_QKV: blocks per head in y, 3 ([q|k|v]) or 4 ([q|k|v|g])
  int ystride;           // MODE_QKV: elements per row of y (parts * nh * d)
  float eps;
};
enum { HEADS_QKV = 0, HEADS_SPLIT = 1 };
hipError_t launch_heads(int mode, int head_dim, const HeadsArgs& a, hipStream_t s);

// ---- routing: tile scores, top-k, pooled branch ------------------------------
struct RouteArgs {
  const float* qbar;    // [nh][nQ][d]
  const float* kbar;    // [nh][nT][d]
  const float* vbar;    // [nh][nT][d]
  float* scores;        // [nh][nQ][nT]
  int* sel;             // [nh][nQ][nsel]
  float* pooled;        // [nh][nQ][d]
  int nh, nQ, nT, npt, top_k, nsel, use_pooled;
};
bool route_shape_ok(int nT, int top_k);
hipError_t launch_route(int head_dim, const RouteArgs& a, hipStream_t s);

// ---- attention ---------------------------------------------------------------
struct AttnArgs {
  const bf16_t* q;          // [nh][Rp][d]
  const bf16_t* k;          // [nh][Rp][d]
  const bf16_t* vt;         // [nh][Rp/32][d][32]
  const int* sel;           // [nh][nQ][nsel]
  const float* scores;      // [nh][nQ][nT]: the tile scores (visiting order of the tiles)
  const float* pooled;      // [nh][nQ][d] or null
  const int* tpstart;       // [nT+1]
  const int* chunk_valid;   // [Rp/32]
  const int4* qblocks;      // [nqb]: (tile, padded row0, nrows, real row0)
  bf16_t* out;              // [R][A]
  const bf16_t* gate;       // null, or the routing gate of row r, head h, column c at
                            // gate[r * gate_stride + h * gate_hstride + c]
  int gate_stride, gate_hstride;
  int nh, Rp, A, nT, npt, nQ, nsel, nqb, nqb_dense, n_prefix_chunks, n_chunks;
  int max_list;             // longest video key list in chunks (prefix + nsel largest tiles)
};
bool attn_shape_ok(int n_chunks, int nsel);
// matrix-core calibration: n_blocks x 4 waves x iters x 16 bf16 products
hipError_t launch_calib_mfma(const void* operands, size_t bytes, int n_blocks, int iters,
                             float* sink, hipStream_t s);
hipError_t launch_attn(int head_dim, const AttnArgs& a, hipStream_t s);

// ---- output heads: vel[r][c] = z[r] . W[c] + b[c] (fp32 out) --------------------
hipError_t launch_out_head(const bf16_t* z, int rows, int H, const bf16_t* w, const bf16_t* b,
                           int C, float* vel, hipStream_t s);

// ---- rows in, time conditioning, Euler -------------------------------------------
struct RowsInArgs {
  const bf16_t* text;                         // [n_text][H]
  const float *audio, *video;                 // [n_audio][c_audio], [n_video][c_video]
  const float *w_audio, *b_audio, *w_video, *b_video;  // [H][c], [H]
  bf16_t* x;                                  // [R][H]
  int n_text, n_audio, n_video, H, c_audio, c_video;
};
hipError_t launch_rows_in(const RowsInArgs& a, hipStream_t s);

constexpr int kTimeEmbedDim = 256;  // width of the timestep frequency embedding

struct TimeGemvArgs {
  const float* in;        // [3][K] fp32, or null: the timestep embedding of sigma (K = 256)
  const bf16_t *w, *b;    // [N][K], [N]
  const bf16_t* table;    // null, or [n_blocks][N]: write out[l][s][o] = v + table[l][o]
  float* out;             // [3][N], or [n_blocks][3][N] with a table
  float sigma[3];
  int K, N, n_blocks, in_silu, out_silu;
};
hipError_t launch_time_gemv(const TimeGemvArgs& a, hipStream_t s);
hipError_t launch_euler(float* x, const float* v, size_t n, double dsigma, hipStream_t s);

// ---- int8 quantization ------------------------------------------------------------
// modnorm (as launch_modnorm over rows [0, rows)) followed by the row's int8 codes
hipError_t launch_modnorm_q(const bf16_t* x, const float* shift, const float* scale,
                            int seg_stride, int rows, int H, int n_text, int n_prefix, float eps,
                            int8_t* q, float* qscale, bf16_t* n_out, hipStream_t s);
bool quant_shape_ok(int K, int G);
// codes of x [rows][K] per group of G columns (G = K: per row); qscale [rows][K/G]
hipError_t launch_quant_rows(const bf16_t* x, int rows, int K, int G, int8_t* q, float* qscale,
                             hipStream_t s);

// ---- token reduction ------------------------------------------------------------
struct TokenArgs {
  const bf16_t* x;     // pool: the full stream [P + V][H]
  bf16_t* red;         // pool: out, the pooled stream [P + Vr][H]; restore: the pooled values kept (base)
  bf16_t* orig;        // pool: out, the video rows kept [V][H]; restore: in
  const bf16_t* cur;   // restore: the pooled stream after the reduced blocks [P + Vr][H]
  bf16_t* out;         // restore: out, the full stream [P + V][H]
  const int* pairs;    // [Vr][2] full video rows of each pooled token (second -1: single)
  int P, V, Vr, H;
};
hipError_t launch_token_pool(const TokenArgs& a, hipStream_t s);
hipError_t launch_token_restore(const TokenArgs& a, hipStream_t s);

// ---- small table upload through kernel arguments ------------------------------
hipError_t launch_poke(int* dst, const int* src, int n, hipStream_t s);

}  // namespace h3
