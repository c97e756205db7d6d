/*
 * h3_ref.h -- plain C++ CPU oracle of the H3-style DiT block and forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library; the product path never
 * does.  It shares no code, header or table with the HIP library.
 *
 * What it computes follows "TensorFold PR #949" (FastH3 DiT forward on Zig +
 * Metal), sections "Precision is the checkpoint's own" (bf16 weights and
 * activations, fp32 sums, fp32 tile means / scores / top-k / pooled branch,
 * softmax weights rounded to bf16 before the value product), "What it adds"
 * (the block: modulated norm, q/k/v products, head layout with q/k norm and
 * rotary, tile means, tile scores, top-k, pooled branch, routed attention,
 * out projection, MLP) and "Kernel contract" (top-k rule: a NaN score ranks as
 * -inf, ties go to the lower tile), and the h3.c README ("Antirez/h3.c:
 * MiniMax H3 inference engine for Mac computers", implementation notes: the
 * gated AdaLN with rounded bf16 residuals, QKV rows interleaved per head, the
 * Q/K norm and RoPE, the final AdaLN and bf16 output heads, F32 rows out).
 *
 * Arithmetic: fp32 throughout.  Every dot product and every reduction is one
 * running fp32 sum taken in ascending index order (descending where a
 * `reverse` flag asks for it: the self-noise measurement of the pages, which
 * reverses the tile sums).  Each fp32 operation is rounded on its own (the
 * library is built without contraction into fused multiply-adds).  bf16
 * rounding is round-to-nearest-even with NaN kept.  libm expf, erff and
 * sqrtf.  OpenMP threads only split independent outputs, so the bytes do not
 * depend on the thread count.
 *
 * bf16 values are raw 16-bit patterns.  All pointers are host pointers owned
 * by the caller.  Functions return 0, or -1 on a bad argument (message from
 * h3r_last_error()).
 */
#ifndef H3_REF_H
#define H3_REF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t n_text, n_audio, n_video;  /* packed rows, in this order */
  int32_t hidden, n_heads, head_dim, ffn;
  int32_t n_tiles, n_prefix_tiles;   /* tile map size; prefix tiles cover the text + audio rows */
  int32_t top_k;                     /* video key tiles kept per (head, video query tile) */
  int32_t pooled;                    /* 1: the pooled branch is added to video rows */
  float norm_eps;
  int32_t mlp;                       /* 0: GELU MLP, 1: SwiGLU (FC1 rows interleaved by 16) */
  int32_t gate;                      /* 1: a fourth per-head QKV block g scales the pooled branch */
} h3r_shape;

typedef struct {
  const uint16_t *w_qkv, *b_qkv;   /* [(3 + gate) A][H] rows [h][q|k|v(|g)][d], [(3 + gate) A] */
  const uint16_t *q_gain, *k_gain; /* [d] */
  const uint16_t *w_o, *b_o;       /* [H][A], [H] */
  const uint16_t *w_fc1, *b_fc1;   /* [F][H] (SwiGLU [2F][H]), [F] ([2F]) */
  const uint16_t *w_fc2, *b_fc2;   /* [H][F], [H] */
} h3r_block_weights;

/* Outputs of one block; every pointer may be NULL except x2.  The first group
 * covers all R rows, the second the n_rows requested rows, in that order. */
typedef struct {
  uint16_t* n1;                 /* [R][H] */
  uint16_t* y;                  /* [R][(3 + gate) A] */
  uint16_t *q, *k, *v, *g;      /* [nh][R][d]: q~, k~ after norm and rotary, v, the gate */
  float *qbar, *kbar, *vbar;    /* [nh][nQ][d], [nh][n_tiles][d], [nh][n_tiles][d] */
  float* scores;                /* [nh][nQ][n_tiles] */
  int32_t* sel;                 /* [nh][nQ][min(top_k, nQ)] */
  float* pooled;                /* [nh][nQ][d] */
  uint16_t* attn;               /* [n_rows][A] */
  uint16_t* o;                  /* [n_rows][H] */
  uint16_t* x1;                 /* [n_rows][H] */
  uint16_t* n2;                 /* [n_rows][H] */
  uint16_t* h;                  /* [n_rows][F] */
  uint16_t* f;                  /* [n_rows][H] */
  uint16_t* x2;                 /* [n_rows][H] */
} h3r_block_out;

/* reverse flags: bit 0 sums each tile mean's rows in descending order, bit 1
 * each tile score's d terms in descending order. */
enum { H3R_REV_MEANS = 1, H3R_REV_SCORES = 2 };

const char* h3r_last_error(void);
int h3r_set_threads(int32_t n);   /* OpenMP threads (n >= 1); returns the previous count */

/* --- steps, for the pins ------------------------------------------------- */
void h3r_round_bf16(const float* x, int64_t n, uint16_t* out);
/* out[r] = bf(x_r (sum_k x_rk^2 / H + eps)^-1/2 (1 + scale[seg_r]) + shift[seg_r]);
 * shift, scale fp32 [3][H]. */
void h3r_modnorm(const uint16_t* x, int32_t n, int32_t H, const int32_t* seg, const float* shift,
                 const float* scale, float eps, uint16_t* out);
/* out[m][o] = (sum_k a[m][k] w[o][k]) + b[o] in fp32, unrounded; b may be NULL. */
void h3r_linear(const uint16_t* a, int32_t M, int32_t K, const uint16_t* w, const uint16_t* b,
                int32_t N, float* out);
/* The same product as the textbook loop, one output at a time (slow; for the
 * check that h3r_linear's loop order changes no bit). */
void h3r_linear_plain(const uint16_t* a, int32_t M, int32_t K, const uint16_t* w,
                      const uint16_t* b, int32_t N, float* out);
void h3r_gelu(const float* z, int64_t n, float* out);   /* 0.5 z (1 + erf(z / sqrt 2)) */
void h3r_silu(const float* z, int64_t n, float* out);   /* z / (1 + e^-z) */
/* u [nh][R][d] bf16 -> bf(rope(u (sum_j u_j^2 / d + eps)^-1/2 gain)); rope fp32
 * [R][d/2][2] (cos, sin) for the pairs (i, i + d/2), or NULL. */
void h3r_qk_norm_rope(const uint16_t* u, int32_t nh, int32_t R, int32_t d, const uint16_t* gain,
                      const float* rope, float eps, uint16_t* out);
/* fp32 means of the listed tiles: u [nh][R][d] bf16 -> out [nh][n_list][d]. */
void h3r_tile_means(const uint16_t* u, int32_t nh, int32_t R, int32_t d, const int32_t* tile_start,
                    const int32_t* tiles, int32_t n_list, int32_t reverse, float* out);
/* S[h][i][j] = (sum_c qbar_ic kbar_jc) d^-1/2, fp32. */
void h3r_tile_scores(const float* qbar, const float* kbar, int32_t nh, int32_t nq, int32_t nk,
                     int32_t d, int32_t reverse, float* out);
/* The k candidates with the largest score (NaN ranks -inf, ties to the lower
 * tile id), ascending; k >= n_cand keeps all.  Writes min(k, n_cand) ids. */
void h3r_topk(const float* scores, const int32_t* cand, int32_t n_cand, int32_t k, int32_t* out);
/* sum_j softmax_j(S) vbar_j over the nk key tiles: vbar [nk][d] -> out [d]. */
void h3r_pooled(const float* scores, const float* vbar, int32_t nk, int32_t d, float* out);
/* Attention of the listed rows (see h3r_block_forward) on head-major q~, k~, v
 * [nh][R][d] with the routing results sel and pooled; gate NULL or [nh][R][d];
 * out [n_rows][nh d] bf16. */
int h3r_attention(const h3r_shape* s, const int32_t* tile_start, const uint16_t* q,
                  const uint16_t* k, const uint16_t* v, const int32_t* sel, const float* pooled,
                  const uint16_t* gate, const int32_t* rows, int32_t n_rows, uint16_t* out);

/* --- the block, the forward, routed attention ----------------------------- */
/* One block on x_in [R][H]; mod fp32 [3][6][H] (shift1, scale1, gate1,
 * shift2, scale2, gate2 per segment); rope fp32 [R][d/2][2] or NULL.  rows:
 * the rows whose attention and MLP are computed (NULL: all rows, n_rows = R);
 * the all-row steps (n1 to the routing) always cover every row. */
int h3r_block_forward(const h3r_shape* s, const int32_t* tile_start, const h3r_block_weights* w,
                      const float* mod, const float* rope, const uint16_t* x_in,
                      const int32_t* rows, int32_t n_rows, int32_t reverse, h3r_block_out* out);

/* Final modulated norm (mod_final fp32 [3][2][H]: shift, scale) of the n rows
 * x [n][H] with segments seg [n], then the heads (bf16 [c][H], [c]) in fp32
 * with no rounding: the video rows, in order, to vel_video [.][c_video], the
 * audio rows to vel_audio [.][c_audio]; text rows produce nothing. */
int h3r_final_heads(const h3r_shape* s, const uint16_t* x, const int32_t* seg, int32_t n,
                    const float* mod_final, const uint16_t* w_video, const uint16_t* b_video,
                    int32_t c_video, const uint16_t* w_audio, const uint16_t* b_audio,
                    int32_t c_audio, float* vel_video, float* vel_audio);

/* n_blocks blocks (mods fp32 [n_blocks][3][6][H]), then h3r_final_heads on
 * every row: vel_video [n_video][c_video], vel_audio [n_audio][c_audio];
 * x_out [R][H] (may be NULL) receives the last block's output. */
int h3r_dit_forward(const h3r_shape* s, int32_t n_blocks, const int32_t* tile_start,
                    const h3r_block_weights* blocks, const float* mods, const float* mod_final,
                    const float* rope, const uint16_t* x_in, const uint16_t* w_video,
                    const uint16_t* b_video, int32_t c_video, const uint16_t* w_audio,
                    const uint16_t* b_audio, int32_t c_audio, int32_t reverse,
                    float* vel_video, float* vel_audio, uint16_t* x_out);

/* Routed attention alone on head-major q, k, v [nh][R][d]: tile means, scores,
 * top-k, pooled branch and attention of the listed rows (NULL: all rows);
 * gate NULL or [nh][R][d].  sel, scores may be NULL. */
int h3r_routed_attn(const h3r_shape* s, const int32_t* tile_start, const uint16_t* q,
                    const uint16_t* k, const uint16_t* v, const uint16_t* gate,
                    const int32_t* rows, int32_t n_rows, int32_t reverse, uint16_t* out,
                    int32_t* sel, float* scores);

#ifdef __cplusplus
}
#endif
#endif /* H3_REF_H */
