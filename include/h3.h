/*
 * h3.h -- C ABI of the MI355X (gfx950) forward of an H3-style joint
 * video+audio diffusion transformer.
 *
 * The computation follows "TensorFold PR #949" (FastH3 DiT forward on Zig +
 * Metal): sections "Precision is the checkpoint's own" (bf16 weights and
 * activations, fp32 sums, fp32 tile means / scores / top-k / pooled branch,
 * softmax weights rounded to bf16 before the value product) and "What it
 * adds" (one block: modulated norm, q/k/v products, head layout with q/k
 * norm and rotary, tile means, tile scores, top-k, pooled branch,
 * tile-routed attention with an online softmax, out projection, MLP), and
 * the h3.c README ("Antirez/h3.c: MiniMax H3 inference engine for Mac
 * computers": fused gated AdaLN with rounded bf16 residuals, QKV rows
 * interleaved per attention head, bf16 output heads, F32 rows out).
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller.  bf16 values
 *     are raw 16-bit patterns (h3_bf16).  Layouts are dense row-major as
 *     written next to each argument; weights follow the [out][in] convention.
 *   - Host structs (h3_shape, weights tables) and tile_start are HOST memory,
 *     read during the call only.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     stream-ordered and asynchronous: shapes are validated on the host
 *     before any launch; device faults surface at the caller's next sync.
 *   - The library allocates no device memory and keeps no pointer after it
 *     returns.  Scratch lives in the caller's workspace `ws` (256-byte
 *     aligned, at least h3_workspace_bytes() bytes).  Concurrent calls need
 *     distinct workspaces.  (One exception, h3_modulation_noalloc: its
 *     scratch is a static device array of the library, see there.)
 *   - Outputs must not alias inputs.  Pointers must be 16-byte aligned.
 *   - Same inputs on the same device give byte-identical outputs (no float
 *     atomics; every reduction has a fixed order).
 *   - Return value: H3_OK, or a negative code with a message available from
 *     h3_last_error() (thread-local).
 *
 * Packed rows: R = n_text + n_audio + n_video rows, in that order; the first
 * P = n_text + n_audio rows are the prefix.  The tile map tile_start[0..n_tiles]
 * is strictly increasing, tile_start[0] = 0, tile_start[n_tiles] = R, and
 * segment boundaries fall on tile boundaries: tiles [0, n_prefix_tiles) cover
 * the prefix rows, the rest cover the video rows (the "video tiles").
 */
#ifndef H3_H
#define H3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t h3_bf16;

enum {
  H3_OK = 0,
  H3_EINVAL = -1,       /* bad shape, tile map or null required pointer */
  H3_EWORKSPACE = -2,   /* ws_bytes smaller than h3_workspace_bytes() */
  H3_EHIP = -3,         /* a HIP launch or runtime error */
  H3_EUNSUPPORTED = -4  /* valid but not supported: head_dim not 64/128, more than 2048 tiles,
                           more than 512 selected tiles, padded rows above 131072, more than
                           2^26 rows */
};

enum { H3_WS_BLOCK = 0, H3_WS_DIT = 1, H3_WS_ATTN = 2, H3_WS_DIT_I8 = 3 };

#define H3_ABI_VERSION 5

typedef struct {
  int32_t n_text, n_audio, n_video;  /* packed in this order; >= 0, at most 2^26 in all */
  int32_t hidden;                    /* H: multiple of 256, <= 8192 */
  int32_t n_heads, head_dim;         /* head_dim in {64, 128}; attention width A = n_heads * head_dim
                                        (may differ from H; (3 + gate) A a multiple of 256) */
  int32_t ffn;                       /* F, multiple of 256 */
  int32_t n_tiles, n_prefix_tiles;   /* tile map size (<= 2048); prefix tiles cover rows [0, P) */
  int32_t top_k;                     /* video key tiles per (head, video query tile); >= nQ keeps all;
                                        min(top_k, nQ) <= 512 */
  int32_t pooled;                    /* 1: add the pooled branch to video rows */
  float norm_eps;                    /* eps of the RMS norms (activation and Q/K) */
  int32_t mlp;                       /* H3_MLP_GELU or H3_MLP_SWIGLU */
  int32_t gate;                      /* 1: the QKV product has a fourth per-head block, the routing
                                        gate g, and video rows get routed + g * pooled */
} h3_shape;

/* MLP of the block.  GELU: h = bf(gelu(n2 W1^T + b1)), W1 [F][H].
 * SwiGLU (TensorFold PR #949, "What it adds": the SwiGLU MLP): W1 [2F][H] whose
 * rows alternate in blocks of 16 (rows 32b .. 32b+15: gate rows of features
 * 16b .. 16b+15; rows 32b+16 .. 32b+31: their up rows), b1 likewise;
 * h = bf(silu(bf(g)) * bf(u)), silu(z) = z / (1 + e^-z). */
enum { H3_MLP_GELU = 0, H3_MLP_SWIGLU = 1 };

/* One block's weights, all bf16, device pointers. */
typedef struct {
  const h3_bf16 *w_qkv, *b_qkv;  /* [(3 + gate) A][H], [(3 + gate) A]; output rows per head
                                    interleaved [h][q|k|v][d], or [h][q|k|v|g][d] with the gate */
  const h3_bf16 *q_gain, *k_gain;/* [d] each: gains of the per-head Q/K RMS norm */
  const h3_bf16 *w_o, *b_o;      /* [H][A], [H] */
  const h3_bf16 *w_fc1, *b_fc1;  /* [F][H], [F]; SwiGLU: [2F][H], [2F] (see H3_MLP_SWIGLU) */
  const h3_bf16 *w_fc2, *b_fc2;  /* [H][F], [H] */
} h3_block_weights;

/* Output heads of the forward (bf16, device). */
typedef struct {
  const h3_bf16 *w_video, *b_video;  /* [c_video][H], [c_video] */
  const h3_bf16 *w_audio, *b_audio;  /* [c_audio][H], [c_audio] */
  int32_t c_video, c_audio;          /* each in [1, 256] */
} h3_head_weights;

/* F32 patch projections of the rows in (device). */
typedef struct {
  const float *w_video, *b_video;  /* [H][c_video], [H] */
  const float *w_audio, *b_audio;  /* [H][c_audio], [H] */
  int32_t c_video, c_audio;        /* patch widths, each in [1, 256] */
} h3_rows_in_weights;

/* Time embedder and modulation projections (bf16, device). */
typedef struct {
  const h3_bf16 *w1, *b1;            /* [H][256], [H] */
  const h3_bf16 *w2, *b2;            /* [H][H], [H] */
  const h3_bf16 *w_mod, *b_mod;      /* [6H][H], [6H] */
  const h3_bf16 *mod_table;          /* [n_blocks][6][H]: per-block offsets */
  const h3_bf16 *w_final, *b_final;  /* [2H][H], [2H] */
} h3_time_weights;

/* Byte offsets of the intermediates inside a block workspace (for tests and
 * diagnostics).  After h3_block_forward returns (and the stream is synced)
 * the workspace holds: n2 (the MLP norm output, [R][H] bf16, in `norm`),
 * the GELU activations ([R][F] bf16, in `big`), the head-major padded
 * q, k ([nh][Rp][d] bf16) and v transposed per 32-row chunk ([nh][Rp/32][d][32]
 * bf16, the 4-row blocks of a chunk in the order 0, 4, 1, 5, 2, 6, 3, 7), the tile
 * means (fp32 [nh][nQ][d], [nh][n_tiles][d] x2), scores (fp32
 * [nh][nQ][n_tiles]), sel (int32 [nh][nQ][min(top_k, nQ)]), pooled (fp32
 * [nh][nQ][d]), attn ([R][H] bf16) and x1 ([R][H] bf16).  Padded row space:
 * tile t occupies rows [tile_pstart[t], tile_pstart[t+1]) with
 * tile_pstart[t+1] - tile_pstart[t] = 32 * ceil(len_t / 32); its first len_t
 * rows are the tile's rows in order, the rest are zero. */
typedef struct {
  size_t tables, norm, big, q, k, vt, qbar, kbar, vbar, scores, sel, pooled, attn, x1;
  size_t xa, xb;         /* residual ping-pong of h3_dit_forward (0 if unused) */
  size_t q8, qscale;     /* int8 forward: activation codes [R][max(H, A, F)], row scales [R] */
  size_t partial;        /* products: partial sums of a split last round (0 if unused) */
  size_t total;
  int32_t padded_rows;   /* Rp */
  int32_t n_query_tiles; /* nQ = n_tiles - n_prefix_tiles */
  int32_t n_sel;         /* min(top_k, nQ) */
} h3_ws_layout;

int h3_abi_version(void);
const char* h3_last_error(void);

/* Bytes of workspace needed by the entry point `which` (H3_WS_*) for this
 * shape and tile map; 0 on invalid input (see h3_last_error).
 * Debugging aid: with the environment variable H3_WS_GUARD=<n> set at
 * planning time, every workspace region (of these calls and of
 * h3_denoise_workspace_bytes / the token-reduction forward) is followed by n
 * bytes, rounded up to 256, that no kernel touches; the sizes and offsets
 * reported here include the bands.  A caller can fill the workspace with a
 * pattern and check the bands after a call.  The same variable must be set
 * when the workspace is sized and when the call runs. */
size_t h3_workspace_bytes(const h3_shape* shape, const int32_t* tile_start, int32_t which);

/* Offsets of the workspace regions (see h3_ws_layout).  Returns H3_OK or an error. */
int h3_workspace_layout(const h3_shape* shape, const int32_t* tile_start, int32_t which,
                        h3_ws_layout* out);

/* One DiT block (TensorFold PR #949, "What it adds": block.zig; GELU MLP):
 *   n1 = bf(x rms(x)^-1 (1 + scale1[seg]) + shift1[seg])
 *   y  = bf(n1 Wqkv^T + b);  per head q, k, v;  q~, k~ = bf(rope(rmsnorm(.) gain))
 *   routing on q~, k~, v: fp32 tile means and scores, top-k video key tiles
 *   (NaN ranks -inf, ties to the lower tile), pooled branch
 *   attn = bf(attention): text/audio rows dense over all rows; video rows over
 *          the prefix rows plus the selected tiles, + pooled if enabled
 *   x1 = bf(x + gate1[seg] bf(attn Wo^T + bo))
 *   n2 = bf(x1 rms(x1)^-1 (1 + scale2[seg]) + shift2[seg])
 *   x2 = bf(x1 + gate2[seg] bf(bf(gelu(n2 W1^T + b1)) W2^T + b2))
 * With shape->mlp = H3_MLP_SWIGLU the MLP hidden row is bf(silu(bf g) bf u)
 * (see H3_MLP_SWIGLU); with shape->gate = 1 the video rows' attention output is
 * bf(routed + g pooled), g the fourth per-head block of y (TensorFold PR #949,
 * "What it adds": q/k/v and the routing gate, the pooled branch).
 * mod:  fp32 [3 segments][6][H], vectors (shift1, scale1, gate1, shift2, scale2, gate2).
 * rope: fp32 [R][d/2][2] (cos, sin) for the pairs (i, i + d/2), or NULL (no rotation).
 * x_in, x_out: [R][H] bf16.  Workspace: H3_WS_BLOCK. */
int h3_block_forward(const h3_shape* shape, const int32_t* tile_start,
                     const h3_block_weights* w, const float* mod, const float* rope,
                     const h3_bf16* x_in, h3_bf16* x_out, void* ws, size_t ws_bytes,
                     void* stream);

/* The forward: n_blocks blocks (blocks: HOST array of n_blocks weight tables;
 * mod: fp32 [n_blocks][3][6][H]), then the final modulated norm of the audio
 * and video rows (mod_final: fp32 [3 segments][2][H], (shift, scale)) and the
 * output heads, F32 with no rounding:
 *   vel_video [n_video][c_video], vel_audio [n_audio][c_audio]  (fp32, device).
 * h3.c README (final audio/video AdaLN, bf16 heads); TensorFold PR #949 (raw
 * f32 rows out).  Workspace: H3_WS_DIT. */
int h3_dit_forward(const h3_shape* shape, int32_t n_blocks, const int32_t* tile_start,
                   const h3_block_weights* blocks, const h3_head_weights* heads,
                   const float* mod, const float* mod_final, const float* rope,
                   const h3_bf16* x_in, float* vel_video, float* vel_audio,
                   void* ws, size_t ws_bytes, void* stream);

/* Routed attention alone on head-major q, k, v ([nh][R][d] bf16): tile
 * means, scores, top-k, pooled branch and attention as in h3_block_forward.
 *   out:    [R][nh*d] bf16.
 *   gate:   NULL, or [R][nh*d] bf16: video rows get routed + gate * pooled
 *           (fp32, then the bf16 rounding); text and audio rows ignore it.
 *   sel:    NULL or int32 [nh][nQ][min(top_k, nQ)]: selected tile ids, ascending.
 *   scores: NULL or fp32 [nh][nQ][n_tiles]: the tile scores.
 * Workspace: H3_WS_ATTN. */
int h3_routed_attn(const h3_shape* shape, const int32_t* tile_start,
                   const h3_bf16* q, const h3_bf16* k, const h3_bf16* v,
                   const h3_bf16* gate, h3_bf16* out, int32_t* sel, float* scores,
                   void* ws, size_t ws_bytes, void* stream);

/* The rows in (h3.c README, implementation notes: the F32 patch projections
 * rounded straight into the packed hidden stream; TensorFold PR #949, "What
 * it adds": the rows in):
 *   x[text rows]  = text_rows (copied)
 *   x[audio rows] = bf(audio_patch W_audio^T + b_audio)   F32 weights, inputs and sums
 *   x[video rows] = bf(video_patch W_video^T + b_video)
 * text_rows [n_text][H] bf16 (the text encoder's output); audio_patch
 * [n_audio][c_audio], video_patch [n_video][c_video] fp32; x [R][H] bf16.
 * All device pointers, 16-byte aligned.  No workspace. */
int h3_rows_in(const h3_shape* shape, const h3_rows_in_weights* w, const h3_bf16* text_rows,
               const float* audio_patch, const float* video_patch, h3_bf16* x, void* stream);

/* The modulation tables of one denoising step from the per-segment timesteps
 * sigma3 (HOST array: text, audio, video), TensorFold PR #949, "What comes
 * next" (the time embedder and modulation tables).  With t = 1000 sigma_s:
 *   e_s = [cos(t w_i)] ++ [sin(t w_i)], w_i = 10000^(-i/128), i < 128
 *   c_s = W2 silu(W1 e_s + b1) + b2
 *   mod[l][s]   = W_mod silu(c_s) + b_mod + mod_table[l]   fp32 [n_blocks][3][6][H]
 *   mod_final[s] = W_final silu(c_s) + b_final             fp32 [3][2][H]
 * ws: h3_modulation_workspace_bytes(shape) bytes of device scratch, 256-byte aligned. */
size_t h3_modulation_workspace_bytes(const h3_shape* shape);
int h3_modulation(const h3_shape* shape, int32_t n_blocks, const h3_time_weights* tw,
                  const float* sigma3, float* mod, float* mod_final, void* ws, size_t ws_bytes,
                  void* stream);

/* h3_modulation for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and outputs, with its scratch (the time embedder's hidden
 * and conditioning vectors, 6 x hidden fp32) in a static device array of the
 * library, 6 x 8192 floats (192 KiB) per GPU, held until the process ends.
 * No workspace argument; the call allocates nothing.  hidden above 8192:
 * H3_EUNSUPPORTED.  Every call on one GPU shares that array, so calls that
 * overlap on one GPU (concurrent streams or threads) race; serialize them.
 * Other errors as h3_modulation. */
int h3_modulation_noalloc(const h3_shape* shape, int32_t n_blocks, const h3_time_weights* tw,
                          const float* sigma3, float* mod, float* mod_final, void* stream);

/* The denoising loop on the device (h3.c README: Euler transitions, video and
 * audio on independent schedules, a terminal zero after the last pass).  For
 * each pass k < n_steps: the rows in from the current latents, the
 * modulation tables of sigmas[k], the n_blocks-block forward and heads, then
 *   video_latent += (sigmas[k+1][2] - sigmas[k][2]) vel_video
 *   audio_latent += (sigmas[k+1][1] - sigmas[k][1]) vel_audio
 * sigmas: HOST array [n_steps + 1][3] (text, audio, video); the latents
 * (fp32 [n_video][c_video], [n_audio][c_audio], device) are updated in place.
 * ws: h3_denoise_workspace_bytes(shape, tile_start, n_blocks) bytes. */
size_t h3_denoise_workspace_bytes(const h3_shape* shape, const int32_t* tile_start,
                                  int32_t n_blocks);
int h3_denoise(const h3_shape* shape, int32_t n_blocks, int32_t n_steps,
               const int32_t* tile_start, const h3_block_weights* blocks,
               const h3_head_weights* heads, const h3_rows_in_weights* rows_w,
               const h3_time_weights* tw, const float* sigmas, const float* rope,
               const h3_bf16* text_rows, float* video_latent, float* audio_latent, void* ws,
               size_t ws_bytes, void* stream);

/* Token reduction (h3.c README, implementation notes: --token-reduction):
 * blocks [reduce_at, restore_at) run on a pooled stream in which pairs of
 * horizontally adjacent video tokens are one token; text and audio rows pass
 * as they are.  At reduce_at the pooled token of pair (a, b) is
 * bf((x[a] + x[b]) / 2) (x[a] for a single token) and the full stream is
 * kept; at restore_at each token of a pair returns as
 * bf(kept + (pooled now - pooled at reduce_at)), a single token as its
 * pooled value, and the remaining blocks run at full resolution.
 *   reduced:    the pooled stream's shape (n_video = number of pooled tokens,
 *               n_tiles / n_prefix_tiles of its tile map; every other field as
 *               in the full shape)
 *   tile_start: HOST [reduced->n_tiles + 1], its tile map
 *   pairs:      DEVICE int32 [reduced->n_video][2]: the full video rows (0-based
 *               within the video segment) of each pooled token, in the pooled
 *               stream's row order; second entry -1 for a single token.
 *               Entries outside [0, n_video) are skipped by the kernels.
 *   rope:       DEVICE fp32 [reduced rows][d/2][2] or NULL: the pooled stream's
 *               rotary table
 *   0 <= reduce_at <= restore_at <= n_blocks (equal: no reduction). */
typedef struct {
  const h3_shape* reduced;
  const int32_t* tile_start;
  const int32_t* pairs;
  const float* rope;
  int32_t reduce_at, restore_at;
} h3_token_reduction;

/* h3_dit_forward with token reduction.  Workspace:
 * h3_dit_forward_tr_workspace_bytes(shape, tile_start, tr) bytes. */
size_t h3_dit_forward_tr_workspace_bytes(const h3_shape* shape, const int32_t* tile_start,
                                         const h3_token_reduction* tr);
int h3_dit_forward_tr(const h3_shape* shape, int32_t n_blocks, const int32_t* tile_start,
                      const h3_token_reduction* tr, const h3_block_weights* blocks,
                      const h3_head_weights* heads, const float* mod, const float* mod_final,
                      const float* rope, const h3_bf16* x_in, float* vel_video,
                      float* vel_audio, void* ws, size_t ws_bytes, void* stream);

/* int8 variant (h3.c README, implementation notes: the int8 QKV,
 * attention-output and MLP products; dynamic activation quantization,
 * per-output-channel weight scales, the quantization folded into the gated
 * AdaLN).  Codes are symmetric: per row (or group of columns) with
 * m = max |x|: code = clamp(rint(x * (127/m)), -127, 127), scale = m / 127,
 * fp32 arithmetic with IEEE division; zero rows have codes 0 and scale 0. */

/* Codes of a bf16 matrix x [rows][cols] per row (group = 0) or per group of
 * `group` consecutive columns: q int8 [rows][cols], scale fp32
 * [rows][cols / group] (or [rows]).  Device pointers; cols and group multiples
 * of 8, group <= 32768 and dividing cols.  Weights are quantized once with this
 * call (per output channel: group = 0). */
int h3_quantize_rows(const h3_bf16* x, int32_t rows, int32_t cols, int32_t group, int8_t* q,
                     float* scale, void* stream);

/* One block's int8 weights: codes and per-output-row scales of the four
 * products (h3_quantize_rows with group 0), the other tensors as in
 * h3_block_weights. */
typedef struct {
  const int8_t* w_qkv; const float* s_qkv; const h3_bf16* b_qkv;
  const h3_bf16 *q_gain, *k_gain;
  const int8_t* w_o;   const float* s_o;   const h3_bf16* b_o;
  const int8_t* w_fc1; const float* s_fc1; const h3_bf16* b_fc1;
  const int8_t* w_fc2; const float* s_fc2; const h3_bf16* b_fc2;
} h3_block_weights_i8;

/* h3_dit_forward with int8 products: each block's QKV, out-projection and
 * FC1 inputs are quantized per row (the norm outputs inside the fused norm
 * kernel), the FC2 input per row (fc2_group = 0) or per row and 1,024
 * channels (fc2_group = 1024, the pages' default; needs an FFN width that is
 * a multiple of 1,024); the products are exact int32 sums scaled by the row
 * (group) and column scales, all else as in h3_dit_forward (attention in
 * bf16).  The hidden, attention and FFN widths (K of the products) must be
 * multiples of 256.  Workspace: H3_WS_DIT_I8. */
int h3_dit_forward_i8(const h3_shape* shape, int32_t n_blocks, const int32_t* tile_start,
                      const h3_block_weights_i8* blocks, const h3_head_weights* heads,
                      const float* mod, const float* mod_final, const float* rope,
                      const h3_bf16* x_in, float* vel_video, float* vel_audio,
                      int32_t fc2_group, void* ws, size_t ws_bytes, void* stream);

/* Kernel-time accounting for diagnostics: while enabled, each kernel launch
 * of the library is bracketed by HIP events on its stream.  h3_prof_read
 * synchronizes those events and returns, for kernel class `cls` (H3_K_*),
 * the launch count and the summed duration in milliseconds; it then forgets
 * the events it has read.  Not thread-safe; for benchmarks. */
enum { H3_K_NORM = 0, H3_K_GEMM_QKV, H3_K_HEADS, H3_K_ROUTE, H3_K_ATTN, H3_K_GEMM_O,
       H3_K_GEMM_FC1, H3_K_GEMM_FC2, H3_K_FINAL, H3_K_TABLES, H3_K_ROWS_IN, H3_K_TIME,
       H3_K_EULER, H3_K_TOKENS, H3_K_QUANT, H3_K_COUNT };
int h3_prof_enable(int on);
int h3_prof_read(int32_t cls, int64_t* launches, double* total_ms);
const char* h3_prof_kernel_name(int32_t cls);

/* Calibration of the matrix cores (measurement only, not a step of the
 * method): n_blocks workgroups of 4 waves, each wave running iters rounds of
 * 16 independent bf16 products v_mfma_f32_16x16x32_bf16 (16,384 FLOP each) on
 * operands read from `operands` (device memory holding random bf16 data,
 * operand_bytes >= 16 and a multiple of 16), so one call performs
 * n_blocks * 4 * iters * 16 * 16,384 FLOP; the caller times it on `stream`.
 * Under such a load the clock settles below the one the published peak is
 * quoted at; the result is the rate the products can reach here.  sink:
 * device, 256 floats (written only if the sums hit a value they cannot
 * reach).  H3_EINVAL on null pointers or sizes out of range. */
int h3_calibrate_mfma(const void* operands, size_t operand_bytes, int32_t n_blocks,
                      int32_t iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* H3_H */
