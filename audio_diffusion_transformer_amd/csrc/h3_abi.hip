// C ABI of the library: argument validation, the workspace plan, and the
// per-block launch sequence on the caller's stream.
//
// Block order (TensorFold PR #949, "What it adds": block.zig), each step one
// kernel of this library:
//   1 modnorm   x  -> n1                     (shift1, scale1)
//   2 gemm      n1 . Wqkv^T + b -> y        (bias, bf16)
//   3 heads     y  -> q~, k~ (norm, gain, rope), v^T, fp32 tile means
//   4 route     tile scores, top-k, pooled branch
//   5 attn      routed / dense attention -> attn [R][H]
//   6 gemm      x1 = bf(x + gate1 * bf(attn . Wo^T + bo))
//   7 modnorm   x1 -> n2                     (shift2, scale2)
//   8 gemm      h  = bf(gelu(n2 . W1^T + b1))
//   9 gemm      x2 = bf(x1 + gate2 * bf(h . W2^T + b2))
// Activation arenas are reused as in the h3.c README's notes on activation
// lifetimes: one [R][H] buffer holds n1 then n2, one [R][max(3H, F)] buffer
// holds the QKV output then the MLP activations.
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>

#include <mutex>
#include <string>
#include <vector>

#include <algorithm>
#include <functional>

#include "common.h"
#include "internal.h"

namespace h3 {

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Rows of a call: far above any product the GEMMs accept (M K < 2^31), low
// enough that every row index and padded row count stays an int.
constexpr int kMaxRows = 1 << 26;

// Guard bands, a debugging aid: with H3_WS_GUARD=<n> in the environment every
// region of a workspace is followed by n bytes (rounded up to 256) that no
// kernel touches, so a caller that fills the workspace with a pattern can
// find a stray write past a region as a changed band.  Unset, or 0: regions
// are packed.  Read at every planning call.
size_t ws_guard() {
  const char* e = getenv("H3_WS_GUARD");
  if (e == nullptr) return 0;
  const long v = strtol(e, nullptr, 10);
  return v > 0 && v <= (1l << 24) ? align256((size_t)v) : 0;
}

struct Plan {
  h3_shape s;
  int R, P, H, D, F, nh, nT, npt, nQ, nsel, Rp, n_chunks, n_prefix_chunks, nqb, nqb_dense;
  int max_list;  // longest video key list in 32-row chunks: prefix + the nsel largest tiles
  int A;      // attention width n_heads * head_dim
  int parts;  // blocks per head in the QKV product: 3, or 4 with the routing gate
  int F1;     // FC1 output width: F (GELU) or 2F (SwiGLU)
  std::vector<int> tstart, tpstart, chunk_valid, qblocks;
  h3_ws_layout lay;
  size_t off_tstart, off_tpstart, off_chunk, off_qb;
  size_t partial_bytes = 0;
};

int make_plan(const h3_shape* s, const int32_t* tile_start, int which, Plan& p) {
  if (!s) return fail(H3_EINVAL, "shape is NULL");
  if (!tile_start) return fail(H3_EINVAL, "tile_start is NULL");
  if (which < H3_WS_BLOCK || which > H3_WS_DIT_I8)
    return fail(H3_EINVAL, "bad workspace kind %d", which);
  p.s = *s;
  if (s->n_text < 0 || s->n_audio < 0 || s->n_video < 0)
    return fail(H3_EINVAL, "negative row count");
  // (summed in 64 bits: three int32 counts can overflow an int)
  if ((long long)s->n_text + s->n_audio + s->n_video > kMaxRows)
    return fail(H3_EUNSUPPORTED, "more than %d rows", kMaxRows);
  p.R = s->n_text + s->n_audio + s->n_video;
  p.P = s->n_text + s->n_audio;
  if (p.R < 1) return fail(H3_EINVAL, "no rows");
  if (s->n_heads < 1 || s->head_dim < 1) return fail(H3_EINVAL, "bad heads");
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(H3_EUNSUPPORTED, "head_dim %d not in {64, 128}", s->head_dim);
  p.D = s->head_dim;
  p.nh = s->n_heads;
  p.A = p.nh * p.D;
  p.H = s->hidden;
  if (s->mlp != H3_MLP_GELU && s->mlp != H3_MLP_SWIGLU) return fail(H3_EINVAL, "bad mlp %d", s->mlp);
  if (s->gate != 0 && s->gate != 1) return fail(H3_EINVAL, "gate must be 0 or 1");
  p.parts = s->gate ? 4 : 3;
  p.F = s->ffn;
  p.F1 = s->mlp == H3_MLP_SWIGLU ? 2 * s->ffn : s->ffn;
  if (which != H3_WS_ATTN) {
    if (p.H % 256 != 0 || p.H > 8192)
      return fail(H3_EUNSUPPORTED, "hidden %d must be a multiple of 256 and <= 8192", p.H);
    if (s->ffn < 128 || s->ffn % 128 != 0 || p.F1 % 256 != 0)
      return fail(H3_EUNSUPPORTED, "ffn %d: the FC1 width must be a positive multiple of 256", s->ffn);
    if ((p.parts * p.A) % 256 != 0 || p.A % 128 != 0)
      return fail(H3_EUNSUPPORTED, "attention width %d: (3 + gate) * width must be a multiple of 256", p.A);
    if (!gemm_shape_ok(p.R, p.parts * p.A, p.H) || !gemm_shape_ok(p.R, p.H, p.A) ||
        !gemm_shape_ok(p.R, p.F1, p.H) || !gemm_shape_ok(p.R, p.H, s->ffn))
      return fail(H3_EUNSUPPORTED, "rows x width too large for the GEMM (R*F must stay below 2^31)");
    if (which == H3_WS_DIT_I8 &&
        (!gemm_i8_shape_ok(p.R, p.parts * p.A, p.H) || !gemm_i8_shape_ok(p.R, p.H, p.A) ||
         !gemm_i8_shape_ok(p.R, p.F1, p.H) || !gemm_i8_shape_ok(p.R, p.H, s->ffn)))
      return fail(H3_EUNSUPPORTED, "int8 products need hidden, attention and FFN widths that are "
                                   "multiples of 256");
  }
  if (!(s->norm_eps >= 0.f)) return fail(H3_EINVAL, "norm_eps must be >= 0");
  p.nT = s->n_tiles;
  p.npt = s->n_prefix_tiles;
  if (p.nT < 1 || p.npt < 0 || p.npt > p.nT) return fail(H3_EINVAL, "bad tile counts");
  if (p.nT > 2048) return fail(H3_EUNSUPPORTED, "n_tiles %d > 2048", p.nT);
  p.tstart.assign(tile_start, tile_start + p.nT + 1);
  if (p.tstart[0] != 0 || p.tstart[p.nT] != p.R)
    return fail(H3_EINVAL, "tile map must start at 0 and end at R=%d", p.R);
  for (int t = 0; t < p.nT; ++t)
    if (p.tstart[t + 1] <= p.tstart[t]) return fail(H3_EINVAL, "tile map not increasing at %d", t);
  if (p.tstart[p.npt] != p.P)
    return fail(H3_EINVAL, "prefix tiles end at row %d, prefix has %d rows", p.tstart[p.npt], p.P);
  {
    // the text/audio boundary must be a tile edge too: a tile holding rows of
    // both segments would mix them in its means
    bool edge = false;
    for (int t = 0; t <= p.npt; ++t) edge = edge || p.tstart[t] == s->n_text;
    if (!edge) return fail(H3_EINVAL, "no tile edge at the text/audio boundary (row %d)", s->n_text);
  }
  p.nQ = p.nT - p.npt;
  if (p.nQ > 0 && s->top_k < 1) return fail(H3_EINVAL, "top_k must be >= 1");
  p.nsel = p.nQ > 0 ? (s->top_k < p.nQ ? s->top_k : p.nQ) : 0;
  if (!route_shape_ok(p.nT, p.nsel)) return fail(H3_EUNSUPPORTED, "top_k too large");

  p.tpstart.resize(p.nT + 1);
  p.tpstart[0] = 0;
  for (int t = 0; t < p.nT; ++t) {
    const int len = p.tstart[t + 1] - p.tstart[t];
    p.tpstart[t + 1] = p.tpstart[t] + ((len + 31) / 32) * 32;
  }
  p.Rp = p.tpstart[p.nT];
  p.n_chunks = p.Rp / 32;
  p.n_prefix_chunks = p.tpstart[p.npt] / 32;
  {
    std::vector<int> vc;
    for (int t = p.npt; t < p.nT; ++t) vc.push_back((p.tpstart[t + 1] - p.tpstart[t]) / 32);
    std::sort(vc.begin(), vc.end(), std::greater<int>());
    p.max_list = p.n_prefix_chunks;
    for (int e = 0; e < p.nsel && e < (int)vc.size(); ++e) p.max_list += vc[e];
  }
  if (!attn_shape_ok(p.n_chunks, p.nsel)) return fail(H3_EUNSUPPORTED, "too many key chunks");
  p.chunk_valid.assign(p.n_chunks, 0);
  for (int t = 0; t < p.nT; ++t) {
    const int len = p.tstart[t + 1] - p.tstart[t];
    for (int o = 0; o < len; o += 32)
      p.chunk_valid[(p.tpstart[t] + o) / 32] = len - o < 32 ? len - o : 32;
  }
  p.qblocks.clear();
  for (int pass = 0; pass < 2; ++pass) {
    for (int t = pass == 0 ? 0 : p.npt; t < (pass == 0 ? p.npt : p.nT); ++t) {
      const int len = p.tstart[t + 1] - p.tstart[t];
      for (int o = 0; o < len; o += 64) {
        p.qblocks.push_back(t);
        p.qblocks.push_back(p.tpstart[t] + o);
        p.qblocks.push_back(len - o < 64 ? len - o : 64);
        p.qblocks.push_back(p.tstart[t] + o);
      }
    }
    if (pass == 0) p.nqb_dense = (int)p.qblocks.size() / 4;
  }
  p.nqb = (int)p.qblocks.size() / 4;

  // ---- workspace layout ----
  h3_ws_layout& L = p.lay;
  L = h3_ws_layout{};
  size_t off = 0;
  const size_t guard = ws_guard();
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes) + guard;
    return o;
  };
  const size_t bf = 2, f4 = 4;
  L.tables = off;
  p.off_tstart = take((size_t)(p.nT + 1) * 4);
  p.off_tpstart = take((size_t)(p.nT + 1) * 4);
  p.off_chunk = take((size_t)p.n_chunks * 4);
  p.off_qb = take((size_t)p.nqb * 16);
  const size_t R = p.R, H = p.H, A = p.A;
  if (which != H3_WS_ATTN) {
    const size_t ywidth = (size_t)p.parts * p.A;  // y (QKV product), then the MLP hidden h
    L.norm = take(R * H * bf);
    L.big = take(R * (ywidth > (size_t)p.F ? ywidth : (size_t)p.F) * bf);
  }
  L.q = take((size_t)p.nh * p.Rp * p.D * bf);
  L.k = take((size_t)p.nh * p.Rp * p.D * bf);
  L.vt = take((size_t)p.nh * p.Rp * p.D * bf);
  L.qbar = take((size_t)p.nh * (p.nQ > 0 ? p.nQ : 1) * p.D * f4);
  L.kbar = take((size_t)p.nh * p.nT * p.D * f4);
  L.vbar = take((size_t)p.nh * p.nT * p.D * f4);
  L.scores = take((size_t)p.nh * (p.nQ > 0 ? p.nQ : 1) * p.nT * f4);
  L.sel = take((size_t)p.nh * (p.nQ > 0 ? p.nQ : 1) * (p.nsel > 0 ? p.nsel : 1) * 4);
  L.pooled = take((size_t)p.nh * (p.nQ > 0 ? p.nQ : 1) * p.D * f4);
  if (which != H3_WS_ATTN) {
    L.attn = take(R * A * bf);
    L.x1 = take(R * H * bf);
  }
  if (which == H3_WS_DIT || which == H3_WS_DIT_I8) {
    L.xa = take(R * H * bf);
    L.xb = take(R * H * bf);
  }
  if (which == H3_WS_DIT_I8) {
    size_t w8 = H > A ? H : A;
    if ((size_t)p.F > w8) w8 = p.F;
    L.q8 = take(R * w8);
    // row scales, or one per row and 1,024 channels of the FC2 input
    const size_t ng = p.F % kFc2Group == 0 ? (size_t)(p.F / kFc2Group) : 1;
    L.qscale = take(R * (ng > 1 ? ng : 1) * f4);
  }
  if (which != H3_WS_ATTN) {  // the products' split-K tails
    const bool i8 = which == H3_WS_DIT_I8;
    const int dims[4][2] = {{p.parts * p.A, p.H}, {p.H, p.A}, {p.F1, p.H}, {p.H, p.F}};
    size_t pb = 0;
    for (const auto& d : dims) {
      const size_t b = gemm_partial_bytes(p.R, d[0], d[1], i8);
      if (b > pb) pb = b;
    }
    p.partial_bytes = pb;
    if (pb) L.partial = take(pb);
  }
  L.total = off;
  L.padded_rows = p.Rp;
  L.n_query_tiles = p.nQ;
  L.n_sel = p.nsel;
  return H3_OK;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int check_ws(const Plan& p, void* ws, size_t ws_bytes) {
  if (!ws) return fail(H3_EINVAL, "workspace is NULL");
  if (((uintptr_t)ws & 255) != 0) return fail(H3_EINVAL, "workspace must be 256-byte aligned");
  if (ws_bytes < p.lay.total)
    return fail(H3_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, p.lay.total);
  return H3_OK;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15) == 0; }

#define H3_TRY(expr)                                                        \
  do {                                                                      \
    hipError_t e_ = (expr);                                                 \
    if (e_ != hipSuccess) return fail(H3_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

int upload_tables(const Plan& p, void* ws, hipStream_t st) {
  prof_begin(H3_K_TABLES, st);
  H3_TRY(launch_poke(at<int>(ws, p.off_tstart), p.tstart.data(), (int)p.tstart.size(), st));
  H3_TRY(launch_poke(at<int>(ws, p.off_tpstart), p.tpstart.data(), (int)p.tpstart.size(), st));
  H3_TRY(launch_poke(at<int>(ws, p.off_chunk), p.chunk_valid.data(), (int)p.chunk_valid.size(), st));
  H3_TRY(launch_poke(at<int>(ws, p.off_qb), p.qblocks.data(), (int)p.qblocks.size(), st));
  prof_end(H3_K_TABLES, st);
  return H3_OK;
}

HeadsArgs heads_args(const Plan& p, void* ws) {
  HeadsArgs a{};
  a.q = at<bf16_t>(ws, p.lay.q);
  a.k = at<bf16_t>(ws, p.lay.k);
  a.vt = at<bf16_t>(ws, p.lay.vt);
  a.qbar = at<float>(ws, p.lay.qbar);
  a.kbar = at<float>(ws, p.lay.kbar);
  a.vbar = at<float>(ws, p.lay.vbar);
  a.tstart = at<int>(ws, p.off_tstart);
  a.tpstart = at<int>(ws, p.off_tpstart);
  a.R = p.R;
  a.Rp = p.Rp;
  a.nh = p.nh;
  a.nT = p.nT;
  a.npt = p.npt;
  a.parts = p.parts;
  a.ystride = p.parts * p.A;
  a.eps = p.s.norm_eps;
  return a;
}

// gate: null, or the routing gate at gate[r * gate_stride + h * gate_hstride + c]
int run_attention(const Plan& p, void* ws, int32_t* sel_out, float* scores_out, bf16_t* out,
                  const bf16_t* gate, int gate_stride, int gate_hstride, hipStream_t st) {
  int* sel = sel_out ? sel_out : at<int>(ws, p.lay.sel);
  float* scores = scores_out ? scores_out : at<float>(ws, p.lay.scores);
  if (p.nQ > 0) {
    RouteArgs r{};
    r.qbar = at<float>(ws, p.lay.qbar);
    r.kbar = at<float>(ws, p.lay.kbar);
    r.vbar = at<float>(ws, p.lay.vbar);
    r.scores = scores;
    r.sel = sel;
    r.pooled = at<float>(ws, p.lay.pooled);
    r.nh = p.nh;
    r.nQ = p.nQ;
    r.nT = p.nT;
    r.npt = p.npt;
    r.top_k = p.s.top_k;
    r.nsel = p.nsel;
    r.use_pooled = p.s.pooled ? 1 : 0;
    prof_begin(H3_K_ROUTE, st);
    H3_TRY(launch_route(p.D, r, st));
    prof_end(H3_K_ROUTE, st);
  }
  AttnArgs a{};
  a.q = at<bf16_t>(ws, p.lay.q);
  a.k = at<bf16_t>(ws, p.lay.k);
  a.vt = at<bf16_t>(ws, p.lay.vt);
  a.sel = sel;
  a.scores = scores;
  a.pooled = p.s.pooled ? at<float>(ws, p.lay.pooled) : nullptr;
  a.tpstart = at<int>(ws, p.off_tpstart);
  a.chunk_valid = at<int>(ws, p.off_chunk);
  a.qblocks = at<int4>(ws, p.off_qb);
  a.out = out;
  a.gate = gate;
  a.gate_stride = gate_stride;
  a.gate_hstride = gate_hstride;
  a.nh = p.nh;
  a.Rp = p.Rp;
  a.A = p.A;
  a.nT = p.nT;
  a.npt = p.npt;
  a.nQ = p.nQ;
  a.nsel = p.nsel;
  a.nqb = p.nqb;
  a.nqb_dense = p.nqb_dense;
  a.n_prefix_chunks = p.n_prefix_chunks;
  a.n_chunks = p.n_chunks;
  a.max_list = p.max_list;
  prof_begin(H3_K_ATTN, st);
  H3_TRY(launch_attn(p.D, a, st));
  prof_end(H3_K_ATTN, st);
  return H3_OK;
}

int check_block_weights(const h3_block_weights* w, int l) {
  if (!w) return fail(H3_EINVAL, "block %d weights NULL", l);
  const void* ptrs[] = {w->w_qkv, w->b_qkv, w->q_gain, w->k_gain, w->w_o,
                        w->b_o,   w->w_fc1, w->b_fc1,  w->w_fc2,  w->b_fc2};
  for (const void* q : ptrs) {
    if (!q) return fail(H3_EINVAL, "block %d: a weight pointer is NULL", l);
    if (!aligned16(q)) return fail(H3_EINVAL, "block %d: a weight pointer is not 16-byte aligned", l);
  }
  return H3_OK;
}

// A product's epilogue arguments with the plan's split-K partial region.
GemmEpi gemm_epi(const Plan& p, void* ws) {
  GemmEpi e{};
  if (p.partial_bytes) {
    e.partial = at<void>(ws, p.lay.partial);
    e.partial_bytes = p.partial_bytes;
  }
  return e;
}

// Steps 1-9 of one block; tables already uploaded.
int run_block(const Plan& p, void* ws, const h3_block_weights* w, const float* mod,
              const float* rope, const bf16_t* x_in, bf16_t* x_out, hipStream_t st) {
  const int R = p.R, H = p.H, F = p.F, A = p.A;
  const int nt = p.s.n_text, np_ = p.P;
  bf16_t* norm = at<bf16_t>(ws, p.lay.norm);
  bf16_t* big = at<bf16_t>(ws, p.lay.big);
  bf16_t* attn = at<bf16_t>(ws, p.lay.attn);
  bf16_t* x1 = at<bf16_t>(ws, p.lay.x1);
  const int ms = 6 * H;  // floats between segments of mod

  prof_begin(H3_K_NORM, st);
  H3_TRY(launch_modnorm(x_in, norm, 0, mod + 0 * H, mod + 1 * H, ms, 0, R, H, nt, np_,
                        p.s.norm_eps, st));
  prof_end(H3_K_NORM, st);

  GemmEpi e = gemm_epi(p, ws);
  e.bias = w->b_qkv;
  e.out = big;
  e.n_text = nt;
  e.n_prefix = np_;
  prof_begin(H3_K_GEMM_QKV, st);
  H3_TRY(launch_gemm(EPI_BIAS, norm, w->w_qkv, R, p.parts * A, H, e, st));
  prof_end(H3_K_GEMM_QKV, st);

  HeadsArgs ha = heads_args(p, ws);
  ha.y = big;
  ha.q_gain = w->q_gain;
  ha.k_gain = w->k_gain;
  ha.rope = rope;
  prof_begin(H3_K_HEADS, st);
  H3_TRY(launch_heads(HEADS_QKV, p.D, ha, st));
  prof_end(H3_K_HEADS, st);

  // the routing gate: the fourth block of each head's rows of y
  const bf16_t* gate = p.s.gate ? big + 3 * p.D : nullptr;
  int rc = run_attention(p, ws, nullptr, nullptr, attn, gate, p.parts * A, p.parts * p.D, st);
  if (rc) return rc;

  e = gemm_epi(p, ws);
  e.bias = w->b_o;
  e.out = x1;
  e.res = x_in;
  e.gate = mod + 2 * H;
  e.gate_seg_stride = ms;
  e.n_text = nt;
  e.n_prefix = np_;
  prof_begin(H3_K_GEMM_O, st);
  H3_TRY(launch_gemm(EPI_BIAS_RESGATE, attn, w->w_o, R, H, A, e, st));
  prof_end(H3_K_GEMM_O, st);

  prof_begin(H3_K_NORM, st);
  H3_TRY(launch_modnorm(x1, norm, 0, mod + 3 * H, mod + 4 * H, ms, 0, R, H, nt, np_,
                        p.s.norm_eps, st));
  prof_end(H3_K_NORM, st);

  e = gemm_epi(p, ws);
  e.bias = w->b_fc1;
  e.out = big;
  prof_begin(H3_K_GEMM_FC1, st);
  H3_TRY(launch_gemm(p.s.mlp == H3_MLP_SWIGLU ? EPI_BIAS_SWIGLU : EPI_BIAS_GELU, norm, w->w_fc1,
                     R, p.F1, H, e, st));
  prof_end(H3_K_GEMM_FC1, st);

  e = gemm_epi(p, ws);
  e.bias = w->b_fc2;
  e.out = x_out;
  e.res = x1;
  e.gate = mod + 5 * H;
  e.gate_seg_stride = ms;
  e.n_text = nt;
  e.n_prefix = np_;
  prof_begin(H3_K_GEMM_FC2, st);
  H3_TRY(launch_gemm(EPI_BIAS_RESGATE, big, w->w_fc2, R, H, F, e, st));
  prof_end(H3_K_GEMM_FC2, st);
  return H3_OK;
}

int check_block_weights_i8(const h3_block_weights_i8* w, int l) {
  if (!w) return fail(H3_EINVAL, "block %d weights NULL", l);
  const void* ptrs[] = {w->w_qkv, w->s_qkv, w->b_qkv, w->q_gain, w->k_gain, w->w_o, w->s_o,
                        w->b_o, w->w_fc1, w->s_fc1, w->b_fc1, w->w_fc2, w->s_fc2, w->b_fc2};
  for (const void* q : ptrs) {
    if (!q) return fail(H3_EINVAL, "block %d: a weight pointer is NULL", l);
    if (!aligned16(q)) return fail(H3_EINVAL, "block %d: a weight pointer is not 16-byte aligned", l);
  }
  return H3_OK;
}

// The block with int8 products: the norms emit row codes, the attention output
// and the MLP hidden are quantized per row before their products.
int run_block_i8(const Plan& p, void* ws, const h3_block_weights_i8* w, const float* mod,
                 const float* rope, const bf16_t* x_in, bf16_t* x_out, bool grouped,
                 hipStream_t st) {
  const int R = p.R, H = p.H, F = p.F, A = p.A;
  const int nt = p.s.n_text, np_ = p.P;
  bf16_t* big = at<bf16_t>(ws, p.lay.big);
  bf16_t* attn = at<bf16_t>(ws, p.lay.attn);
  bf16_t* x1 = at<bf16_t>(ws, p.lay.x1);
  int8_t* q8 = at<int8_t>(ws, p.lay.q8);
  float* qs = at<float>(ws, p.lay.qscale);
  const int ms = 6 * H;

  prof_begin(H3_K_NORM, st);
  H3_TRY(launch_modnorm_q(x_in, mod + 0 * H, mod + 1 * H, ms, R, H, nt, np_, p.s.norm_eps, q8, qs,
                          nullptr, st));
  prof_end(H3_K_NORM, st);

  GemmEpi e = gemm_epi(p, ws);
  e.bias = w->b_qkv;
  e.out = big;
  e.n_text = nt;
  e.n_prefix = np_;
  e.a_scale = qs;
  e.b_scale = w->s_qkv;
  prof_begin(H3_K_GEMM_QKV, st);
  H3_TRY(launch_gemm_i8(EPI_BIAS, q8, w->w_qkv, R, p.parts * A, H, e, st));
  prof_end(H3_K_GEMM_QKV, st);

  HeadsArgs ha = heads_args(p, ws);
  ha.y = big;
  ha.q_gain = w->q_gain;
  ha.k_gain = w->k_gain;
  ha.rope = rope;
  prof_begin(H3_K_HEADS, st);
  H3_TRY(launch_heads(HEADS_QKV, p.D, ha, st));
  prof_end(H3_K_HEADS, st);

  const bf16_t* gate = p.s.gate ? big + 3 * p.D : nullptr;
  int rc = run_attention(p, ws, nullptr, nullptr, attn, gate, p.parts * A, p.parts * p.D, st);
  if (rc) return rc;

  prof_begin(H3_K_QUANT, st);
  H3_TRY(launch_quant_rows(attn, R, A, A, q8, qs, st));
  prof_end(H3_K_QUANT, st);
  e = gemm_epi(p, ws);
  e.bias = w->b_o;
  e.out = x1;
  e.res = x_in;
  e.gate = mod + 2 * H;
  e.gate_seg_stride = ms;
  e.n_text = nt;
  e.n_prefix = np_;
  e.a_scale = qs;
  e.b_scale = w->s_o;
  prof_begin(H3_K_GEMM_O, st);
  H3_TRY(launch_gemm_i8(EPI_BIAS_RESGATE, q8, w->w_o, R, H, A, e, st));
  prof_end(H3_K_GEMM_O, st);

  prof_begin(H3_K_NORM, st);
  H3_TRY(launch_modnorm_q(x1, mod + 3 * H, mod + 4 * H, ms, R, H, nt, np_, p.s.norm_eps, q8, qs,
                          nullptr, st));
  prof_end(H3_K_NORM, st);

  e = gemm_epi(p, ws);
  e.bias = w->b_fc1;
  e.out = big;
  e.a_scale = qs;
  e.b_scale = w->s_fc1;
  prof_begin(H3_K_GEMM_FC1, st);
  H3_TRY(launch_gemm_i8(p.s.mlp == H3_MLP_SWIGLU ? EPI_BIAS_SWIGLU : EPI_BIAS_GELU, q8, w->w_fc1,
                        R, p.F1, H, e, st));
  prof_end(H3_K_GEMM_FC1, st);

  // the FC2 input: per row, or one scale per 1,024 channels
  prof_begin(H3_K_QUANT, st);
  H3_TRY(launch_quant_rows(big, R, F, grouped ? kFc2Group : F, q8, qs, st));
  prof_end(H3_K_QUANT, st);
  e = gemm_epi(p, ws);
  e.bias = w->b_fc2;
  e.out = x_out;
  e.res = x1;
  e.gate = mod + 5 * H;
  e.gate_seg_stride = ms;
  e.n_text = nt;
  e.n_prefix = np_;
  e.a_scale = qs;
  e.b_scale = w->s_fc2;
  prof_begin(H3_K_GEMM_FC2, st);
  if (grouped)
    H3_TRY(launch_gemm_i8g_resgate(q8, w->w_fc2, R, H, F, kFc2Group, e, st));
  else
    H3_TRY(launch_gemm_i8(EPI_BIAS_RESGATE, q8, w->w_fc2, R, H, F, e, st));
  prof_end(H3_K_GEMM_FC2, st);
  return H3_OK;
}

int check_dit_args(int n_blocks, const h3_block_weights* blocks, const h3_head_weights* heads) {
  int rc;
  if (n_blocks < 0) return fail(H3_EINVAL, "n_blocks < 0");
  if (n_blocks > 0 && !blocks) return fail(H3_EINVAL, "blocks is NULL");
  for (int l = 0; l < n_blocks; ++l)
    if ((rc = check_block_weights(&blocks[l], l))) return rc;
  if (!heads || !heads->w_video || !heads->b_video || !heads->w_audio || !heads->b_audio)
    return fail(H3_EINVAL, "head weights are required");
  if (heads->c_video < 1 || heads->c_video > 256 || heads->c_audio < 1 || heads->c_audio > 256)
    return fail(H3_EINVAL, "head widths must be in [1, 256]");
  if (!aligned16(heads->w_video) || !aligned16(heads->w_audio))
    return fail(H3_EINVAL, "tensor pointers must be 16-byte aligned");
  return H3_OK;
}

// L blocks, then the final modulated norm of the audio and video rows and the heads.
int run_dit(const Plan& p, void* ws, int n_blocks, const h3_block_weights* blocks,
            const h3_head_weights* heads, const float* mod, const float* mod_final,
            const float* rope, const bf16_t* x_in, float* vel_video, float* vel_audio,
            hipStream_t st) {
  int rc;
  const bf16_t* x = x_in;
  bf16_t* xa = at<bf16_t>(ws, p.lay.xa);
  bf16_t* xb = at<bf16_t>(ws, p.lay.xb);
  const size_t mstride = (size_t)3 * 6 * p.H;
  for (int l = 0; l < n_blocks; ++l) {
    bf16_t* xo = (l & 1) ? xb : xa;
    if ((rc = run_block(p, ws, &blocks[l], mod + l * mstride, rope, x, xo, st))) return rc;
    x = xo;
  }
  bf16_t* z = at<bf16_t>(ws, p.lay.norm);
  const int H = p.H, nt = p.s.n_text;
  prof_begin(H3_K_FINAL, st);
  H3_TRY(launch_modnorm(x, z, nt, mod_final + 0 * H, mod_final + 1 * H, 2 * H, nt, p.R, H, nt,
                        p.P, p.s.norm_eps, st));
  H3_TRY(launch_out_head(z, p.s.n_audio, H, heads->w_audio, heads->b_audio, heads->c_audio,
                         vel_audio, st));
  H3_TRY(launch_out_head(z + (size_t)p.s.n_audio * H, p.s.n_video, H, heads->w_video,
                         heads->b_video, heads->c_video, vel_video, st));
  prof_end(H3_K_FINAL, st);
  return H3_OK;
}

int check_rows_in(const h3_shape* s, const h3_rows_in_weights* w, const h3_bf16* text,
                  const float* audio, const float* video, const h3_bf16* x) {
  if (!s) return fail(H3_EINVAL, "shape is NULL");
  if (s->n_text < 0 || s->n_audio < 0 || s->n_video < 0) return fail(H3_EINVAL, "negative row count");
  if ((long long)s->n_text + s->n_audio + s->n_video > kMaxRows)
    return fail(H3_EUNSUPPORTED, "more than %d rows", kMaxRows);
  if (s->hidden < 256 || s->hidden % 256 != 0 || s->hidden > 8192)
    return fail(H3_EUNSUPPORTED, "hidden %d must be a positive multiple of 256, <= 8192", s->hidden);
  if (!w) return fail(H3_EINVAL, "rows-in weights are required");
  if (w->c_video < 1 || w->c_video > 256 || w->c_audio < 1 || w->c_audio > 256)
    return fail(H3_EINVAL, "patch widths must be in [1, 256]");
  if ((s->n_video > 0 && (!video || !w->w_video || !w->b_video)) ||
      (s->n_audio > 0 && (!audio || !w->w_audio || !w->b_audio)) || (s->n_text > 0 && !text) || !x)
    return fail(H3_EINVAL, "rows-in inputs, weights and x are required");
  if ((text && !aligned16(text)) || !aligned16(x) || (w->b_video && !aligned16(w->b_video)) ||
      (w->b_audio && !aligned16(w->b_audio)))
    return fail(H3_EINVAL, "text rows, x and the biases must be 16-byte aligned");
  return H3_OK;
}

int run_rows_in(const h3_shape& s, const h3_rows_in_weights* w, const h3_bf16* text,
                const float* audio, const float* video, bf16_t* x, hipStream_t st) {
  RowsInArgs a{};
  a.text = text;
  a.audio = audio;
  a.video = video;
  a.w_audio = w->w_audio;
  a.b_audio = w->b_audio;
  a.w_video = w->w_video;
  a.b_video = w->b_video;
  a.x = x;
  a.n_text = s.n_text;
  a.n_audio = s.n_audio;
  a.n_video = s.n_video;
  a.H = s.hidden;
  a.c_audio = w->c_audio;
  a.c_video = w->c_video;
  prof_begin(H3_K_ROWS_IN, st);
  H3_TRY(launch_rows_in(a, st));
  prof_end(H3_K_ROWS_IN, st);
  return H3_OK;
}

int check_time_weights(const h3_time_weights* tw, int n_blocks) {
  if (!tw || !tw->w1 || !tw->b1 || !tw->w2 || !tw->b2 || !tw->w_final || !tw->b_final ||
      (n_blocks > 0 && (!tw->w_mod || !tw->b_mod || !tw->mod_table)))
    return fail(H3_EINVAL, "time weights are required");
  if (!aligned16(tw->w1) || !aligned16(tw->w2) || !aligned16(tw->w_final) ||
      (tw->w_mod && !aligned16(tw->w_mod)))
    return fail(H3_EINVAL, "time weight matrices must be 16-byte aligned");
  return H3_OK;
}

// scratch: 6H floats (h [3][H], then c [3][H])
int run_modulation(int H, int n_blocks, const h3_time_weights* tw, const float* sigma3,
                   float* mod, float* mod_final, float* scratch, hipStream_t st) {
  float* h = scratch;
  float* c = scratch + 3 * H;
  TimeGemvArgs a{};
  for (int i = 0; i < 3; ++i) a.sigma[i] = sigma3[i];
  prof_begin(H3_K_TIME, st);
  a.in = nullptr; a.w = tw->w1; a.b = tw->b1; a.table = nullptr; a.out = h;
  a.K = kTimeEmbedDim; a.N = H; a.n_blocks = 0; a.in_silu = 0; a.out_silu = 1;
  H3_TRY(launch_time_gemv(a, st));
  a.in = h; a.w = tw->w2; a.b = tw->b2; a.out = c; a.K = H; a.N = H; a.out_silu = 0;
  H3_TRY(launch_time_gemv(a, st));
  if (n_blocks > 0) {
    a.in = c; a.in_silu = 1; a.w = tw->w_mod; a.b = tw->b_mod; a.table = tw->mod_table;
    a.out = mod; a.N = 6 * H; a.n_blocks = n_blocks;
    H3_TRY(launch_time_gemv(a, st));
  }
  a.in = c; a.in_silu = 1; a.w = tw->w_final; a.b = tw->b_final; a.table = nullptr;
  a.out = mod_final; a.N = 2 * H; a.n_blocks = 0;
  H3_TRY(launch_time_gemv(a, st));
  prof_end(H3_K_TIME, st);
  return H3_OK;
}

struct DenoiseLayout {
  size_t x, mod, mod_final, vel_video, vel_audio, time, total;
};

// the forward's workspace, then the denoising loop's own buffers
DenoiseLayout denoise_layout(const Plan& p, int n_blocks) {
  DenoiseLayout d{};
  size_t off = p.lay.total;
  const size_t guard = ws_guard();
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes) + guard;
    return o;
  };
  d.x = take((size_t)p.R * p.H * 2);
  d.mod = take((size_t)(n_blocks > 0 ? n_blocks : 1) * 3 * 6 * p.H * 4);
  d.mod_final = take((size_t)3 * 2 * p.H * 4);
  d.vel_video = take((size_t)(p.s.n_video > 0 ? p.s.n_video : 1) * 256 * 4);
  d.vel_audio = take((size_t)(p.s.n_audio > 0 ? p.s.n_audio : 1) * 256 * 4);
  d.time = take((size_t)6 * p.H * 4);
  d.total = off;
  return d;
}

struct TrLayout {
  size_t orig, red, full, total;
};

// the larger of the two forward workspaces, then the kept video rows, the
// pooled stream as formed (the restore's baseline) and the restored stream
TrLayout tr_layout(const Plan& pf, const Plan& pr) {
  TrLayout t{};
  size_t off = align256(pf.lay.total > pr.lay.total ? pf.lay.total : pr.lay.total);
  const size_t guard = ws_guard();
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes) + guard;
    return o;
  };
  t.orig = take((size_t)(pf.s.n_video > 0 ? pf.s.n_video : 1) * pf.H * 2);
  t.red = take((size_t)pr.R * pr.H * 2);
  t.full = take((size_t)pf.R * pf.H * 2);
  t.total = off;
  return t;
}

int tr_plans(const h3_shape* shape, const int32_t* tile_start, const h3_token_reduction* tr,
             Plan& pf, Plan& pr) {
  int rc = make_plan(shape, tile_start, H3_WS_DIT, pf);
  if (rc) return rc;
  if (!tr || !tr->reduced || !tr->tile_start) return fail(H3_EINVAL, "token reduction is NULL");
  h3_shape rs = *tr->reduced;
  if (rs.n_text != shape->n_text || rs.n_audio != shape->n_audio || rs.hidden != shape->hidden ||
      rs.n_heads != shape->n_heads || rs.head_dim != shape->head_dim || rs.ffn != shape->ffn ||
      rs.top_k != shape->top_k || rs.pooled != shape->pooled || rs.norm_eps != shape->norm_eps ||
      rs.mlp != shape->mlp || rs.gate != shape->gate)
    return fail(H3_EINVAL, "the reduced shape may differ from the full one only in its video rows "
                           "and tile map");
  if (rs.n_video < 0 || rs.n_video > shape->n_video)
    return fail(H3_EINVAL, "the reduced stream has %d video rows, the full one %d", rs.n_video,
                shape->n_video);
  if ((rc = make_plan(&rs, tr->tile_start, H3_WS_DIT, pr))) return rc;
  return H3_OK;
}

// ---------------------------------------------------------------------------
// Kernel-time accounting
// ---------------------------------------------------------------------------
struct Prof {
  bool on = false;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<std::pair<int, std::pair<hipEvent_t, hipEvent_t>>> spans;
  std::vector<hipEvent_t> open;
  int open_cls = -1;
  int64_t launches[H3_K_COUNT] = {};
  double ms[H3_K_COUNT] = {};
} g_prof;

hipEvent_t prof_event() {
  if (g_prof.used == g_prof.pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_prof.pool.push_back(e);
  }
  return g_prof.pool[g_prof.used++];
}

hipEvent_t g_begin_ev = nullptr;

}  // namespace

void prof_begin(int cls, hipStream_t s) {
  if (!g_prof.on) return;
  g_begin_ev = prof_event();
  g_prof.open_cls = cls;
  if (g_begin_ev) (void)hipEventRecord(g_begin_ev, s);
}

void prof_end(int cls, hipStream_t s) {
  if (!g_prof.on || !g_begin_ev) return;
  hipEvent_t e = prof_event();
  if (!e) return;
  (void)hipEventRecord(e, s);
  g_prof.spans.push_back({cls, {g_begin_ev, e}});
  g_begin_ev = nullptr;
}

}  // namespace h3

using namespace h3;

// Scratch of h3_modulation_noalloc, for callers that cannot allocate: the time
// embedder's hidden and conditioning vectors of the three segments, [3][H] and
// [3][H] fp32, for H up to the library's hidden limit.  One copy per GPU, held
// until the process ends; every call on a GPU shares it.
constexpr int kModScratchHidden = 8192;
static __device__ __align__(256) float scratch[6 * kModScratchHidden];

namespace h3 {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices] = {};

// The device address of `scratch` on the current device, taken once per device
// with hipGetSymbolAddress (in host code the array's name is only a host-side
// stand-in, never a device address).
int scratch_on_current_device(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(H3_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(H3_EUNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(H3_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_dev[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_dev[dev];
  return H3_OK;
}

}  // namespace
}  // namespace h3

extern "C" {

int h3_abi_version(void) { return H3_ABI_VERSION; }

const char* h3_last_error(void) { return g_err.c_str(); }

size_t h3_workspace_bytes(const h3_shape* shape, const int32_t* tile_start, int32_t which) {
  Plan p;
  if (make_plan(shape, tile_start, which, p) != H3_OK) return 0;
  return p.lay.total;
}

int h3_workspace_layout(const h3_shape* shape, const int32_t* tile_start, int32_t which,
                        h3_ws_layout* out) {
  if (!out) return fail(H3_EINVAL, "out is NULL");
  Plan p;
  int rc = make_plan(shape, tile_start, which, p);
  if (rc) return rc;
  *out = p.lay;
  return H3_OK;
}

int h3_block_forward(const h3_shape* shape, const int32_t* tile_start, const h3_block_weights* w,
                     const float* mod, const float* rope, const h3_bf16* x_in, h3_bf16* x_out,
                     void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  int rc = make_plan(shape, tile_start, H3_WS_BLOCK, p);
  if (rc) return rc;
  if ((rc = check_ws(p, ws, ws_bytes))) return rc;
  if ((rc = check_block_weights(w, 0))) return rc;
  if (!mod || !x_in || !x_out) return fail(H3_EINVAL, "mod, x_in and x_out are required");
  if (!aligned16(mod) || !aligned16(x_in) || !aligned16(x_out) || (rope && !aligned16(rope)))
    return fail(H3_EINVAL, "tensor pointers must be 16-byte aligned");
  if (x_in == x_out) return fail(H3_EINVAL, "x_out must not alias x_in");
  hipStream_t st = (hipStream_t)stream;
  if ((rc = upload_tables(p, ws, st))) return rc;
  return run_block(p, ws, w, mod, rope, x_in, x_out, st);
}

int h3_dit_forward(const h3_shape* shape, int32_t n_blocks, const int32_t* tile_start,
                   const h3_block_weights* blocks, const h3_head_weights* heads,
                   const float* mod, const float* mod_final, const float* rope,
                   const h3_bf16* x_in, float* vel_video, float* vel_audio, void* ws,
                   size_t ws_bytes, void* stream) {
  Plan p;
  int rc = make_plan(shape, tile_start, H3_WS_DIT, p);
  if (rc) return rc;
  if ((rc = check_ws(p, ws, ws_bytes))) return rc;
  if ((rc = check_dit_args(n_blocks, blocks, heads))) return rc;
  if ((n_blocks > 0 && !mod) || !mod_final || !x_in)
    return fail(H3_EINVAL, "mod, mod_final and x_in are required");
  if ((p.s.n_video > 0 && !vel_video) || (p.s.n_audio > 0 && !vel_audio))
    return fail(H3_EINVAL, "velocity outputs are required");
  if (!aligned16(x_in) || (mod && !aligned16(mod)) || !aligned16(mod_final) ||
      (rope && !aligned16(rope)))
    return fail(H3_EINVAL, "tensor pointers must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  if ((rc = upload_tables(p, ws, st))) return rc;
  return run_dit(p, ws, n_blocks, blocks, heads, mod, mod_final, rope, x_in, vel_video,
                 vel_audio, st);
}

size_t h3_modulation_workspace_bytes(const h3_shape* shape) {
  if (!shape || shape->hidden < 256 || shape->hidden % 256 != 0 || shape->hidden > 8192) {
    fail(H3_EINVAL, "hidden must be a positive multiple of 256, at most 8192");
    return 0;
  }
  return align256((size_t)6 * shape->hidden * sizeof(float));
}

int h3_modulation(const h3_shape* shape, int32_t n_blocks, const h3_time_weights* tw,
                  const float* sigma3, float* mod, float* mod_final, void* ws, size_t ws_bytes,
                  void* stream) {
  const size_t need = h3_modulation_workspace_bytes(shape);
  if (need == 0) return H3_EINVAL;
  if (n_blocks < 0) return fail(H3_EINVAL, "n_blocks < 0");
  if (!sigma3) return fail(H3_EINVAL, "sigma3 is NULL");
  int rc;
  if ((rc = check_time_weights(tw, n_blocks))) return rc;
  if ((n_blocks > 0 && !mod) || !mod_final) return fail(H3_EINVAL, "mod and mod_final are required");
  if (!ws || ((uintptr_t)ws & 255) != 0) return fail(H3_EINVAL, "workspace must be 256-byte aligned");
  if (ws_bytes < need) return fail(H3_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  return run_modulation(shape->hidden, n_blocks, tw, sigma3, mod, mod_final,
                        static_cast<float*>(ws), (hipStream_t)stream);
}

int h3_modulation_noalloc(const h3_shape* shape, int32_t n_blocks, const h3_time_weights* tw,
                          const float* sigma3, float* mod, float* mod_final, void* stream) {
  if (!shape) return fail(H3_EINVAL, "shape is NULL");
  if (shape->hidden > kModScratchHidden)
    return fail(H3_EUNSUPPORTED, "hidden %d exceeds the static scratch (hidden <= %d)",
                shape->hidden, kModScratchHidden);
  if (h3_modulation_workspace_bytes(shape) == 0) return H3_EINVAL;
  if (n_blocks < 0) return fail(H3_EINVAL, "n_blocks < 0");
  if (!sigma3) return fail(H3_EINVAL, "sigma3 is NULL");
  int rc;
  if ((rc = check_time_weights(tw, n_blocks))) return rc;
  if ((n_blocks > 0 && !mod) || !mod_final) return fail(H3_EINVAL, "mod and mod_final are required");
  float* sc = nullptr;
  if ((rc = scratch_on_current_device(&sc))) return rc;
  return run_modulation(shape->hidden, n_blocks, tw, sigma3, mod, mod_final, sc,
                        (hipStream_t)stream);
}

int h3_rows_in(const h3_shape* shape, const h3_rows_in_weights* w, const h3_bf16* text_rows,
               const float* audio_patch, const float* video_patch, h3_bf16* x, void* stream) {
  int rc;
  if ((rc = check_rows_in(shape, w, text_rows, audio_patch, video_patch, x))) return rc;
  return run_rows_in(*shape, w, text_rows, audio_patch, video_patch, x, (hipStream_t)stream);
}

size_t h3_denoise_workspace_bytes(const h3_shape* shape, const int32_t* tile_start,
                                  int32_t n_blocks) {
  Plan p;
  if (make_plan(shape, tile_start, H3_WS_DIT, p) != H3_OK) return 0;
  if (n_blocks < 0) {
    fail(H3_EINVAL, "n_blocks < 0");
    return 0;
  }
  return denoise_layout(p, n_blocks).total;
}

int h3_denoise(const h3_shape* shape, int32_t n_blocks, int32_t n_steps,
               const int32_t* tile_start, const h3_block_weights* blocks,
               const h3_head_weights* heads, const h3_rows_in_weights* rows_w,
               const h3_time_weights* tw, const float* sigmas, const float* rope,
               const h3_bf16* text_rows, float* video_latent, float* audio_latent, void* ws,
               size_t ws_bytes, void* stream) {
  Plan p;
  int rc = make_plan(shape, tile_start, H3_WS_DIT, p);
  if (rc) return rc;
  if (n_steps < 0) return fail(H3_EINVAL, "n_steps < 0");
  if (!sigmas) return fail(H3_EINVAL, "sigmas is NULL");
  const DenoiseLayout dl = denoise_layout(p, n_blocks < 0 ? 0 : n_blocks);
  if (!ws) return fail(H3_EINVAL, "workspace is NULL");
  if (((uintptr_t)ws & 255) != 0) return fail(H3_EINVAL, "workspace must be 256-byte aligned");
  if (ws_bytes < dl.total)
    return fail(H3_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, dl.total);
  if ((rc = check_dit_args(n_blocks, blocks, heads))) return rc;
  if ((rc = check_time_weights(tw, n_blocks))) return rc;
  if (!rows_w || rows_w->c_video != heads->c_video || rows_w->c_audio != heads->c_audio)
    return fail(H3_EINVAL, "rows-in weights must match the head widths");
  bf16_t* x = at<bf16_t>(ws, dl.x);
  if ((rc = check_rows_in(shape, rows_w, text_rows, audio_latent, video_latent, x))) return rc;
  if (rope && !aligned16(rope)) return fail(H3_EINVAL, "tensor pointers must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  if ((rc = upload_tables(p, ws, st))) return rc;
  float* mod = at<float>(ws, dl.mod);
  float* mod_final = at<float>(ws, dl.mod_final);
  float* vv = at<float>(ws, dl.vel_video);
  float* va = at<float>(ws, dl.vel_audio);
  float* tscr = at<float>(ws, dl.time);
  for (int k = 0; k < n_steps; ++k) {
    const float* sg = sigmas + (size_t)3 * k;
    const float* sn = sigmas + (size_t)3 * (k + 1);
    if ((rc = run_rows_in(p.s, rows_w, text_rows, audio_latent, video_latent, x, st))) return rc;
    if ((rc = run_modulation(p.H, n_blocks, tw, sg, mod, mod_final, tscr, st))) return rc;
    if ((rc = run_dit(p, ws, n_blocks, blocks, heads, mod, mod_final, rope, x, vv, va, st)))
      return rc;
    prof_begin(H3_K_EULER, st);
    H3_TRY(launch_euler(video_latent, vv, (size_t)p.s.n_video * heads->c_video,
                        (double)sn[2] - (double)sg[2], st));
    H3_TRY(launch_euler(audio_latent, va, (size_t)p.s.n_audio * heads->c_audio,
                        (double)sn[1] - (double)sg[1], st));
    prof_end(H3_K_EULER, st);
  }
  return H3_OK;
}

size_t h3_dit_forward_tr_workspace_bytes(const h3_shape* shape, const int32_t* tile_start,
                                         const h3_token_reduction* tr) {
  Plan pf, pr;
  if (tr_plans(shape, tile_start, tr, pf, pr) != H3_OK) return 0;
  return tr_layout(pf, pr).total;
}

int h3_dit_forward_tr(const h3_shape* shape, int32_t n_blocks, const int32_t* tile_start,
                      const h3_token_reduction* tr, const h3_block_weights* blocks,
                      const h3_head_weights* heads, const float* mod, const float* mod_final,
                      const float* rope, const h3_bf16* x_in, float* vel_video,
                      float* vel_audio, void* ws, size_t ws_bytes, void* stream) {
  Plan pf, pr;
  int rc = tr_plans(shape, tile_start, tr, pf, pr);
  if (rc) return rc;
  const TrLayout tl = tr_layout(pf, pr);
  if (!ws) return fail(H3_EINVAL, "workspace is NULL");
  if (((uintptr_t)ws & 255) != 0) return fail(H3_EINVAL, "workspace must be 256-byte aligned");
  if (ws_bytes < tl.total)
    return fail(H3_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, tl.total);
  if ((rc = check_dit_args(n_blocks, blocks, heads))) return rc;
  const int r0 = tr->reduce_at, r1 = tr->restore_at;
  if (r0 < 0 || r0 > r1 || r1 > n_blocks)
    return fail(H3_EINVAL, "need 0 <= reduce_at <= restore_at <= n_blocks");
  if (r0 < r1 && !tr->pairs) return fail(H3_EINVAL, "pairs is NULL");
  if ((n_blocks > 0 && !mod) || !mod_final || !x_in)
    return fail(H3_EINVAL, "mod, mod_final and x_in are required");
  if ((pf.s.n_video > 0 && !vel_video) || (pf.s.n_audio > 0 && !vel_audio))
    return fail(H3_EINVAL, "velocity outputs are required");
  if (!aligned16(x_in) || (mod && !aligned16(mod)) || !aligned16(mod_final) ||
      (rope && !aligned16(rope)) || (tr->rope && !aligned16(tr->rope)))
    return fail(H3_EINVAL, "tensor pointers must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  const size_t mstride = (size_t)3 * 6 * pf.H;
  bf16_t* orig = at<bf16_t>(ws, tl.orig);
  bf16_t* red = at<bf16_t>(ws, tl.red);
  bf16_t* full = at<bf16_t>(ws, tl.full);
  TokenArgs ta{};
  ta.pairs = tr->pairs;
  ta.P = pf.P;
  ta.V = pf.s.n_video;
  ta.Vr = pr.s.n_video;
  ta.H = pf.H;
  // full resolution up to reduce_at (blocks alternate between the residual
  // buffers of the full plan)
  if ((rc = upload_tables(pf, ws, st))) return rc;
  const bf16_t* x = x_in;
  // (each block writes the residual buffer its input is not in)
  auto next = [&](const Plan& p, const bf16_t* in) {
    bf16_t* xa = at<bf16_t>(ws, p.lay.xa);
    return in == xa ? at<bf16_t>(ws, p.lay.xb) : xa;
  };
  for (int l = 0; l < r0; ++l) {
    bf16_t* xo = next(pf, x);
    if ((rc = run_block(pf, ws, &blocks[l], mod + l * mstride, rope, x, xo, st))) return rc;
    x = xo;
  }
  if (r0 < r1) {
    ta.x = x;
    ta.red = red;
    ta.orig = orig;
    prof_begin(H3_K_TOKENS, st);
    H3_TRY(launch_token_pool(ta, st));
    prof_end(H3_K_TOKENS, st);
    if ((rc = upload_tables(pr, ws, st))) return rc;
    x = red;
    for (int l = r0; l < r1; ++l) {
      bf16_t* xo = next(pr, x);
      if ((rc = run_block(pr, ws, &blocks[l], mod + l * mstride, tr->rope, x, xo, st))) return rc;
      x = xo;
    }
    ta.cur = x;
    ta.out = full;
    prof_begin(H3_K_TOKENS, st);
    H3_TRY(launch_token_restore(ta, st));
    prof_end(H3_K_TOKENS, st);
    if ((rc = upload_tables(pf, ws, st))) return rc;
    x = full;
  }
  for (int l = r1; l < n_blocks; ++l) {
    bf16_t* xo = next(pf, x);
    if ((rc = run_block(pf, ws, &blocks[l], mod + l * mstride, rope, x, xo, st))) return rc;
    x = xo;
  }
  return run_dit(pf, ws, 0, blocks, heads, mod, mod_final, rope, x, vel_video, vel_audio, st);
}

int h3_quantize_rows(const h3_bf16* x, int32_t rows, int32_t cols, int32_t group, int8_t* q,
                     float* scale, void* stream) {
  if (rows < 0) return fail(H3_EINVAL, "rows < 0");
  const int G = group == 0 ? cols : group;
  if (!quant_shape_ok(cols, G))
    return fail(H3_EINVAL, "cols %d and group %d: multiples of 8, group <= 32768 dividing cols",
                cols, group);
  // one wave per (row, group) must fit a launch of at most 2^31 - 1 workgroups of 4 waves
  if (rows > kMaxRows || (long long)rows * (cols / G) > 4LL * 0x7fffffffLL)
    return fail(H3_EUNSUPPORTED, "%d rows of %d groups: too many", rows, cols / G);
  if (rows > 0 && (!x || !q || !scale)) return fail(H3_EINVAL, "x, q and scale are required");
  if ((x && !aligned16(x)) || (q && ((uintptr_t)q & 7) != 0))
    return fail(H3_EINVAL, "x must be 16-byte and q 8-byte aligned");
  prof_begin(H3_K_QUANT, (hipStream_t)stream);
  H3_TRY(launch_quant_rows(x, rows, cols, G, q, scale, (hipStream_t)stream));
  prof_end(H3_K_QUANT, (hipStream_t)stream);
  return H3_OK;
}

int h3_dit_forward_i8(const h3_shape* shape, int32_t n_blocks, const int32_t* tile_start,
                      const h3_block_weights_i8* blocks, const h3_head_weights* heads,
                      const float* mod, const float* mod_final, const float* rope,
                      const h3_bf16* x_in, float* vel_video, float* vel_audio,
                      int32_t fc2_group, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  int rc = make_plan(shape, tile_start, H3_WS_DIT_I8, p);
  if (rc) return rc;
  if (fc2_group != 0 && fc2_group != kFc2Group)
    return fail(H3_EINVAL, "fc2_group must be 0 or %d", kFc2Group);
  if (fc2_group && p.F % kFc2Group != 0)
    return fail(H3_EUNSUPPORTED, "fc2_group %d needs an FFN width that is a multiple of it",
                fc2_group);
  const bool grouped = fc2_group != 0 && p.F > kFc2Group;  // one group = per row
  if ((rc = check_ws(p, ws, ws_bytes))) return rc;
  if (n_blocks < 0) return fail(H3_EINVAL, "n_blocks < 0");
  if (n_blocks > 0 && !blocks) return fail(H3_EINVAL, "blocks is NULL");
  for (int l = 0; l < n_blocks; ++l)
    if ((rc = check_block_weights_i8(&blocks[l], l))) return rc;
  if ((rc = check_dit_args(0, nullptr, heads))) return rc;
  if ((n_blocks > 0 && !mod) || !mod_final || !x_in)
    return fail(H3_EINVAL, "mod, mod_final and x_in are required");
  if ((p.s.n_video > 0 && !vel_video) || (p.s.n_audio > 0 && !vel_audio))
    return fail(H3_EINVAL, "velocity outputs are required");
  if (!aligned16(x_in) || (mod && !aligned16(mod)) || !aligned16(mod_final) ||
      (rope && !aligned16(rope)))
    return fail(H3_EINVAL, "tensor pointers must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  if ((rc = upload_tables(p, ws, st))) return rc;
  const bf16_t* x = x_in;
  const size_t mstride = (size_t)3 * 6 * p.H;
  for (int l = 0; l < n_blocks; ++l) {
    bf16_t* xa = at<bf16_t>(ws, p.lay.xa);
    bf16_t* xo = x == xa ? at<bf16_t>(ws, p.lay.xb) : xa;
    if ((rc = run_block_i8(p, ws, &blocks[l], mod + l * mstride, rope, x, xo, grouped, st)))
      return rc;
    x = xo;
  }
  return run_dit(p, ws, 0, nullptr, heads, mod, mod_final, rope, x, vel_video, vel_audio, st);
}

int h3_routed_attn(const h3_shape* shape, const int32_t* tile_start, const h3_bf16* q,
                   const h3_bf16* k, const h3_bf16* v, const h3_bf16* gate, h3_bf16* out,
                   int32_t* sel, float* scores, void* ws, size_t ws_bytes, void* stream) {
  Plan p;
  int rc = make_plan(shape, tile_start, H3_WS_ATTN, p);
  if (rc) return rc;
  if ((rc = check_ws(p, ws, ws_bytes))) return rc;
  if (!q || !k || !v || !out) return fail(H3_EINVAL, "q, k, v and out are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (gate && !aligned16(gate)))
    return fail(H3_EINVAL, "tensor pointers must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  if ((rc = upload_tables(p, ws, st))) return rc;
  HeadsArgs ha = heads_args(p, ws);
  ha.q_in = q;
  ha.k_in = k;
  ha.v_in = v;
  prof_begin(H3_K_HEADS, st);
  H3_TRY(launch_heads(HEADS_SPLIT, p.D, ha, st));
  prof_end(H3_K_HEADS, st);
  return run_attention(p, ws, sel, scores, out, gate, p.A, p.D, st);
}

int h3_prof_enable(int on) {
  g_prof.on = on != 0;
  g_prof.spans.clear();
  g_prof.used = 0;
  for (int c = 0; c < H3_K_COUNT; ++c) {
    g_prof.launches[c] = 0;
    g_prof.ms[c] = 0.0;
  }
  return H3_OK;
}

int h3_prof_read(int32_t cls, int64_t* launches, double* total_ms) {
  if (cls < 0 || cls >= H3_K_COUNT) return fail(H3_EINVAL, "bad kernel class");
  for (auto& sp : g_prof.spans) {
    float ms = 0.f;
    if (hipEventSynchronize(sp.second.second) != hipSuccess) return fail(H3_EHIP, "event sync");
    if (hipEventElapsedTime(&ms, sp.second.first, sp.second.second) != hipSuccess)
      return fail(H3_EHIP, "event elapsed");
    g_prof.launches[sp.first] += 1;
    g_prof.ms[sp.first] += ms;
  }
  g_prof.spans.clear();
  g_prof.used = 0;
  if (launches) *launches = g_prof.launches[cls];
  if (total_ms) *total_ms = g_prof.ms[cls];
  return H3_OK;
}

int h3_calibrate_mfma(const void* operands, size_t operand_bytes, int32_t n_blocks,
                      int32_t iters, float* sink, void* stream) {
  if (!operands || !sink) return fail(H3_EINVAL, "operands or sink is NULL");
  if (operand_bytes < 16 || operand_bytes % 16) return fail(H3_EINVAL, "operand_bytes must be a positive multiple of 16");
  if (n_blocks < 1 || n_blocks > (1 << 20) || iters < 1) return fail(H3_EINVAL, "n_blocks or iters out of range");
  H3_TRY(launch_calib_mfma(operands, operand_bytes, n_blocks, iters, sink,
                           static_cast<hipStream_t>(stream)));
  return H3_OK;
}

const char* h3_prof_kernel_name(int32_t cls) {
  static const char* names[H3_K_COUNT] = {"modnorm", "gemm_qkv", "heads", "route", "attn",
                                          "gemm_o", "gemm_fc1", "gemm_fc2", "final", "tables",
                                          "rows_in", "time", "euler", "tokens", "quant"};
  return (cls >= 0 && cls < H3_K_COUNT) ? names[cls] : "";
}

}  // extern "C"
