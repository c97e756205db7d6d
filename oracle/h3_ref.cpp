// h3_ref.cpp -- plain C++ CPU oracle of the H3-style DiT block and forward.
//
// TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
// benchmark's CPU-baseline leg, never by the product path.  It shares no code
// with the HIP library.  The passages each step follows are named beside it;
// the arithmetic rules (fp32, one running sum per output in ascending order,
// no fused multiply-adds, bf16 round-to-nearest-even, OpenMP over independent
// outputs only) are stated in h3_ref.h.
#include "h3_ref.h"

#include <omp.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

namespace {

thread_local std::string g_err;

int fail(const char* msg) {
  g_err = msg;
  return -1;
}

// ---------------------------------------------------------------------------
// Number formats ("Precision is the checkpoint's own": bf16 storage, fp32 sums)
// ---------------------------------------------------------------------------

inline float bf2f(uint16_t u) {
  const uint32_t v = (uint32_t)u << 16;
  float f;
  std::memcpy(&f, &v, 4);
  return f;
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays NaN (quieted).
inline uint16_t f2bf(float f) {
  uint32_t v;
  std::memcpy(&v, &f, 4);
  if ((v & 0x7f800000u) == 0x7f800000u && (v & 0x007fffffu)) return (uint16_t)((v >> 16) | 0x0040u);
  v += 0x7fffu + ((v >> 16) & 1u);
  return (uint16_t)(v >> 16);
}

inline float rbf(float f) { return bf2f(f2bf(f)); }   // the value bf(f)

std::vector<float> widen(const uint16_t* u, size_t n) {
  std::vector<float> out(n);
  for (size_t i = 0; i < n; ++i) out[i] = bf2f(u[i]);
  return out;
}

enum { TEXT = 0, AUDIO = 1, VIDEO = 2 };

struct Dims {
  int T, Au, V, R, P, H, nh, d, A, F, F1, parts, nT, npt, nQ, nsel;
};

int dims_of(const h3r_shape* s, const int32_t* ts, Dims* D) {
  if (!s || !ts) return fail("null shape or tile map");
  D->T = s->n_text;
  D->Au = s->n_audio;
  D->V = s->n_video;
  if (D->T < 0 || D->Au < 0 || D->V < 0) return fail("negative row count");
  D->R = D->T + D->Au + D->V;
  D->P = D->T + D->Au;
  D->H = s->hidden;
  D->nh = s->n_heads;
  D->d = s->head_dim;
  D->A = D->nh * D->d;
  D->F = s->ffn;
  D->F1 = s->mlp == 1 ? 2 * s->ffn : s->ffn;
  D->parts = s->gate ? 4 : 3;
  D->nT = s->n_tiles;
  D->npt = s->n_prefix_tiles;
  D->nQ = D->nT - D->npt;
  D->nsel = D->nQ > 0 ? (s->top_k < D->nQ ? s->top_k : D->nQ) : 0;
  if (D->R < 1 || D->H < 1 || D->nh < 1 || D->d < 2 || (D->d & 1) || D->F < 1)
    return fail("bad widths");
  if (s->mlp == 1 && (D->F % 16)) return fail("SwiGLU needs ffn a multiple of 16");
  if (D->nT < 1 || D->npt < 0 || D->npt > D->nT) return fail("bad tile counts");
  // tile map: starts at 0, ends at R, strictly increasing; segment boundaries
  // (text | audio, prefix | video) are tile edges
  if (ts[0] != 0 || ts[D->nT] != D->R) return fail("tile map must span [0, R)");
  for (int t = 0; t < D->nT; ++t)
    if (ts[t + 1] <= ts[t]) return fail("tile map not increasing");
  if (ts[D->npt] != D->P) return fail("prefix tiles must end at the text + audio rows");
  bool edge = false;
  for (int t = 0; t <= D->npt; ++t) edge = edge || ts[t] == D->T;
  if (!edge) return fail("no tile edge at the text/audio boundary");
  if (D->nQ > 0 && s->top_k < 1) return fail("top_k must be >= 1");
  return 0;
}

inline int seg_of(const Dims& D, int r) { return r < D.T ? TEXT : (r < D.P ? AUDIO : VIDEO); }

// ---------------------------------------------------------------------------
// Plain pieces
// ---------------------------------------------------------------------------

// One running fp32 sum of a[i] b[i], i ascending (descending if rev).
inline float dot(const float* a, const float* b, int n, bool rev = false) {
  float s = 0.f;
  if (!rev)
    for (int i = 0; i < n; ++i) s += a[i] * b[i];
  else
    for (int i = n - 1; i >= 0; --i) s += a[i] * b[i];
  return s;
}

// (mean of squares + eps)^-1/2 of an fp32 row: sum_k x_k^2, ascending, / n.
inline float inv_rms(const float* x, int n, float eps) {
  float s = 0.f;
  for (int k = 0; k < n; ++k) s += x[k] * x[k];
  const float ms = s / (float)n;
  return 1.0f / sqrtf(ms + eps);
}

// Modulated RMS norm (h3.c README: the gated AdaLN, rounded bf16 output;
// TensorFold PR #949 "What it adds": modulated norm):
//   out = bf(x (ms + eps)^-1/2 (1 + scale[seg]) + shift[seg]).
void modnorm_rows(const float* x, int n, int H, const int32_t* seg, const float* shift,
                  const float* scale, float eps, float* out) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < n; ++r) {
    const float* xr = x + (size_t)r * H;
    const float rs = inv_rms(xr, H, eps);
    const float* sh = shift + (size_t)seg[r] * H;
    const float* sc = scale + (size_t)seg[r] * H;
    float* o = out + (size_t)r * H;
    for (int k = 0; k < H; ++k) o[k] = rbf(xr[k] * rs * (1.0f + sc[k]) + sh[k]);
  }
}

// out[m][o] = sum_{k = 0 .. K-1} a[m][k] w[o][k] (+ b[o] after the sum), fp32.
// Each output is one running sum over k in ascending order.  The loops visit
// the outputs in groups of 4 rows x 16 columns so that the 64 running sums of
// a group sit in registers and each weight is read once per group: 16
// neighbouring outputs of a row advance together as two 8-wide float vectors
// (GCC's vector extension; each lane is the ordinary fp32 multiply and add of
// its own output).  This decides which outputs advance together, never the
// order of a sum; linear_plain below is the textbook loop, and a test checks
// that the two agree bit for bit.  w is read through a copy arranged as
// [N/16][K][16] fp32 (a layout change).
typedef float f8 __attribute__((vector_size(32)));
typedef float f8u __attribute__((vector_size(32), aligned(4)));

void linear_f32(const float* a, int M, int K, const uint16_t* w, const uint16_t* b, int N,
                float* out) {
  constexpr int MR = 4, NC = 16;
  const int Mp = (M + MR - 1) / MR * MR, ncb = (N + NC - 1) / NC;
  std::vector<float> wp((size_t)ncb * K * NC, 0.f);
#pragma omp parallel for schedule(static)
  for (int o = 0; o < N; ++o)
    for (int k = 0; k < K; ++k)
      wp[((size_t)(o / NC) * K + k) * NC + o % NC] = bf2f(w[(size_t)o * K + k]);
  std::vector<float> ap;
  const float* A = a;
  if (Mp != M) {
    ap.assign((size_t)Mp * K, 0.f);
    std::memcpy(ap.data(), a, sizeof(float) * (size_t)M * K);
    A = ap.data();
  }
  const int nrb = Mp / MR;
#pragma omp parallel for collapse(2) schedule(static)
  for (int cb = 0; cb < ncb; ++cb)
    for (int rb = 0; rb < nrb; ++rb) {
      const int r0 = rb * MR, o0 = cb * NC;
      const float* wc = wp.data() + (size_t)cb * K * NC;
      f8 acc[MR][2] = {};
      for (int k = 0; k < K; ++k) {
        const f8 w0 = *(const f8u*)(wc + (size_t)k * NC);
        const f8 w1 = *(const f8u*)(wc + (size_t)k * NC + 8);
        for (int i = 0; i < MR; ++i) {
          const float av = A[(size_t)(r0 + i) * K + k];
          acc[i][0] += av * w0;
          acc[i][1] += av * w1;
        }
      }
      for (int i = 0; i < MR && r0 + i < M; ++i)
        for (int j = 0; j < NC && o0 + j < N; ++j) {
          const float sum = acc[i][j / 8][j % 8];
          out[(size_t)(r0 + i) * N + o0 + j] = b ? sum + bf2f(b[o0 + j]) : sum;
        }
    }
}

// The same product as the textbook triple loop (one output at a time).
void linear_plain(const float* a, int M, int K, const uint16_t* w, const uint16_t* b, int N,
                  float* out) {
#pragma omp parallel for schedule(static)
  for (int m = 0; m < M; ++m)
    for (int o = 0; o < N; ++o) {
      float sum = 0.f;
      for (int k = 0; k < K; ++k) sum += a[(size_t)m * K + k] * bf2f(w[(size_t)o * K + k]);
      out[(size_t)m * N + o] = b ? sum + bf2f(b[o]) : sum;
    }
}

// GELU with the exact normal CDF (workload's FFN): 0.5 z (1 + erf(z / sqrt 2)).
inline float gelu(float z) { return 0.5f * z * (1.0f + erff(z / sqrtf(2.0f))); }
// silu(z) = z / (1 + e^-z) (TensorFold PR #949, "What it adds": the SwiGLU MLP).
inline float silu(float z) { return z / (1.0f + expf(-z)); }

// Per-head Q/K RMS norm with gain, then rotary on the pairs (i, i + d/2),
// then bf16 (TensorFold PR #949 "What it adds": head layout with q/k norm and
// rotary; h3.c README: fused Q/K normalization and RoPE).
void qk_norm_rope_rows(const float* u, int nh, int R, int d, const float* gain,
                       const float* rope, float eps, float* out) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int h = 0; h < nh; ++h)
    for (int r = 0; r < R; ++r) {
      const float* x = u + ((size_t)h * R + r) * d;
      float* o = out + ((size_t)h * R + r) * d;
      const float rs = inv_rms(x, d, eps);
      std::vector<float> t(d);
      for (int j = 0; j < d; ++j) t[j] = x[j] * rs * gain[j];
      if (!rope) {
        for (int j = 0; j < d; ++j) o[j] = rbf(t[j]);
        continue;
      }
      const int h2 = d / 2;
      const float* cs = rope + (size_t)r * h2 * 2;
      for (int i = 0; i < h2; ++i) {
        const float a = t[i], b = t[i + h2], c = cs[2 * i], sn = cs[2 * i + 1];
        o[i] = rbf(a * c - b * sn);
        o[i + h2] = rbf(b * c + a * sn);
      }
    }
}

// fp32 mean of each listed tile's rows, divisor the tile's true row count
// (TensorFold PR #949 "Precision": fp32 tile means).
void tile_means_f(const float* u, int nh, int R, int d, const int32_t* ts, const int32_t* tiles,
                  int n_list, bool rev, float* out) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int h = 0; h < nh; ++h)
    for (int i = 0; i < n_list; ++i) {
      const int t = tiles[i], s = ts[t], e = ts[t + 1];
      for (int c = 0; c < d; ++c) {
        float sum = 0.f;
        if (!rev)
          for (int r = s; r < e; ++r) sum += u[((size_t)h * R + r) * d + c];
        else
          for (int r = e - 1; r >= s; --r) sum += u[((size_t)h * R + r) * d + c];
        out[((size_t)h * n_list + i) * d + c] = sum / (float)(e - s);
      }
    }
}

// S[h][i][j] = (qbar_i . kbar_j) d^-1/2 in fp32 (TensorFold PR #949 "What it
// adds": tile scores; "Precision": fp32 scores).
void tile_scores_f(const float* qbar, const float* kbar, int nh, int nq, int nk, int d, bool rev,
                   float* out) {
  const float scale = 1.0f / sqrtf((float)d);
#pragma omp parallel for collapse(2) schedule(static)
  for (int h = 0; h < nh; ++h)
    for (int i = 0; i < nq; ++i)
      for (int j = 0; j < nk; ++j)
        out[((size_t)h * nq + i) * nk + j] =
            dot(qbar + ((size_t)h * nq + i) * d, kbar + ((size_t)h * nk + j) * d, d, rev) * scale;
}

// Top-k under the pages' rule (TensorFold PR #949, "Kernel contract": NaN
// ranks as -inf, ties go to the lower tile).  Brute force: a candidate is kept
// when fewer than k candidates rank above it; the kept ids come out ascending.
void topk_f(const float* S, const int32_t* cand, int n, int k, int32_t* out) {
  if (k >= n) {
    std::vector<int32_t> c(cand, cand + n);
    for (int i = 1; i < n; ++i)
      for (int j = i; j > 0 && c[j - 1] > c[j]; --j) std::swap(c[j - 1], c[j]);
    for (int i = 0; i < n; ++i) out[i] = c[i];
    return;
  }
  auto key = [&](int i) { const float v = S[cand[i]]; return std::isnan(v) ? -INFINITY : v; };
  std::vector<int32_t> kept;
  for (int i = 0; i < n; ++i) {
    int above = 0;
    for (int j = 0; j < n; ++j) {
      if (j == i) continue;
      if (key(j) > key(i) || (key(j) == key(i) && cand[j] < cand[i])) ++above;
    }
    if (above < k) kept.push_back(cand[i]);
  }
  for (size_t i = 1; i < kept.size(); ++i)
    for (size_t j = i; j > 0 && kept[j - 1] > kept[j]; --j) std::swap(kept[j - 1], kept[j]);
  for (int i = 0; i < k; ++i) out[i] = kept[i];
}

// Pooled branch (TensorFold PR #949 "What it adds": the pooled branch over the
// tile means): m = max_j S_j, w_j = e^(S_j - m),
// pooled = (sum_j w_j vbar_j) / sum_j w_j over all key tiles, fp32.  A NaN
// score makes the result NaN.
void pooled_f(const float* S, const float* vbar, int nk, int d, float* out) {
  float m = S[0];
  for (int j = 1; j < nk; ++j)
    if (std::isnan(S[j]) || S[j] > m) m = std::isnan(m) ? m : S[j];
  std::vector<float> w(nk);
  float den = 0.f;
  for (int j = 0; j < nk; ++j) {
    w[j] = expf(S[j] - m);
    den += w[j];
  }
  for (int c = 0; c < d; ++c) {
    float num = 0.f;
    for (int j = 0; j < nk; ++j) num += w[j] * vbar[(size_t)j * d + c];
    out[c] = num / den;
  }
}

struct Routing {
  std::vector<float> qbar, kbar, vbar, S, pooled;
  std::vector<int32_t> sel;
};

void route(const Dims& D, const int32_t* ts, int top_k, const float* q, const float* k,
           const float* v, int rev, Routing* rt) {
  std::vector<int32_t> vid(D.nQ), all(D.nT);
  for (int i = 0; i < D.nQ; ++i) vid[i] = D.npt + i;
  for (int t = 0; t < D.nT; ++t) all[t] = t;
  rt->qbar.assign((size_t)D.nh * D.nQ * D.d, 0.f);
  rt->kbar.assign((size_t)D.nh * D.nT * D.d, 0.f);
  rt->vbar.assign((size_t)D.nh * D.nT * D.d, 0.f);
  rt->S.assign((size_t)D.nh * D.nQ * D.nT, 0.f);
  rt->sel.assign((size_t)D.nh * D.nQ * D.nsel, 0);
  rt->pooled.assign((size_t)D.nh * D.nQ * D.d, 0.f);
  const bool rm = rev & H3R_REV_MEANS, rs = rev & H3R_REV_SCORES;
  if (D.nQ > 0) tile_means_f(q, D.nh, D.R, D.d, ts, vid.data(), D.nQ, rm, rt->qbar.data());
  tile_means_f(k, D.nh, D.R, D.d, ts, all.data(), D.nT, rm, rt->kbar.data());
  tile_means_f(v, D.nh, D.R, D.d, ts, all.data(), D.nT, rm, rt->vbar.data());
  if (D.nQ == 0) return;
  tile_scores_f(rt->qbar.data(), rt->kbar.data(), D.nh, D.nQ, D.nT, D.d, rs, rt->S.data());
#pragma omp parallel for collapse(2) schedule(static)
  for (int h = 0; h < D.nh; ++h)
    for (int i = 0; i < D.nQ; ++i) {
      const float* Srow = rt->S.data() + ((size_t)h * D.nQ + i) * D.nT;
      topk_f(Srow, vid.data(), D.nQ, top_k, rt->sel.data() + ((size_t)h * D.nQ + i) * D.nsel);
      pooled_f(Srow, rt->vbar.data() + (size_t)h * D.nT * D.d, D.nT, D.d,
               rt->pooled.data() + ((size_t)h * D.nQ + i) * D.d);
    }
}

// Attention of the listed rows (TensorFold PR #949: "Precision" -- softmax
// weights rounded to bf16 before the value product, fp32 sums; "What it adds"
// -- tile-routed attention plus the pooled branch; parity notes -- the audio
// rows' attention is dense).  For row r of head h the key rows, ascending, are
// all R rows (text and audio rows) or the prefix rows followed by the rows of
// the selected tiles of r's query tile (video rows).  Then
//   s_c = (q~_r . k~_c) d^-1/2,  m = max_c s_c,  p_c = e^(s_c - m),  l = sum_c p_c,
//   o = (sum_c bf(p_c) v_c) / l  (+ pooled, times the gate g if there is one),
//   out = bf(o).
void attention_rows(const Dims& D, const int32_t* ts, int pooled_on, const float* q,
                    const float* k, const float* v, const int32_t* sel, const float* pooled,
                    const float* g, const int32_t* rows, int n_rows, uint16_t* out) {
  const float scale = 1.0f / sqrtf((float)D.d);
  std::vector<int> tile_of(D.R);
  for (int t = 0; t < D.nT; ++t)
    for (int r = ts[t]; r < ts[t + 1]; ++r) tile_of[r] = t;
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
  for (int n = 0; n < n_rows; ++n)
    for (int h = 0; h < D.nh; ++h) {
      const int r = rows[n];
      const bool video = seg_of(D, r) == VIDEO;
      std::vector<int> keys;
      if (!video) {
        keys.resize(D.R);
        for (int c = 0; c < D.R; ++c) keys[c] = c;
      } else {
        for (int c = 0; c < D.P; ++c) keys.push_back(c);
        const int i = tile_of[r] - D.npt;
        const int32_t* sl = sel + ((size_t)h * D.nQ + i) * D.nsel;
        for (int e = 0; e < D.nsel; ++e)
          for (int c = ts[sl[e]]; c < ts[sl[e] + 1]; ++c) keys.push_back(c);
      }
      const float* qr = q + ((size_t)h * D.R + r) * D.d;
      const size_t nk = keys.size();
      std::vector<float> s(nk), pb(nk);
      for (size_t c = 0; c < nk; ++c)
        s[c] = dot(qr, k + ((size_t)h * D.R + keys[c]) * D.d, D.d) * scale;
      float m = s[0];
      for (size_t c = 1; c < nk; ++c)
        if (std::isnan(s[c]) || s[c] > m) m = std::isnan(m) ? m : s[c];
      float l = 0.f;
      for (size_t c = 0; c < nk; ++c) {
        const float p = expf(s[c] - m);
        l += p;
        pb[c] = rbf(p);
      }
      std::vector<float> o(D.d, 0.f);
      for (size_t c = 0; c < nk; ++c) {
        const float* vc = v + ((size_t)h * D.R + keys[c]) * D.d;
        for (int j = 0; j < D.d; ++j) o[j] += pb[c] * vc[j];
      }
      uint16_t* dst = out + (size_t)n * D.A + (size_t)h * D.d;
      for (int j = 0; j < D.d; ++j) {
        float x = o[j] / l;
        if (video && pooled_on) {
          const int i = tile_of[r] - D.npt;
          const float pj = pooled[((size_t)h * D.nQ + i) * D.d + j];
          x = g ? x + g[((size_t)h * D.R + r) * D.d + j] * pj : x + pj;
        }
        dst[j] = f2bf(x);
      }
    }
}

// Split the projection rows [h][q|k|v(|g)][d] (h3.c README: QKV interleaved
// per attention head; TensorFold PR #949: the fourth "gate" product) into
// head-major [nh][R][d] arrays.
void split_heads(const float* y, const Dims& D, int part, float* out) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int h = 0; h < D.nh; ++h)
    for (int r = 0; r < D.R; ++r)
      for (int j = 0; j < D.d; ++j)
        out[((size_t)h * D.R + r) * D.d + j] =
            y[(size_t)r * D.parts * D.A + ((size_t)h * D.parts + part) * D.d + j];
}

void to_bits(const float* x, size_t n, uint16_t* out) {
  if (!out) return;
  for (size_t i = 0; i < n; ++i) out[i] = f2bf(x[i]);   // x holds bf16 values: exact
}

int check_weights(const h3r_block_weights* w) {
  if (!w || !w->w_qkv || !w->b_qkv || !w->q_gain || !w->k_gain || !w->w_o || !w->b_o ||
      !w->w_fc1 || !w->b_fc1 || !w->w_fc2 || !w->b_fc2)
    return fail("missing block weight");
  return 0;
}

int block(const h3r_shape* s, const Dims& D, const int32_t* ts, const h3r_block_weights* w,
          const float* mod, const float* rope, const float* x, const int32_t* rows, int n_rows,
          int rev, h3r_block_out* out, float* x2f) {
  const int R = D.R, H = D.H, A = D.A;
  std::vector<int32_t> seg(R), rseg(n_rows);
  for (int r = 0; r < R; ++r) seg[r] = seg_of(D, r);
  for (int n = 0; n < n_rows; ++n) rseg[n] = seg[rows[n]];
  // mod [3 segments][6][H] -> per-vector [3][H] tables
  std::vector<float> mv[6];
  for (int i = 0; i < 6; ++i) {
    mv[i].resize((size_t)3 * H);
    for (int sg = 0; sg < 3; ++sg)
      std::memcpy(&mv[i][(size_t)sg * H], mod + ((size_t)sg * 6 + i) * H, sizeof(float) * H);
  }
  const float eps = s->norm_eps;
  // 1. n1 = modulated norm with (shift1, scale1)
  std::vector<float> n1((size_t)R * H);
  modnorm_rows(x, R, H, seg.data(), mv[0].data(), mv[1].data(), eps, n1.data());
  to_bits(n1.data(), n1.size(), out->n1);
  // 2. y = bf(n1 Wqkv^T + b)
  const int NY = D.parts * A;
  std::vector<float> y((size_t)R * NY);
  linear_f32(n1.data(), R, H, w->w_qkv, w->b_qkv, NY, y.data());
  for (auto& e : y) e = rbf(e);
  to_bits(y.data(), y.size(), out->y);
  std::vector<float>().swap(n1);
  // 3. per head q, k, v (and g); q~, k~ = bf(rope(rmsnorm(.) gain))
  const size_t nhr = (size_t)D.nh * R * D.d;
  std::vector<float> q(nhr), k(nhr), v(nhr), g;
  split_heads(y.data(), D, 0, q.data());
  split_heads(y.data(), D, 1, k.data());
  split_heads(y.data(), D, 2, v.data());
  if (s->gate) {
    g.resize(nhr);
    split_heads(y.data(), D, 3, g.data());
  }
  std::vector<float>().swap(y);
  {
    const std::vector<float> qg = widen(w->q_gain, D.d), kg = widen(w->k_gain, D.d);
    std::vector<float> t(nhr);
    qk_norm_rope_rows(q.data(), D.nh, R, D.d, qg.data(), rope, eps, t.data());
    q.swap(t);
    qk_norm_rope_rows(k.data(), D.nh, R, D.d, kg.data(), rope, eps, t.data());
    k.swap(t);
  }
  to_bits(q.data(), nhr, out->q);
  to_bits(k.data(), nhr, out->k);
  to_bits(v.data(), nhr, out->v);
  if (s->gate) to_bits(g.data(), nhr, out->g);
  // 4-7. tile means, scores, top-k, pooled branch
  Routing rt;
  route(D, ts, s->top_k, q.data(), k.data(), v.data(), rev, &rt);
  if (out->qbar) std::memcpy(out->qbar, rt.qbar.data(), sizeof(float) * rt.qbar.size());
  if (out->kbar) std::memcpy(out->kbar, rt.kbar.data(), sizeof(float) * rt.kbar.size());
  if (out->vbar) std::memcpy(out->vbar, rt.vbar.data(), sizeof(float) * rt.vbar.size());
  if (out->scores) std::memcpy(out->scores, rt.S.data(), sizeof(float) * rt.S.size());
  if (out->sel) std::memcpy(out->sel, rt.sel.data(), sizeof(int32_t) * rt.sel.size());
  if (out->pooled) std::memcpy(out->pooled, rt.pooled.data(), sizeof(float) * rt.pooled.size());
  // 8. attention of the requested rows
  std::vector<uint16_t> att((size_t)n_rows * A);
  attention_rows(D, ts, s->pooled, q.data(), k.data(), v.data(), rt.sel.data(),
                 rt.pooled.data(), s->gate ? g.data() : nullptr, rows, n_rows, att.data());
  if (out->attn) std::memcpy(out->attn, att.data(), sizeof(uint16_t) * att.size());
  std::vector<float>().swap(q);
  std::vector<float>().swap(k);
  std::vector<float>().swap(v);
  std::vector<float>().swap(g);
  // 9. o = bf(attn Wo^T + bo); x1 = bf(x + gate1[seg] o)
  std::vector<float> af = widen(att.data(), att.size());
  std::vector<float> o((size_t)n_rows * H);
  linear_f32(af.data(), n_rows, A, w->w_o, w->b_o, H, o.data());
  std::vector<float>().swap(af);
  std::vector<float> x1((size_t)n_rows * H);
  for (int n = 0; n < n_rows; ++n)
    for (int c = 0; c < H; ++c) {
      const size_t i = (size_t)n * H + c;
      o[i] = rbf(o[i]);
      x1[i] = rbf(x[(size_t)rows[n] * H + c] + mv[2][(size_t)rseg[n] * H + c] * o[i]);
    }
  to_bits(o.data(), o.size(), out->o);
  to_bits(x1.data(), x1.size(), out->x1);
  // 10. n2 = modulated norm with (shift2, scale2)
  std::vector<float> n2((size_t)n_rows * H);
  modnorm_rows(x1.data(), n_rows, H, rseg.data(), mv[3].data(), mv[4].data(), eps, n2.data());
  to_bits(n2.data(), n2.size(), out->n2);
  // 11. h = bf(gelu(n2 W1^T + b1)), or the SwiGLU hidden bf(silu(bf g) bf u)
  std::vector<float> z((size_t)n_rows * D.F1);
  linear_f32(n2.data(), n_rows, H, w->w_fc1, w->b_fc1, D.F1, z.data());
  std::vector<float>().swap(n2);
  std::vector<float> hd((size_t)n_rows * D.F);
  if (s->mlp == 1) {
    // FC1 rows 32b .. 32b+15: gate rows of features 16b .. 16b+15; rows
    // 32b+16 .. 32b+31: their up rows (this library family's storage order)
    for (int n = 0; n < n_rows; ++n)
      for (int c = 0; c < D.F; ++c) {
        const int b = c / 16, i = c % 16;
        const float gv = rbf(z[(size_t)n * D.F1 + 32 * b + i]);
        const float uv = rbf(z[(size_t)n * D.F1 + 32 * b + 16 + i]);
        hd[(size_t)n * D.F + c] = rbf(silu(gv) * uv);
      }
  } else {
    for (size_t i = 0; i < hd.size(); ++i) hd[i] = rbf(gelu(z[i]));
  }
  std::vector<float>().swap(z);
  to_bits(hd.data(), hd.size(), out->h);
  // 12. f = bf(h W2^T + b2); x2 = bf(x1 + gate2[seg] f)
  std::vector<float> f((size_t)n_rows * H);
  linear_f32(hd.data(), n_rows, D.F, w->w_fc2, w->b_fc2, H, f.data());
  for (int n = 0; n < n_rows; ++n)
    for (int c = 0; c < H; ++c) {
      const size_t i = (size_t)n * H + c;
      f[i] = rbf(f[i]);
      x2f[i] = rbf(x1[i] + mv[5][(size_t)rseg[n] * H + c] * f[i]);
    }
  to_bits(f.data(), f.size(), out->f);
  to_bits(x2f, (size_t)n_rows * H, out->x2);
  return 0;
}

int heads(const h3r_shape* s, const float* x, const int32_t* seg, int n, const float* mf,
          const uint16_t* wv, const uint16_t* bv, int cv, const uint16_t* wa, const uint16_t* ba,
          int ca, float* vel_video, float* vel_audio) {
  const int H = s->hidden;
  // final modulated norm (mod_final [3][2][H]: shift, scale) of the audio and video rows
  std::vector<float> sh((size_t)3 * H), sc((size_t)3 * H);
  for (int sg = 0; sg < 3; ++sg) {
    std::memcpy(&sh[(size_t)sg * H], mf + ((size_t)sg * 2 + 0) * H, sizeof(float) * H);
    std::memcpy(&sc[(size_t)sg * H], mf + ((size_t)sg * 2 + 1) * H, sizeof(float) * H);
  }
  std::vector<int> vid, aud;
  for (int i = 0; i < n; ++i) {
    if (seg[i] == VIDEO) vid.push_back(i);
    if (seg[i] == AUDIO) aud.push_back(i);
  }
  for (int pass = 0; pass < 2; ++pass) {
    const std::vector<int>& idx = pass == 0 ? vid : aud;
    const int c = pass == 0 ? cv : ca;
    float* vel = pass == 0 ? vel_video : vel_audio;
    if (idx.empty()) continue;
    if (!vel) return fail("missing velocity output");
    std::vector<float> xs((size_t)idx.size() * H), zs((size_t)idx.size() * H);
    std::vector<int32_t> sg(idx.size(), pass == 0 ? VIDEO : AUDIO);
    for (size_t i = 0; i < idx.size(); ++i)
      std::memcpy(&xs[i * H], x + (size_t)idx[i] * H, sizeof(float) * H);
    modnorm_rows(xs.data(), (int)idx.size(), H, sg.data(), sh.data(), sc.data(), s->norm_eps,
                 zs.data());
    // vel = z W_head^T + b, fp32, no rounding (TensorFold PR #949: raw f32 rows out)
    linear_f32(zs.data(), (int)idx.size(), H, pass == 0 ? wv : wa, pass == 0 ? bv : ba, c, vel);
  }
  return 0;
}

}  // namespace

extern "C" {

const char* h3r_last_error(void) { return g_err.c_str(); }

int32_t h3r_set_threads(int32_t n) {
  const int prev = omp_get_max_threads();
  if (n >= 1) omp_set_num_threads(n);
  return prev;
}

void h3r_round_bf16(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f2bf(x[i]);
}

void h3r_modnorm(const uint16_t* x, int32_t n, int32_t H, const int32_t* seg, const float* shift,
                 const float* scale, float eps, uint16_t* out) {
  const std::vector<float> xf = widen(x, (size_t)n * H);
  std::vector<float> o((size_t)n * H);
  modnorm_rows(xf.data(), n, H, seg, shift, scale, eps, o.data());
  to_bits(o.data(), o.size(), out);
}

void h3r_linear(const uint16_t* a, int32_t M, int32_t K, const uint16_t* w, const uint16_t* b,
                int32_t N, float* out) {
  const std::vector<float> af = widen(a, (size_t)M * K);
  linear_f32(af.data(), M, K, w, b, N, out);
}

void h3r_linear_plain(const uint16_t* a, int32_t M, int32_t K, const uint16_t* w,
                      const uint16_t* b, int32_t N, float* out) {
  const std::vector<float> af = widen(a, (size_t)M * K);
  linear_plain(af.data(), M, K, w, b, N, out);
}

void h3r_gelu(const float* z, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = gelu(z[i]);
}

void h3r_silu(const float* z, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = silu(z[i]);
}

void h3r_qk_norm_rope(const uint16_t* u, int32_t nh, int32_t R, int32_t d, const uint16_t* gain,
                      const float* rope, float eps, uint16_t* out) {
  const std::vector<float> uf = widen(u, (size_t)nh * R * d), gf = widen(gain, d);
  std::vector<float> o(uf.size());
  qk_norm_rope_rows(uf.data(), nh, R, d, gf.data(), rope, eps, o.data());
  to_bits(o.data(), o.size(), out);
}

void h3r_tile_means(const uint16_t* u, int32_t nh, int32_t R, int32_t d, const int32_t* tile_start,
                    const int32_t* tiles, int32_t n_list, int32_t reverse, float* out) {
  const std::vector<float> uf = widen(u, (size_t)nh * R * d);
  tile_means_f(uf.data(), nh, R, d, tile_start, tiles, n_list, reverse != 0, out);
}

void h3r_tile_scores(const float* qbar, const float* kbar, int32_t nh, int32_t nq, int32_t nk,
                     int32_t d, int32_t reverse, float* out) {
  tile_scores_f(qbar, kbar, nh, nq, nk, d, reverse != 0, out);
}

void h3r_topk(const float* scores, const int32_t* cand, int32_t n_cand, int32_t k, int32_t* out) {
  topk_f(scores, cand, n_cand, k, out);
}

void h3r_pooled(const float* scores, const float* vbar, int32_t nk, int32_t d, float* out) {
  pooled_f(scores, vbar, nk, d, out);
}

int h3r_attention(const h3r_shape* s, const int32_t* tile_start, const uint16_t* q,
                  const uint16_t* k, const uint16_t* v, const int32_t* sel, const float* pooled,
                  const uint16_t* gate, const int32_t* rows, int32_t n_rows, uint16_t* out) {
  Dims D;
  if (dims_of(s, tile_start, &D)) return -1;
  if (!q || !k || !v || !out || (D.nQ > 0 && (!sel || !pooled))) return fail("null argument");
  const size_t n = (size_t)D.nh * D.R * D.d;
  const std::vector<float> qf = widen(q, n), kf = widen(k, n), vf = widen(v, n);
  std::vector<float> gf;
  if (gate) gf = widen(gate, n);
  std::vector<int32_t> all;
  if (!rows) {
    all.resize(D.R);
    for (int r = 0; r < D.R; ++r) all[r] = r;
    rows = all.data();
    n_rows = D.R;
  }
  for (int i = 0; i < n_rows; ++i)
    if (rows[i] < 0 || rows[i] >= D.R) return fail("row out of range");
  attention_rows(D, tile_start, s->pooled, qf.data(), kf.data(), vf.data(), sel, pooled,
                 gate ? gf.data() : nullptr, rows, n_rows, out);
  return 0;
}

int h3r_block_forward(const h3r_shape* s, const int32_t* tile_start, const h3r_block_weights* w,
                      const float* mod, const float* rope, const uint16_t* x_in,
                      const int32_t* rows, int32_t n_rows, int32_t reverse, h3r_block_out* out) {
  Dims D;
  if (dims_of(s, tile_start, &D)) return -1;
  if (check_weights(w)) return -1;
  if (!mod || !x_in || !out || !out->x2) return fail("null argument");
  std::vector<int32_t> all;
  if (!rows) {
    all.resize(D.R);
    for (int r = 0; r < D.R; ++r) all[r] = r;
    rows = all.data();
    n_rows = D.R;
  }
  for (int i = 0; i < n_rows; ++i)
    if (rows[i] < 0 || rows[i] >= D.R) return fail("row out of range");
  const std::vector<float> x = widen(x_in, (size_t)D.R * D.H);
  std::vector<float> x2((size_t)n_rows * D.H);
  return block(s, D, tile_start, w, mod, rope, x.data(), rows, n_rows, reverse, out, x2.data());
}

int h3r_final_heads(const h3r_shape* s, const uint16_t* x, const int32_t* seg, int32_t n,
                    const float* mod_final, const uint16_t* w_video, const uint16_t* b_video,
                    int32_t c_video, const uint16_t* w_audio, const uint16_t* b_audio,
                    int32_t c_audio, float* vel_video, float* vel_audio) {
  if (!s || !x || !seg || !mod_final || !w_video || !b_video || !w_audio || !b_audio)
    return fail("null argument");
  const std::vector<float> xf = widen(x, (size_t)n * s->hidden);
  return heads(s, xf.data(), seg, n, mod_final, w_video, b_video, c_video, w_audio, b_audio,
               c_audio, vel_video, vel_audio);
}

int h3r_dit_forward(const h3r_shape* s, int32_t n_blocks, const int32_t* tile_start,
                    const h3r_block_weights* blocks, const float* mods, const float* mod_final,
                    const float* rope, const uint16_t* x_in, const uint16_t* w_video,
                    const uint16_t* b_video, int32_t c_video, const uint16_t* w_audio,
                    const uint16_t* b_audio, int32_t c_audio, int32_t reverse,
                    float* vel_video, float* vel_audio, uint16_t* x_out) {
  Dims D;
  if (dims_of(s, tile_start, &D)) return -1;
  if (n_blocks < 0 || (n_blocks > 0 && (!blocks || !mods)) || !mod_final || !x_in)
    return fail("null argument");
  for (int l = 0; l < n_blocks; ++l)
    if (check_weights(&blocks[l])) return -1;
  std::vector<int32_t> rows(D.R), seg(D.R);
  for (int r = 0; r < D.R; ++r) {
    rows[r] = r;
    seg[r] = seg_of(D, r);
  }
  std::vector<float> x = widen(x_in, (size_t)D.R * D.H), x2(x.size());
  for (int l = 0; l < n_blocks; ++l) {
    h3r_block_out o;
    std::memset(&o, 0, sizeof(o));
    std::vector<uint16_t> bits(x.size());
    o.x2 = bits.data();
    if (block(s, D, tile_start, &blocks[l], mods + (size_t)l * 18 * D.H, rope, x.data(),
              rows.data(), D.R, reverse, &o, x2.data()))
      return -1;
    x.swap(x2);
  }
  if (x_out) to_bits(x.data(), x.size(), x_out);
  return heads(s, x.data(), seg.data(), D.R, mod_final, w_video, b_video, c_video, w_audio,
               b_audio, c_audio, vel_video, vel_audio);
}

int h3r_routed_attn(const h3r_shape* s, const int32_t* tile_start, const uint16_t* q,
                    const uint16_t* k, const uint16_t* v, const uint16_t* gate,
                    const int32_t* rows, int32_t n_rows, int32_t reverse, uint16_t* out,
                    int32_t* sel, float* scores) {
  Dims D;
  if (dims_of(s, tile_start, &D)) return -1;
  if (!q || !k || !v || !out) return fail("null argument");
  const size_t n = (size_t)D.nh * D.R * D.d;
  const std::vector<float> qf = widen(q, n), kf = widen(k, n), vf = widen(v, n);
  std::vector<float> gf;
  if (gate) gf = widen(gate, n);
  Routing rt;
  route(D, tile_start, s->top_k, qf.data(), kf.data(), vf.data(), reverse, &rt);
  if (sel) std::memcpy(sel, rt.sel.data(), sizeof(int32_t) * rt.sel.size());
  if (scores) std::memcpy(scores, rt.S.data(), sizeof(float) * rt.S.size());
  std::vector<int32_t> all;
  if (!rows) {
    all.resize(D.R);
    for (int r = 0; r < D.R; ++r) all[r] = r;
    rows = all.data();
    n_rows = D.R;
  }
  for (int i = 0; i < n_rows; ++i)
    if (rows[i] < 0 || rows[i] >= D.R) return fail("row out of range");
  attention_rows(D, tile_start, s->pooled, qf.data(), kf.data(), vf.data(), rt.sel.data(),
                 rt.pooled.data(), gate ? gf.data() : nullptr, rows, n_rows, out);
  return 0;
}

}  // extern "C"
