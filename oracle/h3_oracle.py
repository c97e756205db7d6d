"""CPU oracle for the H3-style joint video+audio DiT forward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.  It
shares no code with the HIP library.

What it computes, and where each step comes from:

* "Antirez/h3.c: MiniMax H3 inference engine for Mac computers" (the h3.c
  README, implementation notes): fused gated AdaLN with a rounded bf16
  residual, QKV rows interleaved per attention head, fused Q/K RMS norm and
  RoPE, bf16 output heads, F32 rows out.
* "TensorFold PR #949" (FastH3 DiT forward on Zig + Metal): sections
  "Precision is the checkpoint's own" (bf16 weights and activations, fp32
  sums, fp32 tile means / scores / top-k / pooled branch, softmax weights
  rounded to bf16 before the value product), "What it adds" (block.zig:
  modulated norm, q/k/v products, head layout with q/k norm and rotary, tile
  means, tile scores, top-k, pooled branch, tile-routed attention with an
  online softmax, out projection, MLP), and "Kernel contract" (top-k rule:
  a NaN score ranks as -inf, ties go to the lower tile).

Arithmetic: every value is carried in float64.  Rounding happens only where
the pages put it: bf16 (round to nearest even) at the activation storage
points, fp32 for the tile means and tile scores, whose fp32 values decide the
top-k.  Matrix products use numpy's matmul (a library primitive) in float64.

Readings where the pages are silent (each listed with its reason in the
design notes): RMS norm without a learned gain, eps 1e-6; modulation as
(1 + scale) and + shift, one set of six vectors per segment (text, audio,
video); gate as x + g * branch; GELU with exact erf; SwiGLU as silu(g) * u on
the stored bf16 gate and up rows; the routing gate as a fourth per-head
product multiplying the pooled branch, with no activation; biases on every linear;
half-split RoPE pairs (i, i + d/2) from caller tables; scale d^-1/2 on row and
tile scores; prefix (text + audio) keys always attended by video rows, top-k
over video key tiles only; tile-mean divisor = true row count; pooled branch =
softmax over all key tiles of the tile scores times the key tiles' value means,
added in full precision before the bf16 rounding of the attention output; text
and audio rows attend densely with no pooled term; softmax denominator uses the
unrounded weights.  For the denoising loop (the pages name its pieces, not
their formulas): the rows in are F32 linear patch projections rounded once to
bf16; the time embedder is a 256-wide cos/sin frequency embedding of
t = 1000 sigma followed by Linear -> silu -> Linear; the modulation tables of
a step are one shared projection of silu(c) per segment plus a per-block
table, stored fp32; each pass ends with an Euler transition of the fp32
latents on the caller's per-segment schedule.  Token reduction: a pair of
horizontally adjacent video tokens pools to the bf16 mean of the two; the
restore adds the pair's update (current minus pooled value) to each token's
value at the pooling point and rounds once; a single token (odd width) takes
its reduced value; the pooled token rotates by its first token's position.

Parity against a released H3 / FastH3 checkpoint is unpinned (no weights,
case file or reference velocities are available); every function here is
pinned by the tests in tests/test_oracle_*.py against closed forms,
invariants, library routines and brute force.
"""
from __future__ import annotations

import time

import numpy as np
from scipy.special import erf as _erf

TEXT, AUDIO, VIDEO = 0, 1, 2


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------

def bf16_to_f64(u16):
    """Raw bf16 bits -> float64 (exact)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def round_bf16(x):
    """float64 -> nearest bf16 value (ties to even), returned as float64.

    bf16 = 1 sign, 8 exponent, 7 fraction bits (fp32's exponent range).
    Normal range: keep the top 7 of the 52 fraction bits of the float64,
    rounding the dropped 45 bits to nearest, ties to even.  Below 2^-126
    (bf16 subnormals) the grid is uniform with step 2^-133.  Results beyond
    the largest finite bf16 become +-inf; NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    fin = np.isfinite(x)
    small = fin & (np.abs(x) < 2.0 ** -126)
    norm = fin & ~small
    bits = x[norm].view(np.uint64)
    half = np.uint64(1) << np.uint64(44)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    bits = (bits + (half - np.uint64(1)) + lsb) & ~((np.uint64(1) << np.uint64(45)) - np.uint64(1))
    r = bits.view(np.float64)
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > bf16_max, np.copysign(np.inf, r), r)
    out[norm] = r
    step = 2.0 ** -133
    out[small] = np.round(x[small] / step) * step   # np.round: half to even
    out[~fin] = x[~fin]
    return out


def f64_to_bf16_bits(x):
    """float64 values that are exactly bf16 -> raw bits (uint16)."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_f32(x):
    """float64 -> nearest float32 (numpy's cast rounds to nearest even), as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# Rows, segments, tiles
# ----------------------------------------------------------------------------

def row_segments(n_text, n_audio, n_video):
    """Segment id of every packed row: text rows, then audio, then video
    (one packed sequence; TensorFold PR #949, opening summary)."""
    return np.concatenate([np.full(n_text, TEXT), np.full(n_audio, AUDIO),
                           np.full(n_video, VIDEO)]).astype(np.int64)


def check_tile_map(tile_start, n_text, n_audio, n_video, n_prefix_tiles):
    ts = np.asarray(tile_start, dtype=np.int64)
    R = n_text + n_audio + n_video
    assert ts[0] == 0 and ts[-1] == R and np.all(np.diff(ts) > 0)
    assert ts[n_prefix_tiles] == n_text + n_audio
    # every segment boundary is a tile edge: text | audio as well as prefix | video
    assert n_text in ts[:n_prefix_tiles + 1]
    return ts


# ----------------------------------------------------------------------------
# Block pieces
# ----------------------------------------------------------------------------

def modulated_rmsnorm(x, shift, scale, seg, eps):
    """Modulated norm (AdaLN): bf( x * (mean_k x_k^2 + eps)^-1/2 * (1 + scale[seg]) + shift[seg] ).

    x: float64 [n][H] (bf16 values); shift, scale: [3][H] per segment; seg:
    the segment id of each of the n rows.
    h3.c README (fused gated AdaLN notes: per-row RMS, rounded bf16 output);
    TensorFold PR #949, "What it adds" (modulated norm)."""
    ms = np.mean(x * x, axis=1, keepdims=True)
    y = x * (ms + eps) ** -0.5 * (1.0 + scale[seg]) + shift[seg]
    return round_bf16(y)


def linear(a, w, b):
    """a @ w^T + b in float64 (weights stored [out][in])."""
    return a @ w.T + b


def gelu(z):
    """GELU with the exact normal CDF: 0.5 z (1 + erf(z / sqrt 2))."""
    return 0.5 * z * (1.0 + _erf(z / np.sqrt(2.0)))


def split_qkv(y, n_heads, head_dim, parts=3):
    """Per-head interleaved projection rows [h][q|k|v][d] (h3.c README, note on
    the checkpoint's QKV layout) -> q, k, v as [nh][R][d].  With parts = 4 the
    fourth block of each head, [h][q|k|v|g][d], is the routing gate g (TensorFold
    PR #949, "What it adds": q/k/v and the routing gate), returned as a fourth
    array."""
    R = y.shape[0]
    t = y.reshape(R, n_heads, parts, head_dim)
    out = [np.ascontiguousarray(t[:, :, i, :].transpose(1, 0, 2)) for i in range(parts)]
    return tuple(out)


def silu(z):
    """z * sigmoid(z) = z / (1 + e^-z)."""
    return z / (1.0 + np.exp(-z))


def split_gate_up(z, ffn):
    """FC1 output of the SwiGLU MLP -> (gate, up), each [R][ffn].  The FC1 rows
    alternate in blocks of 16: rows 32b .. 32b+15 are the gate rows of features
    16b .. 16b+15 and rows 32b+16 .. 32b+31 their up rows (a storage order of
    this library's ABI, like the per-head QKV interleave)."""
    R = z.shape[0]
    t = z.reshape(R, ffn // 16, 2, 16)
    return t[:, :, 0, :].reshape(R, ffn), t[:, :, 1, :].reshape(R, ffn)


def swiglu_hidden(z, ffn):
    """h = bf(silu(bf g) * bf u) from the FC1 output z (float64 before rounding):
    the gate and up products are stored as bf16 like every projection output,
    then combined in full precision and rounded (TensorFold PR #949, "What it
    adds": the SwiGLU MLP; the pages' h3_swiglu kernel takes the stored rows)."""
    g, u = split_gate_up(round_bf16(z), ffn)
    return round_bf16(silu(g) * u)


def qk_norm_rope(u, gain, rope, eps):
    """Per-head RMS norm with gain, then rotary embedding, then bf16.

    u: [nh][R][d] (bf16 values); gain: [d]; rope: fp32 [R][d/2][2] (cos, sin)
    or None (identity).  Pairs are (i, i + d/2):
    (a, b) -> (a cos - b sin, b cos + a sin).
    TensorFold PR #949, "What it adds" (head layout with q/k norm and rotary);
    h3.c README (fused Q/K normalization and RoPE)."""
    d = u.shape[-1]
    ms = np.mean(u * u, axis=-1, keepdims=True)
    t = u * (ms + eps) ** -0.5 * gain
    if rope is None:
        return round_bf16(t)
    c = rope[None, :, :, 0].astype(np.float64)
    s = rope[None, :, :, 1].astype(np.float64)
    a, b = t[..., : d // 2], t[..., d // 2:]
    return round_bf16(np.concatenate([a * c - b * s, b * c + a * s], axis=-1))


def tile_means(u, tile_start, tiles):
    """fp32 mean over each listed tile's rows: [nh][len(tiles)][d]
    (TensorFold PR #949, "Precision": fp32 tile means).  Divisor: the tile's
    true row count."""
    out = np.empty((u.shape[0], len(tiles), u.shape[2]))
    for j, t in enumerate(tiles):
        s, e = tile_start[t], tile_start[t + 1]
        out[:, j, :] = np.sum(u[:, s:e, :], axis=1) / (e - s)
    return round_f32(out)


def tile_scores(qbar, kbar):
    """fp32 tile scores S[h][i][j] = (qbar_i . kbar_j) * d^-1/2 (TensorFold PR
    #949, "What it adds": tile scores; "Precision": fp32 scores)."""
    d = qbar.shape[-1]
    return round_f32(np.einsum("hid,hjd->hij", qbar, kbar) * d ** -0.5)


def topk_tiles(scores_row, cand, k):
    """The k candidate tiles with the largest score, returned ascending.

    Rule from TensorFold PR #949, "Kernel contract": a NaN score ranks as
    -inf and ties go to the lower tile.  k >= len(cand) keeps all of them."""
    cand = np.asarray(cand)
    if k >= len(cand):
        return np.sort(cand)
    s = np.where(np.isnan(scores_row[cand]), -np.inf, scores_row[cand])
    order = np.lexsort((cand, -s))          # primary: larger score; then lower index
    return np.sort(cand[order[:k]])


def pooled_branch(scores_row, vbar):
    """Pooled (coarse) branch for one query tile: softmax over all key tiles
    of the tile scores, times the key tiles' value means (TensorFold PR #949,
    "What it adds": the pooled branch over tile means)."""
    m = np.max(scores_row)
    w = np.exp(scores_row - m)
    return (w @ vbar) / np.sum(w)


def softmax_rows_bf16p(q, kk, vv):
    """Attention of query rows q [n][d] over keys kk/vv [m][d].

    Scores are scaled by d^-1/2; p = exp(s - max s); the value product uses
    p rounded to bf16, the denominator the unrounded sum (TensorFold PR #949,
    "Precision": softmax weights rounded to bf16 before the value product)."""
    d = q.shape[-1]
    s = (q @ kk.T) * d ** -0.5
    m = np.max(s, axis=1, keepdims=True)
    p = np.exp(s - m)
    l = np.sum(p, axis=1, keepdims=True)
    return (round_bf16(p) @ vv) / l


def routing(q, k, v, tile_start, n_prefix_tiles, top_k):
    """Tile means, tile scores, top-k video key tiles and the pooled branch.

    q, k, v: [nh][R][d] float64 (bf16 values).  Returns dict with
    qbar [nh][nQ][d], kbar, vbar [nh][nK][d], scores [nh][nQ][nK] (fp32
    values), sel [nh][nQ][min(k, nQ)] (absolute tile ids), pooled
    [nh][nQ][d]."""
    nK = len(tile_start) - 1
    vid_tiles = list(range(n_prefix_tiles, nK))
    qbar = tile_means(q, tile_start, vid_tiles)
    kbar = tile_means(k, tile_start, range(nK))
    vbar = tile_means(v, tile_start, range(nK))
    S = tile_scores(qbar, kbar)
    nh, nQ = S.shape[0], S.shape[1]
    kk = min(top_k, nQ)
    sel = np.empty((nh, nQ, kk), dtype=np.int64)
    pooled = np.empty((nh, nQ, q.shape[-1]))
    for h in range(nh):
        for i in range(nQ):
            sel[h, i] = topk_tiles(S[h, i], np.asarray(vid_tiles), top_k)
            pooled[h, i] = pooled_branch(S[h, i], vbar[h])
    return dict(qbar=qbar, kbar=kbar, vbar=vbar, scores=S, sel=sel, pooled=pooled)


def attention(q, k, v, tile_start, n_prefix_tiles, n_prefix_rows, rt, use_pooled,
              rows=None, gate=None):
    """Attention output, row-major [len(rows)][nh*d] (float64 before the bf16
    rounding is applied by the caller via round_bf16).

    Text and audio rows attend densely over all rows (TensorFold PR #949,
    parity notes: the audio rows' attention is dense).  A video row in query
    tile i attends the prefix rows, then the rows of the tiles in sel[h][i] in
    ascending order; with the pooled branch on, pooled[h][i] (times the gate,
    if one is given) is added before rounding."""
    nh, R, d = q.shape
    if rows is None:
        rows = np.arange(R)
    rows = np.asarray(rows)
    out = np.zeros((len(rows), nh * d))
    nK = len(tile_start) - 1
    tile_of = np.searchsorted(tile_start, np.arange(R), side="right") - 1
    dense_idx = np.nonzero(rows < n_prefix_rows)[0]
    vid_idx = np.nonzero(rows >= n_prefix_rows)[0]
    for h in range(nh):
        if len(dense_idx):
            rr = rows[dense_idx]
            out[dense_idx, h * d:(h + 1) * d] = softmax_rows_bf16p(q[h, rr], k[h], v[h])
        if len(vid_idx):
            rr = rows[vid_idx]
            tiles = tile_of[rr]
            for t in np.unique(tiles):
                i = t - n_prefix_tiles
                sel_rows = [np.arange(tile_start[j], tile_start[j + 1]) for j in rt["sel"][h, i]]
                keys = np.concatenate([np.arange(n_prefix_rows)] + sel_rows)
                m = tiles == t
                o = softmax_rows_bf16p(q[h, rr[m]], k[h, keys], v[h, keys])
                if use_pooled:
                    pb = rt["pooled"][h, i]
                    if gate is not None:
                        o = o + gate[h, rr[m]] * pb
                    else:
                        o = o + pb
                out[vid_idx[m], h * d:(h + 1) * d] = o
    return out


def block_forward(sh, tile_start, n_prefix_tiles, w, mod, rope, x_in, out_rows=None,
                  timings=None, qw=None, fc2_group=0):
    """One DiT block, steps in the order of TensorFold PR #949 "What it adds"
    (block.zig) with the GELU MLP of the workload description:

      n1 = modnorm(x; shift1, scale1)
      y  = bf(n1 Wqkv^T + b); q, k, v per head; q~, k~ = bf(rope(rmsnorm(.)*gain))
      routing on q~, k~, v (tile means, scores, top-k, pooled)
      a  = bf(attention)
      o  = bf(a Wo^T + bo);            x1 = bf(x + gate1 * o)
      n2 = modnorm(x1; shift2, scale2)
      h  = bf(gelu(n2 W1^T + b1));     f = bf(h W2^T + b2);   x2 = bf(x1 + gate2 * f)

    The pages' own block (sh.mlp = 1, sh.gate = 1) differs in two places: the
    MLP is SwiGLU, h = bf(silu(bf g) * bf u) with [g | u] = n2 W1^T + b1
    (split_gate_up), and y carries a fourth per-head block, the routing gate
    g, which scales the pooled branch of the video rows (o = routed + g *
    pooled).  The attention width nh * d may differ from the hidden width H
    (the pages: H = 5,376, 56 heads x 128 = 7,168).

    sh: object with n_text, n_audio, n_video, n_heads, head_dim, norm_eps,
    top_k, pooled and optionally mlp (0 GELU, 1 SwiGLU), gate (0, 1), ffn.
    w: dict of bf16-bit arrays (see synth.block_weights).  mod: fp32 [3][6][H].
    rope: fp32 [R][d/2][2] or None.  x_in: bf16 bits.
    out_rows: None for all rows, else the rows whose attention / x1 / x2 are
    computed (q, k, v and routing always cover all rows).
    timings: None, or a dict that receives the wall time of the all-row part
    ("all_rows") and of the per-row part ("per_row").
    qw: None, or the int8 codes and scales of the four products
    (quantize_block_int8): each product then quantizes its bf16 input per row
    (the FC2 input per group of fc2_group columns if fc2_group > 0) and
    computes linear_int8 (h3.c README: the int8 QKV, attention-output and MLP
    products); everything else is unchanged.
    Returns a dict of float64 intermediates (bf16 values where rounded)."""
    t0 = time.perf_counter()
    mlp = int(getattr(sh, "mlp", 0))
    use_gate = int(getattr(sh, "gate", 0))
    seg = row_segments(sh.n_text, sh.n_audio, sh.n_video)
    P = sh.n_text + sh.n_audio
    ts = check_tile_map(tile_start, sh.n_text, sh.n_audio, sh.n_video, n_prefix_tiles)
    x = bf16_to_f64(x_in)
    mod = np.asarray(mod, dtype=np.float64)
    shift1, scale1, gate1, shift2, scale2, gate2 = (mod[:, i, :] for i in range(6))
    eps = sh.norm_eps
    f = {k_: bf16_to_f64(v_) for k_, v_ in w.items()}

    def lin(a_, name, group=0):
        if qw is None:
            return linear(a_, f["w_" + name], f["b_" + name])
        qa, sa = quantize_int8(a_, group)
        return linear_int8(qa, sa, qw["w_" + name], qw["s_" + name], f["b_" + name], group)

    n1 = modulated_rmsnorm(x, shift1, scale1, seg, eps)
    y = round_bf16(lin(n1, "qkv"))
    parts = split_qkv(y, sh.n_heads, sh.head_dim, 4 if use_gate else 3)
    q, k, v = parts[:3]
    g = parts[3] if use_gate else None
    qt = qk_norm_rope(q, f["q_gain"], rope, eps)
    kt = qk_norm_rope(k, f["k_gain"], rope, eps)
    rt = routing(qt, kt, v, ts, n_prefix_tiles, sh.top_k)
    rows = np.arange(x.shape[0]) if out_rows is None else np.asarray(out_rows)
    t1 = time.perf_counter()
    a = round_bf16(attention(qt, kt, v, ts, n_prefix_tiles, P, rt, bool(sh.pooled), rows, g))
    sr = seg[rows]
    o = round_bf16(lin(a, "o"))
    x1 = round_bf16(x[rows] + gate1[sr] * o)
    n2 = modulated_rmsnorm(x1, shift2, scale2, sr, eps)
    z1 = lin(n2, "fc1")
    if mlp == 1:
        hdn = swiglu_hidden(z1, z1.shape[1] // 2)
    else:
        hdn = round_bf16(gelu(z1))
    ff = round_bf16(lin(hdn, "fc2", fc2_group))
    x2 = round_bf16(x1 + gate2[sr] * ff)
    if timings is not None:
        timings["all_rows"] = t1 - t0
        timings["per_row"] = time.perf_counter() - t1
    return dict(rows=rows, n1=n1, y=y, q=qt, k=kt, v=v, g=g, attn=a, o=o, x1=x1, n2=n2,
                h=hdn, f=ff, x2=x2, **rt)


def final_heads(sh, x, mod_final, head):
    """Final modulated norm on audio and video rows, then the narrow output
    heads, F32 out with no rounding (h3.c README: final audio/video AdaLN and
    bf16 heads; TensorFold PR #949, "What it adds": rows out as raw f32).

    x: float64 [R][H]; mod_final fp32 [3][2][H] (shift, scale); head: dict of
    bf16 bits w_video [cv][H], b_video, w_audio [ca][H], b_audio."""
    seg = row_segments(sh.n_text, sh.n_audio, sh.n_video)
    mf = np.asarray(mod_final, dtype=np.float64)
    z = modulated_rmsnorm(x, mf[:, 0, :], mf[:, 1, :], seg, sh.norm_eps)
    P = sh.n_text + sh.n_audio
    za = z[sh.n_text:P]
    zv = z[P:]
    vel_video = linear(zv, bf16_to_f64(head["w_video"]), bf16_to_f64(head["b_video"]))
    vel_audio = linear(za, bf16_to_f64(head["w_audio"]), bf16_to_f64(head["b_audio"]))
    return vel_video, vel_audio


def dit_forward(sh, tile_start, n_prefix_tiles, blocks, head, mods, mod_final, rope, x_in,
                qws=None, fc2_group=0):
    """L blocks, then the final norm and heads (TensorFold PR #949 opening
    summary: 50 blocks denoise one packed sequence).  blocks: list of weight
    dicts; mods: [L][3][6][H]; qws: None or the blocks' int8 products
    (quantize_block_int8), see block_forward."""
    x_bits = np.asarray(x_in, dtype=np.uint16)
    x = bf16_to_f64(x_bits)
    for l, w in enumerate(blocks):
        r = block_forward(sh, tile_start, n_prefix_tiles, w, mods[l], rope, x_bits,
                          qw=None if qws is None else qws[l], fc2_group=fc2_group)
        x = r["x2"]
        x_bits = f64_to_bf16_bits(x)
    vv, va = final_heads(sh, x, mod_final, head)
    return dict(x=x, vel_video=vv, vel_audio=va)


def routed_attn(sh, tile_start, n_prefix_tiles, q_bits, k_bits, v_bits, rows=None, gate=None):
    """Stand-alone routed attention on given head-major q, k, v (bf16 bits,
    [nh][R][d]): routing then attention, output bf16 values [rows][nh*d]."""
    q, k, v = bf16_to_f64(q_bits), bf16_to_f64(k_bits), bf16_to_f64(v_bits)
    ts = check_tile_map(tile_start, sh.n_text, sh.n_audio, sh.n_video, n_prefix_tiles)
    rt = routing(q, k, v, ts, n_prefix_tiles, sh.top_k)
    P = sh.n_text + sh.n_audio
    g = None if gate is None else bf16_to_f64(gate)
    out = round_bf16(attention(q, k, v, ts, n_prefix_tiles, P, rt, bool(sh.pooled), rows, g))
    return dict(out=out, **rt)


# ----------------------------------------------------------------------------
# Rows in, time conditioning and the denoising loop
# ----------------------------------------------------------------------------

T_EMBED_DIM = 256        # width of the frequency embedding of the timestep
T_SCALE = 1000.0         # timestep value t = T_SCALE * sigma
T_MAX_PERIOD = 10000.0


def rows_in(sh, text_bits, video_patch, audio_patch, w):
    """The packed hidden stream from the rows: text rows as given (bf16), audio
    and video patches through their F32 projections, F32 weights and inputs,
    the sum rounded once to bf16 (h3.c README, implementation notes: the
    96 -> 5376 video and 32 -> 5376 audio patch projections keep F32 weights,
    inputs and accumulation and round the results straight into the packed
    hidden stream; TensorFold PR #949, "What it adds": the rows in).

    text_bits bf16 [T][H]; video_patch fp32 [V][cv]; audio_patch fp32 [A][ca];
    w: w_video fp32 [H][cv], b_video [H], w_audio [H][ca], b_audio [H].
    Returns float64 bf16 values [R][H] (text, audio, video)."""
    f = lambda a: np.asarray(a, dtype=np.float32).astype(np.float64)
    xv = round_bf16(linear(f(video_patch), f(w["w_video"]), f(w["b_video"])))
    xa = round_bf16(linear(f(audio_patch), f(w["w_audio"]), f(w["b_audio"])))
    xt = bf16_to_f64(np.asarray(text_bits, dtype=np.uint16)).reshape(sh.n_text, sh.hidden)
    return np.concatenate([xt, xa, xv], axis=0)


def timestep_embedding(t, dim=T_EMBED_DIM, max_period=T_MAX_PERIOD):
    """Frequency embedding of a scalar timestep: [cos(t w_i)] ++ [sin(t w_i)],
    w_i = max_period^(-i / (dim/2)), i < dim/2 (the pages name the time
    embedder without its form; this is the usual diffusion-transformer one)."""
    half = dim // 2
    om = max_period ** (-np.arange(half, dtype=np.float64) / half)
    a = float(t) * om
    return np.concatenate([np.cos(a), np.sin(a)])


def time_conditioning(sigma, tw):
    """c = W2 silu(W1 e(T_SCALE sigma) + b1) + b2, [H], bf16 weights, carried
    in float64 (TensorFold PR #949, "What comes next": the time embedder)."""
    e = timestep_embedding(T_SCALE * float(sigma))
    h1 = silu(linear(e[None, :], bf16_to_f64(tw["w1"]), bf16_to_f64(tw["b1"])))
    return linear(h1, bf16_to_f64(tw["w2"]), bf16_to_f64(tw["b2"]))[0]


def modulation_tables(sh, n_blocks, tw, sigma3):
    """Modulation tables of one denoising step from the per-segment timesteps
    sigma3 = (text, audio, video) (TensorFold PR #949, "What comes next": the
    time embedder and modulation tables; h3.c README: video and audio follow
    independent schedules).  For segment s with c_s = time_conditioning:
      m_s        = W_mod silu(c_s) + b_mod                      [6H]
      mod[l][s]  = m_s + table[l]                               [6][H]
      final[s]   = W_final silu(c_s) + b_final                  [2][H]
    stored as fp32 (the tables' storage type).  Returns (mod [L][3][6][H],
    mod_final [3][2][H]) as float64 values of fp32 numbers."""
    H = sh.hidden
    wm, bm = bf16_to_f64(tw["w_mod"]), bf16_to_f64(tw["b_mod"])
    wf, bfin = bf16_to_f64(tw["w_final"]), bf16_to_f64(tw["b_final"])
    table = bf16_to_f64(tw["mod_table"]).reshape(n_blocks, 6, H)
    mod = np.empty((n_blocks, 3, 6, H))
    fin = np.empty((3, 2, H))
    for s in range(3):
        a = silu(time_conditioning(sigma3[s], tw))[None, :]
        m = linear(a, wm, bm)[0].reshape(6, H)
        mod[:, s] = m[None] + table
        fin[s] = linear(a, wf, bfin)[0].reshape(2, H)
    return round_f32(mod), round_f32(fin)


def euler_step(latent, vel, sigma_from, sigma_to):
    """One Euler transition of the flow ODE, x <- x + (sigma_to - sigma_from) v,
    on fp32 latents (h3.c README: the sampler's Euler transitions, video and
    audio on their own schedules, a terminal zero after the last pass)."""
    x = np.asarray(latent, dtype=np.float32).astype(np.float64)
    return round_f32(x + (float(np.float32(sigma_to)) - float(np.float32(sigma_from))) *
                     np.asarray(vel, dtype=np.float64))


def denoise(sh, tile_start, n_prefix_tiles, blocks, head, rows_w, tw, sigmas, rope, text_bits,
            video_latent, audio_latent):
    """The denoising loop: for every pass k, the rows in from the current
    latents, the modulation tables from the timesteps sigmas[k] = (text,
    audio, video), the L-block forward and heads, then one Euler transition of
    the video and audio latents to sigmas[k + 1] (the caller's schedule; its
    last entry is the terminal zero).  Returns the final latents (fp32 values)
    and the velocities of every pass."""
    lat_v = np.asarray(video_latent, dtype=np.float32).astype(np.float64)
    lat_a = np.asarray(audio_latent, dtype=np.float32).astype(np.float64)
    sig = np.asarray(sigmas, dtype=np.float32)
    L = len(blocks)
    vels = []
    for k in range(len(sig) - 1):
        x = rows_in(sh, text_bits, lat_v, lat_a, rows_w)
        mod, fin = modulation_tables(sh, L, tw, sig[k])
        r = dit_forward(sh, tile_start, n_prefix_tiles, blocks, head, mod, fin, rope,
                        f64_to_bf16_bits(x))
        vels.append((r["vel_video"], r["vel_audio"]))
        lat_v = euler_step(lat_v, r["vel_video"], sig[k][2], sig[k + 1][2])
        lat_a = euler_step(lat_a, r["vel_audio"], sig[k][1], sig[k + 1][1])
    return dict(video=lat_v, audio=lat_a, vels=vels)


# ----------------------------------------------------------------------------
# Token reduction
# ----------------------------------------------------------------------------

def token_pool(x, pairs, n_prefix):
    """The reduced stream (h3.c README, implementation notes: token reduction
    pairs adjacent horizontal video tokens and leaves text and audio rows as
    they are): prefix rows unchanged; reduced video row r = bf((x[a] + x[b]) / 2)
    for its pair (a, b) of full video rows, x[a] for a single token.
    x: float64 bf16 values [P + V][H]; pairs int [V'][2] (-1: single).
    Returns [P + V'][H]."""
    P = n_prefix
    v = x[P:]
    a, b = pairs[:, 0], pairs[:, 1]
    single = b < 0
    pooled = round_bf16((v[a] + v[np.where(single, a, b)]) / 2.0)
    pooled[single] = v[a[single]]
    return np.concatenate([x[:P], pooled], axis=0)


def token_restore(x_red, orig, baseline, pairs, n_prefix, n_video):
    """Back to full resolution (h3.c README: each token returns as its
    original value plus the update learned by its pair): video row i of pair r
    = bf(orig[i] + (x_red[r] - baseline[r])), baseline the pair's pooled
    value when it was formed; a single token takes x_red[r]; prefix rows take
    their reduced-stream values.  orig: the full stream when it was reduced."""
    P = n_prefix
    out = np.empty((P + n_video, x_red.shape[1]))
    out[:P] = x_red[:P]
    a, b = pairs[:, 0], pairs[:, 1]
    single = b < 0
    upd = x_red[P:] - baseline[P:]
    out[P + a[single]] = x_red[P:][single]
    out[P + a[~single]] = round_bf16(orig[P + a[~single]] + upd[~single])
    out[P + b[~single]] = round_bf16(orig[P + b[~single]] + upd[~single])
    return out


def dit_forward_reduced(sh, tile_start, n_prefix_tiles, red_sh, red_tile_start, red_npt, pairs,
                        reduce_at, restore_at, blocks, head, mods, mod_final, rope, red_rope, x_in):
    """The forward with token reduction (h3.c README, implementation notes):
    blocks [0, reduce_at) at full resolution, then the pooled stream through
    blocks [reduce_at, restore_at) (its own tile map and rotary table), the
    restore against the full-resolution state kept at the pooling point, and
    blocks [restore_at, L) at full resolution; then the final norm and heads."""
    x_bits = np.asarray(x_in, dtype=np.uint16)
    x = bf16_to_f64(x_bits)
    P = sh.n_text + sh.n_audio
    L = len(blocks)
    assert 0 <= reduce_at <= restore_at <= L
    orig = base = None
    for l in range(L):
        if l == reduce_at and reduce_at < restore_at:
            orig = x
            x = token_pool(x, pairs, P)
            base = x
            x_bits = f64_to_bf16_bits(x)
        if l == restore_at and orig is not None:
            x = token_restore(x, orig, base, pairs, P, sh.n_video)
            x_bits = f64_to_bf16_bits(x)
            orig = None
        if orig is None:
            r = block_forward(sh, tile_start, n_prefix_tiles, blocks[l], mods[l], rope, x_bits)
        else:
            r = block_forward(red_sh, red_tile_start, red_npt, blocks[l], mods[l], red_rope, x_bits)
        x = r["x2"]
        x_bits = f64_to_bf16_bits(x)
    if orig is not None:  # restore_at == L
        x = token_restore(x, orig, base, pairs, P, sh.n_video)
    vv, va = final_heads(sh, x, mod_final, head)
    return dict(x=x, vel_video=vv, vel_audio=va)


# ----------------------------------------------------------------------------
# int8 products
# ----------------------------------------------------------------------------

def quantize_int8(x, group=0):
    """Symmetric int8 codes (h3.c README, implementation notes: the int8 MLP
    quantizes activations dynamically, per-output-channel weight scales, one
    scale per 1,024 channels for the FC2 input).  Per row, or per group of
    `group` consecutive columns: m = max |x|, code = rint(x * (127 / m))
    clamped to [-127, 127], scale = m / 127, all in fp32 arithmetic (the
    codes are decisions, taken in the kernels' precision).  A zero group has
    codes 0 and scale 0.  x: float64 values of bf16 numbers [n][K].
    Returns (codes int8 [n][K], scales fp32 [n] or [n][K/group])."""
    xf = np.asarray(x, dtype=np.float32)
    n, K = xf.shape
    g = K if group == 0 else group
    xg = xf.reshape(n, K // g, g)
    m = np.max(np.abs(xg), axis=2)
    with np.errstate(divide="ignore"):
        inv = np.where(m > 0, np.float32(127.0) / m, np.float32(0.0)).astype(np.float32)
    codes = np.clip(np.rint(xg * inv[:, :, None]), -127, 127).astype(np.int8).reshape(n, K)
    scale = (m / np.float32(127.0)).astype(np.float32)
    return codes, (scale[:, 0] if group == 0 else scale)


def quantize_weight_int8(w_bits):
    """Per-output-channel int8 codes of a bf16 weight [out][in] (rows)."""
    return quantize_int8(bf16_to_f64(w_bits))


def linear_int8(qa, sa, qw, sw, b, group=0):
    """y = sum_k qa qw * sa * sw + b: exact integer sums, then the scales in
    float64.  With `group`, sa is [n][K/group] and each group's sum takes its
    own activation scale."""
    # integer sums in float64 matrix products: every partial sum is an
    # integer below 127^2 K < 2^53, so they are exact
    qa64, qw64 = qa.astype(np.float64), qw.astype(np.float64)
    swf = np.asarray(sw, dtype=np.float64)
    if group == 0:
        acc = qa64 @ qw64.T
        return acc * np.asarray(sa, dtype=np.float64)[:, None] * swf[None, :] + b
    n, K = qa.shape
    y = np.zeros((n, qw.shape[0]))
    for gi in range(K // group):
        sl = slice(gi * group, (gi + 1) * group)
        y += (qa64[:, sl] @ qw64[:, sl].T) * np.asarray(sa, dtype=np.float64)[:, gi:gi + 1]
    return y * swf[None, :] + b


def quantize_block_int8(w):
    """int8 codes and scales of a block's four weight matrices."""
    out = {}
    for name in ("qkv", "o", "fc1", "fc2"):
        out["w_" + name], out["s_" + name] = quantize_weight_int8(w["w_" + name])
    return out
