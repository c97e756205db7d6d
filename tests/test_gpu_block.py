"""GPU parity of h3_block_forward against the CPU oracle, stage by stage,
on seeded inputs (tiny workload and edge shapes).

Two oracles.  The stage-by-stage elementwise bars are taken against the
float64 oracle; the plain C++ fp32 oracle (the contracted one) is checked at
whole-tensor bars (parity.fp32_oracle_checks).  Tolerances, from the
arithmetic: the float64 oracle rounds only at the bf16 points; the GPU sums in
fp32 in another order.  A bf16 result can
therefore land one spacing away where the exact value sits next to a rounding
boundary, and one such flip upstream can move a downstream value by another
spacing: elementwise bars are 2 bf16 spacings plus a small absolute floor
(for values near zero after cancellation).  Attention additionally rounds its
weights against the running rather than the final max (online softmax), a
relative 2^-9 per weight, hence its looser absolute floor.  Tile means and
scores are fp32 sums of values that may differ by those flips (1 spacing / 64
rows)."""
import numpy as np
import pytest
import torch

from audio_diffusion_transformer_amd import synth as S
from oracle import h3_oracle as O
from oracle import h3_ref as O32

import gpu_harness as G
import parity as P

pytestmark = pytest.mark.gpu


def _inputs(sh, seed=42, field=True, ts=None, npt=None):
    if ts is None:
        ts, npt = S.tile_map(sh)
    w = S.block_weights(sh, seed=seed)
    mod = S.modulation(sh, seed=seed)
    rope = S.rope_tables(sh)
    x = S.activations(sh, seed=seed, field=field)
    return ts, npt, w, mod, rope, x


def _check_block(sh, ts, npt, w, mod, rope, x, strict_sel=True, h_frac=2e-2, v_atol=2 ** -11):
    case = (f"block R={sh.rows} H={sh.hidden} nh={sh.n_heads}x{sh.head_dim} F={sh.ffn} "
            f"tiles={len(ts) - 1} k={sh.top_k} pooled={sh.pooled}")
    print("case:", case, flush=True)
    run = G.BlockRun(sh, ts, npt, w, mod, rope, x)
    run.run()
    g = run.read()
    r = O.block_forward(sh, ts, npt, w, mod, rope, x)
    c = G.Checks(case)
    P.block_checks(c, g, r, npt, len(ts) - 1, sh.top_k, sh.pooled, strict_sel=strict_sel,
                   h_frac=h_frac, v_atol=v_atol)
    r32 = O32.block_forward(sh, ts, npt, w, mod, rope, x)
    P.fp32_oracle_checks(c, g, r32, ("q", "k", "v", "attn", "x1", "h", "x2"), npt,
                         sh.top_k if len(ts) - 1 > npt else None)
    # padded rows of the head-major operands are zero
    tp = P.padded_starts(ts)
    pads_zero = all(not g["q_pad"][:, tp[t] + ts[t + 1] - ts[t]:tp[t + 1]].any() and
                    not g["vt_pad"][:, :, tp[t] + ts[t + 1] - ts[t]:tp[t + 1]].any()
                    for t in range(len(ts) - 1))
    c.true("padding", pads_zero)
    c.done()
    return run, g, r


def test_tiny_block_all_stages():
    _check_block(S.TINY, *_inputs(S.TINY))


def test_mid_block_all_rows():
    """One block at mid scale, every row against the oracle: 4,608 rows
    (256 text / 256 audio / 4,096 video), hidden 3072, 24 x 128 heads, GELU
    FFN 12288, tile 64, top-k 16 of 64 video key tiles, pooled.  At hidden
    3072 a 1-spacing flip of one n2 value moves every small GELU output of its
    row by about one spacing, so h is bounded by value (as in the split-K
    tests at the same width).  v: a 1-spacing flip of an n1 value (up to 2^-6
    for entries of 2-4) times a weight of 0.02 moves a product by ~3e-4, which
    exceeds two spacings of a v entry near zero; the bound is 2^-9 as in the
    full-size test."""
    sh = S.MID
    _check_block(sh, *_inputs(sh), h_frac=0.1, v_atol=2 ** -9)


def test_tiny_block_plain_inputs_margin_rule():
    """Plain N(0,1) inputs: tile scores are close together, so selection is
    compared only where the k-th / (k+1)-th margin exceeds 1e-3."""
    _check_block(S.TINY, *_inputs(S.TINY, seed=7, field=False), strict_sel=False)


def test_block_determinism_and_no_state():
    sh = S.TINY
    run = G.BlockRun(sh, *_inputs(sh))
    a = run.run().clone()
    b = run.run(G.T.bf16_empty(a.shape))
    assert torch.equal(a, b)


def test_zero_gates_identity_on_gpu():
    sh = S.TINY
    ts, npt, w, mod, rope, x = _inputs(sh)
    mod = mod.copy()
    mod[:, 2, :] = 0
    mod[:, 5, :] = 0
    run = G.BlockRun(sh, ts, npt, w, mod, rope, x)
    out = run.run()
    np.testing.assert_array_equal(G.T.to_host_bf16(out), x)


def _ragged_tiles(n_text, n_audio, n_video, sizes):
    """Tile map with the given repeating tile sizes inside each segment."""
    starts, r, npt = [], 0, 0
    for seg, n in enumerate((n_text, n_audio, n_video)):
        o, i = 0, 0
        while o < n:
            starts.append(r + o)
            npt += seg < 2
            o += sizes[i % len(sizes)]
            i += 1
        r += n
    starts.append(r)
    return np.asarray(starts, np.int32), npt


@pytest.mark.parametrize("case", [
    # ragged tiles of several sizes, head_dim 128, prefix of text + audio
    dict(sh=S.Shape(5, 30, 300, 256, 2, 128, 256, top_k=3), sizes=[17, 50, 33, 64, 9]),
    # tile size 32 and 128, head_dim 64
    dict(sh=S.Shape(64, 64, 512, 256, 4, 64, 512, tile=32, top_k=5), sizes=None),
    dict(sh=S.Shape(128, 64, 640, 256, 4, 64, 256, tile=128, top_k=2), sizes=None),
    # top_k >= number of video tiles (keep all), pooled off
    dict(sh=S.Shape(64, 64, 256, 256, 4, 64, 256, top_k=99, pooled=0), sizes=None),
    # no text rows; no prefix at all
    dict(sh=S.Shape(0, 40, 300, 256, 2, 128, 256, top_k=2), sizes=None),
    dict(sh=S.Shape(0, 0, 300, 256, 2, 128, 256, top_k=2), sizes=None),
    # a single video tile; a single row of video
    dict(sh=S.Shape(10, 10, 64, 256, 2, 128, 256, top_k=1), sizes=None),
    dict(sh=S.Shape(10, 10, 1, 256, 2, 128, 256, top_k=1), sizes=None),
    # no video rows: every row dense, no routing
    dict(sh=S.Shape(64, 100, 0, 256, 4, 64, 256, top_k=2), sizes=None),
])
def test_edge_shapes(case):
    sh = case["sh"]
    if case["sizes"]:
        ts, npt = _ragged_tiles(sh.n_text, sh.n_audio, sh.n_video, case["sizes"])
    else:
        ts, npt = S.tile_map(sh)
    _check_block(sh, *_inputs(sh, ts=ts, npt=npt), strict_sel=False)


def test_no_rope_table():
    sh = S.TINY
    ts, npt, w, mod, rope, x = _inputs(sh)
    _check_block(sh, ts, npt, w, mod, None, x)


def test_block_at_size_limits():
    """The kernels' limits at once: 2,048 tiles (the routing's 64 lanes x 32
    scores), 4,096 key chunks of 32 padded rows (131,072 rows: the attention's
    chunk table) and top-k 512 (its selection table).  q, k, v and the routing
    are compared for every row, the rest on sampled rows (dense rows attend all
    131,072 keys, video rows the prefix and 512 tiles)."""
    sh = S.Shape(64, 64, 130944, 256, 4, 64, 256, tile=64, top_k=512)
    print("case: block at the size limits (2048 tiles, 4096 chunks, top-k 512)", flush=True)
    ts, npt, w, mod, rope, x = _inputs(sh)
    assert len(ts) - 1 == 2048
    run = G.BlockRun(sh, ts, npt, w, mod, rope, x)
    run.run()
    g = run.read()
    R = sh.rows
    rows = np.unique(np.concatenate([np.arange(0, 3), np.arange(126, 130), np.arange(60000, 60070),
                                     np.arange(R - 70, R)]))
    print("oracle ...", flush=True)
    r = O.block_forward(sh, ts, npt, w, mod, rope, x, out_rows=rows)
    c = G.Checks("block at the size limits")
    c.close("q", g["q"], r["q"], atol=2 ** -5)
    c.close("k", g["k"], r["k"], atol=2 ** -5)
    # 34M values of v: a 1-spacing flip of a large n1 value (spacing 2^-6 for
    # |n1| in [2, 4)) times a weight moves a product by up to ~2^-9, as in the
    # full-size test (seen here on 0.006% of the values)
    c.close("v", g["v"], r["v"], atol=2 ** -9)
    c.true("scores", np.max(np.abs(g["scores"] - r["scores"])) < 1e-3,
           f"{np.max(np.abs(g['scores'] - r['scores'])):.3g}")
    checked, bad, skipped = P.selection_agrees(g["sel"], r["sel"], r["scores"], npt, sh.top_k)
    c.true("sel", bad == 0 and checked > 0, f"checked {checked} bad {bad} skipped {skipped}")
    own = P.selection_follows_scores(g["sel"], g["scores"], npt, sh.top_k)
    c.true("sel = rule top-k of own scores", own == 0, f"{own} rows differ")
    c.true("sel order", bool(np.all(np.diff(g["sel"], axis=-1) > 0)))
    c.true("pooled", np.max(np.abs(g["pooled"] - r["pooled"])) < 1e-3,
           f"{np.max(np.abs(g['pooled'] - r['pooled'])):.3g}")
    m = P.metrics(g["attn"][rows], r["attn"])
    c.true("attn", m["cos"] > 0.99999 and m["rel"] < 4e-3, str(m))
    for name in ("x1", "n2", "h", "x2"):
        c.close(name, g[name][rows], r[name], ulps=2, atol=2 ** -6, frac_1ulp=2e-2)
    c.done()

