"""GPU parity of the products' split-K tail at small sizes.

A product's 256x256 tiles run in rounds of 256 (one per CU).  When the last
round is at most half filled and splitting it saves enough of a tile's K loop,
its tiles are computed as several K ranges whose raw sums are added by a
second launch that runs the epilogue.  The shapes below have a single row of
tiles and a long K, so every product of the block (QKV with and without the
routing gate, out projection, FC1 with GELU and with SwiGLU, FC2) takes that
path; the int8 forward splits its QKV, FC1 and per-row FC2 products.  The
comparison with the oracle and the bars are those of the block and int8
tests (same arithmetic and rounding points; only the fp32 summation order of
the split tiles changes)."""
import pytest
import torch

from audio_diffusion_transformer_amd import binding as B
from audio_diffusion_transformer_amd import synth as S
from oracle import h3_oracle as O

import gpu_harness as G
import parity as P
from test_gpu_block import _check_block, _inputs
from test_gpu_int8 import _i8_case, _run_i8

pytestmark = pytest.mark.gpu

# one row of tiles (R <= 256), K = 3072 = 48 stages: every product splits
WIDE = S.Shape(n_text=32, n_audio=32, n_video=192, hidden=3072, n_heads=24, head_dim=128,
               ffn=3072, tile=64, top_k=2, pooled=1)


def _assert_splits(sh, which):
    ts, npt = S.tile_map(sh)
    lay = B.workspace_layout(B.make_shape(sh, ts, npt), ts, which)
    assert lay.partial > 0, "the plan holds no split-K region: the test would not cover it"


@pytest.mark.parametrize("mlp,gate,rows", [(0, 0, 256), (1, 1, 256), (0, 0, 200), (1, 0, 200)])
def test_split_block_all_stages(mlp, gate, rows):
    # rows 200: the single row of tiles is ragged (rows >= M are clamped and dropped)
    sh = WIDE.replace(mlp=mlp, gate=gate, n_video=rows - 64)
    _assert_splits(sh, B.H3_WS_BLOCK)
    # hidden 3072: a 1-spacing flip of one n2 value (0.15% of them here) moves
    # every small GELU output of its row, so about 2% of h sit one spacing
    # away, with or without the split (the same fraction was measured with the
    # split switched off); h is bounded by value as in the full-size test
    _check_block(sh, *_inputs(sh), h_frac=0.1)


@pytest.mark.parametrize("mlp", [0, 1])
def test_block_ragged_last_tile_row(mlp):
    # 356 rows: the second row of tiles holds 100 rows, so the waves that own
    # its rows 128-255 compute only clamped copies of row 355, which must
    # never reach the output
    sh = WIDE.replace(mlp=mlp, n_video=356 - 64)
    _check_block(sh, *_inputs(sh), h_frac=0.1)


def test_split_block_deterministic():
    """The partial sums are added in a fixed order: two calls give the same bytes."""
    sh = WIDE.replace(mlp=1, gate=1)
    print("case: split block determinism", flush=True)
    run = G.BlockRun(sh, *_inputs(sh))
    a = run.run().clone()
    b = run.run(G.T.bf16_empty(a.shape))
    assert torch.equal(a, b)


@pytest.mark.parametrize("fc2g", [0, 1024])
def test_split_int8_forward(fc2g):
    # K = 5120 int8 = 40 stages: QKV (3 tiles), FC1 (20 tiles) and the per-row
    # FC2 (20 tiles) split; the grouped FC2 product does not
    sh = S.Shape(n_text=32, n_audio=32, n_video=192, hidden=5120, n_heads=4, head_dim=64,
                 ffn=5120, tile=64, top_k=2, pooled=1)
    _assert_splits(sh, B.H3_WS_DIT_I8)
    print(f"case: split int8 forward fc2_group={fc2g}", flush=True)
    ts, npt, blocks, mods, head, mf, rope, x = _i8_case(sh, 1)
    gv, ga = _run_i8(sh, ts, npt, blocks, mods, head, mf, rope, x, fc2g)
    qws = [O.quantize_block_int8(b) for b in blocks]
    r = O.dit_forward(sh, ts, npt, blocks, head, mods, mf, rope, x, qws=qws,
                      fc2_group=fc2g if fc2g and sh.ffn > fc2g else 0)
    for got, ref in ((gv, r["vel_video"]), (ga, r["vel_audio"])):
        m = P.metrics(got, ref)
        assert m["cos"] >= 0.9999 and m["rel"] <= 5e-3, m
