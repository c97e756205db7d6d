"""GPU parity of h3_routed_attn against the CPU oracle: tiny and full-size
(15,435 rows x 40 heads x 128) workloads with a low-rank spatial field in q
and k, the top-k rule cases, and routed-with-all-tiles equals dense."""
import numpy as np
import pytest
import torch

from audio_diffusion_transformer_amd import binding as B
from audio_diffusion_transformer_amd import synth as S
from oracle import h3_oracle as O
from oracle import h3_ref as O32

import gpu_harness as G
import parity as P

pytestmark = pytest.mark.gpu


def attn_shape(n_text, n_audio, n_video, nh, d, tile, top_k, pooled=1):
    return S.Shape(n_text, n_audio, n_video, nh * d, nh, d, 256, tile=tile, top_k=top_k,
                   pooled=pooled)


def _check(sh, rows=None, seed=42, amp=1.0):
    print(f"case: routed attn R={sh.rows} nh={sh.n_heads}x{sh.head_dim} tile={sh.tile} "
          f"k={sh.top_k} pooled={sh.pooled}", flush=True)
    ts, npt = S.tile_map(sh)
    q, k, v = S.attn_qkv(sh, seed=seed, amp=amp)
    g = G.run_routed(sh, ts, npt, q, k, v)
    r = O.routed_attn(sh, ts, npt, q, k, v, rows=rows)
    r32 = O32.routed_attn(sh, ts, npt, q, k, v, rows=rows)
    c = P.Checks(f"routed R={sh.rows} tile={sh.tile} k={sh.top_k}")
    # elementwise against the float64 oracle, whole tensors against the fp32 one
    P.routed_checks(c, g, r, npt, sh.top_k, rows=rows)
    P.fp32_oracle_checks(c, g, r32, ("out",), npt, sh.top_k, rows=rows)
    c.done()
    return g, r, ts, npt, q, k, v


def test_tiny_routed():
    _check(attn_shape(64, 64, 896, 4, 64, 64, 4))


def test_tiny_routed_d128_ragged():
    _check(attn_shape(37, 91, 1001, 3, 128, 64, 5))


def _dense_equivalent(sh, ts, npt, q, k, v):
    """The same rows and tiles, all declared prefix: every row attends densely."""
    shd = sh.replace(n_audio=sh.n_audio + sh.n_video, n_video=0)
    return G.run_routed(shd, ts, len(ts) - 1, q, k, v)


@pytest.mark.parametrize("d", [64, 128])
def test_routed_with_all_tiles_equals_dense(d):
    sh = attn_shape(40, 80, 700, 2, d, 64, 10 ** 6, pooled=0)
    ts, npt = S.tile_map(sh)
    q, k, v = S.attn_qkv(sh)
    routed = G.run_routed(sh, ts, npt, q, k, v)
    dense = _dense_equivalent(sh, ts, npt, q, k, v)
    np.testing.assert_array_equal(routed["out_bits"], dense["out_bits"])


def test_topk_ties_go_to_lower_tiles():
    """q = 0: every tile score is exactly 0 on both sides, so the top-k is
    decided by the tie rule alone: the lowest video tiles."""
    sh = attn_shape(64, 64, 640, 2, 64, 64, 3)
    ts, npt = S.tile_map(sh)
    _, k, v = S.attn_qkv(sh)
    q = np.zeros_like(k)
    g = G.run_routed(sh, ts, npt, q, k, v)
    r = O.routed_attn(sh, ts, npt, q, k, v)
    np.testing.assert_array_equal(g["sel"], r["sel"])
    assert np.all(g["sel"] == np.arange(npt, npt + 3))
    m = P.metrics(g["out"], r["out"])
    assert m["rel"] < 4e-3, m


def test_topk_nan_scores_rank_last():
    """A NaN in one key row makes that tile's mean and score NaN: the tile
    ranks as -inf (kept only if needed) and the selection stays inside its
    row; the oracle applies the same rule."""
    sh = attn_shape(64, 64, 640, 2, 64, 64, 9)   # 10 video tiles, keep 9
    ts, npt = S.tile_map(sh)
    q, k, v = S.attn_qkv(sh)
    k = k.copy()
    k[0, ts[npt + 4] + 3, 5] = 0x7FC0                 # NaN in head 0, video tile 4
    g = G.run_routed(sh, ts, npt, q, k, v)
    r = O.routed_attn(sh, ts, npt, q, k, v)
    assert np.all(np.isnan(g["scores"][0, :, npt + 4]))
    np.testing.assert_array_equal(g["sel"][0], r["sel"][0])
    assert np.all(g["sel"][0] != npt + 4)              # 9 of 10 kept: never the NaN tile
    # the pooled branch of head 0 is NaN for every video tile (as in the oracle)
    vid = slice(sh.n_prefix, sh.rows)
    assert np.array_equal(np.isnan(g["out"][vid, :64]), np.isnan(r["out"][vid, :64]))
    # the text and audio rows of head 0 attend the NaN key itself: NaN, as in the oracle
    pre = slice(0, sh.n_prefix)
    assert np.isnan(r["out"][pre, :64]).all()
    assert np.array_equal(np.isnan(g["out"][pre, :64]), np.isnan(r["out"][pre, :64]))
    assert not np.isnan(g["out"][:, 64:]).any()


def softmax_probe_inputs(sh, seed=3):
    """Every query row's largest score sits in the first key chunk it visits:
    q rows (8, 0, ...); k rows 0 (first of the dense rows' list) and P (the
    first video row: its tile has the highest tile score, so the video rows
    visit it first) are (1.5, 0, ...), all other k rows (0.296875, 0, ...), so
    the other weights are e^-1.203125 = 0.30024, which bf16 rounds up to
    0.30078125; v ~ N(0, 1)."""
    nh, R, d = sh.n_heads, sh.rows, sh.head_dim
    one = lambda x: np.uint16(np.float32(x).view(np.uint32) >> 16)
    q = np.zeros((nh, R, d), np.uint16)
    k = np.zeros((nh, R, d), np.uint16)
    q[:, :, 0] = one(8.0)
    k[:, :, 0] = one(0.296875)
    k[:, 0, 0] = one(1.5)
    k[:, sh.n_text + sh.n_audio, 0] = one(1.5)
    v = S.normal_bf16("test.probe.v", (nh, R, d), 1.0, seed=seed)
    return q, k, v


def test_softmax_rounding_points_probe():
    """The online softmax meets the definition's rounding points exactly when
    the running max is final from the first key chunk: weights rounded to
    bf16 before the value product, an unrounded fp32 denominator.  On the probe
    the output bytes must match the oracle's (bar derived in
    parity.rounding_probe_checks); an unrounded weight or a rounded
    denominator moves a large fraction of them (tests/test_controls.py)."""
    sh = attn_shape(64, 64, 512, 2, 64, 64, 2, pooled=0)
    print("case: softmax rounding probe", flush=True)
    ts, npt = S.tile_map(sh)
    q, k, v = softmax_probe_inputs(sh)
    g = G.run_routed(sh, ts, npt, q, k, v)
    r = O32.routed_attn(sh, ts, npt, q, k, v)
    c = P.Checks("softmax probe")
    P.rounding_probe_checks(c, g["out_bits"], r["out_bits"])
    c.done()


def test_routed_determinism():
    sh = attn_shape(64, 64, 896, 4, 64, 64, 4)
    ts, npt = S.tile_map(sh)
    q, k, v = S.attn_qkv(sh)
    a = G.run_routed(sh, ts, npt, q, k, v)
    b = G.run_routed(sh, ts, npt, q, k, v)
    np.testing.assert_array_equal(a["out_bits"], b["out_bits"])
    np.testing.assert_array_equal(a["sel"], b["sel"])


def _sample_rows(sh, ts, npt):
    """Rows the oracle computes one by one: ends of every segment, the first,
    a middle and the last (ragged) video tile, rows around tile seams."""
    R, P_ = sh.rows, sh.n_prefix
    rows = set()
    for a in (0, sh.n_text, P_):
        rows.update(range(a, min(a + 3, R)))
    for b in (sh.n_text, P_, R):
        rows.update(range(max(b - 3, 0), b))
    nT = len(ts) - 1
    for t in (npt, npt + (nT - npt) // 2, nT - 1):
        rows.update(range(ts[t], ts[t + 1]))
    rows.update(range(ts[npt + 1] - 2, ts[npt + 1] + 2))
    return np.array(sorted(r for r in rows if 0 <= r < R))


FULL_ATTN = attn_shape(512, 543, 14380, 40, 128, 64, 32)


def test_full_size_routed_sampled():
    sh = FULL_ATTN
    ts, npt = S.tile_map(sh)
    _check(sh, rows=_sample_rows(sh, ts, npt))


@pytest.mark.parametrize("tile,top_k", [(32, 8), (128, 8), (64, 8), (32, 32), (128, 32)])
def test_full_size_sweep_sampled(tile, top_k):
    sh = FULL_ATTN.replace(tile=tile, top_k=top_k)
    ts, npt = S.tile_map(sh)
    rows = _sample_rows(sh, ts, npt)[::3]
    _check(sh, rows=rows)


@pytest.mark.parametrize("tile", [32, 64, 128])
def test_full_size_all_tiles_equals_dense(tile):
    sh = FULL_ATTN.replace(tile=tile, top_k=10 ** 6, pooled=0)
    print(f"case: full-size all-tiles vs dense, tile={tile}", flush=True)
    ts, npt = S.tile_map(sh)
    q, k, v = S.attn_qkv(sh)
    routed = G.run_routed(sh, ts, npt, q, k, v)
    dense = _dense_equivalent(sh, ts, npt, q, k, v)
    np.testing.assert_array_equal(routed["out_bits"], dense["out_bits"])


def test_calibration_probe_runs_and_stores_nothing():
    """The matrix-core calibration call (measurement only) runs its products and
    leaves the sink untouched (its sums cannot reach the trigger value)."""
    print("case: h3_calibrate_mfma, 16 workgroups x 50 rounds", flush=True)
    ops = torch.randn(1 << 16, device="cuda").to(torch.bfloat16)
    sink = torch.zeros(256, device="cuda")
    flop = B.calibrate_mfma(ops, 16, 50, sink)
    torch.cuda.synchronize()
    assert flop == 16 * 4 * 50 * 16 * 16384
    assert not sink.any()
