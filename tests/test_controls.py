"""Planted-bug controls (TensorFold PR #949, "Kernel contract": controls that
must go red as planted).  Each control is an implementation with one planted
mistake -- a patched copy of the float64 oracle, on the CPU -- run on the
inputs of a GPU parity test and judged by that test's own checks
(parity.routed_checks, parity.rounding_probe_checks, parity.block_checks)
against the plain C++ oracle, the GPU tests' reference.  The unpatched float64
oracle must pass the same checks, and every planted mistake must fail them."""
import numpy as np
import pytest

from audio_diffusion_transformer_amd import synth as S
from oracle import h3_oracle as O
from oracle import h3_ref as C

import parity as P


def attn_shape(n_text, n_audio, n_video, nh, d, tile, top_k, pooled=1):
    return S.Shape(n_text, n_audio, n_video, nh * d, nh, d, 256, tile=tile, top_k=top_k,
                   pooled=pooled)


def _as_result(r):
    """The float64 oracle's routed result in the layout the checks read."""
    return dict(sel=r["sel"], scores=r["scores"], out=r["out"],
                out_bits=O.f64_to_bf16_bits(r["out"]))


def _routed_failures(sh, ts, npt, q, k, v, strict_sel=True, ts_impl=None):
    ref = C.routed_attn(sh, ts, npt, q, k, v)
    got = _as_result(O.routed_attn(sh, ts if ts_impl is None else ts_impl, npt, q, k, v))
    c = P.Checks("control")
    P.routed_checks(c, got, ref, npt, sh.top_k, strict_sel=strict_sel)
    return c.failures()


def _probe_failures():
    import importlib.util
    import os
    spec = importlib.util.spec_from_file_location(
        "test_gpu_attn_inputs", os.path.join(os.path.dirname(__file__), "test_gpu_attn.py"))
    ta = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(ta)
    sh = attn_shape(64, 64, 512, 2, 64, 64, 2, pooled=0)
    ts, npt = S.tile_map(sh)
    q, k, v = ta.softmax_probe_inputs(sh)
    ref = C.routed_attn(sh, ts, npt, q, k, v)
    got = _as_result(O.routed_attn(sh, ts, npt, q, k, v))
    c = P.Checks("probe control")
    P.rounding_probe_checks(c, got["out_bits"], ref["out_bits"])
    return c.failures()


def _block_failures():
    sh = S.Shape(32, 32, 448, 256, 4, 64, 512, tile=64, top_k=3)
    ts, npt = S.tile_map(sh)
    w, mod, rope = S.block_weights(sh), S.modulation(sh), S.rope_tables(sh)
    x = S.activations(sh, field=True)
    ref = C.block_forward(sh, ts, npt, w, mod, rope, x)
    got = O.block_forward(sh, ts, npt, w, mod, rope, x)
    c = P.Checks("block control")
    P.block_checks(c, got, ref, npt, len(ts) - 1, sh.top_k, sh.pooled)
    return c.failures()


# ----------------------------------------------------------------------------
# The inputs of the GPU tests
# ----------------------------------------------------------------------------

def _tie_case():
    sh = attn_shape(64, 64, 640, 2, 64, 64, 3)
    ts, npt = S.tile_map(sh)
    _, k, v = S.attn_qkv(sh)
    return sh, ts, npt, np.zeros_like(k), k, v


def _ragged_case():
    sh = attn_shape(64, 64, 600, 2, 64, 64, 4)         # last video tile: 24 rows
    ts, npt = S.tile_map(sh)
    q, k, v = S.attn_qkv(sh)
    return sh, ts, npt, q, k, v


def test_unpatched_oracle_passes_every_check():
    sh, ts, npt, q, k, v = _tie_case()
    assert _routed_failures(sh, ts, npt, q, k, v, strict_sel=False) == []
    assert _routed_failures(*_ragged_case()) == []
    assert _probe_failures() == []
    assert _block_failures() == []


def test_control_tie_break_to_the_higher_tile(monkeypatch):
    def topk_higher(scores_row, cand, k):
        cand = np.asarray(cand)
        if k >= len(cand):
            return np.sort(cand)
        s = np.where(np.isnan(scores_row[cand]), -np.inf, scores_row[cand])
        order = np.lexsort((-cand, -s))                # planted: ties to the higher tile
        return np.sort(cand[order[:k]])
    monkeypatch.setattr(O, "topk_tiles", topk_higher)
    sh, ts, npt, q, k, v = _tie_case()
    fails = _routed_failures(sh, ts, npt, q, k, v, strict_sel=False)
    assert "sel = rule top-k of own scores" in fails, fails


def test_control_dropped_ragged_tile(monkeypatch):
    real = O.routing

    def routing_without_last(q, k, v, tile_start, n_prefix_tiles, top_k):
        rt = real(q, k, v, tile_start, n_prefix_tiles, top_k)
        last = len(tile_start) - 2                   # planted: the ragged last tile is
        S_ = rt["scores"].copy()                     # never a candidate
        nh, nQ, _ = S_.shape
        cand = np.arange(n_prefix_tiles, last)
        for h in range(nh):
            for i in range(nQ):
                rt["sel"][h, i] = O.topk_tiles(S_[h, i], cand, top_k)
        return rt
    monkeypatch.setattr(O, "routing", routing_without_last)
    fails = _routed_failures(*_ragged_case())
    assert "sel" in fails and "sel = rule top-k of own scores" in fails, fails


def test_control_off_by_one_tile_map():
    sh, ts, npt, q, k, v = _ragged_case()
    shifted = ts.copy()
    shifted[npt + 1:-1] += 1                        # planted: video tile edges one row late
    fails = _routed_failures(sh, ts, npt, q, k, v, ts_impl=shifted)
    assert "scores" in fails and "out elementwise" in fails, fails


def test_control_unrounded_softmax_weights(monkeypatch):
    def unrounded(q, kk, vv):
        d = q.shape[-1]
        s = (q @ kk.T) * d ** -0.5
        p = np.exp(s - np.max(s, axis=1, keepdims=True))
        return (p @ vv) / np.sum(p, axis=1, keepdims=True)   # planted: p not rounded
    monkeypatch.setattr(O, "softmax_rows_bf16p", unrounded)
    assert "probe bytes" in _probe_failures()


def test_control_rounded_denominator(monkeypatch):
    def rounded_l(q, kk, vv):
        d = q.shape[-1]
        s = (q @ kk.T) * d ** -0.5
        pb = O.round_bf16(np.exp(s - np.max(s, axis=1, keepdims=True)))
        return (pb @ vv) / np.sum(pb, axis=1, keepdims=True)  # planted: l from bf16 weights
    monkeypatch.setattr(O, "softmax_rows_bf16p", rounded_l)
    assert "probe bytes" in _probe_failures()


def test_control_swapped_shift_and_scale(monkeypatch):
    real = O.modulated_rmsnorm

    def swapped(x, shift, scale, seg, eps):
        return real(x, scale, shift, seg, eps)      # planted: shift and scale swapped
    monkeypatch.setattr(O, "modulated_rmsnorm", swapped)
    fails = _block_failures()
    assert {"q", "k", "v", "x2"} <= set(fails), fails
