"""Pins of the plain C++ oracle (oracle/h3_ref.cpp) against facts it does not
compute itself: closed forms, worked examples, textbook constants, library
routines, brute force and the top-k rule as the pages state it; plus its
agreement with the float64 oracle, byte determinism across thread counts, and
the self-noise floor of reversed tile sums.  All run on the CPU."""
import json
import math
import os

import numpy as np
import pytest
import torch

from audio_diffusion_transformer_amd import synth as S
from oracle import h3_oracle as O
from oracle import h3_ref as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32_EPS = 2.0 ** -23


def bits(x):
    """Exactly-bf16 values -> raw bits (through torch, an independent route)."""
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------

def test_round_bf16_known_values_and_torch():
    one = 1.0
    cases = {one + 2 ** -8: one, one + 3 * 2 ** -8: one + 2 ** -6, one + 2 ** -9: one,
             0.3: 0.30078125, -(one + 2 ** -7): -(one + 2 ** -7), 3.4e38: math.inf,
             (2 - 2 ** -7) * 2 ** 127: (2 - 2 ** -7) * 2 ** 127,
             1.5 * 2 ** -133: 2 ** -132, 2.5 * 2 ** -133: 2 * 2 ** -133}
    got = C.round_bf16(np.array(list(cases), np.float32))
    np.testing.assert_array_equal(got, np.array(list(cases.values())))
    assert np.isnan(C.round_bf16(np.array([np.nan], np.float32))[0])
    rng = np.random.default_rng(0)
    x32 = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                          (rng.standard_normal(10000) * 1e-39).astype(np.float32)])
    ref = torch.tensor(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(C.round_bf16(x32), ref)


# ----------------------------------------------------------------------------
# Norm, products, activations
# ----------------------------------------------------------------------------

def test_modnorm_closed_forms():
    H, eps = 8, 1e-6
    seg = np.array([0, 1, 2, 2])
    x = np.zeros((4, H))
    x[0] = 3.0                                   # constant row -> 3 / sqrt(9 + eps)
    x[1] = 0.0                                   # zero row -> the shift
    x[2, :4] = 1.0
    x[2, 4:] = -1.0                              # unit RMS row
    x[3] = np.arange(H)
    shift = np.zeros((3, H), np.float32)
    scale = np.zeros((3, H), np.float32)
    shift[1] = 0.25
    scale[2] = 1.0                               # (1 + 1) doubles the video rows
    y = C.modulated_rmsnorm(bits(x), shift, scale, seg, eps)
    np.testing.assert_array_equal(y[0], np.full(H, 1.0))       # bf(0.99999994) = 1
    np.testing.assert_array_equal(y[1], np.full(H, 0.25))
    np.testing.assert_array_equal(y[2], 2.0 * x[2])
    rms3 = math.sqrt(np.mean(np.arange(H) ** 2.0))
    np.testing.assert_array_equal(y[3], O.round_bf16(2.0 * np.arange(H) / rms3))
    # shift and scale are applied per segment, per column
    sc = np.zeros((3, H), np.float32)
    sc[0, 3] = -0.5
    y2 = C.modulated_rmsnorm(bits(np.ones((1, H))), np.zeros((3, H), np.float32), sc,
                             np.array([0]), 0.0)
    np.testing.assert_array_equal(y2[0], [1, 1, 1, 0.5, 1, 1, 1, 1])


def test_linear_worked_example_and_textbook_loop():
    a = bits([[1.0, 2.0], [3.0, -1.0]])
    w = bits([[1.0, 2.0], [0.0, 1.0]])            # out0 = a0 + 2 a1, out1 = a1
    b = bits([0.5, -0.5])
    np.testing.assert_array_equal(C.linear(a, w, b), [[5.5, 1.5], [1.5, -1.5]])
    # the grouped loop order changes no bit against the one-output-at-a-time
    # loop, on ragged sizes (rows not a multiple of 4, columns not of 16)
    rng = np.random.default_rng(1)
    for M, K, N in ((7, 33, 19), (13, 100, 40), (1, 5, 3)):
        aa = bits(O.round_bf16(rng.standard_normal((M, K))))
        ww = bits(O.round_bf16(rng.standard_normal((N, K)) * 0.05))
        bb = bits(O.round_bf16(rng.standard_normal(N) * 0.05))
        fast = C.linear(aa, ww, bb)
        np.testing.assert_array_equal(fast, C.linear_plain(aa, ww, bb))
        # and the fp32 sum stays within its worst-case bound of the exact sum
        exact = O.bf16_to_f64(aa) @ O.bf16_to_f64(ww).T + O.bf16_to_f64(bb)
        bound = (K + 1) * F32_EPS * (np.abs(O.bf16_to_f64(aa)) @ np.abs(O.bf16_to_f64(ww)).T +
                                     np.abs(O.bf16_to_f64(bb)))
        assert np.all(np.abs(fast - exact) <= bound + 1e-30)


def test_linear_sums_in_ascending_order():
    """fp32 sums are order-dependent: 1 + 2^-24 + 2^-24 = 1 in ascending
    order, but 2^-24 + 2^-24 + 1 = 1 + 2^-23.  The running sum must take the
    terms k = 0, 1, 2 in that order."""
    a = bits([[1.0, 2.0 ** -24, 2.0 ** -24]])
    w = bits([[1.0, 1.0, 1.0]])
    assert C.linear(a, w)[0, 0] == 1.0
    a2 = bits([[2.0 ** -24, 2.0 ** -24, 1.0]])
    assert C.linear(a2, w)[0, 0] == 1.0 + 2.0 ** -23
    assert C.linear_plain(a2, w)[0, 0] == 1.0 + 2.0 ** -23


def test_gelu_textbook_values():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "normal_cdf.txt"))
            if l.strip() and not l.startswith("#")]
    z = np.array([float(r[0]) for r in rows])
    phi = np.array([float(r[1]) for r in rows])
    got = C.gelu(z)
    # fp32 erf: a few units of 2^-24 of the value, plus fp32 rounding of z
    np.testing.assert_allclose(got, z * phi, rtol=8 * F32_EPS, atol=1e-7)
    assert C.gelu(np.array([0.0]))[0] == 0.0
    assert C.gelu(np.array([40.0]))[0] == 40.0


def test_silu_closed_forms():
    # silu(ln 3) = ln 3 * 3/4; silu(0) = 0; silu(-ln 3) = -ln 3 / 4
    l3 = math.log(3.0)
    got = C.silu(np.array([l3, 0.0, -l3, 30.0]))
    np.testing.assert_allclose(got, [0.75 * l3, 0.0, -0.25 * l3, 30.0], rtol=4 * F32_EPS)


def test_qk_norm_gain_rope_quarter_turn_and_identity():
    d = 4
    u = bits(np.array([[[1.0, 1.0, -1.0, -1.0]]]))    # RMS 1
    tab = np.zeros((1, 2, 2), np.float32)
    tab[0, 0] = (0.0, 1.0)                          # pair (0, 2) by 90 degrees
    tab[0, 1] = (1.0, 0.0)                          # pair (1, 3) unchanged
    out = C.qk_norm_rope(u, bits(np.ones(d)), tab, 0.0)
    np.testing.assert_array_equal(out[0, 0], [1.0, 1.0, 1.0, -1.0])
    rng = np.random.default_rng(3)
    u = bits(O.round_bf16(rng.standard_normal((2, 5, 64)) * 3))
    plain = C.qk_norm_rope(u, bits(np.full(64, 2.0)), None, 1e-6)
    np.testing.assert_allclose(np.sqrt(np.mean(plain ** 2, axis=-1)), 2.0, rtol=2 ** -8)
    ident = np.zeros((5, 32, 2), np.float32)
    ident[..., 0] = 1.0
    np.testing.assert_array_equal(C.qk_norm_rope(u, bits(np.full(64, 2.0)), ident, 1e-6), plain)


def test_rope_relative_position():
    rng = np.random.default_rng(4)
    d = 32
    inv = 10000.0 ** (-2.0 * np.arange(d // 2) / d)

    def tables(pos):
        ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]
        t = np.empty((len(pos), d // 2, 2), np.float32)
        t[..., 0], t[..., 1] = np.cos(ang), np.sin(ang)
        return t
    q = np.repeat(O.round_bf16(rng.standard_normal((1, 1, d))), 2, axis=1)
    k = np.repeat(O.round_bf16(rng.standard_normal((1, 1, d))), 2, axis=1)
    a = C.qk_norm_rope(bits(q), bits(np.ones(d)), tables([7, 107]), 1e-6)
    b = C.qk_norm_rope(bits(k), bits(np.ones(d)), tables([3, 103]), 1e-6)
    dots = np.sum(a[0] * b[0], axis=-1)
    assert abs(dots[0] - dots[1]) < 0.05 * np.abs(dots).max() + 0.05


# ----------------------------------------------------------------------------
# Routing
# ----------------------------------------------------------------------------

def test_tile_means_constant_ragged_and_fp32():
    u = np.zeros((1, 7, 2))
    u[0, :4] = 5.0
    u[0, 4:, 0] = [1.0, 2.0, 6.0]
    ts = np.array([0, 4, 7])
    m = C.tile_means(bits(u), ts, [0, 1])
    np.testing.assert_array_equal(m[0], [[5.0, 5.0], [3.0, 0.0]])
    u2 = np.zeros((1, 3, 1))
    u2[0, 0, 0] = 1.0
    assert C.tile_means(bits(u2), np.array([0, 3]), [0])[0, 0, 0] == float(np.float32(1 / 3))
    # ascending vs descending row order: 1 + 2^-24 + 2^-24 vs 2^-24 + 2^-24 + 1
    u3 = np.array([[[1.0], [2.0 ** -24], [2.0 ** -24]]])
    fwd = C.tile_means(bits(u3), np.array([0, 3]), [0])[0, 0, 0]
    rev = C.tile_means(bits(u3), np.array([0, 3]), [0], reverse=True)[0, 0, 0]
    assert fwd == float(np.float32(1.0) / np.float32(3.0))
    assert rev == float(np.float32(1.0 + 2.0 ** -23) / np.float32(3.0)) and rev != fwd


def test_tile_scores_worked_example():
    qbar = np.array([[[1.0, 2.0]]])
    kbar = np.array([[[3.0, 4.0], [-1.0, 0.5]]])
    S_ = C.tile_scores(qbar, kbar)
    scale = np.float32(1.0) / np.sqrt(np.float32(2.0))
    np.testing.assert_array_equal(S_[0, 0], [float(np.float32(11.0) * scale), 0.0])


def test_topk_rule_golden():
    g = json.load(open(os.path.join(GOLDEN, "topk_rule.json")))
    for c in g["cases"]:
        s = np.array([float(v) for v in c["scores"]])
        got = C.topk_tiles(s, np.arange(len(s)), c["k"])
        assert list(got) == c["expect"], c
    got = C.topk_tiles(np.array([9.0, 9.0, 1.0, 3.0, 2.0]), np.arange(2, 5), 2)
    assert list(got) == [3, 4]                      # absolute ids, prefix tiles excluded


def test_topk_brute_force_random_with_ties_and_nan():
    rng = np.random.default_rng(9)
    for _ in range(200):
        n = int(rng.integers(1, 40))
        s = rng.integers(-3, 4, n).astype(np.float64)       # many ties
        s[rng.random(n) < 0.1] = np.nan
        k = int(rng.integers(1, n + 2))
        got = list(C.topk_tiles(s, np.arange(n), k))
        key = [(-(-np.inf if np.isnan(v) else v), j) for j, v in enumerate(s)]
        want = sorted(j for _, j in sorted(key)[:k])
        assert got == want


def test_pooled_closed_forms():
    vbar = np.array([[1.0, 0.0], [0.0, 1.0]])
    np.testing.assert_allclose(C.pooled_branch(np.array([0.0, math.log(3.0)]), vbar),
                               [0.25, 0.75], rtol=4 * F32_EPS)
    np.testing.assert_array_equal(C.pooled_branch(np.array([2.0]), vbar[:1]), [1.0, 0.0])
    np.testing.assert_array_equal(C.pooled_branch(np.array([1.0, 1.0, 1.0]),
                                                  np.array([[3.0], [6.0], [9.0]])), [6.0])
    assert np.all(np.isnan(C.pooled_branch(np.array([0.0, np.nan]), vbar)))


# ----------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------

def _sh(n_text, n_audio, n_video, nh, d, top_k, pooled=1):
    return S.Shape(n_text, n_audio, n_video, nh * d, nh, d, 4 * nh * d, top_k=top_k,
                   pooled=pooled)


def _small_case(seed=7, n_text=5, n_audio=7, n_video=40, tile=8, nh=2, d=16, scale=1.0):
    rng = np.random.default_rng(seed)
    R = n_text + n_audio + n_video
    starts = list(range(0, n_text, tile)) + [n_text + s for s in range(0, n_audio, tile)]
    npt = len(starts)
    starts += [n_text + n_audio + s for s in range(0, n_video, tile)] + [R]
    q, k, v = (O.round_bf16(rng.standard_normal((nh, R, d)) * scale) for _ in range(3))
    return np.array(starts, np.int32), npt, q, k, v


def test_attention_brute_force_float64():
    import parity as P_
    """Tiny routed attention against a float64 brute-force softmax over each
    row's key set, computed here from the definition: the fp32 oracle may
    differ only by fp32 rounding and by bf16 rounding flips of the output."""
    ts, npt, q, k, v = _small_case()
    sh = _sh(5, 7, 40, 2, 16, top_k=2)
    r = C.routed_attn(sh, ts, npt, bits(q), bits(k), bits(v))
    rt = O.routing(q, k, v, ts, npt, 2)
    P, R, d = 12, q.shape[1], q.shape[2]
    tile_of = np.searchsorted(ts, np.arange(R), side="right") - 1
    worst = 0.0
    for h in range(2):
        for row in range(R):
            if row < P:
                keys = np.arange(R)
            else:
                i = tile_of[row] - npt
                keys = np.concatenate([np.arange(P)] +
                                      [np.arange(ts[t], ts[t + 1]) for t in r["sel"][h, i]])
            s = q[h, row] @ k[h, keys].T / math.sqrt(d)
            p = np.exp(s - s.max())
            o = (O.round_bf16(p) @ v[h, keys]) / p.sum()
            # the fp32 weights may round to the neighbouring bf16 value where
            # the exact one sits next to a rounding boundary: 2^-8 relative each
            flip = 2.0 ** -8 * (np.abs(p) @ np.abs(v[h, keys])) / p.sum()
            if row >= P:
                o = o + rt["pooled"][h, tile_of[row] - npt]
            got = r["out"][row, h * d:(h + 1) * d]
            bar = P_.bf16_ulp(o) + flip + 1e-6
            worst = max(worst, float(np.max(np.abs(got - o) / bar)))
    assert worst <= 1.0, worst     # one bf16 spacing of the output plus the weight flips


def test_attention_equal_keys_one_key_and_two_key_closed_form():
    # all keys equal -> every weight 1 -> mean of v; scores 0 and ln 0.3 ->
    # p = (1, 0.3), bf(0.3) = 0.30078125 in the value product, 1.3 below
    d = 4
    sh = _sh(2, 0, 0, 1, d, top_k=1, pooled=0)
    ts = np.array([0, 2], np.int32)
    q = np.zeros((1, 2, d))
    q[0, :, 0] = math.sqrt(d)
    k = np.zeros((1, 2, d))
    k[0, 1, 0] = float(np.float32(math.log(0.3)))
    v = np.zeros((1, 2, d))
    v[0, 0, 0] = 1.0
    v[0, 1, 1] = 1.0
    kb = bits(O.round_bf16(k))
    s1 = float(np.float32(O.bf16_to_f64(kb)[0, 1, 0]))   # the bf16 score ~ ln 0.3
    p1 = float(np.float32(math.exp(s1)))
    out = C.attention(sh, ts, 1, bits(q), kb, bits(v), np.zeros((1, 0, 0)),
                      np.zeros((1, 0, d)))
    want = O.round_bf16(np.array([1.0 / (1.0 + p1), float(O.round_bf16(np.array([p1]))[0]) /
                                  (1.0 + p1), 0, 0]))
    np.testing.assert_array_equal(out[0], want)
    eq = C.attention(sh, ts, 1, bits(np.ones((1, 2, d))), bits(np.ones((1, 2, d))),
                     bits([[[2.0, 0, 0, 0], [4.0, 0, 0, 0]]]), np.zeros((1, 0, 0)),
                     np.zeros((1, 0, d)))
    np.testing.assert_array_equal(eq[:, 0], [3.0, 3.0])


def test_routed_with_all_tiles_equals_dense_bytes():
    ts, npt, q, k, v = _small_case(seed=11)
    nQ = len(ts) - 1 - npt
    sh = _sh(5, 7, 40, 2, 16, top_k=nQ, pooled=0)
    routed = C.routed_attn(sh, ts, npt, bits(q), bits(k), bits(v))
    dense_sh = _sh(52, 0, 0, 2, 16, top_k=1, pooled=0)
    dense = C.routed_attn(dense_sh, np.array([0, 52], np.int32), 1, bits(q), bits(k), bits(v))
    np.testing.assert_array_equal(routed["out_bits"], dense["out_bits"])


def test_attention_key_sets_by_counting():
    """q = 0: each output is the mean of v over the row's key set; one-hot v
    per tile counts the rows of each tile in it (dense prefix rows; prefix plus
    exactly the selected tiles for video rows; pooled only on video rows)."""
    ts = np.array([0, 3, 5, 9, 13, 17, 20], np.int32)
    npt, P, R, d = 2, 5, 20, 8
    tile_of = np.searchsorted(ts, np.arange(R), side="right") - 1
    v = np.zeros((1, R, d))
    v[0, np.arange(R), tile_of] = 1.0
    z = bits(np.zeros((1, R, d)))
    sh = _sh(3, 2, 15, 1, d, top_k=2, pooled=0)
    r = C.routed_attn(sh, ts, npt, z, z, bits(v))
    assert np.all(r["sel"] == [2, 3])                 # equal scores -> lower tiles
    lens = np.diff(ts)
    dense = O.round_bf16(np.concatenate([lens / R, [0, 0]]))
    vid = O.round_bf16(np.array([3, 2, 4, 4, 0, 0, 0, 0]) / (P + lens[2] + lens[3]))
    np.testing.assert_array_equal(r["out"][:P], np.tile(dense, (P, 1)))
    np.testing.assert_array_equal(r["out"][P:], np.tile(vid, (R - P, 1)))
    rp = C.routed_attn(sh.replace(pooled=1), ts, npt, z, z, bits(v))
    np.testing.assert_array_equal(rp["out"][:P], r["out"][:P])
    pooled = np.array([1 / 6.0] * 6 + [0, 0])
    np.testing.assert_array_equal(rp["out"][P:], np.tile(
        O.round_bf16(np.array([3, 2, 4, 4, 0, 0, 0, 0]) / 13.0 + pooled), (R - P, 1)))


def test_routing_selects_a_planted_tile():
    ts = np.array([0, 4, 8, 12, 16, 20], np.int32)     # 1 prefix tile, 4 video tiles
    d = 4
    q = np.zeros((1, 20, d))
    k = np.zeros((1, 20, d))
    q[0, :, 0] = 1.0
    k[0, 12:16, 0] = 2.0
    k[0, 16:20, 0] = -1.0
    sh = _sh(4, 0, 16, 1, d, top_k=1)
    r = C.routed_attn(sh, ts, 1, bits(q), bits(k), bits(np.zeros((1, 20, d))))
    assert np.all(r["sel"][0, :, 0] == 3)
    np.testing.assert_array_equal(r["scores"][0, 0], [0.0, 0.0, 0.0, 1.0, -0.5])


# ----------------------------------------------------------------------------
# Block and forward
# ----------------------------------------------------------------------------

def _tiny_block_inputs(seed=8, **kw):
    sh = S.Shape(8, 8, 48, 32, 2, 16, 64, tile=16, top_k=2, **kw)
    ts, npt = S.tile_map(sh)
    return (sh, ts, npt, S.block_weights(sh, seed=seed), S.modulation(sh, seed=seed),
            S.rope_tables(sh), S.activations(sh, seed=seed, field=True))


def test_block_zero_gates_is_identity():
    sh, ts, npt, w, mod, rope, x = _tiny_block_inputs()
    mod = mod.copy()
    mod[:, 2, :] = 0.0
    mod[:, 5, :] = 0.0
    r = C.block_forward(sh, ts, npt, w, mod, rope, x)
    np.testing.assert_array_equal(r["x2_bits"], x)


def test_block_sampled_rows_match_full():
    sh, ts, npt, w, mod, rope, x = _tiny_block_inputs()
    full = C.block_forward(sh, ts, npt, w, mod, rope, x)
    rows = np.array([0, 9, 17, 40, 63])
    part = C.block_forward(sh, ts, npt, w, mod, rope, x, out_rows=rows)
    np.testing.assert_array_equal(part["x2"], full["x2"][rows])


def test_only_head_v_rows_reach_that_heads_columns():
    sh, ts, npt, w, mod, rope, x = _tiny_block_inputs()
    d, H = sh.head_dim, 32
    w = dict(w)
    wq = np.zeros((3 * H, H), np.uint16)
    rows = np.arange(1 * 3 * d + 2 * d, 1 * 3 * d + 3 * d)
    wq[rows] = w["w_qkv"][rows]
    w["w_qkv"] = wq
    w["b_qkv"] = np.zeros(3 * H, np.uint16)
    a = C.block_forward(sh, ts, npt, w, mod, rope, x)["attn"]
    assert np.all(a[:, :d] == 0) and np.all(a[:, 2 * d:] == 0)
    assert np.count_nonzero(a[:, d:2 * d]) > 0.9 * a[:, d:2 * d].size


def test_pages_block_gate_ones_equals_ungated():
    """The routing gate (a fourth per-head block of y) multiplies the pooled
    branch: gate rows of zero weight and bias 1 give the ungated block."""
    sh, ts, npt, w, mod, rope, x = _tiny_block_inputs(mlp=1)
    shg = sh.replace(gate=1)
    wg = S.block_weights(shg, seed=8)
    d, nh, H = sh.head_dim, sh.n_heads, sh.hidden
    wq = wg["w_qkv"].reshape(nh, 4, d, H).copy()
    bq = wg["b_qkv"].reshape(nh, 4, d).copy()
    wq[:, :3] = w["w_qkv"].reshape(nh, 3, d, H)
    bq[:, :3] = w["b_qkv"].reshape(nh, 3, d)
    wq[:, 3] = 0
    bq[:, 3] = bits(1.0)
    wg = dict(w, w_qkv=wq.reshape(-1, H), b_qkv=bq.reshape(-1))
    a = C.block_forward(sh, ts, npt, w, mod, rope, x)
    b = C.block_forward(shg, ts, npt, wg, mod, rope, x)
    np.testing.assert_array_equal(a["x2"], b["x2"])


def test_final_heads_route_segments():
    sh = S.Shape(2, 3, 4, 4, 1, 4, 16)
    H = 4
    x = np.zeros((9, H))
    x[:2] = 7.0
    x[2:5] = 1.0
    x[5:] = -2.0
    mf = np.zeros((3, 2, H), np.float32)
    head = {"w_video": bits(np.eye(3, H)), "b_video": bits(np.zeros(3)),
            "w_audio": bits(np.ones((2, H))), "b_audio": bits(np.array([0.5, -0.5]))}
    seg = np.array([0, 0, 1, 1, 1, 2, 2, 2, 2])
    vv, va = C.final_heads(sh, bits(x), seg, mf, head)
    np.testing.assert_array_equal(va, np.tile([4.5, 3.5], (3, 1)))   # bf(0.9999995) = 1
    np.testing.assert_array_equal(vv, np.tile([-1.0, -1.0, -1.0], (4, 1)))


def test_dit_forward_with_identity_blocks_is_heads_only():
    sh, ts, npt, w, mod, rope, x = _tiny_block_inputs()
    mod = mod.copy()
    mod[:, 2, :] = 0
    mod[:, 5, :] = 0
    head = S.head_weights(sh)
    mf = S.final_modulation(sh)
    r = C.dit_forward(sh, ts, npt, [w, w], head, np.stack([mod, mod]), mf, rope, x)
    seg = O.row_segments(sh.n_text, sh.n_audio, sh.n_video)
    vv, va = C.final_heads(sh, x, seg, mf, head)
    np.testing.assert_array_equal(r["vel_video"], vv)
    np.testing.assert_array_equal(r["vel_audio"], va)


# ----------------------------------------------------------------------------
# Against the float64 oracle, determinism, self-noise
# ----------------------------------------------------------------------------

def _tiny_forward_inputs(L=2, seed=42):
    sh = S.TINY
    ts, npt = S.tile_map(sh)
    blocks = [S.block_weights(sh, seed=seed + l) for l in range(L)]
    mods = np.stack([S.modulation(sh, block=l, seed=seed) for l in range(L)])
    return (sh, ts, npt, blocks, S.head_weights(sh, seed=seed), mods,
            S.final_modulation(sh, seed=seed), S.rope_tables(sh),
            S.activations(sh, seed=seed, field=True))


def _metrics(got, ref):
    g, r = np.ravel(got), np.ravel(ref)
    return (float(g @ r / (np.linalg.norm(g) * np.linalg.norm(r))),
            float(np.linalg.norm(g - r) / np.linalg.norm(r)))


def test_agrees_with_float64_oracle_on_the_tiny_block_and_forward():
    """Two oracles, one definition: the fp32 sums of this one against the
    float64 sums of the other differ only by rounding, far inside the
    acceptance bar (cos >= 0.998, rel <= 0.06) on every intermediate."""
    sh, ts, npt, blocks, head, mods, mf, rope, x = _tiny_forward_inputs()
    a = O.block_forward(sh, ts, npt, blocks[0], mods[0], rope, x)
    b = C.block_forward(sh, ts, npt, blocks[0], mods[0], rope, x)
    for k_ in ("n1", "y", "q", "k", "v", "qbar", "kbar", "vbar", "scores", "pooled", "attn", "o",
               "x1", "n2", "h", "f", "x2"):
        cos, rel = _metrics(b[k_], a[k_])
        assert cos > 0.99999 and rel < 2e-3, (k_, cos, rel)
    import parity as P
    checked, bad, _ = P.selection_agrees(b["sel"], a["sel"], a["scores"], npt, sh.top_k)
    assert bad == 0 and checked > 0.9 * sh.n_heads * (len(ts) - 1 - npt)
    fa = O.dit_forward(sh, ts, npt, blocks, head, mods, mf, rope, x)
    fb = C.dit_forward(sh, ts, npt, blocks, head, mods, mf, rope, x)
    for k_ in ("vel_video", "vel_audio"):
        cos, rel = _metrics(fb[k_], fa[k_])
        assert cos > 0.99999 and rel < 1e-3, (k_, cos, rel)


def test_bytes_do_not_depend_on_thread_count():
    sh, ts, npt, blocks, head, mods, mf, rope, x = _tiny_forward_inputs()
    prev = C.set_threads(1)
    try:
        outs = []
        for n in (1, 3, 8):
            C.set_threads(n)
            r = C.dit_forward(sh, ts, npt, blocks, head, mods, mf, rope, x)
            outs.append((r["x_bits"].tobytes(), r["vel_video"].tobytes(),
                         r["vel_audio"].tobytes()))
        assert outs[0] == outs[1] == outs[2]
        r2 = C.dit_forward(sh, ts, npt, blocks, head, mods, mf, rope, x)
        assert (r2["x_bits"].tobytes(), r2["vel_video"].tobytes(),
                r2["vel_audio"].tobytes()) == outs[2]
    finally:
        C.set_threads(prev)


def test_self_noise_floor_of_reversed_tile_sums():
    """The pages measure their own floor by summing the tile scores in reverse
    ("TensorFold PR #949", Receipts: the self-noise rows of the parity table).
    Reversing the tile-mean and tile-score sums must change fp32 tile scores
    (else the measurement is vacuous); the velocities it moves must stay far
    inside the acceptance bar.  On this tiny forward no selection flips and
    the floor is exactly zero; the full-size floor is measured by
    tests/golden/make_full_velocity.py."""
    sh, ts, npt, blocks, head, mods, mf, rope, x = _tiny_forward_inputs()
    a = C.block_forward(sh, ts, npt, blocks[0], mods[0], rope, x)
    b = C.block_forward(sh, ts, npt, blocks[0], mods[0], rope, x,
                        reverse=C.REV_MEANS | C.REV_SCORES)
    assert np.count_nonzero(a["scores"] != b["scores"]) > 0.1 * a["scores"].size
    np.testing.assert_allclose(b["scores"], a["scores"], rtol=1e-5, atol=1e-6)
    fwd = C.dit_forward(sh, ts, npt, blocks, head, mods, mf, rope, x)
    rev = C.dit_forward(sh, ts, npt, blocks, head, mods, mf, rope, x,
                        reverse=C.REV_MEANS | C.REV_SCORES)
    for k_ in ("vel_video", "vel_audio"):
        cos, rel = _metrics(rev[k_], fwd[k_])
        assert cos > 0.9999 and rel < 1e-2, (k_, cos, rel)
