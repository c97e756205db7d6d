"""Pins of the CPU oracle against facts it does not compute itself: closed
forms, invariants, library routines, textbook constants and the top-k rule
as the pages state it.  All run on the CPU."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import h3_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


class Sh:
    def __init__(self, n_text, n_audio, n_video, n_heads, head_dim, top_k, pooled=1, eps=1e-6):
        self.n_text, self.n_audio, self.n_video = n_text, n_audio, n_video
        self.n_heads, self.head_dim, self.top_k, self.pooled = n_heads, head_dim, top_k, pooled
        self.norm_eps = eps


def bits(x):
    """float64 bf16-exact values -> bits (via torch, an independent route)."""
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------
# bf16 / fp32 rounding
# ----------------------------------------------------------------------------

def test_round_bf16_known_values():
    one = 1.0
    cases = {
        one: one,
        one + 2 ** -8: one,                       # tie -> even (1.0)
        one + 3 * 2 ** -8: one + 2 ** -6,         # tie -> even (odd lsb rounds up)
        one + 2 ** -8 + 2 ** -40: one + 2 ** -7,  # just above the tie: up
        one + 2 ** -9: one,
        -(one + 2 ** -7): -(one + 2 ** -7),
        0.3: 0.30078125,
        1.5 * 2 ** -133: 2 ** -132,               # subnormal tie -> even
        2.5 * 2 ** -133: 2 * 2 ** -133,
        0.0: 0.0,
        3.5e38: math.inf,                         # beyond the largest finite bf16
        -3.5e38: -math.inf,
        (2 - 2 ** -7) * 2 ** 127: (2 - 2 ** -7) * 2 ** 127,
    }
    xs = np.array(list(cases.keys()))
    got = O.round_bf16(xs)
    np.testing.assert_array_equal(got, np.array(list(cases.values())))
    assert np.isnan(O.round_bf16(np.array([np.nan]))[0])


def test_round_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(0)
    x32 = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 7,
                          (rng.standard_normal(20000) * 1e-39).astype(np.float32)])
    ref = torch.tensor(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(x32.astype(np.float64)), ref)


def test_bf16_bits_roundtrip():
    rng = np.random.default_rng(1)
    x = O.round_bf16(rng.standard_normal(5000) * 3)
    b = O.f64_to_bf16_bits(x)
    np.testing.assert_array_equal(b, bits(x))
    np.testing.assert_array_equal(O.bf16_to_f64(b), x)


def test_round_f32():
    got = O.round_f32(np.array([1 + 2 ** -24, 1 + 3 * 2 ** -24, 1 + 2 ** -23]))
    np.testing.assert_array_equal(got, [1.0, 1 + 2 ** -22, 1 + 2 ** -23])


# ----------------------------------------------------------------------------
# Norm, linear, activation
# ----------------------------------------------------------------------------

def test_modnorm_closed_forms():
    H, eps = 8, 1e-6
    seg = np.array([0, 1, 2, 2])
    x = np.zeros((4, H))
    x[0] = 3.0                                   # constant row
    x[1] = 0.0                                   # zero row -> shift
    x[2, :4] = 1.0; x[2, 4:] = -1.0              # unit RMS row
    x[3] = np.arange(H)
    shift = np.zeros((3, H)); scale = np.zeros((3, H))
    shift[1] = 0.25
    scale[2] = 1.0                               # (1 + 1) doubles video rows
    y = O.modulated_rmsnorm(x, shift, scale, seg, eps)
    np.testing.assert_array_equal(y[0], O.round_bf16(np.full(H, 3.0 / math.sqrt(9.0 + eps))))
    np.testing.assert_array_equal(y[1], np.full(H, 0.25))
    np.testing.assert_array_equal(y[2], O.round_bf16(2.0 * x[2] / math.sqrt(1.0 + eps)))
    rms3 = math.sqrt(np.mean(np.arange(H) ** 2.0) + eps)
    np.testing.assert_array_equal(y[3], O.round_bf16(2.0 * np.arange(H) / rms3))


def test_modnorm_unit_rms_random_rows():
    rng = np.random.default_rng(2)
    x = O.round_bf16(rng.standard_normal((16, 256)) * 5)
    z = np.zeros((3, 256))
    y = O.modulated_rmsnorm(x, z, z, np.zeros(16, dtype=int), 1e-6)
    rms = np.sqrt(np.mean(y * y, axis=1))
    np.testing.assert_allclose(rms, 1.0, atol=2 ** -8)


def test_linear_worked_example():
    a = np.array([[1.0, 2.0], [3.0, -1.0]])
    w = np.array([[1.0, 2.0], [0.0, 1.0]])       # out0 = a0 + 2 a1, out1 = a1
    b = np.array([0.5, -0.5])
    np.testing.assert_array_equal(O.linear(a, w, b), [[5.5, 1.5], [1.5, -1.5]])
    np.testing.assert_array_equal(O.linear(a, np.zeros((3, 2)), np.array([1.0, 2, 3])),
                                  [[1, 2, 3], [1, 2, 3]])


def test_gelu_textbook_values():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "normal_cdf.txt"))
            if l.strip() and not l.startswith("#")]
    z = np.array([float(r[0]) for r in rows])
    phi = np.array([float(r[1]) for r in rows])
    np.testing.assert_allclose(O.gelu(z), z * phi, rtol=1e-13, atol=1e-15)
    assert O.gelu(np.array([40.0]))[0] == 40.0
    assert O.gelu(np.array([-40.0]))[0] == 0.0


# ----------------------------------------------------------------------------
# Heads, QK norm and RoPE
# ----------------------------------------------------------------------------

def test_split_qkv_interleaved_per_head():
    nh, d, R = 3, 2, 2
    y = np.arange(R * nh * 3 * d, dtype=np.float64).reshape(R, nh * 3 * d)
    q, k, v = O.split_qkv(y, nh, d)
    # row 1, head 2: columns [2*3*2 + 0..2) are q, [+2..4) k, [+4..6) v
    base = 1 * nh * 3 * d + 2 * 3 * d
    np.testing.assert_array_equal(q[2, 1], [base, base + 1])
    np.testing.assert_array_equal(k[2, 1], [base + 2, base + 3])
    np.testing.assert_array_equal(v[2, 1], [base + 4, base + 5])


def test_qk_norm_gain_and_identity_tables():
    rng = np.random.default_rng(3)
    d = 64
    u = O.round_bf16(rng.standard_normal((2, 5, d)) * 3)
    gain = np.full(d, 2.0)
    out = O.qk_norm_rope(u, gain, None, 1e-6)
    np.testing.assert_allclose(np.sqrt(np.mean(out ** 2, axis=-1)), 2.0, rtol=2 ** -8)
    tab = np.zeros((5, d // 2, 2), dtype=np.float32)
    tab[..., 0] = 1.0
    np.testing.assert_array_equal(O.qk_norm_rope(u, gain, tab, 1e-6), out)


def test_rope_quarter_turn_and_pairing():
    # d = 4: pairs (0, 2) and (1, 3).  Rotate pair 0 by 90 degrees, pair 1 by 0.
    u = np.array([[[1.0, 1.0, -1.0, -1.0]]])     # RMS 1 -> unchanged by the norm
    tab = np.zeros((1, 2, 2), dtype=np.float32)
    tab[0, 0] = (0.0, 1.0)                       # cos 0, sin 1
    tab[0, 1] = (1.0, 0.0)
    out = O.qk_norm_rope(u, np.ones(4), tab, 0.0)
    # pair 0: (a, b) = (1, -1) -> (a c - b s, b c + a s) = (1, 1); pair 1 unchanged
    np.testing.assert_array_equal(out[0, 0], [1.0, 1.0, 1.0, -1.0])


def test_rope_preserves_norm_and_relative_position():
    rng = np.random.default_rng(4)
    d, R = 32, 40
    inv = 10000.0 ** (-2.0 * np.arange(d // 2) / d)
    def tables(pos):
        ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
        t = np.empty((len(pos), d // 2, 2), dtype=np.float32)
        t[..., 0] = np.cos(ang); t[..., 1] = np.sin(ang)
        return t
    q = O.round_bf16(rng.standard_normal((1, R, d)))
    k = O.round_bf16(rng.standard_normal((1, R, d)))
    base = O.qk_norm_rope(q, np.ones(d), None, 1e-6)
    rq = O.qk_norm_rope(q, np.ones(d), tables(np.arange(R)), 1e-6)
    np.testing.assert_allclose(np.linalg.norm(rq, axis=-1), np.linalg.norm(base, axis=-1),
                               rtol=2 ** -7)
    # q at position m, k at position n: the product depends on m - n only
    q1 = np.repeat(q[:, :1], 2, axis=1)
    k1 = np.repeat(k[:, :1], 2, axis=1)
    a = O.qk_norm_rope(q1, np.ones(d), tables([7, 107]), 1e-6)
    b = O.qk_norm_rope(k1, np.ones(d), tables([3, 103]), 1e-6)
    dots = np.sum(a[0] * b[0], axis=-1)
    assert abs(dots[0] - dots[1]) < 0.05 * np.abs(dots).max() + 0.05


# ----------------------------------------------------------------------------
# Routing
# ----------------------------------------------------------------------------

def test_tile_means_constant_and_ragged_divisor():
    u = np.zeros((1, 7, 2))
    u[0, :4] = 5.0
    u[0, 4:, 0] = [1.0, 2.0, 6.0]
    ts = np.array([0, 4, 7])
    m = O.tile_means(u, ts, [0, 1])
    np.testing.assert_array_equal(m[0, 0], [5.0, 5.0])
    np.testing.assert_array_equal(m[0, 1], [3.0, 0.0])
    # fp32 rounding of the mean: 1/3 is not representable
    u2 = np.zeros((1, 3, 1)); u2[0, 0, 0] = 1.0
    assert O.tile_means(u2, np.array([0, 3]), [0])[0, 0, 0] == float(np.float32(1 / 3))


def test_tile_scores_worked_example():
    qbar = np.array([[[1.0, 2.0]]])
    kbar = np.array([[[3.0, 4.0], [-1.0, 0.5]]])
    S = O.tile_scores(qbar, kbar)
    np.testing.assert_array_equal(S[0, 0], [float(np.float32(11 / math.sqrt(2))), 0.0])


def test_topk_rule_golden():
    g = json.load(open(os.path.join(GOLDEN, "topk_rule.json")))
    for c in g["cases"]:
        s = np.array([float(v) for v in c["scores"]])
        got = O.topk_tiles(s, np.arange(len(s)), c["k"])
        assert list(got) == c["expect"], c


def test_topk_candidates_are_absolute_ids():
    s = np.array([9.0, 9.0, 1.0, 3.0, 2.0])
    got = O.topk_tiles(s, np.arange(2, 5), 2)     # prefix tiles 0, 1 excluded
    assert list(got) == [3, 4]


def test_pooled_closed_forms():
    vbar = np.array([[1.0, 0.0], [0.0, 1.0]])
    np.testing.assert_allclose(O.pooled_branch(np.array([0.0, math.log(3.0)]), vbar),
                               [0.25, 0.75], rtol=1e-15)
    np.testing.assert_array_equal(O.pooled_branch(np.array([2.0]), vbar[:1]), [1.0, 0.0])
    np.testing.assert_allclose(O.pooled_branch(np.array([1.0, 1.0, 1.0]),
                                               np.array([[3.0], [6.0], [9.0]])), [6.0])


# ----------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------

def test_softmax_equal_keys_one_key_and_two_key_closed_form():
    rng = np.random.default_rng(5)
    d = 4
    q = rng.standard_normal((3, d))
    k = np.tile(rng.standard_normal(d), (6, 1))
    v = rng.standard_normal((6, d))
    np.testing.assert_allclose(O.softmax_rows_bf16p(q, k, v), np.tile(v.mean(0), (3, 1)),
                               rtol=1e-14)
    np.testing.assert_allclose(O.softmax_rows_bf16p(q, k[:1], v[:1]), np.tile(v[0], (3, 1)),
                               rtol=1e-15)
    # scores 0 and ln 0.3: p = (1, 0.3), bf(0.3) = 0.30078125, denominator 1.3
    qq = np.array([[math.sqrt(d), 0, 0, 0]])
    kk = np.array([[0.0, 1, 0, 0], [math.log(0.3), 0, 0, 0]])
    vv = np.array([[1.0, 0, 0, 0], [0.0, 1, 0, 0]])
    got = O.softmax_rows_bf16p(qq, kk, vv)
    np.testing.assert_allclose(got[0], [1 / 1.3, 0.30078125 / 1.3, 0, 0], rtol=1e-14)


def test_softmax_near_library_sdpa():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((17, 64)); k = rng.standard_normal((50, 64)); v = rng.standard_normal((50, 64))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None], torch.tensor(k)[None], torch.tensor(v)[None])[0].numpy()
    got = O.softmax_rows_bf16p(q, k, v)
    # the only difference is bf16 rounding of the weights: relative 2^-9 per weight
    assert np.max(np.abs(got - ref)) < 2 ** -8 * np.max(np.abs(v))
    assert np.max(np.abs(got - ref)) > 0          # the rounding is really applied


def _small_case(seed=7, n_text=5, n_audio=7, n_video=40, tile=8, nh=2, d=16):
    rng = np.random.default_rng(seed)
    R = n_text + n_audio + n_video
    starts = list(range(0, n_text, tile)) + [n_text + s for s in range(0, n_audio, tile)]
    npt = len(starts)
    starts += [n_text + n_audio + s for s in range(0, n_video, tile)] + [R]
    q = O.round_bf16(rng.standard_normal((nh, R, d)))
    k = O.round_bf16(rng.standard_normal((nh, R, d)))
    v = O.round_bf16(rng.standard_normal((nh, R, d)))
    return np.array(starts), npt, q, k, v


def test_routed_with_all_tiles_equals_dense():
    ts, npt, q, k, v = _small_case()
    P = 12
    nQ = len(ts) - 1 - npt
    rt = O.routing(q, k, v, ts, npt, nQ)
    routed = O.attention(q, k, v, ts, npt, P, rt, use_pooled=False)
    R = q.shape[1]
    dense = np.concatenate([O.softmax_rows_bf16p(q[h], k[h], v[h]) for h in range(q.shape[0])],
                           axis=1)
    np.testing.assert_array_equal(routed, dense)


def test_attention_key_sets_by_counting():
    """q = 0 makes every score 0, so each row's output is the mean of v over
    its key set; v = one-hot of the key's tile counts the rows of every tile
    in that set.  Pins: dense prefix rows, prefix keys plus exactly the
    selected tiles for video rows, the pooled term added for video rows only."""
    ts = np.array([0, 3, 5, 9, 13, 17, 20])        # 2 prefix tiles, 4 video tiles
    npt, P, R, nT = 2, 5, 20, 6
    d = 8
    tile_of = np.searchsorted(ts, np.arange(R), side="right") - 1
    q = np.zeros((1, R, d))
    k = np.zeros((1, R, d))
    v = np.zeros((1, R, d))
    v[0, np.arange(R), tile_of] = 1.0
    rt = O.routing(q, k, v, ts, npt, 2)
    # all scores equal -> ties to the lower video tiles: 2 and 3
    assert np.all(rt["sel"] == [2, 3])
    np.testing.assert_allclose(rt["pooled"][0, 0], [1 / 6.0] * 6 + [0, 0])
    out = O.attention(q, k, v, ts, npt, P, rt, use_pooled=False)
    lens = np.diff(ts)
    dense = np.concatenate([lens / R, [0, 0]])
    for r in range(P):
        np.testing.assert_allclose(out[r], dense, rtol=1e-15)
    n_keys = P + lens[2] + lens[3]
    vid = np.array([3, 2, 4, 4, 0, 0, 0, 0]) / n_keys
    for r in range(P, R):
        np.testing.assert_allclose(out[r], vid, rtol=1e-15)
    outp = O.attention(q, k, v, ts, npt, P, rt, use_pooled=True)
    np.testing.assert_allclose(outp[:P], out[:P], rtol=0)
    np.testing.assert_allclose(outp[P:], out[P:] + np.array([1 / 6.0] * 6 + [0, 0]), rtol=1e-15)


def test_routing_selects_by_scores():
    """Video tile 3's keys point along q's direction, so every video query
    tile must pick tile 3 first; scores follow the worked formula."""
    ts = np.array([0, 4, 8, 12, 16, 20])          # 1 prefix tile, 4 video tiles
    d = 4
    q = np.zeros((1, 20, d)); k = np.zeros((1, 20, d)); v = np.zeros((1, 20, d))
    q[0, :, 0] = 1.0
    k[0, 12:16, 0] = 2.0
    k[0, 16:20, 0] = -1.0
    rt = O.routing(q, k, v, ts, 1, 1)
    assert np.all(rt["sel"][0, :, 0] == 3)
    np.testing.assert_array_equal(rt["scores"][0, 0], [0.0, 0.0, 0.0, 1.0, -0.5])


# ----------------------------------------------------------------------------
# Block and forward
# ----------------------------------------------------------------------------

def _tiny_block_inputs(seed=8):
    from audio_diffusion_transformer_amd import synth as S
    sh = S.Shape(8, 8, 48, 32, 2, 16, 64, tile=16, top_k=2)
    ts, npt = S.tile_map(sh)
    w = S.block_weights(sh, seed=seed)
    mod = S.modulation(sh, seed=seed)
    rope = S.rope_tables(sh)
    x = S.activations(sh, seed=seed, field=True)
    return sh, ts, npt, w, mod, rope, x


def test_block_zero_gates_is_identity():
    sh, ts, npt, w, mod, rope, x = _tiny_block_inputs()
    mod = mod.copy()
    mod[:, 2, :] = 0.0
    mod[:, 5, :] = 0.0
    r = O.block_forward(sh, ts, npt, w, mod, rope, x)
    np.testing.assert_array_equal(O.f64_to_bf16_bits(r["x2"]), x)


def test_block_gate_wiring_and_determinism():
    sh, ts, npt, w, mod, rope, x = _tiny_block_inputs()
    r1 = O.block_forward(sh, ts, npt, w, mod, rope, x)
    r2 = O.block_forward(sh, ts, npt, w, mod, rope, x)
    np.testing.assert_array_equal(r1["x2"], r2["x2"])
    seg = O.row_segments(sh.n_text, sh.n_audio, sh.n_video)
    g1 = mod[:, 2, :].astype(np.float64)[seg]
    g2 = mod[:, 5, :].astype(np.float64)[seg]
    xf = O.bf16_to_f64(x)
    np.testing.assert_array_equal(r1["x1"], O.round_bf16(xf + g1 * r1["o"]))
    np.testing.assert_array_equal(r1["x2"], O.round_bf16(r1["x1"] + g2 * r1["f"]))
    # only the mlp branch off: x2 == x1
    mod2 = mod.copy(); mod2[:, 5, :] = 0
    r3 = O.block_forward(sh, ts, npt, w, mod2, rope, x)
    np.testing.assert_array_equal(r3["x2"], r1["x1"])


def test_block_sampled_rows_match_full():
    sh, ts, npt, w, mod, rope, x = _tiny_block_inputs()
    full = O.block_forward(sh, ts, npt, w, mod, rope, x)
    rows = np.array([0, 9, 17, 40, 63])
    part = O.block_forward(sh, ts, npt, w, mod, rope, x, out_rows=rows)
    np.testing.assert_array_equal(part["x2"], full["x2"][rows])


def test_only_head_v_rows_reach_that_heads_columns():
    """With W_qkv nonzero only in head 1's v rows (and zero biases), every
    attention output column outside head 1's slot [d, 2d) is zero."""
    sh, ts, npt, w, mod, rope, x = _tiny_block_inputs()
    d, H = sh.head_dim, 32
    w = dict(w)
    wq = np.zeros((3 * H, H), dtype=np.uint16)
    rows = np.arange(1 * 3 * d + 2 * d, 1 * 3 * d + 3 * d)
    wq[rows] = w["w_qkv"][rows]
    w["w_qkv"] = wq
    w["b_qkv"] = np.zeros(3 * H, dtype=np.uint16)
    r = O.block_forward(sh, ts, npt, w, mod, rope, x)
    a = r["attn"]
    assert np.all(a[:, :d] == 0) and np.all(a[:, 2 * d:] == 0)
    assert np.count_nonzero(a[:, d:2 * d]) > 0.9 * a[:, d:2 * d].size


def test_final_heads_route_segments():
    sh = Sh(2, 3, 4, 1, 4, 1)
    H = 4
    x = np.zeros((9, H))
    x[:2] = 7.0            # text rows: must not reach any head
    x[2:5] = 1.0
    x[5:] = -2.0
    mf = np.zeros((3, 2, H), dtype=np.float32)
    head = {"w_video": bits(np.eye(3, H)), "b_video": bits(np.zeros(3)),
            "w_audio": bits(np.ones((2, H))), "b_audio": bits(np.array([0.5, -0.5]))}
    vv, va = O.final_heads(sh, x, mf, head)
    za = float(O.round_bf16(np.array([1.0 / math.sqrt(1.0 + 1e-6)]))[0])
    np.testing.assert_allclose(va, np.tile([4 * za + 0.5, 4 * za - 0.5], (3, 1)), rtol=1e-15)
    np.testing.assert_allclose(vv, np.tile([-za, -za, -za], (4, 1)), rtol=1e-15)


def test_dit_forward_with_identity_blocks_is_heads_only():
    sh, ts, npt, w, mod, rope, x = _tiny_block_inputs()
    from audio_diffusion_transformer_amd import synth as S
    mod = mod.copy(); mod[:, 2, :] = 0; mod[:, 5, :] = 0
    head = S.head_weights(sh)
    mf = S.final_modulation(sh)
    r = O.dit_forward(sh, ts, npt, [w, w], head, [mod, mod], mf, rope, x)
    vv, va = O.final_heads(sh, O.bf16_to_f64(x), mf, head)
    np.testing.assert_array_equal(r["vel_video"], vv)
    np.testing.assert_array_equal(r["vel_audio"], va)


# ----------------------------------------------------------------------------
# The pages' own block: SwiGLU MLP, the routing gate, attention width != hidden,
# cube tiles
# ----------------------------------------------------------------------------

def test_silu_identities():
    x = np.linspace(-8, 8, 161)
    # silu(x) - silu(-x) = x (sigmoid(x) + sigmoid(-x) = 1)
    np.testing.assert_allclose(O.silu(x) - O.silu(-x), x, rtol=0, atol=1e-14)
    assert O.silu(0.0) == 0.0
    # sigmoid(ln 3) = 3/4
    assert abs(O.silu(math.log(3.0)) - 0.75 * math.log(3.0)) < 1e-15
    # large arguments: silu(x) -> x, silu(-x) -> 0 from below
    assert abs(O.silu(40.0) - 40.0) < 1e-12 and -1e-12 < O.silu(-40.0) <= 0.0


def test_swiglu_interleave_against_separate_products():
    """An FC1 weight assembled feature by feature from separate gate and up
    matrices (gate rows of features 16b..16b+15, then their up rows) gives
    bf(silu(bf(n Wg^T + bg)) * bf(n Wu^T + bu))."""
    rng = np.random.default_rng(3)
    R, H, F = 5, 24, 48
    n = O.round_bf16(rng.standard_normal((R, H)))
    wg, wu = O.round_bf16(rng.standard_normal((F, H))), O.round_bf16(rng.standard_normal((F, H)))
    bg, bu = O.round_bf16(rng.standard_normal(F)), O.round_bf16(rng.standard_normal(F))
    w1 = np.zeros((2 * F, H)); b1 = np.zeros(2 * F)
    for f in range(F):
        blk, j = divmod(f, 16)
        w1[32 * blk + j] = wg[f]; b1[32 * blk + j] = bg[f]
        w1[32 * blk + 16 + j] = wu[f]; b1[32 * blk + 16 + j] = bu[f]
    h = O.swiglu_hidden(O.linear(n, w1, b1), F)
    g = O.round_bf16(n @ wg.T + bg)
    u = O.round_bf16(n @ wu.T + bu)
    expect = O.round_bf16(g * u / (1.0 + np.exp(-g)))
    np.testing.assert_array_equal(h, expect)


def test_routed_attention_gate_ones_and_zeros():
    from audio_diffusion_transformer_amd import synth as S
    ts, npt, q, k, v = _small_case()
    nh, R, d = q.shape
    sh = S.Shape(5, 7, 40, nh * d, nh, d, 64, tile=8, top_k=2, pooled=1)
    qb, kb, vb = (O.f64_to_bf16_bits(t) for t in (q, k, v))
    base = O.routed_attn(sh, ts, npt, qb, kb, vb)
    ones = O.routed_attn(sh, ts, npt, qb, kb, vb, gate=np.full((nh, R, d), 0x3F80, np.uint16))
    np.testing.assert_array_equal(ones["out"], base["out"])
    zero = O.routed_attn(sh, ts, npt, qb, kb, vb, gate=np.zeros((nh, R, d), np.uint16))
    no_pool = O.routed_attn(sh.replace(pooled=0), ts, npt, qb, kb, vb)
    np.testing.assert_array_equal(zero["out"], no_pool["out"])
    # a gate of two doubles the pooled term exactly (before the final rounding)
    P = sh.n_text + sh.n_audio
    two = O.routed_attn(sh, ts, npt, qb, kb, vb, gate=np.full((nh, R, d), 0x4000, np.uint16))
    assert not np.array_equal(two["out"][P:], base["out"][P:])
    np.testing.assert_array_equal(two["out"][:P], base["out"][:P])


def _fasth3_tiny_inputs(seed=11):
    from audio_diffusion_transformer_amd import synth as S
    sh = S.Shape(6, 10, 60, 32, 2, 24, 32, tile=16, top_k=3, mlp=1, gate=1,
                 video_grid=(3, 4, 5), cube=2)
    ts, npt = S.tile_map(sh)
    w = S.block_weights(sh, seed=seed)
    mod = S.modulation(sh, seed=seed)
    rope = S.rope_tables(sh)
    x = S.activations(sh, seed=seed, field=True)
    return sh, ts, npt, w, mod, rope, x


def test_fasth3_block_shapes_and_identity():
    """Attention width 48 != hidden 32, SwiGLU and the gate: zero residual gates
    still give the identity, byte for byte."""
    sh, ts, npt, w, mod, rope, x = _fasth3_tiny_inputs()
    assert w["w_qkv"].shape == (4 * 48, 32) and w["w_o"].shape == (32, 48)
    assert w["w_fc1"].shape == (64, 32) and w["w_fc2"].shape == (32, 32)
    r = O.block_forward(sh, ts, npt, w, mod, rope, x)
    assert r["attn"].shape == (sh.rows, 48) and r["h"].shape == (sh.rows, 32)
    m0 = mod.copy(); m0[:, 2, :] = 0.0; m0[:, 5, :] = 0.0
    r0 = O.block_forward(sh, ts, npt, w, m0, rope, x)
    np.testing.assert_array_equal(O.f64_to_bf16_bits(r0["x2"]), x)


def test_fasth3_unit_gate_equals_ungated_block():
    """With the gate rows of the QKV product zero and their bias 1, g = 1 and the
    block equals the block without a gate on the same q/k/v rows: this pins the
    four-part per-head split."""
    sh, ts, npt, w, mod, rope, x = _fasth3_tiny_inputs()
    nh, d, H = sh.n_heads, sh.head_dim, sh.hidden
    wq4 = w["w_qkv"].reshape(nh, 4, d, H).copy()
    bq4 = w["b_qkv"].reshape(nh, 4, d).copy()
    wq4[:, 3] = 0
    bq4[:, 3] = 0x3F80                       # bf16 1.0
    wg = dict(w, w_qkv=wq4.reshape(-1, H), b_qkv=bq4.reshape(-1))
    w3 = dict(w, w_qkv=np.ascontiguousarray(wq4[:, :3]).reshape(-1, H),
              b_qkv=np.ascontiguousarray(bq4[:, :3]).reshape(-1))
    rg = O.block_forward(sh, ts, npt, wg, mod, rope, x)
    r3 = O.block_forward(sh.replace(gate=0), ts, npt, w3, mod, rope, x)
    np.testing.assert_array_equal(rg["x2"], r3["x2"])
    # and a zero gate equals the block with the pooled branch off
    bq4[:, 3] = 0
    wz = dict(w, w_qkv=wq4.reshape(-1, H), b_qkv=bq4.reshape(-1))
    rz = O.block_forward(sh, ts, npt, wz, mod, rope, x)
    rp = O.block_forward(sh.replace(gate=0, pooled=0), ts, npt, w3, mod, rope, x)
    np.testing.assert_array_equal(rz["x2"], rp["x2"])


def test_cube_tiles_cover_the_grid():
    from audio_diffusion_transformer_amd import synth as S
    sh = S.FASTH3
    ts, npt = S.tile_map(sh)
    assert npt == 8 and len(ts) - 1 - npt == 280 and ts[-1] == sh.rows
    sizes = np.diff(ts[npt:])
    assert sizes.max() == 64 and sizes.sum() == sh.n_video
    # the 4x4x4 cube cut of 37 x 15 x 27: edges 1, 3, 3 -> cube sizes are products
    # of {4, 1} x {4, 3} x {4, 3}
    assert set(sizes.tolist()) <= {a * b * c for a in (4, 1) for b in (4, 3) for c in (4, 3)}
    pos = S.video_positions(sh)
    assert np.array_equal(np.sort(pos), np.arange(sh.n_video))   # a permutation
    # every tile is one cube: its raster positions span at most 4 frames, rows, columns
    T, Hh, W = sh.video_grid
    for i in range(len(sizes)):
        p = pos[ts[npt + i] - sh.n_prefix:ts[npt + i + 1] - sh.n_prefix]
        t, h, w = p // (Hh * W), (p // W) % Hh, p % W
        assert t.max() - t.min() < 4 and h.max() - h.min() < 4 and w.max() - w.min() < 4
        assert len(p) == (t.max() - t.min() + 1) * (h.max() - h.min() + 1) * (w.max() - w.min() + 1)


# ----------------------------------------------------------------------------
# Rows in, time conditioning, modulation tables, the Euler loop
# ----------------------------------------------------------------------------

def test_timestep_embedding_closed_forms():
    e0 = O.timestep_embedding(0.0)
    np.testing.assert_array_equal(e0, np.r_[np.ones(128), np.zeros(128)])
    e = O.timestep_embedding(100.0 * math.pi)
    # w_0 = 1 and w_64 = 10000^(-1/2) = 1/100: cos(100 pi) = 1, cos(pi) = -1
    assert abs(e[0] - 1.0) < 1e-12 and abs(e[128]) < 1e-12
    assert abs(e[64] + 1.0) < 1e-12 and abs(e[128 + 64]) < 1e-12
    assert abs(e[127] - math.cos(100.0 * math.pi * 10000.0 ** (-127 / 128))) < 1e-12


def _time_w(H=2, L=1):
    z = lambda *s: np.zeros(s)
    tw = {"w1": z(H, 256), "b1": z(H), "w2": z(H, H), "b2": z(H), "w_mod": z(6 * H, H),
          "b_mod": z(6 * H), "mod_table": z(L, 6, H), "w_final": z(2 * H, H), "b_final": z(2 * H)}
    return tw


def test_time_conditioning_hand_example():
    tw = _time_w()
    tw["w1"][0, 0] = 1.0          # (W1 e)_0 = e_0 = cos(t)
    tw["w1"][1, 0] = -1.0         # (W1 e)_1 = -cos(t)
    tw["w2"][:] = [[0.0, 1.0], [2.0, 0.0]]
    tw["b2"][:] = [0.5, 0.0]
    tb = {k: bits(v) for k, v in tw.items()}
    s1, sm1 = 0.7310585786300049, -0.2689414213699951   # silu(1) = logistic(1), silu(-1)
    c = O.time_conditioning(0.0, tb)                     # t = 0: e_0 = 1
    np.testing.assert_allclose(c, [sm1 + 0.5, 2 * s1], rtol=1e-14)
    c = O.time_conditioning(math.pi / O.T_SCALE, tb)     # t = pi: e_0 = -1
    np.testing.assert_allclose(c, [s1 + 0.5, 2 * sm1], rtol=1e-6)


def test_modulation_tables_layout_and_segments():
    H, L = 2, 3
    tw = _time_w(H, L)
    tw["b_mod"][:] = np.arange(6 * H) * 0.125            # entry j*H + c -> mod[.][.][j][c]
    tw["mod_table"][:] = np.arange(L)[:, None, None] * 4.0
    tw["b_final"][:] = -np.arange(2 * H) * 0.5
    tw["w1"][0, 0] = 1.0
    tw["w2"][0, 0] = 1.0
    tw["w_mod"][:, 0] = 0.25                             # m depends on the segment's timestep
    tb = {k: bits(v) for k, v in tw.items()}
    sh = Sh(1, 1, 1, 1, 2, 1)
    sh.hidden = H
    mod, fin = O.modulation_tables(sh, L, tb, np.array([0.0, 0.5, math.pi / O.T_SCALE]))
    assert mod.shape == (L, 3, 6, H) and fin.shape == (3, 2, H)
    # segment 0 (t = 0): c_0 = silu(1); m = 0.25 silu(c_0) + b_mod
    m0 = 0.25 * float(O.silu(np.array([0.7310585786300049]))[0])
    for l in range(L):
        for j in range(6):
            for c in range(H):
                assert abs(mod[l, 0, j, c] - (m0 + 0.125 * (j * H + c) + 4.0 * l)) < 1e-5
    np.testing.assert_array_equal(fin[:, 0, 1], [-0.5] * 3)
    np.testing.assert_array_equal(fin[:, 1, 1], [-1.5] * 3)
    # the block table shifts every segment alike; the segments differ by their timesteps
    # (each entry is an fp32 value: m + 8 and m round at different spacings)
    np.testing.assert_allclose(mod[2] - mod[0], np.full((3, 6, H), 8.0), atol=2 ** -19)
    assert np.all(mod[0, 0] != mod[0, 2])


def test_rows_in_identity_projection_and_segment_order():
    sh = Sh(2, 3, 4, 1, 4, 1)
    sh.hidden, sh.c_video, sh.c_audio = 128, 96, 32
    H = sh.hidden
    text = bits(np.full((2, H), 3.0))
    pv = (np.arange(4 * 96).reshape(4, 96) % 7 - 3).astype(np.float32) * 0.5
    pa = (np.arange(3 * 32).reshape(3, 32) % 5).astype(np.float32)
    w = {"w_video": np.eye(H, 96, dtype=np.float32), "b_video": np.full(H, 0.25, np.float32),
         "w_audio": 2 * np.eye(H, 32, dtype=np.float32), "b_audio": np.full(H, -1.0, np.float32)}
    x = O.rows_in(sh, text, pv, pa, w)
    np.testing.assert_array_equal(x[:2], 3.0)
    np.testing.assert_array_equal(x[2:5, :32], 2 * pa - 1.0)
    np.testing.assert_array_equal(x[2:5, 32:], -1.0)
    np.testing.assert_array_equal(x[5:, :96], pv + 0.25)
    np.testing.assert_array_equal(x[5:, 96:], 0.25)


def test_rows_in_keeps_f32_weights():
    """A weight 1 + 2^-10 is not a bf16 value: 64 products of it accumulate to
    64 + 2^-4, which rounds to bf16 65.0 only if the weight was not rounded."""
    sh = Sh(0, 0, 1, 1, 4, 1)
    sh.hidden, sh.c_video, sh.c_audio = 1, 64, 1
    w = {"w_video": np.full((1, 64), 1 + 2 ** -10, np.float32), "b_video": np.full(1, 0.5 - 2 ** -5, np.float32),
         "w_audio": np.zeros((1, 1), np.float32), "b_audio": np.zeros(1, np.float32)}
    x = O.rows_in(sh, np.zeros((0, 1), np.uint16), np.ones((1, 64), np.float32),
                  np.zeros((0, 1), np.float32), w)
    # 64 + 1/16 + 1/2 - 1/32 = 64.53125 -> bf16 spacing at 64 is 0.5 -> 64.5
    assert x[0, 0] == 64.5


def test_euler_constant_velocity_closed_form():
    lat = np.array([[1.0, -2.0], [0.5, 3.0]], np.float32)
    v = np.array([[0.25, 1.0], [-2.0, 0.5]])
    x = lat
    for s0, s1 in zip([1.0, 0.5, 0.25], [0.5, 0.25, 0.0]):
        x = O.euler_step(x, v, s0, s1)
    np.testing.assert_array_equal(x, lat - v)


def test_denoise_with_constant_heads_follows_the_schedules():
    """With zero head weights the velocities are the head biases whatever the
    blocks compute, so the loop must land on x0 + (sigma_end - sigma_0) b, per
    segment on its own schedule column (text, audio, video)."""
    from audio_diffusion_transformer_amd import synth as S
    sh = S.TINY.replace(n_text=64, n_audio=64, n_video=128)
    ts, npt = S.tile_map(sh)
    blocks = [S.block_weights(sh, block=0)]
    head = S.head_weights(sh)
    head["w_video"] = np.zeros_like(head["w_video"])
    head["w_audio"] = np.zeros_like(head["w_audio"])
    head["b_video"] = bits(np.full(sh.c_video, 0.5))
    head["b_audio"] = bits(np.full(sh.c_audio, -0.25))
    sig = np.array([[1.0, 1.0, 1.0], [0.5, 0.75, 0.5], [0.25, 0.5, 0.25], [0.0, 0.25, 0.0]],
                   np.float32)
    lv, la = S.latents(sh)
    r = O.denoise(sh, ts, npt, blocks, head, S.rows_in_weights(sh), S.time_weights(sh, 1), sig,
                  S.rope_tables(sh), S.text_rows(sh), lv, la)
    # the same transitions in IEEE float32 arithmetic (each step's sum rounds
    # once; the steps (sigma_to - sigma_from) * b are exact dyadic values)
    ev, ea = lv.copy(), la.copy()
    for k in range(3):
        ev = ev + np.float32((sig[k + 1, 2] - sig[k, 2]) * 0.5)
        ea = ea + np.float32((sig[k + 1, 1] - sig[k, 1]) * -0.25)
    np.testing.assert_array_equal(r["video"], ev.astype(np.float64))
    np.testing.assert_array_equal(r["audio"], ea.astype(np.float64))
    np.testing.assert_allclose(r["video"], lv - 0.5, atol=1e-6)
    np.testing.assert_allclose(r["audio"], la + 0.25 * 0.75, atol=1e-6)
    assert len(r["vels"]) == 3


# ----------------------------------------------------------------------------
# Token reduction
# ----------------------------------------------------------------------------

def test_token_pairs_cover_the_grid_with_horizontal_neighbours():
    from audio_diffusion_transformer_amd import synth as S
    for sh in (S.FASTH3_TINY, S.FASTH3):
        red, pairs, first = S.token_pairs(sh)
        T, Hh, W = sh.video_grid
        assert red.n_video == T * Hh * ((W + 1) // 2)
        used = np.concatenate([pairs[:, 0], pairs[pairs[:, 1] >= 0, 1]])
        np.testing.assert_array_equal(np.sort(used), np.arange(sh.n_video))
        pos = S.video_positions(sh)          # raster index of every full video row
        a, b = pairs[:, 0], pairs[:, 1]
        two = b >= 0
        np.testing.assert_array_equal(pos[a], first)
        np.testing.assert_array_equal(pos[b[two]], pos[a[two]] + 1)   # right-hand neighbour
        np.testing.assert_array_equal(pos[a] % W % 2, 0)              # pairs start on even columns
        assert np.all(pos[a[~two]] % W == W - 1)                      # singles: the odd last column
        assert (~two).sum() == (T * Hh if W % 2 else 0)


def test_token_pool_and_restore_hand_example():
    P = 1
    x = np.array([[9.0, 9.0], [1.0, 2.0], [3.0, 5.0], [7.0, -1.0]])   # prefix, then 3 video rows
    pairs = np.array([[1, 0], [2, -1]])                               # (v1, v0) and v2 single
    r = O.token_pool(x, pairs, P)
    np.testing.assert_array_equal(r, [[9.0, 9.0], [2.0, 3.5], [7.0, -1.0]])
    # no update: exactly the original stream
    np.testing.assert_array_equal(O.token_restore(r, x, r, pairs, P, 3), x)
    # an update d of a pair returns to both its tokens; a single takes its value
    upd = r.copy()
    upd[0] += 0.5
    upd[1] += [0.25, -2.0]
    upd[2] = [4.0, 4.0]
    out = O.token_restore(upd, x, r, pairs, P, 3)
    np.testing.assert_array_equal(out, [[9.5, 9.5], [1.25, 0.0], [3.25, 3.0], [4.0, 4.0]])


def test_token_pool_rounds_the_mean_once():
    # (1 + (1 + 2^-7)) / 2 = 1 + 2^-8: a tie between bf16 1.0 and 1 + 2^-7 -> even (1.0)
    x = np.array([[1.0], [1.0 + 2 ** -7]])
    r = O.token_pool(x, np.array([[0, 1]]), 0)
    assert r[0, 0] == 1.0


def test_reduced_forward_with_identity_middle_equals_the_outer_blocks():
    """Zero gates make the reduced blocks the identity, so the restore must
    give back the pooled-from state bit for bit and the forward equals the
    full forward over the outer blocks alone."""
    from audio_diffusion_transformer_amd import synth as S
    sh = S.FASTH3_TINY
    ts, npt = S.tile_map(sh)
    red, pairs, first = S.token_pairs(sh)
    rts, rnpt = S.tile_map(red)
    L, r0, r1 = 4, 1, 3
    blocks = [S.block_weights(sh, block=l) for l in range(L)]
    mods = np.stack([S.modulation(sh, block=l) for l in range(L)])
    mods[r0:r1, :, 2, :] = 0
    mods[r0:r1, :, 5, :] = 0
    head = S.head_weights(sh)
    mf = S.final_modulation(sh)
    x = S.activations(sh, field=True)
    got = O.dit_forward_reduced(sh, ts, npt, red, rts, rnpt, pairs, r0, r1, blocks, head, mods, mf,
                                S.rope_tables(sh), S.rope_tables(red, first), x)
    keep = [l for l in range(L) if not r0 <= l < r1]
    ref = O.dit_forward(sh, ts, npt, [blocks[l] for l in keep], head, mods[keep], mf,
                        S.rope_tables(sh), x)
    np.testing.assert_array_equal(got["vel_video"], ref["vel_video"])
    np.testing.assert_array_equal(got["vel_audio"], ref["vel_audio"])


# ----------------------------------------------------------------------------
# int8 products
# ----------------------------------------------------------------------------

def test_quantize_int8_exact_grid_and_ties():
    # max 127 * 2^-3: scale 2^-3, and multiples of 2^-3 map to exact integer codes
    x = np.array([[127 / 8, -5 / 8, 0.0, 1 / 8]])
    q, s = O.quantize_int8(x)
    assert s[0] == np.float32(0.125)
    np.testing.assert_array_equal(q, [[127, -5, 0, 1]])
    # max 127 (inv = 1): 2.5 -> 2 and 3.5 -> 4 (round half to even), -2.5 -> -2
    q, s = O.quantize_int8(np.array([[127.0, 2.5, 3.5, -2.5]]))
    np.testing.assert_array_equal(q, [[127, 2, 4, -2]])
    # a zero row: codes 0, scale 0
    q, s = O.quantize_int8(np.zeros((1, 4)))
    assert s[0] == 0 and np.all(q == 0)


def test_quantize_int8_groups_are_independent():
    x = np.array([[1.0, -2.0, 100.0, 50.0]])
    q, s = O.quantize_int8(x, group=2)
    np.testing.assert_array_equal(q, [[64, -127, 127, 64]])      # 1 * 127/2 = 63.5 -> 64 (even)
    np.testing.assert_array_equal(s, np.array([[2.0, 100.0]], np.float32) / np.float32(127))


def test_linear_int8_equals_float_product_on_exact_codes():
    rng = np.random.default_rng(0)
    qa = rng.integers(-127, 128, (5, 256)).astype(np.int8)
    qw = rng.integers(-127, 128, (7, 256)).astype(np.int8)
    sa = np.array([0.5, 0.25, 1.0, 2.0, 0.125], np.float32)
    sw = np.array([1, 2, 4, 0.5, 0.25, 8, 1], np.float32)
    b = np.arange(7) * 0.5
    y = O.linear_int8(qa, sa, qw, sw, b)
    ref = (qa.astype(np.float64) * sa[:, None]) @ (qw.astype(np.float64) * sw[:, None]).T + b
    np.testing.assert_array_equal(y, ref)
    # grouped: one scale per group of 128 columns
    sg = np.stack([sa, 2 * sa], axis=1)
    yg = O.linear_int8(qa, sg, qw, sw, b, group=128)
    ag = qa.astype(np.float64) * np.repeat(sg, 128, axis=1)
    np.testing.assert_array_equal(yg, ag @ (qw.astype(np.float64) * sw[:, None]).T + b)


def test_int8_block_stays_close_to_the_bf16_block():
    sh, ts, npt, w, mod, rope, x = _tiny_block_inputs()
    ref = O.block_forward(sh, ts, npt, w, mod, rope, x)
    q = O.block_forward(sh, ts, npt, w, mod, rope, x, qw=O.quantize_block_int8(w))
    d, r = q["x2"] - O.bf16_to_f64(x), ref["x2"] - O.bf16_to_f64(x)   # the block's update
    cos = float(np.sum(d * r) / np.linalg.norm(d) / np.linalg.norm(r))
    assert cos > 0.99, cos
    # and the int8 path really differs (it is not the bf16 path)
    assert not np.array_equal(q["x2"], ref["x2"])


def test_quantize_weight_int8_rows_from_bf16_bits():
    """Weight codes are per output row of the bf16 weight: row (1, -0.5, 0.25)
    has max 1, so codes rint(127 x) = (127, -64, 32) (-63.5 rounds to even,
    31.75 up) with scale 1/127; row (0, 0, -4) has codes (0, 0, -127), scale
    4/127."""
    w = bits(np.array([[1.0, -0.5, 0.25], [0.0, 0.0, -4.0]]))
    q, s = O.quantize_weight_int8(w)
    np.testing.assert_array_equal(q, [[127, -64, 32], [0, 0, -127]])
    np.testing.assert_array_equal(s, np.array([1.0, 4.0], np.float32) / np.float32(127))


def test_check_tile_map_accepts_and_refuses():
    """A tile map covers rows [0, R) with strictly increasing starts, its
    prefix tiles end exactly where the text and audio rows end, and no tile
    holds rows of two segments."""
    ts = O.check_tile_map([0, 4, 10, 16, 20], 4, 6, 10, 2)
    np.testing.assert_array_equal(ts, [0, 4, 10, 16, 20])
    for bad, npt in (([0, 4, 4, 16, 20], 2),     # an empty tile
                     ([0, 4, 10, 16, 21], 2),    # does not end at R
                     ([1, 4, 10, 16, 20], 2),    # does not start at 0
                     ([0, 4, 12, 16, 20], 2),    # prefix ends inside the audio rows
                     ([0, 2, 10, 16, 20], 2)):   # tile [2, 10) holds text and audio rows
        with pytest.raises(AssertionError):
            O.check_tile_map(bad, 4, 6, 10, npt)
