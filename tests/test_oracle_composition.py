"""A hand-worked tiny block that pins the block's composition in both oracles:
which modulation vectors feed the two norms and the two residuals, where the
out projection, MLP hidden and MLP output are rounded to bf16, and where each
bias sits (TensorFold PR #949, "What it adds": the block's steps in order;
"Precision is the checkpoint's own": bf16 activations; the h3.c README's gated
AdaLN with rounded bf16 residuals).

The block: 1 text, 1 audio and 2 video rows, hidden 4, one head of 4, FFN 4,
tiles [0, 1, 2, 4] (one video tile, top-k 1, no pooled branch), no rotary,
eps 1e-6.  Every row of x is a constant c, so the first norm gives
sign(c) (1 + scale1) + shift1 exactly after rounding.  The q and k projections
are zero (uniform attention over all four rows), the v projection is the
identity, and W_o = W1 = W2 = I, so every later value can be worked out by hand.
scale2 = -1 makes the second norm output its shift.

Modulation per segment (shift1, scale1, gate1, shift2, scale2, gate2), the same
in every column: text (0, 0, 1, 1/2, -1, 1/2), audio (0, 1, 1/2, 1/2, -1, 1),
video (1/4, 1/2, 1, 1/2, -1, 2).  x rows: 1/2, 1, 1/2, -1/2.
Biases: b_o = (5 2^-10, 0, 0, 0), b1 = (0, 1/2, 0, 0), b2 = (0, 2^-9, 3 2^-10, 0).

By hand (bf = round to the nearest bf16, ties to even; bf16 spacing 2^-8 in
[1/2, 1), 2^-7 in [1, 2), 2^-6 in [2, 4)):
  n1 rows: 1, 2, 1.5 + 0.25 = 1.75, -1.5 + 0.25 = -1.25
  attention of every row = bf((1 + 2 + 1.75 - 1.25) / 4) = 0.875 (v = n1, equal weights)
  o = bf(0.875 + b_o) = (bf(0.8798828125) = 0.87890625, 0.875, 0.875, 0.875)
  x1 = bf(x + gate1 o): text 0.5 + 0.87890625 = 1.37890625 is a tie -> 1.375 (an
       unrounded o would give 1.3798828125 -> 1.3828125); audio 1 + 0.439453125
       -> 1.4375; video row 3: -0.5 + 0.87890625 = 0.37890625
  n2 = 0.5 everywhere (shift2)
  h = bf(gelu(0.5 + b1)): gelu(0.5) = 0.5 Phi(0.5) = 0.34573123 -> 0.345703125,
      gelu(1) = Phi(1) = 0.84134475 -> 0.83984375 (bias after the activation would
      give bf(0.84573123) = 0.84765625)
  f = bf(h + b2): column 1 0.84179688 -> 0.84375 (from an unrounded h 0.84329788
      -> 0.84375 as well), column 2 0.3486328125 is a tie -> 0.34765625 (from an
      unrounded h: 0.34866096 -> 0.349609375)
  x2 = bf(x1 + gate2 f), listed below; e.g. video row 3, column 3:
       0.375 + 2 x 0.345703125 = 1.06640625, a tie -> 1.0625.
Each plausible slip changes x2 somewhere: shift and scale swapped or taken
from the other norm, the gates swapped or a segment's vectors taken from
another segment, o, h, f or x1 left unrounded, b1 after the activation, x2
built on x instead of x1.
"""
import numpy as np
import pytest

from audio_diffusion_transformer_amd import synth as S
from oracle import h3_oracle as O
from oracle import h3_ref as C

X2 = [[1.546875, 1.796875, 1.546875, 1.546875],
      [1.78125, 2.28125, 1.78125, 1.78125],
      [2.0625, 3.0625, 2.0625, 2.0625],
      [1.0703125, 2.0625, 1.0703125, 1.0625]]
X1 = [[1.375] * 4, [1.4375] * 4, [1.375] * 4, [0.37890625, 0.375, 0.375, 0.375]]
N1 = [[1.0] * 4, [2.0] * 4, [1.75] * 4, [-1.25] * 4]
O_ROW = [0.87890625, 0.875, 0.875, 0.875]
H_ROW = [0.345703125, 0.83984375, 0.345703125, 0.345703125]
F_ROW = [0.345703125, 0.84375, 0.34765625, 0.345703125]


def _bits(x):
    f = np.asarray(x, dtype=np.float32)
    assert np.all(f.astype(np.float64) == np.asarray(x, np.float64)), "not exactly bf16"
    b = f.view(np.uint32)
    assert np.all(b & 0xFFFF == 0), "not exactly bf16"
    return (b >> 16).astype(np.uint16)


def _case():
    sh = S.Shape(1, 1, 2, 4, 1, 4, 4, tile=1, top_k=1, pooled=0)
    ts = np.array([0, 1, 2, 4], np.int32)
    eye = np.eye(4)
    wqkv = np.zeros((12, 4))
    wqkv[8:12] = eye                                  # head 0: q rows 0-3, k 4-7, v 8-11
    w = dict(w_qkv=_bits(wqkv), b_qkv=_bits(np.zeros(12)), q_gain=_bits(np.ones(4)),
             k_gain=_bits(np.ones(4)), w_o=_bits(eye), b_o=_bits([5 * 2.0 ** -10, 0, 0, 0]),
             w_fc1=_bits(eye), b_fc1=_bits([0, 0.5, 0, 0]), w_fc2=_bits(eye),
             b_fc2=_bits([0, 2.0 ** -9, 3 * 2.0 ** -10, 0]))
    vec = {0: (0, 0, 1, 0.5, -1, 0.5), 1: (0, 1, 0.5, 0.5, -1, 1), 2: (0.25, 0.5, 1, 0.5, -1, 2)}
    mod = np.zeros((3, 6, 4), np.float32)
    for s, v in vec.items():
        mod[s] = np.asarray(v, np.float32)[:, None]
    x = _bits(np.array([0.5, 1.0, 0.5, -0.5])[:, None] * np.ones((1, 4)))
    return sh, ts, w, mod, x


@pytest.mark.parametrize("oracle", [O, C], ids=["float64", "cpp_fp32"])
def test_block_composition_by_hand(oracle):
    sh, ts, w, mod, x = _case()
    r = oracle.block_forward(sh, ts, 2, w, mod, None, x)
    np.testing.assert_array_equal(r["n1"], N1)
    np.testing.assert_array_equal(r["sel"][0, 0], [2])
    np.testing.assert_array_equal(r["attn"], np.full((4, 4), 0.875))
    np.testing.assert_array_equal(r["o"], np.tile(O_ROW, (4, 1)))
    np.testing.assert_array_equal(r["x1"], X1)
    np.testing.assert_array_equal(r["n2"], np.full((4, 4), 0.5))
    np.testing.assert_array_equal(r["h"], np.tile(H_ROW, (4, 1)))
    np.testing.assert_array_equal(r["f"], np.tile(F_ROW, (4, 1)))
    np.testing.assert_array_equal(r["x2"], X2)
