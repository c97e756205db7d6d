"""GPU parity of the int8 variant against the oracle: the quantization codes
(bit-exact: both sides take the decision in fp32 with IEEE division and
round-half-even), and the int8 forward (h3_dit_forward_i8) against the
oracle's int8 forward and, loosely, against the bf16 forward.

Bars: the codes of a given bf16 input are exact.  Inside the forward the GPU
quantizes its own bf16 activations, which may sit one bf16 spacing from the
oracle's (fp32 against float64 sums), so a code may move by one step; the
velocities then carry the forward's bar."""
import numpy as np
import pytest
import torch

from audio_diffusion_transformer_amd import binding as B
from audio_diffusion_transformer_amd import synth as S
from audio_diffusion_transformer_amd import tensors as T
from oracle import h3_oracle as O

import parity as P

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols,group", [(7, 256, 0), (33, 5120, 0), (5, 20480, 1024),
                                             (3, 7168, 0), (9, 4096, 512), (4, 8192, 2048),
                                             (2, 20480, 4096)])
def test_quantize_rows_codes_exact(rows, cols, group):
    print(f"case: quantize {rows}x{cols} group {group}", flush=True)
    x = S.normal_bf16(f"q.{rows}.{cols}", (rows, cols), 1.0)
    x[0, :] = 0                      # a zero row: codes 0, scale 0
    x[1, 5] = S.f32_to_bf16(np.array([40.0], np.float32))[0]   # one large value
    xd = T.to_dev(x)
    q = torch.empty((rows, cols), dtype=torch.int8, device="cuda")
    ns = 1 if group == 0 else cols // group
    sc = torch.empty((rows, ns), dtype=torch.float32, device="cuda")
    B.quantize_rows(xd, q, sc, group)
    torch.cuda.synchronize()
    rq, rs = O.quantize_int8(T.bf16_bits_to_f64(x), group)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    np.testing.assert_array_equal(sc.cpu().numpy().reshape(rs.shape), rs)


def _i8_case(sh, L):
    ts, npt = S.tile_map(sh)
    blocks = [S.block_weights(sh, block=l) for l in range(L)]
    mods = np.stack([S.modulation(sh, block=l) for l in range(L)])
    return ts, npt, blocks, mods, S.head_weights(sh), S.final_modulation(sh), S.rope_tables(sh), \
        S.activations(sh, field=True)


def _run_i8(sh, ts, npt, blocks, mods, head, mf, rope, x, fc2g):
    shape = B.make_shape(sh, ts, npt)
    ws = T.workspace(B.workspace_bytes(shape, ts, B.H3_WS_DIT_I8))
    qb = [B.quantize_block(T.weights_to_dev(b)) for b in blocks]
    vv = torch.empty((sh.n_video, sh.c_video), dtype=torch.float32, device="cuda")
    va = torch.empty((sh.n_audio, sh.c_audio), dtype=torch.float32, device="cuda")
    B.dit_forward_i8(shape, ts, qb, T.weights_to_dev(head), T.to_dev(np.ascontiguousarray(mods)),
                     T.to_dev(mf), T.to_dev(rope), T.to_dev(x), vv, va, ws, fc2_group=fc2g)
    torch.cuda.synchronize()
    # the weight codes the GPU made must be the oracle's
    for n in ("qkv", "fc2"):
        rq, rs = O.quantize_weight_int8(blocks[0]["w_" + n])
        np.testing.assert_array_equal(qb[0]["w_" + n].cpu().numpy(), rq)
        np.testing.assert_array_equal(qb[0]["s_" + n].cpu().numpy(), rs)
    return vv.cpu().numpy(), va.cpu().numpy()


def oracle_group(sh, fc2g):
    """The oracle's FC2 grouping for the ABI's fc2_group: one group that spans
    the whole row is the per-row form."""
    return fc2g if fc2g and sh.ffn > fc2g else 0


@pytest.mark.parametrize("name,fc2g", [("tiny", 1024), ("tiny_grouped_fc2", 1024),
                                       ("tiny_grouped_fc2", 0), ("fasth3_tiny", 0)])
def test_int8_forward(name, fc2g):
    # (the int8 products need K multiples of 256: the pages' block with 8 heads of 64)
    sh = {"tiny": S.TINY, "tiny_grouped_fc2": S.TINY.replace(ffn=3072),
          "fasth3_tiny": S.FASTH3_TINY.replace(n_heads=8)}[name]
    L = 2
    print(f"case: int8 forward {name} L={L} fc2_group={fc2g}", flush=True)
    ts, npt, blocks, mods, head, mf, rope, x = _i8_case(sh, L)
    gv, ga = _run_i8(sh, ts, npt, blocks, mods, head, mf, rope, x, fc2g)
    qws = [O.quantize_block_int8(b) for b in blocks]
    r = O.dit_forward(sh, ts, npt, blocks, head, mods, mf, rope, x, qws=qws,
                      fc2_group=oracle_group(sh, fc2g))
    for got, ref in ((gv, r["vel_video"]), (ga, r["vel_audio"])):
        m = P.metrics(got, ref)
        assert m["cos"] >= 0.9999 and m["rel"] <= 5e-3, m
    # against the bf16 forward: the quantization error itself (reported bar of
    # the variant, loose)
    rb = O.dit_forward(sh, ts, npt, blocks, head, mods, mf, rope, x)
    m = P.metrics(gv, rb["vel_video"])
    print("int8 vs bf16 video velocity:", m, flush=True)
    assert m["cos"] >= 0.99, m


@pytest.mark.parametrize("name,fc2g", [("full", 1024), ("fasth3", 0)])
def test_int8_full_size_block_sampled_rows(name, fc2g):
    """One int8 block at full size through h3_dit_forward_i8 (its output stays
    in the workspace), the oracle on sampled rows.  full: hidden 5120, 40 x 128
    heads, GELU FFN 20480, the FC2 input in 20 groups of 1,024.  fasth3: the
    pages' block (hidden 5,376, 56 x 128 heads, SwiGLU 14,336, routing gate,
    cube tiles) with the FC2 input per row, whose out projection and FC2 (1,281
    tiles) run their last tile as 16 ranges of K."""
    sh = S.FULL if name == "full" else S.FASTH3
    print(f"case: int8 full-size block {name} fc2_group={fc2g} (oracle on sampled rows)", flush=True)
    ts, npt = S.tile_map(sh)
    w = S.block_weights(sh)
    mod = S.modulation(sh)
    rope = S.rope_tables(sh)
    x = S.activations(sh, field=True)
    shape = B.make_shape(sh, ts, npt)
    lay = B.workspace_layout(shape, ts, B.H3_WS_DIT_I8)
    ws = T.workspace(lay.total)
    qb = B.quantize_block(T.weights_to_dev(w))
    vv = torch.empty((sh.n_video, sh.c_video), dtype=torch.float32, device="cuda")
    va = torch.empty((sh.n_audio, sh.c_audio), dtype=torch.float32, device="cuda")
    B.dit_forward_i8(shape, ts, [qb], T.weights_to_dev(S.head_weights(sh)),
                     T.to_dev(mod[None]), T.to_dev(S.final_modulation(sh)), T.to_dev(rope),
                     T.to_dev(x), vv, va, ws, fc2_group=fc2g)
    torch.cuda.synchronize()
    R, H, A = sh.rows, sh.hidden, sh.attn_width
    wsh = ws.cpu().numpy()

    def view(off, shp):
        n = int(np.prod(shp)) * 2
        return T.bf16_bits_to_f64(wsh[off:off + n].view(np.uint16).reshape(shp))
    rows = np.unique(np.concatenate([np.arange(0, 4), np.arange(510, 516), np.arange(1050, 1060),
                                     np.arange(8000, 8040), np.arange(R - 30, R)]))
    print("oracle ...", flush=True)
    r = O.block_forward(sh, ts, npt, w, mod, rope, x, out_rows=rows,
                        qw=O.quantize_block_int8(w), fc2_group=oracle_group(sh, fc2g))
    m = P.metrics(view(lay.attn, (R, A))[rows], r["attn"])
    assert m["cos"] > 0.9999 and m["rel"] < 1e-2, ("attn", m)
    for stage, off in (("x1", lay.x1), ("x2", lay.xa)):
        got = view(off, (R, H))[rows]
        d = P.metrics(got - T.bf16_bits_to_f64(x)[rows], r[stage] - T.bf16_bits_to_f64(x)[rows])
        # the block's update of the residual (a one-step code flip moves a
        # product by about one code step, 1/127 of its row's range)
        assert d["cos"] > 0.999 and d["rel"] < 2e-2, (stage, d)
