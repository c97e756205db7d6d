"""GPU parity of token reduction (h3_dit_forward_tr) against the oracle: the
pages' block on a small video grid with an odd width (pairs and single
tokens), the pooled stream on its own cube tile map.

Bars: the pool and restore are exact operations (one rounding of an exactly
formed sum), so identity middle blocks must give the full forward over the
outer blocks bit for bit on the GPU too; with real middle blocks the
velocities carry the forward's bar."""
import numpy as np
import pytest
import torch

from audio_diffusion_transformer_amd import binding as B
from audio_diffusion_transformer_amd import synth as S
from audio_diffusion_transformer_amd import tensors as T
from oracle import h3_oracle as O

import parity as P

pytestmark = pytest.mark.gpu


def _case(sh, L):
    ts, npt = S.tile_map(sh)
    red, pairs, first = S.token_pairs(sh)
    rts, rnpt = S.tile_map(red)
    blocks = [S.block_weights(sh, block=l) for l in range(L)]
    mods = np.stack([S.modulation(sh, block=l) for l in range(L)])
    return dict(ts=ts, npt=npt, red=red, pairs=pairs, first=first, rts=rts, rnpt=rnpt,
                blocks=blocks, mods=mods, head=S.head_weights(sh), mf=S.final_modulation(sh),
                rope=S.rope_tables(sh), rrope=S.rope_tables(red, first),
                x=S.activations(sh, field=True))


def _run_tr(sh, c, r0, r1):
    shape = B.make_shape(sh, c["ts"], c["npt"])
    tr = B.TokenReduction(B.make_shape(c["red"], c["rts"], c["rnpt"]), c["rts"],
                          T.to_dev(np.ascontiguousarray(c["pairs"])), T.to_dev(c["rrope"]), r0, r1)
    ws = T.workspace(B.dit_forward_tr_workspace_bytes(shape, c["ts"], tr))
    vv = torch.empty((sh.n_video, sh.c_video), dtype=torch.float32, device="cuda")
    va = torch.empty((sh.n_audio, sh.c_audio), dtype=torch.float32, device="cuda")
    B.dit_forward_tr(shape, c["ts"], tr, [T.weights_to_dev(b) for b in c["blocks"]],
                     T.weights_to_dev(c["head"]), T.to_dev(np.ascontiguousarray(c["mods"])),
                     T.to_dev(c["mf"]), T.to_dev(c["rope"]), T.to_dev(c["x"]), vv, va, ws)
    torch.cuda.synchronize()
    return vv.cpu().numpy(), va.cpu().numpy()


def _run_full(sh, c, keep):
    shape = B.make_shape(sh, c["ts"], c["npt"])
    ws = T.workspace(B.workspace_bytes(shape, c["ts"], B.H3_WS_DIT))
    vv = torch.empty((sh.n_video, sh.c_video), dtype=torch.float32, device="cuda")
    va = torch.empty((sh.n_audio, sh.c_audio), dtype=torch.float32, device="cuda")
    B.dit_forward(shape, c["ts"], [T.weights_to_dev(c["blocks"][l]) for l in keep],
                  T.weights_to_dev(c["head"]), T.to_dev(np.ascontiguousarray(c["mods"][keep])),
                  T.to_dev(c["mf"]), T.to_dev(c["rope"]), T.to_dev(c["x"]), vv, va, ws)
    torch.cuda.synchronize()
    return vv.cpu().numpy(), va.cpu().numpy()


def test_token_reduction_identity_middle_is_exact():
    sh = S.FASTH3_TINY
    print("case: token reduction, identity middle", flush=True)
    L, r0, r1 = 4, 1, 3
    c = _case(sh, L)
    c["mods"][r0:r1, :, 2, :] = 0
    c["mods"][r0:r1, :, 5, :] = 0
    got = _run_tr(sh, c, r0, r1)
    ref = _run_full(sh, c, [l for l in range(L) if not r0 <= l < r1])
    np.testing.assert_array_equal(got[0], ref[0])
    np.testing.assert_array_equal(got[1], ref[1])


@pytest.mark.parametrize("r0,r1", [(1, 3), (0, 4), (2, 2)])
def test_token_reduction_forward(r0, r1):
    sh = S.FASTH3_TINY
    print(f"case: token reduction blocks [{r0}, {r1})", flush=True)
    L = 4
    c = _case(sh, L)
    gv, ga = _run_tr(sh, c, r0, r1)
    r = O.dit_forward_reduced(sh, c["ts"], c["npt"], c["red"], c["rts"], c["rnpt"], c["pairs"],
                              r0, r1, c["blocks"], c["head"], c["mods"], c["mf"], c["rope"],
                              c["rrope"], c["x"])
    for got, ref in ((gv, r["vel_video"]), (ga, r["vel_audio"])):
        m = P.metrics(got, ref)
        assert m["cos"] >= 0.9999 and m["rel"] <= 5e-3, m


def test_token_reduction_identity_middle_full_size():
    """The pages' geometry at full size (15,435 rows; 7,770 pooled video rows on
    160 cube tiles), in the launch configuration the benchmark times: with the
    pooled block's gates zero it is the identity, so pooling, the pooled
    stream's own tile map and the restore must give the forward over the other
    blocks bit for bit."""
    sh = S.FASTH3
    print("case: token reduction at full size, identity middle block", flush=True)
    L, r0, r1 = 3, 1, 2
    ts, npt = S.tile_map(sh)
    red, pairs, first = S.token_pairs(sh)
    rts, rnpt = S.tile_map(red)
    blocks = [S.device_block_weights(sh, block=l) for l in range(L)]
    mods = np.stack([S.modulation(sh, block=l) for l in range(L)])
    mods[r0:r1, :, 2, :] = 0
    mods[r0:r1, :, 5, :] = 0
    head = T.weights_to_dev(S.head_weights(sh))
    mf, rope, x = T.to_dev(S.final_modulation(sh)), T.to_dev(S.rope_tables(sh)), \
        T.to_dev(S.activations(sh, field=True))
    shape = B.make_shape(sh, ts, npt)
    tr = B.TokenReduction(B.make_shape(red, rts, rnpt), rts, T.to_dev(np.ascontiguousarray(pairs)),
                          T.to_dev(S.rope_tables(red, first)), r0, r1)
    out = []
    for reduced in (True, False):
        vv = torch.empty((sh.n_video, sh.c_video), dtype=torch.float32, device="cuda")
        va = torch.empty((sh.n_audio, sh.c_audio), dtype=torch.float32, device="cuda")
        if reduced:
            ws = T.workspace(B.dit_forward_tr_workspace_bytes(shape, ts, tr))
            B.dit_forward_tr(shape, ts, tr, blocks, head, T.to_dev(mods), mf, rope, x, vv, va, ws)
        else:
            keep = [l for l in range(L) if not r0 <= l < r1]
            ws = T.workspace(B.workspace_bytes(shape, ts, B.H3_WS_DIT))
            B.dit_forward(shape, ts, [blocks[l] for l in keep], head,
                          T.to_dev(np.ascontiguousarray(mods[keep])), mf, rope, x, vv, va, ws)
        torch.cuda.synchronize()
        out.append((vv.cpu().numpy(), va.cpu().numpy()))
        del ws
    np.testing.assert_array_equal(out[0][0], out[1][0])
    np.testing.assert_array_equal(out[0][1], out[1][1])
