"""GPU parity of the denoising loop's pieces against the oracle: the rows in
(F32 patch projections into the packed bf16 stream), the modulation tables
from the timesteps, and h3_denoise (rows in, tables, forward, Euler) over a
few passes.

Bars, from the arithmetic: the rows in sum in fp32 (the oracle in float64)
and round once to bf16, so an output may sit one bf16 spacing away where the
exact sum lies next to a rounding boundary.  The tables sum about H products
of bf16 weights and fp32 inputs in fp32: relative error about sqrt(H) 2^-24
against float64 (1e-5 absolute at their size).  The latents move by
sum_k (sigma_k+1 - sigma_k) vel_k, so their displacement inherits the
velocity bar of the forward."""
import numpy as np
import pytest
import torch

from audio_diffusion_transformer_amd import binding as B
from audio_diffusion_transformer_amd import synth as S
from audio_diffusion_transformer_amd import tensors as T
from oracle import h3_oracle as O

import parity as P

pytestmark = pytest.mark.gpu


def _dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _rows_in_gpu(sh, rw, text, pa, pv):
    ts, npt = S.tile_map(sh)
    shape = B.make_shape(sh, ts, npt)
    x = T.bf16_empty((sh.rows, sh.hidden))
    B.rows_in(shape, {k: _dev_f32(v) for k, v in rw.items()}, T.to_dev(text), _dev_f32(pa),
              _dev_f32(pv), x)
    torch.cuda.synchronize()
    return T.bf16_bits_to_f64(T.to_host_bf16(x))


@pytest.mark.parametrize("name", ["tiny", "full"])
def test_rows_in(name):
    sh = S.TINY if name == "tiny" else S.FULL
    print(f"case: rows_in {name}", flush=True)
    rw = S.rows_in_weights(sh)
    text = S.text_rows(sh)
    lv, la = S.latents(sh)
    got = _rows_in_gpu(sh, rw, text, la, lv)
    ref = O.rows_in(sh, text, lv, la, rw)
    np.testing.assert_array_equal(got[:sh.n_text], ref[:sh.n_text])
    # an fp32 sum of C products errs by at most C 2^-24 sum |p w| (+ the bias
    # term); the bf16 rounding then adds at most one spacing
    f = lambda a: np.abs(np.asarray(a, np.float64))
    mag = np.concatenate([np.zeros((sh.n_text, sh.hidden)),
                          f(la) @ f(rw["w_audio"]).T + f(rw["b_audio"]),
                          f(lv) @ f(rw["w_video"]).T + f(rw["b_video"])])
    C = np.concatenate([np.ones(sh.n_text), np.full(sh.n_audio, sh.c_audio + 1),
                        np.full(sh.n_video, sh.c_video + 1)])[:, None]
    bound = P.bf16_ulp(ref) + C * 2.0 ** -24 * mag
    err = np.abs(got - ref)
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.all(err <= bound), (worst, got[worst], ref[worst], bound[worst])
    assert np.mean(err > 0) < 2e-3, np.mean(err > 0)


def _modulation_gpu(sh, L, tw, sigma3):
    ts, npt = S.tile_map(sh)
    shape = B.make_shape(sh, ts, npt)
    mod = torch.empty((max(L, 1), 3, 6, sh.hidden), dtype=torch.float32, device="cuda")
    fin = torch.empty((3, 2, sh.hidden), dtype=torch.float32, device="cuda")
    ws = T.workspace(B.modulation_workspace_bytes(shape))
    B.modulation(shape, L, T.weights_to_dev(tw), sigma3, mod, fin, ws)
    torch.cuda.synchronize()
    return mod.cpu().numpy()[:L], fin.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "full"])
def test_modulation_tables(name):
    sh = S.TINY if name == "tiny" else S.FULL
    L = 3
    print(f"case: modulation {name}", flush=True)
    tw = S.time_weights(sh, L)
    sigma3 = np.array([0.9, 0.35, 0.9], np.float32)
    mod, fin = _modulation_gpu(sh, L, tw, sigma3)
    rmod, rfin = O.modulation_tables(sh, L, tw, sigma3)
    np.testing.assert_allclose(mod, rmod, atol=2e-5, rtol=1e-4)
    np.testing.assert_allclose(fin, rfin, atol=2e-5, rtol=1e-4)
    # the segments see their own timesteps: text and video equal, audio differs
    np.testing.assert_array_equal(mod[:, 0], mod[:, 2])
    assert np.max(np.abs(mod[:, 1] - mod[:, 0])) > 1e-3


def _denoise_gpu(sh, L, head, rw, tw, sig, text, lv, la, blocks):
    ts, npt = S.tile_map(sh)
    shape = B.make_shape(sh, ts, npt)
    ws = T.workspace(B.denoise_workspace_bytes(shape, ts, L))
    dv, da = _dev_f32(lv), _dev_f32(la)
    dev_blocks = [b if isinstance(next(iter(b.values())), torch.Tensor) else T.weights_to_dev(b)
                  for b in blocks]
    B.denoise(shape, ts, dev_blocks, T.weights_to_dev(head),
              {k: _dev_f32(v) for k, v in rw.items()}, T.weights_to_dev(tw), sig,
              T.to_dev(S.rope_tables(sh)), T.to_dev(text), dv, da, ws)
    torch.cuda.synchronize()
    return dv.cpu().numpy(), da.cpu().numpy()


def _denoise_case(sh, L, n_steps):
    ts, npt = S.tile_map(sh)
    blocks = [S.block_weights(sh, block=l) for l in range(L)]
    head = S.head_weights(sh)
    rw = S.rows_in_weights(sh)
    tw = S.time_weights(sh, L)
    sig = S.schedule(n_steps)
    text = S.text_rows(sh)
    lv, la = S.latents(sh)
    return ts, npt, blocks, head, rw, tw, sig, text, lv, la


@pytest.mark.parametrize("name", ["tiny", "fasth3_tiny"])
def test_denoise_passes(name):
    sh = S.TINY if name == "tiny" else S.FASTH3_TINY
    L, n = 2, 3
    print(f"case: denoise {name} L={L} steps={n}", flush=True)
    ts, npt, blocks, head, rw, tw, sig, text, lv, la = _denoise_case(sh, L, n)
    gv, ga = _denoise_gpu(sh, L, head, rw, tw, sig, text, lv, la, blocks)
    r = O.denoise(sh, ts, npt, blocks, head, rw, tw, sig, S.rope_tables(sh), text, lv, la)
    for got, ref, x0 in ((gv, r["video"], lv), (ga, r["audio"], la)):
        m = P.metrics(got - x0, ref - x0)
        # the stated bar is cos >= 0.998 and rel <= 0.06 on the velocities; a
        # few passes over two blocks stay far inside it
        assert m["cos"] >= 0.9999 and m["rel"] <= 5e-3, m


@pytest.mark.parametrize("name", ["small", "full"])
def test_denoise_constant_heads_exact(name):
    """Zero head weights: the velocities are the head biases, so the GPU loop
    must equal the float32 Euler steps exactly, on each segment's schedule.
    full: the default geometry (15,435 rows, hidden 5120) with two blocks in
    the benchmark's launch configuration."""
    if name == "small":
        sh = S.TINY.replace(n_text=64, n_audio=64, n_video=128)
        L = 1
    else:
        sh, L = S.FULL, 2
    print(f"case: denoise constant heads {name}", flush=True)
    ts, npt, blocks, head, rw, tw, _, text, lv, la = _denoise_case(sh, 0, 3)
    blocks = ([S.block_weights(sh, block=l) for l in range(L)] if name == "small" else
              [S.device_block_weights(sh, block=l) for l in range(L)])
    tw = S.time_weights(sh, L)
    head["w_video"] = np.zeros_like(head["w_video"])
    head["w_audio"] = np.zeros_like(head["w_audio"])
    head["b_video"] = S.f32_to_bf16(np.full(sh.c_video, 0.5, np.float32))
    head["b_audio"] = S.f32_to_bf16(np.full(sh.c_audio, -0.25, np.float32))
    sig = np.array([[1.0, 1.0, 1.0], [0.5, 0.75, 0.5], [0.25, 0.5, 0.25], [0.0, 0.25, 0.0]],
                   np.float32)
    gv, ga = _denoise_gpu(sh, L, head, rw, tw, sig, text, lv, la, blocks)
    ev, ea = lv.copy(), la.copy()
    for k in range(3):
        ev = ev + np.float32((sig[k + 1, 2] - sig[k, 2]) * 0.5)
        ea = ea + np.float32((sig[k + 1, 1] - sig[k, 1]) * -0.25)
    np.testing.assert_array_equal(gv, ev)
    np.testing.assert_array_equal(ga, ea)


def test_denoise_zero_steps_is_identity():
    sh = S.TINY
    ts, npt, blocks, head, rw, tw, _, text, lv, la = _denoise_case(sh, 1, 1)
    gv, ga = _denoise_gpu(sh, 1, head, rw, tw, np.ones((1, 3), np.float32), text, lv, la, blocks)
    np.testing.assert_array_equal(gv, lv)
    np.testing.assert_array_equal(ga, la)
