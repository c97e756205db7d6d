"""h3_modulation_noalloc (scratch in the library's static device array, no
workspace, no allocation) against h3_modulation (the same kernels with a
caller workspace): byte-identical tables on two calls in a row, the second
with a smaller shape (hidden 256 and 2 blocks after hidden 512 and 3 blocks),
so the second call runs on the array the first one left behind."""
import numpy as np
import pytest
import torch

from audio_diffusion_transformer_amd import binding as B
from audio_diffusion_transformer_amd import synth as S
from audio_diffusion_transformer_amd import tensors as T

pytestmark = pytest.mark.gpu


def _tables(sh, L, tw, sigma3, noalloc):
    ts, npt = S.tile_map(sh)
    shape = B.make_shape(sh, ts, npt)
    mod = torch.full((L, 3, 6, sh.hidden), float("nan"), dtype=torch.float32, device="cuda")
    fin = torch.full((3, 2, sh.hidden), float("nan"), dtype=torch.float32, device="cuda")
    twd = T.weights_to_dev(tw)
    if noalloc:
        B.modulation_noalloc(shape, L, twd, sigma3, mod, fin)
    else:
        ws = T.workspace(B.modulation_workspace_bytes(shape))
        B.modulation(shape, L, twd, sigma3, mod, fin, ws)
    torch.cuda.synchronize()
    return mod.cpu().numpy(), fin.cpu().numpy()


def test_noalloc_modulation_equals_the_workspace_call_twice():
    big = S.TINY.replace(hidden=512, n_heads=8)
    small = S.TINY
    for sh, L, sigma in ((big, 3, (0.9, 0.35, 0.9)), (small, 2, (0.5, 0.2, 0.5))):
        print(f"case: h3_modulation_noalloc hidden={sh.hidden} blocks={L}", flush=True)
        tw = S.time_weights(sh, L)
        sigma3 = np.array(sigma, np.float32)
        want = _tables(sh, L, tw, sigma3, noalloc=False)
        got = _tables(sh, L, tw, sigma3, noalloc=True)
        for g, w in zip(got, want):
            assert not np.isnan(w).any()
            np.testing.assert_array_equal(g.view(np.uint32), w.view(np.uint32))
