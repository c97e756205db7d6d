"""Velocity parity at the full size: h3_dit_forward with two blocks at 15,435
rows against the oracle's velocities of sampled rows, stored in tests/golden/
(written by tests/golden/make_full_velocity.py from the plain C++ oracle on
the same seeded inputs), for two workloads:

- full: 512 text / 543 audio / 14,380 video rows, hidden 5,120, 40 x 128
  heads, GELU FFN 20,480, tile 64, top-k 32 + pooled;
- fasth3: the pages' block and geometry (36 / 414 / 14,985 rows, video in
  4 x 4 x 4 cubes, hidden 5,376, 56 x 128 heads, SwiGLU FFN 14,336, the
  routing gate, top-k 56 + pooled).

Bar: the acceptance bar, cos >= 0.998 and relative L2 <= 0.06, per output
head; the oracle's own self-noise floor (reversed tile sums) on the same rows
is printed beside the GPU's error (TensorFold PR #949, Receipts: Parity, the
first forward's velocities and the self-noise rows)."""
import json
import os
import sys

import numpy as np
import pytest
import torch

from audio_diffusion_transformer_amd import binding as B
from audio_diffusion_transformer_amd import tensors as T

import parity as P

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
sys.path.insert(0, GOLDEN)


@pytest.mark.parametrize("workload", ["full", "fasth3"])
def test_full_size_two_block_velocities(workload):
    import make_full_velocity as MF
    print(f"case: h3_dit_forward, 2 blocks at 15,435 rows ({workload}), sampled rows", flush=True)
    ref = json.load(open(MF.golden_path(workload)))
    sh, ts, npt, blocks, mods, head, mf, rope, x = MF.inputs(workload)
    aud, vid = MF.sample_rows(sh, ts)
    assert aud.tolist() == ref["audio_rows"] and vid.tolist() == ref["video_rows"]
    shape = B.make_shape(sh, ts, npt)
    ws = T.workspace(B.workspace_bytes(shape, ts, B.H3_WS_DIT))
    vv = torch.empty((sh.n_video, sh.c_video), dtype=torch.float32, device="cuda")
    va = torch.empty((sh.n_audio, sh.c_audio), dtype=torch.float32, device="cuda")
    B.dit_forward(shape, ts, [T.weights_to_dev(b) for b in blocks], T.weights_to_dev(head),
                  T.to_dev(np.ascontiguousarray(mods)), T.to_dev(mf), T.to_dev(rope), T.to_dev(x),
                  vv, va, ws)
    torch.cuda.synchronize()
    P_ = sh.n_text + sh.n_audio
    got_v = vv.cpu().numpy()[vid - P_]
    got_a = va.cpu().numpy()[aud - sh.n_text]
    mv = P.metrics(got_v, np.array(ref["vel_video"]))
    ma = P.metrics(got_a, np.array(ref["vel_audio"]))
    print(f"video velocities: GPU vs oracle {mv}; oracle self-noise {ref['self_noise']['video']}")
    print(f"audio velocities: GPU vs oracle {ma}; oracle self-noise {ref['self_noise']['audio']}")
    for m in (mv, ma):
        assert m["cos"] >= 0.998 and m["rel"] <= 0.06, m
