"""The C-ABI library on the CPU: it loads, exports every declared entry point,
and rejects invalid shapes on the host before any launch (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

from audio_diffusion_transformer_amd import binding as B
from audio_diffusion_transformer_amd import synth as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "h3.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(h3_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from audio_diffusion_transformer_amd import build
        build.build_hip()
    return B.lib()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version(lib):
    """The header, the library and the binding agree on the ABI version."""
    src = open(os.path.join(ROOT, "include", "h3.h")).read()
    declared = int(re.search(r"#define H3_ABI_VERSION (\d+)", src).group(1))
    assert lib.h3_abi_version() == declared == B.ABI_VERSION


def _split_ways(M, N, K, es):
    """Host rule for a product's split-K tail: the last round of 256x256 tiles
    (one per CU) is split along K when it is at most half filled, into at most
    16 ranges of >= 2 stages of 128 bytes, when that saves >= 36 stages."""
    tiles = -(-M // 256) * (N // 256)
    tail = tiles % 256
    if tail == 0 or 2 * tail > 256:
        return 0, tail
    kt = K * es // 128
    s = min(256 // tail, 16, kt // 2)
    if s < 2 or kt - -(-kt // s) < 36:
        return 0, tail
    return s, tail


@pytest.mark.parametrize("name", ["TINY", "MID", "FULL", "FASTH3", "FASTH3_TINY"])
def test_split_tail_region(lib, name):
    """The workspace holds the partial sums of the largest split-K tail of the
    block's four products (and none for the attention-only workspace)."""
    sh = getattr(S, name)
    shape, ts = _shape(sh)
    R, H, A, F = sh.rows, sh.hidden, sh.attn_width, sh.ffn
    F1 = 2 * F if sh.mlp else F
    dims = [((3 + sh.gate) * A, H), (H, A), (F1, H), (H, F)]
    for which, es in ((B.H3_WS_BLOCK, 2), (B.H3_WS_DIT, 2), (B.H3_WS_DIT_I8, 1)):
        if which == B.H3_WS_DIT_I8 and any(d[1] % 256 for d in dims):
            continue
        want = 0
        for N, K in dims:
            s, tail = _split_ways(R, N, K, es)
            want = max(want, s * tail * 256 * 256 * 4)
        lay = B.workspace_layout(shape, ts, which)
        if want:
            assert lay.partial % 256 == 0 and lay.partial + want <= lay.total
            assert lay.partial >= max(lay.x1, lay.xb, lay.qscale)
        else:
            assert lay.partial == 0
        assert want <= 64 << 20
    assert B.workspace_layout(shape, ts, B.H3_WS_ATTN).partial == 0


def _shape(sh):
    ts, npt = S.tile_map(sh)
    return B.make_shape(sh, ts, npt), ts


def test_workspace_layout_is_consistent(lib):
    for sh in (S.TINY, S.MID, S.FULL):
        shape, ts = _shape(sh)
        for which in (B.H3_WS_BLOCK, B.H3_WS_DIT, B.H3_WS_ATTN):
            n = B.workspace_bytes(shape, ts, which)
            lay = B.workspace_layout(shape, ts, which)
            assert lay.total == n
            lens = np.diff(ts)
            assert lay.padded_rows == int(np.sum((lens + 31) // 32 * 32))
            assert lay.n_query_tiles == len(ts) - 1 - shape.n_prefix_tiles
            assert lay.n_sel == min(sh.top_k, lay.n_query_tiles)
            offs = [lay.q, lay.k, lay.vt, lay.qbar, lay.kbar, lay.vbar, lay.scores, lay.sel,
                    lay.pooled]
            assert all(o % 256 == 0 for o in offs)
            assert offs == sorted(offs) and offs[-1] < n


@pytest.mark.parametrize("mutate,code", [
    (lambda s, t: setattr(s, "head_dim", 96), B.H3_EUNSUPPORTED),
    (lambda s, t: setattr(s, "hidden", 300), B.H3_EUNSUPPORTED),
    (lambda s, t: setattr(s, "mlp", 2), B.H3_EINVAL),
    (lambda s, t: setattr(s, "gate", 3), B.H3_EINVAL),
    (lambda s, t: setattr(s, "n_heads", 3), B.H3_EUNSUPPORTED),   # 3 x 64 x 3 not a multiple of 256
    (lambda s, t: setattr(s, "ffn", 1000), B.H3_EUNSUPPORTED),
    (lambda s, t: setattr(s, "n_prefix_tiles", 1), B.H3_EINVAL),
    (lambda s, t: t.__setitem__(3, t[2]), B.H3_EINVAL),
    (lambda s, t: t.__setitem__(1, 32), B.H3_EINVAL),   # tile [32, 128) straddles text | audio
    (lambda s, t: t.__setitem__(-1, t[-1] + 1), B.H3_EINVAL),
    (lambda s, t: setattr(s, "top_k", 0), B.H3_EINVAL),
    (lambda s, t: setattr(s, "n_text", -1), B.H3_EINVAL),
    # three row counts whose int32 sum would wrap
    (lambda s, t: (setattr(s, "n_audio", 2 ** 31 - 1), setattr(s, "n_video", 2 ** 31 - 1)),
     B.H3_EUNSUPPORTED),
])
def test_invalid_shapes_rejected_on_host(lib, mutate, code):
    shape, ts = _shape(S.TINY)
    ts = ts.copy()
    mutate(shape, ts)
    lay = B.H3WsLayout()
    rc = lib.h3_workspace_layout(ctypes.byref(shape),
                                 ts.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                 B.H3_WS_BLOCK, ctypes.byref(lay))
    assert rc == code, B.last_error()
    assert B.last_error()
    assert lib.h3_workspace_bytes(ctypes.byref(shape),
                                  ts.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                  B.H3_WS_BLOCK) == 0


def test_quantize_rows_validates_before_launch(lib):
    """Bad widths, missing buffers and launches too large for one grid are
    refused on the host (no GPU is touched)."""
    rc = lib.h3_quantize_rows(None, 4, 100, 0, None, None, None)
    assert rc == B.H3_EINVAL and "multiples of 8" in B.last_error()
    rc = lib.h3_quantize_rows(None, 4, 1024, 256, None, None, None)
    assert rc == B.H3_EINVAL and "required" in B.last_error()
    rc = lib.h3_quantize_rows(None, 2 ** 30, 1024, 1024, None, None, None)
    assert rc == B.H3_EUNSUPPORTED
    rc = lib.h3_quantize_rows(None, 2 ** 26, 2 ** 20, 8, None, None, None)
    assert rc == B.H3_EUNSUPPORTED and "too many" in B.last_error()
    assert lib.h3_quantize_rows(None, 0, 1024, 0, None, None, None) == B.H3_OK  # nothing to do


def test_entry_points_validate_before_launch(lib):
    """Null or undersized arguments are refused with an error code; nothing is
    launched (this runs without a GPU)."""
    shape, ts = _shape(S.TINY)
    tp = ts.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    w = B.H3BlockWeights()
    rc = lib.h3_block_forward(ctypes.byref(shape), tp, ctypes.byref(w), None, None, None, None,
                              None, 0, None)
    assert rc == B.H3_EINVAL and "workspace" in B.last_error()
    rc = lib.h3_block_forward(ctypes.byref(shape), tp, ctypes.byref(w), None, None, None, None,
                              ctypes.c_void_p(256), 16, None)
    assert rc == B.H3_EWORKSPACE
    rc = lib.h3_routed_attn(ctypes.byref(shape), tp, None, None, None, None, None, None, None,
                            ctypes.c_void_p(256), 1 << 40, None)
    assert rc == B.H3_EINVAL
    # a misaligned gate is refused on the host (no launch)
    rc = lib.h3_routed_attn(ctypes.byref(shape), tp, ctypes.c_void_p(256), ctypes.c_void_p(256),
                            ctypes.c_void_p(256), ctypes.c_void_p(258), ctypes.c_void_p(256),
                            None, None, ctypes.c_void_p(256), 1 << 40, None)
    assert rc == B.H3_EINVAL and "aligned" in B.last_error()
    hw = B.H3HeadWeights()
    rc = lib.h3_dit_forward(ctypes.byref(shape), 1, tp, None, ctypes.byref(hw), None, None, None,
                            None, None, None, ctypes.c_void_p(256), 1 << 40, None)
    assert rc == B.H3_EINVAL


def test_pages_block_shapes_are_accepted(lib):
    """Attention width != hidden, SwiGLU and the routing gate (the pages' block):
    the plan sizes y as (3 + gate) A, the attention output as A and the MLP
    hidden as F."""
    for sh in (S.FASTH3_TINY, S.FASTH3):
        shape, ts = _shape(sh)
        lay = B.workspace_layout(shape, ts, B.H3_WS_BLOCK)
        R, H, A, F = sh.rows, sh.hidden, sh.attn_width, sh.ffn
        assert lay.big - lay.norm >= R * H * 2
        big_bytes = lay.q - lay.big
        assert big_bytes >= R * max(4 * A, F) * 2
        assert lay.x1 - lay.attn >= R * A * 2


def test_denoise_entry_points_validate_before_launch(lib):
    shape, ts = _shape(S.TINY)
    tp = ts.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    # rows in: missing weights, bad widths, unsupported hidden
    rc = lib.h3_rows_in(ctypes.byref(shape), None, None, None, None, None, None)
    assert rc == B.H3_EINVAL
    rw = B.H3RowsInWeights(ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_void_p(256),
                           ctypes.c_void_p(256), 300, 32)
    rc = lib.h3_rows_in(ctypes.byref(shape), ctypes.byref(rw), ctypes.c_void_p(256),
                        ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_void_p(256), None)
    assert rc == B.H3_EINVAL and "patch widths" in B.last_error()
    bad = B.H3Shape.from_buffer_copy(shape)
    bad.hidden = 300
    rc = lib.h3_rows_in(ctypes.byref(bad), ctypes.byref(rw), None, None, None, None, None)
    assert rc == B.H3_EUNSUPPORTED
    huge = B.H3Shape.from_buffer_copy(shape)
    huge.n_audio = huge.n_video = 2 ** 31 - 1  # an int32 sum would wrap
    rc = lib.h3_rows_in(ctypes.byref(huge), ctypes.byref(rw), None, None, None, None, None)
    assert rc == B.H3_EUNSUPPORTED and "rows" in B.last_error()
    # modulation: workspace size, missing sigma, missing weights, small workspace
    n = lib.h3_modulation_workspace_bytes(ctypes.byref(shape))
    assert n >= 6 * S.TINY.hidden * 4 and n % 256 == 0
    assert lib.h3_modulation_workspace_bytes(ctypes.byref(bad)) == 0
    tw = B.H3TimeWeights()
    rc = lib.h3_modulation(ctypes.byref(shape), 2, ctypes.byref(tw), None, None, None, None, 0, None)
    assert rc == B.H3_EINVAL and "sigma3" in B.last_error()
    sig = (ctypes.c_float * 3)(1, 1, 1)
    rc = lib.h3_modulation(ctypes.byref(shape), 2, ctypes.byref(tw), sig, None, None, None, 0, None)
    assert rc == B.H3_EINVAL and "time weights" in B.last_error()
    # denoise: its workspace extends the forward's; bad step counts and widths are refused
    nd = lib.h3_denoise_workspace_bytes(ctypes.byref(shape), tp, 2)
    assert nd > lib.h3_workspace_bytes(ctypes.byref(shape), tp, B.H3_WS_DIT)
    assert lib.h3_denoise_workspace_bytes(ctypes.byref(shape), tp, 4) > nd
    sig2 = (ctypes.c_float * 6)(1, 1, 1, 0, 0, 0)
    rc = lib.h3_denoise(ctypes.byref(shape), 0, -1, tp, None, None, None, None, sig2, None, None,
                        None, None, ctypes.c_void_p(256), 1 << 40, None)
    assert rc == B.H3_EINVAL and "n_steps" in B.last_error()
    hw = B.H3HeadWeights(ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_void_p(256),
                         ctypes.c_void_p(256), 96, 32)
    rw2 = B.H3RowsInWeights(ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_void_p(256),
                            ctypes.c_void_p(256), 64, 32)
    tw2 = B.H3TimeWeights(*[ctypes.c_void_p(256)] * 9)
    rc = lib.h3_denoise(ctypes.byref(shape), 0, 1, tp, None, ctypes.byref(hw), ctypes.byref(rw2),
                        ctypes.byref(tw2), sig2, None, None, None, None, ctypes.c_void_p(256),
                        1 << 40, None)
    assert rc == B.H3_EINVAL and "head widths" in B.last_error()


def test_token_reduction_validates_before_launch(lib):
    sh = S.FASTH3_TINY
    shape, ts = _shape(sh)
    tp = ts.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    red, pairs, first = S.token_pairs(sh)
    rshape, rts = _shape(red)
    tr = B.TokenReduction(rshape, rts, None, None, 1, 3)
    n = lib.h3_dit_forward_tr_workspace_bytes(ctypes.byref(shape), tp, ctypes.byref(tr.c))
    assert n > lib.h3_workspace_bytes(ctypes.byref(shape), tp, B.H3_WS_DIT)
    hw = B.H3HeadWeights(ctypes.c_void_p(256), ctypes.c_void_p(256), ctypes.c_void_p(256),
                         ctypes.c_void_p(256), 96, 32)
    w = (B.H3BlockWeights * 4)(*[B.H3BlockWeights(*[ctypes.c_void_p(256)] * 10)] * 4)

    def call(trc, L=4):
        return lib.h3_dit_forward_tr(ctypes.byref(shape), L, tp, ctypes.byref(trc), w,
                                     ctypes.byref(hw), ctypes.c_void_p(256), ctypes.c_void_p(256),
                                     None, ctypes.c_void_p(256), ctypes.c_void_p(256),
                                     ctypes.c_void_p(256), ctypes.c_void_p(256), 1 << 40, None)
    assert call(tr.c) == B.H3_EINVAL and "pairs" in B.last_error()
    bad = B.TokenReduction(rshape, rts, None, None, 3, 1)
    assert call(bad.c) == B.H3_EINVAL and "reduce_at" in B.last_error()
    bad = B.TokenReduction(rshape, rts, None, None, 1, 5)
    assert call(bad.c) == B.H3_EINVAL
    rs2 = B.H3Shape.from_buffer_copy(rshape)
    rs2.hidden = 512
    bad = B.TokenReduction(rs2, rts, None, None, 1, 3)
    assert call(bad.c) == B.H3_EINVAL and "reduced shape" in B.last_error()
    assert lib.h3_dit_forward_tr(ctypes.byref(shape), 4, tp, None, w, ctypes.byref(hw), None,
                                 None, None, None, None, None, None, 0, None) == B.H3_EINVAL


def test_calibration_validates_before_launch(lib):
    rc = lib.h3_calibrate_mfma(None, 1 << 20, 8, 10, ctypes.c_void_p(256), None)
    assert rc == B.H3_EINVAL and "NULL" in B.last_error()
    rc = lib.h3_calibrate_mfma(ctypes.c_void_p(256), 24, 8, 10, ctypes.c_void_p(256), None)
    assert rc == B.H3_EINVAL and "multiple of 16" in B.last_error()
    rc = lib.h3_calibrate_mfma(ctypes.c_void_p(256), 1 << 20, 0, 10, ctypes.c_void_p(256), None)
    assert rc == B.H3_EINVAL


@pytest.mark.parametrize("n_video,top_k,hidden,code", [
    (130944, 512, 256, B.H3_OK),                  # 2,048 tiles, 4,096 chunks, top-k 512
    (131008, 512, 256, B.H3_EUNSUPPORTED),        # 2,049 tiles (and 4,098 chunks)
    (130944, 513, 256, B.H3_EUNSUPPORTED),        # 513 selected tiles
    (1024, 4, 8192, B.H3_OK),                     # the widest hidden the row kernels hold
    (1024, 4, 8448, B.H3_EUNSUPPORTED),
])
def test_size_limits_on_host(lib, n_video, top_k, hidden, code):
    """The plan accepts the kernels' limits and refuses one step beyond, on the
    host (the limits size LDS tables and per-lane score registers)."""
    sh = S.Shape(64, 64, n_video, hidden, 4, 64, 256, tile=64, top_k=top_k)
    shape, ts = _shape(sh)
    lay = B.H3WsLayout()
    rc = lib.h3_workspace_layout(ctypes.byref(shape),
                                 ts.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                 B.H3_WS_BLOCK, ctypes.byref(lay))
    assert rc == code, B.last_error()



def test_binding_refuses_wrong_tensors_before_any_call():
    """The binding checks every tensor's type, element count, layout and device
    against the shape on the host (the C ABI cannot see buffer sizes), so a
    wrong tensor raises H3Error instead of reaching a kernel."""
    import torch
    sh = S.TINY
    shape, ts = _shape(sh)
    R, H, nh, d = sh.rows, sh.hidden, sh.n_heads, sh.head_dim
    bf = lambda n: torch.zeros(n, dtype=torch.int16)
    f32 = lambda n: torch.zeros(n, dtype=torch.float32)
    w = {k: bf(int(np.prod(v))) for k, v in S.block_shapes(sh).items()}
    ws = torch.zeros(256, dtype=torch.uint8)
    mod, rope, x, xo = f32(18 * H), f32(R * d), bf(R * H), bf(R * H)

    def refused(fn, what):
        with pytest.raises(B.H3Error) as e:
            fn()
        assert e.value.code == B.H3_EINVAL and what in str(e.value), str(e.value)

    # right sizes on the host: refused only because they are not device tensors
    refused(lambda: B.block_forward(shape, ts, w, mod, rope, x, xo, ws), "not a device tensor")
    # wrong element counts, types and layouts are named
    refused(lambda: B.block_forward(shape, ts, w, f32(17 * H), rope, x, xo, ws), "mod: ")
    refused(lambda: B.block_forward(shape, ts, w, mod, f32(R * d - 2), x, xo, ws), "rope: ")
    refused(lambda: B.block_forward(shape, ts, w, mod, rope, bf(R * H - 1), xo, ws), "x_in: ")
    refused(lambda: B.block_forward(shape, ts, w, mod, rope, x, f32(R * H), ws), "x_out: dtype")
    bad = dict(w, w_o=bf(H * H + 8))
    refused(lambda: B.block_forward(shape, ts, bad, mod, rope, x, xo, ws), "w_o: ")
    bad = dict(w, w_fc1=bf(2 * H * sh.ffn).view(2 * sh.ffn, H)[::2])
    refused(lambda: B.block_forward(shape, ts, bad, mod, rope, x, xo, ws), "w_fc1: not contiguous")
    q = bf(nh * R * d)
    refused(lambda: B.routed_attn(shape, ts, q, q, bf(nh * R * d - 64), bf(R * H), ws), "v: ")
    refused(lambda: B.routed_attn(shape, ts, q, q, q, bf(R * H), ws,
                                  sel=torch.zeros(3, dtype=torch.int32)), "sel: ")
    head = {k: bf(int(np.prod(v.shape))).view(v.shape) for k, v in S.head_weights(sh).items()}
    vv, va = f32(sh.n_video * sh.c_video), f32(sh.n_audio * sh.c_audio)
    refused(lambda: B.dit_forward(shape, ts, [w, w], head, f32(18 * H), f32(6 * H), rope, x,
                                  vv, va, ws), "mod: ")
    refused(lambda: B.dit_forward(shape, ts, [w], head, mod, f32(6 * H), rope, x,
                                  vv, f32(3), ws), "vel_audio: ")


def test_noalloc_modulation_validates_before_touching_the_gpu(lib):
    """h3_modulation_noalloc refuses a hidden width beyond its static array
    (6 x 8192 floats) and missing arguments on the host, before it looks up
    the array on a device (this runs without a GPU)."""
    shape, ts = _shape(S.TINY)
    tw = B.H3TimeWeights()
    sig = (ctypes.c_float * 3)(1, 1, 1)
    big = B.H3Shape.from_buffer_copy(shape)
    big.hidden = 8448
    rc = lib.h3_modulation_noalloc(ctypes.byref(big), 1, ctypes.byref(tw), sig, None, None, None)
    assert rc == B.H3_EUNSUPPORTED and "static scratch" in B.last_error()
    rc = lib.h3_modulation_noalloc(None, 1, ctypes.byref(tw), sig, None, None, None)
    assert rc == B.H3_EINVAL
    rc = lib.h3_modulation_noalloc(ctypes.byref(shape), 1, ctypes.byref(tw), None, None, None,
                                   None)
    assert rc == B.H3_EINVAL and "sigma3" in B.last_error()
    rc = lib.h3_modulation_noalloc(ctypes.byref(shape), 1, ctypes.byref(tw), sig, None, None, None)
    assert rc == B.H3_EINVAL and "time weights" in B.last_error()


def test_guard_bands_grow_the_plan():
    """CPU-side: the bands add (regions x band) bytes and keep every offset
    256-byte aligned; unset, the plan is the packed one."""
    from guard_bands import GUARD, guard_bands, region_starts
    sh = S.TINY
    ts, npt = S.tile_map(sh)
    shape = B.make_shape(sh, ts, npt)
    with guard_bands(0):
        plain = B.workspace_layout(shape, ts, B.H3_WS_DIT)
    with guard_bands(GUARD):
        banded = B.workspace_layout(shape, ts, B.H3_WS_DIT)
    starts = region_starts(banded, ts)
    assert all(s % 256 == 0 for s in starts)
    assert banded.total == plain.total + (len(starts) + 1) * GUARD
