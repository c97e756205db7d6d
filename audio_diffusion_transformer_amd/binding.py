"""ctypes binding of libh3.so: argument marshalling only.

Every step of the forward runs in the library's HIP kernels; this module only
turns torch tensors into device pointers, numpy tile maps into host arrays and
python shapes into the C structs declared in include/h3.h.  If the built
library is missing, loading fails loudly: there is no other code path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libh3.so")

H3_OK, H3_EINVAL, H3_EWORKSPACE, H3_EHIP, H3_EUNSUPPORTED = 0, -1, -2, -3, -4
H3_WS_BLOCK, H3_WS_DIT, H3_WS_ATTN, H3_WS_DIT_I8 = 0, 1, 2, 3
ABI_VERSION = 5  # must match H3_ABI_VERSION in include/h3.h

KERNEL_CLASSES = ["modnorm", "gemm_qkv", "heads", "route", "attn", "gemm_o", "gemm_fc1",
                  "gemm_fc2", "final", "tables", "rows_in", "time", "euler", "tokens", "quant"]

_vp = ctypes.c_void_p


class H3Shape(ctypes.Structure):
    _fields_ = [("n_text", ctypes.c_int32), ("n_audio", ctypes.c_int32),
                ("n_video", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("n_tiles", ctypes.c_int32),
                ("n_prefix_tiles", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("pooled", ctypes.c_int32), ("norm_eps", ctypes.c_float),
                ("mlp", ctypes.c_int32), ("gate", ctypes.c_int32)]


class H3BlockWeights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("w_qkv", "b_qkv", "q_gain", "k_gain", "w_o", "b_o",
                                   "w_fc1", "b_fc1", "w_fc2", "b_fc2")]


class H3HeadWeights(ctypes.Structure):
    _fields_ = [("w_video", _vp), ("b_video", _vp), ("w_audio", _vp), ("b_audio", _vp),
                ("c_video", ctypes.c_int32), ("c_audio", ctypes.c_int32)]


class H3RowsInWeights(ctypes.Structure):
    _fields_ = [("w_video", _vp), ("b_video", _vp), ("w_audio", _vp), ("b_audio", _vp),
                ("c_video", ctypes.c_int32), ("c_audio", ctypes.c_int32)]


class H3TimeWeights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("w1", "b1", "w2", "b2", "w_mod", "b_mod", "mod_table",
                                   "w_final", "b_final")]


class H3BlockWeightsI8(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("w_qkv", "s_qkv", "b_qkv", "q_gain", "k_gain", "w_o", "s_o",
                                   "b_o", "w_fc1", "s_fc1", "b_fc1", "w_fc2", "s_fc2", "b_fc2")]


class H3TokenReduction(ctypes.Structure):
    _fields_ = [("reduced", ctypes.POINTER(H3Shape)), ("tile_start", ctypes.POINTER(ctypes.c_int32)),
                ("pairs", _vp), ("rope", _vp), ("reduce_at", ctypes.c_int32),
                ("restore_at", ctypes.c_int32)]


class H3WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("tables", "norm", "big", "q", "k", "vt", "qbar",
                                               "kbar", "vbar", "scores", "sel", "pooled",
                                               "attn", "x1", "xa", "xb", "q8", "qscale",
                                               "partial", "total")] + \
               [("padded_rows", ctypes.c_int32), ("n_query_tiles", ctypes.c_int32),
                ("n_sel", ctypes.c_int32)]


class H3Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"h3 error {code}: {msg}")
        self.code = code


_lib = None


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950) first")
    L = ctypes.CDLL(LIB_PATH)
    i32p = ctypes.POINTER(ctypes.c_int32)
    L.h3_abi_version.restype = ctypes.c_int
    L.h3_last_error.restype = ctypes.c_char_p
    L.h3_workspace_bytes.argtypes = [ctypes.POINTER(H3Shape), i32p, ctypes.c_int32]
    L.h3_workspace_bytes.restype = ctypes.c_size_t
    L.h3_workspace_layout.argtypes = [ctypes.POINTER(H3Shape), i32p, ctypes.c_int32,
                                      ctypes.POINTER(H3WsLayout)]
    L.h3_block_forward.argtypes = [ctypes.POINTER(H3Shape), i32p, ctypes.POINTER(H3BlockWeights),
                                   _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.h3_dit_forward.argtypes = [ctypes.POINTER(H3Shape), ctypes.c_int32, i32p,
                                 ctypes.POINTER(H3BlockWeights), ctypes.POINTER(H3HeadWeights),
                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.h3_routed_attn.argtypes = [ctypes.POINTER(H3Shape), i32p, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp, ctypes.c_size_t, _vp]
    L.h3_rows_in.argtypes = [ctypes.POINTER(H3Shape), ctypes.POINTER(H3RowsInWeights), _vp,
                             _vp, _vp, _vp, _vp]
    L.h3_modulation_workspace_bytes.argtypes = [ctypes.POINTER(H3Shape)]
    L.h3_modulation_workspace_bytes.restype = ctypes.c_size_t
    f32p = ctypes.POINTER(ctypes.c_float)
    L.h3_modulation.argtypes = [ctypes.POINTER(H3Shape), ctypes.c_int32,
                                ctypes.POINTER(H3TimeWeights), f32p, _vp, _vp, _vp,
                                ctypes.c_size_t, _vp]
    L.h3_modulation_noalloc.argtypes = [ctypes.POINTER(H3Shape), ctypes.c_int32,
                                        ctypes.POINTER(H3TimeWeights), f32p, _vp, _vp, _vp]
    L.h3_denoise_workspace_bytes.argtypes = [ctypes.POINTER(H3Shape), i32p, ctypes.c_int32]
    L.h3_denoise_workspace_bytes.restype = ctypes.c_size_t
    L.h3_denoise.argtypes = [ctypes.POINTER(H3Shape), ctypes.c_int32, ctypes.c_int32, i32p,
                             ctypes.POINTER(H3BlockWeights), ctypes.POINTER(H3HeadWeights),
                             ctypes.POINTER(H3RowsInWeights), ctypes.POINTER(H3TimeWeights),
                             f32p, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.h3_dit_forward_tr_workspace_bytes.argtypes = [ctypes.POINTER(H3Shape), i32p,
                                                    ctypes.POINTER(H3TokenReduction)]
    L.h3_dit_forward_tr_workspace_bytes.restype = ctypes.c_size_t
    L.h3_dit_forward_tr.argtypes = [ctypes.POINTER(H3Shape), ctypes.c_int32, i32p,
                                    ctypes.POINTER(H3TokenReduction),
                                    ctypes.POINTER(H3BlockWeights), ctypes.POINTER(H3HeadWeights),
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.h3_quantize_rows.argtypes = [_vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp, _vp,
                                   _vp]
    L.h3_dit_forward_i8.argtypes = [ctypes.POINTER(H3Shape), ctypes.c_int32, i32p,
                                    ctypes.POINTER(H3BlockWeightsI8),
                                    ctypes.POINTER(H3HeadWeights), _vp, _vp, _vp, _vp, _vp, _vp,
                                    ctypes.c_int32, _vp, ctypes.c_size_t, _vp]
    L.h3_prof_enable.argtypes = [ctypes.c_int]
    L.h3_prof_read.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                               ctypes.POINTER(ctypes.c_double)]
    L.h3_prof_kernel_name.argtypes = [ctypes.c_int32]
    L.h3_prof_kernel_name.restype = ctypes.c_char_p
    L.h3_calibrate_mfma.argtypes = [_vp, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32, _vp, _vp]
    for f in (L.h3_workspace_layout, L.h3_block_forward, L.h3_dit_forward, L.h3_routed_attn,
              L.h3_rows_in, L.h3_modulation, L.h3_modulation_noalloc, L.h3_denoise,
              L.h3_dit_forward_tr,
              L.h3_quantize_rows, L.h3_dit_forward_i8,
              L.h3_prof_enable, L.h3_prof_read):
        f.restype = ctypes.c_int
    _lib = L
    return L


def last_error():
    return lib().h3_last_error().decode()


def _check(rc):
    if rc != H3_OK:
        raise H3Error(rc, last_error())


def make_shape(sh, tile_start, n_prefix_tiles):
    """sh: any object with the fields of synth.Shape."""
    return H3Shape(sh.n_text, sh.n_audio, sh.n_video, sh.hidden, sh.n_heads, sh.head_dim,
                   sh.ffn, len(tile_start) - 1, n_prefix_tiles, sh.top_k, int(sh.pooled),
                   float(sh.norm_eps), int(getattr(sh, "mlp", 0)), int(getattr(sh, "gate", 0)))


def _tiles(tile_start):
    ts = np.ascontiguousarray(tile_start, dtype=np.int32)
    return ts, ts.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# Host-side checks of the tensors handed to the library.  The C ABI receives
# bare device pointers and cannot see a buffer's size, so a tensor of the wrong
# size, type or device would turn into an out-of-bounds device access; these
# checks refuse it with H3_EINVAL before any call.
_KINDS = {"bf16": ("int16", "uint16", "bfloat16"), "f32": ("float32",), "i32": ("int32",),
          "i8": ("int8",), "u8": ("uint8",)}


class _Checks:
    """Type, size and layout of each tensor are checked as it is named; the
    device of all of them at the end (done), so a wrong size is reported even
    for host tensors."""

    def __init__(self):
        self.named = []

    def __call__(self, t, name, numel, kind, optional=False):
        if t is None:
            if optional:
                return
            raise H3Error(H3_EINVAL, f"{name}: a tensor is required")
        dt = str(t.dtype).replace("torch.", "")
        if dt not in _KINDS[kind]:
            raise H3Error(H3_EINVAL, f"{name}: dtype {dt}, expected {kind}")
        if numel and t.numel() != numel:   # nothing is read or written when numel is 0
            raise H3Error(H3_EINVAL, f"{name}: {t.numel()} elements, expected {numel}")
        if not t.is_contiguous():
            raise H3Error(H3_EINVAL, f"{name}: not contiguous")
        self.named.append((name, t))

    def done(self):
        for name, t in self.named:
            if not t.is_cuda:
                raise H3Error(H3_EINVAL, f"{name}: not a device tensor")


class _Dims:
    """Tensor sizes implied by an H3Shape (see include/h3.h)."""

    def __init__(self, s: H3Shape):
        self.T, self.A_rows, self.V = s.n_text, s.n_audio, s.n_video
        self.R = s.n_text + s.n_audio + s.n_video
        self.H, self.nh, self.d, self.F = s.hidden, s.n_heads, s.head_dim, s.ffn
        self.A = s.n_heads * s.head_dim
        self.parts = 3 + (1 if s.gate else 0)
        self.F1 = 2 * s.ffn if s.mlp == 1 else s.ffn
        self.nT, self.npt = s.n_tiles, s.n_prefix_tiles
        self.nQ = s.n_tiles - s.n_prefix_tiles
        self.nsel = min(s.top_k, self.nQ) if self.nQ > 0 else 0


def _check_block_weights(_expect, w, D: _Dims, tag=""):
    if not isinstance(w, dict):
        return  # a prebuilt struct: the caller vouches for its pointers
    for n, numel in (("w_qkv", D.parts * D.A * D.H), ("b_qkv", D.parts * D.A),
                     ("q_gain", D.d), ("k_gain", D.d), ("w_o", D.H * D.A), ("b_o", D.H),
                     ("w_fc1", D.F1 * D.H), ("b_fc1", D.F1), ("w_fc2", D.H * D.F),
                     ("b_fc2", D.H)):
        _expect(w.get(n), tag + n, numel, "bf16")


def _check_block_weights_i8(_expect, w, D: _Dims, tag=""):
    if not isinstance(w, dict):
        return
    for n, rows, cols in (("qkv", D.parts * D.A, D.H), ("o", D.H, D.A), ("fc1", D.F1, D.H),
                          ("fc2", D.H, D.F)):
        _expect(w.get("w_" + n), tag + "w_" + n, rows * cols, "i8")
        _expect(w.get("s_" + n), tag + "s_" + n, rows, "f32")
        _expect(w.get("b_" + n), tag + "b_" + n, rows, "bf16")
    _expect(w.get("q_gain"), tag + "q_gain", D.d, "bf16")
    _expect(w.get("k_gain"), tag + "k_gain", D.d, "bf16")


def _check_heads(_expect, hw, D: _Dims):
    if not isinstance(hw, dict):
        return
    cv, ca = int(hw["w_video"].shape[0]), int(hw["w_audio"].shape[0])
    _expect(hw["w_video"], "w_video", cv * D.H, "bf16")
    _expect(hw.get("b_video"), "b_video", cv, "bf16")
    _expect(hw["w_audio"], "w_audio", ca * D.H, "bf16")
    _expect(hw.get("b_audio"), "b_audio", ca, "bf16")
    return cv, ca


def _check_forward_io(_expect, D: _Dims, n_blocks, heads, mod, mod_final, rope, x_in, vel_video,
                      vel_audio, ws):
    _expect(mod, "mod", n_blocks * 3 * 6 * D.H, "f32", optional=n_blocks == 0)
    _expect(mod_final, "mod_final", 3 * 2 * D.H, "f32")
    _expect(rope, "rope", D.R * D.d, "f32", optional=True)
    _expect(x_in, "x_in", D.R * D.H, "bf16")
    c = _check_heads(_expect, heads, D)
    if c is not None:
        _expect(vel_video, "vel_video", D.V * c[0], "f32")
        _expect(vel_audio, "vel_audio", D.A_rows * c[1], "f32")
    _expect(ws, "ws", None, "u8")


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def workspace_bytes(shape: H3Shape, tile_start, which):
    ts, tp = _tiles(tile_start)
    n = lib().h3_workspace_bytes(ctypes.byref(shape), tp, which)
    if n == 0:
        raise H3Error(H3_EINVAL, last_error())
    return n


def workspace_layout(shape: H3Shape, tile_start, which) -> H3WsLayout:
    ts, tp = _tiles(tile_start)
    out = H3WsLayout()
    _check(lib().h3_workspace_layout(ctypes.byref(shape), tp, which, ctypes.byref(out)))
    return out


def block_weights_struct(w):
    """w: dict of device torch tensors (bf16 or int16/uint16 raw bits)."""
    return H3BlockWeights(*[_ptr(w[n]) for n, _ in H3BlockWeights._fields_])


def head_weights_struct(hw):
    return H3HeadWeights(_ptr(hw["w_video"]), _ptr(hw["b_video"]), _ptr(hw["w_audio"]),
                         _ptr(hw["b_audio"]), int(hw["w_video"].shape[0]),
                         int(hw["w_audio"].shape[0]))


def block_forward(shape, tile_start, w, mod, rope, x_in, x_out, ws, stream=None):
    D, _expect = _Dims(shape), _Checks()
    _check_block_weights(_expect, w, D)
    _expect(mod, "mod", 3 * 6 * D.H, "f32")
    _expect(rope, "rope", D.R * D.d, "f32", optional=True)
    _expect(x_in, "x_in", D.R * D.H, "bf16")
    _expect(x_out, "x_out", D.R * D.H, "bf16")
    _expect(ws, "ws", None, "u8")
    _expect.done()
    ts, tp = _tiles(tile_start)
    ws_struct = block_weights_struct(w) if isinstance(w, dict) else w
    _check(lib().h3_block_forward(ctypes.byref(shape), tp, ctypes.byref(ws_struct), _ptr(mod),
                                  _ptr(rope), _ptr(x_in), _ptr(x_out), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)))


def dit_forward(shape, tile_start, blocks, heads, mod, mod_final, rope, x_in, vel_video,
                vel_audio, ws, stream=None):
    """blocks: list of weight dicts or a prebuilt (H3BlockWeights * L) array."""
    D, _expect = _Dims(shape), _Checks()
    for l, b in enumerate(blocks if isinstance(blocks, (list, tuple)) else ()):
        _check_block_weights(_expect, b, D, f"block {l} ")
    _check_forward_io(_expect, D, len(blocks), heads, mod, mod_final, rope, x_in, vel_video,
                      vel_audio, ws)
    _expect.done()
    ts, tp = _tiles(tile_start)
    if isinstance(blocks, (list, tuple)):
        arr = (H3BlockWeights * max(len(blocks), 1))(*[block_weights_struct(b) for b in blocks])
        n = len(blocks)
    else:
        arr, n = blocks, len(blocks)
    hw = head_weights_struct(heads) if isinstance(heads, dict) else heads
    _check(lib().h3_dit_forward(ctypes.byref(shape), n, tp, arr, ctypes.byref(hw), _ptr(mod),
                                _ptr(mod_final), _ptr(rope), _ptr(x_in), _ptr(vel_video),
                                _ptr(vel_audio), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)))


def routed_attn(shape, tile_start, q, k, v, out, ws, sel=None, scores=None, gate=None,
                stream=None):
    D, _expect = _Dims(shape), _Checks()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _expect(t, n, D.nh * D.R * D.d, "bf16")
    _expect(gate, "gate", D.R * D.A, "bf16", optional=True)
    _expect(out, "out", D.R * D.A, "bf16")
    _expect(sel, "sel", D.nh * D.nQ * D.nsel, "i32", optional=True)
    _expect(scores, "scores", D.nh * D.nQ * D.nT, "f32", optional=True)
    _expect(ws, "ws", None, "u8")
    _expect.done()
    ts, tp = _tiles(tile_start)
    _check(lib().h3_routed_attn(ctypes.byref(shape), tp, _ptr(q), _ptr(k), _ptr(v), _ptr(gate),
                                _ptr(out), _ptr(sel), _ptr(scores), _ptr(ws),
                                ws.numel() * ws.element_size(), _stream(stream)))


def rows_in_weights_struct(w):
    """w: dict of device fp32 tensors w_video [H][cv], b_video, w_audio [H][ca], b_audio."""
    return H3RowsInWeights(_ptr(w["w_video"]), _ptr(w["b_video"]), _ptr(w["w_audio"]),
                           _ptr(w["b_audio"]), int(w["w_video"].shape[1]),
                           int(w["w_audio"].shape[1]))


def time_weights_struct(tw):
    return H3TimeWeights(*[_ptr(tw[n]) for n, _ in H3TimeWeights._fields_])


def _f32_host(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _check_rows_in(_expect, D: _Dims, w, text_rows):
    if not isinstance(w, dict):
        return None
    cv, ca = int(w["w_video"].shape[1]), int(w["w_audio"].shape[1])
    _expect(w["w_video"], "w_video", D.H * cv, "f32")
    _expect(w.get("b_video"), "b_video", D.H, "f32")
    _expect(w["w_audio"], "w_audio", D.H * ca, "f32")
    _expect(w.get("b_audio"), "b_audio", D.H, "f32")
    _expect(text_rows, "text_rows", D.T * D.H, "bf16")
    return cv, ca


def rows_in(shape, w, text_rows, audio_patch, video_patch, x, stream=None):
    D, _expect = _Dims(shape), _Checks()
    c = _check_rows_in(_expect, D, w, text_rows)
    if c is not None:
        _expect(audio_patch, "audio_patch", D.A_rows * c[1], "f32")
        _expect(video_patch, "video_patch", D.V * c[0], "f32")
    _expect(x, "x", D.R * D.H, "bf16")
    _expect.done()
    ws_ = rows_in_weights_struct(w) if isinstance(w, dict) else w
    _check(lib().h3_rows_in(ctypes.byref(shape), ctypes.byref(ws_), _ptr(text_rows),
                            _ptr(audio_patch), _ptr(video_patch), _ptr(x), _stream(stream)))


def _check_time_weights(_expect, tw, D: _Dims, n_blocks):
    if not isinstance(tw, dict):
        return
    H = D.H
    for n, numel in (("w1", H * 256), ("b1", H), ("w2", H * H), ("b2", H), ("w_mod", 6 * H * H),
                     ("b_mod", 6 * H), ("mod_table", n_blocks * 6 * H), ("w_final", 2 * H * H),
                     ("b_final", 2 * H)):
        _expect(tw.get(n), n, numel, "bf16")


def modulation_workspace_bytes(shape):
    n = lib().h3_modulation_workspace_bytes(ctypes.byref(shape))
    if n == 0:
        raise H3Error(H3_EINVAL, last_error())
    return n


def modulation(shape, n_blocks, tw, sigma3, mod, mod_final, ws, stream=None):
    """sigma3: host (text, audio, video) timesteps."""
    D, _expect = _Dims(shape), _Checks()
    _check_time_weights(_expect, tw, D, n_blocks)
    _expect(mod, "mod", n_blocks * 3 * 6 * D.H, "f32")
    _expect(mod_final, "mod_final", 3 * 2 * D.H, "f32")
    _expect(ws, "ws", None, "u8")
    _expect.done()
    tws = time_weights_struct(tw) if isinstance(tw, dict) else tw
    sg, sp = _f32_host(sigma3)
    _check(lib().h3_modulation(ctypes.byref(shape), n_blocks, ctypes.byref(tws), sp, _ptr(mod),
                               _ptr(mod_final), _ptr(ws), ws.numel() * ws.element_size(),
                               _stream(stream)))


def modulation_noalloc(shape, n_blocks, tw, sigma3, mod, mod_final, stream=None):
    """h3_modulation with the library's static scratch (no workspace argument)."""
    D, _expect = _Dims(shape), _Checks()
    _check_time_weights(_expect, tw, D, n_blocks)
    _expect(mod, "mod", n_blocks * 3 * 6 * D.H, "f32", optional=n_blocks == 0)
    _expect(mod_final, "mod_final", 3 * 2 * D.H, "f32")
    _expect.done()
    tws = time_weights_struct(tw) if isinstance(tw, dict) else tw
    sg, sp = _f32_host(sigma3)
    _check(lib().h3_modulation_noalloc(ctypes.byref(shape), n_blocks, ctypes.byref(tws), sp,
                                       _ptr(mod), _ptr(mod_final), _stream(stream)))


def denoise_workspace_bytes(shape, tile_start, n_blocks):
    ts, tp = _tiles(tile_start)
    n = lib().h3_denoise_workspace_bytes(ctypes.byref(shape), tp, n_blocks)
    if n == 0:
        raise H3Error(H3_EINVAL, last_error())
    return n


def denoise(shape, tile_start, blocks, heads, rows_w, tw, sigmas, rope, text_rows, video_latent,
            audio_latent, ws, stream=None):
    """sigmas: host [n_steps + 1][3]; the latents (fp32 device) are updated in place."""
    D, _expect = _Dims(shape), _Checks()
    for l, b in enumerate(blocks if isinstance(blocks, (list, tuple)) else ()):
        _check_block_weights(_expect, b, D, f"block {l} ")
    _check_time_weights(_expect, tw, D, len(blocks))
    ch = _check_heads(_expect, heads, D)
    ci = _check_rows_in(_expect, D, rows_w, text_rows)
    if ch is not None and ci is not None and ch != ci:
        raise H3Error(H3_EINVAL, f"head widths {ch} differ from the patch widths {ci}")
    c = ch or ci
    if c is not None:
        _expect(video_latent, "video_latent", D.V * c[0], "f32")
        _expect(audio_latent, "audio_latent", D.A_rows * c[1], "f32")
    _expect(rope, "rope", D.R * D.d, "f32", optional=True)
    _expect(ws, "ws", None, "u8")
    _expect.done()
    ts, tp = _tiles(tile_start)
    if isinstance(blocks, (list, tuple)):
        arr = (H3BlockWeights * max(len(blocks), 1))(*[block_weights_struct(b) for b in blocks])
        n = len(blocks)
    else:
        arr, n = blocks, len(blocks)
    hw = head_weights_struct(heads) if isinstance(heads, dict) else heads
    rw = rows_in_weights_struct(rows_w) if isinstance(rows_w, dict) else rows_w
    tws = time_weights_struct(tw) if isinstance(tw, dict) else tw
    sg, sp = _f32_host(sigmas)
    _check(lib().h3_denoise(ctypes.byref(shape), n, len(sg) - 1, tp, arr, ctypes.byref(hw),
                            ctypes.byref(rw), ctypes.byref(tws), sp, _ptr(rope), _ptr(text_rows),
                            _ptr(video_latent), _ptr(audio_latent), _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(stream)))


class TokenReduction:
    """Keeps the C struct and the host arrays it points to alive together."""

    def __init__(self, red_shape: H3Shape, red_tile_start, pairs, rope, reduce_at, restore_at):
        self.shape = red_shape
        self.ts, tp = _tiles(red_tile_start)
        self.pairs, self.rope = pairs, rope
        self.c = H3TokenReduction(ctypes.pointer(self.shape), tp, _ptr(pairs), _ptr(rope),
                                  int(reduce_at), int(restore_at))


def dit_forward_tr_workspace_bytes(shape, tile_start, tr: TokenReduction):
    ts, tp = _tiles(tile_start)
    n = lib().h3_dit_forward_tr_workspace_bytes(ctypes.byref(shape), tp, ctypes.byref(tr.c))
    if n == 0:
        raise H3Error(H3_EINVAL, last_error())
    return n


def dit_forward_tr(shape, tile_start, tr: TokenReduction, blocks, heads, mod, mod_final, rope,
                   x_in, vel_video, vel_audio, ws, stream=None):
    D, _expect = _Dims(shape), _Checks()
    for l, b in enumerate(blocks if isinstance(blocks, (list, tuple)) else ()):
        _check_block_weights(_expect, b, D, f"block {l} ")
    _check_forward_io(_expect, D, len(blocks), heads, mod, mod_final, rope, x_in, vel_video,
                      vel_audio, ws)
    Dr = _Dims(tr.shape)
    _expect(tr.pairs, "pairs", Dr.V * 2, "i32")
    _expect(tr.rope, "reduced rope", Dr.R * Dr.d, "f32", optional=True)
    _expect.done()
    ts, tp = _tiles(tile_start)
    if isinstance(blocks, (list, tuple)):
        arr = (H3BlockWeights * max(len(blocks), 1))(*[block_weights_struct(b) for b in blocks])
        n = len(blocks)
    else:
        arr, n = blocks, len(blocks)
    hw = head_weights_struct(heads) if isinstance(heads, dict) else heads
    _check(lib().h3_dit_forward_tr(ctypes.byref(shape), n, tp, ctypes.byref(tr.c), arr,
                                   ctypes.byref(hw), _ptr(mod), _ptr(mod_final), _ptr(rope),
                                   _ptr(x_in), _ptr(vel_video), _ptr(vel_audio), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)))


def quantize_rows(x, q, scale, group=0, stream=None):
    """int8 codes of the bf16 matrix x [rows][cols] (device tensors)."""
    rows, cols = x.shape
    _expect = _Checks()
    _expect(x, "x", rows * cols, "bf16")
    _expect(q, "q", rows * cols, "i8")
    _expect(scale, "scale", rows * (cols // group if group > 0 else 1), "f32")
    _expect.done()
    _check(lib().h3_quantize_rows(_ptr(x), rows, cols, group, _ptr(q), _ptr(scale),
                                  _stream(stream)))


def quantize_block(w, stream=None):
    """int8 codes and row scales of a block's four products: w is a dict of
    device tensors (bf16 bits); returns the dict of h3_block_weights_i8."""
    import torch
    out = {k: w[k] for k in ("b_qkv", "q_gain", "k_gain", "b_o", "b_fc1", "b_fc2")}
    for n in ("qkv", "o", "fc1", "fc2"):
        m = w["w_" + n]
        out["w_" + n] = torch.empty(m.shape, dtype=torch.int8, device=m.device)
        out["s_" + n] = torch.empty(m.shape[0], dtype=torch.float32, device=m.device)
        quantize_rows(m, out["w_" + n], out["s_" + n], 0, stream)
    return out


def block_weights_i8_struct(w):
    return H3BlockWeightsI8(*[_ptr(w[n]) for n, _ in H3BlockWeightsI8._fields_])


def dit_forward_i8(shape, tile_start, blocks, heads, mod, mod_final, rope, x_in, vel_video,
                   vel_audio, ws, fc2_group=1024, stream=None):
    """blocks: list of int8 weight dicts (quantize_block) or a prebuilt array.
    fc2_group: 1024 (the FC2 input per 1,024 channels) or 0 (per row)."""
    D, _expect = _Dims(shape), _Checks()
    for l, b in enumerate(blocks if isinstance(blocks, (list, tuple)) else ()):
        _check_block_weights_i8(_expect, b, D, f"block {l} ")
    _check_forward_io(_expect, D, len(blocks), heads, mod, mod_final, rope, x_in, vel_video,
                      vel_audio, ws)
    _expect.done()
    ts, tp = _tiles(tile_start)
    if isinstance(blocks, (list, tuple)):
        arr = (H3BlockWeightsI8 * max(len(blocks), 1))(*[block_weights_i8_struct(b) for b in blocks])
        n = len(blocks)
    else:
        arr, n = blocks, len(blocks)
    hw = head_weights_struct(heads) if isinstance(heads, dict) else heads
    _check(lib().h3_dit_forward_i8(ctypes.byref(shape), n, tp, arr, ctypes.byref(hw), _ptr(mod),
                                   _ptr(mod_final), _ptr(rope), _ptr(x_in), _ptr(vel_video),
                                   _ptr(vel_audio), int(fc2_group), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)))


def calibrate_mfma(operands, n_blocks, iters, sink, stream=None):
    """Matrix-core calibration (h3_calibrate_mfma): operands a device tensor of
    random bf16 data, sink a device tensor of >= 256 floats.  Returns the FLOP
    the call performs; the caller times it."""
    _expect = _Checks()
    _expect(operands, "operands", None, "bf16")
    _expect(sink, "sink", None, "f32")
    if sink.numel() < 256:
        raise H3Error(H3_EINVAL, "sink: fewer than 256 floats")
    _expect.done()
    _check(lib().h3_calibrate_mfma(_ptr(operands), operands.numel() * operands.element_size(),
                                   n_blocks, iters, _ptr(sink), _stream(stream)))
    return n_blocks * 4 * iters * 16 * 16384


def prof_enable(on=True):
    _check(lib().h3_prof_enable(1 if on else 0))


def prof_read():
    """{kernel class: (launches, total ms)} for the spans recorded since prof_enable."""
    out = {}
    for c, name in enumerate(KERNEL_CLASSES):
        n = ctypes.c_int64()
        ms = ctypes.c_double()
        _check(lib().h3_prof_read(c, ctypes.byref(n), ctypes.byref(ms)))
        out[name] = (n.value, ms.value)
    return out
