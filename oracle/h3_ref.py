"""ctypes front end of the plain C++ oracle (h3_ref.cpp, libh3ref.so).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.  It
shares no code with the HIP library.

The C++ oracle computes the block in fp32 with one running sum per output in
ascending order, each operation rounded on its own, bf16 round-to-nearest-even
at the storage points and libm expf / erff / sqrtf; see h3_ref.h for the
passages each step follows.  The functions below take and return the same
kinds of arrays as oracle/h3_oracle.py (bf16 bits in, float64 arrays of bf16 or
fp32 values out), so a test can run either oracle.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libh3ref.so")
TEXT, AUDIO, VIDEO = 0, 1, 2
REV_MEANS, REV_SCORES = 1, 2

_vp = ctypes.c_void_p
_lib = None


class Shape(ctypes.Structure):
    _fields_ = [("n_text", ctypes.c_int32), ("n_audio", ctypes.c_int32),
                ("n_video", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("n_tiles", ctypes.c_int32),
                ("n_prefix_tiles", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("pooled", ctypes.c_int32), ("norm_eps", ctypes.c_float),
                ("mlp", ctypes.c_int32), ("gate", ctypes.c_int32)]


class BlockWeights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("w_qkv", "b_qkv", "q_gain", "k_gain", "w_o", "b_o",
                                   "w_fc1", "b_fc1", "w_fc2", "b_fc2")]


class BlockOut(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("n1", "y", "q", "k", "v", "g", "qbar", "kbar", "vbar",
                                   "scores", "sel", "pooled", "attn", "o", "x1", "n2", "h", "f",
                                   "x2")]


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from oracle import build_ref
        build_ref.build()
    L = ctypes.CDLL(LIB_PATH)
    i32, f32, i64 = ctypes.c_int32, ctypes.c_float, ctypes.c_int64
    L.h3r_last_error.restype = ctypes.c_char_p
    L.h3r_set_threads.argtypes = [i32]
    L.h3r_set_threads.restype = i32
    L.h3r_round_bf16.argtypes = [_vp, i64, _vp]
    L.h3r_modnorm.argtypes = [_vp, i32, i32, _vp, _vp, _vp, f32, _vp]
    L.h3r_linear.argtypes = [_vp, i32, i32, _vp, _vp, i32, _vp]
    L.h3r_linear_plain.argtypes = [_vp, i32, i32, _vp, _vp, i32, _vp]
    L.h3r_gelu.argtypes = [_vp, i64, _vp]
    L.h3r_silu.argtypes = [_vp, i64, _vp]
    L.h3r_qk_norm_rope.argtypes = [_vp, i32, i32, i32, _vp, _vp, f32, _vp]
    L.h3r_tile_means.argtypes = [_vp, i32, i32, i32, _vp, _vp, i32, i32, _vp]
    L.h3r_tile_scores.argtypes = [_vp, _vp, i32, i32, i32, i32, i32, _vp]
    L.h3r_topk.argtypes = [_vp, _vp, i32, i32, _vp]
    L.h3r_pooled.argtypes = [_vp, _vp, i32, i32, _vp]
    L.h3r_attention.argtypes = [ctypes.POINTER(Shape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                i32, _vp]
    L.h3r_block_forward.argtypes = [ctypes.POINTER(Shape), _vp, ctypes.POINTER(BlockWeights),
                                    _vp, _vp, _vp, _vp, i32, i32, ctypes.POINTER(BlockOut)]
    L.h3r_final_heads.argtypes = [ctypes.POINTER(Shape), _vp, _vp, i32, _vp, _vp, _vp, i32, _vp,
                                  _vp, i32, _vp, _vp]
    L.h3r_dit_forward.argtypes = [ctypes.POINTER(Shape), i32, _vp, ctypes.POINTER(BlockWeights),
                                  _vp, _vp, _vp, _vp, _vp, _vp, i32, _vp, _vp, i32, i32, _vp,
                                  _vp, _vp]
    L.h3r_routed_attn.argtypes = [ctypes.POINTER(Shape), _vp, _vp, _vp, _vp, _vp, _vp, i32, i32,
                                  _vp, _vp, _vp]
    for f in (L.h3r_attention, L.h3r_block_forward, L.h3r_final_heads, L.h3r_dit_forward,
              L.h3r_routed_attn):
        f.restype = ctypes.c_int
    _lib = L
    return L


def set_threads(n):
    """OpenMP thread count of the oracle; returns the previous count."""
    return lib().h3r_set_threads(int(n))


def _check(rc):
    if rc != 0:
        raise RuntimeError("oracle: " + lib().h3r_last_error().decode())


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return None if a is None else a.ctypes.data


def bits_to_f64(u):
    return ((np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
            .astype(np.float64))


def _bits(a):
    """bf16 input: raw bits (uint16) or float values that are exactly bf16."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return _c(a, np.uint16)
    f = np.ascontiguousarray(a, dtype=np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def make_shape(sh, tile_start, n_prefix_tiles):
    return Shape(sh.n_text, sh.n_audio, sh.n_video, sh.hidden, sh.n_heads, sh.head_dim, sh.ffn,
                 len(tile_start) - 1, n_prefix_tiles, sh.top_k, int(sh.pooled),
                 float(sh.norm_eps), int(getattr(sh, "mlp", 0)), int(getattr(sh, "gate", 0)))


# ----------------------------------------------------------------------------
# Steps
# ----------------------------------------------------------------------------

def round_bf16(x):
    """fp32 values -> bf16 values (round to nearest even), as float64."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().h3r_round_bf16(_p(x), x.size, _p(out))
    return bits_to_f64(out)


def modulated_rmsnorm(x, shift, scale, seg, eps):
    """x: bf16 values or bits [n][H]; shift, scale fp32 [3][H]; seg [n]."""
    xb = _bits(x)
    n, H = xb.shape
    out = np.empty((n, H), np.uint16)
    lib().h3r_modnorm(_p(xb), n, H, _p(_c(seg, np.int32)), _p(_c(shift, np.float32)),
                      _p(_c(scale, np.float32)), float(eps), _p(out))
    return bits_to_f64(out)


def linear(a, w, b=None):
    """fp32 (sum_k a_mk w_ok) + b_o, unrounded; a, w, b bf16 values or bits."""
    ab, wb = _bits(a), _bits(w)
    M, K = ab.shape
    N = wb.shape[0]
    bb = None if b is None else _bits(b)
    out = np.empty((M, N), np.float32)
    lib().h3r_linear(_p(ab), M, K, _p(wb), _p(bb), N, _p(out))
    return out.astype(np.float64)


def linear_plain(a, w, b=None):
    """The textbook loop of linear(), one output at a time."""
    ab, wb = _bits(a), _bits(w)
    M, K = ab.shape
    N = wb.shape[0]
    bb = None if b is None else _bits(b)
    out = np.empty((M, N), np.float32)
    lib().h3r_linear_plain(_p(ab), M, K, _p(wb), _p(bb), N, _p(out))
    return out.astype(np.float64)


def gelu(z):
    z = _c(z, np.float32)
    out = np.empty_like(z)
    lib().h3r_gelu(_p(z), z.size, _p(out))
    return out.astype(np.float64)


def silu(z):
    z = _c(z, np.float32)
    out = np.empty_like(z)
    lib().h3r_silu(_p(z), z.size, _p(out))
    return out.astype(np.float64)


def qk_norm_rope(u, gain, rope, eps):
    ub = _bits(u)
    nh, R, d = ub.shape
    out = np.empty(ub.shape, np.uint16)
    lib().h3r_qk_norm_rope(_p(ub), nh, R, d, _p(_bits(gain)),
                           None if rope is None else _p(_c(rope, np.float32)), float(eps), _p(out))
    return bits_to_f64(out)


def tile_means(u, tile_start, tiles, reverse=False):
    ub = _bits(u)
    nh, R, d = ub.shape
    tl = _c(list(tiles), np.int32)
    out = np.empty((nh, len(tl), d), np.float32)
    lib().h3r_tile_means(_p(ub), nh, R, d, _p(_c(tile_start, np.int32)), _p(tl), len(tl),
                         int(bool(reverse)), _p(out))
    return out.astype(np.float64)


def tile_scores(qbar, kbar, reverse=False):
    q, k = _c(qbar, np.float32), _c(kbar, np.float32)
    nh, nq, d = q.shape
    nk = k.shape[1]
    out = np.empty((nh, nq, nk), np.float32)
    lib().h3r_tile_scores(_p(q), _p(k), nh, nq, nk, d, int(bool(reverse)), _p(out))
    return out.astype(np.float64)


def topk_tiles(scores_row, cand, k):
    s = _c(scores_row, np.float32)
    c = _c(cand, np.int32)
    out = np.empty(min(k, len(c)), np.int32)
    lib().h3r_topk(_p(s), _p(c), len(c), int(k), _p(out))
    return out.astype(np.int64)


def pooled_branch(scores_row, vbar):
    s, v = _c(scores_row, np.float32), _c(vbar, np.float32)
    out = np.empty(v.shape[1], np.float32)
    lib().h3r_pooled(_p(s), _p(v), v.shape[0], v.shape[1], _p(out))
    return out.astype(np.float64)


def attention(sh, tile_start, n_prefix_tiles, q, k, v, sel, pooled, rows=None, gate=None):
    """bf16 attention output [len(rows)][nh d] (as float64 values) of the given
    routing results sel [nh][nQ][nsel], pooled [nh][nQ][d]."""
    shape = make_shape(sh, tile_start, n_prefix_tiles)
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    nh, R, d = qb.shape
    rr = np.arange(R, dtype=np.int32) if rows is None else _c(rows, np.int32)
    out = np.empty((len(rr), nh * d), np.uint16)
    _check(lib().h3r_attention(ctypes.byref(shape), _p(_c(tile_start, np.int32)), _p(qb), _p(kb),
                               _p(vb), _p(_c(sel, np.int32)), _p(_c(pooled, np.float32)),
                               None if gate is None else _p(_bits(gate)), _p(rr), len(rr),
                               _p(out)))
    return bits_to_f64(out)


# ----------------------------------------------------------------------------
# Block, forward, routed attention
# ----------------------------------------------------------------------------

def _weights(w):
    keep = {n: _bits(w[n]) for n, _ in BlockWeights._fields_}
    return BlockWeights(*[_p(keep[n]) for n, _ in BlockWeights._fields_]), keep


def block_forward(sh, tile_start, n_prefix_tiles, w, mod, rope, x_in, out_rows=None, reverse=0):
    """One block; returns the same intermediates as the float64 oracle's
    block_forward (float64 arrays of bf16 / fp32 values; sel as int64)."""
    ts = _c(tile_start, np.int32)
    shape = make_shape(sh, ts, n_prefix_tiles)
    R, H, nh, d, F = sh.rows, sh.hidden, sh.n_heads, sh.head_dim, sh.ffn
    A = nh * d
    parts = 4 if getattr(sh, "gate", 0) else 3
    nT = len(ts) - 1
    nQ = nT - n_prefix_tiles
    nsel = min(sh.top_k, nQ) if nQ > 0 else 0
    rows = np.arange(R, dtype=np.int32) if out_rows is None else _c(out_rows, np.int32)
    n = len(rows)
    bufs = dict(n1=np.empty((R, H), np.uint16), y=np.empty((R, parts * A), np.uint16),
                q=np.empty((nh, R, d), np.uint16), k=np.empty((nh, R, d), np.uint16),
                v=np.empty((nh, R, d), np.uint16),
                g=np.empty((nh, R, d), np.uint16) if parts == 4 else None,
                qbar=np.empty((nh, nQ, d), np.float32), kbar=np.empty((nh, nT, d), np.float32),
                vbar=np.empty((nh, nT, d), np.float32), scores=np.empty((nh, nQ, nT), np.float32),
                sel=np.empty((nh, nQ, nsel), np.int32), pooled=np.empty((nh, nQ, d), np.float32),
                attn=np.empty((n, A), np.uint16), o=np.empty((n, H), np.uint16),
                x1=np.empty((n, H), np.uint16), n2=np.empty((n, H), np.uint16),
                h=np.empty((n, F), np.uint16), f=np.empty((n, H), np.uint16),
                x2=np.empty((n, H), np.uint16))
    out = BlockOut(*[_p(bufs[k_]) for k_, _ in BlockOut._fields_])
    wc, keep = _weights(w)
    _check(lib().h3r_block_forward(ctypes.byref(shape), _p(ts), ctypes.byref(wc),
                                   _p(_c(mod, np.float32)),
                                   None if rope is None else _p(_c(rope, np.float32)),
                                   _p(_bits(x_in)), _p(rows), n, int(reverse), ctypes.byref(out)))
    res = {}
    for k_, a in bufs.items():
        if a is None:
            res[k_] = None
        elif a.dtype == np.uint16:
            res[k_] = bits_to_f64(a)
        elif a.dtype == np.int32:
            res[k_] = a.astype(np.int64)
        else:
            res[k_] = a.astype(np.float64)
    res["rows"] = rows.astype(np.int64)
    res["x2_bits"] = bufs["x2"]
    return res


def final_heads(sh, x, seg, mod_final, head):
    """Final norm and heads of the rows x [n][H] (bf16 values or bits) with
    segments seg [n]: (vel_video of the video rows, vel_audio of the audio rows)."""
    xb = _bits(x)
    seg = _c(seg, np.int32)
    cv, ca = head["w_video"].shape[0], head["w_audio"].shape[0]
    vv = np.empty((int(np.sum(seg == VIDEO)), cv), np.float32)
    va = np.empty((int(np.sum(seg == AUDIO)), ca), np.float32)
    shape = Shape(sh.n_text, sh.n_audio, sh.n_video, sh.hidden, sh.n_heads, sh.head_dim, sh.ffn,
                  1, 0, 1, 0, float(sh.norm_eps), 0, 0)
    hk = {k_: _bits(v_) for k_, v_ in head.items()}
    _check(lib().h3r_final_heads(ctypes.byref(shape), _p(xb), _p(seg), len(seg),
                                 _p(_c(mod_final, np.float32)), _p(hk["w_video"]),
                                 _p(hk["b_video"]), cv, _p(hk["w_audio"]), _p(hk["b_audio"]), ca,
                                 _p(vv), _p(va)))
    return vv.astype(np.float64), va.astype(np.float64)


def dit_forward(sh, tile_start, n_prefix_tiles, blocks, head, mods, mod_final, rope, x_in,
                reverse=0):
    ts = _c(tile_start, np.int32)
    shape = make_shape(sh, ts, n_prefix_tiles)
    L = len(blocks)
    arr = (BlockWeights * max(L, 1))()
    keep = []
    for l, w in enumerate(blocks):
        arr[l], kk = _weights(w)
        keep.append(kk)
    hk = {k_: _bits(v_) for k_, v_ in head.items()}
    cv, ca = hk["w_video"].shape[0], hk["w_audio"].shape[0]
    vv = np.empty((sh.n_video, cv), np.float32)
    va = np.empty((sh.n_audio, ca), np.float32)
    xo = np.empty((sh.rows, sh.hidden), np.uint16)
    md = _c(mods, np.float32) if L else None
    _check(lib().h3r_dit_forward(ctypes.byref(shape), L, _p(ts), arr, _p(md),
                                 _p(_c(mod_final, np.float32)),
                                 None if rope is None else _p(_c(rope, np.float32)),
                                 _p(_bits(x_in)), _p(hk["w_video"]), _p(hk["b_video"]), cv,
                                 _p(hk["w_audio"]), _p(hk["b_audio"]), ca, int(reverse), _p(vv),
                                 _p(va), _p(xo)))
    return dict(x=bits_to_f64(xo), x_bits=xo, vel_video=vv.astype(np.float64),
                vel_audio=va.astype(np.float64))


def routed_attn(sh, tile_start, n_prefix_tiles, q_bits, k_bits, v_bits, rows=None, gate=None,
                reverse=0):
    ts = _c(tile_start, np.int32)
    shape = make_shape(sh, ts, n_prefix_tiles)
    qb, kb, vb = _bits(q_bits), _bits(k_bits), _bits(v_bits)
    nh, R, d = qb.shape
    nT = len(ts) - 1
    nQ = nT - n_prefix_tiles
    nsel = min(sh.top_k, nQ) if nQ > 0 else 0
    rr = np.arange(R, dtype=np.int32) if rows is None else _c(rows, np.int32)
    out = np.empty((len(rr), nh * d), np.uint16)
    sel = np.empty((nh, nQ, nsel), np.int32)
    scores = np.empty((nh, nQ, nT), np.float32)
    _check(lib().h3r_routed_attn(ctypes.byref(shape), _p(ts), _p(qb), _p(kb), _p(vb),
                                 None if gate is None else _p(_bits(gate)), _p(rr), len(rr),
                                 int(reverse), _p(out), _p(sel), _p(scores)))
    return dict(out=bits_to_f64(out), out_bits=out, sel=sel.astype(np.int64),
                scores=scores.astype(np.float64))
