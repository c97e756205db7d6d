"""Comparison metrics for GPU-vs-oracle parity (the pages' parity table uses
cosine, relative error, max abs and per-row median / p99 relative error)."""
import numpy as np


def metrics(got, ref):
    got = np.asarray(got, dtype=np.float64).reshape(len(ref), -1) if np.ndim(ref) > 1 else \
        np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64).reshape(got.shape)
    g, r = got.ravel(), ref.ravel()
    cos = float(g @ r / (np.linalg.norm(g) * np.linalg.norm(r) + 1e-300))
    rel = float(np.linalg.norm(g - r) / (np.linalg.norm(r) + 1e-300))
    out = dict(cos=cos, rel=rel, max_abs=float(np.max(np.abs(g - r))) if g.size else 0.0,
               ref_max=float(np.max(np.abs(r))) if r.size else 0.0)
    if got.ndim == 2 and got.shape[0] > 1:
        rr = np.linalg.norm(got - ref, axis=1) / (np.linalg.norm(ref, axis=1) + 1e-300)
        out["row_rel_median"] = float(np.median(rr))
        out["row_rel_p99"] = float(np.percentile(rr, 99))
    return out


def bf16_ulp(x):
    """Spacing of bf16 values at |x| (normal range)."""
    ax = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def ulp_diff(got, ref):
    """|got - ref| in units of the bf16 spacing at the reference value."""
    return np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)) / bf16_ulp(ref)


def unpad_rows(padded, tile_start, tile_pstart):
    """[..., Rp, X] in the padded tile row space -> [..., R, X]."""
    parts = [padded[..., tile_pstart[t]:tile_pstart[t] + (tile_start[t + 1] - tile_start[t]), :]
             for t in range(len(tile_start) - 1)]
    return np.concatenate(parts, axis=-2)


def padded_starts(tile_start):
    lens = np.diff(np.asarray(tile_start))
    return np.concatenate([[0], np.cumsum((lens + 31) // 32 * 32)])


def selection_agrees(sel_gpu, sel_ref, scores_ref, n_prefix_tiles, k, margin=1e-3):
    """Selected tile sets must agree wherever the oracle's k-th and (k+1)-th
    best video-tile scores differ by more than ``margin``.  Returns (number of
    (head, tile) rows checked, number of disagreements, number skipped)."""
    nh, nQ = sel_ref.shape[:2]
    checked = bad = skipped = 0
    for h in range(nh):
        for i in range(nQ):
            s = scores_ref[h, i, n_prefix_tiles:]
            s = np.where(np.isnan(s), -np.inf, s)
            if k < len(s):
                srt = np.sort(s)[::-1]
                if not (srt[k - 1] - srt[k] > margin):
                    skipped += 1
                    continue
            checked += 1
            if not np.array_equal(np.sort(sel_gpu[h, i]), np.sort(sel_ref[h, i])):
                bad += 1
    return checked, bad, skipped
