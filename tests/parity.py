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


def selection_follows_scores(sel_gpu, scores_gpu, n_prefix_tiles, k):
    """Every (head, query tile) row: the GPU's selection must be exactly the
    rule's top-k of the GPU's own fp32 tile scores (TensorFold PR #949,
    "Kernel contract": NaN ranks as -inf, ties go to the lower tile; ids in
    ascending order).  The rule is applied by the oracle's top-k on those
    same fp32 values, so the decision is taken in the same precision on both
    sides.  Returns the number of rows that differ."""
    from oracle import h3_ref
    nh, nQ = sel_gpu.shape[:2]
    n_tiles = scores_gpu.shape[2]
    cand = np.arange(n_prefix_tiles, n_tiles)
    bad = 0
    for h in range(nh):
        for i in range(nQ):
            want = h3_ref.topk_tiles(scores_gpu[h, i].astype(np.float32), cand, k)
            if not np.array_equal(np.asarray(sel_gpu[h, i]), want):
                bad += 1
    return bad


def close_bf16(got, ref, ulps=2.0, atol=1e-5, frac_1ulp=1e-3):
    """Every element within `ulps` bf16 spacings of the reference plus `atol`,
    and at most a fraction `frac_1ulp` of the elements more than one spacing
    away.  Returns the worst excess over the elementwise bar (<= 0 passes);
    a violated fraction is reported as a positive excess too."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if got.size == 0:
        return 0.0
    err = np.abs(got - ref)
    ulp = bf16_ulp(ref)
    worst = float(np.max(err - ulps * ulp - atol))
    frac = float(np.mean(err > ulp + 1e-12))
    if worst > 0 or frac > frac_1ulp:
        print(f"close_bf16: worst excess {worst:.3g}, fraction beyond 1 spacing {frac:.3g}",
              flush=True)
        return max(worst, frac - frac_1ulp)
    return worst


class Checks:
    """Collects every comparison of a case, prints them all, then asserts."""

    def __init__(self, case):
        self.case = case
        self.failed = []
        self.lines = []

    def close(self, name, got, ref, **kw):
        ex = close_bf16(got, ref, **kw)
        self.lines.append(f"{name}: excess {ex:.3g}")
        if ex > 0:
            self.failed.append(name)

    def true(self, name, cond, info=""):
        self.lines.append(f"{name}: {'ok' if cond else 'FAIL'} {info}")
        if not cond:
            self.failed.append(name)

    def done(self):
        print(f"[{self.case}] " + "; ".join(self.lines), flush=True)
        assert not self.failed, f"{self.case}: failed {self.failed}"

    def failures(self):
        return list(self.failed)


# ----------------------------------------------------------------------------
# The comparisons of the GPU parity tests, as functions of (result under test,
# oracle result), so that the planted controls (tests/test_controls.py) run
# exactly the checks the GPU tests run.
# ----------------------------------------------------------------------------

def routed_checks(c, g, r, n_prefix_tiles, top_k, rows=None, strict_sel=True):
    """Routed attention: selection (margin rule against the oracle; the rule's
    top-k of the result's own scores everywhere), fp32 scores, and the bf16
    output (cos/rel and elementwise, rows = the oracle's rows)."""
    checked, bad, skipped = selection_agrees(g["sel"], r["sel"], r["scores"], n_prefix_tiles,
                                             top_k)
    c.true("sel", bad == 0 and (not strict_sel or checked >= 0.9 * (checked + skipped)),
           f"checked {checked} bad {bad} skipped {skipped}")
    own = selection_follows_scores(g["sel"], g["scores"], n_prefix_tiles, top_k)
    c.true("sel = rule top-k of own scores", own == 0, f"{own} rows differ")
    err = float(np.max(np.abs(g["scores"] - r["scores"]))) if r["scores"].size else 0.0
    c.true("scores", err < 1e-3, f"{err:.3g}")
    got = g["out"] if rows is None else g["out"][rows]
    m = metrics(got, r["out"])
    c.true("out metrics", m["cos"] > 0.99999 and m["rel"] < 4e-3, str(m))
    c.true("out elementwise",
           bool(np.all(np.abs(got - r["out"]) <= 4e-3 + 2 ** -7 * np.abs(r["out"]))))


def rounding_probe_checks(c, got, ref, max_frac=0.01):
    """Attention on the softmax probe (every row's largest score at key row 0):
    the online softmax then rounds its weights against the final max from the
    first key chunk on, so the bf16 outputs must equal the oracle's bit for
    bit except where fp32 sum order decides a rounding (a small fraction)."""
    frac = float(np.mean(np.asarray(got) != np.asarray(ref)))
    c.true("probe bytes", frac <= max_frac, f"fraction differing {frac:.4f}")


def block_checks(c, g, r, n_prefix_tiles, n_tiles, top_k, pooled, strict_sel=True,
                 h_frac=2e-2, v_atol=2 ** -11):
    """One block, stage by stage (q, k, v; tile means, scores, selection,
    pooled; attention; x1, n2, h, x2)."""
    # a flip of one upstream bf16 value (norm output, QKV product) moves the
    # normalised, rotated q/k by up to ~one spacing of the row's largest entry
    c.close("q", g["q"], r["q"], atol=2 ** -5)
    c.close("k", g["k"], r["k"], atol=2 ** -5)
    c.close("v", g["v"], r["v"], atol=v_atol)
    nQ = n_tiles - n_prefix_tiles
    if nQ > 0:
        for name in ("qbar", "kbar", "vbar"):
            c.true(name, np.max(np.abs(g[name] - r[name])) < 2 ** -8,
                   f"{np.max(np.abs(g[name] - r[name])):.3g}")
        c.true("scores", np.max(np.abs(g["scores"] - r["scores"])) < 1e-3,
               f"{np.max(np.abs(g['scores'] - r['scores'])):.3g}")
        checked, bad, skipped = selection_agrees(g["sel"], r["sel"], r["scores"],
                                                 n_prefix_tiles, top_k)
        c.true("sel", bad == 0 and (not strict_sel or checked >= 0.9 * (checked + skipped)),
               f"checked {checked} bad {bad} skipped {skipped}")
        own = selection_follows_scores(g["sel"], g["scores"], n_prefix_tiles, top_k)
        c.true("sel = rule top-k of own scores", own == 0, f"{own} rows differ")
        c.true("sel order", bool(np.all(np.diff(g["sel"], axis=-1) > 0)))
        c.true("sel range", bool(np.all((g["sel"] >= n_prefix_tiles) & (g["sel"] < n_tiles))))
        if pooled:
            c.true("pooled", np.max(np.abs(g["pooled"] - r["pooled"])) < 1e-3,
                   f"{np.max(np.abs(g['pooled'] - r['pooled'])):.3g}")
    m = metrics(g["attn"], r["attn"])
    c.true("attn metrics", m["cos"] > 0.99999 and m["rel"] < 4e-3, str(m))
    c.true("attn elementwise",
           bool(np.all(np.abs(g["attn"] - r["attn"]) <= 4e-3 + 2 ** -7 * np.abs(r["attn"]))))
    for name in ("x1", "n2", "h", "x2"):
        c.close(name, g[name], r[name], ulps=2, atol=2 ** -6,
                frac_1ulp=h_frac if name == "h" else 2e-2)
    m = metrics(g["x2"], r["x2"])
    c.true("x2 metrics", m["cos"] > 0.9999 and m["rel"] < 1e-3, str(m))


def fp32_oracle_checks(c, g, r32, names, n_prefix_tiles=None, top_k=None, rows=None):
    """Against the plain C++ oracle (fp32, ascending sums): whole-tensor bars.
    Its sequential fp32 sums carry a relative error of order sqrt(K) 2^-24 per
    sum (K up to 20,480 terms here), which moves the bf16 rounding of a small
    fraction of its outputs -- more than the float64 oracle's exact sums do --
    so the elementwise bars are taken against the float64 oracle and these
    against the fp32 one: cos >= 0.9999 and relative L2 <= 2e-3 for the
    activations (5e-3 for the MLP hidden, 1e-2 for the attention output, whose
    weights also round against a different running max), and the margin rule
    for the selection."""
    for name in names:
        got = g[name] if rows is None or name not in ("attn", "x1", "n2", "h", "x2", "out") \
            else g[name][rows]
        m = metrics(got, r32[name])
        # (the SwiGLU hidden rounds three times: its gate and up products, then
        # silu(g) u, where a flip of g or u moves h by up to two spacings)
        bar = 1e-2 if name in ("attn", "out") else 5e-3 if name == "h" else 2e-3
        c.true(f"{name} vs fp32 oracle", m["cos"] > 0.9999 and m["rel"] < bar, str(m))
    if top_k is not None and "sel" in r32:
        checked, bad, skipped = selection_agrees(g["sel"], r32["sel"], r32["scores"],
                                                 n_prefix_tiles, top_k)
        c.true("sel vs fp32 oracle", bad == 0, f"checked {checked} bad {bad} skipped {skipped}")
