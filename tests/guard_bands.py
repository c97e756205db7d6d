"""Guard bands around workspace regions (H3_WS_GUARD): the planner's rule,
restated for the checks.  Each region starts 256-byte aligned and is followed
by the band; the four tables at the workspace's head (tile starts, padded
tile starts, chunk counts, query blocks) are not in h3_workspace_layout, so
their starts are derived here from the tile map."""
import contextlib
import os

import numpy as np

GUARD = 4096
FILL = 0xA5
FIELDS = ("norm", "big", "q", "k", "vt", "qbar", "kbar", "vbar", "scores", "sel", "pooled",
          "attn", "x1", "xa", "xb", "q8", "qscale", "partial")


def a256(x):
    return (x + 255) & ~255


@contextlib.contextmanager
def guard_bands(nbytes):
    old = os.environ.get("H3_WS_GUARD")
    os.environ["H3_WS_GUARD"] = str(nbytes)
    try:
        yield
    finally:
        if old is None:
            del os.environ["H3_WS_GUARD"]
        else:
            os.environ["H3_WS_GUARD"] = old


def region_starts(lay, ts):
    """Starts of every region after the first, in the planner's order."""
    ts = np.asarray(ts, np.int64)
    lens = np.diff(ts)
    n_tiles = len(lens)
    n_chunks = lay.padded_rows // 32
    nqb = int(((lens + 63) // 64).sum())
    t1 = lay.tables + a256((n_tiles + 1) * 4) + GUARD
    t2 = t1 + a256((n_tiles + 1) * 4) + GUARD
    t3 = t2 + a256(n_chunks * 4) + GUARD
    after_tables = t3 + a256(nqb * 16) + GUARD
    reported = sorted(getattr(lay, f) for f in FIELDS if getattr(lay, f) != 0)
    assert reported[0] == after_tables, (reported[0], after_tables)
    return [t1, t2, t3] + reported


def check_bands(ws, starts, total):
    """Every band in front of a region start, the one after the last region
    and one past the workspace's end hold FILL (ws: a device byte tensor)."""
    bands = [(s - GUARD, s) for s in starts] + [(total - GUARD, total), (total, total + GUARD)]
    bad = [(a, b) for a, b in bands if not bool((ws[a:b] == FILL).all())]
    assert not bad, f"{len(bad)} of {len(bands)} guard bands written: first {bad[:3]}"
    return len(bands)


