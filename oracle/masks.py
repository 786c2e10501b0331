"""Oracle: mask predicates evaluated element by element (test infrastructure only).

Each mask family is written as a plain predicate over a query row i and a key
column j, following the definitions of the synthetic workloads used to
evaluate CompileMask (paper summary, section 4.1 "Experimental Setup"; the
shared-prompt "Region C" rule [0,b) u [s(i),i+1) of section 3.2.2 "Symbolic
Lowering to Visible Intervals"; the HSTU history/target example of section 2.2
"Motivation").  Nothing here derives intervals symbolically: the predicate is
evaluated at every (i, j) of a row block with numpy broadcasting.

Reading used for rows that no rule names (e.g. a row past the prompt that lies
in no response): such a row sees only the part of its rule that does not refer
to a segment (the prompt or the global prefix); a row of a sample whose
metadata is invalid sees nothing.
"""
from __future__ import annotations

import numpy as np

# Metadata error bits (same meaning as the library's documented flag word).
ERR_NSEG = 1          # n_seg outside [0, seg_cap]
ERR_BOUNDS_ORDER = 2  # segment boundaries decrease somewhere
ERR_BOUNDS_RANGE = 4  # a used boundary lies outside [0, N]
ERR_REF_RANGE = 8     # a used reference lies outside [-1, n_seg)

MASKS = ("causal", "shared_prompt", "hstu", "retrieval", "full", "none")


def validate(md, b: int) -> int:
    """Error bits of sample b's metadata (0 = valid)."""
    n = int(md.n_seg[b])
    cap = md.seg_cap
    if n < 0 or n > cap:
        return ERR_NSEG
    err = 0
    if n >= 1:
        sb = [int(x) for x in md.seg_bounds[b, : n + 1]]
        for s in range(n):
            if sb[s + 1] < sb[s]:
                err |= ERR_BOUNDS_ORDER
        for x in sb:
            if x < 0 or x > md.N:
                err |= ERR_BOUNDS_RANGE
        for s in range(n):
            for r in range(md.n_refs):
                x = int(md.refs[b, s, r])
                if x < -1 or x >= n:
                    err |= ERR_REF_RANGE
    return err


def visible(mask: str, md, b: int, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """Dense boolean visibility for query rows ``rows`` x key columns ``cols``.

    Returns bool[len(rows), len(cols)].
    """
    i = np.asarray(rows, np.int64)[:, None]
    j = np.asarray(cols, np.int64)[None, :]
    shape = (i.shape[0], j.shape[1])
    if validate(md, b) != 0:
        return np.zeros(shape, bool)
    if mask == "none":
        return np.zeros(shape, bool)
    if mask == "full":
        return np.ones(shape, bool)
    if mask == "causal":
        # row i sees keys 0..i
        return j <= i
    if mask == "hstu":
        h = md.scalar("h", b)
        history = (i < h) & (j <= i)
        target = (i >= h) & ((j < h) | (j == i))
        return history | target
    if mask == "shared_prompt":
        # prompt rows are causal; every later row sees the prompt, and a row
        # inside response [s, e) also sees its own response up to itself
        P = md.scalar("P", b)
        ii = i[:, 0]
        out = np.zeros(shape, bool)
        sel = ii < P
        out[sel] = j <= i[sel]
        sel = ii >= P
        out[sel] = np.broadcast_to(j < P, (int(sel.sum()), shape[1]))
        for (s, e) in md.segments(b):
            sel = (ii >= P) & (ii >= s) & (ii < e)
            out[sel] |= (j >= s) & (j <= i[sel])
        return out
    if mask == "retrieval":
        # prefix rows are causal; a row of segment m sees the prefix, its own
        # segment up to itself and every segment m references
        g = md.scalar("g", b)
        segs = md.segments(b)
        ii = i[:, 0]
        out = np.zeros(shape, bool)
        sel = ii < g
        out[sel] = j <= i[sel]
        sel = ii >= g
        out[sel] = np.broadcast_to(j < g, (int(sel.sum()), shape[1]))
        for m, (s, e) in enumerate(segs):
            sel = (ii >= g) & (ii >= s) & (ii < e)
            if not sel.any():
                continue
            see = (j >= s) & (j <= i[sel])
            for r in range(md.n_refs):
                t = int(md.refs[b, m, r])
                if t >= 0:
                    ts, te = segs[t]
                    see = see | ((j >= ts) & (j < te))
            out[sel] |= see
        return out
    raise KeyError(mask)


def dense_mask(mask: str, md, b: int) -> np.ndarray:
    """Full N x N boolean mask of sample b (small N only)."""
    ar = np.arange(md.N)
    return visible(mask, md, b, ar, ar)


def row_block_fn(mask: str, md):
    """Callback (b, r0, r1) -> bool[r1 - r0, N] for the attention oracle."""
    cols = np.arange(md.N)

    def fn(b, r0, r1):
        return visible(mask, md, b, np.arange(r0, r1), cols)

    return fn
