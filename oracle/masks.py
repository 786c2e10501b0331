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
ERR_CU_SEQLENS = 16   # packed batch: cu_seqlens does not run 0 <= ... <= N without decreasing

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


# ---------------------------------------------------------------- packed batches
#
# A packed batch lays its samples end to end as one sequence of md.N tokens;
# md.cu_seqlens[b] is the first token of sample b and cu_seqlens[-1] = N.
# Token i of sample b sees key j exactly when j belongs to the same sample and
# the sample's own rule (evaluated in its coordinates, with its length as N)
# lets local row i - c_b see local key j - c_b.


def cu_valid(md) -> bool:
    cu = [int(x) for x in md.cu_seqlens]
    return cu[0] == 0 and cu[-1] == md.N and all(a <= b for a, b in zip(cu, cu[1:]))


def sample_md(md, b: int):
    """Sample b of a packed batch as a one-sample metadata of its own length."""
    cu = md.cu_seqlens
    out = md.copy()
    out.B = 1
    out.N = int(cu[b + 1]) - int(cu[b])
    out.scalars = md.scalars[b: b + 1].copy()
    out.seg_bounds = md.seg_bounds[b: b + 1].copy()
    out.n_seg = md.n_seg[b: b + 1].copy()
    out.refs = md.refs[b: b + 1].copy()
    out.cu_seqlens = None
    return out


def packed_errors(md):
    """Error word of every sample of a packed batch."""
    n = len(md.cu_seqlens) - 1
    if not cu_valid(md):
        return [ERR_CU_SEQLENS] * n
    return [validate(sample_md(md, b), 0) for b in range(n)]


def packed_visible(mask: str, md, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """Dense visibility of a packed batch for global rows x global columns."""
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    out = np.zeros((len(rows), len(cols)), bool)
    if not cu_valid(md):
        return out
    cu = [int(x) for x in md.cu_seqlens]
    for b in range(len(cu) - 1):
        c0, c1 = cu[b], cu[b + 1]
        rsel = np.nonzero((rows >= c0) & (rows < c1))[0]
        csel = np.nonzero((cols >= c0) & (cols < c1))[0]
        if len(rsel) == 0 or len(csel) == 0:
            continue
        sub = visible(mask, sample_md(md, b), 0, rows[rsel] - c0, cols[csel] - c0)
        out[np.ix_(rsel, csel)] = sub
    return out


def is_packed(md) -> bool:
    return getattr(md, "cu_seqlens", None) is not None


def dense_mask(mask: str, md, b: int) -> np.ndarray:
    """Full N x N boolean mask of sample b (small N only)."""
    ar = np.arange(md.N)
    if is_packed(md):
        return packed_visible(mask, md, ar, ar)
    return visible(mask, md, b, ar, ar)


def row_block_fn(mask: str, md):
    """Callback (b, r0, r1) -> bool[r1 - r0, N] for the attention oracle (a
    packed batch is one sequence: b is then 0)."""
    cols = np.arange(md.N)

    def fn(b, r0, r1):
        if is_packed(md):
            return packed_visible(mask, md, np.arange(r0, r1), cols)
        return visible(mask, md, b, np.arange(r0, r1), cols)

    return fn
