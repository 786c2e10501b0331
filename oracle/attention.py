"""Oracle: dense masked softmax attention and its analytic backward, float64.

Test infrastructure only.  The definition followed (CompileMask paper summary,
section 3.3.2 "Descriptor-Guided Attention Execution"): scores of invisible
(query, key) pairs are replaced by minus infinity before the softmax; the
result is the ordinary softmax attention over the visible keys.

Readings where the pages are silent:
  * scale = 1 / sqrt(d);
  * lse is the natural-log log-sum-exp of the scaled visible scores;
  * a query row with no visible key has O = 0 and lse = -inf, its dQ row is 0
    and it adds nothing to dK or dV;
  * the backward uses D = rowsum(dO * O).  With the default stored_o=None, O
    is the oracle's own float64 O (the exact gradient: D = rowsum(P * dP)).
    With stored_o="bf16", O is that O rounded to bfloat16: the backward
    entry point receives the forward's output `o`, which the library stores
    in bf16, and computes D from it.  The parity tests compare against this
    form; the exact form is what autograd and finite differences pin.

Inputs are numpy or torch arrays [B, H, N, d] (bf16 values are upcast exactly).
``mask_rows(b, r0, r1)`` returns the boolean visibility of rows r0..r1-1
against every key of sample b.
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x) -> np.ndarray:
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, np.float64)


def round_bf16(x) -> np.ndarray:
    """float64 -> nearest bfloat16 value (ties to even), via float32: keep the
    upper 16 bits of the float32 pattern after adding 0x7FFF plus the lowest
    kept bit (finite inputs)."""
    bits = np.asarray(x, np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def _o_for_d(O, stored_o):
    if stored_o is None:
        return O
    if stored_o == "bf16":
        return round_bf16(O)
    raise ValueError(f"stored_o must be None or 'bf16', not {stored_o!r}")


def _scale(d: int, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def forward_head(q, k, v, mask_rows, b: int, rows=None, scale=None, block: int = 1024):
    """Forward of one (b, h) pair.  q, k, v are float64 [N, d].

    Returns O [len(rows), d] and lse [len(rows)] for the given rows (all rows
    by default).
    """
    N, d = q.shape
    sc = _scale(d, scale)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    O = np.zeros((len(rows), d))
    lse = np.full(len(rows), -np.inf)
    for a in range(0, len(rows), block):
        rr = rows[a: a + block]
        M = _rows_mask(mask_rows, b, rr)
        S = (q[rr] @ k.T) * sc
        S[~M] = -np.inf
        m = S.max(axis=1)
        live = np.isfinite(m)
        P = np.zeros_like(S)
        P[live] = np.exp(S[live] - m[live, None])
        l = P.sum(axis=1)
        O[a: a + len(rr)][live] = (P[live] @ v) / l[live, None]
        lse[a: a + len(rr)][live] = m[live] + np.log(l[live])
    return O, lse


def _rows_mask(mask_rows, b, rr):
    """Mask rows rr (in the given order), one mask_rows call per run of
    consecutive indices."""
    rr = np.asarray(rr)
    if len(rr) and np.all(np.diff(rr) == 1):
        return mask_rows(b, int(rr[0]), int(rr[-1]) + 1)
    cuts = np.nonzero(np.diff(rr) != 1)[0] + 1
    return np.vstack([mask_rows(b, int(g[0]), int(g[-1]) + 1) for g in np.split(rr, cuts)])


def probabilities(q, k, lse, M, scale=None):
    """P = exp(S - lse) on visible pairs, 0 elsewhere and on empty rows."""
    d = q.shape[-1]
    S = (q @ k.T) * _scale(d, scale)
    P = np.zeros_like(S)
    live = np.isfinite(lse)
    Sl = S[live]
    Pl = np.exp(Sl - lse[live, None])
    Pl[~M[live]] = 0.0
    P[live] = Pl
    return P


def backward_head(q, k, v, do, mask_rows, b: int, scale=None, block: int = 1024, stored_o=None):
    """Analytic backward of one (b, h) pair; float64 [N, d] inputs.

    Returns dq, dk, dv (float64 [N, d]) and the forward O, lse it used.
    """
    N, d = q.shape
    sc = _scale(d, scale)
    O, lse = forward_head(q, k, v, mask_rows, b, scale=scale, block=block)
    Dvec = np.sum(do * _o_for_d(O, stored_o), axis=1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, N, block):
        r1 = min(N, r0 + block)
        M = mask_rows(b, r0, r1)
        P = probabilities(q[r0:r1], k, lse[r0:r1], M, scale)
        dv += P.T @ do[r0:r1]
        dP = do[r0:r1] @ v.T
        dS = P * (dP - Dvec[r0:r1, None])
        dq[r0:r1] = (dS @ k) * sc
        dk += (dS.T @ q[r0:r1]) * sc
    return dq, dk, dv, O, lse


def backward_rows(q, k, v, do, mask_rows, b: int, r0: int, r1: int, scale=None):
    """The work of query rows r0..r1-1 of one (b, h) pair: their forward and
    their whole share of the backward.  Rows are independent given their own
    lse and D, so summing dk, dv over a partition of the rows gives
    backward_head's dk, dv.  Returns dq rows, dk and dv contributions, O rows
    and lse rows (float64)."""
    d = q.shape[1]
    sc = _scale(d, scale)
    rows = np.arange(r0, r1)
    O, lse = forward_head(q, k, v, mask_rows, b, rows=rows, scale=scale, block=max(1, r1 - r0))
    M = mask_rows(b, r0, r1)
    P = probabilities(q[r0:r1], k, lse, M, scale)
    Dvec = np.sum(do[r0:r1] * O, axis=1)
    dP = do[r0:r1] @ v.T
    dS = P * (dP - Dvec[:, None])
    return (dS @ k) * sc, (dS.T @ q[r0:r1]) * sc, P.T @ do[r0:r1], O, lse


def forward(q, k, v, mask_rows, scale=None, block: int = 1024):
    """All heads: O [B,H,N,d], lse [B,H,N] (float64)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            O[b, h], lse[b, h] = forward_head(q[b, h], k[b, h], v[b, h], mask_rows, b, scale=scale, block=block)
    return O, lse


def backward(q, k, v, do, mask_rows, scale=None, block: int = 1024, stored_o=None):
    """All heads: dq, dk, dv [B,H,N,d] (float64), plus O and lse."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    O = np.zeros_like(q)
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h], O[b, h], lse[b, h] = backward_head(
                q[b, h], k[b, h], v[b, h], do[b, h], mask_rows, b, scale=scale, block=block, stored_o=stored_o)
    return dq, dk, dv, O, lse


def rows_seeing(mask_rows, b: int, N: int, keys, block: int = 2048) -> np.ndarray:
    """Indices of the query rows of sample b that see at least one of `keys`."""
    keys = np.asarray(keys)
    out = []
    for r0 in range(0, N, block):
        r1 = min(N, r0 + block)
        hit = mask_rows(b, r0, r1)[:, keys].any(axis=1)
        out.append(np.nonzero(hit)[0] + r0)
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def tiles_head(q, k, v, do, mask_rows, b: int, rows, keys, scale=None, block: int = 1024, stored_o=None,
               seeing=None):
    """Exact outputs of one (b, h) pair at some query rows and some keys,
    without the whole forward.

    A key's dk and dv sum over the rows that see it (P is zero elsewhere), so
    only those rows need their lse and D, which need only their own scores.
    ``seeing`` may pass rows_seeing(mask_rows, b, N, keys) when the caller
    already has it (it depends on the mask only, not on the head).  Returns
    O, lse, dq at ``rows`` and dk, dv at ``keys`` (float64), as backward_head
    would give them.
    """
    N, d = q.shape
    sc = _scale(d, scale)
    rows = np.asarray(rows)
    keys = np.asarray(keys)
    if seeing is None:
        seeing = rows_seeing(mask_rows, b, N, keys)
    need = np.union1d(rows, seeing)
    O, lse = forward_head(q, k, v, mask_rows, b, rows=need, scale=scale, block=block)
    Dvec = np.sum(do[need] * _o_for_d(O, stored_o), axis=1)
    pos = np.searchsorted(need, rows)
    M = _rows_mask(mask_rows, b, rows)
    P = probabilities(q[rows], k, lse[pos], M, scale)
    dS = P * (do[rows] @ v.T - Dvec[pos, None])
    dq = (dS @ k) * sc
    dk = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), d))
    for a in range(0, len(need), block):
        rr = need[a: a + block]
        Mk = _rows_mask(mask_rows, b, rr)[:, keys]
        Pk = probabilities(q[rr], k[keys], lse[a: a + len(rr)], Mk, scale)
        dv += Pk.T @ do[rr]
        dSk = Pk * (do[rr] @ v[keys].T - Dvec[a: a + len(rr), None])
        dk += (dSk.T @ q[rr]) * sc
    return dict(O=O[pos], lse=lse[pos], dq=dq, dk=dk, dv=dv)


def sampled_head(q, k, v, do, mask_rows, b: int, rows, keys, scale=None, block: int = 1024, stored_o=None):
    """Full-size spot check of one (b, h) pair.

    Runs the whole forward (every row's lse and O are needed by the backward),
    then returns O, lse, dq at ``rows`` and dk, dv at ``keys``.
    """
    N, d = q.shape
    sc = _scale(d, scale)
    O, lse = forward_head(q, k, v, mask_rows, b, scale=scale, block=block)
    Dvec = np.sum(do * _o_for_d(O, stored_o), axis=1)
    rows = np.asarray(rows)
    keys = np.asarray(keys)
    # dq at the sampled rows
    M = _rows_mask(mask_rows, b, rows)
    P = probabilities(q[rows], k, lse[rows], M, scale)
    dS = P * (do[rows] @ v.T - Dvec[rows, None])
    dq = (dS @ k) * sc
    # dk, dv at the sampled keys: sum over every row block
    dk = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), d))
    for r0 in range(0, N, block):
        r1 = min(N, r0 + block)
        Mk = mask_rows(b, r0, r1)[:, keys]
        Pk = probabilities(q[r0:r1], k[keys], lse[r0:r1], Mk, scale)
        dv += Pk.T @ do[r0:r1]
        dSk = Pk * (do[r0:r1] @ v[keys].T - Dvec[r0:r1, None])
        dk += (dSk.T @ q[r0:r1]) * sc
    return dict(O=O[rows], lse=lse[rows], dq=dq, dk=dk, dv=dv, visible_rows=M.sum(axis=1))
