"""Oracle: the Execution Descriptor read off the dense mask (test infrastructure only).

What the descriptor holds (CompileMask paper summary, section 3.3.1 "Execution
Descriptor"): an Interval Table of visible-key intervals per query row, padded
with zero-length intervals up to the per-mask maximum, and Tile-State Bitmaps of
two bits per tile telling empty, full and partial tiles apart.  The backward
pass gets its own table, one per key column over query rows, so that each
direction's intervals follow its traversal (section 3.3 "Online Efficient Mask
Attention Execution").

Readings where the pages are silent (each is frozen here and in the library):
  * a row's intervals are its maximal runs of visible keys, ascending, as
    half-open [start, end) uint32 pairs; unused slots are (0, 0) at the tail;
  * tile codes: 0 = empty, 1 = full, 2 = partial (3 is never written);
    16 tiles per uint32, tile c at bits 2*(c % 16) of word c // 16; unused
    high bits are 0;
  * a tile's state counts only in-range elements (edge tiles are ragged);
  * ``*_tkmax``: per tile row, the largest run count among its rows/columns;
  * descriptors are per sample and shared by all heads;
  * a sample with invalid metadata gets no visible pairs at all.

Byte layout (all uint32, each section starting at a multiple of 256 bytes,
gaps zero):
  header[16]   magic 0x31444D43, B, N, K_r, K_c, fwd_q, fwd_k, bwd_k, bwd_q,
               Tq_f, Tk_f, Tk_b, Tq_b, err_or, seg_cap, n_samples (packed
               batches; 0 otherwise)
  sample_err[B]                 (packed batch: [n_samples])
  row_tkmax[B][Tq_f]
  col_tkmax[B][Tk_b]
  fbm[B][Tq_f][ceil(Tk_f/16)]   forward grid: query tiles x key tiles
  bbm[B][Tk_b][ceil(Tq_b/16)]   backward grid: key tiles x query tiles
  row_iv[B][N][K_r][2]
  col_iv[B][N][K_c][2]
"""
from __future__ import annotations

import math

import numpy as np

from . import masks as _masks

MAGIC = 0x31444D43
EMPTY, FULL, PARTIAL = 0, 1, 2


def _align(x: int, a: int = 256) -> int:
    return (x + a - 1) // a * a


def layout(B: int, N: int, K_r: int, K_c: int, tiles, n_err: int = None):
    """Byte offsets of each section and the total size (n_err sample-error
    words: B, or the sample count of a packed batch)."""
    fq, fk, bk, bq = tiles
    Tq_f, Tk_f = math.ceil(N / fq), math.ceil(N / fk)
    Tk_b, Tq_b = math.ceil(N / bk), math.ceil(N / bq)
    Wf, Wb = math.ceil(Tk_f / 16), math.ceil(Tq_b / 16)
    sizes = [
        ("header", 16 * 4),
        ("sample_err", (B if n_err is None else n_err) * 4),
        ("row_tkmax", B * Tq_f * 4),
        ("col_tkmax", B * Tk_b * 4),
        ("fbm", B * Tq_f * Wf * 4),
        ("bbm", B * Tk_b * Wb * 4),
        ("row_iv", B * N * K_r * 8),
        ("col_iv", B * N * K_c * 8),
    ]
    off, pos = {}, 0
    for name, sz in sizes:
        off[name] = pos
        pos = _align(pos + sz)
    dims = dict(Tq_f=Tq_f, Tk_f=Tk_f, Tk_b=Tk_b, Tq_b=Tq_b, Wf=Wf, Wb=Wb)
    return off, pos, dims


def runs_of_rows(M: np.ndarray):
    """Maximal runs of True along each row: list (per row) of (start, end)."""
    R, C = M.shape
    pad = np.zeros((R, C + 2), np.int8)
    pad[:, 1:-1] = M
    d = np.diff(pad, axis=1)
    sr, sc = np.nonzero(d == 1)
    er, ec = np.nonzero(d == -1)
    out = [[] for _ in range(R)]
    for r, s, e in zip(sr.tolist(), sc.tolist(), ec.tolist()):
        out[r].append((s, e))
    # nonzero is row-major, so per-row starts and ends are both ascending and
    # pair up in order
    assert np.array_equal(sr, er)
    return out


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """codes[R][T] in {0,1,2} -> uint32 words[R][ceil(T/16)]."""
    R, T = codes.shape
    W = math.ceil(T / 16)
    words = np.zeros((R, W), np.uint64)
    for c in range(T):
        words[:, c // 16] |= codes[:, c].astype(np.uint64) << np.uint64(2 * (c % 16))
    return words.astype(np.uint32)


def tile_codes(counts: np.ndarray, row_sizes: np.ndarray, col_sizes: np.ndarray) -> np.ndarray:
    """Tile state from visible counts: none -> empty, all -> full, else partial."""
    area = row_sizes[:, None] * col_sizes[None, :]
    codes = np.full(counts.shape, PARTIAL, np.uint32)
    codes[counts == 0] = EMPTY
    codes[counts == area] = FULL
    return codes


def _tile_starts(N: int, t: int) -> np.ndarray:
    return np.arange(0, N, t)


def _tile_sizes(N: int, t: int) -> np.ndarray:
    st = _tile_starts(N, t)
    return np.minimum(st + t, N) - st


def sample_tables(mask: str, md, b: int, tiles, block_rows: int = 1024):
    """Everything the descriptor holds for sample b, from the dense mask.

    Returns dict with row_runs, col_runs (lists of (start, end)), fwd_counts
    [Tq_f][Tk_f], bwd_counts [Tk_b][Tq_b] (visible counts per tile).
    """
    N = md.N
    fq, fk, bk, bq = tiles
    # row blocks aligned to both query-tile sizes
    step = fq * bq // math.gcd(fq, bq)
    block = max(step, (block_rows // step) * step)
    cols = np.arange(N)
    row_runs = []
    col_starts = [[] for _ in range(N)]
    col_ends = [[] for _ in range(N)]
    fk_st = _tile_starts(N, fk)
    bk_st = _tile_starts(N, bk)
    fwd_counts = np.zeros((math.ceil(N / fq), len(fk_st)), np.int64)
    bwd_counts = np.zeros((len(bk_st), math.ceil(N / bq)), np.int64)
    prev = np.zeros(N, bool)
    for r0 in range(0, N, block):
        r1 = min(N, r0 + block)
        if _masks.is_packed(md):
            M = _masks.packed_visible(mask, md, np.arange(r0, r1), cols)
        else:
            M = _masks.visible(mask, md, b, np.arange(r0, r1), cols)
        row_runs.extend(runs_of_rows(M))
        # column runs: a run starts where a column turns visible going down
        # the rows and ends where it turns invisible
        stacked = np.vstack([prev[None, :], M])
        dm = np.diff(stacked.astype(np.int8), axis=0)
        si, sj = np.nonzero(dm == 1)
        ei, ej = np.nonzero(dm == -1)
        for i_, j_ in zip((si + r0).tolist(), sj.tolist()):
            col_starts[j_].append(i_)
        for i_, j_ in zip((ei + r0).tolist(), ej.tolist()):
            col_ends[j_].append(i_)
        prev = M[-1].copy()
        # visible counts per tile of each grid
        Mi = M.astype(np.int64)
        per_fk = np.add.reduceat(Mi, fk_st, axis=1)           # rows x Tk_f
        rs = np.arange(0, r1 - r0, fq)
        fwd_counts[r0 // fq: r0 // fq + len(rs)] += np.add.reduceat(per_fk, rs, axis=0)
        per_bk = np.add.reduceat(Mi, bk_st, axis=1)           # rows x Tk_b
        rs = np.arange(0, r1 - r0, bq)
        bwd_counts[:, r0 // bq: r0 // bq + len(rs)] += np.add.reduceat(per_bk, rs, axis=0).T
    # close runs still open at the last row
    for j_ in np.nonzero(prev)[0].tolist():
        col_ends[j_].append(N)
    col_runs = []
    for j_ in range(N):
        s, e = sorted(col_starts[j_]), sorted(col_ends[j_])
        assert len(s) == len(e)
        col_runs.append(list(zip(s, e)))
    return dict(row_runs=row_runs, col_runs=col_runs, fwd_counts=fwd_counts, bwd_counts=bwd_counts)


def build(mask: str, md, K_r: int, K_c: int, tiles, block_rows: int = 1024) -> np.ndarray:
    """The whole descriptor as a uint32 array (bytes / 4 words).  A packed
    batch (md.cu_seqlens set) gives the descriptor of its one sequence:
    B = 1, N = the total length, header word 15 = the sample count and one
    error word per sample."""
    packed = _masks.is_packed(md)
    n_samples = len(md.cu_seqlens) - 1 if packed else 0
    B, N = (1, md.N) if packed else (md.B, md.N)
    off, total, dims = layout(B, N, K_r, K_c, tiles, n_samples if packed else None)
    fq, fk, bk, bq = tiles
    words = np.zeros(total // 4, np.uint32)

    def put(section, index_words, values):
        base = off[section] // 4 + index_words
        vals = np.asarray(values, np.uint32).ravel()
        words[base: base + len(vals)] = vals

    errs = _masks.packed_errors(md) if packed else [_masks.validate(md, b) for b in range(B)]
    err_or = 0
    for e in errs:
        err_or |= e
    put("header", 0, [MAGIC, B, N, K_r, K_c, fq, fk, bk, bq,
                      dims["Tq_f"], dims["Tk_f"], dims["Tk_b"], dims["Tq_b"], err_or, md.seg_cap, n_samples])
    put("sample_err", 0, errs)
    Tq_f, Tk_f, Tk_b, Tq_b, Wf, Wb = (dims[k] for k in ("Tq_f", "Tk_f", "Tk_b", "Tq_b", "Wf", "Wb"))
    for b in range(B):
        t = sample_tables(mask, md, b, tiles, block_rows)
        # interval tables
        row_iv = np.zeros((N, K_r, 2), np.uint32)
        for i, runs in enumerate(t["row_runs"]):
            if len(runs) > K_r:
                raise ValueError(f"row {i} has {len(runs)} runs > K_r={K_r}")
            if runs:
                row_iv[i, : len(runs)] = runs
        col_iv = np.zeros((N, K_c, 2), np.uint32)
        for j, runs in enumerate(t["col_runs"]):
            if len(runs) > K_c:
                raise ValueError(f"column {j} has {len(runs)} runs > K_c={K_c}")
            if runs:
                col_iv[j, : len(runs)] = runs
        put("row_iv", b * N * K_r * 2, row_iv)
        put("col_iv", b * N * K_c * 2, col_iv)
        # tile states
        fcodes = tile_codes(t["fwd_counts"], _tile_sizes(N, fq), _tile_sizes(N, fk))
        bcodes = tile_codes(t["bwd_counts"], _tile_sizes(N, bk), _tile_sizes(N, bq))
        put("fbm", b * Tq_f * Wf, pack_codes(fcodes))
        put("bbm", b * Tk_b * Wb, pack_codes(bcodes))
        # largest run count per tile row / tile column
        rcount = np.array([len(r) for r in t["row_runs"]], np.int64)
        ccount = np.array([len(c) for c in t["col_runs"]], np.int64)
        put("row_tkmax", b * Tq_f, [rcount[r * fq: (r + 1) * fq].max() for r in range(Tq_f)])
        put("col_tkmax", b * Tk_b, [ccount[c * bk: (c + 1) * bk].max() for c in range(Tk_b)])
    return words


class View:
    """Named, shaped views into a descriptor word array (either side's)."""

    def __init__(self, words: np.ndarray, B: int, N: int, K_r: int, K_c: int, tiles, n_err: int = None):
        self.words = np.asarray(words, np.uint32)
        self.off, self.total, self.dims = layout(B, N, K_r, K_c, tiles, n_err)
        d = self.dims
        self.B, self.N, self.K_r, self.K_c = B, N, K_r, K_c
        self.shapes = {
            "header": (16,),
            "sample_err": (B if n_err is None else n_err,),
            "row_tkmax": (B, d["Tq_f"]),
            "col_tkmax": (B, d["Tk_b"]),
            "fbm": (B, d["Tq_f"], d["Wf"]),
            "bbm": (B, d["Tk_b"], d["Wb"]),
            "row_iv": (B, N, K_r, 2),
            "col_iv": (B, N, K_c, 2),
        }

    def __getitem__(self, name):
        shp = self.shapes[name]
        n = int(np.prod(shp))
        base = self.off[name] // 4
        return self.words[base: base + n].reshape(shp)

    def codes(self, name: str, b: int) -> np.ndarray:
        """Unpacked tile codes of bitmap ``fbm`` or ``bbm`` for sample b."""
        d = self.dims
        T = d["Tk_f"] if name == "fbm" else d["Tq_b"]
        w = self[name][b].astype(np.uint64)
        c = np.arange(T)
        return ((w[:, c // 16] >> (2 * (c % 16)).astype(np.uint64)) & np.uint64(3)).astype(np.uint32)
