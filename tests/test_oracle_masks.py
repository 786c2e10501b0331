"""Pins of the oracle's masks and descriptors against facts fixed outside it.

Each pin is something the oracle cannot satisfy by construction: closed-form
visible counts derived from the workload definitions, interval formulas
written independently here, a worked example derived by hand
(tests/golden/shared_prompt_tiny.txt), hand-derived ragged tile codes, the
causal tile census, the unsigned-compare identity and the FlashMask
two-masked-interval limit (CompileMask paper summary, section 2.1 "Background"
and section 4.2 "Single-Operator Performance").
"""
import os

import numpy as np
import pytest

from oracle import descriptor as od
from oracle import masks as om
from workloads import WORKLOADS, make_metadata, metadata_from_segments

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers

def merge(intervals):
    """Sort and merge half-open intervals (test's own, independent code)."""
    iv = sorted((s, e) for s, e in intervals if e > s)
    out = []
    for s, e in iv:
        if out and s <= out[-1][1]:
            out[-1] = (out[-1][0], max(out[-1][1], e))
        else:
            out.append((s, e))
    return out


def formula_row(mask, md, b, i):
    """Row i's visible intervals straight from its workload's definition."""
    if mask == "causal":
        return merge([(0, i + 1)])
    if mask == "hstu":
        h = md.scalar("h", b)
        return merge([(0, i + 1)]) if i < h else merge([(0, h), (i, i + 1)])
    segs = md.segments(b)
    if mask == "shared_prompt":
        P = md.scalar("P", b)
        if i < P:
            return merge([(0, i + 1)])
        iv = [(0, P)]
        for (s, e) in segs:
            if s <= i < e:
                iv.append((s, i + 1))
        return merge(iv)
    if mask == "retrieval":
        g = md.scalar("g", b)
        if i < g:
            return merge([(0, i + 1)])
        iv = [(0, g)]
        for m, (s, e) in enumerate(segs):
            if s <= i < e:
                iv.append((s, i + 1))
                for r in range(md.n_refs):
                    t = int(md.refs[b, m, r])
                    if t >= 0:
                        iv.append(segs[t])
        return merge(iv)
    raise KeyError(mask)


def formula_rows(mask, md, b):
    return [formula_row(mask, md, b, i) for i in range(md.N)]


def closed_form_count(mask, md, b):
    """Total visible pairs of sample b, from the closed forms."""
    N = md.N
    if mask == "causal":
        return N * (N + 1) // 2
    if mask == "hstu":
        h = md.scalar("h", b)
        return h * (h + 1) // 2 + (N - h) * (h + 1)
    segs = md.segments(b)
    if mask == "shared_prompt":
        P = md.scalar("P", b)
        return P * (P + 1) // 2 + sum(P * (e - s) + (e - s) * (e - s + 1) // 2 for s, e in segs)
    if mask == "retrieval":
        g = md.scalar("g", b)
        tot = g * (g + 1) // 2
        for m, (s, e) in enumerate(segs):
            L = e - s
            refl = sum(segs[t][1] - segs[t][0] for t in md.refs[b, m] if t >= 0)
            tot += L * g + L * (L + 1) // 2 + L * refl
        return tot
    raise KeyError(mask)


def small_md(mask, N=512, seed=0, B=2):
    """Small random metadata of each family (same shapes as the workloads)."""
    rng = np.random.default_rng(seed)
    if mask == "causal":
        return metadata_from_segments(N, 0, 0, (), [{}] * B)
    if mask == "hstu":
        return metadata_from_segments(N, 0, 0, ("h",), [{"scalars": [int(rng.integers(1, N))]} for _ in range(B)])
    if mask == "shared_prompt":
        out = []
        for _ in range(B):
            P = int(rng.integers(1, N // 2))
            R = int(rng.integers(1, 6))
            cuts = sorted(rng.choice(np.arange(P + 1, N), size=R - 1, replace=False).tolist())
            out.append({"scalars": [P], "bounds": [P] + cuts + [N]})
        return metadata_from_segments(N, 8, 0, ("P",), out)
    if mask == "retrieval":
        out = []
        for _ in range(B):
            g = int(rng.integers(1, 40))
            S = int(rng.integers(3, 10))
            cuts = sorted(rng.choice(np.arange(g + 1, N), size=S - 1, replace=False).tolist())
            refs = []
            for j in range(S):
                if j == 0:
                    refs.append([])
                elif j == 1:
                    refs.append([0])
                else:
                    refs.append(sorted(rng.choice(j, 2, replace=False).tolist()))
            out.append({"scalars": [g], "bounds": [g] + cuts + [N], "refs": refs})
        return metadata_from_segments(N, 12, 2, ("g",), out)
    raise KeyError(mask)


FAMILIES = ["causal", "hstu", "shared_prompt", "retrieval"]


# ---------------------------------------------------------------- pins

@pytest.mark.parametrize("mask", FAMILIES)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_runs_equal_formula_intervals(mask, seed):
    md = small_md(mask, N=384, seed=seed)
    for b in range(md.B):
        t = od.sample_tables(mask, md, b, (64, 64, 64, 64))
        want = formula_rows(mask, md, b)
        assert t["row_runs"] == want
        M = om.dense_mask(mask, md, b)
        # per-row and total counts against the closed form
        assert M.sum() == closed_form_count(mask, md, b)
        assert [sum(e - s for s, e in r) for r in want] == M.sum(axis=1).tolist()
        # column runs are the row runs of the transposed mask
        assert t["col_runs"] == od.runs_of_rows(M.T)


def test_workload_closed_forms_full_size_counts():
    """Closed-form visible counts of the real workloads (no mask needed) and
    the per-row count of the mask on a sample of rows."""
    for name in ["causal_8k", "hstu_4k", "reward_model_32k", "retrieval4_32k"]:
        w = WORKLOADS[name]
        md = make_metadata(w)
        rng = np.random.default_rng(5)
        for b in range(md.B):
            V = closed_form_count(w.mask, md, b)
            rows = rng.choice(w.N, 64, replace=False)
            M = om.visible(w.mask, md, b, rows, np.arange(w.N))
            want = [formula_row(w.mask, md, b, int(i)) for i in rows]
            assert M.sum(axis=1).tolist() == [sum(e - s for s, e in r) for r in want]
            assert od.runs_of_rows(M) == want
            assert V > 0
    md = make_metadata(WORKLOADS["causal_8k"])
    assert 2 * 16 * closed_form_count("causal", md, 0) == 1_073_872_896


def test_worked_example_shared_prompt_tiny():
    gold = {}
    with open(os.path.join(GOLDEN, "shared_prompt_tiny.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, v = line.split(":", 1)
            gold[k.strip()] = v.strip()
    w = WORKLOADS["shared_prompt_tiny"]
    md = make_metadata(w)
    K_r, K_c = int(gold["K_r"]), int(gold["K_c"])
    words = od.build(w.mask, md, K_r, K_c, w.tiles)
    v = od.View(words, md.B, md.N, K_r, K_c, w.tiles)
    assert om.dense_mask(w.mask, md, 0).sum() == int(gold["visible_pairs"])
    codes = [[int(x) for x in r.split()] for r in gold["fbm_codes"].split("|")]
    assert v.codes("fbm", 0).tolist() == codes
    assert v["fbm"][0, :, 0].tolist() == [int(x) for x in gold["fbm_words"].split()]
    assert v["bbm"][0, :, 0].tolist() == [int(x) for x in gold["bbm_words"].split()]
    assert v["row_tkmax"][0].tolist() == [int(x) for x in gold["row_tkmax"].split()]
    assert v["col_tkmax"][0].tolist() == [int(x) for x in gold["col_tkmax"].split()]
    assert v["header"].tolist() == [int(x) for x in gold["header"].split()]
    for key, val in gold.items():
        if key.startswith("row ") or key.startswith("col "):
            kind, idx = key.split()
            want = [int(x) for x in val.split()]
            table = v["row_iv" if kind == "row" else "col_iv"][0, int(idx)].ravel().tolist()
            width = K_r if kind == "row" else K_c
            assert table == want + [0] * (2 * width - len(want)), key
    # census: 9 empty, 3 full, 4 partial
    c = np.array(codes)
    assert [(c == 0).sum(), (c == 1).sum(), (c == 2).sum()] == [9, 3, 4]


@pytest.mark.parametrize("T,t", [(4, 64), (6, 32), (5, 48)])
def test_causal_tile_census(T, t):
    N = T * t
    md = small_md("causal", N=N, B=1)
    words = od.build("causal", md, 1, 1, (t, t, t, t))
    v = od.View(words, 1, N, 1, 1, (t, t, t, t))
    c = v.codes("fbm", 0)
    assert (c == 2).sum() == T
    assert (c == 1).sum() == T * (T - 1) // 2
    assert (c == 0).sum() == T * (T - 1) // 2
    # backward grid of the same shape is the transpose
    assert np.array_equal(v.codes("bbm", 0), c.T)


def test_ragged_tiles_hand_derived():
    # causal, N = 100, forward tiles 48 x 40, backward tiles 40 (keys) x 48 (queries)
    md = small_md("causal", N=100, B=1)
    tiles = (48, 40, 40, 48)
    v = od.View(od.build("causal", md, 1, 1, tiles), 1, 100, 1, 1, tiles)
    assert v.codes("fbm", 0).tolist() == [[2, 2, 0], [1, 2, 2], [1, 1, 2]]
    assert v.codes("bbm", 0).tolist() == [[2, 1, 1], [2, 2, 1], [0, 2, 2]]
    # an all-visible mask: every ragged tile is full
    vf = od.View(od.build("full", md, 1, 1, tiles), 1, 100, 1, 1, tiles)
    assert (vf.codes("fbm", 0) == 1).all() and (vf.codes("bbm", 0) == 1).all()
    assert vf["row_iv"][0, :, 0].tolist() == [[0, 100]] * 100
    # nothing visible: all empty, zero-length padding everywhere
    vn = od.View(od.build("none", md, 2, 2, tiles), 1, 100, 2, 2, tiles)
    assert (vn.codes("fbm", 0) == 0).all() and not vn["row_iv"].any() and not vn["col_iv"].any()
    assert not vn["row_tkmax"].any()


def test_unsigned_check_identity():
    """(s <= j < e)  <=>  uint32(j - s) < uint32(e - s), exhaustively; a
    zero-length (0, 0) slot never matches (section 4.4 "Efficiency of
    Visibility Checks"; section 3.3.1 for zero-length padding)."""
    s = np.arange(65)[:, None, None]
    e = np.arange(65)[None, :, None]
    j = np.arange(64)[None, None, :]
    valid = np.broadcast_to(s <= e, (65, 65, 64))
    direct = (s <= j) & (j < e)
    uns = ((j - s).astype(np.uint32)) < ((e - s).astype(np.uint32))
    assert np.array_equal(direct[valid], uns[valid])
    assert not (((j - 0).astype(np.uint32)) < np.uint32(0)).any()


def masked_runs_per_column(M):
    return np.array([len(r) for r in od.runs_of_rows(~M.T)])


def test_flashmask_two_interval_limit():
    """FlashMask's column form holds at most two masked intervals per column;
    the retrieval mask needs more (sections 2.1 and 4.2)."""
    for mask in ["causal", "hstu", "shared_prompt"]:
        md = small_md(mask, N=256, seed=3)
        for b in range(md.B):
            assert masked_runs_per_column(om.dense_mask(mask, md, b)).max() <= 2
    md = make_metadata(WORKLOADS["shared_prompt_tiny"])
    assert masked_runs_per_column(om.dense_mask("shared_prompt", md, 0)).max() <= 2
    # hand-built retrieval case: prefix g = 4, eight segments of 8 rows;
    # segments 2, 4, 6 reference segment 0, segments 1, 3, 5, 7 do not
    bounds = [4 + 8 * s for s in range(9)]
    refs = [[], [], [0], [1], [0, 1], [2], [0, 3], [5]]
    md = metadata_from_segments(68, 8, 2, ("g",), [{"scalars": [4], "bounds": bounds, "refs": refs}])
    M = om.dense_mask("retrieval", md, 0)
    col = od.runs_of_rows(M.T)[4]          # first key of segment 0
    assert col == [(4, 12), (20, 28), (36, 44), (52, 60)]
    assert masked_runs_per_column(M)[4] >= 3
    # a row of segment 7 (refs {5}) merges to three runs
    row = od.runs_of_rows(M[60:61])[0]
    assert row == [(0, 4), (44, 52), (60, 61)]
    # largest run count per 16-wide tile, counted by hand from the segment
    # table above (columns: own segment tail plus every referencing segment;
    # rows: prefix, own segment head and referenced segments, merged)
    tiles = (16, 16, 16, 16)
    v = od.View(od.build("retrieval", md, 4, 4, tiles), 1, 68, 4, 4, tiles)
    assert v["col_tkmax"][0].tolist() == [4, 2, 2, 2, 1]
    assert v["row_tkmax"][0].tolist() == [2, 3, 3, 3, 3]


def test_metadata_validation_bits_and_empty_sample():
    good = {"scalars": [10], "bounds": [10, 20, 40], "refs": [[-1, -1], [0, -1]]}
    md = metadata_from_segments(40, 4, 2, ("g",), [good, good, good, good, good])
    md.n_seg[1] = 5                      # above seg_cap
    md.seg_bounds[2, 1] = 5              # decreasing
    md.seg_bounds[3, 2] = 41             # past N
    md.refs[4, 1, 0] = 2                 # references a missing segment
    assert [om.validate(md, b) for b in range(5)] == [0, om.ERR_NSEG, om.ERR_BOUNDS_ORDER,
                                                       om.ERR_BOUNDS_RANGE, om.ERR_REF_RANGE]
    tiles = (16, 16, 16, 16)
    v = od.View(od.build("retrieval", md, 3, 3, tiles), 5, 40, 3, 3, tiles)
    assert v["header"][13] == 15
    assert v["sample_err"].tolist() == [0, 1, 2, 4, 8]
    for b in range(1, 5):
        assert not v["row_iv"][b].any() and not v["fbm"][b].any() and not v["bbm"][b].any()
    assert v["row_iv"][0].any()


def test_layout_sections_aligned_and_disjoint():
    off, total, dims = od.layout(3, 1000, 4, 7, (128, 64, 128, 64))
    names = ["header", "sample_err", "row_tkmax", "col_tkmax", "fbm", "bbm", "row_iv", "col_iv"]
    assert all(off[n] % 256 == 0 for n in names)
    assert [off[n] for n in names] == sorted(off[n] for n in names)
    assert dims == dict(Tq_f=8, Tk_f=16, Tk_b=8, Tq_b=16, Wf=1, Wb=1)
    assert total % 256 == 0 and total >= off["col_iv"] + 3 * 1000 * 7 * 8
