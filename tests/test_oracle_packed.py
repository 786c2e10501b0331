"""Pins of the oracle's packed variable-length batches (CPU only).

A packed batch lays its samples end to end as one sequence; a token sees only
keys of its own sample, under the sample's rule evaluated in the sample's own
coordinates.  Pinned by a hand-worked example (tests/golden), by the closed
form visible counts of each sample, by block-diagonality, and by the error
word of an invalid cu_seqlens.
"""
import os

import numpy as np
import pytest

from oracle import descriptor as od
from oracle import masks as om
from tests.test_oracle_masks import FAMILIES, closed_form_count, small_md
from workloads import metadata_from_segments, pack_samples

GOLD = os.path.join(os.path.dirname(__file__), "golden", "packed_causal_tiny.txt")


def read_golden(path):
    out = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        out[key] = vals
    return out


def empty_sample(mask, like):
    """A zero-length sample with the metadata shapes of `like`."""
    m = metadata_from_segments(0, like.seg_cap, like.n_refs, like.scalar_names, [{}])
    return m


def packed_md(mask, lengths, seed=0):
    """Packed metadata of one small random sample per length (0 = empty; an
    HSTU sample of one token is all history)."""
    proto = small_md(mask, N=max(64, max(lengths)), seed=seed, B=1)
    samples = []
    for k, n in enumerate(lengths):
        if n == 0:
            samples.append(empty_sample(mask, proto))
        elif mask == "hstu" and n < 2:
            samples.append(metadata_from_segments(n, proto.seg_cap, proto.n_refs, proto.scalar_names,
                                                  [{"scalars": [n]}]))
        else:
            samples.append(small_md(mask, N=n, seed=seed + 7 * k + 1, B=1))
    return pack_samples(samples)


def test_worked_example_causal():
    g = read_golden(GOLD)
    cu = np.array([int(x) for x in g["cu_seqlens"]], np.int32)
    samples = [metadata_from_segments(int(n), 0, 0, (), [{}]) for n in np.diff(cu)]
    md = pack_samples(samples)
    assert list(md.cu_seqlens) == list(cu)
    tiles = tuple(int(x) for x in g["tiles"])
    words = od.build("causal", md, 1, 1, tiles)
    v = od.View(words, 1, md.N, 1, 1, tiles, n_err=md.B)
    pairs = lambda key: [tuple(int(y) for y in x.split(",")) for x in g[key]]  # noqa: E731
    assert [tuple(r[0]) for r in v["row_iv"][0].tolist()] == pairs("row_runs")
    assert [tuple(r[0]) for r in v["col_iv"][0].tolist()] == pairs("col_runs")
    assert v.codes("fbm", 0).tolist() == [list(p) for p in pairs("fwd_codes")]
    assert v.codes("bbm", 0).tolist() == [list(p) for p in pairs("bwd_codes")]
    assert v["row_tkmax"][0].tolist() == [int(x) for x in g["row_tkmax"]]
    assert v["col_tkmax"][0].tolist() == [int(x) for x in g["col_tkmax"]]
    assert v["sample_err"].tolist() == [int(x) for x in g["sample_err"]]
    h = v["header"]
    assert h[1] == 1 and h[2] == md.N and h[15] == int(g["n_samples"][0]) and h[13] == 0


@pytest.mark.parametrize("mask", FAMILIES)
def test_visible_count_is_sum_of_sample_closed_forms(mask):
    lengths = [70, 0, 129, 64, 200, 0, 65] if mask in ("causal", "hstu") else [70, 129, 64, 200, 65]
    md = packed_md(mask, lengths, seed=3)
    M = om.dense_mask(mask, md, 0)
    want = 0
    for b in range(md.B):
        n = int(md.cu_seqlens[b + 1] - md.cu_seqlens[b])
        if n:
            want += closed_form_count(mask, om.sample_md(md, b), 0)
    assert int(M.sum()) == want


@pytest.mark.parametrize("mask", FAMILIES)
def test_no_visible_pair_crosses_samples(mask):
    md = packed_md(mask, [80, 96, 64, 150], seed=5)
    M = om.dense_mask(mask, md, 0)
    owner = np.repeat(np.arange(md.B), np.diff(md.cu_seqlens))
    i, j = np.nonzero(M)
    assert (owner[i] == owner[j]).all()
    # each diagonal block is the sample's own mask
    for b in range(md.B):
        c0, c1 = int(md.cu_seqlens[b]), int(md.cu_seqlens[b + 1])
        assert np.array_equal(M[c0:c1, c0:c1], om.dense_mask(mask, om.sample_md(md, b), 0))


def test_invalid_cu_seqlens_empties_everything():
    md = packed_md("causal", [10, 20, 30])
    md.cu_seqlens = np.array([0, 25, 20, 60], np.int32)  # decreasing
    assert not om.dense_mask("causal", md, 0).any()
    assert om.packed_errors(md) == [om.ERR_CU_SEQLENS] * 3
    words = od.build("causal", md, 1, 1, (16, 16, 16, 16))
    v = od.View(words, 1, md.N, 1, 1, (16, 16, 16, 16), n_err=3)
    assert v["header"][13] == om.ERR_CU_SEQLENS
    assert not v["row_iv"].any() and not v["fbm"].any()


def test_sample_metadata_errors_stay_in_their_sample():
    md = packed_md("shared_prompt", [100, 90, 120], seed=9)
    md.seg_bounds[1, int(md.n_seg[1]):] = 95  # last bound beyond sample 1's own length 90
    errs = om.packed_errors(md)
    assert errs[1] == om.ERR_BOUNDS_RANGE and errs[0] == 0 and errs[2] == 0
    M = om.dense_mask("shared_prompt", md, 0)
    assert not M[100:190].any() and M[:100].any() and M[190:].any()
