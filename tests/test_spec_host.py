"""Host-side checks of the C ABI library (no GPU needed).

* the library loads and exports every entry point include/compilemask.h declares;
* MaskSpec lowering: slot counts per Region (the "Region C" rule needs two
  slots, CompileMask paper summary, section 3.2.2), canonicalisation merges
  what is provably adjacent over the whole Region, errors are reported;
* the lowered program, evaluated on the host for one index at a time, gives
  the oracle's runs for every row and column of random small batches;
* argument checks return the documented status without touching the GPU.
"""
import os
import re

import numpy as np
import pytest

import runtime_metadata_attention_amd as cm
from runtime_metadata_attention_amd import specs
from oracle import descriptor as od
from oracle import masks as om
from tests.test_oracle_masks import small_md
from workloads import WORKLOADS, make_metadata, metadata_from_segments

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "compilemask.h")


def test_library_exports_every_declared_symbol():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(cm_\w+)\s*\(", text, re.M))
    assert declared == set(cm.EXPORTS)
    lib = cm.library()
    for name in declared:
        assert hasattr(lib, name), name
    assert "gfx950" in cm.cm_version()


@pytest.mark.parametrize("mask,K", [("causal", (1, 1)), ("shared_prompt", (2, 1)), ("hstu", (2, 1)),
                                    ("retrieval", (4, 1 + 64))])
def test_slot_counts(mask, K):
    s = cm.cm_spec_compile(specs.BY_MASK[mask])
    assert cm.cm_spec_info(s, 64)[:2] == K


def test_region_c_needs_two_slots_and_provable_merge_needs_one():
    s = cm.cm_spec_compile(specs.SHARED_PROMPT)
    dump = cm.cm_spec_dump(s)
    resp = dump.split("region response")[1].split("region")[0]
    assert resp.count("slot") == 2
    # [0,P) u [P,i+1) over rows i >= P is provably one interval
    s2 = cm.cm_spec_compile("param P\nforward\n region r: i >= P => j < P | (j >= P & j <= i)\n"
                            "backward\n region c: true => i >= j\n")
    assert cm.cm_spec_info(s2, 0)[0] == 1
    assert "slot j in [0, i + 1)" in cm.cm_spec_dump(s2)
    # without the guard the two cannot be merged
    s3 = cm.cm_spec_compile("param P\nforward\n region r: true => j < P | (j >= P & j <= i)\n"
                            "backward\n region c: true => i >= j\n")
    assert cm.cm_spec_info(s3, 0)[0] == 2


def test_lowering_forms():
    txt = """param a
    forward
      region r: i < 10 | i >= 20 => !(j < i - 3 | j > i) & j != i - 1
    backward
      region c: true => seg(i) == seg(j) | (i in [j, j] )
    """
    s = cm.cm_spec_compile(txt)
    d = cm.cm_spec_dump(s)
    # guard disjunction -> two regions; j != i-1 splits the window in two
    assert d.count("region r") == 2
    assert cm.cm_spec_info(s, 4)[0] == 2
    N = 40
    for i in range(N):
        runs, err = cm.cm_spec_eval_host(s, 0, N, i, [7], [0], 0, [], 0)
        want = [] if 10 <= i < 20 else [(s_, e_) for (s_, e_) in [(max(0, i - 3), max(0, i - 1)), (i, i + 1)] if e_ > s_]
        assert runs == want, i
    # backward: own segment, or the diagonal
    bounds = [0, 5, 12, 40]
    for j in range(N):
        runs, _ = cm.cm_spec_eval_host(s, 1, N, j, [7], bounds, 3, [], 0)
        sg = max(t for t in range(3) if bounds[t] <= j)
        assert runs == [(bounds[sg], bounds[sg + 1])], j


@pytest.mark.parametrize("bad,msg", [
    ("forward region a: true => j < \nbackward region b: true => i >= j", "incomplete"),
    ("forward region a: true => j * 2 < i\nbackward region b: true => i >= j", "unexpected character"),
    ("forward region a: true => 2 + j + j < i\nbackward region b: true => i >= j", "coefficient"),
    ("forward region a: j < 3 => j <= i\nbackward region b: true => i >= j", "guard"),
    ("forward region a: true => !exists k (j in k)\nbackward region b: true => i >= j", "negated exists"),
    ("forward region a: true => j <= i", "backward"),
    ("forward region a: true => j <= Q\nbackward region b: true => i >= j", "unknown name"),
    ("refs 1\nforward region a: true => j in ref(seg(i), 1)\nbackward region b: true => i >= j", "reference index"),
])
def test_parse_errors(bad, msg):
    with pytest.raises(cm.CompileMaskError) as e:
        cm.cm_spec_compile(bad)
    assert e.value.status == -3 and msg in str(e.value)


def _host_tables(spec, md, b, direction):
    out = []
    sb = md.seg_bounds[b]
    for x in range(md.N):
        runs, err = cm.cm_spec_eval_host(spec, direction, md.N, x, md.scalars[b], sb, int(md.n_seg[b]),
                                         md.refs[b], md.n_refs)
        assert err == 0
        out.append(runs)
    return out


@pytest.mark.parametrize("mask", ["causal", "hstu", "shared_prompt", "retrieval"])
@pytest.mark.parametrize("seed", [0, 1])
def test_lowered_program_matches_oracle_runs(mask, seed):
    spec = cm.cm_spec_compile(specs.BY_MASK[mask])
    md = small_md(mask, N=200, seed=seed)
    for b in range(md.B):
        t = od.sample_tables(mask, md, b, (64, 64, 64, 64))
        assert _host_tables(spec, md, b, 0) == t["row_runs"]
        assert _host_tables(spec, md, b, 1) == t["col_runs"]


def test_lowered_program_matches_oracle_on_tiny_workload_and_c5_rows():
    w = WORKLOADS["shared_prompt_tiny"]
    md = make_metadata(w)
    spec = cm.cm_spec_compile(specs.BY_MASK[w.mask])
    t = od.sample_tables(w.mask, md, 0, w.tiles)
    assert _host_tables(spec, md, 0, 0) == t["row_runs"]
    assert _host_tables(spec, md, 0, 1) == t["col_runs"]
    # full-size retrieval metadata: sampled rows and columns
    w = WORKLOADS["retrieval4_32k"]
    md = make_metadata(w)
    spec = cm.cm_spec_compile(specs.BY_MASK[w.mask])
    rng = np.random.default_rng(0)
    idx = rng.choice(w.N, 48, replace=False)
    M = om.visible(w.mask, md, 0, idx, np.arange(w.N))
    rows = od.runs_of_rows(M)
    Mc = om.visible(w.mask, md, 0, np.arange(w.N), idx).T
    cols = od.runs_of_rows(Mc)
    for a, x in enumerate(idx.tolist()):
        r, _ = cm.cm_spec_eval_host(spec, 0, w.N, x, md.scalars[0], md.seg_bounds[0], int(md.n_seg[0]), md.refs[0], 2)
        c, _ = cm.cm_spec_eval_host(spec, 1, w.N, x, md.scalars[0], md.seg_bounds[0], int(md.n_seg[0]), md.refs[0], 2)
        assert r == rows[a] and c == cols[a], x


def test_metadata_errors_match_oracle_validation():
    good = {"scalars": [10], "bounds": [10, 20, 40], "refs": [[-1, -1], [0, -1]]}
    md = metadata_from_segments(40, 4, 2, ("g",), [good] * 5)
    md.n_seg[1] = 5
    md.seg_bounds[2, 1] = 5
    md.seg_bounds[3, 2] = 41
    md.refs[4, 1, 0] = 2
    spec = cm.cm_spec_compile(specs.RETRIEVAL)
    for b in range(5):
        runs, err = cm.cm_spec_eval_host(spec, 0, 40, 30, md.scalars[b], md.seg_bounds[b], int(md.n_seg[b]),
                                         md.refs[b], 2)
        assert err == om.validate(md, b)
        assert (runs == []) == (err != 0)


def test_desc_size_matches_documented_layout():
    for mask, tiles in [("retrieval", (128, 64, 128, 64)), ("causal", (48, 40, 40, 48)), ("hstu", (64, 64, 64, 64))]:
        spec = cm.cm_spec_compile(specs.BY_MASK[mask])
        for B, N, cap in [(1, 256, 4), (3, 1000, 9), (2, 4097, 64)]:
            K_r, K_c = cm.cm_spec_info(spec, cap)[:2]
            assert cm.cm_desc_size(spec, B, N, cap, tiles) == od.layout(B, N, K_r, K_c, tiles)[1]


def test_argument_checks_without_gpu():
    spec = cm.cm_spec_compile(specs.CAUSAL)
    with pytest.raises(cm.CompileMaskError) as e:
        cm.cm_desc_size(spec, 0, 128, 0, (64, 64, 64, 64))
    assert e.value.status == -2
    with pytest.raises(cm.CompileMaskError) as e:
        cm.cm_desc_size(spec, 1, 128, 0, (0, 64, 64, 64))
    assert e.value.status == -2
    args = cm.cm_attn_args(1, 1, 128, 96, 0, 0, 0, 0.0, 0)
    with pytest.raises(cm.CompileMaskError) as e:
        cm.library()
        st = cm.library().cm_attn_fwd(args, 16, 16, 16, None, 16, 16, None)
        cm._check(st, "cm_attn_fwd")
    assert e.value.status == -5
    args = cm.cm_attn_args(1, 1, 128, 64, 0, 0, 0, 0.0, 0)
    st = cm.library().cm_attn_fwd(args, 16, 16, 16, None, 16, 16, None)
    assert st == -1  # non-causal needs a descriptor
    args = cm.cm_attn_args(1, 1, 128, 64, 0, 0, 0, 0.0, 1, 2)
    st = cm.library().cm_attn_fwd(args, 16, 16, 16, None, 16, 16, None)
    assert st == -2  # no such partial-tile check
    # size limits: at most 2^27 rows per call, one head's rows within 4 GiB
    args = cm.cm_attn_args(1 << 7, 1 << 4, (1 << 16) + 1, 128, 0, 0, 0, 0.0, 1)
    assert cm.library().cm_attn_fwd(args, 16, 16, 16, None, 16, 16, None) == -5
    args = cm.cm_attn_args(1, 1, 1 << 20, 128, 1 << 40, 1 << 40, 4096, 0.0, 1)
    assert cm.library().cm_attn_fwd(args, 16, 16, 16, None, 16, 16, None) == -5
    # just inside both limits: the size checks pass, the missing q is reported
    args = cm.cm_attn_args(1, 1, 1 << 20, 128, 1 << 40, 1 << 40, 2048, 0.0, 1)
    assert cm.library().cm_attn_fwd(args, None, 16, 16, None, 16, 16, None) == -1
    args = cm.cm_attn_args(1 << 7, 1 << 4, 1 << 16, 128, 0, 0, 0, 0.0, 1)
    assert cm.library().cm_attn_fwd(args, None, 16, 16, None, 16, 16, None) == -1
    assert cm.cm_status_str(-4) == "descriptor/spec/argument mismatch"
    # operand precision: only 0 and 1, and the split precision only with the default check
    args = cm.cm_attn_args(1, 1, 128, 64, 0, 0, 0, 0.0, 1, 0, 2)
    assert cm.library().cm_attn_fwd(args, 16, 16, 16, None, 16, 16, None) == -2
    args = cm.cm_attn_args(1, 1, 128, 64, 0, 0, 0, 0.0, 1, cm.CM_CHECK_UNSIGNED, cm.CM_PRECISION_SPLIT)
    assert cm.library().cm_attn_fwd(args, 16, 16, 16, None, 16, 16, None) == -5
    args = cm.cm_attn_args(1, 1, 128, 64, 0, 0, 0, 0.0, 1, cm.CM_CHECK_RUN_BITS, cm.CM_PRECISION_SPLIT)
    assert cm.library().cm_attn_fwd(args, None, 16, 16, None, 16, 16, None) == -1  # checks pass, q missing
    # the fixed-workspace backward: more rows than its array holds is refused
    # before any HIP call
    big = cm.CM_NOALLOC_MAX_ROWS + 1
    args = cm.cm_attn_args(1, 1, big, 128, 0, 0, 0, 0.0, 1)
    assert cm.library().cm_attn_bwd_noalloc(args, 16, 16, 16, 16, 16, 16, None, 16, 16, 16, None) == -6
    assert "rows" in cm.cm_last_error()


def test_specialised_source_embeds_the_program_and_compiles():
    """The generated preprocess source holds the lowered program as a constant
    array and builds for gfx950 against the library's own headers."""
    import os
    import subprocess
    import tempfile

    spec = cm.cm_spec_compile(specs.RETRIEVAL)
    src = cm.cm_spec_codegen(spec)
    assert "kProgram[" in src and "preprocess_body(a, kProgram)" in src
    words = src.split("kProgram[")[1].split("]")[0]
    assert int(words) > 10
    csrc = os.path.join(os.path.dirname(cm.__file__), "csrc")
    with tempfile.TemporaryDirectory() as d:
        f = os.path.join(d, "spec.hip")
        open(f, "w").write("#include <hip/hip_runtime.h>\n" + src)
        r = subprocess.run(["/opt/rocm/bin/hipcc", "-std=c++17", "-O1", "--offload-arch=gfx950", "--cuda-device-only",
                            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                            "-I", csrc, "-c", f, "-o", os.path.join(d, "spec.o")], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]


def test_binding_rejects_tensors_that_do_not_match_q():
    """The binding checks every tensor against q (shape, strides, dtype,
    device) and lse's shape, dtype and layout before calling the library: the
    C ABI applies q's strides to every tensor."""
    import torch

    B, H, N, d = 2, 3, 64, 128
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16)
    args = cm.attn_args(q, causal=True)
    good = dict(k=q.clone(), v=q.clone(), o=q.clone())
    lse = torch.zeros(B, H, N)
    cases = [
        ("k", torch.zeros(B, H, N + 1, d, dtype=torch.bfloat16), "shape"),
        ("v", torch.zeros(B, H, N, d, dtype=torch.float16), "bfloat16"),
        ("o", torch.zeros(B, N, H, d, dtype=torch.bfloat16).transpose(1, 2), "strides"),
    ]
    for name, bad, what in cases:
        kw = dict(good)
        kw[name] = bad
        with pytest.raises(ValueError, match=what):
            cm.cm_attn_fwd(args, q, kw["k"], kw["v"], None, kw["o"], lse)
    with pytest.raises(ValueError, match="lse"):
        cm.cm_attn_fwd(args, q, good["k"], good["v"], None, good["o"], torch.zeros(B, H, N, dtype=torch.float64))
    with pytest.raises(ValueError, match="lse"):
        cm.cm_attn_fwd(args, q, good["k"], good["v"], None, good["o"], torch.zeros(B, N, H).transpose(1, 2))
    with pytest.raises(ValueError, match="args"):
        cm.cm_attn_fwd(cm.attn_args(q[:, :, :32]), q, good["k"], good["v"], None, good["o"], lse)
    with pytest.raises(ValueError, match="GPU"):
        cm.cm_attn_fwd(args, q, good["k"], good["v"], None, good["o"], lse)
    ws = torch.zeros(16, dtype=torch.float64)
    with pytest.raises(ValueError, match="workspace"):
        cm.cm_attn_bwd(args, q, q, q, q, lse, q, None, q, q, q, ws)
    with pytest.raises(ValueError, match="dq"):
        cm.cm_attn_bwd(args, q, q, q, q, lse, q, None, q[:, :, :32], q, q, torch.zeros(16))
