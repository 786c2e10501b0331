"""GPU parity of the attention kernels against the float64 oracle.

O, dQ, dK, dV must match the oracle within max-abs 2e-2 and relative L2 1e-2
(bf16 inputs, fp32 accumulation); lse within 1e-3 absolute with identical
-inf positions (rows with no visible key).  The backward's D = rowsum(dO * o)
uses the o it is given, the forward's bf16 output; the oracle therefore takes
D from its own O rounded to bf16.

The outputs are bf16 tensors.  Where the exact value has magnitude 8 or more
the nearest bf16 value can itself lie up to 2^-5 away, more than 2e-2, so
there the max-abs bar is 2e-2 plus half the bf16 spacing at that magnitude;
below 8 storage costs at most 2^-6 and the bar is 2e-2 exactly.  Every
comparison records its worst excess over the plain 2e-2 (negative = margin)
for the parity report (conftest.py writes it when CM_PARITY_REPORT names a
file).

Every output buffer is filled with NaN before the kernels run, so a tile that
no work-group writes fails the finiteness check.  The descriptor path and the
maskless causal path of the same kernels must agree bit for bit on the
causal mask.  Inputs are the seeded workloads' bf16 tensors; sizes span
several tiles and end in a ragged tile.  Both operand precisions are tested
(CM_PRECISION_BF16, the default, and CM_PRECISION_SPLIT).
"""
import math

import numpy as np
import pytest
import torch

import runtime_metadata_attention_amd as cm
from runtime_metadata_attention_amd import specs
from oracle import attention as oa
from oracle import masks as om
from tests.test_oracle_masks import small_md
from workloads import WORKLOADS, make_metadata, make_tensors, metadata_from_segments

pytestmark = pytest.mark.gpu

ATOL, RL2, LSE_ATOL = 2e-2, 1e-2, 1e-3
STORAGE_FLOOR = 8.0          # |exact| from which bf16 storage alone can exceed ATOL
PRECISIONS = {"bf16": cm.CM_PRECISION_BF16, "split": cm.CM_PRECISION_SPLIT}

# case id -> {output name: worst excess of |got - exact| over the plain ATOL}
PARITY_REPORT = {}
_CASE = ["?"]


def set_case(name):
    _CASE[0] = name


def run_gpu(spec_text, md, t, tiles, causal=False, desc=None, spec=None, check=cm.CM_CHECK_RUN_BITS,
            precision=cm.CM_PRECISION_BF16):
    """Build the descriptor (unless causal) and run forward + backward into
    NaN-filled outputs."""
    q, k, v, do = (t[n].cuda() for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    if not causal:
        spec = spec or cm.cm_spec_compile(spec_text)
        if desc is None:
            packed = md.B if om.is_packed(md) else 0
            desc = cm.Descriptor(spec, B, N, md.seg_cap, tiles, packed=packed)
        cm.cm_build_descriptor(spec, cm.device_metadata(md), desc)
    args = cm.attn_args(q, causal=causal, check=check, precision=precision)
    nan = float("nan")
    o = torch.full_like(q, nan)
    lse = torch.full((B, H, N), nan, dtype=torch.float32, device="cuda")
    cm.cm_attn_fwd(args, q, k, v, None if causal else desc, o, lse)
    dq, dk, dv = torch.full_like(q, nan), torch.full_like(k, nan), torch.full_like(v, nan)
    ws = torch.empty(cm.cm_attn_bwd_workspace(args) // 4, dtype=torch.float32, device="cuda")
    cm.cm_attn_bwd(args, q, k, v, o, lse, do, None if causal else desc, dq, dk, dv, ws)
    torch.cuda.synchronize()
    return {n: x.cpu() for n, x in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv).items()}


def bf16_half_step(w):
    """Half the spacing of bf16 values around |w| (8 significant bits)."""
    mag = np.maximum(np.abs(w), np.finfo(np.float64).tiny)
    return 0.5 * np.exp2(np.floor(np.log2(mag)) - 7)


def max_abs_bar(w, atol=ATOL):
    """The max-abs bar per element: atol, plus the bf16 storage error where
    |exact| >= 8 (there the nearest bf16 value can be 2^-5 away)."""
    return atol + np.where(np.abs(w) >= STORAGE_FLOOR, bf16_half_step(w), 0.0)


def compare(name, got, want, atol=ATOL, rl2=RL2):
    g = got.double().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    assert np.isfinite(g).all(), f"{name}: non-finite values (an output element was not written)"
    err = np.abs(g - w)
    rel = np.linalg.norm(g - w) / max(np.linalg.norm(w), 1e-30)
    worst = float(err.max() - atol) if err.size else -atol
    rec = PARITY_REPORT.setdefault(_CASE[0], {})
    rec[name] = max(rec.get(name, -1.0), round(worst, 6))
    over = err - max_abs_bar(w, atol)
    assert over.max() <= 0 and (rel <= rl2 or np.linalg.norm(w) < 1e-6), \
        f"{name}: max-abs {err.max():.3e} (at {np.unravel_index(err.argmax(), err.shape)}, |exact| " \
        f"{np.abs(w).flat[err.argmax()]:.3g}), worst excess over the bar {over.max():.3e}, rel-L2 {rel:.3e}"
    return err.max(), rel


def compare_lse(got, want):
    g = got.double().numpy()
    w = np.asarray(want)
    assert not np.isnan(g).any(), "lse: an element was not written"
    assert np.array_equal(np.isneginf(g), np.isneginf(w)), "lse: -inf rows differ"
    fin = np.isfinite(w)
    if fin.any():
        assert np.abs(g[fin] - w[fin]).max() <= LSE_ATOL, f"lse: max-abs {np.abs(g[fin] - w[fin]).max():.3e}"


def check_all(out, t, mask, md):
    dq, dk, dv, O, lse = oa.backward(t["q"], t["k"], t["v"], t["do"], om.row_block_fn(mask, md), stored_o="bf16")
    compare("O", out["o"], O)
    compare_lse(out["lse"], lse)
    compare("dq", out["dq"], dq)
    compare("dk", out["dk"], dk)
    compare("dv", out["dv"], dv)


SMALL = [
    # mask, N, d, tiles, seed
    ("causal", 700, 128, (128, 64, 128, 64), 11),
    ("hstu", 517, 128, (128, 64, 128, 64), 12),
    ("shared_prompt", 900, 128, (128, 64, 128, 64), 13),
    ("retrieval", 777, 128, (128, 64, 128, 64), 14),
    ("shared_prompt", 333, 64, (64, 64, 64, 64), 15),
    ("retrieval", 450, 64, (128, 64, 64, 64), 16),
    ("hstu", 300, 128, (64, 64, 128, 64), 17),
]


@pytest.mark.parametrize("prec", list(PRECISIONS))
@pytest.mark.parametrize("mask,N,d,tiles,seed", SMALL)
def test_small_ragged_parity(mask, N, d, tiles, seed, prec):
    print(f"[attention] {mask} N={N} d={d} tiles={tiles} precision={prec}", flush=True)
    set_case(f"small {mask} N={N} d={d} seed={seed} {prec}")
    md = small_md(mask, N=N, seed=seed, B=2)
    t = make_tensors(2, 2, N, d, seed)
    out = run_gpu(specs.BY_MASK[mask], md, t, tiles, precision=PRECISIONS[prec])
    check_all(out, t, mask, md)


def tiny_sequences():
    """Sequences shorter than one wave's 32 rows, each sample a degenerate
    shape of its family: no history (HSTU rows that see only themselves), a
    prompt that fills the sequence, a segment of one token, a reference to a
    one-token segment."""
    seg = metadata_from_segments
    return [
        ("causal", seg(1, 0, 0, (), [{}] * 2)),
        ("causal", seg(5, 0, 0, (), [{}] * 2)),
        ("hstu", seg(1, 0, 0, ("h",), [{"scalars": [0]}, {"scalars": [1]}])),
        ("hstu", seg(5, 0, 0, ("h",), [{"scalars": [0]}, {"scalars": [5]}])),
        ("shared_prompt", seg(1, 2, 0, ("P",), [{"scalars": [1]}, {"scalars": [0], "bounds": [0, 1]}])),
        ("shared_prompt", seg(5, 2, 0, ("P",), [{"scalars": [2], "bounds": [2, 3, 5]}, {"scalars": [5]}])),
        ("retrieval", seg(5, 3, 2, ("g",), [{"scalars": [1], "bounds": [1, 3, 5], "refs": [[], [0]]},
                                            {"scalars": [0], "bounds": [0, 2, 3, 5], "refs": [[], [], [0]]}])),
    ]


@pytest.mark.parametrize("prec", list(PRECISIONS))
@pytest.mark.parametrize("d,tiles", [(128, (128, 64, 128, 64)), (64, (64, 64, 64, 64))])
def test_tiny_sequences_parity(d, tiles, prec):
    for i, (mask, md) in enumerate(tiny_sequences()):
        print(f"[attention-tiny] {mask} N={md.N} d={d} tiles={tiles} precision={prec}", flush=True)
        set_case(f"tiny {mask} N={md.N} d={d} #{i} {prec}")
        t = make_tensors(md.B, 2, md.N, d, 40 + i)
        out = run_gpu(specs.BY_MASK[mask], md, t, tiles, precision=PRECISIONS[prec])
        check_all(out, t, mask, md)
        if mask == "causal":
            check_all(run_gpu(None, md, t, tiles, causal=True, precision=PRECISIONS[prec]), t, mask, md)


@pytest.mark.parametrize("prec", list(PRECISIONS))
def test_tiny_workload_parity(prec):
    w = WORKLOADS["shared_prompt_tiny"]
    set_case(f"workload shared_prompt_tiny {prec}")
    md = make_metadata(w)
    t = make_tensors(w.B, w.H, w.N, w.d, w.seed)
    out = run_gpu(specs.BY_MASK[w.mask], md, t, w.tiles, precision=PRECISIONS[prec])
    check_all(out, t, w.mask, md)


def test_empty_rows_give_zero_output_and_no_gradient():
    # retrieval with no prefix and segments that leave gaps: gap rows see nothing
    N = 300
    bounds = [20, 90, 150, 260]
    md = metadata_from_segments(N, 4, 2, ("g",), [{"scalars": [0], "bounds": bounds, "refs": [[], [0], [0, 1]]}])
    t = make_tensors(1, 2, N, 128, 21)
    out = run_gpu(specs.RETRIEVAL, md, t, (128, 64, 128, 64))
    check_all(out, t, "retrieval", md)
    empty = np.r_[0:20, 260:300]
    assert torch.isneginf(out["lse"][0, :, empty]).all()
    assert (out["o"][0, :, empty].float() == 0).all() and (out["dq"][0, :, empty].float() == 0).all()


def test_causal_descriptor_path_equals_maskless_path_bitwise():
    N = 1000
    md = small_md("causal", N=N, B=2)
    t = make_tensors(2, 3, N, 128, 31)
    a = run_gpu(specs.CAUSAL, md, t, (128, 64, 128, 64))
    b = run_gpu(None, md, t, None, causal=True)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[n], b[n]), n
    check_all(b, t, "causal", md)


def many_column_runs_md(N=640):
    """Retrieval metadata whose first segment is referenced by every other
    later segment, so its key columns carry more runs than the kernels hold
    in registers."""
    L = 40
    bounds = list(range(L, N + 1, L))
    n = len(bounds) - 1
    refs = [[]] + [[0] if i % 2 == 0 else [max(0, i - 1)] for i in range(1, n)]
    return metadata_from_segments(N, n + 1, 2, ("g",), [{"scalars": [L], "bounds": bounds, "refs": refs}])


ABLATION = [
    # mask, N, d, tiles, seed
    ("hstu", 517, 128, (128, 64, 128, 64), 12),
    ("shared_prompt", 333, 64, (64, 64, 64, 64), 15),
    ("retrieval", 777, 128, (128, 64, 128, 64), 14),
    ("many_runs", 640, 128, (128, 64, 128, 64), 18),
]


@pytest.mark.parametrize("mask,N,d,tiles,seed", ABLATION)
def test_ablation_checks_equal_the_default_check_bitwise(mask, N, d, tiles, seed):
    """The per-element unsigned-compare kernels and the ablation kernels
    (ordinary compares on masked intervals) decide the same visibility as the
    default run-bitmask kernels, so every output is equal."""
    print(f"[ablation] {mask} N={N} d={d} tiles={tiles}", flush=True)
    if mask == "many_runs":
        md, mask = many_column_runs_md(N), "retrieval"
        m = om.dense_mask(mask, md, 0).astype(np.int8)
        starts = np.diff(np.vstack([np.zeros((1, N), np.int8), m]), axis=0) == 1
        assert starts.sum(axis=0).max() > 4, "the case must exceed the register copy of column runs"
    else:
        md = small_md(mask, N=N, seed=seed, B=2)
    t = make_tensors(md.B, 2, N, d, seed)
    a = run_gpu(specs.BY_MASK[mask], md, t, tiles)
    check_all(a, t, mask, md)
    for check in (cm.CM_CHECK_UNSIGNED, cm.CM_CHECK_ORDINARY_MASKED):
        b = run_gpu(specs.BY_MASK[mask], md, t, tiles, check=check)
        for n in ("o", "lse", "dq", "dk", "dv"):
            assert torch.equal(a[n], b[n]), (check, n)


def test_columns_with_twenty_runs_parity():
    """Key columns with 20 visible-row runs: the dK/dV kernel's memory path for
    runs beyond its register copy, and the preprocess's beyond 16 intervals."""
    L, S = 40, 40
    N = 40 + L * S
    bounds = [40 + L * k for k in range(S + 1)]
    refs = [[], []] + [[0] if k % 2 == 0 else [1, k - 1] for k in range(2, S)]
    md = metadata_from_segments(N, S, 2, ("g",), [{"scalars": [40], "bounds": bounds, "refs": refs}])
    t = make_tensors(1, 2, N, 128, 61)
    out = run_gpu(specs.RETRIEVAL, md, t, (128, 64, 128, 64))
    check_all(out, t, "retrieval", md)


def test_ablation_checks_on_the_causal_path():
    N = 700
    md = small_md("causal", N=N, B=1)
    t = make_tensors(1, 2, N, 128, 32)
    a = run_gpu(None, md, t, None, causal=True)
    for check in (cm.CM_CHECK_UNSIGNED, cm.CM_CHECK_ORDINARY_MASKED):
        b = run_gpu(None, md, t, None, causal=True, check=check)
        for n in ("o", "lse", "dq", "dk", "dv"):
            assert torch.equal(a[n], b[n]), (check, n)


def test_strided_layout_matches_contiguous():
    """[B, N, H, d] storage through the stride arguments."""
    mask, N = "shared_prompt", 400
    md = small_md(mask, N=N, seed=3, B=2)
    t = make_tensors(2, 2, N, 128, 41)
    a = run_gpu(specs.BY_MASK[mask], md, t, (128, 64, 128, 64))
    ts = {n: x.transpose(1, 2).contiguous().transpose(1, 2) for n, x in t.items()}
    assert ts["q"].stride()[1] == 128
    b = run_gpu(specs.BY_MASK[mask], md, ts, (128, 64, 128, 64))
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[n], b[n]), n


def test_forward_bitwise_repeatable_and_desc_reuse():
    mask, N = "hstu", 640
    md = small_md(mask, N=N, seed=4, B=2)
    t = make_tensors(2, 2, N, 128, 51)
    spec = cm.cm_spec_compile(specs.HSTU)
    desc = cm.Descriptor(spec, 2, N, md.seg_cap, (128, 64, 128, 64))
    a = run_gpu(None, md, t, None, desc=desc, spec=spec)
    b = run_gpu(None, md, t, None, desc=desc, spec=spec)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[n], b[n]), n


def _busy(stream_cycles):
    """Keep the current stream busy for a while (spin kernel, else matmuls)."""
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(stream_cycles)
        return
    a = torch.full((2048, 2048), 1e-3, device="cuda")
    for _ in range(40):
        a = a @ a


def test_launches_follow_the_callers_stream():
    """Every call enqueues on the stream it is given (here torch's current
    stream inside a side-stream context, as the binding passes it): inputs
    that the side stream writes only after a delay are the ones read, and
    the outputs equal a default-stream run bit for bit."""
    mask, N, d, tiles = "shared_prompt", 900, 128, (128, 64, 128, 64)
    md = small_md(mask, N=N, seed=21, B=2)
    t = make_tensors(2, 2, N, d, 21)
    ref = run_gpu(specs.BY_MASK[mask], md, t, tiles)
    src = {n: t[n].cuda() for n in ("q", "k", "v", "do")}
    x = {n: torch.zeros_like(a) for n, a in src.items()}
    spec = cm.cm_spec_compile(specs.BY_MASK[mask])
    desc = cm.Descriptor(spec, 2, N, md.seg_cap, tiles)
    dmd = cm.device_metadata(md)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        _busy(100_000_000)
        for n in x:
            x[n].copy_(src[n])
        cm.cm_build_descriptor(spec, dmd, desc)
        args = cm.attn_args(x["q"])
        o = torch.empty_like(x["q"])
        lse = torch.empty(2, 2, N, dtype=torch.float32, device="cuda")
        cm.cm_attn_fwd(args, x["q"], x["k"], x["v"], desc, o, lse)
        dq, dk, dv = torch.empty_like(o), torch.empty_like(o), torch.empty_like(o)
        ws = torch.empty(cm.cm_attn_bwd_workspace(args) // 4, dtype=torch.float32, device="cuda")
        cm.cm_attn_bwd(args, x["q"], x["k"], x["v"], o, lse, x["do"], desc, dq, dk, dv, ws)
    side.synchronize()
    for n, got in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv).items():
        assert torch.equal(got.cpu(), ref[n]), n


BESIDE_CASES = [
    # B, H, N, seed: hstu_4k's shape (the dK/dV grid holds two work-groups per CU), smaller grids
    (4, 8, 4096, 1003),
    (2, 2, 1000, 41),
    (1, 3, 700, 42),
]


@pytest.mark.parametrize("B,H,N,seed", BESIDE_CASES)
def test_backward_with_dq_beside_dkdv_equals_the_kernels_one_by_one(B, H, N, seed):
    """On short grids cm_attn_bwd runs dQ on a second stream beside dK/dV,
    after D on the caller's stream, and the caller's stream waits for both.
    The result equals the three backward kernels called one by one
    (cm_attn_bwd_stage) bit for bit.  The call runs on a side stream whose
    inputs are written only after a delay, and the outputs are copied on
    that stream right after the call: a missing fork or join would read or
    copy unfinished data."""
    print(f"[attention-beside] hstu B={B} H={H} N={N} seed={seed}", flush=True)
    if N == 4096:
        md = make_metadata(WORKLOADS["hstu_4k"])
    else:
        md = small_md("hstu", N=N, seed=seed, B=B)
    t = make_tensors(B, H, N, 128, seed)
    tiles = (128, 64, 128, 64)
    src = {n: t[n].cuda() for n in ("q", "k", "v", "do")}
    spec = cm.cm_spec_compile(specs.HSTU)
    desc = cm.Descriptor(spec, B, N, md.seg_cap, tiles)
    cm.cm_build_descriptor(spec, cm.device_metadata(md), desc)
    args = cm.attn_args(src["q"])
    o = torch.empty_like(src["q"])
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    cm.cm_attn_fwd(args, src["q"], src["k"], src["v"], desc, o, lse)
    ws = torch.empty(cm.cm_attn_bwd_workspace(args) // 4, dtype=torch.float32, device="cuda")
    ref = [torch.full_like(src["q"], float("nan")) for _ in range(3)]
    for stage in range(3):
        cm.cm_attn_bwd_stage(stage, args, src["q"], src["k"], src["v"], o, lse, src["do"], desc, *ref, ws)
    torch.cuda.synchronize()
    x = {n: torch.zeros_like(a) for n, a in src.items()}
    got = [torch.full_like(src["q"], float("nan")) for _ in range(3)]
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        _busy(100_000_000)
        for n in x:
            x[n].copy_(src[n])
        cm.cm_attn_bwd(args, x["q"], x["k"], x["v"], o, lse, x["do"], desc, *got, ws)
        copies = [g.clone() for g in got]
    side.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), copies, ref):
        assert torch.equal(a, b), name


def test_backward_from_two_host_threads_on_their_own_streams():
    """Two host threads call cm_attn_bwd at the same time, each on its own
    stream with its own tensors, on a grid short enough that the library runs
    dQ on its side stream (shared by every caller on the device): each
    thread's results equal the kernels called one by one, bit for bit."""
    import threading

    B, H, N = 2, 2, 1000
    print(f"[attention-threads] hstu B={B} H={H} N={N}", flush=True)
    cases = []
    for seed in (61, 62):
        md = small_md("hstu", N=N, seed=seed, B=B)
        t = make_tensors(B, H, N, 128, seed)
        x = {n: t[n].cuda() for n in ("q", "k", "v", "do")}
        spec = cm.cm_spec_compile(specs.HSTU)
        desc = cm.Descriptor(spec, B, N, md.seg_cap, (128, 64, 128, 64))
        cm.cm_build_descriptor(spec, cm.device_metadata(md), desc)
        args = cm.attn_args(x["q"])
        o = torch.empty_like(x["q"])
        lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
        cm.cm_attn_fwd(args, x["q"], x["k"], x["v"], desc, o, lse)
        ws = torch.empty(cm.cm_attn_bwd_workspace(args) // 4, dtype=torch.float32, device="cuda")
        ref = [torch.full_like(o, float("nan")) for _ in range(3)]
        for stage in range(3):
            cm.cm_attn_bwd_stage(stage, args, x["q"], x["k"], x["v"], o, lse, x["do"], desc, *ref, ws)
        cases.append(dict(x=x, desc=desc, args=args, o=o, lse=lse, ref=ref,
                          ws=torch.empty_like(ws), stream=torch.cuda.Stream()))
    torch.cuda.synchronize()
    errors = []

    def run(c):
        try:
            with torch.cuda.stream(c["stream"]):
                for _ in range(4):
                    got = [torch.full_like(c["o"], float("nan")) for _ in range(3)]
                    cm.cm_attn_bwd(c["args"], c["x"]["q"], c["x"]["k"], c["x"]["v"], c["o"], c["lse"], c["x"]["do"],
                                   c["desc"], *got, c["ws"])
                    c["stream"].synchronize()
                    for name, a, b in zip(("dq", "dk", "dv"), got, c["ref"]):
                        if not torch.equal(a, b):
                            errors.append(name)
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=run, args=(c,)) for c in cases]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=100)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors


_FIRST_CALL_CAPTURED = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
import runtime_metadata_attention_amd as cm
from runtime_metadata_attention_amd import specs
from tests.test_oracle_masks import small_md
from workloads import make_tensors
B, H, N = 2, 2, 1000
md = small_md("hstu", N=N, seed=51, B=B)
t = make_tensors(B, H, N, 128, 51)
x = {n: t[n].cuda() for n in ("q", "k", "v", "do")}
spec = cm.cm_spec_compile(specs.HSTU)
desc = cm.Descriptor(spec, B, N, md.seg_cap, (128, 64, 128, 64))
cm.cm_build_descriptor(spec, cm.device_metadata(md), desc)
args = cm.attn_args(x["q"])
o = torch.empty_like(x["q"])
lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
cm.cm_attn_fwd(args, x["q"], x["k"], x["v"], desc, o, lse)
ws = torch.empty(cm.cm_attn_bwd_workspace(args) // 4, dtype=torch.float32, device="cuda")
got = [torch.full_like(o, float("nan")) for _ in range(3)]
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g):
    cm.cm_attn_bwd(args, x["q"], x["k"], x["v"], o, lse, x["do"], desc, *got, ws)
ref = [torch.full_like(o, float("nan")) for _ in range(3)]
for stage in range(3):
    cm.cm_attn_bwd_stage(stage, args, x["q"], x["k"], x["v"], o, lse, x["do"], desc, *ref, ws)
for rep in range(3):
    for a in got:
        a.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), (rep, name)
    print("replay", rep, "ok", flush=True)
"""


def test_first_backward_call_inside_a_graph_capture():
    """A process whose first cm_attn_bwd call is captured into a HIP graph
    (the library creates no stream inside a capture and runs that backward
    on the caller's stream): every replay equals the kernels called one by
    one.  Runs in a child process, so that no earlier call has set anything
    up."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    print("[attention-capture-first] child process", flush=True)
    r = subprocess.run([sys.executable, "-c", _FIRST_CALL_CAPTURED, root], cwd=root, capture_output=True,
                       text=True, timeout=100)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.count("ok") == 3


def test_step_captured_in_a_hip_graph_replays_with_new_metadata():
    """Descriptor build, forward and backward captured once into a HIP graph
    (the hot calls allocate, copy and clear nothing) and replayed with new
    metadata written into the same device buffers: every replay equals the
    eager step on that metadata bit for bit, with eager work and
    synchronisation between the replays."""
    mask, N, d, tiles = "hstu", 1000, 128, (128, 64, 128, 64)
    mds = [small_md(mask, N=N, seed=s, B=2) for s in (31, 32, 33)]
    t = make_tensors(2, 2, N, d, 31)
    eager = [run_gpu(specs.BY_MASK[mask], md, t, tiles) for md in mds]
    spec = cm.cm_spec_compile(specs.BY_MASK[mask])
    desc = cm.Descriptor(spec, 2, N, mds[0].seg_cap, tiles)
    dmd = cm.device_metadata(mds[0])
    x = {n: t[n].cuda() for n in ("q", "k", "v", "do")}
    args = cm.attn_args(x["q"])
    out = dict(o=torch.empty_like(x["q"]), lse=torch.empty(2, 2, N, dtype=torch.float32, device="cuda"),
               dq=torch.empty_like(x["q"]), dk=torch.empty_like(x["q"]), dv=torch.empty_like(x["q"]))
    ws = torch.empty(cm.cm_attn_bwd_workspace(args) // 4, dtype=torch.float32, device="cuda")

    def step():
        cm.cm_build_descriptor(spec, dmd, desc)
        cm.cm_attn_fwd(args, x["q"], x["k"], x["v"], desc, out["o"], out["lse"])
        cm.cm_attn_bwd(args, x["q"], x["k"], x["v"], out["o"], out["lse"], x["do"], desc,
                       out["dq"], out["dk"], out["dv"], ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(2):
        for i, (md, want) in enumerate(zip(mds, eager)):
            print(f"[graph] replay {rep}.{i}", flush=True)
            for name in ("scalars", "seg_bounds", "n_seg", "refs"):
                dev = getattr(dmd, name)
                if dev is not None:
                    dev.copy_(torch.as_tensor(getattr(md, name), dtype=torch.int32).reshape(dev.shape))
            g.replay()
            torch.cuda.synchronize()
            for n, got in out.items():
                assert torch.equal(got.cpu(), want[n]), (rep, i, n)
            run_gpu(specs.BY_MASK[mask], mds[(i + 1) % 3], t, tiles)  # eager work between replays


def test_argument_errors_launch_nothing():
    spec = cm.cm_spec_compile(specs.CAUSAL)
    md = small_md("causal", N=256, B=1)
    desc = cm.Descriptor(spec, 1, 256, md.seg_cap, (128, 64, 128, 64))
    q = torch.zeros(1, 1, 128, 128, dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 7.0)
    lse = torch.zeros(1, 1, 128, device="cuda")
    with pytest.raises(cm.CompileMaskError) as e:
        cm.cm_attn_fwd(cm.attn_args(q), q, q, q, desc, o, lse)      # N mismatch
    assert e.value.status == -4
    bad = cm.Descriptor(spec, 1, 128, 0, (64, 32, 128, 64))
    with pytest.raises(cm.CompileMaskError) as e:
        cm.cm_attn_fwd(cm.attn_args(q), q, q, q, bad, o, lse)       # no kernel for 64x32 tiles
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert (o == 7.0).all()


FULL = ["causal_8k", "hstu_4k", "reward_model_32k", "retrieval4_32k", "hstu_packed_64k"]


def key_tile_rows(fn, b, N, bk, block=2048):
    """Per key tile of width bk: how many query rows of sample b see a key in it."""
    T = (N + bk - 1) // bk
    counts = np.zeros(T, np.int64)
    for r0 in range(0, N, block):
        M = fn(b, r0, min(N, r0 + block))
        pad = np.zeros((M.shape[0], T * bk), bool)
        pad[:, :N] = M
        counts += pad.reshape(M.shape[0], T, bk).any(axis=2).sum(axis=0)
    return counts


def full_size_tiles(w, md, fn, b):
    """Whole tiles to check for every head of sample b: the first and last
    query tiles (rows), the last key tile and the partial key tile seen by the
    fewest rows (keys), plus the rows that see those keys."""
    fq, bk = w.tiles[0], w.tiles[2]
    Tq = (w.N + fq - 1) // fq
    counts = key_tile_rows(fn, b, w.N, bk)
    cand = [t for t in range(len(counts) - 1) if 0 < counts[t] < w.N]
    kt = min(cand, key=lambda t: counts[t]) if cand else 0
    keys = np.unique(np.r_[kt * bk: min(w.N, kt * bk + bk), (len(counts) - 1) * bk: w.N])
    rows_fixed = np.r_[0:fq, (Tq - 1) * fq: w.N]
    return Tq, fq, rows_fixed, keys, oa.rows_seeing(fn, b, w.N, keys)


@pytest.mark.parametrize("name", FULL)
def test_full_size_parity_every_head(name):
    """Full workload on the GPU in both precisions, into NaN-filled outputs:
    every element of every output must be written.  Every (sample, head) is
    then checked against the oracle on whole tiles: the first, the last and
    one other query tile (O, lse, dq), the last key tile and the partial key
    tile that the fewest rows see (dk, dv).  One head is also checked on the
    first key tile and random rows and keys, with its whole forward."""
    w = WORKLOADS[name]
    md = make_metadata(w)
    t = make_tensors(w.B, w.H, w.N, w.d, w.seed)
    outs = {}
    for prec in PRECISIONS:
        print(f"[attention-full] {name} precision={prec}", flush=True)
        outs[prec] = run_gpu(specs.BY_MASK[w.mask], md, t, w.tiles, precision=PRECISIONS[prec])
        for n in ("o", "lse", "dq", "dk", "dv"):
            assert not torch.isnan(outs[prec][n]).any(), (prec, n, "not written")
    fn = om.row_block_fn(w.mask, md)
    rng = np.random.default_rng(w.seed)
    f = lambda x, b, h: oa._f64(x[b, h])  # noqa: E731
    for b in range(w.B):
        Tq, fq, rows_fixed, keys, seeing = full_size_tiles(w, md, fn, b)
        for h in range(w.H):
            mid = int(rng.integers(1, max(2, Tq - 1)))
            rows = np.unique(np.r_[rows_fixed, mid * fq: min(w.N, mid * fq + fq)])
            ref = oa.tiles_head(f(t["q"], b, h), f(t["k"], b, h), f(t["v"], b, h), f(t["do"], b, h), fn, b, rows,
                                keys, stored_o="bf16", seeing=seeing)
            for prec, out in outs.items():
                set_case(f"full {name} {prec}")
                compare("O", out["o"][b, h, rows], ref["O"])
                compare_lse(out["lse"][b, h, rows], ref["lse"])
                compare("dq", out["dq"][b, h, rows], ref["dq"])
                compare("dk", out["dk"][b, h, keys], ref["dk"])
                compare("dv", out["dv"][b, h, keys], ref["dv"])
        print(f"[attention-full] {name} sample {b}: {w.H} heads, {len(rows_fixed) + fq} rows, {len(keys)} keys, "
              f"{len(seeing)} rows seeing them", flush=True)
    b, h = w.B - 1, w.H // 2
    rows = np.unique(np.r_[rng.choice(w.N, 24, replace=False), 0, w.N - 1])
    keys = np.unique(np.r_[rng.choice(w.N, 24, replace=False), 0:w.tiles[2], w.N - 1])
    ref = oa.sampled_head(f(t["q"], b, h), f(t["k"], b, h), f(t["v"], b, h), f(t["do"], b, h), fn, b, rows, keys,
                          block=2048 if w.N <= 32768 else 1024, stored_o="bf16")
    for prec, out in outs.items():
        set_case(f"full {name} {prec}")
        compare("O", out["o"][b, h, rows], ref["O"])
        compare_lse(out["lse"][b, h, rows], ref["lse"])
        compare("dq", out["dq"][b, h, rows], ref["dq"])
        compare("dk", out["dk"][b, h, keys], ref["dk"])
        compare("dv", out["dv"][b, h, keys], ref["dv"])


# Whole-tensor cases whose B * H is a multiple of the 8 XCDs, so the
# kernels' XCD-aware work-group order is in effect: fewer than 128 tiles per
# head (heads dealt tile by tile) and 128 or more (head by head), on the
# descriptor path and on the maskless causal path.
XCD_CASES = [
    # mask, B, H, N, tiles, causal path, seed
    ("retrieval", 2, 4, 1000, (128, 64, 128, 64), False, 91),
    ("shared_prompt", 2, 8, 700, (128, 64, 128, 64), False, 92),
    ("hstu", 1, 8, 8192, (64, 64, 64, 64), False, 93),
    ("causal", 2, 4, 1000, None, True, 94),
]


@pytest.mark.parametrize("prec", list(PRECISIONS))
@pytest.mark.parametrize("mask,B,H,N,tiles,causal,seed", XCD_CASES)
def test_xcd_orders_whole_tensor(mask, B, H, N, tiles, causal, seed, prec):
    print(f"[attention-xcd] {mask} B={B} H={H} N={N} tiles={tiles} causal={causal} precision={prec}", flush=True)
    set_case(f"xcd {mask} B={B} H={H} N={N} {prec}")
    md = small_md(mask, N=N, seed=seed, B=B)
    t = make_tensors(B, H, N, 128, seed)
    out = run_gpu(specs.BY_MASK[mask], md, t, tiles, causal=causal, precision=PRECISIONS[prec])
    check_all(out, t, mask, md)


def test_causal_path_head_by_head_order():
    """The maskless causal path with 128 query tiles per head (N = 16384,
    head-by-head order) equals the descriptor path bit for bit over every
    head, and the oracle over two whole heads."""
    N, B, H = 16384, 1, 8
    md = small_md("causal", N=N, B=B)
    t = make_tensors(B, H, N, 128, 95)
    print("[attention-xcd] causal N=16384 B=1 H=8, both paths", flush=True)
    a = run_gpu(None, md, t, None, causal=True)
    d = run_gpu(specs.CAUSAL, md, t, (128, 64, 128, 64))
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[n], d[n]), n
    set_case("xcd causal N=16384 bf16")
    fn = om.row_block_fn("causal", md)
    for h in (0, H - 1):
        f = lambda x: oa._f64(x[0, h])  # noqa: E731
        dq, dk, dv, O, lse = oa.backward_head(f(t["q"]), f(t["k"]), f(t["v"]), f(t["do"]), fn, 0, block=2048,
                                              stored_o="bf16")
        compare("O", a["o"][0, h], O)
        compare_lse(a["lse"][0, h], lse)
        compare("dq", a["dq"][0, h], dq)
        compare("dk", a["dk"][0, h], dk)
        compare("dv", a["dv"][0, h], dv)


WIDE_CASES = [
    # mask, B, H, N, d, seed: unpacked batches with N >= 2048, where the dK/dV
    # kernel with 64 keys per wave runs; N ragged and an odd number of 128-key
    # tiles (the last work-group's second tile is empty); B * H = 8 engages
    # the XCD order; retrieval gives key columns several visible-row runs
    ("shared_prompt", 1, 2, 8269, 128, 96),
    ("causal", 1, 2, 8200, 64, 97),
    ("hstu", 2, 4, 2100, 128, 98),
    ("retrieval", 1, 2, 3000, 64, 99),
]


@pytest.mark.parametrize("mask,B,H,N,d,seed", WIDE_CASES)
def test_wide_dkdv_whole_tensor(mask, B, H, N, d, seed):
    print(f"[attention-wide] {mask} B={B} H={H} N={N} d={d}", flush=True)
    md = small_md(mask, N=N, seed=seed, B=B)
    t = make_tensors(B, H, N, d, seed)
    out = run_gpu(specs.BY_MASK[mask], md, t, (128, 64, 128, 64))
    check_all(out, t, mask, md)
