"""GPU tests of the predicate baseline (FlexAttention-style masking).

cm_build_blockmask evaluates a mask family's predicate at every element to
build the tile bitmaps; attention with check = CM_CHECK_PREDICATE evaluates
it again at every element of a partial tile.  Its bitmaps must equal the
oracle's tile codes (and the preprocess's), and its attention outputs must
equal the interval path's bit for bit: same tiles, same visibility, same
arithmetic.
"""
import numpy as np
import pytest
import torch

import runtime_metadata_attention_amd as cm
from runtime_metadata_attention_amd import specs
from oracle import descriptor as od
from oracle import masks as om
from tests.test_gpu_attention import check_all, run_gpu
from tests.test_oracle_masks import small_md
from workloads import WORKLOADS, make_metadata, make_tensors

pytestmark = pytest.mark.gpu

CASES = [
    # mask, N, tiles, seed
    ("causal", 700, (128, 64, 128, 64), 1),
    ("hstu", 517, (128, 64, 128, 64), 2),
    ("shared_prompt", 900, (128, 64, 128, 64), 3),
    ("retrieval", 777, (128, 64, 128, 64), 4),
    ("shared_prompt", 333, (64, 64, 64, 64), 5),
    ("retrieval", 450, (48, 40, 40, 48), 6),
]


def blockmask(mask, md, tiles):
    spec = cm.cm_spec_compile(specs.BY_MASK[mask])
    desc = cm.Descriptor(spec, md.B, md.N, md.seg_cap, tiles)
    dmd = cm.device_metadata(md)
    cm.cm_build_blockmask(mask, dmd, desc)
    torch.cuda.synchronize()
    return desc


@pytest.mark.parametrize("mask,N,tiles,seed", CASES)
def test_blockmask_bitmaps_equal_oracle_codes(mask, N, tiles, seed):
    print(f"[blockmask] {mask} N={N} tiles={tiles}", flush=True)
    md = small_md(mask, N=N, seed=seed, B=2)
    desc = blockmask(mask, md, tiles)
    words = desc.words()
    want = od.build(mask, md, desc.K_r, desc.K_c, tiles)
    g = od.View(words, md.B, N, desc.K_r, desc.K_c, tiles)
    o = od.View(want, md.B, N, desc.K_r, desc.K_c, tiles)
    for name in ("fbm", "bbm", "sample_err"):
        assert np.array_equal(g[name], o[name]), name
    assert np.array_equal(g["header"][:15], o["header"][:15])


def test_blockmask_flags_invalid_metadata():
    md = small_md("retrieval", N=300, seed=8, B=2)
    md.refs[1, 2, 0] = 40  # beyond n_seg
    desc = blockmask("retrieval", md, (128, 64, 128, 64))
    g = od.View(desc.words(), md.B, md.N, desc.K_r, desc.K_c, (128, 64, 128, 64))
    assert g["sample_err"][1] == om.ERR_REF_RANGE and g["sample_err"][0] == 0
    assert not g["fbm"][1].any() and not g["bbm"][1].any()


@pytest.mark.parametrize("mask,N,tiles,seed", [c for c in CASES if c[2][1] == 64])
def test_predicate_attention_equals_interval_attention_bitwise(mask, N, tiles, seed):
    print(f"[predicate-attn] {mask} N={N} tiles={tiles}", flush=True)
    md = small_md(mask, N=N, seed=seed, B=2)
    t = make_tensors(2, 2, N, 128, seed)
    a = run_gpu(specs.BY_MASK[mask], md, t, tiles)
    spec = cm.cm_spec_compile(specs.BY_MASK[mask])
    desc = blockmask(mask, md, tiles)
    q, k, v, do = (t[n].cuda() for n in ("q", "k", "v", "do"))
    args = cm.attn_args(q, check=cm.CM_CHECK_PREDICATE)
    o = torch.empty_like(q)
    lse = torch.empty(2, 2, N, dtype=torch.float32, device="cuda")
    cm.cm_attn_fwd(args, q, k, v, desc, o, lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(cm.cm_attn_bwd_workspace(args) // 4, dtype=torch.float32, device="cuda")
    cm.cm_attn_bwd(args, q, k, v, o, lse, do, desc, dq, dk, dv, ws)
    torch.cuda.synchronize()
    b = {n: x.cpu() for n, x in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv).items()}
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[n], b[n]), n
    check_all(b, t, mask, md)


def test_check_and_descriptor_kind_must_match():
    md = small_md("hstu", N=256, seed=1, B=1)
    spec = cm.cm_spec_compile(specs.HSTU)
    interval = cm.Descriptor(spec, 1, 256, md.seg_cap, (128, 64, 128, 64))
    cm.cm_build_descriptor(spec, cm.device_metadata(md), interval)
    bm = blockmask("hstu", md, (128, 64, 128, 64))
    q = torch.zeros(1, 1, 256, 128, dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 7.0)
    lse = torch.zeros(1, 1, 256, device="cuda")
    with pytest.raises(cm.CompileMaskError) as e:
        cm.cm_attn_fwd(cm.attn_args(q, check=cm.CM_CHECK_PREDICATE), q, q, q, interval, o, lse)
    assert e.value.status == -4
    with pytest.raises(cm.CompileMaskError) as e:
        cm.cm_attn_fwd(cm.attn_args(q), q, q, q, bm, o, lse)
    assert e.value.status == -4
    with pytest.raises(cm.CompileMaskError) as e:
        cm.cm_attn_fwd(cm.attn_args(q, causal=True, check=cm.CM_CHECK_PREDICATE), q, q, q, None, o, lse)
    assert e.value.status == -2
    torch.cuda.synchronize()
    assert (o == 7.0).all()


@pytest.mark.parametrize("name", ["reward_model_32k", "retrieval4_32k"])
def test_full_size_blockmask_equals_preprocess_bitmaps(name):
    w = WORKLOADS[name]
    md = make_metadata(w)
    print(f"[blockmask-full] {name}", flush=True)
    spec = cm.cm_spec_compile(specs.BY_MASK[w.mask])
    d1 = cm.Descriptor(spec, w.B, w.N, w.seg_cap, w.tiles)
    cm.cm_build_descriptor(spec, cm.device_metadata(md), d1)
    d2 = blockmask(w.mask, md, w.tiles)
    g1 = od.View(d1.words(), w.B, w.N, d1.K_r, d1.K_c, w.tiles)
    g2 = od.View(d2.words(), w.B, w.N, d2.K_r, d2.K_c, w.tiles)
    for n in ("fbm", "bbm", "sample_err"):
        assert np.array_equal(g1[n], g2[n]), n
