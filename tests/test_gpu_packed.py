"""GPU parity of packed variable-length batches (cu_seqlens).

The preprocess builds the descriptor of the one packed sequence; it must be
bit-exact against the oracle's (which reads it off the block-diagonal dense
mask), and the unchanged attention kernels, run on [1, H, T, d] tensors with
it, must match the oracle within the usual tolerances.  Cases mix empty,
short and long samples so that tiles straddle sample boundaries.
"""
import numpy as np
import pytest
import torch

import runtime_metadata_attention_amd as cm
from runtime_metadata_attention_amd import specs
from oracle import descriptor as od
from oracle import masks as om
from tests.test_gpu_attention import check_all, run_gpu
from tests.test_gpu_descriptor import explain, gpu_descriptor
from tests.test_oracle_packed import packed_md
from workloads import make_tensors

pytestmark = pytest.mark.gpu

CASES = [
    # mask, lengths, tiles, seed
    ("causal", [70, 0, 129, 64, 200, 0, 65], (128, 64, 128, 64), 1),
    ("hstu", [300, 5, 1, 0, 260, 77], (128, 64, 128, 64), 2),
    ("hstu", [33, 40, 17, 90], (48, 40, 40, 48), 3),
    ("shared_prompt", [150, 64, 300, 90], (128, 64, 128, 64), 4),
    ("retrieval", [200, 90, 260], (128, 64, 128, 64), 5),
    ("retrieval", [120, 64, 64, 140], (64, 64, 64, 64), 6),
]


def widths(mask, md):
    spec = cm.cm_spec_compile(specs.BY_MASK[mask])
    return cm.cm_spec_info(spec, md.seg_cap)[:2]


@pytest.mark.parametrize("mask,lengths,tiles,seed", CASES)
def test_packed_descriptor_bit_exact(mask, lengths, tiles, seed):
    print(f"[packed-desc] {mask} lengths={lengths} tiles={tiles}", flush=True)
    md = packed_md(mask, lengths, seed)
    K_r, K_c = widths(mask, md)
    words, desc, spec = gpu_descriptor(mask, md, tiles, guard_bytes=256)
    want = od.build(mask, md, K_r, K_c, tiles)
    assert words.shape == want.shape
    if not np.array_equal(words, want):
        pytest.fail(explain(words, want, 1, md.N, K_r, K_c, tiles, n_err=md.B))
    assert (desc.buffer[desc.bytes:].cpu().numpy() == 0xA5).all()


@pytest.mark.parametrize("mask,lengths,tiles,seed", [c for c in CASES if c[2][1] == 64])
def test_packed_attention_parity(mask, lengths, tiles, seed):
    print(f"[packed-attn] {mask} lengths={lengths} tiles={tiles}", flush=True)
    md = packed_md(mask, lengths, seed)
    t = make_tensors(1, 2, md.N, 128, seed)
    out = run_gpu(specs.BY_MASK[mask], md, t, tiles)
    check_all(out, t, mask, md)


def test_invalid_cu_seqlens_flags_and_empties():
    md = packed_md("hstu", [100, 60, 90], 7)
    md.cu_seqlens = np.array([0, 100, 90, 250], np.int32)  # decreasing
    K_r, K_c = widths("hstu", md)
    words, desc, spec = gpu_descriptor("hstu", md, (128, 64, 128, 64))
    want = od.build("hstu", md, K_r, K_c, (128, 64, 128, 64))
    assert np.array_equal(words, want)
    v = od.View(words, 1, md.N, K_r, K_c, (128, 64, 128, 64), n_err=md.B)
    assert v["header"][13] == om.ERR_CU_SEQLENS and not v["row_iv"].any()


def test_packed_and_padded_metadata_are_not_mixed():
    md = packed_md("causal", [100, 28])
    spec = cm.cm_spec_compile(specs.CAUSAL)
    padded = cm.Descriptor(spec, 1, md.N, md.seg_cap, (128, 64, 128, 64))
    with pytest.raises(cm.CompileMaskError) as e:
        cm.cm_build_descriptor(spec, cm.device_metadata(md), padded)
    assert e.value.status == -4
    packed = cm.Descriptor(spec, 1, md.N, md.seg_cap, (128, 64, 128, 64), packed=md.B)
    md.cu_seqlens = None
    with pytest.raises(cm.CompileMaskError) as e:
        cm.cm_build_descriptor(spec, cm.device_metadata(md), packed)
    assert e.value.status == -1
