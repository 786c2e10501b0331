"""cm_attn_bwd_noalloc (the backward with the library's fixed per-GPU
workspace) against cm_attn_bwd (a caller workspace), through the C ABI.

Both run the same kernels, so the outputs must be equal bit for bit.  Two
calls in a row, the second on a smaller input, check that the fixed array
keeps no state that matters between calls.  A call above the array's row
limit must fail with CM_ERR_SIZE before anything runs.
"""
import numpy as np
import pytest
import torch

import runtime_metadata_attention_amd as cm
from runtime_metadata_attention_amd import specs
from tests.test_oracle_masks import small_md
from workloads import make_tensors

pytestmark = pytest.mark.gpu


def _both(mask, md, t, tiles, causal=False):
    q, k, v, do = (t[n].cuda() for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    desc = None
    if not causal:
        spec = cm.cm_spec_compile(specs.BY_MASK[mask])
        desc = cm.Descriptor(spec, B, N, md.seg_cap, tiles)
        cm.cm_build_descriptor(spec, cm.device_metadata(md), desc)
    args = cm.attn_args(q, causal=causal)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    cm.cm_attn_fwd(args, q, k, v, desc, o, lse)
    ref = [torch.full_like(q, float("nan")) for _ in range(3)]
    ws = torch.empty(cm.cm_attn_bwd_workspace(args) // 4, dtype=torch.float32, device="cuda")
    cm.cm_attn_bwd(args, q, k, v, o, lse, do, desc, *ref, ws)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    cm.cm_attn_bwd_noalloc(args, q, k, v, o, lse, do, desc, *got)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.isfinite(b.float()).all(), name
        assert torch.equal(a.cpu(), b.cpu()), name


def test_noalloc_equals_workspace_backward_on_two_calls():
    tiles = (128, 64, 128, 64)
    print("[no-alloc] retrieval B=2 H=3 N=900, then shared_prompt B=1 H=2 N=300", flush=True)
    md = small_md("retrieval", N=900, seed=5, B=2)
    _both("retrieval", md, make_tensors(2, 3, 900, 128, 71), tiles)
    md = small_md("shared_prompt", N=300, seed=6, B=1)
    _both("shared_prompt", md, make_tensors(1, 2, 300, 128, 72), tiles)
    print("[no-alloc] causal path B=1 H=2 N=500", flush=True)
    _both("causal", None, make_tensors(1, 2, 500, 128, 73), tiles, causal=True)


def test_noalloc_rejects_more_rows_than_the_fixed_array():
    rows = cm.CM_NOALLOC_MAX_ROWS
    q = torch.zeros(1, 1, 64, 128, dtype=torch.bfloat16, device="cuda")
    args = cm.cm_attn_args(2, 1, rows // 2 + 64, 128, 0, 0, 0, 0.0, 1)
    p = q.data_ptr()  # the size check comes first: nothing is read or launched
    st = cm.library().cm_attn_bwd_noalloc(args, p, p, p, p, p, p, None, p, p, p, None)
    assert st == -6 and "rows" in cm.cm_last_error()
