"""Seeded sweep of small configurations against the oracle (GPU).

Each case draws from its own seed:
* the mask family and N (1 to 700);
* d (64 or 128), B and H (1 to 3);
* tile shapes the attention kernels take;
* a padded or a packed batch (packed: 1 to 4 samples, some of them empty);
* contiguous or [B, N, H, d] storage.

Descriptor words must equal the oracle's.  O, lse, dQ, dK and dV must meet
the parity bars of test_gpu_attention.
"""
import numpy as np
import pytest

from runtime_metadata_attention_amd import specs
from oracle import descriptor as od
from oracle import masks as om
from tests.test_gpu_attention import check_all, run_gpu
from tests.test_gpu_descriptor import explain, gpu_descriptor
from tests.test_oracle_masks import small_md
from tests.test_oracle_packed import packed_md
from workloads import make_tensors

pytestmark = pytest.mark.gpu

FAMILIES = ["causal", "hstu", "shared_prompt", "retrieval"]
TILES = [(128, 64, 128, 64), (64, 64, 64, 64), (128, 64, 64, 64), (64, 64, 128, 64)]


def draw_case(seed):
    rng = np.random.default_rng(10_000 + seed)
    mask = FAMILIES[int(rng.integers(len(FAMILIES)))]
    d = int(rng.choice([64, 128]))
    tiles = TILES[int(rng.integers(len(TILES)))]
    H = int(rng.integers(1, 4))
    strided = bool(rng.integers(2))
    # families with segments need room for a prompt or prefix and a few segments
    lo = 2 if mask in ("causal", "hstu") else 64
    if rng.integers(3) == 0:
        lengths = [int(rng.integers(lo, 300)) if rng.integers(4) else 0 for _ in range(int(rng.integers(1, 5)))]
        if sum(lengths) == 0:
            lengths[0] = lo
        md = packed_md(mask, lengths, seed=seed)
        B = 1
    else:
        B = int(rng.integers(1, 4))
        md = small_md(mask, N=int(rng.integers(lo, 701)), seed=seed, B=B)
    return mask, md, B, H, d, tiles, strided


@pytest.mark.parametrize("seed", range(64))
def test_random_small_configuration(seed):
    mask, md, B, H, d, tiles, strided = draw_case(seed)
    packed = om.is_packed(md)
    print(f"[sweep] seed={seed} {mask} N={md.N} B={B} H={H} d={d} tiles={tiles} "
          f"packed={md.B if packed else 0} strided={strided}", flush=True)
    words, desc, _ = gpu_descriptor(mask, md, tiles)
    want = od.build(mask, md, desc.K_r, desc.K_c, tiles)
    n_err = md.B if packed else None
    assert np.array_equal(words, want), explain(words, want, B, md.N, desc.K_r, desc.K_c, tiles, n_err=n_err)
    t = make_tensors(B, H, md.N, d, 500 + seed)
    if strided:
        t = {n: x.transpose(1, 2).contiguous().transpose(1, 2) for n, x in t.items()}
    out = run_gpu(specs.BY_MASK[mask], md, t, tiles)
    check_all(out, t, mask, md)
