"""GPU tests of the spec-specialised preprocess (cm_spec_specialize).

The run-time compiled kernel carries the lowered program as a constant; its
descriptors must be bit-identical to the interpreting kernel's and to the
oracle's, for every mask family, packed batches, invalid metadata and the
full-size workloads (recorded oracle hashes).
"""
import hashlib
import json
import os

import numpy as np
import pytest
import torch

import runtime_metadata_attention_amd as cm
from runtime_metadata_attention_amd import specs
from oracle import descriptor as od
from oracle import masks as om
from tests.test_gpu_descriptor import GOLDEN, gpu_descriptor
from tests.test_oracle_masks import small_md
from tests.test_oracle_packed import packed_md
from workloads import WORKLOADS, make_metadata

pytestmark = pytest.mark.gpu

_SPECIALISED = {}


def specialised(mask):
    """One specialised spec per mask family for the whole module (compiled once)."""
    if mask not in _SPECIALISED:
        spec = cm.cm_spec_compile(specs.BY_MASK[mask])
        cm.cm_spec_specialize(spec)
        cm.cm_spec_specialize(spec)  # idempotent
        _SPECIALISED[mask] = spec
    return _SPECIALISED[mask]


CASES = [
    ("causal", 777, (128, 64, 128, 64), 1),
    ("hstu", 513, (64, 64, 64, 64), 2),
    ("shared_prompt", 333, (16, 80, 24, 8), 5),
    ("retrieval", 777, (128, 64, 128, 64), 7),
    ("retrieval", 450, (48, 40, 40, 48), 8),
]


@pytest.mark.parametrize("mask,N,tiles,seed", CASES)
def test_specialised_equals_interpreted_and_oracle(mask, N, tiles, seed):
    print(f"[specialise] {mask} N={N} tiles={tiles}", flush=True)
    md = small_md(mask, N=N, seed=seed, B=2)
    if seed == 8:
        md.refs[1, 1, 0] = 99  # an invalid sample too
    a, desc, _ = gpu_descriptor(mask, md, tiles)
    b, _, _ = gpu_descriptor(mask, md, tiles, spec=specialised(mask))
    assert np.array_equal(a, b)
    assert np.array_equal(b, od.build(mask, md, desc.K_r, desc.K_c, tiles))


def test_specialised_packed_batch():
    md = packed_md("shared_prompt", [150, 64, 300, 90], 4)
    a, desc, _ = gpu_descriptor("shared_prompt", md, (128, 64, 128, 64))
    b, _, _ = gpu_descriptor("shared_prompt", md, (128, 64, 128, 64), spec=specialised("shared_prompt"))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_specialised_full_size_bit_exact(name):
    w = WORKLOADS[name]
    md = make_metadata(w)
    gold = json.load(open(GOLDEN))[name]
    print(f"[specialise-full] {name}", flush=True)
    words, desc, _ = gpu_descriptor(w.mask, md, w.tiles, spec=specialised(w.mask))
    assert hashlib.sha256(words.tobytes()).hexdigest() == gold["sha256"]


def test_concurrent_specialise_and_build_on_one_spec():
    """Two threads specialise one spec while a third keeps building
    descriptors with it: one module is kept, and every descriptor (from the
    interpreting or the specialised kernel) is the oracle's."""
    import threading

    mask, N, tiles = "shared_prompt", 900, (128, 64, 128, 64)
    md = small_md(mask, N=N, seed=41, B=2)
    spec = cm.cm_spec_compile(specs.BY_MASK[mask])
    _, desc, _ = gpu_descriptor(mask, md, tiles, spec=spec)
    want = od.build(mask, md, desc.K_r, desc.K_c, tiles)
    errors, builds = [], []
    done = threading.Event()

    def specialise():
        try:
            cm.cm_spec_specialize(spec)
        except Exception as e:  # noqa: BLE001 -- reported below
            errors.append(e)

    def build():
        try:
            while not done.is_set() or not builds:
                words, _, _ = gpu_descriptor(mask, md, tiles, spec=spec)
                builds.append(np.array_equal(words, want))
        except Exception as e:  # noqa: BLE001
            errors.append(e)

    workers = [threading.Thread(target=specialise), threading.Thread(target=specialise)]
    builder = threading.Thread(target=build)
    builder.start()
    for t in workers:
        t.start()
    for t in workers:
        t.join()
    done.set()
    builder.join()
    assert not errors, errors
    assert builds and all(builds)
    words, _, _ = gpu_descriptor(mask, md, tiles, spec=spec)
    assert np.array_equal(words, want)
