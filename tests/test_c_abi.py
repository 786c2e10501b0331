"""The C ABI driven from plain C (tests/c_driver.c), without the Python binding.

* CPU: include/compilemask.h compiles as C11 with every warning enabled, and
  the driver links against the library.
* GPU: the driver's descriptor equals the oracle's, and its outputs equal
  the Python binding's on the same inputs bit for bit (same kernels; this
  checks the C view of the structs and calls).
"""
import os
import struct
import subprocess

import numpy as np
import pytest
import torch

import runtime_metadata_attention_amd as cm
from runtime_metadata_attention_amd import specs
from oracle import descriptor as od
from oracle import masks as om
from tests.test_gpu_attention import run_gpu
from tests.test_oracle_masks import small_md
from workloads import make_tensors

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.dirname(cm.LIB_PATH)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_driver(out_dir):
    exe = os.path.join(out_dir, "c_driver")
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-O1", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c_driver.c"), "-L", LIB_DIR, "-lcompilemask",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{LIB_DIR}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_header_is_c_and_driver_links(tmp_path):
    assert os.access(build_driver(str(tmp_path)), os.X_OK)


@pytest.mark.gpu
def test_c_driver_matches_python_binding(tmp_path):
    mask, N, d, tiles = "shared_prompt", 300, 128, (128, 64, 128, 64)
    B, H = 2, 2
    md = small_md(mask, N=N, seed=8, B=B)
    t = make_tensors(B, H, N, d, 81)
    # metadata the device must flag: sample 0 claims more segments than the
    # capacity, sample 1 starts its first segment past the sequence end
    bad = md.copy()
    bad.n_seg[0] = md.seg_cap + 1
    bad.seg_bounds[1, 0] = N + 5
    want_err = [om.validate(bad, b) for b in range(B)]
    assert want_err[0] and want_err[1]
    text = specs.BY_MASK[mask].encode()
    job = tmp_path / "job.bin"
    with open(job, "wb") as f:
        f.write(struct.pack("<12i", B, H, N, d, md.n_scalars, md.seg_cap, md.n_refs, *tiles, len(text)))
        f.write(text)
        for a in (md.scalars, md.seg_bounds, md.n_seg, md.refs):
            f.write(np.ascontiguousarray(a, dtype=np.int32).tobytes())
        for n in ("q", "k", "v", "do"):
            f.write(t[n].contiguous().view(torch.int16).numpy().tobytes())
        f.write(struct.pack("<i", 1))
        for a in (bad.scalars, bad.seg_bounds, bad.n_seg, bad.refs):
            f.write(np.ascontiguousarray(a, dtype=np.int32).tobytes())
    exe = build_driver(str(tmp_path))
    res = tmp_path / "res.bin"
    print(f"[c-abi] {mask} B={B} H={H} N={N} d={d}", flush=True)
    r = subprocess.run([exe, str(job), str(res)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    raw = res.read_bytes()
    n = B * H * N * d
    outs = {}
    pos = 0
    for name in ("o", "dq", "dk", "dv"):
        outs[name] = torch.from_numpy(np.frombuffer(raw, np.int16, n, pos).copy()).view(torch.bfloat16)
        outs[name] = outs[name].reshape(B, H, N, d)
        pos += 2 * n
    outs["lse"] = torch.from_numpy(np.frombuffer(raw, np.float32, B * H * N, pos).copy()).reshape(B, H, N)
    pos += 4 * B * H * N
    spec = cm.cm_spec_compile(specs.BY_MASK[mask])
    desc = cm.Descriptor(spec, B, N, md.seg_cap, tiles)
    words = np.frombuffer(raw, np.uint32, desc.bytes // 4, pos)
    pos += desc.bytes
    flags = int(np.frombuffer(raw, np.uint32, 1, pos)[0])
    per = np.frombuffer(raw, np.uint32, B, pos + 4).tolist()
    bad_words = np.frombuffer(raw, np.uint32, desc.bytes // 4, pos + 4 + 4 * B)
    # the invalid batch: its error words through cm_desc_errors, its whole
    # descriptor through cm_desc_download, both against the oracle
    assert per == want_err, (per, want_err)
    assert flags == (want_err[0] | want_err[1])
    assert np.array_equal(bad_words, od.build(mask, bad, desc.K_r, desc.K_c, tiles))

    assert words.nbytes == desc.bytes
    assert np.array_equal(words, od.build(mask, md, desc.K_r, desc.K_c, tiles))
    ref = run_gpu(specs.BY_MASK[mask], md, t, tiles, spec=spec, desc=desc)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(outs[name], ref[name]), name


def test_run_bitmask_matches_the_run_definition(tmp_path):
    """The partial-tile run bitmask (per run and tile: two clamped element
    counts and a bit range) against the element-by-element definition of a
    run, exhaustively over runs [s, e) within 200 indices, every 64-wide
    tile and both lane halves (tests/run_bits_check.cpp, host code)."""
    exe = str(tmp_path / "run_bits_check")
    src = os.path.join(ROOT, "tests", "run_bits_check.cpp")
    cmd = [os.path.join(ROCM, "bin", "hipcc"), "-std=c++17", "-O1", "-x", "hip", "--cuda-host-only",
           "-I", os.path.join(ROOT, "include"), src, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe, "200"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
