"""Seeded synthetic workloads shared by the oracle and the GPU path.

This module only *draws* inputs: batch metadata (per-sample scalars, segment
boundaries, segment references) and the bf16 Q/K/V/dO tensors.  It holds no
part of the masking or attention arithmetic: it never decides which key a
query row may see.  Both sides (the CPU oracle and the HIP library) receive the
same arrays and compute from them independently.

Workloads follow the five synthetic mask settings measured for CompileMask
(CompileMask paper summary, section 4.1 "Experimental Setup": HSTU,
shared-prompt reward model, CLEAR-like multi-interval and causal masks at
synthetic lengths 1K-32K).  The CLEAR traces and the KuaiRand-1K logs are not
available, so ``retrieval4_32k`` (a 4-interval retrieval mask) and
``hstu_4k`` (synthetic history lengths) stand in for them.

Readings of underspecified draws (all integer ranges are inclusive):
  * ``hstu_4k``: one history length h ~ U[1024, 3840] per sample.
  * ``reward_model_32k``: P ~ U[4096, 16384]; R ~ U{4..16}; response r has
    length 64 + floor(w_r * (N - P - 64 R)) with w ~ Dirichlet(1,...,1); the
    rounding remainder goes to the last response.
  * ``retrieval4_32k``: g = 512; segment lengths ~ U[512, 2048] are drawn
    until they cover N - g; the last segment is truncated to the remainder.
    Segment 0 references nothing, segment 1 references {0}, segment j >= 2
    references two distinct segments drawn uniformly from {0..j-1}, ascending.
  * ``hstu_packed_64k`` (stands in for the KuaiRand-1K histories, which are
    packed variable-length sequences): sample lengths n ~ lognormal(ln 1024,
    1) floored and clipped to [64, 16384], drawn until they cover 65536 tokens
    (the last truncated to the remainder); per sample h = max(1, floor(u n)),
    u ~ U[0.25, 0.94], in the sample's coordinates.
  * Tensors: ``torch.Generator('cpu').manual_seed(seed)``; q, k, v, dO drawn in
    that order with ``randn(B, H, N, d)`` in float32, then rounded to bfloat16.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "Metadata",
    "Workload",
    "WORKLOADS",
    "make_workload",
    "make_metadata",
    "make_tensors",
    "metadata_from_segments",
    "pack_samples",
]


@dataclasses.dataclass
class Metadata:
    """Per-batch mask metadata, as int32 host arrays.

    scalars    [B, n_scalars]      named per-sample scalars (``scalar_names``)
    seg_bounds [B, seg_cap + 1]    segment s of sample b is
                                   [seg_bounds[b, s], seg_bounds[b, s + 1])
                                   for s < n_seg[b]; unused tail entries repeat
                                   the last bound
    n_seg      [B]                 number of segments per sample
    refs       [B, seg_cap, n_refs] referenced segment ids, -1 = none
    """

    B: int
    N: int
    scalars: np.ndarray
    seg_bounds: np.ndarray
    n_seg: np.ndarray
    refs: np.ndarray
    scalar_names: Tuple[str, ...] = ()
    # packed batches: [B + 1] first token of each sample, cu_seqlens[B] = N
    # (the B samples are laid end to end as one sequence of N tokens and each
    # sample's scalars and boundaries are in its own coordinates); None for a
    # padded batch of B sequences of N tokens
    cu_seqlens: Optional[np.ndarray] = None

    @property
    def seg_cap(self) -> int:
        return int(self.seg_bounds.shape[1] - 1)

    @property
    def n_refs(self) -> int:
        return int(self.refs.shape[2])

    @property
    def n_scalars(self) -> int:
        return int(self.scalars.shape[1])

    def scalar(self, name: str, b: int) -> int:
        return int(self.scalars[b, self.scalar_names.index(name)])

    def segments(self, b: int):
        """List of (start, end) of sample b's segments."""
        n = int(self.n_seg[b])
        sb = self.seg_bounds[b]
        return [(int(sb[s]), int(sb[s + 1])) for s in range(n)]

    def copy(self) -> "Metadata":
        return Metadata(self.B, self.N, self.scalars.copy(), self.seg_bounds.copy(),
                        self.n_seg.copy(), self.refs.copy(), tuple(self.scalar_names),
                        None if self.cu_seqlens is None else self.cu_seqlens.copy())


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    mask: str           # mask family: causal | shared_prompt | hstu | retrieval | ...
    B: int
    H: int
    N: int
    d: int
    seed: int
    tiles: Tuple[int, int, int, int]   # (fwd_q, fwd_k, bwd_k, bwd_q)
    seg_cap: int
    n_refs: int
    scalar_names: Tuple[str, ...]
    description: str
    packed: bool = False   # B = 1 packed sequence of N tokens holding many samples


_T128 = (128, 64, 128, 64)

WORKLOADS: Dict[str, Workload] = {
    "shared_prompt_tiny": Workload(
        "shared_prompt_tiny", "shared_prompt", 1, 1, 256, 64, 1001, (64, 64, 64, 64), 4, 0, ("P",),
        "prompt rows 0..63 causal; responses [64,128) [128,192) [192,256) see [0,64) u [s,i+1)"),
    "causal_8k": Workload(
        "causal_8k", "causal", 2, 16, 8192, 128, 1002, _T128, 0, 0, (),
        "row i sees [0,i+1)"),
    "hstu_4k": Workload(
        "hstu_4k", "hstu", 4, 8, 4096, 128, 1003, _T128, 0, 0, ("h",),
        "history rows i<h see [0,i+1); target rows see [0,h) u [i,i+1); h ~ U[1024,3840]"),
    "reward_model_32k": Workload(
        "reward_model_32k", "shared_prompt", 1, 16, 32768, 128, 1004, _T128, 16, 0, ("P",),
        "prompt P ~ U[4096,16384] causal; R ~ U{4..16} responses see [0,P) u [s,i+1)"),
    "retrieval4_32k": Workload(
        "retrieval4_32k", "retrieval", 1, 16, 32768, 128, 1005, _T128, 64, 2, ("g",),
        "prefix g=512 causal; segment rows see [0,g) u [s_j,i+1) u seg(r1) u seg(r2)"),
    "hstu_packed_64k": Workload(
        "hstu_packed_64k", "hstu", 1, 8, 65536, 128, 1006, _T128, 0, 0, ("h",),
        "packed HSTU batch: heavy-tailed sample lengths n ~ lognormal(ln 1024, 1) clipped to [64, 16384] "
        "filling 65536 tokens (the last truncated); h = floor(u n), u ~ U[0.25, 0.94]", packed=True),
}


def _empty_md(B: int, N: int, seg_cap: int, n_refs: int, scalar_names) -> Metadata:
    return Metadata(
        B=B, N=N,
        scalars=np.zeros((B, len(scalar_names)), np.int32),
        seg_bounds=np.zeros((B, seg_cap + 1), np.int32),
        n_seg=np.zeros((B,), np.int32),
        refs=np.full((B, seg_cap, n_refs), -1, np.int32),
        scalar_names=tuple(scalar_names),
    )


def metadata_from_segments(N: int, seg_cap: int, n_refs: int, scalar_names, per_sample) -> Metadata:
    """Build a Metadata from a list (one entry per sample) of dicts with keys
    ``scalars`` (list), ``bounds`` (list of n_seg+1 ints) and optionally
    ``refs`` (list of per-segment lists of referenced segment ids)."""
    B = len(per_sample)
    md = _empty_md(B, N, seg_cap, n_refs, scalar_names)
    for b, s in enumerate(per_sample):
        sc = list(s.get("scalars", []))
        md.scalars[b, : len(sc)] = sc
        bounds = list(s.get("bounds", []))
        if bounds:
            n = len(bounds) - 1
            if n > seg_cap:
                raise ValueError("more segments than seg_cap")
            md.n_seg[b] = n
            md.seg_bounds[b, : n + 1] = bounds
            md.seg_bounds[b, n + 1:] = bounds[-1]
        for j, rl in enumerate(s.get("refs", [])):
            for r, v in enumerate(rl):
                md.refs[b, j, r] = v
    return md


def pack_samples(samples) -> Metadata:
    """One packed-batch Metadata from one-sample Metadata objects (each with its
    own length N and the same seg_cap / n_refs / scalar names), laid end to end
    in the given order."""
    lens = [int(m.N) for m in samples]
    cu = np.zeros(len(samples) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    first = samples[0]
    return Metadata(
        B=len(samples), N=int(cu[-1]),
        scalars=np.concatenate([m.scalars[:1] for m in samples]).astype(np.int32),
        seg_bounds=np.concatenate([m.seg_bounds[:1] for m in samples]).astype(np.int32),
        n_seg=np.concatenate([m.n_seg[:1] for m in samples]).astype(np.int32),
        refs=np.concatenate([m.refs[:1] for m in samples]).astype(np.int32),
        scalar_names=tuple(first.scalar_names),
        cu_seqlens=cu,
    )


def _draw_packed_lengths(rng: np.random.Generator, T: int):
    lens = []
    while sum(lens) < T:
        n = int(np.clip(np.floor(rng.lognormal(np.log(1024.0), 1.0)), 64, 16384))
        lens.append(n)
    lens[-1] = T - sum(lens[:-1])
    return lens


def _draw_shared_prompt(rng: np.random.Generator, N: int, seg_cap: int):
    P = int(rng.integers(4096, 16384 + 1))
    R = int(rng.integers(4, 16 + 1))
    if R > seg_cap:
        raise ValueError("seg_cap too small")
    w = rng.dirichlet(np.ones(R))
    free = N - P - 64 * R
    lens = [64 + int(np.floor(w[r] * free)) for r in range(R)]
    lens[-1] += (N - P) - sum(lens)
    bounds = [P]
    for L in lens:
        bounds.append(bounds[-1] + L)
    assert bounds[-1] == N and min(lens) >= 64
    return {"scalars": [P], "bounds": bounds}


def _draw_retrieval(rng: np.random.Generator, N: int, g: int, seg_cap: int):
    lens = []
    total = N - g
    while sum(lens) < total:
        lens.append(int(rng.integers(512, 2048 + 1)))
    lens[-1] = total - sum(lens[:-1])
    if len(lens) > seg_cap:
        raise ValueError("seg_cap too small")
    bounds = [g]
    for L in lens:
        bounds.append(bounds[-1] + L)
    refs = []
    for j in range(len(lens)):
        if j == 0:
            refs.append([])
        elif j == 1:
            refs.append([0])
        else:
            pick = rng.choice(j, size=2, replace=False)
            refs.append(sorted(int(x) for x in pick))
    return {"scalars": [g], "bounds": bounds, "refs": refs}


def make_metadata(w: Workload, seed: Optional[int] = None) -> Metadata:
    """Seeded metadata for workload ``w`` (seed defaults to the workload's)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    N, B = w.N, w.B
    if w.name == "shared_prompt_tiny":
        return metadata_from_segments(N, w.seg_cap, w.n_refs, w.scalar_names,
                                      [{"scalars": [64], "bounds": [64, 128, 192, 256]}] * B)
    if w.packed and w.mask == "hstu":
        samples = []
        for n in _draw_packed_lengths(rng, N):
            m = _empty_md(1, n, w.seg_cap, w.n_refs, w.scalar_names)
            m.scalars[0, 0] = max(1, int(np.floor(rng.uniform(0.25, 0.94) * n)))
            samples.append(m)
        return pack_samples(samples)
    if w.mask == "causal":
        return _empty_md(B, N, w.seg_cap, w.n_refs, w.scalar_names)
    if w.mask == "hstu":
        md = _empty_md(B, N, w.seg_cap, w.n_refs, w.scalar_names)
        md.scalars[:, 0] = rng.integers(1024, 3840 + 1, size=B)
        return md
    if w.mask == "shared_prompt":
        return metadata_from_segments(N, w.seg_cap, w.n_refs, w.scalar_names,
                                      [_draw_shared_prompt(rng, N, w.seg_cap) for _ in range(B)])
    if w.mask == "retrieval":
        return metadata_from_segments(N, w.seg_cap, w.n_refs, w.scalar_names,
                                      [_draw_retrieval(rng, N, 512, w.seg_cap) for _ in range(B)])
    raise KeyError(w.name)


def make_tensors(B: int, H: int, N: int, d: int, seed: int, with_grad: bool = True):
    """bf16 q, k, v (and dO) drawn from N(0, 1) in float32, then rounded."""
    import torch

    g = torch.Generator("cpu").manual_seed(seed)
    names = ("q", "k", "v", "do") if with_grad else ("q", "k", "v")
    out = {}
    for n in names:
        out[n] = torch.randn(B, H, N, d, dtype=torch.float32, generator=g).to(torch.bfloat16)
    return out


def make_workload(name: str, seed: Optional[int] = None, with_tensors: bool = True):
    """Return (workload, metadata, tensors-or-None)."""
    w = WORKLOADS[name]
    md = make_metadata(w, seed)
    t = make_tensors(w.B, w.H, w.N, w.d, w.seed if seed is None else seed) if with_tensors else None
    return w, md, t
