"""Pins of the float64 attention oracle.

Reductions to independent implementations: torch's scaled_dot_product_attention
in float64 on the CPU (no mask, causal, boolean mask) with its autograd
backward, scipy's logsumexp, and central finite differences of the oracle's own
forward.  Invariants: rows of P sum to one, an empty row gives O = 0, lse = -inf
and no gradient, heads permute with their outputs.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import attention as oa
from oracle import masks as om
from workloads import WORKLOADS, make_metadata, make_tensors, metadata_from_segments


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _mask_fn(M):
    """mask_rows callback over a fixed dense mask M[b] (N x N)."""
    return lambda b, r0, r1: M[b][r0:r1]


def _sdpa(q, k, v, do, mask=None, causal=False):
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=None if mask is None else torch.tensor(mask), is_causal=causal)
    o.backward(torch.tensor(do))
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("kind", ["none", "causal", "random"])
def test_matches_sdpa_and_autograd(kind):
    B, H, N, d = 2, 3, 67, 16
    q, k, v, do = (_rand((B, H, N, d), s) for s in range(4))
    if kind == "none":
        M = np.ones((B, N, N), bool)
        ref = _sdpa(q, k, v, do)
    elif kind == "causal":
        M = np.broadcast_to(np.tril(np.ones((N, N), bool)), (B, N, N))
        ref = _sdpa(q, k, v, do, causal=True)
    else:
        M = np.random.default_rng(9).random((B, N, N)) < 0.3
        M[:, np.arange(N), np.arange(N)] = True          # no empty rows for SDPA
        ref = _sdpa(q, k, v, do, mask=M[:, None])
    dq, dk, dv, O, lse = oa.backward(q, k, v, do, _mask_fn(M))
    np.testing.assert_allclose(O, ref[0], atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(dq, ref[1], atol=1e-11, rtol=1e-9)
    np.testing.assert_allclose(dk, ref[2], atol=1e-11, rtol=1e-9)
    np.testing.assert_allclose(dv, ref[3], atol=1e-11, rtol=1e-9)
    # lse against scipy on the visible scaled scores
    for b in range(B):
        for h in range(H):
            S = q[b, h] @ k[b, h].T / math.sqrt(d)
            want = logsumexp(np.where(M[b], S, -np.inf), axis=1)
            np.testing.assert_allclose(lse[b, h], want, rtol=1e-12, atol=1e-12)


def test_finite_differences_with_empty_row():
    N, d = 9, 4
    rng = np.random.default_rng(3)
    q, k, v, do = (rng.standard_normal((1, 1, N, d)) for _ in range(4))
    M = rng.random((1, N, N)) < 0.5
    M[0, 4, :] = False                                    # an empty row
    M[0, 5, :] = True
    fn = _mask_fn(M)
    dq, dk, dv, O, lse = oa.backward(q, k, v, do, fn)

    def loss(qq, kk, vv):
        o, _ = oa.forward(qq, kk, vv, fn)
        return float(np.sum(o * do))

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = loss(args["q"], args["k"], args["v"])
            args[name] = xm
            fm = loss(args["q"], args["k"], args["v"])
            num[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=1e-7, rtol=1e-6, err_msg=name)
    # the empty row: O = 0, lse = -inf, zero dq row
    assert np.all(O[0, 0, 4] == 0) and lse[0, 0, 4] == -np.inf and np.all(dq[0, 0, 4] == 0)


def test_empty_row_contributes_nothing():
    N, d = 24, 8
    rng = np.random.default_rng(4)
    q, k, v, do = (rng.standard_normal((1, 1, N, d)) for _ in range(4))
    M = np.tril(np.ones((N, N), bool))[None].copy()
    M[0, 7, :] = False
    _, dk, dv, _, _ = oa.backward(q, k, v, do, _mask_fn(M))
    # the same computation with row 7's upstream gradient removed
    do2 = do.copy(); do2[0, 0, 7] = 0
    q2 = q.copy(); q2[0, 0, 7] = 123.0
    _, dk2, dv2, _, _ = oa.backward(q2, k, v, do2, _mask_fn(M))
    np.testing.assert_array_equal(dk, dk2)
    np.testing.assert_array_equal(dv, dv2)


def test_rows_of_p_sum_to_one():
    w = WORKLOADS["shared_prompt_tiny"]
    md = make_metadata(w)
    t = make_tensors(w.B, w.H, w.N, w.d, w.seed)
    q, k, v = (oa._f64(t[n])[0, 0] for n in ("q", "k", "v"))
    fn = om.row_block_fn(w.mask, md)
    O, lse = oa.forward_head(q, k, v, fn, 0)
    P = oa.probabilities(q, k, lse, fn(0, 0, w.N))
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)
    assert (P[~fn(0, 0, w.N)] == 0).all()


def test_head_permutation_equivariance():
    B, H, N, d = 1, 4, 40, 8
    q, k, v, do = (_rand((B, H, N, d), 10 + s) for s in range(4))
    md = metadata_from_segments(N, 0, 0, ("h",), [{"scalars": [17]}])
    fn = om.row_block_fn("hstu", md)
    dq, dk, dv, O, lse = oa.backward(q, k, v, do, fn)
    p = [2, 0, 3, 1]
    dq2, dk2, dv2, O2, lse2 = oa.backward(q[:, p], k[:, p], v[:, p], do[:, p], fn)
    for a, b_ in ((dq, dq2), (dk, dk2), (dv, dv2), (O, O2), (lse, lse2)):
        np.testing.assert_array_equal(a[:, p], b_)


def test_sampled_head_equals_full_backward():
    w = WORKLOADS["shared_prompt_tiny"]
    md = make_metadata(w)
    t = make_tensors(w.B, w.H, w.N, w.d, w.seed)
    q, k, v, do = (oa._f64(t[n])[0, 0] for n in ("q", "k", "v", "do"))
    fn = om.row_block_fn(w.mask, md)
    dq, dk, dv, O, lse = oa.backward_head(q, k, v, do, fn, 0, block=100)
    rows = [0, 63, 64, 130, 255]
    keys = [0, 5, 64, 191, 255]
    s = oa.sampled_head(q, k, v, do, fn, 0, rows, keys, block=77)
    np.testing.assert_allclose(s["O"], O[rows], atol=1e-13)
    np.testing.assert_allclose(s["dq"], dq[rows], atol=1e-12)
    np.testing.assert_allclose(s["dk"], dk[keys], atol=1e-12)
    np.testing.assert_allclose(s["dv"], dv[keys], atol=1e-12)


@pytest.mark.parametrize("mask", ["causal", "hstu", "shared_prompt", "retrieval"])
def test_tiles_head_equals_full_backward(mask):
    """The restricted computation (forward only for the rows that the chosen
    keys see) gives backward_head's values at those rows and keys."""
    from tests.test_oracle_masks import small_md
    md = small_md(mask, N=300, seed=3, B=2)
    t = make_tensors(2, 1, 300, 32, 77)
    fn = om.row_block_fn(mask, md)
    for b in range(2):
        q, k, v, do = (oa._f64(t[n])[b, 0] for n in ("q", "k", "v", "do"))
        dq, dk, dv, O, lse = oa.backward_head(q, k, v, do, fn, b, block=64, stored_o="bf16")
        rows = np.r_[0:40, 150:171, 290:300]
        keys = np.r_[0:3, 200:264, 299]
        s = oa.tiles_head(q, k, v, do, fn, b, rows, keys, block=50, stored_o="bf16")
        np.testing.assert_allclose(s["O"], O[rows], atol=1e-13)
        np.testing.assert_array_equal(np.isneginf(s["lse"]), np.isneginf(lse[rows]))
        fin = np.isfinite(lse[rows])
        np.testing.assert_allclose(s["lse"][fin], lse[rows][fin], atol=1e-13)
        np.testing.assert_allclose(s["dq"], dq[rows], atol=1e-12)
        np.testing.assert_allclose(s["dk"], dk[keys], atol=1e-12)
        np.testing.assert_allclose(s["dv"], dv[keys], atol=1e-12)
        # the row set it needs is exactly the rows that see a chosen key
        M = fn(b, 0, 300)
        seeing = oa.rows_seeing(fn, b, 300, keys, block=37)
        assert np.array_equal(seeing, np.nonzero(M[:, keys].any(axis=1))[0])
        s2 = oa.tiles_head(q, k, v, do, fn, b, rows, keys, block=50, stored_o="bf16", seeing=seeing)
        for n in ("dq", "dk", "dv"):
            np.testing.assert_array_equal(s2[n], s[n])


def test_row_partition_sums_to_full_backward():
    w = WORKLOADS["shared_prompt_tiny"]
    md = make_metadata(w)
    t = make_tensors(w.B, w.H, w.N, w.d, w.seed)
    q, k, v, do = (oa._f64(t[n])[0, 0] for n in ("q", "k", "v", "do"))
    fn = om.row_block_fn(w.mask, md)
    dq, dk, dv, O, lse = oa.backward_head(q, k, v, do, fn, 0)
    sdk, sdv = np.zeros_like(dk), np.zeros_like(dv)
    for r0, r1 in [(0, 50), (50, 64), (64, 200), (200, 256)]:
        pq, pk, pv, pO, pl = oa.backward_rows(q, k, v, do, fn, 0, r0, r1)
        np.testing.assert_allclose(pq, dq[r0:r1], atol=1e-12)
        np.testing.assert_allclose(pO, O[r0:r1], atol=1e-13)
        np.testing.assert_allclose(pl, lse[r0:r1], atol=1e-13)
        sdk += pk
        sdv += pv
    np.testing.assert_allclose(sdk, dk, atol=1e-11)
    np.testing.assert_allclose(sdv, dv, atol=1e-11)


def test_round_bf16_matches_torch_conversion():
    """The oracle's bf16 rounding (ties to even, through float32) against
    torch's float32 -> bfloat16 conversion, including exact ties."""
    import torch

    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(4096) * 10.0 ** rng.integers(-4, 4, 4096),
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5 - 2.0 ** -7, 0.0, -0.0, 65504.0])])
    x32 = x.astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oa.round_bf16(x32.astype(np.float64)), want)


def test_stored_o_bf16_changes_only_d():
    """stored_o="bf16" takes D from the bf16-rounded O.  When O is exactly a
    bf16 value (one visible key per row: O = that key's bf16 v row), both
    forms agree exactly; the sampled and the full backward agree with it on."""
    N, d = 12, 16
    rng = np.random.default_rng(6)
    q, k, v, do = (oa._f64(torch_bf16(rng.standard_normal((1, 1, N, d)))) for _ in range(4))
    fn = _mask_fn(np.eye(N, dtype=bool)[None])
    a = oa.backward(q, k, v, do, fn)
    b = oa.backward(q, k, v, do, fn, stored_o="bf16")
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    fn = _mask_fn(np.tril(np.ones((N, N), dtype=bool))[None])
    full = oa.backward_head(q[0, 0], k[0, 0], v[0, 0], do[0, 0], fn, 0, stored_o="bf16")
    s = oa.sampled_head(q[0, 0], k[0, 0], v[0, 0], do[0, 0], fn, 0, [0, 5, 11], [0, 7, 11], block=5, stored_o="bf16")
    np.testing.assert_allclose(s["dq"], full[0][[0, 5, 11]], atol=1e-12)
    np.testing.assert_allclose(s["dk"], full[1][[0, 7, 11]], atol=1e-12)
    exact = oa.backward_head(q[0, 0], k[0, 0], v[0, 0], do[0, 0], fn, 0)
    assert np.abs(exact[0] - full[0]).max() > 0  # the rounding of O does reach dq


def torch_bf16(x):
    import torch

    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)
