"""Pins for the backward oracle (dQ, dK, dV), dense and on the ring.

* library routine: torch float64 autograd through scaled_dot_product_attention
  (full and is_causal);
* brute force: central finite differences of sum(O * dO) on tiny inputs;
* exact invariants: the rows of dS sum to zero, so the dK of all keys sums to
  zero; the weights of a row sum to one, so the dV of all keys sums to the
  dO of all queries; V with equal rows makes O constant, so dQ = dK = 0;
* the ring backward (vibeengines.com method step 6: dK, dV accumulators
  travel with the blocks) equals the dense gradients for even and uneven
  blocks, causal layouts and any fold order, and the residents' shares add
  up to the full dK, dV;
* planted mistakes are caught.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import backward as ob
from oracle import layouts

torch = pytest.importorskip("torch")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _autograd(q, k, v, do, causal=False, scale=None):
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [None, 0.3])
def test_dense_backward_matches_autograd(causal, scale):
    q, k, v, do = (_rand((2, 3, 24, 8), s, 1.5) for s in (1, 2, 3, 4))
    pos = np.arange(24) if causal else None
    got = ob.dense_attention_backward(q, k, v, do, scale, pos, pos)
    want = _autograd(q, k, v, do, causal, scale)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=0, atol=1e-12)


def test_dense_backward_finite_differences():
    q, k, v = _rand((5, 3), 5), _rand((4, 3), 6), _rand((4, 2), 7)
    do = _rand((5, 2), 8)
    dq, dk, dv = ob.dense_attention_backward(q, k, v, do)
    h = 1e-6

    def loss(q_, k_, v_):
        s = q_ @ k_.T / math.sqrt(3)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        return float(((p @ v_) * do).sum())

    for x, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=0, atol=1e-8)


def test_backward_invariants():
    q, k, v, do = (_rand((3, 16, 8), s) for s in (9, 10, 11, 12))
    dq, dk, dv = ob.dense_attention_backward(q, k, v, do)
    np.testing.assert_allclose(dk.sum(axis=-2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=-2), do.sum(axis=-2), atol=1e-12)
    vc = np.broadcast_to(_rand((3, 1, 8), 13), v.shape).copy()
    dq0, dk0, _ = ob.dense_attention_backward(q, k, vc, do)
    np.testing.assert_allclose(dq0, 0.0, atol=1e-12)
    np.testing.assert_allclose(dk0, 0.0, atol=1e-12)


@pytest.mark.parametrize("N,P", [(24, 4), (23, 4), (10, 3), (9, 9), (16, 1)])
def test_ring_backward_equals_dense(N, P):
    q, k, v, do = (_rand((2, 1, N, 6), s, 1.5) for s in (14, 15, 16, 17))
    want = ob.dense_attention_backward(q, k, v, do)
    got = ob.ring_attention_backward(q, k, v, do, P)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g, w, rtol=0, atol=1e-11)
    rev = ob.ring_attention_backward(q, k, v, do, P, order=lambda i: list(range(P))[::-1])
    for g, w in zip(rev, want):
        np.testing.assert_allclose(g, w, rtol=0, atol=1e-11)


@pytest.mark.parametrize("layout,N,P", [("contiguous", 24, 4), ("striped", 24, 4), ("zigzag", 24, 3),
                                        ("contiguous", 23, 5), ("striped", 19, 4)])
def test_ring_backward_causal_equals_dense(layout, N, P):
    q, k, v, do = (_rand((1, 2, N, 6), s, 1.5) for s in (18, 19, 20, 21))
    pos = np.arange(N)
    want = ob.dense_attention_backward(q, k, v, do, None, pos, pos)
    ql, kl, vl, dol = (layouts.to_layout(x, layout, P) for x in (q, k, v, do))
    got = ob.ring_attention_backward(ql, kl, vl, dol, P, causal_layout=layout)
    for g, w in zip(got, want):
        np.testing.assert_allclose(layouts.from_layout(g, layout, P), w, rtol=0, atol=1e-11)


def test_ring_backward_resident_shares_add_up():
    N, P = 22, 4
    q, k, v, do = (_rand((1, 1, N, 5), s) for s in (22, 23, 24, 25))
    full = ob.ring_attention_backward(q, k, v, do, P)
    bounds = oracle.block_bounds(N, P)
    dk_sum = np.zeros_like(k)
    dv_sum = np.zeros_like(v)
    for part in ([3, 1], [0], [2]):
        rows = np.concatenate([np.arange(*bounds[i]) for i in part])
        dq, dk, dv = ob.ring_attention_backward(q[..., rows, :], k, v, do[..., rows, :], P, query_blocks=part)
        np.testing.assert_allclose(dq, full[0][..., rows, :], rtol=0, atol=1e-12)
        dk_sum += dk
        dv_sum += dv
    np.testing.assert_allclose(dk_sum, full[1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv_sum, full[2], rtol=0, atol=1e-12)


@pytest.mark.parametrize("mistake", ["no_D", "dS_transposed_scale", "P_unnormalised", "dV_uses_dP"])
def test_planted_backward_mistakes_are_caught(monkeypatch, mistake):
    def bad(q_blk, k_blk, v_blk, do_blk, lse, dd, scale, q_pos=None, k_pos=None):
        s = ob._scores(q_blk, k_blk, scale, q_pos, k_pos)
        p = np.exp(s - lse[..., None])
        if mistake == "P_unnormalised":
            p = np.exp(s)
        dp = do_blk @ np.swapaxes(v_blk, -1, -2)
        ds = p * (dp - (0.0 if mistake == "no_D" else dd[..., None]))
        dv = np.swapaxes(dp if mistake == "dV_uses_dP" else p, -1, -2) @ do_blk
        dq = scale * ds @ k_blk
        dk = (1.0 if mistake == "dS_transposed_scale" else scale) * np.swapaxes(ds, -1, -2) @ q_blk
        return dq, dk, dv

    q, k, v, do = (_rand((1, 1, 12, 4), s, 1.5) for s in (26, 27, 28, 29))
    want = _autograd(q, k, v, do)
    monkeypatch.setattr(ob, "fold_backward", bad)
    got = ob.ring_attention_backward(q, k, v, do, 3)
    assert any(not np.allclose(g, w, atol=1e-6) for g, w in zip(got, want))


def test_backward_rows_matches_autograd():
    """The streaming row sampler against torch fp64 autograd on a sequence
    long enough to need several row chunks."""
    n, d = 300, 16
    q, k, v, do = (_rand((n, d), s, 1.2) for s in (31, 32, 33, 34))
    rows_q = np.array([0, 7, 150, 299])
    rows_k = np.array([1, 64, 200, 299])
    want = _autograd(q, k, v, do)
    for chunk in (1024, 64, 7):
        dq, dk, dv = ob.backward_rows(q, k, v, do, rows_q, rows_k, row_chunk=chunk)
        np.testing.assert_allclose(dq, want[0][rows_q], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk, want[1][rows_k], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv, want[2][rows_k], rtol=0, atol=1e-12)
    dq, dk, dv = ob.backward_rows(q, k, v, do, rows_q, rows_k, scale=0.4, row_chunk=50)
    want = _autograd(q, k, v, do, scale=0.4)
    np.testing.assert_allclose(dk, want[1][rows_k], rtol=0, atol=1e-12)


@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
def test_backward_rows_causal_matches_autograd(layout):
    """With positions: equals torch fp64 autograd through the causal attention
    of the sequence in position order, at the rows' positions."""
    P, b, d = 4, 40, 8
    n = P * b
    pos = layouts.positions(layout, P, b).reshape(-1)
    q, k, v, do = (_rand((n, d), s, 1.3) for s in (41, 42, 43, 44))
    # in position order the mask is plain is_causal; row r sits at position pos[r]
    order = np.argsort(pos)
    want_sorted = _autograd(q[order], k[order], v[order], do[order], causal=True)
    want = [np.empty_like(w) for w in want_sorted]
    for w, ws in zip(want, want_sorted):
        w[order] = ws
    rows = np.array([0, 11, 77, n - 1])
    dq, dk, dv = ob.backward_rows(q, k, v, do, rows, rows, row_chunk=33, pos=pos)
    np.testing.assert_allclose(dq, want[0][rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, want[1][rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, want[2][rows], rtol=0, atol=1e-12)


@pytest.mark.parametrize("mistake", ["no_D", "lse_without_log"])
def test_backward_rows_planted_mistakes_are_caught(monkeypatch, mistake):
    """Mistakes planted in the sampler's first pass fail the autograd comparison."""
    n, d = 120, 8
    q, k, v, do = (_rand((n, d), s) for s in (35, 36, 37, 38))
    rows = np.array([3, 90])
    want = _autograd(q, k, v, do)
    real = ob._lse_and_dd

    def bad(q_, k_, v_, do_, scale, chunk, masked=None):
        lse, dd = real(q_, k_, v_, do_, scale, chunk)
        if mistake == "no_D":
            return lse, np.zeros_like(dd)
        s = q_ @ k_.T * scale
        return s.max(axis=1) + (np.exp(s - s.max(axis=1, keepdims=True))).sum(axis=1), dd

    monkeypatch.setattr(ob, "_lse_and_dd", bad)
    dq, dk, dv = ob.backward_rows(q, k, v, do, rows, rows, row_chunk=32)
    assert not (np.allclose(dq, want[0][rows], atol=1e-6) and np.allclose(dk, want[1][rows], atol=1e-6)
                and np.allclose(dv, want[2][rows], atol=1e-6))
