"""Pins for the causal part of the oracle (a query sees keys at or before it).

* library routine: torch's float64 CPU scaled_dot_product_attention with
  is_causal=True;
* brute force in pure Python on tiny inputs;
* the ring over each layout (contiguous, striped, zig-zag) equals the dense
  causal result after undoing the layout permutation;
* the load-balance facts the pages state: a contiguous split leaves about half
  of the compute slots unused, striped and zig-zag splits even it out;
* a block a row cannot see leaves that row's state as it was.
"""

import math

import numpy as np
import pytest

import oracle
import oracle.ring as oring
from oracle import layouts


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_dense_causal_matches_library_sdpa():
    torch = pytest.importorskip("torch")
    g = torch.Generator().manual_seed(5)
    q, k, v = (torch.randn(2, 3, 48, 16, generator=g, dtype=torch.float64) for _ in range(3))
    want = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True).numpy()
    pos = np.arange(48)
    got = oracle.dense_attention(q.numpy(), k.numpy(), v.numpy(), q_pos=pos, k_pos=pos)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_dense_causal_brute_force():
    rng = np.random.default_rng(3)
    n, d = 6, 3
    q, k, v = rng.uniform(-2, 2, (n, d)), rng.uniform(-2, 2, (n, d)), rng.uniform(-2, 2, (n, 2))
    scale = 1 / math.sqrt(d)
    want = []
    for i in range(n):
        w = [math.exp(scale * math.fsum(q[i, c] * k[j, c] for c in range(d))) for j in range(i + 1)]
        z = math.fsum(w)
        want.append([math.fsum(w[j] * v[j, c] for j in range(i + 1)) / z for c in range(2)])
    pos = np.arange(n)
    np.testing.assert_allclose(oracle.dense_attention(q, k, v, q_pos=pos, k_pos=pos), want, atol=1e-13)


@pytest.mark.parametrize("layout", layouts.LAYOUTS)
@pytest.mark.parametrize("P", [1, 2, 3, 4])
def test_positions_are_a_permutation(layout, P):
    b = 6
    pos = layouts.positions(layout, P, b)
    assert sorted(pos.reshape(-1).tolist()) == list(range(P * b))
    x = _rand((1, P * b, 2), 1)
    np.testing.assert_array_equal(layouts.from_layout(layouts.to_layout(x, layout, P), layout, P), x)


def test_zigzag_and_striped_shapes():
    """Zig-zag: device j holds chunk j and its mirror 2P-1-j; striped: device j
    holds every P-th token starting at j (vibeengines.com, "The causal-mask
    catch")."""
    P, b = 4, 6
    z = layouts.positions("zigzag", P, b)
    h = b // 2
    for j in range(P):
        assert set(z[j, :h] // h) == {j} and set(z[j, h:] // h) == {2 * P - 1 - j}
    s = layouts.positions("striped", P, b)
    assert np.all(s % P == np.arange(P)[:, None])


@pytest.mark.parametrize("layout", layouts.LAYOUTS)
@pytest.mark.parametrize("P,b", [(1, 8), (2, 6), (4, 4), (3, 10)])
def test_ring_causal_equals_dense_causal(layout, P, b):
    n = P * b
    q, k, v = _rand((2, 1, n, 8), 7, 2.0), _rand((2, 1, n, 8), 8, 2.0), _rand((2, 1, n, 8), 9)
    pos = np.arange(n)
    want = oracle.dense_attention(q, k, v, q_pos=pos, k_pos=pos)
    ql, kl, vl = (layouts.to_layout(x, layout, P) for x in (q, k, v))
    got = oracle.ring_attention(ql, kl, vl, P, causal_layout=layout)
    np.testing.assert_allclose(layouts.from_layout(got, layout, P), want, rtol=0, atol=1e-12)
    # any fold order gives the same causal result too
    got2 = oracle.ring_attention(ql, kl, vl, P, causal_layout=layout, order=lambda i: list(range(P))[::-1])
    np.testing.assert_allclose(got2, got, rtol=0, atol=1e-12)


def _work_per_device(layout, P, b):
    pos = layouts.positions(layout, P, b)
    # visible (query, key) pairs of device i over the whole ring
    return np.array([sum(int((pos[j][None, :] <= pos[i][:, None]).sum()) for j in range(P)) for i in range(P)])


def test_contiguous_causal_leaves_about_half_idle():
    """Math page, causal section, and vibeengines.com: with contiguous blocks
    and a lockstep ring, about half of the compute slots do nothing; striped
    and zig-zag splits balance the work."""
    P, b = 8, 16
    w = _work_per_device("contiguous", P, b)
    idle = 1 - w.mean() / w.max()
    assert 0.4 < idle < 0.5  # exactly (P - 1) / (2 P) up to the diagonal blocks
    z = _work_per_device("zigzag", P, b)
    assert z.max() == z.min()  # zig-zag: every device does the same work
    s = _work_per_device("striped", P, b)
    assert (s.max() - s.min()) / s.max() < 2.0 / b + 1e-9  # one diagonal row of difference per row
    assert w.sum() == z.sum() == s.sum() == P * b * (P * b + 1) // 2


def test_invisible_block_leaves_state_unchanged():
    st = oracle.init_state((), 3, 2)
    st = oring.fold_scores(st, np.array([[1.0, 2.0], [0.5, -1.0], [3.0, 3.0]]), np.ones((2, 2)))
    masked = np.full((3, 2), -np.inf)
    st2 = oring.fold_scores(st, masked, np.ones((2, 2)) * 7)
    np.testing.assert_array_equal(st2.m, st.m)
    np.testing.assert_array_equal(st2.l, st.l)
    np.testing.assert_array_equal(st2.o, st.o)
    fresh = oracle.init_state((), 3, 2)
    st3 = oring.fold_scores(fresh, masked, np.ones((2, 2)))
    assert np.all(np.isneginf(st3.m)) and np.all(st3.l == 0) and np.all(st3.o == 0)


def test_planted_mask_mistake_is_caught(monkeypatch):
    """Masking keys at the query's own position too (>= instead of >) must fail
    the library pin."""
    torch = pytest.importorskip("torch")

    def bad_fold(state, q_blk, k_blk, v_blk, scale=None, q_pos=None, k_pos=None):
        q_blk, k_blk, v_blk = (np.asarray(x, dtype=np.float64) for x in (q_blk, k_blk, v_blk))
        s = q_blk @ np.swapaxes(k_blk, -1, -2) * (scale or 1 / math.sqrt(q_blk.shape[-1]))
        s = np.where(np.asarray(k_pos)[None, :] >= np.asarray(q_pos)[:, None], -np.inf, s)
        return oring.fold_scores(state, s, v_blk)

    monkeypatch.setattr(oring, "fold", bad_fold)
    g = torch.Generator().manual_seed(2)
    q, k, v = (torch.randn(1, 1, 16, 8, generator=g, dtype=torch.float64) for _ in range(3))
    want = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True).numpy()
    got = oracle.ring_attention(q.numpy(), k.numpy(), v.numpy(), 4, causal_layout="contiguous")
    assert not np.allclose(got, want, atol=1e-6)
