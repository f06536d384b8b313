"""Pins for the oracle when N is not a multiple of P (uneven shards).

bembew.net "Ring Attention", "Implementation Considerations": a sequence
length that P does not divide needs padding or uneven partitioning.  The
oracle splits into shards whose sizes differ by at most one row, the first
N mod P shards one row longer.  Pinned by:

* the split equals ``numpy.array_split`` (a library routine) and covers every
  row once;
* the ring over uneven shards equals dense attention (itself pinned against
  torch's fp64 attention in test_oracle.py), for every resident subset and in
  any fold order;
* striped shards have exactly the contiguous sizes; the causal ring over
  uneven contiguous or striped shards equals dense causal attention;
* a planted split that drops the remainder rows is caught.
"""

import numpy as np
import pytest

import oracle
import oracle.ring as oring
from oracle import layouts


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("N,P", [(10, 3), (37, 5), (7, 7), (9, 2), (64, 6), (1000, 16), (12, 4)])
def test_block_bounds_match_array_split(N, P):
    bounds = oring.block_bounds(N, P)
    parts = np.array_split(np.arange(N), P)
    assert [(int(p[0]), int(p[-1]) + 1) for p in parts] == bounds
    sizes = [b - a for a, b in bounds]
    assert sum(sizes) == N and max(sizes) - min(sizes) <= 1
    assert sizes == layouts.block_sizes(P, N)
    assert all(sizes[j] == N // P + 1 for j in range(N % P))


@pytest.mark.parametrize("N,P", [(10, 3), (37, 5), (9, 2), (23, 4), (5, 5)])
def test_ring_uneven_equals_dense(N, P):
    q, k, v = _rand((2, 1, N, 6), 1, 2.0), _rand((2, 1, N, 6), 2, 2.0), _rand((2, 1, N, 6), 3)
    want = oracle.dense_attention(q, k, v)
    np.testing.assert_allclose(oracle.ring_attention(q, k, v, P), want, rtol=0, atol=1e-12)
    # a resident subset, stacked in the order given
    qb = [P - 1, 0] if P > 1 else [0]
    bounds = oring.block_bounds(N, P)
    sub = np.concatenate([want[..., bounds[i][0]:bounds[i][1], :] for i in qb], axis=-2)
    np.testing.assert_allclose(oracle.ring_attention(q, k, v, P, query_blocks=qb), sub, rtol=0, atol=1e-12)
    # any fold order
    rev = oracle.ring_attention(q, k, v, P, order=lambda i: list(range(P))[::-1])
    np.testing.assert_allclose(rev, want, rtol=0, atol=1e-12)


def test_ring_rejects_more_devices_than_rows():
    x = _rand((1, 1, 3, 4), 0)
    with pytest.raises(ValueError):
        oracle.ring_attention(x, x, x, 4)


@pytest.mark.parametrize("layout", ["contiguous", "striped"])
@pytest.mark.parametrize("N,P", [(10, 3), (37, 5), (26, 4), (9, 9)])
def test_causal_uneven_equals_dense_causal(layout, N, P):
    blocks = layouts.block_positions(layout, P, N)
    assert [len(b) for b in blocks] == layouts.block_sizes(P, N)
    flat = np.concatenate(blocks)
    assert sorted(flat.tolist()) == list(range(N))
    assert all(np.all(np.diff(b) > 0) for b in blocks)  # positions rise along each shard
    q, k, v = _rand((1, 2, N, 8), 4, 2.0), _rand((1, 2, N, 8), 5, 2.0), _rand((1, 2, N, 8), 6)
    pos = np.arange(N)
    want = oracle.dense_attention(q, k, v, q_pos=pos, k_pos=pos)
    ql, kl, vl = (layouts.to_layout(x, layout, P) for x in (q, k, v))
    got = oracle.ring_attention(ql, kl, vl, P, causal_layout=layout)
    np.testing.assert_allclose(layouts.from_layout(got, layout, P), want, rtol=0, atol=1e-12)


def test_striped_uneven_deals_round_robin():
    blocks = layouts.block_positions("striped", 4, 10)
    assert [b.tolist() for b in blocks] == [[0, 4, 8], [1, 5, 9], [2, 6], [3, 7]]
    blocks = layouts.block_positions("contiguous", 4, 10)
    assert [b.tolist() for b in blocks] == [[0, 1, 2], [3, 4, 5], [6, 7], [8, 9]]


def test_zigzag_needs_multiple_of_2P():
    with pytest.raises(ValueError):
        layouts.block_positions("zigzag", 3, 10)
    assert [len(b) for b in layouts.block_positions("zigzag", 3, 12)] == [4, 4, 4]


def test_planted_split_dropping_remainder_is_caught(monkeypatch):
    N, P = 11, 3

    def bad_bounds(n, p):
        b = n // p
        return [(j * b, (j + 1) * b) for j in range(p)]  # the last n mod p rows never visit

    q, k, v = _rand((1, 1, N, 4), 7), _rand((1, 1, N, 4), 8), _rand((1, 1, N, 4), 9)
    want = oracle.dense_attention(q, k, v)
    monkeypatch.setattr(oring, "block_bounds", bad_bounds)
    got = oracle.ring_attention(q, k, v, P)
    assert got.shape != want.shape or not np.allclose(got, want, atol=1e-6)
