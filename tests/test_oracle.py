"""Pins for the CPU oracle: it is checked against things other than itself.

* values printed by the math page's worked two-block example
  (tests/golden/worked_example.json) and their exact closed forms;
* a brute-force scalar evaluation of the softmax definition in pure Python
  (math.exp, math.fsum) on tiny inputs;
* a library routine: torch's float64 CPU scaled_dot_product_attention;
* closed forms (equal value rows, zero queries, convex hull);
* invariants the pages state: order independence (block size, ring start,
  random order), P = 1 is ordinary attention, the ring visits every block once;
* the wrong scheme the pages warn about (normalise each block then average)
  is caught;
* planted mistakes in the oracle's fold are caught by these pins.
"""

import json
import math
import os
import random

import numpy as np
import pytest

import oracle
import oracle.ring as oring

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")
PRINT_TOL = 5e-4  # the page prints three decimals


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _fold_worked_example():
    g = _golden()
    st = oracle.init_state((), 1, 1)
    steps = []
    for blk in g["blocks"]:
        m_old = st.m.copy()
        s = np.array([blk["s"]])
        v = np.array(blk["v"])[:, None]
        st = oring.fold_scores(st, s, v)
        alpha = float(np.exp(m_old - st.m)[0])
        p = np.exp(s - st.m[:, None])[0]
        steps.append(dict(m=float(st.m[0]), alpha=alpha, p=p, l=float(st.l[0]), o=float(st.o[0, 0])))
    out = float(oracle.finalize(st)[0, 0])
    return steps, out


def check_worked_example():
    g = _golden()
    steps, out = _fold_worked_example()
    for got, want in zip(steps, g["steps"]):
        assert abs(got["m"] - want["m"]) <= PRINT_TOL
        assert abs(got["alpha"] - want["alpha"]) <= PRINT_TOL
        assert np.all(np.abs(got["p"] - np.array(want["p"])) <= PRINT_TOL)
        assert abs(got["l"] - want["l"]) <= PRINT_TOL
        assert abs(got["o"] - want["o"]) <= PRINT_TOL
    assert abs(out - g["out"]) <= PRINT_TOL


def test_worked_example_printed_values():
    check_worked_example()


def test_worked_example_closed_forms():
    e = math.e
    # step A: m = 2, l = e^-1 + 1, o = e^-1*1 + 1*2
    l_a = math.exp(-1) + 1.0
    o_a = math.exp(-1) * 1 + 2.0
    # step B: alpha = e^-1, terms exp(3-3)=1 and exp(0-3)=e^-3
    l_b = math.exp(-1) * l_a + 1.0 + math.exp(-3)
    o_b = math.exp(-1) * o_a + 3.0 + 4.0 * math.exp(-3)
    steps, out = _fold_worked_example()
    assert steps[0]["l"] == pytest.approx(l_a, abs=1e-15)
    assert steps[0]["o"] == pytest.approx(o_a, abs=1e-15)
    assert steps[1]["l"] == pytest.approx(l_b, abs=1e-14)
    assert steps[1]["o"] == pytest.approx(o_b, abs=1e-14)
    assert out == pytest.approx(o_b / l_b, abs=1e-14)
    assert o_b / l_b == pytest.approx(2.6208871, abs=1e-7)
    # direct softmax over [1, 2, 3, 0] with values [1, 2, 3, 4]
    w = [e ** 1, e ** 2, e ** 3, e ** 0]
    direct = math.fsum(wi * vi for wi, vi in zip(w, [1, 2, 3, 4])) / math.fsum(w)
    assert out == pytest.approx(direct, abs=1e-14)
    # and the dense oracle on the same numbers (d = 1, scale 1 since s is given scaled)
    q = np.array([[1.0]])
    k = np.array([[1.0], [2.0], [3.0], [0.0]])
    v = np.array([[1.0], [2.0], [3.0], [4.0]])
    assert oracle.dense_attention(q, k, v, scale=1.0)[0, 0] == pytest.approx(direct, abs=1e-14)


def test_normalize_then_average_is_caught():
    """The math page's closing note: normalising per block and averaging is wrong."""
    g = _golden()
    per_block = []
    for blk in g["blocks"]:
        w = np.exp(np.array(blk["s"]))
        per_block.append(float((w * np.array(blk["v"])).sum() / w.sum()))
    wrong = sum(per_block) / len(per_block)
    assert wrong == pytest.approx(2.389, abs=PRINT_TOL)
    # the bf16 tolerance (2e-2 max-abs) would flag this scheme
    assert abs(wrong - g["out"]) > 0.2


def _brute_force(q, k, v, scale):
    """Softmax attention by the definition, scalar loops, exact summation."""
    nq, d = len(q), len(q[0])
    nk, dv = len(k), len(v[0])
    out = []
    for i in range(nq):
        s = [scale * math.fsum(q[i][c] * k[j][c] for c in range(d)) for j in range(nk)]
        w = [math.exp(x) for x in s]
        z = math.fsum(w)
        out.append([math.fsum(w[j] * v[j][c] for j in range(nk)) / z for c in range(dv)])
    return out


@pytest.mark.parametrize("nq,nk,d,dv,seed", [(1, 1, 1, 1, 0), (3, 5, 2, 3, 1), (8, 8, 4, 4, 2), (5, 7, 3, 2, 3)])
def test_dense_matches_brute_force(nq, nk, d, dv, seed):
    rng = random.Random(seed)
    q = [[rng.uniform(-2, 2) for _ in range(d)] for _ in range(nq)]
    k = [[rng.uniform(-2, 2) for _ in range(d)] for _ in range(nk)]
    v = [[rng.uniform(-2, 2) for _ in range(dv)] for _ in range(nk)]
    scale = 1.0 / math.sqrt(d)
    want = np.array(_brute_force(q, k, v, scale))
    got = oracle.dense_attention(np.array(q), np.array(k), np.array(v))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)
    # the ring loop on the same tiny input, every P dividing nk
    for P in [p for p in range(1, nk + 1) if nk % p == 0]:
        # the ring shards the sequence, so queries and keys have the same length
        if nq != nk:
            continue
        got_r = oracle.ring_attention(np.array(q), np.array(k), np.array(v), P)
        np.testing.assert_allclose(got_r, want, rtol=0, atol=1e-13)


def test_dense_matches_library_sdpa():
    torch = pytest.importorskip("torch")
    g = torch.Generator().manual_seed(11)
    q = torch.randn(2, 3, 40, 16, generator=g, dtype=torch.float64)
    k = torch.randn(2, 3, 56, 16, generator=g, dtype=torch.float64)
    v = torch.randn(2, 3, 56, 24, generator=g, dtype=torch.float64)
    want = torch.nn.functional.scaled_dot_product_attention(q, k, v).numpy()
    got = oracle.dense_attention(q.numpy(), k.numpy(), v.numpy())
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    got_s = oracle.dense_attention(q.numpy(), k.numpy(), v.numpy(), scale=0.3)
    want_s = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=0.3).numpy()
    np.testing.assert_allclose(got_s, want_s, rtol=0, atol=1e-12)


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8])
def test_ring_equals_dense(P):
    n = 24 * P
    q, k, v = _rand((2, 2, n, 8), 1), _rand((2, 2, n, 8), 2), _rand((2, 2, n, 8), 3)
    np.testing.assert_allclose(oracle.ring_attention(q, k, v, P), oracle.dense_attention(q, k, v), rtol=0, atol=1e-12)


def test_p1_is_ordinary_attention():
    """vibeengines.com, "At the extremes": with P = 1 the loop runs once."""
    q, k, v = _rand((1, 3, 50, 6), 4), _rand((1, 3, 50, 6), 5), _rand((1, 3, 50, 6), 6)
    out, states = oracle.ring_attention(q, k, v, 1, return_states=True)
    assert len(states) == 1 and len(states[0]) == 1
    np.testing.assert_allclose(out, oracle.dense_attention(q, k, v), rtol=0, atol=1e-13)


def test_order_independence():
    """Math page, worked example closing remark; vibeengines.com method step 4."""
    P, b = 6, 10
    q, k, v = _rand((1, 2, P * b, 5), 7, 3.0), _rand((1, 2, P * b, 5), 8, 3.0), _rand((1, 2, P * b, 5), 9)
    ref = oracle.ring_attention(q, k, v, P)
    rng = random.Random(0)
    for _ in range(5):
        perms = {i: rng.sample(range(P), P) for i in range(P)}
        got = oracle.ring_attention(q, k, v, P, order=lambda i: perms[i])
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    for off in range(P):  # a different ring start offset
        got = oracle.ring_attention(q, k, v, P, order=lambda i: [(i + off - t) % P for t in range(P)])
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    ascending = oracle.ring_attention(q, k, v, P, order=lambda i: list(range(P)))
    np.testing.assert_allclose(ascending, ref, rtol=0, atol=1e-12)
    # block size: the same sequence cut into a different number of blocks
    for P2 in (1, 2, 3, 12):
        np.testing.assert_allclose(oracle.ring_attention(q, k, v, P2), ref, rtol=0, atol=1e-12)


def test_subset_of_query_blocks():
    P, b = 4, 16
    q, k, v = _rand((1, 1, P * b, 8), 10), _rand((1, 1, P * b, 8), 11), _rand((1, 1, P * b, 8), 12)
    full = oracle.dense_attention(q, k, v)
    got = oracle.ring_attention(q, k, v, P, query_blocks=[2, 0])
    np.testing.assert_allclose(got[..., :b, :], full[..., 2 * b:3 * b, :], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[..., b:, :], full[..., :b, :], rtol=0, atol=1e-12)
    rows = np.array([5, 17, 63])
    np.testing.assert_allclose(oracle.dense_attention_rows(q, k, v, rows), full[..., rows, :], rtol=0, atol=1e-13)


def test_per_step_state_meaning():
    """After folding blocks B_0..B_t: m is the max score seen, l * e^m is the
    sum of e^s seen, and o / l is attention over the keys seen so far."""
    P, b, d = 4, 8, 4
    q, k, v = _rand((1, 1, P * b, d), 13, 2.0), _rand((1, 1, P * b, d), 14, 2.0), _rand((1, 1, P * b, d), 15)
    _, states = oracle.ring_attention(q, k, v, P, return_states=True)
    scale = 1 / math.sqrt(d)
    for i in range(P):
        qi = q[..., i * b:(i + 1) * b, :]
        seen = []
        for t, st in enumerate(states[i]):
            j = (i - t) % P
            seen.extend(range(j * b, (j + 1) * b))
            s = (qi @ np.swapaxes(k[..., seen, :], -1, -2)) * scale
            np.testing.assert_allclose(st.m, s.max(-1), rtol=0, atol=1e-13)
            np.testing.assert_allclose(st.l * np.exp(st.m), np.exp(s).sum(-1), rtol=1e-13)
            np.testing.assert_allclose(st.o / st.l[..., None], oracle.dense_attention(qi, k[..., seen, :], v[..., seen, :]), atol=1e-13)


def test_closed_forms():
    n, d = 32, 8
    k = _rand((1, 1, n, d), 16)
    q = _rand((1, 1, n, d), 17)
    row = _rand((d,), 18)
    v_same = np.broadcast_to(row, (1, 1, n, d)).copy()
    np.testing.assert_allclose(oracle.ring_attention(q, k, v_same, 4), np.broadcast_to(row, (1, 1, n, d)), atol=1e-13)
    v = _rand((1, 1, n, d), 19)
    zero_q = np.zeros_like(q)
    np.testing.assert_allclose(oracle.ring_attention(zero_q, k, v, 4), np.broadcast_to(v.mean(-2, keepdims=True), (1, 1, n, d)), atol=1e-13)
    out = oracle.ring_attention(q * 4, k, v, 4)
    assert np.all(out <= v.max(-2, keepdims=True) + 1e-12) and np.all(out >= v.min(-2, keepdims=True) - 1e-12)


def test_empty_block_and_unfolded_rows():
    st = oracle.init_state((1,), 3, 2)
    st2 = oring.fold_scores(st, np.zeros((1, 3, 0)), np.zeros((1, 0, 2)))
    assert np.all(np.isneginf(st2.m)) and np.all(st2.l == 0) and np.all(st2.o == 0)
    assert np.all(oracle.finalize(st2) == 0)


@pytest.mark.parametrize("P", [1, 2, 5, 16, 17, 64])
def test_ring_schedule_is_a_ring(P):
    """Math page, "The ring schedule": each device sees every block once, and
    each step is one send to i+1 and one receive from i-1 per device."""
    for i in range(P):
        assert sorted(oracle.ring_schedule(P, i)) == list(range(P))
        assert oracle.ring_schedule(P, i)[0] == i  # starts with its own block
    for t in range(P):
        held = [oracle.ring_schedule(P, i)[t] for i in range(P)]
        assert sorted(held) == list(range(P))
        if t + 1 < P:
            nxt = [oracle.ring_schedule(P, i)[t + 1] for i in range(P)]
            assert all(nxt[i] == held[(i - 1) % P] for i in range(P))


# ---------------------------------------------------------------------------
# Planted mistakes: each mutant replaces the oracle's fold and must fail a pin.


def _mutant_no_alpha_on_l(state, s, v):
    m_new = np.maximum(state.m, s.max(-1))
    a = np.exp(state.m - m_new)
    p = np.exp(s - m_new[..., None])
    return oring.State(m_new, state.l + p.sum(-1), a[..., None] * state.o + p @ v)


def _mutant_wrong_alpha_sign(state, s, v):
    m_new = np.maximum(state.m, s.max(-1))
    a = np.exp(np.where(np.isinf(state.m), -np.inf, m_new - state.m))
    p = np.exp(s - m_new[..., None])
    return oring.State(m_new, a * state.l + p.sum(-1), a[..., None] * state.o + p @ v)


def _mutant_block_max(state, s, v):
    m_new = s.max(-1)  # forgets the running max
    a = np.exp(np.minimum(state.m - m_new, 0.0))
    p = np.exp(s - m_new[..., None])
    return oring.State(m_new, a * state.l + p.sum(-1), a[..., None] * state.o + p @ v)


def _mutant_transposed_v(state, s, v):
    m_new = np.maximum(state.m, s.max(-1))
    a = np.exp(state.m - m_new)
    p = np.exp(s - m_new[..., None])
    vt = np.swapaxes(v, -1, -2) if v.shape[-1] == v.shape[-2] else v[..., ::-1, :]
    return oring.State(m_new, a * state.l + p.sum(-1), a[..., None] * state.o + p @ vt)


@pytest.mark.parametrize("mutant", [_mutant_no_alpha_on_l, _mutant_wrong_alpha_sign, _mutant_block_max, _mutant_transposed_v])
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(oring, "fold_scores", mutant)
    caught = 0
    try:
        check_worked_example()
    except AssertionError:
        caught += 1
    P, b = 4, 8
    q, k, v = _rand((1, 1, P * b, 8), 20, 3.0), _rand((1, 1, P * b, 8), 21, 3.0), _rand((1, 1, P * b, 8), 22)
    got = oracle.ring_attention(q, k, v, P)
    if not np.allclose(got, oracle.dense_attention(q, k, v), atol=1e-9):
        caught += 1
    assert caught >= 1
