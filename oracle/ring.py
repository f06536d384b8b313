"""Naive blockwise ring loop with the online-softmax fold, in float64.

Oracle (test infrastructure only; see the package docstring).

Sources:
* aicassindra.com "Ring Attention, math":
  - "Sharding the sequence": P contiguous blocks of b = N/P rows; device i
    owns block i.
  - "The online-softmax identity ...": per query keep (m, l, o); for each
    incoming block take the new maximum m', rescale the old l and o by
    alpha = exp(m - m'), then add exp(s - m') and exp(s - m') v.
  - "The ring schedule": on step t device i holds the block of device
    (i - t) mod P; after P steps it has seen every block once.
  - "Accumulation math, step by step": start from (-inf, 0, 0) with the own
    block, fold P times, finish with O_i = o / l.
* bembew.net "Ring Attention", "Conceptual Algorithm": the same loop with
  m_new = max(m, rowmax S), alpha = exp(m - m_new), beta = exp(S - m_new).
* bembew.net "Implementation Considerations", load balancing: when N is not a
  multiple of P the shards cannot be equal; here the first N mod P devices
  hold one row more (block j starts at j (N // P) + min(j, N mod P)).

The steps below follow those passages in order, one block at a time, with no
tiling inside a block and no reordering.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Callable, Sequence

import numpy as np

from .attention import _as_f64


@dataclass
class State:
    """Running per-row state: m, l of shape [..., rows]; o of shape [..., rows, dv]."""

    m: np.ndarray
    l: np.ndarray
    o: np.ndarray

    def copy(self) -> "State":
        return State(self.m.copy(), self.l.copy(), self.o.copy())


def init_state(lead_shape: tuple, rows: int, dv: int) -> State:
    """(m, l, o) = (-inf, 0, 0) for every query row (math page, loop set-up)."""
    return State(
        m=np.full(lead_shape + (rows,), -np.inf, dtype=np.float64),
        l=np.zeros(lead_shape + (rows,), dtype=np.float64),
        o=np.zeros(lead_shape + (rows, dv), dtype=np.float64),
    )


def fold_scores(state: State, s: np.ndarray, v_blk: np.ndarray) -> State:
    """Fold one block of (already scaled) scores into the state.

    s: [..., rows, nk] scores of this block; v_blk: [..., nk, dv].
    Math page, per-query pseudo-code under the identity section:
      m' = max(m, max_j s_j); alpha = exp(m - m');
      l' = alpha l + sum_j exp(s_j - m'); o' = alpha o + sum_j exp(s_j - m') v_j.
    A block with no keys leaves the state as it is.
    """
    s = np.asarray(s, dtype=np.float64)
    v_blk = np.asarray(v_blk, dtype=np.float64)
    if s.shape[-1] == 0:
        return state.copy()
    m_new = np.maximum(state.m, s.max(axis=-1))
    # A row that has still seen no visible key (every score so far -inf, only
    # possible under a causal mask) keeps its state: alpha = 1, weights 0.
    none = np.isneginf(m_new)
    m_safe = np.where(none, 0.0, m_new)
    alpha = np.where(none, 1.0, np.exp(state.m - m_safe))  # exp(-inf) = 0 on the first block
    p = np.exp(s - m_safe[..., None])
    l_new = alpha * state.l + p.sum(axis=-1)
    o_new = alpha[..., None] * state.o + np.matmul(p, v_blk)
    return State(m_new, l_new, o_new)


def fold(state: State, q_blk, k_blk, v_blk, scale: float | None = None, q_pos=None, k_pos=None) -> State:
    """S = Q_i K_blk^T / sqrt(d), then ``fold_scores`` (math page loop body).
    With positions, keys after a query's position are masked to -inf (causal)."""
    q_blk = _as_f64(q_blk)
    k_blk = _as_f64(k_blk)
    v_blk = _as_f64(v_blk)
    if scale is None:
        scale = 1.0 / math.sqrt(q_blk.shape[-1])
    s = np.matmul(q_blk, np.swapaxes(k_blk, -1, -2)) * scale
    if q_pos is not None:
        s = np.where(np.asarray(k_pos)[None, :] > np.asarray(q_pos)[:, None], -np.inf, s)
    return fold_scores(state, s, v_blk)


def finalize(state: State) -> np.ndarray:
    """O = o / l after the last block (math page).  Rows never folded (l = 0)
    give 0: the pages leave 0/0 undefined and this is the convention chosen."""
    l = state.l[..., None]
    safe = np.where(l > 0, l, 1.0)
    return np.where(l > 0, state.o / safe, 0.0)


def block_bounds(N: int, P: int) -> list[tuple[int, int]]:
    """[start, stop) rows of each device's block: N // P rows each, one more
    for the first N mod P devices."""
    b, rem = divmod(N, P)
    starts = [j * b + min(j, rem) for j in range(P + 1)]
    return [(starts[j], starts[j + 1]) for j in range(P)]


def ring_schedule(P: int, i: int) -> list[int]:
    """Block held by device i on steps t = 0..P-1: (i - t) mod P (math page,
    "The ring schedule")."""
    return [(i - t) % P for t in range(P)]


def ring_attention(
    q,
    k,
    v,
    P: int,
    query_blocks: Sequence[int] | None = None,
    scale: float | None = None,
    order: Callable[[int], Sequence[int]] | None = None,
    return_states: bool = False,
    causal_layout: str | None = None,
):
    """Run the per-device loop for each resident query block.

    q, k, v: [..., N, d], the whole sequence, any N >= P (uneven blocks when
      N is not a multiple of P, see ``block_bounds``).
    query_blocks: which devices' query blocks to compute (default 0..P-1).
    order: maps a device index i to the sequence of blocks it folds
      (default: the ring schedule (i - t) mod P).  The math page's worked
      example and vibeengines.com method step 4 say the result does not depend
      on the order; tests use other orders to check exactly that.
    causal_layout: None for full attention, or "contiguous", "striped" or
      "zigzag": then q, k, v are in that layout's device order (see
      ``oracle.layouts``) and a query sees only keys at or before its position.
    Returns O for the resident blocks stacked along the row axis
    ([..., sum of their sizes, dv]); with ``return_states`` also the list,
    per resident block, of the state after every step.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    n = k.shape[-2]
    if not 1 <= P <= n:
        raise ValueError(f"need 1 <= P={P} <= N={n}")
    bounds = block_bounds(n, P)
    if query_blocks is None:
        query_blocks = range(P)
    if order is None:
        order = lambda i: ring_schedule(P, i)  # noqa: E731
    lead = q.shape[:-2]
    dv = v.shape[-1]
    pos = None
    if causal_layout is not None:
        from .layouts import block_positions

        pos = block_positions(causal_layout, P, n)
    outs = []
    all_states = []
    for i in query_blocks:
        q_i = q[..., bounds[i][0]:bounds[i][1], :]
        state = init_state(lead, q_i.shape[-2], dv)
        states = []
        for j in order(i):
            qp, kp = (None, None) if pos is None else (pos[i], pos[j])
            k_j = k[..., bounds[j][0]:bounds[j][1], :]
            v_j = v[..., bounds[j][0]:bounds[j][1], :]
            state = fold(state, q_i, k_j, v_j, scale, qp, kp)
            states.append(state.copy())
        outs.append(finalize(state))
        all_states.append(states)
    out = np.concatenate(outs, axis=-2)
    if return_states:
        return out, all_states
    return out
