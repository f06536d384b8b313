"""Backward pass of attention, dense and on the ring, in float64.

Oracle (test infrastructure only; see the package docstring).

Sources:
* vibeengines.com "Ring attention, explained", method step 6: the backward
  pass runs on the same ring; the key/value blocks travel with their gradient
  accumulators, so each device adds its share of dK and dV to the block it
  holds and keeps its own dQ.
* The gradients are those of the plain definition O = softmax(s Q K^T) V
  (aicassindra.com "Ring Attention, math", the identity section), written out
  with the standard derivatives of softmax: with P the attention weights,
    dV = P^T dO,   dP = dO V^T,   D_i = sum_j P_ij dP_ij = dO_i . O_i,
    dS = P * (dP - D),   dQ = s dS K,   dK = s dS^T Q.
* On the ring the weights of a visiting block are rebuilt from the running
  maximum and sum the forward kept: P_ij = exp(s_ij - L_i) with
  L_i = m_i + log l_i (the log of the softmax denominator).

Rows that see no key (possible only under a causal mask) have P = 0 and get
zero gradients, matching the forward's O = 0 for them.
"""

from __future__ import annotations

import math
from typing import Callable, Sequence

import numpy as np

from .attention import _as_f64
from .ring import block_bounds, ring_schedule


def _scores(q, k, scale, q_pos, k_pos):
    s = np.matmul(q, np.swapaxes(k, -1, -2)) * scale
    if q_pos is not None:
        s = np.where(np.asarray(k_pos)[None, :] > np.asarray(q_pos)[:, None], -np.inf, s)
    return s


def dense_attention_backward(q, k, v, do, scale: float | None = None, q_pos=None, k_pos=None):
    """(dQ, dK, dV) of O = softmax(scale Q K^T) V for the upstream gradient dO.

    q, do: [..., Nq, d]; k, v: [..., Nk, d].  With positions, keys after a
    query's position are masked (causal)."""
    q, k, v, do = (_as_f64(x) for x in (q, k, v, do))
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    s = _scores(q, k, scale, q_pos, k_pos)
    m = s.max(axis=-1, keepdims=True)
    none = np.isneginf(m)
    e = np.exp(s - np.where(none, 0.0, m))
    z = e.sum(axis=-1, keepdims=True)
    p = np.where(z > 0, e / np.where(z > 0, z, 1.0), 0.0)
    o = np.matmul(p, v)
    dv = np.matmul(np.swapaxes(p, -1, -2), do)
    dp = np.matmul(do, np.swapaxes(v, -1, -2))
    dd = (do * o).sum(axis=-1, keepdims=True)
    ds = p * (dp - dd)
    dq = scale * np.matmul(ds, k)
    dk = scale * np.matmul(np.swapaxes(ds, -1, -2), q)
    return dq, dk, dv


def fold_backward(q_blk, k_blk, v_blk, do_blk, lse, dd, scale, q_pos=None, k_pos=None):
    """One (resident query block, visiting block) pair of the ring backward.

    lse: [..., nq] = m + log l from the forward; dd: [..., nq] = rowsum(dO * O).
    Returns the contributions (dQ_i, dK_j, dV_j) of this pair."""
    s = _scores(q_blk, k_blk, scale, q_pos, k_pos)
    lse_safe = np.where(np.isneginf(lse), 0.0, lse)[..., None]
    p = np.where(np.isneginf(lse)[..., None], 0.0, np.exp(s - lse_safe))
    dv = np.matmul(np.swapaxes(p, -1, -2), do_blk)
    dp = np.matmul(do_blk, np.swapaxes(v_blk, -1, -2))
    ds = p * (dp - dd[..., None])
    dq = scale * np.matmul(ds, k_blk)
    dk = scale * np.matmul(np.swapaxes(ds, -1, -2), q_blk)
    return dq, dk, dv


def ring_attention_backward(
    q,
    k,
    v,
    do,
    P: int,
    query_blocks: Sequence[int] | None = None,
    scale: float | None = None,
    order: Callable[[int], Sequence[int]] | None = None,
    causal_layout: str | None = None,
):
    """The backward on the ring for the resident query blocks.

    q, do: [..., rows, d] -- the resident blocks' query rows and upstream
    gradients stacked in query_blocks order (the whole sequence when every
    block is resident); k, v: [..., N, d].  Each resident device i first runs
    the forward ring (for O and L = m + log l), then on step t folds block
    (i - t) mod P: its dQ_i grows locally and its share is added to the
    visiting block's travelling dK_j, dV_j.
    Returns dQ like q, and dK, dV like k, v holding the residents' shares
    (the full gradients when every block is resident)."""
    q, k, v, do = (_as_f64(x) for x in (q, k, v, do))
    n = k.shape[-2]
    bounds = block_bounds(n, P)
    if query_blocks is None:
        query_blocks = list(range(P))
    if order is None:
        order = lambda i: ring_schedule(P, i)  # noqa: E731
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    pos = None
    if causal_layout is not None:
        from .layouts import block_positions

        pos = block_positions(causal_layout, P, n)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    row0 = 0
    for i in query_blocks:
        a, b = bounds[i]
        rows = slice(row0, row0 + (b - a))
        row0 += b - a
        q_i, do_i = q[..., rows, :], do[..., rows, :]
        # the forward of this device: O_i and its final (m, l) give L and D
        o_i, st = _forward_block(q_i, k, v, i, order(i), scale, pos, bounds)
        lse = np.where(st.l > 0, st.m + np.log(np.where(st.l > 0, st.l, 1.0)), -np.inf)
        dd = (do_i * o_i).sum(axis=-1)
        for j in order(i):
            c0, c1 = bounds[j]
            qp, kp = (None, None) if pos is None else (pos[i], pos[j])
            gq, gk, gv = fold_backward(q_i, k[..., c0:c1, :], v[..., c0:c1, :], do_i, lse, dd, scale, qp, kp)
            dq[..., rows, :] += gq
            dk[..., c0:c1, :] += gk
            dv[..., c0:c1, :] += gv
    return dq, dk, dv


def _forward_block(q_i, k, v, i, blocks, scale, pos, bounds):
    """The forward loop of one resident block over ``blocks``: (O_i, final state)."""
    from .ring import finalize, fold, init_state

    state = init_state(q_i.shape[:-2], q_i.shape[-2], v.shape[-1])
    for j in blocks:
        c0, c1 = bounds[j]
        qp, kp = (None, None) if pos is None else (pos[i], pos[j])
        state = fold(state, q_i, k[..., c0:c1, :], v[..., c0:c1, :], scale, qp, kp)
    return finalize(state), state


def backward_rows(q, k, v, do, q_rows, k_rows, scale: float | None = None, row_chunk: int = 1024, pos=None):
    """Selected rows of (dQ, dK, dV) for one (batch, head) -- [N, d] inputs --
    for checking full-size runs the dense backward cannot hold in memory.

    dQ_i needs only row i: its softmax weights P_i, dP_i = dO_i V^T and
    D_i = dO_i . O_i.  dK_j and dV_j need column j of P and dS over every
    query row, so every row's log-sum-exp L_i and D_i are computed first in a
    streaming pass over ``row_chunk`` query rows at a time (same formulas as
    ``dense_attention_backward``: dV = P^T dO, dS = P * (dP - D),
    dQ = s dS K, dK = s dS^T Q).  With ``pos`` (the position of every row,
    queries and keys alike) keys after a query's position are masked.
    Returns (dq[len(q_rows), d], dk[len(k_rows), d], dv[len(k_rows), dv])."""
    q, k, v, do = (_as_f64(x) for x in (q, k, v, do))
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    n = q.shape[0]
    pos = None if pos is None else np.asarray(pos)

    def masked(s, qi, kj_idx):
        # -inf where the key comes after the query (positions of rows qi, keys kj_idx)
        if pos is None:
            return s
        return np.where(pos[kj_idx][None, :] > pos[qi][:, None], -np.inf, s)

    lse, dd = _lse_and_dd(q, k, v, do, scale, row_chunk, masked)
    kj = k[k_rows]
    dk = np.zeros((len(k_rows), q.shape[1]))
    dv = np.zeros((len(k_rows), v.shape[1]))
    # pass 2: the chosen key rows' dK, dV over every query row
    all_k = np.arange(k.shape[0])
    for a in range(0, n, row_chunk):
        qi = np.arange(a, min(a + row_chunk, n))
        p = np.exp(masked((q[a:a + row_chunk] @ kj.T) * scale, qi, k_rows) - lse[a:a + row_chunk, None])
        dpj = do[a:a + row_chunk] @ v[k_rows].T
        dsj = p * (dpj - dd[a:a + row_chunk, None])
        dv += p.T @ do[a:a + row_chunk]
        dk += scale * dsj.T @ q[a:a + row_chunk]
    # the chosen query rows' dQ
    s = masked((q[q_rows] @ k.T) * scale, q_rows, all_k)
    p = np.exp(s - lse[q_rows, None])
    dp = do[q_rows] @ v.T
    dq = scale * (p * (dp - dd[q_rows, None])) @ k
    return dq, dk, dv


def _lse_and_dd(q, k, v, do, scale, row_chunk, masked=lambda s, qi, kj: s):
    """Pass 1 of ``backward_rows``: every query row's L_i = m_i + log l_i and
    D_i = dO_i . O_i, ``row_chunk`` rows at a time.  (Every row sees at least
    its own key under a causal mask, so no row is empty.)"""
    n = q.shape[0]
    lse = np.empty(n)
    dd = np.empty(n)
    all_k = np.arange(k.shape[0])
    for a in range(0, n, row_chunk):
        qi = np.arange(a, min(a + row_chunk, n))
        s = masked((q[a:a + row_chunk] @ k.T) * scale, qi, all_k)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        lse[a:a + row_chunk] = (m + np.log(z))[:, 0]
        o = (e / z) @ v
        dd[a:a + row_chunk] = (do[a:a + row_chunk] * o).sum(axis=1)
    return lse, dd
