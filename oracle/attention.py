"""Dense softmax attention in float64 -- the plain definition the ring reaches.

Oracle (test infrastructure only; see the package docstring).

Source: aicassindra.com "Ring Attention, math", section "Why one device runs
out of room" (scores S = Q K^T / sqrt(d_k)) and section "The online-softmax
identity that makes streaming legal" (the output of a query is the
softmax-weighted sum of the values; subtracting any constant m, taken as the
row maximum, leaves the ratio unchanged).  The same page's worked example
closes with the direct softmax over all four scores, and vibeengines.com
"Ring attention, explained", method step 4, says the ring result equals full
attention up to floating-point rounding.  So the reference result is this
function.
"""

from __future__ import annotations

import math

import numpy as np


def _as_f64(x) -> np.ndarray:
    """Exact upcast to float64 (bf16 and fp32 values are representable)."""
    if hasattr(x, "detach"):  # a torch tensor: read its exact values
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def dense_attention(q, k, v, scale: float | None = None, row_chunk: int = 1024, q_pos=None,
                    k_pos=None) -> np.ndarray:
    """O = softmax(Q K^T * scale) V for every leading (batch, head) index.

    q: [..., Nq, d], k: [..., Nk, d], v: [..., Nk, dv] (leading dims equal).
    scale defaults to 1/sqrt(d) (the pages' 1/sqrt(d_k)).  The row maximum is
    subtracted before exp, which the identity section shows cancels in the
    ratio; it only keeps exp in range.  Computed in float64, ``row_chunk``
    query rows at a time so memory stays bounded; chunking rows does not change
    any row's arithmetic.

    With ``q_pos`` [Nq] and ``k_pos`` [Nk] (sequence positions) the attention
    is causal: a query sees only keys at or before its own position (math
    page, "Causal masking, load balance, and other wrinkles").  A row that sees
    no key at all gives 0.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nq = q.shape[-2]
    out = np.empty(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
    kt = np.swapaxes(k, -1, -2)
    causal = q_pos is not None
    if causal:
        q_pos = np.asarray(q_pos)
        k_pos = np.asarray(k_pos)
    for r0 in range(0, nq, row_chunk):
        r1 = min(nq, r0 + row_chunk)
        s = np.matmul(q[..., r0:r1, :], kt) * scale  # [..., rows, Nk]
        if causal:
            s = np.where(k_pos[None, :] > q_pos[r0:r1, None], -np.inf, s)
            mx = s.max(axis=-1, keepdims=True)
            p = np.exp(s - np.where(np.isneginf(mx), 0.0, mx))
            z = p.sum(axis=-1, keepdims=True)
            out[..., r0:r1, :] = np.matmul(p, v) / np.where(z > 0, z, 1.0)
            continue
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        out[..., r0:r1, :] = np.matmul(p, v) / p.sum(axis=-1, keepdims=True)
    return out


def dense_attention_rows(q, k, v, rows, scale: float | None = None) -> np.ndarray:
    """Dense attention for a chosen subset of query rows only.

    q: [..., Nq, d]; rows: 1-D integer index array into the Nq axis.  Each
    output row depends only on its own query row, so this is exactly the
    corresponding rows of ``dense_attention(q, k, v)``.  Used to check
    outputs of full-size runs the oracle cannot compute whole.
    """
    rows = np.asarray(rows, dtype=np.int64)
    if hasattr(q, "detach"):  # pick the rows before the float64 copy
        import torch

        q = q[..., torch.from_numpy(rows).to(q.device), :]
    else:
        q = np.asarray(q)[..., rows, :]
    return dense_attention(q, k, v, scale=scale)
