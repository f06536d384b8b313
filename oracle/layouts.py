"""Token-to-device layouts of the ring, for causal masking.

Oracle (test infrastructure only; see the package docstring).

Sources:
* aicassindra.com "Ring Attention, math", "Sharding the sequence": P
  contiguous blocks of b = N/P tokens, device i owns block i.
* same page, "Causal masking, load balance, and other wrinkles", and
  vibeengines.com "Ring attention, explained", "The causal-mask catch": a query
  attends only to keys at or before its own position; striped attention deals
  tokens to hosts round-robin; the zig-zag split gives each host one early
  chunk and its mirror-image late chunk.

``positions(layout, P, b)`` returns pos[j, r], the position in the whole
sequence of row r of device j's shard.  A tensor "in layout order" holds
device j's shard as rows [j*b, (j+1)*b) of its sequence axis.
"""

from __future__ import annotations

import numpy as np

LAYOUTS = ("contiguous", "striped", "zigzag")


def positions(layout: str, P: int, b: int) -> np.ndarray:
    j = np.arange(P)[:, None]
    r = np.arange(b)[None, :]
    if layout == "contiguous":
        return j * b + r
    if layout == "striped":  # token t goes to device t mod P, as its (t // P)-th row
        return r * P + j
    if layout == "zigzag":  # 2P chunks of b/2; device j holds chunks j and 2P-1-j
        if b % 2:
            raise ValueError("zig-zag needs an even block size")
        h = b // 2
        return np.where(r < h, j * h + r, (2 * P - 1 - j) * h + (r - h))
    raise ValueError(f"unknown layout {layout!r}")


def to_layout(x, layout: str, P: int):
    """Reorder the sequence axis (-2) of x from natural order to layout order."""
    n = x.shape[-2]
    perm = positions(layout, P, n // P).reshape(-1)
    return x[..., perm, :]


def from_layout(x, layout: str, P: int):
    """Inverse of ``to_layout``."""
    n = x.shape[-2]
    perm = positions(layout, P, n // P).reshape(-1)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(n)
    return x[..., inv, :]
