"""Token-to-device layouts of the ring, for causal masking.

Oracle (test infrastructure only; see the package docstring).

Sources:
* aicassindra.com "Ring Attention, math", "Sharding the sequence": P
  contiguous blocks of b = N/P tokens, device i owns block i.
* same page, "Causal masking, load balance, and other wrinkles", and
  vibeengines.com "Ring attention, explained", "The causal-mask catch": a query
  attends only to keys at or before its own position; the striped split hands
  tokens to the devices in turn; the zig-zag split gives each device an early
  chunk together with the matching chunk counted from the end.

``positions(layout, P, b)`` returns pos[j, r], the position in the whole
sequence of row r of device j's shard.  A tensor "in layout order" holds
device j's shard as rows [j*b, (j+1)*b) of its sequence axis.

When N is not a multiple of P (bembew.net "Ring Attention", "Implementation
Considerations": padding or dynamic partitioning is needed), the shards are
uneven: ``block_positions(layout, P, N)`` lists each device's positions.  The
contiguous split gives the first N mod P devices one token more (the sizes
``numpy.array_split`` makes); handing tokens out in turn (striped) gives
exactly the same sizes.  The zig-zag split needs N to be a multiple of 2P.
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


def block_sizes(P: int, N: int) -> list[int]:
    """Rows of each device's shard: N // P, plus one for the first N mod P."""
    return [N // P + (1 if j < N % P else 0) for j in range(P)]


def block_positions(layout: str, P: int, N: int) -> list[np.ndarray]:
    """Positions held by each device, in row order, for any N >= P."""
    if N % P == 0:
        return list(positions(layout, P, N // P))
    sizes = block_sizes(P, N)
    if layout == "contiguous":
        starts = np.concatenate([[0], np.cumsum(sizes)])
        return [np.arange(starts[j], starts[j] + sizes[j]) for j in range(P)]
    if layout == "striped":
        return [j + P * np.arange(sizes[j]) for j in range(P)]
    if layout == "zigzag":
        raise ValueError("zig-zag needs N to be a multiple of 2P")
    raise ValueError(f"unknown layout {layout!r}")


def _perm(layout: str, P: int, n: int) -> np.ndarray:
    return np.concatenate(block_positions(layout, P, n))


def to_layout(x, layout: str, P: int):
    """Reorder the sequence axis (-2) of x from natural order to layout order."""
    return x[..., _perm(layout, P, x.shape[-2]), :]


def from_layout(x, layout: str, P: int):
    """Inverse of ``to_layout``."""
    n = x.shape[-2]
    perm = _perm(layout, P, n)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(n)
    return x[..., inv, :]
