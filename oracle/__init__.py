"""CPU oracle for Ring Attention's per-step online-softmax fold.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path (no kernels, headers, helpers or constants) and imports nothing
from it.

Everything here is plain NumPy in float64, written from the pages:

* ``dense_attention`` -- the plain definition softmax(Q K^T / sqrt(d)) V
  ("Ring Attention, math" page, sections "Why one device runs out of room"
  and "The online-softmax identity that makes streaming legal").
* ``fold`` -- one application of the running (m, l, o) recurrence to one
  visiting block (same page, the per-query pseudo-code under the identity
  section; bembew.net "Conceptual Algorithm").
* ``ring_attention`` -- the naive per-device loop over P blocks in ring order
  (i - t) mod P, finished with o / l (math page, "The ring schedule" and
  "Accumulation math, step by step").
* ``ring_schedule`` -- the block a device holds at each step.
* ``block_bounds`` -- the rows of each device's block; when N is not a
  multiple of P the first N mod P blocks hold one row more (bembew.net
  "Implementation Considerations", load balancing).
* ``backward`` -- dQ, dK, dV: the dense gradients and the ring backward in
  which dK, dV accumulators travel with the blocks (vibeengines.com method
  step 6).
* ``layouts`` -- contiguous, striped and zig-zag token layouts and the causal
  positions they imply (math page "Causal masking, load balance, and other
  wrinkles"; vibeengines.com "The causal-mask catch").

Every function here is pinned (``tests/test_oracle.py``, ``test_oracle_causal.py``,
``test_oracle_ragged.py``, ``test_oracle_backward.py``) against values the
pages print (the worked two-block example), closed forms, a brute-force
pure-Python evaluation, a library routine (torch's fp64 CPU attention) and
invariants the pages state (order independence, P = 1).
"""

from . import backward, layouts
from .attention import dense_attention, dense_attention_rows
from .ring import (
    State,
    block_bounds,
    finalize,
    fold,
    init_state,
    ring_attention,
    ring_schedule,
)

__all__ = [
    "State",
    "backward",
    "block_bounds",
    "layouts",
    "dense_attention",
    "dense_attention_rows",
    "finalize",
    "fold",
    "init_state",
    "ring_attention",
    "ring_schedule",
]
