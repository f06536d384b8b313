"""The ring's hand-off (the stand-in for the send to i + 1 / receive from
i - 1 of the math page's "Accumulation math, step by step", where a device
waits for the transfer before it takes the next block) under stress.

* RA_DEBUG_POISON=1 fills every double-buffer slot with NaN right after the
  fold that reads it: a refill ordered before that fold has finished, or a
  fold that starts before its copy has landed, puts NaN into the output.
* RA_DEBUG_DELAY_US holds the side stream before every hand-off, so a fold
  that does not wait for its copy reads the block of two steps earlier.

Each mode must give the output of the plain run bit for bit, on the rotated
hand-off (every block resident in ring order: the bf16 fold writes the next
step's slot itself, other dtypes use two contiguous copies per tensor) and on
the block-by-block one (a subset or another order of resident blocks, uneven
blocks).  The hand-offs are also compared with each other.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads  # noqa: E402
from tests.helpers import check_output, to64  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    import blockwise_online_softmax_fold_amd as ra

    ra.load()
    return ra


def _say(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _resident_q(q_all, N, P, blocks):
    bounds = oracle.block_bounds(N, P)
    return torch.cat([q_all[:, :, bounds[i][0]:bounds[i][1]] for i in blocks], dim=2).contiguous()


# (dtype, B, H, N, d, P, query_blocks): rotated path first, then block by block
CASES = [
    ("bf16", 1, 4, 8192, 128, 8, None),
    ("bf16", 2, 2, 4096, 256, 4, None),
    ("f32", 1, 2, 2048, 64, 4, None),
    ("bf16", 1, 4, 8192 + 13, 128, 8, (7, 2, 5)),
    ("bf16", 1, 3, 6000, 64, 5, (4, 3, 2, 1, 0)),
    ("f32", 1, 2, 1500 + 3, 64, 6, (0, 5)),
]


def _ids(c):
    dt, B, H, N, d, P, qb = c
    return f"{dt}-B{B}H{H}N{N}d{d}P{P}-{'rotated' if qb is None else 'blocks' + ''.join(map(str, qb))}"


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
@pytest.mark.parametrize("mode", ["poison", "delay", "poison+delay"])
def test_handoff_hazard_modes_are_bitwise_equal(ra, monkeypatch, case, mode):
    dt, B, H, N, d, P, qb = case
    _say(f"hand-off {mode} {_ids(case)}")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    q_all, k, v = workloads.make_small(B, H, N, d, tdt, seed=N + P + d)
    blocks = list(range(P)) if qb is None else list(qb)
    q = _resident_q(q_all, N, P, blocks)
    plain = ra.ra_ring_forward(q, k, v, P, query_blocks=qb)
    torch.cuda.synchronize()
    if "poison" in mode:
        monkeypatch.setenv("RA_DEBUG_POISON", "1")
    if "delay" in mode:
        monkeypatch.setenv("RA_DEBUG_DELAY_US", "3000")
    got = ra.ra_ring_forward(q, k, v, P, query_blocks=qb)
    torch.cuda.synchronize()
    assert torch.isfinite(got).all(), "a poisoned slot reached the output"
    assert torch.equal(got, plain)
    # the plain run itself is right
    ref = oracle.ring_attention(to64(q_all), to64(k), to64(v), P, query_blocks=blocks)
    check_output(plain, ref, dt, "plain ring")


# (dtype, B, H, N, d, P): every block resident in ring order
FUSED = [
    ("bf16", 1, 4, 8192, 128, 8),
    ("bf16", 1, 2, 8 * 1000, 128, 8),   # ragged last tile (1000 = 15 x 64 + 40)
    ("bf16", 2, 3, 4 * 100, 128, 4),    # a block shorter than a workgroup's 256 rows
    ("bf16", 1, 2, 6 * 640, 64, 6),
    ("bf16", 2, 2, 4096, 256, 4),       # padded LDS rows: duplicated units written twice
    ("bf16", 1, 1, 66 * 64, 128, 66),   # two launches per step (more than 64 residents)
]


@pytest.mark.parametrize("case", FUSED, ids=[f"{c[0]}-B{c[1]}H{c[2]}N{c[3]}d{c[4]}P{c[5]}" for c in FUSED])
@pytest.mark.parametrize("mode", ["plain", "poison"])
def test_fused_hand_off_equals_side_stream_copies(ra, monkeypatch, case, mode):
    """With every block resident (bf16, no mask) the fold writes the block it
    visits into the next step's slot itself; RA_HANDOFF_COPY=1 moves it with
    the side-stream copies instead.  The folds read the same bytes either way,
    so the outputs are equal bit for bit; with RA_DEBUG_POISON the slot a fold
    has read is NaN until the next fold overwrites it, so a tile the fused
    hand-off misses shows up as NaN."""
    dt, B, H, N, d, P = case
    _say(f"fused vs copied hand-off ({mode}) {dt} B{B} H{H} N{N} d{d} P{P}")
    q, k, v = workloads.make_small(B, H, N, d, torch.bfloat16, seed=N + 7 * P + d)
    if mode == "poison":
        monkeypatch.setenv("RA_DEBUG_POISON", "1")
    fused = ra.ra_ring_forward(q, k, v, P)
    torch.cuda.synchronize()
    monkeypatch.setenv("RA_HANDOFF_COPY", "1")
    copied = ra.ra_ring_forward(q, k, v, P)
    torch.cuda.synchronize()
    assert torch.isfinite(fused).all(), "a poisoned slot reached the output"
    assert torch.equal(fused, copied)
    if mode == "plain":
        ref = oracle.ring_attention(to64(q), to64(k), to64(v), P)
        check_output(fused, ref, dt, "fused hand-off ring")


def test_poison_is_seen_when_a_slot_is_read_after_it(ra, monkeypatch):
    """The poison check can fail: folding a poisoned slot by hand (the fold
    reads what the hand-off left after the poison) gives NaN.  A P = 3 ring
    poisons slot 0 after step 1 and never refills it; reading that workspace
    slot afterwards must show the NaN pattern."""
    _say("poison pattern present after the last reader, bf16 B1 H2 N768 d64 P3")
    B, H, N, d, P = 1, 2, 768, 64, 3
    q, k, v = workloads.make_small(B, H, N, d, torch.bfloat16, seed=3)
    nbytes = ra.ra_ring_workspace_bytes(torch.bfloat16, B, H, N, d, P, P)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    monkeypatch.setenv("RA_DEBUG_POISON", "1")
    ra.ra_ring_forward(q, k, v, P, workspace=ws)
    torch.cuda.synchronize()
    words = ws.view(torch.int32)
    assert int((words == 0x7FC07FC0).sum()) > 0


@pytest.mark.parametrize("dt,B,H,N,d,P", [
    ("bf16", 1, 4, 8192, 128, 8),
    ("bf16", 2, 2, 8192, 256, 16),
    ("f32", 1, 2, 2048, 64, 4),
])
def test_rotated_and_block_by_block_hand_off_agree(ra, dt, B, H, N, d, P):
    """Every block resident in ring order takes the rotated hand-off; the same
    residents in reversed order take the block-by-block one.  Each row's
    arithmetic is the same, so after undoing the permutation of rows the two
    outputs are equal bit for bit."""
    _say(f"rotated vs block-by-block {dt} B{B} H{H} N{N} d{d} P{P}")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    q_all, k, v = workloads.make_small(B, H, N, d, tdt, seed=77 + P)
    rotated = ra.ra_ring_forward(q_all, k, v, P)
    rev = list(range(P))[::-1]
    q_rev = _resident_q(q_all, N, P, rev)
    blockwise = ra.ra_ring_forward(q_rev, k, v, P, query_blocks=rev)
    torch.cuda.synchronize()
    b = N // P
    undone = torch.cat([blockwise[:, :, (P - 1 - i) * b:(P - i) * b] for i in range(P)], dim=2)
    assert torch.equal(undone, rotated)
    ref = oracle.ring_attention(to64(q_all), to64(k), to64(v), P)
    check_output(rotated, ref, dt, "rotated ring")
    assert np.all(np.isfinite(to64(rotated)))
