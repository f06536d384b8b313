"""ra_ring_forward_noalloc (collected last: it shares a device-wide scratch): the ring forward in the library's static device
scratch, for callers that cannot allocate.  Through the C ABI its output must
equal ra_ring_forward's (the same kernels on the same data, so bit for bit),
on two calls in a row, the second with a smaller ring, and rings needing more
workspace than the scratch holds are refused before any GPU work."""

from __future__ import annotations

import sys

import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads  # noqa: E402
from tests.helpers import check_output, to64  # noqa: E402


@pytest.fixture(scope="module")
def ra():
    import blockwise_online_softmax_fold_amd as ra

    ra.load()
    return ra


def _say(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


# (dtype, B, H, N, d, P, query_blocks): the first needs most of the scratch,
# the second is smaller, with uneven blocks and a resident subset
CASES = [
    ("bf16", 1, 8, 4096, 128, 8, None),
    ("f32", 1, 2, 1000, 64, 3, (2, 0)),
]


@pytest.mark.gpu
def test_noalloc_equals_ring_forward_on_consecutive_calls(ra):
    outs = []
    for dt, B, H, N, d, P, qb in CASES:
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        blocks = list(range(P)) if qb is None else list(qb)
        need = ra.ra_ring_workspace_bytes(tdt, B, H, N, d, P, len(blocks))
        _say(f"noalloc ring {dt} B{B} H{H} N{N} d{d} P{P} residents {blocks}: workspace {need} bytes")
        assert 0 < need <= ra.NOALLOC_SCRATCH_BYTES
        q_all, k, v = workloads.make_small(B, H, N, d, tdt, seed=N + d)
        bounds = oracle.block_bounds(N, P)
        q = torch.cat([q_all[:, :, bounds[i][0]:bounds[i][1]] for i in blocks], dim=2).contiguous()
        want = ra.ra_ring_forward(q, k, v, P, query_blocks=qb)
        out = torch.full_like(q, float("nan"))
        got = ra.ra_ring_forward_noalloc(q, k, v, P, query_blocks=qb, out=out)
        torch.cuda.synchronize()
        assert got is out
        assert torch.equal(got, want)
        check_output(got, oracle.ring_attention(to64(q_all), to64(k), to64(v), P, query_blocks=blocks), dt,
                     "noalloc vs oracle")
        outs.append(got.clone())
    # the first call's result is unaffected by the second call's use of the scratch
    dt, B, H, N, d, P, qb = CASES[0]
    q_all, k, v = workloads.make_small(B, H, N, d, torch.bfloat16, seed=N + d)
    again = ra.ra_ring_forward_noalloc(q_all, k, v, P)
    torch.cuda.synchronize()
    assert torch.equal(again, outs[0])


@pytest.mark.gpu
def test_noalloc_refuses_rings_beyond_the_scratch(ra):
    _say("noalloc refuses a ring larger than the scratch (bf16 B1 H16 N16384 d128 P8)")
    B, H, N, d, P = 1, 16, 16384, 128, 8
    need = ra.ra_ring_workspace_bytes(torch.bfloat16, B, H, N, d, P, P)
    assert need > ra.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ra.RaError, match="static scratch"):
        ra.ra_ring_forward_noalloc(q, q, q, P, out=torch.empty_like(q))
