"""GPU parity of the ring backward (dQ, dK, dV) and of the forward's row
log-sum-exp against the fp64 CPU oracle (oracle/backward.py, pinned to torch
autograd, finite differences and exact invariants).

vibeengines.com "Ring attention, explained", method step 6: the backward runs
on the same ring, dK and dV accumulators travelling with the blocks.  The
gradient bars are the output bars scaled by each gradient's magnitude
(tests/helpers.py check_grad).
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from oracle import backward as ob  # noqa: E402
from oracle import layouts  # noqa: E402
from tests.helpers import check_grad, check_output, to64  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    import blockwise_online_softmax_fold_amd as ra

    ra.load()
    return ra


def _say(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _dt(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def _inputs(B, H, N, d, dtype, seed, n=4):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    return [torch.randn((B, H, N, d), generator=gen, device="cuda").to(_dt(dtype)) for _ in range(n)]


def _lse_oracle(q, k, v, P, layout):
    """m + ln l of every row from the oracle's ring states (all blocks resident)."""
    _, states = oracle.ring_attention(q, k, v, P, return_states=True, causal_layout=layout)
    return np.concatenate([st[-1].m + np.log(st[-1].l) for st in states], axis=-1)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", [None, "contiguous", "striped", "zigzag"])
def test_forward_lse(ra, layout, dtype):
    N, P, d = 1024, 4, 128
    _say(f"forward lse layout={layout} dtype={dtype}")
    q, k, v = _inputs(1, 2, N, d, dtype, 31, 3)
    out, lse = ra.ra_ring_forward_ex(q, k, v, P, layout)
    out2 = ra.ra_ring_forward(q, k, v, P) if layout is None else ra.ra_ring_forward_causal(q, k, v, P, layout)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)  # the lse output changes nothing else
    want = _lse_oracle(to64(q), to64(k), to64(v), P, layout)
    tol = 2e-3 if dtype == "bf16" else 1e-5
    np.testing.assert_allclose(to64(lse), want, rtol=0, atol=tol * (1 + np.abs(want).max()))


def _check_backward(ra, q, k, v, do, P, layout, dtype, what, query_blocks=None):
    out, lse = ra.ra_ring_forward_ex(q, k, v, P, layout, query_blocks=query_blocks)
    dq, dk, dv = ra.ra_ring_backward(q, k, v, out, do, lse, P, layout, query_blocks=query_blocks)
    torch.cuda.synchronize()
    want = ob.ring_attention_backward(to64(q), to64(k), to64(v), to64(do), P, query_blocks=query_blocks,
                                      causal_layout=layout)
    for name, g, w in zip(("dQ", "dK", "dV"), (dq, dk, dv), want):
        check_grad(g, w, dtype, f"{what} {name}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,P,d", [(512, 4, 128), (384, 3, 64), (256, 2, 256), (300, 1, 128), (1000, 3, 128)])
def test_ring_backward(ra, N, P, d, dtype):
    _say(f"ring backward N={N} P={P} d={d} dtype={dtype}")
    q, k, v, do = _inputs(1, 2, N, d, dtype, 41 + N + d)
    _check_backward(ra, q, k, v, do, P, None, dtype, f"N={N} P={P} d={d}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("N,P,d", [(512, 4, 128), (768, 3, 64), (384, 2, 256)])
def test_ring_backward_causal(ra, layout, N, P, d, dtype):
    _say(f"ring backward causal layout={layout} N={N} P={P} d={d} dtype={dtype}")
    q, k, v, do = _inputs(1, 2, N, d, dtype, 51 + N)
    _check_backward(ra, q, k, v, do, P, layout, dtype, f"causal {layout}")


@pytest.mark.parametrize("layout", [None, "contiguous", "striped"])
def test_ring_backward_uneven_causal(ra, layout):
    N, P, d = 1003, 4, 128
    _say(f"ring backward uneven N={N} P={P} layout={layout}")
    q, k, v, do = _inputs(2, 2, N, d, "bf16", 61)
    _check_backward(ra, q, k, v, do, P, layout, "bf16", f"uneven {layout}")


@pytest.mark.parametrize("qb", [(0,), (3, 1), (2, 0, 3)])
def test_ring_backward_resident_shares(ra, qb):
    """Resident subsets: dQ of those rows; dK, dV hold only their shares."""
    N, P, d = 640, 4, 128
    _say(f"ring backward residents {qb}")
    q, k, v, do = _inputs(1, 2, N, d, "bf16", 71)
    bounds = oracle.block_bounds(N, P)
    rows = torch.from_numpy(np.concatenate([np.arange(*bounds[i]) for i in qb])).cuda()
    _check_backward(ra, q[:, :, rows].contiguous(), k, v, do[:, :, rows].contiguous(), P, None, "bf16",
                    f"residents {qb}", query_blocks=list(qb))


def test_ring_backward_16k(ra):
    """B1 H4 d128 N4096 P8 bf16, every gradient compared in full."""
    N, P, d = 4096, 8, 128
    _say(f"ring backward N={N} P={P}")
    q, k, v, do = _inputs(1, 4, N, d, "bf16", 81)
    out, lse = ra.ra_ring_forward_ex(q, k, v, P)
    dq, dk, dv = ra.ra_ring_backward(q, k, v, out, do, lse, P)
    torch.cuda.synchronize()
    want = ob.dense_attention_backward(to64(q), to64(k), to64(v), to64(do))
    for name, g, w in zip(("dQ", "dK", "dV"), (dq, dk, dv), want):
        check_grad(g, w, "bf16", f"N={N} {name}")


def test_ring_backward_caller_workspace_and_determinism(ra):
    N, P, d = 512, 4, 64
    _say("ring backward caller workspace, repeat")
    q, k, v, do = _inputs(1, 2, N, d, "bf16", 91)
    out, lse = ra.ra_ring_forward_ex(q, k, v, P)
    ws = torch.empty(ra.ra_ring_backward_workspace_bytes(torch.bfloat16, 1, 2, N, d, P, P), dtype=torch.uint8,
                     device="cuda")
    a = ra.ra_ring_backward(q, k, v, out, do, lse, P, workspace=ws)
    b = ra.ra_ring_backward(q, k, v, out, do, lse, P)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    with pytest.raises(ra.RaError):
        ra.ra_ring_backward(q, k, v, out, do, lse, P, workspace=ws[:-256])


@pytest.mark.parametrize("d", [64, 128])
def test_ring_backward_strided_layout(ra, d):
    """Q, K, V, dO stored [B, N, H, d] and viewed as [B, H, N, d] (row stride
    H d), so every streamed LDS tile -- K and V in the dQ kernel, Q, dO and
    the V rows in the dK/dV kernel -- is gathered with a non-trivial row
    stride; gradients written into contiguous tensors."""
    B, H, N, P = 1, 8, 700, 3
    _say(f"ring backward strided [B,N,H,d] views d={d}")
    gen = torch.Generator(device="cuda").manual_seed(101 + d)
    base = [torch.randn((B, N, H, d), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(4)]
    q, k, v, do = (t.permute(0, 2, 1, 3) for t in base)
    assert q.stride(2) == H * d
    _check_backward(ra, q, k, v, do, P, None, "bf16", f"strided d={d}")


@pytest.mark.parametrize("layout", [None, "striped"])
def test_ring_backward_many_devices(ra, layout):
    """P = 70 devices: more resident blocks than one backward launch takes (64),
    so each step's dQ and dK/dV passes are split into two launches."""
    N, P, d = 280, 70, 64
    _say(f"ring backward P={P} N={N} layout={layout}")
    q, k, v, do = _inputs(1, 2, N, d, "bf16", 111)
    _check_backward(ra, q, k, v, do, P, layout, "bf16", f"P={P} {layout}")


@pytest.mark.parametrize("layout", [None, "zigzag"])
def test_ring_backward_explicit_scale(ra, layout):
    """A caller-given scale through ra_ring_forward_ex and ra_ring_backward, B = 2."""
    N, P, d, sc = 512, 4, 128, 0.25
    _say(f"ring backward explicit scale={sc} layout={layout}")
    q, k, v, do = _inputs(2, 2, N, d, "bf16", 121)
    out, lse = ra.ra_ring_forward_ex(q, k, v, P, layout, scale=sc)
    dq, dk, dv = ra.ra_ring_backward(q, k, v, out, do, lse, P, layout, scale=sc)
    torch.cuda.synchronize()
    want = ob.ring_attention_backward(to64(q), to64(k), to64(v), to64(do), P, scale=sc, causal_layout=layout)
    for name, g, w in zip(("dQ", "dK", "dV"), (dq, dk, dv), want):
        check_grad(g, w, "bf16", f"scale={sc} {layout} {name}")


def test_ring_backward_128k_sampled(ra):
    """The headline shape (B1 H32 d128 N131072 P16, all blocks resident), as
    bench.py --backward launches it: head 0's dQ on 64 sampled query rows and
    dK, dV on 64 sampled key rows against the oracle's streaming row sampler
    (one full fp64 pass over head 0, about a minute of CPU time); every
    gradient finite."""
    import workloads
    from tests.helpers import sample_rows

    w = workloads.WORKLOADS[3]
    _say(f"ring backward full size {w.describe()}")
    q, k, v = workloads.make_inputs(w, device="cuda")
    do = torch.randn(q.shape, generator=torch.Generator(device="cuda").manual_seed(w.seed + 7),
                     device="cuda").to(q.dtype)
    out, lse = ra.ra_ring_forward_ex(q, k, v, w.P)
    dq, dk, dv = ra.ra_ring_backward(q, k, v, out, do, lse, w.P)
    torch.cuda.synchronize()
    for g in (dq, dk, dv):
        assert torch.isfinite(g).all()
    rows = sample_rows(w.P, w.b, 4, seed=w.seed)
    print(f"[case] oracle pass over head 0 ({len(rows)} query and key rows)", flush=True)
    want = ob.backward_rows(to64(q[0, 0]), to64(k[0, 0]), to64(v[0, 0]), to64(do[0, 0]), rows, rows, row_chunk=2048)
    print("[case] oracle done", flush=True)
    idx = torch.from_numpy(rows).cuda()
    for name, g, ww in zip(("dQ", "dK", "dV"), (dq, dk, dv), want):
        check_grad(g[0, 0, idx], ww, "bf16", f"128K {name}")


def test_ring_backward_128k_causal_sampled(ra):
    """The headline shape under the zig-zag causal layout: head 0's dQ, dK, dV
    on 64 sampled rows against the oracle's streaming row sampler with the
    rows' positions (one full fp64 pass over head 0)."""
    import workloads
    from tests.helpers import sample_rows

    w = workloads.WORKLOADS[3]
    layout = "zigzag"
    _say(f"ring backward full size causal {layout} {w.describe()}")
    q, k, v = workloads.make_inputs(w, device="cuda")
    do = torch.randn(q.shape, generator=torch.Generator(device="cuda").manual_seed(w.seed + 9),
                     device="cuda").to(q.dtype)
    out, lse = ra.ra_ring_forward_ex(q, k, v, w.P, layout)
    dq, dk, dv = ra.ra_ring_backward(q, k, v, out, do, lse, w.P, layout)
    torch.cuda.synchronize()
    for g in (dq, dk, dv):
        assert torch.isfinite(g).all()
    rows = sample_rows(w.P, w.b, 4, seed=w.seed + 1)
    pos = layouts.positions(layout, w.P, w.b).reshape(-1)
    print(f"[case] oracle pass over head 0 ({len(rows)} query and key rows)", flush=True)
    want = ob.backward_rows(to64(q[0, 0]), to64(k[0, 0]), to64(v[0, 0]), to64(do[0, 0]), rows, rows,
                            row_chunk=2048, pos=pos)
    print("[case] oracle done", flush=True)
    idx = torch.from_numpy(rows).cuda()
    for name, g, ww in zip(("dQ", "dK", "dV"), (dq, dk, dv), want):
        check_grad(g[0, 0, idx], ww, "bf16", f"128K causal {name}")
