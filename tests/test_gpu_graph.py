"""The ring forward and backward captured into a HIP graph (stream capture
through torch.cuda.graph) and replayed: every replay, with unrelated eager work
and synchronisations in between, must equal the eager call bit for bit, and a
replay after the inputs change in place must equal the eager call on the new
inputs.  The ring driver's hand-off copies, side stream and events all become
graph nodes; the caller passes the workspace, so nothing is allocated during
capture."""

from __future__ import annotations

import sys

import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    import blockwise_online_softmax_fold_amd as ra

    ra.load()
    return ra


def _say(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _inputs(B, H, N, d, dtype, seed, n=3):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    return [torch.randn((B, H, N, d), generator=gen, device="cuda").to(dtype) for _ in range(n)]


def _eager_noise():
    x = torch.randn(4096, device="cuda")
    return float((x * x).sum().item())


@pytest.mark.parametrize("dtype,N,P,d,layout", [(torch.float32, 1024, 4, 64, None),
                                                 (torch.bfloat16, 2048, 4, 128, None),
                                                 (torch.bfloat16, 1536, 3, 128, "zigzag"),
                                                 (torch.bfloat16, 1040, 4, 256, None),
                                                 (torch.bfloat16, 768, 3, 256, "striped")])
def test_ring_forward_graph_replay(ra, dtype, N, P, d, layout):
    _say(f"graph replay ring forward dtype={dtype} N={N} P={P} d={d} layout={layout}")
    q, k, v = _inputs(1, 2, N, d, dtype, 7 + N)
    ws = torch.empty(ra.ra_ring_workspace_bytes(dtype, 1, 2, N, d, P, P), dtype=torch.uint8, device="cuda")
    fwd = (lambda out: ra.ra_ring_forward(q, k, v, P, out=out, workspace=ws)) if layout is None else \
        (lambda out: ra.ra_ring_forward_causal(q, k, v, P, layout, out=out, workspace=ws))
    want = torch.empty_like(q)
    fwd(want)
    torch.cuda.synchronize()
    out = torch.zeros_like(q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(out)
    torch.cuda.synchronize()
    for rep in range(3):
        _eager_noise()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {rep} differs from the eager call"
    q2, k2, v2 = _inputs(1, 2, N, d, dtype, 99 + N)
    q.copy_(q2)
    k.copy_(k2)
    v.copy_(v2)
    g.replay()
    want2 = torch.empty_like(q)
    fwd(want2)
    torch.cuda.synchronize()
    assert torch.equal(out, want2), "replay on new inputs differs from the eager call"


def test_ring_backward_graph_replay(ra):
    N, P, d = 1024, 4, 128
    _say(f"graph replay ring backward N={N} P={P} d={d}")
    q, k, v, do = _inputs(1, 2, N, d, torch.bfloat16, 17, 4)
    out, lse = ra.ra_ring_forward_ex(q, k, v, P)
    ws = torch.empty(ra.ra_ring_backward_workspace_bytes(torch.bfloat16, 1, 2, N, d, P, P), dtype=torch.uint8,
                     device="cuda")
    want = ra.ra_ring_backward(q, k, v, out, do, lse, P, workspace=ws)
    torch.cuda.synchronize()
    grads = [torch.zeros_like(q) for _ in range(3)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ra.ra_ring_backward(q, k, v, out, do, lse, P, dq=grads[0], dk=grads[1], dv=grads[2], workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        _eager_noise()
        for t in grads:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), grads, want):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
