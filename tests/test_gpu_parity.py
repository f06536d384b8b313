"""GPU parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Small cases are compared element by element, full-size workloads on a seeded
row sample.  Tolerances: bf16 max-abs <= 2e-2 and mean-abs <= 2e-3; fp32
max|err| <= 1e-5 max|O_ref|.
"""

from __future__ import annotations

import math
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads  # noqa: E402
from tests.helpers import check_output, oracle_rows, sample_rows, to64  # noqa: E402

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


def _new_state(B, H, rows, d):
    m = torch.empty((B, H, rows), device="cuda", dtype=torch.float32)
    l = torch.empty_like(m)
    o = torch.empty((B, H, rows, d), device="cuda", dtype=torch.float32)
    return m, l, o


# ---------------------------------------------------------------------------
# state init / finalize


def test_state_init_and_finalize(ra):
    _say("state_init + finalize B2 H3 rows 37 d64")
    m, l, o = _new_state(2, 3, 37, 64)
    ra.ra_state_init(m, l, o)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(m)) and torch.all(l == 0) and torch.all(o == 0)
    # finalize: o / l, rows with l == 0 give 0
    l.copy_(torch.rand_like(l) + 0.5)
    l[0, 1, 5] = 0.0
    o.copy_(torch.randn_like(o))
    for dt in (torch.float32, torch.bfloat16):
        out = torch.empty((2, 3, 37, 64), device="cuda", dtype=dt)
        ra.ra_finalize(l, o, out)
        torch.cuda.synchronize()
        ref = to64(o) / np.where(to64(l) > 0, to64(l), 1.0)[..., None]
        ref[0, 1, 5] = 0.0
        tol = 1e-6 if dt == torch.float32 else 2 ** -8
        np.testing.assert_allclose(to64(out), ref, rtol=tol, atol=tol)


# ---------------------------------------------------------------------------
# fold_block: per-step state parity, ragged shapes


def _oracle_steps(q, ks, vs, scale=None):
    st = oracle.init_state(tuple(q.shape[:2]), q.shape[2], q.shape[3])
    out = []
    for k, v in zip(ks, vs):
        st = oracle.ring.fold(st, to64(q), to64(k), to64(v), scale)
        out.append(st.copy())
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("q_rows,kv_rows", [(256, 192), (200, 77), (1, 1), (129, 300)])
def test_fold_block_state_per_step(ra, dtype, d, q_rows, kv_rows):
    _say(f"fold_block dtype={dtype} d={d} q_rows={q_rows} kv_rows={kv_rows} seed=7")
    B, H, steps = 1, 2, 3
    gen = torch.Generator(device="cuda").manual_seed(7 + d + q_rows)
    q = torch.randn((B, H, q_rows, d), generator=gen, device="cuda").to(_dt(dtype))
    ks = [torch.randn((B, H, kv_rows, d), generator=gen, device="cuda").mul(1.0 + t).to(_dt(dtype)) for t in range(steps)]
    vs = [torch.randn((B, H, kv_rows, d), generator=gen, device="cuda").to(_dt(dtype)) for t in range(steps)]
    m, l, o = _new_state(B, H, q_rows, d)
    ra.ra_state_init(m, l, o)
    ref = _oracle_steps(q, ks, vs)
    for t in range(steps):
        ra.ra_fold_block(q, ks[t], vs[t], m, l, o)
        torch.cuda.synchronize()
        r = ref[t]
        # m: the running max of the scaled scores (fp32 scores vs exact ones)
        np.testing.assert_allclose(to64(m), r.m, rtol=0, atol=2e-4 * (1 + np.abs(r.m).max()))
        # l relative to the oracle (bf16 weights carry 2^-9 rounding each)
        ltol = 1e-2 if dtype == "bf16" else 1e-5
        np.testing.assert_allclose(to64(l), r.l, rtol=ltol)
        # o / l is attention over the keys folded so far
        check_output(to64(o) / to64(l)[..., None], r.o / r.l[..., None], dtype, f"step {t} o/l")


# Visiting-block lengths that take every path of the d = 256 tile loop (32-key
# tiles in padded LDS rows, two buffers, full tiles two per loop iteration): a
# lone ragged tile, one full tile, a full tile plus a ragged one, whole pairs,
# a pair plus a single full tile, and a ragged last tile after either; 130
# query rows leave the second 128-row workgroup two rows.
@pytest.mark.parametrize("kv_rows", [31, 32, 33, 64, 95, 96, 97, 128, 161, 224, 225])
def test_fold_block_d256_tile_ring(ra, kv_rows):
    _say(f"fold_block d=256 q_rows=130 kv_rows={kv_rows} seed=11")
    B, H, q_rows, d, steps = 1, 2, 130, 256, 2
    gen = torch.Generator(device="cuda").manual_seed(11 + kv_rows)
    q = torch.randn((B, H, q_rows, d), generator=gen, device="cuda").to(torch.bfloat16)
    ks = [torch.randn((B, H, kv_rows, d), generator=gen, device="cuda").mul(1.0 + t).to(torch.bfloat16) for t in range(steps)]
    vs = [torch.randn((B, H, kv_rows, d), generator=gen, device="cuda").to(torch.bfloat16) for t in range(steps)]
    m, l, o = _new_state(B, H, q_rows, d)
    ra.ra_state_init(m, l, o)
    ref = _oracle_steps(q, ks, vs)
    for t in range(steps):
        ra.ra_fold_block(q, ks[t], vs[t], m, l, o)
        torch.cuda.synchronize()
        r = ref[t]
        np.testing.assert_allclose(to64(m), r.m, rtol=0, atol=2e-4 * (1 + np.abs(r.m).max()))
        np.testing.assert_allclose(to64(l), r.l, rtol=1e-2)
        check_output(to64(o) / to64(l)[..., None], r.o / r.l[..., None], "bf16", f"step {t} o/l")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fold_block_large_max_jumps(ra, d):
    """Scores whose running maximum jumps far (hundreds of base-2 units) inside
    one block and across blocks, and rows whose maximum comes first: the
    reference-maximum bookkeeping must rescale exactly when needed."""
    _say(f"fold_block large maximum jumps d={d}")
    B, H, q_rows, kv_rows = 1, 2, 160, 300
    gen = torch.Generator(device="cuda").manual_seed(99 + d)
    q = torch.randn((B, H, q_rows, d), generator=gen, device="cuda")
    ks, vs = [], []
    for t in range(3):
        k = torch.randn((B, H, kv_rows, d), generator=gen, device="cuda")
        # key rows grow in magnitude along the block (later tiles dominate),
        # and a few rows of q see their largest scores in the first tile
        k = k * torch.linspace(0.5, 6.0 + 4 * t, kv_rows, device="cuda")[None, None, :, None]
        k[:, :, :8] *= 12.0
        ks.append(k.bfloat16())
        vs.append(torch.randn((B, H, kv_rows, d), generator=gen, device="cuda").bfloat16())
    q = q.bfloat16()
    m, l, o = _new_state(B, H, q_rows, d)
    ra.ra_state_init(m, l, o)
    ref = _oracle_steps(q, ks, vs)
    for t in range(3):
        ra.ra_fold_block(q, ks[t], vs[t], m, l, o)
        torch.cuda.synchronize()
        r = ref[t]
        np.testing.assert_allclose(to64(m), r.m, rtol=1e-5, atol=1e-3)
        assert np.all(np.isfinite(to64(l))) and np.all(np.isfinite(to64(o)))
        np.testing.assert_allclose(to64(l), r.l, rtol=1e-2)
        check_output(to64(o) / to64(l)[..., None], r.o / r.l[..., None], "bf16", f"step {t} o/l")


def test_fold_block_zero_rows_is_noop(ra):
    _say("fold_block kv_rows=0 / q_rows=0")
    q = torch.randn((1, 1, 64, 128), device="cuda").bfloat16()
    k = torch.randn((1, 1, 0, 128), device="cuda").bfloat16()
    m, l, o = _new_state(1, 1, 64, 128)
    ra.ra_state_init(m, l, o)
    ra.ra_fold_block(q, k, k, m, l, o)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(m)) and torch.all(l == 0) and torch.all(o == 0)
    out = torch.empty_like(q)
    ra.ra_finalize(l, o, out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    # no query rows at all
    q0 = torch.empty((1, 1, 0, 128), device="cuda", dtype=torch.bfloat16)
    m0, l0, o0 = _new_state(1, 1, 0, 128)
    kk = torch.randn((1, 1, 64, 128), device="cuda").bfloat16()
    ra.ra_state_init(m0, l0, o0)
    ra.ra_fold_block(q0, kk, kk, m0, l0, o0)
    ra.ra_finalize(l0, o0, q0)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# ring_forward: small rings compared element by element


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,H,N,d,P,qb", [
    (1, 2, 512, 128, 1, None),
    (2, 3, 768, 64, 3, None),
    (1, 2, 1280, 128, 5, None),
    (1, 1, 640, 256, 2, None),
    (1, 2, 2048, 128, 8, (6, 1, 1)),
    (1, 1, 200, 64, 4, None),  # blocks of 50 rows: ragged tiles everywhere
])
def test_ring_forward_small(ra, dtype, B, H, N, d, P, qb):
    _say(f"ring_forward dtype={dtype} B={B} H={H} N={N} d={d} P={P} query_blocks={qb}")
    q_all, k, v = workloads.make_small(B, H, N, d, _dt(dtype), seed=N + d + P)
    blocks = list(range(P)) if qb is None else list(qb)
    b = N // P
    q = torch.cat([q_all[:, :, i * b:(i + 1) * b] for i in blocks], dim=2).contiguous()
    out = ra.ra_ring_forward(q, k, v, P, query_blocks=qb)
    torch.cuda.synchronize()
    ref = oracle.ring_attention(to64(q_all), to64(k), to64(v), P, query_blocks=blocks)
    check_output(out, ref, dtype, "ring_forward")
    # and the dense definition
    dense = oracle.dense_attention(to64(q), to64(k), to64(v))
    check_output(out, dense, dtype, "ring_forward vs dense")


def test_ring_forward_strided_layout(ra):
    """Tensors stored [B, N, H, d] and viewed as [B, H, N, d] (head stride < row
    stride); output written into a strided view as well."""
    _say("ring_forward strided [B,N,H,d] views, bf16 H=4 N=1024 d=128 P=4")
    B, N, H, d, P = 1, 1024, 4, 128, 4
    gen = torch.Generator(device="cuda").manual_seed(99)
    base = [torch.randn((B, N, H, d), generator=gen, device="cuda").bfloat16() for _ in range(3)]
    q, k, v = (t.permute(0, 2, 1, 3) for t in base)
    out_store = torch.zeros((B, N, H, d), device="cuda", dtype=torch.bfloat16)
    out = out_store.permute(0, 2, 1, 3)
    ra.ra_ring_forward(q, k, v, P, out=out)
    torch.cuda.synchronize()
    check_output(out, oracle.dense_attention(to64(q), to64(k), to64(v)), "bf16", "strided")


def test_ring_forward_deterministic_and_overlap_free(ra, monkeypatch):
    """Bitwise equal run to run, and equal to the run with the hand-off
    serialised on the caller's stream (no overlap)."""
    _say("ring_forward determinism / RA_SYNC_EACH_STEP, bf16 H=8 N=8192 d=128 P=8")
    q, k, v = workloads.make_small(1, 8, 8192, 128, torch.bfloat16, seed=5)
    a = ra.ra_ring_forward(q, k, v, 8)
    b_ = ra.ra_ring_forward(q, k, v, 8)
    monkeypatch.setenv("RA_SYNC_EACH_STEP", "1")
    c = ra.ra_ring_forward(q, k, v, 8)
    torch.cuda.synchronize()
    assert torch.equal(a, b_)
    assert torch.equal(a, c)


def test_checkpoint_resume_bitwise(ra):
    """(m, l, o) is the whole state between steps: copy it to the host after
    step 2, restore it into fresh buffers and finish; the output is identical."""
    _say("checkpoint/resume via fold_block, bf16 H=2 N=2048 d=128 P=4")
    P, B, H, N, d = 4, 1, 2, 2048, 128
    q_all, k, v = workloads.make_small(B, H, N, d, torch.bfloat16, seed=21)
    b = N // P
    i = 1
    q = q_all[:, :, i * b:(i + 1) * b]
    order = oracle.ring_schedule(P, i)

    def run(split):
        m, l, o = _new_state(B, H, b, d)
        ra.ra_state_init(m, l, o)
        for t, j in enumerate(order):
            if t == split:
                host = [x.cpu() for x in (m, l, o)]
                m, l, o = _new_state(B, H, b, d)
                for dst, src in zip((m, l, o), host):
                    dst.copy_(src)
            ra.ra_fold_block(q, k[:, :, j * b:(j + 1) * b], v[:, :, j * b:(j + 1) * b], m, l, o)
        out = torch.empty_like(q)
        ra.ra_finalize(l, o, out)
        return out

    a, c = run(-1), run(2)
    torch.cuda.synchronize()
    assert torch.equal(a, c)
    # the fold_block loop agrees with ring_forward for that block; not bit for
    # bit: inside the ring the spilled state stays relative to the kernel's
    # reference maximum (kRefState), while fold_block's state is relative to
    # the running maximum, so the bf16 weights round differently
    full = ra.ra_ring_forward(q_all, k, v, P)
    torch.cuda.synchronize()
    check_output(full[:, :, i * b:(i + 1) * b], to64(a), "bf16", "ring vs fold_block loop")


def test_ring_rising_max_every_step(ra):
    """Resident block 0 of a P = 8 ring whose visiting blocks arrive with scores
    6 higher at every step (natural units): every step raises the running
    maximum by about 8.7 in base 2, so inside the ring each step's first tile
    takes the reference-raising path (the weights' sums exceed 2^8).  The
    output against the oracle; the math page's worked example is this rescale,
    repeated."""
    _say("ring_forward rising max every step, bf16 B1 H2 N8192 d128 P8, resident block 0")
    P, B, H, N, d = 8, 1, 2, 8192, 128
    b = N // P
    gen = torch.Generator(device="cuda").manual_seed(91)
    u = torch.randn((d,), generator=gen, device="cuda")
    u = u / torch.linalg.vector_norm(u)
    q = (torch.randn((B, H, b, d), generator=gen, device="cuda") + math.sqrt(d) * u).bfloat16()
    # block j carries shift 6 ((P - j) mod P): resident 0 visits j = 0, P-1, ..., 1
    shift = torch.tensor([6.0 * ((P - j) % P) for j in range(P)], device="cuda").repeat_interleave(b)
    k = (torch.randn((B, H, N, d), generator=gen, device="cuda") + shift[:, None] * u).bfloat16()
    v = (torch.rand((B, H, N, d), generator=gen, device="cuda") * 2 - 1).bfloat16()
    out = ra.ra_ring_forward(q, k, v, P, query_blocks=[0])
    torch.cuda.synchronize()
    ref = oracle.dense_attention(to64(q), to64(k), to64(v))
    check_output(out, ref, "bf16", "rising max, resident 0")


def test_fold_order_invariance(ra):
    """Ascending order and ring order agree within tolerance (the math page's
    worked example: the order of blocks does not change the result)."""
    _say("fold order invariance, bf16 H=2 N=4096 d=128 P=8")
    P, B, H, N, d = 8, 1, 2, 4096, 128
    q_all, k, v = workloads.make_small(B, H, N, d, torch.bfloat16, seed=33, scale=1.5)
    b = N // P
    ref = oracle.dense_attention(to64(q_all), to64(k), to64(v))
    for i in (0, 5):
        q = q_all[:, :, i * b:(i + 1) * b]
        for order in (oracle.ring_schedule(P, i), list(range(P)), list(range(P))[::-1]):
            m, l, o = _new_state(B, H, b, d)
            ra.ra_state_init(m, l, o)
            for j in order:
                ra.ra_fold_block(q, k[:, :, j * b:(j + 1) * b], v[:, :, j * b:(j + 1) * b], m, l, o)
            out = torch.empty_like(q)
            ra.ra_finalize(l, o, out)
            torch.cuda.synchronize()
            check_output(out, ref[:, :, i * b:(i + 1) * b], "bf16", f"block {i} order {order[:3]}...")


def test_caller_workspace(ra):
    _say("ring_forward with caller workspace, bf16 H=4 N=4096 d=128 P=4")
    q, k, v = workloads.make_small(1, 4, 4096, 128, torch.bfloat16, seed=44)
    nbytes = ra.ra_ring_workspace_bytes(torch.bfloat16, 1, 4, 4096, 128, 4, 4)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a = ra.ra_ring_forward(q, k, v, 4, workspace=ws)
    b_ = ra.ra_ring_forward(q, k, v, 4)
    torch.cuda.synchronize()
    assert torch.equal(a, b_)
    with pytest.raises(ra.RaError):
        ra.ra_ring_forward(q, k, v, 4, workspace=ws[: nbytes - 256])


# ---------------------------------------------------------------------------
# the five workloads


def _run_workload(ra, w):
    q, k, v = workloads.make_inputs(w, device="cuda")
    out = ra.ra_ring_forward(q, k, v, w.P, query_blocks=w.query_blocks)
    torch.cuda.synchronize()
    return q, k, v, out


def test_workload1_full(ra):
    w = workloads.WORKLOADS[1]
    _say(f"workload 1 {w.describe()}")
    q, k, v, out = _run_workload(ra, w)
    ref = oracle.ring_attention(to64(q), to64(k), to64(v), w.P)
    check_output(out, ref, "f32", "workload 1 vs ring oracle")
    check_output(out, oracle.dense_attention(to64(q), to64(k), to64(v)), "f32", "workload 1 vs dense")


# Rows compared per (batch, head, resident block), every head: about 2e12
# oracle FLOP (some 15 s on the host) for each of the three large workloads.
# Workload 2 is compared whole.
@pytest.mark.parametrize("wid,per_block,heads", [(2, 2048, None), (3, 64, None), (4, 128, None), (5, 128, None)])
def test_workload_sampled(ra, wid, per_block, heads):
    w = workloads.WORKLOADS[wid]
    _say(f"workload {wid} {w.describe()} sample {per_block} rows/block heads={heads}")
    q, k, v, out = _run_workload(ra, w)
    rows = sample_rows(w.n_q, w.b, per_block, seed=w.seed)
    ref = oracle_rows(q, k, v, rows, heads=heads)
    hsel = list(range(w.H)) if heads is None else heads
    got = out[:, hsel][:, :, torch.from_numpy(rows).cuda()]
    figs = check_output(got, ref, w.dtype, f"workload {wid}")
    print(f"[parity] workload {wid}: {figs}", flush=True)
    # properties that hold at every row: finite, inside the value range
    assert torch.isfinite(out).all()
    vmax = v.abs().amax().float()
    assert out.float().abs().amax() <= vmax * 1.01


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 256)])
def test_ring_forward_explicit_scale(ra, dtype, d):
    """A caller-given softmax scale (0.3, not 1/sqrt(d)) through the ABI, B = 2,
    against the dense oracle with the same scale."""
    B, H, N, P, sc = 2, 2, 600, 3, 0.3
    _say(f"ring_forward explicit scale={sc} dtype={dtype} B={B} H={H} N={N} d={d} P={P}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = workloads.make_small(B, H, N, d, tdt, seed=44 + d)
    out = ra.ra_ring_forward(q, k, v, P, scale=sc)
    torch.cuda.synchronize()
    check_output(out, oracle.dense_attention(to64(q), to64(k), to64(v), scale=sc), dtype, "explicit scale")
