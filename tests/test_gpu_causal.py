"""GPU parity of the causal entry points against the fp64 CPU oracle.

A query sees only keys at or before its position (math page, "Causal masking,
load balance, and other wrinkles"), under the contiguous, striped and zig-zag
token layouts (vibeengines.com, "The causal-mask catch").  The oracle masks
the scores of each pair with the positions ``oracle.layouts`` assigns; the
HIP path derives the same positions from (layout, P, block ids) on its own.
Tolerances are those of the non-causal tests.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import oracle.ring as oring  # noqa: E402
from oracle import layouts  # noqa: E402
from tests.helpers import check_output, sample_rows, to64  # noqa: E402

pytestmark = pytest.mark.gpu

LAYOUTS = ("contiguous", "striped", "zigzag")


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


def _rand(shape, gen, dtype, mul=1.0):
    return torch.randn(shape, generator=gen, device="cuda").mul(mul).to(_dt(dtype))


def _check_state(m, l, o, ref, dtype, what):
    """State parity; rows the oracle has never given a visible key must hold
    exactly (-inf, 0, 0)."""
    gm, gl, go = to64(m), to64(l), to64(o)
    empty = ref.l == 0
    assert np.all(np.isneginf(gm[empty])) and np.all(gl[empty] == 0) and np.all(go[empty] == 0), what
    seen = ~empty
    if not seen.any():
        return
    assert np.all(gl[seen] > 0), what
    np.testing.assert_allclose(gm[seen], ref.m[seen], rtol=0, atol=2e-4 * (1 + np.abs(ref.m[seen]).max()))
    np.testing.assert_allclose(gl[seen], ref.l[seen], rtol=1e-2 if dtype == "bf16" else 1e-5)
    check_output(go[seen] / gl[seen][:, None], ref.o[seen] / ref.l[seen][:, None], dtype, what)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_fold_block_causal_every_pair(ra, layout, d, dtype):
    """Every (query block, visiting block) pair of a P = 3 ring with b = 200
    rows (two query tiles, ragged key tiles), folded onto a state that has
    already seen a random block, then onto a fresh state."""
    P, b, B, H = 3, 200, 1, 2
    _say(f"fold_block_causal layout={layout} d={d} dtype={dtype} P={P} b={b}")
    gen = torch.Generator(device="cuda").manual_seed(11 + d)
    pos = layouts.positions(layout, P, b)
    q = [_rand((B, H, b, d), gen, dtype) for _ in range(P)]
    k = [_rand((B, H, b, d), gen, dtype, 1.5) for _ in range(P)]
    v = [_rand((B, H, b, d), gen, dtype) for _ in range(P)]
    k0, v0 = _rand((B, H, b, d), gen, dtype), _rand((B, H, b, d), gen, dtype)
    for i in range(P):
        for j in range(P):
            # pre-folded state: one unmasked block
            st = oring.fold(oracle.init_state((B, H), b, d), to64(q[i]), to64(k0), to64(v0))
            m, l, o = (torch.from_numpy(x).float().cuda() for x in (st.m, st.l, st.o))
            m0, l0, o0 = m.clone(), l.clone(), o.clone()
            ra.ra_fold_block_causal(q[i], k[j], v[j], m, l, o, layout, P, i, j)
            torch.cuda.synchronize()
            ref = oring.fold(st, to64(q[i]), to64(k[j]), to64(v[j]), None, pos[i], pos[j])
            _check_state(m, l, o, ref, dtype, f"pre-folded pair ({i}, {j})")
            # rows that see no key of block j keep their state bit for bit
            blind = np.array([not np.any(pos[j] <= pos[i][r]) for r in range(b)])
            if blind.any():
                for got, was in ((m, m0), (l, l0), (o, o0)):
                    assert torch.equal(got[:, :, torch.from_numpy(blind).cuda()],
                                       was[:, :, torch.from_numpy(blind).cuda()]), f"pair ({i}, {j}) touched a blind row"
            # fresh state
            m, l, o = (torch.empty_like(x) for x in (m, l, o))
            ra.ra_state_init(m, l, o)
            ra.ra_fold_block_causal(q[i], k[j], v[j], m, l, o, layout, P, i, j)
            torch.cuda.synchronize()
            ref = oring.fold(oracle.init_state((B, H), b, d), to64(q[i]), to64(k[j]), to64(v[j]), None, pos[i],
                             pos[j])
            _check_state(m, l, o, ref, dtype, f"fresh pair ({i}, {j})")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fold_block_causal_none_layout_is_fold_block(ra, dtype):
    _say(f"fold_block_causal layout=none equals fold_block dtype={dtype}")
    gen = torch.Generator(device="cuda").manual_seed(5)
    q, k, v = (_rand((1, 3, 130, 128), gen, dtype) for _ in range(3))
    outs = []
    for causal in (False, True):
        m = torch.empty((1, 3, 130), device="cuda")
        l, o = torch.empty_like(m), torch.empty((1, 3, 130, 128), device="cuda")
        ra.ra_state_init(m, l, o)
        if causal:
            ra.ra_fold_block_causal(q, k, v, m, l, o, None, 1, 0, 0)
        else:
            ra.ra_fold_block(q, k, v, m, l, o)
        outs.append((m, l, o))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_invisible_block_leaves_state_bitwise(ra, layout):
    """A block entirely in the future of every row of the resident block."""
    P, b, d = 4, 256, 128
    _say(f"invisible block layout={layout}")
    pos = layouts.positions(layout, P, b)
    pairs = [(i, j) for i in range(P) for j in range(P) if pos[j].min() > pos[i].max()]
    if layout == "contiguous":
        assert len(pairs) == P * (P - 1) // 2
    gen = torch.Generator(device="cuda").manual_seed(3)
    q, k, v = (_rand((1, 2, b, d), gen, "bf16") for _ in range(3))
    for i, j in pairs:
        m = torch.randn((1, 2, b), generator=gen, device="cuda")
        l = torch.rand((1, 2, b), generator=gen, device="cuda") + 0.5
        o = torch.randn((1, 2, b, d), generator=gen, device="cuda")
        before = [x.clone() for x in (m, l, o)]
        ra.ra_fold_block_causal(q, k, v, m, l, o, layout, P, i, j)
        torch.cuda.synchronize()
        for x, y in zip((m, l, o), before):
            assert torch.equal(x, y)


def _causal_ring_case(ra, layout, dtype, B, H, P, b, d, query_blocks, seed):
    N = P * b
    gen = torch.Generator(device="cuda").manual_seed(seed)
    # the sequence in position order, then dealt to devices in the layout's order
    qs, ks, vs = (_rand((B, H, N, d), gen, dtype) for _ in range(3))
    pos = layouts.positions(layout, P, b).reshape(-1)
    perm = torch.from_numpy(pos).cuda()
    ql, kl, vl = (x[:, :, perm].contiguous() for x in (qs, ks, vs))
    qb = list(range(P)) if query_blocks is None else list(query_blocks)
    q_res = torch.cat([ql[:, :, i * b:(i + 1) * b] for i in qb], dim=2).contiguous()
    out = ra.ra_ring_forward_causal(q_res, kl, vl, P, layout, query_blocks=query_blocks)
    torch.cuda.synchronize()
    return to64(out), to64(q_res), to64(kl), to64(vl), pos, qb


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("P,b,d", [(4, 256, 128), (3, 200, 64), (5, 96, 256), (1, 130, 128)])
def test_ring_causal_small(ra, layout, dtype, P, b, d):
    B, H = 1, 2
    _say(f"ring causal layout={layout} dtype={dtype} P={P} b={b} d={d}")
    got, q, k, v, pos, qb = _causal_ring_case(ra, layout, dtype, B, H, P, b, d, None, 40 + P + d)
    ref = oracle.dense_attention(q, k, v, q_pos=pos, k_pos=pos)
    check_output(got, ref, dtype, f"causal ring {layout}")
    # and the oracle's own causal ring in layout order agrees with its dense form
    if P * b <= 512:
        ring_ref = oracle.ring_attention(q, k, v, P, causal_layout=layout)
        np.testing.assert_allclose(ring_ref, ref, rtol=0, atol=1e-10)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_ring_causal_resident_subset(ra, layout):
    P, b, d = 6, 128, 128
    qb = (5, 0, 3)
    _say(f"ring causal resident subset {qb} layout={layout}")
    got, q, k, v, pos, qbl = _causal_ring_case(ra, layout, "bf16", 1, 2, P, b, d, qb, 77)
    q_pos = np.concatenate([pos[i * b:(i + 1) * b] for i in qbl])
    ref = oracle.dense_attention(q, k, v, q_pos=q_pos, k_pos=pos)
    check_output(got, ref, "bf16", "causal ring, resident subset")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_ring_causal_16k(ra, layout):
    """B1 H16 d128 N16384 P8 (b 2048) under each causal layout; 48 sampled rows
    per block of two heads against the dense causal oracle."""
    B, H, P, b, d = 1, 16, 8, 2048, 128
    _say(f"ring causal 16K layout={layout}")
    got, q, k, v, pos, qb = _causal_ring_case(ra, layout, "bf16", B, H, P, b, d, None, 2002)
    rows = sample_rows(P, b, 48, 2002)
    for hi in (0, H - 1):
        ref = oracle.dense_attention(q[0, hi, rows], k[0, hi], v[0, hi], q_pos=pos[rows], k_pos=pos)
        check_output(got[0, hi, rows], ref, "bf16", f"causal 16K head {hi}")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_ring_causal_many_devices(ra, layout):
    """P = 70 devices of 4 rows: more resident blocks than one fold launch takes
    (64), so every ring step is split into two launches."""
    P, b, d = 70, 4, 64
    _say(f"ring causal P={P} b={b} layout={layout}")
    got, q, k, v, pos, qb = _causal_ring_case(ra, layout, "bf16", 1, 2, P, b, d, None, 303)
    ref = oracle.dense_attention(q, k, v, q_pos=pos, k_pos=pos)
    check_output(got, ref, "bf16", f"causal ring P={P} {layout}")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_ring_causal_batch_and_scale(ra, layout):
    """B = 2 batches and a caller-given scale under each causal layout."""
    B, H, P, b, d, sc = 2, 2, 4, 96, 128, 0.2
    _say(f"ring causal B={B} scale={sc} layout={layout}")
    N = P * b
    gen = torch.Generator(device="cuda").manual_seed(505)
    q, k, v = (_rand((B, H, N, d), gen, "bf16") for _ in range(3))
    out = ra.ra_ring_forward_causal(q, k, v, P, layout, scale=sc)
    torch.cuda.synchronize()
    pos = layouts.positions(layout, P, b).reshape(-1)
    ref = oracle.dense_attention(to64(q), to64(k), to64(v), scale=sc, q_pos=pos, k_pos=pos)
    check_output(out, ref, "bf16", f"causal {layout} B={B} scale={sc}")


@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
def test_ring_causal_128k_sampled(ra, layout):
    """The headline shape (B1 H32 d128 N131072 P16) as bench.py --causal runs
    it: random inputs taken as already dealt in ``layout``'s device order;
    48 sampled rows per block of heads 0 and 31 against the dense causal
    oracle at those rows' positions."""
    import workloads

    w = workloads.WORKLOADS[3]
    _say(f"ring causal full size {layout} {w.describe()}")
    q, k, v = workloads.make_inputs(w, device="cuda")
    out = ra.ra_ring_forward_causal(q, k, v, w.P, layout)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    pos = layouts.positions(layout, w.P, w.b).reshape(-1)
    rows = sample_rows(w.P, w.b, 48, 3003)
    idx = torch.from_numpy(rows).cuda()
    for hi in (0, w.H - 1):
        ref = oracle.dense_attention(to64(q[0, hi, idx]), to64(k[0, hi]), to64(v[0, hi]), q_pos=pos[rows], k_pos=pos)
        check_output(to64(out[0, hi, idx]), ref, "bf16", f"causal 128K {layout} head {hi}")
