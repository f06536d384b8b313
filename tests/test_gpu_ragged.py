"""GPU parity when N is not a multiple of P (uneven blocks), against the fp64
CPU oracle.

bembew.net "Ring Attention", "Implementation Considerations": a sequence
length P does not divide needs padding or uneven partitioning.  Both sides
give the first N mod P devices one row more; the oracle's split is pinned to
numpy.array_split (tests/test_oracle_ragged.py), the library derives its own
from (N, P).  Tolerances are those of the other parity tests.
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


def _inputs(B, H, N, d, dtype, seed):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    return [torch.randn((B, H, N, d), generator=gen, device="cuda").to(_dt(dtype)) for _ in range(3)]


def _resident_rows(N, P, qb):
    bounds = oring.block_bounds(N, P)
    return np.concatenate([np.arange(*bounds[i]) for i in qb])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,P,d", [(1000, 3, 128), (1031, 8, 64), (777, 7, 256), (2053, 16, 128), (130, 129, 64)])
def test_ring_uneven_blocks(ra, N, P, d, dtype):
    _say(f"ring uneven N={N} P={P} d={d} dtype={dtype}")
    q, k, v = _inputs(1, 2, N, d, dtype, 300 + N + d)
    out = ra.ra_ring_forward(q, k, v, P)
    torch.cuda.synchronize()
    ref = oracle.dense_attention(to64(q), to64(k), to64(v))
    check_output(out, ref, dtype, f"uneven ring N={N} P={P}")


@pytest.mark.parametrize("qb", [(0,), (5,), (4, 0, 2), (6, 5, 4, 3, 2, 1, 0)])
def test_ring_uneven_resident_subsets(ra, qb):
    """Residents of both sizes (7 blocks over 1003 rows: three of 144, four of
    143), stacked in the order given."""
    N, P, d = 1003, 7, 128
    _say(f"ring uneven residents {qb} N={N} P={P}")
    q, k, v = _inputs(2, 2, N, d, "bf16", 71)
    rows = _resident_rows(N, P, qb)
    q_res = q[:, :, torch.from_numpy(rows).cuda()].contiguous()
    out = ra.ra_ring_forward(q_res, k, v, P, query_blocks=list(qb))
    torch.cuda.synchronize()
    ref = oracle.dense_attention(to64(q_res), to64(k), to64(v))
    check_output(out, ref, "bf16", f"uneven residents {qb}")
    with pytest.raises(ValueError):  # q must hold exactly the residents' rows
        ra.ra_ring_forward(q[:, :, : rows.size - 1], k, v, P, query_blocks=list(qb))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["contiguous", "striped"])
@pytest.mark.parametrize("N,P,d", [(1000, 3, 128), (517, 6, 64), (1101, 4, 256)])
def test_ring_causal_uneven_blocks(ra, layout, N, P, d, dtype):
    _say(f"ring causal uneven layout={layout} N={N} P={P} d={d} dtype={dtype}")
    qs, ks, vs = _inputs(1, 2, N, d, dtype, 500 + N)
    perm = np.concatenate(layouts.block_positions(layout, P, N))
    pt = torch.from_numpy(perm).cuda()
    ql, kl, vl = (x[:, :, pt].contiguous() for x in (qs, ks, vs))
    out = ra.ra_ring_forward_causal(ql, kl, vl, P, layout)
    torch.cuda.synchronize()
    ref = oracle.dense_attention(to64(ql), to64(kl), to64(vl), q_pos=perm, k_pos=perm)
    check_output(out, ref, dtype, f"causal uneven {layout}")


def test_zigzag_rejects_uneven(ra):
    q, k, v = _inputs(1, 1, 1001, 64, "bf16", 1)
    with pytest.raises(ra.RaError):
        ra.ra_ring_forward_causal(q, k, v, 4, "zigzag")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", [None, "contiguous", "striped"])
def test_fold_block_causal_uneven_pairs(ra, layout, dtype):
    """Every (query block, visiting block) pair of N = 459 over P = 4 (blocks
    of 115, 115, 115, 114 rows) from a fresh state."""
    N, P, d, B, H = 459, 4, 128, 1, 2
    _say(f"fold_block_causal uneven layout={layout} dtype={dtype}")
    q, k, v = _inputs(B, H, N, d, dtype, 900)
    bounds = oring.block_bounds(N, P)
    pos = layouts.block_positions(layout or "contiguous", P, N)
    # tensors in layout order
    perm = torch.from_numpy(np.concatenate(pos)).cuda()
    ql, kl, vl = (x[:, :, perm].contiguous() for x in (q, k, v))
    for i in range(P):
        for j in range(P):
            qi = ql[:, :, bounds[i][0]:bounds[i][1]].contiguous()
            kj = kl[:, :, bounds[j][0]:bounds[j][1]].contiguous()
            vj = vl[:, :, bounds[j][0]:bounds[j][1]].contiguous()
            rows = qi.shape[2]
            m = torch.empty((B, H, rows), device="cuda")
            l, o = torch.empty_like(m), torch.empty((B, H, rows, d), device="cuda")
            ra.ra_state_init(m, l, o)
            ra.ra_fold_block_causal(qi, kj, vj, m, l, o, layout, P, i, j, N=N)
            torch.cuda.synchronize()
            qp, kp = (pos[i], pos[j]) if layout else (None, None)
            ref = oring.fold(oracle.init_state((B, H), rows, d), to64(qi), to64(kj), to64(vj), None, qp, kp)
            seen = ref.l > 0
            gl, go = to64(l), to64(o)
            assert np.all(gl[~seen] == 0) and np.all(go[~seen] == 0)
            if seen.any():
                check_output(go[seen] / gl[seen][:, None], ref.o[seen] / ref.l[seen][:, None], dtype,
                             f"pair ({i}, {j})")


def test_ring_uneven_16k(ra):
    """B1 H8 d128 over N = 16384 + 13 tokens, P = 8 (blocks of 2050 and 2049),
    sampled rows of two heads against the dense oracle."""
    B, H, N, P, d = 1, 8, 16384 + 13, 8, 128
    _say(f"ring uneven N={N} P={P}")
    q, k, v = _inputs(B, H, N, d, "bf16", 16397)
    out = ra.ra_ring_forward(q, k, v, P)
    torch.cuda.synchronize()
    rows = sample_rows(1, N, 256, 16397)
    got, q64, k64, v64 = to64(out), to64(q), to64(k), to64(v)
    for hi in (0, H - 1):
        ref = oracle.dense_attention_rows(q64[0, hi], k64[0, hi], v64[0, hi], rows)
        check_output(got[0, hi, rows], ref, "bf16", f"uneven 16K head {hi}")
