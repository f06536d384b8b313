"""The rescale-stress workload (B2 H8 d256 N32768 P32, b = 1024; key block j
shifted by +0.25 j along a direction Q shares) folded in ASCENDING block
order with ra_fold_block, so the running maximum of most rows rises on many
steps and the state is rescaled by alpha = exp(m - m') each time -- the step
the math page's "A worked numeric example" walks through (the second block
lifts the maximum and l, o are multiplied by alpha).

In ring order (i - t) mod P the shifted blocks arrive in falling order and the
maximum jumps once, at the wrap; that order is covered by the full-size ring
parity test.  Here the oracle's own fold loop, run on a row sample in the same
ascending order, reports how often each row's maximum rose and the smallest
alpha it took, and the test asserts that the stress is real before it
compares the GPU's state after every step and its final output.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads  # noqa: E402
from tests.helpers import check_output, sample_rows, to64  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    import blockwise_online_softmax_fold_amd as ra

    ra.load()
    return ra


@pytest.fixture(scope="module")
def stress_inputs():
    w = workloads.WORKLOADS[5]
    q, k, v = workloads.make_inputs(w, device="cuda")
    torch.cuda.synchronize()
    return w, q, k, v


def _say(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("i", [0, 15, 31])
def test_rescale_stress_ascending_order(ra, stress_inputs, i):
    w, q, k, v = stress_inputs
    b, P, B, H, d = w.b, w.P, w.B, w.H, w.d
    _say(f"rescale stress, ascending fold order, resident block {i}: {w.describe()}")
    rows = sample_rows(1, b, 128, seed=w.seed + i)  # rows of block i, the same in every (batch, head)
    assert len(rows) == 128
    q_i = q[:, :, i * b:(i + 1) * b]
    rsel = torch.from_numpy(rows).cuda()

    # the oracle's fold loop on the sampled rows, blocks 0, 1, ..., P - 1
    q_s = to64(q_i[:, :, rsel])
    k64, v64 = to64(k), to64(v)
    st = oracle.init_state((B, H), len(rows), d)
    ref_states = []
    for j in range(P):
        st = oracle.fold(st, q_s, k64[:, :, j * b:(j + 1) * b], v64[:, :, j * b:(j + 1) * b])
        ref_states.append(st.copy())
    ms = np.stack([s.m for s in ref_states])  # [P, B, H, rows]
    rises = (ms[1:] > ms[:-1]).sum(axis=0)
    alpha_min = np.exp(ms[:-1] - ms[1:]).min(axis=0)
    print(f"[stress] block {i}: rises per row median {np.median(rises):.0f} (min {rises.min()}, "
          f"max {rises.max()}) of {P - 1} steps; smallest alpha {alpha_min.min():.3g} "
          f"(median over rows {np.median(alpha_min):.3g})", flush=True)
    # the workload is a stress only if most steps rescale most rows
    assert np.median(rises) >= 10, "the running maximum does not rise on most steps"
    assert np.mean(rises >= 8) >= 0.9
    assert alpha_min.min() < 0.2

    # the GPU: the same order through ra_fold_block, state checked every step
    m = torch.empty((B, H, b), device="cuda", dtype=torch.float32)
    l = torch.empty_like(m)
    o = torch.empty((B, H, b, d), device="cuda", dtype=torch.float32)
    ra.ra_state_init(m, l, o)
    gpu_rises = np.zeros((B, H, len(rows)), dtype=np.int64)
    m_prev = None
    for j in range(P):
        ra.ra_fold_block(q_i, k[:, :, j * b:(j + 1) * b], v[:, :, j * b:(j + 1) * b], m, l, o)
        m_s = to64(m[:, :, rsel])
        r = ref_states[j]
        np.testing.assert_allclose(m_s, r.m, rtol=0, atol=2e-4 * (1 + np.abs(r.m).max()), err_msg=f"m, step {j}")
        np.testing.assert_allclose(to64(l[:, :, rsel]), r.l, rtol=1e-2, err_msg=f"l, step {j}")
        check_output(to64(o[:, :, rsel]) / to64(l[:, :, rsel])[..., None], r.o / r.l[..., None], "bf16",
                     f"o/l, step {j}")
        if m_prev is not None:
            gpu_rises += m_s > m_prev
        m_prev = m_s
    # the GPU's stored maximum rose where the oracle's did (up to rounding ties)
    assert np.mean(gpu_rises == rises) >= 0.99
    out = torch.empty_like(q_i)
    ra.ra_finalize(l, o, out)
    torch.cuda.synchronize()
    got = out[:, :, rsel]
    figs = check_output(got, oracle.finalize(ref_states[-1]), "bf16", f"block {i} ascending vs oracle loop")
    dense = np.stack([np.stack([oracle.dense_attention_rows(q_i[bi, hi], k[bi, hi], v[bi, hi], rows)
                                for hi in range(H)]) for bi in range(B)])
    check_output(got, dense, "bf16", f"block {i} ascending vs dense")
    print(f"[parity] stress ascending block {i}: {figs}", flush=True)
