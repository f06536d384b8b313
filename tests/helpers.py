"""Shared test helpers: tolerance checks and oracle sampling."""

from __future__ import annotations

import math

import numpy as np

# bf16 inputs: max-abs and mean-abs error of the output against the fp64 oracle
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
# fp32 inputs: norm-wise relative error  max|O - O_ref| <= 1e-5 max|O_ref|
F32_REL = 1e-5


def to64(t) -> np.ndarray:
    import torch

    return t.detach().to("cpu", torch.float64).numpy()


def check_output(got, ref: np.ndarray, dtype: str, what: str = "") -> dict:
    """Assert the workload tolerance; return the error figures."""
    g = to64(got) if not isinstance(got, np.ndarray) else got
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    figs = dict(max_abs=float(err.max()), mean_abs=float(err.mean()), ref_max=float(np.abs(ref).max()))
    if dtype == "bf16":
        assert figs["max_abs"] <= BF16_MAX_ABS, f"{what}: max-abs {figs['max_abs']:.3g} > {BF16_MAX_ABS}"
        assert figs["mean_abs"] <= BF16_MEAN_ABS, f"{what}: mean-abs {figs['mean_abs']:.3g} > {BF16_MEAN_ABS}"
    else:
        bound = F32_REL * figs["ref_max"]
        assert figs["max_abs"] <= bound, f"{what}: max-abs {figs['max_abs']:.3g} > 1e-5 * max|ref| = {bound:.3g}"
    return figs


def sample_rows(n_blocks: int, b: int, per_block: int, seed: int) -> np.ndarray:
    """Seeded row sample: ``per_block`` rows of every block, always including
    each block's first and last row, sorted."""
    rng = np.random.default_rng(seed)
    rows = []
    for i in range(n_blocks):
        k = min(per_block, b)
        pick = set([0, b - 1]) if k >= 2 else {0}
        rest = rng.choice(b, size=k, replace=False)
        for r in rest:
            if len(pick) >= k:
                break
            pick.add(int(r))
        rows.extend(i * b + r for r in sorted(pick))
    return np.array(rows, dtype=np.int64)


def oracle_rows(q, k, v, rows: np.ndarray, heads=None, scale=None) -> np.ndarray:
    """fp64 dense attention for the chosen rows of q (all batches, chosen
    heads), head by head to bound host memory.  Returns [B, len(heads), rows, d]."""
    import oracle

    B, H = q.shape[0], q.shape[1]
    heads = list(range(H)) if heads is None else list(heads)
    out = np.empty((B, len(heads), len(rows), v.shape[-1]))
    for bi in range(B):
        for n, hi in enumerate(heads):
            out[bi, n] = oracle.dense_attention_rows(q[bi, hi], k[bi, hi], v[bi, hi], rows, scale=scale)
    return out


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def check_grad(got, ref: np.ndarray, dtype: str, what: str = "") -> dict:
    """Gradient parity, norm-wise: the output bars scaled by the gradient's own
    magnitude (a gradient has no fixed scale, unlike O, a convex combination of
    V rows): bf16 max|err| <= 2e-2 max|ref| and mean|err| <= 2e-3 max|ref|;
    fp32 max|err| <= 1e-5 max|ref|."""
    g = to64(got) if not isinstance(got, np.ndarray) else got
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    err = np.abs(g - ref)
    scale = float(np.abs(ref).max())
    figs = dict(max_abs=float(err.max()), mean_abs=float(err.mean()), ref_max=scale)
    if scale == 0.0:
        assert figs["max_abs"] == 0.0, f"{what}: expected zeros"
        return figs
    if dtype == "bf16":
        assert figs["max_abs"] <= BF16_MAX_ABS * scale, f"{what}: max-abs {figs['max_abs']:.3g} > 2e-2 * {scale:.3g}"
        assert figs["mean_abs"] <= BF16_MEAN_ABS * scale, f"{what}: mean-abs {figs['mean_abs']:.3g} > 2e-3 * {scale:.3g}"
    else:
        assert figs["max_abs"] <= F32_REL * scale, f"{what}: max-abs {figs['max_abs']:.3g} > 1e-5 * {scale:.3g}"
    return figs
