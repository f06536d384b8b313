"""Seeded synthetic workloads shared by the tests, smoke() and bench.py.

Holds the five workload shapes and the input generators only -- none of the
method's arithmetic.  Both the HIP path and the CPU oracle consume the same
tensors produced here; the oracle reads back their exact values.

Recipe (all non-causal, layout [B, H, rows, d], d contiguous):
* one ``torch.Generator`` on the target device, seeded with the workload seed;
  tensors drawn in the order Q, K, V (cfg 5 draws its direction u first),
  head by head, in float32, then rounded to the workload dtype (bf16: round to
  nearest even);
* N(0, 1) entries for Q, K, V unless stated otherwise;
* the rescale-stress workload: Q0, K0 ~ N(0, 1), u a random unit vector,
  K block j += 0.25 j u and Q += sqrt(d) u, so that the expected score of any
  query against block j is raised by 0.25 j; V ~ U(-1, 1);
* when only some query blocks are resident, Q holds just those blocks' rows.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    id: int
    name: str
    B: int
    H: int
    d: int
    N: int
    P: int
    dtype: str  # "f32" or "bf16"
    seed: int
    query_blocks: tuple | None = None  # None: every block is resident
    stress: bool = False
    note: str = ""

    @property
    def b(self) -> int:
        return self.N // self.P

    @property
    def n_q(self) -> int:
        return self.P if self.query_blocks is None else len(self.query_blocks)

    @property
    def resident(self) -> list:
        return list(range(self.P)) if self.query_blocks is None else list(self.query_blocks)

    def flops(self) -> float:
        """4 B H Nq Nk d: two dense products (scores and values) per (query, key) pair."""
        return 4.0 * self.B * self.H * (self.n_q * self.b) * self.N * self.d

    def exps(self) -> float:
        return float(self.B) * self.H * (self.n_q * self.b) * self.N

    def torch_dtype(self):
        import torch

        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def describe(self) -> dict:
        return dict(workload=self.name, B=self.B, H=self.H, d=self.d, N=self.N, P=self.P, b=self.b,
                    resident_query_blocks=self.n_q, dtype=self.dtype, seed=self.seed)


WORKLOADS = {
    1: Workload(1, "tiny-ring-fp32", B=1, H=1, d=64, N=1024, P=4, dtype="f32", seed=1001,
                note="fp32 N(0,1), all 4 query blocks"),
    2: Workload(2, "ring-16k-P8", B=1, H=16, d=128, N=16384, P=8, dtype="bf16", seed=1002,
                note="bf16 N(0,1), all 8 query blocks"),
    3: Workload(3, "ring-128k-P16", B=1, H=32, d=128, N=131072, P=16, dtype="bf16", seed=1003,
                note="bf16 N(0,1), all 16 query blocks, double-buffered hand-off"),
    4: Workload(4, "ring-1M-P64-device0", B=1, H=32, d=128, N=1048576, P=64, dtype="bf16", seed=1004,
                query_blocks=(0,), note="bf16 N(0,1), only query block 0 resident"),
    5: Workload(5, "rescale-stress-d256-P32", B=2, H=8, d=256, N=32768, P=32, dtype="bf16", seed=1005,
                stress=True, note="Q,K ~ N(0,1) + direction u; K block j shifted 0.25 j; V ~ U(-1,1)"),
}


def make_generator(seed: int, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, gen, device, dtype):
    """float32 N(0, 1) drawn head by head (bounded temporaries), rounded to dtype."""
    import torch

    B, H, rows, d = shape
    out = torch.empty(shape, dtype=dtype, device=device)
    for bi in range(B):
        for hi in range(H):
            out[bi, hi] = torch.randn((rows, d), generator=gen, device=device, dtype=torch.float32).to(dtype)
    return out


def make_inputs(w: Workload, device="cuda", dtype=None):
    """Q, K, V of workload ``w`` on ``device``.  Q has the resident rows only."""
    import torch

    dtype = dtype or w.torch_dtype()
    gen = make_generator(w.seed, device)
    B, H, N, d, b = w.B, w.H, w.N, w.d, w.b
    q_rows = w.n_q * b
    if not w.stress:
        q_full = _normal((B, H, q_rows, d), gen, device, dtype)
        k = _normal((B, H, N, d), gen, device, dtype)
        v = _normal((B, H, N, d), gen, device, dtype)
        return q_full, k, v
    u = torch.randn((d,), generator=gen, device=device, dtype=torch.float32)
    u = u / torch.linalg.vector_norm(u)
    q = torch.empty((B, H, q_rows, d), dtype=dtype, device=device)
    k = torch.empty((B, H, N, d), dtype=dtype, device=device)
    v = torch.empty((B, H, N, d), dtype=dtype, device=device)
    shift = (0.25 * torch.arange(w.P, device=device, dtype=torch.float32)).repeat_interleave(b)  # [N]
    for bi in range(B):
        for hi in range(H):
            q0 = torch.randn((q_rows, d), generator=gen, device=device, dtype=torch.float32)
            q[bi, hi] = (q0 + math.sqrt(d) * u).to(dtype)
    for bi in range(B):
        for hi in range(H):
            k0 = torch.randn((N, d), generator=gen, device=device, dtype=torch.float32)
            k[bi, hi] = (k0 + shift[:, None] * u).to(dtype)
    for bi in range(B):
        for hi in range(H):
            v[bi, hi] = (torch.rand((N, d), generator=gen, device=device, dtype=torch.float32) * 2 - 1).to(dtype)
    return q, k, v


def make_small(B, H, N, d, dtype, seed, device="cuda", q_rows=None, scale=1.0):
    """Generic seeded N(0, scale^2) inputs for parity cases of arbitrary shape."""
    import torch

    gen = make_generator(seed, device)
    q_rows = N if q_rows is None else q_rows
    q = (torch.randn((B, H, q_rows, d), generator=gen, device=device) * scale).to(dtype)
    k = (torch.randn((B, H, N, d), generator=gen, device=device) * scale).to(dtype)
    v = torch.randn((B, H, N, d), generator=gen, device=device).to(dtype)
    return q, k, v
