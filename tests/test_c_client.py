"""The ABI from plain C (tests/c/ring_forward_c.c: gcc, C11, no C++, Python or
torch on its side).

CPU: the client compiles against include/ra.h and libra.so and its argument
checks see the library's rejections.  GPU: the in-tree client (built by
__graft_entry__.build()) runs the whole bf16 ring on files the test writes,
and its output is compared with the fp64 oracle.
"""

from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest

from blockwise_online_softmax_fold_amd import build as rabuild


def _have_toolchain() -> bool:
    return shutil.which(os.environ.get("CC", "gcc")) is not None and os.path.exists(
        os.path.join(rabuild.ROCM, "lib", "libamdhip64.so"))


@pytest.mark.skipif(not os.path.exists(rabuild.LIB_PATH), reason="libra.so not built")
@pytest.mark.skipif(not _have_toolchain(), reason="gcc or the HIP runtime library is missing")
def test_c_client_compiles_and_sees_rejections(tmp_path):
    exe = str(tmp_path / "ring_forward_c")
    res = subprocess.run(rabuild.c_client_command(exe), capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe, "check"], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    assert run.stdout.count("rejected") == 2
    assert "P=0" in run.stdout and "head dim" in run.stdout


@pytest.mark.gpu
def test_c_client_ring_forward(tmp_path):
    """B1 H2 N1000 d128 P4 (uneven blocks) bf16 through the C client."""
    import sys

    torch = pytest.importorskip("torch")
    import oracle
    import workloads
    from tests.helpers import check_output

    exe = rabuild.C_CLIENT_PATH
    assert os.path.exists(exe), f"{exe} is missing: run __graft_entry__.build()"
    B, H, N, d, P = 1, 2, 1000, 128, 4
    print(f"\n[case] C client ring forward B={B} H={H} N={N} d={d} P={P}", flush=True)
    sys.stdout.flush()
    q, k, v = workloads.make_small(B, H, N, d, torch.bfloat16, seed=707, device="cuda")
    paths = [str(tmp_path / f"{n}.bin") for n in ("q", "k", "v", "out")]
    for t, path in zip((q, k, v), paths):
        t.contiguous().cpu().view(torch.int16).numpy().tofile(path)
    run = subprocess.run([exe, "run", str(B), str(H), str(N), str(d), str(P), *paths], capture_output=True,
                         text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    raw = np.fromfile(paths[3], dtype=np.int16)
    out = torch.from_numpy(raw).view(torch.bfloat16).reshape(B, H, N, d)
    f64 = lambda t: t.to(torch.float64).cpu().numpy()  # noqa: E731
    ref = oracle.ring_attention(f64(q), f64(k), f64(v), P)
    check_output(f64(out), ref, "bf16", "C client")
