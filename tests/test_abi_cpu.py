"""The C ABI without a GPU: the library loads, exports every symbol
include/ra.h declares, and rejects bad arguments on the host before any HIP
call (so these run in a GPU-less container)."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ra.h")


@pytest.fixture(scope="module")
def lib():
    import blockwise_online_softmax_fold_amd as ra

    if not os.path.exists(ra.lib_path()):
        from blockwise_online_softmax_fold_amd import build

        build.build()
    return ra.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    import blockwise_online_softmax_fold_amd as ra

    assert _declared() == sorted(ra.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    # and nothing of the kernels' internals leaks
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert {n for n in exported if n.startswith("ra_")} == set(_declared())


def test_version(lib):
    assert re.match(r"^\d+\.\d+\.\d+$", lib.ra_version().decode())


# fake, well-aligned device addresses: every call below must fail validation
# before it could use them
A = ctypes.c_void_p(0x10000)
S_BF16 = (ctypes.c_int64 * 3)(16 * 1024 * 128, 1024 * 128, 128)
BF16, F32 = 1, 0


def _fold(lib, q=A, qs=S_BF16, k=A, ks=S_BF16, v=A, vs=S_BF16, dt=BF16, B=1, H=16, q_rows=1024, kv_rows=1024,
          d=128, scale=0.0, m=A, l=A, o=A):
    return lib.ra_fold_block(q, qs, k, ks, v, vs, dt, B, H, q_rows, kv_rows, d, ctypes.c_float(scale), m, l, o, None)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(q=ctypes.c_void_p(None)), 1, "q is NULL"),
    (dict(k=ctypes.c_void_p(0x10008)), 1, "16-byte aligned"),
    (dict(d=96), 2, "head dim"),
    (dict(dt=7), 1, "dtype"),
    (dict(B=0), 1, "must be >= 1"),
    (dict(q_rows=-1), 1, ">= 0"),
    (dict(scale=-1.0), 1, "scale"),
    (dict(scale=float("nan")), 1, "scale"),
    (dict(vs=(ctypes.c_int64 * 3)(16, 8, 4)), 1, "multiple of 8"),
    (dict(m=ctypes.c_void_p(None)), 1, "NULL"),
    (dict(o=ctypes.c_void_p(0x10004)), 1, "o is not 16-byte aligned"),
    (dict(ks=(ctypes.c_int64 * 3)(1 << 35, 1 << 34, 1 << 24)), 2, "k row stride"),
    (dict(vs=(ctypes.c_int64 * 3)(1 << 35, 1 << 34, 1 << 24)), 2, "v row stride"),
])
def test_fold_block_rejects(lib, kwargs, status, needle):
    assert _fold(lib, **kwargs) == status
    assert needle in lib.ra_last_error().decode()


def test_fold_block_empty_is_ok_without_gpu(lib):
    N = ctypes.c_void_p(None)
    assert _fold(lib, q_rows=0) == 0
    assert _fold(lib, q_rows=0, q=N, k=N, v=N, m=N, l=N, o=N) == 0
    assert _fold(lib, kv_rows=0) == 0
    assert _fold(lib, kv_rows=0, k=N, v=N) == 0
    assert lib.ra_last_error().decode() == ""
    assert _fold(lib, kv_rows=0, q=N) == 1  # query rows still need q


def _ring(lib, dt=BF16, B=1, H=32, N=131072, d=128, P=16, qb=None, n_q=16, scale=0.0, ws=None, ws_bytes=0,
          q=A, out=A):
    qbp = None if qb is None else (ctypes.c_int32 * len(qb))(*qb)
    return lib.ra_ring_forward(q, S_BF16, A, S_BF16, A, S_BF16, out, S_BF16, dt, B, H, N, d, P, qbp, n_q,
                               ctypes.c_float(scale), ws if ws is not None else ctypes.c_void_p(None), ws_bytes,
                               None)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(P=0), 1, "P=0"),
    (dict(N=8, P=16), 1, ">= P"),
    (dict(n_q=4), 1, "n_q=4 != P=16"),
    (dict(qb=[0, 16], n_q=2), 1, "outside"),
    (dict(qb=[-1], n_q=1), 1, "outside"),
    (dict(d=32), 2, "head dim"),
    (dict(out=ctypes.c_void_p(None)), 1, "out is NULL"),
    (dict(ws=ctypes.c_void_p(0x10000), ws_bytes=1024), 1, "smaller than"),
    (dict(scale=float("inf")), 1, "scale"),
])
def test_ring_forward_rejects(lib, kwargs, status, needle):
    assert _ring(lib, **kwargs) == status
    assert needle in lib.ra_last_error().decode()


def test_ring_workspace_is_two_blocks_not_P(lib):
    """Math page, "Memory": besides its own shard a device holds at most two
    visiting K/V blocks, whatever P is."""
    B, H, d, n_q = 1, 8, 128, 1
    sizes = {}
    for P in (1, 2, 4, 16, 64):
        b = 4096
        N = b * P
        sizes[P] = lib.ra_ring_workspace_bytes(BF16, B, H, N, d, P, n_q)
        state = B * H * b * (d + 2) * 4
        blocks = min(2, P - 1) * 2 * B * H * b * d * 2  # K and V, bf16
        assert state + blocks <= sizes[P] <= state + blocks + 5 * 256
    assert sizes[4] == sizes[16] == sizes[64]
    assert lib.ra_ring_workspace_bytes(BF16, 1, 1, 8, 128, 16, 1) == 0  # rejected shape: N < P


def test_ring_workspace_uneven_blocks(lib):
    """N not a multiple of P: every slot and state row is sized for the
    longest block, N // P + 1 rows."""
    B, H, d, n_q = 1, 2, 64, 3
    even = lib.ra_ring_workspace_bytes(BF16, B, H, 16 * 4097, d, 16, n_q)
    uneven = lib.ra_ring_workspace_bytes(BF16, B, H, 16 * 4096 + 5, d, 16, n_q)
    assert uneven == even > 0


def test_state_init_and_finalize_reject(lib):
    assert lib.ra_state_init(A, A, ctypes.c_void_p(0x10004), 1, 1, 4, 64, None) == 1
    assert lib.ra_state_init(A, A, A, 1, 1, 4, 48, None) == 2
    assert lib.ra_state_init(A, A, A, 1, 1, 0, 64, None) == 0
    assert lib.ra_finalize(A, A, ctypes.c_void_p(None), S_BF16, BF16, 1, 1, 4, 64, None) == 1
    assert lib.ra_finalize(A, A, A, S_BF16, 9, 1, 1, 4, 64, None) == 1


def _fold_causal(lib, layout=1, P=4, qb=0, kb=0, N=4096, dt=BF16, d=128, q=A, k=A, m=A):
    return lib.ra_fold_block_causal(q, S_BF16, k, S_BF16, A, S_BF16, dt, 1, 16, N, d, ctypes.c_float(0.0),
                                    layout, P, qb, kb, m, A, A, None)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(layout=9), 1, "unknown causal layout"),
    (dict(layout=-1), 1, "unknown causal layout"),
    (dict(P=0), 1, "P=0"),
    (dict(qb=4), 1, "must lie in [0, P=4)"),
    (dict(kb=-1), 1, "must lie in [0, P=4)"),
    (dict(N=3), 1, "N=3 must be >= P=4"),
    (dict(layout=3, N=4100), 1, "multiple of 2P"),
    (dict(layout=2, P=1024, N=1 << 31), 2, "do not fit 32 bits"),
    (dict(q=ctypes.c_void_p(None)), 1, "q is NULL"),
    (dict(m=ctypes.c_void_p(None)), 1, "NULL"),
    (dict(d=80), 2, "head dim"),
])
def test_fold_block_causal_rejects(lib, kwargs, status, needle):
    assert _fold_causal(lib, **kwargs) == status
    assert needle in lib.ra_last_error().decode()


def test_fold_block_causal_uneven_blocks_are_checked_on_host(lib):
    # N = 4097 over P = 4: block 0 has 1025 rows, the others 1024 -- still host-side
    # validation only: a NULL q is caught before any GPU work
    assert _fold_causal(lib, N=4097, qb=0, kb=3, q=ctypes.c_void_p(None)) == 1
    assert "q is NULL" in lib.ra_last_error().decode()
    assert _fold_causal(lib, layout=0, N=4097, qb=1, kb=2, m=ctypes.c_void_p(None)) == 1


def _ring_causal(lib, layout=1, N=131072, P=16, n_q=16, d=128):
    return lib.ra_ring_forward_causal(A, S_BF16, A, S_BF16, A, S_BF16, A, S_BF16, BF16, 1, 32, N, d, P, None, n_q,
                                      ctypes.c_float(0.0), layout, ctypes.c_void_p(None), 0, None)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(layout=4), 1, "unknown causal layout"),
    (dict(layout=3, N=16 * 1001), 1, "multiple of 2P"),
    (dict(layout=3, N=16 * 1000 + 3), 1, "multiple of 2P"),
    (dict(layout=1, N=10), 1, ">= P"),
    (dict(layout=2, d=48), 2, "head dim"),
])
def test_ring_forward_causal_rejects(lib, kwargs, status, needle):
    assert _ring_causal(lib, **kwargs) == status
    assert needle in lib.ra_last_error().decode()


def _bwd(lib, lse=A, dout=A, layout=0, N=4096, P=4, ws=None, ws_bytes=0, d=128, qs=S_BF16, ds=S_BF16):
    S = S_BF16
    return lib.ra_ring_backward(A, qs, A, S, A, S, A, S, dout, ds, lse, A, S, A, S, A, S, BF16, 1, 16, N, d, P, None,
                                P, ctypes.c_float(0.0), layout, ws if ws is not None else ctypes.c_void_p(None),
                                ws_bytes, None)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(lse=ctypes.c_void_p(None)), 1, "lse is NULL"),
    (dict(lse=ctypes.c_void_p(0x10002)), 1, "lse is not 4-byte aligned"),
    (dict(dout=ctypes.c_void_p(None)), 1, "dout is NULL"),
    (dict(layout=7), 1, "unknown causal layout"),
    (dict(layout=3, N=4100), 1, "multiple of 2P"),
    (dict(d=96), 2, "head dim"),
    (dict(ws=ctypes.c_void_p(0x10000), ws_bytes=4096), 1, "smaller than"),
    # Q and dO rows are streamed through LDS tiles in the dK/dV kernel
    (dict(qs=(ctypes.c_int64 * 3)(1 << 35, 1 << 34, 1 << 24)), 2, "q row stride"),
    (dict(ds=(ctypes.c_int64 * 3)(1 << 35, 1 << 34, 1 << 24)), 2, "dout row stride"),
])
def test_ring_backward_rejects(lib, kwargs, status, needle):
    assert _bwd(lib, **kwargs) == status
    assert needle in lib.ra_last_error().decode()


def test_ring_backward_rejects_repeated_blocks(lib):
    """Two residents of one block would race on that block's dK/dV
    accumulators; the backward refuses them (the forward allows them)."""
    S = S_BF16
    P = 4
    for qb in ((1, 1), (0, 2, 3, 2)):
        arr = (ctypes.c_int32 * len(qb))(*qb)
        st = lib.ra_ring_backward(A, S, A, S, A, S, A, S, A, S, A, A, S, A, S, A, S, BF16, 1, 16, 4096, 128, P, arr,
                                  len(qb), ctypes.c_float(0.0), 0, ctypes.c_void_p(None), 0, None)
        assert st == 1
        assert "repeats a block" in lib.ra_last_error().decode()


def test_ring_backward_workspace_size(lib):
    B, H, N, d, P = 1, 2, 1000, 64, 3
    got = lib.ra_ring_backward_workspace_bytes(BF16, B, H, N, d, P, P)
    rows = P * (N // P + 1)
    need = 2 * B * H * rows * 4 + B * H * rows * d * 4 + 2 * B * H * N * d * 4
    assert need <= got <= need + 5 * 256
    assert lib.ra_ring_backward_workspace_bytes(BF16, B, H, 2, d, 3, 3) == 0  # N < P


def test_ring_forward_ex_rejects_misaligned_lse(lib):
    st = lib.ra_ring_forward_ex(A, S_BF16, A, S_BF16, A, S_BF16, A, S_BF16, ctypes.c_void_p(0x10001), BF16, 1, 32,
                                131072, 128, 16, None, 16, ctypes.c_float(0.0), 0, ctypes.c_void_p(None), 0, None)
    assert st == 1 and "lse" in lib.ra_last_error().decode()


def test_noalloc_refuses_rings_beyond_its_scratch_on_the_host(lib):
    """ra_ring_forward_noalloc runs in a static scratch of RA_NOALLOC_SCRATCH_BYTES
    (64 MiB); a ring needing more workspace is refused before any HIP call."""
    import blockwise_online_softmax_fold_amd as ra

    assert ra.NOALLOC_SCRATCH_BYTES == 64 << 20
    text = open(HEADER).read()
    assert "#define RA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text
    need = lib.ra_ring_workspace_bytes(BF16, 1, 16, 16384, 128, 8, 8)
    assert need > ra.NOALLOC_SCRATCH_BYTES
    st = lib.ra_ring_forward_noalloc(A, S_BF16, A, S_BF16, A, S_BF16, A, S_BF16, BF16, 1, 16, 16384, 128, 8, None, 8,
                                     ctypes.c_float(0.0), None)
    assert st == 1
    assert "static scratch" in lib.ra_last_error().decode()
    # and argument checks come first, as in ra_ring_forward
    st = lib.ra_ring_forward_noalloc(A, S_BF16, A, S_BF16, A, S_BF16, A, S_BF16, BF16, 1, 16, 16384, 96, 8, None, 8,
                                     ctypes.c_float(0.0), None)
    assert st == 2 and "head dim" in lib.ra_last_error().decode()
