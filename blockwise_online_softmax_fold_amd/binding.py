"""ctypes binding of libra.so (include/ra.h), with the same entry-point names.

This layer only marshals arguments: torch tensors become device pointers and
element strides, the current torch stream becomes the hipStream_t.  Every step
of the computation runs in the library's HIP kernels.  If the library is not
built, every call raises; nothing falls back to another implementation.
"""

from __future__ import annotations

import ctypes
import os
from typing import Sequence

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libra.so")
_lib = None

RA_OK = 0
RA_E_INVALID_ARG = 1
RA_E_UNSUPPORTED = 2
RA_E_HIP = 3
RA_E_OOM = 4
RA_DTYPE_F32 = 0
RA_DTYPE_BF16 = 1
RA_CAUSAL_NONE = 0
RA_CAUSAL_CONTIGUOUS = 1
RA_CAUSAL_STRIPED = 2
RA_CAUSAL_ZIGZAG = 3

#: token layouts of a causal ring by name (None: full attention)
CAUSAL_LAYOUTS = {None: RA_CAUSAL_NONE, "contiguous": RA_CAUSAL_CONTIGUOUS, "striped": RA_CAUSAL_STRIPED,
                  "zigzag": RA_CAUSAL_ZIGZAG}

#: every symbol include/ra.h declares
EXPORTED = (
    "ra_state_init",
    "ra_fold_block",
    "ra_fold_block_causal",
    "ra_finalize",
    "ra_ring_workspace_bytes",
    "ra_ring_forward",
    "ra_ring_forward_noalloc",
    "ra_ring_forward_causal",
    "ra_ring_forward_ex",
    "ra_ring_backward_workspace_bytes",
    "ra_ring_backward",
    "ra_last_error",
    "ra_version",
    "ra_profile_folds",
    "ra_profile_read",
)

_STATUS_NAMES = {0: "RA_OK", 1: "RA_E_INVALID_ARG", 2: "RA_E_UNSUPPORTED", 3: "RA_E_HIP", 4: "RA_E_OOM"}


class RaError(RuntimeError):
    """A non-zero ra_status_t; ``status`` holds the code, the message ra_last_error()."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libra.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m blockwise_online_softmax_fold_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation"
        )
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, f32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    strides = ctypes.POINTER(ctypes.c_int64)
    lib.ra_state_init.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp]
    lib.ra_state_init.restype = ctypes.c_int
    lib.ra_fold_block.argtypes = [vp, strides, vp, strides, vp, strides, ctypes.c_int, i64, i64, i64, i64, i64, f32,
                                  vp, vp, vp, vp]
    lib.ra_fold_block.restype = ctypes.c_int
    lib.ra_fold_block_causal.argtypes = [vp, strides, vp, strides, vp, strides, ctypes.c_int, i64, i64, i64, i64,
                                         f32, ctypes.c_int, i32, i32, i32, vp, vp, vp, vp]  # (..., B, H, N, d, ...)
    lib.ra_fold_block_causal.restype = ctypes.c_int
    lib.ra_finalize.argtypes = [vp, vp, vp, strides, ctypes.c_int, i64, i64, i64, i64, vp]
    lib.ra_finalize.restype = ctypes.c_int
    lib.ra_ring_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i64, i64, i32, i32]
    lib.ra_ring_workspace_bytes.restype = sz
    lib.ra_ring_forward.argtypes = [vp, strides, vp, strides, vp, strides, vp, strides, ctypes.c_int, i64, i64, i64,
                                    i64, i32, ctypes.POINTER(ctypes.c_int32), i32, f32, vp, sz, vp]
    lib.ra_ring_forward.restype = ctypes.c_int
    lib.ra_ring_forward_noalloc.argtypes = [vp, strides, vp, strides, vp, strides, vp, strides, ctypes.c_int, i64,
                                            i64, i64, i64, i32, ctypes.POINTER(ctypes.c_int32), i32, f32, vp]
    lib.ra_ring_forward_noalloc.restype = ctypes.c_int
    lib.ra_ring_forward_causal.argtypes = [vp, strides, vp, strides, vp, strides, vp, strides, ctypes.c_int, i64,
                                           i64, i64, i64, i32, ctypes.POINTER(ctypes.c_int32), i32, f32,
                                           ctypes.c_int, vp, sz, vp]
    lib.ra_ring_forward_causal.restype = ctypes.c_int
    lib.ra_ring_forward_ex.argtypes = [vp, strides, vp, strides, vp, strides, vp, strides, vp, ctypes.c_int, i64, i64,
                                       i64, i64, i32, ctypes.POINTER(ctypes.c_int32), i32, f32, ctypes.c_int, vp, sz,
                                       vp]
    lib.ra_ring_forward_ex.restype = ctypes.c_int
    lib.ra_ring_backward_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i64, i64, i32, i32]
    lib.ra_ring_backward_workspace_bytes.restype = sz
    lib.ra_ring_backward.argtypes = [vp, strides, vp, strides, vp, strides, vp, strides, vp, strides, vp, vp, strides,
                                     vp, strides, vp, strides, ctypes.c_int, i64, i64, i64, i64, i32,
                                     ctypes.POINTER(ctypes.c_int32), i32, f32, ctypes.c_int, vp, sz, vp]
    lib.ra_ring_backward.restype = ctypes.c_int
    lib.ra_last_error.argtypes = []
    lib.ra_last_error.restype = ctypes.c_char_p
    lib.ra_version.argtypes = []
    lib.ra_version.restype = ctypes.c_char_p
    lib.ra_profile_folds.argtypes = [ctypes.c_int]
    lib.ra_profile_folds.restype = ctypes.c_int
    lib.ra_profile_read.argtypes = [ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    lib.ra_profile_read.restype = ctypes.c_int
    _lib = lib
    return lib


def ra_last_error() -> str:
    return load().ra_last_error().decode()


def ra_version() -> str:
    return load().ra_version().decode()


def _check(status: int) -> None:
    if status != RA_OK:
        raise RaError(status, ra_last_error())


# ---------------------------------------------------------------------------
# torch marshalling helpers


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return RA_DTYPE_BF16
    if t.dtype == torch.float32:
        return RA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _strides(t):
    """Element strides {batch, head, row} of a [B, H, rows, d] tensor."""
    if t.dim() != 4:
        raise ValueError(f"expected a [B, H, rows, d] tensor, got shape {tuple(t.shape)}")
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError("the last (d) axis must be contiguous")
    return (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))


def _dev(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _state_ok(m, l, o):
    import torch

    for name, t in (("m", m), ("l", l), ("o", o)):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"state {name} must be a contiguous float32 tensor")


# ---------------------------------------------------------------------------
# entry points


def ra_state_init(m, l, o, stream=None) -> None:
    """(m, l, o) = (-inf, 0, 0).  m, l: [B, H, rows]; o: [B, H, rows, d]."""
    _state_ok(m, l, o)
    B, H, rows, d = o.shape
    _check(load().ra_state_init(_dev(m, "m"), _dev(l, "l"), _dev(o, "o"), B, H, rows, d, _stream(stream)))


def ra_fold_block(q, k, v, m, l, o, scale: float = 0.0, stream=None) -> None:
    """Fold one visiting block (k, v: [B, H, kv_rows, d]) into the state of q's rows."""
    _state_ok(m, l, o)
    B, H, q_rows, d = q.shape
    kv_rows = k.shape[2]
    if k.shape != v.shape or k.shape[:2] != q.shape[:2] or k.shape[3] != d:
        raise ValueError(f"shapes q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)} do not match")
    if tuple(o.shape) != (B, H, q_rows, d) or tuple(m.shape) != (B, H, q_rows) or tuple(l.shape) != (B, H, q_rows):
        raise ValueError("state shapes do not match q")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must have one dtype")
    _check(load().ra_fold_block(
        _dev(q, "q"), _strides(q), _dev(k, "k"), _strides(k), _dev(v, "v"), _strides(v), _dtype_code(q),
        B, H, q_rows, kv_rows, d, float(scale), _dev(m, "m"), _dev(l, "l"), _dev(o, "o"), _stream(stream)))


def _layout_code(layout) -> int:
    if isinstance(layout, int):
        return layout
    if layout not in CAUSAL_LAYOUTS:
        raise ValueError(f"unknown causal layout {layout!r}: use one of {sorted(k for k in CAUSAL_LAYOUTS if k)}")
    return CAUSAL_LAYOUTS[layout]


def block_sizes(N: int, P: int) -> list:
    """Rows of each device's block: N // P, one more for the first N % P."""
    return [N // P + (1 if j < N % P else 0) for j in range(P)]


def ra_fold_block_causal(q, k, v, m, l, o, layout, P: int, q_block: int, kv_block: int, N: int | None = None,
                         scale: float = 0.0, stream=None) -> None:
    """Fold device kv_block's block into device q_block's state under the causal
    mask of a P-device ring over N tokens in ``layout`` ("contiguous",
    "striped", "zigzag"); q: [B, H, n_qblock, d], k, v: [B, H, n_kvblock, d].
    N defaults to P * rows when q and k have the same row count."""
    _state_ok(m, l, o)
    B, H, rows, d = q.shape
    if N is None:
        if k.shape[2] != rows:
            raise ValueError("N is needed when the two blocks differ in size")
        N = P * rows
    if P >= 1 and N >= P and 0 <= q_block < P and 0 <= kv_block < P:
        sizes = block_sizes(N, P)
        if rows != sizes[q_block] or k.shape[2] != sizes[kv_block]:
            raise ValueError(f"blocks {q_block} and {kv_block} of N={N} over P={P} have {sizes[q_block]} and "
                             f"{sizes[kv_block]} rows; q has {rows}, k has {k.shape[2]}")
    if k.shape != v.shape or k.shape[:2] != q.shape[:2] or k.shape[3] != d:
        raise ValueError(f"shapes q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)} do not match")
    if tuple(o.shape) != (B, H, rows, d) or tuple(m.shape) != (B, H, rows) or tuple(l.shape) != (B, H, rows):
        raise ValueError("state shapes do not match q")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must have one dtype")
    _check(load().ra_fold_block_causal(
        _dev(q, "q"), _strides(q), _dev(k, "k"), _strides(k), _dev(v, "v"), _strides(v), _dtype_code(q),
        B, H, int(N), d, float(scale), _layout_code(layout), int(P), int(q_block), int(kv_block),
        _dev(m, "m"), _dev(l, "l"), _dev(o, "o"), _stream(stream)))


def ra_finalize(l, o, out, stream=None) -> None:
    """out = o / l (0 where l == 0), cast to out's dtype."""
    B, H, rows, d = o.shape
    _check(load().ra_finalize(_dev(l, "l"), _dev(o, "o"), _dev(out, "out"), _strides(out), _dtype_code(out),
                              B, H, rows, d, _stream(stream)))


def ra_ring_workspace_bytes(dtype, B: int, H: int, N: int, d: int, P: int, n_q: int) -> int:
    import torch

    code = RA_DTYPE_BF16 if dtype == torch.bfloat16 else RA_DTYPE_F32 if dtype == torch.float32 else -1
    return int(load().ra_ring_workspace_bytes(code, B, H, N, d, P, n_q))


def ra_ring_forward(q, k, v, P: int, query_blocks: Sequence[int] | None = None, out=None, scale: float = 0.0,
                    workspace=None, stream=None):
    """The whole ring for the resident query blocks; returns out ([B, H, n_q*b, d])."""
    return _ring(q, k, v, P, query_blocks, out, scale, workspace, stream, None)


#: bytes of the static scratch ra_ring_forward_noalloc runs in (RA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


def ra_ring_forward_noalloc(q, k, v, P: int, query_blocks: Sequence[int] | None = None, out=None,
                            scale: float = 0.0, stream=None):
    """ra_ring_forward in the library's static device scratch: allocates
    nothing (``out`` must then be given by a caller that cannot allocate).
    Rings needing more than NOALLOC_SCRATCH_BYTES of workspace are refused."""
    return _ring(q, k, v, P, query_blocks, out, scale, None, stream, None, noalloc=True)


def ra_ring_forward_causal(q, k, v, P: int, layout, query_blocks: Sequence[int] | None = None, out=None,
                           scale: float = 0.0, workspace=None, stream=None):
    """The causal ring: q, k, v in ``layout``'s device order; returns out."""
    return _ring(q, k, v, P, query_blocks, out, scale, workspace, stream, layout)


def ra_ring_forward_ex(q, k, v, P: int, layout=None, query_blocks: Sequence[int] | None = None, out=None, lse=None,
                       scale: float = 0.0, workspace=None, stream=None):
    """The ring forward (causal when ``layout`` is given) that also returns each
    resident row's log-sum-exp: (out, lse), lse float32 [B, H, rows]."""
    import torch

    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must be a contiguous float32 [B, H, rows] tensor")
    out = _ring(q, k, v, P, query_blocks, out, scale, workspace, stream, layout, lse=lse)
    return out, lse


def ra_ring_backward_workspace_bytes(dtype, B: int, H: int, N: int, d: int, P: int, n_q: int) -> int:
    import torch

    code = RA_DTYPE_BF16 if dtype == torch.bfloat16 else RA_DTYPE_F32 if dtype == torch.float32 else -1
    return int(load().ra_ring_backward_workspace_bytes(code, B, H, N, d, P, n_q))


def ra_ring_backward(q, k, v, out, dout, lse, P: int, layout=None, query_blocks: Sequence[int] | None = None,
                     dq=None, dk=None, dv=None, scale: float = 0.0, workspace=None, stream=None):
    """Gradients on the ring: (dq, dk, dv).  q, k, v, P, layout, query_blocks and
    scale as given to the forward; out, lse from ra_ring_forward_ex; dout like
    out.  dk, dv hold the resident blocks' shares (full gradients when every
    block is resident)."""
    import torch

    B, H, N, d = k.shape
    _ring_shape_check(q, k, v, P, query_blocks)
    for name, t in (("out", out), ("dout", dout)):
        if t.shape != q.shape:
            raise ValueError(f"{name} must have q's shape")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must be a contiguous float32 [B, H, rows] tensor")
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype):
        raise TypeError("q, k, v, out and dout must have one dtype")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("dq, dk, dv must have the shapes of q, k, v")
    n_q = P if query_blocks is None else len(query_blocks)
    qb = None if query_blocks is None else (ctypes.c_int32 * max(1, n_q))(*[int(x) for x in query_blocks])
    ws_ptr, ws_bytes = ctypes.c_void_p(None), 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    _check(load().ra_ring_backward(
        _dev(q, "q"), _strides(q), _dev(k, "k"), _strides(k), _dev(v, "v"), _strides(v), _dev(out, "out"),
        _strides(out), _dev(dout, "dout"), _strides(dout), _dev(lse, "lse"), _dev(dq, "dq"), _strides(dq),
        _dev(dk, "dk"), _strides(dk), _dev(dv, "dv"), _strides(dv), _dtype_code(q), B, H, N, d, int(P), qb, n_q,
        float(scale), _layout_code(layout), ws_ptr, ws_bytes, _stream(stream)))
    return dq, dk, dv


def _ring_shape_check(q, k, v, P, query_blocks):
    B, H, N, d = k.shape
    if v.shape != k.shape:
        raise ValueError("k and v must have the same shape")
    if 1 <= P <= N:
        sizes = block_sizes(N, P)
        qb = range(P) if query_blocks is None else query_blocks
        rows = sum(sizes[i] for i in qb if 0 <= i < P)
        if q.shape[:2] != k.shape[:2] or q.shape[3] != d or q.shape[2] != rows:
            raise ValueError(f"q must be [B, H, rows of the resident blocks, d] = [{B}, {H}, {rows}, {d}], "
                             f"got {tuple(q.shape)}")


def _ring(q, k, v, P, query_blocks, out, scale, workspace, stream, layout, lse=None, noalloc=False):
    import torch

    B, H, N, d = k.shape
    _ring_shape_check(q, k, v, P, query_blocks)
    n_q = P if query_blocks is None else len(query_blocks)
    if out is not None and out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if out is None:
        out = torch.empty_like(q)
    qb = None
    if query_blocks is not None:
        qb = (ctypes.c_int32 * max(1, n_q))(*[int(x) for x in query_blocks])
    ws_ptr, ws_bytes = ctypes.c_void_p(None), 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    if not (q.dtype == k.dtype == v.dtype == out.dtype):
        raise TypeError("q, k, v and out must have one dtype")
    args = (_dev(q, "q"), _strides(q), _dev(k, "k"), _strides(k), _dev(v, "v"), _strides(v), _dev(out, "out"),
            _strides(out), _dtype_code(q), B, H, N, d, int(P), qb, n_q, float(scale))
    if noalloc:
        _check(load().ra_ring_forward_noalloc(*args, _stream(stream)))
    elif lse is not None:
        _check(load().ra_ring_forward_ex(*args[:8], _dev(lse, "lse"), *args[8:], _layout_code(layout), ws_ptr,
                                         ws_bytes, _stream(stream)))
    elif layout is None:
        _check(load().ra_ring_forward(*args, ws_ptr, ws_bytes, _stream(stream)))
    else:
        _check(load().ra_ring_forward_causal(*args, _layout_code(layout), ws_ptr, ws_bytes, _stream(stream)))
    return out


def ra_profile_folds(enable: bool) -> None:
    """Time every fold launch of ra_ring_forward with HIP events on its stream."""
    _check(load().ra_profile_folds(1 if enable else 0))


def ra_profile_read():
    """(launches, total_ms, max_ms) of the fold launches timed since the last read."""
    n, tot, mx = ctypes.c_int64(), ctypes.c_double(), ctypes.c_double()
    _check(load().ra_profile_read(ctypes.byref(n), ctypes.byref(tot), ctypes.byref(mx)))
    return int(n.value), float(tot.value), float(mx.value)
