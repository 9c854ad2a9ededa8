"""MI355X (gfx950) selective-scan forward (S6): a thin Python binding over libselscan.so.

Every step of the computation runs in the HIP kernels of ``csrc/``; this module only
marshals torch tensors (device memory) and the current HIP stream into the C ABI declared
in ``include/selscan.h``, and raises on a non-zero status.  There is no fallback: if the
library is not built, importing the binding's functions raises.

    y, last = selective_scan_fwd(u, delta, A, B, C, Dskip, z, return_last_state=True)

Shapes (torch tensors on the current GPU):
    u, z           [batch, L, D]        float32 or bfloat16 (same dtype for u, delta, B, C, z)
    delta          [batch, L, D]        (selective) or [D] (time-invariant)
    A              [D, N] float32
    B, C           [batch, L, N]        (selective) or [D, N] (time-invariant)
    Dskip          [D] float32 or None
Options: ``discretization="euler"`` (Bbar = delta * B instead of the ZOH coefficient),
``delta_softplus=True`` and ``delta_bias`` ([D] float32): the step size is
softplus(delta + delta_bias) (the bias alone is added without softplus).
The innermost axis of every tensor must be unit-stride; other strides are passed through
(zero strides, i.e. expanded views, are allowed).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libselscan.so")

SELSCAN_ABI_VERSION = 2
SELSCAN_F32, SELSCAN_BF16 = 0, 1
SELSCAN_OK = 0
SELSCAN_ERR_NULL, SELSCAN_ERR_DIMS, SELSCAN_ERR_UNSUPPORTED = -1, -2, -3
SELSCAN_ERR_ALIGN, SELSCAN_ERR_HIP, SELSCAN_ERR_WORKSPACE, SELSCAN_ERR_ABI = -4, -5, -6, -7
SELSCAN_ERR_SCRATCH_LIMIT = -8
NOALLOC_SCRATCH_BYTES = 64 << 20          # SELSCAN_NOALLOC_SCRATCH_BYTES
PATHS = {"auto": 0, "single": 1, "chunked": 2, "conv": 3}   # conv: fixed coefficients only
FLAG_SCALAR_IO = 0x100   # tests only: force the general per-element kernel
DISCRETIZATIONS = {"zoh": 0, "euler": 1}


class SelscanDims(ctypes.Structure):
    """Mirror of ``selscan_dims`` in include/selscan.h (same field order and types)."""
    _fields_ = [
        ("abi_version", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("dim", ctypes.c_int64), ("dstate", ctypes.c_int64),
        ("u_sb", ctypes.c_int64), ("u_sl", ctypes.c_int64),
        ("delta_sb", ctypes.c_int64), ("delta_sl", ctypes.c_int64),
        ("z_sb", ctypes.c_int64), ("z_sl", ctypes.c_int64),
        ("y_sb", ctypes.c_int64), ("y_sl", ctypes.c_int64),
        ("B_sb", ctypes.c_int64), ("B_sl", ctypes.c_int64), ("B_sd", ctypes.c_int64),
        ("C_sb", ctypes.c_int64), ("C_sl", ctypes.c_int64), ("C_sd", ctypes.c_int64),
        ("path", ctypes.c_int32), ("chunk_len", ctypes.c_int32),
        ("discretization", ctypes.c_int32), ("delta_softplus", ctypes.c_int32),
    ]


class SelscanError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = "%s failed: %s (status %d)" % (where, strerror(status), status)
        if status == SELSCAN_ERR_HIP:
            msg += ", hipError %d" % last_hip_error()
        super().__init__(msg)


_lib = None

# (name, restype, argtypes) of every exported entry point
_VP = ctypes.c_void_p
_SIGNATURES = [
    ("selscan_dims_init", None, [ctypes.POINTER(SelscanDims), ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_int]),
    ("selective_scan_fwd", ctypes.c_int, [_VP] * 9 + [ctypes.POINTER(SelscanDims), _VP]),
    ("selective_scan_workspace_size", ctypes.c_size_t, [ctypes.POINTER(SelscanDims)]),
    ("selective_scan_plan_path", ctypes.c_int, [ctypes.POINTER(SelscanDims)]),
    ("selective_scan_fwd_ws", ctypes.c_int, [_VP] * 9 + [ctypes.POINTER(SelscanDims), _VP, ctypes.c_size_t, _VP]),
    ("selective_scan_fwd_ex", ctypes.c_int, [_VP] * 11 + [ctypes.POINTER(SelscanDims), _VP, ctypes.c_size_t, _VP]),
    ("selective_scan_fwd_noalloc", ctypes.c_int, [_VP] * 11 + [ctypes.POINTER(SelscanDims), _VP]),
    ("selective_scan_step", ctypes.c_int, [_VP] * 10 + [ctypes.POINTER(SelscanDims), _VP]),
    ("selective_scan_bwd", ctypes.c_int, [_VP] * 20 + [ctypes.POINTER(SelscanDims), _VP, ctypes.c_size_t, _VP]),
    ("selective_scan_bwd_workspace_size", ctypes.c_size_t, [ctypes.POINTER(SelscanDims)]),
    ("selective_scan_ssd_fwd", ctypes.c_int, [_VP] * 10 + [ctypes.c_void_p, _VP, ctypes.c_size_t, _VP]),
    ("selective_scan_ssd_workspace_size", ctypes.c_size_t, [ctypes.c_void_p]),
    ("selective_scan_strerror", ctypes.c_char_p, [ctypes.c_int]),
    ("selective_scan_last_hip_error", ctypes.c_int, []),
    ("selective_scan_abi_version", ctypes.c_int, []),
]


def lib():
    """The loaded libselscan.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libselscan.so is not built (expected at %s); run "
                               "`python -m selective_state_space_s6_amd.build`" % LIB_PATH)
        # PyTorch's wheel carries its own HIP runtime; it is loaded first so that this library
        # binds to the runtime that owns PyTorch's streams and memory (loaded the other way
        # round, HIP calls from here fail with hipErrorNoDevice)
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        handle = ctypes.CDLL(LIB_PATH)
        for name, res, args in _SIGNATURES:
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        if handle.selective_scan_abi_version() != SELSCAN_ABI_VERSION:
            raise RuntimeError("libselscan.so ABI version mismatch")
        _lib = handle
    return _lib


def strerror(status: int) -> str:
    return lib().selective_scan_strerror(int(status)).decode()


def last_hip_error() -> int:
    return int(lib().selective_scan_last_hip_error())


def abi_version() -> int:
    return int(lib().selective_scan_abi_version())


def dims_init(io_dtype: int, batch: int, seqlen: int, dim: int, dstate: int, time_invariant: bool = False) -> SelscanDims:
    d = SelscanDims()
    lib().selscan_dims_init(ctypes.byref(d), int(io_dtype), int(batch), int(seqlen), int(dim), int(dstate),
                            1 if time_invariant else 0)
    return d


def workspace_size(dims: SelscanDims) -> int:
    return int(lib().selective_scan_workspace_size(ctypes.byref(dims)))


def plan_path(dims: SelscanDims) -> str:
    """The path a forward call with these dims takes ("single", "chunked" or "conv")."""
    code = int(lib().selective_scan_plan_path(ctypes.byref(dims)))
    if code < 0:
        raise SelscanError(code, "selective_scan_plan_path")
    return {v: k for k, v in PATHS.items()}[code]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _io_code(dtype):
    import torch
    if dtype == torch.float32:
        return SELSCAN_F32
    if dtype == torch.bfloat16:
        return SELSCAN_BF16
    raise TypeError("u/delta/B/C/z/y must be float32 or bfloat16, got %s" % dtype)


def _strides_bld(t, name, batch, L, D):
    """(sb, sl) element strides of a [batch, L, D] tensor whose last axis is unit-stride."""
    if t.dim() != 3 or tuple(t.shape) != (batch, L, D):
        raise ValueError("%s must have shape %s, got %s" % (name, (batch, L, D), tuple(t.shape)))
    if D > 1 and t.stride(2) != 1:
        raise ValueError("%s: the channel axis must be unit-stride" % name)
    return t.stride(0), t.stride(1)


def make_dims(u, delta, A, B, C, z=None, y=None, *, path: str = "auto", chunk_len: int = 0,
              scalar_io: bool = False, discretization: str = "zoh", delta_softplus: bool = False) -> SelscanDims:
    """Build selscan_dims from tensor shapes and strides (see the module docstring)."""
    if u.dim() != 3:
        raise ValueError("u must be [batch, L, D]")
    batch, L, D = (int(x) for x in u.shape)
    if A.dim() != 2 or int(A.shape[0]) != D:
        raise ValueError("A must be [D, N]")
    N = int(A.shape[1])
    d = SelscanDims()
    d.abi_version = SELSCAN_ABI_VERSION
    d.io_dtype = _io_code(u.dtype)
    d.batch, d.seqlen, d.dim, d.dstate = batch, L, D, N
    d.u_sb, d.u_sl = _strides_bld(u, "u", batch, L, D)
    if delta.dim() == 1:
        if int(delta.shape[0]) != D or (D > 1 and delta.stride(0) != 1):
            raise ValueError("per-channel delta must be a contiguous [D] tensor")
        d.delta_sb = d.delta_sl = 0
    else:
        d.delta_sb, d.delta_sl = _strides_bld(delta, "delta", batch, L, D)
    for name, t in (("B", B), ("C", C)):
        if t.dim() == 2:
            if tuple(t.shape) != (D, N) or (N > 1 and t.stride(1) != 1):
                raise ValueError("per-channel %s must be [D, N] with a unit-stride state axis" % name)
            sb, sl, sd = 0, 0, t.stride(0)
        elif t.dim() == 3:
            if tuple(t.shape) != (batch, L, N) or (N > 1 and t.stride(2) != 1):
                raise ValueError("per-token %s must be [batch, L, N] with a unit-stride state axis" % name)
            sb, sl, sd = t.stride(0), t.stride(1), 0
        else:
            raise ValueError("%s must be [batch, L, N] or [D, N]" % name)
        setattr(d, name + "_sb", sb)
        setattr(d, name + "_sl", sl)
        setattr(d, name + "_sd", sd)
    if z is not None:
        d.z_sb, d.z_sl = _strides_bld(z, "z", batch, L, D)
    if y is not None:
        d.y_sb, d.y_sl = _strides_bld(y, "y", batch, L, D)
    d.path = PATHS[path] | (FLAG_SCALAR_IO if scalar_io else 0)
    d.chunk_len = int(chunk_len)
    d.discretization = DISCRETIZATIONS[discretization]
    d.delta_softplus = 1 if delta_softplus else 0
    return d


def _check_dskip(Dskip, D):
    """Dskip is read as Dskip[d] for every channel d < D: anything but a contiguous float32
    [D] GPU tensor is rejected before any launch."""
    import torch
    if Dskip is not None and (Dskip.dtype != torch.float32 or tuple(Dskip.shape) != (D,)
                              or not Dskip.is_contiguous() or not Dskip.is_cuda):
        raise ValueError("Dskip must be a contiguous float32 [D] GPU tensor (D = %d), got %s %s"
                         % (D, tuple(Dskip.shape), Dskip.dtype))


def _check_bias(delta_bias, D):
    import torch
    if delta_bias is not None and (delta_bias.dtype != torch.float32 or tuple(delta_bias.shape) != (D,)
                                   or not delta_bias.is_contiguous() or not delta_bias.is_cuda):
        raise ValueError("delta_bias must be a contiguous float32 [D] GPU tensor")


def selective_scan_fwd(u, delta, A, B, C, Dskip=None, z=None, y=None, last_state=None, *,
                       initial_state=None, delta_bias=None, delta_softplus: bool = False,
                       discretization: str = "zoh", return_last_state: bool = False, path: str = "auto",
                       chunk_len: int = 0, scalar_io: bool = False, workspace=None,
                       stream=None) -> Tuple["object", Optional["object"]]:
    """Selective-scan forward on the GPU.  Returns (y, last_state or None).

    ``y`` / ``last_state`` may be given (outputs are written in place) or are allocated.
    ``initial_state`` ([batch, D, N] float32, selective coefficients only) is the state the
    sequence continues from; it may be the ``last_state`` tensor itself (continue in place).

    ``workspace`` (a uint8 CUDA tensor of at least ``workspace_size`` bytes) selects the
    non-allocating entry point; when it is omitted and the call needs one, it is taken from
    torch's caching allocator.  ``stream`` defaults to torch's current stream."""
    import torch
    io = u.dtype
    for name, t in (("delta", delta), ("B", B), ("C", C), ("z", z), ("y", y)):
        if t is not None and t.dtype != io:
            raise TypeError("%s has dtype %s, expected %s like u" % (name, t.dtype, io))
    if A.dtype != torch.float32 or not A.is_contiguous():
        raise TypeError("A must be a contiguous float32 [D, N] tensor")
    if u.dim() != 3:
        raise ValueError("u must be [batch, L, D]")
    _check_dskip(Dskip, int(u.shape[2]))
    for name, t in (("u", u), ("delta", delta), ("A", A), ("B", B), ("C", C), ("Dskip", Dskip), ("z", z), ("y", y),
                    ("last_state", last_state)):
        if t is not None and not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
    if y is None:
        y = torch.empty(u.shape, dtype=io, device=u.device)
    batch, L, D = (int(x) for x in u.shape)
    N = int(A.shape[1])
    if last_state is None and return_last_state:
        last_state = torch.empty((batch, D, N), dtype=torch.float32, device=u.device)
    for name, t in (("last_state", last_state), ("initial_state", initial_state)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (batch, D, N)
                              or not t.is_cuda):
            raise ValueError("%s must be a contiguous float32 [batch, D, N] GPU tensor" % name)
    _check_bias(delta_bias, D)
    dims = make_dims(u, delta, A, B, C, z, y, path=path, chunk_len=chunk_len, scalar_io=scalar_io,
                     discretization=discretization, delta_softplus=delta_softplus)
    torch_stream = stream if (stream is None or hasattr(stream, "cuda_stream")) else None
    if stream is None:
        stream = torch.cuda.current_stream(u.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    if workspace is None and (torch_stream is not None or stream == torch.cuda.current_stream(u.device).cuda_stream):
        # Scratch of the chunked path from torch's caching allocator (the C entry point
        # would allocate it stream-ordered on every call); a raw stream handle that is not
        # torch's current stream keeps the library's own allocation.
        need = workspace_size(dims)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=u.device)
            if torch_stream is not None:
                workspace.record_stream(torch_stream)
    if initial_state is not None or delta_bias is not None:
        ws_args = ((_ptr(workspace), int(workspace.numel() * workspace.element_size())) if workspace is not None
                   else (None, 0))
        st = lib().selective_scan_fwd_ex(_ptr(u), _ptr(delta), _ptr(delta_bias), _ptr(A), _ptr(B), _ptr(C),
                                         _ptr(Dskip), _ptr(z), _ptr(y), _ptr(initial_state), _ptr(last_state),
                                         ctypes.byref(dims), ws_args[0], ws_args[1], ctypes.c_void_p(stream))
        if st != SELSCAN_OK:
            raise SelscanError(st, "selective_scan_fwd_ex")
        return y, last_state
    args = [_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(z), _ptr(y), _ptr(last_state),
            ctypes.byref(dims)]
    if workspace is not None:
        st = lib().selective_scan_fwd_ws(*args, _ptr(workspace), int(workspace.numel() * workspace.element_size()),
                                         ctypes.c_void_p(stream))
        where = "selective_scan_fwd_ws"
    else:
        st = lib().selective_scan_fwd(*args, ctypes.c_void_p(stream))
        where = "selective_scan_fwd"
    if st != SELSCAN_OK:
        raise SelscanError(st, where)
    return y, last_state


def selective_scan_fwd_noalloc(u, delta, A, B, C, Dskip=None, z=None, *, y, last_state=None, initial_state=None,
                               delta_bias=None, delta_softplus: bool = False, discretization: str = "zoh",
                               path: str = "auto", chunk_len: int = 0, stream=None):
    """The forward pass through selective_scan_fwd_noalloc, which allocates nothing: the
    chunked path's scratch is the library's own per-GPU array (NOALLOC_SCRATCH_BYTES).  The
    outputs ``y`` (and ``last_state`` if wanted) must be given; nothing is allocated here
    either.  Arguments otherwise as selective_scan_fwd.  Calls that overlap on one GPU race
    on the shared scratch.  Returns (y, last_state)."""
    import torch
    io = u.dtype
    if u.dim() != 3:
        raise ValueError("u must be [batch, L, D]")
    batch, L, D = (int(x) for x in u.shape)
    _check_dskip(Dskip, D)
    for name, t in (("delta", delta), ("B", B), ("C", C), ("z", z), ("y", y)):
        if t is not None and (t.dtype != io or not t.is_cuda):
            raise TypeError("%s must be a GPU tensor of dtype %s like u" % (name, io))
    if A.dtype != torch.float32 or not A.is_contiguous() or not A.is_cuda:
        raise TypeError("A must be a contiguous float32 [D, N] GPU tensor")
    N = int(A.shape[1])
    for name, t in (("last_state", last_state), ("initial_state", initial_state)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (batch, D, N)
                              or not t.is_cuda):
            raise ValueError("%s must be a contiguous float32 [batch, D, N] GPU tensor" % name)
    _check_bias(delta_bias, D)
    dims = make_dims(u, delta, A, B, C, z, y, path=path, chunk_len=chunk_len, discretization=discretization,
                     delta_softplus=delta_softplus)
    if stream is None:
        stream = torch.cuda.current_stream(u.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    st = lib().selective_scan_fwd_noalloc(_ptr(u), _ptr(delta), _ptr(delta_bias), _ptr(A), _ptr(B), _ptr(C),
                                          _ptr(Dskip), _ptr(z), _ptr(y), _ptr(initial_state), _ptr(last_state),
                                          ctypes.byref(dims), ctypes.c_void_p(stream))
    if st != SELSCAN_OK:
        raise SelscanError(st, "selective_scan_fwd_noalloc")
    return y, last_state


def selective_scan_step(u, delta, A, B, C, Dskip=None, z=None, y=None, *, state, time_invariant: bool = False,
                        delta_bias=None, delta_softplus: bool = False, discretization: str = "zoh", stream=None):
    """One recurrent decode step (one token per batch row); ``state`` ([batch, D, N] float32,
    contiguous) is read as the running state and overwritten with the new one.

    u, z, y: [batch, D]; A: [D, N]; Dskip: [D].  Selective coefficients: delta [batch, D]
    (or [D] shared by the batch), B, C [batch, N].  time_invariant=True: delta [D], B, C
    [D, N].  delta_bias, delta_softplus, discretization: as selective_scan_fwd.  Returns y."""
    import torch
    if u.dim() != 2:
        raise ValueError("u must be [batch, D] (one token per batch row)")
    batch, D = (int(x) for x in u.shape)
    _check_dskip(Dskip, D)
    if A.dim() != 2 or int(A.shape[0]) != D or A.dtype != torch.float32 or not A.is_contiguous():
        raise ValueError("A must be a contiguous float32 [D, N] tensor")
    N = int(A.shape[1])
    io = u.dtype
    if y is None:
        y = torch.empty((batch, D), dtype=io, device=u.device)
    for name, t in (("delta", delta), ("B", B), ("C", C), ("z", z), ("y", y)):
        if t is not None and (t.dtype != io or not t.is_cuda):
            raise TypeError("%s must be a GPU tensor of dtype %s like u" % (name, io))
    if (state.dtype != torch.float32 or not state.is_contiguous() or tuple(state.shape) != (batch, D, N)
            or not state.is_cuda):
        raise ValueError("state must be a contiguous float32 [batch, D, N] GPU tensor")

    def rows(t, name, width):                  # [batch, width] with a unit-stride last axis
        if t.dim() != 2 or tuple(t.shape) != (batch, width) or (width > 1 and t.stride(1) != 1):
            raise ValueError("%s must be [batch, %d] with a unit-stride last axis" % (name, width))
        return t.stride(0)

    _check_bias(delta_bias, D)
    d = SelscanDims()
    d.abi_version = SELSCAN_ABI_VERSION
    d.io_dtype = _io_code(io)
    d.batch, d.seqlen, d.dim, d.dstate = batch, 1, D, N
    d.discretization = DISCRETIZATIONS[discretization]
    d.delta_softplus = 1 if delta_softplus else 0
    d.u_sb = rows(u, "u", D)
    d.u_sl = D
    d.y_sb = rows(y, "y", D)
    d.y_sl = D                                 # rows of different batch entries must not overlap
    if z is not None:
        d.z_sb = rows(z, "z", D)
        d.z_sl = D
    if delta.dim() == 1:
        if int(delta.shape[0]) != D or (D > 1 and delta.stride(0) != 1):
            raise ValueError("per-channel delta must be a contiguous [D] tensor")
        d.delta_sb = d.delta_sl = 0
    else:
        d.delta_sb = rows(delta, "delta", D)
        d.delta_sl = D
    if time_invariant and delta.dim() != 1:
        raise ValueError("time-invariant coefficients take a per-channel [D] delta")
    for name, t in (("B", B), ("C", C)):
        if time_invariant:
            if t.dim() != 2 or tuple(t.shape) != (D, N) or (N > 1 and t.stride(1) != 1):
                raise ValueError("per-channel %s must be [D, N] with a unit-stride state axis" % name)
            sb, sl, sd = 0, 0, t.stride(0)
        else:
            sb, sl, sd = rows(t, name, N), N, 0
        setattr(d, name + "_sb", sb)
        setattr(d, name + "_sl", sl)
        setattr(d, name + "_sd", sd)
    if stream is None:
        stream = torch.cuda.current_stream(u.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    st = lib().selective_scan_step(_ptr(u), _ptr(delta), _ptr(delta_bias), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip),
                                   _ptr(z), _ptr(y), _ptr(state), ctypes.byref(d), ctypes.c_void_p(stream))
    if st != SELSCAN_OK:
        raise SelscanError(st, "selective_scan_step")
    return y


def bwd_workspace_size(dims: SelscanDims) -> int:
    return int(lib().selective_scan_bwd_workspace_size(ctypes.byref(dims)))


def selective_scan_bwd(u, delta, A, B, C, Dskip=None, z=None, *, dy, dlast_state=None, initial_state=None,
                       delta_bias=None, delta_softplus: bool = False, discretization: str = "zoh", workspace=None,
                       stream=None) -> dict:
    """Gradients of selective_scan_fwd (same inputs and options) given dy, the gradient of y,
    and optionally dlast_state, the gradient of last_state.

    Returns a dict: du, ddelta, dz (if z) as [batch, L, D] and dB, dC as [batch, L, N], in
    u's dtype; dA [D, N], dDskip [D] (if Dskip), ddelta_bias [D] (if delta_bias) and
    dinitial_state [batch, D, N] (if initial_state), in float32.  With fixed coefficients
    (delta [D], B and C [D, N]) ddelta is [D] and dB, dC are [D, N], in u's dtype.
    ``workspace`` (a uint8 GPU tensor of bwd_workspace_size bytes) is taken from torch's
    caching allocator when omitted."""
    import torch
    io = u.dtype
    if u.dim() != 3:
        raise ValueError("u must be [batch, L, D]")
    batch, L, D = (int(x) for x in u.shape)
    _check_dskip(Dskip, D)
    for name, t in (("delta", delta), ("B", B), ("C", C), ("z", z), ("dy", dy)):
        if t is not None and (t.dtype != io or not t.is_cuda):
            raise TypeError("%s must be a GPU tensor of dtype %s like u" % (name, io))
    if A.dtype != torch.float32 or not A.is_contiguous():
        raise TypeError("A must be a contiguous float32 [D, N] tensor")
    N = int(A.shape[1])
    for name, t in (("dlast_state", dlast_state), ("initial_state", initial_state)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (batch, D, N)
                              or not t.is_cuda):
            raise ValueError("%s must be a contiguous float32 [batch, D, N] GPU tensor" % name)
    _check_bias(delta_bias, D)
    dims = make_dims(u, delta, A, B, C, z, dy, discretization=discretization, delta_softplus=delta_softplus)
    dev = u.device
    ti = delta.dim() == 1 and B.dim() == 2 and C.dim() == 2      # fixed coefficients
    g = {"du": torch.empty((batch, L, D), dtype=io, device=dev),
         "ddelta": torch.empty((D,) if ti else (batch, L, D), dtype=io, device=dev),
         "dA": torch.empty((D, N), dtype=torch.float32, device=dev),
         "dB": torch.empty((D, N) if ti else (batch, L, N), dtype=io, device=dev),
         "dC": torch.empty((D, N) if ti else (batch, L, N), dtype=io, device=dev)}
    if z is not None:
        g["dz"] = torch.empty((batch, L, D), dtype=io, device=dev)
    if Dskip is not None:
        g["dDskip"] = torch.empty((D,), dtype=torch.float32, device=dev)
    if delta_bias is not None:
        g["ddelta_bias"] = torch.empty((D,), dtype=torch.float32, device=dev)
    if initial_state is not None:
        g["dinitial_state"] = torch.empty((batch, D, N), dtype=torch.float32, device=dev)
    torch_stream = stream if (stream is None or hasattr(stream, "cuda_stream")) else None
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    if workspace is None and (torch_stream is not None or stream == torch.cuda.current_stream(dev).cuda_stream):
        need = bwd_workspace_size(dims)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
            if torch_stream is not None:
                workspace.record_stream(torch_stream)
    ws = (_ptr(workspace), int(workspace.numel() * workspace.element_size())) if workspace is not None else (None, 0)
    st = lib().selective_scan_bwd(
        _ptr(u), _ptr(delta), _ptr(delta_bias), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(z), _ptr(initial_state),
        _ptr(dy), _ptr(dlast_state), _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g.get("ddelta_bias")), _ptr(g["dA"]),
        _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g.get("dDskip")), _ptr(g.get("dz")), _ptr(g.get("dinitial_state")),
        ctypes.byref(dims), ws[0], ws[1], ctypes.c_void_p(stream))
    if st != SELSCAN_OK:
        raise SelscanError(st, "selective_scan_bwd")
    return g


class SsdDims(ctypes.Structure):
    """Mirror of ``selscan_ssd_dims`` in include/selscan.h."""
    _fields_ = [("abi_version", ctypes.c_int32), ("discretization", ctypes.c_int32), ("batch", ctypes.c_int64),
                ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("path", ctypes.c_int32), ("segments", ctypes.c_int32)]


SSD_PATHS = {"auto": 0, "fused": 1, "chunked": 2, "segmented": 3}


def ssd_dims(batch, seqlen, nheads, headdim, dstate, discretization="zoh", path="auto", segments=0) -> SsdDims:
    d = SsdDims()
    d.abi_version = SELSCAN_ABI_VERSION
    d.discretization = DISCRETIZATIONS[discretization]
    d.path = SSD_PATHS[path]
    d.segments = int(segments)
    d.batch, d.seqlen, d.nheads, d.headdim, d.dstate = int(batch), int(seqlen), int(nheads), int(headdim), int(dstate)
    return d


def ssd_workspace_size(dims: SsdDims) -> int:
    return int(lib().selective_scan_ssd_workspace_size(ctypes.byref(dims)))


def selective_scan_ssd_fwd(x, delta, A, B, C, Dskip=None, z=None, y=None, *, initial_state=None,
                           return_last_state: bool = False, discretization: str = "zoh", path: str = "auto",
                           segments: int = 0, workspace=None, stream=None):
    """The scalar-decay (Mamba-2) layer on the GPU (bf16 x, delta, B, C, z, y; fp32 A, Dskip,
    states).  x, z: [batch, L, H, 64]; delta: [batch, L, H]; A: [H]; B, C: [batch, L, N] with
    N = 64 or 128; Dskip: [H * 64]; initial_state: [batch, H, 64, N].  All contiguous.
    path: "auto", "fused" (on chip), "chunked" (chunk-parallel) or "segmented" (on chip over
    `segments` sequence segments, 0 = chosen by the library).  Returns (y, last_state or None)."""
    import torch
    if x.dim() != 4:
        raise ValueError("x must be [batch, L, H, headdim]")
    batch, L, H, P = (int(v) for v in x.shape)
    N = int(B.shape[-1])
    for name, t in (("x", x), ("delta", delta), ("B", B), ("C", C), ("z", z), ("y", y)):
        if t is not None and (t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda):
            raise TypeError("%s must be a contiguous bfloat16 GPU tensor" % name)
    if tuple(delta.shape) != (batch, L, H) or tuple(B.shape) != (batch, L, N) or tuple(C.shape) != (batch, L, N):
        raise ValueError("delta must be [batch, L, H]; B, C [batch, L, N]")
    for name, t, shape in (("A", A, (H,)), ("Dskip", Dskip, (H * P,)), ("initial_state", initial_state, (batch, H, P, N))):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != shape or not t.is_cuda):
            raise ValueError("%s must be a contiguous float32 %s GPU tensor" % (name, shape))
    if y is None:
        y = torch.empty_like(x)
    last = torch.empty((batch, H, P, N), dtype=torch.float32, device=x.device) if return_last_state else None
    dims = ssd_dims(batch, L, H, P, N, discretization, path, segments)
    torch_stream = stream if (stream is None or hasattr(stream, "cuda_stream")) else None
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    if workspace is None and (torch_stream is not None or stream == torch.cuda.current_stream(x.device).cuda_stream):
        need = ssd_workspace_size(dims)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
            if torch_stream is not None:
                workspace.record_stream(torch_stream)
    ws = (_ptr(workspace), int(workspace.numel() * workspace.element_size())) if workspace is not None else (None, 0)
    st = lib().selective_scan_ssd_fwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(z), _ptr(y),
                                      _ptr(initial_state), _ptr(last), ctypes.byref(dims), ws[0], ws[1],
                                      ctypes.c_void_p(stream))
    if st != SELSCAN_OK:
        raise SelscanError(st, "selective_scan_ssd_fwd")
    return y, last


__all__ = ["selective_scan_fwd", "selective_scan_step", "selective_scan_bwd", "bwd_workspace_size",
           "selective_scan_ssd_fwd", "ssd_dims", "ssd_workspace_size", "SsdDims", "make_dims", "dims_init", "workspace_size", "strerror", "last_hip_error",
           "abi_version", "lib", "SelscanDims", "SelscanError", "LIB_PATH"]
