"""Independent CPU oracle for the S6 selective-scan forward pass.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()`` and by
the CPU-baseline leg of ``bench.py``.  The GPU library never imports, links or calls
anything here, and nothing here imports the GPU library.

Two independent statements of the method live here:

* ``fwd`` -- the plain sequential recurrence in double precision (``ssm_oracle.c``),
  following the zero-order-hold discretisation and the recurrence/readout as written on
  the "state-space models" page (aarnphm.xyz, sections "From continuous time to tokens"
  and "One recurrence, one convolution") and the Algenta "Sequence and state-space
  models" page (section on ``state_space_models``), with the feed-through and SiLU gate
  of the TorchLean "Selective Mamba" page (``step``).  Options: an initial state, the
  first-order input coefficient Bbar = delta * B (Algenta, ``mamba_selective_scan_step``),
  and the step-size transform softplus(delta + per-channel bias) (TorchLean, ``step``).
* ``ssd_fwd`` / ``ssd_quadratic`` -- the scalar-decay (Mamba-2) layer: as the recurrence above
  with one decay per head, and in its pairwise masked form ("state-space models", section
  "Mamba-2 and state-space duality").
* ``bwd`` -- the gradients of that forward (its vector-Jacobian product) by the reverse-time
  recurrence over the cached states, as the rustytorch commit log describes its hand-written
  VJP of the selective scan.
* ``conv_ti`` -- for fixed (time-invariant) coefficients, the causal-convolution form of
  the same layer with lag kernel K_k = C Abar^k Bbar ("state-space models", section "One
  recurrence, one convolution"), written with numpy in float64 and sharing no code with
  the recurrence.  Abar^k is evaluated as exp(k * delta * a), the exact composition of
  k steps, not as a repeated product.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libssm_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile ssm_oracle.c with gcc (-O2, no fast-math) into libssm_oracle.so."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fno-fast-math", "-o", tmp, _SRC,
                               "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class OracleLib:
    """ctypes view of one compiled oracle library (the default one, or a test-built variant)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        fp = ctypes.POINTER(ctypes.c_float)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.ssm_oracle_fwd.restype = ctypes.c_int
        lib.ssm_oracle_fwd.argtypes = [fp, fp, fp, fp, fp, fp, fp, fp, fp, dp, dp, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int]
        for name in ("ssm_oracle_discretize", "ssm_oracle_discretize_euler"):
            getattr(lib, name).restype = None
            getattr(lib, name).argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double, dp, dp]
        lib.ssm_oracle_softplus.restype = ctypes.c_double
        lib.ssm_oracle_softplus.argtypes = [ctypes.c_double]
        lib.ssm_oracle_bwd.restype = ctypes.c_int
        lib.ssm_oracle_bwd.argtypes = [fp] * 11 + [dp] * 9 + [ctypes.c_int64] * 4 + [ctypes.c_int] * 3
        self.lib = lib
        self.path = path

    def discretize(self, a: float, b: float, delta: float, euler: bool = False):
        """Coefficients (Abar, Bbar) of one scalar state: ZOH, or the first-order input
        coefficient with euler=True."""
        ab = ctypes.c_double()
        bb = ctypes.c_double()
        fn = self.lib.ssm_oracle_discretize_euler if euler else self.lib.ssm_oracle_discretize
        fn(float(a), float(b), float(delta), ctypes.byref(ab), ctypes.byref(bb))
        return ab.value, bb.value

    def softplus(self, x: float) -> float:
        return self.lib.ssm_oracle_softplus(float(x))

    def fwd(self, u, delta, A, B, C, Dskip=None, z=None, *, h0=None, delta_bias=None, euler=False,
            delta_softplus=False, time_invariant=False, want_last=True, nthreads=None):
        """Run the fp64 recurrence.  Returns (y [batch,L,D] float64, last_state [batch,D,N] float64
        or None).

        u, z: [batch, L, D]; delta: [batch, L, D] (time-invariant: [D]); B, C: [batch, L, N]
        (time-invariant: [D, N]); A: [D, N]; Dskip: [D]; h0: [batch, D, N] initial state (None:
        zero); delta_bias: [D] added to delta (None: zero).  euler: Bbar = delta * B;
        delta_softplus: the step size is softplus(delta + delta_bias).  Inputs are converted to
        float32 first, the precision the GPU library receives.
        """
        u = _f32(u)
        delta = _f32(delta)
        A = _f32(A)
        B = _f32(B)
        C = _f32(C)
        Dskip = _f32(Dskip)
        z = _f32(z)
        h0 = _f32(h0)
        delta_bias = _f32(delta_bias)
        batch, L, D = u.shape
        N = A.shape[1]
        assert A.shape == (D, N)
        if time_invariant:
            assert delta.shape == (D,) and B.shape == (D, N) and C.shape == (D, N)
        else:
            assert delta.shape == (batch, L, D) and B.shape == (batch, L, N) and C.shape == (batch, L, N)
        if Dskip is not None:
            assert Dskip.shape == (D,)
        if z is not None:
            assert z.shape == (batch, L, D)
        if h0 is not None:
            assert h0.shape == (batch, D, N)
        if delta_bias is not None:
            assert delta_bias.shape == (D,)
        y = np.empty((batch, L, D), dtype=np.float64)
        last = np.empty((batch, D, N), dtype=np.float64) if want_last else None
        if nthreads is None:
            nthreads = os.cpu_count() or 1
        rc = self.lib.ssm_oracle_fwd(
            _fptr(u), _fptr(delta), _fptr(A), _fptr(B), _fptr(C), _fptr(Dskip), _fptr(z), _fptr(h0),
            _fptr(delta_bias), y.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
            None if last is None else last.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
            batch, L, D, N, 1 if time_invariant else 0, 1 if euler else 0, 1 if delta_softplus else 0,
            int(nthreads))
        if rc != 0:
            raise RuntimeError("ssm_oracle_fwd failed with %d" % rc)
        return y, last


    def bwd(self, u, delta, A, B, C, Dskip=None, z=None, *, dy, dlast=None, h0=None, delta_bias=None, euler=False,
            delta_softplus=False, time_invariant=False):
        """Gradients of the forward pass (the vector-Jacobian product with dy, plus dlast at the
        final state), in float64, by the reverse-time recurrence over the cached states.
        Returns a dict with du, ddelta, dA, dB, dC, dz (always), dDskip (if Dskip),
        ddelta_bias (if delta_bias) and dh0 (if h0); shapes follow the inputs."""
        u, delta, A, B, C, Dskip, z, h0, delta_bias = map(_f32, (u, delta, A, B, C, Dskip, z, h0, delta_bias))
        dy, dlast = _f32(dy), _f32(dlast)
        batch, L, D = u.shape
        N = A.shape[1]
        assert dy.shape == (batch, L, D)
        if dlast is not None:
            assert dlast.shape == (batch, D, N)
        out = {"du": np.empty((batch, L, D)), "dz": np.empty((batch, L, D)),
               "ddelta": np.empty((D,) if time_invariant else (batch, L, D)), "dA": np.empty((D, N)),
               "dB": np.empty((D, N) if time_invariant else (batch, L, N)),
               "dC": np.empty((D, N) if time_invariant else (batch, L, N))}
        if Dskip is not None:
            out["dDskip"] = np.empty(D)
        if delta_bias is not None:
            out["ddelta_bias"] = np.empty(D)
        if h0 is not None:
            out["dh0"] = np.empty((batch, D, N))
        dpt = lambda k: out[k].ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if k in out else None
        rc = self.lib.ssm_oracle_bwd(
            _fptr(u), _fptr(delta), _fptr(A), _fptr(B), _fptr(C), _fptr(Dskip), _fptr(z), _fptr(h0),
            _fptr(delta_bias), _fptr(dy), _fptr(dlast),
            dpt("du"), dpt("ddelta"), dpt("dA"), dpt("dB"), dpt("dC"), dpt("dDskip"), dpt("dz"),
            dpt("ddelta_bias"), dpt("dh0"), batch, L, D, N, 1 if time_invariant else 0, 1 if euler else 0,
            1 if delta_softplus else 0)
        if rc != 0:
            raise RuntimeError("ssm_oracle_bwd failed with %d" % rc)
        if z is None:
            out["dz"][...] = 0.0
        return out


def _load() -> OracleLib:
    global _lib
    if _lib is None:
        _lib = OracleLib(build())
    return _lib


def _fptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _f32(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float32)


def discretize(a: float, b: float, delta: float, euler: bool = False):
    """Coefficients (Abar, Bbar) of one scalar state, from the C oracle (ZOH, or the
    first-order input coefficient with euler=True)."""
    return _load().discretize(a, b, delta, euler)


def softplus(x: float) -> float:
    """softplus(x) = log(1 + e^x) in double, from the C oracle."""
    return _load().softplus(x)


def fwd(u, delta, A, B, C, Dskip=None, z=None, *, h0=None, delta_bias=None, euler=False, delta_softplus=False,
        time_invariant=False, want_last=True, nthreads=None):
    """The fp64 recurrence of the default oracle library; see ``OracleLib.fwd``."""
    return _load().fwd(u, delta, A, B, C, Dskip, z, h0=h0, delta_bias=delta_bias, euler=euler,
                       delta_softplus=delta_softplus, time_invariant=time_invariant, want_last=want_last,
                       nthreads=nthreads)


def bwd(u, delta, A, B, C, Dskip=None, z=None, *, dy, dlast=None, h0=None, delta_bias=None, euler=False,
        delta_softplus=False, time_invariant=False):
    """Gradients of the forward pass from the default oracle library; see ``OracleLib.bwd``."""
    return _load().bwd(u, delta, A, B, C, Dskip, z, dy=dy, dlast=dlast, h0=h0, delta_bias=delta_bias, euler=euler,
                       delta_softplus=delta_softplus, time_invariant=time_invariant)


def ssd_as_s6(x, delta, A_head, Dskip=None):
    """The scalar-decay (Mamba-2 "SSD") layer as an S6 layer: Abar_t = a_t I within a head
    ("state-space models", section "Mamba-2 and state-space duality") is the diagonal S6
    transition with A[d, n] = A_head[h] for every state n and every channel d = h * P + p of
    head h, and one step size per (token, head) shared by the head's P channels.  Returns the
    S6 per-token operands (u [b, L, H*P], delta [b, L, H*P]); ssd_fwd builds A and runs fwd."""
    x = np.asarray(x, np.float32)
    b, L, H, P = x.shape
    u = x.reshape(b, L, H * P)
    dl = np.repeat(np.asarray(delta, np.float32), P, axis=2)
    return u, dl


def ssd_fwd(x, delta, A_head, B, C, Dskip=None, z=None, *, h0=None, euler=False, want_last=True, nthreads=None):
    """The scalar-decay layer by the fp64 recurrence of ``fwd``: x, z [b, L, H, P]; delta
    [b, L, H]; A_head [H]; B, C [b, L, N] (one group shared by every head); Dskip [H*P].
    Returns (y [b, L, H, P], last_state [b, H, P, N] or None)."""
    x = np.asarray(x, np.float32)
    b, L, H, P = x.shape
    N = np.asarray(B).shape[2]
    u, dl = ssd_as_s6(x, delta, A_head)
    A = np.repeat(np.asarray(A_head, np.float32), P)[:, None].repeat(N, axis=1)
    zz = None if z is None else np.asarray(z, np.float32).reshape(b, L, H * P)
    y, last = fwd(u, dl, A, B, C, Dskip, zz, h0=None if h0 is None else np.asarray(h0, np.float32).reshape(b, H * P, N),
                  euler=euler, want_last=want_last, nthreads=nthreads)
    return y.reshape(b, L, H, P), None if last is None else last.reshape(b, H, P, N)


def ssd_quadratic(x, delta, A_head, B, C, euler=False):
    """The same layer in its pairwise form Y = (L o Q K^T) V per head, in float64 (O(L^2)):
    L[t, s] = prod_{k=s+1..t} a_k for s <= t (else 0), Q = C, K rows = Bbar_s = c_s B_s, V = x
    ("state-space models", section "Mamba-2 and state-space duality": the unrolled sum and
    its masked-attention form).  a_k = exp(delta_k A_h); c_s = (a_s - 1)/A_h (ZOH; delta_s
    when A_h == 0) or delta_s (first order).  No feed-through, no gate."""
    x = np.asarray(x, np.float64)
    b, L, H, P = x.shape
    dl = np.asarray(delta, np.float64)
    A = np.asarray(A_head, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    y = np.zeros_like(x)
    for bi in range(b):
        QK = C[bi] @ B[bi].T                                    # [L, L]: C_t . B_s
        for h in range(H):
            logs = dl[bi, :, h] * A[h]                          # log a_k
            cum = np.concatenate([[0.0], np.cumsum(logs)])      # cum[t+1] = sum_{k<=t} log a_k
            Lmask = np.tril(np.exp(cum[1:, None] - cum[None, 1:]))   # prod_{k=s+1..t} a_k
            if euler or A[h] == 0.0:
                c = dl[bi, :, h]
            else:
                c = np.expm1(logs) / A[h]
            y[bi, :, h, :] = (Lmask * QK * c[None, :]) @ x[bi, :, h, :]
    return y


def kernel_element(c: float, abar_power: float, bbar: float) -> float:
    """One lag-kernel term C * Abar^k * Bbar for a single state (the factor the caller
    sums over states and lags)."""
    return float(c) * float(abar_power) * float(bbar)


def ti_kernel(delta, A, B, C, L: int):
    """Lag kernel K[k, d] = sum_n C[d,n] * exp(k*delta[d]*A[d,n]) * Bbar[d,n], k = 0..L-1,
    in float64, with Bbar = expm1(delta*a)/a * b (delta * b when a == 0)."""
    delta = np.asarray(delta, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    dA = delta[:, None] * A
    with np.errstate(divide="ignore", invalid="ignore"):
        coeff = np.where(A != 0.0, np.expm1(dA) / np.where(A != 0.0, A, 1.0), delta[:, None])
    bbar = coeff * B
    k = np.arange(L, dtype=np.float64)[:, None, None]
    powers = np.exp(k * dA[None, :, :])                      # Abar^k = exp(k * delta * a)
    return np.einsum("kdn,dn->kd", powers * C[None], bbar)    # [L, D]


def conv_ti(u, delta, A, B, C, Dskip=None):
    """Causal convolution y[b,t,d] = sum_{j<=t} K[t-j,d] u[b,j,d] + Dskip[d] u[b,t,d] (float64).

    Uses an FFT of length >= 2L per channel (zero padded, so the circular product equals the
    linear causal one)."""
    u = np.asarray(u, dtype=np.float64)
    batch, L, D = u.shape
    K = ti_kernel(delta, A, B, C, L)
    nfft = 1
    while nfft < 2 * L:
        nfft *= 2
    Kf = np.fft.rfft(K, n=nfft, axis=0)                       # [F, D]
    Uf = np.fft.rfft(u, n=nfft, axis=1)                       # [batch, F, D]
    y = np.fft.irfft(Uf * Kf[None], n=nfft, axis=1)[:, :L, :]
    if Dskip is not None:
        y = y + np.asarray(Dskip, dtype=np.float64)[None, None, :] * u
    return y


def conv_ti_direct(u, delta, A, B, C, Dskip=None):
    """The same causal convolution as an explicit double sum (O(L^2) per channel); for
    small inputs."""
    u = np.asarray(u, dtype=np.float64)
    batch, L, D = u.shape
    K = ti_kernel(delta, A, B, C, L)
    y = np.zeros_like(u)
    for t in range(L):
        # sum_j K[t-j] u[j], j = 0..t
        y[:, t, :] = np.einsum("jd,bjd->bd", K[t::-1], u[:, : t + 1, :])
    if Dskip is not None:
        y = y + np.asarray(Dskip, dtype=np.float64)[None, None, :] * u
    return y
