"""Seeded synthetic inputs for the S6 selective-scan forward.

This module only draws random numbers and lays them out; it holds none of the scan's
arithmetic.  It is shared by the tests, the smoke check and the benchmark so that the
GPU library and the oracle always see the same inputs.

Distributions follow the canonical S6 initialisation described in the rustytorch commit
log ("canonical S6 init": A = -(1..N) from A_log = ln(1..N), a time step whose softplus is
about 0.01, D = 1): A[d, n] = -(n + 1), Dskip = 1, and log-uniform step sizes in
[1e-3, 1e-1].  u, B, C and z are standard normal.  Every workload below is synthetic;
the pages measure nothing on a public dataset for this path.

Draw order inside one workload: u, delta (or the softplus pre-activation g), B, C, z,
each drawn in float64 from numpy's PCG64 with seed 1000 + workload number, then cast to
float32 and, for bf16-I/O workloads, rounded to bfloat16 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# name -> spec.  "number" fixes the seed (1000 + number).
WORKLOADS = {
    "tiny_f32": dict(number=1, batch=1, L=64, D=4, N=4, io="f32", gate=False, last=True, ti=False,
                     a_scale=1.0, delta="loguniform"),
    "small_f32": dict(number=2, batch=2, L=1024, D=256, N=16, io="f32", gate=True, last=True, ti=False,
                      a_scale=1.0, delta="loguniform"),
    "mamba130m_f32": dict(number=3, batch=8, L=2048, D=1536, N=16, io="f32", gate=True, last=True, ti=False,
                          a_scale=1.0, delta="loguniform"),
    "longctx_bf16": dict(number=4, batch=4, L=16384, D=2560, N=16, io="bf16", gate=True, last=False,
                         ti=False, a_scale=1.0, delta="softplus_normal"),
    "s4d_ti_f32": dict(number=5, batch=4, L=8192, D=1024, N=64, io="f32", gate=False, last=False, ti=True,
                       a_scale=0.5, delta="loguniform"),
    # one recurrent decode step for 512 sequences of the long-context model's width: one
    # token per batch row, the running state [512, 2560, 16] fp32 read and written once
    "decode_bf16": dict(number=6, batch=512, L=1, D=2560, N=16, io="bf16", gate=True, last=True, ti=False,
                        a_scale=1.0, delta="softplus_normal", decode=True),
}

# Scalar-decay (Mamba-2) layers: x [batch, L, H, 64], delta [batch, L, H], B, C [batch, L, N].
# Widths of the Mamba-2 130M (24 heads) and 2.7B (80 heads) layers, 64-wide heads, 128 states.
SSD_WORKLOADS = {
    "ssd_mamba2_130m_bf16": dict(number=7, batch=8, L=2048, H=24, N=128),
    "ssd_mamba2_2p7b_bf16": dict(number=8, batch=4, L=8192, H=80, N=128),
}

VARIANTS = ("default", "scan_only", "active", "active_const")


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32 values
    that are exactly representable in bfloat16.  Inputs here are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The bfloat16 bit patterns (uint16) of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def softplus(x: np.ndarray) -> np.ndarray:
    """log(1 + e^x) in the overflow-free form log1p(e^-|x|) + max(x, 0); used only to draw
    the step sizes of the long-context workload from a pre-activation."""
    x = np.asarray(x, dtype=np.float64)
    return np.log1p(np.exp(-np.abs(x))) + np.maximum(x, 0.0)


@dataclasses.dataclass
class Inputs:
    """One workload's tensors as float32 numpy arrays (bf16 workloads: bf16-exact values)."""
    name: str
    io: str                       # "f32" or "bf16"
    ti: bool                      # time-invariant: delta [D], B and C [D, N]
    u: np.ndarray                 # [batch, L, D]
    delta: np.ndarray             # [batch, L, D] or [D]
    A: np.ndarray                 # [D, N]
    B: np.ndarray                 # [batch, L, N] or [D, N]
    C: np.ndarray                 # [batch, L, N] or [D, N]
    Dskip: Optional[np.ndarray]   # [D] or None
    z: Optional[np.ndarray]       # [batch, L, D] or None
    want_last: bool

    @property
    def shape(self):
        b, L, D = self.u.shape
        return b, L, D, self.A.shape[1]

    @property
    def elements(self) -> int:
        b, L, D, N = self.shape
        return b * L * D * N


def spec(name: str) -> dict:
    return dict(WORKLOADS[name])


def generate(name: str, variant: str = "default", *, seed: Optional[int] = None, batch: Optional[int] = None,
             L: Optional[int] = None, D: Optional[int] = None, N: Optional[int] = None,
             gate: Optional[bool] = None) -> Inputs:
    """Draw a workload's inputs.  ``batch``/``L``/``D``/``N`` override the sizes (for
    reduced parity cases); ``variant`` is one of VARIANTS:

    * default      -- the workload as specified;
    * scan_only    -- no feed-through and no gate, so y is the scan term alone;
    * active       -- step sizes log-uniform in [0.1, 1] (large per-step decay);
    * active_const -- every step size equal to 0.69 (about log 2).
    """
    if variant not in VARIANTS:
        raise ValueError("unknown variant %r" % variant)
    s = spec(name)
    b = s["batch"] if batch is None else batch
    Lq = s["L"] if L is None else L
    Dq = s["D"] if D is None else D
    Nq = s["N"] if N is None else N
    use_gate = s["gate"] if gate is None else gate
    rng = np.random.Generator(np.random.PCG64(1000 + s["number"] if seed is None else seed))
    ti = s["ti"]

    u = rng.standard_normal((b, Lq, Dq))
    dshape = (Dq,) if ti else (b, Lq, Dq)
    if variant == "active":
        delta = np.exp(rng.uniform(np.log(0.1), np.log(1.0), dshape))
    elif variant == "active_const":
        delta = np.full(dshape, 0.69)
    elif s["delta"] == "loguniform":
        delta = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), dshape))
    elif s["delta"] == "softplus_normal":
        delta = softplus(rng.normal(-4.6, 0.5, dshape))
    else:
        raise ValueError(s["delta"])
    bcshape = (Dq, Nq) if ti else (b, Lq, Nq)
    B = rng.standard_normal(bcshape)
    C = rng.standard_normal(bcshape)
    z = rng.standard_normal((b, Lq, Dq)) if use_gate else None
    A = -(np.arange(Nq, dtype=np.float64) + 1.0)[None, :].repeat(Dq, axis=0) * s["a_scale"]
    Dskip = np.ones(Dq)

    f32 = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.float32)
    u, delta, B, C, z, A, Dskip = map(f32, (u, delta, B, C, z, A, Dskip))
    if s["io"] == "bf16":
        u, delta, B, C = bf16_round(u), bf16_round(delta), bf16_round(B), bf16_round(C)
        z = None if z is None else bf16_round(z)
    if variant == "scan_only":
        Dskip, z = None, None
    return Inputs(name=name, io=s["io"], ti=ti, u=u, delta=delta, A=A, B=B, C=C, Dskip=Dskip, z=z,
                  want_last=s["last"])


@dataclasses.dataclass
class SsdInputs:
    """One scalar-decay workload (float32 arrays holding bf16-exact values; A, Dskip fp32)."""
    name: str
    x: np.ndarray        # [batch, L, H, 64]
    delta: np.ndarray    # [batch, L, H]
    A: np.ndarray        # [H]
    B: np.ndarray        # [batch, L, N]
    C: np.ndarray        # [batch, L, N]
    Dskip: np.ndarray    # [H * 64]
    z: np.ndarray        # [batch, L, H, 64]


def generate_ssd(name: str, *, seed: Optional[int] = None) -> SsdInputs:
    """Draw a scalar-decay workload: x, B, C, z standard normal; delta log-uniform in
    [1e-3, 1e-1] (the canonical time-step range); A_h = -exp(U(0, ln 16)) per head (Mamba-2
    draws its per-head rate from a range of that kind); Dskip = 1.  Draw order x, delta, A, B, C, z;
    bf16 rounding (nearest even) for x, delta, B, C, z."""
    s = SSD_WORKLOADS[name]
    rng = np.random.Generator(np.random.PCG64(1000 + s["number"] if seed is None else seed))
    b, L, H, N = s["batch"], s["L"], s["H"], s["N"]
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    x = bf16_round(f32(rng.standard_normal((b, L, H, 64))))
    delta = bf16_round(f32(np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), (b, L, H)))))
    A = f32(-np.exp(rng.uniform(0.0, np.log(16.0), H)))
    B = bf16_round(f32(rng.standard_normal((b, L, N))))
    C = bf16_round(f32(rng.standard_normal((b, L, N))))
    z = bf16_round(f32(rng.standard_normal((b, L, H, 64))))
    return SsdInputs(name=name, x=x, delta=delta, A=A, B=B, C=C, Dskip=np.ones(H * 64, np.float32), z=z)


# Rates whose product with a step of 1e-3 is 1e-6 .. 1e-10, and zero: the ZOH input
# coefficient (exp(delta a) - 1)/a cancels there in float32.
SMALL_RATES = (-1e-3, -1e-5, -1e-7, 0.0)


def small_rates(batch: int, L: int, D: int, N: int, io: str = "f32", seed: int = 31,
                step: float = 1e-3, block: int = 64) -> Inputs:
    """Inputs with rates near zero.  Channels come in blocks of ``block``; block k is of
    kind k mod 3: (0) every rate small, cycling over SMALL_RATES by channel and state; (1)
    small and canonical rates alternating over the states; (2) canonical rates only,
    A[d, n] = -(n + 1).  Channels that own a small rate take the constant step ``step``, so
    that every token rounds the same way; the others draw log-uniform steps in [1e-3, 1e-1].
    u, B, C ~ N(0, 1); no feed-through and no gate, so y is the scan's term alone.  Draw
    order: u, delta, B, C."""
    rng = np.random.Generator(np.random.PCG64(seed))
    u = rng.standard_normal((batch, L, D))
    delta = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), (batch, L, D)))
    B = rng.standard_normal((batch, L, N))
    C = rng.standard_normal((batch, L, N))
    A = -(np.arange(N, dtype=np.float64) + 1.0)[None, :].repeat(D, axis=0)
    kind = (np.arange(D) // block) % 3
    for d in range(D):
        for n in range(N):
            if kind[d] == 0 or (kind[d] == 1 and n % 2 == 0):
                A[d, n] = SMALL_RATES[(d + n) % len(SMALL_RATES)]
    delta[..., kind != 2] = step
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    u, delta, B, C, A = map(f32, (u, delta, B, C, A))
    if io == "bf16":
        u, delta, B, C = bf16_round(u), bf16_round(delta), bf16_round(B), bf16_round(C)
    return Inputs(name="small_rates", io=io, ti=False, u=u, delta=delta, A=A, B=B, C=C, Dskip=None, z=None,
                  want_last=True)


def running_state(inp: Inputs, seed: int = 11, scale: float = 0.1) -> np.ndarray:
    """A seeded [batch, D, N] float32 state to continue from (the decode workload's running
    state): normal with standard deviation ``scale``."""
    b, _, D, N = inp.shape
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.ascontiguousarray(rng.standard_normal((b, D, N)) * scale, dtype=np.float32)


def raw_step_sizes(inp: Inputs, seed: int = 17, spread: float = 0.5):
    """Inputs for the fused step-size transform: (raw, bias) with raw shaped like ``inp.delta``
    (float32; bf16-exact for bf16 workloads) and bias [D] float32, so that the step size is
    softplus(raw + bias).  bias[d] is the inverse softplus of a log-uniform step in
    [1e-3, 1e-1] (the canonical S6 time-step initialisation), raw is normal with standard
    deviation ``spread`` (a projection's output around it)."""
    D = inp.A.shape[0]
    rng = np.random.Generator(np.random.PCG64(seed))
    dt0 = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), D))
    bias = np.log(np.expm1(dt0))
    raw = rng.normal(0.0, spread, inp.delta.shape)
    raw = np.ascontiguousarray(raw, dtype=np.float32)
    if inp.io == "bf16":
        raw = bf16_round(raw)
    return raw, np.ascontiguousarray(bias, dtype=np.float32)


def sample_channels(D: int, count: int, seed: int = 7) -> np.ndarray:
    """A sorted, seeded sample of channel indices that always includes the first and last
    channel (ragged edges) and a few channel-tile boundaries."""
    rng = np.random.Generator(np.random.PCG64(seed))
    must = {0, D - 1, min(D - 1, 3), min(D - 1, 4), min(D - 1, 63), min(D - 1, 64)}
    extra = rng.choice(D, size=min(D, max(0, count - len(must))), replace=False)
    return np.array(sorted(must.union(int(x) for x in extra)), dtype=np.int64)


def select_channels(inp: Inputs, ch) -> Inputs:
    """The same workload restricted to channels ``ch``.  In the selective mode B and C are
    shared by all channels of a token, so the restriction is exact."""
    ch = np.asarray(ch)
    sub = lambda a: None if a is None else np.ascontiguousarray(a[..., ch])
    return Inputs(
        name=inp.name, io=inp.io, ti=inp.ti, u=sub(inp.u),
        delta=np.ascontiguousarray(inp.delta[ch]) if inp.ti else sub(inp.delta),
        A=np.ascontiguousarray(inp.A[ch]),
        B=np.ascontiguousarray(inp.B[ch]) if inp.ti else inp.B,
        C=np.ascontiguousarray(inp.C[ch]) if inp.ti else inp.C,
        Dskip=None if inp.Dskip is None else np.ascontiguousarray(inp.Dskip[ch]),
        z=sub(inp.z), want_last=inp.want_last)
