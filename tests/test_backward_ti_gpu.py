"""GPU parity of the backward pass with fixed (time-invariant) coefficients -- delta [D], B and
C [D, N] shared by every batch row and token -- against the oracle's reverse-time recurrence
(rustytorch commit log: hand-written VJP of the selective scan, which differentiates every
block parameter), gradient by gradient: max|g - g_ref| / max|g_ref| <= 1e-4 (fp32 I/O) or 2e-2
(bf16 I/O, whose du, dz, ddelta, dB and dC are rounded to bf16).  ddelta [D], dB and dC [D, N]
are the sums over batch rows and tokens.  Cases span ragged 16-token tiles, sequence chunks
(the chunk end states composed by the prefix, the chunk adjoints combined), every state layout,
both discretisations, the fused softplus step size, an initial state and a gradient reaching
the final state, no gate, an empty sequence, and the full time-invariant workload on sampled
channels."""
import numpy as np
import pytest

import oracle
import s6_workloads
from tests.gpu_common import TOL, dev, log_errors, rel_err

pytestmark = pytest.mark.gpu


def torch():
    import torch as t
    return t


def run_ti(inp, *, delta=None, bias=None, softplus=False, euler=False, h0=None, dlast=None, seed=5, ref=True):
    import selective_state_space_s6_amd as ss
    t = torch()
    rng = np.random.default_rng(seed)
    b, L, D, N = inp.shape
    dy = rng.standard_normal((b, L, D)).astype(np.float32)
    if inp.io == "bf16":
        dy = s6_workloads.bf16_round(dy)
    dl = inp.delta if delta is None else delta
    io = inp.io
    g = ss.selective_scan_bwd(
        dev(inp.u, io), dev(dl, io), t.from_numpy(inp.A).cuda(), dev(inp.B, io), dev(inp.C, io),
        None if inp.Dskip is None else t.from_numpy(inp.Dskip).cuda(), dev(inp.z, io), dy=dev(dy, io),
        dlast_state=None if dlast is None else t.from_numpy(dlast).cuda(),
        initial_state=None if h0 is None else t.from_numpy(h0).cuda(),
        delta_bias=None if bias is None else t.from_numpy(bias).cuda(), delta_softplus=softplus,
        discretization="euler" if euler else "zoh")
    t.cuda.synchronize()
    out = {k: v.float().cpu().numpy() for k, v in g.items()}
    if not ref:
        return out, dy
    r = oracle.bwd(inp.u, dl, inp.A, inp.B, inp.C, inp.Dskip, inp.z, dy=dy, dlast=dlast, h0=h0, delta_bias=bias,
                   euler=euler, delta_softplus=softplus, time_invariant=True)
    names = {"dinitial_state": "dh0"}
    return {k: rel_err(v, r[names.get(k, k)]) for k, v in out.items()}, None


def to_bf16(inp):
    bf = s6_workloads.bf16_round
    inp.u, inp.delta, inp.B, inp.C = bf(inp.u), bf(inp.delta), bf(inp.B), bf(inp.C)
    inp.z = None if inp.z is None else bf(inp.z)
    inp.io = "bf16"
    return inp


def check(errs, io, case):
    log_errors("bwd_ti/" + case, io=io, **errs)
    bad = {k: e for k, e in errs.items() if not e <= TOL[io]}
    assert not bad, (case, errs)


@pytest.mark.parametrize("N", [4, 16, 24, 32, 64])
@pytest.mark.parametrize("L", [1, 15, 16, 17, 333])
def test_ti_backward_state_counts_and_lengths(N, L):
    inp = s6_workloads.generate("s4d_ti_f32", "active", batch=2, L=L, D=20, N=N, gate=True)
    errs, _ = run_ti(inp, seed=N + L)
    assert errs["ddelta"] >= 0 and "dz" in errs
    check(errs, "f32", "N=%d L=%d" % (N, L))


@pytest.mark.parametrize("batch,L,D,N", [(1, 1000, 24, 16), (2, 700, 40, 64), (3, 2100, 8, 32)])
def test_ti_backward_sequence_chunks(batch, L, D, N):
    """Few (batch row, channel group) items: the plan splits the sequence into chunks."""
    inp = s6_workloads.generate("s4d_ti_f32", "active", batch=batch, L=L, D=D, N=N, gate=True)
    check(run_ti(inp, seed=L)[0], "f32", "chunks b=%d L=%d D=%d N=%d" % (batch, L, D, N))


@pytest.mark.parametrize("variant", ["default", "scan_only", "active_const"])
def test_ti_backward_variants_bf16(variant):
    inp = to_bf16(s6_workloads.generate("s4d_ti_f32", variant, batch=2, L=300, D=44, N=64, gate=True))
    check(run_ti(inp)[0], "bf16", "bf16/" + variant)


@pytest.mark.parametrize("euler", [False, True])
@pytest.mark.parametrize("softplus", [False, True])
def test_ti_backward_options(euler, softplus):
    inp = s6_workloads.generate("s4d_ti_f32", batch=2, L=500, D=16, N=32, gate=True)
    bias = None
    delta = None
    if softplus:
        delta, bias = s6_workloads.raw_step_sizes(inp)
    errs, _ = run_ti(inp, delta=delta, bias=bias, softplus=softplus, euler=euler)
    if softplus:
        assert "ddelta_bias" in errs
    check(errs, "f32", "euler=%s softplus=%s" % (euler, softplus))


@pytest.mark.parametrize("L", [40, 900])
def test_ti_backward_initial_and_final_state(L):
    inp = s6_workloads.generate("s4d_ti_f32", "active", batch=2, L=L, D=24, N=16, gate=True)
    b, _, D, N = inp.shape
    h0 = np.random.default_rng(3).standard_normal((b, D, N)).astype(np.float32)
    dlast = np.random.default_rng(4).standard_normal((b, D, N)).astype(np.float32)
    errs, _ = run_ti(inp, h0=h0, dlast=dlast)
    assert "dinitial_state" in errs
    check(errs, "f32", "h0+dlast L=%d" % L)


def test_ti_backward_small_and_zero_rates():
    inp = s6_workloads.generate("s4d_ti_f32", batch=2, L=200, D=16, N=16, gate=True)
    A = inp.A.copy()
    A[:, 0], A[:, 1], A[:, 2], A[:, 3] = 0.0, -1e-7, -1e-5, -1e-3
    inp.A = A
    check(run_ti(inp)[0], "f32", "small rates")


def test_ti_backward_without_gate_or_feedthrough_and_empty():
    inp = s6_workloads.generate("s4d_ti_f32", "scan_only", batch=2, L=70, D=24, N=16)
    errs, _ = run_ti(inp)
    assert "dz" not in errs and "dDskip" not in errs
    check(errs, "f32", "scan_only")
    # no tokens: every sum is empty (zero) and the initial state's gradient is dlast
    import selective_state_space_s6_amd as ss
    t = torch()
    D, N = 24, 16
    e = lambda *sh: t.zeros(sh, dtype=t.float32, device="cuda")
    dlast = t.randn(2, D, N, device="cuda")
    g = ss.selective_scan_bwd(e(2, 0, D), t.full((D,), 0.05, device="cuda"), -t.ones(D, N, device="cuda"),
                              t.randn(D, N, device="cuda"), t.randn(D, N, device="cuda"), t.ones(D, device="cuda"),
                              e(2, 0, D), dy=e(2, 0, D), dlast_state=dlast, initial_state=e(2, D, N))
    t.cuda.synchronize()
    for k in ("ddelta", "dB", "dC", "dA", "dDskip"):
        assert g[k].shape[0] == D and not g[k].any(), k
    assert t.equal(g["dinitial_state"], dlast)


def test_ti_backward_deterministic():
    inp = s6_workloads.generate("s4d_ti_f32", "active", batch=2, L=800, D=24, N=32, gate=True)
    a, _ = run_ti(inp, ref=False)
    b, _ = run_ti(inp, ref=False)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_ti_backward_full_size_sampled_channels():
    """The full time-invariant workload (batch 4, L 8192, D 1024, N 64, fp32), with a gate, on
    every channel; checked against the oracle on sampled channels (each channel's gradients
    depend on that channel only)."""
    inp = s6_workloads.generate("s4d_ti_f32", gate=True)
    out, dy = run_ti(inp, ref=False)
    for k, v in out.items():
        assert np.all(np.isfinite(v)), k
    ch = s6_workloads.sample_channels(inp.u.shape[2], 24)
    sub = s6_workloads.select_channels(inp, ch)
    r = oracle.bwd(sub.u, sub.delta, sub.A, sub.B, sub.C, sub.Dskip, sub.z, dy=np.ascontiguousarray(dy[..., ch]),
                   time_invariant=True)
    errs = {"du": rel_err(out["du"][..., ch], r["du"]), "dz": rel_err(out["dz"][..., ch], r["dz"]),
            "ddelta": rel_err(out["ddelta"][ch], r["ddelta"]), "dA": rel_err(out["dA"][ch], r["dA"]),
            "dB": rel_err(out["dB"][ch], r["dB"]), "dC": rel_err(out["dC"][ch], r["dC"]),
            "dDskip": rel_err(out["dDskip"][ch], r["dDskip"])}
    check(errs, "f32", "full/s4d_ti_f32")
