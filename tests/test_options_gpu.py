"""GPU parity of the discretisation options against the oracle: the first-order input
coefficient Bbar = delta * B (Algenta "Sequence and state-space models",
mamba_selective_scan_step; TorchLean "Selective Mamba", step) and the fused step-size
transform softplus(delta + bias[d]) (TorchLean "Selective Mamba", step: softplus of the
projection plus dtBias).  Every kernel is covered: the software-pipelined one (N % 4 == 0,
aligned rows), the per-element one (forced, or for N of 3 and 6), both chunked passes, the
time-invariant kernels and the decode step.  Same bar as the forward pass:
max|y - y_ref| / max|y_ref| <= 1e-4 (fp32 I/O), 2e-2 (bf16 I/O); states (fp32) <= 1e-4."""
import numpy as np
import pytest

import oracle
import s6_workloads
from tests.gpu_common import TOL, TOL_STATE, dev, log_errors, rel_err

pytestmark = pytest.mark.gpu

CASES = {
    "small_f32": dict(batch=2, L=300, D=40),
    "mamba130m_f32": dict(batch=2, L=530, D=100),
    "longctx_bf16": dict(batch=2, L=700, D=36),
    "s4d_ti_f32": dict(batch=2, L=400, D=44),
}


def torch():
    import torch as t
    return t


def to_gpu(inp, delta=None):
    t = torch()
    return dict(u=dev(inp.u, inp.io), delta=dev(inp.delta if delta is None else delta, inp.io), B=dev(inp.B, inp.io),
                C=dev(inp.C, inp.io), z=dev(inp.z, inp.io), A=t.from_numpy(inp.A).cuda(),
                Dskip=None if inp.Dskip is None else t.from_numpy(inp.Dskip).cuda())


def run_both(inp, *, delta=None, bias=None, softplus=False, euler=False, h0=None, path="auto", scalar_io=False):
    import selective_state_space_s6_amd as ss
    t = torch()
    dl = inp.delta if delta is None else delta
    y_ref, l_ref = oracle.fwd(inp.u, dl, inp.A, inp.B, inp.C, inp.Dskip, inp.z, h0=h0, delta_bias=bias,
                              delta_softplus=softplus, euler=euler, time_invariant=inp.ti)
    g = to_gpu(inp, dl)
    y, last = ss.selective_scan_fwd(
        g["u"], g["delta"], g["A"], g["B"], g["C"], g["Dskip"], g["z"], return_last_state=True, path=path,
        scalar_io=scalar_io, initial_state=None if h0 is None else t.from_numpy(h0).cuda(),
        delta_bias=None if bias is None else t.from_numpy(bias).cuda(), delta_softplus=softplus,
        discretization="euler" if euler else "zoh")
    t.cuda.synchronize()
    return rel_err(y.float().cpu().numpy(), y_ref), rel_err(last.cpu().numpy(), l_ref)


@pytest.mark.parametrize("scalar_io", [False, True])
@pytest.mark.parametrize("path", ["single", "chunked"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_euler_parity(name, path, scalar_io):
    inp = s6_workloads.generate(name, "active", **CASES[name])
    e_y, e_l = run_both(inp, euler=True, path=path, scalar_io=scalar_io)
    log_errors("euler/%s/%s/%s" % (name, path, scalar_io), y=e_y, last_state=e_l, io=inp.io)
    assert e_y <= TOL[inp.io] and e_l <= TOL_STATE, (e_y, e_l)


@pytest.mark.parametrize("euler", [False, True])
@pytest.mark.parametrize("scalar_io", [False, True])
@pytest.mark.parametrize("path", ["single", "chunked"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_softplus_parity(name, path, scalar_io, euler):
    inp = s6_workloads.generate(name, **CASES[name])
    raw, bias = s6_workloads.raw_step_sizes(inp)
    e_y, e_l = run_both(inp, delta=raw, bias=bias, softplus=True, euler=euler, path=path, scalar_io=scalar_io)
    log_errors("softplus/%s/%s/%s/%s" % (name, path, scalar_io, euler), y=e_y, last_state=e_l, io=inp.io)
    assert e_y <= TOL[inp.io] and e_l <= TOL_STATE, (e_y, e_l)


@pytest.mark.parametrize("N", [3, 6, 12, 32, 64])
@pytest.mark.parametrize("path", ["single", "chunked"])
def test_options_state_counts(N, path):
    """Every lane layout: N = 3 and 6 (per-element kernel, 4 and 8 lanes per channel), 12
    (padded quads), 32 and 64 (two and four states per lane)."""
    inp = s6_workloads.generate("mamba130m_f32", batch=2, L=333, D=52, N=N)
    raw, bias = s6_workloads.raw_step_sizes(inp, seed=N)
    e_y, e_l = run_both(inp, delta=raw, bias=bias, softplus=True, euler=(N % 2 == 0), path=path)
    assert e_y <= TOL["f32"] and e_l <= TOL_STATE, (N, e_y, e_l)


def test_bias_without_softplus():
    """The bias alone shifts the step size (no softplus)."""
    inp = s6_workloads.generate("small_f32", batch=2, L=260, D=40)
    bias = np.full(40, 0.01, np.float32) * (1 + np.arange(40, dtype=np.float32) % 3)
    for path in ("single", "chunked"):
        for scalar_io in (False, True):
            e_y, e_l = run_both(inp, bias=bias, path=path, scalar_io=scalar_io)
            assert e_y <= TOL["f32"] and e_l <= TOL_STATE, (path, scalar_io, e_y, e_l)


def test_softplus_per_channel_delta_selective():
    """Selective B/C with a per-channel (zero-stride) delta, transformed once per channel."""
    inp = s6_workloads.generate("small_f32", batch=2, L=300, D=40)
    raw = np.random.default_rng(5).normal(-4.0, 1.0, 40).astype(np.float32)
    bias = np.random.default_rng(6).normal(0.0, 0.5, 40).astype(np.float32)
    full = np.ascontiguousarray(np.broadcast_to(raw, inp.u.shape))
    import selective_state_space_s6_amd as ss
    t = torch()
    y_ref, l_ref = oracle.fwd(inp.u, full, inp.A, inp.B, inp.C, inp.Dskip, inp.z, delta_bias=bias,
                              delta_softplus=True)
    g = to_gpu(inp)
    for path in ("single", "chunked"):
        y, last = ss.selective_scan_fwd(g["u"], t.from_numpy(raw).cuda(), g["A"], g["B"], g["C"], g["Dskip"], g["z"],
                                        return_last_state=True, path=path, delta_bias=t.from_numpy(bias).cuda(),
                                        delta_softplus=True)
        t.cuda.synchronize()
        assert rel_err(y.cpu().numpy(), y_ref) <= TOL["f32"]
        assert rel_err(last.cpu().numpy(), l_ref) <= TOL_STATE


@pytest.mark.parametrize("path", ["single", "chunked"])
def test_options_with_initial_state(path):
    inp = s6_workloads.generate("longctx_bf16", batch=2, L=640, D=36)
    raw, bias = s6_workloads.raw_step_sizes(inp)
    h0 = s6_workloads.running_state(inp, scale=1.0)
    e_y, e_l = run_both(inp, delta=raw, bias=bias, softplus=True, euler=True, h0=h0, path=path)
    assert e_y <= TOL["bf16"] and e_l <= TOL_STATE, (e_y, e_l)


STEP_CASES = [("longctx_bf16", 16, 36), ("mamba130m_f32", 16, 7), ("mamba130m_f32", 64, 36),
              ("small_f32", 17, 36), ("s4d_ti_f32", 64, 36), ("s4d_ti_f32", 4, 7)]


@pytest.mark.parametrize("euler", [False, True])
@pytest.mark.parametrize("name,N,D", STEP_CASES)
def test_step_options_parity(name, N, D, euler):
    """The decode step with the step-size transform (and the first-order coefficient)
    against the oracle run over one token from the same state."""
    import selective_state_space_s6_amd as ss
    t = torch()
    inp = s6_workloads.generate(name, batch=9, L=1, D=D, N=N)
    raw, bias = s6_workloads.raw_step_sizes(inp)
    h0 = s6_workloads.running_state(inp, scale=1.0)
    y_ref, l_ref = oracle.fwd(inp.u, raw, inp.A, inp.B, inp.C, inp.Dskip, inp.z, h0=h0, delta_bias=bias,
                              delta_softplus=True, euler=euler, time_invariant=inp.ti)
    g = to_gpu(inp, raw)
    state = t.from_numpy(h0).cuda()
    rows = lambda x: None if x is None else x[:, 0]
    y = ss.selective_scan_step(rows(g["u"]), g["delta"] if inp.ti else rows(g["delta"]), g["A"],
                               g["B"] if inp.ti else rows(g["B"]), g["C"] if inp.ti else rows(g["C"]), g["Dskip"],
                               rows(g["z"]), state=state, time_invariant=inp.ti,
                               delta_bias=t.from_numpy(bias).cuda(), delta_softplus=True,
                               discretization="euler" if euler else "zoh")
    t.cuda.synchronize()
    e_y = rel_err(y.float().cpu().numpy(), y_ref[:, 0])
    e_l = rel_err(state.cpu().numpy(), l_ref)
    log_errors("step_options/%s/%d/%d/%s" % (name, N, D, euler), y=e_y, last_state=e_l, io=inp.io)
    assert e_y <= TOL[inp.io] and e_l <= TOL_STATE, (e_y, e_l)


def test_decode_loop_with_options_equals_scan():
    """Twelve decode steps with the transform and the first-order coefficient give the
    scan's outputs and final state."""
    import selective_state_space_s6_amd as ss
    t = torch()
    inp = s6_workloads.generate("small_f32", batch=3, L=12, D=40)
    raw, bias = s6_workloads.raw_step_sizes(inp)
    g = to_gpu(inp, raw)
    tb = t.from_numpy(bias).cuda()
    y_scan, l_scan = ss.selective_scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["Dskip"], g["z"],
                                           return_last_state=True, delta_bias=tb, delta_softplus=True,
                                           discretization="euler")
    state = t.zeros((3, 40, 16), dtype=t.float32, device="cuda")
    ys = []
    for l in range(12):
        ys.append(ss.selective_scan_step(g["u"][:, l], g["delta"][:, l], g["A"], g["B"][:, l], g["C"][:, l],
                                         g["Dskip"], g["z"][:, l], state=state, delta_bias=tb, delta_softplus=True,
                                         discretization="euler"))
    t.cuda.synchronize()
    y_loop = t.stack(ys, dim=1)
    assert rel_err(y_loop.cpu().numpy(), y_scan.cpu().numpy()) <= 1e-5
    assert rel_err(state.cpu().numpy(), l_scan.cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("option", ["softplus", "euler"])
def test_full_size_longctx_options(option):
    """The long-context forward at full size in the benchmark's launch configuration, with the
    fused step size softplus(raw + bias[d]) (TorchLean "Selective Mamba", step) or with the
    first-order coefficient (Algenta "Sequence and state-space models",
    mamba_selective_scan_step), against the oracle on sampled channels of every batch row."""
    import dataclasses
    import selective_state_space_s6_amd as ss
    t = torch()
    inp = s6_workloads.generate("longctx_bf16")
    bias = None
    if option == "softplus":
        raw, bias = s6_workloads.raw_step_sizes(inp)
        inp = dataclasses.replace(inp, delta=raw)
    g = to_gpu(inp)
    y, _ = ss.selective_scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["Dskip"], g["z"],
                                 delta_bias=None if bias is None else t.from_numpy(bias).cuda(),
                                 delta_softplus=option == "softplus", discretization=option if option == "euler" else "zoh")
    t.cuda.synchronize()
    ch = s6_workloads.sample_channels(inp.u.shape[2], 24)
    sub = s6_workloads.select_channels(inp, ch)
    y_ref, _ = oracle.fwd(sub.u, sub.delta, sub.A, sub.B, sub.C, sub.Dskip, sub.z,
                          delta_bias=None if bias is None else np.ascontiguousarray(bias[ch]),
                          delta_softplus=option == "softplus", euler=option == "euler", want_last=False)
    e_y = rel_err(y.float().cpu().numpy()[..., ch], y_ref)
    log_errors("full/longctx/%s" % option, y=e_y, io="bf16")
    assert e_y <= TOL["bf16"], e_y
