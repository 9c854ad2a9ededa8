"""GPU parity of the backward pass (selective_scan_bwd) against the oracle's reverse-time
recurrence (rustytorch commit log: hand-written VJP of the selective scan), gradient by
gradient: max|g - g_ref| / max|g_ref| <= 1e-4 (fp32 I/O) or 2e-2 (bf16 I/O, whose du, ddelta,
dz, dB and dC are rounded to bf16), for every gradient the call returns.  Cases span several
16-token tiles with ragged tails, channel groups with a partial last group, every state
layout (one, two and four states per lane, padded states), both discretisations, the fused
softplus step size, an initial state and a gradient reaching the final state."""
import numpy as np
import pytest

import oracle
import s6_workloads
from tests.gpu_common import TOL, dev, log_errors, rel_err

pytestmark = pytest.mark.gpu


def torch():
    import torch as t
    return t


def run_case(inp, *, delta=None, bias=None, softplus=False, euler=False, h0=None, dlast=None, seed=5, row_pad=0):
    """row_pad > 0: u, delta, z and dy are views into rows of D + row_pad elements."""
    import selective_state_space_s6_amd as ss
    t = torch()
    rng = np.random.default_rng(seed)
    b, L, D, N = inp.shape
    dy = rng.standard_normal((b, L, D)).astype(np.float32)
    if inp.io == "bf16":
        dy = s6_workloads.bf16_round(dy)
    dl = inp.delta if delta is None else delta
    ref = oracle.bwd(inp.u, dl, inp.A, inp.B, inp.C, inp.Dskip, inp.z, dy=dy, dlast=dlast, h0=h0, delta_bias=bias,
                     euler=euler, delta_softplus=softplus)
    io = inp.io

    def tok(x):
        if x is None or row_pad == 0:
            return dev(x, io)
        wide = np.zeros(x.shape[:2] + (D + row_pad,), np.float32)
        wide[..., :D] = x
        return dev(wide, io)[..., :D]

    g = ss.selective_scan_bwd(
        tok(inp.u), tok(dl), t.from_numpy(inp.A).cuda(), dev(inp.B, io), dev(inp.C, io),
        None if inp.Dskip is None else t.from_numpy(inp.Dskip).cuda(), tok(inp.z), dy=tok(dy),
        dlast_state=None if dlast is None else t.from_numpy(dlast).cuda(),
        initial_state=None if h0 is None else t.from_numpy(h0).cuda(),
        delta_bias=None if bias is None else t.from_numpy(bias).cuda(), delta_softplus=softplus,
        discretization="euler" if euler else "zoh")
    t.cuda.synchronize()
    names = {"dinitial_state": "dh0"}
    errs = {}
    for k, v in g.items():
        errs[k] = rel_err(v.float().cpu().numpy(), ref[names.get(k, k)])
    return errs


def check(errs, io, case):
    log_errors("bwd/" + case, io=io, **errs)
    bad = {k: e for k, e in errs.items() if not e <= TOL[io]}
    assert not bad, (case, errs)


CASES = {
    "small_f32": dict(batch=2, L=100, D=40),
    "mamba130m_f32": dict(batch=2, L=130, D=36),
    "longctx_bf16": dict(batch=2, L=150, D=36),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_parity(name):
    inp = s6_workloads.generate(name, "active", **CASES[name])
    check(run_case(inp), inp.io, name)


@pytest.mark.parametrize("name", ["mamba130m_f32", "longctx_bf16"])
@pytest.mark.parametrize("layout", ["odd_channels", "padded_rows"])
def test_backward_element_staging(name, layout):
    """Layouts that the 4-channel vector staging does not take -- a channel count off the
    4-channel grid, rows of u, delta, z and dy 2 elements longer than D -- take the element-wise
    staging; same bar."""
    D = 18 if layout == "odd_channels" else 20
    inp = s6_workloads.generate(name, "active", batch=2, L=150, D=D)
    check(run_case(inp, row_pad=2 if layout == "padded_rows" else 0), inp.io, "%s/%s" % (name, layout))


@pytest.mark.parametrize("N", [3, 8, 16, 17, 32, 48, 64])
@pytest.mark.parametrize("L", [1, 16, 37])
def test_backward_state_counts_and_lengths(N, L):
    inp = s6_workloads.generate("mamba130m_f32", "active", batch=2, L=L, D=20, N=N)
    check(run_case(inp, seed=N + L), "f32", "N=%d L=%d" % (N, L))


@pytest.mark.parametrize("name", ["small_f32", "longctx_bf16"])
def test_backward_options(name):
    inp = s6_workloads.generate(name, **CASES[name])
    raw, bias = s6_workloads.raw_step_sizes(inp)
    check(run_case(inp, delta=raw, bias=bias, softplus=True), inp.io, name + "/softplus")
    check(run_case(inp, euler=True), inp.io, name + "/euler")
    check(run_case(inp, delta=raw, bias=bias, softplus=True, euler=True), inp.io, name + "/softplus+euler")


@pytest.mark.parametrize("name", ["mamba130m_f32", "longctx_bf16"])
def test_backward_initial_and_final_state(name):
    inp = s6_workloads.generate(name, "active", **CASES[name])
    b, L, D, N = inp.shape
    h0 = s6_workloads.running_state(inp, scale=1.0)
    dlast = np.random.default_rng(9).standard_normal((b, D, N)).astype(np.float32)
    check(run_case(inp, h0=h0, dlast=dlast), inp.io, name + "/h0+dlast")


def test_backward_without_gate_or_feedthrough():
    inp = s6_workloads.generate("small_f32", "scan_only", batch=2, L=70, D=24)
    errs = run_case(inp)
    assert "dz" not in errs and "dDskip" not in errs
    check(errs, "f32", "scan_only")


def test_backward_empty_sequence():
    """No tokens: every sum is empty and the initial state's gradient is dlast."""
    import selective_state_space_s6_amd as ss
    t = torch()
    D, N = 8, 16
    e = lambda *s: t.zeros(s, dtype=t.float32, device="cuda")
    dlast = t.randn(2, D, N, device="cuda")
    g = ss.selective_scan_bwd(e(2, 0, D), e(2, 0, D), -t.ones(D, N, device="cuda"), e(2, 0, N), e(2, 0, N),
                              t.ones(D, device="cuda"), dy=e(2, 0, D), dlast_state=dlast, initial_state=e(2, D, N))
    t.cuda.synchronize()
    assert not g["dA"].any() and not g["dDskip"].any()
    assert t.equal(g["dinitial_state"], dlast)


def test_backward_deterministic():
    import selective_state_space_s6_amd as ss
    t = torch()
    inp = s6_workloads.generate("small_f32", batch=2, L=90, D=40)
    args = (dev(inp.u, "f32"), dev(inp.delta, "f32"), t.from_numpy(inp.A).cuda(), dev(inp.B, "f32"),
            dev(inp.C, "f32"), t.from_numpy(inp.Dskip).cuda(), dev(inp.z, "f32"))
    dy = t.randn(2, 90, 40, device="cuda")
    g1 = ss.selective_scan_bwd(*args, dy=dy)
    g2 = ss.selective_scan_bwd(*args, dy=dy)
    t.cuda.synchronize()
    assert all(t.equal(g1[k], g2[k]) for k in g1)


@pytest.mark.parametrize("N", [4, 16, 32, 64])
@pytest.mark.parametrize("L", [333, 1000])
def test_backward_sequence_chunks(N, L):
    """Few (batch row, channel group) items and a long sequence: the backward splits the
    sequence into chunks (ragged last chunk), carrying states forward and adjoints back."""
    inp = s6_workloads.generate("mamba130m_f32", "active", batch=1, L=L, D=24, N=N)
    b, _, D, _ = inp.shape
    h0 = s6_workloads.running_state(inp, scale=1.0)
    dlast = np.random.default_rng(L).standard_normal((b, D, N)).astype(np.float32)
    check(run_case(inp, h0=h0, dlast=dlast, seed=L + N), "f32", "chunks N=%d L=%d" % (N, L))


def test_backward_sequence_chunks_options_bf16():
    inp = s6_workloads.generate("longctx_bf16", batch=1, L=900, D=40)
    raw, bias = s6_workloads.raw_step_sizes(inp)
    check(run_case(inp, delta=raw, bias=bias, softplus=True, euler=True), "bf16", "chunks bf16 options")


def test_backward_full_size_sampled_channels():
    """The benchmark's backward (mamba130m_f32 at full size, automatic chunking): the
    per-channel gradients (du, ddelta, dz, dA, dDskip) against the oracle on sampled channels;
    dB and dC, sums over every channel, by additivity: the full call's dB equals the sum of
    the calls on the two halves of the channels."""
    import selective_state_space_s6_amd as ss
    t = torch()
    inp = s6_workloads.generate("mamba130m_f32")
    b, L, D, N = inp.shape
    dy = np.random.default_rng(4).standard_normal((b, L, D)).astype(np.float32)

    def gpu(sub, dys):
        return ss.selective_scan_bwd(dev(sub.u, "f32"), dev(sub.delta, "f32"), t.from_numpy(sub.A).cuda(),
                                     dev(sub.B, "f32"), dev(sub.C, "f32"), t.from_numpy(sub.Dskip).cuda(),
                                     dev(sub.z, "f32"), dy=dev(dys, "f32"))

    g = gpu(inp, dy)
    ch = s6_workloads.sample_channels(D, 16)
    sub = s6_workloads.select_channels(inp, ch)
    ref = oracle.bwd(sub.u, sub.delta, sub.A, sub.B, sub.C, sub.Dskip, sub.z, dy=np.ascontiguousarray(dy[..., ch]))
    t.cuda.synchronize()
    errs = {k: rel_err(g[k][..., ch].cpu().numpy() if k in ("du", "ddelta", "dz") else
                       (g[k][ch].cpu().numpy()), ref[k]) for k in ("du", "ddelta", "dz", "dA", "dDskip")}
    check(errs, "f32", "full/mamba130m sampled")
    half = D // 2
    parts = [gpu(s6_workloads.select_channels(inp, np.arange(lo, hi)), np.ascontiguousarray(dy[..., lo:hi]))
             for lo, hi in ((0, half), (half, D))]
    t.cuda.synchronize()
    for k in ("dB", "dC"):
        whole = g[k].cpu().numpy().astype(np.float64)
        summed = sum(pp[k].cpu().numpy().astype(np.float64) for pp in parts)
        assert rel_err(whole, summed) <= 1e-5, (k, rel_err(whole, summed))


def test_backward_full_size_longctx_against_oracle():
    """The long-context backward at full size (batch 4, L 16384, D 2560, N 16, bf16 I/O; the
    planner splits the sequence into chunks), in the launch configuration the benchmark times:
    du, ddelta, dz, dA and dDskip against the oracle on sampled channels over every batch row,
    and dB and dC, sums over every channel, against the oracle over all channels of batch row 0
    (rustytorch commit log: hand-written VJP of the selective scan)."""
    import selective_state_space_s6_amd as ss
    t = torch()
    inp = s6_workloads.generate("longctx_bf16")
    b, L, D, N = inp.shape
    dy = s6_workloads.bf16_round(np.random.default_rng(4).standard_normal((b, L, D)).astype(np.float32))
    g = ss.selective_scan_bwd(dev(inp.u, "bf16"), dev(inp.delta, "bf16"), t.from_numpy(inp.A).cuda(),
                              dev(inp.B, "bf16"), dev(inp.C, "bf16"), t.from_numpy(inp.Dskip).cuda(),
                              dev(inp.z, "bf16"), dy=dev(dy, "bf16"))
    t.cuda.synchronize()
    g = {k: v.float().cpu().numpy() for k, v in g.items()}
    ch = s6_workloads.sample_channels(D, 16)
    sub = s6_workloads.select_channels(inp, ch)
    ref = oracle.bwd(sub.u, sub.delta, sub.A, sub.B, sub.C, sub.Dskip, sub.z, dy=np.ascontiguousarray(dy[..., ch]))
    errs = {k: rel_err(g[k][..., ch] if k in ("du", "ddelta", "dz") else g[k][ch], ref[k])
            for k in ("du", "ddelta", "dz", "dA", "dDskip")}
    row = lambda a: np.ascontiguousarray(a[:1])
    ref0 = oracle.bwd(row(inp.u), row(inp.delta), inp.A, row(inp.B), row(inp.C), inp.Dskip, row(inp.z), dy=row(dy))
    for k in ("dB", "dC", "du", "ddelta", "dz"):
        errs[k + "[row 0, all channels]"] = rel_err(g[k][:1], ref0[k])
    check(errs, "bf16", "full/longctx")
