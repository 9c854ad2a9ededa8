"""GPU parity of the convolution mode of fixed (time-invariant) coefficients (path "conv"):
y = K * u with the lag kernel K_k = sum_n C_n Abar_n^k Bbar_n ("state-space models"
(aarnphm.xyz), section "One recurrence, one convolution"; Algenta "Sequence and state-space
models", s4_kernel_element), computed as 16-token block Toeplitz products on the fp32 matrix
cores with the state carried between blocks.  Checked against the oracle's FFT convolution
(oracle.conv_ti) and its fp64 recurrence (gate, options, final state), on every state-block
count (N 16..64, padded N 24 and 40), ragged blocks and super-tiles, several channel groups,
both element types, and at the full time-invariant workload on sampled channels.  Bar as for
the recurrence: max|err| / max|ref| <= 1e-4 (fp32 I/O), 2e-2 (bf16 I/O); states <= 1e-4."""
import numpy as np
import pytest

import oracle
import s6_workloads
from tests.gpu_common import TOL, TOL_STATE, dev, log_errors, rel_err

pytestmark = pytest.mark.gpu


def torch():
    import torch as t
    return t


def run_conv(inp, *, bias=None, softplus=False, euler=False, want_last=True, path="conv"):
    import selective_state_space_s6_amd as ss
    t = torch()
    io = inp.io
    y, last = ss.selective_scan_fwd(dev(inp.u, io), dev(inp.delta, io), t.from_numpy(inp.A).cuda(), dev(inp.B, io),
                                    dev(inp.C, io), None if inp.Dskip is None else t.from_numpy(inp.Dskip).cuda(),
                                    dev(inp.z, io), return_last_state=want_last, path=path,
                                    delta_bias=None if bias is None else t.from_numpy(bias).cuda(),
                                    delta_softplus=softplus, discretization="euler" if euler else "zoh")
    t.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), None if last is None else last.cpu().numpy()


@pytest.mark.parametrize("N", [16, 24, 32, 40, 64])
@pytest.mark.parametrize("L", [1, 15, 16, 17, 255, 256, 257, 700])
def test_conv_against_fft_convolution(N, L):
    inp = s6_workloads.generate("s4d_ti_f32", batch=2, L=L, D=20, N=N)
    y, last = run_conv(inp)
    y_ref = oracle.conv_ti(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip)
    _, l_ref = oracle.fwd(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, None, time_invariant=True)
    e_y, e_l = rel_err(y, y_ref), rel_err(last, l_ref)
    log_errors("conv N=%d L=%d" % (N, L), y=e_y, last_state=e_l, io="f32")
    assert e_y <= TOL["f32"] and e_l <= TOL_STATE, (e_y, e_l)


@pytest.mark.parametrize("variant", ["scan_only", "active", "active_const"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_variants_and_gate(variant, io):
    inp = s6_workloads.generate("s4d_ti_f32", variant, batch=2, L=600, D=44, N=64, gate=True)
    if io == "bf16":
        bf = s6_workloads.bf16_round
        inp.u, inp.delta, inp.B, inp.C = bf(inp.u), bf(inp.delta), bf(inp.B), bf(inp.C)
        inp.z = None if inp.z is None else bf(inp.z)
        inp.io = "bf16"
    y, last = run_conv(inp)
    y_ref, l_ref = oracle.fwd(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z, time_invariant=True)
    e_y, e_l = rel_err(y, y_ref), rel_err(last, l_ref)
    log_errors("conv/%s/%s" % (variant, io), y=e_y, last_state=e_l, io=io)
    assert e_y <= TOL[io] and e_l <= TOL_STATE, (e_y, e_l)


@pytest.mark.parametrize("euler", [False, True])
@pytest.mark.parametrize("softplus", [False, True])
def test_conv_options(euler, softplus):
    inp = s6_workloads.generate("s4d_ti_f32", batch=2, L=333, D=16, N=32)
    bias = None
    if softplus:
        raw, bias = s6_workloads.raw_step_sizes(inp)
        inp.delta = raw
    y, last = run_conv(inp, bias=bias, softplus=softplus, euler=euler)
    y_ref, l_ref = oracle.fwd(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, None, time_invariant=True,
                              delta_bias=bias, delta_softplus=softplus, euler=euler)
    e_y, e_l = rel_err(y, y_ref), rel_err(last, l_ref)
    log_errors("conv/options euler=%s softplus=%s" % (euler, softplus), y=e_y, last_state=e_l, io="f32")
    assert e_y <= TOL["f32"] and e_l <= TOL_STATE, (e_y, e_l)


def test_conv_matches_recurrence_and_is_deterministic():
    inp = s6_workloads.generate("s4d_ti_f32", batch=2, L=1000, D=24, N=64)
    y1, l1 = run_conv(inp)
    y2, l2 = run_conv(inp)
    assert np.array_equal(y1, y2) and np.array_equal(l1, l2)
    y_rec, l_rec = run_conv(inp, path="auto")
    assert rel_err(y1, y_rec) <= 1e-5 and rel_err(l1, l_rec) <= 1e-5


def test_conv_full_size_sampled_channels():
    """The full time-invariant workload (batch 4, L 8192, D 1024, N 64, fp32) through the
    convolution mode, against the oracle's FFT convolution on sampled channels."""
    inp = s6_workloads.generate("s4d_ti_f32")
    y, _ = run_conv(inp, want_last=False)
    assert np.all(np.isfinite(y))
    ch = s6_workloads.sample_channels(inp.u.shape[2], 24)
    sub = s6_workloads.select_channels(inp, ch)
    y_ref = oracle.conv_ti(sub.u, sub.delta, sub.A, sub.B, sub.C, sub.Dskip)
    e_y = rel_err(y[..., ch], y_ref)
    log_errors("conv/full/s4d_ti_f32", y=e_y, io="f32")
    assert e_y <= TOL["f32"], e_y


def test_conv_refuses_selective_coefficients_and_initial_state():
    import selective_state_space_s6_amd as ss
    t = torch()
    inp = s6_workloads.generate("small_f32", batch=1, L=64, D=8)
    g = {k: dev(getattr(inp, k), "f32") for k in ("u", "delta", "B", "C")}
    with pytest.raises(ss.SelscanError):
        ss.selective_scan_fwd(g["u"], g["delta"], t.from_numpy(inp.A).cuda(), g["B"], g["C"], path="conv")
    ti = s6_workloads.generate("s4d_ti_f32", batch=1, L=64, D=8, N=16)
    gt = {k: dev(getattr(ti, k), "f32") for k in ("u", "delta", "B", "C")}
    with pytest.raises(ss.SelscanError):
        ss.selective_scan_fwd(gt["u"], gt["delta"], t.from_numpy(ti.A).cuda(), gt["B"], gt["C"], path="conv",
                              initial_state=t.zeros(1, 8, 16, device="cuda"))
