"""GPU parity of the initial-state input and the one-token decode step against the oracle
(TorchLean "Selective Mamba": step / runArray carry an explicit hidden state; aarnphm
"state-space models", "One recurrence, one convolution": the recurrent form).  Same bar as
the forward pass: max|y - y_ref| / max|y_ref| <= 1e-4 (fp32 I/O), 2e-2 (bf16 I/O); states
(fp32) <= 1e-4."""
import numpy as np
import pytest

import oracle
import s6_workloads
from tests.gpu_common import TOL, TOL_STATE, dev, log_errors, rel_err

pytestmark = pytest.mark.gpu


def torch():
    import torch as t
    return t


def to_gpu(inp):
    t = torch()
    return dict(u=dev(inp.u, inp.io), delta=dev(inp.delta, inp.io), B=dev(inp.B, inp.io), C=dev(inp.C, inp.io),
                z=dev(inp.z, inp.io), A=t.from_numpy(inp.A).cuda(),
                Dskip=None if inp.Dskip is None else t.from_numpy(inp.Dskip).cuda())


def initial_state(inp, seed=3):
    b, _, D, N = inp.shape
    return np.random.default_rng(seed).standard_normal((b, D, N)).astype(np.float32)


CASES = {
    "small_f32": dict(batch=2, L=300, D=40),
    "mamba130m_f32": dict(batch=2, L=530, D=100),
    "longctx_bf16": dict(batch=2, L=700, D=36),
}


@pytest.mark.parametrize("scalar_io", [False, True])
@pytest.mark.parametrize("path", ["single", "chunked"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_initial_state_parity(name, path, scalar_io):
    import selective_state_space_s6_amd as ss
    t = torch()
    inp = s6_workloads.generate(name, "active", **CASES[name])
    h0 = initial_state(inp)
    y_ref, l_ref = oracle.fwd(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z, h0=h0)
    g = to_gpu(inp)
    y, last = ss.selective_scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["Dskip"], g["z"],
                                    initial_state=t.from_numpy(h0).cuda(), return_last_state=True, path=path,
                                    scalar_io=scalar_io)
    t.cuda.synchronize()
    e_y = rel_err(y.float().cpu().numpy(), y_ref)
    e_l = rel_err(last.cpu().numpy(), l_ref)
    log_errors("h0/%s/%s/%s" % (name, path, scalar_io), y=e_y, last_state=e_l, io=inp.io)
    assert e_y <= TOL[inp.io] and e_l <= TOL_STATE, (e_y, e_l)


@pytest.mark.parametrize("path", ["single", "chunked"])
def test_continuation_in_place(path):
    """Two calls, the second continuing in place from the first's last_state, against the
    oracle over the whole sequence."""
    import selective_state_space_s6_amd as ss
    t = torch()
    inp = s6_workloads.generate("mamba130m_f32", "active", batch=2, L=777, D=44)
    y_ref, l_ref = oracle.fwd(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z)
    g = to_gpu(inp)
    k = 300
    state = t.empty((2, 44, inp.A.shape[1]), dtype=t.float32, device="cuda")
    y1, _ = ss.selective_scan_fwd(g["u"][:, :k], g["delta"][:, :k], g["A"], g["B"][:, :k], g["C"][:, :k], g["Dskip"],
                                  g["z"][:, :k], last_state=state, path=path)
    y2, _ = ss.selective_scan_fwd(g["u"][:, k:], g["delta"][:, k:], g["A"], g["B"][:, k:], g["C"][:, k:], g["Dskip"],
                                  g["z"][:, k:], last_state=state, initial_state=state, path=path)
    t.cuda.synchronize()
    y = np.concatenate([y1.cpu().numpy(), y2.cpu().numpy()], axis=1)
    assert rel_err(y, y_ref) <= TOL["f32"]
    assert rel_err(state.cpu().numpy(), l_ref) <= TOL_STATE


def test_empty_sequence_hands_back_initial_state():
    import selective_state_space_s6_amd as ss
    t = torch()
    h0 = t.randn((2, 5, 3), device="cuda")
    u = t.zeros((2, 0, 5), device="cuda")
    Bm = t.zeros((2, 0, 3), device="cuda")
    A = -t.ones((5, 3), device="cuda")
    _, last = ss.selective_scan_fwd(u, u, A, Bm, Bm, initial_state=h0, return_last_state=True)
    same = h0.clone()
    ss.selective_scan_fwd(u, u, A, Bm, Bm, initial_state=same, last_state=same)
    t.cuda.synchronize()
    assert t.equal(last, h0) and t.equal(same, h0)


def test_time_invariant_initial_state_is_rejected():
    import selective_state_space_s6_amd as ss
    t = torch()
    inp = s6_workloads.generate("s4d_ti_f32", batch=1, L=32, D=8)
    g = to_gpu(inp)
    with pytest.raises(ss.SelscanError) as err:
        ss.selective_scan_fwd(g["u"], g["delta"], g["A"], g["B"], g["C"], g["Dskip"],
                              initial_state=t.zeros((1, 8, 64), device="cuda"))
    assert err.value.status == ss.SELSCAN_ERR_UNSUPPORTED


def step_inputs(name, variant, batch, D, N, seed):
    inp = s6_workloads.generate(name, variant, batch=batch, L=1, D=D, N=N)
    return inp, initial_state(inp, seed)


@pytest.mark.parametrize("N", [4, 16, 17, 64])
@pytest.mark.parametrize("D", [7, 36])
@pytest.mark.parametrize("name", ["small_f32", "longctx_bf16", "s4d_ti_f32"])
def test_step_parity(name, D, N):
    import selective_state_space_s6_amd as ss
    t = torch()
    inp, h0 = step_inputs(name, "active", 3, D, N, seed=D + N)
    y_ref, l_ref = oracle.fwd(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z, h0=h0,
                              time_invariant=inp.ti)
    g = to_gpu(inp)
    sq = lambda x: None if x is None else x[:, 0]       # [batch, 1, ...] -> [batch, ...]
    delta = g["delta"] if inp.ti else sq(g["delta"])
    B = g["B"] if inp.ti else sq(g["B"])
    C = g["C"] if inp.ti else sq(g["C"])
    state = t.from_numpy(h0).cuda()
    y = ss.selective_scan_step(sq(g["u"]), delta, g["A"], B, C, g["Dskip"], sq(g["z"]), state=state,
                               time_invariant=inp.ti)
    t.cuda.synchronize()
    e_y = rel_err(y.float().cpu().numpy(), y_ref[:, 0])
    e_l = rel_err(state.cpu().numpy(), l_ref)
    log_errors("step/%s/D%d/N%d" % (name, D, N), y=e_y, last_state=e_l, io=inp.io)
    assert e_y <= TOL[inp.io] and e_l <= TOL_STATE, (e_y, e_l)


@pytest.mark.parametrize("name", ["small_f32", "s4d_ti_f32"])
def test_decode_loop_equals_scan(name):
    """Decoding L tokens one step at a time gives the forward pass over the L tokens."""
    import selective_state_space_s6_amd as ss
    t = torch()
    inp = s6_workloads.generate(name, "active", batch=2, L=40, D=12, N=16)
    y_ref, l_ref = oracle.fwd(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z, time_invariant=inp.ti)
    g = to_gpu(inp)
    state = t.zeros((2, 12, 16), device="cuda")
    ys = []
    for l in range(40):
        delta = g["delta"] if inp.ti else g["delta"][:, l]
        B = g["B"] if inp.ti else g["B"][:, l]
        C = g["C"] if inp.ti else g["C"][:, l]
        z = None if g["z"] is None else g["z"][:, l]
        ys.append(ss.selective_scan_step(g["u"][:, l], delta, g["A"], B, C, g["Dskip"], z, state=state,
                                         time_invariant=inp.ti))
    t.cuda.synchronize()
    y = t.stack(ys, dim=1).cpu().numpy()
    assert rel_err(y, y_ref) <= TOL["f32"]
    assert rel_err(state.cpu().numpy(), l_ref) <= TOL_STATE


def test_decode_step_full_size():
    """The decode workload at its full size (512 sequences x 2560 channels x 16 states) in the
    benchmark's call, against the oracle over all of it."""
    import selective_state_space_s6_amd as ss
    t = torch()
    inp = s6_workloads.generate("decode_bf16")
    h0 = s6_workloads.running_state(inp)
    y_ref, l_ref = oracle.fwd(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z, h0=h0)
    g = to_gpu(inp)
    row = lambda x: x[:, 0].contiguous()
    state = t.from_numpy(h0).cuda()
    y = ss.selective_scan_step(row(g["u"]), row(g["delta"]), g["A"], row(g["B"]), row(g["C"]), g["Dskip"], row(g["z"]),
                               state=state)
    t.cuda.synchronize()
    e_y = rel_err(y.float().cpu().numpy(), y_ref[:, 0])
    e_l = rel_err(state.cpu().numpy(), l_ref)
    log_errors("decode/full", y=e_y, last_state=e_l, io="bf16")
    assert e_y <= TOL["bf16"] and e_l <= TOL_STATE, (e_y, e_l)
