"""The caller's workspace carries no information into a call: filled with 0xFF bytes (a NaN
in every fp32 slot) instead of zeros, it must give bit-identical outputs.  A read of a slot
the call did not write first would turn up as NaN or as a difference.  Covered: the chunked
forward through the workspace entry point (one chunk, several, a ragged last chunk, the
time-invariant kernels, an initial state and a fused step size), and the backward pass with
and without sequence chunks.  The chunked path's workspace holds each chunk's end state and
step sum, which the prefix composes into carried-in states (chipfoundry glossary, Appendix
Lab 3: the associative combine)."""
import numpy as np
import pytest

import oracle
import s6_workloads
from tests.gpu_common import TOL, dev, rel_err

pytestmark = pytest.mark.gpu


def torch():
    import torch as t
    return t


def forward_twice(inp, chunk_len, h0=None, bias=None):
    """y, last_state from a zero-filled and from a 0xFF-filled workspace."""
    import selective_state_space_s6_amd as ss
    t = torch()
    io = inp.io
    u, dl, B, C, z = (dev(x, io) for x in (inp.u, inp.delta, inp.B, inp.C, inp.z))
    A = t.from_numpy(inp.A).cuda()
    Ds = None if inp.Dskip is None else t.from_numpy(inp.Dskip).cuda()
    need = ss.workspace_size(ss.make_dims(u, dl, A, B, C, z, u, path="chunked", chunk_len=chunk_len,
                                          delta_softplus=bias is not None))
    assert need > 0
    out = []
    for fill in (0, 255):
        ws = t.full((need,), fill, dtype=t.uint8, device="cuda")
        y, last = ss.selective_scan_fwd(u, dl, A, B, C, Ds, z, return_last_state=True, path="chunked",
                                        chunk_len=chunk_len, workspace=ws,
                                        initial_state=None if h0 is None else t.from_numpy(h0).cuda(),
                                        delta_bias=None if bias is None else t.from_numpy(bias).cuda(),
                                        delta_softplus=bias is not None)
        t.cuda.synchronize()
        out.append((y.clone(), last.clone()))
    return out


@pytest.mark.parametrize("L,chunk_len", [(300, 512), (300, 64), (333, 64), (333, 112), (1000, 0)])
@pytest.mark.parametrize("name", ["small_f32", "longctx_bf16", "s4d_ti_f32"])
def test_forward_workspace_fill_does_not_matter(name, L, chunk_len):
    t = torch()
    inp = s6_workloads.generate(name, batch=2, L=L, D=40)
    (y0, l0), (y1, l1) = forward_twice(inp, chunk_len)
    assert t.equal(y0, y1) and t.equal(l0, l1), name
    assert bool(t.isfinite(y1.float()).all()) and bool(t.isfinite(l1).all())
    y_ref, l_ref = oracle.fwd(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z, time_invariant=inp.ti)
    assert rel_err(y1.float().cpu().numpy(), y_ref) <= TOL[inp.io]
    assert rel_err(l1.cpu().numpy(), l_ref) <= 1e-4


@pytest.mark.parametrize("chunk_len", [512, 64, 112])
def test_forward_workspace_fill_with_initial_state_and_step_size(chunk_len):
    t = torch()
    inp = s6_workloads.generate("mamba130m_f32", "active", batch=2, L=333, D=36)
    raw, bias = s6_workloads.raw_step_sizes(inp)
    inp.delta = raw
    h0 = s6_workloads.running_state(inp, scale=1.0)
    (y0, l0), (y1, l1) = forward_twice(inp, chunk_len, h0=h0, bias=bias)
    assert t.equal(y0, y1) and t.equal(l0, l1)
    y_ref, l_ref = oracle.fwd(inp.u, raw, inp.A, inp.B, inp.C, inp.Dskip, inp.z, h0=h0, delta_bias=bias,
                              delta_softplus=True)
    assert rel_err(y1.cpu().numpy(), y_ref) <= TOL["f32"] and rel_err(l1.cpu().numpy(), l_ref) <= 1e-4


@pytest.mark.parametrize("batch,L,D", [(2, 100, 40), (1, 1000, 24), (1, 333, 40)])
def test_backward_workspace_fill_does_not_matter(batch, L, D):
    import selective_state_space_s6_amd as ss
    t = torch()
    inp = s6_workloads.generate("mamba130m_f32", "active", batch=batch, L=L, D=D)
    u, dl, B, C, z = (dev(x, "f32") for x in (inp.u, inp.delta, inp.B, inp.C, inp.z))
    A = t.from_numpy(inp.A).cuda()
    Ds = t.from_numpy(inp.Dskip).cuda()
    h0 = t.from_numpy(s6_workloads.running_state(inp, scale=1.0)).cuda()
    dy = t.from_numpy(np.random.default_rng(L).standard_normal(inp.u.shape).astype(np.float32)).cuda()
    dlast = t.from_numpy(np.random.default_rng(D).standard_normal((batch, D, 16)).astype(np.float32)).cuda()
    need = ss.bwd_workspace_size(ss.make_dims(u, dl, A, B, C, z, dy))
    out = []
    for fill in (0, 255):
        ws = t.full((need,), fill, dtype=t.uint8, device="cuda")
        g = ss.selective_scan_bwd(u, dl, A, B, C, Ds, z, dy=dy, dlast_state=dlast, initial_state=h0, workspace=ws)
        t.cuda.synchronize()
        out.append({k: v.clone() for k, v in g.items()})
    for k in out[0]:
        assert t.equal(out[0][k], out[1][k]), k
        assert bool(t.isfinite(out[1][k]).all()), k
