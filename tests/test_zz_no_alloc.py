"""selective_scan_fwd_noalloc, the forward for callers that cannot allocate, against
selective_scan_fwd_ex given a workspace (the entry point it is a variant of): the same kernels
and plan, so the outputs must agree bit for bit, and both within the parity bar of the oracle.
Two calls in a row share the library's per-GPU scratch, the second on a smaller input, so
that the second call runs over what the first left there."""
import numpy as np
import pytest

import oracle
import s6_workloads
from tests.gpu_common import TOL, TOL_STATE, dev, rel_err

pytestmark = pytest.mark.gpu


def torch():
    import torch as t
    return t


def both(inp, *, path="auto", chunk_len=0, h0=None, bias=None):
    """(y, last) from the no-allocation entry point and from selective_scan_fwd_ex with a
    workspace, on the same inputs."""
    import selective_state_space_s6_amd as ss
    t = torch()
    io = inp.io
    u, dl, B, C, z = (dev(x, io) for x in (inp.u, inp.delta, inp.B, inp.C, inp.z))
    A = t.from_numpy(inp.A).cuda()
    Ds = None if inp.Dskip is None else t.from_numpy(inp.Dskip).cuda()
    h0_t = None if h0 is None else t.from_numpy(h0).cuda()
    bias_t = None if bias is None else t.from_numpy(bias).cuda()
    b, L, D, N = inp.shape
    opts = dict(initial_state=h0_t, delta_bias=bias_t, delta_softplus=bias is not None, path=path,
                chunk_len=chunk_len)
    y1, l1 = t.empty_like(u), t.empty((b, D, N), dtype=t.float32, device="cuda")
    ss.selective_scan_fwd_noalloc(u, dl, A, B, C, Ds, z, y=y1, last_state=l1, **opts)
    need = ss.workspace_size(ss.make_dims(u, dl, A, B, C, z, u, path=path, chunk_len=chunk_len,
                                          delta_softplus=bias is not None))
    ws = t.empty(max(need, 256), dtype=t.uint8, device="cuda")
    y2, l2 = ss.selective_scan_fwd(u, dl, A, B, C, Ds, z, return_last_state=True, workspace=ws, **opts)
    t.cuda.synchronize()
    return (y1, l1), (y2, l2), need


def check(inp, got, ref, h0=None, bias=None):
    t = torch()
    (y1, l1), (y2, l2) = got, ref
    assert t.equal(y1, y2) and t.equal(l1, l2)
    y_ref, l_ref = oracle.fwd(inp.u, inp.delta, inp.A, inp.B, inp.C, inp.Dskip, inp.z, h0=h0, delta_bias=bias,
                              delta_softplus=bias is not None, time_invariant=inp.ti)
    assert rel_err(y1.float().cpu().numpy(), y_ref) <= TOL[inp.io]
    assert rel_err(l1.cpu().numpy(), l_ref) <= TOL_STATE


@pytest.mark.parametrize("name", ["small_f32", "longctx_bf16", "s4d_ti_f32"])
def test_noalloc_two_calls_second_smaller(name):
    first = s6_workloads.generate(name, batch=2, L=1100, D=96)
    second = s6_workloads.generate(name, batch=1, L=333, D=40, seed=77)
    for inp, chunk_len in ((first, 0), (second, 64)):
        y1, y2, need = both(inp, path="chunked", chunk_len=chunk_len)
        assert need > 0                      # the chunked path ran through the scratch
        check(inp, y1, y2)


def test_noalloc_initial_state_and_step_size():
    import dataclasses
    inp = s6_workloads.generate("mamba130m_f32", "active", batch=2, L=700, D=36)
    raw, bias = s6_workloads.raw_step_sizes(inp)
    inp = dataclasses.replace(inp, delta=raw)
    h0 = s6_workloads.running_state(inp, scale=1.0)
    for chunk_len in (112, 48):              # the second call: more, shorter chunks
        got, ref, need = both(inp, path="chunked", chunk_len=chunk_len, h0=h0, bias=bias)
        assert need > 0
        check(inp, got, ref, h0=h0, bias=bias)


def test_noalloc_automatic_paths():
    """The automatic path: chunked for the small workload (128 wavefronts), one pass for a
    well-filled one (no scratch touched), then chunked again."""
    for name, kw in (("small_f32", {}), ("mamba130m_f32", dict(batch=8, L=300, D=512)),
                     ("small_f32", dict(batch=1, L=600, D=64))):
        inp = s6_workloads.generate(name, **kw)
        got, ref, _ = both(inp)
        check(inp, got, ref)
