"""GPU parity where the zero-order-hold input coefficient (exp(delta a) - 1)/a cancels in
float32: rates a with |delta a| from 1e-6 down to 1e-10, and zero, at a constant step of 1e-3
("state-space models" (aarnphm.xyz), section "From continuous time to tokens"; Algenta
"Sequence and state-space models", ssm_discretize_b).  Formed as (exp(x) - 1)/a from a rounded
exp(x), the coefficient would lose every correct digit at |x| = 1e-7 and vanish below; the
oracle takes expm1.  Inputs (s6_workloads.small_rates) mix channel blocks whose rates are all
small, half small, and canonical, so that both forms of the coefficient run in one call.  No
feed-through and no gate: y is the scan's term alone.  Covered: the pipelined and per-element
kernels on the single and chunked paths, both element types, 16 and 64 states, the decode
step, the backward pass (unsplit and with sequence chunks) and the scalar-decay layer on both
of its paths.  Bar as everywhere: max|err| / max|ref| <= 1e-4 (fp32 I/O), 2e-2 (bf16 I/O)."""
import numpy as np
import pytest

import oracle
import s6_workloads
from tests.gpu_common import TOL, TOL_STATE, dev, log_errors, rel_err, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def torch():
    import torch as t
    return t


@pytest.mark.parametrize("scalar_io", [False, True])
@pytest.mark.parametrize("path", ["single", "chunked"])
@pytest.mark.parametrize("N", [16, 64])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_forward_small_rates(io, N, path, scalar_io):
    inp = s6_workloads.small_rates(2, 300, 192, N, io=io)
    y_ref, l_ref = run_oracle(inp)
    y, last = run_gpu(inp, path=path, scalar_io=scalar_io)
    e_y, e_l = rel_err(y, y_ref), rel_err(last, l_ref)
    case = "small_rates/%s/N=%d/%s/%s" % (io, N, path, scalar_io)
    log_errors(case, y=e_y, last_state=e_l, io=io)
    assert e_y <= TOL[io] and e_l <= TOL_STATE, (case, e_y, e_l)
    # the channels whose every rate is small, on their own: their scan must not vanish
    ch = np.arange(64)
    assert rel_err(y[..., ch], y_ref[..., ch]) <= TOL[io], case


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_steps_small_rates(io):
    """Twelve decode steps from a running state against the oracle's scan over the same
    twelve tokens from that state."""
    import selective_state_space_s6_amd as ss
    t = torch()
    inp = s6_workloads.small_rates(4, 12, 192, 16, io=io)
    b, L, D, N = inp.shape
    h0 = s6_workloads.running_state(inp, scale=1.0)
    y_ref, l_ref = oracle.fwd(inp.u, inp.delta, inp.A, inp.B, inp.C, None, None, h0=h0)
    state = t.from_numpy(h0).cuda()
    A = t.from_numpy(inp.A).cuda()
    g = {k: dev(getattr(inp, k), io) for k in ("u", "delta", "B", "C")}
    ys = []
    for l in range(L):
        ys.append(ss.selective_scan_step(g["u"][:, l].contiguous(), g["delta"][:, l].contiguous(), A,
                                         g["B"][:, l].contiguous(), g["C"][:, l].contiguous(), None, None,
                                         state=state))
    t.cuda.synchronize()
    y = t.stack(ys, dim=1).float().cpu().numpy()
    e_y, e_l = rel_err(y, y_ref), rel_err(state.cpu().numpy(), l_ref)
    log_errors("small_rates/step/%s" % io, y=e_y, last_state=e_l, io=io)
    assert e_y <= TOL[io] and e_l <= TOL_STATE, (e_y, e_l)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("batch,L", [(2, 100), (1, 1000)])   # the second splits the sequence into chunks
def test_backward_small_rates(io, batch, L):
    import selective_state_space_s6_amd as ss
    t = torch()
    inp = s6_workloads.small_rates(batch, L, 192, 16, io=io)
    dy = np.random.default_rng(L).standard_normal(inp.u.shape).astype(np.float32)
    if io == "bf16":
        dy = s6_workloads.bf16_round(dy)
    ref = oracle.bwd(inp.u, inp.delta, inp.A, inp.B, inp.C, None, None, dy=dy)
    g = ss.selective_scan_bwd(dev(inp.u, io), dev(inp.delta, io), t.from_numpy(inp.A).cuda(), dev(inp.B, io),
                              dev(inp.C, io), None, None, dy=dev(dy, io))
    t.cuda.synchronize()
    errs = {k: rel_err(v.float().cpu().numpy(), ref[k]) for k, v in g.items()}
    log_errors("small_rates/bwd/%s/%d/%d" % (io, batch, L), io=io, **errs)
    assert all(e <= TOL[io] for e in errs.values()), errs


@pytest.mark.parametrize("path", ["fused", "chunked"])
def test_ssd_small_rates(path):
    """The scalar-decay layer with per-head rates near zero at a constant step."""
    import selective_state_space_s6_amd as ss
    t = torch()
    rng = np.random.default_rng(41)
    bf = s6_workloads.bf16_round
    b, L, H, N = 2, 200, 8, 64
    x = bf(rng.standard_normal((b, L, H, 64)).astype(np.float32))
    dl = bf(np.full((b, L, H), 1e-3, np.float32))
    A = np.array([-1e-3, -1e-5, -1e-7, 0.0, -1.0, -2.0, -0.1, -4.0], np.float32)
    B = bf(rng.standard_normal((b, L, N)).astype(np.float32))
    C = bf(rng.standard_normal((b, L, N)).astype(np.float32))
    g = lambda a: t.from_numpy(a).cuda().to(t.bfloat16)
    y, last = ss.selective_scan_ssd_fwd(g(x), g(dl), t.from_numpy(A).cuda(), g(B), g(C), None, None,
                                        return_last_state=True, path=path)
    t.cuda.synchronize()
    y_ref, l_ref = oracle.ssd_fwd(x, dl, A, B, C, None, None)
    e_y, e_l = rel_err(y.float().cpu().numpy(), y_ref), rel_err(last.cpu().numpy(), l_ref)
    log_errors("small_rates/ssd/%s" % path, y=e_y, last_state=e_l, io="bf16")
    assert e_y <= TOL["bf16"] and e_l <= TOL["bf16"], (e_y, e_l)
    # the heads with small rates alone
    assert rel_err(y.float().cpu().numpy()[:, :, :4], y_ref[:, :, :4]) <= TOL["bf16"]
