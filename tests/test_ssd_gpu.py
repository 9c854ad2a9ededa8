"""GPU parity of the scalar-decay (Mamba-2) layer, selective_scan_ssd_fwd, against the oracle
(the fp64 recurrence with one decay per head, itself pinned to the pairwise masked form of
"state-space models", section "Mamba-2 and state-space duality").  Operands are bf16 and the
chunk products run on bf16 matrix cores with fp32 accumulation, so the bar is the bf16 one:
max|y - y_ref| / max|y_ref| <= 2e-2, and the same for the final state.  Cases: several 64-token
chunks with a ragged last one, one chunk, a single token, both state sizes, both input
coefficients, with and without gate and feed-through, an initial state, and the on-chip walk
over sequence segments (forced segment counts, ragged segments, both workgroup widths)."""
import numpy as np
import pytest

import oracle
import s6_workloads
from tests.gpu_common import TOL, log_errors, rel_err

pytestmark = pytest.mark.gpu


def torch():
    import torch as t
    return t


def make(rng, b, L, H, N, gate=True, dskip=True):
    bf = s6_workloads.bf16_round
    x = bf(rng.standard_normal((b, L, H, 64)).astype(np.float32))
    dl = bf(np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), (b, L, H))).astype(np.float32))
    A = (-np.exp(rng.uniform(np.log(1.0), np.log(16.0), H))).astype(np.float32)
    B = bf(rng.standard_normal((b, L, N)).astype(np.float32))
    C = bf(rng.standard_normal((b, L, N)).astype(np.float32))
    Ds = rng.standard_normal(H * 64).astype(np.float32) if dskip else None
    z = bf(rng.standard_normal((b, L, H, 64)).astype(np.float32)) if gate else None
    return x, dl, A, B, C, Ds, z


def run_gpu(inp, h0=None, euler=False, path="auto", segments=0):
    import selective_state_space_s6_amd as ss
    t = torch()
    x, dl, A, B, C, Ds, z = inp
    g = lambda a: None if a is None else t.from_numpy(a).cuda().to(t.bfloat16)
    y, last = ss.selective_scan_ssd_fwd(g(x), g(dl), t.from_numpy(A).cuda(), g(B), g(C),
                                        None if Ds is None else t.from_numpy(Ds).cuda(), g(z),
                                        initial_state=None if h0 is None else t.from_numpy(h0).cuda(),
                                        return_last_state=True, discretization="euler" if euler else "zoh",
                                        path=path, segments=segments)
    t.cuda.synchronize()
    return y.float().cpu().numpy(), last.cpu().numpy()


def run(inp, h0=None, euler=False, path="auto", segments=0):
    y, last = run_gpu(inp, h0=h0, euler=euler, path=path, segments=segments)
    x, dl, A, B, C, Ds, z = inp
    y_ref, l_ref = oracle.ssd_fwd(x, dl, A, B, C, Ds, z, h0=h0, euler=euler)
    return rel_err(y, y_ref), rel_err(last, l_ref)


@pytest.mark.parametrize("path", ["fused", "chunked"])
@pytest.mark.parametrize("euler", [False, True])
@pytest.mark.parametrize("N", [64, 128])
@pytest.mark.parametrize("L", [1, 64, 200])
def test_ssd_parity(L, N, euler, path):
    rng = np.random.default_rng(L + N + euler)
    e_y, e_l = run(make(rng, 2, L, 3, N), euler=euler, path=path)
    log_errors("ssd/%s L=%d N=%d euler=%s" % (path, L, N, euler), y=e_y, last_state=e_l, io="bf16")
    assert e_y <= TOL["bf16"] and e_l <= TOL["bf16"], (e_y, e_l)


@pytest.mark.parametrize("path", ["fused", "chunked"])
def test_ssd_without_gate_or_feedthrough(path):
    rng = np.random.default_rng(7)
    e_y, e_l = run(make(rng, 1, 150, 2, 64, gate=False, dskip=False), path=path)
    assert e_y <= TOL["bf16"] and e_l <= TOL["bf16"], (e_y, e_l)


@pytest.mark.parametrize("path", ["fused", "chunked"])
def test_ssd_initial_state(path):
    rng = np.random.default_rng(8)
    inp = make(rng, 2, 130, 2, 128)
    h0 = rng.standard_normal((2, 2, 64, 128)).astype(np.float32)
    e_y, e_l = run(inp, h0=h0, path=path)
    assert e_y <= TOL["bf16"] and e_l <= TOL["bf16"], (e_y, e_l)


@pytest.mark.parametrize("path", ["auto", "fused", "chunked"])
def test_ssd_many_heads_long(path):
    """A longer sequence (33 chunks) over 8 heads: the carried state crosses many chunks."""
    rng = np.random.default_rng(9)
    e_y, e_l = run(make(rng, 1, 2100, 8, 128), path=path)
    assert e_y <= TOL["bf16"] and e_l <= TOL["bf16"], (e_y, e_l)


@pytest.mark.parametrize("segments", [2, 3, 5, 100])
@pytest.mark.parametrize("N", [64, 128])
@pytest.mark.parametrize("L", [200, 1000])
def test_ssd_segmented_parity(L, N, segments):
    """On chip over sequence segments: segment end states from zero, composed across segments,
    then each segment walked from its carried-in state.  Ragged last chunks and segments, a
    segment count above the chunk count (one chunk per segment), an initial state."""
    rng = np.random.default_rng(L + N + segments)
    h0 = rng.standard_normal((2, 3, 64, N)).astype(np.float32) if segments % 2 else None
    e_y, e_l = run(make(rng, 2, L, 3, N), h0=h0, path="segmented", segments=segments)
    log_errors("ssd/segmented L=%d N=%d segments=%d" % (L, N, segments), y=e_y, last_state=e_l, io="bf16")
    assert e_y <= TOL["bf16"] and e_l <= TOL["bf16"], (e_y, e_l)


@pytest.mark.parametrize("euler", [False, True])
def test_ssd_segmented_four_wavefront_workgroups(euler):
    """More than 256 (batch, segment, head) workgroups: the four-wavefront output pass.  The
    oracle runs on three of the heads (heads are independent given B and C)."""
    rng = np.random.default_rng(11 + euler)
    x, dl, A, B, C, Ds, z = make(rng, 2, 700, 66, 64)
    h0 = rng.standard_normal((2, 66, 64, 64)).astype(np.float32)
    y, last = run_gpu((x, dl, A, B, C, Ds, z), h0=h0, euler=euler, path="segmented", segments=3)
    hs = np.array([0, 31, 65])
    ch = (hs[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
    y_ref, l_ref = oracle.ssd_fwd(x[:, :, hs], dl[:, :, hs], A[hs], B, C, Ds[ch], z[:, :, hs], h0=h0[:, hs],
                                  euler=euler)
    e_y, e_l = rel_err(y[:, :, hs], y_ref), rel_err(last[:, hs], l_ref)
    log_errors("ssd/segmented/nw4 euler=%s" % euler, y=e_y, last_state=e_l, io="bf16")
    assert e_y <= TOL["bf16"] and e_l <= TOL["bf16"], (e_y, e_l)


def test_ssd_one_segment_is_the_on_chip_walk():
    """One segment is the on-chip path itself: the same kernel, bit for bit."""
    rng = np.random.default_rng(12)
    inp = make(rng, 2, 333, 3, 128)
    a = run_gpu(inp, path="fused")
    b = run_gpu(inp, path="segmented", segments=1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


_FULL_REF = {}


def _full_reference(name):
    """Workload inputs and the oracle's output on three of its heads (heads are independent
    given B and C), computed once per workload."""
    if name not in _FULL_REF:
        inp = s6_workloads.generate_ssd(name)
        H = inp.x.shape[2]
        hs = np.array([0, H // 2, H - 1])
        ch = (hs[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
        y_ref, l_ref = oracle.ssd_fwd(inp.x[:, :, hs], inp.delta[:, :, hs], inp.A[hs], inp.B, inp.C, inp.Dskip[ch],
                                      inp.z[:, :, hs])
        _FULL_REF[name] = (inp, hs, y_ref, l_ref)
    return _FULL_REF[name]


@pytest.mark.parametrize("path", ["auto", "fused", "segmented", "chunked"])
@pytest.mark.parametrize("name", sorted(s6_workloads.SSD_WORKLOADS))
def test_ssd_full_size_sampled_heads(name, path):
    """The benchmark's workloads at full size (the automatic path, which the benchmark times,
    and every forced one), checked against the oracle on three heads."""
    import selective_state_space_s6_amd as ss
    t = torch()
    inp, hs, y_ref, l_ref = _full_reference(name)
    g = lambda a: t.from_numpy(a).cuda().to(t.bfloat16)
    y, last = ss.selective_scan_ssd_fwd(g(inp.x), g(inp.delta), t.from_numpy(inp.A).cuda(), g(inp.B), g(inp.C),
                                        t.from_numpy(inp.Dskip).cuda(), g(inp.z), return_last_state=True, path=path)
    t.cuda.synchronize()
    e_y = rel_err(y[:, :, hs].float().cpu().numpy(), y_ref)
    e_l = rel_err(last[:, hs].cpu().numpy(), l_ref)
    log_errors("ssd/full/%s/%s" % (name, path), y=e_y, last_state=e_l, io="bf16")
    assert e_y <= TOL["bf16"] and e_l <= TOL["bf16"], (e_y, e_l)
