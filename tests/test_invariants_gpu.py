"""GPU invariants the pages fix for the S6 block (the rustytorch commit log lists causality
and seeded determinism among its selective-scan tests): bitwise run-to-run determinism,
causality, batch independence; plus equality of the two entry points and stream use."""
import numpy as np
import pytest

import s6_workloads
from tests.gpu_common import TOL, rel_err, run_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,kw", [("small_f32", {}), ("longctx_bf16", dict(batch=2, L=600, D=80)),
                                     ("s4d_ti_f32", dict(batch=2, L=300, D=40))])
def test_deterministic(name, kw):
    inp = s6_workloads.generate(name, **kw)
    for path in ("single", "chunked"):
        y1, l1 = run_gpu(inp, path=path)
        y2, l2 = run_gpu(inp, path=path)
        assert np.array_equal(y1, y2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("path", ["single", "chunked"])
def test_causal(path):
    inp = s6_workloads.generate("mamba130m_f32", "active", batch=2, L=400, D=20)
    y0, _ = run_gpu(inp, path=path)
    for t0 in (0, 17, 255, 399):
        pert = s6_workloads.generate("mamba130m_f32", "active", batch=2, L=400, D=20)
        pert.u[:, t0, :] += 1.0
        y1, _ = run_gpu(pert, path=path)
        assert np.array_equal(y0[:, :t0], y1[:, :t0]), t0
        assert not np.array_equal(y0[:, t0], y1[:, t0])


def test_batch_rows_independent():
    inp = s6_workloads.generate("small_f32", batch=3, L=200, D=36)
    y, last = run_gpu(inp, path="single")
    for b in range(3):
        one = s6_workloads.generate("small_f32", batch=3, L=200, D=36)
        for f in ("u", "delta", "B", "C", "z"):
            setattr(one, f, np.ascontiguousarray(getattr(one, f)[b:b + 1]))
        yb, lb = run_gpu(one, path="single")
        assert np.array_equal(yb[0], y[b]) and np.array_equal(lb[0], last[b])


def test_single_and_chunked_agree():
    inp = s6_workloads.generate("small_f32", "active")
    ys, ls = run_gpu(inp, path="single")
    yc, lc = run_gpu(inp, path="chunked")
    assert rel_err(yc, ys) <= TOL["f32"] and rel_err(lc, ls) <= 1e-4


def test_workspace_entry_point_matches():
    inp = s6_workloads.generate("small_f32")
    for path in ("auto", "chunked", "single"):
        y1, l1 = run_gpu(inp, path=path)
        y2, l2 = run_gpu(inp, path=path, workspace=True)
        assert np.array_equal(y1, y2) and np.array_equal(l1, l2)


def test_side_stream():
    import torch
    inp = s6_workloads.generate("small_f32", L=256)
    y1, _ = run_gpu(inp)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y2, _ = run_gpu(inp, stream=s)
    assert np.array_equal(y1, y2)


def test_library_allocated_workspace_on_raw_stream():
    """The C entry point that allocates its own (stream-ordered) workspace: reached from the
    binding with a raw stream handle that is not torch's current stream."""
    import torch
    inp = s6_workloads.generate("small_f32")
    y1, l1 = run_gpu(inp, path="chunked")
    s = torch.cuda.Stream()
    y2, l2 = run_gpu(inp, path="chunked", stream=s.cuda_stream)
    torch.cuda.synchronize()
    assert np.array_equal(y1, y2) and np.array_equal(l1, l2)
