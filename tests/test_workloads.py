"""Input generator checks (CPU): shapes, seeding, distributions, bf16 rounding."""
import numpy as np
import pytest
import torch

import s6_workloads as w


def test_softplus_printed_values(golden):
    g = golden("softplus_values.txt")
    v = w.softplus(np.array([0.0, 1.0]))
    assert v[0] == pytest.approx(g["softplus_0"], abs=1e-16)
    assert v[1] == pytest.approx(g["softplus_1"], abs=1e-15)
    # overflow-free for large arguments
    assert np.isfinite(w.softplus(np.array([1000.0, -1000.0]))).all()


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-6, 6, 200000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(w.bf16_round(x), ref)
    assert np.array_equal(w.bf16_bits(ref).astype(np.uint32) << 16, ref.view(np.uint32))


@pytest.mark.parametrize("name", sorted(w.WORKLOADS))
def test_reduced_shapes_and_determinism(name):
    a = w.generate(name, batch=1, L=32, D=8)
    b = w.generate(name, batch=1, L=32, D=8)
    s = w.spec(name)
    assert a.u.shape == (1, 32, 8) and a.A.shape == (8, s["N"])
    assert np.array_equal(a.u, b.u) and np.array_equal(a.delta, b.delta)
    if s["ti"]:
        assert a.delta.shape == (8,) and a.B.shape == (8, s["N"])
    else:
        assert a.delta.shape == (1, 32, 8) and a.B.shape == (1, 32, s["N"])
    assert (a.z is not None) == s["gate"]
    assert np.all(a.A < 0) and np.all(a.delta > 0)
    if s["io"] == "bf16":
        for t in (a.u, a.delta, a.B, a.C, a.z):
            assert np.array_equal(w.bf16_round(t), t)


def test_distributions_small_workload():
    x = w.generate("small_f32")
    assert x.delta.min() >= 1e-3 * (1 - 1e-6) and x.delta.max() <= 1e-1 * (1 + 1e-6)
    ld = np.log(x.delta)
    assert abs(ld.mean() - 0.5 * (np.log(1e-3) + np.log(1e-1))) < 0.02
    assert abs(x.u.std() - 1.0) < 0.01
    np.testing.assert_array_equal(x.A[5], -(np.arange(16) + 1.0))
    np.testing.assert_array_equal(x.Dskip, np.ones(256))


def test_longctx_delta_distribution():
    x = w.generate("longctx_bf16", batch=1, L=256, D=256)
    med = np.median(x.delta)
    assert 0.0085 < med < 0.0115
    xs = w.generate("s4d_ti_f32", batch=1, L=16, D=16)
    np.testing.assert_array_equal(xs.A[0], -(np.arange(64) + 1.0) / 2)


def test_variants():
    x = w.generate("small_f32", "scan_only", L=16)
    assert x.Dskip is None and x.z is None
    y = w.generate("small_f32", "active", L=16)
    assert y.delta.min() >= 0.1 * (1 - 1e-6) and y.delta.max() <= 1.0 + 1e-6
    c = w.generate("small_f32", "active_const", L=16)
    assert np.all(c.delta == np.float32(0.69))


def test_sample_channels():
    s = w.sample_channels(2560, 32)
    assert s[0] == 0 and s[-1] == 2559 and len(set(s.tolist())) == len(s) and len(s) >= 30
    assert np.array_equal(s, w.sample_channels(2560, 32))
