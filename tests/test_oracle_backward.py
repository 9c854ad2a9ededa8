"""Pins for the oracle's backward pass (the reverse-time recurrence over the cached states,
as the rustytorch commit log describes its hand-written VJP of the selective scan).

* Reverse-mode automatic differentiation (torch, float64, CPU) through a forward written
  here directly from the method's definition (per-token loop, vectorised over batch,
  channels and states): every gradient, every option, to rounding.
* Central finite differences of the pure-Python brute-force unroll (float64), on sampled
  elements of every gradient, well inside the pages' own bound (5e-3 + 5e-2 |fd|, the
  rustytorch commit log's finite-difference test).
* The zero-rate limit dA = sum lambda delta^2/2 * B u at A == 0, which the autograd forward
  cannot give (its A == 0 branch does not depend on A), by finite differences at A = +-eps.
* Linearity in the output gradient.
"""
import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import brute_force


def torch():
    import torch as t
    return t


def torch_forward(u, raw, A, B, C, Dskip, z, h0, bias, euler, softplus, ti):
    """The forward pass from its definition, in float64 torch ops (differentiable)."""
    t = torch()
    batch, L, D = u.shape
    N = A.shape[1]
    x = raw + (bias if bias is not None else 0.0)
    dt = t.logaddexp(t.zeros_like(x), x) if softplus else x          # softplus(x) = log(e^0 + e^x)
    h = h0.clone() if h0 is not None else t.zeros(batch, D, N, dtype=t.float64)
    A_safe = t.where(A == 0, t.ones_like(A), A)
    ys = []
    for l in range(L):
        d_l = dt if ti else dt[:, l, :]                               # [D] or [batch, D]
        dA_ = d_l[..., None] * A                                      # delta * a
        abar = t.exp(dA_)
        if euler:
            c = d_l[..., None].expand_as(dA_)
        else:
            c = t.where(A == 0, d_l[..., None].expand_as(dA_), t.expm1(d_l[..., None] * A_safe) / A_safe)
        Bl = B[None] if ti else B[:, l, None, :]
        Cl = C[None] if ti else C[:, l, None, :]
        h = abar * h + c * Bl * u[:, l, :, None]
        yl = (Cl * h).sum(-1)
        if Dskip is not None:
            yl = yl + Dskip * u[:, l, :]
        if z is not None:
            yl = yl * z[:, l, :] * t.sigmoid(z[:, l, :])
        ys.append(yl)
    return t.stack(ys, dim=1), h


def autograd_grads(inp, dy, dlast=None, h0=None, bias=None, euler=False, softplus=False, ti=False):
    t = torch()
    u, raw, A, B, C, Dskip, z = inp
    leaf = lambda a: None if a is None else t.tensor(np.asarray(a, np.float64), requires_grad=True)
    tu, traw, tA, tB, tC, tD, tz, th0, tbias = map(leaf, (u, raw, A, B, C, Dskip, z, h0, bias))
    y, hl = torch_forward(tu, traw, tA, tB, tC, tD, tz, th0, tbias, euler, softplus, ti)
    loss = (y * t.tensor(np.asarray(dy, np.float64))).sum()
    if dlast is not None:
        loss = loss + (hl * t.tensor(np.asarray(dlast, np.float64))).sum()
    loss.backward()
    g = {"du": tu.grad, "ddelta": traw.grad, "dA": tA.grad, "dB": tB.grad, "dC": tC.grad}
    if tD is not None:
        g["dDskip"] = tD.grad
    if tz is not None:
        g["dz"] = tz.grad
    if th0 is not None:
        g["dh0"] = th0.grad
    if tbias is not None:
        g["ddelta_bias"] = tbias.grad
    return {k: v.numpy() for k, v in g.items()}


def rand_case(rng, batch, L, D, N, ti=False, gate=True, dskip=True, softplus=False, zero_a=False):
    u = rng.standard_normal((batch, L, D)).astype(np.float32)
    dshape = (D,) if ti else (batch, L, D)
    if softplus:
        raw = rng.normal(-1.0, 1.5, dshape).astype(np.float32)
    else:
        raw = np.exp(rng.uniform(np.log(1e-2), 0.0, dshape)).astype(np.float32)
    A = (-rng.uniform(0.2, 3.0, (D, N))).astype(np.float32)
    if zero_a:
        A[0, 0] = 0.0
    bc = (D, N) if ti else (batch, L, N)
    B = rng.standard_normal(bc).astype(np.float32)
    C = rng.standard_normal(bc).astype(np.float32)
    Ds = rng.standard_normal(D).astype(np.float32) if dskip else None
    z = rng.standard_normal((batch, L, D)).astype(np.float32) if gate else None
    return u, raw, A, B, C, Ds, z


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


OPTS = [dict(), dict(euler=True), dict(softplus=True), dict(softplus=True, bias=True, euler=True),
        dict(h0=True, dlast=True), dict(ti=True), dict(ti=True, softplus=True, bias=True)]


@pytest.mark.parametrize("opt", OPTS, ids=lambda o: "-".join(sorted(o)) or "plain")
def test_backward_equals_autograd(opt):
    rng = np.random.default_rng(100 + len(opt))
    batch, L, D, N = 2, 7, 3, 4
    ti = opt.get("ti", False)
    inp = rand_case(rng, batch, L, D, N, ti=ti, softplus=opt.get("softplus", False))
    dy = rng.standard_normal((batch, L, D)).astype(np.float32)
    h0 = rng.standard_normal((batch, D, N)).astype(np.float32) if opt.get("h0") else None
    dlast = rng.standard_normal((batch, D, N)).astype(np.float32) if opt.get("dlast") else None
    bias = rng.normal(0.0, 0.5, D).astype(np.float32) if opt.get("bias") else None
    euler, sp = opt.get("euler", False), opt.get("softplus", False)
    g = oracle.bwd(*inp, dy=dy, dlast=dlast, h0=h0, delta_bias=bias, euler=euler, delta_softplus=sp,
                   time_invariant=ti)
    ref = autograd_grads(inp, dy, dlast=dlast, h0=h0, bias=bias, euler=euler, softplus=sp, ti=ti)
    assert set(ref) <= set(g)
    for k, v in ref.items():
        assert rel(g[k], v) < 1e-11, (k, rel(g[k], v))


def test_backward_without_gate_or_feedthrough():
    rng = np.random.default_rng(7)
    inp = rand_case(rng, 1, 9, 2, 5, gate=False, dskip=False)
    dy = rng.standard_normal((1, 9, 2)).astype(np.float32)
    g = oracle.bwd(*inp, dy=dy)
    ref = autograd_grads(inp, dy)
    for k, v in ref.items():
        assert rel(g[k], v) < 1e-11, k
    assert not g["dz"].any() and "dDskip" not in g


def fd_grad(fn, x, idx, eps):
    xp = x.astype(np.float64).copy()
    xm = x.astype(np.float64).copy()
    xp[idx] += eps
    xm[idx] -= eps
    return (fn(xp) - fn(xm)) / (2 * eps)


@pytest.mark.parametrize("euler", [False, True])
def test_backward_central_differences(euler):
    """At least 30 sampled gradient elements of every input against central differences of
    the brute-force unroll (float64), with a zero rate among the states."""
    rng = np.random.default_rng(17 + euler)
    batch, L, D, N = 2, 6, 3, 3
    u, delta, A, B, C, Ds, z = rand_case(rng, batch, L, D, N, zero_a=True)
    dy = rng.standard_normal((batch, L, D))
    g = oracle.bwd(u, delta, A, B, C, Ds, z, dy=dy, euler=euler)
    args = dict(u=u, delta=delta, A=A, B=B, C=C, Dskip=Ds, z=z)

    def loss_of(name):
        def f(x):
            a = dict(args)
            a[name] = x
            y, _ = brute_force(a["u"], a["delta"], a["A"], a["B"], a["C"], a["Dskip"], a["z"], euler=euler)
            return float(np.sum(y * dy))
        return f

    checked = 0
    for name, key in (("u", "du"), ("delta", "ddelta"), ("A", "dA"), ("B", "dB"), ("C", "dC"), ("Dskip", "dDskip"),
                      ("z", "dz")):
        x = args[name]
        flat = rng.choice(x.size, size=min(x.size, 6), replace=False)
        for f_i in flat:
            idx = np.unravel_index(f_i, x.shape)
            if name == "A" and x[idx] == 0.0:
                continue                                    # the limit is pinned below
            fd = fd_grad(loss_of(name), x, idx, 1e-6)
            assert abs(g[key][idx] - fd) <= 1e-6 * (1 + abs(fd)), (name, idx, g[key][idx], fd)
            assert abs(g[key][idx] - fd) <= 5e-3 + 5e-2 * abs(fd)          # the pages' own bound
            checked += 1
    assert checked >= 30


def test_zero_rate_limit_of_da():
    """dA at A == 0 is the limit delta^2/2 B u lambda: compare with central differences
    across a = 0 (the brute force uses delta * B exactly at 0 and expm1 elsewhere)."""
    rng = np.random.default_rng(23)
    u, delta, A, B, C, Ds, z = rand_case(rng, 1, 6, 2, 3)
    A[1, 2] = 0.0
    dy = rng.standard_normal((1, 6, 2))
    g = oracle.bwd(u, delta, A, B, C, Ds, z, dy=dy)

    def f(Ax):
        y, _ = brute_force(u, delta, Ax, B, C, Ds, z)
        return float(np.sum(y * dy))

    fd = fd_grad(f, A, (1, 2), 1e-5)
    assert abs(g["dA"][1, 2] - fd) <= 1e-7 * (1 + abs(fd))


def test_backward_linear_in_output_gradient():
    rng = np.random.default_rng(29)
    inp = rand_case(rng, 2, 8, 3, 4)
    d1 = rng.standard_normal((2, 8, 3)).astype(np.float32)
    d2 = rng.standard_normal((2, 8, 3)).astype(np.float32)
    g1 = oracle.bwd(*inp, dy=d1)
    g2 = oracle.bwd(*inp, dy=d2)
    g12 = oracle.bwd(*inp, dy=(d1.astype(np.float64) + d2).astype(np.float32))
    for k in g1:
        assert rel(g12[k], g1[k] + g2[k]) < 1e-6, k
    g0 = oracle.bwd(*inp, dy=np.zeros_like(d1))
    assert all(not v.any() for v in g0.values())


# ---- sharpness: plausible mistakes planted in a copy of the backward fail the battery above

import os
import tempfile

from tests.test_oracle_mutants import SRC, _build

MUTANTS_BWD = {
    "state_after_step_in_delta_term": ("const double hp = hs[l * N + n], bn", "const double hp = hs[(l + 1) * N + n], bn"),
    "adjoint_not_decayed": ("lam[n] = abar * ln;", "lam[n] = ln;"),
    "coefficient_term_of_ddelta_dropped": ("g_dt += ln * (a * abar * hp + dc_ddt * bn * uu);",
                                           "g_dt += ln * (a * abar * hp);"),
    "silu_derivative_wrong": ("dz[tok] = dyp * yp * sg * (1.0 + zz * (1.0 - sg));", "dz[tok] = dyp * yp * sg;"),
    "gate_not_applied_to_adjoint": ("dyp *= zz * sg;", ";"),
    "da_coefficient_term_dropped": ("dA[d * N + n] += ln * (dt * abar * hp + dc_da * bn * uu);",
                                    "dA[d * N + n] += ln * (dt * abar * hp);"),
    "db_without_input": ("dBrow[n] += ln * c * uu;", "dBrow[n] += ln * c;"),
    "dc_uses_previous_state": ("dCrow[n] += dyp * hs[(l + 1) * N + n];", "dCrow[n] += dyp * hs[l * N + n];"),
    "softplus_chain_dropped": ("g_dt * (delta_softplus ? sigmoid(", "g_dt * (0 ? sigmoid("),
    "dlast_ignored": ("lam[n] = dlast ? (double)dlast[(b * D + d) * N + n] : 0.0;", "lam[n] = 0.0;"),
    "zero_rate_da_limit_wrong": ("(a == 0.0 ? 0.5 * dt * dt : zoh_coeff_da(dt, a))", "(a == 0.0 ? 0.0 : zoh_coeff_da(dt, a))"),
    "euler_uses_zoh_derivative": ("const double dc_ddt = euler ? 1.0 : abar;", "const double dc_ddt = abar;"),
}


def bwd_battery(lib):
    failed = []
    rng = np.random.default_rng(31)
    for i, opt in enumerate([dict(), dict(euler=True), dict(softplus=True, bias=True), dict(h0=True, dlast=True)]):
        inp = rand_case(rng, 2, 6, 3, 4, softplus=opt.get("softplus", False))
        dy = rng.standard_normal((2, 6, 3)).astype(np.float32)
        h0 = rng.standard_normal((2, 3, 4)).astype(np.float32) if opt.get("h0") else None
        dlast = rng.standard_normal((2, 3, 4)).astype(np.float32) if opt.get("dlast") else None
        bias = rng.normal(0.0, 0.5, 3).astype(np.float32) if opt.get("bias") else None
        kw = dict(dlast=dlast, h0=h0, bias=bias, euler=opt.get("euler", False), softplus=opt.get("softplus", False))
        g = lib.bwd(*inp, dy=dy, dlast=dlast, h0=h0, delta_bias=bias, euler=kw["euler"], delta_softplus=kw["softplus"])
        ref = autograd_grads(inp, dy, **kw)
        if any(rel(g[k], v) > 1e-11 for k, v in ref.items()):
            failed.append("autograd%d" % i)
    # the zero-rate limit
    u, delta, A, B, C, Ds, z = rand_case(rng, 1, 6, 2, 3)
    A[1, 2] = 0.0
    dy = rng.standard_normal((1, 6, 2))
    g = lib.bwd(u, delta, A, B, C, Ds, z, dy=dy)
    fd = fd_grad(lambda Ax: float(np.sum(brute_force(u, delta, Ax, B, C, Ds, z)[0] * dy)), A, (1, 2), 1e-5)
    if abs(g["dA"][1, 2] - fd) > 1e-7 * (1 + abs(fd)):
        failed.append("zero_rate")
    return failed


@pytest.fixture(scope="module")
def tmpdir_bwd():
    with tempfile.TemporaryDirectory() as d:
        yield d


def test_unmodified_backward_passes_battery(tmpdir_bwd):
    with open(SRC) as f:
        assert bwd_battery(_build(f.read(), tmpdir_bwd, "unmodified_bwd")) == []


@pytest.mark.parametrize("name", sorted(MUTANTS_BWD))
def test_backward_mutant_is_caught(name, tmpdir_bwd):
    with open(SRC) as f:
        text = f.read()
    old, new = MUTANTS_BWD[name]
    assert text.count(old) == 1, "mutation site not found exactly once: %s" % name
    assert bwd_battery(_build(text.replace(old, new), tmpdir_bwd, name)), "mutant %s passed every pin" % name
