"""Sharpness of the oracle pins: plant one plausible mistake at a time in a copy of the
oracle's C source (on the CPU, in a temporary directory), build it, and check that the pin
battery below rejects every mutant while accepting the unmodified oracle.

The battery uses only references the pages or the mathematics fix: the printed worked ZOH
and first-order examples, the printed softplus values, the halving closed form, a
brute-force unrolled sum (also fed step sizes transformed with numpy's logaddexp), the
causal-convolution form for fixed coefficients, scipy's logistic function for the gate, and
the integrator closed form for a zero continuous rate.
"""
import math
import os
import subprocess
import tempfile

import numpy as np
import pytest
import scipy.special

import oracle
from tests.conftest import read_golden
from tests.test_oracle_pins import brute_force, rel_err

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssm_oracle.c")

# the forward's decay line (the backward has a line of the same text)
FWD_ABAR = "const double abar = exp(dt * a);\n      const double bbar"

MUTANTS = {
    "first_order_input_coeff": ("return expm1(dt * a) / a;", "return dt;"),
    "readout_before_update": (
        "      h[n] = abar * h[n] + bbar * uu;\n      acc += (double)Crow[n] * h[n];",
        "      acc += (double)Crow[n] * h[n];\n      h[n] = abar * h[n] + bbar * uu;"),
    "dropped_feedthrough": ("if (j->Dskip) yv += (double)j->Dskip[d] * uu;", ";"),
    "sigmoid_instead_of_silu": ("yv *= zz / (1.0 + exp(-zz));", "yv *= 1.0 / (1.0 + exp(-zz));"),
    "wrong_sign_decay": (FWD_ABAR, FWD_ABAR.replace("exp(dt * a)", "exp(-dt * a)")),
    "b_and_c_swapped": ("const double bbar = (j->euler ? dt : zoh_input_coeff(dt, a)) * (double)Brow[n];",
                        "const double bbar = (j->euler ? dt : zoh_input_coeff(dt, a)) * (double)Crow[n];"),
    "a_transposed": ("const double a = (double)j->A[d * N + n];", "const double a = (double)j->A[n * D + d];"),
    "zero_rate_fallback_dropped": ("if (a == 0.0) return dt;", "if (a == 0.0) return 0.0;"),
    "feedthrough_after_gate": (
        "    if (j->Dskip) yv += (double)j->Dskip[d] * uu;\n    if (j->z) {\n      const double zz = (double)j->z[tok];\n      yv *= zz / (1.0 + exp(-zz));\n    }",
        "    if (j->z) {\n      const double zz = (double)j->z[tok];\n      yv *= zz / (1.0 + exp(-zz));\n    }\n    if (j->Dskip) yv += (double)j->Dskip[d] * uu;"),
    "euler_decay": (FWD_ABAR, FWD_ABAR.replace("exp(dt * a)", "1.0 + dt * a")),
    "ti_b_layout_transposed": ("const float* Brow = j->time_invariant ? j->B + d * N : j->B + (b * L + l) * N;",
                               "const float* Brow = j->time_invariant ? j->B + d : j->B + (b * L + l) * N;"),
    "state_not_reset": ("h[n] = j->h0 ? (double)j->h0[(b * D + d) * N + n] : 0.0;",
                        "h[n] = j->h0 ? (double)j->h0[(b * D + d) * N + n] : 1e-3;"),
    "initial_state_ignored": ("h[n] = j->h0 ? (double)j->h0[(b * D + d) * N + n] : 0.0;", "h[n] = 0.0;"),
    "initial_state_wrong_index": ("h[n] = j->h0 ? (double)j->h0[(b * D + d) * N + n] : 0.0;",
                                  "h[n] = j->h0 ? (double)j->h0[(d * j->batch + b) * N + n] : 0.0;"),
    "euler_flag_ignored": ("(j->euler ? dt : zoh_input_coeff(dt, a))", "zoh_input_coeff(dt, a)"),
    "euler_also_linearises_decay": (FWD_ABAR, FWD_ABAR.replace("exp(dt * a)", "j->euler ? 1.0 + dt * a : exp(dt * a)")),
    "softplus_not_applied": ("return j->delta_softplus ? softplus(x) : x;", "return x;"),
    "softplus_wrong_branch": ("log1p(exp(-fabs(x))) + fmax(x, 0.0)", "log1p(exp(-fabs(x))) + fmax(-x, 0.0)"),
    "bias_not_per_channel": ("if (j->delta_bias) x += (double)j->delta_bias[d];",
                             "if (j->delta_bias) x += (double)j->delta_bias[0];"),
    "bias_after_softplus": ("  double x = raw;\n  if (j->delta_bias) x += (double)j->delta_bias[d];\n  return j->delta_softplus ? softplus(x) : x;",
                            "  double x = j->delta_softplus ? softplus(raw) : raw;\n  if (j->delta_bias) x += (double)j->delta_bias[d];\n  return x;"),
}


def _build(text, tmpdir, name):
    c = os.path.join(tmpdir, name + ".c")
    so = os.path.join(tmpdir, name + ".so")
    with open(c, "w") as f:
        f.write(text)
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-o", so, c, "-lm", "-lpthread"])
    return oracle.OracleLib(so)


def pin_battery(lib):
    """Returns the list of failed pin names (empty = all pins hold)."""
    failed = []
    g = read_golden("zoh_scalar_example.txt")
    # printed worked example through the recurrence
    u = np.array([[[g["x"]], [0.0]]], np.float32)
    y, last = lib.fwd(u, np.full((1, 2, 1), g["delta"], np.float32), np.array([[g["a"]]], np.float32),
                      np.full((1, 2, 1), g["b"], np.float32), np.ones((1, 2, 1), np.float32))
    if abs(y[0, 0, 0] - g["h1_zoh"]) > 1e-15 or abs(y[0, 1, 0] - g["abar"] * g["h1_zoh"]) > 1e-15:
        failed.append("worked_example")
    # halving closed form
    L = 20
    dt32 = np.float32(math.log(2.0))
    ui = np.zeros((1, L, 1), np.float32)
    ui[0, 0, 0] = 1.0
    y, _ = lib.fwd(ui, np.full((1, L, 1), dt32, np.float32), -np.ones((1, 1), np.float32),
                   np.ones((1, L, 1), np.float32), np.ones((1, L, 1), np.float32))
    if np.max(np.abs(y[0, :, 0] - 0.5 ** (np.arange(L) + 1))) > 1e-7:
        failed.append("halving")
    # brute force, random selective inputs with feed-through, gate and a zero rate
    rng = np.random.default_rng(1234)
    b, L, D, N = 2, 8, 3, 4
    args = (rng.standard_normal((b, L, D)).astype(np.float32),
            np.exp(rng.uniform(np.log(1e-2), 0.0, (b, L, D))).astype(np.float32),
            (-rng.uniform(0.2, 3.0, (D, N))).astype(np.float32),
            rng.standard_normal((b, L, N)).astype(np.float32),
            rng.standard_normal((b, L, N)).astype(np.float32),
            rng.standard_normal(D).astype(np.float32),
            rng.standard_normal((b, L, D)).astype(np.float32))
    args[2][1, 2] = 0.0
    y, last = lib.fwd(*args)
    yb, lb = brute_force(*args)
    if rel_err(y, yb) > 1e-12 or rel_err(last, lb) > 1e-12:
        failed.append("brute_force")
    # gate is SiLU
    yu, _ = lib.fwd(*args[:6])
    z64 = args[6].astype(np.float64)
    if np.max(np.abs(y - yu * z64 * scipy.special.expit(z64))) > 1e-12:
        failed.append("gate")
    # convolution identity for fixed coefficients
    D2, N2 = 3, 5
    u2 = rng.standard_normal((2, 64, D2)).astype(np.float32)
    dl = np.exp(rng.uniform(np.log(1e-2), 0.0, D2)).astype(np.float32)
    A2 = (-rng.uniform(0.2, 2.0, (D2, N2))).astype(np.float32)
    B2 = rng.standard_normal((D2, N2)).astype(np.float32)
    C2 = rng.standard_normal((D2, N2)).astype(np.float32)
    Ds2 = rng.standard_normal(D2).astype(np.float32)
    y, _ = lib.fwd(u2, dl, A2, B2, C2, Ds2, time_invariant=True)
    if rel_err(y, oracle.conv_ti_direct(u2, dl, A2, B2, C2, Ds2)) > 1e-12:
        failed.append("convolution")
    # zero continuous rate integrates delta * B * u
    u3 = rng.standard_normal((1, 10, 1)).astype(np.float32)
    d3 = rng.uniform(0.01, 0.5, (1, 10, 1)).astype(np.float32)
    B3 = rng.standard_normal((1, 10, 2)).astype(np.float32)
    C3 = rng.standard_normal((1, 10, 2)).astype(np.float32)
    y, _ = lib.fwd(u3, d3, np.zeros((1, 2), np.float32), B3, C3)
    h = np.cumsum(d3[0].astype(np.float64) * B3[0] * u3[0], axis=0)
    if np.max(np.abs(y[0, :, 0] - np.sum(C3[0] * h, axis=1))) > 1e-12:
        failed.append("zero_rate")
    # initial state against the brute-force unroll
    h0 = rng.standard_normal((b, D, N)).astype(np.float32)
    y, last = lib.fwd(*args, h0=h0)
    yb, lb = brute_force(*args, h0=h0)
    if rel_err(y, yb) > 1e-12 or rel_err(last, lb) > 1e-12:
        failed.append("initial_state")
    # printed first-order example through the recurrence
    y, _ = lib.fwd(u, np.full((1, 2, 1), g["delta"], np.float32), np.array([[g["a"]]], np.float32),
                   np.full((1, 2, 1), g["b"], np.float32), np.ones((1, 2, 1), np.float32), euler=True)
    if y[0, 0, 0] != g["h1_first_order"] or abs(y[0, 1, 0] - g["abar"] * g["h1_first_order"]) > 1e-15:
        failed.append("first_order_example")
    # printed softplus values
    sp = read_golden("softplus_values.txt")
    if abs(lib.softplus(0.0) - sp["softplus_0"]) > 1e-16 or abs(lib.softplus(1.0) - sp["softplus_1"]) > 1e-15:
        failed.append("softplus_values")
    # bias per channel, then softplus, against the brute force fed logaddexp(0, raw + bias)
    raw = rng.normal(-1.0, 1.5, args[0].shape).astype(np.float32)
    bias = rng.normal(0.0, 1.0, D).astype(np.float32)
    y, last = lib.fwd(args[0], raw, *args[2:], delta_bias=bias, delta_softplus=True)
    dt = np.logaddexp(0.0, raw.astype(np.float64) + bias.astype(np.float64)[None, None, :])
    yb, lb = brute_force(args[0], dt, *args[2:])
    if rel_err(y, yb) > 1e-12 or rel_err(last, lb) > 1e-12:
        failed.append("fused_softplus")
    return failed


@pytest.fixture(scope="module")
def tmpdir_mod():
    with tempfile.TemporaryDirectory() as d:
        yield d


def test_unmodified_oracle_passes_battery(tmpdir_mod):
    with open(SRC) as f:
        text = f.read()
    assert pin_battery(_build(text, tmpdir_mod, "unmodified")) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmpdir_mod):
    with open(SRC) as f:
        text = f.read()
    old, new = MUTANTS[name]
    assert text.count(old) == 1, "mutation site not found exactly once: %s" % name
    failed = pin_battery(_build(text.replace(old, new), tmpdir_mod, name))
    assert failed, "mutant %s passed every pin" % name
