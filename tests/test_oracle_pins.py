"""Pins for the CPU oracle: each checks it against something the pages or the mathematics
fix, not against a re-typed copy of its own loop.

* the worked scalar ZOH example printed on the Algenta "Sequence and state-space models"
  page (tests/golden/zoh_scalar_example.txt);
* the closed form of the scalar example on the "state-space models" page (aarnphm.xyz,
  section "From continuous time to tokens"): A = -1, B = C = 1 gives
  h_t = e^-delta h_{t-1} + (1 - e^-delta) x_t, which halves at delta = log 2;
* the recurrence/convolution identity for fixed coefficients (same page, section "One
  recurrence, one convolution"), through an FFT and through an explicit double sum;
* the unrolled sum of the "Mamba-2 and state-space duality" section, generalised from a
  scalar decay a_k to a per-state decay Abar_k[n], evaluated by brute force on tiny inputs;
* the associative combine of the chipfoundry glossary's Lab 3 (sequential vs parallel scan);
* invariants: causality, linearity, batch independence, determinism, stability of Abar;
* the SiLU gate against scipy's logistic function;
* the first-order ("Euler") input coefficient: the worked value h_1 = 1.0 printed on the
  Algenta page beside the ZOH one, its geometric-series closed form, and the brute-force
  unroll with Bbar = delta * B;
* softplus of the step size: the two values printed on the Algenta page (mamba_delta_softplus),
  numpy's logaddexp(0, x) = log(e^0 + e^x), and the fused transform (per-channel bias, then
  softplus, as in TorchLean "Selective Mamba", step) against the brute-force unroll fed the
  transformed step sizes.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
import s6_workloads


def _rand_s6(rng, batch, L, D, N, gate=True, dskip=True, zero_a=False):
    u = rng.standard_normal((batch, L, D)).astype(np.float32)
    delta = np.exp(rng.uniform(np.log(1e-2), np.log(1.0), (batch, L, D))).astype(np.float32)
    A = (-rng.uniform(0.2, 3.0, (D, N))).astype(np.float32)
    if zero_a:
        A[0, 0] = 0.0
        A[-1, -1] = 0.0
    B = rng.standard_normal((batch, L, N)).astype(np.float32)
    C = rng.standard_normal((batch, L, N)).astype(np.float32)
    Ds = rng.standard_normal(D).astype(np.float32) if dskip else None
    z = rng.standard_normal((batch, L, D)).astype(np.float32) if gate else None
    return u, delta, A, B, C, Ds, z


def brute_force(u, delta, A, B, C, Dskip=None, z=None, h0=None, euler=False):
    """y_t = sum_n C_t[n] [(prod_{k=0..t} Abar_k[n]) h0[n] + sum_{s<=t} (prod_{k=s+1..t} Abar_k[n])
    Bbar_s[n] u_s] + D u_t, then the gate; and the final state h[n] = (prod_k Abar_k[n]) h0[n] +
    sum_s (prod_{k=s+1..L-1} Abar_k[n]) Bbar_s[n] u_s.  h0 (the initial state) defaults to zero.
    Bbar is the ZOH coefficient, or delta * B with euler=True.  delta may be given in float64 (a
    step size already transformed by the caller).
    Pure Python loops in float64 -- O(L^2 N) per channel, for tiny inputs only."""
    u = np.asarray(u, np.float64)
    delta = np.asarray(delta, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    batch, L, D = u.shape
    N = A.shape[1]
    y = np.zeros((batch, L, D))
    last = np.zeros((batch, D, N))

    def decay(abar, s, t, n):          # prod_{k=s+1..t} Abar_k[n]; the empty product is 1
        prod = 1.0
        for k in range(s + 1, t + 1):
            prod *= abar[k][n]
        return prod

    for b in range(batch):
        for d in range(D):
            abar, bbar = [], []
            for t in range(L):
                dt = delta[b, t, d]
                abar.append([math.exp(dt * A[d, n]) for n in range(N)])
                bbar.append([(dt if euler else math.expm1(dt * A[d, n]) / A[d, n] if A[d, n] != 0.0 else dt)
                             * B[b, t, n] for n in range(N)])
            for t in range(L):
                total = 0.0
                for n in range(N):
                    if h0 is not None:
                        total += C[b, t, n] * decay(abar, -1, t, n) * float(h0[b, d, n])
                    for s in range(t + 1):
                        total += C[b, t, n] * decay(abar, s, t, n) * bbar[s][n] * u[b, s, d]
                if Dskip is not None:
                    total += float(Dskip[d]) * u[b, t, d]
                if z is not None:
                    zz = float(z[b, t, d])
                    total *= zz * scipy.special.expit(zz)
                y[b, t, d] = total
            for n in range(N):
                last[b, d, n] = sum(decay(abar, s, L - 1, n) * bbar[s][n] * u[b, s, d] for s in range(L))
                if h0 is not None:
                    last[b, d, n] += decay(abar, -1, L - 1, n) * float(h0[b, d, n])
    return y, last


def rel_err(a, ref):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(ref))) / max(np.max(np.abs(ref)), 1e-300))


# ---------------------------------------------------------------------------------------------
# Printed worked example


def test_zoh_scalar_example_coefficients(golden):
    g = golden("zoh_scalar_example.txt")
    abar, bbar = oracle.discretize(g["a"], g["b"], g["delta"])
    assert abar == pytest.approx(g["abar"], abs=1e-15)
    assert bbar == pytest.approx(g["bbar_zoh"], abs=1e-15)
    # the first-order coefficient delta*b is a different method: the page's 1.0 must NOT match
    assert abs(bbar * g["x"] - g["h1_first_order"]) > 0.2


def test_zoh_scalar_example_through_recurrence(golden):
    g = golden("zoh_scalar_example.txt")
    # one channel, one state, two tokens: x then 0; C = 1 reads the state out directly
    u = np.array([[[g["x"]], [0.0]]], np.float32)
    delta = np.full((1, 2, 1), g["delta"], np.float32)
    A = np.array([[g["a"]]], np.float32)
    B = np.full((1, 2, 1), g["b"], np.float32)
    C = np.ones((1, 2, 1), np.float32)
    y, last = oracle.fwd(u, delta, A, B, C)
    assert y[0, 0, 0] == pytest.approx(g["h1_zoh"], abs=1e-15)          # readout of the updated state
    assert y[0, 1, 0] == pytest.approx(g["abar"] * g["h1_zoh"], abs=1e-15)
    assert last[0, 0, 0] == pytest.approx(g["abar"] * g["h1_zoh"], abs=1e-15)


def test_singular_a_uses_delta_b():
    # a == 0: the ZOH integral is delta (state integrates the input)
    abar, bbar = oracle.discretize(0.0, 2.0, 0.5)
    assert abar == 1.0 and bbar == 1.0
    # continuity: tiny |a| approaches the same value
    _, bbar_small = oracle.discretize(-1e-12, 2.0, 0.5)
    assert bbar_small == pytest.approx(1.0, rel=1e-9)


def test_abar_in_unit_interval_for_stable_a():
    rng = np.random.default_rng(3)
    for _ in range(200):
        a = -float(rng.uniform(1e-3, 50))
        dt = float(np.exp(rng.uniform(np.log(1e-4), np.log(2.0))))
        abar, bbar = oracle.discretize(a, 1.0, dt)
        assert 0.0 < abar < 1.0
        assert 0.0 < bbar <= dt  # (1 - e^{-|a|dt})/|a| is positive and below dt


# ---------------------------------------------------------------------------------------------
# Closed form of the scalar example


@pytest.mark.parametrize("L", [1, 7, 40])
def test_halving_closed_form(L):
    dt32 = np.float32(math.log(2.0))
    u_imp = np.zeros((1, L, 1), np.float32)
    u_imp[0, 0, 0] = 1.0
    u_step = np.ones((1, L, 1), np.float32)
    delta = np.full((1, L, 1), dt32, np.float32)
    A = -np.ones((1, 1), np.float32)
    B = np.ones((1, L, 1), np.float32)
    C = np.ones((1, L, 1), np.float32)
    y_imp, _ = oracle.fwd(u_imp, delta, A, B, C)
    y_step, _ = oracle.fwd(u_step, delta, A, B, C)
    t = np.arange(L)
    q = math.exp(-float(dt32))                 # exact decay for the fp32 step that was passed
    np.testing.assert_allclose(y_imp[0, :, 0], (1 - q) * q ** t, rtol=1e-13, atol=0)
    np.testing.assert_allclose(y_step[0, :, 0], 1 - q ** (t + 1), rtol=1e-13, atol=1e-16)
    # and the page's statement: each update keeps half and adds half
    np.testing.assert_allclose(y_imp[0, :, 0], 0.5 ** (t + 1), rtol=1e-7)
    np.testing.assert_allclose(y_step[0, :, 0], 1 - 0.5 ** (t + 1), rtol=1e-7)


def test_zero_a_integrates():
    rng = np.random.default_rng(11)
    L, N = 30, 3
    u = rng.standard_normal((1, L, 1)).astype(np.float32)
    delta = rng.uniform(0.01, 0.5, (1, L, 1)).astype(np.float32)
    A = np.zeros((1, N), np.float32)
    B = rng.standard_normal((1, L, N)).astype(np.float32)
    C = rng.standard_normal((1, L, N)).astype(np.float32)
    y, last = oracle.fwd(u, delta, A, B, C)
    h = np.cumsum(delta[0, :, 0:1].astype(np.float64) * B[0].astype(np.float64) * u[0, :, 0:1], axis=0)
    np.testing.assert_allclose(y[0, :, 0], np.sum(C[0] * h, axis=1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(last[0, 0], h[-1], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------------------------
# Recurrence == causal convolution for fixed coefficients


def test_kernel_element_printed_value(golden):
    g = golden("s4_kernel_element.txt")
    assert oracle.kernel_element(g["c"], g["abar_power"], g["b"]) == pytest.approx(g["kernel_element"], abs=1e-16)
    # Abar^2 = exp(2 * delta * a) composes exactly: delta = 0.5, a = -1
    K = oracle.ti_kernel(np.array([0.5]), np.array([[-1.0]]), np.array([[1.0]]), np.array([[1.0]]), 3)
    abar, bbar = oracle.discretize(-1.0, 1.0, 0.5)
    assert K[2, 0] == pytest.approx(abar * abar * bbar, rel=1e-15)
    assert K[2, 0] / bbar == pytest.approx(g["abar_power"], rel=1e-15)


@pytest.mark.parametrize("D,N", [(3, 5), (6, 2)])
def test_time_invariant_recurrence_equals_convolution(D, N):
    rng = np.random.default_rng(100 + D)
    batch, L = 2, 160
    u = rng.standard_normal((batch, L, D)).astype(np.float32)
    delta = np.exp(rng.uniform(np.log(1e-2), np.log(1.0), D)).astype(np.float32)
    A = (-(np.arange(N) + 1.0)[None, :] * rng.uniform(0.2, 1.0, (D, 1))).astype(np.float32)
    A[0, 0] = 0.0   # one singular state: Bbar = delta * B
    B = rng.standard_normal((D, N)).astype(np.float32)
    C = rng.standard_normal((D, N)).astype(np.float32)
    Ds = rng.standard_normal(D).astype(np.float32)
    y, _ = oracle.fwd(u, delta, A, B, C, Ds, time_invariant=True)
    assert rel_err(y, oracle.conv_ti_direct(u, delta, A, B, C, Ds)) < 1e-12
    assert rel_err(y, oracle.conv_ti(u, delta, A, B, C, Ds)) < 1e-12


def test_time_invariant_mode_equals_selective_mode_for_one_channel():
    rng = np.random.default_rng(7)
    batch, L, N = 2, 50, 4
    u = rng.standard_normal((batch, L, 1)).astype(np.float32)
    delta = np.array([0.3], np.float32)
    A = -rng.uniform(0.1, 2.0, (1, N)).astype(np.float32)
    B = rng.standard_normal((1, N)).astype(np.float32)
    C = rng.standard_normal((1, N)).astype(np.float32)
    y_ti, l_ti = oracle.fwd(u, delta, A, B, C, time_invariant=True)
    y_s6, l_s6 = oracle.fwd(u, np.full((batch, L, 1), 0.3, np.float32), A,
                            np.broadcast_to(B, (batch, L, N)).copy(), np.broadcast_to(C, (batch, L, N)).copy())
    assert np.array_equal(y_ti, y_s6) and np.array_equal(l_ti, l_s6)


# ---------------------------------------------------------------------------------------------
# Brute-force unrolled sum


@pytest.mark.parametrize("gate,dskip,zero_a", [(False, False, False), (True, True, False), (True, False, True)])
def test_brute_force_unroll_random(gate, dskip, zero_a):
    rng = np.random.default_rng(5 + gate + 2 * dskip + 4 * zero_a)
    inp = _rand_s6(rng, 2, 9, 3, 4, gate=gate, dskip=dskip, zero_a=zero_a)
    y, last = oracle.fwd(*inp)
    yb, lb = brute_force(*inp)
    assert rel_err(y, yb) < 1e-12
    assert rel_err(last, lb) < 1e-12


def test_brute_force_tiny_workload():
    x = s6_workloads.generate("tiny_f32")
    y, last = oracle.fwd(x.u, x.delta, x.A, x.B, x.C, x.Dskip, x.z)
    yb, lb = brute_force(x.u, x.delta, x.A, x.B, x.C, x.Dskip, x.z)
    assert rel_err(y, yb) < 1e-12
    assert rel_err(last, lb) < 1e-12
    xs = s6_workloads.generate("tiny_f32", "scan_only")
    y, _ = oracle.fwd(xs.u, xs.delta, xs.A, xs.B, xs.C)
    yb, _ = brute_force(xs.u, xs.delta, xs.A, xs.B, xs.C)
    assert rel_err(y, yb) < 1e-12


# ---------------------------------------------------------------------------------------------
# Associative combine: sequential == chunked composition (Lab 3)


def test_chunk_composition_of_final_state():
    rng = np.random.default_rng(21)
    u, delta, A, B, C, _, _ = _rand_s6(rng, 2, 60, 4, 6, gate=False, dskip=False)
    _, full = oracle.fwd(u, delta, A, B, C)
    h = np.zeros_like(full)
    for lo, hi in [(0, 17), (17, 18), (18, 45), (45, 60)]:
        _, part = oracle.fwd(u[:, lo:hi], delta[:, lo:hi], A, B[:, lo:hi], C[:, lo:hi])
        # chunk map (P, H): P = prod Abar = exp(a * sum delta), H = end state from zero
        P = np.exp(A[None].astype(np.float64) * delta[:, lo:hi].astype(np.float64).sum(axis=1)[:, :, None])
        h = P * h + part                                  # (P2 P1, P2 H1 + H2)
    assert np.max(np.abs(h - full)) < 1e-12


def test_lab3_sequential_vs_parallel_scan():
    rng = np.random.default_rng(2)
    seq, st = 30, 6
    abar = rng.uniform(0.5, 0.95, (seq, st))
    bx = rng.standard_normal((seq, st)) * 0.3
    # the oracle as the sequential scan: one channel per state, Abar = exp(delta*a) with delta=1,
    # a = log(abar), B = bx/Bbar-factor, u = 1
    a = np.log(abar).astype(np.float64)
    # run each state as its own channel with per-token decay: emulate through delta, fixed a = -1
    delta = (-a).astype(np.float32)                    # exp(-delta) = abar (to fp32 rounding)
    A = -np.ones((st, 1), np.float32)
    d64 = delta.astype(np.float64)
    coeff = -np.expm1(-d64)                            # (Abar - 1)/A with A = -1
    Bv = (bx / coeff).astype(np.float32)
    u = np.ones((1, seq, st), np.float32)
    # per-channel B differs, so run one state-channel at a time
    states = np.zeros((seq, st))
    for s in range(st):
        y, _ = oracle.fwd(u[:, :, s:s + 1], delta[None, :, s:s + 1], A[s:s + 1], Bv[None, :, s:s + 1],
                          np.ones((1, seq, 1), np.float32))
        states[:, s] = y[0, :, 0]
    # parallel scan by associative combine over the exact pairs the oracle used
    pa = np.exp(-d64)
    pb = coeff * Bv.astype(np.float64)
    acc_a, acc_b = pa[0].copy(), pb[0].copy()
    par = [acc_b.copy()]
    for t in range(1, seq):
        acc_a, acc_b = pa[t] * acc_a, pa[t] * acc_b + pb[t]
        par.append(acc_b.copy())
    assert np.max(np.abs(states - np.stack(par))) < 1e-8


# ---------------------------------------------------------------------------------------------
# Invariants


def test_causality_and_u_zero():
    rng = np.random.default_rng(31)
    u, delta, A, B, C, Ds, z = _rand_s6(rng, 1, 50, 3, 4)
    y0, _ = oracle.fwd(u, delta, A, B, C, Ds, z)
    for t0 in (0, 13, 49):
        u2 = u.copy()
        u2[:, t0, :] += 1.0
        y2, _ = oracle.fwd(u2, delta, A, B, C, Ds, z)
        assert np.array_equal(y0[:, :t0], y2[:, :t0])
        assert not np.array_equal(y0[:, t0], y2[:, t0])
    yz, lz = oracle.fwd(np.zeros_like(u), delta, A, B, C, Ds, z)
    assert not yz.any() and not lz.any()


def test_linear_in_u_without_gate_and_batch_independent():
    rng = np.random.default_rng(41)
    u, delta, A, B, C, Ds, _ = _rand_s6(rng, 3, 40, 2, 5, gate=False)
    u2 = rng.standard_normal(u.shape).astype(np.float32)
    y1, _ = oracle.fwd(u, delta, A, B, C, Ds)
    y2, _ = oracle.fwd(u2, delta, A, B, C, Ds)
    y12, _ = oracle.fwd(u.astype(np.float64) * 2 + u2, delta, A, B, C, Ds)
    # u*2 + u2 is exact in fp32 only approximately; compare with a loose bound
    assert rel_err(y12, 2 * y1 + y2) < 1e-6
    for b in range(3):
        yb, _ = oracle.fwd(u[b:b + 1], delta[b:b + 1], A, B[b:b + 1], C[b:b + 1], Ds)
        assert np.array_equal(yb[0], y1[b])


def test_small_delta_preserves_state():
    rng = np.random.default_rng(51)
    u, delta, A, B, C, _, _ = _rand_s6(rng, 1, 20, 2, 3, gate=False, dskip=False)
    _, l1 = oracle.fwd(u, delta, A, B, C)
    tail = np.full((1, 10, 2), 1e-9, np.float32)
    u2 = np.concatenate([u, rng.standard_normal((1, 10, 2)).astype(np.float32)], axis=1)
    d2 = np.concatenate([delta, tail], axis=1)
    B2 = np.concatenate([B, rng.standard_normal((1, 10, 3)).astype(np.float32)], axis=1)
    C2 = np.concatenate([C, rng.standard_normal((1, 10, 3)).astype(np.float32)], axis=1)
    _, l2 = oracle.fwd(u2, d2, A, B2, C2)
    np.testing.assert_allclose(l2, l1, rtol=1e-6, atol=1e-7)


def test_deterministic_across_thread_counts():
    rng = np.random.default_rng(61)
    inp = _rand_s6(rng, 3, 64, 17, 8)
    y1, l1 = oracle.fwd(*inp, nthreads=1)
    y8, l8 = oracle.fwd(*inp, nthreads=8)
    assert np.array_equal(y1, y8) and np.array_equal(l1, l8)


def test_gate_is_silu():
    rng = np.random.default_rng(71)
    u, delta, A, B, C, Ds, z = _rand_s6(rng, 2, 30, 3, 4)
    yg, lg = oracle.fwd(u, delta, A, B, C, Ds, z)
    yu, lu = oracle.fwd(u, delta, A, B, C, Ds, None)
    z64 = z.astype(np.float64)
    np.testing.assert_allclose(yg, yu * z64 * scipy.special.expit(z64), rtol=1e-13, atol=1e-15)
    assert np.array_equal(lg, lu)  # the gate never touches the state
    # SiLU(0) = 0
    yz, _ = oracle.fwd(u, delta, A, B, C, Ds, np.zeros_like(z))
    assert not yz.any()


def test_feedthrough_only_when_b_is_zero():
    rng = np.random.default_rng(81)
    u, delta, A, B, C, Ds, z = _rand_s6(rng, 2, 25, 3, 4)
    y, last = oracle.fwd(u, delta, A, np.zeros_like(B), C, Ds, z)
    u64, z64 = u.astype(np.float64), z.astype(np.float64)
    ref = Ds.astype(np.float64)[None, None] * u64 * z64 * scipy.special.expit(z64)
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-16)
    assert not last.any()


def test_empty_sequence_gives_zero_state():
    A = -np.ones((2, 3), np.float32)
    u = np.zeros((1, 0, 2), np.float32)
    y, last = oracle.fwd(u, np.zeros((1, 0, 2), np.float32), A, np.zeros((1, 0, 3), np.float32),
                         np.zeros((1, 0, 3), np.float32))
    assert y.shape == (1, 0, 2) and last.shape == (1, 2, 3) and not last.any()


# ---- initial state (continuation of a previous call; TorchLean "Selective Mamba", step /
# runArray with an explicit state; aarnphm "One recurrence, one convolution": the recurrent form)

def test_initial_state_zero_input_closed_form():
    """A = -1, B = C = 1, delta = ln 2, no input, h0 = 1: the state halves every step, so
    y_t = 2^-(t+1) exactly (the zero-input half of the aarnphm halving example)."""
    L = 24
    dt32 = np.float32(math.log(2.0))
    y, last = oracle.fwd(np.zeros((1, L, 1), np.float32), np.full((1, L, 1), dt32, np.float32),
                         -np.ones((1, 1), np.float32), np.ones((1, L, 1), np.float32),
                         np.ones((1, L, 1), np.float32), h0=np.ones((1, 1, 1), np.float32))
    # delta is the fp32 value nearest ln 2, so the exact decay per step is exp(-delta)
    e = math.exp(-float(dt32))
    np.testing.assert_allclose(y[0, :, 0], e ** (np.arange(L) + 1.0), rtol=1e-12, atol=0)
    np.testing.assert_allclose(y[0, :, 0], 0.5 ** (np.arange(L) + 1.0), rtol=1e-7, atol=0)
    assert abs(last[0, 0, 0] - e ** L) < 1e-12 * e ** L


def test_initial_state_brute_force():
    rng = np.random.default_rng(77)
    b, L, D, N = 3, 7, 4, 3
    u = rng.standard_normal((b, L, D)).astype(np.float32)
    dl = np.exp(rng.uniform(np.log(1e-2), 0.0, (b, L, D))).astype(np.float32)
    A = (-rng.uniform(0.2, 3.0, (D, N))).astype(np.float32)
    A[2, 1] = 0.0
    Bm = rng.standard_normal((b, L, N)).astype(np.float32)
    Cm = rng.standard_normal((b, L, N)).astype(np.float32)
    Ds = rng.standard_normal(D).astype(np.float32)
    z = rng.standard_normal((b, L, D)).astype(np.float32)
    h0 = rng.standard_normal((b, D, N)).astype(np.float32)
    y, last = oracle.fwd(u, dl, A, Bm, Cm, Ds, z, h0=h0)
    yb, lb = brute_force(u, dl, A, Bm, Cm, Ds, z, h0=h0)
    assert rel_err(y, yb) < 1e-12 and rel_err(last, lb) < 1e-12


def test_continuation_equals_concatenation():
    """Two calls with the state carried (rounded to fp32, as the GPU library hands it over)
    equal one call over the concatenated tokens."""
    rng = np.random.default_rng(5)
    b, L, D, N = 2, 40, 3, 4
    u = rng.standard_normal((b, L, D)).astype(np.float32)
    dl = np.exp(rng.uniform(np.log(1e-2), 0.0, (b, L, D))).astype(np.float32)
    A = (-rng.uniform(0.2, 3.0, (D, N))).astype(np.float32)
    Bm = rng.standard_normal((b, L, N)).astype(np.float32)
    Cm = rng.standard_normal((b, L, N)).astype(np.float32)
    Ds = np.ones(D, np.float32)
    y, last = oracle.fwd(u, dl, A, Bm, Cm, Ds)
    k = 17
    y1, l1 = oracle.fwd(u[:, :k], dl[:, :k], A, Bm[:, :k], Cm[:, :k], Ds)
    y2, l2 = oracle.fwd(u[:, k:], dl[:, k:], A, Bm[:, k:], Cm[:, k:], Ds, h0=l1.astype(np.float32))
    assert np.array_equal(y1, y[:, :k])
    assert rel_err(y2, y[:, k:]) < 1e-6 and rel_err(l2, last) < 1e-6


def test_empty_call_hands_back_initial_state():
    """No tokens: the state is handed back unchanged (TorchLean: an empty chunk preserves
    the state)."""
    h0 = np.arange(2 * 3 * 4, dtype=np.float32).reshape(2, 3, 4) - 5.0
    e = np.zeros((2, 0, 3), np.float32)
    _, last = oracle.fwd(e, e, -np.ones((3, 4), np.float32), np.zeros((2, 0, 4), np.float32),
                         np.zeros((2, 0, 4), np.float32), h0=h0)
    assert np.array_equal(last, h0.astype(np.float64))


# ---- first-order input coefficient ("Euler"): Algenta "Sequence and state-space models",
# mamba_selective_scan_step and its worked example; TorchLean "Selective Mamba", step

def test_euler_scalar_example(golden):
    g = golden("zoh_scalar_example.txt")
    abar, bbar = oracle.discretize(g["a"], g["b"], g["delta"], euler=True)
    assert abar == pytest.approx(g["abar"], abs=1e-15)              # the same exact Abar
    assert bbar * g["x"] + abar * g["h_prev"] == g["h1_first_order"]  # 1.0 exactly
    u = np.array([[[g["x"]], [0.0]]], np.float32)
    y, last = oracle.fwd(u, np.full((1, 2, 1), g["delta"], np.float32), np.array([[g["a"]]], np.float32),
                         np.full((1, 2, 1), g["b"], np.float32), np.ones((1, 2, 1), np.float32), euler=True)
    assert y[0, 0, 0] == g["h1_first_order"]
    assert y[0, 1, 0] == pytest.approx(g["abar"] * g["h1_first_order"], abs=1e-15)
    assert last[0, 0, 0] == pytest.approx(g["abar"] * g["h1_first_order"], abs=1e-15)
    # the printed gap between the two methods at this step size (about 27 %)
    assert (g["h1_first_order"] - g["h1_zoh"]) / g["h1_zoh"] == pytest.approx(0.27, abs=0.005)


@pytest.mark.parametrize("L", [1, 9, 60])
def test_euler_geometric_closed_form(L):
    """Constant delta, a, b and a unit input: h_t = delta b (1 - Abar^(t+1)) / (1 - Abar)."""
    dt, a, b = np.float32(0.37), np.float32(-1.3), np.float32(0.8)
    y, _ = oracle.fwd(np.ones((1, L, 1), np.float32), np.full((1, L, 1), dt, np.float32),
                      np.full((1, 1), a, np.float32), np.full((1, L, 1), b, np.float32),
                      np.ones((1, L, 1), np.float32), euler=True)
    q = math.exp(float(dt) * float(a))
    t = np.arange(L)
    np.testing.assert_allclose(y[0, :, 0], float(dt) * float(b) * (1 - q ** (t + 1)) / (1 - q), rtol=1e-13)


def test_euler_brute_force_and_zero_rate():
    rng = np.random.default_rng(91)
    inp = _rand_s6(rng, 2, 9, 3, 4, zero_a=True)
    y, last = oracle.fwd(*inp, euler=True)
    yb, lb = brute_force(*inp, euler=True)
    assert rel_err(y, yb) < 1e-12 and rel_err(last, lb) < 1e-12
    h0 = rng.standard_normal((2, 3, 4)).astype(np.float32)
    y, last = oracle.fwd(*inp, h0=h0, euler=True)
    yb, lb = brute_force(*inp, h0=h0, euler=True)
    assert rel_err(y, yb) < 1e-12 and rel_err(last, lb) < 1e-12
    # with every rate zero the two discretisations coincide (both integrate delta * B * u)
    u, delta, A, B, C, Ds, z = inp
    A0 = np.zeros_like(A)
    assert np.array_equal(oracle.fwd(u, delta, A0, B, C, Ds, z, euler=True)[0], oracle.fwd(u, delta, A0, B, C, Ds, z)[0])


def test_euler_approaches_zoh_for_small_steps():
    """Bbar_zoh / Bbar_euler = expm1(delta a) / (delta a) = 1 + delta a / 2 + O((delta a)^2)."""
    for dt in (1e-2, 1e-3, 1e-4):
        _, bz = oracle.discretize(-2.0, 1.0, dt)
        _, be = oracle.discretize(-2.0, 1.0, dt, euler=True)
        assert be == dt
        assert bz / be - 1.0 == pytest.approx(-dt, rel=2 * dt)


def test_euler_time_invariant_equals_selective():
    rng = np.random.default_rng(93)
    batch, L, N = 2, 40, 3
    u = rng.standard_normal((batch, L, 1)).astype(np.float32)
    A = -rng.uniform(0.1, 2.0, (1, N)).astype(np.float32)
    B = rng.standard_normal((1, N)).astype(np.float32)
    C = rng.standard_normal((1, N)).astype(np.float32)
    y_ti, l_ti = oracle.fwd(u, np.array([0.3], np.float32), A, B, C, euler=True, time_invariant=True)
    y_s6, l_s6 = oracle.fwd(u, np.full((batch, L, 1), 0.3, np.float32), A, np.broadcast_to(B, (batch, L, N)).copy(),
                            np.broadcast_to(C, (batch, L, N)).copy(), euler=True)
    assert np.array_equal(y_ti, y_s6) and np.array_equal(l_ti, l_s6)


# ---- softplus of the step size: Algenta page, mamba_delta_softplus; TorchLean "Selective
# Mamba", step (softplus of the projection plus dtBias)

def test_softplus_printed_values_and_identities(golden):
    g = golden("softplus_values.txt")
    assert oracle.softplus(0.0) == pytest.approx(g["softplus_0"], abs=1e-16)
    assert oracle.softplus(1.0) == pytest.approx(g["softplus_1"], abs=1e-15)
    xs = np.concatenate([np.linspace(-40, 40, 801), [-700.0, -80.0, 80.0, 700.0, 1e-9, -1e-9]])
    got = np.array([oracle.softplus(float(x)) for x in xs])
    np.testing.assert_allclose(got, np.logaddexp(0.0, xs), rtol=4e-16, atol=0)
    np.testing.assert_allclose(got - np.array([oracle.softplus(-float(x)) for x in xs]), xs, rtol=1e-12, atol=1e-15)
    assert oracle.softplus(1000.0) == 1000.0 and 0.0 < oracle.softplus(-700.0) < 1e-300


@pytest.mark.parametrize("euler", [False, True])
def test_fused_step_size_transform_brute_force(euler):
    rng = np.random.default_rng(95 + euler)
    u, _, A, B, C, Ds, z = _rand_s6(rng, 2, 9, 3, 4, zero_a=True)
    raw = rng.normal(-1.0, 1.5, u.shape).astype(np.float32)
    bias = rng.normal(0.0, 1.0, 3).astype(np.float32)
    x64 = raw.astype(np.float64) + bias.astype(np.float64)[None, None, :]
    # bias, then softplus
    y, last = oracle.fwd(u, raw, A, B, C, Ds, z, delta_bias=bias, delta_softplus=True, euler=euler)
    yb, lb = brute_force(u, np.logaddexp(0.0, x64), A, B, C, Ds, z, euler=euler)
    assert rel_err(y, yb) < 1e-12 and rel_err(last, lb) < 1e-12
    # softplus without a bias
    y, _ = oracle.fwd(u, raw, A, B, C, Ds, z, delta_softplus=True, euler=euler)
    yb, _ = brute_force(u, np.logaddexp(0.0, raw.astype(np.float64)), A, B, C, Ds, z, euler=euler)
    assert rel_err(y, yb) < 1e-12
    # a bias alone shifts the step size (positive inputs keep it positive)
    pos = np.abs(raw) + np.float32(0.05)
    bpos = np.abs(bias) * np.float32(0.1)
    y, _ = oracle.fwd(u, pos, A, B, C, Ds, z, delta_bias=bpos, euler=euler)
    yb, _ = brute_force(u, pos.astype(np.float64) + bpos.astype(np.float64)[None, None, :], A, B, C, Ds, z,
                        euler=euler)
    assert rel_err(y, yb) < 1e-12


def test_fused_step_size_time_invariant():
    rng = np.random.default_rng(97)
    D, N, L = 3, 4, 50
    u = rng.standard_normal((2, L, D)).astype(np.float32)
    raw = rng.normal(-2.0, 1.0, D).astype(np.float32)
    bias = rng.normal(0.0, 0.5, D).astype(np.float32)
    A = (-rng.uniform(0.2, 2.0, (D, N))).astype(np.float32)
    B = rng.standard_normal((D, N)).astype(np.float32)
    C = rng.standard_normal((D, N)).astype(np.float32)
    y, _ = oracle.fwd(u, raw, A, B, C, delta_bias=bias, delta_softplus=True, time_invariant=True)
    dt = np.logaddexp(0.0, raw.astype(np.float64) + bias.astype(np.float64))
    assert rel_err(y, oracle.conv_ti_direct(u, dt, A, B, C)) < 1e-12
