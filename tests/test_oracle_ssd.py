"""Pins for the scalar-decay (Mamba-2, "SSD") layer of the oracle ("state-space models",
section "Mamba-2 and state-space duality"): the recurrence with one decay per head equals the
pairwise masked form Y = (L o Q K^T) V written out from the page's equation (state-space
duality), for both input coefficients; the one-token case is C . Bbar x by hand; and a head
whose decay is 1 (A = 0) integrates (a cumulative sum)."""
import numpy as np
import pytest

import oracle


def rand_ssd(rng, b, L, H, P, N):
    x = rng.standard_normal((b, L, H, P)).astype(np.float32)
    dl = np.exp(rng.uniform(np.log(1e-2), 0.0, (b, L, H))).astype(np.float32)
    A = (-rng.uniform(0.2, 3.0, H)).astype(np.float32)
    B = rng.standard_normal((b, L, N)).astype(np.float32)
    C = rng.standard_normal((b, L, N)).astype(np.float32)
    return x, dl, A, B, C


@pytest.mark.parametrize("euler", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1), (2, 37, 3, 4, 5), (1, 80, 2, 8, 16)])
def test_recurrence_equals_pairwise_form(shape, euler):
    rng = np.random.default_rng(sum(shape) + euler)
    x, dl, A, B, C = rand_ssd(rng, *shape)
    y_rec, _ = oracle.ssd_fwd(x, dl, A, B, C, euler=euler)
    y_quad = oracle.ssd_quadratic(x, dl, A, B, C, euler=euler)
    scale = max(np.max(np.abs(y_quad)), 1e-300)
    assert np.max(np.abs(y_rec - y_quad)) / scale < 1e-12


def test_one_token_by_hand():
    x = np.array([[[[2.0, -1.0]]]], np.float32)          # b=1, L=1, H=1, P=2
    dl = np.array([[[0.5]]], np.float32)
    A = np.array([-1.0], np.float32)
    B = np.array([[[1.0, 3.0]]], np.float32)
    C = np.array([[[0.5, -2.0]]], np.float32)
    cb = 0.5 * 1.0 + (-2.0) * 3.0                         # C . B
    c_zoh = np.expm1(-0.5) / -1.0
    y, last = oracle.ssd_fwd(x, dl, A, B, C)
    np.testing.assert_allclose(y[0, 0, 0], cb * c_zoh * np.array([2.0, -1.0]), rtol=1e-13)
    np.testing.assert_allclose(last[0, 0], c_zoh * np.outer([2.0, -1.0], [1.0, 3.0]), rtol=1e-13)
    y_e, _ = oracle.ssd_fwd(x, dl, A, B, C, euler=True)
    np.testing.assert_allclose(y_e[0, 0, 0], cb * 0.5 * np.array([2.0, -1.0]), rtol=1e-13)


def test_unit_decay_integrates():
    rng = np.random.default_rng(3)
    x, dl, A, B, C = rand_ssd(rng, 1, 30, 2, 3, 4)
    A[:] = 0.0                                            # a_t = 1: h_t = sum_s delta_s B_s x_s
    y, _ = oracle.ssd_fwd(x, dl, A, B, C)
    for h in range(2):
        hist = np.cumsum(dl[0, :, h, None, None].astype(np.float64) * B[0][:, :, None] * x[0, :, h][:, None, :], axis=0)
        ref = np.einsum("tn,tnp->tp", C[0].astype(np.float64), hist)
        np.testing.assert_allclose(y[0, :, h], ref, rtol=1e-12, atol=1e-12)
