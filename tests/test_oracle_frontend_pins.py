"""Pins of the front-end oracle to facts that do not come from itself: closed
forms of RMSNorm and rotary embedding, the rotation's invariants, and the
rounding rule, so that a dropped term, a wrong sign or a swapped half fails."""
import numpy as np

from oracle import qsa_frontend_oracle as F


def test_projection_of_unit_hidden_is_the_weight_column():
    rng = np.random.default_rng(0)
    H, D = 48, 8
    w = rng.standard_normal((2 * D, H))
    h = np.zeros((1, H))
    h[0, 5] = 1.0
    q, k = F.project(h, w, D)
    assert np.array_equal(q[0], w[:D, 5]) and np.array_equal(k[0], w[D:, 5])


def test_rmsnorm_closed_forms():
    g = np.array([0.0, 0.5, -0.25, 1.0])
    y = F.rmsnorm(np.full((1, 4), -3.0), g)
    assert np.allclose(y[0], -(1 + g) * 3.0 / np.sqrt(9.0 + F.RMS_EPS), rtol=0, atol=1e-12)
    y = F.rmsnorm(np.array([[3.0, 4.0, 0.0, 0.0]]), np.zeros(4))   # rms = 2.5
    assert np.allclose(y[0], np.array([3, 4, 0, 0]) / np.sqrt(6.25 + F.RMS_EPS), atol=1e-12)


def test_rope_position_zero_is_identity_and_first_pair_closed_form():
    x = np.random.default_rng(1).standard_normal((1, 16))
    assert np.array_equal(F.rope(x, np.array([0]), 10000.0), x)
    e0 = np.zeros((1, 16))
    e0[0, 0] = 1.0          # pair (0, 8) rotates by p * base^0 = p radians
    y = F.rope(e0, np.array([3]), 10000.0)
    assert np.isclose(y[0, 0], np.cos(3.0)) and np.isclose(y[0, 8], np.sin(3.0))
    assert np.allclose(np.delete(y[0], [0, 8]), 0.0)
    e1 = np.zeros((1, 16))
    e1[0, 1] = 1.0          # pair (1, 9) rotates by p * base^(-2/16)
    y = F.rope(e1, np.array([5]), 10000.0)
    a = 5 * 10000.0 ** (-2.0 / 16)
    assert np.isclose(y[0, 1], np.cos(a)) and np.isclose(y[0, 9], np.sin(a))


def test_rope_keeps_pair_norms_and_depends_on_relative_position_only():
    rng = np.random.default_rng(2)
    x, y = rng.standard_normal((1, 32)), rng.standard_normal((1, 32))
    for m, n, d in [(7, 3, 100), (0, 1000, 12345), (999983, 5, 17)]:
        xm = F.rope(x, np.array([m]), 10000.0)
        assert np.allclose(xm[0, :16] ** 2 + xm[0, 16:] ** 2, x[0, :16] ** 2 + x[0, 16:] ** 2)
        a = (xm @ F.rope(y, np.array([n]), 10000.0).T).item()
        b = (F.rope(x, np.array([m + d]), 10000.0) @ F.rope(y, np.array([n + d]), 10000.0).T).item()
        assert np.isclose(a, b, rtol=0, atol=1e-8)


def test_quantize_rounds_half_to_even_and_clamps_symmetrically():
    v = np.array([0.5, 1.5, 2.5, -0.5, -1.5, 126.49, 126.5, 127.5, 300.0, -300.0, -127.5])
    assert F.quantize(v, 1.0).tolist() == [0, 2, 2, 0, -2, 126, 126, 127, 127, -127, -127]
    assert F.quantize(np.array([0.25]), 6.0).tolist() == [2]   # 1.5 -> 2


def test_norm_then_rope_differs_from_rope_then_norm_when_gains_differ():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 8))
    g = rng.standard_normal(8)
    a = F.rope(F.rmsnorm(x, g), np.array([11]), 10000.0)
    b = F.rmsnorm(F.rope(x, np.array([11]), 10000.0), g)
    assert not np.allclose(a, b)     # the order F3 fixes matters
    z = np.zeros(8)
    assert np.allclose(F.rope(F.rmsnorm(x, z), np.array([11]), 10000.0),
                       F.rmsnorm(F.rope(x, np.array([11]), 10000.0), z))   # with unit gains it does not
