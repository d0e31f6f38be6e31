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


def _composed_case(pos, base=10000.0):
    """A unit hidden vector e_3 whose q projection is e_0 and k projection 2 e_1
    (column 3 of the weight), non-uniform gains, distinct q and k scales."""
    rng = np.random.default_rng(4)
    H, D = 16, 8
    w = rng.standard_normal((2 * D, H))
    w[:, 3] = 0.0
    w[0, 3] = 1.0            # q row 0
    w[D + 1, 3] = 2.0        # k row 1
    h = np.zeros((1, H))
    h[0, 3] = 1.0
    g_q = np.linspace(-0.5, 0.75, D)
    g_q[0], g_q[D // 2] = 0.5, -0.25
    g_k = np.linspace(0.3, -0.6, D)
    g_k[1], g_k[1 + D // 2] = -0.4, 0.6
    res = F.indexer_frontend(h, np.array([pos]), w, g_q, g_k, base, 20.0, 7.0, D, prequant=True)
    return res, g_q, g_k, D, base


def test_composed_front_end_at_position_zero():
    """Position 0: no rotation; q = e_0 normalised (rms sqrt(1/D)) times (1 + g_q[0])
    times q_scale, k = 2 e_1 normalised (rms 2 sqrt(1/D)) times (1 + g_k[1]) times k_scale."""
    (qi, ki, qf, kf), g_q, g_k, D, _ = _composed_case(0)
    want_q = np.zeros(D)
    want_q[0] = 20.0 * (1 + g_q[0]) / np.sqrt(1.0 / D + F.RMS_EPS)
    want_k = np.zeros(D)
    want_k[1] = 7.0 * 2.0 * (1 + g_k[1]) / np.sqrt(4.0 / D + F.RMS_EPS)
    assert np.allclose(qf[0], want_q, atol=1e-12) and np.allclose(kf[0], want_k, atol=1e-12)
    assert qi[0].tolist() == np.rint(want_q).astype(int).tolist()
    assert ki[0].tolist() == np.rint(want_k).astype(int).tolist()


def test_composed_front_end_at_position_p():
    """Position p: the normalised q's pair (0, D/2) turns by p radians and k's pair
    (1, 1 + D/2) by p * base^(-2/D), after the gains (norm first, then rotation)."""
    p = 3
    (qi, ki, qf, kf), g_q, g_k, D, base = _composed_case(p)
    vq = 20.0 * (1 + g_q[0]) / np.sqrt(1.0 / D + F.RMS_EPS)
    vk = 7.0 * 2.0 * (1 + g_k[1]) / np.sqrt(4.0 / D + F.RMS_EPS)
    a = p * base ** (-2.0 / D)
    want_q = np.zeros(D)
    want_q[0], want_q[D // 2] = vq * np.cos(p), vq * np.sin(p)
    want_k = np.zeros(D)
    want_k[1], want_k[1 + D // 2] = vk * np.cos(a), vk * np.sin(a)
    assert np.allclose(qf[0], want_q, atol=1e-12) and np.allclose(kf[0], want_k, atol=1e-12)
    assert qi[0].tolist() == np.clip(np.rint(want_q), -127, 127).astype(int).tolist()
    assert ki[0].tolist() == np.clip(np.rint(want_k), -127, 127).astype(int).tolist()


# ---- MRoPE (F5): three position components, contiguous frequency sections ----

def _unit(D, i):
    e = np.zeros((1, D))
    e[0, i] = 1.0
    return e


def test_mrope_with_equal_components_is_the_1d_rotation():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 16))
    p = np.array([0, 7, 4096, 999983])
    assert np.array_equal(F.mrope(x, np.stack([p, p, p]), 10000.0, (2, 3, 3)), F.rope(x, p, 10000.0))


def test_mrope_each_section_turns_with_its_own_component_only():
    """D = 16, sections (2, 3, 3): pairs 0-1 follow the temporal component,
    2-4 the height, 5-7 the width.  A position with one non-zero component
    turns exactly that section's pairs, each by p * base^(-2i/D) (closed form)."""
    D, base, p = 16, 10000.0, 11
    sec = (2, 3, 3)
    owner = [0, 0, 1, 1, 1, 2, 2, 2]
    for c in range(3):
        pos3 = np.zeros((3, 1), dtype=np.int64)
        pos3[c, 0] = p
        for i in range(D // 2):
            y = F.mrope(_unit(D, i), pos3, base, sec)
            a = p * base ** (-2.0 * i / D) if owner[i] == c else 0.0
            want = np.zeros(D)
            want[i], want[i + D // 2] = np.cos(a), np.sin(a)
            assert np.allclose(y[0], want, rtol=0, atol=1e-12), (c, i)


def test_mrope_first_pair_of_each_section_closed_form():
    D, base = 64, 10000.0
    sec = (8, 12, 12)
    pos3 = np.array([[3], [5], [7]])
    for i, p in [(0, 3), (8, 5), (20, 7)]:
        y = F.mrope(_unit(D, i), pos3, base, sec)
        a = p * base ** (-2.0 * i / D)
        assert np.isclose(y[0, i], np.cos(a), atol=1e-12) and np.isclose(y[0, i + D // 2], np.sin(a), atol=1e-12)


def test_mrope_keeps_pair_norms_and_depends_on_relative_positions_only():
    rng = np.random.default_rng(6)
    x, y = rng.standard_normal((1, 32)), rng.standard_normal((1, 32))
    sec = (4, 6, 6)
    m, n, d = np.array([[7], [30], [2]]), np.array([[3], [1], [50]]), np.array([[100], [-13], [4096]])
    xm = F.mrope(x, m, 10000.0, sec)
    assert np.allclose(xm[0, :16] ** 2 + xm[0, 16:] ** 2, x[0, :16] ** 2 + x[0, 16:] ** 2)
    a = (xm @ F.mrope(y, n, 10000.0, sec).T).item()
    b = (F.mrope(x, m + d, 10000.0, sec) @ F.mrope(y, n + d, 10000.0, sec).T).item()
    assert np.isclose(a, b, rtol=0, atol=1e-8)


def test_composed_front_end_with_mrope():
    """The composed front end at position (p_t, p_h, p_w) with sections (1, 1, 2)
    of D = 8: q = e_0 normalised lies in pair 0 (temporal) and turns by p_t; k = 2 e_1
    lies in pair 1 (height) and turns by p_h * base^(-2/D)."""
    rng = np.random.default_rng(4)
    H, D, base = 16, 8, 10000.0
    w = rng.standard_normal((2 * D, H))
    w[:, 3] = 0.0
    w[0, 3] = 1.0
    w[D + 1, 3] = 2.0
    h = np.zeros((1, H))
    h[0, 3] = 1.0
    g_q = np.linspace(-0.5, 0.75, D)
    g_k = np.linspace(0.3, -0.6, D)
    pt, ph, pw = 5, 9, 40
    qi, ki, qf, kf = F.indexer_frontend(h, np.array([[pt], [ph], [pw]]), w, g_q, g_k, base, 20.0, 7.0, D,
                                        prequant=True, mrope_sections=(1, 1, 2))
    vq = 20.0 * (1 + g_q[0]) / np.sqrt(1.0 / D + F.RMS_EPS)
    vk = 7.0 * 2.0 * (1 + g_k[1]) / np.sqrt(4.0 / D + F.RMS_EPS)
    a = ph * base ** (-2.0 / D)
    want_q = np.zeros(D)
    want_q[0], want_q[D // 2] = vq * np.cos(pt), vq * np.sin(pt)
    want_k = np.zeros(D)
    want_k[1], want_k[1 + D // 2] = vk * np.cos(a), vk * np.sin(a)
    assert np.allclose(qf[0], want_q, atol=1e-12) and np.allclose(kf[0], want_k, atol=1e-12)
    assert qi[0].tolist() == np.clip(np.rint(want_q), -127, 127).astype(int).tolist()
    assert ki[0].tolist() == np.clip(np.rint(want_k), -127, 127).astype(int).tolist()
