"""Pins for the oracle's schedule, guidance combine, DDIM / Euler steps and
rel-MAE (CPU only).

Pins come from closed forms and exact arithmetic, not from the oracle's own
formulas: exact-rational DDIM steps (tests/golden/ddim_worked.txt), the DDIM
trajectory that must land exactly on a chosen x0, the sum-of-squares closed
form of the scaled-linear betas, exact-rational timestep rounding, the Euler
telescoping sum, and the special values of rel-MAE.
"""
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------- schedule
def test_beta_endpoints_and_first_alpha_bar():
    b = oracle.scaled_linear_betas(1000, 0.00085, 0.012)
    assert b.shape == (1000,)
    assert abs(b[0] - 0.00085) < 1e-18
    assert abs(b[-1] - 0.012) < 1e-17
    a = oracle.alphas_cumprod(b)
    assert abs(a[0] - (1 - 0.00085)) < 1e-16   # abar_0 = 1 - beta_0, not 1
    assert np.all(np.diff(a) < 0)


def test_beta_sum_closed_form():
    # sum_{i=0}^{n} (a + h i)^2 = (n+1) a^2 + a h n (n+1) + h^2 n (n+1)(2n+1)/6.
    # Linear-in-beta betas would sum to 1000 * (b0 + b1)/2 = 6.425 instead.
    a = math.sqrt(0.00085)
    n = 999
    h = (math.sqrt(0.012) - a) / n
    closed = (n + 1) * a * a + a * h * n * (n + 1) + h * h * n * (n + 1) * (2 * n + 1) / 6
    b = oracle.scaled_linear_betas(1000, 0.00085, 0.012)
    assert abs(b.sum() - closed) < 1e-12
    assert abs(closed - 6.425) > 1.0


def test_alpha_bar_against_high_precision_product():
    getcontext().prec = 50
    a = Decimal("0.00085").sqrt()
    bb = Decimal("0.012").sqrt()
    prod = Decimal(1)
    ref = {}
    for i in range(1000):
        r = a + (bb - a) * Decimal(i) / Decimal(999)
        prod *= (1 - r * r)
        ref[i] = prod
    abar = oracle.alphas_cumprod(oracle.scaled_linear_betas(1000, 0.00085, 0.012))
    for t in (0, 1, 111, 500, 888, 999):
        assert abs(abar[t] - float(ref[t])) < 1e-13 * max(1.0, float(ref[t]))


def _half_even_round(fr: Fraction) -> int:
    fl = math.floor(fr)
    rem = fr - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


@pytest.mark.parametrize("S", [1, 2, 10, 28, 50, 100])
def test_timesteps_exact_rational_rounding(S):
    ts = oracle.ddim_timesteps(1000, S)
    if S == 1:
        assert list(ts) == [0]
        return
    expect = [_half_even_round(Fraction(999 * i, S - 1)) for i in range(S)]
    assert list(ts) == expect
    if S == 10:
        assert list(ts) == list(range(0, 1000, 111))


# ----------------------------------------------------------------- guidance
def test_cfg_special_weights():
    r = _rng(1)
    gc, gu = r.standard_normal(50), r.standard_normal(50)
    np.testing.assert_allclose(oracle.cfg_combine(gc, gu, 1.0), gc, rtol=0, atol=1e-15)
    np.testing.assert_array_equal(oracle.cfg_combine(gc, gu, 0.0), gu)
    np.testing.assert_array_equal(oracle.cfg_combine(gu, gu, 7.5), gu)
    f0, f1, f2 = (oracle.cfg_combine(gc, gu, w) for w in (0.0, 1.0, 2.0))
    np.testing.assert_allclose(f2 - f1, f1 - f0, rtol=0, atol=1e-14)
    # w = 7.5 pushes 7.5x further from the unconditional prediction
    np.testing.assert_allclose(oracle.cfg_combine(gc, gu, 7.5) - gu, 7.5 * (gc - gu),
                               rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------------- DDIM
def test_ddim_hand_worked_golden():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "ddim_worked.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) >= 7
    for at, ap, last, x, e, want in rows:
        got = oracle.ddim_step(np.array([float(x)]), np.array([float(e)]),
                               float(at), float(ap), bool(int(last)))
        assert abs(got[0] - float(want)) < 1e-14, (at, ap, last, x, e, want, got)


@pytest.mark.parametrize("steps,w", [(10, 7.5), (50, 7.5), (10, 0.0)])
def test_ddim_trajectory_lands_on_x0(steps, w):
    # If x_T = sqrt(abar_T) x0* + sqrt(1-abar_T) eps* and the guided
    # prediction is eps* at every step, every x0 estimate is x0* and the
    # last step returns exactly x0*.  The pair (g_c, g_u) is built so that
    # g_u + w (g_c - g_u) = eps* while g_c and g_u themselves differ.
    r = _rng(steps)
    x0 = r.standard_normal(64)
    eps = r.standard_normal(64)
    delta = r.standard_normal(64)
    g_u = eps - w * delta
    g_c = g_u + delta
    sch = oracle.DDIMSchedule(steps)
    abar_T = sch.abar[sch.ts[-1]]
    x = math.sqrt(abar_T) * x0 + math.sqrt(1 - abar_T) * eps
    for i in range(steps):
        x, _ = sch.step(x, g_c, g_u, w, i)
    np.testing.assert_allclose(x, x0, rtol=0, atol=1e-11)


def test_ddim_step_order():
    sch = oracle.DDIMSchedule(10)
    at, ap, last = sch.step_args(0)
    assert (at, ap, last) == (sch.abar[999], sch.abar[888], False)
    at, ap, last = sch.step_args(9)
    assert (at, ap, last) == (sch.abar[0], 1.0, True)


def test_ddim_identity_step():
    x = _rng(3).standard_normal(10)
    e = _rng(4).standard_normal(10)
    np.testing.assert_allclose(oracle.ddim_step(x, e, 0.3, 0.3, False), x, rtol=0, atol=1e-14)


# -------------------------------------------------------------------- Euler
def test_flow_sigmas():
    s = oracle.flow_sigmas(28)
    assert s.shape == (29,)
    assert s[0] == 1.0 and s[-1] == 0.0
    np.testing.assert_allclose(np.diff(s), -1 / 28, rtol=0, atol=1e-15)


def test_euler_constant_velocity_telescopes():
    r = _rng(5)
    x1 = r.standard_normal(32)
    vstar = r.standard_normal(32)
    delta = r.standard_normal(32)
    w = 3.5
    v_u = vstar - w * delta
    v_c = v_u + delta
    sch = oracle.EulerSchedule(28)
    x = x1.copy()
    for i in range(28):
        x, _ = sch.step(x, v_c, v_u, w, i)
        np.testing.assert_allclose(x, x1 - (1 - sch.sigmas[i + 1]) * vstar, rtol=0, atol=1e-13)
    np.testing.assert_allclose(x, x1 - vstar, rtol=0, atol=1e-13)


# ------------------------------------------------------------------ rel-MAE
def test_relmae_special_values():
    r = _rng(6)
    gu = r.standard_normal(1000)
    assert oracle.relmae(gu, gu) == 0.0
    for alpha in (0.25, -0.6, 3.0):
        assert abs(oracle.relmae((1 + alpha) * gu, gu) - abs(alpha)) < 1e-14
    assert abs(oracle.relmae(-gu, gu) - 2.0) < 1e-15
    gc = r.standard_normal(1000)
    assert abs(oracle.relmae(5 * gc, 5 * gu) - oracle.relmae(gc, gu)) < 1e-14
    # the unconditional prediction is the reference (denominator)
    assert abs(oracle.relmae(np.ones(4), 2 * np.ones(4)) - 0.5) < 1e-16
    assert math.isnan(oracle.relmae(np.zeros(3), np.zeros(3)))
    assert math.isinf(oracle.relmae(np.ones(3), np.zeros(3)))


def test_relmae_tiny_brute_force():
    gc = [1.5, -2.0, 0.25]
    gu = [1.0, 1.0, -0.75]
    # |0.5| + |-3| + |1| = 4.5 ; |1| + |1| + |0.75| = 2.75
    assert abs(oracle.relmae(gc, gu) - 4.5 / 2.75) < 1e-15


def test_relmae_iid_gaussian_near_sqrt2():
    # Statistical sanity only: E|X - Y| / E|Y| = sqrt(2) for iid normals.
    r = _rng(7)
    val = oracle.relmae(r.standard_normal(200000), r.standard_normal(200000))
    assert abs(val - math.sqrt(2)) < 0.01


# ------------------------------------------------------------ DDIM with eta > 0
def test_ddim_eta_zero_is_the_deterministic_step():
    rng = np.random.default_rng(21)
    x, e, z = (rng.standard_normal(64) for _ in range(3))
    for last in (False, True):
        np.testing.assert_array_equal(oracle.ddim_step_eta(x, e, z, 0.3, 0.7, 0.0, last),
                                      oracle.ddim_step(x, e, 0.3, 0.7, last))


@pytest.mark.parametrize("eta", [0.25, 0.5, 1.0])
@pytest.mark.parametrize("abar_t,abar_prev", [(0.2, 0.45), (0.004660098513077238, 0.016009281935883385),
                                              (0.8803525730500632, 0.99915)])
def test_ddim_eta_preserves_the_forward_marginal(eta, abar_t, abar_prev):
    """Whatever eta, a step from x_t = sqrt(abar_t) x0 + sqrt(1 - abar_t) eps
    with the exact eps lands on sqrt(abar_prev) x0 + c_e eps + c_z z with
    c_e^2 + c_z^2 = 1 - abar_prev: the same N(sqrt(abar_prev) x0, 1 - abar_prev)
    marginal as the forward process at the previous timestep (DDIM's defining
    property).  The coefficients are read off the oracle by unit inputs."""
    x0 = np.array([0.7])
    unit, zero = np.array([1.0]), np.array([0.0])
    def run(eps, z):
        x = np.sqrt(abar_t) * x0 + np.sqrt(1.0 - abar_t) * eps
        return oracle.ddim_step_eta(x, eps, z, abar_t, abar_prev, eta, False)[0]
    base = run(zero, zero)
    np.testing.assert_allclose(base, np.sqrt(abar_prev) * x0[0], rtol=0, atol=1e-13)
    c_e = run(unit, zero) - base
    c_z = run(zero, unit) - base
    assert c_z > 0
    np.testing.assert_allclose(c_e ** 2 + c_z ** 2, 1.0 - abar_prev, rtol=1e-12, atol=0)


def test_ddim_eta_one_noise_is_the_posterior_scale():
    """At eta = 1 the added noise has the scale of the Gaussian posterior
    q(x_prev | x_t, x0) of the forward process, derived here from the forward
    process alone: with a = abar_prev, b = abar_t / abar_prev, the posterior
    variance is (1 - a) (1 - b) / (1 - a b)."""
    a_t, a_p = 0.2, 0.45
    unit, zero = np.array([1.0]), np.array([0.0])
    x = np.array([0.3])
    c_z = (oracle.ddim_step_eta(x, zero, unit, a_t, a_p, 1.0, False)
           - oracle.ddim_step_eta(x, zero, zero, a_t, a_p, 1.0, False))[0]
    a, b = a_p, a_t / a_p
    np.testing.assert_allclose(c_z ** 2, (1 - a) * (1 - b) / (1 - a * b), rtol=1e-13)


def test_ddim_eta_last_step_adds_no_noise():
    rng = np.random.default_rng(22)
    x, e, z = (rng.standard_normal(16) for _ in range(3))
    np.testing.assert_array_equal(oracle.ddim_step_eta(x, e, z, 0.9, 1.0, 1.0, True),
                                  oracle.ddim_step(x, e, 0.9, 1.0, True))


# --------------------------------------------------- three-phase switch points
def test_switch_clean_u_curve_switches_at_its_minimum():
    """On a clean U (M_t = (t - c)^2 / S + 0.1) the averaged slope turns
    non-negative only L/2 steps after the minimum, so the cap decides:
    tau1 = c, tau2 = c + k."""
    S, c = 50, 23
    t = np.arange(S)
    M = (t - c) ** 2 / S + 0.1
    for L in (1, 2, 4):
        assert oracle.switch_points(M, L, 0.05, 5) == (c, c + 5)


def test_switch_plateau_before_the_minimum():
    """A fast drop to a flat plateau, then a deeper minimum later: the first
    flat point (slope 0 over the last L steps) wins over the cap."""
    M = np.concatenate([np.linspace(1.0, 0.1, 11),        # steps 0..10 drop
                        np.full(20, 0.1),                   # 11..30 flat
                        [0.08, 0.06, 0.05, 0.07, 0.1, 0.2]])  # minimum at step 33
    assert oracle.switch_points(M, 2, 1e-3, 5) == (12, 17)
    assert oracle.switch_points(M, 4, 1e-3, 5) == (14, 19)


def test_switch_slope_bound_is_strict_and_rising_curves_fall_back_to_the_cap():
    M = np.array([1.0, 0.5, 0.5 + 0.02, 0.4, 0.3, 0.35])
    # step 2: G = 0.02 over L = 1; only counts when g_slope > 0.02
    assert oracle.switch_points(M, 1, 0.02, 1) == (4, 5)
    assert oracle.switch_points(M, 1, 0.021, 1) == (2, 3)
    # strictly decreasing: no flat point, the cap is the last step, tau2 clamps
    assert oracle.switch_points(np.linspace(1, 0, 10), 2, 0.1, 5) == (9, 10)


def test_switch_ties_and_properties_on_random_series():
    rng = np.random.default_rng(5)
    assert oracle.switch_points([0.3, 0.1, 0.2, 0.1], 1, 0.0, 2) == (1, 3)   # first minimum
    for _ in range(200):
        S = int(rng.integers(1, 40))
        L = int(rng.integers(1, 6))
        g = float(rng.uniform(0.0, 0.2))
        M = rng.uniform(0.0, 1.0, S)
        t1, t2 = oracle.switch_points(M, L, g, 5)
        cap = int(np.argmin(M))
        assert 0 <= t1 <= cap and t2 == min(t1 + 5, S)
        if t1 < cap:                       # chosen by the slope rule: first such step
            G = (M[t1] - M[t1 - L]) / L
            assert t1 >= L and 0 <= G < g
        for t in range(L, t1):             # no earlier step qualifies
            G = (M[t] - M[t - L]) / L
            assert not (0 <= G < g)
