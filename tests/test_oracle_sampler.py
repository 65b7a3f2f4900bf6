"""Pins of the sampler-update oracle (CPU only)."""

import math

import numpy as np
import pytest
from scipy import integrate

from oracle import sampler


def _vp(t):
    """A variance-preserving schedule point: alpha^2 + sigma^2 = 1."""
    a = math.cos(0.5 * math.pi * t)
    return a, math.sqrt(1.0 - a * a)


@pytest.mark.parametrize("t_s,t_t", [(0.9, 0.7), (0.5, 0.45), (0.3, 0.05)])
def test_etd1_coefficients_match_the_exact_integral(t_s, t_t):
    """With the data prediction constant over the step, the exact step is
    x_t = (sigma_t/sigma_s) x_s + sigma_t * int e^lambda dlambda * x0: the
    integral is taken by adaptive quadrature, independent of the formula."""
    a_s, s_s = _vp(t_s)
    a_t, s_t = _vp(t_t)
    decay, coeff = sampler.etd1_coefficients(a_s, s_s, a_t, s_t)
    lam_s, lam_t = math.log(a_s / s_s), math.log(a_t / s_t)
    integral, err = integrate.quad(math.exp, lam_s, lam_t, epsabs=0, epsrel=1e-13)
    assert decay == pytest.approx(s_t / s_s, rel=1e-13)
    assert coeff == pytest.approx(s_t * integral, rel=1e-12)


def test_etd1_is_exact_over_many_steps_for_a_constant_prediction():
    """Chained ETD1 steps from t = 0.95 to 0.02 equal the one-step exact
    solution when x0_hat is constant (the linear part is solved exactly)."""
    rng = np.random.default_rng(80)
    x = rng.standard_normal(64)
    x0 = rng.standard_normal(64)
    ts = np.linspace(0.95, 0.02, 12)
    y = x.copy()
    for s, t in zip(ts[:-1], ts[1:]):
        y = sampler.etd1_update(y, x0, *sampler.etd1_coefficients(*_vp(s), *_vp(t)))
    a0, s0 = _vp(ts[0])
    a1, s1 = _vp(ts[-1])
    exact = (s1 / s0) * x + s1 * (a1 / s1 - a0 / s0) * x0
    assert np.allclose(y, exact, rtol=1e-12, atol=1e-12)


def test_etd2_equal_predictions_and_first_step_reduce_to_etd1():
    rng = np.random.default_rng(81)
    x, x0, x0p = rng.standard_normal((3, 32))
    args = (*_vp(0.6), *_vp(0.5))
    d1, c = sampler.etd1_coefficients(*args)
    d, c0, c1 = sampler.etd2_coefficients(*args, first_step=False)
    assert d == d1 and c0 == 0.75 * c and c1 == 0.25 * c
    assert np.allclose(sampler.etd2_update(x, x0, x0, d, c0, c1), sampler.etd1_update(x, x0, d1, c), rtol=1e-15)
    d, c0, c1 = sampler.etd2_coefficients(*args, first_step=True)
    assert (d, c0, c1) == (d1, c, 0.0)
    # the previous prediction enters with weight 1/4 of the coefficient
    out = sampler.etd2_update(x, x0, x0p, *sampler.etd2_coefficients(*args, first_step=False))
    assert np.allclose(out - sampler.etd1_update(x, x0, d1, c), 0.25 * c * (x0p - x0), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("p", [1, 2])
def test_richardson_cancels_the_leading_error(p):
    """fine = x* + C (h/2)^p, coarse = x* + C h^p: the combine returns x*."""
    rng = np.random.default_rng(90 + p)
    xs, c = rng.standard_normal((2, 50))
    h = 0.1
    fine = xs + c * (h / 2) ** p
    coarse = xs + c * h ** p
    out = sampler.richardson_combine(fine, coarse, 2.0 ** p)
    assert np.allclose(out, xs, rtol=0, atol=1e-14)
    if p == 1:
        assert np.allclose(out, 2 * fine - coarse, rtol=0, atol=1e-15)
    else:
        assert np.allclose(out, (4 * fine - coarse) / 3, rtol=0, atol=1e-15)
