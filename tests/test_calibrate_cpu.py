"""Pins of the depth-calibration arithmetic (LoopSpec page, section 2.4: eq. 7 envelope, eq. 8
closed-form depths, eq. 11 commit-cost bound; section 3.1 and Figure 3 for the fitted
parameters).

* eq. 8 reproduces the depths the page prints: (beta, alpha) = (0.175, 1.03) gives about
  (1.26, 8.85) and (0.207, 1.08) gives about (1.41, 9.17), with R = 32;
* eq. 8 is the minimum of eq. 11: a numerical minimisation of the bound from several starts
  lands on it, and the bound's gradient vanishes there;
* the envelope fit returns exact power laws exactly, and over noisy curves lies on or above
  every point and touches at least one;
* the integer depths minimise eq. 11 over their search space and sit next to the
  continuous optimum.
"""

import numpy as np
import pytest
from scipy.optimize import minimize

from looped_transformer_self_amd import calibrate as cal


@pytest.mark.parametrize("beta,alpha,want", [(0.175, 1.03, (1.26, 8.85)), (0.207, 1.08, (1.41, 9.17))])
def test_closed_form_depths_match_the_page(beta, alpha, want):
    d1, d2 = cal.continuous_optimum(alpha, beta, 32)
    assert (round(d1, 2), round(d2, 2)) == want


@pytest.mark.parametrize("beta,alpha,R", [(0.175, 1.03, 32), (0.207, 1.08, 32), (0.3, 0.8, 16), (0.1, 1.5, 64)])
def test_closed_form_is_the_minimum_of_the_bound(beta, alpha, R):
    d1, d2 = cal.continuous_optimum(alpha, beta, R)
    f = lambda x: cal.commit_cost_bound(x[0], x[1], alpha, beta, R) if min(x) > 0 else np.inf
    for start in ((1.0, 2.0), (3.0, 12.0), (0.5, 20.0)):
        res = minimize(f, np.array(start), method="Nelder-Mead", options={"xatol": 1e-9, "fatol": 1e-12,
                                                                           "maxiter": 20000})
        assert abs(res.x[0] - d1) < 1e-4 * max(1, d1) and abs(res.x[1] - d2) < 1e-4 * max(1, d2), (res.x, d1, d2)
    h = 1e-6
    g1 = (f((d1 + h, d2)) - f((d1 - h, d2))) / (2 * h)
    g2 = (f((d1, d2 + h)) - f((d1, d2 - h))) / (2 * h)
    assert abs(g1) < 1e-5 and abs(g2) < 1e-5


def test_envelope_of_an_exact_power_law():
    r = np.array([1, 2, 3, 4, 6, 8, 12, 16], float)
    alpha, beta = cal.fit_envelope(r, 0.175 * r ** -1.03)
    assert abs(alpha - 1.03) < 1e-12 and abs(beta - 0.175) < 1e-12


def test_envelope_lies_above_noisy_points():
    rng = np.random.Generator(np.random.PCG64(3))
    r = np.array([1, 2, 3, 4, 6, 8, 12, 16, 24], float)
    for _ in range(20):
        tv = 0.3 * r ** -0.9 * np.exp(0.2 * rng.standard_normal(len(r)))
        alpha, beta = cal.fit_envelope(r, tv)
        env = beta * r ** -alpha
        assert np.all(env >= tv * (1 - 1e-12))
        assert np.min(env / tv) < 1 + 1e-9
    # depths whose TV is zero (the full depth) are left out of the fit
    a2, b2 = cal.fit_envelope(np.append(r, 32), np.append(0.2 * r ** -1.1, 0.0))
    assert abs(a2 - 1.1) < 1e-12 and abs(b2 - 0.2) < 1e-12


@pytest.mark.parametrize("beta,alpha", [(0.175, 1.03), (0.207, 1.08), (0.4, 0.7)])
def test_integer_depths_near_the_continuous_optimum(beta, alpha):
    R = 32
    d1, d2, c = cal.best_integer_depths(alpha, beta, R)
    d1c, d2c = cal.continuous_optimum(alpha, beta, R)
    assert abs(d1 - d1c) <= 1.5 and abs(d2 - d2c) <= 1.5
    assert c >= cal.commit_cost_bound(d1c, d2c, alpha, beta, R) - 1e-12
    m1, m2, cm = cal.best_integer_depths(alpha, beta, R, multiples=True)
    assert m2 % m1 == 0 and R % m1 == 0 and cm >= c


@pytest.mark.parametrize("R", [4, 8, 32])
def test_depth_passes_cover_the_depths(R):
    passes = cal.depth_passes(R)
    assert all(p[-1] == R and len(p) <= cal.MAX_DEPTHS and list(p) == sorted(set(p)) for p in passes)
    got = {r for p in passes for r in p if r < R}
    if R <= cal.MAX_DEPTHS:
        assert got == set(range(1, R))
    else:
        assert {1, 2, 4, 8, 16} <= got and len(got) >= 10
