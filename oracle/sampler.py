"""Diffusion-sampler update steps: ETD1, ETD2 and the Richardson combine.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "拡散サンプリングの高速化：数値計算手法とスコアベースモデルの出会い"
(Accelerating diffusion sampling: numerical methods meet score-based models),
sections on the exponential integrator (ETD1, ETD2), Richardson
extrapolation and the fused update kernels.

In log-SNR time lambda = log(alpha / sigma) the exact step from s to t is
    x_t = (sigma_t / sigma_s) x_s + sigma_t * integral_{lambda_s}^{lambda_t}
          e^lambda x0_hat(lambda) dlambda,
and the ETD methods solve the linear part exactly and approximate only the
integral of the network's data prediction x0_hat.

* ETD1: x0_hat held at its value at the start of the step:
      x_{n+1} = decay * x_n + coeff * x0^(n),
      decay = e^-h * alpha_{n+1} / alpha_n (= sigma_{n+1} / sigma_n),
      coeff = alpha_{n+1} * (1 - e^-h),  h = lambda_{n+1} - lambda_n.
  Reading: the page prints e^h where the exact solution above needs e^-h
  for h = lambda_{n+1} - lambda_n > 0; the sign that reproduces the exact
  solution is taken (the two agree if h is read as lambda_n - lambda_{n+1}).
* ETD2: the same decay and coefficient applied to (3/4) x0^(n) + (1/4)
  x0^(n-1), as the page writes it (c0 = 3/4 coeff, c1 = 1/4 coeff); the
  first step, with no previous prediction, is ETD1.
* Richardson: with results x_N (N steps) and x_2N (2N steps) of an order-p
  method, x = (2^p x_2N - x_N) / (2^p - 1); the page's kernel form is
  (scale * fine - coarse) / (scale - 1), scale = 2^p.

The updates are elementwise; they are written out in float64 on whatever
array shapes they are given.
"""

import math

import numpy as np


def log_snr(alpha, sigma):
    return math.log(alpha / sigma)


def etd1_coefficients(alpha_s, sigma_s, alpha_t, sigma_t):
    """(decay, coeff) of the ETD1 step from (alpha_s, sigma_s) to (alpha_t, sigma_t)."""
    h = log_snr(alpha_t, sigma_t) - log_snr(alpha_s, sigma_s)
    decay = math.exp(-h) * alpha_t / alpha_s
    coeff = alpha_t * (1.0 - math.exp(-h))
    return decay, coeff


def etd2_coefficients(alpha_s, sigma_s, alpha_t, sigma_t, first_step):
    """(decay, c0, c1) of the ETD2 step; the first step falls back to ETD1."""
    decay, coeff = etd1_coefficients(alpha_s, sigma_s, alpha_t, sigma_t)
    if first_step:
        return decay, coeff, 0.0
    return decay, 0.75 * coeff, 0.25 * coeff


def etd1_update(x, x0, decay, coeff):
    return decay * np.asarray(x, dtype=np.float64) + coeff * np.asarray(x0, dtype=np.float64)


def etd2_update(x, x0, x0_prev, decay, c0, c1):
    return (decay * np.asarray(x, dtype=np.float64) + c0 * np.asarray(x0, dtype=np.float64)
            + c1 * np.asarray(x0_prev, dtype=np.float64))


def richardson_combine(fine, coarse, scale):
    """(scale * fine - coarse) / (scale - 1); scale = 2^p for an order-p method."""
    fine = np.asarray(fine, dtype=np.float64)
    coarse = np.asarray(coarse, dtype=np.float64)
    return (scale * fine - coarse) / (scale - 1.0)
