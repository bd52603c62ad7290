"""Pins for the oracle's quantizer constants and storage accounting (CPU only)."""

import json
import math
import os

import numpy as np
import pytest
from scipy import integrate, optimize

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _round_to(x, digits):
    return float(f"{x:.{digits}f}")


def test_lloyd_max_matches_published_table():
    g = _golden("lloyd_max_gaussian4.json")
    tau, a, b, mse = oracle.lloyd_max_gaussian()
    dg = g["printed_digits"]
    assert _round_to(tau, dg["threshold"]) == g["threshold"]
    assert _round_to(a, dg["level_inner"]) == g["level_inner"]
    assert _round_to(b, dg["level_outer"]) == g["level_outer"]
    assert _round_to(mse, dg["mse"]) == g["mse"]


def test_lloyd_max_conditions_hold():
    tau, a, b, _ = oracle.lloyd_max_gaussian()
    pdf = lambda x: math.exp(-x * x / 2) / math.sqrt(2 * math.pi)
    num_a, _ = integrate.quad(lambda x: x * pdf(x), 0, tau)
    den_a, _ = integrate.quad(pdf, 0, tau)
    num_b, _ = integrate.quad(lambda x: x * pdf(x), tau, np.inf)
    den_b, _ = integrate.quad(pdf, tau, np.inf)
    assert abs(a - num_a / den_a) < 1e-10
    assert abs(b - num_b / den_b) < 1e-10
    assert abs(tau - 0.5 * (a + b)) < 1e-12


def test_lloyd_max_is_the_mse_minimiser():
    # Direct numeric minimisation of the integrated distortion over (tau, a, b).
    pdf = lambda x: math.exp(-x * x / 2) / math.sqrt(2 * math.pi)

    def distortion(p):
        t, a, b = p
        d1, _ = integrate.quad(lambda x: (x - a) ** 2 * pdf(x), 0, t)
        d2, _ = integrate.quad(lambda x: (x - b) ** 2 * pdf(x), t, np.inf)
        return 2 * (d1 + d2)

    res = optimize.minimize(distortion, x0=[1.2, 0.3, 1.3], method="Nelder-Mead",
                            options=dict(xatol=1e-9, fatol=1e-13, maxiter=4000))
    tau, a, b, mse = oracle.lloyd_max_gaussian()
    assert np.allclose(res.x, [tau, a, b], atol=2e-5)
    assert abs(res.fun - mse) < 1e-9
    assert abs(oracle.quantizer_mse(tau, a, b) - distortion([tau, a, b])) < 1e-10


def test_response_matches_pages_and_monte_carlo():
    g = _golden("quantizer_response.json")
    tau, a, b, _ = oracle.lloyd_max_gaussian()
    r = oracle.quantizer_response(tau, a, b)
    assert _round_to(r, g["printed_digits"]) == g["mse_optimal_response"]
    # The centroid condition gives E[xQ] = E[Q^2], so MSE = 1 - E[xQ].
    assert abs(r - (1 - oracle.quantizer_mse(tau, a, b))) < 1e-12
    # Monte Carlo E[x Q(x)] with an independent sampler.
    rng = np.random.default_rng(7)
    x = rng.standard_normal(4_000_000)
    q = np.where(x >= tau, b, np.where(x >= 0, a, np.where(x >= -tau, -a, -b)))
    assert abs(np.mean(x * q) - r) < 3e-3
    # Coupled gain restores unit response (kappa = 1).
    gain = oracle.coupled_gain(tau, a, b)
    assert abs(gain * r - g["coupled_response"]) < 1e-12
    assert abs(np.mean(x * gain * q) - 1.0) < 4e-3


def test_response_is_mse_optimal_gain_times_one():
    # d/dg MSE(g) = 0 at g* = E[xQ]/E[Q^2]; for Lloyd-Max g* = 1.
    tau, a, b, _ = oracle.lloyd_max_gaussian()
    gs = np.linspace(0.8, 1.2, 4001)
    mses = [oracle.quantizer_mse(tau, a, b, g) for g in gs]
    assert abs(gs[int(np.argmin(mses))] - 1.0) < 2e-4


def test_storage_accounting_matches_pages():
    g = _golden("storage_accounting.json")
    ds = g["deepseek_v2_lite"]
    bpt = oracle.bytes_per_token(ds["d_c"], ds["d_r"], ds["bits"], ds["group"])
    assert bpt == ds["bytes_per_token"]
    assert oracle.bf16_bytes_per_token(ds["d_c"], ds["d_r"]) == ds["bf16_bytes_per_token"]
    assert round(bpt * 8 / (ds["d_c"] + ds["d_r"]), 3) == ds["effective_bits"]
    ceiling = oracle.bf16_bytes_per_token() / oracle.bytes_per_token()
    assert round(ceiling, 3) == ds["capacity_ceiling"]
    # Components as itemised on the pages.
    assert ds["d_c"] * ds["bits"] / 8 == ds["code_bytes"]
    assert ds["d_c"] / ds["group"] * 2 * 4 == ds["meta_bytes"]
    assert ds["d_r"] * 2 == ds["rope_bytes"]
    mc = g["minicpm3"]
    assert oracle.bytes_per_token(mc["d_c"], mc["d_r"], mc["bits"], mc["group"]) == mc["bytes_per_token"]
    # The measured ratio sits below the arithmetic ceiling, and the measured
    # token capacities describe the same memory budget to within 1%.
    assert g["measured_capacity_ratio"] <= ceiling
    bf16_budget = g["measured_tokens_bf16"] * ds["bf16_bytes_per_token"]
    rlq_budget = g["measured_tokens_rlq"] * ds["bytes_per_token"]
    assert abs(bf16_budget / rlq_budget - 1) < 0.01


def test_storage_accounting_other_widths():
    # 4-bit codes at group 128: 256 + 32 + 128 bytes.
    assert oracle.bytes_per_token(bits=4) == 416
    # group 64 doubles the statistics: 128 + 64 + 128.
    assert oracle.bytes_per_token(group=64) == 320
