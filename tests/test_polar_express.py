"""Pins of the Polar Express schedule (CPU only): the printed rows, the
minimax property of every step, and what the composed schedule does to
singular values."""

import os

import numpy as np
import pytest
from scipy.optimize import linprog

import oracle
from gpt_pretraining_step_gemms_amd import polar_express as pe
from gpt_pretraining_step_gemms_amd.configs import NS_POLAR_EXPRESS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def printed_rows():
    rows = []
    for line in open(os.path.join(GOLDEN, "polar_express_rows.txt")):
        if line.strip() and not line.startswith("#"):
            rows.append(np.array([float(x) for x in line.split()]))
    return rows


def test_first_two_rows_match_the_printed_rows_to_their_digits():
    # printed with three decimals: within half a unit of the last digit
    table = pe.polar_express_table()
    for got, want in zip(table[:2], printed_rows()):
        assert np.max(np.abs(np.array(got) - want)) < 5e-4, (got, want)
    assert NS_POLAR_EXPRESS == table and len(table) == 5


def test_remez_step_matches_a_linear_program_on_a_grid():
    # the minimax quintic found another way: minimise t subject to
    # |1 - p(x_j)| <= t on 4001 points of [l, u]
    for l, u in [(0.02, 1.0), (0.3, 1.7), (0.85, 1.15)]:
        a, b, c, E = pe.remez_odd_quintic(l, u)
        x = np.linspace(l, u, 4001)
        V = np.stack([x, x ** 3, x ** 5], 1)
        A = np.block([[V, -np.ones((x.size, 1))], [-V, -np.ones((x.size, 1))]])
        rhs = np.concatenate([np.ones(x.size), -np.ones(x.size)])
        res = linprog([0, 0, 0, 1], A_ub=A, b_ub=rhs, bounds=[(None, None)] * 4, method="highs")
        assert res.status == 0
        np.testing.assert_allclose([a, b, c], res.x[:3], rtol=2e-4, atol=2e-4 * abs(a))
        assert abs(abs(E) - res.x[3]) < 1e-6 * max(1.0, abs(E))


def test_every_step_equioscillates():
    l, u = pe.L0, 1.0
    for a, b, c in NS_POLAR_EXPRESS:
        lo = max(l, pe.FLOOR * u)
        a0, b0, c0, E = pe.remez_odd_quintic(lo, u)
        x = np.linspace(lo, u, 200001)
        err = 1 - pe.poly(a0, b0, c0, x)
        assert np.max(np.abs(err)) <= abs(E) * (1 + 1e-9)
        # four alternating extrema of size |E|: the two ends and two interior points
        ext = [err[0], err[np.argmin(err)], err[np.argmax(err[1:-1]) + 1], err[-1]]
        assert abs(err[0] - E) < 1e-12 and abs(err[-1] + E) < 1e-12
        assert abs(np.min(err) + abs(E)) < 1e-9 and abs(np.max(err) - abs(E)) < 1e-9
        assert np.all(np.abs(np.abs(ext) - abs(E)) < 1e-9)
        # the rows are the recentred, slowed copies of these polynomials
        k = 2.0 / (pe.poly(a0, b0, c0, l) + pe.poly(a0, b0, c0, u))
        g = 1 + pe.SAFETY
        np.testing.assert_allclose([a, b, c], [a0 * k / g, b0 * k / g ** 3, c0 * k / g ** 5],
                                   rtol=1e-14)
        l = pe.poly(a, b, c, l)
        u = 2 - l


def test_composed_schedule_maps_singular_values_near_one():
    s = np.geomspace(pe.L0, 1.0, 100001)
    l, u = pe.L0, 1.0
    for a, b, c in NS_POLAR_EXPRESS:
        s = pe.poly(a, b, c, s)
        l = pe.poly(a, b, c, l)
        u = 2 - l
        assert s.min() >= l - 1e-12 and s.max() <= u + 1e-12    # stays in the tracked interval
    assert s.min() > 0.84 and s.max() < 1.15


@pytest.mark.parametrize("shape", [(16, 16), (12, 40), (40, 12)])
def test_oracle_newton_schulz_with_the_schedule_acts_on_singular_values(shape):
    rng = np.random.default_rng(3 + shape[0])
    M = rng.standard_normal(shape)
    X = oracle.newton_schulz(M, NS_POLAR_EXPRESS, eps=1e-7)
    U, s, Vt = np.linalg.svd(M, full_matrices=False)
    s = s / (np.linalg.norm(M) + 1e-7)
    for a, b, c in NS_POLAR_EXPRESS:
        s = a * s + b * s ** 3 + c * s ** 5
    np.testing.assert_allclose(X, (U * s) @ Vt, atol=1e-10)
