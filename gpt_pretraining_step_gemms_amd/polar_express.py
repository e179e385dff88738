"""Polar Express coefficient schedule for Muon's Newton-Schulz iteration.

apidog.com, "Cara Melatih ChatGPT Sendiri dengan Budget 50 Dolar", section
"2. Pengoptimal Muon (nanochat/optim.py)", names the quintic iteration
"Polar Express" and prints the first two of its five (a, b, c) rows before
the listing breaks off.  The construction behind the name is published
(N. Amsel, D. Persson, C. Musco, R. M. Gower, "The Polar Express: Optimal
Matrix Sign Methods and Their Application to the Muon Algorithm", 2025):

* the singular values of X0 = M / ||M||_F lie in an interval [l, u]
  (l0 = 1e-3, u0 = 1);
* step i uses the odd quintic p(x) = a x + b x^3 + c x^5 that best
  approximates 1 in the max norm on that interval (Remez exchange on four
  alternation points), fitted on [max(l, floor * u), u] so that the first
  steps are not pulled towards the tiny l;
* p is rescaled so that p(l) + p(u) = 2 (centred on 1 over the whole
  interval), then slowed by a safety factor, p(x) -> p(x / (1 + safety)),
  which keeps bf16 rounding from pushing values past the fixed point;
* the next interval is [p(l), 2 - p(l)].

The floor and the safety factor are not printed.  They are taken here as
the values that bring the first row within rounding of the printed
(8.156, -22.483, 15.879): floor = 0.020075, safety = 0.019942 (a minimax fit
of those two numbers to that one row).  With them the second row comes out
as (4.0429, -2.8088, 0.5000), the printed (4.043, -2.809, 0.500) to every
printed digit, which checks the construction.  Rows three to five follow
from the same construction; the pages do not show them.

Host-side configuration data only: the library takes any table of rows.
"""

import numpy as np

L0 = 1e-3
FLOOR = 0.020075
SAFETY = 0.019942


def poly(a, b, c, x):
    return a * x + b * x ** 3 + c * x ** 5


def remez_odd_quintic(l, u, iters=100):
    """Odd quintic minimising max_{x in [l, u]} |1 - p(x)|, by Remez
    exchange: solve p(x_j) + s_j E = 1 on four alternation points with signs
    s = (+, -, +, -), move the two interior points to the extrema of p, repeat.
    Returns (a, b, c, E); |E| is the minimax error."""
    xs = np.array([l, l + (u - l) / 3, l + 2 * (u - l) / 3, u], dtype=np.float64)
    s = np.array([1.0, -1.0, 1.0, -1.0])
    for _ in range(iters):
        M = np.stack([xs, xs ** 3, xs ** 5, s], axis=1)
        a, b, c, E = np.linalg.solve(M, np.ones(4))
        # interior extrema: p'(x) = a + 3 b x^2 + 5 c x^4 = 0, a quadratic in x^2
        disc = 9 * b * b - 20 * a * c
        if disc < 0 or c == 0:
            break
        r2 = np.array([(-3 * b - np.sqrt(disc)) / (10 * c), (-3 * b + np.sqrt(disc)) / (10 * c)])
        r = np.sort(np.sqrt(r2[r2 > 0]))
        r = r[(r > l) & (r < u)]
        if r.size != 2:
            break
        new = np.array([l, r[0], r[1], u])
        if np.max(np.abs(new - xs)) <= 1e-15 * u:
            break
        xs = new
    return float(a), float(b), float(c), float(E)


def polar_express_table(n=5, l0=L0, floor=FLOOR, safety=SAFETY):
    """The n (a, b, c) rows of the schedule (see the module docstring)."""
    l, u = l0, 1.0
    rows = []
    for _ in range(n):
        a, b, c, _ = remez_odd_quintic(max(l, floor * u), u)
        k = 2.0 / (poly(a, b, c, l) + poly(a, b, c, u))
        a, b, c = a * k, b * k, c * k
        g = 1.0 + safety
        a, b, c = a / g, b / g ** 3, c / g ** 5
        rows.append((a, b, c))
        l = poly(a, b, c, l)
        u = 2.0 - l
    return rows
