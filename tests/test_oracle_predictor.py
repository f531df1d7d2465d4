"""Pins for the predictor oracle.

  * exact rational arithmetic: floor(x + eps) of the positive root is found
    by integer search on the quadratic with fractions.Fraction (no floating
    point, no quadratic formula), and must equal the oracle's;
  * closed forms: L = 0 returns base; f(L+x) - f(L) = T for the raw root;
    as a -> 0+ the root tends to T/b; T = f(base) - f(0);
  * the fit recovers noise-free coefficients and satisfies the normal
    equations (residual orthogonal to the design) on noisy data;
  * invariants of the post-processing: alignment, minimum, clamps,
    non-increasing chunk size in L, the walk covers the prompt exactly.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle.predictor import (EPS_FLOOR, PredictorConfig, fit_quadratic,
                              latency, next_chunk, profile_sizes, raw_chunk,
                              schedule, target)

CFG = PredictorConfig()  # 2048 base, align 128, min 64, max 2048, 32768


def test_profile_sizes_are_2048_down_to_32_by_32():
    s = profile_sizes(2048, 64, 32)
    assert s == [2048 - 32 * i for i in range(64)]
    assert len(set(s)) == 64


def test_fit_recovers_noise_free_quadratic():
    a, b, c = 3.2e-7, 4.1e-3, 0.37
    l = np.array(profile_sizes(2048), dtype=float)
    t = a * l * l + b * l + c
    fa, fb, fc = fit_quadratic(l, t)
    assert abs(fa - a) <= 1e-9 * a
    assert abs(fb - b) <= 1e-9 * b
    assert abs(fc - c) <= 1e-9 * c


def test_fit_satisfies_normal_equations():
    rng = np.random.default_rng(0)
    l = np.array(profile_sizes(2048), dtype=float)
    t = 1e-6 * l * l + 2e-3 * l + 0.5 + rng.normal(0, 0.05, l.size)
    a, b, c = fit_quadratic(l, t)
    r = t - (a * l * l + b * l + c)
    u = l / 2048.0
    for col in (u * u, u, np.ones_like(u)):
        assert abs(float(col @ r)) <= 1e-9 * float(np.abs(col) @ np.abs(t))


def test_target_is_f_base_minus_f_zero():
    a, b, c = 1e-6, 1e-3, 0.25
    assert math.isclose(target(a, b, 2048), latency(a, b, c, 2048) - latency(a, b, c, 0),
                        rel_tol=1e-15)
    assert math.isclose(target(a, b, 2048), 6.242304, rel_tol=1e-15)


def _exact_floor(a, b, T, L):
    """max integer k with q(k - eps) <= 0, q(y) = a*y^2 + (2aL+b)*y - T, in
    exact rationals; equals floor(x + eps) for the positive root x."""
    A, Bf, Tq = Fraction(a), 2 * Fraction(a) * L + Fraction(b), Fraction(T)
    eps = Fraction(EPS_FLOOR)

    def q(y):
        return A * y * y + Bf * y - Tq

    k = max(0, int(raw_chunk(a, b, T, L, 2048)))  # start near the root
    while q(k - eps) <= 0:
        k += 1
    while k > 0 and q(k - eps) > 0:
        k -= 1
    x_exact_plus_eps_near_int = abs(float(q(Fraction(k + 1) - eps))) < 1e-18
    return k, x_exact_plus_eps_near_int


@pytest.mark.parametrize("seed", range(6))
def test_root_floor_matches_exact_rational(seed):
    rng = np.random.default_rng(seed)
    for _ in range(60):
        a = float(10 ** rng.uniform(-8, -5))
        b = float(10 ** rng.uniform(-4, -2))
        T = target(a, b, 2048)
        L = int(rng.integers(0, 32768))
        x = raw_chunk(a, b, T, L, 2048)
        k, tie = _exact_floor(a, b, T, L)
        if tie:
            continue
        assert int(math.floor(x + EPS_FLOOR)) == k


def test_root_closes_the_latency_equation():
    for a in (1e-8, 3e-7, 1e-6, 1e-5):
        for b in (0.0, 1e-4, 1e-3, 1e-2):
            T = target(a, b, 2048)
            for L in (0, 100, 2048, 9999, 30000):
                x = raw_chunk(a, b, T, L, 2048)
                lhs = latency(a, b, 0.0, L + x) - latency(a, b, 0.0, L)
                assert math.isclose(lhs, T, rel_tol=1e-9)


def test_zero_history_returns_base():
    for a in (1e-8, 1e-6, 1e-5):
        for b in (0.0, 1e-4, 1e-2):
            T = target(a, b, 2048)
            chunk, x = next_chunk(CFG, a, b, T, 0, 1 << 20)
            assert chunk == 2048
            assert abs(x - 2048) < 1e-9


def test_small_a_limit_is_linear():
    b = 1e-3
    T = target(1e-14, b, 2048)
    x = raw_chunk(1e-14, b, T, 5000, 2048)
    assert math.isclose(x, T / (2e-14 * 5000 + b), rel_tol=1e-4)
    # a <= 0 (degenerate fit): linear solve T/b
    assert raw_chunk(0.0, b, 2.048, 5000, 2048) == 2.048 / b
    assert raw_chunk(-1e-9, 0.0, 2.0, 10, 2048) == 2048.0


def test_worked_walk_first_chunks():
    """a=1e-6, b=1e-3 (ms): T = 6.242304 ms; at L=2048 the root is 1020.56...
    and aligns down to 896; the next prefix 2944 gives 810.8... -> 768."""
    a, b = 1e-6, 1e-3
    T = target(a, b, 2048)
    c1, x1 = next_chunk(CFG, a, b, T, 2048, 1 << 20)
    assert c1 == 896 and 1020.5 < x1 < 1020.6
    c2, x2 = next_chunk(CFG, a, b, T, 2944, 1 << 20)
    assert c2 == 768 and 810.8 < x2 < 810.9


def test_post_processing_invariants():
    rng = np.random.default_rng(3)
    for _ in range(300):
        a = float(10 ** rng.uniform(-9, -5))
        b = float(10 ** rng.uniform(-5, -2))
        T = target(a, b, 2048)
        L = int(rng.integers(0, 32768))
        rem = int(rng.integers(1, 40000))
        chunk, _ = next_chunk(CFG, a, b, T, L, rem)
        caps = min(2048, 32768 - L, rem)
        assert 0 < chunk <= caps
        assert chunk % 128 == 0 or chunk == 64 or chunk == caps


def test_chunks_non_increasing_and_walk_covers_prompt():
    a, b = 5e-7, 2e-3
    T = target(a, b, 2048)
    walk = schedule(CFG, a, b, T, 32768)
    assert sum(c for _, c, _ in walk) == 32768
    Ls = [L for L, _, _ in walk]
    assert Ls == sorted(Ls) and Ls[0] == 0
    sizes = [c for _, c, _ in walk[:-1]]
    assert all(x >= y for x, y in zip(sizes, sizes[1:]))


def test_smoothing_blends_with_base():
    cfg = PredictorConfig(smooth_factor=0.5, align=1, min_chunk=1)
    a, b = 1e-6, 1e-3
    T = target(a, b, 2048)
    chunk, x = next_chunk(cfg, a, b, T, 2048, 1 << 20)
    assert chunk == math.floor(0.5 * x + 0.5 * 2048 + EPS_FLOOR)
