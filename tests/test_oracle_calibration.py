"""Pins of oracle/calibration.py (the online two-variable latency model of the
CPP design, section "online calibration"), each against something other than
the oracle's own formulas: exact recovery from noise-free data, an
independent least-squares route, the one-variable fit it must reduce to, the
root's defining equation checked in exact rational arithmetic, and the
window policy."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import calibration as cal
from oracle.predictor import PredictorConfig, fit_quadratic


def synth(rng, n, a, b, c, noise=0.0):
    feats, ms = [], []
    for _ in range(n):
        N = int(rng.integers(1, 5))
        C = rng.integers(16, 2048, N)
        H = rng.integers(0, 30000, N)
        f = cal.features(C, H)
        t = sum(a * x * (x + h) + b * (x + h) + c for x, h in zip(C.astype(float), H.astype(float)))
        feats.append(f)
        ms.append(t + (rng.normal(0, noise) if noise else 0.0))
    return feats, ms


def test_features_by_hand():
    # chunk 3 at history 5, chunk 0 (skipped), chunk 2 at history 0
    assert cal.features([3, 0, 2], [5, 9, 0]) == (3 * 8 + 2 * 2, 8 + 2, 2.0)


@pytest.mark.parametrize("seed", range(6))
def test_fit_recovers_noise_free_model(seed):
    rng = np.random.default_rng(seed)
    a, b, c = 10 ** rng.uniform(-9, -6), 10 ** rng.uniform(-5, -3), rng.uniform(0.01, 0.5)
    feats, ms = synth(rng, 30, a, b, c)
    ga, gb, gc = cal.fit(feats, ms)
    assert ga == pytest.approx(a, rel=1e-9)
    assert gb == pytest.approx(b, rel=1e-9)
    assert gc == pytest.approx(c, rel=1e-9)


def test_fit_matches_normal_equations():
    # An independent route: the normal equations solved in exact rationals.
    rng = np.random.default_rng(11)
    feats, ms = synth(rng, 12, 2e-8, 3e-4, 0.05, noise=0.01)
    F = [[Fraction(v) for v in f] for f in feats]
    t = [Fraction(v) for v in ms]
    A = [[sum(F[k][i] * F[k][j] for k in range(len(F))) for j in range(3)] for i in range(3)]
    y = [sum(F[k][i] * t[k] for k in range(len(F))) for i in range(3)]
    # Gauss-Jordan in exact arithmetic
    M = [row[:] + [y[i]] for i, row in enumerate(A)]
    for col in range(3):
        piv = next(r for r in range(col, 3) if M[r][col] != 0)
        M[col], M[piv] = M[piv], M[col]
        for r in range(3):
            if r != col:
                f = M[r][col] / M[col][col]
                M[r] = [M[r][k] - f * M[col][k] for k in range(4)]
    exact = [float(M[i][3] / M[i][i]) for i in range(3)]
    got = cal.fit(feats, ms)
    for g, e in zip(got, exact):
        assert g == pytest.approx(e, rel=1e-8)


def test_reduces_to_one_variable_fit_without_history():
    # H = 0 and one sequence per batch: F = (C^2, C, 1), the 1-D design.
    rng = np.random.default_rng(3)
    C = np.arange(2048, 0, -32)
    ms = 3e-7 * C * C + 2e-4 * C + 0.02 + rng.normal(0, 1e-3, C.size)
    two = cal.fit([cal.features([x], [0]) for x in C], ms)
    one = fit_quadratic(C, ms)
    for g, e in zip(two, one):
        assert g == pytest.approx(e, rel=1e-9, abs=1e-15)


def test_root_solves_the_model_equation_exactly():
    a, b, c = 1.3e-7, 4.1e-4, 0.07
    base = 2048
    T = cal.target(a, b, c, base)
    for H in (0, 1, 777, 4096, 30000):
        x = cal.raw_chunk(a, b, c, T, H, base)
        # f(x, H) - T' in exact arithmetic at the fp64 root: tiny relative to T'
        fa, fb, fc, fx, fH, fT = map(Fraction, (a, b, c, x, H, T))
        resid = fa * fx * (fx + fH) + fb * (fx + fH) + fc - fT
        assert abs(float(resid)) <= 1e-9 * T
        # positive exactly when the history alone costs less than T'
        assert (x > 0) == (b * H + c < T)


def test_root_at_zero_history_is_base():
    cfg = PredictorConfig()
    for a, b, c in [(1e-6, 1e-3, 0.0), (1.234e-7, 7.77e-4, 0.3), (5e-9, 1e-2, 2.0)]:
        T = cal.target(a, b, c, cfg.base_chunk_size)
        chunk, x = cal.next_chunk(cfg, a, b, c, T, 0, 1 << 20)
        assert x == pytest.approx(2048.0, rel=1e-12)
        assert chunk == 2048


def test_chunk_shrinks_with_history():
    cfg = PredictorConfig(align=16)
    a, b, c = 2e-7, 3e-4, 0.05
    T = cal.target(a, b, c, cfg.base_chunk_size)
    prev = None
    for H in range(0, 32768, 512):
        x = cal.raw_chunk(a, b, c, T, H, cfg.base_chunk_size)
        if prev is not None:
            assert x <= prev
        prev = x


def test_degenerate_models():
    base = 2048
    # a = 0: linear solve (T - bH - c) / b
    assert cal.raw_chunk(0.0, 2e-3, 0.1, 4.196, 100, base) == pytest.approx((4.196 - 0.2 - 0.1) / 2e-3)
    # a < 0 and a*H + b <= 0: base
    assert cal.raw_chunk(-1.0, 1e-3, 0.0, 1.0, 10, base) == base
    # non-finite: base
    assert cal.raw_chunk(float("nan"), 1e-3, 0.0, 1.0, 10, base) == base
    # history alone exceeds the target: negative root -> min_chunk after clamps
    cfg = PredictorConfig()
    chunk, x = cal.next_chunk(cfg, 1e-7, 1e-3, 5.0, 0.01, 30000, 10000)
    assert x < 0 and chunk == cfg.min_chunk


def test_calibrator_window_and_threshold():
    rng = np.random.default_rng(5)
    calib = cal.Calibrator(min_points=5, window=30)
    fa, ma = synth(rng, 10, 9e-7, 1e-3, 0.5)     # an old regime
    fb, mb = synth(rng, 30, 2e-8, 4e-4, 0.05)    # the current one
    for i, (f, m) in enumerate(zip(fa[:4], ma[:4])):
        assert calib.record(f, m) is False
    assert calib.record(fa[4], ma[4]) is True
    for f, m in zip(fa[5:] + fb, ma[5:] + mb):
        calib.record(f, m)
    a, b, c = calib.coef
    assert a == pytest.approx(2e-8, rel=1e-9)
    assert b == pytest.approx(4e-4, rel=1e-9)
    assert c == pytest.approx(0.05, rel=1e-9)


def test_constant_chunk_size_does_not_determine_the_model():
    # C fixed: C*(C+H) = C * (C+H), the first two columns are proportional.
    feats = [cal.features([1024], [h]) for h in range(0, 10240, 1024)]
    ms = [1e-7 * f[0] + 1e-3 * f[1] + 0.1 for f in feats]
    with pytest.raises(ValueError):
        cal.fit(feats, ms)
    calib = cal.Calibrator(min_points=5, window=30)
    good = [cal.features([c], [h]) for c, h in [(64, 0), (2048, 0), (512, 4096), (128, 9000), (1000, 20000)]]
    for f in good:
        calib.record(f, 2e-8 * f[0] + 3e-4 * f[1] + 0.02)
    before = calib.coef
    # a window holding only the constant-size records cannot be fitted
    small = cal.Calibrator(min_points=5, window=5)
    for f, m in zip(feats, ms):
        assert small.record(f, m) is False
    assert calib.coef == before
