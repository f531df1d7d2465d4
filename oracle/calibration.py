"""fp64 oracle: online calibration of the two-variable latency model.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Follows the vllm-ascend design "dynamic chunked pipeline parallel (CPP)",
section "online calibration": profiling only covers lengths up to the token
budget, so at run time the extended model

    f(C, H) = a * C * (C + H) + b * (C + H) + c

(C the chunk size, H the prefix history) is refitted by least squares from
what each executed batch records: the feature vector
[sum (C+H)*C, sum (C+H), N] over its N sequences and the measured time,
once enough points (5 to 30) have been collected. The section "runtime:
dynamic prediction" supplies the rest: an equal-latency target and the same
smoothing / alignment / caps as the one-variable predictor.

Readings where the section is silent:
  * the fitted model sums the per-sequence model over the batch, so the
    constant multiplies N: time ~ a*F0 + b*F1 + c*F2 with F = the features;
  * "5 to 30 points": refit after every record once at least min_points (5)
    are held, over the most recent window (30) records;
  * the columns are scaled by their largest magnitude in the window before
    the least-squares solve (a well-conditioned 3-column design);
  * a window that does not determine three coefficients (e.g. one chunk
    size throughout: C*(C+H) and C+H are then proportional, so a and b are
    confounded) is not fitted; the previous model stays;
  * the per-chunk target is T' = f(base, 0) = a*base^2 + b*base + c, the
    modelled latency of a base-size chunk without history; the next chunk
    at history H solves f(C, H) = T', i.e.
        a*C^2 + (a*H + b)*C + (b*H + c - T') = 0,
    positive root by the quadratic formula;
  * degenerate models: a <= 0 or a non-finite value -> C = (T' - b*H - c) /
    (a*H + b) when a*H + b > 0, else base; a negative discriminant -> base;
  * post-processing exactly as predictor.next_chunk (smooth, floor(x+1e-6),
    align down, min_chunk, caps).
"""
from __future__ import annotations

import math
from collections import deque

import numpy as np

from .predictor import EPS_FLOOR, PredictorConfig, _XI_CAP


def features(chunk_lens, hist_lens) -> tuple[float, float, float]:
    """[sum C*(C+H), sum (C+H), N] over the sequences with C > 0."""
    f0 = f1 = 0.0
    n = 0
    for C, H in zip(chunk_lens, hist_lens):
        if C <= 0:
            continue
        f0 += float(C) * float(C + H)
        f1 += float(C + H)
        n += 1
    return f0, f1, float(n)


def fit(feats, ms) -> tuple[float, float, float]:
    """Least squares (a, b, c) for ms ~ a*F0 + b*F1 + c*F2."""
    F = np.asarray(feats, dtype=np.float64).reshape(-1, 3)
    t = np.asarray(ms, dtype=np.float64).reshape(-1)
    if F.shape[0] != t.size or t.size < 3:
        raise ValueError("need at least 3 (features, ms) records")
    scale = np.max(np.abs(F), axis=0)
    if np.any(scale <= 0):
        raise ValueError("a feature column is all zero")
    coef, _, rank, _ = np.linalg.lstsq(F / scale, t, rcond=None)
    if rank < 3:
        raise ValueError("records do not determine three coefficients")
    coef = coef / scale
    return float(coef[0]), float(coef[1]), float(coef[2])


def target(a: float, b: float, c: float, base: int) -> float:
    """T' = f(base, 0) = a*base^2 + b*base + c."""
    return a * base * base + b * base + c


def raw_chunk(a: float, b: float, c: float, T: float, H: int, base: int) -> float:
    """Positive root C of a*C^2 + (a*H + b)*C + (b*H + c - T) = 0, or the
    stated fallback."""
    fin = all(math.isfinite(v) for v in (a, b, c, T))
    if a > 0 and fin:
        B = a * H + b
        K = b * H + c - T
        disc = B * B - 4.0 * a * K
        if disc >= 0.0:
            return (-B + math.sqrt(disc)) / (2.0 * a)
        return float(base)
    if fin:
        B = a * H + b
        if B > 0:
            return (T - b * H - c) / B
    return float(base)


def next_chunk(cfg: PredictorConfig, a: float, b: float, c: float, T: float,
               history_len: int, remaining: int) -> tuple[int, float]:
    """(chunk size, raw root) at prefix history_len under the 2-variable model."""
    base = cfg.base_chunk_size
    x = raw_chunk(a, b, c, T, history_len, base)
    s = cfg.smooth_factor
    xs = s * x + (1.0 - s) * base
    xf = xs + EPS_FLOOR
    if not xf >= 0.0:
        xi = 0
    elif xf >= _XI_CAP:
        xi = int(_XI_CAP)
    else:
        xi = int(math.floor(xf))
    xa = (xi // cfg.align) * cfg.align
    xa = max(xa, cfg.min_chunk)
    chunk = min(xa, cfg.max_chunk, cfg.max_model_len - history_len, remaining)
    return max(chunk, 0), x


class Calibrator:
    """Record window and refit policy of the online calibration."""

    def __init__(self, min_points: int = 5, window: int = 30):
        if min_points < 3 or window < min_points:
            raise ValueError("need 3 <= min_points <= window")
        self.min_points = min_points
        self.records: deque = deque(maxlen=window)
        self.coef: tuple[float, float, float] | None = None

    def record(self, feat, ms: float) -> bool:
        """Adds one batch; refits once min_points are held. True if a model
        is available afterwards."""
        self.records.append((tuple(float(v) for v in feat), float(ms)))
        if len(self.records) >= self.min_points:
            try:
                self.coef = fit([r[0] for r in self.records], [r[1] for r in self.records])
            except ValueError:
                pass  # the window does not determine the model: keep the last one
        return self.coef is not None
