"""fp64 oracle: the profiled chunk-size predictor.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Follows the vllm-ascend design "dynamic chunked pipeline parallel (CPP)":
  * section "quadratic latency model": f(l) = a*l^2 + b*l + c;
  * section "startup: profiling": 64 distinct chunk sizes sampled evenly
    from base_chunk_size down to near zero, each timed (ms), a least-squares
    fit of the quadratic, and a per-chunk target from base_chunk_size;
  * section "runtime: dynamic prediction": T = f(base) - f(0); solve
    f(L+x) - f(L) = T, i.e. a*x^2 + (2aL+b)*x - T = 0, by the quadratic
    formula (positive root); then smooth with smooth_factor, align down to a
    multiple of the page size (at least 64), and cap at
    max_model_len - history_len and at the scheduler's token cap.

Readings where that section is silent:
  * sample sizes: round(base - i*(base-lo)/(n-1)), i = 0..n-1 (2048..32
    in steps of exactly 32 for base 2048, lo 32, n 64);
  * smoothing: xs = s*x + (1-s)*base, s = smooth_factor (s = 1: none);
  * rounding x to tokens: floor(xs + 1e-6). The 1e-6 absorbs fp64 rounding
    of roots that are integers in exact arithmetic (at L = 0 the root is
    exactly base) and is far below one token;
  * the alignment quantum is a parameter (the page size by default);
  * order: smooth, floor, align down, raise to min_chunk, then cap at
    max_chunk, max_model_len - L and the tokens remaining in the prompt;
  * degenerate fits (a <= 0 or a non-finite coefficient): linear solve
    x = T/b when b > 0, else base;
  * a negative discriminant (only possible when T < 0): x = base.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

EPS_FLOOR = 1e-6
_XI_CAP = 9.0e15   # keeps float -> int conversion exact and finite


@dataclass(frozen=True)
class PredictorConfig:
    base_chunk_size: int = 2048
    align: int = 128
    min_chunk: int = 64
    max_chunk: int = 2048
    max_model_len: int = 32768
    smooth_factor: float = 1.0


def profile_sizes(base: int, n: int = 64, lo: int = 32) -> list[int]:
    """n distinct sizes evenly spaced from base down to lo."""
    return [int(round(base - i * (base - lo) / (n - 1))) for i in range(n)]


def fit_quadratic(lens, ms, base: float | None = None):
    """Least squares (a, b, c) for ms ~ a*l^2 + b*l + c.

    The columns are scaled by 1/base (l/base in [0, 1]) so the 3-column
    design is well conditioned; the solve is numpy's least-squares routine
    on that design, and the coefficients are unscaled afterwards.
    """
    l = np.asarray(lens, dtype=np.float64)
    t = np.asarray(ms, dtype=np.float64)
    if l.shape != t.shape or l.size < 3:
        raise ValueError("need at least 3 (size, ms) pairs")
    if base is None:
        base = float(np.max(np.abs(l))) or 1.0
    u = l / base
    design = np.stack([u * u, u, np.ones_like(u)], axis=1)
    coef, *_ = np.linalg.lstsq(design, t, rcond=None)
    return float(coef[0] / (base * base)), float(coef[1] / base), float(coef[2])


def latency(a: float, b: float, c: float, l: float) -> float:
    return a * l * l + b * l + c


def target(a: float, b: float, base: int) -> float:
    """T = f(base) - f(0) = a*base^2 + b*base (the constant cancels)."""
    return a * base * base + b * base


def raw_chunk(a: float, b: float, T: float, L: int, base: int) -> float:
    """Positive root x of a*x^2 + (2aL+b)*x - T = 0 (or the stated fallback)."""
    if a > 0 and math.isfinite(a) and math.isfinite(b) and math.isfinite(T):
        B = 2.0 * a * L + b
        disc = B * B + 4.0 * a * T
        if disc >= 0.0:
            return (-B + math.sqrt(disc)) / (2.0 * a)
        return float(base)
    if b > 0 and math.isfinite(b) and math.isfinite(T):
        return T / b
    return float(base)


def next_chunk(cfg: PredictorConfig, a: float, b: float, T: float,
               history_len: int, remaining: int) -> tuple[int, float]:
    """(chunk size, raw root x) for the next chunk at prefix history_len."""
    base = cfg.base_chunk_size
    x = raw_chunk(a, b, T, history_len, base)
    s = cfg.smooth_factor
    xs = s * x + (1.0 - s) * base
    xf = xs + EPS_FLOOR
    if not xf >= 0.0:          # negative or NaN
        xi = 0
    elif xf >= _XI_CAP:
        xi = int(_XI_CAP)
    else:
        xi = int(math.floor(xf))
    xa = (xi // cfg.align) * cfg.align
    xa = max(xa, cfg.min_chunk)
    chunk = min(xa, cfg.max_chunk, cfg.max_model_len - history_len, remaining)
    return max(chunk, 0), x


def schedule(cfg: PredictorConfig, a: float, b: float, T: float,
             prompt_len: int, history_len: int = 0):
    """Chunk walk over a prompt: list of (L, chunk, raw_x) until done."""
    out = []
    L = history_len
    end = history_len + prompt_len
    while L < end:
        chunk, x = next_chunk(cfg, a, b, T, L, end - L)
        if chunk <= 0:
            break
        out.append((L, chunk, x))
        L += chunk
    return out
