"""Pins of oracle/scheduler.py (token-budget batch former of the vLLM
Chunked-Prefills article, section 3.1, with the chunk caps of its section
3.2.2 and of the CPP design's runtime phase): a hand-worked request stream,
invariants over random streams, the progressive sizes, and the single-prompt
walk that must equal the predictor's own schedule."""
import numpy as np
import pytest

from oracle import predictor as P
from oracle import scheduler as S


def run(sched, max_steps=10000):
    steps = []
    while not sched.finished():
        steps.append(sched.form())
        sched.commit()
        assert len(steps) < max_steps
    return steps


def test_hand_worked_stream():
    s = S.Scheduler(512, S.Rule(S.RULE_FIXED, fixed=512))
    a = s.add(1000, 2)
    b = s.add(300, 1)
    assert run(s) == [
        [(a, 512, 512)],                      # A's first chunk uses the whole budget
        [(a, 488, 1000), (b, 24, 24)],        # A finishes its prompt, B is admitted with 24
        [(a, 1, 1001), (b, 276, 300)],        # decode row first, then B's rest
        [(a, 1, 1002), (b, 1, 301)],          # two decode rows; A and B then done
    ]


def test_arrival_order_and_late_arrivals():
    s = S.Scheduler(100, S.Rule(S.RULE_FIXED, fixed=64))
    a = s.add(50, 0, arrival=2)
    b = s.add(50, 0, arrival=0)
    steps = run(s)
    assert steps[0] == [(b, 50, 50)]
    assert steps[1] == []
    assert steps[2] == [(a, 50, 50)]


@pytest.mark.parametrize("seed", range(8))
def test_invariants_on_random_streams(seed):
    rng = np.random.default_rng(seed)
    budget = int(rng.choice([256, 512, 2048]))
    kind = seed % 3
    rule = S.Rule(kind, fixed=int(rng.choice([128, 512])), cfg=P.PredictorConfig(align=16),
                  a=1e-7, b=1e-3, T=P.target(1e-7, 1e-3, 2048))
    if kind == S.RULE_PROGRESSIVE:
        rule.sizes = (2048, 1024, 512)
    s = S.Scheduler(budget, rule)
    reqs = [(int(rng.integers(1, 6000)), int(rng.integers(0, 20)), int(rng.integers(0, 30)))
            for _ in range(int(rng.integers(1, 12)))]
    for p, m, t in reqs:
        s.add(p, m, t)
    prefilled = [0] * len(reqs)
    generated = [0] * len(reqs)
    admitted_at = {}
    for step_no, batch in enumerate(run(s)):
        assert sum(q for _, q, _ in batch) <= budget
        kinds = []
        for rid, q, n in batch:
            p, m, t = reqs[rid]
            assert step_no >= t
            if prefilled[rid] == p:                     # decode row
                assert q == 1 and n == p + generated[rid] + 1
                generated[rid] += 1
                kinds.append(0)
            else:
                assert n == prefilled[rid] + q and 0 < q <= p - prefilled[rid]
                admitted_at.setdefault(rid, step_no)
                prefilled[rid] += q
                kinds.append(1)
        assert kinds == sorted(kinds)                    # decode rows first
    assert prefilled == [p for p, _, _ in reqs]
    assert generated == [m for _, m, _ in reqs]
    # admission follows arrival order (ties by insertion order)
    assert s.admitted == sorted(s.admitted, key=lambda r: (reqs[r][2], r))
    assert sorted(s.admitted) == list(range(len(reqs)))


def test_progressive_sizes():
    s = S.Scheduler(1 << 20, S.Rule(S.RULE_PROGRESSIVE, sizes=(2048, 1024, 512)))
    s.add(5000, 0)
    assert [b[0][1] for b in run(s)] == [2048, 1024, 512, 512, 512, 392]


def test_predictor_rule_walk_equals_predictor_schedule():
    cfg = P.PredictorConfig()
    a, b = 1e-6, 1e-3
    T = P.target(a, b, 2048)
    s = S.Scheduler(1 << 20, S.Rule(S.RULE_PREDICTOR, cfg=cfg, a=a, b=b, T=T))
    s.add(32768, 0)
    got = [(batch[0][2] - batch[0][1], batch[0][1]) for batch in run(s)]
    exp = [(L, c) for L, c, _ in P.schedule(cfg, a, b, T, 32768)]
    assert got == exp


def test_unlimited_budget_prefills_everything_at_once():
    s = S.Scheduler(1 << 20, S.Rule(S.RULE_FIXED, fixed=1 << 20))
    ids = [s.add(p, 1) for p in (10, 5000, 77)]
    steps = run(s)
    assert steps[0] == [(ids[0], 10, 10), (ids[1], 5000, 5000), (ids[2], 77, 77)]
    assert steps[1] == [(ids[0], 1, 11), (ids[1], 1, 5001), (ids[2], 1, 78)]
    assert len(steps) == 2
