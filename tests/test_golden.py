"""Worked settings the pages print (tests/golden/*.json, each with its
citation), run through the oracle's token-budget batch former and through
the library's cpa_sched_* (host code, no GPU). The fixtures hold the
printed figures; where a figure follows from them by arithmetic (a chunk
count), the fixture says so."""
import json
import os

import pytest

from oracle import scheduler as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        d = json.load(f)
    assert d["citation"]
    return d


def run_oracle(budget, rule, requests):
    s = S.Scheduler(budget, rule)
    for p, m, t in requests:
        s.add(p, m, t)
    steps = []
    while not s.finished():
        steps.append(s.form())
        s.commit()
        assert len(steps) < 10000
    return steps


def run_library(cpa, cfg, requests):
    s = cpa.Sched(cfg)
    for p, m, t in requests:
        s.add(p, m, t)
    steps = []
    while not s.status()[0]:
        steps.append(s.form())
        s.commit()
        assert len(steps) < 10000
    return steps


@pytest.fixture(scope="module")
def cpa():
    from chunked_prefill_attention_slot_amd import binding
    return binding


def test_sixteen_prompts_fit_one_step(cpa):
    d = load("budget_16384_sixteen_prompts.json")
    rule = S.Rule(S.RULE_FIXED, fixed=d["fixed_chunk"])
    steps = run_oracle(d["budget"], rule, d["requests"])
    first = steps[0]
    pr = d["printed"]
    assert len(first) == pr["first_step_rows"] == 16
    assert sum(q for _, q, _ in first) == pr["first_step_tokens"] == 4096
    assert all(q == n == pr["chunk_of_each_prompt"] for _, q, n in first)
    # then one decode row per request per step until each has its 32 tokens
    assert all(len(b) == 16 and all(q == 1 for _, q, _ in b) for b in steps[1:])
    assert len(steps) == 1 + 32
    lib = run_library(cpa, cpa.sched_cfg(d["budget"], cpa.CPA_RULE_FIXED,
                                         fixed_chunk=d["fixed_chunk"]), d["requests"])
    assert lib == steps


def test_long_prompt_is_cut_into_budget_chunks(cpa):
    d = load("budget_320_long_prompt.json")
    rule = S.Rule(S.RULE_FIXED, fixed=d["fixed_chunk"])
    steps = run_oracle(d["budget"], rule, d["requests"])
    pr = d["printed"]
    chunks = [b[0][1] for b in steps if b and b[0][2] <= pr["prompt_tokens"]]
    assert len(chunks) == pr["prefill_chunks"] == pr["prompt_tokens"] // pr["chunk_tokens"]
    assert all(q == pr["chunk_tokens"] for q in chunks)
    assert [b[0][2] for b in steps[:3]] == [320, 640, 960]      # prefix grows one chunk a step
    assert steps[-1] == [(0, 1, pr["prompt_tokens"] + 1)]       # then the one decode row
    lib = run_library(cpa, cpa.sched_cfg(d["budget"], cpa.CPA_RULE_FIXED,
                                         fixed_chunk=d["fixed_chunk"]), d["requests"])
    assert lib == steps


def test_fixed_and_progressive_chunks_of_one_prompt(cpa):
    d = load("budget_2048_chunk_512.json")
    (p, m, t), = d["requests"]
    for rule, cfg, want in (
            (S.Rule(S.RULE_FIXED, fixed=512),
             cpa.sched_cfg(d["budget"], cpa.CPA_RULE_FIXED, fixed_chunk=512),
             d["fixed_chunks"]),
            (S.Rule(S.RULE_PROGRESSIVE, sizes=tuple(d["progressive_sizes"])),
             cpa.sched_cfg(d["budget"], cpa.CPA_RULE_PROGRESSIVE,
                           sizes=tuple(d["progressive_sizes"])),
             d["progressive_chunks"])):
        steps = run_oracle(d["budget"], rule, d["requests"])
        chunks = [b[0][1] for b in steps if b and b[0][2] <= p]
        assert chunks == want and sum(want) == p
        assert steps[-1] == [(0, 1, p + 1)]
        assert run_library(cpa, cfg, d["requests"]) == steps
