"""Oracle: the token-budget batch former of chunked prefill.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Follows the vLLM "Chunked-Prefills" article, section 3.1 (non-blocking
scheduling under a token budget): each step has a budget of tokens; decode
requests are scheduled first at one token each, then the unfinished
prefills take chunks of at most what remains of their prompt and of the
budget, and finally new requests are admitted, in order, while budget is
left. Section 3.2.2 and the vllm-ascend CPP design ("runtime: dynamic
prediction", step 1: the scheduler asks the predictor) supply the chunk
caps: a fixed size (512), the progressive sizes [2048, 1024, 512], or the
predictor's size for the prompt's current prefix.

Readings where the pages are silent:
  * one request = (prompt_len, max_new, arrival_step); it can be admitted
    from its arrival step on, in arrival order (ties by insertion order);
    decode rows and unfinished prefills are visited in admission order;
  * a request whose prompt finishes prefilling in a step becomes a decode
    request from the next step on; a decode row handles one new token at
    position prompt_len + generated (query_len 1, seq_len that + 1); the
    request finishes once max_new tokens were generated (max_new = 0: done
    when the prompt is prefilled);
  * the chunk of a prefill is min(remaining prompt, budget left, cap), where
    the cap is evaluated at the request's prefix L and remaining prompt; a
    cap of 0 schedules nothing for that request this step;
  * progressive sizes: the k-th chunk of a request is capped by
    sizes[min(k, len(sizes) - 1)];
  * the batch lists decode rows, then prefill chunks, in the order taken
    (that is also the order of the flattened token axis);
  * if the unfinished prefills stop early because the budget ran out, no
    new request is admitted in that step.
"""
from __future__ import annotations

from dataclasses import dataclass, field

from . import predictor as P
from . import calibration as CAL

RULE_FIXED, RULE_PROGRESSIVE, RULE_PREDICTOR, RULE_CALIBRATED = 0, 1, 2, 3


@dataclass
class Rule:
    kind: int = RULE_FIXED
    fixed: int = 512
    sizes: tuple = (2048, 1024, 512)
    cfg: P.PredictorConfig = field(default_factory=P.PredictorConfig)
    a: float = 0.0
    b: float = 0.0
    c: float = 0.0
    T: float = 0.0

    def cap(self, L: int, remaining: int, k: int) -> int:
        if self.kind == RULE_FIXED:
            return self.fixed
        if self.kind == RULE_PROGRESSIVE:
            return self.sizes[min(k, len(self.sizes) - 1)]
        if self.kind == RULE_PREDICTOR:
            return P.next_chunk(self.cfg, self.a, self.b, self.T, L, remaining)[0]
        return CAL.next_chunk(self.cfg, self.a, self.b, self.c, self.T, L, remaining)[0]


@dataclass
class Request:
    rid: int
    prompt_len: int
    max_new: int
    arrival: int
    prefilled: int = 0
    generated: int = 0
    chunks: int = 0
    admitted: bool = False

    @property
    def done(self) -> bool:
        return self.prefilled == self.prompt_len and self.generated >= self.max_new


class Scheduler:
    def __init__(self, budget: int, rule: Rule):
        if budget <= 0:
            raise ValueError("budget must be > 0")
        self.budget = budget
        self.rule = rule
        self.requests: list[Request] = []
        self.admitted: list[int] = []     # request ids in admission order
        self.step_no = 0
        self.pending: list | None = None

    def add(self, prompt_len: int, max_new: int, arrival: int = 0) -> int:
        if prompt_len <= 0 or max_new < 0:
            raise ValueError("need prompt_len > 0 and max_new >= 0")
        rid = len(self.requests)
        self.requests.append(Request(rid, prompt_len, max_new, arrival))
        return rid

    def form(self):
        """The batch of the current step: list of (rid, query_len, seq_len)."""
        left = self.budget
        batch = []
        live = [self.requests[i] for i in self.admitted if not self.requests[i].done]
        for r in live:                                   # decode rows first
            if r.prefilled == r.prompt_len and left > 0:
                pos = r.prompt_len + r.generated
                batch.append((r.rid, 1, pos + 1))
                left -= 1
        ran_out = False
        for r in live:                                   # unfinished prefills
            if r.prefilled < r.prompt_len:
                if left <= 0:
                    ran_out = True
                    break
                rem = r.prompt_len - r.prefilled
                chunk = min(rem, left, self.rule.cap(r.prefilled, rem, r.chunks))
                if chunk > 0:
                    batch.append((r.rid, chunk, r.prefilled + chunk))
                    left -= chunk
        if not ran_out:                                  # new requests, by arrival
            waiting = sorted((r for r in self.requests
                              if not r.admitted and r.arrival <= self.step_no),
                             key=lambda r: (r.arrival, r.rid))
            for r in waiting:
                if left <= 0:
                    break
                chunk = min(r.prompt_len, left, self.rule.cap(0, r.prompt_len, 0))
                if chunk <= 0:
                    break
                r.admitted = True
                self.admitted.append(r.rid)
                batch.append((r.rid, chunk, chunk))
                left -= chunk
        self.pending = batch
        return batch

    def commit(self):
        """Advance the requests by the formed batch, then the step counter."""
        assert self.pending is not None, "form() first"
        for rid, q, n in self.pending:
            r = self.requests[rid]
            if r.prefilled == r.prompt_len:              # decode row
                r.generated += 1
            else:
                r.prefilled += q
                r.chunks += 1
        self.pending = None
        self.step_no += 1

    def finished(self) -> bool:
        return all(r.done for r in self.requests)
