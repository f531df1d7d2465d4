"""fp64/int oracle: the two-micro-batch split of a flattened batch.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Follows the Ascend dual-stream article (Qwen3 dense), section 3.1 "data
split": one batch on the flattened token axis becomes two micro-batches.

  * split point, simple method: seq_split = batch_size // 2 and
    token_split = sum(query_lens[:seq_split]) (the batch size is read off
    query_lens, since the token axis merges batch and length);
  * split point, balanced method: aim at total_tokens // 2, walk query_lens
    keeping the running token count, take the sequence boundary whose count
    is nearest the aim; refuse the split (no dual stream) when the two
    micro-batches differ by more than balance_threshold relative to the
    smaller one, or when either is shorter than length_threshold;
  * per-field split: token-indexed fields (slot_mapping, the number of
    tokens, queries and outputs) at token_split; sequence-indexed fields
    (seq_lens, query_lens, block_table rows) at seq_split. The article also
    slices an explicit attention mask; this path has none (the causal mask
    follows from query_lens and seq_lens).

Readings where the section is silent:
  * a split needs two non-empty sequence ranges: seq_split in 1 .. S-1
    (the simple method with S < 2 gives no split);
  * "nearest": the smallest k in 1 .. S-1 minimising
    |sum(query_lens[:k]) - total // 2| (ties to the smaller k);
  * the micro-batch "lengths" the thresholds compare are their token counts;
    a zero-token micro-batch is infinitely unbalanced (refused).
"""
from __future__ import annotations

import numpy as np


def simple_split(query_lens) -> tuple[int, int] | None:
    """(seq_split, token_split) by batch_size // 2, or None if S < 2."""
    S = len(query_lens)
    k = S // 2
    if k < 1 or k > S - 1:
        return None
    return k, int(sum(int(q) for q in query_lens[:k]))


def balanced_split(query_lens, balance_threshold: float, length_threshold: int):
    """(seq_split, token_split) nearest total // 2, or None when refused."""
    S = len(query_lens)
    if S < 2:
        return None
    total = sum(int(q) for q in query_lens)
    aim = total // 2
    best = None
    cumu = 0
    for k in range(1, S):
        cumu += int(query_lens[k - 1])
        if best is None or abs(cumu - aim) < abs(best[1] - aim):
            best = (k, cumu)
    k, tsp = best
    n1, n2 = tsp, total - tsp
    if min(n1, n2) <= 0:
        return None
    if abs(n1 - n2) / min(n1, n2) > balance_threshold:
        return None
    if n1 < length_threshold or n2 < length_threshold:
        return None
    return k, tsp


def split_metadata(meta: dict, seq_split: int, token_split: int) -> tuple[dict, dict]:
    """Two micro-batch metadata dicts. Token-indexed keys: slot_mapping, q,
    out (leading axis = tokens); sequence-indexed: seq_lens, query_lens,
    block_table. num_tokens is recomputed."""
    token_keys = ("slot_mapping", "q", "k_new", "v_new", "out")
    seq_keys = ("seq_lens", "query_lens", "block_table")
    pre, post = {}, {}
    for key, val in meta.items():
        if key in token_keys:
            pre[key], post[key] = val[:token_split], val[token_split:]
        elif key in seq_keys:
            pre[key], post[key] = val[:seq_split], val[seq_split:]
        else:
            pre[key] = post[key] = val
    pre["num_tokens"] = int(np.sum(pre["query_lens"]))
    post["num_tokens"] = int(np.sum(post["query_lens"]))
    return pre, post
