"""fp64 oracle: paged chunked-prefill self-attention.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is computed (vLLM "Chunked-Prefills" article, section 3.2.1, chunked
attention): the chunk's queries attend over the concatenation of the cached
keys/values and the chunk's own, scores = Q.K^T times a scale, softmax over
keys, weighted sum of values. Readings where that passage is silent or
garbled:
  * causal: the query at absolute position H+i (H = prefix length) sees keys
    0..H+i and nothing after (the dynamic-chunking design's O(n^2)
    self-attention cost; the printed pseudocode has no mask);
  * scale = 1/sqrt(head_dim) (the printed sqrt(H) uses the hidden size);
  * GQA: query head h uses KV head h // (Hq/Hkv) (contiguous groups);
  * metadata as in the Ascend dual-stream article, section 3.1: seq_lens
    include this step's tokens, so H = seq_len - query_len; tokens of all
    sequences are concatenated in order; block_table maps logical page
    j // P of a sequence to a physical page of the cache [NB, Hkv, P, d].
The result has a plain definition, so this module writes the definition out:
per (sequence, query head) one dense score matrix, masked, softmaxed in
fp64, times V. bf16 inputs are widened exactly to fp64.
"""
from __future__ import annotations

import numpy as np


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def gather_sequence(cache_bits: np.ndarray, block_row: np.ndarray, n: int,
                    page_size: int) -> np.ndarray:
    """Logical positions 0..n-1 of one sequence out of a paged cache.

    cache [NB, Hkv, P, d]; position j lives in physical page
    block_row[j // P] at offset j % P. Returns [n, Hkv, d] bits.
    """
    j = np.arange(n)
    phys = np.asarray(block_row)[j // page_size]
    return cache_bits[phys, :, j % page_size, :]


def causal_chunk_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                           hist: int, scale: float,
                           return_lse: bool = False):
    """One head: q [C, d] at absolute positions hist..hist+C-1; k, v [n, d]
    with n >= hist + C. Row i sees keys 0..hist+i. fp64 throughout."""
    C = q.shape[0]
    n = k.shape[0]
    scores = (q @ k.T) * scale                     # [C, n]
    visible = np.arange(n)[None, :] <= (hist + np.arange(C))[:, None]
    scores = np.where(visible, scores, -np.inf)
    m = scores.max(axis=1, keepdims=True)
    w = np.exp(scores - m)
    z = w.sum(axis=1, keepdims=True)
    out = (w @ v) / z
    if return_lse:
        return out, (m + np.log(z))[:, 0]
    return out


def paged_attention(q_bits: np.ndarray, k_cache_bits: np.ndarray,
                    v_cache_bits: np.ndarray, block_table: np.ndarray,
                    query_lens, seq_lens, num_kv_heads: int, page_size: int,
                    scale: float | None = None,
                    rows: dict | None = None) -> np.ndarray:
    """All query tokens of a flattened batch; returns out [T, Hq, d] fp64.

    q [T, Hq, d] bits; caches [NB, Hkv, P, d] bits already holding every
    visible key (prefix and this step's tokens). `rows`, if given, maps a
    sequence index to the list of its query rows (0-based within the chunk)
    to compute; other outputs stay NaN. That is how large workloads are
    checked on samples.
    """
    T, Hq, d = q_bits.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    G = Hq // num_kv_heads
    out = np.full((T, Hq, d), np.nan)
    t0 = 0
    for s, (ql, n) in enumerate(zip(query_lens, seq_lens)):
        ql, n = int(ql), int(n)
        hist = n - ql
        sel = None if rows is None else rows.get(s)
        if ql > 0 and (rows is None or sel):
            k = widen_bf16(gather_sequence(k_cache_bits, block_table[s], n, page_size))
            v = widen_bf16(gather_sequence(v_cache_bits, block_table[s], n, page_size))
            qs = widen_bf16(q_bits[t0:t0 + ql])
            for h in range(Hq):
                g = h // G
                if sel is None:
                    out[t0:t0 + ql, h] = causal_chunk_attention(
                        qs[:, h], k[:, g], v[:, g], hist, scale)
                else:
                    for i in sel:
                        # one row at absolute position hist+i sees hist+i+1 keys
                        out[t0 + i, h] = causal_chunk_attention(
                            qs[i:i + 1, h], k[:hist + i + 1, g],
                            v[:hist + i + 1, g], hist + i, scale)[0]
        t0 += ql
    return out


def paged_attention_rowloop(q_bits, k_cache_bits, v_cache_bits, block_table,
                            query_lens, seq_lens, num_kv_heads, page_size,
                            scale=None) -> np.ndarray:
    """The same definition as paged_attention, one scalar at a time.

    For tiny shapes only: every score, max, exponential and weighted sum is
    an explicit Python loop over fp64 scalars, so it can be read against the
    definition directly.
    """
    T, Hq, d = q_bits.shape
    if scale is None:
        scale = 1.0 / float(np.sqrt(d))
    G = Hq // num_kv_heads
    q = widen_bf16(q_bits)
    out = np.zeros((T, Hq, d))
    t0 = 0
    for s in range(len(query_lens)):
        ql, n = int(query_lens[s]), int(seq_lens[s])
        hist = n - ql
        for i in range(ql):
            p = hist + i
            for h in range(Hq):
                g = h // G
                z = []
                for j in range(p + 1):
                    blk = int(block_table[s][j // page_size])
                    kj = widen_bf16(k_cache_bits[blk, g, j % page_size])
                    acc = 0.0
                    for e in range(d):
                        acc += float(q[t0 + i, h, e]) * float(kj[e])
                    z.append(acc * scale)
                m = max(z)
                w = [float(np.exp(x - m)) for x in z]
                tot = sum(w)
                for j in range(p + 1):
                    blk = int(block_table[s][j // page_size])
                    vj = widen_bf16(v_cache_bits[blk, g, j % page_size])
                    out[t0 + i, h] += (w[j] / tot) * vj
        t0 += ql
    return out
