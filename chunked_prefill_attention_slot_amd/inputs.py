"""Seeded synthetic inputs for paged chunked-prefill attention.

This module draws random numbers and lays them out; it holds none of the
attention, KV-write or predictor arithmetic. The HIP path's tests and bench
and the fp64 oracle's tests all take their inputs from here, so both sides
see the same bf16 bit patterns.

Layouts (the metadata fields of the Ascend dual-stream article, section 3.1
"data split": slot_mapping, seq_lens, query_lens, block_table):
  q            [T, Hq, d]            bf16 bits (uint16)
  k_new, v_new [T, Hkv, d]           bf16 bits: the chunk's own keys/values
  k_cache,     [NB, Hkv, P, d]       bf16 bits: paged cache holding every
  v_cache                            sequence's prefix (positions < H);
                                     all other slots hold a sentinel
  block_table  [S, max_blocks] int32 physical page of logical page j;
                                     unused entries are -1
  slot_mapping [T] int32             page*P + offset of each new token
  query_lens   [S] int32             tokens of this step per sequence
  seq_lens     [S] int32             prefix + this step's tokens
Tokens of all sequences are concatenated on one flat axis in sequence order
(the vLLM chunked-prefill article, "selective batching": a flattened
[sum L, hidden] token axis).

Draw order for one batch, from numpy's PCG64 seeded with `seed`:
  1. the page-pool permutation (rng.permutation(num_blocks));
  2. K of every sequence, positions 0..n-1, sequence by sequence;
  3. V likewise;
  4. Q for all T query tokens.
Each value is an fp32 N(0,1) draw rounded to bf16 (round to nearest even).
Random sequence lengths, when a workload wants them, are drawn by the caller
from its own generator before calling make_batch.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Sequence

import numpy as np

# Finite, conspicuous fill for cache slots that hold no token. A kernel that
# writes a wrong slot or reads past a sequence shows up against these.
SENTINEL_K = np.uint16(0x4B80)  # bf16 +2^24
SENTINEL_V = np.uint16(0xCB80)  # bf16 -2^24


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Inputs are finite N(0,1) draws, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


@dataclass
class Batch:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_blocks: int
    max_blocks_per_seq: int
    query_lens: np.ndarray
    seq_lens: np.ndarray
    block_table: np.ndarray
    slot_mapping: np.ndarray
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    # Logical per-sequence K/V ([n_s, Hkv, d] bits), kept for tests that
    # compare against unpaged attention. Empty when keep_logical=False.
    k_logical: list = field(default_factory=list)
    v_logical: list = field(default_factory=list)

    @property
    def num_seqs(self) -> int:
        return int(self.query_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.query_lens.sum())

    @property
    def query_start_loc(self) -> np.ndarray:
        out = np.zeros(self.num_seqs + 1, dtype=np.int32)
        np.cumsum(self.query_lens, out=out[1:])
        return out


def make_batch(seed: int, *, num_q_heads: int, num_kv_heads: int,
               head_dim: int, page_size: int,
               query_lens: Sequence[int], seq_lens: Sequence[int],
               extra_pages: int = 0, max_blocks_per_seq: int | None = None,
               keep_logical: bool = False) -> Batch:
    """Draw one flattened batch.

    Sequence s owns ceil(seq_lens[s]/page_size) pages taken in order from a
    seeded permutation of the pool (pages of different sequences are
    disjoint). Prefix positions p < seq_lens[s]-query_lens[s] are placed in
    the cache; the query_lens[s] new tokens come out as k_new/v_new with
    their slots in slot_mapping.
    """
    ql = np.asarray(query_lens, dtype=np.int32)
    sl = np.asarray(seq_lens, dtype=np.int32)
    if ql.shape != sl.shape or ql.ndim != 1:
        raise ValueError("query_lens and seq_lens must be 1-D and equally long")
    if np.any(ql < 0) or np.any(ql > sl):
        raise ValueError("need 0 <= query_len <= seq_len")
    P = int(page_size)
    pages = [(int(n) + P - 1) // P for n in sl]
    mbs = max_blocks_per_seq if max_blocks_per_seq is not None else max(1, max(pages))
    if max(pages) > mbs:
        raise ValueError("max_blocks_per_seq too small")
    NB = sum(pages) + int(extra_pages)
    rng = np.random.default_rng(seed)
    perm = rng.permutation(NB).astype(np.int32)

    S = ql.shape[0]
    block_table = np.full((S, mbs), -1, dtype=np.int32)
    off = 0
    for s in range(S):
        block_table[s, :pages[s]] = perm[off:off + pages[s]]
        off += pages[s]

    Hq, Hkv, d = num_q_heads, num_kv_heads, head_dim
    k_log = [normal_bf16(rng, (int(n), Hkv, d)) for n in sl]
    v_log = [normal_bf16(rng, (int(n), Hkv, d)) for n in sl]
    T = int(ql.sum())
    q = normal_bf16(rng, (T, Hq, d))

    k_cache = np.full((NB, Hkv, P, d), SENTINEL_K, dtype=np.uint16)
    v_cache = np.full((NB, Hkv, P, d), SENTINEL_V, dtype=np.uint16)
    k_new = np.empty((T, Hkv, d), dtype=np.uint16)
    v_new = np.empty((T, Hkv, d), dtype=np.uint16)
    slot_mapping = np.empty(T, dtype=np.int32)
    t0 = 0
    for s in range(S):
        n, c = int(sl[s]), int(ql[s])
        hist = n - c
        pos = np.arange(hist)
        phys = block_table[s, pos // P]
        k_cache[phys, :, pos % P, :] = k_log[s][:hist]
        v_cache[phys, :, pos % P, :] = v_log[s][:hist]
        newpos = np.arange(hist, n)
        slot_mapping[t0:t0 + c] = block_table[s, newpos // P] * P + newpos % P
        k_new[t0:t0 + c] = k_log[s][hist:n]
        v_new[t0:t0 + c] = v_log[s][hist:n]
        t0 += c

    return Batch(num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, page_size=P,
                 num_blocks=NB, max_blocks_per_seq=mbs, query_lens=ql,
                 seq_lens=sl, block_table=block_table,
                 slot_mapping=slot_mapping, q=q, k_new=k_new, v_new=v_new,
                 k_cache=k_cache, v_cache=v_cache,
                 k_logical=k_log if keep_logical else [],
                 v_logical=v_log if keep_logical else [])


# --- The workloads -------------------------------------------------------
# Shapes follow the pages: P1's history sweep 0/4k/8k/12k (dynamic chunked
# pipeline parallel design, "problem statement"), P3's 512-token chunks and
# 2048-token budget (vLLM chunked-prefill article, sections 3.1 and 4.1),
# LLaMA-13B (40 heads) and Llama-3-8B (32/8 heads) attention layers.

def small_parity(seed: int = 1, keep_logical: bool = False) -> Batch:
    """One sequence, 4/4 heads, d=64, H=192 cached, C=64 new, page 16,
    block table a permutation of 16 pages."""
    return make_batch(seed, num_q_heads=4, num_kv_heads=4, head_dim=64,
                      page_size=16, query_lens=[64], seq_lens=[256],
                      keep_logical=keep_logical)


def llama3_8b_chunk(hist: int, seed: int = 2, chunk: int = 512) -> Batch:
    """Llama-3-8B attention layer (32 q / 8 kv heads, d=128), page 128,
    one chunk of `chunk` tokens at prefix `hist`; 8 spare pages in the pool."""
    return make_batch(seed, num_q_heads=32, num_kv_heads=8, head_dim=128,
                      page_size=128, query_lens=[chunk],
                      seq_lens=[hist + chunk], extra_pages=8)


def mixed_llama13b(seed: int = 4, num_decode: int = 16,
                   prefill_hists: Sequence[int] = (2048, 6144),
                   chunk: int = 512) -> Batch:
    """LLaMA-13B attention (40/40 heads, d=128), page 128. Decode rows come
    first on the flat axis (query_len 1, seq_len uniform in [1024, 8192]),
    then prefill chunks of `chunk` tokens at the given prefixes."""
    rng = np.random.default_rng(seed)
    dec = rng.integers(1024, 8193, size=num_decode).astype(np.int32)
    ql = [1] * num_decode + [chunk] * len(prefill_hists)
    sl = [int(n) for n in dec] + [h + chunk for h in prefill_hists]
    return make_batch(seed + 1000, num_q_heads=40, num_kv_heads=40,
                      head_dim=128, page_size=128, query_lens=ql,
                      seq_lens=sl)


def long_context_chunk(hist: int, seed: int = 5, chunk: int = 2048,
                       max_model_len: int = 32768) -> Batch:
    """70B-like layer (64 q / 8 kv heads, d=128), page 128, one chunk at
    prefix `hist`; the block table spans max_model_len."""
    return make_batch(seed, num_q_heads=64, num_kv_heads=8, head_dim=128,
                      page_size=128, query_lens=[chunk],
                      seq_lens=[hist + chunk],
                      max_blocks_per_seq=math.ceil(max_model_len / 128))


# --- A request stream over many steps -----------------------------------
# The token-budget step loop (vLLM chunked-prefill article, section 3.1)
# prefills each prompt over several steps and then decodes one token per
# step, all into one paged cache. ServingStream fixes each request's pages
# up front and, for every formed batch, lays out that step's flattened
# metadata and draws its new tokens.

@dataclass
class StepInputs:
    query_lens: np.ndarray        # [S] int32
    seq_lens: np.ndarray          # [S] int32
    block_table: np.ndarray       # [S, max_blocks] int32, -1 past a request's pages
    slot_mapping: np.ndarray      # [T] int32
    q: np.ndarray | None          # [T, Hq, d] bf16 bits (None when not drawn)
    k_new: np.ndarray | None      # [T, Hkv, d]
    v_new: np.ndarray | None

    @property
    def num_tokens(self) -> int:
        return int(self.query_lens.sum())


class ServingStream:
    """Seeded pages and per-step tokens for a stream of requests.

    requests: (prompt_len, max_new, arrival_step) triples. Request r owns
    ceil((prompt_len + max_new) / page_size) pages, taken in order from a
    seeded permutation of a pool of that many pages plus `extra_pages`; its
    token at absolute position p goes to slot page[p // P] * P + p % P.
    `step(batch)` takes a formed batch, a list of (request id, query_len,
    seq_len) rows, and returns that step's metadata; with draw=True it also
    draws q, k_new and v_new for the step's tokens from the stream's
    generator (fp32 N(0,1) rounded to bf16, q first, then K, then V), so the
    draws depend on the sequence of batches and on nothing else.
    `initial_caches()` returns the pool's caches with every slot holding the
    sentinels.
    """

    def __init__(self, seed: int, *, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 page_size: int, requests: Sequence[tuple], extra_pages: int = 0):
        self.num_q_heads, self.num_kv_heads = int(num_q_heads), int(num_kv_heads)
        self.head_dim, self.page_size = int(head_dim), int(page_size)
        self.requests = [(int(p), int(m), int(a)) for p, m, a in requests]
        P = self.page_size
        counts = [(p + m + P - 1) // P for p, m, _ in self.requests]
        self.num_blocks = sum(counts) + int(extra_pages)
        self.max_blocks_per_seq = max([1] + counts)
        self.rng = np.random.default_rng(seed)
        perm = self.rng.permutation(self.num_blocks).astype(np.int32)
        self.pages, off = [], 0
        for n in counts:
            self.pages.append(perm[off:off + n])
            off += n

    def initial_caches(self):
        shape = (self.num_blocks, self.num_kv_heads, self.page_size, self.head_dim)
        return (np.full(shape, SENTINEL_K, dtype=np.uint16),
                np.full(shape, SENTINEL_V, dtype=np.uint16))

    def step(self, batch, draw: bool = True) -> StepInputs:
        P = self.page_size
        S = len(batch)
        ql = np.array([q for _, q, _ in batch], dtype=np.int32).reshape(S)
        sl = np.array([n for _, _, n in batch], dtype=np.int32).reshape(S)
        bt = np.full((max(S, 1), self.max_blocks_per_seq), -1, dtype=np.int32)[:S]
        slots = []
        for s, (rid, q, n) in enumerate(batch):
            pg = self.pages[rid]
            if (n + P - 1) // P > len(pg):
                raise ValueError(f"request {rid}: seq_len {n} exceeds its pages")
            bt[s, :len(pg)] = pg
            pos = np.arange(n - q, n)
            slots.append(pg[pos // P] * P + pos % P)
        sm = (np.concatenate(slots) if slots else np.zeros(0, np.int64)).astype(np.int32)
        T = int(ql.sum())
        q = k = v = None
        if draw:
            q = normal_bf16(self.rng, (T, self.num_q_heads, self.head_dim))
            k = normal_bf16(self.rng, (T, self.num_kv_heads, self.head_dim))
            v = normal_bf16(self.rng, (T, self.num_kv_heads, self.head_dim))
        return StepInputs(ql, sl, bt, sm, q, k, v)


def llama3_8b_request_stream(seed: int = 41, num_requests: int = 16):
    """A request stream for the step loop at the Llama-3-8B layer: prompts
    uniform in [2048, 16384] tokens (the history range of the dynamic-chunking
    design's sweep and beyond), 16..128 generated tokens, arrivals uniform over
    the first 32 steps. Returns (prompt_len, max_new, arrival_step) triples."""
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(2048, 16385)), int(rng.integers(16, 129)),
             int(rng.integers(0, 33))) for _ in range(num_requests)]
