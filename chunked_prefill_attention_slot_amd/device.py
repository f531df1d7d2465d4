"""Device-side holder for one seeded batch: copies the inputs of an
inputs.Batch into torch device tensors, builds and uploads the attention
plan, and calls libcpa's KV write and attention on them. Marshalling only;
the work happens in libcpa."""
from __future__ import annotations

import numpy as np
import torch

from . import binding as cpa


def to_dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def to_dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def from_dev_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


class DeviceBatch:
    def __init__(self, b, out_dtype=cpa.CPA_DTYPE_BF16, options=None, scale=None):
        self.b = b
        self.desc = cpa.layer_desc(b.num_q_heads, b.num_kv_heads, b.head_dim, b.page_size,
                                   b.num_blocks, b.max_blocks_per_seq, scale=scale,
                                   out_dtype=out_dtype)
        self.q = to_dev_u16(b.q)
        self.k_new = to_dev_u16(b.k_new)
        self.v_new = to_dev_u16(b.v_new)
        self.k_cache = to_dev_u16(b.k_cache)
        self.v_cache = to_dev_u16(b.v_cache)
        self.slot_mapping = to_dev_i32(b.slot_mapping)
        self.block_table = to_dev_i32(b.block_table)
        self.plan = cpa.cpa_plan_create(self.desc, b.query_lens, b.seq_lens, options)
        self.workspace = torch.empty(max(self.plan.workspace_bytes, 256), dtype=torch.uint8,
                                     device="cuda")
        cpa.cpa_plan_upload(self.plan, self.workspace)
        dt = torch.float32 if out_dtype == cpa.CPA_DTYPE_F32 else torch.int16
        self.out = torch.full((b.num_tokens, b.num_q_heads, b.head_dim), -7777,
                              dtype=dt, device="cuda")

    def kv_write(self):
        cpa.cpa_kv_write(self.desc, self.k_new, self.v_new, self.slot_mapping,
                         self.k_cache, self.v_cache)

    def attention(self):
        cpa.cpa_attention(self.plan, self.q, self.k_cache, self.v_cache, self.block_table,
                          self.out, self.workspace)

    def run(self):
        self.kv_write()
        self.attention()
        torch.cuda.synchronize()

    def kv_write_attention(self):
        """The fused call: the same results as kv_write() then attention()."""
        cpa.cpa_kv_write_attention(self.plan, self.q, self.k_new, self.v_new,
                                   self.slot_mapping, self.k_cache, self.v_cache,
                                   self.block_table, self.out, self.workspace)

    def bound_fused(self):
        """kv_write_attention with its arguments marshalled once, on the
        current stream."""
        return cpa.bind_kv_write_attention(self.plan, self.q, self.k_new, self.v_new,
                                           self.slot_mapping, self.k_cache, self.v_cache,
                                           self.block_table, self.out, self.workspace)

    def bound(self):
        """(kv_write, attention) with their arguments marshalled once, on the
        current stream."""
        return (cpa.bind_kv_write(self.desc, self.k_new, self.v_new, self.slot_mapping,
                                  self.k_cache, self.v_cache),
                cpa.bind_attention(self.plan, self.q, self.k_cache, self.v_cache,
                                   self.block_table, self.out, self.workspace))

    def out_f64(self) -> np.ndarray:
        if self.out.dtype == torch.float32:
            return self.out.cpu().numpy().astype(np.float64)
        return self.out.view(torch.bfloat16).to(torch.float64).cpu().numpy()


class MicroBatchPair:
    """A DeviceBatch split into two micro-batches at (seq_split,
    token_split) (cpa_split_point): each half gets its own plan and
    workspace, and attention() runs the halves on two streams, ordered after
    the current stream's work and joined back into it. Marshalling only:
    both halves are cpa_attention calls on row-offset views."""

    def __init__(self, db: DeviceBatch, seq_split: int, token_split: int, options=None):
        b = db.b
        self.db = db
        ql, sl = np.asarray(b.query_lens), np.asarray(b.seq_lens)
        bounds = ((0, seq_split, 0, token_split),
                  (seq_split, len(ql), token_split, int(b.num_tokens)))
        self.parts = []
        for s0, s1, t0, t1 in bounds:
            plan = cpa.cpa_plan_create(db.desc, ql[s0:s1], sl[s0:s1], options)
            ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
            cpa.cpa_plan_upload(plan, ws)
            self.parts.append((plan, ws, s0, s1, t0, t1))
        self.streams = [torch.cuda.Stream(), torch.cuda.Stream()]

    def attention(self):
        db = self.db
        cur = torch.cuda.current_stream()
        ready = torch.cuda.Event()
        ready.record(cur)
        for (plan, ws, s0, s1, t0, t1), st in zip(self.parts, self.streams):
            st.wait_event(ready)
            cpa.cpa_attention(plan, db.q[t0:t1], db.k_cache, db.v_cache, db.block_table[s0:s1],
                              db.out[t0:t1], ws, stream=st)
        for st in self.streams:
            cur.wait_stream(st)


class ServingCaches:
    """Device K/V caches of a ServingStream's page pool, kept across steps,
    and the marshalling of one step: upload its metadata (and tokens), build
    and upload its plan, then KV write and attention through libcpa.
    `init="sentinel"` copies the stream's sentinel-filled caches to the
    device; `init="zeros"` only allocates and zeroes them (the content of a
    slot is never read before the step that writes it)."""

    def __init__(self, stream, out_dtype=cpa.CPA_DTYPE_BF16, options=None, init="sentinel"):
        self.stream = stream
        self.options = options
        self.out_dtype = out_dtype
        self.desc = cpa.layer_desc(stream.num_q_heads, stream.num_kv_heads, stream.head_dim,
                                   stream.page_size, stream.num_blocks,
                                   stream.max_blocks_per_seq, out_dtype=out_dtype)
        if init == "sentinel":
            kc, vc = stream.initial_caches()
            self.k_cache, self.v_cache = to_dev_u16(kc), to_dev_u16(vc)
        else:
            shape = (stream.num_blocks, stream.num_kv_heads, stream.page_size, stream.head_dim)
            self.k_cache = torch.zeros(shape, dtype=torch.int16, device="cuda")
            self.v_cache = torch.zeros(shape, dtype=torch.int16, device="cuda")
        self.workspace = torch.empty(256, dtype=torch.uint8, device="cuda")
        self.num_tokens = 0

    def load(self, st, q=None, k_new=None, v_new=None):
        """Take one step's StepInputs. Token tensors default to the drawn
        ones in `st`; device tensors of at least the step's token count may
        be passed instead (their leading rows are used)."""
        T = st.num_tokens
        self.num_tokens = T
        if T == 0:
            return
        self.q = q[:T] if q is not None else to_dev_u16(st.q)
        self.k_new = k_new[:T] if k_new is not None else to_dev_u16(st.k_new)
        self.v_new = v_new[:T] if v_new is not None else to_dev_u16(st.v_new)
        self.slot_mapping = to_dev_i32(st.slot_mapping)
        self.block_table = to_dev_i32(st.block_table)
        self.plan = cpa.cpa_plan_create(self.desc, st.query_lens, st.seq_lens, self.options)
        if self.plan.workspace_bytes > self.workspace.numel():
            self.workspace = torch.empty(self.plan.workspace_bytes, dtype=torch.uint8,
                                         device="cuda")
        cpa.cpa_plan_upload(self.plan, self.workspace)
        dt = torch.float32 if self.out_dtype == cpa.CPA_DTYPE_F32 else torch.int16
        self.out = torch.empty((T, self.stream.num_q_heads, self.stream.head_dim), dtype=dt,
                               device="cuda")

    def kv_write(self):
        if self.num_tokens:
            cpa.cpa_kv_write(self.desc, self.k_new, self.v_new, self.slot_mapping,
                             self.k_cache, self.v_cache)

    def attention(self):
        if self.num_tokens:
            cpa.cpa_attention(self.plan, self.q, self.k_cache, self.v_cache, self.block_table,
                              self.out, self.workspace)

    def out_f64(self) -> np.ndarray:
        if self.out.dtype == torch.float32:
            return self.out.cpu().numpy().astype(np.float64)
        return self.out.view(torch.bfloat16).to(torch.float64).cpu().numpy()
