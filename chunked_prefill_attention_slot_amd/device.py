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
