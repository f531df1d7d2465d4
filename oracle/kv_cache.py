"""Oracle: writing a chunk's K/V into the paged cache (a byte copy).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Ascend dual-stream article, section 3.1: slot_mapping ([bs] on the flat
token axis) maps each token to the cache slot its K/V go to; the vLLM
chunked-prefill article, section 3.1: each chunk computes and caches its KV.
Readings (the pages give no formula or layout): slot = page*P + offset, the
cache is [NB, Hkv, P, d] with separate K and V buffers, and a negative slot
means "no write" (padding token). The result is a byte copy, compared bit
for bit.
"""
from __future__ import annotations

import numpy as np


def kv_write(k_cache_bits: np.ndarray, v_cache_bits: np.ndarray,
             k_new_bits: np.ndarray, v_new_bits: np.ndarray,
             slot_mapping, page_size: int):
    """Return copies of both caches with token t's K/V ([Hkv, d]) stored at
    page slot // P, offset slot % P for every slot >= 0."""
    kc = k_cache_bits.copy()
    vc = v_cache_bits.copy()
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), page_size)
        kc[blk, :, off, :] = k_new_bits[t]
        vc[blk, :, off, :] = v_new_bits[t]
    return kc, vc
