"""Plain, slow fp64 CPU oracle for paged chunked-prefill attention.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call anything in this package; the product
path (chunked_prefill_attention_slot_amd) never does, and shares no code
with it.

Modules and the passages they follow:
  attention  -- chunked attention: the vLLM "Chunked-Prefills" article,
                section 3.2.1 (concatenate cached K/V with the chunk's own,
                scores, softmax, weighted V), with the causal offset by the
                prefix length and the paged-cache metadata of the Ascend
                dual-stream article, section 3.1.
  kv_cache   -- the slot_mapping write of the chunk's K/V (dual-stream
                article, section 3.1; chunked-prefill article, section 3.1:
                each chunk caches its KV).
  predictor  -- the quadratic latency model, least-squares fit, target and
                chunk solve with smoothing/alignment/clamps: the vllm-ascend
                dynamic chunked pipeline parallel design, sections
                "quadratic latency model", "startup: profiling",
                "runtime: dynamic prediction".
  calibration -- the online two-variable model f(C,H) of the same design,
                section "online calibration".
  split      -- the two-micro-batch split point of the dual-stream article,
                section 3.1.

Every function states the reading it takes where the pages are silent.
"""
