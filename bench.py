"""Bench: paged chunked-prefill attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs ...] [--no-cpu]

One step = one pass of the hot path over the headline workload: a
Llama-3-8B attention layer (32 q / 8 kv heads, d=128, bf16, 128-token
pages) taking one 512-token chunk at each prefix H in {0, 4096, 8192,
12288} (the history sweep of the dynamic-chunking design's problem
statement; 512-token chunks of the vLLM chunked-prefill article): for each
H, one call writes the chunk's K/V into the paged cache through
slot_mapping and runs attention over prefix + chunk. Metadata planning and
upload happen once per workload, outside the timed region (a plan serves
every layer of a batch step). Inputs are resident in HBM before timing.

The printed JSON line (last line of stdout) carries:
  value        -- algorithmic TFLOP/s of the whole step, FLOP per chunk =
                  4*Hq*d*C*(H + C/2), over K steps timed with no events
                  between the launches, after the per-call event passes
                  (the median of three such timed regions; all are
                  reported);
  roofline     -- the step's call (prefill MFMA kernel with the KV write
                  inside, then the split combine) against bf16 dense MFMA
                  peak, averaged over the four H; a call's duration is the
                  span of K back-to-back calls between two HIP events, / K;
and one object per further leg (all run by default; --legs selects):
  small        -- the 4/4-head d=64 parity chunk (H=192, C=64);
  decode       -- LLaMA-13B decode rows (16 rows, seq_len U[1024, 8192],
                  40/40 heads): algorithmic K+V+Q+O bytes / time vs HBM peak;
  mixed_batch  -- the LLaMA-13B mixed batch (decode rows + two 512-token
                  chunks): whole call, the chunks alone in TFLOP/s, and the
                  two-micro-batch split on two streams;
  long_context -- 70B-like layer, 16 chunks of 2048 from H=0 to 30720,
                  TFLOP/s per chunk;
  predictor    -- dynamic chunking at the 4/4-head d=64 shape: 64 profiled
                  sizes, quadratic fit, T, the 32768-token walk at align 128
                  and 16 with per-chunk ratios to T and to the model, and
                  two online-calibrated walks (the record window seeded
                  with the profile's runs, and unseeded);
  chunk_schedule -- the token-budget step loop under fixed 512, progressive
                  [2048, 1024, 512], predictor and calibrated chunk rules
                  (a 16-request stream and one 32768-token prompt), and the
                  cost of chunk sizes around 512;
  cpu_baseline -- the fp64 oracle on host cores over the same workloads,
                  with GPU/oracle ratios and element-wise parity against
                  this run's GPU outputs.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
HIST_SWEEP = (0, 4096, 8192, 12288)
CHUNK = 512
REPEATS = 3                      # event-free timed regions of the headline step


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def flops_chunk(hq, d, c, h):
    return 4.0 * hq * d * c * (h + c / 2.0)


_HIP = None


class Event:
    """A HIP timing event on torch's current stream, created with
    hipEventDisableSystemFence. A default event record ends with a
    system-scope fence: it writes back and invalidates the caches, which
    costs time inside the bracket and slows the work after it. Timing-only
    events do not need it (HIP's own documentation of the flag says so).
    Same interface as torch.cuda.Event: record(), synchronize(),
    elapsed_time(end) in ms."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        import torch
        global _HIP
        if _HIP is None:
            torch.cuda.init()
            # The HIP runtime torch (and libcpa) already use in this process.
            path = [l.split()[-1] for l in open("/proc/self/maps").read().splitlines()
                    if "libamdhip64" in l][0]
            _HIP = ctypes.CDLL(path)
        self._ctypes = ctypes
        # Recorded on the stream current at creation (the timed loops run there).
        self._stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.h = ctypes.c_void_p()
        rc = _HIP.hipEventCreateWithFlags(ctypes.byref(self.h),
                                          ctypes.c_uint(self.DISABLE_SYSTEM_FENCE))
        assert rc == 0, f"hipEventCreateWithFlags: {rc}"

    def record(self):
        rc = _HIP.hipEventRecord(self.h, self._stream)
        assert rc == 0, f"hipEventRecord: {rc}"

    def synchronize(self):
        rc = _HIP.hipEventSynchronize(self.h)
        assert rc == 0, f"hipEventSynchronize: {rc}"

    def elapsed_time(self, end):
        ms = self._ctypes.c_float()
        rc = _HIP.hipEventElapsedTime(self._ctypes.byref(ms), self.h, end.h)
        assert rc == 0, f"hipEventElapsedTime: {rc}"
        return ms.value

    def __del__(self):
        if _HIP is not None and self.h:
            _HIP.hipEventDestroy(self.h)


def median_ms(fn, reps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(Event(), Event()) for _ in range(reps)]
    for s, e in ev:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    t = sorted(s.elapsed_time(e) for s, e in ev)
    return {"median_ms": t[len(t) // 2], "p10_ms": t[len(t) // 10], "p90_ms": t[(9 * len(t)) // 10],
            "mean_ms": sum(t) / len(t)}


# ---------------------------------------------------------------------------
def headline(args):
    import torch
    from chunked_prefill_attention_slot_amd.inputs import llama3_8b_chunk
    from chunked_prefill_attention_slot_amd.device import DeviceBatch

    dbs = []
    for h in args.hist:
        b = llama3_8b_chunk(h)
        db = DeviceBatch(b)
        dbs.append((h, db))
        log(f"[bench] llama3-8b C{CHUNK} H{h}: plan {db.plan.info()}")
    hq, d = 32, 128
    flops = [flops_chunk(hq, d, CHUNK, h) for h in args.hist]

    # Each call's arguments are marshalled once (binding.bind_*): the timed
    # loop then costs one foreign call per launch on the host. A step issues
    # cpa_kv_write_attention per chunk (the KV write inside the attention
    # launch); the same step through the two separate calls, cpa_kv_write
    # then cpa_attention, is timed beside it.
    calls = [db.bound() for _, db in dbs]
    fused = [db.bound_fused() for _, db in dbs]

    def step():
        for f in fused:
            f()

    def step_separate():
        for kv_write, attention in calls:
            kv_write()
            attention()

    for _ in range(args.warmup):
        step()
        step_separate()
    torch.cuda.synchronize()
    # Event passes first (they also finish warming the clocks): K steps with
    # one event before the first call and one after every call, on the
    # launch stream (torch's current stream); each call's bracketed time is
    # the span between the events around it, so it includes its launch and
    # one event's overhead.
    n = len(dbs)
    evs = [[Event() for _ in range(n + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for k in range(args.steps):
        e = evs[k]
        e[0].record()
        for i, f in enumerate(fused):
            f()
            e[i + 1].record()
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t1
    evs_sep = [[Event() for _ in range(2 * n + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        e = evs_sep[k]
        e[0].record()
        for i, (kv_write, attention) in enumerate(calls):
            kv_write()
            e[2 * i + 1].record()
            attention()
            e[2 * i + 2].record()
    torch.cuda.synchronize()
    # Per-call durations without per-call event overhead: for each H, K
    # back-to-back calls of that chunk between one pair of events on the
    # launch stream; the duration of a call is the span over K. This is the
    # figure `per_H` and `roofline` use; the bracketed spans above (each call
    # between two events of its own) are kept beside it.
    per_call = []
    for f in fused:
        e0, e1 = Event(), Event()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            f()
        e1.record()
        e1.synchronize()
        per_call.append(e0.elapsed_time(e1) / args.steps)
    torch.cuda.synchronize()
    # Timed regions: K steps exactly as a caller issues them, with no event
    # between the launches (a recorded event costs 1.5-2 us of stream time,
    # its own packet between two kernels). The fused step is timed
    # REPEATS times after the event passes, each region exactly K steps;
    # `value` is the median region (the clock still settles over the first
    # regions after a short warm-up), and every repeat is reported.
    walls = []
    for _ in range(REPEATS):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
    wall = sorted(walls)[len(walls) // 2]
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_separate()
    torch.cuda.synchronize()
    wall_sep = time.perf_counter() - t0
    per_h = []
    call_ms_tot = 0.0
    for i, h in enumerate(args.hist):
        c = sorted(e[i].elapsed_time(e[i + 1]) for e in evs)
        a = sorted(e[2 * i + 1].elapsed_time(e[2 * i + 2]) for e in evs_sep)
        kv = sorted(e[2 * i].elapsed_time(e[2 * i + 1]) for e in evs_sep)
        cm = per_call[i]
        call_ms_tot += cm
        per_h.append({"H": h, "call_us_mean": cm * 1e3,
                      "call_us_bracketed_mean": sum(c) / len(c) * 1e3,
                      "call_us_bracketed_median": c[len(c) // 2] * 1e3,
                      "call_us_bracketed_p10": c[len(c) // 10] * 1e3,
                      "call_us_bracketed_p90": c[(9 * len(c)) // 10] * 1e3,
                      "attn_us_mean": sum(a) / len(a) * 1e3,
                      "kv_write_us_mean": sum(kv) / len(kv) * 1e3,
                      "tflops": flops[i] / (cm * 1e-3) / 1e12,
                      "mfma_frac": flops[i] / (cm * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS})
        log(f"[bench] H={h}: kv_write_attention {cm*1e3:.1f} us -> {per_h[-1]['tflops']:.1f} "
            f"TFLOP/s ({100*per_h[-1]['mfma_frac']:.1f}% of bf16 peak; {sum(c) / len(c) * 1e3:.1f}"
            f" us between events of its own); separate calls: "
            f"kv_write {per_h[-1]['kv_write_us_mean']:.1f} us + attention "
            f"{per_h[-1]['attn_us_mean']:.1f} us (events of their own)")
    ms_per_step = wall * 1e3 / args.steps
    log(f"[bench] step: {ms_per_step*1e3:.1f} us without events (median of repeats "
        + ", ".join(f"{w * 1e6 / args.steps:.1f}" for w in walls)
        + f"; {wall_ev*1e6/args.steps:.1f} us with {n+1} events); separate calls "
        f"{wall_sep*1e6/args.steps:.1f} us")
    total_flops = sum(flops)
    achieved = (total_flops / n) / (call_ms_tot / n * 1e-3) / 1e12
    # The timed steps' outputs (bf16 bits), for the parity figure of the
    # CPU baseline leg.
    outs = {h: db.out.cpu().numpy().view(np.uint16).copy() for h, db in dbs}
    return {
        "outputs": outs,
        "ms_per_step": ms_per_step,
        "ms_per_step_repeats": [w * 1e3 / args.steps for w in walls],
        "ms_per_step_with_events": wall_ev * 1e3 / args.steps,
        "ms_per_step_separate_calls": wall_sep * 1e3 / args.steps,
        "value": total_flops / (ms_per_step * 1e-3) / 1e12,
        "per_H": per_h,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": None,
                     "kernel": "cpa_kv_write_attention (prefill_kernel<128, fused> + "
                               "combine_kernel<128> when tiles are split)",
                     "duration": "mean call duration, K back-to-back calls per H between "
                                 "two HIP events on the launch stream, averaged over the H",
                     "flop_per_launch": total_flops / n},
    }


def small_leg(args):
    """The small workload (4/4 heads, d=64, H=192 cached, C=64 new, 16-token
    pages): the fused call's time. Far too small to load the GPU; it is the
    parity case, timed for the record."""
    import torch
    from chunked_prefill_attention_slot_amd.inputs import small_parity
    from chunked_prefill_attention_slot_amd.device import DeviceBatch
    b = small_parity()
    db = DeviceBatch(b)
    r = median_ms(db.bound_fused(), 50, 10)
    f = flops_chunk(4, 64, 64, 192)
    torch.cuda.synchronize()
    out = db.out.cpu().numpy().view(np.uint16).copy()
    res = {"workload": "4/4 heads, d=64, page 16, H=192, C=64 (fused KV write + attention)",
           "us_median": r["median_ms"] * 1e3, "us_mean": r["mean_ms"] * 1e3, "flop": f,
           "tflops": f / (r["median_ms"] * 1e-3) / 1e12}
    log(f"[bench] small: {res['us_median']:.1f} us per fused call")
    return res, (b, out)


def decode_rows(args, mixed):
    """LLaMA-13B decode rows alone: a plan over the 16 query_len-1 rows of
    the mixed batch (its prefill chunks get query_len 0)."""
    import torch
    from chunked_prefill_attention_slot_amd import binding as cpa
    b, db = mixed
    nd = 16
    ql = [1] * nd + [0] * (b.num_seqs - nd)
    plan = cpa.cpa_plan_create(db.desc, ql, b.seq_lens)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
    cpa.cpa_plan_upload(plan, ws)
    q = db.q[:nd]
    out = db.out[:nd]
    r = median_ms(cpa.bind_attention(plan, q, db.k_cache, db.v_cache, db.block_table, out, ws),
                  args.decode_reps, 5)
    hkv, d = b.num_kv_heads, b.head_dim
    kv_bytes = float(sum(int(n) for n in b.seq_lens[:nd])) * hkv * d * 2 * 2
    qo_bytes = nd * b.num_q_heads * d * 2 * 2
    gbs = (kv_bytes + qo_bytes) / (r["mean_ms"] * 1e-3) / 1e9
    res = {"workload": "llama13b 16 decode rows, seq_len U[1024,8192], 40/40 heads, d=128",
           "bytes": kv_bytes + qo_bytes, "us_mean": r["mean_ms"] * 1e3,
           "us_median": r["median_ms"] * 1e3, "GB_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
           "plan": plan.info()}
    log(f"[bench] decode rows: {res['us_mean']:.1f} us, {gbs:.0f} GB/s "
        f"({100*gbs/HBM_PEAK_GBS:.1f}% of HBM peak)")
    return res


def mixed_leg(args, mixed):
    """The LLaMA-13B mixed batch on one flattened axis (16 decode rows, then
    two 512-token chunks at H = 2048 and 6144; 1040 tokens of a 2048-token
    budget): (i) the whole mixed call, (ii) its prefill chunks alone ->
    TFLOP/s, (iii) the two-micro-batch split (dual-stream article, section
    3.1) on two streams. Decode rows alone are the decode leg."""
    import torch
    from chunked_prefill_attention_slot_amd import binding as cpa
    b, db = mixed
    r_all = median_ms(db.bound()[1], args.decode_reps, 3)
    torch.cuda.synchronize()
    out_all = db.out.cpu().numpy().view(np.uint16).copy()
    nd = 16
    ql = [0] * nd + [int(x) for x in b.query_lens[nd:]]
    plan = cpa.cpa_plan_create(db.desc, ql, b.seq_lens)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
    cpa.cpa_plan_upload(plan, ws)
    r_pf = median_ms(cpa.bind_attention(plan, db.q[nd:], db.k_cache, db.v_cache,
                                        db.block_table, db.out[nd:], ws),
                     args.decode_reps, 3)
    pf_flops = sum(flops_chunk(40, 128, int(c), int(n) - int(c))
                   for c, n in zip(b.query_lens[nd:], b.seq_lens[nd:]))
    res = {"workload": "llama13b mixed batch: 16 decode rows + 2 chunks of 512 at H=2048, 6144",
           "mixed_call_us": r_all["mean_ms"] * 1e3,
           "prefill_only_us": r_pf["mean_ms"] * 1e3, "prefill_flop": pf_flops,
           "prefill_only_tflops": pf_flops / (r_pf["mean_ms"] * 1e-3) / 1e12,
           "prefill_only_mfma_frac":
               pf_flops / (r_pf["mean_ms"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    log(f"[bench] llama13b mixed call {res['mixed_call_us']:.1f} us; prefill chunks alone "
        f"{res['prefill_only_us']:.1f} us = {res['prefill_only_tflops']:.1f} TFLOP/s")
    from chunked_prefill_attention_slot_amd.device import MicroBatchPair
    for mode, name in ((cpa.CPA_SPLIT_BALANCED, "balanced"), (cpa.CPA_SPLIT_SIMPLE, "simple")):
        split = cpa.cpa_split_point(b.query_lens, mode, 0.5, 64)
        if split is None:
            res[f"micro_batches_{name}"] = None
            continue
        pair = MicroBatchPair(db, *split)
        r_mb = median_ms(pair.attention, args.decode_reps, 3)
        res[f"micro_batches_{name}"] = {"split": list(split), "two_stream_us": r_mb["mean_ms"] * 1e3}
        log(f"[bench] llama13b micro-batches ({name}, split {split}): two streams "
            f"{r_mb['mean_ms'] * 1e3:.1f} us vs one call {res['mixed_call_us']:.1f} us")
    return res, out_all


def long_context(args):
    """70B-like layer (64 q / 8 kv heads): one 32768-token prompt prefilled in
    16 chunks of 2048; each chunk = one fused KV write + attention call,
    FLOP counted as 4*heads*d*C*(H + C/2). Returns the result and the last
    chunk's GPU output."""
    import torch
    from chunked_prefill_attention_slot_amd import binding as cpa
    from chunked_prefill_attention_slot_amd.inputs import make_batch
    from chunked_prefill_attention_slot_amd.device import DeviceBatch
    b = make_batch(5, num_q_heads=64, num_kv_heads=8, head_dim=128, page_size=128,
                   query_lens=[32768], seq_lens=[32768])
    db = DeviceBatch(b)
    run = chunk_runner(db, cpa, torch)
    rows = []
    tot_f, tot_ms = 0.0, 0.0
    for c in range(16):
        h = 2048 * c
        r = median_ms(run(h, 2048), 10, 2)
        f = flops_chunk(64, 128, 2048, h)
        tot_f += f
        tot_ms += r["median_ms"]
        rows.append({"H": h, "us": r["median_ms"] * 1e3,
                     "tflops": f / (r["median_ms"] * 1e-3) / 1e12,
                     "mfma_frac": f / (r["median_ms"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS})
    torch.cuda.synchronize()
    last = db.out[30720:].cpu().numpy().view(np.uint16).copy()
    res = {"workload": "70B-like layer 64/8 heads, d=128, page 128: 16 chunks of 2048, "
                       "H = 0..30720, fused KV write + attention per chunk",
           "chunks": rows, "total_ms": tot_ms, "tflops": tot_f / (tot_ms * 1e-3) / 1e12,
           "mfma_frac": tot_f / (tot_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    log(f"[bench] 70b-like 16x2048: {tot_ms:.2f} ms total, {res['tflops']:.1f} TFLOP/s; last "
        f"chunk {rows[-1]['tflops']:.0f} TFLOP/s")
    return res, (b, last)


PREDICTOR_SHAPES = {
    # the profiling shape of the predictor workload: 4/4 heads, d=64, page 16
    "tiny": dict(num_q_heads=4, num_kv_heads=4, head_dim=64, page_size=16),
    # a Llama-3-8B attention layer, where the chunk cost grows with history
    "llama3_8b": dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=128),
}


def chunk_runner(db, cpa, torch):
    """runner(L, c) -> a closure doing the KV write + attention of the chunk
    [L, L + c) of db's single sequence in one fused call
    (cpa_kv_write_attention), the unit every chunk of a prefill pays."""
    def runner(L, c):
        plan = cpa.cpa_plan_create(db.desc, [c], [L + c])
        ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
        cpa.cpa_plan_upload(plan, ws)
        sl = slice(L, L + c)
        f = cpa.bind_kv_write_attention(plan, db.q[sl], db.k_new[sl], db.v_new[sl],
                                        db.slot_mapping[sl], db.k_cache, db.v_cache,
                                        db.block_table, db.out[sl], ws)
        f.plan = plan
        return f
    return runner


def profile_fit(runner):
    """Startup profiling (dynamic-chunking design, "startup"): median ms of
    KV write + attention for a fresh chunk of each of the 64 sizes 2048,
    2016, .., 32, and the least-squares quadratic through them."""
    from chunked_prefill_attention_slot_amd import binding as cpa
    sizes = cpa.cpa_predictor_profile_sizes(2048, 64, 32)
    ms = [median_ms(runner(0, l), 21, 3)["median_ms"] for l in sizes]
    return sizes, ms, cpa.cpa_predictor_fit(sizes, ms)


def _ratio_stats(r, ok=None):
    r = np.asarray(r, dtype=np.float64)
    out = {"min": float(r.min()), "max": float(r.max()), "mean": float(r.mean()),
           "cv": float(r.std() / r.mean()) if r.mean() else None,
           "frac_within_10pct": float(np.mean(np.abs(r - 1) <= 0.1))}
    if ok is not None:
        out["frac_within_10pct_not_alignment_limited"] = \
            float(np.mean(np.abs(r[ok] - 1) <= 0.1)) if ok.any() else None
    return out


def predictor_walk(runner, fit, align, prompt, cfg_kw=None):
    """Prefill `prompt` tokens with chunks from cpa_predictor_next_chunk under
    the profiled fit; time each chunk (median of 11 fused calls) and compare
    it with the target and with the model (dynamic-chunking design,
    "runtime: dynamic prediction"). Per chunk: measured/T, the model's own
    ratio [f(L+x) - f(L)]/T (below 0.9 = alignment-limited: the align-down
    removed more than a tenth of the solved chunk), measured/model,
    (measured - c)/T (the measured time beyond the fitted per-call constant
    c, which f(L+x) - f(L) cancels), and measured/f(base)."""
    from chunked_prefill_attention_slot_amd import binding as cpa
    a, b, c = fit
    cfg = cpa.predictor_cfg(align=align, **(cfg_kw or {}))
    T = cpa.cpa_predictor_target(cfg, a, b)
    f_base = a * 2048.0 * 2048.0 + b * 2048.0 + c

    def f(x):
        return a * x * x + b * x + c
    rows = []
    L = 0
    while L < prompt:
        ch, x = cpa.cpa_predictor_next_chunk(cfg, a, b, T, L, prompt - L)
        if ch <= 0:
            break
        m = median_ms(runner(L, ch), 11, 2)["median_ms"]
        model = f(L + ch) - f(L)
        rows.append((L, ch, x, m, model))
        L += ch
    Ls, ch, raw, ms, model = (np.array(v, dtype=np.float64) for v in zip(*rows))
    model_over_T = model / T
    ok = model_over_T >= 0.9
    return {"align": align, "T_ms": T, "f_base_ms": f_base, "num_chunks": len(rows),
            "degenerate_fit": not (a > 0),
            "meas_over_T": _ratio_stats(ms / T, ok),
            "meas_minus_c_over_T": _ratio_stats((ms - c) / T, ok),
            # a degenerate fit (a <= 0) models some chunks at <= 0 ms
            "meas_over_model": _ratio_stats(ms / model) if np.all(model > 0) else None,
            "meas_over_f_base": _ratio_stats(ms / f_base, ok),
            "alignment_limited_chunks": int((~ok).sum()),
            "chunks": {"L": Ls.astype(int).tolist(), "chunk": ch.astype(int).tolist(),
                       "raw_x": [round(v, 3) for v in raw],
                       "ms": [round(v, 5) for v in ms],
                       "model_over_T": [round(v, 4) for v in model_over_T]}}


def seed_calibration(calib, sizes, ms):
    """Start the online calibration's record window with the startup
    profile's timed runs (dynamic-chunking design, "startup: profiling" and
    "online calibration"): each is a chunk of l tokens at H = 0, i.e. the
    features [l*l, l, 1], added in ascending size so that the sizes nearest
    the base stay longest in the window. Without them, a single prompt whose
    profile model repeats one chunk size never gets a refit: C*(C+H) and
    C+H then stay proportional and the window does not determine a, b, c."""
    from chunked_prefill_attention_slot_amd import binding as cpa
    for l, m in sorted(zip(sizes, ms)):
        calib.record(cpa.cpa_calib_features([int(l)], [0]), float(m))


def online_walk(calib, cfg, fit, prompt, measure):
    """Prefill `prompt` tokens with chunks sized by the online calibration
    (dynamic-chunking design, "online calibration"): each chunk solves the
    current two-variable model for T' = f(base, 0) of that model (R22),
    falling back to the profiled one-variable predictor while the window
    holds no model; measure(L, chunk) -> ms runs and times the chunk, whose
    features and time are recorded before the next solve. Returns the rows
    (L, chunk, ms, T' used) and the number of refused refits."""
    from chunked_prefill_attention_slot_amd import binding as cpa
    a, b, c = fit
    T = cpa.cpa_predictor_target(cfg, a, b)
    f_base = a * 2048.0 * 2048.0 + b * 2048.0 + c
    rows, refused, L = [], 0, 0
    while L < prompt:
        try:
            a2, b2, c2 = calib.model()
            T2 = cpa.cpa_calib_target(cfg, a2, b2, c2)
            ch, _ = cpa.cpa_calib_next_chunk(cfg, a2, b2, c2, T2, L, prompt - L)
        except cpa.CpaError:
            T2 = f_base
            ch, _ = cpa.cpa_predictor_next_chunk(cfg, a, b, T, L, prompt - L)
        if ch <= 0:
            break
        m = measure(L, ch)
        try:
            calib.record(cpa.cpa_calib_features([ch], [L]), m)
        except cpa.CpaError:
            refused += 1       # window does not determine the model (e.g. one chunk size)
        rows.append((L, ch, m, T2))
        L += ch
    return rows, refused


def predictor_run(args, shape="tiny", prompt=32768, aligns=(128, 16)):
    """The dynamic-chunking workload: profile the fused KV write + attention
    at 64 sizes (2048 down to 32, H = 0), fit f(l) = a l^2 + b l + c, set
    T = f(2048) - f(0), then prefill a 32768-token prompt with predicted
    chunks at each alignment quantum (128 as the workload states, 16 as the
    side run). Then the same prompt again with online calibration of the
    two-variable model f(C, H) (refitted from each chunk's measured time once
    5 are held), twice: with the record window seeded by the startup
    profile's timed runs (seed_calibration), and unseeded (the one-variable
    model sizes the chunks until a refit exists).
    Returns the result and the GPU outputs of the align-128 walk."""
    import torch
    from chunked_prefill_attention_slot_amd import binding as cpa
    from chunked_prefill_attention_slot_amd.inputs import make_batch
    from chunked_prefill_attention_slot_amd.device import DeviceBatch
    b = make_batch(3, query_lens=[prompt], seq_lens=[prompt], **PREDICTOR_SHAPES[shape])
    db = DeviceBatch(b)
    runner = chunk_runner(db, cpa, torch)
    sizes, ms, (a, bb, c) = profile_fit(runner)
    prof = np.array(ms)
    res = {"shape": shape, "prompt": prompt, "fit": {"a": a, "b": bb, "c": c},
           "profile_ms": [round(v, 5) for v in ms], "profile_sizes": [int(v) for v in sizes],
           # sizes run from 2048 down to 32: a rising profile has ms[i] >= ms[i+1]
           "profile_monotone_violations": int(np.sum(prof[:-1] < prof[1:] - 1e-4)),
           "fit_rms_ms": float(np.sqrt(np.mean((a * np.array(sizes, float) ** 2 +
                                                bb * np.array(sizes, float) + c - prof) ** 2)))}
    outputs = None
    for al in aligns:
        w = predictor_walk(runner, (a, bb, c), al, prompt)
        res[f"align{al}"] = w
        if outputs is None:
            torch.cuda.synchronize()
            outputs = (b, w["chunks"], db.out.cpu().numpy().view(np.uint16).copy())
        log(f"[bench] predictor {shape} align {al}: a={a:.3e} b={bb:.3e} c={c:.3e} "
            f"T={w['T_ms']:.4f} ms, {w['num_chunks']} chunks ({w['alignment_limited_chunks']} "
            f"alignment-limited); meas/T mean {w['meas_over_T']['mean']:.2f} "
            f"(within 10%: {w['meas_over_T']['frac_within_10pct']:.2f}); "
            f"(meas-c)/T mean {w['meas_minus_c_over_T']['mean']:.2f} "
            f"(within 10%: {w['meas_minus_c_over_T']['frac_within_10pct']:.2f}, not alignment-"
            f"limited {w['meas_minus_c_over_T']['frac_within_10pct_not_alignment_limited']}); "
            + (f"meas/model mean {w['meas_over_model']['mean']:.2f} cv "
               f"{w['meas_over_model']['cv']:.2f}" if w["meas_over_model"] else
               "model degenerate (a <= 0)"))

    # Online calibration of f(C, H) = a*C*(C+H) + b*(C+H) + c over the same prompt.
    cfg = cpa.predictor_cfg(align=aligns[0])
    f_base = a * 2048.0 * 2048.0 + bb * 2048.0 + c
    for key, seeded in (("online", True), ("online_unseeded", False)):
        calib = cpa.Calib(min_points=5, window=30)
        if seeded:
            seed_calibration(calib, sizes, ms)
        online, refused = online_walk(
            calib, cfg, (a, bb, c), prompt,
            lambda L, ch: median_ms(runner(L, ch), 11, 2)["median_ms"])
        try:
            fin = list(calib.model())
        except cpa.CpaError:
            fin = None
        om = np.array([r[2] for r in online])
        res[key] = {"seeded_with_profile": seeded, "num_chunks": len(online), "final_fit": fin,
                    "refused_refits": refused,
                    # T' of the model that sized each chunk (f(base) of the profile fit
                    # while no refit exists)
                    "meas_over_T_used": _ratio_stats(om / np.array([r[3] for r in online])),
                    "meas_over_f_base": _ratio_stats(om / f_base),
                    "chunk": [int(r[1]) for r in online]}
        log(f"[bench] predictor {shape} online calibration ({'seeded' if seeded else 'unseeded'}): "
            f"{len(online)} chunks, {refused} refits refused; meas/T' mean "
            f"{res[key]['meas_over_T_used']['mean']:.2f} cv {res[key]['meas_over_T_used']['cv']:.3f} "
            f"(within 10%: {res[key]['meas_over_T_used']['frac_within_10pct']:.2f}); meas/f(base) "
            f"cv {res[key]['meas_over_f_base']['cv']:.3f} vs "
            f"{res['align128']['meas_over_f_base']['cv']:.3f} profiled")
    return res, outputs


LLAMA3_8B = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=128)


def step_loop(requests, budget, rule, fit, seed=7, align=128, profile=None):
    """One pass of the token-budget step loop (vLLM chunked-prefill article,
    section 3.1) over a request stream at the Llama-3-8B layer: libcpa's
    batch former forms each step, the stream lays out its metadata, and the
    step's KV write + attention run on one cache kept across steps. Each
    step's GPU time comes from events around its two calls, after which the
    host waits for the step (so host work is outside the figure). rule is
    ("fixed", size) | ("progressive", sizes) | ("predictor",) |
    ("calibrated",): the last refits f(C, H) online from every step's
    features and time, its window seeded with the startup profile's runs
    (profile = (sizes, ms); seed_calibration), and hands the model to the
    former."""
    import torch
    from chunked_prefill_attention_slot_amd import binding as cpa
    from chunked_prefill_attention_slot_amd.device import ServingCaches
    from chunked_prefill_attention_slot_amd.inputs import ServingStream
    a, b, c = fit
    pcfg = cpa.predictor_cfg(align=align)
    kind = rule[0]
    if kind == "fixed":
        cfg = cpa.sched_cfg(budget, cpa.CPA_RULE_FIXED, fixed_chunk=rule[1])
    elif kind == "progressive":
        cfg = cpa.sched_cfg(budget, cpa.CPA_RULE_PROGRESSIVE, sizes=rule[1])
    elif kind == "predictor":
        cfg = cpa.sched_cfg(budget, cpa.CPA_RULE_PREDICTOR, pred=pcfg, a=a, b=b,
                            T=cpa.cpa_predictor_target(pcfg, a, b))
    else:   # the one-variable fit is f(C, 0) of the two-variable model until refits exist
        cfg = cpa.sched_cfg(budget, cpa.CPA_RULE_CALIBRATED, pred=pcfg, a=a, b=b, c=c,
                            T=cpa.cpa_calib_target(pcfg, a, b, c))
    sched = cpa.Sched(cfg)
    for p, m, t in requests:
        sched.add(p, m, t)
    calib = cpa.Calib(min_points=5, window=30) if kind == "calibrated" else None
    if calib is not None and profile is not None:
        seed_calibration(calib, *profile)
        a2, b2, c2 = calib.model()
        sched.set_model(a2, b2, c2, cpa.cpa_calib_target(pcfg, a2, b2, c2))
    stream = ServingStream(seed, requests=requests, **LLAMA3_8B)
    dev = ServingCaches(stream, init="zeros")
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    hq, hkv, d = LLAMA3_8B["num_q_heads"], LLAMA3_8B["num_kv_heads"], LLAMA3_8B["head_dim"]

    def pool(h):
        return torch.randn((budget, h, d), generator=g, device="cuda").to(torch.bfloat16) \
            .view(torch.int16)
    pools = (pool(hq), pool(hkv), pool(hkv))
    e0, e1 = Event(), Event()
    steps, refused, host_s = [], 0, 0.0
    first_tok, dec_times = {}, {}
    cum = 0.0
    while True:
        done, step_no = sched.status()
        if done:
            break
        h0 = time.perf_counter()
        batch = sched.form()
        st = stream.step(batch, draw=False)
        dev.load(st, *pools)
        host_s += time.perf_counter() - h0
        if step_no == 0:                      # warm the kernels on the first step's shapes
            for _ in range(2):
                dev.kv_write()
                dev.attention()
        e0.record()
        dev.kv_write()
        dev.attention()
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1) if st.num_tokens else 0.0
        start, cum = cum, cum + ms
        n_dec = 0
        for rid, q, n in batch:
            p, _, arr = requests[rid]
            if n > p:
                n_dec += 1
                dec_times.setdefault(rid, []).append(cum)
            elif n == p:
                first_tok[rid] = (arr, cum)
        steps.append({"tokens": st.num_tokens, "rows": len(batch), "decode_rows": n_dec,
                      "ms": ms, "start_ms": start})
        if calib is not None and st.num_tokens:
            try:
                calib.record(cpa.cpa_calib_features(st.query_lens, st.seq_lens - st.query_lens),
                             ms)
            except cpa.CpaError:
                refused += 1
            try:
                a2, b2, c2 = calib.model()
                sched.set_model(a2, b2, c2, cpa.cpa_calib_target(pcfg, a2, b2, c2))
            except cpa.CpaError:
                pass
        sched.commit()
    # time to first token: from the start of the arrival step to the end of
    # the step that finishes the prompt; inter-token gaps between a request's
    # token-producing steps
    start_of = [s["start_ms"] for s in steps]
    ttft = [end - start_of[min(arr, len(start_of) - 1)] for arr, end in first_tok.values()]
    itl = []
    for rid, ts in dec_times.items():
        prev = first_tok[rid][1]
        for t in ts:
            itl.append(t - prev)
            prev = t
    busy_idx = [i for i, s in enumerate(steps) if s["tokens"] > s["decode_rows"]]  # with prefill
    busy = [steps[i]["ms"] for i in busy_idx]

    def stats(v):
        v = np.asarray(v, dtype=np.float64)
        if v.size == 0:
            return None
        return {"mean": float(v.mean()), "p50": float(np.percentile(v, 50)),
                "p90": float(np.percentile(v, 90)), "max": float(v.max()),
                "cv": float(v.std() / v.mean()) if v.mean() > 0 else 0.0}
    tot = sum(s["ms"] for s in steps)
    ntok = sum(s["tokens"] for s in steps)
    res = {"rule": list(rule) if len(rule) > 1 else [kind], "steps": len(steps),
           "gpu_ms_total": tot, "tokens": ntok,
           "prefill_chunks": sum(s["rows"] - s["decode_rows"] for s in steps),
           "tokens_per_s": ntok / (tot * 1e-3) if tot else None,
           "step_ms_with_prefill": stats(busy),
           "slowest_step": (lambda i: {"index": i, **steps[i]})(max(busy_idx, key=lambda i:
                                                                       steps[i]["ms"]))
           if busy_idx else None,
           "ttft_ms": stats(ttft), "itl_ms": stats(itl),
           "host_ms_per_step": host_s * 1e3 / max(1, len(steps))}
    if calib is not None:
        res["refused_refits"] = refused
        try:
            res["final_model"] = list(calib.model())
        except cpa.CpaError:
            res["final_model"] = None
    return res


def serving_run(args):
    """The step loop at the Llama-3-8B layer under four chunk rules, on a
    seeded stream of 16 requests (budget 2048) and on one 32768-token prompt
    alone (the chunk-schedule comparison: fixed 512, progressive
    [2048, 1024, 512], predictor-sized, calibrated). The predictor rules use
    a fit profiled at this layer at startup."""
    import torch
    from chunked_prefill_attention_slot_amd import binding as cpa
    from chunked_prefill_attention_slot_amd.inputs import llama3_8b_request_stream, make_batch
    from chunked_prefill_attention_slot_amd.device import DeviceBatch
    b = make_batch(3, query_lens=[2048], seq_lens=[2048], **LLAMA3_8B)
    db = DeviceBatch(b)
    sizes, ms, fit = profile_fit(chunk_runner(db, cpa, torch))
    del db
    rules = [("fixed", 512), ("progressive", (2048, 1024, 512)), ("predictor",), ("calibrated",)]
    out = {"fit": list(fit), "budget": 2048}
    for name, reqs in (("stream16", llama3_8b_request_stream()), ("single32k", [(32768, 0, 0)])):
        rows = []
        for rule in rules:
            r = step_loop(reqs, 2048, rule, fit, profile=(sizes, ms))
            rows.append(r)
            bs = r["step_ms_with_prefill"]
            log(f"[bench] step loop {name} {r['rule']}: {r['steps']} steps, {r['gpu_ms_total']:.1f} "
                f"ms GPU, {r['prefill_chunks']} chunks, prefill-step ms mean {bs['mean']:.3f} "
                f"p90 {bs['p90']:.3f} max {bs['max']:.3f} cv {bs['cv']:.3f}"
                + (f", ttft mean {r['ttft_ms']['mean']:.1f} ms" if r["ttft_ms"] else "")
                + (f", itl p90 {r['itl_ms']['p90']:.3f} ms" if r["itl_ms"] else ""))
            torch.cuda.empty_cache()
        out[name] = {"requests": len(reqs), "prompt_tokens": sum(p for p, _, _ in reqs),
                     "decode_tokens": sum(m for _, m, _ in reqs), "rules": rows}
    return out


def alignment_study(args, hists=(0, 4096, 12288),
                    sizes=(384, 448, 496, 511, 512, 513, 528, 544, 576, 640)):
    """Chunk-size sweep around 512 at the Llama-3-8B layer (KV write +
    attention of one chunk at prefix H): the cost of a chunk one token past a
    tile multiple, which the vLLM chunked-prefill article prices at +32%
    for 512 -> 513 on its GPU."""
    import torch
    from chunked_prefill_attention_slot_amd import binding as cpa
    from chunked_prefill_attention_slot_amd.inputs import make_batch
    from chunked_prefill_attention_slot_amd.device import DeviceBatch
    n = max(hists) + max(sizes)
    b = make_batch(6, query_lens=[n], seq_lens=[n], **LLAMA3_8B)
    db = DeviceBatch(b)
    db.kv_write()
    run = chunk_runner(db, cpa, torch)
    out = {}
    for h in hists:
        row = {int(c): median_ms(run(h, c), 31, 3)["median_ms"] * 1e3 for c in sizes}
        out[str(h)] = {"us": row, "ratio_513_over_512": row[513] / row[512],
                       "ratio_511_over_512": row[511] / row[512]}
        log(f"[bench] alignment H={h}: " + " ".join(f"{c}:{u:.1f}" for c, u in row.items())
            + f" us; 513/512 = {row[513] / row[512]:.3f}")
    return out


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads")}
                for i in threadpool_info()]
        return blas, max([i["threads"] or 1 for i in blas] or [1])
    except Exception:
        return [], os.cpu_count()


class _Parity:
    """Running max / mean of |gpu - oracle| over compared elements."""

    def __init__(self):
        self.mx, self.tot, self.n = 0.0, 0.0, 0

    def add(self, gpu_bits, ref):
        g = (np.asarray(gpu_bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        e = np.abs(g - ref)
        self.mx = max(self.mx, float(e.max()))
        self.tot += float(e.sum())
        self.n += e.size

    def result(self):
        return {"max_abs": self.mx, "mean_abs": self.tot / max(1, self.n), "elements": self.n,
                "within_bar": self.mx <= 2e-2 and self.tot / max(1, self.n) <= 2e-3}


def cpu_baseline(gpu, budget_s=8.0):
    """The fp64 oracle on host cores, timed on the same workloads as the GPU
    legs of this run, and compared element by element with their GPU
    outputs (bar: max-abs 2e-2, mean-abs 2e-3):
      * headline: whole passes of the Llama-3-8B step (C=512 at H = 0, 4096,
        8192, 12288, all 32 query heads, including the page gather) until
        budget_s has passed -- `value` is its FLOP rate;
      * small: the 4/4-head d=64 chunk, in full;
      * predictor: the chunk walk over the 32768-token prompt (the oracle's
        schedule from the GPU fit's coefficients, checked equal to the
        library's) and the attention of every chunk, in full;
      * mixed: the LLaMA-13B mixed batch, every row, in full;
      * long_context (subset): the last 2048-token chunk (H = 30720) for the
        8 query heads of KV head 0, of the 64.
    gpu: dict of the GPU legs' outputs and times."""
    from chunked_prefill_attention_slot_amd.inputs import llama3_8b_chunk
    from oracle.attention import (causal_chunk_attention, gather_sequence, paged_attention,
                                  widen_bf16)
    from oracle.kv_cache import kv_write
    from oracle import predictor as opred
    blas, threads = _blas_threads()
    per = {}

    # headline step (config 2)
    prepared = []
    for h in HIST_SWEEP:
        b = llama3_8b_chunk(h)
        kc, vc = kv_write(b.k_cache, b.v_cache, b.k_new, b.v_new, b.slot_mapping, b.page_size)
        prepared.append((h, b, kc, vc))
    head_out = gpu.get("headline")
    passes = 0
    par = {h: _Parity() for h in HIST_SWEEP}
    t0 = time.perf_counter()
    while True:
        for h, b, kc, vc in prepared:
            n = h + CHUNK
            k = widen_bf16(gather_sequence(kc, b.block_table[0], n, b.page_size))
            v = widen_bf16(gather_sequence(vc, b.block_table[0], n, b.page_size))
            q = widen_bf16(b.q)
            for head in range(32):
                o = causal_chunk_attention(q[:, head], k[:, head // 4], v[:, head // 4], h,
                                           1.0 / math.sqrt(128))
                if passes == 0 and head_out is not None and h in head_out["outputs"]:
                    par[h].add(head_out["outputs"][h][:, head], o)
        passes += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    f = passes * sum(flops_chunk(32, 128, CHUNK, h) for h in HIST_SWEEP)
    per["headline"] = {"seconds": dt, "passes": passes, "oracle_tflops": f / dt / 1e12,
                       "oracle_ms_per_step": dt / passes * 1e3}
    if head_out is not None:
        per["headline"]["gpu_ms_per_step"] = head_out["ms_per_step"]
        per["headline"]["gpu_over_oracle"] = dt / passes * 1e3 / head_out["ms_per_step"]
        per["headline"]["parity_vs_gpu"] = {str(h): p.result() for h, p in par.items()}
    res = {"value": f / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{passes} pass(es) of the headline step (Llama-3-8B, C=512 at H=0/4096/"
                     f"8192/12288, all 32 query heads), fp64 NumPy oracle incl. gather; {dt:.1f} s",
           "seconds": dt, "cpu_count": os.cpu_count(), "blas": blas}
    try:
        res["affinity"] = len(os.sched_getaffinity(0))
    except Exception:
        res["affinity"] = os.cpu_count()

    def timed(name, fn, gpu_ms, flop, note):
        t = time.perf_counter()
        p = fn()
        d = time.perf_counter() - t
        per[name] = {"seconds": d, "flop": flop, "oracle_tflops": flop / d / 1e12 if flop else None,
                     "gpu_ms": gpu_ms, "gpu_over_oracle": d * 1e3 / gpu_ms if gpu_ms else None,
                     "covers": note, "parity_vs_gpu": p.result() if p is not None else None}
        log(f"[bench] cpu oracle {name}: {d:.2f} s"
            + (f", GPU {d * 1e3 / gpu_ms:.0f}x faster" if gpu_ms else "")
            + (f"; parity max_abs {p.mx:.2e} mean_abs {p.tot / max(1, p.n):.2e}" if p else ""))

    if "small" in gpu:
        b, out, us = gpu["small"]

        def run_small():
            p = _Parity()
            kc, vc = kv_write(b.k_cache, b.v_cache, b.k_new, b.v_new, b.slot_mapping, b.page_size)
            p.add(out, paged_attention(b.q, kc, vc, b.block_table, b.query_lens, b.seq_lens,
                                       b.num_kv_heads, b.page_size))
            return p
        timed("small", run_small, us * 1e-3, flops_chunk(4, 64, 64, 192), "every element")

    if "predictor" in gpu:
        b, chunks, out, fit, gpu_ms = gpu["predictor"]

        def run_pred():
            a, bb, c = fit
            cfg = opred.PredictorConfig(align=128)
            T = opred.target(a, bb, cfg.base_chunk_size)
            sched = opred.schedule(cfg, a, bb, T, b.num_tokens)
            per_chunks_equal = ([ch for _, ch, _ in sched] == chunks["chunk"] and
                                [L for L, _, _ in sched] == chunks["L"])
            p = _Parity()
            kc, vc = kv_write(b.k_cache, b.v_cache, b.k_new, b.v_new, b.slot_mapping, b.page_size)
            n = b.num_tokens
            k = widen_bf16(gather_sequence(kc, b.block_table[0], n, b.page_size))
            v = widen_bf16(gather_sequence(vc, b.block_table[0], n, b.page_size))
            q = widen_bf16(b.q)
            sc = 1.0 / math.sqrt(b.head_dim)
            for L, ch, _ in sched:
                for h in range(b.num_q_heads):
                    g = h // (b.num_q_heads // b.num_kv_heads)
                    o = causal_chunk_attention(q[L:L + ch, h], k[:L + ch, g], v[:L + ch, g], L, sc)
                    p.add(out[L:L + ch, h], o)
            per_chunks_ok.append(per_chunks_equal)
            return p
        per_chunks_ok = []
        n = b.num_tokens
        timed("predictor", run_pred, gpu_ms, 4.0 * b.num_q_heads * b.head_dim * n * n / 2.0,
              "oracle schedule + attention of every chunk of the align-128 walk, every element")
        per["predictor"]["schedule_equals_library"] = bool(per_chunks_ok[0])

    if "mixed" in gpu:
        b, out, us, pf_flops = gpu["mixed"]

        def run_mixed():
            p = _Parity()
            kc, vc = kv_write(b.k_cache, b.v_cache, b.k_new, b.v_new, b.slot_mapping, b.page_size)
            p.add(out, paged_attention(b.q, kc, vc, b.block_table, b.query_lens, b.seq_lens,
                                       b.num_kv_heads, b.page_size))
            return p
        timed("mixed", run_mixed, us * 1e-3, pf_flops,
              "every row (16 decode rows, 2 prefill chunks); flop counts the chunks only")

    if "long" in gpu:
        b, last, us_last = gpu["long"]

        def run_long():
            p = _Parity()
            kc, vc = kv_write(b.k_cache, b.v_cache, b.k_new, b.v_new, b.slot_mapping, b.page_size)
            n = b.num_tokens
            k = widen_bf16(gather_sequence(kc, b.block_table[0], n, b.page_size)[:, 0])
            v = widen_bf16(gather_sequence(vc, b.block_table[0], n, b.page_size)[:, 0])
            q = widen_bf16(b.q[30720:, :8])
            for h in range(8):
                p.add(last[:, h], causal_chunk_attention(q[:, h], k, v, 30720,
                                                         1.0 / math.sqrt(128)))
            return p
        # the GPU time of the same subset: the last chunk's call, 8 of its 64 heads
        timed("long_context_subset", run_long, us_last * 1e-3 * 8 / 64,
              flops_chunk(8, 128, 2048, 30720),
              "last chunk (H=30720), query heads 0-7 of 64; GPU time prorated by heads")
    res["per_config"] = per
    bars = [v.get("parity_vs_gpu") for v in per.values()]
    flat = [x for b_ in bars if b_ for x in (b_.values() if "max_abs" not in b_ else [b_])]
    if flat:
        res["parity_vs_gpu"] = {"max_abs": max(x["max_abs"] for x in flat),
                                "all_within_bar": all(x["within_bar"] for x in flat)}
    log(f"[bench] cpu oracle headline: {passes} passes in {dt:.1f} s -> {res['value']*1e3:.2f} "
        f"GFLOP/s on {threads} threads")
    return res


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling rocprofv3's FETCH_SIZE /
    WRITE_SIZE counters into bytes: each launch reads and writes nbytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": reps}), flush=True)


def kernel_source_digest(*paths):
    """sha256[:16] of one or more C++/HIP sources, in order, with comments and
    whitespace removed: it changes when the code does, not when only a
    comment does."""
    import hashlib
    import re
    h = hashlib.sha256()
    for path in paths:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


# The sources that decide what the prefill launch reads and writes: the
# kernel itself, the planner (tiles, splits, partial rows) and the shared
# layouts.
_CSRC = os.path.join(ROOT, "chunked_prefill_attention_slot_amd", "csrc")
TRAFFIC_SOURCES = tuple(os.path.join(_CSRC, f) for f in
                        ("prefill_attn.hip", "api.cpp", "cpa_internal.h"))


def load_traffic(sources=TRAFFIC_SOURCES):
    """HBM bytes per launch of the prefill kernel from the committed counter
    summary, or None if it was taken on different code."""
    path = os.path.join(ROOT, "profiles", "prefill_attn_llama3_8b_c512_traffic.txt")
    try:
        fields = dict(l.split(":", 1) for l in open(path).read().splitlines() if ":" in l)
    except OSError:
        return None, "no counter summary"
    sha = kernel_source_digest(*sources)
    if fields.get("kernel_code_digest", "").strip() != sha:
        return None, "kernel changed since the counters were taken"
    return float(fields["hbm_bytes_per_launch"]), fields.get("note", "").strip()


LEGS = ("headline", "small", "decode", "mixed", "long", "predictor", "schedule")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--decode-reps", type=int, default=30)
    ap.add_argument("--legs", default=",".join(LEGS),
                    help="comma-separated subset of " + ",".join(LEGS) +
                         " (the headline always runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--hist", type=int, nargs="+", default=list(HIST_SWEEP),
                    help="prefixes of the headline sweep (profiling subsets)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    legs = set(x for x in args.legs.split(",") if x)
    unknown = legs - set(LEGS)
    if unknown:
        ap.error(f"unknown legs {sorted(unknown)}")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(each GPU would run its own heads or sequences with no exchange).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration()
        return
    props = torch.cuda.get_device_properties(0)
    log(f"[bench] device {props.name} CUs={props.multi_processor_count}")
    t_start = time.perf_counter()

    head = headline(args)
    out = {
        "metric": "chunked-prefill attn TFLOP/s (% MFMA peak) at C=512, H=0..12k; decode GB/s",
        "value": head["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Llama-3-8B attention layer (32 q / 8 kv heads, d=128), "
                               "page 128, one 512-token chunk at each H in 0/4096/8192/12288; "
                               "KV write + attention per chunk in one call "
                               "(cpa_kv_write_attention)",
                   "chunk": CHUNK, "hist": list(args.hist), "page_size": 128},
        "roofline": head["roofline"], "per_H": head["per_H"],
        "ms_per_step_repeats": head["ms_per_step_repeats"],
        "ms_per_step_with_events": head["ms_per_step_with_events"],
        "ms_per_step_separate_calls": head["ms_per_step_separate_calls"],
    }
    traffic, note = load_traffic()
    out["roofline"]["traffic"] = traffic
    out["roofline"]["traffic_note"] = note
    # Algorithmic bytes per launch averaged over the sweep: K and V of every
    # visible key once, Q in, O out (bf16).
    alg = sum((h + CHUNK) * 8 * 128 * 2 * 2 + CHUNK * 32 * 128 * 2 * 2 for h in args.hist)
    out["roofline"]["algorithmic_bytes_per_launch"] = alg / len(args.hist)
    gpu = {"headline": {"outputs": head.pop("outputs"), "ms_per_step": head["ms_per_step"]}}
    if "small" in legs:
        out["small"], (b, o) = small_leg(args)
        gpu["small"] = (b, o, out["small"]["us_median"])
    if legs & {"decode", "mixed"}:
        from chunked_prefill_attention_slot_amd.inputs import mixed_llama13b
        from chunked_prefill_attention_slot_amd.device import DeviceBatch
        b = mixed_llama13b()
        mixed = (b, DeviceBatch(b))
        mixed[1].kv_write()
        torch.cuda.synchronize()
        if "decode" in legs:
            out["decode"] = decode_rows(args, mixed)
        if "mixed" in legs:
            out["mixed_batch"], o = mixed_leg(args, mixed)
            gpu["mixed"] = (b, o, out["mixed_batch"]["mixed_call_us"],
                            out["mixed_batch"]["prefill_flop"])
        del mixed
        torch.cuda.empty_cache()
    if "long" in legs:
        out["long_context"], (b, last) = long_context(args)
        gpu["long"] = (b, last, out["long_context"]["chunks"][-1]["us"])
        torch.cuda.empty_cache()
    if "predictor" in legs:
        # the workload as stated (4/4 heads, d=64, 16-token pages) ...
        out["predictor"], (b, chunks, o) = predictor_run(args)
        fit = out["predictor"]["fit"]
        gpu["predictor"] = (b, chunks, o, (fit["a"], fit["b"], fit["c"]),
                            float(sum(chunks["ms"])))
        torch.cuda.empty_cache()
        # ... and the same procedure at the headline layer
        out["predictor_llama3_8b"], _ = predictor_run(args, shape="llama3_8b", aligns=(128,))
        torch.cuda.empty_cache()
    if "schedule" in legs:
        out["chunk_schedule"] = {"step_loop": serving_run(args),
                                 "sizes_around_512": alignment_study(args)}
        torch.cuda.empty_cache()
    out["gpu_legs_seconds"] = time.perf_counter() - t_start
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(gpu)
    out["context_from_pages"] = {
        "note": "whole-model figures on A100 from the vLLM chunked-prefill article, "
                "section 2.1; not this kernel, not comparable",
        "llama13b_2048_token_prefill_ms": 120, "decode_ms_per_token": 25}
    out["total_seconds"] = time.perf_counter() - t_start
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
