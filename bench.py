"""Bench: paged chunked-prefill attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--extras] [--no-cpu]

One step = one pass of the hot path over the headline workload: a
Llama-3-8B attention layer (32 q / 8 kv heads, d=128, bf16, 128-token
pages) taking one 512-token chunk at each prefix H in {0, 4096, 8192,
12288} (the history sweep of the dynamic-chunking design's problem
statement; 512-token chunks of the vLLM chunked-prefill article): for each
H, the chunk's K/V are written into the paged cache through slot_mapping,
then attention runs over prefix + chunk. Metadata planning and upload
happen once per workload, outside the timed region (a plan serves every
layer of a batch step). Inputs are resident in HBM before timing starts.

The printed JSON line (last line of stdout) carries:
  value      -- algorithmic TFLOP/s of the whole step (KV writes included),
                FLOP per chunk = 4*Hq*d*C*(H + C/2), over K steps timed
                with no events between the launches;
  roofline   -- the step's call (cpa_kv_write_attention: the prefill MFMA
                kernel with the KV write inside, then the split combine)
                against bf16 dense MFMA peak, averaged over the four H, its
                duration from HIP events in a second pass of K steps;
  decode     -- LLaMA-13B decode rows (16 rows, seq_len U[1024, 8192],
                40/40 heads): algorithmic K+V+Q+O bytes / time vs HBM peak;
  cpu_baseline -- the fp64 oracle on a bounded sample of the H=12288 chunk.
--extras adds the mixed batch, the 70B-like long-context sweep, the
chunk-size predictor runs, the token-budget step loop under four chunk
rules and the chunk-size sweep around 512 as extra fields (--serving adds
only the last two).
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
    # Per-launch durations first (they also finish warming the clocks): K
    # steps with one event before the first call and one after every call,
    # on the launch stream (torch's current stream); each call's time is the
    # span between the events that bracket it, so it includes its launch and
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
    # Timed regions: K steps exactly as a caller issues them, with no event
    # between the launches (a recorded event costs 1.5-2 us of stream time,
    # its own packet between two kernels). The fused step is timed
    # REPEATS times after the event passes; `value` is the first of these,
    # and every repeat is reported.
    walls = []
    for _ in range(REPEATS):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
    wall = walls[0]
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
        cm = sum(c) / len(c)
        call_ms_tot += cm
        per_h.append({"H": h, "call_us_mean": cm * 1e3, "call_us_median": c[len(c) // 2] * 1e3,
                      "attn_us_mean": sum(a) / len(a) * 1e3,
                      "kv_write_us_mean": sum(kv) / len(kv) * 1e3,
                      "tflops": flops[i] / (cm * 1e-3) / 1e12,
                      "mfma_frac": flops[i] / (cm * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS})
        log(f"[bench] H={h}: kv_write_attention {cm*1e3:.1f} us -> {per_h[-1]['tflops']:.1f} "
            f"TFLOP/s ({100*per_h[-1]['mfma_frac']:.1f}% of bf16 peak); separate calls: "
            f"kv_write {per_h[-1]['kv_write_us_mean']:.1f} us + attention "
            f"{per_h[-1]['attn_us_mean']:.1f} us")
    ms_per_step = wall * 1e3 / args.steps
    log(f"[bench] step: {ms_per_step*1e3:.1f} us without events (repeats "
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
                               "combine_kernel<128>)",
                     "flop_per_launch": total_flops / n},
    }


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


def mixed_extras(args, mixed):
    import torch
    from chunked_prefill_attention_slot_amd import binding as cpa
    b, db = mixed
    r_all = median_ms(db.bound()[1], args.decode_reps, 3)
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
    res = {"mixed_call_us": r_all["mean_ms"] * 1e3,
           "prefill_only_us": r_pf["mean_ms"] * 1e3,
           "prefill_only_tflops": pf_flops / (r_pf["mean_ms"] * 1e-3) / 1e12}
    log(f"[bench] llama13b mixed call {res['mixed_call_us']:.1f} us; prefill chunks alone "
        f"{res['prefill_only_us']:.1f} us = {res['prefill_only_tflops']:.1f} TFLOP/s")
    # Two micro-batches (dual-stream article, section 3.1) on two streams.
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
    return res


def long_context(args):
    """70B-like layer (64 q / 8 kv heads): one 32768-token prompt prefilled in
    16 chunks of 2048; each chunk = KV write + attention."""
    import torch
    from chunked_prefill_attention_slot_amd import binding as cpa
    from chunked_prefill_attention_slot_amd.inputs import make_batch
    from chunked_prefill_attention_slot_amd.device import DeviceBatch
    b = make_batch(5, num_q_heads=64, num_kv_heads=8, head_dim=128, page_size=128,
                   query_lens=[32768], seq_lens=[32768])
    db = DeviceBatch(b)
    rows = []
    tot_f, tot_ms = 0.0, 0.0
    for c in range(16):
        h = 2048 * c
        plan = cpa.cpa_plan_create(db.desc, [2048], [h + 2048])
        ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
        cpa.cpa_plan_upload(plan, ws)
        sl = slice(h, h + 2048)
        kn, vn, sm = db.k_new[sl], db.v_new[sl], db.slot_mapping[sl]
        q, out = db.q[sl], db.out[sl]

        kv_write = cpa.bind_kv_write(db.desc, kn, vn, sm, db.k_cache, db.v_cache)
        attention = cpa.bind_attention(plan, q, db.k_cache, db.v_cache, db.block_table, out, ws)

        def chunk():
            kv_write()
            attention()
        r = median_ms(chunk, 10, 2)
        f = flops_chunk(64, 128, 2048, h)
        tot_f += f
        tot_ms += r["median_ms"]
        rows.append({"H": h, "us": r["median_ms"] * 1e3,
                     "tflops": f / (r["median_ms"] * 1e-3) / 1e12})
    res = {"chunks": rows, "total_ms": tot_ms, "tflops": tot_f / (tot_ms * 1e-3) / 1e12,
           "mfma_frac": tot_f / (tot_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    log(f"[bench] 70b-like 16x2048: {tot_ms:.2f} ms total, {res['tflops']:.1f} TFLOP/s")
    return res


PREDICTOR_SHAPES = {
    # the profiling shape of the predictor workload: 4/4 heads, d=64, page 16
    "tiny": dict(num_q_heads=4, num_kv_heads=4, head_dim=64, page_size=16),
    # a Llama-3-8B attention layer, where the chunk cost grows with history
    "llama3_8b": dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=128),
}


def chunk_runner(db, cpa, torch):
    """runner(L, c) -> a closure doing KV write + attention of the chunk
    [L, L + c) of db's single sequence."""
    def runner(L, c):
        plan = cpa.cpa_plan_create(db.desc, [c], [L + c])
        ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
        cpa.cpa_plan_upload(plan, ws)
        sl = slice(L, L + c)
        kn, vn, sm, q, out = db.k_new[sl], db.v_new[sl], db.slot_mapping[sl], db.q[sl], db.out[sl]

        kv_write = cpa.bind_kv_write(db.desc, kn, vn, sm, db.k_cache, db.v_cache)
        attention = cpa.bind_attention(plan, q, db.k_cache, db.v_cache, db.block_table, out, ws)

        def f():
            kv_write()
            attention()
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


def predictor_run(args, align=128, shape="tiny", prompt=32768):
    """Startup profiling at 64 sizes (2048 down to 32, H=0) of KV write +
    attention, least-squares fit, target T = f(2048) - f(0), then a prompt
    prefilled with predicted chunks (one-variable model); then the same
    prompt again with online calibration of the two-variable model f(C,H)
    (refitted from each chunk's measured time once 5 are held; before that
    the one-variable model sizes the chunks). Reports measured/T per chunk."""
    import torch
    from chunked_prefill_attention_slot_amd import binding as cpa
    from chunked_prefill_attention_slot_amd.inputs import make_batch
    from chunked_prefill_attention_slot_amd.device import DeviceBatch
    b = make_batch(3, query_lens=[prompt], seq_lens=[prompt], **PREDICTOR_SHAPES[shape])
    db = DeviceBatch(b)
    runner = chunk_runner(db, cpa, torch)

    sizes, ms, (a, bb, c) = profile_fit(runner)
    cfg = cpa.predictor_cfg(align=align)
    T = cpa.cpa_predictor_target(cfg, a, bb)
    f_base = a * 2048.0 * 2048.0 + bb * 2048.0 + c   # modelled latency of a base chunk at H=0

    def f_model(x):
        return a * x * x + bb * x + c

    def summary(chunks, key):
        r = np.array([cch[key] for cch in chunks])
        return {"min": float(r.min()), "max": float(r.max()), "mean": float(r.mean()),
                "cv": float(r.std() / r.mean()),
                "frac_within_10pct": float(np.mean(np.abs(r - 1) <= 0.1))}

    chunks = []
    L = 0
    while L < prompt:
        ch, x = cpa.cpa_predictor_next_chunk(cfg, a, bb, T, L, prompt - L)
        if ch <= 0:
            break
        m = median_ms(runner(L, ch), 11, 2)["median_ms"]
        model_ratio = (f_model(L + ch) - f_model(L)) / T
        chunks.append({"L": L, "chunk": ch, "raw_x": x, "ms": m, "meas_over_T": m / T,
                       "model_over_T": model_ratio, "meas_over_f_base": m / f_base,
                       "alignment_limited": model_ratio < 0.9})
        L += ch
    r = np.array([cch["meas_over_T"] for cch in chunks])
    ok = np.array([not cch["alignment_limited"] for cch in chunks])

    # Online calibration of f(C, H) = a*C*(C+H) + b*(C+H) + c over the same prompt.
    calib = cpa.Calib(min_points=5, window=30)
    online = []
    L = 0
    while L < prompt:
        try:
            a2, b2, c2 = calib.model()
            T2 = cpa.cpa_calib_target(cfg, a2, b2, c2)
            ch, x = cpa.cpa_calib_next_chunk(cfg, a2, b2, c2, T2, L, prompt - L)
            src = "online"
        except cpa.CpaError:
            ch, x = cpa.cpa_predictor_next_chunk(cfg, a, bb, T, L, prompt - L)
            src = "profiled"
        if ch <= 0:
            break
        m = median_ms(runner(L, ch), 11, 2)["median_ms"]
        try:
            calib.record(cpa.cpa_calib_features([ch], [L]), m)
            refit = True
        except cpa.CpaError:
            refit = False   # window does not determine the model (e.g. one chunk size)
        online.append({"L": L, "chunk": ch, "raw_x": x, "ms": m, "model": src, "refit": refit,
                       "meas_over_f_base": m / f_base})
        L += ch
    try:
        a2, b2, c2 = calib.model()
    except cpa.CpaError:
        a2 = b2 = c2 = None

    res = {"shape": shape, "prompt": prompt, "align": align, "fit": {"a": a, "b": bb, "c": c},
           "T_ms": T, "f_base_ms": f_base,
           "profile_ms": dict(zip(map(int, sizes), ms)), "num_chunks": len(chunks),
           "meas_over_T": summary(chunks, "meas_over_T"),
           "frac_within_10pct": float(np.mean(np.abs(r - 1) <= 0.1)),
           "frac_within_10pct_not_alignment_limited":
               float(np.mean(np.abs(r[ok] - 1) <= 0.1)) if ok.any() else None,
           "meas_over_f_base": summary(chunks, "meas_over_f_base"),
           "chunks": chunks,
           "online": {"num_chunks": len(online), "final_fit": {"a": a2, "b": b2, "c": c2},
                      "refused_refits": sum(1 for o in online if not o["refit"]),
                      "meas_over_f_base": summary(online, "meas_over_f_base"),
                      "chunks": online}}
    log(f"[bench] predictor {shape} align {align}: a={a:.3e} b={bb:.3e} c={c:.3e} T={T:.4f} ms, "
        f"{len(chunks)} chunks, meas/T in [{r.min():.2f}, {r.max():.2f}]; online: "
        f"{len(online)} chunks, meas/f(base) cv {res['online']['meas_over_f_base']['cv']:.3f} "
        f"vs {res['meas_over_f_base']['cv']:.3f}")
    return res


LLAMA3_8B = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=128)


def step_loop(requests, budget, rule, fit, seed=7, align=128):
    """One pass of the token-budget step loop (vLLM chunked-prefill article,
    section 3.1) over a request stream at the Llama-3-8B layer: libcpa's
    batch former forms each step, the stream lays out its metadata, and the
    step's KV write + attention run on one cache kept across steps. Each
    step's GPU time comes from events around its two calls, after which the
    host waits for the step (so host work is outside the figure). rule is
    ("fixed", size) | ("progressive", sizes) | ("predictor",) |
    ("calibrated",): the last refits f(C, H) online from every step's
    features and time and hands the model to the former."""
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
            r = step_loop(reqs, 2048, rule, fit)
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


def cpu_baseline(budget_s=10.0, gpu_outputs=None):
    """The fp64 oracle on host cores over the headline step: the Llama-3-8B
    chunk at H = 0, 4096, 8192, 12288, every query head, repeated until
    budget_s seconds have passed (whole passes only). Its first pass is also
    compared element by element with the outputs of the timed GPU steps
    (gpu_outputs: H -> bf16 bits [512, 32, 128])."""
    from chunked_prefill_attention_slot_amd.inputs import llama3_8b_chunk
    from oracle.attention import causal_chunk_attention, gather_sequence, widen_bf16
    from oracle.kv_cache import kv_write
    try:
        from threadpoolctl import threadpool_info
        blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads")}
                for i in threadpool_info()]
        threads = max([i["threads"] or 1 for i in blas] or [1])
    except Exception:
        blas, threads = [], os.cpu_count()
    prepared = []
    for h in HIST_SWEEP:
        b = llama3_8b_chunk(h)
        kc, vc = kv_write(b.k_cache, b.v_cache, b.k_new, b.v_new, b.slot_mapping, b.page_size)
        prepared.append((h, b, kc, vc))
    passes = 0
    parity = {}
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
                if passes == 0 and gpu_outputs is not None and h in gpu_outputs:
                    g = (gpu_outputs[h][:, head].astype(np.uint32) << 16).view(np.float32)
                    e = np.abs(g.astype(np.float64) - o)
                    acc = parity.setdefault(h, [0.0, 0.0, 0])
                    acc[0] = max(acc[0], float(e.max()))
                    acc[1] += float(e.sum())
                    acc[2] += e.size
        passes += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    f = passes * sum(flops_chunk(32, 128, CHUNK, h) for h in HIST_SWEEP)
    try:
        aff = len(os.sched_getaffinity(0))
    except Exception:
        aff = os.cpu_count()
    res = {"value": f / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{passes} pass(es) of the headline step (Llama-3-8B, C=512 at H=0/4096/"
                     f"8192/12288, all 32 query heads), fp64 NumPy oracle incl. gather; {dt:.1f} s",
           "seconds": dt, "cpu_count": os.cpu_count(), "affinity": aff, "blas": blas}
    if parity:
        res["parity_vs_gpu"] = {
            "note": "oracle vs the timed GPU steps' bf16 outputs, every element; bar: "
                    "max-abs 2e-2, mean-abs 2e-3",
            "per_H": {str(h): {"max_abs": m, "mean_abs": t / c} for h, (m, t, c) in parity.items()},
            "max_abs": max(m for m, _, _ in parity.values()),
            "mean_abs": sum(t for _, t, _ in parity.values()) / sum(c for _, _, c in parity.values())}
        log(f"[bench] parity of the timed steps vs the oracle: max_abs "
            f"{res['parity_vs_gpu']['max_abs']:.2e}, mean_abs {res['parity_vs_gpu']['mean_abs']:.2e}")
    log(f"[bench] cpu oracle: {passes} passes in {dt:.1f} s -> {res['value']*1e3:.2f} GFLOP/s")
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--decode-reps", type=int, default=30)
    ap.add_argument("--extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--hist", type=int, nargs="+", default=list(HIST_SWEEP),
                    help="prefixes of the headline sweep (profiling subsets)")
    ap.add_argument("--serving", action="store_true",
                    help="add the step-loop and chunk-alignment legs (also part of --extras)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
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
    if not args.no_decode or args.extras:
        from chunked_prefill_attention_slot_amd.inputs import mixed_llama13b
        from chunked_prefill_attention_slot_amd.device import DeviceBatch
        b = mixed_llama13b()
        mixed = (b, DeviceBatch(b))
        mixed[1].kv_write()
        torch.cuda.synchronize()
        if not args.no_decode:
            out["decode"] = decode_rows(args, mixed)
        if args.extras:
            out["mixed_batch"] = mixed_extras(args, mixed)
        del mixed
        torch.cuda.empty_cache()
    if args.extras:
        out["long_context"] = long_context(args)
        out["predictor"] = predictor_run(args, 128)
        out["predictor_align16"] = predictor_run(args, 16)
        out["predictor_llama3_8b"] = predictor_run(args, 128, shape="llama3_8b")
    if args.extras or args.serving:
        out["step_loop"] = serving_run(args)
        out["alignment"] = alignment_study(args)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(gpu_outputs=head.pop("outputs"))
    out["context_from_pages"] = {
        "note": "whole-model figures on A100 from the vLLM chunked-prefill article, "
                "section 2.1; not this kernel, not comparable",
        "llama13b_2048_token_prefill_ms": 120, "decode_ms_per_token": 25}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
