#!/usr/bin/env python3
"""Benchmark: weight-absorbed MLA decode on one MI355X.

Workload: DeepSeek-V2 dims (128 heads, latent 512, rotary 64, head dim 128),
BF16 latent cache in 64-token pages shuffled across one pool, batch 64 with
per-request contexts uniform in [16,384, 32,768]; one decode step per request.
A step is the whole path: absorb_q -> decode_attn -> combine + out_up (one
launch, mla_combine_out_up), on one stream, inputs resident in HBM before
timing starts.

Prints one JSON line.  `value` is the latent-KV read rate of the whole step:
cache bytes read per step (each visible position's 1,152-byte item once) over
the step time.  Also reported: decode tokens/s, the attention kernel's own
rate against the HBM roofline (HIP events around every attention launch in
the timed region), the float64 CPU oracle timed on whole requests of the
same workload on the host cores (about 15 s of work), each launch's time with
the matrix-core utilisation of the attention and the weight rate of the two
head GEMMs ("parts"), and a plain streaming read for reference.  --long adds
one layer of the long-context workload (1 request x 131,072 positions);
--fp8-topk adds the FP8-cache, top-2,048 workload, with one scale per token
and, from the same draw, with one scale per 128 latent channels.  --indexer
adds the lightning indexer scan and top-k pick over 32 x 65,536 positions
(and, with --fp8-topk, the whole sparse decode step fed by its picks).
--prefill adds prefill of a 4,096-token prompt on the expanded path.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_FLOPS = 2.5e15  # dense MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attn_v2_batched_traffic.json")
# Sources that define the timed attention kernel (decode_bf16_kernel): the
# traffic counters are used only while they match.
KERNEL_SRCS = [os.path.join(ROOT, "mla_latent_kv_absorb_amd", "csrc", f)
               for f in ("decode_attn_bf16.hip", "attn_common.h", "tile_space.h", "mla_internal.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per attention launch from committed rocprofv3 counter runs,
    if they were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256_16") != kernel_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(inp, budget_s=15.0):
    """The float64 oracle, as it stands, on whole requests of the same
    workload (all heads, unabsorbed) on the host cores: requests 0, 1, ...
    until about budget_s seconds have passed.  Rate in the metric's unit:
    cache bytes of the requests done per second."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    item = (inp.D_C + inp.D_R) * 2
    done_bytes, done, positions = 0, 0, 0
    t0 = time.perf_counter()
    for b in range(inp.B):
        lo, hi = inp.request(b)
        oracle.decode_unabsorbed(inp.c_kv[lo:hi], inp.k_rope[lo:hi], inp.q_nope[b], inp.q_rope[b], inp.w_uk,
                                 inp.w_uv, inp.scale)
        done += 1
        positions += hi - lo
        done_bytes += (hi - lo) * item
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": round(done_bytes / dt / 1e9, 6),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"requests 0..{done - 1} of {inp.B} ({positions} positions, all {inp.H} heads) in "
                  f"{dt:.1f} s; float64 numpy, unabsorbed (expands keys and values per head)",
        "seconds_per_request": round(dt / done, 3),
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def read_ceiling(torch, gib=2, reps=10):
    """A plain streaming read for reference: torch's sum over a 2 GiB float64
    buffer resident in HBM (bytes read / time, HIP events); of the reductions
    tried it reads fastest."""
    x = torch.ones((gib << 30) // 8, dtype=torch.float64, device="cuda")
    x.sum()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        x.sum()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del x
    return {"GBps": round((gib << 30) / (ms * 1e-3) / 1e9, 1), "kind": "torch.sum over 2 GiB float64"}


def long_context_layer(torch, I, runner, num_cus, layers=4, reps=8):
    """One decode step of the long-context workload (1 request, 131,072
    positions) per layer: four independent layer draws are cycled so that
    every launch reads its cache from HBM rather than from the last-level
    cache.  Reports the average step time per layer and the per-token rate
    over the workload's 60 layers."""
    ws = []
    for layer in range(layers):
        inp = I.make_inputs("v2_long", layer=layer)
        ws.append(runner.DeviceWorkload(inp, split=True, num_cus=num_cus))
    cache_bytes = I.cache_bytes_read(inp)
    for w in ws:
        w.step_fused()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        for w in ws:
            w.step_fused()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (reps * layers)
    return {"us_per_layer": round(us, 2), "cache_GBps": round(cache_bytes / (us * 1e-6) / 1e9, 1),
            "tokens_per_s_60_layers": round(1e6 / (60 * us), 1), "workers": ws[0].plan.num_workers}


def fp8_topk_step(torch, I, runner, num_cus, inp, lists=8, reps=10):
    """The FP8-cache workload with a top-2,048 index list per request.  One
    step reads 42 MB out of a 1.35 GB pool, which would otherwise stay in the
    last-level cache, so the steps cycle over `lists` independently drawn
    index-list sets (338 MB of distinct rows).  Reports the step and attention
    times, the cache rate and both roofline fractions (HBM, and BF16 matrix
    cores: the FP8 latent is dequantised to BF16 for the MFMAs)."""
    w = runner.DeviceWorkload(inp, split=True, num_cus=num_cus)
    rng = np.random.default_rng(5005)
    sets = []
    for _ in range(lists):
        idx = np.stack([np.sort(rng.choice(int(inp.seq_lens[b]), inp.topk_idx.shape[1], replace=False))
                        for b in range(inp.B)]).astype(np.int32)
        sets.append(torch.from_numpy(idx).to(w.topk_idx.device))
    cache_bytes = I.cache_bytes_read(inp)
    n_pos = int(np.sum(inp.topk_idx >= 0))
    flop = float(n_pos) * 2 * inp.H * (inp.D_C + inp.D_R + inp.D_C)
    for t in sets:
        w.topk_idx = t
        w.step_fused()
    torch.cuda.synchronize()
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    att = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps * lists)]
    step_ev[0].record()
    for r in range(reps):
        for i, t in enumerate(sets):
            w.topk_idx = t
            w.absorb()
            att[r * lists + i][0].record()
            w.attend()
            att[r * lists + i][1].record()
            w.combine_up()
    step_ev[1].record()
    torch.cuda.synchronize()
    step_us = step_ev[0].elapsed_time(step_ev[1]) * 1e3 / (reps * lists)
    attn_us = float(np.mean([a.elapsed_time(b) for a, b in att])) * 1e3
    return {"step_us": round(step_us, 2), "attn_us": round(attn_us, 2),
            "cache_bytes_per_step": int(cache_bytes),
            "attn_cache_GBps": round(cache_bytes / (attn_us * 1e-6) / 1e9, 1),
            "attn_hbm_frac": round(cache_bytes / (attn_us * 1e-6) / (HBM_PEAK_GBPS * 1e9), 4),
            "attn_mfma_util": round(flop / (attn_us * 1e-6) / BF16_PEAK_FLOPS, 4),
            "tokens_per_s": round(inp.B / (step_us * 1e-6), 1), "workers": w.plan.num_workers}


def prefill_leg(torch, I, runner, T=4096, reps=10):
    """Prefill of a T-token prompt of one request at V2 dims on the expanded
    path: expansion of the cached latent per head (two GEMMs over the 512
    latent channels) and causal attention of the T queries.  Reports the time
    of each and their matrix-core rates (dense BF16 peak)."""
    inp = I.make_inputs("v2_single", ctx=(T, T))
    qn, qr = I.make_prefill_queries(inp, T, seed=56)
    w = runner.PrefillWorkload(inp, qn, qr)
    w.step()
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        w.expand()
        e[1].record()
        w.attend()
        e[2].record()
        ev.append(e)
    torch.cuda.synchronize()
    exp_us = float(np.median([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
    att_us = float(np.median([e[1].elapsed_time(e[2]) for e in ev])) * 1e3
    H = inp.H
    exp_flop = 2.0 * T * inp.D_C * H * (inp.D_N + inp.D_V)
    pairs = T * (T + 1) / 2.0                       # causal (query, key) pairs
    att_flop = 2.0 * pairs * H * (inp.D_N + inp.D_R + inp.D_V)
    return {"tokens": T, "expand_us": round(exp_us, 1), "attn_us": round(att_us, 1),
            "expand_TFLOPs": round(exp_flop / (exp_us * 1e-6) / 1e12, 1),
            "attn_TFLOPs": round(att_flop / (att_us * 1e-6) / 1e12, 1),
            "attn_mfma_util": round(att_flop / (att_us * 1e-6) / BF16_PEAK_FLOPS, 4),
            "prefill_tokens_per_s": round(T / ((exp_us + att_us) * 1e-6), 1)}


def cache_append_part(torch, I, w, reps=200):
    """mla_cache_append for the workload's 64 requests (one token each, with
    RoPE from float32 tables), timed after the decode steps; it rewrites each
    request's last cached position, so the timed steps are unaffected."""
    from mla_latent_kv_absorb_amd import binding as B
    inp = w.inp
    rows = int(inp.seq_lens.max())
    theta = 10000.0 ** (-np.arange(0, inp.D_R, 2) / inp.D_R)
    ang = np.arange(rows)[:, None] * theta[None, :]
    cos = torch.from_numpy(np.cos(ang).astype(np.float32)).cuda()
    sin = torch.from_numpy(np.sin(ang).astype(np.float32)).cuda()
    rng = np.random.default_rng(77)
    c_new = torch.from_numpy(rng.standard_normal((inp.B, inp.D_C)).astype(np.float32)).cuda().bfloat16()
    k_new = torch.from_numpy(rng.standard_normal((inp.B, inp.D_R)).astype(np.float32)).cuda().bfloat16()
    pos = (w.seq_lens - 1).contiguous()
    call = lambda: B.mla_cache_append(w.cfg, c_new, k_new, pos, w.pool, w.table, cos, sin)
    call()
    torch.cuda.synchronize()
    # A single call is shorter than its launch from Python, so the calls are
    # captured once in a HIP graph (the kernel records no memset) and the
    # replays are timed: device time per call, without the host's share.
    per_graph = 20
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(per_graph):
                call()
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps // per_graph):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (reps // per_graph * per_graph)
    return {"us": round(us, 2), "bytes_written": int(inp.B * (inp.D_C + inp.D_R) * 2),
            "timing": "HIP graph replays of 20 calls"}


def indexer_step(torch, I, runner, reps=10, layers=4, attn=None):
    """The lightning indexer over 32 requests x 65,536 positions (64 heads x
    128, FP8 search keys, 132 B per position), then the top-2,048 pick, as two
    calls and as one (mla_indexer_topk).  Four independent draws (277 MB of
    keys each) are cycled so the scans read HBM.  With ``attn`` (an FP8 top-k
    DeviceWorkload of the same shape) it also times the whole sparse decode
    step: scores and pick (one call), absorb, attention over the picked
    positions, merge + up-projection."""
    ws = []
    for layer in range(layers):
        inp = I.make_indexer_inputs(seed=600 + layer)
        ws.append(runner.IndexerWorkload(inp))
    key_bytes = I.key_bytes_read(inp)
    n_pos = int(np.sum(inp.seq_lens.astype(np.int64)))
    flop = float(n_pos) * 2 * inp.H_I * inp.d_I
    for w in ws:
        w.step()
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        for w in ws:
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            w.score()
            e[1].record()
            w.select()
            e[2].record()
            ev.append(e)
    torch.cuda.synchronize()
    score_us = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
    select_us = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e3
    # both steps as one call (the first histogram built by the score kernel)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        for w in ws:
            w.score_and_select()
    b.record()
    torch.cuda.synchronize()
    fused_us = a.elapsed_time(b) * 1e3 / (reps * layers)
    res = {"score_us": round(score_us, 2), "select_us": round(select_us, 2),
           "score_and_select_one_call_us": round(fused_us, 2),
           "key_bytes_per_step": int(key_bytes),
           "score_key_GBps": round(key_bytes / (score_us * 1e-6) / 1e9, 1),
           "score_hbm_frac": round(key_bytes / (score_us * 1e-6) / (HBM_PEAK_GBPS * 1e9), 4),
           "score_mfma_util": round(flop / (score_us * 1e-6) / BF16_PEAK_FLOPS, 4)}
    if attn is not None:
        # the picked lists of each draw drive the attention over the FP8 cache
        for w in ws:
            w.score_and_select()
            attn.topk_idx = w.idx
            attn.step_fused()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            for w in ws:
                w.score_and_select()
                attn.topk_idx = w.idx
                attn.step_fused()
        b.record()
        torch.cuda.synchronize()
        step_us = a.elapsed_time(b) * 1e3 / (reps * layers)
        res["sparse_decode_step_us"] = round(step_us, 2)
        res["sparse_decode_tokens_per_s"] = round(inp.B / (step_us * 1e-6), 1)
        res["sparse_decode_cache"] = attn.inp.cache_dtype
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device-to-device copy (counter calibration)")
    ap.add_argument("--long", action="store_true",
                    help="also time one layer of the long-context workload (1 request, 131,072 positions)")
    ap.add_argument("--prefill", action="store_true",
                    help="also time prefill of a 4,096-token prompt on the expanded path")
    ap.add_argument("--indexer", action="store_true",
                    help="also time the lightning indexer and top-k pick (32 x 65,536 positions), and with "
                         "--fp8-topk the whole sparse decode step")
    ap.add_argument("--fp8-topk", action="store_true",
                    help="also time the FP8-cache, top-2,048 workload (32 requests x 65,536 positions)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported in this build "
              "(the path shards by request with no communication; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(1)
    from mla_latent_kv_absorb_amd import inputs as I
    from mla_latent_kv_absorb_amd import runner

    t0 = time.time()
    inp = I.make_inputs("v2_batched")
    log(f"inputs drawn in {time.time() - t0:.1f} s; contexts {inp.seq_lens.min()}..{inp.seq_lens.max()}")
    num_cus = torch.cuda.get_device_properties(0).multi_processor_count
    w = runner.DeviceWorkload(inp, split=True, num_cus=num_cus)
    torch.cuda.synchronize()
    log(f"resident on GPU after {time.time() - t0:.1f} s; workers {w.plan.num_workers}, "
        f"workspace {w.plan.workspace_bytes / 1e6:.1f} MB")
    cache_bytes = I.cache_bytes_read(inp)

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        w.step_fused()
    torch.cuda.synchronize()
    log("warmup done")

    stream = torch.cuda.current_stream()
    # events between the three launches of every timed step, on the launch
    # stream: absorb, attention, merge + up-projection (one launch)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        ev[k][0].record(stream)
        w.absorb()
        ev[k][1].record(stream)
        w.attend()
        ev[k][2].record(stream)
        w.combine_up()
        ev[k][3].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(stop)
    part_ms = lambda i: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in ev]))
    absorb_ms, attn_avg_ms, tail_ms = part_ms(0), part_ms(1), part_ms(2)
    ms_per_step = total_ms / args.steps
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (wall {wall:.3f} s), "
        f"attention {attn_avg_ms * 1e3:.1f} us")

    gbps = cache_bytes / (ms_per_step * 1e-3) / 1e9
    attn_gbps = cache_bytes / (attn_avg_ms * 1e-3) / 1e9
    tokens_per_s = inp.B / (ms_per_step * 1e-3)

    # matrix-core view of the same launches (dense BF16 peak), and the head
    # GEMMs against their weight read
    attn_flop = float(np.sum(inp.seq_lens.astype(np.int64))) * 2 * inp.H * (inp.D_C + inp.D_R + inp.D_C)
    gemm_flop = 2.0 * inp.B * inp.H * inp.D_C * inp.D_N
    w_bytes = inp.H * inp.D_C * inp.D_N * 2
    gemm = lambda ms, act_bytes: {"us": round(ms * 1e3, 2), "weight_GBps": round(w_bytes / (ms * 1e-3) / 1e9, 1),
                                  "bytes_GBps": round((w_bytes + act_bytes) / (ms * 1e-3) / 1e9, 1),
                                  "mfma_util": round(gemm_flop / (ms * 1e-3) / BF16_PEAK_FLOPS, 5)}
    part_bytes = w.plan.num_slots * inp.H * (inp.D_C * 2 + 4)  # BF16 partials + lse
    parts = {
        "absorb": gemm(absorb_ms, inp.B * inp.H * (inp.D_N + inp.D_C) * 2),
        "attention": {"us": round(attn_avg_ms * 1e3, 2), "mfma_util": round(attn_flop / (attn_avg_ms * 1e-3) / BF16_PEAK_FLOPS, 4)},
        "combine_out_up": gemm(tail_ms, part_bytes + inp.B * inp.H * inp.D_V * 2),
    }
    parts["cache_append"] = cache_append_part(torch, I, w)
    ceiling = read_ceiling(torch)
    long_layer = long_context_layer(torch, I, runner, num_cus) if args.long else None
    fp8 = fp8g = None
    if args.fp8_topk:
        # one draw, both FP8 formats: one scale per token, and one per 128
        # latent channels (the 656-byte item)
        fp8_inp = I.make_inputs("v2_fp8_topk")
        fp8 = fp8_topk_step(torch, I, runner, num_cus, fp8_inp)
        g_inp = I.requantize(fp8_inp, I.DTYPE_FP8_G128)
        del fp8_inp
        fp8g = fp8_topk_step(torch, I, runner, num_cus, g_inp)
    pre = prefill_leg(torch, I, runner) if args.prefill else None
    idx = None
    if args.indexer:
        attn = runner.DeviceWorkload(g_inp, split=True, num_cus=num_cus) if args.fp8_topk else None
        idx = indexer_step(torch, I, runner, attn=attn)
        del attn

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on whole requests (about 15 s)")
        cpu = cpu_baseline(inp)

    result = {
        "metric": "MLA decode latent-KV read GB/s (% HBM peak) + tokens/s, B=64 ctx=32K",
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) latents/rotary keys/queries, N(0,1/512) weights)",
        "config": {
            "workload": "V2-dims batched decode: B=64, contexts uniform in [16384, 32768] "
                        "(seeded), BF16 latent cache, 64-token pages shuffled in one pool, "
                        "H=128, D_C=512, D_R=64, D_N=D_V=128",
            "global_batch": int(inp.B),
            "seq_len": int(inp.seq_lens.max()),
            "total_context": int(inp.seq_lens.sum()),
            "cache_bytes_per_step": int(cache_bytes),
            "parallelism": "single GPU; split-KV over %d workers" % w.plan.num_workers,
        },
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(tokens_per_s, 1),
        "attn_us": round(attn_avg_ms * 1e3, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": "mla_decode_attn (decode_bf16_kernel<split>)",
            "achieved": round(attn_gbps, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(attn_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic_from_profile(),
        },
        "cpu_baseline": cpu,
        "parts": parts,
        "read_ceiling": ceiling,
    }
    if long_layer is not None:
        result["v2_long_layer"] = long_layer
    if fp8 is not None:
        result["fp8_topk_step"] = fp8
        result["fp8_g128_topk_step"] = fp8g
    if idx is not None:
        result["indexer_step"] = idx
    if pre is not None:
        result["prefill_4096"] = pre
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
