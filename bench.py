#!/usr/bin/env python3
"""Benchmark: weight-absorbed MLA decode on one MI355X.

Headline workload: DeepSeek-V2 dims (128 heads, latent 512, rotary 64, head
dim 128), BF16 latent cache in 64-token pages shuffled across one pool, batch
64 with per-request contexts uniform in [16,384, 32,768]; one decode step per
request.  A step is the whole path: absorb_q -> decode_attn -> combine +
out_up (one launch, mla_combine_out_up), on one stream, inputs resident in HBM
before timing starts.  Before the W warmup steps, untimed steps run for
--settle-s seconds so the GPU clock has left its idle level; a clock probe
around the timed region reports the mean shader clock over it.

Prints one JSON line.  `value` is the latent-KV read rate of the whole step:
cache bytes read per step (each visible position's 1,152-byte item once) over
the step time.  Also reported: decode tokens/s, the attention kernel's own
rate against the HBM roofline (HIP events around every attention launch in
the timed region), each launch's time (mean and median) with the matrix-core
utilisation of the attention and the weight rate of the two head GEMMs
("parts"), a hand-written streaming read for reference, and the float64 CPU
oracle on whole requests of the same workload on the host cores.

`configs` times the other workloads in the same process, each beside its
oracle time: the tiny float32 step; the single 4,096-token request (cycled
over 64 pool copies so it reads HBM); one token of the 131,072-token workload
over 60 independent layers (one HIP graph); the FP8 top-2,048 workload with
one scale per position and with one per 128 channels.  The long-context and
FP8 workloads are drawn on the device (see device_inputs.py).  --indexer adds
the lightning indexer scan and pick, and the sparse decode step they feed;
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
               for f in ("decode_attn_bf16.hip", "attn_common.h", "tile_space.h", "mla_internal.h", "mla_args.h")]


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


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def _oracle_requests(inp, requests):
    """Run the float64 oracle on whole requests (all heads, unabsorbed);
    returns per-request seconds."""
    import oracle
    times = []
    for b in requests:
        lo, hi = inp.request(b)
        if inp.cache_dtype in ("fp8_e4m3", "fp8_e4m3_g128"):
            c = oracle.dequant_fp8_latent(inp.c_codes[lo:hi], inp.c_scales[lo:hi])
        else:
            c = inp.c_kv[lo:hi]
        picked = None if inp.topk_idx is None else inp.topk_idx[b]
        t = time.perf_counter()
        oracle.decode_unabsorbed(c, inp.k_rope[lo:hi], inp.q_nope[b], inp.q_rope[b], inp.w_uk, inp.w_uv,
                                 inp.scale, picked=picked)
        times.append(time.perf_counter() - t)
    return times


def cpu_baseline(inp, budget_s=12.0, full=False):
    """The float64 oracle, as it stands, on whole requests of the batched
    workload (all heads, unabsorbed) on the host cores: requests 0, 1, ...
    until about budget_s seconds have passed (every request with full=True).
    Rate in the metric's unit: cache bytes of the requests done per second
    (their total over their total time; the median per-request rate is given
    beside it)."""
    item = (inp.D_C + inp.D_R) * 2
    times, done = [], []
    t0 = time.perf_counter()
    for b in range(inp.B):
        times += _oracle_requests(inp, [b])
        done.append(b)
        if not full and time.perf_counter() - t0 >= budget_s:
            break
    lens = np.array([int(inp.seq_lens[b]) for b in done], dtype=np.float64)
    t = np.array(times)
    return {
        "value": round(float(lens.sum()) * item / t.sum() / 1e9, 6),
        "unit": "GB/s",
        "cores": _blas_threads(),
        "kind": "oracle",
        "sample": (f"all {inp.B} requests" if len(done) == inp.B else f"requests 0..{done[-1]} of {inp.B}")
                  + f" ({int(lens.sum())} positions, all {inp.H} heads) in {t.sum():.1f} s; float64 numpy, "
                    "unabsorbed (expands keys and values per head)",
        "median_GBps_per_request": round(float(np.median(lens * item / t)) / 1e9, 6),
        "seconds_per_request_median": round(float(np.median(t)), 3),
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def cpu_baselines_other(I):
    """The oracle on the other configurations, on the host cores: the tiny
    float32 one and the single 4,096-token request in full, one layer of the
    131,072-token workload (times 60 for a token), and the sparse FP8
    workload's 32 requests x 2,048 picked positions (the oracle reads only the
    picked rows, so the context is drawn at 4,096 positions to keep the host
    draw short; the work timed is that of the full workload)."""
    res = {}
    cores = _blas_threads()

    def one(name, inp, item, scale_to=1, note=""):
        t = _oracle_requests(inp, list(range(inp.B)))
        n = int(np.sum(inp.topk_idx >= 0)) if inp.topk_idx is not None else int(np.sum(inp.seq_lens))
        total = float(np.sum(t)) * scale_to
        res[name] = {"seconds": round(total, 4), "GBps": round(n * item * scale_to / total / 1e9, 6),
                     "cores": cores, "kind": "oracle", "sample": note}

    one("tiny_fp32", I.make_inputs("tiny_fp32"), (16 + 8) * 4, note="the whole step (1 request x 64 positions)")
    one("v2_single", I.make_inputs("v2_single"), 1152, note="the whole step (1 request x 4,096 positions)")
    one("v2_long_token", I.make_inputs("v2_long", layer=0), 1152, scale_to=60,
        note="layer 0 (131,072 positions, all heads) timed, times 60 layers per token")
    one("v2_fp8_topk", I.make_inputs("v2_fp8_topk", ctx=(4096, 4096)), 644,
        note="32 requests x 2,048 picked positions (all heads); contexts drawn at 4,096")
    return res


class ClockProbe:
    """Mean shader clock over a region of the stream: each probe launch records
    s_memtime (shader clock counter) and s_memrealtime (100 MHz) per XCD;
    the clock over the region is delta(memtime) / delta(realtime) between two
    probes, per XCD.  Also drives the hand-written streaming read."""

    GROUPS = 256

    def __init__(self, torch):
        import ctypes
        path = os.path.join(ROOT, "mla_latent_kv_absorb_amd", "libmla_bench.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run the build first")
        self.lib = ctypes.CDLL(path)
        self.lib.mlab_clock_probe.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
        self.lib.mlab_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p,
                                              ctypes.c_void_p]
        self.lib.mlab_stamp.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.torch = torch
        self.bufs = []

    def mark(self):
        t = self.torch.zeros(self.GROUPS * 4, dtype=self.torch.int64, device="cuda")
        st = self.lib.mlab_clock_probe(t.data_ptr(), self.GROUPS, self.torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"clock probe failed ({st})")
        self.bufs.append(t)
        return len(self.bufs) - 1

    def mhz(self, i0, i1):
        """Mean clock between two marks, from the work-groups of the two probes
        that ran on the same compute unit (same XCD, shader engine, array and
        CU id): the median over those units, with the per-XCD medians."""
        a = self.bufs[i0].cpu().numpy().reshape(-1, 4)
        b = self.bufs[i1].cpu().numpy().reshape(-1, 4)
        unit = lambda r: (int(r[2]), int(r[3]) & 0xFF00)   # xcc, (se, sh, cu) bits of HW_ID
        first = {}
        for r in a:
            first.setdefault(unit(r), r)
        per_unit = []
        for r in b:
            u = unit(r)
            if u in first:
                dm, dr = float(r[0] - first[u][0]), float(r[1] - first[u][1])
                if dr > 0 and dm > 0:
                    per_unit.append((u[0], dm / dr * 100.0))
        if not per_unit:
            return {"mean_MHz": None, "units": 0}
        vals = np.array([v for _, v in per_unit])
        per_xcd = {}
        for x in sorted({x for x, _ in per_unit}):
            per_xcd[str(x)] = round(float(np.median([v for xx, v in per_unit if xx == x])), 1)
        return {"mean_MHz": round(float(np.median(vals)), 1), "units": len(per_unit), "per_xcd_MHz": per_xcd,
                "realtime_ticks": int(np.median(b[:, 1]) - np.median(a[:, 1]))}

    def stamp(self, buf, i):
        """Real-time stamp (100 MHz ticks) into buf[i] when the stream gets there."""
        st = self.lib.mlab_stamp(buf.data_ptr() + 8 * i, self.torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"stamp failed ({st})")

    def stream_read(self, buf, groups):
        sink = self.torch.zeros(groups, dtype=self.torch.int32, device="cuda")
        st = self.lib.mlab_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), groups, sink.data_ptr(),
                                       self.torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"stream read failed ({st})")


def _run_ms(torch, fn, reps):
    """Average time of fn() over reps back-to-back calls, HIP events only at
    the two ends (an event between launches adds a gap and a cache flush)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def _graph_ms(torch, calls, reps):
    """Average time per call of a list of launches captured once in a HIP
    graph and replayed reps times (HIP events at the two ends): for legs whose
    launches are shorter than their launch from Python.  None of the captured
    calls records a memset."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for c in calls:
                c()
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    ms = _run_ms(torch, g.replay, reps)
    del g
    return ms / len(calls)


def _median_ms(torch, fn, reps):
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    return float(np.median(ms))


def read_ceiling(torch, probe, gib=4, reps=10):
    """A plain streaming read for reference, written here: every byte of a
    4 GiB buffer resident in HBM loaded once with 16-byte loads (median over
    reps, HIP events).  torch's float64 sum over the same buffer is given
    beside it."""
    x = torch.ones((gib << 30) // 8, dtype=torch.float64, device="cuda")
    nbytes = gib << 30
    out = {}
    for groups in (1024, 2048, 4096):
        probe.stream_read(x, groups)
        torch.cuda.synchronize()
        out[groups] = nbytes / (_median_ms(torch, lambda: probe.stream_read(x, groups), reps) * 1e-3) / 1e9
    best = max(out, key=out.get)
    x.sum()
    torch.cuda.synchronize()
    torch_gbps = nbytes / (_median_ms(torch, lambda: x.sum(), reps) * 1e-3) / 1e9
    del x
    return {"GBps": round(out[best], 1), "kind": f"hand-written streaming read, 4 GiB, {best} work-groups",
            "by_groups_GBps": {str(k): round(v, 1) for k, v in out.items()},
            "torch_sum_GBps": round(torch_gbps, 1)}


def tiny_leg(torch, I, runner, reps=200):
    """The tiny float32 configuration (4 heads, latent 16, 64 positions): the
    four calls, direct mode; launch-latency bound."""
    inp = I.make_inputs("tiny_fp32")
    w = runner.DeviceWorkload(inp, split=False)
    w.step()
    torch.cuda.synchronize()
    us = _graph_ms(torch, [w.step] * 20, reps // 20) * 1e3
    return {"step_us": round(us, 2), "cache_bytes_per_step": int(I.cache_bytes_read(inp)),
            "note": "absorb, attention (direct mode), up-projection, timed as HIP graph replays; "
                    "launch-latency bound"}


def single_leg(torch, I, runner, num_cus, copies=64, reps=4):
    """The single 4,096-token request: its 4.7 MB of cache would sit in the
    last-level cache, so the step cycles over `copies` copies of the pool at
    different addresses (302 MB in all) and every launch reads HBM.  The
    steps are shorter than their launch from Python, so they are timed as HIP
    graph replays."""
    inp = I.make_inputs("v2_single")
    w = runner.DeviceWorkload(inp, split=True, num_cus=num_cus)
    n = w.pool.shape[0]
    big = w.pool.repeat(copies, 1)
    tables = [(w.table + i * n).contiguous() for i in range(copies)]
    w.pool = big
    for t in tables:
        w.table = t
        w.step_fused()
    torch.cuda.synchronize()

    def on_copy(t, fn):
        def call():
            w.table = t
            fn()
        return call

    cache_bytes = I.cache_bytes_read(inp)
    step_us = _graph_ms(torch, [on_copy(t, w.step_fused) for t in tables], reps) * 1e3
    attn_us = _graph_ms(torch, [on_copy(t, w.attend) for t in tables], reps) * 1e3
    return {"step_us": round(step_us, 2), "attn_us": round(attn_us, 2),
            "cache_GBps": round(cache_bytes / (step_us * 1e-6) / 1e9, 1),
            "attn_GBps": round(cache_bytes / (attn_us * 1e-6) / 1e9, 1),
            "tokens_per_s": round(1e6 / step_us, 1), "cache_bytes_per_step": int(cache_bytes),
            "workers": w.plan.num_workers, "copies": copies}


def long_context_token(torch, I, runner, DI, num_cus, layers=60, tokens=10):
    """One generated token of the long-context workload: 60 independent layers
    (1 request x 131,072 positions each, 9.06 GB of cache in all), each layer
    absorb -> attention -> merge + up-projection.  The layers are drawn on the
    device (seed 4000 + layer).  The 180 launches of a token are captured in
    one HIP graph and the graph is replayed; the 60 attention launches alone,
    back to back, give the per-layer attention time."""
    ws = []
    for layer in range(layers):
        t = DI.draw_bf16_layer(torch, 4000 + layer, [131072])
        ws.append(runner.DeviceWorkload(t["shell"], split=True, num_cus=num_cus, tensors=t))
    cache_bytes = I.cache_bytes_read(ws[0].inp) * layers
    for w in ws:
        w.step_fused()
    torch.cuda.synchronize()
    attn_us = _run_ms(torch, lambda: [w.attend() for w in ws], 3) * 1e3 / layers
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for w in ws:
                w.step_fused()
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    tok_ms = _median_ms(torch, g.replay, tokens)
    eager_ms = _median_ms(torch, lambda: [w.step_fused() for w in ws], 3)
    del g, ws
    return {"ms_per_token_median": round(tok_ms, 3), "tokens_per_s": round(1e3 / tok_ms, 1),
            "cache_GBps": round(cache_bytes / (tok_ms * 1e-3) / 1e9, 1),
            "cache_bytes_per_token": int(cache_bytes), "layers": layers,
            "attn_us_per_layer": round(attn_us, 2),
            "attn_GBps": round(cache_bytes / layers / (attn_us * 1e-6) / 1e9, 1),
            "eager_ms_per_token": round(eager_ms, 3), "tokens_timed": tokens,
            "timing": "HIP graph of the 60 layers' 180 launches, replayed; layers drawn on the device"}


def fp8_topk_step(torch, I, runner, DI, num_cus, group128, lists=16, reps=6):
    """The FP8-cache workload with a top-2,048 index list per request (32
    requests x 65,536 positions, drawn on the device; one scale per position,
    or one per 128 latent channels).  One step reads 42 MB out of a 1.35 GB
    pool, which would otherwise stay in the last-level cache, so the steps
    cycle over `lists` independently drawn index-list sets (675 MB of distinct
    rows).  Steps and single launches are timed as HIP graph replays (they
    are shorter than their launch from Python).  Reports the step and
    attention times, the cache rate and
    both roofline fractions (HBM, and BF16 matrix cores: the FP8 latent is
    widened to BF16 for the MFMAs).  Returns (result, workload)."""
    log(f"fp8 top-k leg ({'group' if group128 else 'per-position'} scales): drawing inputs")
    t = DI.draw_fp8_topk(torch, 5, group128=group128)
    w = runner.DeviceWorkload(t["shell"], split=True, num_cus=num_cus, tensors=t)
    inp = w.inp
    g = torch.Generator(device="cuda")
    g.manual_seed(5005)
    sets = [DI.draw_topk_lists(torch, g, inp.seq_lens, w.topk) for _ in range(lists)]
    cache_bytes = I.cache_bytes_read(inp)
    n_pos = inp.B * w.topk
    flop = float(n_pos) * 2 * inp.H * (inp.D_C + inp.D_R + inp.D_C)
    for s_ in sets:
        w.topk_idx = s_
        w.step_fused()
    torch.cuda.synchronize()
    log(f"fp8 top-k leg: {lists} index sets resident; timing")

    def on_set(t, fn):
        def call():
            w.topk_idx = t
            fn()
        return call

    step_us = _graph_ms(torch, [on_set(t, w.step_fused) for t in sets], reps) * 1e3
    attn_us = _graph_ms(torch, [on_set(t, w.attend) for t in sets], reps) * 1e3
    absorb_us = _graph_ms(torch, [w.absorb] * lists, reps) * 1e3
    tail_us = _graph_ms(torch, [w.combine_up] * lists, reps) * 1e3
    res = {"step_us": round(step_us, 2), "attn_us": round(attn_us, 2),
           "absorb_us": round(absorb_us, 2), "combine_out_up_us": round(tail_us, 2),
           "cache_bytes_per_step": int(cache_bytes),
           "attn_cache_GBps": round(cache_bytes / (attn_us * 1e-6) / 1e9, 1),
           "attn_hbm_frac": round(cache_bytes / (attn_us * 1e-6) / (HBM_PEAK_GBPS * 1e9), 4),
           "attn_mfma_util": round(flop / (attn_us * 1e-6) / BF16_PEAK_FLOPS, 4),
           "tokens_per_s": round(inp.B / (step_us * 1e-6), 1), "workers": w.plan.num_workers,
           "data": "drawn on the device (seed 5), index sets cycled"}
    return res, w


def prefill_leg(torch, I, runner, T=4096, reps=10, name="v2_single"):
    """Prefill of a T-token prompt of one request at V2 dims on the expanded
    path: expansion of the cached latent per head (two GEMMs over the 512
    latent channels) and causal attention of the T queries.  Reports the time
    of each and their matrix-core rates (dense BF16 peak).  ``name`` picks the
    cache: BF16 (v2_single) or FP8 with one scale per position (v2_fp8_topk)
    or per 128 channels (v2_fp8g_topk)."""
    inp = I.make_inputs(name, batch=1, ctx=(T, T), topk=0) if name != "v2_single" else \
        I.make_inputs(name, ctx=(T, T))
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
            "prefill_tokens_per_s": round(T / ((exp_us + att_us) * 1e-6), 1), "cache": inp.cache_dtype}


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
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of untimed steps before the warmup steps, so the GPU clock has settled "
                         "at its loaded level when timing starts")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the oracle on all 64 requests of the batched workload (about 1.5 minutes)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device-to-device copy (counter calibration)")
    ap.add_argument("--main-only", action="store_true",
                    help="time only the batched workload (no other configurations, no reference read)")
    ap.add_argument("--configs", default="tiny_fp32,v2_single,v2_long_token,v2_fp8_topk,v2_fp8g_topk",
                    help="comma-separated configuration legs to run after the batched workload (default: all)")
    ap.add_argument("--fp8-lists", type=int, default=16,
                    help="index-list sets the FP8 top-k legs cycle through (fewer for counter runs)")
    ap.add_argument("--fp8-reps", type=int, default=6, help="graph replays per FP8 top-k timing")
    ap.add_argument("--prefill", action="store_true",
                    help="also time prefill of a 4,096-token prompt on the expanded path")
    ap.add_argument("--indexer", action="store_true",
                    help="also time the lightning indexer and top-k pick (32 x 65,536 positions) and the whole "
                         "sparse decode step fed by its picks")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported in this build "
              "(the path shards by request with no communication; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(1)
    from mla_latent_kv_absorb_amd import device_inputs as DI
    from mla_latent_kv_absorb_amd import inputs as I
    from mla_latent_kv_absorb_amd import runner

    t0 = time.time()
    inp = I.make_inputs("v2_batched")
    log(f"inputs drawn in {time.time() - t0:.1f} s; contexts {inp.seq_lens.min()}..{inp.seq_lens.max()}")
    num_cus = torch.cuda.get_device_properties(0).multi_processor_count
    w = runner.DeviceWorkload(inp, split=True, num_cus=num_cus)
    probe = ClockProbe(torch)
    # The first launch of a kernel loads its code object, which stalls the
    # host for tens of milliseconds; the GPU idles meanwhile and its clock
    # drops, and the steps that follow run up to twice as long until it has
    # recovered.  So every kernel the timed region and its probes use is
    # launched once here, before the settle.
    probe.mark()
    probe.stream_read(torch.zeros(16 * 256 * 8, dtype=torch.uint8, device="cuda"), 1)
    w.step_fused()
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

    # settle: untimed steps until the clock has reached its loaded level
    settle_steps = 0
    ts = time.perf_counter()
    while time.perf_counter() - ts < args.settle_s:
        for _ in range(20):
            w.step_fused()
        settle_steps += 20
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        w.step_fused()
    torch.cuda.synchronize()
    log(f"settle {settle_steps} steps, warmup {args.warmup} done")

    stream = torch.cuda.current_stream()
    # The timed region: K whole steps, HIP events only at its two ends (an
    # event recorded between two launches slows the launch after it).  The
    # passes that time single launches are queued right behind it, each after
    # a bridge of untimed steps, and the host does not wait in between: a
    # GPU left idle for a few milliseconds drops its clock, and the launches
    # after the gap run slow until it has recovered.
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0 = probe.mark()
    start.record(stream)
    for _ in range(args.steps):
        w.step_fused()
    stop.record(stream)
    c1 = probe.mark()
    # Per-launch times: the same K steps with a one-wave stamp kernel between
    # the launches that writes the real-time counter (100 MHz).  A stamp is an
    # ordinary launch on the stream, without the cache writeback and
    # invalidate of an event.
    stamps = torch.zeros((args.steps, 4), dtype=torch.int64, device="cuda")
    for _ in range(20):
        w.step_fused()
    c2 = probe.mark()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    for k in range(args.steps):
        probe.stamp(stamps[k], 0)
        w.absorb()
        probe.stamp(stamps[k], 1)
        w.attend()
        probe.stamp(stamps[k], 2)
        w.combine_up()
        probe.stamp(stamps[k], 3)
    p1.record(stream)
    c3 = probe.mark()
    # and with HIP events around the attention launches, for comparison
    for _ in range(20):
        w.step_fused()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for k in range(args.steps):
        w.absorb()
        ev[k][0].record(stream)
        w.attend()
        ev[k][1].record(stream)
        w.combine_up()
    torch.cuda.synchronize()
    clock = probe.mhz(c0, c1)
    ms_per_step = start.elapsed_time(stop) / args.steps
    clock_parts = probe.mhz(c2, c3)
    stamped_ms_per_step = p0.elapsed_time(p1) / args.steps
    ticks = stamps.cpu().numpy().astype(np.float64)
    part = lambda i: (ticks[:, i + 1] - ticks[:, i]) / 1e5   # 100 MHz ticks -> ms
    absorb_ms, attn_ms, tail_ms = part(0), part(1), part(2)
    absorb_avg_ms, attn_avg_ms, tail_avg_ms = float(absorb_ms.mean()), float(attn_ms.mean()), float(tail_ms.mean())
    attn_event_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step, clock {clock['mean_MHz']} MHz; "
        f"with stamps: {stamped_ms_per_step * 1e3:.1f} us/step, attention {attn_avg_ms * 1e3:.1f} us, "
        f"absorb {absorb_avg_ms * 1e3:.1f} us, merge + up-projection {tail_avg_ms * 1e3:.1f} us; "
        f"attention between HIP events {attn_event_ms * 1e3:.1f} us")

    gbps = cache_bytes / (ms_per_step * 1e-3) / 1e9
    attn_gbps = cache_bytes / (attn_avg_ms * 1e-3) / 1e9
    tokens_per_s = inp.B / (ms_per_step * 1e-3)

    # matrix-core view of the same launches (dense BF16 peak), and the head
    # GEMMs against their weight read
    attn_flop = float(np.sum(inp.seq_lens.astype(np.int64))) * 2 * inp.H * (inp.D_C + inp.D_R + inp.D_C)
    gemm_flop = 2.0 * inp.B * inp.H * inp.D_C * inp.D_N
    w_bytes = inp.H * inp.D_C * inp.D_N * 2

    def gemm(m, act_bytes):
        return {"us": round(m * 1e3, 2),
                "weight_GBps": round(w_bytes / (m * 1e-3) / 1e9, 1),
                "bytes_GBps": round((w_bytes + act_bytes) / (m * 1e-3) / 1e9, 1),
                "mfma_util": round(gemm_flop / (m * 1e-3) / BF16_PEAK_FLOPS, 5)}

    part_bytes = w.plan.num_slots * inp.H * (inp.D_C * 2 + 4)  # BF16 partials + lse
    parts = {
        "absorb": gemm(absorb_avg_ms, inp.B * inp.H * (inp.D_N + inp.D_C) * 2),
        "attention": {"us": round(attn_avg_ms * 1e3, 2), "us_median": round(float(np.median(attn_ms)) * 1e3, 2),
                      "mfma_util": round(attn_flop / (attn_avg_ms * 1e-3) / BF16_PEAK_FLOPS, 4)},
        "combine_out_up": gemm(tail_avg_ms, part_bytes + inp.B * inp.H * inp.D_V * 2),
        "step_us_with_stamps": round(stamped_ms_per_step * 1e3, 2),
        "attention_us_between_hip_events": round(attn_event_ms * 1e3, 2),
    }
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
            "timing": "average attention launch duration in a pass of the K steps with a one-wave stamp kernel "
                      "(real-time counter) between launches; with HIP events between launches the launch takes "
                      "attention_us_between_hip_events",
        },
        "cpu_baseline": None,
        "parts": parts,
        "parts_timing": "a second pass of the K steps with a one-wave kernel between the launches on the launch "
                        "stream stamping the real-time counter (100 MHz): average launch duration",
        "clock_timed_region": clock,
        "clock_parts_pass": clock_parts,
        "settle": {"seconds": args.settle_s, "steps": settle_steps},
    }
    if not args.main_only:
        parts["cache_append"] = cache_append_part(torch, I, w)
        del w
        torch.cuda.empty_cache()
        result["read_ceiling"] = read_ceiling(torch, probe)
        log(f"read ceiling {result['read_ceiling']['GBps']} GB/s")
        legs = set(args.configs.split(",")) if args.configs else set()
        configs = {}
        if "tiny_fp32" in legs:
            configs["tiny_fp32"] = tiny_leg(torch, I, runner)
        if "v2_single" in legs:
            configs["v2_single"] = single_leg(torch, I, runner, num_cus)
            log(f"v2_single {configs['v2_single']['step_us']} us/step")
        if "v2_long_token" in legs:
            configs["v2_long_token"] = long_context_token(torch, I, runner, DI, num_cus)
            log(f"v2_long {configs['v2_long_token']['ms_per_token_median']} ms/token")
            torch.cuda.empty_cache()
        if "v2_fp8_topk" in legs:
            fp8, _ = fp8_topk_step(torch, I, runner, DI, num_cus, group128=False, lists=args.fp8_lists,
                                   reps=args.fp8_reps)
            configs["v2_fp8_topk"] = fp8
            log(f"fp8 top-k step {fp8['step_us']} us")
            torch.cuda.empty_cache()
        wg = None
        if "v2_fp8g_topk" in legs or args.indexer:
            fp8g, wg = fp8_topk_step(torch, I, runner, DI, num_cus, group128=True, lists=args.fp8_lists,
                                     reps=args.fp8_reps)
            configs["v2_fp8g_topk"] = fp8g
            log(f"fp8 top-k step, group scales {fp8g['step_us']} us")
        if args.indexer:
            result["indexer_step"] = indexer_step(torch, I, runner, attn=wg)
        del wg
        torch.cuda.empty_cache()
        if args.prefill:
            result["prefill_4096"] = prefill_leg(torch, I, runner)
            result["prefill_4096_fp8"] = prefill_leg(torch, I, runner, name="v2_fp8_topk")
            result["prefill_4096_fp8g"] = prefill_leg(torch, I, runner, name="v2_fp8g_topk")
        result["configs"] = configs

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on whole requests")
        result["cpu_baseline"] = cpu_baseline(inp, full=args.cpu_full)
        if not args.main_only:
            other = cpu_baselines_other(I)
            for k, v in other.items():
                result["configs"].setdefault(k, {})["cpu_baseline"] = v
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
