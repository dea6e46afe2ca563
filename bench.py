"""Benchmark of the GQA KV-cache attention path on one MI355X.

One step = one pass of the whole path over the 16K session workload: a
16384-token prompt (8 query heads sharing 1 KV head, head_dim 256, bf16
cache) prefilled as 21 chunks of 768 rows plus one of 256 -- each chunk one
ka_attn_append_prefill_chunk call (the append of its K/V rows and the prefill
of its query rows) -- followed by 64 decode steps, each one
ka_attn_decode_step call (the append of the step's row and its decode).  Inputs are
seeded synthetic draws (module ``synth``), resident in HBM before timing.

Printed: one JSON line.  ``value`` is the 16K prefill throughput in rows/s
(16384 rows / GPU time of the 22 chunk calls; the same chunks as separate
append and prefill calls are reported beside it).  The line also
carries the decode time per token at 16K (in-session, and cache-cold over 64
rotated cache copies) and at 128K (4 sessions batched), the roofline of the
prefill kernel (bf16 MFMA) and of the 128K decode (HBM), and the CPU oracle
timed on a bounded sample of the same workload.

GPU times come from HIP events recorded on the stream the library launches
on.  While the host enqueues a timed phase the GPU is held by a short spin
kernel (recorded before the phase's first event), so the events time the
GPU, not Python's call overhead.  A timed phase carries events at its two
ends only: an event recorded between two calls stalls the queue (about 5 us
on this GPU), so per-call figures come from separate runs of the same call
repeated back to back, as (time of 2n calls - time of n calls) / n, which
cancels the fixed cost of the bracketing events.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import kv_cache_attention_amd as ka  # noqa: E402
from synth import WORKLOADS, draw_batch  # noqa: E402

METRIC = "prefill rows/s at 16K ctx; decode µs/token at 16K & 128K; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3   # MI355X dense FP32 MFMA, AMD's published figure


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "session16k_decode128k_hbm_traffic.md")


def kernel_source_hash():
    """SHA-256 over the library's kernel sources (names and contents, sorted)."""
    import hashlib
    csrc = os.path.join(ROOT, "kv_cache_attention_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        h.update(f.encode())
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, or {} when the
    kernels have changed since those counters were taken."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                k, sep, v = line.partition(":")
                if sep and k.strip() and " " not in k.strip():
                    kv[k.strip()] = v.strip()
        if kv.get("traffic_source_sha256") != kernel_source_hash():
            return {}
        return {k: int(v) for k, v in kv.items() if k.endswith("_bytes_per_launch")}
    except (OSError, ValueError):
        return {}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


class Hold:
    """Keeps the GPU busy while the host enqueues a phase (torch's spin kernel)."""

    def __init__(self):
        self.cycles = 0
        if not hasattr(torch.cuda, "_sleep"):
            return
        # calibrate: cycles for ~1 ms
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(1_000_000)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        self.per_ms = 1_000_000 / max(ms, 1e-3)

    def __call__(self, ms):
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(int(self.per_ms * ms))


def prefill_flops(w):
    """Algorithmic flops of the session's prefill: causal pairs x Hq x D x 4."""
    pairs = sum(R * s + R * (R + 1) // 2 for s, R in w.chunks)
    return pairs * w.num_q_heads * w.head_dim * 4 * w.batch, pairs


def decode_bytes(w, ctx, batch, kv_dtype=None):
    """Algorithmic HBM bytes of one decode call: K and V rows once, q and out.
    int8-K caches: per row D code bytes and a 4-byte scale for K, 2 D for V."""
    kv_dtype = kv_dtype or w.kv_dtype
    if kv_dtype == "i8k":
        kv = batch * w.num_kv_heads * ctx * (3 * w.head_dim + 4)
        qo = 2 * batch * w.num_q_heads * w.head_dim * 4
        return kv + qo
    el = 2 if kv_dtype == "bf16" else 4
    kv = 2 * batch * w.num_kv_heads * ctx * w.head_dim * el
    qo = 2 * batch * w.num_q_heads * w.head_dim * 4
    return kv + qo


class Session16K:
    """Device state of the 16K session workload."""

    def __init__(self, kv_dtype="bf16"):
        self.w = w = WORKLOADS[4]
        c = draw_batch(w)
        self.k = dev(c.k)          # [1][P][1][256]
        self.v = dev(c.v)
        self.q = dev(c.q)          # [1][16448][8][256]
        self.shape = ka.Shape(1, 8, 1, 256, w.capacity, kv_dtype)
        self.kc = ka.alloc_cache(self.shape, fill_byte=0xFF)
        self.vc = ka.alloc_cache(self.shape, fill_byte=0xFF)
        self.out_p = torch.empty(768 * 8 * 256, device="cuda")
        self.out_d = torch.empty(8 * 256, device="cuda")
        n = max(ka.append_prefill_workspace_bytes(self.shape, 768),
                ka.prefill_workspace_bytes(self.shape, 768),
                ka.decode_workspace_bytes(self.shape, w.capacity), 1)
        self.ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        # contiguous per-call views
        self.chunk_views = []
        qrow = 0
        for s, R in w.chunks:
            self.chunk_views.append((s, R, self.k[:, s:s + R], self.v[:, s:s + R],
                                     self.q[:, qrow:qrow + R], self.out_p[: R * 8 * 256]))
            qrow += R
        self.dec_views = []
        for t, p in enumerate(w.decode_positions):
            self.dec_views.append((p, self.k[:, p:p + 1], self.v[:, p:p + 1], self.q[0, qrow + t]))

    def prefill_phase(self):
        """22 chunk calls, each ka_attn_append_prefill_chunk (the chunk's append
        and its prefill in one call)."""
        sh = self.shape
        for s, R, kk, vv, qq, oo in self.chunk_views:
            ka.append_prefill_chunk(sh, qq, kk, vv, self.kc, self.vc, oo, s, R, self.w.scale,
                                    self.ws)

    def prefill_phase_separate(self):
        """The same 22 chunks as ka_attn_append_kv + ka_attn_prefill_chunk."""
        sh = self.shape
        for s, R, kk, vv, qq, oo in self.chunk_views:
            ka.append_kv(sh, self.kc, self.vc, kk, vv, s, R)
            ka.prefill_chunk(sh, qq, self.kc, self.vc, oo, s, R, self.w.scale, self.ws)

    def decode_phase(self):
        """64 decode steps, each one ka_attn_decode_step (append + attend)."""
        sh = self.shape
        for p, kk, vv, qq in self.dec_views:
            ka.decode_step(sh, qq, kk, vv, self.kc, self.vc, self.out_d, [p], self.w.scale, self.ws)


def ev_pair():
    return (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))


def span_ms(f, n, hold, hold_ms=2.0):
    """GPU time of n back-to-back calls f(i), events at the two ends only.
    The spin kernel before the first event must outlast the host's enqueue
    of the n calls, or the GPU would wait for the host."""
    a, b = ev_pair()
    hold(hold_ms)
    a.record()
    for i in range(n):
        f(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def per_call_ms(f, hold, n=8, reps=5):
    """Per-call GPU time of f, back to back: median over reps of
    (span of 2n calls - span of n calls) / n."""
    f(0)
    torch.cuda.synchronize()
    hold_ms = 1.0 + 0.15 * 2 * n
    ts = []
    for _ in range(reps):
        t1 = span_ms(f, n, hold, hold_ms)
        t2 = span_ms(f, 2 * n, hold, hold_ms)
        ts.append((t2 - t1) / n)
    return float(np.median(ts))


def bench_session(steps, warmup, hold):
    """The timed steps: the 22 chunk calls and the 64 decode steps, each phase
    back to back with events at its two ends.  Then, untimed for the step,
    each chunk's prefill call and the last decode step alone (per_call_ms)."""
    s = Session16K()
    log("16K session: inputs resident")
    for _ in range(warmup):
        s.prefill_phase()
        s.decode_phase()
    torch.cuda.synchronize()
    rec = []
    t0 = time.perf_counter()
    for _ in range(steps):
        ph, dh = ev_pair(), ev_pair()
        hold(6.0)
        ph[0].record()
        s.prefill_phase()
        ph[1].record()
        hold(10.0)
        dh[0].record()
        s.decode_phase()
        dh[1].record()
        rec.append((ph, dh))
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    phase_p = [r[0][0].elapsed_time(r[0][1]) for r in rec]
    phase_d = [r[1][0].elapsed_time(r[1][1]) for r in rec]
    log("16K session: timed steps done")
    sep = [span_ms(lambda i: s.prefill_phase_separate(), 1, hold, 6.0) for _ in range(3)]
    sh = s.shape
    fused_calls, pre_calls = [], []
    for (st, R, kk, vv, qq, oo) in s.chunk_views:
        # each call appends the same rows again: the cache ends as one pass leaves it
        fused_calls.append(per_call_ms(
            lambda i: ka.append_prefill_chunk(sh, qq, kk, vv, s.kc, s.vc, oo, st, R, s.w.scale, s.ws),
            hold, n=6, reps=3))
        pre_calls.append(per_call_ms(
            lambda i: ka.prefill_chunk(sh, qq, s.kc, s.vc, oo, st, R, s.w.scale, s.ws), hold, n=6, reps=3))
    p, kk, vv, qq = s.dec_views[-1]
    dec_call = per_call_ms(
        lambda i: ka.decode_step(sh, qq, kk, vv, s.kc, s.vc, s.out_d, [p], s.w.scale, s.ws), hold, n=16)
    return dict(w=s.w, wall_ms=wall * 1e3, prefill_phase_ms=float(np.median(phase_p)),
                prefill_phase_separate_ms=float(np.median(sep)), fused_calls_ms=np.array(fused_calls),
                decode_phase_ms=float(np.median(phase_d)), prefill_calls_ms=np.array(pre_calls),
                decode_call_ms=dec_call, session=s)


def bench_decode_cold_16k(s, hold, copies=64, reps=3):
    """The decode step at 16K over `copies` caches in rotation (more bytes
    than the MALL), back to back: GPU time per step."""
    w = s.w
    p = w.decode_positions[-1]
    kcs = [s.kc.clone() for _ in range(copies)]
    vcs = [s.vc.clone() for _ in range(copies)]
    _, kk, vv, qq = s.dec_views[-1]
    torch.cuda.synchronize()
    times = []
    for r in range(reps + 1):
        a, b = ev_pair()
        hold(10.0)
        a.record()
        for i in range(copies):
            ka.decode_step(s.shape, qq, kk, vv, kcs[i], vcs[i], s.out_d, [p], w.scale, s.ws)
        b.record()
        torch.cuda.synchronize()
        if r:
            times.append(a.elapsed_time(b) / copies)
    del kcs, vcs
    return float(np.median(times))


def copy_calibration(mib=256, reps=5):
    """A plain device-to-device copy of known size: its measured bandwidth is
    printed beside the HBM peak, and under a counter profiler its FETCH_SIZE /
    WRITE_SIZE per dispatch give the factor that turns those counters into
    bytes (it reads and writes exactly ``mib`` MiB)."""
    n = mib * 2**20 // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = ev_pair()
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    nbytes = 2 * n * 4
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_read": n * 4, "bytes_written": n * 4,
            "gbs": round(nbytes / (float(np.median(times)) * 1e-3) / 1e9, 1)}


def bench_decode_128k(hold, steps=32, kv_dtype="bf16"):
    w = WORKLOADS[5]
    c = draw_batch(w)
    log("128K: drawn")
    shape = ka.Shape(w.batch, 8, 1, 256, w.capacity, kv_dtype)
    kc = ka.alloc_cache(shape, fill_byte=0xFF)
    vc = ka.alloc_cache(shape, fill_byte=0xFF)
    for s0 in range(0, w.positions, 16384):
        e = min(w.positions, s0 + 16384)
        ka.append_kv(shape, kc, vc, dev(c.k[:, s0:e]), dev(c.v[:, s0:e]), s0, e - s0)
    torch.cuda.synchronize()
    # every position is now appended once; the timed steps re-append their
    # own rows (identical values) as part of each decode step
    kd = [dev(c.k[:, p:p + 1]) for p in w.decode_positions]
    vd = [dev(c.v[:, p:p + 1]) for p in w.decode_positions]
    qd = [dev(c.q[:, t]) for t in range(len(w.decode_positions))]
    out = torch.empty(w.batch * 8 * 256, device="cuda")
    ws = torch.empty(max(ka.decode_workspace_bytes(shape, w.capacity), 1), dtype=torch.uint8, device="cuda")
    del c
    log("128K: filled")

    def step(t):
        p = w.decode_positions[t % steps]
        ka.decode_step(shape, qd[t % steps], kd[t % steps], vd[t % steps], kc, vc, out,
                       [p] * w.batch, w.scale, ws)

    step(0)
    torch.cuda.synchronize()
    # the 32 steps back to back, events at the ends
    step_ms = [span_ms(step, steps, hold, 6.0) / steps for _ in range(5)]
    # one step alone: the last one (context 131072), repeated (it re-appends
    # the same row, so every repeat does the same work)
    last = lambda i: step(steps - 1)
    call_ms = per_call_ms(last, hold, n=8)
    ctx_mean = int(np.mean([p + 1 for p in w.decode_positions[:steps]]))
    return dict(w=w, step_ms=float(np.median(step_ms)), call_ms=call_ms,
                bytes=decode_bytes(w, ctx_mean, w.batch, kv_dtype), ctx_mean=ctx_mean)


def bench_prefill_f32(hold, reps=10):
    """The f32 chunk workload: a 768-row chunk at 3072 over 3072 cached rows
    (8 query heads / 1 KV head, head_dim 256, f32 cache): per-call time."""
    w = WORKLOADS[3]
    c = draw_batch(w)
    shape = ka.Shape(1, 8, 1, 256, w.capacity, "f32")
    kc = ka.alloc_cache(shape, fill_byte=0xFF)
    vc = ka.alloc_cache(shape, fill_byte=0xFF)
    (s0, R), = w.chunks
    ka.append_kv(shape, kc, vc, dev(c.k[:, :s0 + R]), dev(c.v[:, :s0 + R]), 0, s0 + R)
    q = dev(c.q)
    out = torch.empty(R * 8 * 256, device="cuda")
    ws = torch.empty(max(ka.prefill_workspace_bytes(shape, R), 1), dtype=torch.uint8, device="cuda")
    del c
    ms = per_call_ms(lambda i: ka.prefill_chunk(shape, q, kc, vc, out, s0, R, w.scale, ws), hold,
                     n=6, reps=reps)
    pairs = R * s0 + R * (R + 1) // 2
    flops = pairs * 8 * 256 * 4
    return dict(ms=ms, rows=R, flops=flops)


def bench_decode_f32_4k(hold, copies=64):
    """The f32 decode workload: 8 query heads on one KV head, head_dim 256,
    4096 cached rows; each step appends row 4096 and attends to 4097 keys
    (ka_attn_decode_step on an f32 cache).  Warm: one cache, the step
    repeated (8.4 MB of K/V, resident in the 256 MB MALL); cold: `copies`
    caches in rotation (545 MB), back to back."""
    w = WORKLOADS[2]
    c = draw_batch(w)
    shape = ka.Shape(1, 8, 1, 256, w.capacity, "f32")
    kc = ka.alloc_cache(shape, fill_byte=0xFF)
    vc = ka.alloc_cache(shape, fill_byte=0xFF)
    ka.append_kv(shape, kc, vc, dev(c.k[:, :w.fill_rows]), dev(c.v[:, :w.fill_rows]), 0, w.fill_rows)
    p = w.decode_positions[0]
    kn, vn, q = dev(c.k[:, p]), dev(c.v[:, p]), dev(c.q[:, 0])
    out = torch.empty(8 * 256, device="cuda")
    ws = torch.empty(max(ka.decode_workspace_bytes(shape, p + 1), 1), dtype=torch.uint8, device="cuda")
    del c
    warm = per_call_ms(lambda i: ka.decode_step(shape, q, kn, vn, kc, vc, out, [p], w.scale, ws), hold,
                       n=16)
    kcs = [kc.clone() for _ in range(copies)]
    vcs = [vc.clone() for _ in range(copies)]
    torch.cuda.synchronize()
    f = lambda i: ka.decode_step(shape, q, kn, vn, kcs[i % copies], vcs[i % copies], out, [p],
                                 w.scale, ws)
    f(0)
    cold = float(np.median([span_ms(f, copies, hold, 10.0) / copies for _ in range(3)]))
    del kcs, vcs
    torch.cuda.empty_cache()
    return dict(warm_ms=warm, cold_ms=cold, bytes=decode_bytes(w, p + 1, 1, "f32"))


def bench_rope(hold, reps=20):
    """Rotary entry points at the session's chunk shape: a 768-row append
    whose K rows are rotated on the way into the bf16 cache, and the rotation
    of the chunk's 768 x 8 query rows (per-call times, back to back)."""
    w = WORKLOADS[4]
    shape = ka.Shape(1, 8, 1, 256, w.capacity, "bf16")
    kc = ka.alloc_cache(shape)
    vc = ka.alloc_cache(shape)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    R, s0 = 768, 7680
    k = torch.randn(R * 256, device="cuda", generator=g)
    v = torch.randn(R * 256, device="cuda", generator=g)
    q = torch.randn(R * 8 * 256, device="cuda", generator=g)
    qo = torch.empty_like(q)
    pos = torch.arange(s0, s0 + R, device="cuda", dtype=torch.float64)[:, None]
    inv = 10000.0 ** (-torch.arange(128, device="cuda", dtype=torch.float64) * 2.0 / 256)
    cos = torch.cos(pos * inv).float().contiguous()
    sin = torch.sin(pos * inv).float().contiguous()
    calls = {"append_kv_rope_768_us": lambda: ka.append_kv_rope(shape, kc, vc, k, v, cos, sin, s0, R),
             "rope_rows_768x8_us": lambda: ka.rope_rows(shape, q, qo, cos, sin, R),
             "append_kv_768_us": lambda: ka.append_kv(shape, kc, vc, k, v, s0, R)}
    res = {}
    for name, f in calls.items():
        res[name] = round(per_call_ms(lambda i, f=f: f(), hold, n=16) * 1e3, 2)
    return res


def bench_int8(hold):
    """The 16K session and the 4 x 131K decode steps on int8-K caches (int8 K
    codes with row scales, bf16 V, integer scores): the session's 22 chunk
    calls and 64 decode steps, and the 128K steps with their HBM rate."""
    ka.int8_self_test()
    s = Session16K("i8k")
    s.prefill_phase()
    s.decode_phase()
    torch.cuda.synchronize()
    pre, dec = [], []
    for _ in range(3):
        pre.append(span_ms(lambda i: s.prefill_phase(), 1, hold, 6.0))
        dec.append(span_ms(lambda i: s.decode_phase(), 1, hold, 10.0) / len(s.dec_views))
    rows = sum(R for _, R in s.w.chunks)
    pm = float(np.median(pre))
    res = {"prefill_16k_ms": round(pm, 4), "prefill_16k_rows_per_s": round(rows / (pm * 1e-3), 1),
           "decode_us_per_token_16k": round(float(np.median(dec)) * 1e3, 3)}
    del s
    torch.cuda.empty_cache()
    d = bench_decode_128k(hold, kv_dtype="i8k")
    gbs = d["bytes"] / (d["step_ms"] * 1e-3) / 1e9
    res["decode_us_per_step_128k_x4"] = round(d["step_ms"] * 1e3, 3)
    res["decode_us_per_call_128k_x4"] = round(d["call_ms"] * 1e3, 3)
    res["roofline_decode_128k"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                   "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                   "algorithmic_bytes_per_launch": d["bytes"],
                                   "time": "32 steps back to back"}
    torch.cuda.empty_cache()
    return res


def bench_few_rows(hold, reps=20):
    """Chunks of 1 .. 15 rows (the band between decode and the M-tile
    prefill) ending at context 16384 and 131072 of one session, 8 query heads
    on one KV head, head_dim 256, bf16 cache: per-call times, back to back."""
    res = {}
    for ctx in (16384, 131072):
        shape = ka.Shape(1, 8, 1, 256, ctx, "bf16")
        kc = ka.alloc_cache(shape)
        vc = ka.alloc_cache(shape)
        g = torch.Generator(device="cuda")
        g.manual_seed(11)
        k = torch.randn(ctx * 256, device="cuda", generator=g)
        v = torch.randn(ctx * 256, device="cuda", generator=g)
        ka.append_kv(shape, kc, vc, k, v, 0, ctx)
        del k, v
        q = torch.randn(15 * 8 * 256, device="cuda", generator=g)
        o = torch.empty_like(q)
        ws = torch.zeros(max(1, ka.prefill_workspace_bytes(shape, 15)), dtype=torch.uint8,
                         device="cuda")
        row = {}
        for R in (1, 2, 4, 8, 15):
            n = R * 8 * 256
            f = lambda i, n=n, R=R: ka.prefill_chunk(shape, q[:n], kc, vc, o[:n], ctx - R, R, 1 / 16, ws)
            row[str(R)] = round(per_call_ms(f, hold, n=12) * 1e3, 2)
        res[f"ctx_{ctx}_us_by_rows"] = row
        del kc, vc, q, o, ws
        torch.cuda.empty_cache()
    return res


def bench_ragged(hold, reps=20):
    """Eight sessions of one 16K-capacity bf16 cache (8 query heads, one KV
    head, head_dim 256), each with a chunk at its own position: one ragged
    call against one chunk call per session (per-call times, back to back)."""
    B, C = 8, 16384
    shape = ka.Shape(B, 8, 1, 256, C, "bf16")
    one = ka.Shape(1, 8, 1, 256, C, "bf16")
    kc = ka.alloc_cache(shape)
    vc = ka.alloc_cache(shape)
    g = torch.Generator(device="cuda")
    g.manual_seed(13)
    k = torch.randn(B * C * 256, device="cuda", generator=g)
    v = torch.randn(B * C * 256, device="cuda", generator=g)
    ka.append_kv(shape, kc, vc, k, v, 0, C)
    del k, v
    slab = ka.cache_bytes(one)
    res = {}
    for name, rows in (("64_rows_each", [64] * B), ("mixed_768_to_1", [768, 16, 300, 1, 64, 128, 5, 512])):
        starts = [C - r - 1000 * i for i, r in enumerate(rows)]
        T = sum(rows)
        q = torch.randn(T * 2048, device="cuda", generator=g)
        o = torch.empty_like(q)
        ws = torch.empty(max(ka.prefill_ragged_workspace_bytes(shape, T),
                             ka.prefill_workspace_bytes(one, 768)), dtype=torch.uint8, device="cuda")

        def ragged():
            ka.prefill_ragged(shape, q, kc, vc, o, starts, rows, 1 / 16, ws)

        def per_session():
            r0 = 0
            for b in range(B):
                n = rows[b]
                ka.prefill_chunk(one, q[r0 * 2048:(r0 + n) * 2048], kc[b * slab:(b + 1) * slab],
                                 vc[b * slab:(b + 1) * slab], o[r0 * 2048:(r0 + n) * 2048],
                                 starts[b], n, 1 / 16, ws)
                r0 += n

        row = {"rows": rows}
        for nm, f in (("ragged_call_us", ragged), ("per_session_calls_us", per_session)):
            row[nm] = round(per_call_ms(lambda i, f=f: f(), hold, n=8) * 1e3, 2)
        res[name] = row
    del kc, vc
    torch.cuda.empty_cache()
    return res


def cpu_baseline(session_w, budget_s=15.0):
    """The oracle (as written) on a bounded sample of the 16K prefill: 16-row
    blocks spaced evenly over all 16384 prompt rows (so the mean context is the
    session's), as many as fit the time budget, plus one 16K decode step."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    w = session_w
    c = draw_batch(w)
    ks = oracle.stored_values(c.k, "bf16")[0]
    vs = oracle.stored_values(c.v, "bf16")[0]
    rows = sum(R for _, R in w.chunks)           # prompt rows = positions 0..rows-1
    q = c.q[0]

    def run(nblocks):
        starts = np.linspace(0, rows - 16, nblocks).astype(np.int64)
        t = time.perf_counter()
        for s0 in starts:
            oracle.attend_rows(q[s0:s0 + 16], ks, vs, np.arange(s0, s0 + 16), w.scale)
        return time.perf_counter() - t

    ctxm = threadpool_limits(limits=cores) if threadpool_limits else None
    try:
        t_cal = run(8)
        nblocks = int(min(rows // 16, max(8, 8 * budget_s / max(t_cal, 1e-3))))
        dt = run(nblocks)
        p = w.decode_positions[0]
        t = time.perf_counter()
        oracle.attend_rows(q[rows][None], ks, vs, [p], w.scale)
        dt_dec = time.perf_counter() - t
    finally:
        if ctxm is not None:
            ctxm.__exit__(None, None, None)
    n = nblocks * 16
    extras = oracle_extras(oracle, threadpool_limits, cores)
    # the scalar oracle (pure Python, one core) on the tiny workload in full
    w1 = WORKLOADS[1]
    c1 = draw_batch(w1)
    (s1, R1), = w1.chunks
    t = time.perf_counter()
    oracle.attend_rows_scalar(c1.q[0], c1.k[0], c1.v[0], list(range(s1, s1 + R1)), w1.scale)
    extras["scalar_tiny_prefill_1_core"] = {
        "rows_per_s": round(R1 / (time.perf_counter() - t), 2),
        "seconds": round(time.perf_counter() - t, 2),
        "sample": "all 128 rows of the tiny f32 prefill (2 query heads, head_dim 64), "
                  "pure-Python math.fsum oracle, one core"}
    return {"value": round(n / dt, 2), "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": (f"{n} of the 16384 prompt rows of the 16K session (16-row blocks evenly spaced "
                       f"over positions 0..16383, each row against its full causal context; 8 heads, "
                       f"head_dim 256, bf16-stored K/V), numpy float64 two-pass softmax with "
                       f"{cores} BLAS threads, {dt:.1f} s; plus one decode step at 16384 "
                       f"({dt_dec * 1e3:.1f} ms)"),
            "decode_16k_us_per_token": round(dt_dec * 1e6, 1),
            "other_workloads": extras}


def oracle_extras(oracle, threadpool_limits, cores):
    """The oracle on samples of the other timed workloads, with all host cores
    and with one BLAS thread: 64 of the 768 rows of the f32 chunk at 3072
    (evenly spaced, each against its full causal context), and one decode step
    of the first of the four 131K sessions."""
    from synth import draw_session
    res = {}
    w3 = WORKLOADS[3]
    c3 = draw_batch(w3)
    (s0, R), = w3.chunks
    pick = np.linspace(0, R - 1, 64).astype(np.int64)
    w5 = WORKLOADS[5]
    p5 = w5.decode_positions[0]
    c5 = draw_session(w5, 0, q_positions=[p5])
    k5, v5 = oracle.stored_values(c5.k, "bf16"), oracle.stored_values(c5.v, "bf16")
    for threads in (cores, 1):
        ctxm = threadpool_limits(limits=threads) if threadpool_limits else None
        try:
            t = time.perf_counter()
            oracle.attend_rows(c3.q[0][pick], c3.k[0], c3.v[0], s0 + pick, w3.scale)
            dt3 = time.perf_counter() - t
            t = time.perf_counter()
            oracle.attend_rows(c5.q, k5, v5, [p5], w5.scale)
            dt5 = time.perf_counter() - t
        finally:
            if ctxm is not None:
                ctxm.__exit__(None, None, None)
        res[f"threads_{threads}"] = {
            "f32_chunk_3072_768_rows_per_s": round(len(pick) / dt3, 2),
            "decode_131k_us_per_session_token": round(dt5 * 1e6, 1)}
    res["sample"] = ("64 of the 768 rows of the f32 chunk at 3072 (evenly spaced, full causal "
                     "context each); one decode step at position 131040 of one of the four 131K "
                     "sessions (bf16-stored K/V, 8 heads)")
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-128k", action="store_true")
    ap.add_argument("--no-cold", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) is not "
              f"supported: the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ka.lib()
    torch.cuda.set_device(0)
    hold = Hold()
    copy = copy_calibration()
    traffic = measured_traffic()

    r = bench_session(args.steps, args.warmup, hold)
    w = r["w"]
    flops, pairs = prefill_flops(w)
    fused_calls = r["fused_calls_ms"]                   # [22] fused append + prefill calls
    fused_ms = float(fused_calls.sum())
    pre_calls = r["prefill_calls_ms"]                   # [22] prefill calls alone (no append)
    pre_kernel_ms = float(pre_calls.sum())
    achieved_tf = flops / (pre_kernel_ms * 1e-3) / 1e12
    rows = sum(R for _, R in w.chunks)
    value = rows / (r["prefill_phase_ms"] * 1e-3)        # 22 fused append + prefill calls
    dec16_step = r["decode_phase_ms"] / len(w.decode_positions)
    last_chunk_ms = float(pre_calls[-2])
    s_last, R_last = w.chunks[-2]
    flops_last = (R_last * s_last + R_last * (R_last + 1) // 2) * 8 * 256 * 4

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(r["prefill_phase_ms"] + r["decode_phase_ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": ("16K session: 8 query heads / 1 KV head, head_dim 256, bf16 KV "
                                "cache (f32 accumulate), 16384-row prompt as 21x768 + 256 chunks "
                                "(one fused append + prefill call each), then 64 decode steps "
                                "(one fused append + decode call each)"),
                   "global_batch": 1, "seq_len": 16384, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved_tf, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved_tf / BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic.get("prefill_call_bytes_per_launch"), "traffic_unit": "B/launch",
                     "kernel": "prefill call (ka_attn_prefill_chunk: prefill_mtile_kernel<256, false, "
                               "false>, which stages f32 Q, and its merge kernel), average over the "
                               "22 chunks; the session's fused chunk call runs the same loop on a "
                               "bf16 Q copy its append writes",
                     "algorithmic_flops_per_step": flops, "causal_pairs": pairs,
                     "avg_launch_ms": round(pre_kernel_ms / len(w.chunks), 5),
                     "time": "each chunk's prefill call back to back, (2n - n calls) / n"},
        "wall_ms_per_step": round(r["wall_ms"], 3),
        "prefill_16k_ms": round(r["prefill_phase_ms"], 4),
        "prefill_16k_ms_separate_calls": round(r["prefill_phase_separate_ms"], 4),
        "prefill_16k_ms_chunk_calls_only": round(fused_ms, 4),
        "prefill_16k_ms_prefill_calls_only": round(pre_kernel_ms, 4),
        "prefill_last768_chunk_call_us": round(float(fused_calls[-2]) * 1e3, 2),
        "prefill_last768_rows_per_s": round(R_last / (last_chunk_ms * 1e-3), 1),
        "prefill_last768_tflops": round(flops_last / (last_chunk_ms * 1e-3) / 1e12, 2),
        "decode_us_per_token_16k": round(dec16_step * 1e3, 3),
        "decode_us_per_call_16k": round(r["decode_call_ms"] * 1e3, 3),
    }
    out["copy_calibration"] = copy
    b16 = decode_bytes(w, w.decode_positions[-1] + 1, 1)
    if not args.no_cold:
        cold = bench_decode_cold_16k(r["session"], hold)
        out["decode_us_per_token_16k_cold"] = round(cold * 1e3, 3)
        out["decode_16k_cold_hbm_frac"] = round(b16 / (cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    out["decode_16k_in_session_hbm_frac"] = round(b16 / (dec16_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    del r
    torch.cuda.empty_cache()
    if not args.no_128k:
        d = bench_decode_128k(hold)
        gbs = d["bytes"] / (d["step_ms"] * 1e-3) / 1e9
        out["decode_us_per_step_128k_x4"] = round(d["step_ms"] * 1e3, 3)
        out["decode_us_per_token_128k"] = round(d["step_ms"] * 1e3 / d["w"].batch, 3)
        out["decode_us_per_call_128k_x4"] = round(d["call_ms"] * 1e3, 3)
        out["roofline_decode_128k"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                       "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                       "frac_of_measured_copy": round(gbs / copy["gbs"], 4),
                                       "traffic": traffic.get("decode_128k_call_bytes_per_launch"),
                                       "traffic_unit": "B/launch",
                                       "kernel": "decode step call (decode_mfma_kernel with the "
                                                 "row append + decode_merge_kernel), 4 sessions "
                                                 "at ctx 131041..131072",
                                       "algorithmic_bytes_per_launch": d["bytes"],
                                       "time": "32 steps back to back"}
        torch.cuda.empty_cache()
    d2 = bench_decode_f32_4k(hold)
    out["decode_f32_4097"] = {
        "us_per_step_warm": round(d2["warm_ms"] * 1e3, 3),
        "hbm_frac_warm": round(d2["bytes"] / (d2["warm_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "us_per_step_cold": round(d2["cold_ms"] * 1e3, 3),
        "hbm_frac_cold": round(d2["bytes"] / (d2["cold_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes": d2["bytes"],
        "note": "warm: 8.4 MB of K/V resident in the 256 MB MALL; cold: 64 caches in rotation"}
    f = bench_prefill_f32(hold)
    tf = f["flops"] / (f["ms"] * 1e-3) / 1e12
    out["prefill_f32_3072_768_us"] = round(f["ms"] * 1e3, 2)
    out["prefill_f32_3072_768_rows_per_s"] = round(f["rows"] / (f["ms"] * 1e-3), 1)
    out["roofline_prefill_f32"] = {"bound": "mfma", "achieved": round(tf, 2), "peak": FP32_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": round(tf / FP32_PEAK_TFLOPS, 4),
                                   "kernel": "f32 prefill chunk call (prefill_seq_kernel + merge), "
                                             "768 rows at 3072",
                                   "algorithmic_flops_per_launch": f["flops"]}
    torch.cuda.empty_cache()
    out["rope"] = bench_rope(hold)
    out["few_row_chunks"] = bench_few_rows(hold)
    out["ragged_8_sessions_16k"] = bench_ragged(hold)
    out["int8_k"] = bench_int8(hold)
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
