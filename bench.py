"""Benchmark of the fused-attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

The bench line's workload is causal prefill in the Llama2-7B attention shape
(B4 H32 T1024 D128, bf16 Q/K/V i.i.d. N(0,1), fp32 accumulation, scale
1/sqrt(128)); one step is one attn_prefill launch over one batch.  `value`
is its throughput in algorithmic TFLOP/s: 4*D flop per attended
(query, key) pair, T(T+1)/2 pairs per (b, h) under the causal mask.

The paged-decode workloads (MHA B32, GQA 32/8 B128, the same two over an
FP8 E4M3 cache, shared-prefix cascade over bf16 and FP8 caches) are timed in
the same run and reported under "decode" in KV GB/s: unique K+V bytes read
(one byte per element for FP8), the shared prefix counted once; "decode"
also holds 8-layer decode steps launched eagerly and replayed as a HIP
graph.  Chunked prefill against the paged cache is reported under
"prefill_paged" in algorithmic TFLOP/s, the same prefill without the mask
under "prefill_noncausal", the fp32 test mode (B1 H1 T128 D64) under
"prefill_f32_test_mode", and the flat GEMM of the decode
projections (one Llama2-7B layer's four weights, m = 1, 16, 64 tokens) under
"flat_gemm" in GB/s of weight + activation bytes.

Timing: an untimed spin-up (the same step repeated for 50 ms: the GPU drops
its clocks while the host prepares each section's inputs), W untimed warm-up
steps, then K steps bracketed by a device synchronisation on both sides; HIP events on the launch stream give each
launch's duration (the roofline uses their mean).  The prefill rotates
through three input sets so the 256 MB last-level cache cannot hold the
working set; the cascade flushes it before every timed repetition.

The CPU baseline runs the fp64 oracle on a bounded sample of the same
workload (a few (b, h) pairs, ~10-30 s of CPU work) on the host's cores; the
MHA, GQA and cascade decode sections time it on their sequences too
(~4 s each, in KV GB/s), reported under cpu_baseline["decode"].  Every
line carries the p10/p50/p90 of its per-launch durations (launch_us).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from attention_tiled_fmha_amd import attn  # noqa: E402
from attention_tiled_fmha_amd import workloads as wl  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")


def dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


SPINUP_S = 0.05   # untimed spin-up before each section's warm-up, seconds


def spin_up(fn, before=None, seconds=SPINUP_S):
    """Run the step back to back until `seconds` of wall time have passed.
    The bench prepares each section's inputs on the host while the GPU idles,
    and an idle GPU drops its clocks: measured after W = 10 warm-up launches
    alone, the causal prefill ran at 460-478 TFLOP/s, after ~28 ms of the
    same launches at 557.  The spin-up brings the GPU back to the state it
    holds under sustained load before the W warm-up and K timed steps."""
    t0 = time.perf_counter()
    i = 0
    while True:
        if before:
            before(i)
        fn(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                break
    torch.cuda.synchronize()


def time_launches(fn, steps, warmup, before=None):
    """Per-launch durations (ms) from HIP events on the current stream, plus
    the span of the K timed steps and its wall time.  An untimed spin-up
    (spin_up) runs before the W warm-up steps.

    Without a per-step ``before`` the K steps are enqueued back to back
    between one pair of events (the span; the mean is span / K), then K more
    with an event after each for the distribution.  With ``before`` (e.g. a
    cache flush) each step gets its own event pair and ``before`` stays
    outside the timed spans."""
    spin_up(fn, before)
    for i in range(warmup):
        if before:
            before(i)
        fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if before is None:
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            fn(i)
        end.record()
        torch.cuda.synchronize()
        span = start.elapsed_time(end)
        wall = time.perf_counter() - t0
        # a second pass of K launches with an event between each two gives
        # the per-launch distribution (the events add small gaps, so the
        # mean stays the back-to-back span / K)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record()
        for i in range(steps):
            fn(i)
            evs[i + 1].record()
        torch.cuda.synchronize()
        return [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)], span, wall
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        before(i)
        starts[i].record()
        fn(i)
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    durs = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return durs, float(np.sum(durs)), wall


def percentiles_us(durs):
    p10, p50, p90 = np.percentile(np.asarray(durs, np.float64) * 1e3, [10, 50, 90])
    return dict(p10=round(float(p10), 2), p50=round(float(p50), 2), p90=round(float(p90), 2))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "attention_tiled_fmha_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(name, digest):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    or None when there is none or the kernel source changed since."""
    path = os.path.join(PROFILES, f"{name}_counters.json")
    try:
        with open(path) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("source_digest") != digest:
        return None
    return c.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------

def bench_prefill(steps, warmup):
    sets = []
    for s in range(3):
        inp = wl.workload(wl.PREFILL_CAUSAL, seed=1002 + 100 * s)
        sets.append(tuple(dev(inp[x]) for x in ("q", "k", "v")))
    B, H, T, D = 4, 32, 1024, 128
    o = torch.empty((B, H, T, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, T), device="cuda")
    scale = 1.0 / math.sqrt(D)

    def step(i):
        q, k, v = sets[i % 3]
        attn.attn_prefill(q, k, v, o, lse, causal=True, scale=scale)

    durs, span, wall = time_launches(step, steps, warmup)
    flops = 4.0 * D * (T * (T + 1) / 2) * B * H
    mean_ms = span / steps
    achieved = flops / (mean_ms * 1e-3) / 1e12
    digest = source_digest("prefill_bf16.hip", "common.h")
    traffic = measured_traffic("prefill_bf16_causal_b4h32t1024d128", digest)
    return dict(
        ms_per_step=span / steps, mean_launch_ms=mean_ms, launch_us=percentiles_us(durs),
        tflops=flops / (span / steps * 1e-3) / 1e12, flops=flops, wall_s=wall,
        roofline=dict(bound="mfma", achieved=round(achieved, 2), peak=PEAK_BF16_TFLOPS,
                      unit="TFLOP/s", frac=round(achieved / PEAK_BF16_TFLOPS, 4),
                      traffic=traffic, kernel="prefill_bf16_kernel<128,true,false>",
                      algorithmic_bytes=int(4 * B * H * T * D * 2 + B * H * T * 4),
                      source_digest=digest))


def bench_prefill_noncausal(steps, warmup):
    """The causal prefill shape without the mask (B4 H32 T1024 D128 bf16): every
    (query, key) pair attended, 4 D flop each; three input sets rotate."""
    sets = []
    for s in range(3):
        inp = wl.workload(wl.PREFILL_CAUSAL, seed=1002 + 100 * s)
        sets.append(tuple(dev(inp[x]) for x in ("q", "k", "v")))
    B, H, T, D = 4, 32, 1024, 128
    o = torch.empty((B, H, T, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, T), device="cuda")

    def step(i):
        q, k, v = sets[i % 3]
        attn.attn_prefill(q, k, v, o, lse, causal=False, scale=1.0 / math.sqrt(D))

    durs, span, _ = time_launches(step, steps, warmup)
    flops = 4.0 * D * T * T * B * H
    mean_ms = span / steps
    return dict(workload="non-causal prefill B4 H32 T1024 D128 bf16", mean_ms=mean_ms,
                launch_us=percentiles_us(durs),
                tflops=round(flops / (mean_ms * 1e-3) / 1e12, 2),
                frac_mfma=round(flops / (mean_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4))


def bench_torch_sdpa(steps, warmup):
    """Context, not the product: PyTorch's own fused attention
    (scaled_dot_product_attention restricted to its flash, then its
    memory-efficient backend, never the unfused math path) on the prefill
    shape, causal and not, timed like the prefill lines."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    sets = []
    for s in range(3):
        inp = wl.workload(wl.PREFILL_CAUSAL, seed=1002 + 100 * s)
        sets.append(tuple(dev(inp[x]) for x in ("q", "k", "v")))
    B, H, T, D = 4, 32, 1024, 128
    out = dict(library="torch.nn.functional.scaled_dot_product_attention", torch=torch.__version__)
    for name, backend in (("flash", SDPBackend.FLASH_ATTENTION),
                          ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
        try:
            with sdpa_kernel([backend]):
                for causal in (True, False):
                    def step(i):
                        q, k, v = sets[i % 3]
                        torch.nn.functional.scaled_dot_product_attention(
                            q, k, v, is_causal=causal, scale=1.0 / math.sqrt(D))

                    _, span, _ = time_launches(step, steps, warmup)
                    flops = 4.0 * D * (T * (T + 1) / 2 if causal else T * T) * B * H
                    out["causal_tflops" if causal else "noncausal_tflops"] = round(
                        flops / (span / steps * 1e-3) / 1e12, 2)
            out["backend"] = name
            return out
        except RuntimeError as e:
            out[f"{name}_unavailable"] = str(e)[:160]
    return out


def bench_prefill_f32(steps, warmup):
    """The fp32 test mode, non-causal B1 H1 T128 D64 (4.19 MFLOP;
    launch-latency bound, reported in microseconds and against the fp32
    vector peak of 157.3 TFLOP/s)."""
    inp = wl.workload(wl.PREFILL_F32)
    q, k, v = (dev(inp[x]) for x in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], device="cuda")

    def step(i):
        attn.attn_prefill(q, k, v, o, lse, causal=False, scale=inp["scale"])

    durs, span, _ = time_launches(step, steps, warmup)
    flops = 4.0 * 64 * 128 * 128
    mean_ms = span / steps
    return dict(workload="non-causal prefill B1 H1 T128 D64 fp32 (test mode)",
                us=round(mean_ms * 1e3, 2),
                tflops=round(flops / (mean_ms * 1e-3) / 1e12, 4),
                frac_fp32_peak=round(flops / (mean_ms * 1e-3) / 1e12 / 157.3, 5))


def bench_prefill_paged(steps, warmup):
    """Chunked prefill: a 512-token chunk per sequence against its paged
    cache (B4 Hq32 Hkv8 D128 bf16, kv_len U[2048, 8192], causal with the
    diagonal at kv_len - 512); three input sets rotate.  Algorithmic flops:
    4 D per visible (query, key) pair."""
    B, Hq, Hkv, Tq, D = 4, 32, 8, 512, 128
    sets, flops = [], []
    for s in range(3):
        d = wl.paged_prefill_inputs(B, Hq, Hkv, Tq, D, "bf16", 1009 + 100 * s,
                                    length_range=(2048, 8192))
        sets.append((dev(d["q"]), dev(d["k_pages"]), dev(d["v_pages"]), dev(d["block_table"]),
                     dev(d["kv_lens"]), d["scale"]))
        L = d["kv_lens"].astype(np.float64)
        flops.append(4.0 * D * Hq * float(np.sum(Tq * (L - Tq) + Tq * (Tq + 1) / 2)))
    o = torch.empty((B, Hq, Tq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, Tq), device="cuda")

    def step(i):
        q, kp, vp, bt, kl, scale = sets[i % 3]
        attn.attn_prefill_paged(q, kp, vp, bt, kl, o, lse, causal=True, scale=scale)

    durs, span, _ = time_launches(step, steps, warmup)
    mean_flops = float(np.mean([flops[i % 3] for i in range(steps)]))
    mean_ms = span / steps
    return dict(workload="chunked prefill B4 Hq32 Hkv8 D128 bf16, 512-token chunk against a "
                         "paged cache, kv_len U[2048,8192], causal (bottom-right), page 16",
                mean_ms=mean_ms, launch_us=percentiles_us(durs),
                tflops=round(mean_flops / (mean_ms * 1e-3) / 1e12, 2),
                frac_mfma=round(mean_flops / (mean_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4))


def kv_bytes(lengths, hkv, d, elem=2):
    return int(np.sum(np.asarray(lengths, np.int64))) * hkv * d * 2 * elem


DECODE_SOURCES = ("decode_mfma.hip", "decode.hip", "common.h")


def hbm_roofline(nbytes, mean_ms, kernels, counters, digest):
    """Roofline object of an HBM-bound step: ``nbytes`` algorithmic bytes
    over the mean step duration; traffic from the committed counters of the
    same source (None when absent or stale)."""
    achieved = nbytes / (mean_ms * 1e-3) / 1e9
    return dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                frac=round(achieved / PEAK_HBM_GBS, 4), traffic=measured_traffic(counters, digest),
                kernel=kernels, algorithmic_bytes=int(nbytes), source_digest=digest)


def decode_kernels(D, fp8, max_splits):
    k = f"decode_mfma_kernel<{D},{'true' if fp8 else 'false'}>"
    return k + (f" + decode_combine_kernel<{D}>" if max_splits > 1 else "")


def cpu_decode_sample(d, target_s, prefix_len=0):
    """The fp64 oracle on the sequences of a decode workload in order (one
    call per batch of sequences, sized from the rate so far to end near
    ``target_s``; the workload starts over when it runs out), in KV GB/s:
    each sampled sequence's K+V bytes (bf16) over the oracle's time.  With
    ``prefix_len`` (the cascade) each request attends the shared prefix + its
    suffix, and the rate is the whole workload's bytes (prefix once) over
    the sample's time scaled to every request."""
    import oracle
    threads = oracle.default_threads()
    if prefix_len:
        lens, run = d["suffix_lens"], lambda sl: oracle.cascade_decode(
            d["q"][sl], d["k_pages"], d["v_pages"], d["prefix_pages"], prefix_len,
            d["suffix_table"][sl], d["suffix_lens"][sl], d["scale"], threads=threads)
    else:
        lens, run = d["kv_lens"], lambda sl: oracle.decode_paged(
            d["q"][sl], d["k_pages"], d["v_pages"], d["block_table"][sl], d["kv_lens"][sl],
            d["scale"], threads=threads)
    B, Hkv, D = len(lens), d["Hkv"], d["D"]
    done, tokens, t_used, n = 0, 0, 0.0, 1
    t0 = time.perf_counter()
    while t_used < target_s:
        lo = done % B
        sl = slice(lo, min(B, lo + n))
        run(sl)
        done += sl.stop - lo
        tokens += int(np.sum(lens[sl]))
        t_used = time.perf_counter() - t0
        n = max(1, int((target_s - t_used) / (t_used / done)))
    if prefix_len:
        nbytes = kv_bytes([prefix_len], Hkv, D) + kv_bytes(lens, Hkv, D)
        rate = nbytes / (t_used * B / done) / 1e9
        what = (f"{done} requests (the workload's {B} in order, repeated; each the "
                f"{prefix_len}-token prefix + its suffix), {t_used:.1f} s, fp64, "
                f"rate scaled to one pass over the {B}")
    else:
        rate = tokens * Hkv * D * 2 * 2 / t_used / 1e9
        what = (f"{done} sequences (the workload's {B} in order, repeated; {tokens} KV "
                f"tokens), {t_used:.1f} s, fp64")
    return dict(value=round(rate, 4), unit="GB/s", cores=threads, kind="oracle", sample=what,
                seconds=round(t_used, 2))


def bench_decode(name, steps, warmup, cpu_s=0.0):
    d = wl.workload(name)
    q = dev(d["q"])
    kp, vp = dev(d["k_pages"]), dev(d["v_pages"])
    bt, kl = dev(d["block_table"]), dev(d["kv_lens"])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], device="cuda")
    maxlen = int(d["kv_lens"].max())
    split = d.get("split_tokens", 0)
    ws_bytes = attn.attn_decode_workspace_bytes(d["B"], d["Hq"], d["Hkv"], d["D"], maxlen, split)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def step(i):
        attn.attn_decode_paged(q, kp, vp, bt, kl, o, lse, max_kv_len=maxlen, scale=d["scale"],
                               workspace=ws, split_tokens=split)

    durs, span, _ = time_launches(step, steps, warmup)
    nbytes = kv_bytes(d["kv_lens"], d["Hkv"], d["D"])
    mean_ms = span / steps
    split_used, nsplit = attn.attn_decode_plan(d["B"], d["Hkv"], maxlen, 0, split)
    del kp, vp
    digest = source_digest(*DECODE_SOURCES)
    r = dict(workload=wl.WORKLOADS[name], kv_bytes=nbytes, sum_kv_len=int(d["kv_lens"].sum()),
             mean_ms=mean_ms, launch_us=percentiles_us(durs),
             gbs=nbytes / (mean_ms * 1e-3) / 1e9,
             frac_hbm=round(nbytes / (mean_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
             split_tokens=split_used, max_splits=nsplit,
             roofline=hbm_roofline(nbytes, mean_ms, decode_kernels(d["D"], False, nsplit),
                                   name, digest))
    if cpu_s > 0:
        r["cpu_oracle"] = cpu_decode_sample(d, cpu_s)
    return r


def bench_decode_fp8(name, steps, warmup):
    """Workload n's shapes and lengths over an FP8 (OCP E4M3) cache; KV bytes
    are one byte per element."""
    d = wl.fp8_workload(name)
    q = dev(d["q"])
    kp, vp = dev(d["k_pages"]), dev(d["v_pages"])
    bt, kl = dev(d["block_table"]), dev(d["kv_lens"])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], device="cuda")
    maxlen = int(d["kv_lens"].max())
    split = d.get("split_tokens", 0)
    ws_bytes = attn.attn_decode_workspace_bytes(d["B"], d["Hq"], d["Hkv"], d["D"], maxlen, split)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def step(i):
        attn.attn_decode_paged_fp8(q, kp, vp, d["k_scale"], d["v_scale"], bt, kl, o, lse,
                                   max_kv_len=maxlen, scale=d["scale"], workspace=ws,
                                   split_tokens=split)

    durs, span, _ = time_launches(step, steps, warmup)
    nbytes = kv_bytes(d["kv_lens"], d["Hkv"], d["D"], elem=1)
    mean_ms = span / steps
    _, nsplit = attn.attn_decode_plan(d["B"], d["Hkv"], maxlen, 0, split)
    del kp, vp
    return dict(workload=wl.FP8_WORKLOADS[name], kv_bytes=nbytes, sum_kv_len=int(d["kv_lens"].sum()),
                mean_ms=mean_ms, launch_us=percentiles_us(durs),
                gbs=nbytes / (mean_ms * 1e-3) / 1e9,
                frac_hbm=round(nbytes / (mean_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                tokens_per_s=int(d["kv_lens"].sum()) * d["Hkv"] / (mean_ms * 1e-3),
                roofline=hbm_roofline(nbytes, mean_ms, decode_kernels(d["D"], True, nsplit),
                                      name + "_fp8", source_digest(*DECODE_SOURCES)))


def bench_cascade(steps, warmup, fp8=False, cpu_s=0.0):
    """Shared-prefix cascade decode (64 requests, 4096-token prefix, suffixes
    U[128, 1024], H32 D128): prefix stage + suffix decode + merge on one stream, timed as
    one step.  With fp8 the cache is OCP E4M3 bytes with per-tensor scales."""
    c = wl.fp8_workload(wl.CASCADE) if fp8 else wl.workload(wl.CASCADE)
    q = dev(c["q"])
    kp, vp = dev(c["k_pages"]), dev(c["v_pages"])
    pp, st, sl = dev(c["prefix_pages"]), dev(c["suffix_table"]), dev(c["suffix_lens"])
    R, H, D = q.shape
    o_p, o_s = torch.empty_like(q), torch.empty_like(q)
    l_p, l_s = (torch.empty((R, H), device="cuda") for _ in range(2))
    maxlen = int(c["suffix_lens"].max())
    cache_dt = attn.FP8_E4M3 if fp8 else attn.BF16
    ws_p = torch.empty(max(1, attn.attn_shared_prefix_workspace_bytes(R, H, c["Hkv"], D,
                                                                          c["prefix_len"],
                                                                          cache_dt)),
                       dtype=torch.uint8, device="cuda")
    ws_s = torch.empty(max(1, attn.attn_decode_workspace_bytes(R, H, c["Hkv"], D, maxlen)),
                       dtype=torch.uint8, device="cuda")
    flush = torch.zeros(128 << 20, dtype=torch.float32, device="cuda")

    def before(i):
        # evict the last-level cache (256 MB) between repetitions by reading
        # 512 MB; a write would leave dirty lines whose write-back then
        # competes with the timed reads
        flush.sum()

    def step(i):
        if fp8:
            attn.attn_decode_shared_prefix_fp8(q, kp, vp, c["k_scale"], c["v_scale"], pp,
                                               c["prefix_len"], o_p, l_p, scale=c["scale"],
                                               workspace=ws_p)
            attn.attn_decode_paged_fp8(q, kp, vp, c["k_scale"], c["v_scale"], st, sl, o_s, l_s,
                                       max_kv_len=maxlen, scale=c["scale"], workspace=ws_s)
        else:
            attn.attn_decode_shared_prefix(q, kp, vp, pp, c["prefix_len"], o_p, l_p,
                                           scale=c["scale"], workspace=ws_p)
            attn.attn_decode_paged(q, kp, vp, st, sl, o_s, l_s, max_kv_len=maxlen,
                                   scale=c["scale"], workspace=ws_s)
        attn.attn_merge_states(o_p, l_p, o_s, l_s)

    durs, span, _ = time_launches(step, steps, warmup, before=before)
    elem = 1 if fp8 else 2
    nbytes = (kv_bytes([c["prefix_len"]], c["Hkv"], D, elem=elem)
              + kv_bytes(c["suffix_lens"], c["Hkv"], D, elem=elem))
    mean_ms = float(np.mean(durs))
    _, nsplit = attn.attn_decode_plan(R, c["Hkv"], maxlen, 0, 0)
    kernels = (f"prefix_mfma_kernel<{D},{'true' if fp8 else 'false'}> + "
               f"decode_combine_kernel<{D}> (prefix chunks) + "
               + decode_kernels(D, fp8, nsplit) + " + merge_states_kernel")
    r = dict(workload=(wl.FP8_WORKLOADS if fp8 else wl.WORKLOADS)[wl.CASCADE], kv_bytes=nbytes,
             mean_ms=mean_ms, launch_us=percentiles_us(durs),
             gbs=nbytes / (mean_ms * 1e-3) / 1e9,
             frac_hbm=round(nbytes / (mean_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
             roofline=hbm_roofline(nbytes, mean_ms, kernels, wl.CASCADE + ("_fp8" if fp8 else ""),
                                   source_digest("prefix_mfma.hip", "merge.hip",
                                                 *DECODE_SOURCES)))
    if cpu_s > 0 and not fp8:
        r["cpu_oracle"] = cpu_decode_sample(c, cpu_s, prefix_len=c["prefix_len"])
    return r


def bench_graph_decode(steps, warmup, B, length_range, layers=8):
    """The attention of one decode step of a model with ``layers`` layers: per
    layer a GQA paged decode (B Hq32 Hkv8 D128 bf16, L~U[length_range], split
    decode + combine) over the layer's own cache.  Launched eagerly from
    Python, then replayed as one captured HIP graph; both timed back to back,
    so host launch gaps count."""
    per_layer = []
    for layer in range(layers):
        d = wl.paged_decode_inputs(B, 32, 8, 128, "bf16", 1100 + layer, length_range=length_range)
        maxlen = int(d["kv_lens"].max())
        t = dict(q=dev(d["q"]), kp=dev(d["k_pages"]), vp=dev(d["v_pages"]),
                 bt=dev(d["block_table"]), kl=dev(d["kv_lens"]), maxlen=maxlen, scale=d["scale"],
                 nbytes=kv_bytes(d["kv_lens"], 8, 128),
                 ws=torch.empty(max(1, attn.attn_decode_workspace_bytes(B, 32, 8, 128, maxlen)),
                                dtype=torch.uint8, device="cuda"))
        t["o"] = torch.empty_like(t["q"])
        t["lse"] = torch.empty(t["q"].shape[:2], device="cuda")
        per_layer.append(t)

    def step(i=0):
        for t in per_layer:
            attn.attn_decode_paged(t["q"], t["kp"], t["vp"], t["bt"], t["kl"], t["o"], t["lse"],
                                   max_kv_len=t["maxlen"], scale=t["scale"], workspace=t["ws"])

    eager, _, _ = time_launches(step, steps, warmup)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    graph, _, _ = time_launches(lambda i: g.replay(), steps, warmup)
    nbytes = sum(t["nbytes"] for t in per_layer)
    eager_ms, graph_ms = float(np.mean(eager)), float(np.mean(graph))
    lo, hi = length_range
    return dict(workload=f"{layers} layers x paged decode GQA B{B} Hq32 Hkv8 D128 bf16, "
                         f"L~U[{lo},{hi}], page 16, each layer its own cache",
                kv_bytes=nbytes, eager_us=round(eager_ms * 1e3, 2), graph_us=round(graph_ms * 1e3, 2),
                eager_gbs=round(nbytes / (eager_ms * 1e-3) / 1e9, 1),
                graph_gbs=round(nbytes / (graph_ms * 1e-3) / 1e9, 1))


def bench_flat_gemm(steps, warmup, ms=(1, 16, 64)):
    """Flat GEMM C = A W^T of the decode phase over the four projection
    shapes of one Llama2-7B layer (bf16 A [m, k], W [n, k], bf16 C), for
    m tokens per step.  Each shape rotates through enough device copies of W
    (>= 768 MB) that the 256 MB last-level cache cannot hold them; launches
    run back to back.  Bytes: W + A + C (W dominates)."""
    res = {m: {} for m in ms}
    for name, (n, k) in wl.LLAMA2_7B_PROJECTIONS.items():
        d = wl.flat_gemm_inputs(max(ms), n, k, 1200)
        w0 = dev(d["w"])
        copies = max(2, -(-(768 << 20) // (n * k * 2)))
        ws = [w0] + [w0.clone() for _ in range(copies - 1)]
        for m in ms:
            a = dev(d["a"][:m])
            c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")

            def step(i):
                attn.attn_flat_gemm(a, ws[i % copies], c)

            durs, span, _ = time_launches(step, steps, warmup)
            mean_ms = span / steps
            nbytes = n * k * 2 + m * k * 2 + m * n * 2
            res[m][name] = dict(n=n, k=k, us=round(mean_ms * 1e3, 2), bytes=nbytes,
                                gbs=round(nbytes / (mean_ms * 1e-3) / 1e9, 1),
                                frac_hbm=round(nbytes / (mean_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
        del ws, w0
        torch.cuda.empty_cache()
    out = {}
    for m in ms:
        r = res[m]
        tot_ms = sum(v["us"] for v in r.values()) * 1e-3
        tot_bytes = sum(v.pop("bytes") for v in r.values())
        r["layer"] = dict(us=round(tot_ms * 1e3, 2), gbs=round(tot_bytes / (tot_ms * 1e-3) / 1e9, 1),
                          frac_hbm=round(tot_bytes / (tot_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
        out[f"m{m}"] = r
    return dict(workload="flat GEMM C = A W^T, the four decode projections of one Llama2-7B "
                         "layer (qkv 12288x4096, o 4096x4096, gate_up 22016x4096, "
                         "down 4096x11008), bf16, m tokens", results=out)


def bench_hbm_read(reps=10):
    """The HBM read rate plain 16-byte loads reach on this GPU (a read-only
    kernel of the library over 4 GiB): 4 KiB blocks in place order and in a
    seeded random order (the scattered pages of a paged cache).  The
    memory-bound lines are also given as a fraction of the random-order rate."""
    blk = attn.load().attn_probe_block_bytes()
    nbytes = 4 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    n = nbytes // blk
    order = torch.from_numpy(np.random.default_rng(2024).permutation(n).astype(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = {}
    for key, o in (("in_order_4k_blocks", None), ("random_4k_blocks", order)):
        attn.attn_probe_hbm_read(buf, o, sink)
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            attn.attn_probe_hbm_read(buf, o, sink)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        med = float(np.median(ts))
        out[key] = dict(gbs=round(nbytes / (med * 1e-3) / 1e9, 1),
                        frac_hbm=round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                        us=round(med * 1e3, 1))
    del buf, order
    torch.cuda.empty_cache()
    return dict(workload="read-only kernel, 4 GiB as 4 KiB blocks, 16-byte loads, "
                         "two blocks per wavefront in flight, median of 10", **out)


GRAPH_CASES = (("decode_step_graph_b1", 1, (256, 1024)), ("decode_step_graph_b4", 4, (1024, 4096)))
DECODE_CPU_S = 4.0   # seconds of oracle time per decode workload sample


def cpu_baseline(target_s=10.0):
    """The fp64 oracle on (b, h) pairs of the prefill workload, timed on the
    host cores; throughput in the bench's unit (algorithmic causal TFLOP/s)."""
    import oracle
    inp = wl.workload(wl.PREFILL_CAUSAL)
    T, D = 1024, 128
    threads = oracle.default_threads()
    pairs, flops, t_used = 0, 0.0, 0.0
    t0 = time.perf_counter()
    while t_used < target_s:
        # (b, h) pairs in order, starting over after all 128
        n = max(1, min(threads, 128 - pairs % 128))
        idx = [((p % 128) // 32, p % 32) for p in range(pairs, pairs + n)]
        q = np.stack([inp["q"][b, h] for b, h in idx])[:, None]
        k = np.stack([inp["k"][b, h] for b, h in idx])[:, None]
        v = np.stack([inp["v"][b, h] for b, h in idx])[:, None]
        oracle.attention(q, k, v, True, inp["scale"], threads=threads)
        pairs += n
        flops += n * 4.0 * D * T * (T + 1) / 2
        t_used = time.perf_counter() - t0
    return dict(value=flops / t_used / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"{pairs} (b,h) pairs (the workload's 128 in order, repeated) of the "
                       f"causal B4 H32 T1024 D128 prefill, {t_used:.1f} s, fp64, full score matrix",
                seconds=round(t_used, 2))


SECTIONS = ("prefill", "prefill_noncausal", "torch_sdpa", "prefill_f32", "prefill_paged",
            "decode_mha",
            "decode_gqa", "decode_mha_fp8", "decode_gqa_fp8", "cascade", "cascade_fp8", "graph",
            "flat_gemm", "hbm_read")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true")
    ap.add_argument("--flat-gemm-only", action="store_true",
                    help="time only the flat GEMM of the decode projections (prints its JSON)")
    ap.add_argument("--only", choices=SECTIONS,
                    help="time one section and print its JSON instead of the bench line "
                         "(for profiling one workload)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB read + 1 GiB write elementwise kernel, "
                         "the reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        log("copy calibration: 3 x (1 GiB read + 1 GiB write)")

    K, W = args.steps, args.warmup
    if args.flat_gemm_only:
        args.only = "flat_gemm"
    if args.only:
        run = {
            "prefill": lambda: bench_prefill(K, W),
            "prefill_noncausal": lambda: bench_prefill_noncausal(K, W),
            "torch_sdpa": lambda: bench_torch_sdpa(K, W),
            "prefill_f32": lambda: bench_prefill_f32(K, W),
            "prefill_paged": lambda: bench_prefill_paged(K, W),
            "decode_mha": lambda: bench_decode(wl.DECODE_MHA, K, W),
            "decode_gqa": lambda: bench_decode(wl.DECODE_GQA, K, W),
            "decode_mha_fp8": lambda: bench_decode_fp8(wl.DECODE_MHA, K, W),
            "decode_gqa_fp8": lambda: bench_decode_fp8(wl.DECODE_GQA, K, W),
            "cascade": lambda: bench_cascade(K, W),
            "cascade_fp8": lambda: bench_cascade(K, W, fp8=True),
            "graph": lambda: {k: bench_graph_decode(K, W, B, lr) for k, B, lr in GRAPH_CASES},
            "flat_gemm": lambda: bench_flat_gemm(K, W),
            "hbm_read": lambda: bench_hbm_read(),
        }[args.only]
        log(f"{args.only} ...")
        print(json.dumps(run()), flush=True)
        return

    cpu_s = 0.0 if args.no_cpu_baseline else DECODE_CPU_S
    log("prefill B4 H32 T1024 D128 causal bf16 ...")
    pre = bench_prefill(K, W)
    log(f"  {pre['tflops']:.1f} TFLOP/s, mean launch {pre['mean_launch_ms'] * 1e3:.1f} us")
    decode = {}
    paged_prefill = None
    flat = None
    noncausal = bench_prefill_noncausal(K, W)
    log(f"  non-causal: {noncausal['tflops']:.1f} TFLOP/s")
    log("torch's fused attention on the same shape (context) ...")
    try:
        library = bench_torch_sdpa(K, W)
    except Exception as e:   # context only: never let it stop the bench
        library = dict(unavailable=f"{type(e).__name__}: {str(e)[:160]}")
    if "causal_tflops" in library:
        library["this_library_causal_ratio"] = round(pre["tflops"] / library["causal_tflops"], 3)
        log(f"  {library.get('backend')}: causal {library['causal_tflops']:.1f}, non-causal "
            f"{library.get('noncausal_tflops', float('nan')):.1f} TFLOP/s")
    f32_mode = bench_prefill_f32(K, W)
    log(f"  fp32 test mode (B1 H1 T128 D64): {f32_mode['us']:.1f} us per launch")
    ceiling = None
    if not args.prefill_only:
        log("HBM read rate of plain loads (4 GiB, 4 KiB blocks) ...")
        ceiling = bench_hbm_read()
        log(f"  in order {ceiling['in_order_4k_blocks']['gbs']:.0f} GB/s, "
            f"random {ceiling['random_4k_blocks']['gbs']:.0f} GB/s")
        log("chunked prefill against the paged cache ...")
        paged_prefill = bench_prefill_paged(K, W)
        log(f"  {paged_prefill['tflops']:.1f} TFLOP/s")
        torch.cuda.empty_cache()
        for name in (wl.DECODE_MHA, wl.DECODE_GQA):
            log(f"{name} ...")
            decode[name] = bench_decode(name, K, W, cpu_s=cpu_s)
            log(f"  {decode[name]['gbs']:.0f} GB/s")
            torch.cuda.empty_cache()
        for name in (wl.DECODE_MHA, wl.DECODE_GQA):
            log(f"{name}, FP8 cache ...")
            decode[name + "_fp8"] = bench_decode_fp8(name, K, W)
            log(f"  {decode[name + '_fp8']['gbs']:.0f} GB/s")
            torch.cuda.empty_cache()
        log(f"{wl.CASCADE} ...")
        decode[wl.CASCADE] = bench_cascade(K, W, cpu_s=cpu_s)
        log(f"  {decode[wl.CASCADE]['gbs']:.0f} GB/s")
        torch.cuda.empty_cache()
        log(f"{wl.CASCADE}, FP8 cache ...")
        decode[wl.CASCADE + "_fp8"] = bench_cascade(K, W, fp8=True)
        log(f"  {decode[wl.CASCADE + '_fp8']['gbs']:.0f} GB/s")
        for key, B, lr in GRAPH_CASES:
            log(f"8-layer decode step B{B}, eager vs graph replay ...")
            decode[key] = bench_graph_decode(K, W, B, lr)
            log(f"  eager {decode[key]['eager_us']:.1f} us, graph {decode[key]['graph_us']:.1f} us")
        log("flat GEMM, Llama2-7B decode projections ...")
        flat = bench_flat_gemm(K, W)
        for mk, r in flat["results"].items():
            log(f"  {mk}: layer {r['layer']['us']:.1f} us, {r['layer']['gbs']:.0f} GB/s")
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle) ...")
        cpu = cpu_baseline()
        cpu["cpu_model"] = cpu_model()
        # the decode workloads' oracle samples, timed in their own sections
        cpu["decode"] = {k: v.pop("cpu_oracle") for k, v in decode.items() if "cpu_oracle" in v}
        log(f"  {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads")

    if ceiling is not None:
        top = ceiling["random_4k_blocks"]["gbs"]
        for v in decode.values():
            if "gbs" in v:
                v["frac_of_read_ceiling"] = round(v["gbs"] / top, 4)
        if flat is not None:
            for r in flat["results"].values():
                r["layer"]["frac_of_read_ceiling"] = round(r["layer"]["gbs"] / top, 4)

    line = {
        "metric": "prefill attn TFLOP/s + decode attn KV GB/s, % of MI355X roofline",
        "value": round(pre["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "spinup_s_per_section": SPINUP_S,
        "ms_per_step": round(pre["ms_per_step"], 5),
        "launch_us": pre["launch_us"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal prefill B4 H32 T1024 D128 bf16 (Llama2-7B attention "
                               "shape), scale 1/sqrt(128), seeded N(0,1) inputs",
                   "global_batch": 4, "seq_len": 1024, "heads": 32, "head_dim": 128},
        "roofline": pre["roofline"],
        "cpu_baseline": cpu,
        "decode": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                       for kk, vv in v.items()} for k, v in decode.items()},
        "prefill_paged": paged_prefill,
        "prefill_noncausal": noncausal,
        "prefill_library_reference": library,
        "prefill_f32_test_mode": f32_mode,
        "flat_gemm": flat,
        "hbm_read_ceiling": ceiling,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
