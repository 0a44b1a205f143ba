"""Benchmark of the paged KV cache hot path on one MI355X.

A step is one decode step of a single Qwen3-0.6B-shaped layer, issued as one
library call (pa_decode_step): the cache write of the 64 new tokens (bf16)
followed by paged decode attention over the whole batch, inputs resident in HBM.
Default workload: batch 64, H_Q=16, H_KV=8, d_h=128, block_size 16, context
lengths uniform in [512, 4096], 32,768-block bf16 pool.

Prints ONE JSON line. ``value`` is the step's KV-read throughput: the K/V bytes
attention must read (2 * sum(ctx) * H_KV * d_h * 2 B) divided by the measured
time per step (write + attention). ``roofline`` is for the dominant kernel
(decode attention) against MI355X's 8 TB/s; ``cpu_baseline`` is the CPU oracle
timed on this host on the same step; ``bulk_cache_write`` is the 32,768-token
bf16 -> fp8 cache write measured in the same run with a cold Infinity Cache;
``fp8_decode_b256`` and ``mla_k_write`` the other reported configurations, and
``prefill_chunks`` and ``mla_decode_b64`` the chunked-prefill and MLA latent
decode workloads, all timed in the same process, each after at least 100 ms of its
own untimed calls.

Other workloads (parity-test configurations, for measurement only):
``--workload decode_fp8_b256 | decode_b64_tp2 | decode_b64_bs8 | prefill_fp8 | mla_concat_swa | mla_fused |
prefill_chunks | prefill_chunks_fp8 | engine_decode_b64 | mla_decode_b64``.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MALL_FLUSH_BYTES = 1 << 30   # > 256 MB Infinity Cache
READ_PROBE_BYTES = 2 << 30   # streaming-read reference size
COPY_CAL_BYTES = 512 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # kernels in the first ~10 ms of GPU work after start-up were measured up
    # to 15% slower, so the default warm-up covers well past that
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--workload", default="decode_b64",
                   choices=["decode_b64", "decode_b64_tp2", "decode_b64_bs8", "prefill_fp8", "decode_fp8_b256",
                            "mla_concat_swa",
                            "mla_fused", "prefill_chunks", "prefill_chunks_fp8", "engine_decode_b64",
                            "mla_decode_b64"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--profile-steps", type=int, default=0,
                   help="only run --warmup then this many untimed steps (for rocprofv3 runs)")
    return p.parse_args()


class Timer:
    """Event pairs on one stream; mean duration in ms."""

    def __init__(self, torch, stream):
        self.torch, self.stream, self.pairs = torch, stream, []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs.append([e, None])

    def stop(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs[-1][1] = e

    def mean_ms(self):
        return float(np.mean([a.elapsed_time(b) for a, b in self.pairs]))

    def percentiles_ms(self, qs=(10, 50, 90)):
        return [round(float(x), 5) for x in np.percentile([a.elapsed_time(b) for a, b in self.pairs], qs)]


def gpu_spin_up(torch, pkv, min_ms: float = 200.0):
    """Untimed streaming reads for at least min_ms of wall time before any warm-up:
    GPU work in the first ~10 ms after start-up was measured up to 15% slower, and
    a short --warmup would otherwise leave that inside the timed region."""
    buf = torch.empty(READ_PROBE_BYTES // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty((pkv.ops.HBM_READ_SINK_UNITS, 4), dtype=torch.int32, device="cuda")
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(8):
            pkv.hbm_read(buf, sink)
        torch.cuda.synchronize()
    del buf, sink


SETTLE_MS = 100.0


def settle(torch, call, min_calls: int, min_ms: float = SETTLE_MS) -> int:
    """Untimed calls call(i) of one workload, at least min_calls and at least min_ms
    of wall time, before its timed calls: the clocks ramp over the first ~30 ms of a
    new kind of work (chunked-prefill calls measured 352 -> 237 us over their first
    120 calls, and the same again after 2 s idle), so a short warm-up would time
    the ramp, not the kernel. Returns the number of calls made."""
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(8):
            call(n)
            n += 1
        torch.cuda.synchronize()
        if n >= min_calls and (time.perf_counter() - t0) * 1e3 >= min_ms:
            return n


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


# --------------------------------------------------------------------------- #
# decode step (default)
# --------------------------------------------------------------------------- #

def setup_decode(torch, pkv, workloads, w):
    B, HQ, HKV, D, BS, NB = (w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_size,
                             w.block_size, w.num_blocks)
    dev = "cuda"
    if w.cache_dtype == "fp8":
        kc = workloads.device_fp8((NB, BS, HKV, D), dev, w.seed, w.k_scale)
        vc = workloads.device_fp8((NB, BS, HKV, D), dev, w.seed + 1, w.v_scale)
    else:
        kc = workloads.device_normal((NB, BS, HKV, D), torch.bfloat16, dev, w.seed)
        vc = workloads.device_normal((NB, BS, HKV, D), torch.bfloat16, dev, w.seed + 1)
    t = dict(kc=kc, vc=vc)
    t["q"] = workloads.device_normal((B, HQ, D), torch.bfloat16, dev, w.seed + 2)
    t["new_k"] = workloads.device_normal((B, HKV, D), torch.bfloat16, dev, w.seed + 3)
    t["new_v"] = workloads.device_normal((B, HKV, D), torch.bfloat16, dev, w.seed + 4)
    t["slots"] = torch.from_numpy(w.new_token_slots).to(dev)
    t["bt"] = torch.from_numpy(w.block_tables).to(dev)
    t["cl"] = torch.from_numpy(w.context_lens).to(dev)
    t["out"] = torch.empty((B, HQ, D), dtype=torch.bfloat16, device=dev)
    t["ks"] = None if w.k_scale is None else torch.tensor([w.k_scale], device=dev)
    t["vs"] = None if w.v_scale is None else torch.tensor([w.v_scale], device=dev)
    need = pkv.decode_attention_workspace_size(B, HQ, HKV, D, w.width, BS)
    t["ws"] = torch.zeros(need, dtype=torch.uint8, device=dev)
    return t


def decode_write(pkv, t, w):
    if w.cache_dtype == "fp8":
        pkv.reshape_and_cache(t["new_k"], t["new_v"], t["kc"], t["vc"], t["slots"],
                              k_scale=t["ks"], v_scale=t["vs"])
    else:
        pkv.reshape_and_cache(t["new_k"], t["new_v"], t["kc"], t["vc"], t["slots"])


def decode_attn(pkv, t, w):
    pkv.decode_attention(t["out"], t["q"], t["kc"], t["vc"], t["bt"], t["cl"], w.softmax_scale,
                         t["ks"], t["vs"], workspace=t["ws"])


def decode_step(pkv, t, w):
    """The whole step in one library call: the write, then the attention."""
    pkv.decode_step(t["new_k"], t["new_v"], t["slots"], t["out"], t["q"], t["kc"], t["vc"], t["bt"],
                    t["cl"], w.softmax_scale, t["ks"], t["vs"], workspace=t["ws"])


def decode_bytes(w):
    """Algorithmic HBM bytes of one attention call and of the new-token write."""
    ctx = w.context_lens.astype(np.int64)
    e_kv = 1 if w.cache_dtype == "fp8" else 2
    kv = int(2 * ctx.sum() * w.num_kv_heads * w.head_size * e_kv)
    qo = int(w.num_seqs * w.num_q_heads * w.head_size * (2 + 2))
    meta = int(np.sum(-(-ctx // w.block_size)) * 4 + 4 * w.num_seqs)
    scales = 8 if w.k_scale is not None else 0
    write = int(w.num_seqs * (8 + 2 * w.num_kv_heads * w.head_size * (2 + e_kv)))
    return kv, kv + qo + meta + scales, write


CPU_BASELINE_MIN_S = 10.0  # each CPU baseline repeats its sample for at least this long


def repeat_for(fn, min_s=CPU_BASELINE_MIN_S):
    """Run fn until at least min_s seconds have passed; (runs, seconds)."""
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        dt = time.perf_counter() - t0
        if dt >= min_s:
            return n, dt


def cpu_baseline_decode(torch, t, w, oracle):
    """The oracle on the same step (new-token write + attention), with all host
    threads and with one."""
    cdt = oracle.FP8_E4M3FN if w.cache_dtype == "fp8" else oracle.BF16
    raw = torch.uint8 if w.cache_dtype == "fp8" else torch.int16
    npv = np.uint8 if w.cache_dtype == "fp8" else np.uint16
    kc = t["kc"].view(raw).cpu().numpy().view(npv)
    vc = t["vc"].view(raw).cpu().numpy().view(npv)
    q = t["q"].view(torch.int16).cpu().numpy().view(np.uint16)
    nk = t["new_k"].view(torch.int16).cpu().numpy().view(np.uint16)
    nv = t["new_v"].view(torch.int16).cpu().numpy().view(np.uint16)
    kv_bytes, _, _ = decode_bytes(w)

    def step():
        oracle.reshape_and_cache(nk, nv, oracle.BF16, kc, vc, cdt, w.new_token_slots,
                                 k_scale=w.k_scale, v_scale=w.v_scale)
        oracle.decode_attention(q, oracle.BF16, kc, vc, cdt, w.block_tables, w.context_lens,
                                w.softmax_scale, w.k_scale, w.v_scale)
    threads = oracle.max_threads()
    n, dt = repeat_for(step)
    oracle.set_num_threads(1)  # the same sample on one thread
    try:
        n1, dt1 = repeat_for(step)
    finally:
        oracle.set_num_threads(threads)
    sample = (f"the whole step ({w.num_seqs} sequences, {int(w.context_lens.sum())} cached tokens): "
              "oracle write of the new tokens + fp64 attention, KV-read bytes / time")
    return {"value": round(n * kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "sample": f"{sample}; {n} steps in {dt:.1f} s", "cpu_model": cpu_model(),
            "single_thread": {"value": round(n1 * kv_bytes / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"{n1} steps in {dt1:.1f} s"}}


def run_decode(args, torch, pkv, workloads, w, metric_name):
    t = setup_decode(torch, pkv, workloads, w)
    stream = torch.cuda.current_stream()
    if args.profile_steps:
        copy_calibration(torch, pkv)
        for _ in range(args.warmup + args.profile_steps):
            decode_step(pkv, t, w)
        # the launches roofline.achieved times: attention calls back to back
        for _ in range(args.profile_steps):
            decode_attn(pkv, t, w)
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps, "workload": w.name}))
        return
    gpu_spin_up(torch, pkv)
    for _ in range(args.warmup):
        decode_step(pkv, t, w)
    torch.cuda.synchronize()
    # (1) the contract: K back-to-back steps between two synchronisations
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        decode_step(pkv, t, w)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    # (2) per-launch durations on the launch stream: K attention calls (split
    # pass + merge pass) back to back between two events, then K new-token writes
    ta, tw = Timer(torch, stream), Timer(torch, stream)
    ta.start()
    for _ in range(args.steps):
        decode_attn(pkv, t, w)
    ta.stop()
    tw.start()
    for _ in range(args.steps):
        decode_write(pkv, t, w)
    tw.stop()
    torch.cuda.synchronize()
    # (3) cold: the 256 MB Infinity Cache flushed before every attention call
    flush_src = torch.empty(MALL_FLUSH_BYTES // 2, dtype=torch.uint8, device="cuda")
    flush_dst = torch.empty_like(flush_src)
    tc = Timer(torch, stream)
    for _ in range(max(10, args.steps // 2)):
        pkv.hbm_copy(flush_dst, flush_src)
        tc.start()
        decode_attn(pkv, t, w)
        tc.stop()
    torch.cuda.synchronize()
    # (4) the streaming-copy reference on the same device (read + write bytes)
    tcopy = Timer(torch, stream)
    for _ in range(5):
        tcopy.start()
        pkv.hbm_copy(flush_dst, flush_src)
        tcopy.stop()
    torch.cuda.synchronize()
    copy_gbps = 2 * flush_src.numel() / (tcopy.mean_ms() * 1e-3) / 1e9
    del flush_src, flush_dst
    # (5) the streaming-read reference (2 GiB, well past the Infinity Cache)
    rd = torch.empty(READ_PROBE_BYTES // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty((pkv.ops.HBM_READ_SINK_UNITS, 4), dtype=torch.int32, device="cuda")
    for _ in range(3):
        pkv.hbm_read(rd, sink)
    tread = Timer(torch, stream)
    tread.start()
    for _ in range(10):
        pkv.hbm_read(rd, sink)
    tread.stop()
    torch.cuda.synchronize()
    read_gbps = READ_PROBE_BYTES / (tread.mean_ms() / 10 * 1e-3) / 1e9
    del rd, sink

    kv, attn_bytes, write_bytes = decode_bytes(w)
    attn_ms, write_ms, cold_ms = ta.mean_ms() / args.steps, tw.mean_ms() / args.steps, tc.mean_ms()
    achieved = attn_bytes / (attn_ms * 1e-3) / 1e9
    value = kv / (ms_per_step * 1e-3) / 1e9
    res = {
        "metric": metric_name,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.cache_dtype == "bf16" else "fp8_e4m3fn",
        "data": "synthetic (seeded N(0,1) K/V/q of Qwen3-0.6B shapes)",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_size": w.head_size,
                   "block_size": w.block_size, "num_blocks": w.num_blocks,
                   "context_lens": f"{int(w.context_lens.min())}..{int(w.context_lens.max())} "
                                   f"(sum {int(w.context_lens.sum())})",
                   "kv_read_bytes_per_step": kv},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(w.num_seqs / (ms_per_step * 1e-3), 1),
        "attention": {"ms": round(attn_ms, 5), "bytes": attn_bytes,
                      "GBps": round(achieved, 2), "cold_ms": round(cold_ms, 5),
                      "cold_GBps": round(attn_bytes / (cold_ms * 1e-3) / 1e9, 2),
                      "cold_p10_p50_p90_ms": tc.percentiles_ms()},
        "new_token_write": {"ms": round(write_ms, 5), "bytes": write_bytes,
                            "GBps": round(write_bytes / (write_ms * 1e-3) / 1e9, 2),
                            "tokens": w.num_seqs},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profiles("decode_attention", w.name),
                     "dominant_kernel": kernel_trace_from_profiles("decode_attention", w.name, attn_bytes)},
        "hbm_copy_GBps": round(copy_gbps, 1),
        "frac_of_copy": round(achieved / copy_gbps, 4),
        "hbm_read_GBps": round(read_gbps, 1),
        "frac_of_read": round(achieved / read_gbps, 4),
    }
    if args.workload == "decode_b64":
        # the cache-write target is quoted on the bulk write (a 64-token write is
        # launch-latency bound), so the default line carries it too
        res["bulk_cache_write"] = measure_bulk_write(args, torch, pkv, workloads)
        # the other reported configurations, timed in the same process: the
        # batch-256 fp8 decode and the MLA K assembly + SWA write (fused and not)
        res["fp8_decode_b256"] = measure_fp8_decode(args, torch, pkv, workloads)
        torch.cuda.empty_cache()
        res["mla_k_write"] = measure_mla_k_write(args, torch, pkv, workloads)
        torch.cuda.empty_cache()
        # the hot path's next rows, timed in the same process: chunked prefill
        # and MLA latent decode
        res["prefill_chunks"] = measure_prefill_chunks(args, torch, pkv, workloads)
        torch.cuda.empty_cache()
        res["mla_decode_b64"] = measure_mla_decode(args, torch, pkv, workloads)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        import oracle
        res["cpu_baseline"] = cpu_baseline_decode(torch, t, w, oracle)
    print(json.dumps(res))


def measure_fp8_decode(args, torch, pkv, workloads):
    """Batch-256 mixed-length decode over the 65,536-block fp8 pool: K attention
    calls back to back on HIP events (the roofline's launches), and K whole steps
    (new-token write + attention in one call)."""
    w = workloads.mixed_decode_fp8()
    t = setup_decode(torch, pkv, workloads, w)
    stream = torch.cuda.current_stream()
    settle(torch, lambda i: decode_attn(pkv, t, w), max(8, args.warmup))
    ta, ts = Timer(torch, stream), Timer(torch, stream)
    ta.start()
    for _ in range(args.steps):
        decode_attn(pkv, t, w)
    ta.stop()
    ts.start()
    for _ in range(args.steps):
        decode_step(pkv, t, w)
    ts.stop()
    torch.cuda.synchronize()
    kv, attn_bytes, _ = decode_bytes(w)
    ms, step_ms = ta.mean_ms() / args.steps, ts.mean_ms() / args.steps
    gbps = attn_bytes / (ms * 1e-3) / 1e9
    del t
    return {"workload": w.name, "ms": round(ms, 5), "bytes": attn_bytes, "kv_read_bytes": kv,
            "GBps": round(gbps, 2), "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "step_ms": round(step_ms, 5), "tokens_per_s": round(w.num_seqs / (step_ms * 1e-3), 1),
            "traffic": traffic_from_profiles("decode_attention", w.name),
            "dominant_kernel": kernel_trace_from_profiles("decode_attention", w.name, attn_bytes)}


def measure_mla_k_write(args, torch, pkv, workloads):
    """The MLA K assembly + SWA-remapped K-only write (16,384 tokens x 128 heads):
    the unfused path (concat to fp32, then the write) and the fused kernel, each
    K calls back to back (working sets of 4.3 and 1.2 GB, far past the Infinity
    Cache)."""
    stream = torch.cuda.current_stream()
    out = {}
    for label, builder in (("unfused", mla_unfused_step), ("fused", mla_fused_step)):
        step, nbytes, kernel, name, T = builder(torch, pkv, workloads)
        settle(torch, lambda i: step(), max(3, min(args.warmup, 10)))
        tm = Timer(torch, stream)
        tm.start()
        for _ in range(args.steps):
            step()
        tm.stop()
        torch.cuda.synchronize()
        ms = tm.mean_ms() / args.steps
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[label] = {"workload": name, "ms": round(ms, 5), "bytes": nbytes, "GBps": round(gbps, 2),
                      "frac": round(gbps / HBM_PEAK_GBPS, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
                      "traffic": traffic_from_profiles(kernel, name)}
        del step
        torch.cuda.empty_cache()
    return out


def copy_calibration(torch, pkv):
    """Three 512 MiB streaming copies (the reference kernel for profiler byte
    counters: 512 MiB read and 512 MiB written per launch)."""
    src = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        pkv.hbm_copy(dst, src)
    torch.cuda.synchronize()
    del src, dst


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on
    the current kernel source; otherwise None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.md")
    src = os.path.join(ROOT, "paged_kv_cache_304_amd", "csrc", f"{kernel}.hip")
    if not os.path.exists(path) or not os.path.exists(src):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256_16") != sha:
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def kernel_trace_from_profiles(kernel: str, workload: str, nbytes: int):
    """The dominant kernel's average duration from the committed kernel-trace
    summary (rocprofv3 --stats over the same launches), if it was taken on the
    current kernel source, and the algorithmic bytes of the whole call over that
    duration as a fraction of HBM peak; otherwise None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.md")
    src = os.path.join(ROOT, "paged_kv_cache_304_amd", "csrc", f"{kernel}.hip")
    if not os.path.exists(path) or not os.path.exists(src):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256_16") != sha or "dominant_avg_ns" not in fields:
        return None
    ns = float(fields["dominant_avg_ns"])
    gbps = nbytes / ns
    return {"kernel": fields.get("dominant_kernel"), "avg_ns": ns, "GBps": round(gbps, 2),
            "frac": round(gbps / HBM_PEAK_GBPS, 4)}


# --------------------------------------------------------------------------- #
# other workloads (measurement of the parity-test configurations)
# --------------------------------------------------------------------------- #

def bulk_write_bytes(w) -> int:
    """Algorithmic bytes of the bulk write: every token's slot, and for each kept
    token its bf16 K and V rows read and its fp8 K and V rows written."""
    kept = int((w["slot_mapping"] >= 0).sum())
    return 8 * w["num_tokens"] + kept * 2 * w["num_heads"] * w["head_size"] * (2 + 1)


def bulk_write_setup(torch, pkv, workloads):
    """The bulk bf16 -> fp8 write (32,768 tokens, 5% skipped) on four independent
    source/cache sets (191 MB each): calls that rotate over them find none of
    their data in the 256 MB Infinity Cache. Returns (call(i), algorithmic bytes,
    tokens)."""
    w = workloads.prefill_write_fp8()
    T, H, D, BS, NB = w["num_tokens"], w["num_heads"], w["head_size"], w["block_size"], w["num_blocks"]
    slots = torch.from_numpy(w["slot_mapping"]).cuda()
    ks = torch.tensor([w["k_scale"]], device="cuda")
    vs = torch.tensor([w["v_scale"]], device="cuda")
    sets = []
    for i in range(4):
        key = workloads.device_normal((T, H, D), torch.bfloat16, "cuda", w["seed"], std=w["std"])
        val = workloads.device_normal((T, H, D), torch.bfloat16, "cuda", w["seed"] + 1, std=w["std"])
        kc = torch.empty((NB, BS, H, D), dtype=torch.float8_e4m3fn, device="cuda")
        sets.append((key, val, kc, torch.empty_like(kc)))

    def call(i):
        key, val, kc, vc = sets[i % len(sets)]
        pkv.reshape_and_cache(key, val, kc, vc, slots, k_scale=ks, v_scale=vs)

    return call, bulk_write_bytes(w), T


BULK_WRITE_NAME = "bulk_prefill_write_32768_bf16_to_fp8"


def run_prefill_fp8(args, torch, pkv, workloads):
    call, nbytes, T = bulk_write_setup(torch, pkv, workloads)
    return generic(args, torch, pkv, lambda: call(0), nbytes, "reshape_and_cache", BULK_WRITE_NAME,
                   "fp8_e4m3fn", T, "tokens_per_s", rotating=call)


def measure_bulk_write(args, torch, pkv, workloads):
    """The cache-write target's workload measured beside the decode step: K calls
    back to back rotating over the four sets (cold Infinity Cache)."""
    call, nbytes, T = bulk_write_setup(torch, pkv, workloads)
    stream = torch.cuda.current_stream()
    settle(torch, call, max(8, args.warmup))
    tm = Timer(torch, stream)
    tm.start()
    for i in range(args.steps):
        call(i)
    tm.stop()
    torch.cuda.synchronize()
    ms = tm.mean_ms() / args.steps
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"workload": BULK_WRITE_NAME, "ms": round(ms, 5), "bytes": nbytes, "GBps": round(gbps, 2),
            "frac": round(gbps / HBM_PEAK_GBPS, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "traffic": traffic_from_profiles("reshape_and_cache", BULK_WRITE_NAME)}


def mla_unfused_step(torch, pkv, workloads):
    """Workload 5 unfused: concat to an fp32 K, then the K-only bf16 write through
    the SWA table. Returns (step, algorithmic bytes, kernel, workload name, tokens)."""
    w = workloads.mla_concat_swa()
    T, H, nope, rope, BS, NB = (w["num_tokens"], w["num_heads"], w["nope_dim"], w["rope_dim"],
                                w["block_size"], w["num_blocks"])
    kn = workloads.device_normal((T, H, nope), torch.bfloat16, "cuda", w["seed"])
    kr = workloads.device_normal((T, 1, rope), torch.bfloat16, "cuda", w["seed"] + 1)
    k = torch.empty((T, H, nope + rope), dtype=torch.float32, device="cuda")
    cache = torch.empty((NB, BS, H, nope + rope), dtype=torch.bfloat16, device="cuda")
    slots = torch.from_numpy(w["slot_mapping"]).cuda()
    swa = torch.from_numpy(w["swa_slot_mapping"]).cuda()

    def step():
        pkv.concat_and_cast_mla_k(k, kn, kr)
        pkv.reshape_and_cache(k, None, cache, None, slots, swa)

    kept = int((oracle_free_resolve(w) >= 0).sum())
    cat_bytes = T * H * nope * 2 + T * rope * 2 + T * H * (nope + rope) * 4
    write_bytes = 8 * T + 8 * T + kept * H * (nope + rope) * (4 + 2)
    return step, cat_bytes + write_bytes, "concat_and_cast", "mla_concat_16384x128_then_swa_write", T


def mla_fused_step(torch, pkv, workloads):
    """Workload 5 fused: one kernel writes the bf16 cache rows straight from
    k_nope / k_rope through the SWA table."""
    w = workloads.mla_concat_swa()
    T, H, nope, rope, BS, NB = (w["num_tokens"], w["num_heads"], w["nope_dim"], w["rope_dim"],
                                w["block_size"], w["num_blocks"])
    kn = workloads.device_normal((T, H, nope), torch.bfloat16, "cuda", w["seed"])
    kr = workloads.device_normal((T, 1, rope), torch.bfloat16, "cuda", w["seed"] + 1)
    cache = torch.empty((NB, BS, H, nope + rope), dtype=torch.bfloat16, device="cuda")
    slots = torch.from_numpy(w["slot_mapping"]).cuda()
    swa = torch.from_numpy(w["swa_slot_mapping"]).cuda()

    def step():
        pkv.concat_and_cache_mla_k(kn, kr, cache, slots, swa)

    final = oracle_free_resolve(w)
    kept = int((final >= 0).sum())
    kept1 = int((w["slot_mapping"] >= 0).sum())
    # kept tokens read their k_nope and k_rope rows; every token reads its slot,
    # tokens past stage one read their SWA entry; kept rows are written once
    nbytes = 8 * T + 8 * kept1 + kept * (H * nope * 2 + rope * 2) + kept * H * (nope + rope) * 2
    return step, nbytes, "concat_and_cast", "mla_fused_concat_and_cache_16384x128_swa", T


def run_mla(args, torch, pkv, workloads):
    step, nbytes, kernel, name, T = mla_unfused_step(torch, pkv, workloads)
    return generic(args, torch, pkv, step, nbytes, kernel, name, "bf16", T, "tokens_per_s")


def run_mla_fused(args, torch, pkv, workloads):
    """The same MLA K assembly and SWA write as run_mla, fused into one kernel."""
    step, nbytes, kernel, name, T = mla_fused_step(torch, pkv, workloads)
    return generic(args, torch, pkv, step, nbytes, kernel, name, "bf16", T, "tokens_per_s")


def oracle_free_resolve(w):
    """Final slot per token for the MLA workload's two-stage table (host bookkeeping)."""
    s = w["slot_mapping"]
    fin = np.where(s >= 0, w["swa_slot_mapping"][np.maximum(s, 0)], -1)
    return fin


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak


def prefill_flops(w) -> int:
    """Algorithmic flops of one chunked-prefill call: every (query, q head) pair
    does a D-long dot product and a D-long weighted sum (2 flops each per element)
    for every position it attends to (its own included)."""
    total = 0
    cu, ctx = w["cu_seqlens_q"], w["context_lens"]
    for b in range(w["num_seqs"]):
        n, L = int(cu[b + 1] - cu[b]), int(ctx[b])
        pos = L - n + np.arange(n)
        total += int(np.maximum(pos + 1, 0).sum())
    return total * w["num_q_heads"] * w["head_size"] * 4


def prefill_setup(torch, pkv, workloads, fp8=False):
    """Tensors of the chunked-prefill workload (bf16 or the same over an fp8 pool)
    and one call of it."""
    w = workloads.prefill_chunks()
    B, HQ, HKV, D, BS, NB, T = (w["num_seqs"], w["num_q_heads"], w["num_kv_heads"], w["head_size"],
                                w["block_size"], w["num_blocks"], w["num_tokens"])
    ks = vs = None
    if fp8:  # the same workload over an fp8 e4m3fn pool (k/v scales 0.05/0.04)
        w = dict(w, name=w["name"].replace("_bf16", "_fp8"))
        kc = workloads.device_fp8((NB, BS, HKV, D), "cuda", w["seed"], 0.05)
        vc = workloads.device_fp8((NB, BS, HKV, D), "cuda", w["seed"] + 1, 0.04)
        ks = torch.tensor([0.05], dtype=torch.float32, device="cuda")
        vs = torch.tensor([0.04], dtype=torch.float32, device="cuda")
    else:
        kc = workloads.device_normal((NB, BS, HKV, D), torch.bfloat16, "cuda", w["seed"])
        vc = workloads.device_normal((NB, BS, HKV, D), torch.bfloat16, "cuda", w["seed"] + 1)
    q = workloads.device_normal((T, HQ, D), torch.bfloat16, "cuda", w["seed"] + 2)
    out = torch.empty_like(q)
    cu = torch.from_numpy(w["cu_seqlens_q"]).cuda()
    bt = torch.from_numpy(w["block_tables"]).cuda()
    cl = torch.from_numpy(w["context_lens"]).cuda()

    def step():
        pkv.prefill_attention(out, q, cu, kc, vc, bt, cl, w["softmax_scale"], ks, vs)

    return w, step, q, kc, vc


def measure_prefill_chunks(args, torch, pkv, workloads):
    """The bf16 chunked-prefill workload (16 sequences, a 512-token chunk each),
    K calls back to back on HIP events: rate against the dense bf16 MFMA peak."""
    w, step, q, kc, vc = prefill_setup(torch, pkv, workloads)
    stream = torch.cuda.current_stream()
    settle(torch, lambda i: step(), max(5, min(args.warmup, 20)))
    tm = Timer(torch, stream)
    tm.start()
    for _ in range(args.steps):
        step()
    tm.stop()
    torch.cuda.synchronize()
    ms = tm.mean_ms() / args.steps
    flops = prefill_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    del step, q, kc, vc
    return {"workload": w["name"], "ms": round(ms, 5), "flops": flops, "TFLOPs": round(tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS, "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "tokens_per_s": round(w["num_tokens"] / (ms * 1e-3), 1),
            "traffic": traffic_from_profiles("prefill_attention", w["name"])}


def run_prefill_chunks(args, torch, pkv, workloads, fp8=False):
    w, step, q, kc, vc = prefill_setup(torch, pkv, workloads, fp8)
    B, HQ, HKV, D, BS, T = (w["num_seqs"], w["num_q_heads"], w["num_kv_heads"], w["head_size"],
                            w["block_size"], w["num_tokens"])
    flops = prefill_flops(w)
    kv_bytes = int(2 * int(w["context_lens"].astype(np.int64).sum()) * HKV * D * (1 if fp8 else 2))
    stream = torch.cuda.current_stream()
    if args.profile_steps:
        copy_calibration(torch, pkv)
        for _ in range(args.warmup + args.profile_steps):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps, "workload": w["name"]}))
        return
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    call_ms = ms  # a step is one call, launched back to back
    tflops = flops / (call_ms * 1e-3) / 1e12
    res = {
        "metric": "chunked-prefill paged attention TFLOP/s (1 MI355X)",
        "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 (fp8_e4m3fn cache)" if fp8 else "bf16",
        "data": "synthetic (seeded N(0,1) K/V/q of Qwen3-0.6B shapes)",
        "config": {"workload": w["name"], "num_seqs": B, "num_tokens": T, "num_q_heads": HQ,
                   "num_kv_heads": HKV, "head_size": D, "block_size": BS,
                   "context_lens": f"{int(w['context_lens'].min())}..{int(w['context_lens'].max())}",
                   "flops_per_step": flops, "kv_bytes_per_step": kv_bytes},
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_from_profiles("prefill_attention", w["name"])},
        "kv_read_GBps": round(kv_bytes / (call_ms * 1e-3) / 1e9, 1),
    }
    if not args.no_cpu_baseline:
        import oracle
        res["cpu_baseline"] = cpu_baseline_prefill(torch, q, kc, vc, w, oracle, fp8)
    print(json.dumps(res))


def cpu_baseline_prefill(torch, q, kc, vc, w, oracle, fp8=False):
    """The oracle on the whole call (every sequence, row and head; about ten
    seconds on 16 host cores), reported in the metric's unit."""
    qh = q.view(torch.int16).cpu().numpy().view(np.uint16)
    if fp8:
        kh, vh = kc.view(torch.uint8).cpu().numpy(), vc.view(torch.uint8).cpu().numpy()
        cdt, ks, vs = oracle.FP8_E4M3FN, 0.05, 0.04
    else:
        kh = kc.view(torch.int16).cpu().numpy().view(np.uint16)
        vh = vc.view(torch.int16).cpu().numpy().view(np.uint16)
        cdt, ks, vs = oracle.BF16, None, None
    n, dt = repeat_for(lambda: oracle.prefill_attention(
        qh, oracle.BF16, w["cu_seqlens_q"], kh, vh, cdt, w["block_tables"], w["context_lens"],
        w["softmax_scale"], ks, vs))
    flops = prefill_flops(w)
    return {"value": round(n * flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"the whole call ({w['num_tokens']} query rows x {w['num_q_heads']} heads, "
                      f"{flops / 1e9:.1f} GFLOP), {n} calls in {dt:.1f} s"}


def engine_prefill_rounds(plan, lens, chunk=16):
    """Give every sequence its first lens[b] positions in rounds of `chunk` tokens
    per sequence, all sequences per round (a chunked prefill): each sequence's
    blocks then interleave with the others' instead of lying side by side."""
    left = lens.astype(np.int64).copy()
    while left.any():
        seqs = np.nonzero(left)[0].astype(np.int32)
        num = np.minimum(left[seqs], chunk).astype(np.int32)
        plan(seqs, num)
        left[seqs] -= num


def engine_width(args, w) -> int:
    """Table width that holds every context after all the steps this run takes."""
    loops = args.warmup + max(2 * args.steps, args.profile_steps)
    return -(-(int(w.context_lens.max()) + loops) // w.block_size)


def run_engine_decode(args, torch, pkv, workloads):
    """The batch-64 decode workload driven the way an engine drives it: each step
    the native block manager plans one new token per sequence (slots, tables,
    lengths), one host-to-device copy uploads that metadata, and pa_decode_step
    writes and attends. Contexts grow by one token per step; planning of step
    k+1 overlaps the GPU work of step k (two pinned staging blobs)."""
    import dataclasses
    w = workloads.qwen3_decode_b64()
    B, HQ, HKV, D, BS, NB = (w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_size,
                             w.block_size, w.num_blocks)
    W = engine_width(args, w)
    bm = pkv.BlockManager(NB, BS, B, W, B, 16 * B)
    lens = w.context_lens.astype(np.int64) - 1          # positions cached before the first step
    engine_prefill_rounds(lambda s, n: bm.plan_host(s, n), lens)
    stager = pkv.StepStager(bm)
    dev = "cuda"
    kc = workloads.device_normal((NB, BS, HKV, D), torch.bfloat16, dev, w.seed)
    vc = workloads.device_normal((NB, BS, HKV, D), torch.bfloat16, dev, w.seed + 1)
    q = workloads.device_normal((B, HQ, D), torch.bfloat16, dev, w.seed + 2)
    nk = workloads.device_normal((B, HKV, D), torch.bfloat16, dev, w.seed + 3)
    nv = workloads.device_normal((B, HKV, D), torch.bfloat16, dev, w.seed + 4)
    out = torch.empty_like(q)
    ws = torch.zeros(pkv.decode_attention_workspace_size(B, HQ, HKV, D, W, BS), dtype=torch.uint8,
                     device=dev)
    seqs = np.arange(B, dtype=np.int32)
    ones = np.ones(B, dtype=np.int32)
    stream = torch.cuda.current_stream()

    def step():
        d = stager.step(seqs, ones, stream=stream)
        pkv.decode_step(nk, nv, d.slot_mapping, out, q, kc, vc, d.block_tables, d.context_lens,
                        w.softmax_scale, workspace=ws, stream=stream)
        lens[:] += 1
        return d

    def kv_bytes():
        return int(2 * lens.sum() * HKV * D * 2)

    if args.profile_steps:
        copy_calibration(torch, pkv)
        for _ in range(args.warmup + args.profile_steps):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps, "workload": "engine_decode_b64"}))
        return
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # (1) K whole steps (plan + upload + write + attention) between two synchronisations
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    kv = 0
    h0 = time.perf_counter()
    t0.record(stream)
    for _ in range(args.steps):
        step()
        kv += kv_bytes()
    t1.record(stream)
    h1 = time.perf_counter()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    host_us_per_step = (h1 - h0) / args.steps * 1e6
    # (2) the parts: host planning, the upload copy, decode attention on the uploaded metadata
    blob = stager.host[0]
    plan_s = 0.0
    tu, ta = Timer(torch, stream), Timer(torch, stream)
    attn_bytes = 0
    for _ in range(args.steps):
        torch.cuda.synchronize()
        s0 = time.perf_counter()
        rows, toks, _ = bm.plan_into(blob.data_ptr(), blob.numel(), seqs, ones)
        plan_s += time.perf_counter() - s0
        lens[:] += 1
        tu.start()
        pkv._lib.check(pkv._lib.lib.pa_bm_upload(bm._h, blob.data_ptr(), stager.dev.data_ptr(), rows,
                                                 stream.cuda_stream))
        tu.stop()
        lay = bm.layout
        d = stager.dev
        bt = d[lay.block_tables:lay.block_tables + 4 * B * W].view(torch.int32).view(B, W)
        cl = d[lay.context_lens:lay.context_lens + 4 * B].view(torch.int32)
        ta.start()
        pkv.decode_attention(out, q, kc, vc, bt, cl, w.softmax_scale, workspace=ws)
        ta.stop()
        attn_bytes += decode_bytes(dataclasses.replace(w, context_lens=lens.astype(np.int32)))[1]
    torch.cuda.synchronize()
    attn_ms, up_ms = ta.mean_ms(), tu.mean_ms()
    attn_bytes //= args.steps
    achieved = attn_bytes / (attn_ms * 1e-3) / 1e9
    up_bytes = int(bm.layout.block_tables + 4 * B * W)
    value = kv / args.steps / (ms_per_step * 1e-3) / 1e9
    res = {
        "metric": "paged decode attn KV-read GB/s & % HBM peak; cache-write GB/s (1 MI355X)",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) K/V/q of Qwen3-0.6B shapes)",
        "config": {"workload": "engine_decode_b64", "num_seqs": B, "num_q_heads": HQ,
                   "num_kv_heads": HKV, "head_size": D, "block_size": BS, "num_blocks": NB,
                   "context_lens": f"{int(w.context_lens.min())}..{int(w.context_lens.max())} "
                                   "at the first step, +1 per step",
                   "allocation": "native block manager, 16-token chunked prefill rounds"},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "host": {"plan_us": round(plan_s / args.steps * 1e6, 2),
                 "enqueue_us_per_step": round(host_us_per_step, 2),
                 "upload_us": round(up_ms * 1e3, 2), "upload_bytes": up_bytes},
        "attention": {"ms": round(attn_ms, 5), "bytes": attn_bytes, "GBps": round(achieved, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        import oracle
        res["cpu_baseline"] = cpu_baseline_engine(torch, w, W, oracle, kc, vc, q, nk, nv, lens)
    print(json.dumps(res))


def cpu_baseline_engine(torch, w, W, oracle, kc, vc, q, nk, nv, lens):
    """The oracle on one engine step: its block pool brought to the same state
    (untimed), then -- timed -- planning the step, the new-token write and fp64
    attention."""
    from oracle.block_pool import BlockPool
    B, BS = w.num_seqs, w.block_size
    pool = BlockPool(w.num_blocks, BS, W)
    engine_prefill_rounds(lambda s, n: pool.step(s, n), w.context_lens.astype(np.int64) - 1)
    grown = lens - (w.context_lens.astype(np.int64) - 1)   # steps the GPU side has taken
    for _ in range(int(grown[0])):
        pool.step(range(B), [1] * B)
    kch = kc.view(torch.int16).cpu().numpy().view(np.uint16)
    vch = vc.view(torch.int16).cpu().numpy().view(np.uint16)
    qh = q.view(torch.int16).cpu().numpy().view(np.uint16)
    nkh = nk.view(torch.int16).cpu().numpy().view(np.uint16)
    nvh = nv.view(torch.int16).cpu().numpy().view(np.uint16)
    t0 = time.perf_counter()
    sm, bt, cl, _ = pool.step_arrays(range(B), [1] * B, W)
    plan_s = time.perf_counter() - t0

    def attend():
        oracle.reshape_and_cache(nkh, nvh, oracle.BF16, kch, vch, oracle.BF16, sm)
        oracle.decode_attention(qh, oracle.BF16, kch, vch, oracle.BF16, bt, cl, w.softmax_scale)
    n, dt = repeat_for(attend)
    per_step = plan_s + dt / n
    kv = int(2 * cl.astype(np.int64).sum() * w.num_kv_heads * w.head_size * 2)
    return {"value": round(kv / per_step / 1e9, 4), "unit": "GB/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"one engine step ({B} sequences, {int(cl.sum())} tokens): oracle block-pool "
                      f"planning ({plan_s * 1e6:.0f} us, once) + write + fp64 attention ({n} times in "
                      f"{dt:.1f} s), KV-read bytes / time per step"}


def mla_segments(ctx: np.ndarray, grid: int, tile: int = 32) -> int:
    """(workgroup, sequence) segments of the persistent MLA split: the work of
    all sequences in sequence order forms one list of units (a sequence with
    tiles of 32 positions contributes one unit for its absorbed query, then one
    per tile), cut into ``grid`` even ranges (the first T % grid ranges one unit
    longer); a segment is a sequence's tiles within one range."""
    tiles = -(-ctx.astype(np.int64) // tile)
    units = np.where(tiles > 0, tiles + 1, 0)
    ts = np.concatenate([[0], np.cumsum(units)])
    T = int(ts[-1])
    q, r = divmod(T, grid)
    starts = np.array([w * q + min(w, r) for w in range(grid + 1)], dtype=np.int64)
    n = 0
    for w in range(grid):
        t0, t1 = starts[w], starts[w + 1]
        if t1 > t0:  # a sequence's tiles are units ts[b] + 1 .. ts[b + 1] - 1
            n += int(np.sum((np.minimum(t1, ts[1:]) > np.maximum(t0, ts[:-1] + 1))))
    return n


def mla_bytes(w, grid: int = 256) -> dict:
    """HBM bytes of one MLA decode call. ``algorithmic``: the latent rows, block
    tables and lengths, weights and queries read once and the output written
    (what the roofline is measured on). ``call``: that plus the workspace
    traffic of this design on a ``grid``-workgroup split -- the absorbed query
    (hi + lo) written once and read once per segment, the segments' partial
    outputs written and read once, the tile plan written and read."""
    ctx = w["context_lens"].astype(np.int64)
    B, H, QK, R, DC, DV = (w["num_seqs"], w["num_heads"], w["qk_nope_dim"], w["rope_dim"],
                           w["kv_lora_rank"], w["v_dim"])
    row = DC + R
    segs = mla_segments(ctx, grid)
    latent = int(ctx.sum() * row * 2)
    tables = int(np.sum(-(-ctx // w["block_size"])) * 4 + 4 * B)
    weights = DC * H * (QK + DV) * 2
    q = B * H * (QK + R) * 2
    qt = B * H * row * 2 * 2
    partial = segs * H * (DC + 2) * 4
    plan = (B + 1) * 4
    out = B * H * DV * 2
    split = latent + tables + segs * H * row * 2 * 2 + partial
    return {"latent": latent, "split": split, "segments": segs,
            "algorithmic": latent + tables + weights + q + out,
            "call": (latent + tables + weights + q + qt + segs * H * row * 2 * 2 + 2 * partial
                     + 2 * plan + out)}


def mla_setup(torch, pkv, workloads):
    """Tensors of the batch-64 MLA decode workload, its decode step (the new
    latent rows written, then the attention: one pa_mla_decode_step call) and
    its attention call alone."""
    w = workloads.mla_decode_b64()
    B, H, QK, R, DC, DV = (w["num_seqs"], w["num_heads"], w["qk_nope_dim"], w["rope_dim"],
                           w["kv_lora_rank"], w["v_dim"])
    BS, NB, s = w["block_size"], w["num_blocks"], w["seed"]
    cache = workloads.device_normal((NB, BS, DC + R), torch.bfloat16, "cuda", s)
    q_nope = workloads.device_normal((B, H, QK), torch.bfloat16, "cuda", s + 1)
    q_rope = workloads.device_normal((B, H, R), torch.bfloat16, "cuda", s + 2)
    w_uk = workloads.device_normal((DC, H * QK), torch.bfloat16, "cuda", s + 3, std=w["w_std"])
    w_uv = workloads.device_normal((DC, H * DV), torch.bfloat16, "cuda", s + 4, std=w["w_std"])
    new_c = workloads.device_normal((B, 1, DC), torch.bfloat16, "cuda", s + 5)
    new_r = workloads.device_normal((B, 1, R), torch.bfloat16, "cuda", s + 6)
    slots = torch.from_numpy(w["new_token_slots"]).cuda()
    bt = torch.from_numpy(w["block_tables"]).cuda()
    cl = torch.from_numpy(w["context_lens"]).cuda()
    out = torch.empty((B, H, DV), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(pkv.mla_decode_workspace_size(B, H, QK, R, DC, DV, bt.shape[1], BS), dtype=torch.uint8,
                     device="cuda")

    def step():
        pkv.mla_decode_step(new_c, new_r, slots, out, q_nope, q_rope, w_uk, w_uv, cache, bt, cl,
                            w["softmax_scale"], workspace=ws)

    def attend():
        pkv.mla_decode_attention(out, q_nope, q_rope, w_uk, w_uv, cache, bt, cl, w["softmax_scale"],
                                 workspace=ws)

    return w, step, attend, (cache, q_nope, q_rope, w_uk, w_uv)


def measure_mla_decode(args, torch, pkv, workloads):
    """The batch-64 MLA latent decode: K attention calls back to back on HIP
    events (absorb + split + merge; the roofline's launches) and K whole steps
    (latent write + attention in one pa_mla_decode_step call)."""
    w, step, attend, tensors = mla_setup(torch, pkv, workloads)
    stream = torch.cuda.current_stream()
    settle(torch, lambda i: step(), max(5, min(args.warmup, 20)))
    ta, ts = Timer(torch, stream), Timer(torch, stream)
    ta.start()
    for _ in range(args.steps):
        attend()
    ta.stop()
    ts.start()
    for _ in range(args.steps):
        step()
    ts.stop()
    torch.cuda.synchronize()
    ms, step_ms = ta.mean_ms() / args.steps, ts.mean_ms() / args.steps
    nb = mla_bytes(w, grid=min(256, torch.cuda.get_device_properties(0).multi_processor_count))
    gbps = nb["algorithmic"] / (ms * 1e-3) / 1e9
    del step, attend, tensors
    return {"workload": w["name"], "ms": round(ms, 5), "bytes": nb["algorithmic"], "GBps": round(gbps, 2),
            "frac": round(gbps / HBM_PEAK_GBPS, 4), "bytes_with_workspace": nb["call"],
            "step_ms": round(step_ms, 5), "tokens_per_s": round(w["num_seqs"] / (step_ms * 1e-3), 1),
            "traffic": traffic_from_profiles("mla_decode", w["name"])}


def run_mla_decode(args, torch, pkv, workloads):
    """MLA decode step over a latent paged cache (synthetic DeepSeek-V2-Lite shapes):
    the batch's new latent rows written, then the attention, in one
    pa_mla_decode_step call."""
    w, step, attend, (cache, q_nope, q_rope, w_uk, w_uv) = mla_setup(torch, pkv, workloads)
    B, H, QK, R, DC, DV = (w["num_seqs"], w["num_heads"], w["qk_nope_dim"], w["rope_dim"],
                           w["kv_lora_rank"], w["v_dim"])
    BS, NB = w["block_size"], w["num_blocks"]
    stream = torch.cuda.current_stream()

    if args.profile_steps:
        copy_calibration(torch, pkv)
        for _ in range(args.warmup + args.profile_steps):
            step()
        # the launches roofline.achieved times: attention calls back to back
        for _ in range(args.profile_steps):
            attend()
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps, "workload": w["name"]}))
        return
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    ta = Timer(torch, stream)  # K calls back to back
    ta.start()
    for _ in range(args.steps):
        attend()
    ta.stop()
    torch.cuda.synchronize()
    attn_ms = ta.mean_ms() / args.steps
    nb = mla_bytes(w, grid=min(256, torch.cuda.get_device_properties(0).multi_processor_count))
    value = nb["latent"] / (ms * 1e-3) / 1e9
    achieved = nb["algorithmic"] / (attn_ms * 1e-3) / 1e9
    ctx = w["context_lens"]
    res = {
        "metric": "paged decode attn KV-read GB/s & % HBM peak; cache-write GB/s (1 MI355X)",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) latent rows and queries, N(0,1/512) weights)",
        "config": {"workload": w["name"], "num_seqs": B, "num_heads": H, "qk_nope_dim": QK,
                   "rope_dim": R, "kv_lora_rank": DC, "v_dim": DV, "block_size": BS,
                   "num_blocks": NB, "context_lens": f"{int(ctx.min())}..{int(ctx.max())} "
                                                     f"(sum {int(ctx.sum())})",
                   "latent_read_bytes_per_step": nb["latent"]},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(B / (ms * 1e-3), 1),
        "attention": {"ms": round(attn_ms, 5), "bytes": nb["algorithmic"], "GBps": round(achieved, 2),
                      "bytes_with_workspace": nb["call"],
                      "GBps_with_workspace": round(nb["call"] / (attn_ms * 1e-3) / 1e9, 2),
                      "note": "the whole call (absorb + split + merge), K calls back to back on HIP events"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profiles("mla_decode", w["name"])},
    }
    if not args.no_cpu_baseline:
        import oracle
        res["cpu_baseline"] = cpu_baseline_mla(torch, w, oracle, cache, q_nope, q_rope, w_uk, w_uv)
    print(json.dumps(res))


def cpu_baseline_mla(torch, w, oracle, cache, q_nope, q_rope, w_uk, w_uv):
    """The oracle (K and V written out from the latent, fp64) on four of the
    batch's sequences; latent-read bytes of those sequences / time."""
    h16 = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
    ch, qn, qr, wk, wv = h16(cache), h16(q_nope), h16(q_rope), h16(w_uk), h16(w_uv)
    pick = np.arange(4)
    ctx = w["context_lens"][pick]
    n, dt = repeat_for(lambda: oracle.mla_decode(qn[pick], qr[pick], wk, wv, ch, w["block_tables"][pick], ctx,
                                                 w["softmax_scale"]))
    row = w["kv_lora_rank"] + w["rope_dim"]
    nbytes = int(ctx.astype(np.int64).sum()) * row * 2
    return {"value": round(n * nbytes / dt / 1e9, 5), "unit": "GB/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"sequences 0..3 of the batch ({int(ctx.sum())} cached tokens): fp64 MLA decode with "
                      f"K/V up-projected per position, {n} runs in {dt:.1f} s, latent-read bytes / time"}


def run_decode_tp2(args, torch, pkv, workloads):
    """The batch-64 decode step at one GPU's share under 2-way tensor parallelism:
    4 KV heads and their 8 q heads per GPU, same contexts and block tables."""
    import dataclasses
    w = workloads.qwen3_decode_b64(num_q_heads=8, num_kv_heads=4)
    w = dataclasses.replace(w, name="qwen3_0.6b_decode_b64_bf16_tp2_shard")
    return run_decode(args, torch, pkv, workloads, w,
                      "paged decode attn KV-read GB/s & % HBM peak; cache-write GB/s (1 MI355X)")


def run_decode_bs8(args, torch, pkv, workloads):
    """The batch-64 decode step with 8-position cache blocks (same contexts,
    twice the blocks): a block size that is not a multiple of 16 runs the
    vector-ALU split kernel instead of the matrix-core persistent one."""
    import dataclasses
    w = workloads.qwen3_decode_b64(block_size=8, num_blocks=65536, width=512)
    w = dataclasses.replace(w, name="qwen3_0.6b_decode_b64_bf16_bs8")
    return run_decode(args, torch, pkv, workloads, w,
                      "paged decode attn KV-read GB/s & % HBM peak; cache-write GB/s (1 MI355X)")


def run_decode_fp8(args, torch, pkv, workloads):
    w = workloads.mixed_decode_fp8()
    return run_decode(args, torch, pkv, workloads, w,
                      "paged decode attn KV-read GB/s & % HBM peak; cache-write GB/s (1 MI355X)")


def generic(args, torch, pkv, step, nbytes, kernel, name, dtype, units, unit_name, rotating=None):
    """K back-to-back steps (warm). Cold: with `rotating(i)` (call i on one of
    several buffer sets that together exceed the Infinity Cache), K such calls back
    to back; otherwise each call timed alone after a 512 MiB copy."""
    stream = torch.cuda.current_stream()
    if args.profile_steps:
        copy_calibration(torch, pkv)
        for i in range(args.warmup + args.profile_steps):
            rotating(i) if rotating is not None else step()  # the launches the roofline times
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps, "workload": name}))
        return
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    gbps = nbytes / (ms * 1e-3) / 1e9
    # cold: the 256 MB Infinity Cache flushed before every call (a working set
    # below its size is otherwise partly served from it); the roofline uses this
    tc = Timer(torch, stream)
    if rotating is not None:
        for i in range(8):
            rotating(i)
        tc.start()
        for i in range(args.steps):
            rotating(i)
        tc.stop()
        torch.cuda.synchronize()
        cold_ms = tc.mean_ms() / args.steps
    else:
        flush_src = torch.empty(MALL_FLUSH_BYTES // 2, dtype=torch.uint8, device="cuda")
        flush_dst = torch.empty_like(flush_src)
        for _ in range(max(3, args.steps // 5)):
            pkv.hbm_copy(flush_dst, flush_src)
            tc.start()
            step()
            tc.stop()
        torch.cuda.synchronize()
        del flush_src, flush_dst
        cold_ms = tc.mean_ms()
    cold = nbytes / (cold_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "paged decode attn KV-read GB/s & % HBM peak; cache-write GB/s (1 MI355X)",
        "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": name, "bytes_per_step": nbytes},
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        unit_name: round(units / (ms * 1e-3), 1),
        "cold": {"ms": round(cold_ms, 5), "GBps": round(cold, 2)},
        "roofline": {"bound": "hbm", "achieved": round(cold, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(cold / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profiles(kernel, name)},
    }))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the paged "
              "KV cache kernels shard by sequence or KV head with no exchange between GPUs, so "
              "one GPU's share at its real shape is the measured unit)", file=sys.stderr)
        sys.exit(2)
    import torch

    import paged_kv_cache_304_amd as pkv
    import workloads
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    metric = "paged decode attn KV-read GB/s & % HBM peak; cache-write GB/s (1 MI355X)"
    if args.workload == "decode_b64":
        run_decode(args, torch, pkv, workloads, workloads.qwen3_decode_b64(), metric)
    elif args.workload == "decode_b64_tp2":
        run_decode_tp2(args, torch, pkv, workloads)
    elif args.workload == "decode_b64_bs8":
        run_decode_bs8(args, torch, pkv, workloads)
    elif args.workload == "decode_fp8_b256":
        run_decode_fp8(args, torch, pkv, workloads)
    elif args.workload == "prefill_fp8":
        run_prefill_fp8(args, torch, pkv, workloads)
    elif args.workload == "prefill_chunks":
        run_prefill_chunks(args, torch, pkv, workloads)
    elif args.workload == "prefill_chunks_fp8":
        run_prefill_chunks(args, torch, pkv, workloads, fp8=True)
    elif args.workload == "mla_fused":
        run_mla_fused(args, torch, pkv, workloads)
    elif args.workload == "engine_decode_b64":
        run_engine_decode(args, torch, pkv, workloads)
    elif args.workload == "mla_decode_b64":
        run_mla_decode(args, torch, pkv, workloads)
    else:
        run_mla(args, torch, pkv, workloads)


if __name__ == "__main__":
    main()
