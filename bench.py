#!/usr/bin/env python3
"""Benchmark of the MXFP4 paged-cache store on one MI355X.

A step is one MXFP4 store of the whole batch: 4,500,000 tokens x 512 bf16
(uniform in [-4, 4]) into a random permutation of the slots of a flat
1.224 GB cache; inputs are resident in HBM before timing.  For this dense
scattered batch the library advises its slot-order form, so a step is
mxfp4_build_inverse + mxfp4_store_by_slot; the scatter form (mxfp4_store) is
timed beside it.  The roofline entry is for the dominant kernel (the
slot-order store): HIP events around its launch in every timed step give
its average duration there.  The companions (gather-dequant, ring save,
CR1 norm, the read-side attention in one pass and in the split-key decode
form, the three RoPE+quant inserts) are timed after it, each on its own
workload, and reported under "companions".

Output: one JSON line (see the fields below).  `--sweep` prints further
lines for the token-count / slot-pattern sweep with the Infinity Cache
flushed between repetitions, then the pad-heavy batches.  Other modes (no
headline line): `--probes` (memory-system probes next to the store),
`--pads` (pad-heavy batches), `--counters [--counter-set ...]` (launches
only, for rocprofv3 --pmc).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
BYTES_PER_TOKEN = 1024 + 272 + 8  # latent read + row written + slot read
BYTES_PER_PAD = 8
# The slot-order store reads one int32 inverse entry per slot instead of the
# 8-byte slot of each token.
BY_SLOT_BYTES_PER_TOKEN = 1024 + 272
BY_SLOT_BYTES_PER_SLOT = 4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mxfp4_store_large_traffic.txt")
# tokens of the compress-ratio-1 norm's benchmark batch (2M fp32 rows of 512)
NORM_TOKENS = 1 << 21
# the store kernel's source and the headers it includes
STORE_SRCS = tuple(os.path.join(ROOT, "mxfp4_paged_cache_store_amd", "csrc", f)
                   for f in ("mxfp4_store.hip", "device_common.hpp", "kernels.hpp"))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--tokens", type=int, default=4_500_000)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-companions", action="store_true")
    p.add_argument("--sweep", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=4_500_000)
    p.add_argument("--scatter", action="store_true", help="time the scatter form as the step")
    p.add_argument("--counters", action="store_true",
                   help="for rocprofv3 --pmc: a 1 GiB copy (calibration) then 3 launches of each "
                        "kernel of --counter-set, no JSON")
    p.add_argument("--counter-set", choices=("store", "companions", "probes", "pads", "lds"), default="store",
                   help="what --counters runs: the store step, the companions, the probes, the "
                        "pad-heavy batches, or the LDS access patterns")
    p.add_argument("--only", default="",
                   help="comma-separated companion names to run (default: all)")
    p.add_argument("--probes", action="store_true",
                   help="time the memory-system probes of libmxprobe.so (one JSON line each)")
    p.add_argument("--pads", action="store_true",
                   help="time the scatter store on pad-heavy batches (one JSON line each)")
    return p.parse_args()


def source_digest(paths) -> str:
    """Digest of kernel sources' code (in the order given): comments and blank
    space removed, so that counters taken on a kernel stay attached to it
    across comment-only edits."""
    import re

    text = "\n".join(open(p, encoding="utf-8").read() for p in paths)
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    code = " ".join(text.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def measured_traffic(tokens: int, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source and this token
    count."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != source_digest(STORE_SRCS):
        return None
    if int(kv.get("tokens", -1)) != tokens or kv.get("kernel") != kernel:
        return None
    return int(float(kv["hbm_bytes_per_launch"]))


def time_launches(fn, steps: int, warmup: int, torch):
    """Wall time and HIP-event time of `steps` back-to-back launches on the
    current stream (the one every launch here uses)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        fn()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, ev0.elapsed_time(ev1) / 1000.0


def time_graph(fn, per_graph: int, replays: int, torch) -> float:
    """Seconds per launch of `fn` captured `per_graph` times into one HIP
    graph and replayed `replays` times (HIP events around the replays): the
    device's back-to-back rate without the host's per-call submission cost,
    which bounds eager launches of latency-bound kernels."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(replays):
        graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    del graph
    return ev0.elapsed_time(ev1) / 1000.0 / (replays * per_graph)


GRAPH_LAUNCHES = 50  # launches per captured graph for the latency-bound companions
GRAPH_REPLAYS = 10


def cpu_threads() -> tuple[int, int]:
    """(threads for the all-cores leg, logical CPUs the OS reports).  The
    all-cores leg uses the CPUs this process may run on, at most 16 (one
    GPU's share of a shared host)."""
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return max(1, min(16, usable)), os.cpu_count() or 1


def cpu_baseline(sample: int):
    """The oracle's store (plain C, scalar) on the host: all cores over
    contiguous token ranges on `sample` tokens, and one thread on
    sample / threads tokens (about the same wall time).  Data generation is
    outside the timed calls."""
    import numpy as np

    import oracle
    import workloads

    threads, nproc = cpu_threads()
    src, slots = workloads.large_sample_host(sample)
    cache = np.full(sample * 272, 0xA5, dtype=np.uint8)
    t0 = time.perf_counter()
    oracle.mxfp4_store(src, slots, cache, 1, sample, sample, threads=threads)
    dt = time.perf_counter() - t0
    one = max(1, sample // threads)
    src1 = np.ascontiguousarray(src[:one])
    slots1 = np.empty(one, dtype=np.int64)
    slots1[np.argsort(slots[:one], kind="stable")] = np.arange(one, dtype=np.int64)
    cache1 = np.full(one * 272, 0xA5, dtype=np.uint8)
    t0 = time.perf_counter()
    oracle.mxfp4_store(src1, slots1, cache1, 1, one, one, threads=1)
    dt1 = time.perf_counter() - t0
    return {
        "value": round(sample / dt, 1),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{sample} tokens x 512 bf16 uniform in [-4, 4], random-permutation slots "
                  f"into a flat cache (same distribution as the timed batch), "
                  f"{threads} threads over contiguous token ranges, {dt:.2f} s wall "
                  f"({threads * dt:.0f} thread-seconds); nproc {nproc}",
        "GBps": round(sample * BYTES_PER_TOKEN / dt / 1e9, 2),
        "nproc": nproc,
        "single_thread": {"value": round(one / dt1, 1), "unit": "tokens/s",
                          "GBps": round(one * BYTES_PER_TOKEN / dt1 / 1e9, 3),
                          "sample": f"first {one} tokens, their slots ranked into a {one}-slot "
                                    f"cache, {dt1:.2f} s"},
    }


def small_stores(torch, ops, workloads, steps, warmup):
    """The store on the decode-shaped batch (256 tokens into a paged cache
    with other layers' rows interleaved) and on the prefill chunk (16,384
    tokens in 32 request runs, then gather-dequant of the stored slots):
    both are latency-bound, so they are reported in microseconds per launch:
    HIP events over back-to-back eager launches (the host's per-call cost
    included) and over replays of a HIP graph of the same launches."""
    out = {}
    reps = max(20, steps)
    for name, case in (("mxfp4_store_decode", workloads.decode_case()),
                       ("mxfp4_store_prefill", workloads.prefill_case())):
        src = torch.from_numpy(case.src.view("int16")).cuda().view(torch.bfloat16)
        slots = torch.from_numpy(case.slots).cuda()
        cache = torch.from_numpy(case.fresh_cache()).cuda()
        nb, bs, bsr = case.num_blocks, case.block_size, case.block_stride_rows
        store = lambda: ops.mxfp4_store(src, slots, cache, nb, bs, bsr)  # noqa: E731
        _, ev = time_launches(store, reps, warmup, torch)
        per = ev / reps
        per_graph = time_graph(store, GRAPH_LAUNCHES, GRAPH_REPLAYS, torch)
        valid = int((case.slots >= 0).sum())
        entry = {
            "workload": f"{case.src.shape[0]} tokens ({valid} valid) into {nb} blocks x {bs} slots, "
                        f"block stride {bsr} rows",
            "us_per_launch": round(per * 1e6, 2),
            "tokens_per_s": round(valid / per, 1),
            "graph_us_per_launch": round(per_graph * 1e6, 2),
            "graph_tokens_per_s": round(valid / per_graph, 1),
        }
        if case.gather_slots is not None:
            gs = torch.from_numpy(case.gather_slots).cuda()
            dq = torch.empty((gs.numel(), 512), dtype=torch.bfloat16, device="cuda")
            gather = lambda: ops.mxfp4_gather_dequant(cache, nb, bs, bsr, 512, gs, dq)  # noqa: E731
            _, ev = time_launches(gather, reps, warmup, torch)
            entry["gather_dequant_us_per_launch"] = round(ev / reps * 1e6, 2)
            entry["gather_dequant_graph_us_per_launch"] = round(
                time_graph(gather, GRAPH_LAUNCHES, GRAPH_REPLAYS, torch) * 1e6, 2)
        out[name] = entry
    return out


COMPANIONS = ("mxfp4_gather_dequant", "save_ring_rows", "fused_save_compress_norm_cr1",
              "rope_store", "rope_store_large", "sparse_mla_attention",
              "sparse_mla_attention_decode", "small_stores")


def companions(torch, ops, workloads, steps, warmup, cache, n_tokens, only=(), counters=False):
    """Each companion on its own workload.  `only`: names from COMPANIONS to
    run (all when empty).  With `counters`, each kernel is launched three
    times and nothing is timed (for rocprofv3 --pmc)."""
    out = {}
    want = lambda name: not only or name in only  # noqa: E731

    def timed(fn, reps):
        if counters:
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            return None
        _, ev = time_launches(fn, reps, warmup, torch)
        return ev / reps

    if want("mxfp4_gather_dequant"):
        # gather-dequant of every slot of the large cache back to bf16
        slots = torch.arange(n_tokens, dtype=torch.int64, device="cuda")
        dq = torch.empty((n_tokens, 512), dtype=torch.bfloat16, device="cuda")
        per = timed(lambda: ops.mxfp4_gather_dequant(cache, 1, n_tokens, n_tokens, 512, slots, dq),
                    max(3, steps // 3))
        if per is not None:
            out["mxfp4_gather_dequant"] = {
                "workload": f"{n_tokens} slots of the flat cache -> bf16 [{n_tokens}, 512]",
                "us_per_launch": round(per * 1e6, 2),
                "slots_per_s": round(n_tokens / per, 1),
                "GBps": round(n_tokens * 1304 / per / 1e9, 1),
                "frac_hbm_peak": round(n_tokens * 1304 / per / 1e9 / HBM_PEAK_GBS, 4),
            }
        del dq, slots
    if want("save_ring_rows"):
        # ring-state save: 262,144 fp32 [kv, score] rows (1024 wide) to
        # scattered slots of an 8192-block x 32-row ring
        rows, ring_slots, ring_shape = workloads.ring_large_device()
        n_rows = rows.shape[0]
        ring = torch.zeros(ring_shape, dtype=torch.float32, device="cuda")
        per = timed(lambda: ops.save_ring_rows(rows, ring_slots, ring), steps)
        if per is not None:
            out["save_ring_rows"] = {
                "workload": f"{n_rows} fp32 rows x 1024 -> scattered slots of an 8192 x 32 ring",
                "us_per_launch": round(per * 1e6, 2),
                "GBps": round(n_rows * (4096 + 4096 + 8) / per / 1e9, 1),
                "frac_hbm_peak": round(n_rows * (4096 + 4096 + 8) / per / 1e9 / HBM_PEAK_GBS, 4),
            }
        del rows, ring, ring_slots
    if want("fused_save_compress_norm_cr1"):
        # compress-ratio-1 RMSNorm: 2,097,152 fp32 [512] rows -> bf16, all valid
        n_norm = NORM_TOKENS
        kv = torch.empty((n_norm, 512), dtype=torch.float32, device="cuda").normal_()
        norm_slots = torch.arange(n_norm, dtype=torch.int64, device="cuda")
        w = torch.empty(512, dtype=torch.float32, device="cuda").normal_(0.8, 0.5).to(torch.bfloat16)
        latent_out = torch.empty((n_norm, 512), dtype=torch.bfloat16, device="cuda")
        per = timed(lambda: ops.fused_save_compress_norm_cr1(kv, norm_slots, w, 1e-6, latent_out), steps)
        if per is not None:
            out["fused_save_compress_norm_cr1"] = {
                "workload": f"{n_norm} fp32 rows x 512 -> bf16 RMSNorm, all tokens valid",
                "us_per_launch": round(per * 1e6, 2),
                "tokens_per_s": round(n_norm / per, 1),
                "GBps": round(n_norm * (2048 + 1024 + 8) / per / 1e9, 1),
                "frac_hbm_peak": round(n_norm * (2048 + 1024 + 8) / per / 1e9 / HBM_PEAK_GBS, 4),
            }
        del kv, norm_slots, w, latent_out
    if want("rope_store"):
        # RoPE inserts on the 16384-token, compress-ratio-4 workload
        case = workloads.rope_case()
        lat = torch.from_numpy(case.latent.view("int16")).cuda().view(torch.bfloat16)
        pos = torch.from_numpy(case.positions).cuda()
        cs = torch.from_numpy(case.cos_sin).cuda()
        sl = torch.from_numpy(case.slots).cuda()
        written = int(((case.positions + 1) % case.compress_ratio == 0).sum())
        for name, fn, width in (("mxfp8_rope_store", ops.mxfp8_rope_store, 528),
                                ("nvfp4_rope_store", ops.nvfp4_rope_store, 288),
                                ("v4_rope_store", ops.v4_rope_store, 584)):
            kv = torch.zeros((case.num_blocks, case.block, width), dtype=torch.uint8, device="cuda")
            insert = lambda: fn(lat, pos, cs, kv, sl, case.compress_ratio)  # noqa: E731
            per = timed(insert, steps)
            if per is not None:
                per_graph = time_graph(insert, GRAPH_LAUNCHES, GRAPH_REPLAYS, torch)
                nbytes = written * (1024 + 256 + 16 + width) + (case.latent.shape[0] - written) * 16
                out[name] = {
                    "workload": f"{case.latent.shape[0]} tokens, CR {case.compress_ratio} ({written} "
                                f"written), {width}-byte records",
                    "us_per_launch": round(per * 1e6, 2),
                    "GBps": round(nbytes / per / 1e9, 1),
                    "graph_us_per_launch": round(per_graph * 1e6, 2),
                }
        del lat, pos, sl, kv
    if want("rope_store_large"):
        # the same inserts at bandwidth scale: 1,048,576 tokens, compress
        # ratio 1 (every token written), random positions and a permutation
        # of the slots
        lat, pos, cs, sl = workloads.rope_large_device()
        n_big = lat.shape[0]
        for name, fn, width in (("mxfp8_rope_store", ops.mxfp8_rope_store, 528),
                                ("nvfp4_rope_store", ops.nvfp4_rope_store, 288),
                                ("v4_rope_store", ops.v4_rope_store, 584)):
            kv = torch.zeros((n_big // 64, 64, width), dtype=torch.uint8, device="cuda")
            per = timed(lambda: fn(lat, pos, cs, kv, sl, 1), max(10, steps))
            if per is not None:
                nbytes = n_big * (1024 + 256 + 16 + width)
                out[name + "_large"] = {
                    "workload": f"{n_big} tokens, CR 1 (all written), {width}-byte records, "
                                f"scattered slots",
                    "us_per_launch": round(per * 1e6, 2),
                    "GBps": round(nbytes / per / 1e9, 1),
                    "frac_hbm_peak": round(nbytes / per / 1e9 / HBM_PEAK_GBS, 4),
                }
            del kv
        del lat, pos, cs, sl
    if want("sparse_mla_attention"):
        # sparse MLA attention over the packed cache (after the HBM-bound
        # companions: its matrix-core load can lower the clock for the
        # launches that follow): the last 4,096 queries of a 16,384-token
        # prefill, 32 heads, top-2048 causal slots
        q, acache, aidx, ascale = workloads.attention_workload_device()
        aout = torch.empty_like(q)
        attn = lambda: ops.sparse_mla_attention(q, acache, aidx, ascale, out=aout, splits=1)  # noqa: E731
        if counters:
            per = timed(attn, 3)
        else:
            # After the HBM-bound companions its first 30-40 launches run up
            # to 20% slower while the clock comes up; the steady state is
            # timed after ATTN_WARMUP untimed launches.
            _, ev = time_launches(attn, ATTN_REPS, ATTN_WARMUP, torch)
            per = ev / ATTN_REPS
        if per is not None:
            valid = int((aidx >= 0).sum())
            flops = 4.0 * q.shape[1] * 512 * valid
            out["sparse_mla_attention"] = {
                "workload": f"{q.shape[0]} queries x {q.shape[1]} heads, top-{aidx.shape[1]} of a "
                            f"{acache.shape[0]}-token MXFP4 cache ({valid} valid slot reads)",
                "us_per_launch": round(per * 1e6, 2),
                "TFLOPs": round(flops / per / 1e12, 1),
                "frac_bf16_mfma_peak": round(flops / per / 1e12 / BF16_PEAK_TFLOPS, 4),
            }
        del q, acache, aidx, aout
    if want("sparse_mla_attention_decode"):
        # decode: the last 64 queries of the same context, in the advised
        # split form
        q, acache, aidx, ascale = workloads.attention_workload_device(tokens=64)
        aout = torch.empty_like(q)
        splits = ops.sparse_mla_attention_splits_advised(64, q.shape[1], aidx.shape[1])
        ws = torch.empty(max(256, ops.sparse_mla_attention_workspace_bytes(64, q.shape[1], splits)),
                         dtype=torch.uint8, device="cuda")
        decode = lambda: ops.sparse_mla_attention(q, acache, aidx, ascale, out=aout,  # noqa: E731
                                                  splits=splits, workspace=ws)
        per = timed(decode, max(10, steps))
        if per is not None:
            per_graph = time_graph(decode, GRAPH_LAUNCHES, GRAPH_REPLAYS, torch)
            valid = int((aidx >= 0).sum())
            flops = 4.0 * q.shape[1] * 512 * valid
            out["sparse_mla_attention_decode"] = {
                "workload": f"{q.shape[0]} decode queries x {q.shape[1]} heads, top-{aidx.shape[1]} "
                            f"of a {acache.shape[0]}-token MXFP4 cache, {splits} key ranges + merge",
                "us_per_call": round(per * 1e6, 2),
                "TFLOPs": round(flops / per / 1e12, 1),
                "graph_us_per_call": round(per_graph * 1e6, 2),
            }
        del q, acache, aidx, aout, ws
    return out


PROBE_REPS = 20
PAD_TOKENS = (16384, 262144)
PAD_FRACTIONS = (0.0, 0.5, 0.9)


def run_pads(torch, ops, counters: bool = False) -> None:
    """The scatter store on batches where a share of the slots are pads (-1,
    at random positions, as in a batch padded to a captured size): 16,384 and
    262,144 tokens x 512 into a flat cache with four slots per token, valid
    tokens on distinct random slots.  Bytes per launch count 1304 per valid
    token and 8 per pad.  Median of PROBE_REPS HIP-event times of single
    launches after a 1 GiB read (flushed) and back to back (warm); with
    `counters`, three launches of each case, untimed."""
    import statistics

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    for n in PAD_TOKENS:
        src = torch.empty((n, 512), dtype=torch.bfloat16, device="cuda").uniform_(-4, 4, generator=g)
        num_slots = 4 * n
        cache = torch.zeros(num_slots * 272, dtype=torch.uint8, device="cuda")
        for frac in PAD_FRACTIONS:
            slots = torch.randperm(num_slots, generator=g, device="cuda")[:n].contiguous()
            pad = torch.rand(n, generator=g, device="cuda") < frac
            slots[pad] = -1
            valid = int((slots >= 0).sum())
            fn = lambda: ops.mxfp4_store(src, slots, cache, 1, num_slots, num_slots)  # noqa: E731
            if counters:
                for _ in range(3):
                    fn()
                torch.cuda.synchronize()
                continue
            nbytes = valid * BYTES_PER_TOKEN + (n - valid) * BYTES_PER_PAD
            for state in ("flushed", "warm"):
                times = []
                for _ in range(PROBE_REPS + 2):
                    if state == "flushed":
                        flush.sum()
                    torch.cuda.synchronize()
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    fn()
                    e1.record()
                    torch.cuda.synchronize()
                    times.append(e0.elapsed_time(e1) / 1000.0)
                t = statistics.median(times[2:])
                print(json.dumps({"pads": "mxfp4_store", "tokens": n, "valid": valid,
                                  "pad_fraction": frac, "cache": state, "reps": PROBE_REPS,
                                  "us": round(t * 1e6, 2), "bytes": nbytes,
                                  "GBps": round(nbytes / t / 1e9, 1)}), flush=True)
            del slots, pad
        del src, cache
    del flush


def run_probes(torch, workloads, n: int, counters: bool = False) -> None:
    """The memory-system probes of libmxprobe.so next to the store on the
    same buffers (4.5M tokens: 4.608 GB of latent, a 1.224 GB cache, a random
    permutation): read-only, write-only, the store's traffic as a plain copy
    (1 KiB read + 272-byte row written per token) in sequential and in
    slot order (gathered through the inverse map), and the store's slot-order
    kernel and whole step; the inverse map's traffic (a sequential write of
    its size, scattered 4-byte writes) beside its build; a copy of 262,144 rows of 4 KiB in order and to a
    permutation of the rows, beside save_ring_rows on the same shapes; the
    gather-dequant's traffic (272-byte rows to 1 KiB rows, in order) and the
    CR1 norm's (2 KiB rows to 1 KiB rows) as plain copies beside those
    kernels; then the small-batch floors (an empty launch of
    the store's grid, a plain read of the batch's latent, a copy with the
    store's traffic) beside the store with in-order slots at 16,384 and
    65,536 tokens; last, the LDS and matrix-core rates of a CU (contiguous
    LDS reads, transposing reads and writes; bf16 MFMAs alone).  One JSON
    line per probe: median of PROBE_REPS HIP-event times of single launches,
    each after a 1 GiB read that flushes the Infinity Cache (the LDS and MFMA
    probes: median of 5, no flush).  With `counters`, three launches of each
    HBM probe, untimed."""
    import ctypes
    import statistics

    from mxfp4_paged_cache_store_amd import build, ops

    if not os.path.exists(build.PROBE_LIB_PATH):
        build.build_probes()
    lib = ctypes.CDLL(build.PROBE_LIB_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.probe_read.argtypes = [vp, i64, vp, vp]
    lib.probe_write.argtypes = [vp, i64, ctypes.c_int, vp]
    lib.probe_copy_rows.argtypes = [vp, i64, vp, vp, ctypes.c_int, vp]
    lib.probe_empty.argtypes = [i64, vp]
    lib.probe_copy_wide.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.probe_copy_expand.argtypes = [vp, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp]
    lib.probe_scatter_dwords.argtypes = [vp, i64, ctypes.c_int, vp, vp]
    lib.probe_lds.argtypes = [ctypes.c_int, i64, ctypes.c_int, vp, vp]
    for f in (lib.probe_read, lib.probe_write, lib.probe_copy_rows, lib.probe_empty, lib.probe_copy_wide,
              lib.probe_copy_expand, lib.probe_scatter_dwords, lib.probe_lds):
        f.restype = ctypes.c_int

    def ok(rc):
        if rc != 0:
            raise RuntimeError(f"probe launch failed ({rc})")

    st = lambda: int(torch.cuda.current_stream().cuda_stream)  # noqa: E731
    src, slots = workloads.large_case_device(n)
    cache = torch.zeros(n * 272, dtype=torch.uint8, device="cuda")
    inv = ops.mxfp4_inverse_workspace(1, n)
    ops.mxfp4_build_inverse(slots, 1, n, inv)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    read_bytes = (n * 1024) // 16384 * 16384
    write_bytes = (n * 272) // 16384 * 16384
    rows = n // 16 * 16

    def store_kernel():
        ops.mxfp4_store_by_slot(src, n, inv, cache, 1, n, n)

    def store_step():
        ops.mxfp4_build_inverse(slots, 1, n, inv)
        store_kernel()

    cases = [
        ("read_only", read_bytes, lambda: ok(lib.probe_read(src.data_ptr(), read_bytes, sink.data_ptr(), st()))),
    ]
    # each write probe with plain stores and written through (NT + SC1), as
    # the slot-order store writes
    for through, tag in ((0, ""), (1, "_through")):
        cases += [
            ("write_only" + tag, write_bytes,
             lambda w=through: ok(lib.probe_write(cache.data_ptr(), write_bytes, w, st()))),
            ("copy_rows_sequential" + tag, rows * 1296,
             lambda w=through: ok(lib.probe_copy_rows(src.data_ptr(), rows, None, cache.data_ptr(), w, st()))),
            ("copy_rows_slot_order" + tag, rows * 1300,
             lambda w=through: ok(lib.probe_copy_rows(src.data_ptr(), rows, inv.data_ptr(), cache.data_ptr(), w,
                                                      st()))),
        ]
    cases += [
        ("store_by_slot_kernel", n * 1300, store_kernel),
        ("store_slot_order_step", n * BYTES_PER_TOKEN, store_step),
    ]
    # the inverse map's traffic: a sequential write of its size (the fill) and
    # n scattered 4-byte writes to the positions the permutation names (an
    # 8-byte index read + 4 bytes written each), 1-8 per thread, next to the
    # library's build of the same map (fill + inversion)
    scat = torch.empty(n, dtype=torch.int32, device="cuda")
    map_bytes = (n * 4) // 16384 * 16384
    cases.append(("write_map_sequential", map_bytes,
                  lambda: ok(lib.probe_write(scat.data_ptr(), map_bytes, 0, st()))))
    for per in (1, 2, 4, 8):
        cases.append((f"scatter_dwords_{per}_per_thread", n * 12,
                      lambda p=per: ok(lib.probe_scatter_dwords(slots.data_ptr(), n, p, scat.data_ptr(), st()))))
    cases.append(("inverse_map_build", n * 16, lambda: ops.mxfp4_build_inverse(slots, 1, n, inv)))
    # the ring-state save's traffic: 262,144 rows of 4 KiB, in order or to a
    # permutation of the rows, next to save_ring_rows on the same shapes
    ring_rows, ring_slots, ring_shape = workloads.ring_large_device()
    n_ring = ring_rows.shape[0]
    ring = torch.zeros(ring_shape, dtype=torch.float32, device="cuda")
    ring_dst = torch.empty_like(ring_rows)
    ring_perm = torch.randperm(n_ring, device="cuda")
    cases += [
        ("copy_wide_sequential", n_ring * 8192,
         lambda: ok(lib.probe_copy_wide(ring_rows.data_ptr(), n_ring, 4096, None, ring_dst.data_ptr(), st()))),
        ("copy_wide_scattered", n_ring * 8200,
         lambda: ok(lib.probe_copy_wide(ring_rows.data_ptr(), n_ring, 4096, ring_perm.data_ptr(),
                                        ring_dst.data_ptr(), st()))),
        ("save_ring_rows", n_ring * 8200, lambda: ops.save_ring_rows(ring_rows, ring_slots, ring)),
    ]
    # the gather-dequant's traffic (272-byte rows in order -> 1 KiB bf16 rows,
    # non-temporal stores) and the CR1 norm's (2 KiB fp32 rows -> 1 KiB bf16
    # rows, written through), each next to its kernel on the same shapes
    dq_out = torch.empty((n, 512), dtype=torch.bfloat16, device="cuda")
    dq_slots = torch.arange(n, dtype=torch.int64, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9)
    kv = torch.randn((NORM_TOKENS, 512), generator=gen, dtype=torch.float32, device="cuda")
    kv_out = torch.empty((NORM_TOKENS, 512), dtype=torch.bfloat16, device="cuda")
    kv_slots = torch.arange(NORM_TOKENS, dtype=torch.int64, device="cuda")
    weight = torch.ones(512, dtype=torch.bfloat16, device="cuda")
    # (the copies with 1, 2, 4 and 8 rows per wave: the fastest is the ceiling)
    for rpw in (1, 2, 4, 8):
        cases.append((f"copy_272_to_1024_nt_{rpw}_rows_per_wave", n * 1296,
                      lambda r=rpw: ok(lib.probe_copy_expand(cache.data_ptr(), n, 272, 1024, 2, r,
                                                             dq_out.data_ptr(), st()))))
    cases.append(("gather_dequant_in_order", n * 1304,
                  lambda: ops.mxfp4_gather_dequant(cache, 1, n, n, 512, dq_slots, dq_out)))
    for rpw in (1, 2, 4, 8):
        cases.append((f"copy_2048_to_1024_through_{rpw}_rows_per_wave", NORM_TOKENS * 3072,
                      lambda r=rpw: ok(lib.probe_copy_expand(kv.data_ptr(), NORM_TOKENS, 2048, 1024, 18, r,
                                                             kv_out.data_ptr(), st()))))
    cases.append(("compress_norm_cr1", NORM_TOKENS * 3080,
                  lambda: ops.fused_save_compress_norm_cr1(kv, kv_slots, weight, 1e-6, kv_out)))
    seq_slots = torch.arange(65536, dtype=torch.int64, device="cuda")
    for tokens in (16384, 65536):
        tpw = 2 if tokens <= 16384 else 4
        grid = tokens // (4 * tpw)  # the scatter store's workgroups at this size
        nbytes = tokens * 1024
        cases.append((f"empty_launch_{tokens}", 0, lambda g=grid: ok(lib.probe_empty(g, st()))))
        cases.append((f"read_latent_{tokens}", nbytes,
                      lambda b=nbytes: ok(lib.probe_read(src.data_ptr(), b, sink.data_ptr(), st()))))
        # the store's own traffic and write form at this size (1 KiB read,
        # 272-byte row written per token, in order) beside the scatter store
        # on the same batch with slot t = t
        cases.append((f"copy_rows_sequential_{tokens}", tokens * 1296,
                      lambda k=tokens: ok(lib.probe_copy_rows(src.data_ptr(), k, None, cache.data_ptr(), 0,
                                                              st()))))
        cases.append((f"store_in_order_{tokens}", tokens * BYTES_PER_TOKEN,
                      lambda k=tokens: ops.mxfp4_store(src[:k], seq_slots[:k], cache, 1, n, n)))
    for name, nbytes, fn in cases:
        if counters:
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            continue
        fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(PROBE_REPS):
            flush.sum()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / 1000.0)
        t = statistics.median(times)
        line = {"probe": name, "bytes": nbytes, "reps": PROBE_REPS, "cache": "flushed",
                "us": round(t * 1e6, 2)}
        if nbytes:
            line["GBps"] = round(nbytes / t / 1e9, 1)
            line["frac_hbm_peak"] = round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)
        print(json.dumps(line), flush=True)
    del src, slots, cache, inv, flush, ring_rows, ring_slots, ring, ring_dst, ring_perm
    del dq_out, dq_slots, kv, kv_out, kv_slots, scat, seq_slots
    # LDS and matrix-core rates of a CU (no HBM traffic): 1,024 workgroups of
    # 1,024 threads (one per CU at a time), LDS_ITERS x 8 accesses per wave
    # (or x 16 MFMAs); median of 5 launches
    lds_out = torch.empty(1024 * 1024, dtype=torch.int32, device="cuda")
    waves = 1024 * 16
    for kind, name, per_instr in ((0, "lds_read_b128", 1024), (1, "lds_read_b64_tr_b16", 512),
                                  (2, "lds_write_b128", 1024), (3, "lds_write_b64", 512),
                                  (4, "mfma_bf16_16x16x32", 0)):
        fn = lambda k=kind: ok(lib.probe_lds(k, 1024, LDS_ITERS, lds_out.data_ptr(), st()))  # noqa: E731
        fn()
        torch.cuda.synchronize()
        if counters:
            continue
        times = []
        for _ in range(5):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / 1000.0)
        t = statistics.median(times)
        line = {"probe": name, "reps": 5, "us": round(t * 1e6, 2)}
        if per_instr:
            line["lds_GBps_per_CU"] = round(waves * LDS_ITERS * 8 * per_instr / t / 1e9 / 256, 1)
        else:
            flops = waves * LDS_ITERS * 16 * (16 * 16 * 32 * 2)
            line["TFLOPs"] = round(flops / t / 1e12, 1)
            line["frac_bf16_mfma_peak"] = round(flops / t / 1e12 / BF16_PEAK_TFLOPS, 4)
        print(json.dumps(line), flush=True)
    del lds_out


LDS_ITERS = 1024


def lds_patterns():
    """Lane -> 16-byte LDS unit maps of the attention kernel's accesses (32
    heads per workgroup), its earlier layouts, and plain strides.  Partial
    scores: 4 producers x 4 key tiles x 2 head tiles x 64 lanes of f32x4.
    Weights: bf16 rows 160 bytes apart, [head][key]."""
    def cur_slot(v, ht, q, li, kk):  # rows of 128 B per (producer, head tile, sub-block, head)
        return (((v * 2 + ht) * 2 + q) * 16 + li) * 8 + (kk ^ (li & 7))
    pats = {
        "contiguous": lambda l: l,
        "stride_32B": lambda l: 2 * l,
        "stride_64B": lambda l: 4 * l,
        "rows_160B_apart": lambda l: 10 * l,
        # current: writer lane (li, lq) of key tile 2, head tile 1; owner lane
        # 8hh + kk of producer 0 reading producer 1's partials
        "partial_write": lambda l: cur_slot(0, 1, (l >> 4) & 1, l & 15, 4 + ((l >> 4) >> 1)),
        "partial_read": lambda l: cur_slot(1, 0, 0, l >> 3, l & 7),
        # earlier: slot 16lq + (li ^ 4lq) per (producer, key tile, head
        # tile), owner lane hh + 8kk
        "partial_write_earlier": lambda l: ((0 * 4 + 2) * 2 + 1) * 64 + 16 * (l >> 4) + ((l & 15) ^ (4 * (l >> 4))),
        "partial_read_earlier": lambda l: (((l >> 3) >> 1) * 2) * 64 + 16 * (2 * ((l >> 3) & 1))
                                          + ((l & 7) ^ (4 * (2 * ((l >> 3) & 1)))),
        # the first layout tried with owner lane 8hh + kk: slot
        # 16lq + ((li + 4kt + lq) & 15)
        "partial_read_first_try": lambda l: (((l & 7) >> 1) * 2) * 64 + 16 * (2 * (l & 1))
                                            + (((l >> 3) + 4 * ((l & 7) >> 1) + 2 * (l & 1)) & 15),
        "weights_write": lambda l: ((l >> 3) * 160 + 16 * (l & 7)) // 16,
        "weights_write_earlier": lambda l: ((l & 7) * 160 + 16 * (l >> 3)) // 16,
        "weights_read": lambda l: ((l & 15) * 160 + 16 * (l >> 4)) // 16,
    }
    return {k: [f(l) for l in range(64)] for k, f in pats.items()}


def run_lds_patterns(torch):
    """One read and one write launch per pattern of lds_patterns() (2,048
    one-wave workgroups, LDS_PATTERN_ITERS accesses per lane), for
    rocprofv3's SQ_LDS_BANK_CONFLICT; dispatch order = print order."""
    import ctypes
    from mxfp4_paged_cache_store_amd import build

    if not os.path.exists(build.PROBE_LIB_PATH):
        build.build_probes()
    lib = ctypes.CDLL(build.PROBE_LIB_PATH)
    lib.probe_lds_pattern.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_lds_pattern.restype = ctypes.c_int
    out = torch.empty(2048 * 64, dtype=torch.int32, device="cuda")
    st = int(torch.cuda.current_stream().cuda_stream)
    for name, units in lds_patterns().items():
        if min(units) < 0 or max(units) >= 4096:
            raise ValueError(f"pattern {name} leaves the 64 KB probe buffer")
        dev = torch.tensor(units, dtype=torch.int32, device="cuda")
        for write in (0, 1):
            if lib.probe_lds_pattern(dev.data_ptr(), write, 2048, LDS_PATTERN_ITERS, out.data_ptr(), st) != 0:
                raise RuntimeError("probe launch failed")
            torch.cuda.synchronize()
            print(json.dumps({"lds_pattern": name, "access": "write" if write else "read",
                              "workgroups": 2048, "iters": LDS_PATTERN_ITERS}), flush=True)


LDS_PATTERN_ITERS = 1000
ATTN_WARMUP = 40   # untimed launches of the attention companion before its timed ones
ATTN_REPS = 20

SWEEP_TOKENS = (16384, 65536, 262144, 1048576, 4500000)
SWEEP_REPS = 20


def run_sweep(torch, ops, workloads):
    """Store throughput vs token count and slot pattern, both forms.  Slot
    patterns: prefill-style runs (requests of U[448, 512) tokens, each in its
    own 512-slot chunk, chunks in random order) and a random permutation.
    Each case is timed SWEEP_REPS times with the Infinity Cache flushed
    before every repetition by reading a 1 GiB buffer (a write-flush would
    leave dirty lines to be written back during the timed kernel), then
    SWEEP_REPS times warm (back to back, labelled "warm"); medians of HIP
    event times around single launches, two untimed repetitions first.  The
    dispatches come in the order the lines are printed (flushed before
    warm), so a kernel trace of this run splits the same way."""
    import statistics

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    for n in SWEEP_TOKENS:
        for pattern in ("runs", "random"):
            src = torch.empty((n, 512), dtype=torch.bfloat16, device="cuda").uniform_(-4, 4)
            if pattern == "random":
                slots, num_slots = torch.randperm(n, device="cuda"), n
            else:
                host, num_slots = workloads.request_runs_slots(n)
                slots = torch.from_numpy(host).to("cuda")
            cache = torch.zeros(num_slots * 272, dtype=torch.uint8, device="cuda")
            inv = ops.mxfp4_inverse_workspace(1, num_slots)
            forms = {"scatter": lambda: ops.mxfp4_store(src, slots, cache, 1, num_slots, num_slots)}
            if ops.mxfp4_slot_order_advised(n, 512, 1, num_slots):
                def slot_order():
                    ops.mxfp4_build_inverse(slots, 1, num_slots, inv)
                    ops.mxfp4_store_by_slot(src, n, inv, cache, 1, num_slots, num_slots)
                forms["slot_order"] = slot_order
            for form, fn in forms.items():
                for state in ("flushed", "warm"):
                    times = []
                    for _ in range(SWEEP_REPS + 2):
                        if state == "flushed":
                            flush.sum()
                        torch.cuda.synchronize()
                        e0 = torch.cuda.Event(enable_timing=True)
                        e1 = torch.cuda.Event(enable_timing=True)
                        e0.record()
                        fn()
                        e1.record()
                        torch.cuda.synchronize()
                        times.append(e0.elapsed_time(e1) / 1000.0)
                    t = statistics.median(times[2:])
                    gbs = n * BYTES_PER_TOKEN / t / 1e9
                    print(json.dumps({"sweep": "mxfp4_store", "form": form, "tokens": n, "slots": pattern,
                                      "cache": state, "reps": SWEEP_REPS, "us": round(t * 1e6, 2),
                                      "GBps": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}),
                          flush=True)
            del src, slots, cache, inv


LAYERS_SHARING_MAPPING = (1, 4, 16, 64)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the store has "
              "no cross-GPU step, so run it with --gpus 1 on each GPU's share", file=sys.stderr)
        sys.exit(2)

    only = tuple(x for x in args.only.split(",") if x)
    unknown = [x for x in only if x not in COMPANIONS]
    if unknown:
        print(f"unknown companion(s) {unknown}; known: {', '.join(COMPANIONS)}", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads
    from mxfp4_paged_cache_store_amd import build, ops

    if not os.path.exists(build.LIB_PATH):
        build.build()
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)

    n = args.tokens
    if args.counters:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)  # calibration: 1 GiB read + 1 GiB written
        torch.cuda.synchronize()
        del a, b
        if args.counter_set == "probes":
            run_probes(torch, workloads, n, counters=True)
            print("[bench] counters run done", file=sys.stderr, flush=True)
            return
        if args.counter_set == "lds":
            run_lds_patterns(torch)
            print("[bench] counters run done", file=sys.stderr, flush=True)
            return
        if args.counter_set == "pads":
            run_pads(torch, ops, counters=True)
            print("[bench] counters run done", file=sys.stderr, flush=True)
            return
        if args.counter_set == "companions":
            cache = workloads.random_cache_device(n)
            companions(torch, ops, workloads, args.steps, args.warmup, cache, n, only, counters=True)
            print("[bench] counters run done", file=sys.stderr, flush=True)
            return
    if args.probes:
        print(f"[bench] probes over {n} tokens", file=sys.stderr, flush=True)
        run_probes(torch, workloads, n)
        return
    if args.pads:
        print("[bench] pad-heavy batches", file=sys.stderr, flush=True)
        run_pads(torch, ops)
        return

    print(f"[bench] generating {n} tokens on the device", file=sys.stderr, flush=True)
    src, slots = workloads.large_case_device(n)
    cache = torch.zeros(n * 272, dtype=torch.uint8, device="cuda")
    valid = n  # a permutation: no pad slots
    num_slots = n
    slot_order = ops.mxfp4_slot_order_advised(n, 512, 1, num_slots) and not args.scatter
    inv = ops.mxfp4_inverse_workspace(1, num_slots)

    def scatter_step():
        ops.mxfp4_store(src, slots, cache, 1, num_slots, num_slots)

    def store_by_slot():
        ops.mxfp4_store_by_slot(src, n, inv, cache, 1, num_slots, num_slots)

    def slot_order_step():
        ops.mxfp4_build_inverse(slots, 1, num_slots, inv)
        store_by_slot()

    step = slot_order_step if slot_order else scatter_step

    if args.counters:
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        print("[bench] counters run done", file=sys.stderr, flush=True)
        return

    print(f"[bench] timing {args.steps} steps ({'slot order' if slot_order else 'scatter'})",
          file=sys.stderr, flush=True)
    # The timed region: K steps back to back.  HIP events around the store
    # kernel's launch inside each step give its average duration there (all
    # launches go to torch's current stream).
    stream = torch.cuda.current_stream()
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]

    def timed_step(i):
        if slot_order:
            ops.mxfp4_build_inverse(slots, 1, num_slots, inv)
        kev[i][0].record(stream)
        store_by_slot() if slot_order else scatter_step()
        kev[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        timed_step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_s = ev0.elapsed_time(ev1) / 1000.0 / args.steps
    per_launch = sum(a.elapsed_time(b) for a, b in kev) / 1000.0 / args.steps
    if slot_order:
        kernel = "mxfp4_store_by_slot_kernel<512>"
        kernel_bytes = valid * BY_SLOT_BYTES_PER_TOKEN + num_slots * BY_SLOT_BYTES_PER_SLOT
    else:
        kernel = "mxfp4_store_kernel<512>"
        kernel_bytes = valid * BYTES_PER_TOKEN + (n - valid) * BYTES_PER_PAD
    # The metric's bytes: 1024 read + 272 written + 8 slot bytes per token.
    algo_bytes = valid * BYTES_PER_TOKEN + (n - valid) * BYTES_PER_PAD
    _, sev = time_launches(scatter_step, args.steps, args.warmup, torch)
    scatter_s = sev / args.steps
    achieved = algo_bytes / per_launch / 1e9
    step_gbs = algo_bytes / step_s / 1e9
    traffic = measured_traffic(n, kernel)
    inverse_s = step_s - per_launch

    result = {
        "metric": "MXFP4 store tokens/s and effective HBM GB/s (% of MI355X peak), 1 GPU",
        "value": round(valid * args.steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"mxfp4_store: {n} tokens x 512 bf16 uniform in [-4, 4], random-permutation "
                        f"slots, flat cache of {n} x 272-byte rows, group 32",
            "tokens": n,
            "latent": 512,
            "row_bytes": 272,
            "form": "slot order (build_inverse + store_by_slot)" if slot_order else "scatter (mxfp4_store)",
            "parallelism": "single GPU",
        },
        "effective_GBps": round(valid * BYTES_PER_TOKEN * args.steps / wall / 1e9, 1),
        "frac_hbm_peak_whole_step": round(step_gbs / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": algo_bytes,
            "bytes_per_token": BYTES_PER_TOKEN,
            "kernel_us_per_launch": round(per_launch * 1e6, 2),
            "kernel_own_bytes_per_launch": kernel_bytes,
            "traffic_bytes_per_token": None if traffic is None else round(traffic / valid, 1),
            "whole_step_us": round(step_s * 1e6, 2),
            "whole_step_achieved": round(step_gbs, 1),
            "whole_step_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        },
        "scatter_form": {
            "kernel": "mxfp4_store_kernel<512>",
            "us_per_launch": round(scatter_s * 1e6, 2),
            "GBps": round(valid * BYTES_PER_TOKEN / scatter_s / 1e9, 1),
            "frac_hbm_peak": round(valid * BYTES_PER_TOKEN / scatter_s / 1e9 / HBM_PEAK_GBS, 4),
        },
    }
    if slot_order:
        # One inverse map serves every layer that stores with the same slot
        # mapping in a step: per-layer cost with the map built once for L
        # layers (L = 1 is the headline step above).
        result["per_layer_shared_mapping"] = [
            {"layers": L, "us_per_layer": round((per_launch + inverse_s / L) * 1e6, 2),
             "frac_hbm_peak": round(algo_bytes / (per_launch + inverse_s / L) / 1e9 / HBM_PEAK_GBS, 4)}
            for L in LAYERS_SHARING_MAPPING]
    if not args.no_companions:
        print("[bench] companions", file=sys.stderr, flush=True)
        result["companions"] = companions(torch, ops, workloads, args.steps, args.warmup, cache, n, only)
        if not only or "small_stores" in only:
            result["companions"].update(small_stores(torch, ops, workloads, args.steps, args.warmup))
    del src, slots, inv
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(args.cpu_sample)
    print(json.dumps(result), flush=True)
    if args.sweep:
        del cache
        torch.cuda.empty_cache()
        run_sweep(torch, ops, workloads)
        run_pads(torch, ops)


if __name__ == "__main__":
    main()
