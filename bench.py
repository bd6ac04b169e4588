"""Benchmark of the sparse GQA decode path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch of synthetic input, with every input
resident in HBM (or, for host-resident rows, in pinned host memory) before the timed region.

Default (--workload all): every workload below runs in this one process, one after the other.
The headline — `value`, `ms_per_step`, `roofline`, `cpu_baseline` of the JSON line — is the
largest single-GPU configuration, per_head (131072 tokens, 1.23 GB per step), timed over
exactly --steps steps after --warmup untimed ones; every other workload is reported in the
line's "workloads" object with its own step count, step GB/s, roofline and CPU baseline.

Workloads:
  block        Llama-3-8B-shaped layer: batch 8, 32/8 heads, d 128, 32768 cached tokens, bf16.
               Predictor scores of mean-pooled 64-token blocks -> top-32 blocks -> attention over
               the blocks plus 4 sinks and the 512 most recent tokens.  Steps rotate through 8
               layer caches with fresh queries, so no step finds the previous rows in the 256 MB
               last-level cache.
  block_windowed  the same layer with the predictor scoring overlapping compression windows
               (kernel 32, stride 16) of the keys; each 64-token block takes the largest score
               of the windows it overlaps -> top-32 blocks -> the same attention.
  per_head     batch 4, 32/8 heads, 131072 tokens, 1% outlier keys; every query head keeps its own
               exact top-2% (2622) tokens; each KV group fetches the union of its heads' sets.
  spec_verify  batch 16, 4 draft tokens, 32/8 heads, 65536 tokens; group-mean top-2048 per token;
               the union per KV group is fetched once; 10% of each group's rows live in pinned
               host memory and are read over PCIe inside the attention kernel.
  tiers        batch 32, 28 layers, 28/4 heads, 64 decode steps growing 4096 -> 16384 tokens:
               tier classification -> attention over T0 ∪ T1 in all layers -> importance update.
  block_lookahead  the block layer through 8 layers whose caches keep a seeded 1.8 % of the
               blocks (about 1.4 % of the selected rows) only in pinned host memory: timed with
               lookahead (layer l+1's blocks chosen before layer l attends, their host rows
               copied into HBM by a persistent kernel on a second stream meanwhile), without it
               (host rows read inside the attention) and with every row in HBM.
  tiers_offload  the same episode with every row in pinned host memory and --hbm-rows slots
               per sequence in HBM (default 8192): every --reassign-every steps (default 8) the
               resident set is recomputed and only newly resident rows are copied over PCIe;
               the attention reads the other selected rows from host memory.  Timed with the
               copies before the first layer and overlapped layer by layer with the attention.
  tiers_offload_t2  the offload episode with a T2 tier: the rows ranked 75-95 % are attended
               from their 8-bit copy in pinned host memory (staged into HBM, fetched when new
               to T2), the last 5 % evicted; timed against the same rows at full precision.
  tiers_offload_32k  the offload episode at batch 8 growing 8192 -> 32768 tokens, 16384 HBM
               slots per sequence; every step's outputs are checked bit for bit against the
               same episode with every row in HBM.

Prints ONE JSON line.  `value` is the step's algorithmic bytes (index keys read + selected K/V
rows) per second; `roofline` reports the dominant kernel against the 8 TB/s HBM peak with its
duration measured by HIP events on its own stream; `cpu_baseline` times the fp64 CPU oracle on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import torch

HBM_PEAK_GBS = 8000.0
PCIE_PEAK_GBS = 64.0   # PCIe 5.0 x16, one direction
METRIC = "sparse decode attn: selected-KV GB/s (% of HBM peak), decode steps/s"
ROW_BYTES = 2 * 128 * 2  # one token's K and V for one KV head, bf16, d = 128


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="all",
                    choices=["all", "block", "block_windowed", "per_head", "spec_verify", "tiers",
                             "tiers_offload", "tiers_offload_32k", "tiers_offload_t2",
                             "block_lookahead"])
    ap.add_argument("--hbm-rows", type=int, default=None,
                    help="tiers_offload: HBM slots per sequence (the rest stays in host memory; "
                         "default half the final context)")
    ap.add_argument("--reassign-every", type=int, default=8,
                    help="tiers_offload: tiered steps between residency reassignments")
    ap.add_argument("--layers", type=int, default=8, help="block: layer caches to rotate")
    ap.add_argument("--host-frac", type=float, default=None,
                    help="block_lookahead: fraction of the eligible blocks kept only in host memory "
                         "(default: the workload's)")
    ap.add_argument("--copy-workgroups", type=int, default=None,
                    help="block_lookahead: workgroups of the persistent copy kernel (default: one "
                         "per (batch, kv-head) group)")
    ap.add_argument("--slices", type=int, default=None,
                    help="spec_verify: batch slices the step pipelines over two streams "
                         "(default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run a plain device-to-device copy of this many MiB four times "
                         "(the reference point for hardware byte counters)")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def host(t):
    """CPU copy for the oracle: bf16 as raw uint16 bits, float as float32."""
    import numpy as np
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cores():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        if n and n[0]:
            return int(n[0])
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def event_time_ms(fn, reps, stream, per_call=None):
    """Median duration of fn() bracketed by HIP events recorded on `stream`."""
    evs = []
    with torch.cuda.stream(stream):
        for i in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn(i)
            b.record(stream)
            evs.append((a, b))
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in evs)
    return t[len(t) // 2]


_HIP = None


def _hip():
    """The HIP runtime torch has loaded (ctypes), for events created with explicit flags."""
    global _HIP
    if _HIP is None:
        import ctypes
        h = ctypes.CDLL("libamdhip64.so")
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                          ctypes.c_void_p]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _HIP = h
    return _HIP


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


def gather_kernel_ms(call, reps, stream):
    """Median duration of the attention's gather kernel (the launch that reads the selected
    K/V rows): the library records a pair of HIP events around that launch, on `stream`.  The
    events skip the system-scope cache fence a default event record performs, which would
    otherwise add about 2 us to a kernel of about 20 us."""
    import ctypes
    import sparse_top_kv_gqa_amd as spk
    hip = _hip()
    pairs = []
    for _ in range(reps):
        a, b = ctypes.c_void_p(), ctypes.c_void_p()
        if (hip.hipEventCreateWithFlags(ctypes.byref(a), HIP_EVENT_DISABLE_SYSTEM_FENCE) or
                hip.hipEventCreateWithFlags(ctypes.byref(b), HIP_EVENT_DISABLE_SYSTEM_FENCE)):
            raise RuntimeError("hipEventCreateWithFlags failed")
        pairs.append((a, b))
    L = spk.lib()
    try:
        with torch.cuda.stream(stream):
            for i, (a, b) in enumerate(pairs):
                if L.spk_set_attn_timing_events(a, b) != 0:
                    raise RuntimeError(L.spk_last_error().decode())
                call(i)
    finally:
        L.spk_set_attn_timing_events(None, None)
    torch.cuda.synchronize()
    t = []
    for a, b in pairs:
        f = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(f), a, b):
            raise RuntimeError("hipEventElapsedTime failed")
        t.append(f.value)
        hip.hipEventDestroy(a)
        hip.hipEventDestroy(b)
    t.sort()
    return t[len(t) // 2]


def stream_ceiling_gbs(nbytes, stream, reps=12):
    """HBM read ceiling at this size: the best median rate of the library's plain streaming read
    (spk_stream_read, nontemporal 16-byte loads) over a buffer of `nbytes`, across workgroup
    counts.  The buffers cycle
    through at least 768 MiB so none is still in the 256 MB last-level cache, and a long read
    queued first lets the host enqueue every timed launch ahead of the GPU, so each event pair
    brackets one kernel and no host time."""
    import ctypes
    import sparse_top_kv_gqa_amd as spk
    hip = _hip()
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    nbytes = (int(nbytes) + 15) // 16 * 16
    nbuf = max(4, -(-(768 << 20) // nbytes))
    pool = torch.empty(nbuf * nbytes, dtype=torch.uint8, device="cuda")
    bufs = [pool[i * nbytes:(i + 1) * nbytes] for i in range(nbuf)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    sh = ctypes.c_void_p(stream.cuda_stream)
    best = 0.0
    for wgs in (1024, 2048, 4096, 8192, 16384, 32768):
        pairs = []
        for _ in range(reps):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            if (hip.hipEventCreateWithFlags(ctypes.byref(a), HIP_EVENT_DISABLE_SYSTEM_FENCE) or
                    hip.hipEventCreateWithFlags(ctypes.byref(b), HIP_EVENT_DISABLE_SYSTEM_FENCE)):
                raise RuntimeError("hipEventCreateWithFlags failed")
            pairs.append((a, b))
        for i in range(nbuf):
            spk.stream_read(bufs[i], wgs, sink, stream)          # first touch of every page
        spk.stream_read(pool, 96, sink, stream)                  # long read: the host runs ahead
        for i, (a, b) in enumerate(pairs):
            hip.hipEventRecord(a, sh)
            spk.stream_read(bufs[i % nbuf], wgs, sink, stream)
            hip.hipEventRecord(b, sh)
        torch.cuda.synchronize()
        t = []
        for a, b in pairs:
            f = ctypes.c_float()
            if hip.hipEventElapsedTime(ctypes.byref(f), a, b):
                raise RuntimeError("hipEventElapsedTime failed")
            t.append(f.value)
            hip.hipEventDestroy(a)
            hip.hipEventDestroy(b)
        t.sort()
        best = max(best, nbytes / (t[len(t) // 2] * 1e-3) / 1e9)
    del bufs, pool
    torch.cuda.empty_cache()
    return round(best, 1)


def host_read_ceiling_gbs(nbytes, stream, reps=6, cap=256 << 20):
    """Host-link read ceiling at this size (at most `cap` bytes): the best median rate of the
    library's streaming read of pinned host memory (spk_stream_read_host, the device address of
    the pinned buffer, as the attention reads host-resident rows) across workgroup counts."""
    import ctypes
    import sparse_top_kv_gqa_amd as spk
    hip = _hip()
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    nbytes = (min(int(nbytes), cap) + 15) // 16 * 16
    if nbytes <= 0:
        return None
    buf = torch.zeros(nbytes, dtype=torch.uint8, pin_memory=True)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    sh = ctypes.c_void_p(stream.cuda_stream)
    best = 0.0
    for wgs in (256, 1024, 4096):
        pairs = []
        for _ in range(reps):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            if (hip.hipEventCreateWithFlags(ctypes.byref(a), HIP_EVENT_DISABLE_SYSTEM_FENCE) or
                    hip.hipEventCreateWithFlags(ctypes.byref(b), HIP_EVENT_DISABLE_SYSTEM_FENCE)):
                raise RuntimeError("hipEventCreateWithFlags failed")
            pairs.append((a, b))
        spk.stream_read_host(buf, wgs, sink, stream)             # lead-in: the host runs ahead
        for a, b in pairs:
            hip.hipEventRecord(a, sh)
            spk.stream_read_host(buf, wgs, sink, stream)
            hip.hipEventRecord(b, sh)
        torch.cuda.synchronize()
        t = []
        for a, b in pairs:
            f = ctypes.c_float()
            if hip.hipEventElapsedTime(ctypes.byref(f), a, b):
                raise RuntimeError("hipEventElapsedTime failed")
            t.append(f.value)
            hip.hipEventDestroy(a)
            hip.hipEventDestroy(b)
        t.sort()
        best = max(best, nbytes / (t[len(t) // 2] * 1e-3) / 1e9)
    del buf
    return round(best, 1)


def with_ceiling(roof, stream):
    """Adds the measured read ceiling at the roofline kernel's byte count: HBM for an HBM-bound
    roofline record, the host link (pinned host memory read by a kernel) for a PCIe-bound one."""
    if roof.get("bound") == "hbm":
        c = stream_ceiling_gbs(roof["algorithmic_bytes_per_launch"], stream)
        roof["stream_read_ceiling_GBs"] = c
        roof["frac_of_stream_ceiling"] = round(roof["achieved"] / c, 4) if c > 0 else None
    elif roof.get("bound") == "pcie":
        c = host_read_ceiling_gbs(roof["algorithmic_bytes_per_launch"], stream)
        roof["host_read_ceiling_GBs"] = c
        roof["frac_of_host_read_ceiling"] = round(roof["achieved"] / c, 4) if c else None
    return roof


def copy_calibration(mib):
    """A plain copy of known size, for scaling FETCH_SIZE / WRITE_SIZE counter readings."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {mib} MiB four times (calibration)")
    del src, dst


def timed_loop(run_step, K, W, stream):
    """W untimed steps, then exactly K steps bracketed by synchronisations and events."""
    with torch.cuda.stream(stream):
        for i in range(W):
            run_step(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(K):
            run_step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    return e0.elapsed_time(e1), wall


def cold_step_ms(run_step, reps, stream, flush_mib=1024):
    """Median time of one step after a plain streaming read of `flush_mib` MiB (outside the
    timed pair) has replaced whatever the last-level cache held: the step with every byte from
    HBM.  With flush_mib = 0 the same event pairs time steps queued behind nothing, which
    separates the cost of timing one step alone from the cache's part."""
    import sparse_top_kv_gqa_amd as spk
    flush = torch.empty(max(flush_mib, 1) << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    evs = []
    with torch.cuda.stream(stream):
        for i in range(reps):
            if flush_mib > 0:
                spk.stream_read(flush, 8192, sink, stream)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run_step(i)
            b.record(stream)
            evs.append((a, b))
    torch.cuda.synchronize()
    del flush
    t = sorted(a.elapsed_time(b) for a, b in evs)
    return t[len(t) // 2]


def base_result(w, K, W, ms_step, step_bytes, config):
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    return {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_step, 5), "steps_per_s": round(1e3 / ms_step, 2),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16)", "config": config,
    }


# Bytes the roofline kernel of each workload moves per launch, from two rocprofv3 --pmc runs of
# this script (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch, mean over the dispatches of the
# timed kernel loop).  Each counter is scaled by what it reads for a plain 512 MiB device copy
# in the same runs (FETCH_SIZE 262167 KiB -> x2.0, WRITE_SIZE 524288 KiB -> x1.0).  A reading
# belongs to the kernel sources it was taken on (digest of the files listed): once they change
# it is reported as null until the counters are taken again.
COPY_KIB = 512 * 1024
FETCH_COPY_KIB, WRITE_COPY_KIB = 262167.0, 524288.0
TRAFFIC = {
    "per_head": (('index_score.hip', 'spk_internal.h', 'select_common.h'), "b5e7d593716d4c9d", 524470.5, 65536.0),
    "block": (('attn.hip', 'spk_internal.h', 'select_common.h'), "618b9af45143852f", 41685.54, 1442.0),
    "block_windowed": (('attn.hip', 'spk_internal.h', 'select_common.h'), "618b9af45143852f", 41823.41, 1442.01),
    "spec_verify": (('attn.hip', 'spk_internal.h', 'select_common.h'), "618b9af45143852f", 272558.97, 8544.51),
    "tiers": (('attn.hip', 'spk_internal.h', 'select_common.h'), "618b9af45143852f", 401309.22, 51551.92),
}


def _src_digest(files):
    import hashlib
    h = hashlib.sha256()
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sparse_top_kv_gqa_amd", "csrc")
    for f in files:
        with open(os.path.join(here, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the roofline kernel (counter readings scaled by the copy
    calibration), or None when the kernel's sources changed since the readings."""
    if workload not in TRAFFIC:
        return None
    files, digest, fetch_kib, write_kib = TRAFFIC[workload]
    if _src_digest(files) != digest:
        return None
    fetch = fetch_kib * COPY_KIB / FETCH_COPY_KIB
    write = write_kib * COPY_KIB / WRITE_COPY_KIB
    return int((fetch + write) * 1024)


def roofline(kernel, bytes_per_launch, ms, traffic=None, note=None, bound="hbm",
             peak=HBM_PEAK_GBS):
    gbs = bytes_per_launch / (ms * 1e-3) / 1e9
    r = {"bound": bound, "kernel": kernel, "achieved": round(gbs, 1), "peak": peak,
         "unit": "GB/s", "frac": round(gbs / peak, 4), "traffic": traffic,
         "avg_launch_us": round(ms * 1e3, 3), "algorithmic_bytes_per_launch": int(bytes_per_launch)}
    if note:
        r["note"] = note
    return r


# ------------------------------------------------------------------------------ block

def union_rows_block(idx, n_tokens, bs, n_sink, n_recent):
    """Rows the (b, kvh) groups fetch for a block selection (setup-time bookkeeping)."""
    G = idx.shape[0] * idx.shape[2]
    blocks = idx.reshape(G, -1).long()
    mask = torch.zeros((G, n_tokens), dtype=torch.bool, device=idx.device)
    tok = (blocks[:, :, None] * bs + torch.arange(bs, device=idx.device)).reshape(G, -1)
    mask.scatter_(1, tok.clamp(0, n_tokens - 1), True)
    mask[:, :n_sink] = True
    mask[:, n_tokens - n_recent:] = True
    return int(mask.sum())


def block_fetch_lists(idx, count, n_tokens, bs, n_sink, n_recent):
    """Each (b, kvh) group's fetch list as token ids: the sinks, the recent window, then the
    selected blocks' rows not already listed; -1 marks a hole.  The rows the attention reads,
    for the gather reference (setup-time bookkeeping)."""
    dev = idx.device
    G = idx.shape[0] * idx.shape[2]
    blocks = idx.reshape(G, -1).long()
    nsel = count.reshape(G, 1).long()
    tok = blocks[:, :, None] * bs + torch.arange(bs, device=dev)
    live = (torch.arange(blocks.shape[1], device=dev)[None, :] < nsel)[:, :, None]
    tok = tok.reshape(G, -1)
    live = live.expand(-1, -1, bs).reshape(G, -1)
    ns = min(n_sink, n_tokens)
    rs = max(n_tokens - n_recent, 0)
    forced_tok = torch.cat([torch.arange(ns, device=dev), torch.arange(max(rs, ns), n_tokens, device=dev)])
    keep = live & (tok < n_tokens) & (tok >= ns) & (tok < rs)
    sel = torch.where(keep, tok, torch.full_like(tok, -1))
    return torch.cat([forced_tok[None, :].expand(G, -1), sel], dim=1).to(torch.int32).contiguous()


def gather_ceiling_gbs(caches, lists, stream, reps=12):
    """HBM rate of a plain gather of exactly the attention's rows: the best median over
    workgroups per group of the library's gather reference (spk_gather_read), rotating over
    the layer caches like the timed steps, with a long read queued first so each event pair
    brackets one kernel."""
    import ctypes
    import sparse_top_kv_gqa_amd as spk
    hip = _hip()
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    pad = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    sh = ctypes.c_void_p(stream.cuda_stream)
    L = len(caches)
    nbytes = [int((x >= 0).sum()) * (k.shape[-1] * k.element_size() * 2)
              for x, (k, _) in zip(lists, caches)]
    best = 0.0
    for wpg in (11, 22, 44, 64):
        pairs = []
        for _ in range(reps):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            if (hip.hipEventCreateWithFlags(ctypes.byref(a), HIP_EVENT_DISABLE_SYSTEM_FENCE) or
                    hip.hipEventCreateWithFlags(ctypes.byref(b), HIP_EVENT_DISABLE_SYSTEM_FENCE)):
                raise RuntimeError("hipEventCreateWithFlags failed")
            pairs.append((a, b))
        with torch.cuda.stream(stream):
            for i in range(L):
                spk.gather_read(caches[i][0], caches[i][1], lists[i], wpg, sink, stream)
            spk.stream_read(pad, 48, sink, stream)                 # the host runs ahead
            for i, (a, b) in enumerate(pairs):
                hip.hipEventRecord(a, sh)
                spk.gather_read(caches[i % L][0], caches[i % L][1], lists[i % L], wpg, sink, stream)
                hip.hipEventRecord(b, sh)
        torch.cuda.synchronize()
        rates = []
        for i, (a, b) in enumerate(pairs):
            f = ctypes.c_float()
            if hip.hipEventElapsedTime(ctypes.byref(f), a, b):
                raise RuntimeError("hipEventElapsedTime failed")
            rates.append(nbytes[i % L] / (f.value * 1e-3) / 1e9)
            hip.hipEventDestroy(a)
            hip.hipEventDestroy(b)
        rates.sort()
        best = max(best, rates[len(rates) // 2])
    del pad
    return round(best, 1)


def bench_block(args, windowed=False):
    import workloads as W
    from sparse_top_kv_gqa_amd import sparse_decode_attn, window_count
    from sparse_top_kv_gqa_amd.decode import BlockSparseDecode

    w = W.LLAMA8B_BLOCK_WIN if windowed else W.LLAMA8B_BLOCK
    K = args.steps or 400
    Wm = args.warmup if args.warmup is not None else 40
    L = args.layers
    log(f"generating {L} layer caches of {w.name}")
    decs, qs, preds = [], [], []
    for l in range(L):
        k = W.kv_cache(w, "k", layer=l, device="cuda")
        v = W.kv_cache(w, "v", layer=l, device="cuda")
        d = BlockSparseDecode(k, v, w.N, w.Hq, w.block_size, w.k, w.n_sink, w.n_recent,
                              window=w.window, stride=w.stride)
        d.pool(W.predictors(w, step=0, layer=l, device="cuda"))   # key pooling, once per cache
        decs.append(d)
        qs.append(W.queries(w, step=1, layer=l, device="cuda"))
        preds.append(W.predictors(w, step=1, layer=l, device="cuda"))
    torch.cuda.synchronize()
    rows = []
    for l in range(L):
        decs[l].step(qs[l], preds[l])
        rows.append(union_rows_block(decs[l].idx, w.N, w.block_size, w.n_sink, w.n_recent))
    # fp32 pooled keys: one per block, or one per overlapping compression window
    n_keys = window_count(w.N, w.window, w.stride) if windowed else w.N // w.block_size
    index_bytes = w.B * w.Hkv * n_keys * w.d * 4
    sel_bytes = [r * ROW_BYTES for r in rows]
    step_bytes = [index_bytes + s for s in sel_bytes]

    stream = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(stream):
        for l in range(L):
            decs[l].step(qs[l], preds[l])
        torch.cuda.synchronize()
        for l in range(L):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                decs[l].step(qs[l], preds[l])
            graphs.append(g)
    torch.cuda.synchronize()
    ms_total, wall = timed_loop(lambda i: graphs[i % L].replay(), K, Wm, stream)
    ms_step = ms_total / K
    cold_ms = cold_step_ms(lambda i: graphs[i % L].replay(), 64, stream)
    single_ms = cold_step_ms(lambda i: graphs[i % L].replay(), 64, stream, flush_mib=0)
    # graph replays reproduce an eager step bit for bit
    for l in range(min(L, 2)):
        graphs[l].replay()
        torch.cuda.synchronize()
        ref = decs[l].out.clone()
        decs[l].step(qs[l], preds[l])
        torch.cuda.synchronize()
        assert torch.equal(ref, decs[l].out), "graph replay differs from eager step"

    # the step's attention launch: with the selection inside it (the default) it also reads the
    # group's score row, which counts among its algorithmic bytes
    in_attn = decs[0].topk_in_attn
    score_bytes = w.B * w.Hkv * (w.N // w.block_size) * 4 if in_attn else 0

    def attn(i):
        d = decs[i % L]
        if in_attn:
            d.attend_scores(qs[i % L], stream=stream)
        else:
            sparse_decode_attn(qs[i % L], d.k, d.v, d.idx, d.count, "per_kv_head", d.n_tokens,
                               gran=d.bs, n_sink=d.n_sink, n_recent=d.n_recent,
                               sm_scale=d.sm_scale, out=d.out, lse=d.lse, ws=d.ws, stream=stream)
    att_ms = event_time_ms(attn, 8 * L, stream)
    gather_ms = gather_kernel_ms(attn, 8 * L, stream)
    att_bytes = sum(sel_bytes) / L + score_bytes
    idx_ms = event_time_ms(lambda i: decs[i % L].score(preds[i % L]), 8 * L, stream)
    bytes_avg = sum(step_bytes[i % L] for i in range(K)) / K
    res = base_result(w, K, Wm, ms_step, bytes_avg, {
        "workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
        "context": w.N, "block_size": w.block_size, "top_blocks": w.k, "sinks": w.n_sink,
        "recent": w.n_recent, "layer_caches_rotated": L, "bytes_per_step": int(bytes_avg),
        "selected_rows_per_step": int(sum(sel_bytes) / L / ROW_BYTES),
        "wall_s_timed": round(wall, 4),
        "single_step_ms": round(single_ms, 5), "cold_single_step_ms": round(cold_ms, 5),
        "attention_call_ms": round(att_ms, 4), "index_call_ms": round(idx_ms, 4),
        "index_GBs": round(index_bytes / (idx_ms * 1e-3) / 1e9, 1)})
    if windowed:
        res["config"].update({"window": w.window, "stride": w.stride,
                              "windows_per_group": n_keys})
    kname = ("attn_partial_mfma_kernel (sparse_topk_decode_attn: top-k + gather)" if in_attn
             else "attn_partial_mfma_kernel (sparse_decode_attn gather)")
    res["roofline"] = roofline(kname, att_bytes, gather_ms,
                               traffic=measured_traffic("block_windowed" if windowed else "block"))
    # the rate a plain gather of the same rows reaches (no selection, no arithmetic)
    lists = [block_fetch_lists(d.idx, d.count, d.n_tokens, d.bs, d.n_sink, d.n_recent)
             for d in decs]
    gc = gather_ceiling_gbs([(d.k, d.v) for d in decs], lists, stream)
    res["roofline"]["gather_read_ceiling_GBs"] = gc
    res["roofline"]["frac_of_gather_ceiling"] = round(res["roofline"]["achieved"] / gc, 4)
    ctx = dict(w=w, dec=decs[0], q=qs[0], pred=preds[0], windowed=windowed)
    return res, ctx


def cpu_block(ctx, seconds):
    """The fp64 oracle, untuned, on a bounded sample: whole (b, kvh) groups of one step."""
    import oracle
    from oracle import steps as osteps
    w, d0, q, pred = ctx["w"], ctx["dec"], ctx["q"], ctx["pred"]
    scale = oracle.softmax_scale(w.d)
    groups = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    done, spent, G = 0, 0.0, w.G
    qh, ph = host(q), host(pred)
    for (b, h) in groups:
        kh, vh = host(d0.k[b, h]), host(d0.v[b, h])
        kpool = d0.kpool[b, h].cpu().numpy()
        t0 = time.perf_counter()
        if ctx.get("windowed"):
            nw = oracle.window_count(w.N, w.window, w.stride)
            osteps.block_windowed_group(ph[b, 0, h], kh, vh, qh[b, 0, h * G:(h + 1) * G], w.k,
                                        w.block_size, w.window, w.stride, w.n_sink, w.n_recent,
                                        scale, kwin=kpool[:nw])
        else:
            osteps.block_group(ph[b, 0, h], kh, vh, qh[b, 0, h * G:(h + 1) * G], w.k,
                               w.block_size, w.n_sink, w.n_recent, scale, kpool=kpool)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= seconds:
            break
    layers = ctx.get("layers", 1)
    per_step = spent / done * len(groups) * layers
    return {"value": round(1.0 / per_step, 4), "unit": "decode steps/s", "cores": _cores(),
            "kind": "oracle",
            "sample": f"{done} of {len(groups)} (batch, kv-head) groups of one layer "
                      f"({spent:.1f} s), scaled to the whole step ({layers} layer(s))"}


# ------------------------------------------------------------------------------ token sparse

def _row_mask(ids, N):
    """[G, N] mask of the values in [0, N) of each row of ids [G, M] (int64); anything else
    marks nothing (column N of a scratch mask takes it)."""
    ids = torch.where((ids >= 0) & (ids < N), ids, torch.full_like(ids, N))
    mask = torch.zeros((ids.shape[0], N + 1), dtype=torch.bool, device=ids.device)
    mask.scatter_(1, ids, True)
    return mask[:, :N]


def _distinct_rows(ids, N):
    """Distinct values in [0, N) per row of ids [G, M]."""
    return _row_mask(ids, N).sum(dim=1)


def _counted(idx, count):
    """idx [..., k] as int64 with the entries at or past count[...] set to -1."""
    k = idx.shape[-1]
    live = torch.arange(k, device=idx.device) < count.unsqueeze(-1).long()
    return torch.where(live, idx.long(), torch.full_like(idx, -1, dtype=torch.long))


def union_rows_tokens(idx, count, per_group_rows, N):
    """Rows each (b, kvh) group fetches: union of the selection rows that map to it.
    idx [B, T, Hs, k] int32; count [B, T, Hs]; per_group_rows: selection rows per group along
    (T, Hs/Hkv).  Only the first count entries of a row are read."""
    B, T, Hs, k = idx.shape
    Hkv = Hs // per_group_rows
    ids = _counted(idx, count)
    sel = ids.reshape(B, T, Hkv, per_group_rows, k).permute(0, 2, 1, 3, 4).reshape(B * Hkv, -1)
    return _distinct_rows(sel, N)


def bench_token(args, which):
    import workloads as W
    import sparse_top_kv_gqa_amd as spk
    from sparse_top_kv_gqa_amd.decode import TokenSparseDecode

    w = W.PER_HEAD_2PCT if which == "per_head" else W.SPEC_VERIFY
    K = args.steps or 20
    Wm = args.warmup if args.warmup is not None else 3
    P = 4  # query sets rotated through
    log(f"generating {w.name}")
    k = W.kv_cache(w, "k", device="cuda")
    v = W.kv_cache(w, "v", device="cuda")
    qs = [W.queries(w, step=s, device="cuda") for s in range(P)]
    kh_pool = vh_pool = loc = None
    host_rows_total = 0
    if w.host_frac > 0:
        # a seeded 10% of every group's rows live in pinned host memory
        n_host = int(round(w.host_frac * w.N))
        loc = torch.arange(w.N, dtype=torch.int32, device="cuda").repeat(w.B, w.Hkv, 1)
        kh_pool = torch.empty((w.B, w.Hkv, n_host, w.d), dtype=torch.bfloat16, pin_memory=True)
        vh_pool = torch.empty_like(kh_pool).pin_memory()
        for b in range(w.B):
            for h in range(w.Hkv):
                rows = W.host_rows(w, b, h, torch.arange(w.N)).to("cuda")
                kh_pool[b, h].copy_(k[b, h, rows].cpu())
                vh_pool[b, h].copy_(v[b, h, rows].cpu())
                loc[b, h, rows] = ~torch.arange(rows.numel(), dtype=torch.int32, device="cuda")
        host_rows_total = w.B * w.Hkv * n_host
    mode = "token_per_head" if which == "per_head" else "token_group_mean"
    slices = (args.slices if args.slices is not None else w.slices) \
        if which == "spec_verify" else 1
    dec = TokenSparseDecode(k, v, w.N, w.Hq, w.T, w.k, mode, k_host=kh_pool, v_host=vh_pool,
                            loc=loc, slices=slices)
    torch.cuda.synchronize()
    # bytes: every key read by the indexer + the union rows of each step
    per_group_rows = w.G if which == "per_head" else 1
    union = []
    host_frac = []
    # the rows of one gather launch: the last slice's groups (the whole batch unsliced)
    b0, b1 = dec.ranges[-1] if dec.parts is not None else (0, w.B)
    launch_rows = launch_host_rows = None
    for s in range(P):
        dec.step(qs[s])
        u = union_rows_tokens(dec.idx, dec.count, per_group_rows if which == "per_head" else 1, w.N) \
            if which == "per_head" else None
        if which != "per_head":
            # spec verify: rows of (b, kvh) = union over the T draft tokens
            B, T, Hkv, kk = dec.idx.shape
            sel = _counted(dec.idx, dec.count).permute(0, 2, 1, 3).reshape(B * Hkv, T * kk)
            m = _row_mask(sel, w.N)
            u = m.sum(dim=1)
            hm = (loc.reshape(B * Hkv, w.N) < 0) & m
            host_frac.append(float(hm.sum()) / float(m.sum()))
            if s == 0:
                launch_rows = int(u[b0 * Hkv:b1 * Hkv].sum())
                launch_host_rows = int(hm[b0 * Hkv:b1 * Hkv].sum())
        union.append(int(u.sum()))
        if s == 0 and launch_rows is None:
            launch_rows = int(u.sum())
    index_bytes = w.B * w.Hkv * w.N * w.d * 2
    sel_bytes = [u * ROW_BYTES for u in union]
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    ms_total, wall = timed_loop(lambda i: dec.step(qs[i % P], stream=stream), K, Wm, stream)
    ms_step = ms_total / K
    idx_ms = event_time_ms(lambda i: dec.index(qs[i % P], stream=stream), 10, stream)
    dec.select(qs[0], stream=stream)
    torch.cuda.synchronize()
    att_ms = event_time_ms(lambda i: dec.attend(qs[0], stream=stream), 10, stream)
    gather_ms = gather_kernel_ms(lambda i: dec.attend(qs[0], stream=stream), 10, stream)
    topk_ms = event_time_ms(lambda i: dec.select_topk(stream=stream), 10, stream)
    bytes_avg = index_bytes + sum(sel_bytes) / P
    cfg = {"workload": w.name, "batch": w.B, "query_tokens": w.T, "q_heads": w.Hq,
           "kv_heads": w.Hkv, "head_dim": w.d, "context": w.N, "topk": w.k,
           "bytes_per_step": int(bytes_avg), "index_bytes": index_bytes,
           "selected_rows_per_step": int(sum(union) / P), "wall_s_timed": round(wall, 4),
           "union_pipeline": bool(dec.union),
           "index_ms": round(idx_ms, 4), "topk_ms": round(topk_ms, 4),
           "attention_ms": round(att_ms, 4), "attention_gather_kernel_ms": round(gather_ms, 4),
           "attention_selected_GBs": round(launch_rows * ROW_BYTES / (gather_ms * 1e-3) / 1e9, 1)}
    if dec.parts is not None:
        # attention_ms sums the slices' attentions run one after another; the gather kernel's
        # time and rates are those of one launch, the last slice's (sequences b0 .. b1 - 1)
        cfg["batch_slices"] = len(dec.parts)
        cfg["gather_launch_sequences"] = b1 - b0
    res = base_result(w, K, Wm, ms_step, bytes_avg, cfg)
    if w.host_frac > 0:
        # the gather kernel dominates; its host-resident rows cross PCIe inside it
        cfg["host_fraction_of_selected_rows"] = round(sum(host_frac) / len(host_frac), 4)
        cfg["host_rows_resident"] = host_rows_total
        hb = launch_host_rows * ROW_BYTES
        cfg["hbm_part_GBs_in_gather"] = round((launch_rows - launch_host_rows) * ROW_BYTES /
                                              (gather_ms * 1e-3) / 1e9, 1)
        res["roofline"] = roofline("attn_partial_mfma_kernel (sparse_decode_attn gather), "
                                   "host-resident rows", hb, gather_ms, bound="pcie",
                                   peak=PCIE_PEAK_GBS,
                                   traffic=measured_traffic(which) if slices == w.slices else None,
                                   note="traffic counts every byte the kernel reads (HBM rows "
                                        "and host rows)")
    else:
        kname = f"index_rows_kernel (sparse_index_score {mode})"
        res["roofline"] = roofline(kname, index_bytes, idx_ms, traffic=measured_traffic(which))
    ctx = dict(w=w, k=k, v=v, q=qs[0], which=which)
    return res, ctx


def cpu_token(ctx, seconds):
    import oracle
    from oracle import steps as osteps
    w, k, v, q = ctx["w"], ctx["k"], ctx["v"], ctx["q"]
    scale = oracle.softmax_scale(w.d)
    groups = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    done, spent, G = 0, 0.0, w.G
    qh = host(q)
    for (b, h) in groups:
        kh, vh = host(k[b, h]), host(v[b, h])
        t0 = time.perf_counter()
        if ctx["which"] == "per_head":
            osteps.per_head_group(qh[b, 0, h * G:(h + 1) * G], kh, vh, w.k, scale)
        else:
            osteps.group_mean_group(qh[b, :, h * G:(h + 1) * G], kh, vh, w.k, scale)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= seconds:
            break
    per_step = spent / done * len(groups)
    return {"value": round(1.0 / per_step, 5), "unit": "decode steps/s", "cores": _cores(),
            "kind": "oracle",
            "sample": f"{done} of {len(groups)} (batch, kv-head) groups of one step "
                      f"({spent:.1f} s), scaled to the whole step"}


# ------------------------------------------------------------------------------ tiers

def bench_tiers(args):
    import workloads as W
    import sparse_top_kv_gqa_amd as spk
    from sparse_top_kv_gqa_amd.decode import TieredDecode

    w = W.REASONING_TIERS
    steps = w.steps
    K = args.steps or steps
    Wm = args.warmup if args.warmup is not None else 0
    log(f"generating {w.layers} layer caches of {w.name}")
    caches = [(W.kv_cache(w, "k", l, "cuda", n_cap=w.N), W.kv_cache(w, "v", l, "cuda", n_cap=w.N))
              for l in range(w.layers)]
    qs = [[W.queries(w, step=t, layer=l, device="cuda") for l in range(w.layers)]
          for t in range(steps)]
    dec = TieredDecode(caches, w.Hq, w.N, w.n_sink, w.n_recent, w.t0_permille, w.t01_permille)
    torch.cuda.synchronize()
    n_at = [w.n_start + w.grow_per_step * (t + 1) for t in range(steps)]
    stream = torch.cuda.Stream()

    def run_episode(record_rows=None):
        dec.s.zero_()
        dec.evicted.zero_()
        for t in range(min(K, steps)):
            dec.step(qs[t], n_at[t], dense=(t == 0))
            if record_rows is not None:
                record_rows.append(int(dec.count.sum()))

    rows = []
    with torch.cuda.stream(stream):
        run_episode(rows)            # warm-up episode, records the rows each step reads
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        run_episode()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    n_steps = min(K, steps)
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / n_steps
    # bytes per step: every layer's KV groups read their sequence's T0 ∪ T1 rows
    sel_bytes = [r * w.Hkv * w.layers * ROW_BYTES for r in rows]
    bytes_avg = sum(sel_bytes) / n_steps
    # attention of one layer at the last step (largest N), events on the stream
    k0, v0 = caches[0]
    n_last = n_at[n_steps - 1]

    def attn(i):
        spk.sparse_decode_attn(qs[n_steps - 1][0], k0, v0, dec.sel, dec.count, "per_seq", n_last,
                               out=dec.out[0], lse=dec.lse[0], logits=dec.logits[0], ws=dec.ws,
                               stream=stream)
    att_ms = event_time_ms(attn, 10, stream)
    gather_ms = gather_kernel_ms(attn, 10, stream)
    att_bytes = rows[n_steps - 1] * w.Hkv * ROW_BYTES
    s_copy = dec.s.clone()
    tb = torch.empty_like(dec.tier)
    sb = torch.empty_like(dec.sel)
    cb = torch.empty_like(dec.count)
    tier_ms = event_time_ms(lambda i: spk.tier_classify(s_copy, n_last, w.n_sink, w.n_recent,
                                                        w.t0_permille, w.t01_permille, tier=tb,
                                                        sel_idx=sb, sel_count=cb, stream=stream),
                            5, stream)
    imp_ms = event_time_ms(lambda i: spk.importance_accumulate(s_copy, dec.sel, dec.count,
                                                               dec.logits, dec.lse, n_last,
                                                               stream=stream), 5, stream)
    res = base_result(w, n_steps, Wm, ms_step, bytes_avg, {
        "workload": w.name, "batch": w.B, "layers": w.layers, "q_heads": w.Hq, "kv_heads": w.Hkv,
        "head_dim": w.d, "context_start": w.n_start, "context_end": n_at[n_steps - 1],
        "grow_per_step": w.grow_per_step, "decode_steps": n_steps,
        "bytes_per_step_avg": int(bytes_avg), "rows_last_step_per_layer_kvh": rows[n_steps - 1],
        "episode_s": round(ms_total / 1e3, 4), "wall_s_timed": round(wall, 4),
        "attention_layer_ms_last_step": round(att_ms, 4), "tier_classify_ms": round(tier_ms, 4),
        "importance_ms": round(imp_ms, 4)})
    res["roofline"] = roofline("attn_partial_mfma_kernel (sparse_decode_attn gather, one layer at "
                               f"{n_last} tokens)", att_bytes, gather_ms,
                               traffic=measured_traffic("tiers"))
    # the rate a plain gather of the same rows reaches: each KV group reads its sequence's list
    # (trimmed to the longest list: a skipped entry still costs the reference a cached load)
    ld = int(dec.count.max())
    sel = dec.sel.reshape(dec.sel.shape[0], -1)[:, :ld]
    live = torch.arange(ld, device=sel.device)[None, :] < dec.count.reshape(-1, 1)
    seq_rows = torch.where(live, sel, torch.full_like(sel, -1))
    lists = [seq_rows.repeat_interleave(w.Hkv, dim=0).contiguous()]
    gc = gather_ceiling_gbs([(k0, v0)], lists, stream)
    res["roofline"]["gather_read_ceiling_GBs"] = gc
    res["roofline"]["frac_of_gather_ceiling"] = round(res["roofline"]["achieved"] / gc, 4)
    ctx = dict(w=w, caches=caches, qs=qs, n_last=n_last)
    return res, ctx


def bench_tiers_offload(args, w=None, check_identity=False):
    """The tiered episode with the memory hierarchy: every row lives in pinned host memory
    (the DDR tier), HBM holds HBM_ROWS slots per sequence; every REASSIGN tiered steps the
    resident set is recomputed (T0, then the most important T1 rows while slots remain) and
    only rows that newly need a slot are copied host -> HBM.  The attention reads every other
    selected row over PCIe.  Rows appended since the last reassignment have no slot yet and are
    read from host memory until the next one.  The episode is timed twice: with the copies of
    a reassignment done before the first layer, and overlapped layer by layer with the
    attention on a second stream.  check_identity: the warm-up episode runs beside the same
    episode with every row in HBM, and every step's outputs, lse and the importance state must
    match bit for bit (Proposition 1)."""
    import workloads as W
    import sparse_top_kv_gqa_amd as spk
    from sparse_top_kv_gqa_amd.decode import TieredDecode

    w = W.REASONING_TIERS if w is None else w
    steps = w.steps
    K = args.steps or steps
    cap, every = (args.hbm_rows or w.N // 2), args.reassign_every
    log(f"generating {w.layers} layer caches of {w.name} into pinned host memory")
    host_pools, hbm, full = [], [], []
    for l in range(w.layers):
        pair, fpair = [], []
        for which in ("k", "v"):
            t = W.kv_cache(w, which, l, "cuda", n_cap=w.N)
            h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
            h.copy_(t)
            pair.append(h)
            fpair.append(t)     # the rows as the layer produced them, on the device
            del t
        host_pools.append(tuple(pair))
        full.append(tuple(fpair))
        hbm.append((torch.zeros((w.B, w.Hkv, cap, w.d), dtype=torch.bfloat16, device="cuda"),
                    torch.zeros((w.B, w.Hkv, cap, w.d), dtype=torch.bfloat16, device="cuda")))
    torch.cuda.synchronize()
    qs = [[W.queries(w, step=t, layer=l, device="cuda") for l in range(w.layers)]
          for t in range(steps)]
    mk = dict(host_caches=host_pools, hbm_rows=cap, reassign_every=every, producer_caches=full)
    dec = TieredDecode(hbm, w.Hq, w.N, w.n_sink, w.n_recent, w.t0_permille, w.t01_permille, **mk)
    dec_ov = TieredDecode(hbm, w.Hq, w.N, w.n_sink, w.n_recent, w.t0_permille, w.t01_permille,
                          overlap_prefetch=True, **mk)
    ref = (TieredDecode(full, w.Hq, w.N, w.n_sink, w.n_recent, w.t0_permille, w.t01_permille)
           if check_identity else None)
    n_at = [w.n_start + w.grow_per_step * (t + 1) for t in range(steps)]
    n_steps = min(K, steps)
    stream = torch.cuda.Stream()

    def run_episode(d, record=None):
        d.reset()
        if ref is not None and record is not None:
            ref.reset()
        for t in range(n_steps):
            d.step(qs[t], n_at[t], dense=(t == 0))
            if record is not None:
                sel = d.dense_idx if t == 0 else d.sel
                m = torch.arange(w.N, device="cuda")[None, :] < d.count[:, None].long()
                ids = sel.long().clamp(0, w.N - 1)     # entries past the count are unused
                host_rows = ((torch.gather(d.loc, 1, ids) < 0) & m).sum()
                record.append((int(d.count.sum()), int(host_rows), int(d.copies),
                               int(d.appended)))
                if ref is not None:
                    ref.step(qs[t], n_at[t], dense=(t == 0))
                    assert torch.equal(d.out, ref.out) and torch.equal(d.lse, ref.lse), \
                        f"offload step {t} differs from the all-HBM step"
                    assert torch.equal(d.s, ref.s), f"importance after step {t} differs"

    rec = []
    with torch.cuda.stream(stream):
        run_episode(dec, rec)       # warm-up episode: rows read, rows read from host, copies
        torch.cuda.synchronize()

        def timed(d):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            e0.record(stream)
            run_episode(d)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1), time.perf_counter() - t0
        ms_total, wall = timed(dec)
        run_episode(dec_ov)         # warm-up of the overlapped variant
        s_seq = dec.s.clone()
        ms_total_ov, _ = timed(dec_ov)
        assert torch.equal(dec_ov.s, s_seq) and torch.equal(dec_ov.out, dec.out), \
            "overlapped prefetch changed a result"
    if ref is not None:
        del ref
    ms_step = ms_total / n_steps
    per_layer = w.Hkv * w.layers * ROW_BYTES
    sel_bytes = [r[0] * per_layer for r in rec]
    pcie_attn = sum(r[1] for r in rec) * per_layer
    copies = rec[-1][2]
    appended = rec[-1][3]
    pcie_copy = copies * per_layer
    bytes_avg = sum(sel_bytes) / n_steps
    # the last step's attention in one layer: its host rows cross PCIe inside the gather
    n_last = n_at[n_steps - 1]
    (k0, v0), (kh0, vh0) = hbm[0], host_pools[0]

    def attn(i):
        spk.sparse_decode_attn(qs[n_steps - 1][0], k0, v0, dec.sel, dec.count, "per_seq", n_last,
                               out=dec.out[0], lse=dec.lse[0], logits=dec.logits[0], ws=dec.ws,
                               k_host=kh0, v_host=vh0, loc=dec.loc_view, stream=stream)
    att_ms = event_time_ms(attn, 5, stream)
    gather_ms = gather_kernel_ms(attn, 5, stream)
    host_last = rec[-1][1] * w.Hkv * ROW_BYTES
    res = base_result(w, n_steps, 0, ms_step, bytes_avg, {
        "workload": w.name + "_offload", "batch": w.B, "layers": w.layers, "q_heads": w.Hq,
        "kv_heads": w.Hkv, "head_dim": w.d, "context_start": w.n_start,
        "context_end": n_last, "grow_per_step": w.grow_per_step, "decode_steps": n_steps,
        "hbm_rows_per_sequence": cap, "reassign_every": every,
        "ms_per_step_prefetch_overlapped": round(ms_total_ov / n_steps, 5),
        "bit_identical_to_all_hbm_every_step": bool(check_identity),
        "bytes_per_step_avg": int(bytes_avg),
        "pcie_share_of_step_bytes": round((pcie_attn + pcie_copy) / max(1, sum(sel_bytes)), 4),
        "host_fetch_fraction": round(sum(r[1] for r in rec) / max(1, sum(r[0] for r in rec)), 4),
        "rows_appended_to_hbm_episode": appended,
        "pcie_attention_bytes_per_step": int(pcie_attn / n_steps),
        "prefetch_bytes_episode": int(pcie_copy), "rows_copied_episode": copies,
        "episode_s": round(ms_total / 1e3, 4), "wall_s_timed": round(wall, 4),
        "attention_layer_ms_last_step": round(att_ms, 4),
        "pcie_GBs_episode": round((pcie_attn + pcie_copy) / (ms_total * 1e-3) / 1e9, 2)})
    res["roofline"] = roofline(f"attn_partial_mfma_kernel (host rows of one layer at {n_last} "
                               "tokens, over PCIe)", host_last, gather_ms, bound="pcie",
                               peak=PCIE_PEAK_GBS,
                               note=f"HBM rows of the same launch: "
                                    f"{(rec[-1][0] - rec[-1][1]) * w.Hkv * ROW_BYTES} bytes")
    ctx = dict(w=w, caches=host_pools, qs=qs, n_last=n_last)
    return res, ctx


def bench_tiers_t2(args):
    """The offload episode with the T2 tier: rows ranked between 75 % and 95 % of the unprotected
    ones are attended from their 8-bit copy in pinned host memory (staged into HBM rows,
    fetched only when new to T2), the last 5 % evicted.  Timed against the same episode with
    those rows in T1 (full precision, read from host memory where they hold no HBM slot): the
    same attended rows, twice the PCIe bytes for each."""
    import workloads as W
    import sparse_top_kv_gqa_amd as spk
    from sparse_top_kv_gqa_amd.decode import TieredDecode

    w = W.REASONING_TIERS
    p012 = 950
    steps = w.steps
    n_steps = min(args.steps or steps, steps)
    cap, every = (args.hbm_rows or w.N // 2), args.reassign_every
    stage = (w.N * (p012 - w.t01_permille)) // 1000 + 1
    log(f"generating {w.layers} layer caches of {w.name}, pinned host pools and 8-bit codes")
    host_pools, codes, hbm, produced = [], [], [], []
    for l in range(w.layers):
        pair, cpair, ppair = [], [], []
        for which in ("k", "v"):
            t = W.kv_cache(w, which, l, "cuda", n_cap=w.N)
            h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
            h.copy_(t)
            c = torch.empty(t.shape, dtype=torch.int8, pin_memory=True)
            sc = torch.empty(t.shape[:3], dtype=torch.float32, pin_memory=True)
            spk.kv_quantize_int8(t, c, sc)
            torch.cuda.synchronize()
            pair.append(h)
            cpair.append((c, sc))
            ppair.append(t)     # the rows as the layer produced them, on the device
            del t
        host_pools.append(tuple(pair))
        produced.append(tuple(ppair))
        codes.append((cpair[0][0], cpair[1][0], cpair[0][1], cpair[1][1]))
        hbm.append((torch.zeros((w.B, w.Hkv, cap + stage, w.d), dtype=torch.bfloat16, device="cuda"),
                    torch.zeros((w.B, w.Hkv, cap + stage, w.d), dtype=torch.bfloat16, device="cuda")))
    qs = [[W.queries(w, step=t, layer=l, device="cuda") for l in range(w.layers)]
          for t in range(steps)]
    t2 = TieredDecode(hbm, w.Hq, w.N, w.n_sink, w.n_recent, w.t0_permille, w.t01_permille,
                      host_caches=host_pools, hbm_rows=cap, reassign_every=every,
                      t012_permille=p012, t2_codes=codes, producer_caches=produced)
    full = TieredDecode(hbm, w.Hq, w.N, w.n_sink, w.n_recent, w.t0_permille, p012,
                        host_caches=host_pools, hbm_rows=cap, reassign_every=every,
                        producer_caches=produced)
    n_at = [w.n_start + w.grow_per_step * (t + 1) for t in range(steps)]
    stream = torch.cuda.Stream()

    def run_episode(d, record=None):
        d.reset()
        for t in range(n_steps):
            d.step(qs[t], n_at[t], dense=(t == 0))
            if record is not None:
                ids = (d.dense_idx if t == 0 else d.sel).long().clamp(0, w.N - 1)
                m = torch.arange(w.N, device="cuda")[None, :] < d.count[:, None].long()
                loc = d.loc_attn if (d.t2 and t > 0) else d.loc
                host_rows = ((torch.gather(loc, 1, ids) < 0) & m).sum()
                t2_rows = ((d.tier[:, :n_at[t]] == 2).sum() if t > 0 else torch.zeros(()))
                record.append((int(d.count.sum()), int(host_rows), int(t2_rows),
                               int(d.t2_fetched) if d.t2 else 0))

    def timed(d):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run_episode(d)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    rec_t2, rec_full = [], []
    with torch.cuda.stream(stream):
        run_episode(t2, rec_t2)
        torch.cuda.synchronize()
        out_t2 = t2.out.clone()
        run_episode(full, rec_full)
        torch.cuda.synchronize()
        diff = (t2.out - full.out).abs().max().item() / full.out.abs().max().item()
        ms_t2 = timed(t2)
        ms_full = timed(full)
        assert torch.equal(t2.out, out_t2), "T2 episode not reproducible"
    per_row = w.Hkv * w.layers * ROW_BYTES                        # K and V, every layer and head
    per_code = w.Hkv * w.layers * (2 * w.d + 2 * 4)               # codes and scales of K and V
    fetched = rec_t2[-1][3]
    pcie_t2 = (sum(h for _, h, _, _ in rec_t2) * per_row + fetched * per_code) / n_steps
    pcie_full = sum(h for _, h, _, _ in rec_full) * per_row / n_steps
    sel_bytes = sum(r for r, _, _, _ in rec_t2) * per_row / n_steps
    res = base_result(w, n_steps, 0, ms_t2 / n_steps, sel_bytes, {
        "workload": w.name + "_offload_t2", "batch": w.B, "layers": w.layers, "q_heads": w.Hq,
        "kv_heads": w.Hkv, "head_dim": w.d, "context_start": w.n_start,
        "context_end": n_at[n_steps - 1], "decode_steps": n_steps,
        "tier_permille": [w.t0_permille, w.t01_permille, p012],
        "hbm_rows_per_sequence": cap, "t2_staging_rows_per_sequence": stage,
        "reassign_every": every,
        "ms_per_step_same_rows_full_precision": round(ms_full / n_steps, 5),
        "pcie_bytes_per_step_t2": int(pcie_t2), "pcie_bytes_per_step_full_precision": int(pcie_full),
        "t2_rows_per_step_avg": round(sum(r for _, _, r, _ in rec_t2) / max(1, n_steps - 1), 1),
        "t2_rows_fetched_per_step_avg": round(fetched / max(1, n_steps - 1), 1),
        "max_rel_output_change_vs_full_precision_last_step": float(f"{diff:.3e}")})
    # the last step's attention of one layer, rows staged or resident in HBM or on the host
    k0, v0 = hbm[0]
    kh0, vh0 = host_pools[0]
    n_last = n_at[n_steps - 1]

    def attn(i):
        spk.sparse_decode_attn(qs[n_steps - 1][0], k0, v0, t2.sel, t2.count, "per_seq", n_last,
                               out=t2.out[0], lse=t2.lse[0], logits=t2.logits[0], ws=t2.ws,
                               k_host=kh0, v_host=vh0, loc=t2.loc_attn_view, stream=stream)
    gather_ms = gather_kernel_ms(attn, 5, stream)
    host_last = rec_t2[-1][1] * w.Hkv * ROW_BYTES
    res["roofline"] = roofline(f"attn_partial_mfma_kernel (host rows of one layer at {n_last} "
                               "tokens, T2 rows staged in HBM)", host_last, gather_ms,
                               bound="pcie", peak=PCIE_PEAK_GBS,
                               note=f"HBM rows of the same launch: "
                                    f"{(rec_t2[-1][0] - rec_t2[-1][1]) * w.Hkv * ROW_BYTES} bytes")
    ctx = dict(w=w, caches=host_pools, qs=qs, n_last=n_last, t012=p012)
    return res, ctx


def bench_lookahead(args):
    """Block decode through 8 layers with host-only blocks: lookahead vs none vs all in HBM."""
    import workloads as W
    from sparse_top_kv_gqa_amd.decode import BlockLookaheadDecode, BlockSparseDecode

    w = W.LOOKAHEAD_BLOCK
    if args.host_frac is not None:
        w = W.scaled(w, host_frac=args.host_frac)
    K = args.steps or 50
    Wm = args.warmup if args.warmup is not None else 5
    bs, kb = w.block_size, w.k
    P = 4
    log(f"generating {w.layers} layers of {w.name}")
    full, layers, host_rows_total = [], [], 0
    for l in range(w.layers):
        kf = W.kv_cache(w, "k", layer=l, device="cuda")
        vf = W.kv_cache(w, "v", layer=l, device="cuda")
        full.append((kf, vf))
        home = torch.arange(w.N, dtype=torch.int32).repeat(w.B, w.Hkv, 1)
        rows_g = []
        for b in range(w.B):
            for h in range(w.Hkv):
                blks = W.host_blocks(w, b, h, l)
                rows = (blks[:, None] * bs + torch.arange(bs)).reshape(-1)
                home[b, h, rows] = ~torch.arange(rows.numel(), dtype=torch.int32)
                rows_g.append(rows)
        nh = max(1, max(r.numel() for r in rows_g))
        kh = torch.zeros((w.B, w.Hkv, nh, w.d), dtype=torch.bfloat16, pin_memory=True)
        vh = torch.zeros_like(kh).pin_memory()
        k = torch.empty((w.B, w.Hkv, w.N + kb * bs, w.d), dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        k[:, :, :w.N] = kf
        v[:, :, :w.N] = vf
        i = 0
        for b in range(w.B):
            for h in range(w.Hkv):
                rows = rows_g[i]
                i += 1
                host_rows_total += rows.numel()
                rd = rows.to("cuda")
                kh[b, h, :rows.numel()].copy_(kf[b, h, rd].cpu())
                vh[b, h, :rows.numel()].copy_(vf[b, h, rd].cpu())
                k[b, h, rd] = float("nan")           # the HBM copies of host rows are never read
                v[b, h, rd] = float("nan")
        layers.append((k, v, kh, vh, home.to("cuda")))
    pool_keys = [kf for kf, _ in full]
    qs = [[W.queries(w, step=s, layer=l, device="cuda") for l in range(w.layers)] for s in range(P)]
    preds = [[W.predictors(w, step=s, layer=l, device="cuda") for l in range(w.layers)]
             for s in range(P)]
    la = BlockLookaheadDecode(layers, pool_keys, w.N, w.Hq, bs, kb, w.n_sink, w.n_recent,
                              lookahead=True, workgroups=args.copy_workgroups)
    no = BlockLookaheadDecode(layers, pool_keys, w.N, w.Hq, bs, kb, w.n_sink, w.n_recent,
                              lookahead=False)
    hbm = [BlockSparseDecode(kf, vf, w.N, w.Hq, bs, kb, w.n_sink, w.n_recent, topk_in_attn=False)
           for kf, vf in full]
    pred0 = [W.predictors(w, step=99, layer=l, device="cuda") for l in range(w.layers)]
    la.pool(pred0)
    no.pool(pred0)
    for d_, p_ in zip(hbm, pred0):
        d_.pool(p_)
    stream = torch.cuda.Stream()

    def hbm_step(i):
        for l in range(w.layers):
            hbm[l].select(preds[i % P][l])
            hbm[l].attend(qs[i % P][l])

    # rows per step, host rows among them, bit identity of the three ways
    sel_rows, host_sel = [], []
    with torch.cuda.stream(stream):
        for s_ in range(P):
            la.step(qs[s_], preds[s_], stream=stream)
            o_la = la.out.clone()
            no.step(qs[s_], preds[s_], stream=stream)
            hbm_step(s_)
            torch.cuda.synchronize()
            tot = host = 0
            for l in range(w.layers):
                assert torch.equal(o_la[l], hbm[l].out) and torch.equal(no.out[l], hbm[l].out), \
                    "lookahead, in-kernel host reads and all-HBM differ"
                tot += union_rows_block(hbm[l].idx, w.N, bs, w.n_sink, w.n_recent)
                sel = hbm[l].idx.reshape(w.B * w.Hkv, -1).long()
                toks = (sel[:, :, None] * bs + torch.arange(bs, device="cuda")).reshape(w.B * w.Hkv, -1)
                hm = layers[l][4].reshape(w.B * w.Hkv, w.N)
                host += int((torch.gather(hm, 1, toks.clamp(0, w.N - 1)) < 0).sum())
            sel_rows.append(tot)
            host_sel.append(host)
    index_bytes = w.layers * w.B * w.Hkv * (w.N // bs) * w.d * 4
    step_bytes = index_bytes + sum(sel_rows) / P * ROW_BYTES
    # every variant's step (all layers) captured once per input set and replayed: the timed loops
    # measure the GPU, not the host's launch rate
    def capture(fn):
        gs = []
        with torch.cuda.stream(stream):
            for s_ in range(P):
                fn(s_)
            torch.cuda.synchronize()
            for s_ in range(P):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    fn(s_)
                gs.append(g)
        torch.cuda.synchronize()
        return gs
    g_la = capture(lambda i: la.step(qs[i], preds[i], stream=stream))
    g_no = capture(lambda i: no.step(qs[i], preds[i], stream=stream))
    g_hbm = capture(hbm_step)
    # replays reproduce the eager results bit for bit
    for s_ in range(P):
        g_la[s_].replay()
        g_hbm[s_].replay()
        torch.cuda.synchronize()
        for l in range(w.layers):
            assert torch.equal(la.out[l], hbm[l].out), "graph replay differs"
    ms_la, wall = timed_loop(lambda i: g_la[i % P].replay(), K, Wm, stream)
    ms_no, _ = timed_loop(lambda i: g_no[i % P].replay(), K, Wm, stream)
    ms_hbm, _ = timed_loop(lambda i: g_hbm[i % P].replay(), K, Wm, stream)
    ms_step = ms_la / K
    pcie = sum(host_sel) / P * ROW_BYTES
    # the attention of one layer after its prefetch (every row it reads is in HBM)
    l0 = w.layers - 1

    def attn(i):
        la._attend(l0, qs[0][l0], la.loc[l0], stream)
    la.step(qs[0], preds[0], stream=stream)
    torch.cuda.synchronize()
    gather_ms = gather_kernel_ms(attn, 20, stream)
    att_bytes = sel_rows[0] / w.layers * ROW_BYTES
    res = base_result(w, K, Wm, ms_step, step_bytes, {
        "workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
        "context": w.N, "layers": w.layers, "block_size": bs, "top_blocks": kb,
        "sinks": w.n_sink, "recent": w.n_recent, "bytes_per_step": int(step_bytes),
        "host_rows_resident": host_rows_total,
        "host_block_fraction": w.host_frac,
        "host_fraction_of_selected_rows": round(sum(host_sel) / max(1, sum(sel_rows)), 4),
        "pcie_bytes_per_step": int(pcie), "wall_s_timed": round(wall, 4),
        "ms_per_step_lookahead": round(ms_la / K, 5),
        "ms_per_step_no_lookahead": round(ms_no / K, 5),
        "ms_per_step_all_hbm": round(ms_hbm / K, 5),
        "lookahead_speedup": round(ms_no / ms_la, 3),
        "copy_kernel_workgroups": la.workgroups or w.B * w.Hkv, "timing": "HIP graph replays of the whole step"})
    res["roofline"] = roofline("attn_partial_mfma_kernel (sparse_decode_attn gather, one layer, "
                               "host blocks already staged)", att_bytes, gather_ms)
    ctx = dict(w=w, dec=hbm[0], q=qs[0][0], pred=preds[0][0], windowed=False, layers=w.layers)
    return res, ctx


def cpu_tiers(ctx, seconds):
    """One dense decode step of whole sequences (all layers), the oracle as it stands."""
    import numpy as np
    import oracle
    from oracle import steps as osteps
    w, caches, qs = ctx["w"], ctx["caches"], ctx["qs"]
    n = ctx["n_last"]
    scale = oracle.softmax_scale(w.d)
    done, spent = 0, 0.0
    for b in range(w.B):
        qb = np.stack([host(qs[-1][l])[b, 0] for l in range(w.layers)])
        kb = np.stack([host(caches[l][0][b, :, :n]) for l in range(w.layers)])
        vb = np.stack([host(caches[l][1][b, :, :n]) for l in range(w.layers)])
        s_prev = np.random.default_rng(b).random(n).astype(np.float32)
        t0 = time.perf_counter()
        osteps.tiered_sequence_step(s_prev, None, qb, kb, vb, n, scale, w.n_sink, w.n_recent,
                                    w.t0_permille, w.t01_permille,
                                    t012_permille=ctx.get("t012"))
        spent += time.perf_counter() - t0
        done += 1
        if spent >= seconds:
            break
    per_step = spent / done * w.B
    return {"value": round(1.0 / per_step, 5), "unit": "decode steps/s", "cores": _cores(),
            "kind": "oracle",
            "sample": f"{done} of {w.B} sequences of one tiered step at {n} tokens, all "
                      f"{w.layers} layers ({spent:.1f} s), scaled to the whole batch"}


HEADLINE = "per_head"
ORDER = ["per_head", "block", "block_windowed", "spec_verify", "tiers", "tiers_offload",
         "tiers_offload_32k", "tiers_offload_t2", "block_lookahead"]


def run_workload(name, args):
    """Runs one workload: its timed steps, the read ceiling at its roofline kernel's size and
    (unless switched off) the oracle on the host cores.  Returns the result record."""
    if name in ("block", "block_windowed"):
        res, ctx = bench_block(args, windowed=name == "block_windowed")
        cpu = cpu_block
    elif name in ("per_head", "spec_verify"):
        res, ctx = bench_token(args, name)
        cpu = cpu_token
    elif name == "tiers_offload":
        res, ctx = bench_tiers_offload(args)
        cpu = cpu_tiers
    elif name == "tiers_offload_t2":
        res, ctx = bench_tiers_t2(args)
        cpu = cpu_tiers
    elif name == "tiers_offload_32k":
        import workloads as W
        res, ctx = bench_tiers_offload(args, W.REASONING_TIERS_32K, check_identity=True)
        cpu = cpu_tiers
    elif name == "block_lookahead":
        res, ctx = bench_lookahead(args)
        cpu = cpu_block
    else:
        res, ctx = bench_tiers(args)
        cpu = cpu_tiers
    log(f"{name}: measuring the read ceiling at the roofline kernel's size")
    res["roofline"] = with_ceiling(res["roofline"], torch.cuda.Stream())
    if not args.no_cpu_baseline:
        log(f"{name}: timing the CPU oracle")
        cb = cpu(ctx, args.cpu_seconds)
        cb["cpu_model"] = _cpu_model()
        res["cpu_baseline"] = cb
    del ctx
    return res


def _free():
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def sub_record(res):
    """The per-workload object of the combined line."""
    keep = ("value", "unit", "ms_per_step", "steps_per_s", "pct_of_hbm_peak", "steps", "warmup",
            "config", "roofline", "cpu_baseline")
    return {k: res[k] for k in keep if k in res}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the sparse decode "
              "path shards by (batch, KV head) with no exchange between shards, so N GPUs would "
              "each run this single-GPU step on their share; no multi-GPU figure is produced.",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import copy
    import sparse_top_kv_gqa_amd as spk
    spk.lib()
    if args.calibrate_copy_mib > 0:
        copy_calibration(args.calibrate_copy_mib)
    if args.workload != "all":
        res = run_workload(args.workload, args)
        print(json.dumps(res), flush=True)
        return
    t_all = time.perf_counter()
    head = run_workload(HEADLINE, args)
    _free()
    subs = {}
    for name in ORDER:
        if name == HEADLINE:
            continue
        sub_args = copy.copy(args)
        sub_args.steps = None          # each workload's own step count
        sub_args.warmup = None
        log(f"workload {name}")
        subs[name] = sub_record(run_workload(name, sub_args))
        _free()
    head["workloads"] = subs
    head["config"]["all_workloads_wall_s"] = round(time.perf_counter() - t_all, 1)
    print(json.dumps(head), flush=True)


if __name__ == "__main__":
    main()
