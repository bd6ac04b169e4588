"""Benchmark of the sparse GQA decode path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch of synthetic input, with every input
resident in HBM before the timed region.  Default workload: a Llama-3-8B-shaped layer (batch 8,
32 query / 8 KV heads, d 128, 32768 cached tokens, bf16 K/V): predictor scores of mean-pooled
64-token blocks -> top-32 blocks -> exact attention over the blocks plus 4 sinks and the 512
most recent tokens.  Steps rotate through 8 independent layer caches and fresh queries, so
no step finds the previous step's rows in the 256 MB last-level cache.

Prints ONE JSON line.  `value` is the step's algorithmic bytes (index keys read + selected K/V
rows) per second; `roofline` reports the attention kernel against the 8 TB/s HBM peak;
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="block", choices=["block", "per_head", "spec_verify",
                                                            "tiers", "tiny"])
    ap.add_argument("--layers", type=int, default=8, help="independent layer caches to rotate")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------------------ block workload

def union_rows_block(idx, count, n_tokens, bs, n_sink, n_recent):
    """Rows each (b, kvh) group fetches for a block selection (setup-time bookkeeping)."""
    G = idx.shape[0] * idx.shape[2]
    blocks = idx.reshape(G, -1).long()
    mask = torch.zeros((G, n_tokens), dtype=torch.bool, device=idx.device)
    tok = (blocks[:, :, None] * bs + torch.arange(bs, device=idx.device)).reshape(G, -1)
    mask.scatter_(1, tok.clamp(max=n_tokens - 1), True)
    mask[:, :n_sink] = True
    mask[:, n_tokens - n_recent:] = True
    return int(mask.sum())


def bench_block(args):
    import workloads as W
    from sparse_top_kv_gqa_amd.decode import BlockSparseDecode

    w = W.LLAMA8B_BLOCK
    dev = "cuda"
    L = args.layers
    log(f"generating {L} layer caches of {w.name}")
    decs, qs, preds = [], [], []
    for l in range(L):
        k = W.kv_cache(w, "k", layer=l, device=dev)
        v = W.kv_cache(w, "v", layer=l, device=dev)
        d = BlockSparseDecode(k, v, w.N, w.Hq, w.block_size, w.k, w.n_sink, w.n_recent)
        d.pool(W.predictors(w, step=0, layer=l, device=dev))
        decs.append(d)
        qs.append(W.queries(w, step=1, layer=l, device=dev))
        preds.append(W.predictors(w, step=1, layer=l, device=dev))
    torch.cuda.synchronize()
    # bytes of each step (selection depends on the step's predictor)
    rows = []
    for l in range(L):
        decs[l].step(qs[l], preds[l])
        rows.append(union_rows_block(decs[l].idx, decs[l].count, w.N, w.block_size, w.n_sink,
                                     w.n_recent))
    row_bytes = 2 * w.d * 2                                     # K + V, bf16
    index_bytes = w.B * w.Hkv * (w.N // w.block_size) * w.d * 4  # fp32 pooled keys
    sel_bytes = [r * row_bytes for r in rows]
    step_bytes = [index_bytes + s for s in sel_bytes]

    # one HIP graph per layer slot: index -> top-k -> attention
    graphs = []
    stream = torch.cuda.Stream()
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

    K, Wm = args.steps, args.warmup
    with torch.cuda.stream(stream):
        for i in range(Wm):
            graphs[i % L].replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(K):
            graphs[i % L].replay()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / K
    # graph replays must reproduce an eager step bit for bit
    ref = []
    for l in range(min(L, 2)):
        graphs[l].replay()
        torch.cuda.synchronize()
        ref.append(decs[l].out.clone())
        decs[l].step(qs[l], preds[l])
        torch.cuda.synchronize()
        assert torch.equal(ref[-1], decs[l].out), "graph replay differs from eager step"

    bytes_avg = sum(step_bytes[i % L] for i in range(K)) / K
    sel_avg = sum(sel_bytes[i % L] for i in range(K)) / K

    # attention kernel alone, same stream, eager launches bracketed by events
    att_ms = []
    with torch.cuda.stream(stream):
        for rep in range(3):
            for l in range(L):
                decs[l].step(qs[l], preds[l])
        torch.cuda.synchronize()
        n_rep = 0
        tot = 0.0
        from sparse_top_kv_gqa_amd import sparse_decode_attn
        for rep in range(max(4, K // L // 4)):
            for l in range(L):
                d = decs[l]
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                sparse_decode_attn(qs[l], d.k, d.v, d.idx, d.count, "per_kv_head", d.n_tokens,
                                   gran=d.bs, n_sink=d.n_sink, n_recent=d.n_recent,
                                   sm_scale=d.sm_scale, out=d.out, lse=d.lse, ws=d.ws,
                                   stream=stream)
                b.record(stream)
                att_ms.append((a, b, sel_bytes[l]))
        torch.cuda.synchronize()
    att_time = sum(a.elapsed_time(b) for a, b, _ in att_ms) / len(att_ms)
    att_bytes = sum(x for _, _, x in att_ms) / len(att_ms)
    att_gbs = att_bytes / (att_time * 1e-3) / 1e9

    gbs = bytes_avg / (ms_step * 1e-3) / 1e9
    res = {
        "metric": "sparse decode attn: selected-KV GB/s (% of HBM peak), decode steps/s",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_step, 5),
        "steps_per_s": round(1e3 / ms_step, 1),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.d, "context": w.N, "block_size": w.block_size,
                   "top_blocks": w.k, "sinks": w.n_sink, "recent": w.n_recent,
                   "layer_caches_rotated": L, "bytes_per_step": int(bytes_avg),
                   "selected_rows_per_step": int(sel_avg / row_bytes),
                   "wall_s_timed": round(wall, 4)},
        "roofline": {"bound": "hbm", "kernel": "sparse_decode_attn", "achieved": round(att_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(att_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "avg_launch_us": round(att_time * 1e3, 3),
                     "algorithmic_bytes_per_launch": int(att_bytes)},
    }
    ctx = dict(w=w, decs=decs, qs=qs, preds=preds)
    return res, ctx


def cpu_baseline_block(ctx, seconds):
    """The fp64 oracle, untuned, on a bounded sample: whole (b, kvh) groups of one step."""
    import numpy as np
    import oracle
    from oracle import steps as osteps
    w, d0 = ctx["w"], ctx["decs"][0]
    q, pred = ctx["qs"][0], ctx["preds"][0]

    def host(t):
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    scale = oracle.softmax_scale(w.d)
    groups = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    done = 0
    spent = 0.0
    G = w.G
    for (b, h) in groups:
        kh, vh = host(d0.k[b, h]), host(d0.v[b, h])
        kpool = d0.kpool[b, h].cpu().numpy()
        t0 = time.perf_counter()
        osteps.block_group(host(pred)[b, 0, h], kh, vh, host(q)[b, 0, h * G:(h + 1) * G], w.k,
                           w.block_size, w.n_sink, w.n_recent, scale, kpool=kpool)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= seconds:
            break
    per_step = spent / done * len(groups)
    return {"value": round(1.0 / per_step, 4), "unit": "decode steps/s", "cores": _cores(),
            "kind": "oracle",
            "sample": f"{done} of {len(groups)} (batch, kv-head) groups of one step "
                      f"({spent:.1f} s), scaled to the whole step"}


def _cores():
    try:
        import numpy  # noqa: F401
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        if n and n[0]:
            return int(n[0])
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the sparse decode "
              "path shards by (batch, KV head) with no exchange, so N GPUs would each run this "
              "single-GPU step on their share.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import sparse_top_kv_gqa_amd as spk
    spk.lib()
    if args.workload != "block":
        print(f"workload {args.workload} is not wired into the bench yet", file=sys.stderr)
        sys.exit(2)
    res, ctx = bench_block(args)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline_block(ctx, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
