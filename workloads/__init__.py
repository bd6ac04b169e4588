"""Seeded synthetic workloads for sparse GQA decode attention.

This module only draws and shapes inputs.  It holds none of the method's
arithmetic (no scores, no selection, no softmax), so the HIP path and the CPU
oracle can both take their inputs from it without sharing any computation.

Every tensor is drawn from its own ``torch.Generator`` seeded from a stable
hash of (workload, tensor name, batch, layer, kv head, step), so any single
(b, kv-head) group can be drawn again on its own.  Floating point data is
fp32 N(0, 1); bf16 tensors are that fp32 draw rounded to nearest-even by
``Tensor.to(torch.bfloat16)``.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional

import torch

BASE_SEED = 20261202


def seed_of(*parts) -> int:
    """Stable 63-bit seed from a tuple of ints/strings (independent of PYTHONHASHSEED)."""
    h = hashlib.blake2b(repr(tuple(parts)).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(BASE_SEED, *parts))
    return g


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and structure of one decode-step workload.

    name         short identifier used in seeds and reports
    B, T         batch, query tokens per sequence (T>1: speculative verify)
    Hq, Hkv, d   query heads, KV heads, head dim
    N            cached tokens (context) at the measured step
    kv_dtype     "f32" or "bf16" for Q/K/V
    index_mode   "token_group_mean" | "token_per_head" | "block_pooled" | None
    scope        "per_kv_head" | "per_q_head" | "per_seq"
    k            top-k (tokens, or blocks when block_size > 1)
    block_size   1 for token selection, else the pooling block
    n_sink, n_recent   always-kept rows
    window, stride     overlapping compression windows scored instead of whole blocks (0: none)
    slices       runs of whole sequences the token decode step pipelines over two streams (the
                 selection of one run beside the attention of the previous one); a schedule only,
                 the results do not depend on it
    """

    name: str
    B: int
    T: int
    Hq: int
    Hkv: int
    d: int
    N: int
    kv_dtype: str
    index_mode: Optional[str]
    scope: str
    k: int
    block_size: int = 1
    n_sink: int = 0
    n_recent: int = 0
    layers: int = 1
    outlier_frac: float = 0.0      # fraction of K rows per group scaled by outlier_scale
    outlier_scale: float = 4.0
    host_frac: float = 0.0         # fraction of rows per group resident in pinned host memory
    # tiering (reasoning-chain workload)
    n_start: int = 0
    grow_per_step: int = 0
    steps: int = 1
    t0_permille: int = 250
    t01_permille: int = 750
    window: int = 0
    stride: int = 0
    slices: int = 1

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


TINY = Workload("tiny_b1_h4x1_d64_n1024", B=1, T=1, Hq=4, Hkv=1, d=64, N=1024,
                kv_dtype="f32", index_mode="token_group_mean", scope="per_kv_head", k=64)

LLAMA8B_BLOCK = Workload("llama3_8b_b8_n32k_block64_top32", B=8, T=1, Hq=32, Hkv=8, d=128,
                         N=32768, kv_dtype="bf16", index_mode="block_pooled",
                         scope="per_kv_head", k=32, block_size=64, n_sink=4, n_recent=512)

LLAMA8B_BLOCK_WIN = Workload("llama3_8b_b8_n32k_win32s16_block64_top32", B=8, T=1, Hq=32, Hkv=8,
                             d=128, N=32768, kv_dtype="bf16", index_mode="block_windowed",
                             scope="per_kv_head", k=32, block_size=64, n_sink=4, n_recent=512,
                             window=32, stride=16)

PER_HEAD_2PCT = Workload("per_head_b4_n128k_top2pct", B=4, T=1, Hq=32, Hkv=8, d=128,
                         N=131072, kv_dtype="bf16", index_mode="token_per_head",
                         scope="per_q_head", k=math.ceil(0.02 * 131072),
                         outlier_frac=0.01, outlier_scale=4.0)

SPEC_VERIFY = Workload("spec_verify_b16_t4_n64k_top2048", B=16, T=4, Hq=32, Hkv=8, d=128,
                       N=65536, kv_dtype="bf16", index_mode="token_group_mean",
                       scope="per_kv_head", k=2048, host_frac=0.10)

REASONING_TIERS = Workload("tiers_b32_l28_h28x4_n4k_to_16k", B=32, T=1, Hq=28, Hkv=4, d=128,
                           N=16384, kv_dtype="bf16", index_mode=None, scope="per_seq",
                           k=0, n_sink=4, n_recent=512, layers=28, n_start=4096,
                           grow_per_step=192, steps=64)

# The same reasoning episode at twice the context (8192 -> 32768 tokens over 64 steps) for the
# memory hierarchy: batch 8 keeps the pinned host pools of all 28 layers at 15 GB.
REASONING_TIERS_32K = Workload("tiers_b8_l28_h28x4_n8k_to_32k", B=8, T=1, Hq=28, Hkv=4, d=128,
                               N=32768, kv_dtype="bf16", index_mode=None, scope="per_seq",
                               k=0, n_sink=4, n_recent=512, layers=28, n_start=8192,
                               grow_per_step=384, steps=64)

# The block layer over 8 layers with a few blocks of every (group, layer) living only in pinned
# host memory: host_frac is the fraction of the eligible blocks (complete blocks other than
# block 0 and those reaching into the recent window) that are host-resident, chosen so that about
# 1.4 % of the selected rows are host rows.
LOOKAHEAD_BLOCK = Workload("llama3_8b_b8_n32k_block64_top32_l8_hostblocks",
                           B=8, T=1, Hq=32, Hkv=8, d=128, N=32768, kv_dtype="bf16",
                           index_mode="block_pooled", scope="per_kv_head", k=32, block_size=64,
                           n_sink=4, n_recent=512, layers=8, host_frac=0.018)

ALL = {w.name: w for w in (TINY, LLAMA8B_BLOCK, LLAMA8B_BLOCK_WIN, PER_HEAD_2PCT, SPEC_VERIFY,
                           REASONING_TIERS, REASONING_TIERS_32K, LOOKAHEAD_BLOCK)}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(w, **changes)


def torch_dtype(kv_dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[kv_dtype]


def normal(shape, dtype, device, *key) -> torch.Tensor:
    """fp32 N(0,1) draw of ``shape`` from the generator keyed by ``key``, cast to dtype."""
    x = torch.randn(tuple(shape), generator=_gen(device, *key), device=device,
                    dtype=torch.float32)
    return x.to(dtype)


def kv_cache(w: Workload, which: str, layer: int = 0, device="cpu", n_cap: Optional[int] = None,
             groups=None) -> torch.Tensor:
    """K or V cache ``[B, Hkv, n_cap, d]``; row n of group (b, kvh) never depends on n_cap.

    Rows are drawn in chunks of 4096 from per-(group, chunk) generators so that a
    growing cache can be extended without redrawing what exists.
    ``groups``: optional iterable of (b, kvh) to fill (others stay zero).
    K gets the workload's outlier rows (a seeded subset scaled by outlier_scale).
    """
    n_cap = w.N if n_cap is None else n_cap
    dt = torch_dtype(w.kv_dtype)
    out = torch.zeros((w.B, w.Hkv, n_cap, w.d), dtype=dt, device=device)
    todo = groups if groups is not None else [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    for b, h in todo:
        out[b, h] = kv_group(w, which, b, h, layer, device, n_cap)
    return out


CHUNK = 4096


def kv_group(w: Workload, which: str, b: int, h: int, layer: int = 0, device="cpu",
             n_cap: Optional[int] = None) -> torch.Tensor:
    """One group's K or V rows ``[n_cap, d]`` (see kv_cache)."""
    n_cap = w.N if n_cap is None else n_cap
    dt = torch_dtype(w.kv_dtype)
    parts = []
    for c0 in range(0, n_cap, CHUNK):
        rows = min(CHUNK, n_cap - c0)
        x = torch.randn((CHUNK, w.d), generator=_gen(device, w.name, which, b, layer, h, c0),
                        device=device, dtype=torch.float32)[:rows]
        parts.append(x)
    x = torch.cat(parts, 0)
    if which == "k" and w.outlier_frac > 0:
        rows = outlier_rows(w, b, h, device)
        rows = rows[rows < n_cap]
        x[rows] *= w.outlier_scale
    return x.to(dt)


def outlier_rows(w: Workload, b: int, h: int, device="cpu") -> torch.Tensor:
    """Exactly round(outlier_frac * N) distinct rows of group (b, h), by seeded permutation."""
    n_out = int(round(w.outlier_frac * w.N))
    perm = torch.randperm(w.N, generator=_gen("cpu", w.name, "outlier", b, h), device="cpu")
    return perm[:n_out].to(device)


def queries(w: Workload, step: int = 0, layer: int = 0, device="cpu") -> torch.Tensor:
    """Query vectors ``[B, T, Hq, d]`` for one decode step (drawn afresh per step)."""
    return normal((w.B, w.T, w.Hq, w.d), torch_dtype(w.kv_dtype), device, w.name, "q", step, layer)


def predictors(w: Workload, step: int = 0, layer: int = 0, device="cpu") -> torch.Tensor:
    """Forecast/predictor vectors ``[B, T, Hkv, d]``: one per GQA group, drawn per step."""
    return normal((w.B, w.T, w.Hkv, w.d), torch_dtype(w.kv_dtype), device, w.name, "pred", step,
                  layer)


def host_rows(w: Workload, b: int, h: int, candidates: torch.Tensor) -> torch.Tensor:
    """Exactly round(host_frac * len(candidates)) of ``candidates`` (1-D token ids), chosen by
    a seeded permutation: the rows that live in pinned host memory."""
    n = candidates.numel()
    n_host = int(round(w.host_frac * n))
    perm = torch.randperm(n, generator=_gen("cpu", w.name, "host", b, h), device="cpu")
    return candidates.cpu()[perm[:n_host]].sort().values


def host_blocks(w: Workload, b: int, h: int, layer: int = 0) -> torch.Tensor:
    """Block ids of group (b, h) in layer ``layer`` that live only in pinned host memory: exactly
    round(host_frac * eligible) of the eligible blocks [1, (N - n_recent) // block_size - 1),
    chosen by a seeded permutation, ascending."""
    bs = w.block_size
    n_elig = max(0, (w.N - w.n_recent) // bs - 1)
    n_host = int(round(w.host_frac * n_elig))
    perm = torch.randperm(n_elig, generator=_gen("cpu", w.name, "hostblk", b, h, layer),
                          device="cpu")
    return (perm[:n_host] + 1).sort().values


def bf16_bits(t: torch.Tensor):
    """The raw uint16 bit patterns of a bf16 tensor as a numpy array (CPU copy)."""
    import numpy as np
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
