"""Decode-step runners: the library's entry points chained on one stream with every buffer
allocated up front, so a step can be captured in a HIP graph and replayed.  Orchestration
only — each step of the path is a libspk call.

BlockSparseDecode   predictor scores pooled blocks -> top-k blocks -> attention over the blocks
                    plus sinks and recent window (SparDA-style compact indexer)
TokenSparseDecode   per-head or group-mean token scores -> top-k tokens -> attention over each
                    query's own set, the group's union fetched once (optionally with some rows in
                    pinned host memory)
TieredDecode        tier classification by cumulative importance -> attention over T0 ∪ T1
                    (∪ T2, read from its 8-bit copy) in every layer -> importance update
BlockLookaheadDecode  the block step through several layers whose caches keep some blocks only
                    in pinned host memory; with lookahead, layer l+1's blocks are chosen before
                    layer l attends and their host rows are copied into HBM meanwhile
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import torch

from . import (attn_workspace_size, fused_index_topk_ok, sparse_decode_attn, sparse_index_score,
               sparse_index_score_windowed, sparse_index_topk, sparse_topk_decode_attn,
               sparse_window_pool, topk_attn_workspace_size, topk_select, topk_workspace_size,
               importance_accumulate, tier_classify, window_count, residency_update,
               residency_prefetch, topk_select_union, topk_union_workspace_size,
               sparse_decode_attn_union, attn_union_workspace_size, union_sets,
               lookahead_prefetch, TIERS_T2, t2_fetch, t2_locations, residency_append)

from .streams import cu_partition_streams

UNION_MIN_TOKENS = 16385   # wide rows: the union pipeline (narrower rows fit one workgroup)


class BlockSparseDecode:
    """One layer's block-sparse decode step over a KV cache ``[B, Hkv, Ncap, d]``."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, n_tokens: int, Hq: int, block_size: int,
                 k_blocks: int, n_sink: int, n_recent: int, sm_scale: Optional[float] = None,
                 fused: bool = False, topk_in_attn: bool = True, window: int = 0,
                 stride: int = 0):
        self.k, self.v = k, v
        # window > 0: the predictor scores overlapping compression windows (kernel window,
        # stride stride) and each block takes the largest score of the windows it overlaps
        self.window, self.stride = window, stride
        B, Hkv, _, d = k.shape
        self.B, self.Hkv, self.Hq, self.d = B, Hkv, Hq, d
        self.n_tokens, self.bs, self.kb = n_tokens, block_size, k_blocks
        self.n_sink, self.n_recent = n_sink, n_recent
        self.sm_scale = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
        self.nb = n_tokens // block_size
        # fused=True: scoring and top-k in one launch (one workgroup per KV group; it pays off
        # when there are many groups with short rows, and loses to the two calls when a few
        # dozen groups leave most of the chip idle)
        self.fused = fused and window == 0 and fused_index_topk_ok("block_pooled", 1, 1, self.nb)
        # topk_in_attn (default): the attention launch selects the top-k blocks from the scores
        # itself, one launch fewer; every split workgroup repeats the selection of its group's
        # short score row in its prologue (registers, one barrier per radix pass), which costs
        # less than the separate top-k launch and the gap before the attention
        # (the fused launch walks the sinks, the recent window and the blocks in list order,
        # which needs room for all of them in the context)
        ok = (k.dtype == torch.bfloat16 and self.nb <= 4096 and k_blocks <= 62
              and n_tokens >= k_blocks * block_size + n_sink + n_recent)
        self.topk_in_attn = bool(topk_in_attn) and ok
        if self.topk_in_attn:
            self.fused = False
        dev = k.device
        if window > 0:
            self.kpool = torch.empty((B, Hkv, max(window_count(n_tokens, window, stride), 1), d),
                                     dtype=torch.float32, device=dev)
        else:
            self.kpool = torch.empty((B, Hkv, self.nb, d), dtype=torch.float32, device=dev)
        self.scores = torch.empty((B, 1, Hkv, self.nb), dtype=torch.float32, device=dev)
        kk = min(k_blocks, self.nb)
        self.idx = torch.empty((B, 1, Hkv, max(kk, 1)), dtype=torch.int32, device=dev)
        self.count = torch.empty((B, 1, Hkv), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, 1, Hq, d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, 1, Hq), dtype=torch.float32, device=dev)
        ws = attn_workspace_size("per_kv_head", B, 1, Hq, Hkv, d, n_tokens, self.idx.shape[-1],
                                 block_size, n_sink, n_recent)
        if self.topk_in_attn:
            ws = max(ws, topk_attn_workspace_size(B, Hq, Hkv, d, n_tokens, self.nb, k_blocks,
                                                  block_size, n_sink, n_recent))
        self.ws = torch.zeros(max(ws, 1), dtype=torch.uint8, device=dev)

    def pool(self, pred: torch.Tensor):
        """Mean-pool every complete block (or compression window) of the keys into ``kpool``
        (once per cache; block pooling also scores ``pred`` as a by-product)."""
        if self.window > 0:
            sparse_window_pool(self.k, self.n_tokens, self.window, self.stride, out=self.kpool)
            return
        sparse_index_score("block_raw", pred, self.k, self.n_tokens, self.bs, scores=self.scores,
                           pooled_out=self.kpool)

    def score(self, pred: torch.Tensor):
        """Predictor scores of the blocks (pooled blocks, or windows max-pooled onto blocks)."""
        if self.window > 0:
            sparse_index_score_windowed(pred, self.kpool, self.n_tokens, self.window, self.stride,
                                        self.bs, scores=self.scores)
        else:
            sparse_index_score("block_pooled", pred, self.kpool, self.n_tokens, self.bs,
                               scores=self.scores)

    def select(self, pred: torch.Tensor):
        """Predictor scores of the pooled blocks -> the top-k blocks (idx, count)."""
        if self.fused:
            sparse_index_topk("block_pooled", pred, self.kpool, self.n_tokens, self.kb, self.bs,
                              scores=self.scores, idx=self.idx, count=self.count)
        else:
            self.score(pred)
            topk_select(self.scores, self.kb, idx=self.idx, count=self.count)

    def attend(self, q: torch.Tensor):
        """Attention over the selected blocks, the sinks and the recent window."""
        sparse_decode_attn(q, self.k, self.v, self.idx, self.count, "per_kv_head", self.n_tokens,
                           gran=self.bs, n_sink=self.n_sink, n_recent=self.n_recent,
                           sm_scale=self.sm_scale, out=self.out, lse=self.lse, ws=self.ws)
        return self.out, self.lse

    def attend_scores(self, q: torch.Tensor, stream=None):
        """Top-k of ``scores`` and the attention over the chosen blocks, the sinks and the
        recent window in one launch (also writes idx and count)."""
        sparse_topk_decode_attn(self.scores, self.kb, q, self.k, self.v, self.n_tokens,
                                gran=self.bs, n_sink=self.n_sink, n_recent=self.n_recent,
                                sm_scale=self.sm_scale, out=self.out, lse=self.lse,
                                sel_idx=self.idx.view(-1, self.idx.shape[-1]),
                                sel_count=self.count.view(-1), ws=self.ws, stream=stream)
        return self.out, self.lse

    def step(self, q: torch.Tensor, pred: torch.Tensor):
        if self.topk_in_attn:
            self.score(pred)
            return self.attend_scores(q)
        self.select(pred)
        return self.attend(q)


class TokenSparseDecode:
    """Token-sparse decode step with ``T`` query tokens per sequence.

    mode "token_per_head": every query head keeps its own top-k (scope per_q_head);
    mode "token_group_mean": each (token, KV head) keeps the top-k of the group-mean score
    (scope per_kv_head).  ``index_keys`` is the key array the indexer streams (defaults to k);
    host pools and ``loc`` put some rows in pinned host memory for the attention gather.

    With wide rows and at most 4 selection sets per KV head (``union`` None = automatic) the
    step runs the union pipeline: the per-set top-k and the group's union in one call, then the
    attention over that union (no assembly).

    slices > 1 splits the batch into that many runs of whole sequences and pipelines them over
    two streams: the caller's stream scores and selects slice after slice, and a second stream
    attends to each slice as soon as its selection is made, so that the indexer (bound by HBM)
    of slice i + 1 can run while the attention of slice i reads its host-resident rows (bound
    by PCIe).  The buffers (scores, idx, count, out, lse) are the same full-batch tensors, each
    slice working on its own rows of them.  Scores and selections are bit-identical to
    slices = 1; each slice's attention is bit-identical to the slice run as a batch of its own,
    and against slices = 1 it can differ in rounding, since a launch cuts a group's rows into
    split-K workgroups by its own group count.  Measured on the speculative-verify workload
    (10 % of the rows in host memory) two slices gain about 2 % and more slices lose: beside
    each other both phases run slower than alone.  With every row in HBM it loses.

    attn_cus > 0 (with slices > 1) would also split the compute units: the attentions on a
    stream limited to attn_cus CUs, the selections on one limited to the rest.  The attention's
    workgroups stay resident for as long as their host reads take; on shared CUs they hold the
    slots the indexer needs, and each phase runs slower beside the other than alone.  The
    CU-partitioned streams are switched off for now (streams.cu_partition_streams raises).
    """

    def __init__(self, k: torch.Tensor, v: torch.Tensor, n_tokens: int, Hq: int, T: int, topk: int,
                 mode: str, sm_scale: Optional[float] = None,
                 index_keys: Optional[torch.Tensor] = None, k_host=None, v_host=None, loc=None,
                 union: Optional[bool] = None, slices: int = 1, attn_cus: int = 0,
                 _buffers=None):
        self.k, self.v = k, v
        self.index_keys = k if index_keys is None else index_keys
        self.k_host, self.v_host, self.loc = k_host, v_host, loc
        B, Hkv, _, d = k.shape
        self.B, self.Hkv, self.Hq, self.T, self.d = B, Hkv, Hq, T, d
        self.n_tokens, self.topk, self.mode = n_tokens, topk, mode
        self.scope = "per_q_head" if mode == "token_per_head" else "per_kv_head"
        self.sm_scale = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
        dev = k.device
        Hs = Hq if mode == "token_per_head" else Hkv
        kk = max(1, min(topk, n_tokens))
        if _buffers is not None:
            self.scores, self.idx, self.count, self.out, self.lse = _buffers
        else:
            self.scores = torch.empty((B, T, Hs, n_tokens), dtype=torch.float32, device=dev)
            self.idx = torch.empty((B, T, Hs, kk), dtype=torch.int32, device=dev)
            self.count = torch.empty((B, T, Hs), dtype=torch.int32, device=dev)
            self.out = torch.empty((B, T, Hq, d), dtype=torch.float32, device=dev)
            self.lse = torch.empty((B, T, Hq), dtype=torch.float32, device=dev)
        slices = max(1, min(int(slices), B))
        self.parts = None
        if slices > 1:
            # runs of whole sequences, the last ones one longer when slices does not divide B
            cuts = [b * B // slices for b in range(slices + 1)]
            self.ranges = [(cuts[i], cuts[i + 1]) for i in range(slices)]
            sl = lambda t, b0, b1: None if t is None else t[b0:b1]
            self.parts = [
                TokenSparseDecode(k[b0:b1], v[b0:b1], n_tokens, Hq, T, topk, mode, self.sm_scale,
                                  self.index_keys[b0:b1], sl(k_host, b0, b1), sl(v_host, b0, b1),
                                  sl(loc, b0, b1), union,
                                  _buffers=(self.scores[b0:b1], self.idx[b0:b1],
                                            self.count[b0:b1], self.out[b0:b1], self.lse[b0:b1]))
                for b0, b1 in self.ranges]
            self.union = self.parts[0].union
            if attn_cus > 0:
                self.select_stream, self.attn_stream = cu_partition_streams(attn_cus, dev)
            else:
                self.select_stream, self.attn_stream = None, torch.cuda.Stream(device=dev)
            self.attn_cus = attn_cus
            self._chosen = [torch.cuda.Event() for _ in self.parts]
            self._called = torch.cuda.Event()
            self._attended = torch.cuda.Event()
            return
        S = union_sets(self.scope, T, Hq, Hkv)
        self.union = (S <= 4 and n_tokens >= UNION_MIN_TOKENS) if union is None else bool(union)
        if self.union:
            rows = B * T * Hs
            u_ld = max(1, min(n_tokens, S * min(topk, n_tokens)))
            self.u_list = torch.empty((B * Hkv, u_ld), dtype=torch.int32, device=dev)
            self.u_mask = torch.empty((B * Hkv, u_ld), dtype=torch.int32, device=dev)
            self.u_count = torch.empty((B * Hkv,), dtype=torch.int32, device=dev)
            uws = topk_union_workspace_size(B, T, Hq, Hkv, self.scope, n_tokens, topk)
            self.topk_ws = torch.empty(max(uws, 1), dtype=torch.uint8, device=dev)
            aws = attn_union_workspace_size(self.scope, B, T, Hq, Hkv, d, n_tokens, u_ld)
            self.ws = torch.empty(max(aws, 1), dtype=torch.uint8, device=dev)
        else:
            ws = attn_workspace_size(self.scope, B, T, Hq, Hkv, d, n_tokens, kk)
            self.ws = torch.zeros(max(ws, 1), dtype=torch.uint8, device=dev)
            tws = topk_workspace_size(B * T * Hs, n_tokens, topk)
            self.topk_ws = torch.empty(max(tws, 1), dtype=torch.uint8, device=dev)

    def _each(self, name: str, q: Optional[torch.Tensor], stream):
        """The phase ``name`` of every slice in turn, on one stream (phase timings)."""
        for p, (b0, b1) in zip(self.parts, self.ranges):
            if q is None:
                getattr(p, name)(stream)
            else:
                getattr(p, name)(q[b0:b1], stream)

    def index(self, q: torch.Tensor, stream=None):
        """The indexer's scores."""
        if self.parts is not None:
            return self._each("index", q, stream)
        sparse_index_score(self.mode, q, self.index_keys, self.n_tokens, scores=self.scores,
                           stream=stream)

    def select_topk(self, stream=None):
        """Top-k of the current scores (and, on the union pipeline, each group's union)."""
        if self.parts is not None:
            return self._each("select_topk", None, stream)
        if self.union:
            topk_select_union(self.scores, self.topk, self.scope, self.Hkv,
                              idx=self.idx, count=self.count, u_list=self.u_list,
                              u_mask=self.u_mask, u_count=self.u_count, ws=self.topk_ws,
                              stream=stream)
        else:
            topk_select(self.scores, self.topk, idx=self.idx, count=self.count, ws=self.topk_ws,
                        stream=stream)

    def select(self, q: torch.Tensor, stream=None):
        self.index(q, stream)
        self.select_topk(stream)

    def attend(self, q: torch.Tensor, stream=None):
        if self.parts is not None:
            self._each("attend", q, stream)
            return self.out, self.lse
        if self.union:
            sparse_decode_attn_union(q, self.k, self.v, self.u_list, self.u_mask, self.u_count,
                                     self.scope, self.n_tokens, sm_scale=self.sm_scale,
                                     k_host=self.k_host, v_host=self.v_host, loc=self.loc,
                                     out=self.out, lse=self.lse, ws=self.ws, stream=stream)
        else:
            sparse_decode_attn(q, self.k, self.v, self.idx, self.count, self.scope, self.n_tokens,
                               sm_scale=self.sm_scale, k_host=self.k_host, v_host=self.v_host,
                               loc=self.loc, out=self.out, lse=self.lse, ws=self.ws,
                               stream=stream)
        return self.out, self.lse

    def step(self, q: torch.Tensor, stream=None):
        if self.parts is None:
            self.select(q, stream)
            return self.attend(q, stream)
        caller = torch.cuda.current_stream() if stream is None else stream
        s0, s1 = self.select_stream, self.attn_stream
        if s0 is None:
            s0 = caller
        else:
            # the selection stream starts after everything queued on the caller's stream
            self._called.record(caller)
            s0.wait_event(self._called)
        for p, (b0, b1), ev in zip(self.parts, self.ranges, self._chosen):
            qi = q[b0:b1]
            p.select(qi, s0)
            # the attention stream starts slice i's attention once its selection is made (and,
            # through the same event, after everything queued before it)
            ev.record(s0)
            s1.wait_event(ev)
            p.attend(qi, s1)
        # the caller's stream resumes after the last attention, which comes after the last
        # selection: the next step's selection may then overwrite what the attentions read
        self._attended.record(s1)
        caller.wait_event(self._attended)
        return self.out, self.lse


class TieredDecode:
    """Decode steps of a batch of sequences under the T0/T1/T3 hierarchy, all layers.

    caches: per-layer (k, v) ``[B, Hkv, Ncap, d]``.  State: importance ``s`` fp32
    ``[B, Ncap]`` and the sticky evicted mask ``[B, Ncap]``.

    host_caches / hbm_rows: the hierarchy in memory.  ``host_caches`` are per-layer pinned
    (k, v) host pools holding every row (the DDR tier); HBM then holds ``hbm_rows`` slots per
    sequence (the same slots in every layer and KV head, ``caches`` are those HBM pools, shape
    ``[B, Hkv, hbm_rows, d]``).  Every ``reassign_every`` tiered steps the resident set is
    recomputed (T0 first, then the most important T1 rows while slots remain) and only rows
    that newly need a slot are copied host -> HBM; the attention reads every other selected
    row from the host pools over PCIe.  The results are bit-identical to the all-HBM layout.

    overlap_prefetch: the copies of a reassignment run layer by layer on a second stream
    (default priority), and each layer's attention waits only for its own layer's copy, so
    layer l+1's copy overlaps layer l's attention.

    producer_caches: per-layer device (k, v) pools ``[B, Hkv, >= n_cap, d]`` holding the K/V
    each layer produced for every row (with host_caches).  The rows a sequence gains between two
    steps are then written into free HBM slots (residency_append, lowest slots first; a row
    finding none stays in host memory until the next reassignment), so the protected recent
    rows are read from HBM while memory allows.

    t012_permille / t2_codes: the T2 tier (rows ranked between t01 and t012 are attended from
    their 8-bit copy).  t2_codes are per-layer (codes_k, codes_v, scale_k, scale_v) written by
    kv_quantize_int8 (pinned host memory, or device memory), and needs host_caches.  Every
    tiered step the T2 rows hold staging rows [hbm_rows, hbm_rows + stage_rows) of the HBM
    pools (a row that stays in T2 keeps its staging row; only rows new to T2 are fetched and
    dequantized), and the attention reads them there.
    """

    def __init__(self, caches: Sequence, Hq: int, n_cap: int, n_sink: int, n_recent: int,
                 t0_permille: int = 250, t01_permille: int = 750,
                 sm_scale: Optional[float] = None, host_caches: Optional[Sequence] = None,
                 hbm_rows: int = 0, reassign_every: int = 1, overlap_prefetch: bool = False,
                 t012_permille: Optional[int] = None, t2_codes: Optional[Sequence] = None,
                 producer_caches: Optional[Sequence] = None):
        self.caches = list(caches)
        k0 = self.caches[0][0]
        B, Hkv, _, d = k0.shape
        self.B, self.Hkv, self.Hq, self.d, self.L = B, Hkv, Hq, d, len(self.caches)
        self.n_cap, self.n_sink, self.n_recent = n_cap, n_sink, n_recent
        self.p0, self.p01 = t0_permille, t01_permille
        self.sm_scale = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
        dev = k0.device
        self.s = torch.zeros((B, n_cap), dtype=torch.float32, device=dev)
        self.evicted = torch.zeros((B, n_cap), dtype=torch.uint8, device=dev)
        self.tier = torch.zeros((B, n_cap), dtype=torch.uint8, device=dev)
        self.sel = torch.empty((B, n_cap), dtype=torch.int32, device=dev)
        self.count = torch.empty((B,), dtype=torch.int32, device=dev)
        self.dense_idx = torch.arange(n_cap, dtype=torch.int32, device=dev).repeat(B, 1)
        self.logits = torch.empty((self.L, B, 1, Hq, n_cap), dtype=torch.float32, device=dev)
        self.out = torch.empty((self.L, B, 1, Hq, d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((self.L, B, 1, Hq), dtype=torch.float32, device=dev)
        ws = attn_workspace_size("per_seq", B, 1, Hq, Hkv, d, n_cap, n_cap)
        self.ws = torch.zeros(max(ws, 1), dtype=torch.uint8, device=dev)
        self.host = list(host_caches) if host_caches is not None else None
        self.hbm_rows, self.reassign_every = hbm_rows, max(1, reassign_every)
        self.tiered_steps = 0
        if self.host is not None:
            if len(self.host) != self.L or self.caches[0][0].shape[2] < hbm_rows:
                raise ValueError("one host pool per layer and HBM pools of hbm_rows slots")
            # every row starts in host memory only
            self.loc = (~torch.arange(n_cap, dtype=torch.int32, device=dev)).repeat(B, 1)
            self.loc_view = self.loc.unsqueeze(1).expand(B, Hkv, n_cap)   # shared by KV heads
            self.copy_tok = torch.zeros((B, max(hbm_rows, 1)), dtype=torch.int32, device=dev)
            self.copy_slot = torch.zeros((B, max(hbm_rows, 1)), dtype=torch.int32, device=dev)
            self.copy_count = torch.zeros((B,), dtype=torch.int32, device=dev)
            self.copies = torch.zeros((), dtype=torch.int64, device=dev)   # rows copied so far
        self.overlap = overlap_prefetch and self.host is not None
        self.copy_stream = torch.cuda.Stream(device=dev) if self.overlap else None
        self._copied = None      # per-layer events of the pending overlapped copies
        self.producer = list(producer_caches) if producer_caches is not None else None
        if self.producer is not None:
            if self.host is None or len(self.producer) != self.L:
                raise ValueError("producer_caches need host_caches, one pair per layer")
            self.app_tok = torch.zeros((B, max(1, min(hbm_rows, n_cap))), dtype=torch.int32,
                                       device=dev)
            self.app_slot = torch.zeros_like(self.app_tok)
            self.app_count = torch.zeros((B,), dtype=torch.int32, device=dev)
            self.appended = torch.zeros((), dtype=torch.int64, device=dev)   # rows so far
        self.n_prev = None       # tokens at the previous step (rows past it are new)
        self.p012 = t01_permille if t012_permille is None else t012_permille
        self.t2 = self.p012 > t01_permille
        if self.t2:
            if self.host is None or t2_codes is None or len(t2_codes) != self.L:
                raise ValueError("the T2 tier needs host_caches and per-layer t2_codes")
            self.codes = list(t2_codes)
            # at most floor(M*t012/1000) - floor(M*t01/1000) <= this many T2 rows per sequence
            self.stage_rows = (n_cap * (self.p012 - t01_permille)) // 1000 + 1
            if self.caches[0][0].shape[2] < hbm_rows + self.stage_rows:
                raise ValueError(f"HBM pools need hbm_rows + {self.stage_rows} staging rows")
            self.loc_t2 = (~torch.arange(n_cap, dtype=torch.int32, device=dev)).repeat(B, 1)
            self.loc_attn = torch.empty((B, n_cap), dtype=torch.int32, device=dev)
            self.loc_attn_view = self.loc_attn.unsqueeze(1).expand(B, Hkv, n_cap)
            self.t2_tok = torch.zeros((B, self.stage_rows), dtype=torch.int32, device=dev)
            self.t2_slot = torch.zeros((B, self.stage_rows), dtype=torch.int32, device=dev)
            self.t2_count = torch.zeros((B,), dtype=torch.int32, device=dev)
            self.t2_fetched = torch.zeros((), dtype=torch.int64, device=dev)   # rows so far

    def reset(self):
        """Back to an empty history: importance, evictions, residency and T2 staging."""
        self.s.zero_()
        self.evicted.zero_()
        if self.host is not None:
            dev = self.loc.device
            home = ~torch.arange(self.n_cap, dtype=torch.int32, device=dev)
            self.loc.copy_(home.repeat(self.B, 1))
            self.tiered_steps = 0
            self.copies.zero_()
        if self.t2:
            self.loc_t2.copy_(home.repeat(self.B, 1))
            self.t2_fetched.zero_()
        if self.producer is not None:
            self.appended.zero_()
        self.n_prev = None

    def append(self, n_tokens: int):
        """Free HBM slots for the rows gained since the previous step, and their K/V written
        there from the pools that produced them, in every layer."""
        n_old = self.n_prev
        if self.producer is None or n_old is None or n_tokens <= n_old:
            return
        residency_append(self.loc, n_old, n_tokens, self.hbm_rows, self.app_tok, self.app_slot,
                         self.app_count)
        m = min(n_tokens - n_old, self.app_tok.shape[1])
        for (pk, pv), (k, v) in zip(self.producer, self.caches):
            residency_prefetch(pk, pv, k, v, self.app_tok, self.app_slot, self.app_count, m)
        self.appended += self.app_count.sum()

    def reassign(self, n_tokens: int):
        """Resident set of every sequence for the current tiers, and the differential copy of
        the rows that newly hold a slot, in every layer."""
        residency_update(self.tier, self.s, n_tokens, self.hbm_rows, self.loc, self.copy_tok,
                         self.copy_slot, self.copy_count)
        self.copies += self.copy_count.sum()
        if not self.overlap:
            for (kh, vh), (k, v) in zip(self.host, self.caches):
                residency_prefetch(kh, vh, k, v, self.copy_tok, self.copy_slot, self.copy_count,
                                   self.hbm_rows)
            return
        s1, s2 = torch.cuda.current_stream(), self.copy_stream
        s2.wait_stream(s1)            # the copy list, and the previous step's reads of the pools
        self._copied = []
        for (kh, vh), (k, v) in zip(self.host, self.caches):
            residency_prefetch(kh, vh, k, v, self.copy_tok, self.copy_slot, self.copy_count,
                               self.hbm_rows, stream=s2)
            e = torch.cuda.Event()
            e.record(s2)
            self._copied.append(e)

    def step(self, qs: Sequence[torch.Tensor], n_tokens: int, dense: bool = False):
        """One decode step at ``n_tokens`` cached tokens.  qs: per-layer Q ``[B, 1, Hq, d]``.
        dense=True attends over every token (no importance exists yet)."""
        self.append(n_tokens)
        if dense:
            self.count.fill_(n_tokens)
            sel = self.dense_idx
        else:
            tier_classify(self.s, n_tokens, self.n_sink, self.n_recent, self.p0, self.p01,
                          evicted=self.evicted, tier=self.tier, sel_idx=self.sel,
                          sel_count=self.count, t012_permille=self.p012)
            sel = self.sel
            if self.host is not None and self.tiered_steps % self.reassign_every == 0:
                self.reassign(n_tokens)
            self.tiered_steps += 1
        staged = self.t2 and not dense
        if staged:
            # T2 rows keep their staging rows while they stay in T2; rows new to T2 are listed
            residency_update(self.tier, self.s, n_tokens, self.stage_rows, self.loc_t2,
                             self.t2_tok, self.t2_slot, self.t2_count, tier_classes=TIERS_T2)
            t2_locations(self.tier, self.loc, self.loc_t2, self.loc_attn, n_tokens, self.hbm_rows)
            self.t2_fetched += self.t2_count.sum()
        for l, (k, v) in enumerate(self.caches):
            if self.host is not None:
                kh, vh = self.host[l]
                if self._copied is not None:
                    torch.cuda.current_stream().wait_event(self._copied[l])
                if staged:
                    ck, cv, sk, sv = self.codes[l]
                    t2_fetch(ck, cv, sk, sv, k, v, self.hbm_rows, self.t2_tok, self.t2_slot,
                             self.t2_count, self.stage_rows)
                sparse_decode_attn(qs[l], k, v, sel, self.count, "per_seq", n_tokens,
                                   sm_scale=self.sm_scale, out=self.out[l], lse=self.lse[l],
                                   logits=self.logits[l], ws=self.ws, k_host=kh, v_host=vh,
                                   loc=self.loc_attn_view if staged else self.loc_view)
            else:
                sparse_decode_attn(qs[l], k, v, sel, self.count, "per_seq", n_tokens,
                                   sm_scale=self.sm_scale, out=self.out[l], lse=self.lse[l],
                                   logits=self.logits[l], ws=self.ws)
        self._copied = None
        importance_accumulate(self.s, sel, self.count, self.logits, self.lse, n_tokens)
        self.n_prev = n_tokens
        return self.out, self.lse


class BlockLookaheadDecode:
    """Block-sparse decode through L layers with some blocks of every layer only in pinned host
    memory (SparDA §2, lookahead selection and the persistent copy kernel).

    layers: per layer (k, v, k_host, v_host, loc_home): HBM caches ``[B, Hkv, C, d]`` with
    C >= n_tokens + k_blocks * block_size (the rows past n_tokens are staging rows), pinned host
    pools ``[B, Hkv, Nh, d]`` and the int32 home location of every row ``[B, Hkv, n_tokens]``
    (>= 0: HBM row, < 0: host row ~loc).  The pooled keys are taken from ``pool_keys`` (the keys
    of every row, pooled before any row left HBM).

    lookahead=True: layer l+1's blocks are selected on the caller's stream before layer l
    attends; a second stream (default priority) runs lookahead_prefetch, a persistent kernel of
    ``workgroups`` workgroups (default one per (b, kvh) group), which copies the selected
    blocks' host rows into staging rows and redirects their locations while layer l attends;
    layer l+1's attention waits for it.
    lookahead=False: every layer selects, then attends, reading its host rows in the attention
    kernel itself.  Both give bit-identical results (the reduction order never depends on where
    a row is read from).
    """

    def __init__(self, layers, pool_keys, n_tokens: int, Hq: int, block_size: int, k_blocks: int,
                 n_sink: int, n_recent: int, lookahead: bool = True,
                 workgroups: Optional[int] = None,
                 sm_scale: Optional[float] = None):
        self.layers = list(layers)
        self.L = len(self.layers)
        k0 = self.layers[0][0]
        B, Hkv, C, d = k0.shape
        self.B, self.Hkv, self.Hq, self.d = B, Hkv, Hq, d
        self.n_tokens, self.bs, self.kb = n_tokens, block_size, k_blocks
        self.n_sink, self.n_recent = n_sink, n_recent
        self.lookahead, self.workgroups = lookahead, workgroups
        self.sm_scale = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
        self.stage_base = n_tokens
        if C < n_tokens + k_blocks * block_size:
            raise ValueError("HBM caches need n_tokens + k_blocks * block_size rows")
        dev = k0.device
        # selection per layer: pooled keys, scores, top-k blocks (two launches)
        self.sel = []
        for l, (k, v, _, _, _) in enumerate(self.layers):
            d_l = BlockSparseDecode(k, v, n_tokens, Hq, block_size, k_blocks, n_sink, n_recent,
                                    sm_scale=self.sm_scale, fused=False, topk_in_attn=False)
            self.sel.append(d_l)
        kk = self.sel[0].idx.shape[-1]
        self.loc = [h.clone() for (_, _, _, _, h) in self.layers]
        self.staged = [torch.full((B * Hkv, kk * block_size), -1, dtype=torch.int32, device=dev)
                       for _ in range(self.L)]
        self.staged_count = [torch.zeros((B * Hkv,), dtype=torch.int32, device=dev)
                             for _ in range(self.L)]
        self.out = torch.empty((self.L, B, 1, Hq, d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((self.L, B, 1, Hq), dtype=torch.float32, device=dev)
        ws = attn_workspace_size("per_kv_head", B, 1, Hq, Hkv, d, n_tokens, kk, block_size, n_sink,
                                 n_recent)
        self.ws = torch.zeros(max(ws, 1), dtype=torch.uint8, device=dev)
        self.copy_stream = torch.cuda.Stream(device=dev)
        self.pool_keys = pool_keys

    def pool(self, preds):
        """Pool every layer's complete blocks (from the keys of every row) into its selection."""
        for l, d_l in enumerate(self.sel):
            sparse_index_score("block_raw", preds[l], self.pool_keys[l], self.n_tokens, self.bs,
                               scores=d_l.scores, pooled_out=d_l.kpool)

    def _attend(self, l: int, q: torch.Tensor, loc: torch.Tensor, stream):
        k, v, kh, vh, _ = self.layers[l]
        d_l = self.sel[l]
        sparse_decode_attn(q, k, v, d_l.idx, d_l.count, "per_kv_head", self.n_tokens, gran=self.bs,
                           n_sink=self.n_sink, n_recent=self.n_recent, sm_scale=self.sm_scale,
                           k_host=kh, v_host=vh, loc=loc, out=self.out[l], lse=self.lse[l],
                           ws=self.ws, stream=stream)

    def _prefetch(self, l: int, stream):
        k, v, kh, vh, home = self.layers[l]
        d_l = self.sel[l]
        lookahead_prefetch(d_l.idx, d_l.count, self.bs, self.n_tokens, kh, vh, k, v,
                           self.stage_base, home, self.loc[l], self.staged[l],
                           self.staged_count[l], self.workgroups, stream=stream)

    def step(self, qs, preds, stream=None):
        """One decode step through every layer.  qs / preds: per layer ``[B, 1, Hq, d]`` and
        ``[B, 1, Hkv, d]``."""
        s1 = torch.cuda.current_stream() if stream is None else stream
        if not self.lookahead:
            with torch.cuda.stream(s1):
                for l in range(self.L):
                    self.sel[l].select(preds[l])
                    self._attend(l, qs[l], self.layers[l][4], s1)
            return self.out, self.lse
        s2 = self.copy_stream
        with torch.cuda.stream(s1):
            self.sel[0].select(preds[0])
        done = []
        s2.wait_stream(s1)
        self._prefetch(0, s2)
        e = torch.cuda.Event()
        e.record(s2)
        done.append(e)
        for l in range(self.L):
            if l + 1 < self.L:
                with torch.cuda.stream(s1):
                    self.sel[l + 1].select(preds[l + 1])      # layer l+1's blocks, ahead of time
                s2.wait_stream(s1)
                self._prefetch(l + 1, s2)                     # overlaps layer l's attention
                e = torch.cuda.Event()
                e.record(s2)
                done.append(e)
            s1.wait_event(done[l])
            self._attend(l, qs[l], self.loc[l], s1)
        return self.out, self.lse
