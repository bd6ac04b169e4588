"""Python binding of libspk — sparse top-k KV decode attention (GQA) for AMD MI355X.

Argument marshalling only: every step of the path runs in the HIP kernels of libspk.so.
PyTorch supplies device memory, pinned host memory and the current HIP stream.  The
library must be built (``python -m sparse_top_kv_gqa_amd._build``); importing works without
it, but every call raises if it is missing — there is no fallback path.

Entry points mirror include/spk.h: ``sparse_index_score``, ``topk_select``,
``sparse_decode_attn``, ``importance_accumulate``, ``tier_classify``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

# SPK_LIB names another build of the same library (the AddressSanitizer build of the host code)
LIB_PATH = os.environ.get("SPK_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                     "libspk.so")

# enums of spk.h
F32, BF16 = 0, 1
IDX_TOKEN_GROUP_MEAN, IDX_TOKEN_PER_HEAD, IDX_BLOCK_POOLED, IDX_BLOCK_RAW = 0, 1, 2, 3
SEL_PER_SEQ, SEL_PER_KV_HEAD, SEL_PER_Q_HEAD = 0, 1, 2
STATUS = {0: "SPK_OK", 1: "SPK_EINVAL", 2: "SPK_EUNSUPPORTED", 3: "SPK_EWORKSPACE", 4: "SPK_EHIP"}

MODES = {"token_group_mean": IDX_TOKEN_GROUP_MEAN, "token_per_head": IDX_TOKEN_PER_HEAD,
         "block_pooled": IDX_BLOCK_POOLED, "block_raw": IDX_BLOCK_RAW}
SCOPES = {"per_seq": SEL_PER_SEQ, "per_kv_head": SEL_PER_KV_HEAD, "per_q_head": SEL_PER_Q_HEAD}

EXPORTS = ("spk_last_error", "spk_version", "sparse_index_score", "topk_select_workspace_size",
           "topk_select", "sparse_decode_attn_workspace_size", "sparse_decode_attn",
           "importance_accumulate", "tier_classify_workspace_size", "tier_classify",
           "spk_set_attn_timing_events", "sparse_index_topk",
           "sparse_topk_decode_attn_workspace_size", "sparse_topk_decode_attn",
           "sparse_window_pool", "sparse_index_score_windowed", "residency_update",
           "residency_prefetch", "spk_stream_read", "spk_stream_read_host", "spk_gather_read",
           "sparse_decode_attn_noalloc", "sparse_decode_attn_noalloc_max_bytes",
           "topk_select_union_workspace_size", "topk_select_union",
           "sparse_decode_attn_union_workspace_size", "sparse_decode_attn_union",
           "lookahead_prefetch", "residency_update_tiers", "kv_quantize_int8", "t2_fetch",
           "t2_locations", "residency_append")


class SpkError(RuntimeError):
    def __init__(self, status: int, where: str, text: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}: {text}")
        self.status = status


_lib = None

P = ctypes.c_void_p
I = ctypes.c_int
I64 = ctypes.c_int64
SZ = ctypes.c_size_t
FL = ctypes.c_float


def lib() -> ctypes.CDLL:
    """Load libspk.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m sparse_top_kv_gqa_amd._build` (no fallback path exists)")
    L = ctypes.CDLL(LIB_PATH)
    L.spk_last_error.restype = ctypes.c_char_p
    L.spk_last_error.argtypes = []
    L.spk_version.restype = I
    L.sparse_index_score.restype = I
    L.sparse_index_score.argtypes = [I, P, I, P, I, I64, I64, I64, I, I, I, I, I, I, I, P, I64, P, P]
    L.topk_select_workspace_size.restype = I
    L.topk_select_workspace_size.argtypes = [I, I, I, ctypes.POINTER(SZ)]
    L.topk_select.restype = I
    L.topk_select.argtypes = [P, I64, I, I, I, P, I64, P, P, SZ, P]
    L.sparse_decode_attn_workspace_size.restype = I
    L.sparse_decode_attn_workspace_size.argtypes = [I, I, I, I, I, I, I, I64, I, I, I,
                                                    ctypes.POINTER(SZ)]
    L.sparse_decode_attn.restype = I
    L.sparse_decode_attn.argtypes = [P, I, P, P, I, I64, I64, I64, P, P, I64, I64, I64, I64, P, I64,
                                     I64, I64, P, P, I64, I, I, I, I, I, I, I, I, I, I, FL, P, P, P, I64, P,
                                     SZ, P]
    L.sparse_decode_attn_noalloc.restype = I
    L.sparse_decode_attn_noalloc.argtypes = L.sparse_decode_attn.argtypes[:-3] + [P]
    L.sparse_decode_attn_noalloc_max_bytes.restype = SZ
    L.sparse_decode_attn_noalloc_max_bytes.argtypes = []
    L.topk_select_union_workspace_size.restype = I
    L.topk_select_union_workspace_size.argtypes = [I, I, I, I, I, I, I, ctypes.POINTER(SZ)]
    L.topk_select_union.restype = I
    L.topk_select_union.argtypes = [P, I64, I, I, I, I, I, I, I, P, I64, P, P, P, P, I64, P, SZ, P]
    L.sparse_decode_attn_union_workspace_size.restype = I
    L.sparse_decode_attn_union_workspace_size.argtypes = [I, I, I, I, I, I, I, I64,
                                                          ctypes.POINTER(SZ)]
    L.sparse_decode_attn_union.restype = I
    L.sparse_decode_attn_union.argtypes = [P, I, P, P, I, I64, I64, I64, P, P, I64, I64, I64, I64, P,
                                           I64, I64, I64, P, P, P, I64, I, I, I, I, I, I, I, FL, P, P,
                                           P, I64, P, SZ, P]
    L.lookahead_prefetch.restype = I
    L.lookahead_prefetch.argtypes = [P, P, I64, I, I, I, I, I, I, P, P, I64, I64, I64, I64, P, P,
                                     I64, I64, I64, I64, I64, P, P, I64, I64, P, P, I, P]
    L.importance_accumulate.restype = I
    L.importance_accumulate.argtypes = [P, I64, I, I, P, P, I64, P, I64, P, I, I, P]
    L.tier_classify_workspace_size.restype = I
    L.tier_classify_workspace_size.argtypes = [I, I, ctypes.POINTER(SZ)]
    L.tier_classify.restype = I
    L.tier_classify.argtypes = [P, I64, I, I, I, I, I, I, I, P, I64, P, I64, P, P, I64, P, SZ, P]
    L.spk_set_attn_timing_events.restype = I
    L.spk_set_attn_timing_events.argtypes = [P, P]
    L.spk_stream_read.restype = I
    L.spk_stream_read.argtypes = [P, SZ, I, P, P]
    L.spk_stream_read_host.restype = I
    L.spk_stream_read_host.argtypes = [P, SZ, I, P, P]
    L.spk_gather_read.restype = I
    L.spk_gather_read.argtypes = [P, P, I64, I64, I64, I64, P, I64, I, I, P, P]
    L.sparse_topk_decode_attn_workspace_size.restype = I
    L.sparse_topk_decode_attn_workspace_size.argtypes = [I, I, I, I, I, I, I, I, I, I,
                                                         ctypes.POINTER(SZ)]
    L.sparse_topk_decode_attn.restype = I
    L.sparse_topk_decode_attn.argtypes = [P, I64, I, I, P, I, P, P, I, I64, I64, I64, I, I, I, I, I,
                                          I, I, I, FL, P, P, P, P, I64, P, SZ, P]
    L.sparse_index_topk.restype = I
    L.sparse_index_topk.argtypes = [I, P, I, P, I, I64, I64, I64, I, I, I, I, I, I, I, I, P, I64,
                                    P, I64, P, P]
    L.sparse_window_pool.restype = I
    L.sparse_window_pool.argtypes = [P, I, I64, I64, I64, I, I, I, I, I, I, P, I64, P]
    L.sparse_index_score_windowed.restype = I
    L.sparse_index_score_windowed.argtypes = [P, I, P, I64, I, I, I, I, I, I, I, I, P, I64, P]
    L.residency_update.restype = I
    L.residency_update.argtypes = [P, I64, P, I64, I, I, I, P, I64, P, P, I64, P, P]
    L.residency_update_tiers.restype = I
    L.residency_update_tiers.argtypes = [P, I64, P, I64, I, I, I, I, P, I64, P, P, I64, P, P]
    L.kv_quantize_int8.restype = I
    L.kv_quantize_int8.argtypes = [P, I, I64, I64, I64, I, I, I, I, I, P, I64, I64, I64, P, I64,
                                   I64, P]
    L.t2_fetch.restype = I
    L.t2_fetch.argtypes = [P, P, I64, I64, I64, P, P, I64, I64, I64, P, P, I, I64, I64, I64, I64,
                           I64, I, I, I, P, P, I64, P, I, P]
    L.t2_locations.restype = I
    L.t2_locations.argtypes = [P, I64, P, I64, P, I64, P, I64, I, I, I64, P]
    L.residency_append.restype = I
    L.residency_append.argtypes = [P, I64, I, I, I, I, P, P, I64, P, P]
    L.residency_prefetch.restype = I
    L.residency_prefetch.argtypes = [P, P, I64, I64, I64, I64, P, P, I64, I64, I64, I64, I, I, I,
                                     I, P, P, I64, P, I, P]
    _lib = L
    return L


def _check(status: int, where: str):
    if status != 0:
        raise SpkError(status, where, lib().spk_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ----------------------------------------------------------------------------- validation
#
# The C ABI receives bare pointers and cannot see extents, so every wrapper checks here, before
# any library call, that each tensor has the dtype, device, shape and row layout the kernels
# will index: a mis-shaped tensor raises ValueError and nothing is launched.

def _is_dev(t: torch.Tensor) -> bool:
    return t.is_cuda


def _is_pinned(t: torch.Tensor) -> bool:
    return (not t.is_cuda) and t.is_pinned()


def _need_dev(t, name: str, dtypes=None):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if not _is_dev(t):
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)} (got {t.dtype})")
    return t


def _need_shape(t: torch.Tensor, name: str, shape):
    """`shape`: one entry per dim; an int must match exactly, ('>=', m) is a lower bound,
    None matches anything."""
    if t.dim() != len(shape):
        raise ValueError(f"{name} must have {len(shape)} dims (got shape {tuple(t.shape)})")
    for i, want in enumerate(shape):
        got = t.shape[i]
        if want is None:
            continue
        if isinstance(want, tuple):
            if got < want[1]:
                raise ValueError(f"{name} dim {i} is {got}, needs >= {want[1]} "
                                 f"(shape {tuple(t.shape)})")
        elif got != want:
            raise ValueError(f"{name} dim {i} is {got}, needs {want} (shape {tuple(t.shape)})")
    return t


def _row_ld(t: torch.Tensor, name: str, rows: int, min_len: int) -> int:
    """Checks that `t` is `rows` rows of at least `min_len` contiguous elements, row r starting
    at r·ld (the layout of a [rows, ld] matrix, possibly a column slice of a wider one), and
    returns ld."""
    if t.dim() < 1 or (t.numel() and t.stride(-1) != 1 and t.shape[-1] > 1):
        raise ValueError(f"{name} must have a contiguous last dim")
    lead = t.shape[:-1]
    nrows = int(math.prod(lead)) if len(lead) else 1
    if nrows != rows:
        raise ValueError(f"{name} holds {nrows} rows (shape {tuple(t.shape)}), needs {rows}")
    if t.shape[-1] < min_len:
        raise ValueError(f"{name} rows hold {t.shape[-1]} elements, need >= {min_len}")
    if t.numel() == 0:
        return t.shape[-1]          # empty rows (or none): no element is ever addressed
    ld = t.stride(-2) if t.dim() >= 2 else t.shape[-1]
    expect = ld
    for i in range(t.dim() - 2, -1, -1):
        if t.shape[i] != 1 and t.stride(i) != expect:
            raise ValueError(f"{name}: rows are not evenly spaced (strides {t.stride()})")
        expect *= t.shape[i]
    if rows > 1 and ld < t.shape[-1]:
        raise ValueError(f"{name}: rows overlap (row stride {ld} < {t.shape[-1]})")
    return max(ld, t.shape[-1]) if rows <= 1 else ld


def _need_contig_n(t, name: str, n: int, dtypes):
    """A contiguous device tensor of exactly n elements."""
    _need_dev(t, name, dtypes)
    if t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous with {n} elements (shape {tuple(t.shape)})")
    return t


def _need_cache(t, name: str, B: int, H: int, n_min: int, d: int, dtypes=(torch.float32, torch.bfloat16),
                device=True):
    """A [>=B, H, >=n_min, d] cache view with a contiguous last dim (device or pinned host)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if device:
        _need_dev(t, name, dtypes)
    else:
        if not _is_pinned(t):
            raise ValueError(f"{name} must be pinned host memory")
        if t.dtype not in dtypes:
            raise ValueError(f"{name} has dtype {t.dtype}")
    _need_shape(t, name, [(">=", B), H, (">=", n_min), d])
    _rows_view(t, name)
    return t


F32S, KVS, I32S, U8S = (torch.float32,), (torch.float32, torch.bfloat16), (torch.int32,), (torch.uint8,)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _rows_view(t: torch.Tensor, name: str):
    """(b, h, n, d) strides of a 4-D cache view whose last dim is contiguous."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError(f"{name} must be a 4-D [B, H, N, d] view with a contiguous last dim")
    return t.stride(0), t.stride(1), t.stride(2)


def _contig(t: torch.Tensor, name: str):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


# ----------------------------------------------------------------------------- index scores

def sparse_index_score(mode, q: torch.Tensor, keys: torch.Tensor, n_tokens: int,
                       block_size: int = 1, Hq: Optional[int] = None,
                       scores: Optional[torch.Tensor] = None,
                       pooled_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Indexer scores (no softmax).  q: [B,T,Hq,d] (token modes) or predictor [B,T,Hkv,d]
    (block modes); keys: [B,Hkv,*,d] cache view (or pooled keys).  Returns fp32
    [B,T,Hs,n_cand] (Hs = Hq for per-head, else Hkv)."""
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    _need_dev(q, "q", KVS)
    _contig(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, d]")
    B, T, Hx, d = q.shape
    if keys.dim() != 4:
        raise ValueError("keys must be a [B, Hkv, N, d] view")
    Hkv = keys.shape[1]
    block = m in (IDX_BLOCK_POOLED, IDX_BLOCK_RAW)
    if Hq is None:
        Hq = Hkv if block else Hx
    if block_size < 1 or n_tokens < 0:
        raise ValueError("block_size must be >= 1 and n_tokens >= 0")
    if Hx != (Hkv if block else Hq):
        raise ValueError(f"q has {Hx} heads, needs {Hkv if block else Hq}")
    n_cand = n_tokens // block_size if block else n_tokens
    key_rows = n_cand if m == IDX_BLOCK_POOLED else n_tokens
    _need_cache(keys, "keys", B, Hkv, key_rows, d)
    Hs = Hq if m == IDX_TOKEN_PER_HEAD else Hkv
    if scores is None:
        scores = torch.empty((B, T, Hs, n_cand), dtype=torch.float32, device=q.device)
    _need_dev(scores, "scores", F32S)
    s_ld = _row_ld(scores, "scores", B * T * Hs, n_cand)
    if pooled_out is not None:
        if m != IDX_BLOCK_RAW:
            raise ValueError("pooled_out is written by the block_raw mode only")
        _need_dev(pooled_out, "pooled_out", F32S)
        _contig(pooled_out, "pooled_out")
        _need_shape(pooled_out, "pooled_out", [B, Hkv, (">=", n_cand), d])
        if pooled_out.shape[2] != n_cand:
            raise ValueError(f"pooled_out must be [B, Hkv, {n_cand}, d]")
    sb, sh, sn = _rows_view(keys, "keys")
    st = lib().sparse_index_score(m, _ptr(q), _dt(q), _ptr(keys), _dt(keys), sb, sh, sn, B, T, Hq,
                                  Hkv, d, n_tokens, block_size, _ptr(scores), s_ld,
                                  _ptr(pooled_out), _stream(stream))
    _check(st, "sparse_index_score")
    return scores


def window_count(n_tokens: int, window: int, stride: int) -> int:
    """Complete compression windows [stride*w, stride*w + window) inside n_tokens tokens."""
    return 0 if n_tokens < window else (n_tokens - window) // stride + 1


def sparse_window_pool(keys: torch.Tensor, n_tokens: int, window: int, stride: int,
                       out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Mean of the keys of every complete overlapping compression window.  keys: [B,Hkv,*,d]
    cache view; returns fp32 [B,Hkv,w_cap,d] (w_cap >= the window count; rows past it are not
    written)."""
    if keys.dim() != 4:
        raise ValueError("keys must be a [B, Hkv, N, d] view")
    B, Hkv, _, d = keys.shape
    _need_cache(keys, "keys", B, Hkv, n_tokens, d)
    if window < 1 or stride < 1 or n_tokens < 0:
        raise ValueError("window and stride must be >= 1, n_tokens >= 0")
    nw = window_count(n_tokens, window, stride)
    if out is None:
        out = torch.empty((B, Hkv, max(nw, 1), d), dtype=torch.float32, device=keys.device)
    _need_dev(out, "out", F32S)
    _contig(out, "out")
    _need_shape(out, "out", [B, Hkv, (">=", nw), d])
    sb, sh, sn = _rows_view(keys, "keys")
    st = lib().sparse_window_pool(_ptr(keys), _dt(keys), sb, sh, sn, B, Hkv, d, n_tokens, window,
                                  stride, _ptr(out), out.shape[2], _stream(stream))
    _check(st, "sparse_window_pool")
    return out


def sparse_index_score_windowed(pred: torch.Tensor, kwin: torch.Tensor, n_tokens: int, window: int,
                                stride: int, block_size: int,
                                scores: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Block scores from overlapping compression windows: the predictor [B,T,Hkv,d] scores
    every window of kwin [B,Hkv,w_cap,d] (fp32) and each block takes the largest score of the
    windows it overlaps.  Returns fp32 [B,T,Hkv,n_tokens // block_size]."""
    _need_dev(pred, "pred", KVS)
    _contig(pred, "pred")
    if pred.dim() != 4:
        raise ValueError("pred must be [B, T, Hkv, d]")
    _need_dev(kwin, "kwin", F32S)
    _contig(kwin, "kwin")
    B, T, Hkv, d = pred.shape
    if window < 1 or stride < 1 or block_size < 1 or n_tokens < 0:
        raise ValueError("window, stride and block_size must be >= 1, n_tokens >= 0")
    _need_shape(kwin, "kwin", [B, Hkv, (">=", window_count(n_tokens, window, stride)), d])
    nb = n_tokens // block_size
    if scores is None:
        scores = torch.empty((B, T, Hkv, max(nb, 1)), dtype=torch.float32, device=pred.device)
    _need_dev(scores, "scores", F32S)
    s_ld = _row_ld(scores, "scores", B * T * Hkv, nb)
    st = lib().sparse_index_score_windowed(_ptr(pred), _dt(pred), _ptr(kwin), kwin.shape[2], B, T,
                                           Hkv, d, n_tokens, window, stride, block_size,
                                           _ptr(scores), s_ld, _stream(stream))
    _check(st, "sparse_index_score_windowed")
    return scores


FUSED_MAX_VECTORS, FUSED_MAX_CAND, FUSED_MAX_SCORES = 4, 8192, 16384


def fused_index_topk_ok(mode, T: int, G: int, n_cand: int) -> bool:
    """Whether sparse_index_topk accepts this shape (else use the two separate calls)."""
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    ns = T * G if m == IDX_TOKEN_PER_HEAD else T
    return (m != IDX_BLOCK_RAW and ns <= FUSED_MAX_VECTORS and n_cand <= FUSED_MAX_CAND
            and ns * n_cand <= FUSED_MAX_SCORES)


def sparse_index_topk(mode, q: torch.Tensor, keys: torch.Tensor, n_tokens: int, k: int,
                      block_size: int = 1, Hq: Optional[int] = None,
                      scores: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                      count: Optional[torch.Tensor] = None, want_scores: bool = False,
                      stream=None):
    """Indexer scores and their top-k in one launch (short candidate rows).  Returns
    (idx int32 [B,T,Hs,min(k,n_cand)] ascending, count int32 [B,T,Hs], scores or None)."""
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    _need_dev(q, "q", KVS)
    _contig(q, "q")
    if q.dim() != 4 or keys.dim() != 4:
        raise ValueError("q must be [B, T, H, d] and keys a [B, Hkv, N, d] view")
    B, T, Hx, d = q.shape
    Hkv = keys.shape[1]
    block = m in (IDX_BLOCK_POOLED, IDX_BLOCK_RAW)
    if Hq is None:
        Hq = Hkv if block else Hx
    if block_size < 1 or n_tokens < 0:
        raise ValueError("block_size must be >= 1 and n_tokens >= 0")
    if Hx != (Hkv if block else Hq):
        raise ValueError(f"q has {Hx} heads, needs {Hkv if block else Hq}")
    n_cand = n_tokens // block_size if block else n_tokens
    _need_cache(keys, "keys", B, Hkv, n_cand if m == IDX_BLOCK_POOLED else n_tokens, d)
    Hs = Hq if m == IDX_TOKEN_PER_HEAD else Hkv
    kk = max(0, min(k, n_cand))
    if scores is None and want_scores:
        scores = torch.empty((B, T, Hs, max(n_cand, 1)), dtype=torch.float32, device=q.device)
    if idx is None:
        idx = torch.empty((B, T, Hs, max(kk, 1)), dtype=torch.int32, device=q.device)
    if count is None:
        count = torch.empty((B, T, Hs), dtype=torch.int32, device=q.device)
    s_ld = 0
    if scores is not None:
        _need_dev(scores, "scores", F32S)
        s_ld = _row_ld(scores, "scores", B * T * Hs, n_cand)
    _need_dev(idx, "idx", I32S)
    i_ld = _row_ld(idx, "idx", B * T * Hs, kk)
    _need_contig_n(count, "count", B * T * Hs, I32S)
    sb, sh, sn = _rows_view(keys, "keys")
    st = lib().sparse_index_topk(m, _ptr(q), _dt(q), _ptr(keys), _dt(keys), sb, sh, sn, B, T, Hq,
                                 Hkv, d, n_tokens, block_size, k, _ptr(scores), s_ld, _ptr(idx),
                                 i_ld, _ptr(count), _stream(stream))
    _check(st, "sparse_index_topk")
    return idx, count, scores


# ----------------------------------------------------------------------------- top-k

def topk_workspace_size(rows: int, n: int, k: int) -> int:
    out = SZ(0)
    _check(lib().topk_select_workspace_size(rows, n, k, ctypes.byref(out)),
           "topk_select_workspace_size")
    return out.value


def topk_select(scores: torch.Tensor, k: int, n: Optional[int] = None,
                idx: Optional[torch.Tensor] = None, count: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None, stream=None):
    """Exact top-k of each row of ``scores`` (any leading shape, last dim contiguous).
    Returns (idx int32 [..., min(k, n)] ascending, count int32 [...])."""
    _need_dev(scores, "scores", F32S)
    if scores.dim() < 1:
        raise ValueError("scores must have at least one dim")
    lead = scores.shape[:-1]
    rows = int(math.prod(lead)) if len(lead) else 1
    n = scores.shape[-1] if n is None else n
    if n < 0 or n > scores.shape[-1]:
        raise ValueError(f"n = {n} outside [0, {scores.shape[-1]}]")
    kk = max(0, min(k, n))
    s_ld = _row_ld(scores, "scores", rows, n)
    if idx is None:
        idx = torch.empty((*lead, kk), dtype=torch.int32, device=scores.device)
    if count is None:
        count = torch.empty(lead, dtype=torch.int32, device=scores.device)
    _need_dev(idx, "idx", I32S)
    i_ld = _row_ld(idx, "idx", rows, kk)
    _need_contig_n(count, "count", rows, I32S)
    wsz = topk_workspace_size(rows, n, k)
    if wsz and (ws is None or ws.numel() < wsz):
        ws = torch.empty(wsz, dtype=torch.uint8, device=scores.device)
    if wsz:
        _need_dev(ws, "ws", U8S)
    st = lib().topk_select(_ptr(scores), s_ld, rows, n, k, _ptr(idx), i_ld, _ptr(count),
                           _ptr(ws) if wsz else None, wsz, _stream(stream))
    _check(st, "topk_select")
    return idx, count


def union_sets(scope, T: int, Hq: int, Hkv: int) -> int:
    """Selection sets per KV group: T * G per-head sets, or T per-token sets."""
    sc = SCOPES[scope] if isinstance(scope, str) else int(scope)
    return T * (Hq // Hkv) if sc == SEL_PER_Q_HEAD else T


def topk_union_workspace_size(B, T, Hq, Hkv, scope, n, k) -> int:
    sc = SCOPES[scope] if isinstance(scope, str) else int(scope)
    out = SZ(0)
    _check(lib().topk_select_union_workspace_size(B, T, Hq, Hkv, sc, n, k, ctypes.byref(out)),
           "topk_select_union_workspace_size")
    return out.value


def topk_select_union(scores: torch.Tensor, k: int, scope, Hkv: int, n: Optional[int] = None,
                      idx: Optional[torch.Tensor] = None, count: Optional[torch.Tensor] = None,
                      u_list: Optional[torch.Tensor] = None, u_mask: Optional[torch.Tensor] = None,
                      u_count: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                      stream=None):
    """Per-set exact top-k of scores [B, T, Hs, n] (Hs = Hq for per_q_head, Hkv for
    per_kv_head) and each KV group's union of its sets with a set mask per row.
    Returns (idx int32 [B,T,Hs,min(k,n)], count int32 [B,T,Hs], u_list int32 [B*Hkv, u_ld],
    u_mask int32 [B*Hkv, u_ld], u_count int32 [B*Hkv])."""
    sc = SCOPES[scope] if isinstance(scope, str) else int(scope)
    if sc not in (SEL_PER_Q_HEAD, SEL_PER_KV_HEAD):
        raise ValueError("topk_select_union: scope must be per_q_head or per_kv_head")
    _need_dev(scores, "scores", F32S)
    if scores.dim() != 4:
        raise ValueError("scores must be [B, T, Hs, n]")
    B, T, Hs, _ = scores.shape
    n = scores.shape[-1] if n is None else n
    if n < 0 or n > scores.shape[-1]:
        raise ValueError(f"n = {n} outside [0, {scores.shape[-1]}]")
    Hq = Hs if sc == SEL_PER_Q_HEAD else Hkv
    if sc == SEL_PER_KV_HEAD and Hs != Hkv:
        raise ValueError(f"per_kv_head scores need {Hkv} rows per token, got {Hs}")
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"{Hq} heads are not a multiple of Hkv = {Hkv}")
    rows = B * T * Hs
    s_ld = _row_ld(scores, "scores", rows, n)
    kk = max(0, min(k, n))
    S = union_sets(sc, T, Hq, Hkv)
    u_ld = max(1, min(n, S * kk))
    dev = scores.device
    if idx is None:
        idx = torch.empty((B, T, Hs, max(kk, 1)), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((B, T, Hs), dtype=torch.int32, device=dev)
    if u_list is None:
        u_list = torch.empty((B * Hkv, u_ld), dtype=torch.int32, device=dev)
    if u_mask is None:
        u_mask = torch.empty((B * Hkv, u_ld), dtype=torch.int32, device=dev)
    if u_count is None:
        u_count = torch.empty((B * Hkv,), dtype=torch.int32, device=dev)
    _need_dev(idx, "idx", I32S)
    i_ld = _row_ld(idx, "idx", rows, kk)
    _need_contig_n(count, "count", rows, I32S)
    for t, nm in ((u_list, "u_list"), (u_mask, "u_mask")):
        _need_dev(t, nm, I32S)
        _contig(t, nm)
        _need_shape(t, nm, [B * Hkv, (">=", min(n, S * kk))])
    if u_mask.shape != u_list.shape:
        raise ValueError("u_list and u_mask must have one shape")
    _need_contig_n(u_count, "u_count", B * Hkv, I32S)
    wsz = topk_union_workspace_size(B, T, Hq, Hkv, sc, n, k)
    if ws is None or ws.numel() < wsz:
        ws = torch.empty(max(wsz, 1), dtype=torch.uint8, device=dev)
    _need_dev(ws, "ws", U8S)
    st = lib().topk_select_union(_ptr(scores), s_ld, B, T, Hq, Hkv, sc, n, k,
                                 _ptr(idx), i_ld, _ptr(count), _ptr(u_list), _ptr(u_mask),
                                 _ptr(u_count), u_list.shape[1], _ptr(ws), ws.numel(),
                                 _stream(stream))
    _check(st, "topk_select_union")
    return idx, count, u_list, u_mask, u_count


# ----------------------------------------------------------------------------- attention

def attn_workspace_size(scope, B, T, Hq, Hkv, d, n_tokens, sel_ld, gran=1, n_sink=0,
                        n_recent=0) -> int:
    sc = SCOPES[scope] if isinstance(scope, str) else int(scope)
    out = SZ(0)
    _check(lib().sparse_decode_attn_workspace_size(sc, B, T, Hq, Hkv, d, n_tokens, sel_ld, gran,
                                                   n_sink, n_recent, ctypes.byref(out)),
           "sparse_decode_attn_workspace_size")
    return out.value


def fetch_list_bound(scope, T, G, sel_ld, gran, n_sink, n_recent, n_tokens) -> int:
    """Upper bound of a group's fetch list (the rows of logits), as spk.h defines it."""
    sc = SCOPES[scope] if isinstance(scope, str) else int(scope)
    sets = 1 if sc == SEL_PER_SEQ else (T if sc == SEL_PER_KV_HEAD else T * G)
    return min(n_tokens, sets * sel_ld * gran + n_sink + n_recent)


def _attn_call_args(q, k, v, sel_idx, sel_count, scope, n_tokens, gran, n_sink, n_recent, sm_scale,
                    k_host, v_host, loc, out, lse, logits, u_mask=None):
    """Validates the arguments of sparse_decode_attn (every tensor against the shapes the
    kernels index) and returns (C arguments up to logits_ld, out, lse, sizes for the
    workspace query)."""
    sc = SCOPES[scope] if isinstance(scope, str) else int(scope)
    if sc not in (SEL_PER_SEQ, SEL_PER_KV_HEAD, SEL_PER_Q_HEAD):
        raise ValueError(f"unknown scope {scope}")
    _need_dev(q, "q", KVS)
    _contig(q, "q")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [B, T, Hq, d] and k, v [B, Hkv, N, d] views")
    B, T, Hq, d = q.shape
    Hkv = k.shape[1]
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq = {Hq} is not a multiple of Hkv = {Hkv}")
    if n_tokens < 0 or gran < 1 or n_sink < 0 or n_recent < 0:
        raise ValueError("negative n_tokens, n_sink, n_recent or gran < 1")
    _need_cache(k, "k", B, Hkv, 0 if loc is not None else n_tokens, d)
    _need_cache(v, "v", B, Hkv, 0 if loc is not None else n_tokens, d, dtypes=(k.dtype,))
    _need_dev(sel_idx, "sel_idx", I32S)
    if u_mask is None:
        sel_rows = {SEL_PER_SEQ: B, SEL_PER_KV_HEAD: B * T * Hkv, SEL_PER_Q_HEAD: B * T * Hq}[sc]
    else:
        sel_rows = B * Hkv                    # one assembled union per (b, kvh) group
        _need_dev(u_mask, "u_mask", I32S)
        if u_mask.shape != sel_idx.shape or not u_mask.is_contiguous():
            raise ValueError("u_mask must be contiguous with the shape of u_list")
    if sel_idx.dim() < 1:
        raise ValueError("sel_idx must have at least one dim")
    sel_ld = _row_ld(sel_idx, "sel_idx", sel_rows, 0)
    sel_ld = sel_idx.shape[-1] if sel_rows <= 1 else sel_ld
    if sel_rows > 1 and sel_ld != sel_idx.shape[-1]:
        raise ValueError("sel_idx rows must be contiguous (row stride = row length)")
    if u_mask is not None and sel_ld < 1:
        raise ValueError("u_list rows must hold at least one entry")
    _need_contig_n(sel_count, "sel_count", sel_rows, I32S)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    kb, kh, kn = _rows_view(k, "k")
    if _rows_view(v, "v") != (kb, kh, kn):
        raise ValueError("k and v must share strides")
    hb = hh = hn = host_slots = 0
    if (k_host is None) != (v_host is None):
        raise ValueError("give both host pools or neither")
    if k_host is not None:
        if loc is None:
            raise ValueError("host pools need loc")
        _need_cache(k_host, "k_host", B, Hkv, 0, d, dtypes=(k.dtype,), device=False)
        _need_cache(v_host, "v_host", B, Hkv, 0, d, dtypes=(k.dtype,), device=False)
        hb, hh, hn = _rows_view(k_host, "k_host")
        if _rows_view(v_host, "v_host") != (hb, hh, hn):
            raise ValueError("k_host and v_host must share strides")
        host_slots = min(k_host.shape[2], v_host.shape[2])
    lb = lh = 0
    if loc is not None:
        if k_host is None:
            raise ValueError("loc needs the host pools k_host, v_host")
        _need_dev(loc, "loc", I32S)
        if loc.dim() != 3 or loc.stride(2) != 1:
            raise ValueError("loc must be int32 [B, Hkv, N] with a contiguous last dim")
        _need_shape(loc, "loc", [(">=", B), Hkv, (">=", n_tokens)])
        lb, lh = loc.stride(0), loc.stride(1)
    hbm_slots = min(k.shape[2], v.shape[2])
    if out is None:
        out = torch.empty((B, T, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, T, Hq), dtype=torch.float32, device=q.device)
    _need_contig_n(out, "out", B * T * Hq * d, F32S)
    _need_shape(out, "out", [B, T, Hq, d])
    _need_contig_n(lse, "lse", B * T * Hq, F32S)
    lg_ld = 0
    if logits is not None:
        _need_dev(logits, "logits", F32S)
        bound = (min(n_tokens, sel_ld) if u_mask is not None else
                 fetch_list_bound(sc, T, Hq // Hkv, sel_ld, gran, n_sink, n_recent, n_tokens))
        lg_ld = _row_ld(logits, "logits", B * T * Hq, bound)
    cargs = [_ptr(q), _dt(q), _ptr(k), _ptr(v), _dt(k), kb, kh, kn,
             _ptr(k_host), _ptr(v_host), hb, hh, hn, host_slots, _ptr(loc), lb, lh, hbm_slots,
             _ptr(sel_idx), _ptr(sel_count), sel_ld, sc, gran, n_sink, n_recent,
             B, T, Hq, Hkv, d, n_tokens, float(sm_scale), _ptr(out), _ptr(lse), _ptr(logits), lg_ld]
    return cargs, out, lse, (sc, B, T, Hq, Hkv, d, n_tokens, sel_ld, gran, n_sink, n_recent)


def sparse_decode_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sel_idx: torch.Tensor,
                       sel_count: torch.Tensor, scope, n_tokens: int, gran: int = 1,
                       n_sink: int = 0, n_recent: int = 0, sm_scale: Optional[float] = None,
                       k_host: Optional[torch.Tensor] = None, v_host: Optional[torch.Tensor] = None,
                       loc: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                       ws: Optional[torch.Tensor] = None, stream=None):
    """Exact attention over the selected rows.  q [B,T,Hq,d]; k, v [B,Hkv,*,d] views;
    sel_idx [rows, sel_ld] int32 (rows per `scope`), sel_count [rows] int32.
    Host pools k_host/v_host: pinned [B,Hkv,*,d] views, used where loc [B,Hkv,>=n_tokens] < 0.
    Returns (out fp32 [B,T,Hq,d], lse fp32 [B,T,Hq])."""
    cargs, out, lse, sizes = _attn_call_args(q, k, v, sel_idx, sel_count, scope, n_tokens, gran,
                                             n_sink, n_recent, sm_scale, k_host, v_host, loc, out,
                                             lse, logits)
    wsz = attn_workspace_size(*sizes)
    if ws is None or ws.numel() < wsz:
        ws = torch.zeros(max(wsz, 1), dtype=torch.uint8, device=q.device)
    _need_dev(ws, "ws", U8S)
    st = lib().sparse_decode_attn(*cargs, _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "sparse_decode_attn")
    return out, lse


def noalloc_max_bytes() -> int:
    """Size of the library's fixed scratch array (the workspace sparse_decode_attn_noalloc
    uses on each GPU)."""
    return int(lib().sparse_decode_attn_noalloc_max_bytes())


def sparse_decode_attn_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                               sel_idx: torch.Tensor, sel_count: torch.Tensor, scope,
                               n_tokens: int, out: torch.Tensor, lse: torch.Tensor, gran: int = 1,
                               n_sink: int = 0, n_recent: int = 0,
                               sm_scale: Optional[float] = None,
                               k_host: Optional[torch.Tensor] = None,
                               v_host: Optional[torch.Tensor] = None,
                               loc: Optional[torch.Tensor] = None,
                               logits: Optional[torch.Tensor] = None, stream=None):
    """sparse_decode_attn with no workspace argument: the library's fixed scratch array serves
    as the workspace and nothing is allocated (the caller passes out and lse).  Calls that
    overlap in time on one GPU race."""
    if out is None or lse is None:
        raise ValueError("sparse_decode_attn_noalloc: pass out and lse (it allocates nothing)")
    cargs, out, lse, _ = _attn_call_args(q, k, v, sel_idx, sel_count, scope, n_tokens, gran,
                                         n_sink, n_recent, sm_scale, k_host, v_host, loc, out,
                                         lse, logits)
    st = lib().sparse_decode_attn_noalloc(*cargs, _stream(stream))
    _check(st, "sparse_decode_attn_noalloc")
    return out, lse


def attn_union_workspace_size(scope, B, T, Hq, Hkv, d, n_tokens, u_ld) -> int:
    sc = SCOPES[scope] if isinstance(scope, str) else int(scope)
    out = SZ(0)
    _check(lib().sparse_decode_attn_union_workspace_size(sc, B, T, Hq, Hkv, d, n_tokens, u_ld,
                                                         ctypes.byref(out)),
           "sparse_decode_attn_union_workspace_size")
    return out.value


def sparse_decode_attn_union(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                             u_list: torch.Tensor, u_mask: torch.Tensor, u_count: torch.Tensor,
                             scope, n_tokens: int, sm_scale: Optional[float] = None,
                             k_host: Optional[torch.Tensor] = None,
                             v_host: Optional[torch.Tensor] = None,
                             loc: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                             lse: Optional[torch.Tensor] = None,
                             logits: Optional[torch.Tensor] = None,
                             ws: Optional[torch.Tensor] = None, stream=None):
    """Exact attention over fetch lists already assembled (topk_select_union's union):
    u_list / u_mask int32 [B*Hkv, u_ld], u_count int32 [B*Hkv].  Other arguments as
    sparse_decode_attn.  Returns (out fp32 [B,T,Hq,d], lse fp32 [B,T,Hq])."""
    sc = SCOPES[scope] if isinstance(scope, str) else int(scope)
    if sc not in (SEL_PER_Q_HEAD, SEL_PER_KV_HEAD):
        raise ValueError("sparse_decode_attn_union: scope must be per_q_head or per_kv_head")
    cargs, out, lse, sizes = _attn_call_args(q, k, v, u_list, u_count, sc, n_tokens, 1, 0, 0,
                                             sm_scale, k_host, v_host, loc, out, lse, logits,
                                             u_mask=u_mask)
    sc_, B, T, Hq, Hkv, d, n, u_ld = sizes[:8]
    wsz = attn_union_workspace_size(sc, B, T, Hq, Hkv, d, n, u_ld)
    if ws is None or ws.numel() < wsz:
        ws = torch.empty(max(wsz, 1), dtype=torch.uint8, device=q.device)
    _need_dev(ws, "ws", U8S)
    # C argument order of the union call: the selection arguments are (list, mask, count, ld)
    head, tail = cargs[:18], cargs[25:]
    st = lib().sparse_decode_attn_union(*head, _ptr(u_list), _ptr(u_mask), _ptr(u_count), u_ld, sc,
                                        *tail, _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "sparse_decode_attn_union")
    return out, lse


# ----------------------------------------------------------------------------- importance / tiers

def importance_accumulate(s: torch.Tensor, sel_idx: torch.Tensor, sel_count: torch.Tensor,
                          logits: torch.Tensor, lse: torch.Tensor, n_tokens: int, stream=None):
    """s [B, s_ld] fp32 updated in place; sel_idx [B, sel_ld]; logits [L, B, Hq, logits_ld]
    (or [L, B, 1, Hq, logits_ld]); lse [L, B, Hq] (or [L, B, 1, Hq])."""
    _need_dev(s, "s", F32S)
    if s.dim() != 2 or n_tokens < 0:
        raise ValueError("s must be [B, >= n_tokens] and n_tokens >= 0")
    B = s.shape[0]
    s_ld = _row_ld(s, "s", B, n_tokens)
    _need_dev(sel_idx, "sel_idx", I32S)
    _contig(sel_idx, "sel_idx")
    _need_shape(sel_idx, "sel_idx", [B, None])
    sel_ld = sel_idx.shape[-1]
    _need_contig_n(sel_count, "sel_count", B, I32S)
    _need_dev(logits, "logits", F32S)
    if logits.dim() not in (4, 5) or (logits.dim() == 5 and logits.shape[2] != 1):
        raise ValueError("logits must be [L, B, Hq, ld] or [L, B, 1, Hq, ld]")
    L = logits.shape[0]
    Hq = logits.shape[-2]
    if logits.shape[1] != B:
        raise ValueError(f"logits batch {logits.shape[1]} != {B}")
    lg_ld = _row_ld(logits, "logits", L * B * Hq, sel_ld)
    _need_contig_n(lse, "lse", L * B * Hq, F32S)
    st = lib().importance_accumulate(_ptr(s), s_ld, B, n_tokens, _ptr(sel_idx),
                                     _ptr(sel_count), sel_ld, _ptr(logits), lg_ld, _ptr(lse), L, Hq,
                                     _stream(stream))
    _check(st, "importance_accumulate")
    return s


def tier_classify(s: torch.Tensor, n_tokens: int, n_sink: int, n_recent: int,
                  t0_permille: int = 250, t01_permille: int = 750,
                  evicted: Optional[torch.Tensor] = None, tier: Optional[torch.Tensor] = None,
                  sel_idx: Optional[torch.Tensor] = None, sel_count: Optional[torch.Tensor] = None,
                  stream=None, t012_permille: Optional[int] = None):
    """Tiers of each sequence's tokens.  s [B, s_ld] fp32.  Returns (tier uint8 [B, n_tokens],
    sel_idx int32 [B, n_tokens] (T0 ∪ T1 ∪ T2 ascending), sel_count int32 [B]).
    t012_permille None: no T2 (the T2 quota equals t01_permille)."""
    if t012_permille is None:
        t012_permille = t01_permille
    _need_dev(s, "s", F32S)
    if s.dim() != 2 or n_tokens < 0:
        raise ValueError("s must be [B, >= n_tokens] and n_tokens >= 0")
    B = s.shape[0]
    dev = s.device
    s_ld = _row_ld(s, "s", B, n_tokens)
    if tier is None:
        tier = torch.empty((B, n_tokens), dtype=torch.uint8, device=dev)
    if sel_idx is None:
        sel_idx = torch.empty((B, max(n_tokens, 1)), dtype=torch.int32, device=dev)
    if sel_count is None:
        sel_count = torch.empty((B,), dtype=torch.int32, device=dev)
    _need_dev(tier, "tier", U8S)
    t_ld = _row_ld(tier, "tier", B, n_tokens)
    ev_ld = 0
    if evicted is not None:
        _need_dev(evicted, "evicted", U8S)
        ev_ld = _row_ld(evicted, "evicted", B, n_tokens)
    _need_dev(sel_idx, "sel_idx", I32S)
    sl = _row_ld(sel_idx, "sel_idx", B, n_tokens)
    _need_contig_n(sel_count, "sel_count", B, I32S)
    st = lib().tier_classify(_ptr(s), s_ld, B, n_tokens, n_sink, n_recent, t0_permille,
                             t01_permille, t012_permille, _ptr(evicted), ev_ld, _ptr(tier), t_ld,
                             _ptr(sel_idx),
                             _ptr(sel_count), sl, None, 0, _stream(stream))
    _check(st, "tier_classify")
    return tier, sel_idx, sel_count


def set_attn_timing_events(begin: Optional[torch.cuda.Event] = None,
                           end: Optional[torch.cuda.Event] = None):
    """Bracket the gather kernel of every following sparse_decode_attn call with two recorded
    events (a measurement hook); call with no arguments to switch it off.  The events must have
    been created with enable_timing=True and recorded once (torch creates them lazily)."""
    if (begin is None) != (end is None):
        raise ValueError("give both events or neither")
    b = None if begin is None else ctypes.c_void_p(begin.cuda_event)
    e = None if end is None else ctypes.c_void_p(end.cuda_event)
    if begin is not None and (not b.value or not e.value):
        raise ValueError("record the events once before handing them over")
    _check(lib().spk_set_attn_timing_events(b, e), "spk_set_attn_timing_events")


def stream_read(buf: torch.Tensor, workgroups: int, sink: torch.Tensor, stream=None):
    """Measurement reference: a plain streaming read of the whole device tensor ``buf`` split
    into ``workgroups`` chunks (``sink``: one int32 device element, written practically never)."""
    _contig(buf, "buf")
    if not buf.is_cuda or not sink.is_cuda:
        raise ValueError("stream_read: buf and sink must be device tensors")
    _check(lib().spk_stream_read(_ptr(buf), buf.numel() * buf.element_size(), int(workgroups),
                                 _ptr(sink), _stream(stream)), "spk_stream_read")


def stream_read_host(buf: torch.Tensor, workgroups: int, sink: torch.Tensor, stream=None):
    """Measurement reference: a plain streaming read of the whole pinned host tensor ``buf``
    over the host link, split into ``workgroups`` chunks (``sink`` as in stream_read)."""
    _contig(buf, "buf")
    if not _is_pinned(buf) or not sink.is_cuda:
        raise ValueError("stream_read_host: buf must be a pinned host tensor, sink a device tensor")
    _check(lib().spk_stream_read_host(_ptr(buf), buf.numel() * buf.element_size(),
                                      int(workgroups), _ptr(sink), _stream(stream)),
           "spk_stream_read_host")


def gather_read(k: torch.Tensor, v: torch.Tensor, rows: torch.Tensor, wg_per_group: int,
                sink: torch.Tensor, stream=None):
    """Measurement reference: reads the K and V rows each group's list names (``rows`` int32
    [groups, rows_ld], entries < 0 skipped), once each, for caches ``k``, ``v``
    [B, Hkv, N, d] (or [groups, N, d]) views sharing strides, with ``wg_per_group``
    workgroups per group (``sink`` as in stream_read)."""
    if not (k.is_cuda and v.is_cuda and rows.is_cuda and sink.is_cuda):
        raise ValueError("gather_read: device tensors expected")
    if k.dim() == 4:
        if k.stride(0) != k.shape[1] * k.stride(1) or v.stride() != k.stride():
            raise ValueError("gather_read: k and v must share strides, groups evenly spaced")
        groups, sg, sn = k.shape[0] * k.shape[1], k.stride(1), k.stride(2)
    elif k.dim() == 3 and v.stride() == k.stride():
        groups, sg, sn = k.shape[0], k.stride(0), k.stride(1)
    else:
        raise ValueError("gather_read: k, v must be [B, H, N, d] or [groups, N, d] views")
    if k.stride(-1) != 1 or rows.dim() != 2 or rows.shape[0] != groups or rows.dtype != torch.int32:
        raise ValueError("gather_read: contiguous rows of k/v and an int32 [groups, ld] list")
    _contig(rows, "rows")
    e = k.element_size()
    _check(lib().spk_gather_read(_ptr(k), _ptr(v), k.shape[-1] * e, sg * e, sn * e, k.shape[-2],
                                 _ptr(rows), rows.shape[1], groups, int(wg_per_group), _ptr(sink),
                                 _stream(stream)), "spk_gather_read")


def topk_attn_workspace_size(B, Hq, Hkv, d, n_tokens, n_cand, k, gran=1, n_sink=0,
                             n_recent=0) -> int:
    out = SZ(0)
    _check(lib().sparse_topk_decode_attn_workspace_size(B, Hq, Hkv, d, n_tokens, n_cand, k, gran,
                                                        n_sink, n_recent, ctypes.byref(out)),
           "sparse_topk_decode_attn_workspace_size")
    return out.value


def sparse_topk_decode_attn(scores: torch.Tensor, k: int, q: torch.Tensor, kc: torch.Tensor,
                            vc: torch.Tensor, n_tokens: int, gran: int = 1, n_sink: int = 0,
                            n_recent: int = 0, sm_scale: Optional[float] = None,
                            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                            sel_idx: Optional[torch.Tensor] = None,
                            sel_count: Optional[torch.Tensor] = None,
                            ws: Optional[torch.Tensor] = None, stream=None):
    """Top-k of each (b, kvh) score row and exact attention over the selection, one launch.
    scores [B, 1, Hkv, >=n_cand] fp32 (n_cand = scores.shape[-1]); q [B, 1, Hq, d] bf16.
    Returns (out fp32 [B,1,Hq,d], lse fp32 [B,1,Hq])."""
    _need_dev(q, "q", KVS)
    _contig(q, "q")
    if q.dim() != 4 or kc.dim() != 4 or vc.dim() != 4:
        raise ValueError("q must be [B, 1, Hq, d] and k, v [B, Hkv, N, d] views")
    B, T, Hq, d = q.shape
    if T != 1:
        raise ValueError("one query token per sequence")
    Hkv = kc.shape[1]
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq = {Hq} is not a multiple of Hkv = {Hkv}")
    if n_tokens < 0 or gran < 1 or n_sink < 0 or n_recent < 0:
        raise ValueError("negative n_tokens, n_sink, n_recent or gran < 1")
    _need_dev(scores, "scores", F32S)
    n_cand = scores.shape[-1]
    s_ld = _row_ld(scores, "scores", B * Hkv, n_cand)
    _need_cache(kc, "k", B, Hkv, n_tokens, d)
    _need_cache(vc, "v", B, Hkv, n_tokens, d, dtypes=(kc.dtype,))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    kb, kh, kn = _rows_view(kc, "k")
    if _rows_view(vc, "v") != (kb, kh, kn):
        raise ValueError("k and v must share strides")
    if out is None:
        out = torch.empty((B, 1, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, 1, Hq), dtype=torch.float32, device=q.device)
    _need_contig_n(out, "out", B * Hq * d, F32S)
    _need_contig_n(lse, "lse", B * Hq, F32S)
    if (sel_idx is None) != (sel_count is None):
        raise ValueError("give sel_idx and sel_count together")
    sl = 0
    if sel_idx is not None:
        _need_dev(sel_idx, "sel_idx", I32S)
        sl = _row_ld(sel_idx, "sel_idx", B * Hkv, max(0, min(k, n_cand)))
        _need_contig_n(sel_count, "sel_count", B * Hkv, I32S)
    wsz = topk_attn_workspace_size(B, Hq, Hkv, d, n_tokens, n_cand, k, gran, n_sink, n_recent)
    if ws is None or ws.numel() < wsz:
        ws = torch.zeros(max(wsz, 1), dtype=torch.uint8, device=q.device)
    _need_dev(ws, "ws", U8S)
    st = lib().sparse_topk_decode_attn(_ptr(scores), s_ld, n_cand, k, _ptr(q), _dt(q),
                                       _ptr(kc), _ptr(vc), _dt(kc), kb, kh, kn, gran, n_sink,
                                       n_recent, B, Hq, Hkv, d, n_tokens, float(sm_scale),
                                       _ptr(out), _ptr(lse), _ptr(sel_idx), _ptr(sel_count), sl,
                                       _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "sparse_topk_decode_attn")
    return out, lse


def lookahead_prefetch(sel_idx: torch.Tensor, sel_count: torch.Tensor, block_size: int,
                       n_tokens: int, k_host: torch.Tensor, v_host: torch.Tensor, k: torch.Tensor,
                       v: torch.Tensor, stage_base: int, loc_home: torch.Tensor,
                       loc: torch.Tensor, staged: torch.Tensor, staged_count: torch.Tensor,
                       workgroups: Optional[int] = None, stream=None):
    """Copy the host-resident rows of the selected blocks (sel_idx [B, 1, Hkv, sel_ld] block ids,
    sel_count [B, 1, Hkv]) into the staging rows [stage_base, stage_base + sel_ld*block_size) of
    the HBM caches k, v [B, Hkv, C, d], pointing loc [B, Hkv, >=n_tokens] there; the rows the
    previous call redirected go back to loc_home first.  staged int32 [B*Hkv, sel_ld*block_size],
    staged_count int32 [B*Hkv] (zero before the first call): the compact list of the tokens the
    last call redirected, for the next call with the same sel_ld and block_size.  A persistent
    kernel of ``workgroups`` workgroups (default one per (b, kvh) group)."""
    if k.dim() != 4:
        raise ValueError("k must be a [B, Hkv, C, d] view")
    B, Hkv, C, d = k.shape
    _need_cache(k, "k", B, Hkv, 0, d)
    _need_cache(v, "v", B, Hkv, 0, d, dtypes=(k.dtype,))
    _need_cache(k_host, "k_host", B, Hkv, 0, d, dtypes=(k.dtype,), device=False)
    _need_cache(v_host, "v_host", B, Hkv, 0, d, dtypes=(k.dtype,), device=False)
    _need_dev(sel_idx, "sel_idx", I32S)
    sel_ld = _row_ld(sel_idx, "sel_idx", B * Hkv, 0)
    if B * Hkv > 1 and sel_ld != sel_idx.shape[-1]:
        raise ValueError("sel_idx rows must be contiguous")
    sel_ld = sel_idx.shape[-1]
    _need_contig_n(sel_count, "sel_count", B * Hkv, I32S)
    for t, nm in ((loc_home, "loc_home"), (loc, "loc")):
        _need_dev(t, nm, I32S)
        if t.dim() != 3 or t.stride(2) != 1:
            raise ValueError(f"{nm} must be int32 [B, Hkv, N] with a contiguous last dim")
        _need_shape(t, nm, [(">=", B), Hkv, (">=", n_tokens)])
    if loc.stride() != loc_home.stride():
        raise ValueError("loc and loc_home must share strides")
    _need_contig_n(staged, "staged", B * Hkv * sel_ld * block_size, I32S)
    _need_contig_n(staged_count, "staged_count", B * Hkv, I32S)
    if not (n_tokens <= stage_base and stage_base + sel_ld * block_size <= C):
        raise ValueError(f"staging rows [{stage_base}, {stage_base + sel_ld * block_size}) must lie "
                         f"past the {n_tokens} tokens and inside the {C} HBM rows")
    hb, hh, hn = _rows_view(k_host, "k_host")
    if _rows_view(v_host, "v_host") != (hb, hh, hn):
        raise ValueError("k_host and v_host must share strides")
    kb, kh, kn = _rows_view(k, "k")
    if _rows_view(v, "v") != (kb, kh, kn):
        raise ValueError("k and v must share strides")
    st = lib().lookahead_prefetch(_ptr(sel_idx), _ptr(sel_count), sel_ld, block_size, B, Hkv, d,
                                  _dt(k), n_tokens, _ptr(k_host), _ptr(v_host), hb, hh, hn,
                                  min(k_host.shape[2], v_host.shape[2]), _ptr(k), _ptr(v), kb, kh,
                                  kn, min(k.shape[2], v.shape[2]), stage_base, _ptr(loc_home),
                                  _ptr(loc), loc.stride(0), loc.stride(1), _ptr(staged),
                                  _ptr(staged_count),
                                  int(B * Hkv if workgroups is None else workgroups),
                                  _stream(stream))
    _check(st, "lookahead_prefetch")


# ----------------------------------------------------------------------------- residency

TIERS_T0_T1 = 0xF4   # residency classes: T0 ranked first, T1 second, T2 and T3 never resident
TIERS_T2 = 0xCF      # every T2 row resident (the staging of the 8-bit tier)


def residency_update(tier: torch.Tensor, s: torch.Tensor, n_tokens: int, capacity: int,
                     loc: torch.Tensor, copy_tok: torch.Tensor, copy_slot: torch.Tensor,
                     copy_count: torch.Tensor, stream=None, tier_classes: int = TIERS_T0_T1):
    """HBM slots after a tier reassignment (loc updated in place) and the rows to copy.
    tier uint8 [B,*], s fp32 [B,*], loc int32 [B,*]; copy_tok/copy_slot int32 [B,copy_ld],
    copy_count int32 [B].  tier_classes: the tiers' roles (2 bits per tier code; the default
    ranks T0 then T1, TIERS_T2 stages every T2 row)."""
    B = tier.shape[0]
    for t, nm, dts in ((tier, "tier", U8S), (s, "s", F32S), (loc, "loc", I32S),
                       (copy_tok, "copy_tok", I32S), (copy_slot, "copy_slot", I32S),
                       (copy_count, "copy_count", I32S)):
        _need_dev(t, nm, dts)
        _contig(t, nm)
    if n_tokens < 0 or capacity < 0:
        raise ValueError("n_tokens and capacity must be >= 0")
    for t, nm in ((tier, "tier"), (s, "s"), (loc, "loc")):
        _need_shape(t, nm, [B, (">=", n_tokens)])
    for t, nm in ((copy_tok, "copy_tok"), (copy_slot, "copy_slot")):
        _need_shape(t, nm, [B, (">=", min(capacity, n_tokens))])
    if copy_slot.shape != copy_tok.shape:
        raise ValueError("copy_tok and copy_slot must have one shape")
    _need_contig_n(copy_count, "copy_count", B, I32S)
    st = lib().residency_update_tiers(_ptr(tier), tier.shape[1], _ptr(s), s.shape[1], B,
                                      n_tokens, capacity, int(tier_classes), _ptr(loc),
                                      loc.shape[1], _ptr(copy_tok), _ptr(copy_slot),
                                      copy_tok.shape[1], _ptr(copy_count), _stream(stream))
    _check(st, "residency_update")


def residency_append(loc: torch.Tensor, n_old: int, n_new: int, capacity: int,
                     copy_tok: torch.Tensor, copy_slot: torch.Tensor, copy_count: torch.Tensor,
                     stream=None):
    """HBM slots for the rows [n_old, n_new) of every sequence (loc int32 [B, >= n_new] updated
    in place): the free slots, lowest first, in token order; the rows given one are listed in
    copy_tok / copy_slot int32 [B, >= min(n_new - n_old, capacity)], their number in
    copy_count int32 [B]."""
    for t, nm in ((loc, "loc"), (copy_tok, "copy_tok"), (copy_slot, "copy_slot")):
        _need_dev(t, nm, I32S)
        _contig(t, nm)
    B = loc.shape[0]
    if not 0 <= n_old <= n_new or capacity < 0:
        raise ValueError("need 0 <= n_old <= n_new and capacity >= 0")
    _need_shape(loc, "loc", [B, (">=", n_new)])
    listed = min(n_new - n_old, capacity)
    for t, nm in ((copy_tok, "copy_tok"), (copy_slot, "copy_slot")):
        _need_shape(t, nm, [B, (">=", listed)])
    if copy_slot.shape != copy_tok.shape:
        raise ValueError("copy_tok and copy_slot must have one shape")
    _need_contig_n(copy_count, "copy_count", B, I32S)
    st = lib().residency_append(_ptr(loc), loc.shape[1], B, n_old, n_new, capacity,
                                _ptr(copy_tok), _ptr(copy_slot), copy_tok.shape[1],
                                _ptr(copy_count), _stream(stream))
    _check(st, "residency_append")


def residency_prefetch(k_host: torch.Tensor, v_host: torch.Tensor, k_hbm: torch.Tensor,
                       v_hbm: torch.Tensor, copy_tok: torch.Tensor, copy_slot: torch.Tensor,
                       copy_count: torch.Tensor, max_copies: int, stream=None):
    """Copy the listed rows of the source pools [B,Hkv,Nh,d] (pinned host memory, or device
    memory holding rows produced on the GPU) into their slots of the HBM pools [B,Hkv,C,d]
    (one layer, every KV head)."""
    if k_hbm.dim() != 4:
        raise ValueError("k_hbm must be a [B, Hkv, C, d] view")
    B, Hkv, _, d = k_hbm.shape
    _need_cache(k_hbm, "k_hbm", B, Hkv, 0, d)
    _need_cache(v_hbm, "v_hbm", B, Hkv, 0, d, dtypes=(k_hbm.dtype,))
    for t, nm in ((k_host, "k_host"), (v_host, "v_host")):
        _dev_or_pinned(t, nm, (k_hbm.dtype,))
        _need_cache(t, nm, B, Hkv, 0, d, dtypes=(k_hbm.dtype,), device=_is_dev(t))
    for t, nm in ((copy_tok, "copy_tok"), (copy_slot, "copy_slot")):
        _need_dev(t, nm, I32S)
        _contig(t, nm)
        _need_shape(t, nm, [B, (">=", max_copies)])
    _need_contig_n(copy_count, "copy_count", B, I32S)
    hsb, hsh, hsn = _rows_view(k_host, "k_host")
    dsb, dsh, dsn = _rows_view(k_hbm, "k_hbm")
    if _rows_view(v_host, "v_host") != (hsb, hsh, hsn) or _rows_view(v_hbm, "v_hbm") != (dsb, dsh, dsn):
        raise ValueError("k and v pools must share their strides")
    st = lib().residency_prefetch(_ptr(k_host), _ptr(v_host), hsb, hsh, hsn, k_host.shape[2],
                                  _ptr(k_hbm), _ptr(v_hbm), dsb, dsh, dsn, k_hbm.shape[2],
                                  _dt(k_hbm), B, Hkv, d, _ptr(copy_tok), _ptr(copy_slot),
                                  copy_tok.shape[1], _ptr(copy_count), max_copies, _stream(stream))
    _check(st, "residency_prefetch")


# ----------------------------------------------------------------------------- T2 (8-bit tier)

def _dev_or_pinned(t, name: str, dtypes):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if not (_is_dev(t) or _is_pinned(t)):
        raise ValueError(f"{name} must be a device tensor or pinned host memory")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)} (got {t.dtype})")
    return t


def _codes_view(codes: torch.Tensor, scales: torch.Tensor, name: str, B: int, Hkv: int,
                n_min: int, d: int):
    _dev_or_pinned(codes, f"{name} codes", (torch.int8,))
    _dev_or_pinned(scales, f"{name} scales", F32S)
    _need_shape(codes, f"{name} codes", [(">=", B), Hkv, (">=", n_min), d])
    _need_shape(scales, f"{name} scales", [(">=", B), Hkv, (">=", n_min)])
    if codes.stride(3) != 1 or scales.stride(2) != 1:
        raise ValueError(f"{name}: codes and scales need a contiguous last dim")
    if min(codes.shape[2], scales.shape[2]) < n_min:
        raise ValueError(f"{name}: fewer than {n_min} rows")
    return codes.stride(0), codes.stride(1), codes.stride(2), scales.stride(0), scales.stride(1)


def kv_quantize_int8(src: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                     row_begin: int = 0, row_end: Optional[int] = None, stream=None):
    """8-bit codes and fp32 scales of the rows [row_begin, row_end) of a K or V cache view
    src [B, Hkv, N, d] (bf16 or fp32; device or pinned host) into codes int8 [B, Hkv, >=N, d]
    and scales fp32 [B, Hkv, >=N] (device or pinned host)."""
    _dev_or_pinned(src, "src", KVS)
    sb, sh, sn = _rows_view(src, "src")
    B, Hkv, N, d = src.shape
    row_end = N if row_end is None else row_end
    if not 0 <= row_begin <= row_end <= N:
        raise ValueError(f"rows [{row_begin}, {row_end}) outside the {N} rows of src")
    csb, csh, csn, ssb, ssh = _codes_view(codes, scales, "kv_quantize_int8", B, Hkv, row_end, d)
    st = lib().kv_quantize_int8(_ptr(src), _dt(src), sb, sh, sn, B, Hkv, d, row_begin, row_end,
                                _ptr(codes), csb, csh, csn, _ptr(scales), ssb, ssh,
                                _stream(stream))
    _check(st, "kv_quantize_int8")


def t2_fetch(codes_k: torch.Tensor, codes_v: torch.Tensor, scale_k: torch.Tensor,
             scale_v: torch.Tensor, k: torch.Tensor, v: torch.Tensor, stage_base: int,
             copy_tok: torch.Tensor, copy_slot: torch.Tensor, copy_count: torch.Tensor,
             max_copies: int, stream=None):
    """Rows copy_tok[b, r] of the 8-bit pools, dequantized to bf16 into rows
    stage_base + copy_slot[b, r] of the HBM pools k, v [B, Hkv, C, d] (one layer, every KV
    head), r < min(copy_count[b], max_copies)."""
    if k.dim() != 4:
        raise ValueError("k must be a [B, Hkv, C, d] view")
    B, Hkv, C, d = k.shape
    _need_cache(k, "k", B, Hkv, 0, d, dtypes=(torch.bfloat16,))
    _need_cache(v, "v", B, Hkv, 0, d, dtypes=(torch.bfloat16,))
    kb, kh, kn = _rows_view(k, "k")
    if _rows_view(v, "v") != (kb, kh, kn) or v.shape[2] != C:
        raise ValueError("k and v must share shape and strides")
    g = _codes_view(codes_k, scale_k, "t2_fetch K", B, Hkv, 0, d)
    if _codes_view(codes_v, scale_v, "t2_fetch V", B, Hkv, 0, d) != g:
        raise ValueError("the K and V code pools must share strides")
    rows = min(codes_k.shape[2], codes_v.shape[2], scale_k.shape[2], scale_v.shape[2])
    for t, nm in ((copy_tok, "copy_tok"), (copy_slot, "copy_slot")):
        _need_dev(t, nm, I32S)
        _contig(t, nm)
        _need_shape(t, nm, [B, (">=", max_copies)])
    if copy_slot.shape != copy_tok.shape:
        raise ValueError("copy_tok and copy_slot must have one shape")
    _need_contig_n(copy_count, "copy_count", B, I32S)
    if stage_base < 0:
        raise ValueError("stage_base must be >= 0")
    st = lib().t2_fetch(_ptr(codes_k), _ptr(codes_v), g[0], g[1], g[2], _ptr(scale_k),
                        _ptr(scale_v), g[3], g[4], rows, _ptr(k), _ptr(v), _dt(k), kb, kh, kn, C,
                        stage_base, B, Hkv, d, _ptr(copy_tok), _ptr(copy_slot), copy_tok.shape[1],
                        _ptr(copy_count), max_copies, _stream(stream))
    _check(st, "t2_fetch")


def t2_locations(tier: torch.Tensor, loc_res: torch.Tensor, loc_t2: torch.Tensor,
                 loc_out: torch.Tensor, n_tokens: int, stage_base: int, stream=None):
    """loc_out = stage_base + loc_t2 for T2 rows holding a staging slot, else loc_res; every
    array [B, >= n_tokens] on the device (tier uint8, the locations int32)."""
    B = tier.shape[0]
    for t, nm, dts in ((tier, "tier", U8S), (loc_res, "loc_res", I32S), (loc_t2, "loc_t2", I32S),
                       (loc_out, "loc_out", I32S)):
        _need_dev(t, nm, dts)
        _contig(t, nm)
        _need_shape(t, nm, [B, (">=", n_tokens)])
    st = lib().t2_locations(_ptr(tier), tier.shape[1], _ptr(loc_res), loc_res.shape[1],
                            _ptr(loc_t2), loc_t2.shape[1], _ptr(loc_out), loc_out.shape[1], B,
                            n_tokens, stage_base, _stream(stream))
    _check(st, "t2_locations")
