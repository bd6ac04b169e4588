"""Per-group definitions of the sparse decode path, in fp64 NumPy (test infrastructure only).

Conventions: a "group" is one (batch, KV head) pair.  Keys and values of a group
are ``[n, d]`` arrays; query vectors are ``[m, d]``.  All arithmetic is fp64 on
the exact values of the (fp32 or bf16) inputs.
"""
from __future__ import annotations

import math

import numpy as np


# --------------------------------------------------------------------------- inputs

def decode_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values: a bf16 is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def encode_bf16(x) -> np.ndarray:
    """fp32 values -> bf16 bit patterns (uint16): round to nearest, ties to even (the low 16
    bits decide, with the kept part's last bit breaking ties); a NaN stays a quiet NaN."""
    xf = np.asarray(x, dtype=np.float32)
    u = xf.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    r = np.where(np.isnan(xf), ((u >> np.uint64(16)) | np.uint64(0x40)) & np.uint64(0xFFFF), r)
    return r.astype(np.uint16)


def to_f64(x) -> np.ndarray:
    """Exact fp64 copy of a float array, or of bf16 bit patterns given as uint16."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return decode_bf16(x)
    return x.astype(np.float64)


# --------------------------------------------------------------------------- a0 / a1

def block_pool(keys, block_size: int) -> np.ndarray:
    """Mean of the keys of each complete block of ``block_size`` consecutive tokens.

    SparDA, "Estratégia de Treinamento": the indexer scores keys compressed on a
    block grid.  Reading taken: non-overlapping windows (kernel = stride =
    block_size), mean pooling, only complete blocks.  Returns ``[n // bs, d]``.
    """
    k = to_f64(keys)
    nb = k.shape[0] // block_size
    return k[: nb * block_size].reshape(nb, block_size, k.shape[1]).mean(axis=1)


def scores_token_group_mean(q_group, keys) -> np.ndarray:
    """Token score of one GQA group: the mean over the group's query heads of q_h·k_j.

    SparDA §2 "Indexador de Previsão Compacto": one score per GQA group instead of
    a scoring loop per query head, and no softmax.  ``q_group`` is ``[G, d]``,
    ``keys`` ``[n, d]``; returns ``[n]``.  Unscaled dot products.
    """
    q = to_f64(q_group)
    k = to_f64(keys)
    per_head = k @ q.T                      # [n, G]
    return per_head.mean(axis=1)


def scores_token_per_head(q_group, keys) -> np.ndarray:
    """Per-query-head token scores q_h·k_j, ``[G, n]``.

    "Esparsidade de Contexto ...", §2 "Oracle Top-K": exact scores of every token,
    selected independently per query head (per-head sparsity patterns).
    """
    q = to_f64(q_group)
    k = to_f64(keys)
    return q @ k.T


def scores_block(pred, kpool) -> np.ndarray:
    """Block scores p·Kpool_j of one predictor vector (no softmax), ``[nb]``.

    SparDA §2 "Indexador de Previsão Compacto" (one predictor head per GQA group)
    and "Seleção Esparsa de Lookahead Treinável" (the predictor ranks KV blocks).
    """
    return to_f64(kpool) @ to_f64(pred)


def window_count(n_tokens: int, window: int, stride: int) -> int:
    """Number of complete compression windows [stride*w, stride*w + window) inside n tokens."""
    return 0 if n_tokens < window else (n_tokens - window) // stride + 1


def window_pool(keys, window: int, stride: int) -> np.ndarray:
    """Mean of the keys of every complete compression window.

    SparDA, "Estratégia de Treinamento": at inference the keys are compressed with
    overlapping windows of kernel 32 and stride 16.  Window w covers tokens
    [stride*w, stride*w + window); only complete windows exist.  Returns ``[nw, d]``.
    """
    k = to_f64(keys)
    nw = window_count(k.shape[0], window, stride)
    out = np.empty((nw, k.shape[1]))
    for w in range(nw):
        out[w] = k[stride * w: stride * w + window].mean(axis=0)
    return out


def scores_block_windowed(pred, kwin, n_tokens: int, window: int, stride: int,
                          block_size: int) -> np.ndarray:
    """Block scores on the selection grid from scores on the compression grid.

    SparDA, "Estratégia de Treinamento": scores on one window grid are max-pooled onto
    another grid.  Reading taken for the block indexer: the predictor scores every
    complete compression window (p·Kwin_w, no softmax), and the score of block j
    (tokens [bs*j, bs*j + bs), complete blocks only) is the largest score among the
    windows that share at least one token with the block; -inf if there is none.
    Returns ``[n_tokens // block_size]``.
    """
    ws = to_f64(kwin) @ to_f64(pred)
    nw = ws.shape[0]
    nb = n_tokens // block_size
    out = np.full(nb, -np.inf)
    for j in range(nb):
        lo_tok, hi_tok = block_size * j, block_size * j + block_size     # [lo, hi)
        for w in range(nw):
            if stride * w < hi_tok and stride * w + window > lo_tok:
                out[j] = max(out[j], ws[w])
    return out


# --------------------------------------------------------------------------- a2

def topk(x, k: int) -> np.ndarray:
    """Exact top-k of a score row: the k largest scores, ties to the lowest index.

    "Esparsidade de Contexto ...", §2 "Oracle Top-K" (exact top-k); the tie rule
    and the ascending output order are this library's definition.  A stable sort
    of -x keeps equal scores in index order; -0 and +0 compare equal; NaN sorts
    after every number (NumPy puts NaN last).  k > n returns all n; k <= 0 none.
    Returns the chosen indices in ascending order (int64).
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    k = max(0, min(int(k), n))
    order = np.argsort(-x, kind="stable")
    return np.sort(order[:k])


# --------------------------------------------------------------------------- a3

def selection_tokens(sel, granularity: int, n_tokens: int, n_sink: int = 0,
                     n_recent: int = 0) -> np.ndarray:
    """Token ids one selection row makes an attention query read, ascending and unique.

    SparDA: selected blocks expand to their tokens; "Nem Todos os Pensamentos ...",
    §1: attention sinks and the recent window are always kept.  Reading taken: the
    union of the expanded selection with the first ``n_sink`` and the last
    ``n_recent`` tokens, deduplicated.  Entries outside [0, n_tokens) are dropped.
    """
    toks = set()
    for s in np.asarray(sel, dtype=np.int64).ravel():
        for t in range(int(s) * granularity, int(s) * granularity + granularity):
            if 0 <= t < n_tokens:
                toks.add(t)
    toks.update(range(0, min(n_sink, n_tokens)))
    toks.update(range(max(0, n_tokens - n_recent), n_tokens))
    return np.array(sorted(toks), dtype=np.int64)


# --------------------------------------------------------------------------- a4 / a5

def attend(q_vecs, keys_sel, vals_sel, sm_scale: float):
    """Exact softmax attention of each query vector over the gathered rows only.

    "Esparsidade de Contexto ...", §3C: sparse decoding reads O(k·d) instead of
    O(N·d) and the result is ordinary attention restricted to the selection.
    o = softmax(sm_scale · q·K_Sᵀ) · V_S, computed textbook-style (max-shifted).

    ``q_vecs`` ``[m, d]``; ``keys_sel``/``vals_sel`` ``[r, d]``.  Returns
    (out ``[m, d]``, lse ``[m]`` natural-log sum-exp of the scaled logits,
    logits ``[m, r]`` scaled).  With r = 0 the output is 0 and lse = -inf.
    """
    q = to_f64(q_vecs)
    k = to_f64(keys_sel)
    v = to_f64(vals_sel)
    m = q.shape[0]
    if k.shape[0] == 0:
        return np.zeros((m, v.shape[1])), np.full(m, -np.inf), np.zeros((m, 0))
    logits = sm_scale * (q @ k.T)                       # [m, r]
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    z = e.sum(axis=1, keepdims=True)
    p = e / z
    out = p @ v
    lse = (mx + np.log(z))[:, 0]
    return out, lse, logits


# --------------------------------------------------------------------------- a6

def importance_update(s_prev, alpha) -> np.ndarray:
    """One step of cumulative attention importance.

    "Nem Todos os Pensamentos Necessitam de HBM", §2 "Pontuação de Importância":
    s_i(t) = s_i(t-1) + (1/|L|) Σ_ℓ (1/H) Σ_h α_ℓ,h(t)[i].

    ``s_prev`` ``[n]`` (the fp32 state), ``alpha`` ``[L, H, n]`` attention
    probabilities of this step (0 for rows not attended).  The increment is
    formed in fp64 and the state is stored back as fp32.
    """
    a = np.asarray(alpha, dtype=np.float64)
    L, H = a.shape[0], a.shape[1]
    delta = np.zeros(a.shape[2])
    for l in range(L):
        delta += a[l].sum(axis=0) / H
    delta /= L
    return (np.asarray(s_prev, dtype=np.float64) + delta).astype(np.float32)


# --------------------------------------------------------------------------- a7

def tier_classify(s, n_tokens: int, n_sink: int, n_recent: int, t0_permille: int = 250,
                  t01_permille: int = 750, evicted=None, t012_permille=None):
    """Four-tier classification by cumulative importance.

    "Nem Todos os Pensamentos Necessitam de HBM", §1 "Classificação de Quatro
    Níveis": protected tokens (attention sinks, recent window) and the most
    important tokens stay in T0; middle importance goes to T1 (full precision,
    fetched before attention); low importance may go to T2 (kept at reduced
    precision); only the least important tail goes to T3 (evicted for good).
    Readings taken:

    * protected = tokens [0, n_sink) and [n_tokens - n_recent, n_tokens) -> T0;
    * the M other tokens are ranked by (not evicted first, s descending, index
      ascending); rank < floor(M·t0/1000) -> T0, rank < floor(M·t01/1000) -> T1,
      rank < floor(M·t012/1000) -> T2, every other token -> T3 (t012 = t01, the
      default, uses no T2);
    * an evicted token stays T3 whatever its rank (eviction is permanent).

    Returns (tier ``[n_tokens]`` uint8 with 0/1/2/3, ascending int64 list of the
    attended rows T0 ∪ T1 ∪ T2).
    """
    if t012_permille is None:
        t012_permille = t01_permille
    s = np.asarray(s, dtype=np.float64)[:n_tokens]
    ev = np.zeros(n_tokens, dtype=bool) if evicted is None else \
        np.asarray(evicted, dtype=bool)[:n_tokens]
    prot = np.zeros(n_tokens, dtype=bool)
    prot[: min(n_sink, n_tokens)] = True
    prot[max(0, n_tokens - n_recent):] = True
    tier = np.full(n_tokens, 3, dtype=np.uint8)
    tier[prot] = 0
    cand = np.nonzero(~prot)[0]
    M = cand.shape[0]
    n0 = (M * t0_permille) // 1000
    n01 = (M * t01_permille) // 1000
    n012 = (M * t012_permille) // 1000
    # sort key: live before evicted, then larger s, then lower index.  A NaN score
    # ranks with the evicted rows (after every number), by index.
    def key(i):
        last = bool(ev[i]) or bool(np.isnan(s[i]))
        return (last, 0.0 if last else -s[i], i)
    order = sorted(cand.tolist(), key=key)
    for r, i in enumerate(order):
        if ev[i]:
            continue
        if r < n0:
            tier[i] = 0
        elif r < n01:
            tier[i] = 1
        elif r < n012:
            tier[i] = 2
    lst = np.nonzero(tier <= 2)[0].astype(np.int64)
    return tier, lst


def quantize_int8(rows):
    """T2 storage of K or V rows: symmetric 8-bit codes with one fp32 scale per row.

    "Nem Todos os Pensamentos Necessitam de HBM", §1 "Classificação de Quatro Níveis" (T2:
    low-importance rows kept on the CPU at reduced precision, for instance 8-bit quantization;
    §4 "Sensibilidade à Precisão" reports what it costs in accuracy).  The pages name no
    scheme; reading taken: per row (one token of one KV head, K and V separately) m is the
    largest |x| over the row's finite elements, scale = fp32(m / 127), and every element gets
    the code rint(fp32(x · fp32(127 / m))) (ties to even) clamped to [-127, 127]; a non-finite
    element gets code 0; a row with m = 0 gets codes 0 and scale 0.  The fp32 quotients and
    products decide integers, so they are taken in fp32, as the kernel takes them.

    rows: ``[..., d]`` values (float, or bf16 bit patterns as uint16).
    Returns (codes int8 ``[..., d]``, scale fp32 ``[...]``).
    """
    x = np.asarray(rows)
    x = decode_bf16(x).astype(np.float32) if x.dtype == np.uint16 else x.astype(np.float32)
    fin = np.isfinite(x)
    a = np.where(fin, np.abs(x), np.float32(0)).astype(np.float32)
    m = a.max(axis=-1) if x.shape[-1] else np.zeros(x.shape[:-1], np.float32)
    pos = m > 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        scale = np.where(pos, m / np.float32(127), np.float32(0)).astype(np.float32)
        inv = np.where(pos, np.float32(127) / m, np.float32(0)).astype(np.float32)
        y = (x * inv[..., None]).astype(np.float32)
    c = np.clip(np.rint(np.where(fin, y, np.float32(0))), -127, 127)
    return c.astype(np.int8), scale


def dequantize_int8(codes, scale) -> np.ndarray:
    """A T2 row as the attention reads it: fp32(code · scale), rounded to bf16 (ties to even),
    the dtype of the cache it stands in for.  Returns bf16 bit patterns (uint16)."""
    c = np.asarray(codes).astype(np.float32)
    sc = np.asarray(scale, dtype=np.float32)[..., None]
    return encode_bf16((c * sc).astype(np.float32))


def residency_update(tier, s, loc_old, n_tokens: int, capacity: int):
    """HBM residency of one sequence's rows after a tier reassignment, and the rows to copy.

    "Nem Todos os Pensamentos Necessitam de HBM", §1 "Classificação de Quatro Níveis" (T0
    stays in HBM; T1 lives in host DDR at full precision and reaches the attention from there)
    and §4 "Implementação do Sistema" (asynchronous differential prefetch: only newly promoted
    rows cross PCIe); "O Fim do Gargalo de Memória ...", "A Inovação" (optional residency:
    rows stay in HBM while memory allows).  Readings taken:

    * HBM holds at most ``capacity`` rows of the sequence, in slots 0..capacity-1 (the same
      slot in every layer and KV head); every row also lives in host memory at its token index.
    * the resident set R: the rows of T0 ∪ T1 ranked by (tier ascending, s descending, index
      ascending), the first min(capacity, |T0 ∪ T1|) of them — T0 first, then the most
      important T1 rows while slots remain.  A NaN score ranks last in its tier, by index.
    * a row of R that already holds a slot (0 <= loc_old < capacity) keeps it; the other rows
      of R, in ascending token order, take the slots no kept row holds, in ascending slot
      order, and are copied host -> HBM.
    * loc[tok] = slot for tok in R, else ~tok (the row is read from host slot tok).

    Returns (loc_new ``[n_tokens]`` int64, copies: list of (tok, slot), ascending tok).
    """
    tier = np.asarray(tier)[:n_tokens]
    sv = np.asarray(s, dtype=np.float64)[:n_tokens]
    old = np.asarray(loc_old, dtype=np.int64)[:n_tokens]

    def key(i):
        bad = bool(np.isnan(sv[i]))
        return (int(tier[i]), bad, 0.0 if bad else -sv[i], i)

    live = [i for i in range(n_tokens) if tier[i] <= 1]
    ranked = sorted(live, key=key)
    R = sorted(ranked[: min(capacity, len(ranked))])
    held = {i: int(old[i]) for i in R if 0 <= old[i] < capacity}
    taken = set(held.values())
    free = [sl for sl in range(capacity) if sl not in taken]
    loc = np.array([~i for i in range(n_tokens)], dtype=np.int64)
    copies = []
    for i in R:
        if i in held:
            loc[i] = held[i]
        else:
            sl = free[len(copies)]
            loc[i] = sl
            copies.append((i, sl))
    return loc, copies


def residency_append(loc_old, n_old: int, n_new: int, capacity: int):
    """HBM slots of the rows a sequence gained since the last step.

    "Nem Todos os Pensamentos Necessitam de HBM", §1 "Classificação de Quatro Níveis" (the
    recent window is protected, so a new row is T0, and T0 stays in HBM); "O Fim do Gargalo de
    Memória ...", "A Inovação" (rows are kept in HBM while memory allows).  Reading taken: a
    row's K/V are produced on the GPU, so each new row is written into an HBM slot if one is
    free: the new rows [n_old, n_new), in ascending token order, take the slots 0..capacity-1
    that no row below n_old holds (0 <= loc_old < capacity), in ascending slot order; rows left
    without a slot are read from host memory (~tok) until the next reassignment.

    Returns (loc_new ``[n_new]`` int64, copies: list of (tok, slot), ascending tok).
    """
    old = np.asarray(loc_old, dtype=np.int64)[:n_old]
    held = {int(x) for x in old if 0 <= x < capacity}
    free = [sl for sl in range(capacity) if sl not in held]
    loc = np.concatenate([old, np.array([~t for t in range(n_old, n_new)], dtype=np.int64)])
    copies = []
    for t in range(n_old, n_new):
        if len(copies) < len(free):
            loc[t] = free[len(copies)]
            copies.append((t, free[len(copies)]))
    return loc, copies


def softmax_scale(d: int) -> float:
    """Softmax temperature 1/sqrt(d) (the pages do not state one; the usual choice)."""
    return 1.0 / math.sqrt(d)
