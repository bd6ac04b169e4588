"""One decode step of each workload shape, composed from the per-group definitions
(test infrastructure only).  Each function works on one (batch, KV head) group
— or one sequence for the tiered step — so large caches can be checked a group
at a time.  All arrays are NumPy; bf16 inputs are passed as uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

from .core import (attend, block_pool, decode_bf16, dequantize_int8, importance_update,
                   quantize_int8, scores_block, scores_block_windowed, window_pool,
                   scores_token_group_mean, scores_token_per_head, selection_tokens,
                   tier_classify, to_f64, topk)


def block_group(pred, keys, vals, q_group, k_blocks, block_size, n_sink, n_recent, sm_scale,
                kpool=None):
    """Block-sparse step of one GQA group (predictor indexer over pooled blocks).

    SparDA §2: one predictor vector per GQA group scores mean-pooled block keys
    (no softmax); the top-k blocks are read; the group's query heads attend over
    them exactly.  The sinks and the recent window are always kept ("Nem Todos os
    Pensamentos ...", §1).  Top-k runs over all complete blocks; the forced rows
    are merged afterwards and deduplicated.
    """
    n = np.asarray(keys).shape[0]
    kp = block_pool(keys, block_size) if kpool is None else to_f64(kpool)
    sc = scores_block(pred, kp)
    blocks = topk(sc, k_blocks)
    toks = selection_tokens(blocks, block_size, n, n_sink, n_recent)
    kf, vf = to_f64(keys), to_f64(vals)
    out, lse, _ = attend(q_group, kf[toks], vf[toks], sm_scale)
    return dict(kpool=kp, scores=sc, blocks=blocks, tokens=toks, out=out, lse=lse)


def block_layers(preds, keys_layers, vals_layers, q_layers, k_blocks, block_size, n_sink,
                 n_recent, sm_scale):
    """Block-sparse decode of one GQA group through L layers with lookahead selection.

    SparDA §2 "Seleção Esparsa de Lookahead Treinável": the blocks layer l+1 reads are chosen
    by that layer's predictor vector, which is available while layer l still runs, so the
    selection of every layer is made before the layer before it attends and never depends on
    another layer's attention; each layer then reads its chosen blocks (with the sinks and the
    recent window) and attends exactly, as block_group.  Where a row lives (HBM, or host memory
    copied in ahead of use) does not enter: "Nem Todos os Pensamentos ...", §3 (Proposition 1).

    preds ``[L, d]``; keys_layers / vals_layers ``[L, n, d]``; q_layers ``[L, G, d]``.
    Returns the list of block_group results, one per layer.
    """
    L = len(preds)
    return [block_group(preds[l], keys_layers[l], vals_layers[l], q_layers[l], k_blocks,
                        block_size, n_sink, n_recent, sm_scale) for l in range(L)]


def block_windowed_group(pred, keys, vals, q_group, k_blocks, block_size, window, stride,
                         n_sink, n_recent, sm_scale, kwin=None):
    """Block-sparse step of one GQA group with the predictor scoring overlapping compression
    windows (SparDA, "Estratégia de Treinamento": kernel 32, stride 16 at inference) whose
    scores are max-pooled onto the block grid; then as ``block_group``.
    """
    n = np.asarray(keys).shape[0]
    kw = window_pool(keys, window, stride) if kwin is None else to_f64(kwin)
    sc = scores_block_windowed(pred, kw, n, window, stride, block_size)
    blocks = topk(sc, k_blocks)
    toks = selection_tokens(blocks, block_size, n, n_sink, n_recent)
    kf, vf = to_f64(keys), to_f64(vals)
    out, lse, _ = attend(q_group, kf[toks], vf[toks], sm_scale)
    return dict(kwin=kw, scores=sc, blocks=blocks, tokens=toks, out=out, lse=lse)


def group_mean_group(q_tokens, keys, vals, k, sm_scale, n_sink=0, n_recent=0):
    """Token-sparse step of one GQA group with group-mean scoring, T query tokens.

    ``q_tokens`` ``[T, G, d]``.  For each query token t: score every cached key by
    the mean over the group's heads of q·k, keep the top-k, and let the G heads of
    token t attend over token t's own set.  "O Fim do Gargalo de Memória ...",
    "Metodologia e Eficiência de Carga": queries verified together share the
    retrieval of missing rows — the union of the T sets is the fetch unit only.
    """
    q = np.asarray(q_tokens)
    n = np.asarray(keys).shape[0]
    kf, vf = to_f64(keys), to_f64(vals)
    T = q.shape[0]
    scores, sels, outs, lses = [], [], [], []
    for t in range(T):
        sc = scores_token_group_mean(q[t], keys)
        sel = topk(sc, k)
        toks = selection_tokens(sel, 1, n, n_sink, n_recent)
        out, lse, _ = attend(q[t], kf[toks], vf[toks], sm_scale)
        scores.append(sc), sels.append(sel), outs.append(out), lses.append(lse)
    union = np.unique(np.concatenate(sels)) if T else np.zeros(0, np.int64)
    return dict(scores=np.stack(scores), sel=np.stack(sels), union=union,
                out=np.stack(outs), lse=np.stack(lses))


def per_head_group(q_group, keys, vals, k, sm_scale):
    """Per-query-head exact top-k step of one GQA group ("Esparsidade de Contexto ...",
    §2 "Oracle Top-K" and "Implementação de Hardware": each query head keeps its
    own top-k tokens).  ``q_group`` ``[G, d]``.  The group's union is the fetch unit.
    """
    q = np.asarray(q_group)
    kf, vf = to_f64(keys), to_f64(vals)
    sc = scores_token_per_head(q, keys)                 # [G, n]
    G = sc.shape[0]
    sels, outs, lses = [], [], []
    for h in range(G):
        sel = topk(sc[h], k)
        out, lse, _ = attend(q[h:h + 1], kf[sel], vf[sel], sm_scale)
        sels.append(sel), outs.append(out[0]), lses.append(lse[0])
    union = np.unique(np.concatenate(sels)) if G else np.zeros(0, np.int64)
    return dict(scores=sc, sel=np.stack(sels), union=union, out=np.stack(outs),
                lse=np.array(lses))


def tiered_sequence_step(s_prev, evicted, q_layers, k_layers, v_layers, n_tokens, sm_scale,
                         n_sink, n_recent, t0_permille=250, t01_permille=750, dense=False,
                         t012_permille=None):
    """One decode step of one sequence under the tiered KV hierarchy.

    "Nem Todos os Pensamentos Necessitam de HBM": classify tokens into tiers by the
    importance of the previous step (§1), attend exactly over T0 ∪ T1 ∪ T2 in every
    layer and head (T1 rows come back at full precision, §3; T2 rows are read from
    their 8-bit copy, ``core.quantize_int8`` then ``core.dequantize_int8``, §1), then
    add this step's attention, averaged over layers and heads, to the importance (§2).
    ``dense=True`` is the first step, before any importance exists: attend over
    every token and classify nothing.  ``t012_permille`` None: no T2.

    q_layers ``[L, Hq, d]``; k_layers / v_layers ``[L, Hkv, >=n_tokens, d]``;
    ``s_prev`` fp32 ``[>=n_tokens]``; ``evicted`` bool ``[>=n_tokens]`` or None.
    Returns dict(tier, tokens, out [L, Hq, d], lse [L, Hq], s (fp32 [n_tokens]),
    evicted (bool [n_tokens])).
    """
    q = np.asarray(q_layers)
    L, Hq = q.shape[0], q.shape[1]
    Hkv = np.asarray(k_layers).shape[1]
    G = Hq // Hkv
    s_prev = np.asarray(s_prev, dtype=np.float32)[:n_tokens]
    ev = np.zeros(n_tokens, bool) if evicted is None else np.asarray(evicted, bool)[:n_tokens]
    if dense:
        tier = np.zeros(n_tokens, np.uint8)
        toks = np.arange(n_tokens, dtype=np.int64)
    else:
        tier, toks = tier_classify(s_prev, n_tokens, n_sink, n_recent, t0_permille,
                                   t01_permille, ev, t012_permille)
    t2 = tier[toks] == 2                    # attended rows read from their 8-bit copy
    alpha = np.zeros((L, Hq, n_tokens))
    outs = np.zeros((L, Hq, q.shape[2]))
    lses = np.zeros((L, Hq))

    def rows(src):
        x = np.asarray(src)[:n_tokens][toks]
        f = to_f64(x)
        if t2.any():
            f[t2] = decode_bf16(dequantize_int8(*quantize_int8(x[t2])))
        return f
    for l in range(L):
        for kvh in range(Hkv):
            kf = rows(k_layers[l, kvh])
            vf = rows(v_layers[l, kvh])
            out, lse, logits = attend(q[l, kvh * G:(kvh + 1) * G], kf, vf, sm_scale)
            outs[l, kvh * G:(kvh + 1) * G] = out
            lses[l, kvh * G:(kvh + 1) * G] = lse
            alpha[l, kvh * G:(kvh + 1) * G][:, toks] = np.exp(logits - lse[:, None])
    s_new = importance_update(s_prev, alpha)
    return dict(tier=tier, tokens=toks, out=outs, lse=lses, s=s_new, evicted=ev | (tier == 3))


# Bars of the parity checks.  TOL is the stated one (2e-3 max relative error); the
# elementwise check counts an element's error against max(|ref_i|, ELEM_FLOOR·max|ref|); the
# attention outputs also meet ATTN_REGRESSION_BOUND, which sits between what fp32 accumulation
# with P kept to ~16 bits reaches (a few 1e-6) and what rounding P to bf16 alone costs
# (~1.5e-3 to 2e-3 on these shapes, under TOL): a regression to the latter fails it.
TOL = 2e-3
ELEM_FLOOR = 1e-2
ATTN_REGRESSION_BOUND = 1e-4


def rel_err(x, ref) -> float:
    """Normwise relative error max|x - ref| / max|ref| (the absolute error when ref is all
    zero; 0 for empty arrays)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise ValueError(f"shape mismatch {x.shape} vs {ref.shape}")
    if ref.size == 0:
        return 0.0
    den = np.max(np.abs(ref))
    num = np.max(np.abs(x - ref))
    if den == 0.0:
        return float(num)
    return float(num / den)


def elem_rel_err(x, ref, floor_frac: float = ELEM_FLOOR) -> float:
    """Largest elementwise relative error, each element's error taken against
    max(|ref_i|, floor_frac·max|ref|): elements far below the row's scale are held to an
    absolute floor instead of their own magnitude.  0 for empty arrays; a NaN anywhere
    gives inf."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise ValueError(f"shape mismatch {x.shape} vs {ref.shape}")
    if ref.size == 0:
        return 0.0
    diff = np.abs(x - ref)
    if np.isnan(diff).any():
        return float("inf")
    scale = np.maximum(np.abs(ref), floor_frac * np.max(np.abs(ref)))
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(diff == 0.0, 0.0, diff / scale)
    return float(np.max(r))


def topk_band_ok(gpu_idx, scores_ref, k, tol) -> bool:
    """Selection check when the GPU ranked scores it computed itself.

    The selection must hold exactly min(k, n) distinct indices in [0, n).  The GPU and
    oracle scores may differ in the last bits, so a differing choice is accepted only for
    elements whose oracle score lies within ``tol·max|x|`` of the k-th largest oracle
    score: every element clearly above that threshold must be chosen and every one clearly
    below must not.
    """
    x = np.asarray(scores_ref, dtype=np.float64)
    n = x.shape[0]
    k = max(0, min(int(k), n))
    idx = np.asarray(gpu_idx).astype(np.int64).ravel()
    if idx.shape[0] != k:
        return False
    if k and (idx.min() < 0 or idx.max() >= n):
        return False
    if np.unique(idx).shape[0] != k:
        return False
    chosen = np.zeros(n, bool)
    chosen[idx] = True
    if k == 0 or k == n:
        return True
    thr = np.sort(x)[::-1][k - 1]
    band = tol * np.max(np.abs(x))
    must = x > thr + band
    must_not = x < thr - band
    return bool(np.all(chosen[must]) and not np.any(chosen[must_not]))
