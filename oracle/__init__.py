"""CPU oracle for sparse GQA decode attention — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct fp64 NumPy implementation of what the sparse
decode path computes, written from the source pages' definitions.  It shares
no code with the HIP library and imports nothing from it.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path never does.

Every function cites the passage it follows by page title and section:

* "SparDA: Atenção Esparsa Desacoplada ..." — §2 Metodologia, subsection
  "Indexador de Previsão Compacto" (one predictor head per GQA group, no
  softmax) and "Seleção Esparsa de Lookahead Treinável" (top-k blocks);
  "Estratégia de Treinamento" (the compression window of the block grid, and
  the overlapping (32, 16) compression windows max-pooled onto another grid).
* "Esparsidade de Contexto no Tempo de Inferência: Ilusão ou Oportunidade?"
  — §2 Metodologia "Oracle Top-K" (exact top-k tokens) and "Implementação de
  Hardware" (per-token, per-query, per-head sparsity); §3C (traffic O(k·d)).
* "Nem Todos os Pensamentos Necessitam de HBM" — Metodologia §1 (four-tier
  classification, T2 kept at 8 bits), §2 (cumulative importance equation), §3
  (Proposition 1), §4 (reassignment period Δ).
* "O Fim do Gargalo de Memória: ... Adaptive DHiSparse" — "Metodologia e
  Eficiência de Carga" (queries share the retrieval of missing rows), "A Inovação"
  (optional residency of rows in HBM while memory allows).
* "Nem Todos os Pensamentos Necessitam de HBM" §4 "Implementação do Sistema"
  (differential prefetch of newly promoted rows) — residency_update; §1 (the recent window is
  protected T0) — residency_append, the slots of rows added since the last step.

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
closed forms, invariants, brute force on tiny inputs or an independent library
routine, and so are the checkers every parity assertion goes through
(``steps.rel_err``, ``steps.elem_rel_err``, ``steps.topk_band_ok``: hand values, sign
flips, outliers, zero references, wrong counts, duplicates and out-of-range indices).  Nothing in this package is "parity unpinned" except
the pages' published throughput figures, which it does not model.
"""
from .core import (  # noqa: F401
    decode_bf16,
    encode_bf16,
    quantize_int8,
    dequantize_int8,
    to_f64,
    block_pool,
    window_count,
    window_pool,
    scores_block_windowed,
    scores_token_group_mean,
    scores_token_per_head,
    scores_block,
    topk,
    selection_tokens,
    attend,
    importance_update,
    tier_classify,
    residency_update,
    residency_append,
    softmax_scale,
)
from . import steps  # noqa: F401
