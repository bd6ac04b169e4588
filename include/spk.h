/*
 * spk.h — C ABI of libspk: sparse top-k KV decode attention with GQA on AMD MI355X (gfx950).
 *
 * One decode step over a long KV cache reads only a chosen part of it:
 *   sparse_index_score   a compact indexer scores cached keys (or pooled block keys), no softmax
 *   topk_select          exact top-k of each score row, ties to the lowest index
 *   sparse_index_topk    both of the above in one launch, for short candidate rows
 *   sparse_topk_decode_attn  top-k of a score row and the attention over it, in one launch
 *   sparse_decode_attn   gathers the chosen K/V rows once per GQA group (HBM or pinned host
 *                        memory) and runs exact softmax attention over them only
 *   topk_select_union, sparse_decode_attn_union
 *                        for wide rows with up to 4 selection sets per KV head: the per-set
 *                        top-k and the group's union with set masks, and the attention over
 *                        that union
 *   lookahead_prefetch   copies the host rows of the next layer's chosen blocks into HBM
 *                        staging rows while the current layer attends
 *   importance_accumulate  cumulative attention importance s_i += mean over layers, heads of α[i]
 *   tier_classify        T0/T1/T3 tiers by importance, sinks and recent window protected
 *
 * Conventions shared by every call
 *   - Tensors are row-major with a contiguous last dimension; strides and leading dimensions
 *     are in ELEMENTS of the tensor's own type.  "Device" pointers are HIP device memory (or
 *     device-mapped pinned host memory where stated); "host" pointers are ordinary CPU memory.
 *   - Shapes: B batch, T query tokens per sequence, Hq query heads, Hkv KV heads (Hq % Hkv == 0,
 *     G = Hq / Hkv), d head dim (64 or 128), n_tokens cached tokens.  Query head h belongs to
 *     KV head h / G.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the null stream) and
 *     returns; nothing synchronises the host.  Faults during execution surface as HIP errors
 *     at the caller's next synchronisation.
 *   - Ownership: the caller owns every buffer (inputs, outputs, workspace, host pools).  The
 *     library never allocates or frees memory and keeps no state between calls except a cached
 *     per-device property table and the fixed scratch array of sparse_decode_attn_noalloc;
 *     calls are re-entrant and may run on concurrent streams when their output buffers and
 *     workspaces are distinct.
 *   - Errors: arguments are validated before any launch; on a non-OK return nothing was
 *     launched and nothing was written, and spk_last_error() (thread-local) says why.
 *       SPK_EINVAL       null required pointer, inconsistent shapes, bad strides or sizes
 *       SPK_EUNSUPPORTED d not in {64, 128}, or a dtype combination without a kernel
 *       SPK_EWORKSPACE   workspace smaller than the *_workspace_size query asks for
 *       SPK_EHIP         a HIP launch failed (text in spk_last_error())
 *   - Index entries that fall outside the valid range are skipped (never dereferenced).
 */
#ifndef SPK_H
#define SPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define SPK_API __attribute__((visibility("default")))
#else
#define SPK_API
#endif

typedef enum {
  SPK_OK = 0,
  SPK_EINVAL = 1,
  SPK_EUNSUPPORTED = 2,
  SPK_EWORKSPACE = 3,
  SPK_EHIP = 4
} spk_status;

typedef enum { SPK_F32 = 0, SPK_BF16 = 1 } spk_dtype;

typedef enum {
  SPK_IDX_TOKEN_GROUP_MEAN = 0, /* score[b,t,kvh,j] = mean over the G heads of kvh of q[b,t,h]·k[b,kvh,j] */
  SPK_IDX_TOKEN_PER_HEAD = 1,   /* score[b,t,h,j]   = q[b,t,h]·k[b,h/G,j]                               */
  SPK_IDX_BLOCK_POOLED = 2,     /* score[b,t,kvh,j] = p[b,t,kvh]·Kpool[b,kvh,j]  (pooled keys given)     */
  SPK_IDX_BLOCK_RAW = 3         /* same, pooling raw keys on the fly (optionally writing Kpool)        */
} spk_index_mode;

typedef enum {
  SPK_SEL_PER_SEQ = 0,     /* one list per sequence b, read by every query vector of b            */
  SPK_SEL_PER_KV_HEAD = 1, /* one list per (b, t, kvh), read by the G heads of kvh at token t      */
  SPK_SEL_PER_Q_HEAD = 2   /* one list per (b, t, h), read by query head h at token t only         */
} spk_sel_scope;

/* Thread-local text describing the last non-OK status returned on this thread ("" if none). */
SPK_API const char* spk_last_error(void);

/* ABI version of this header (bumped on any incompatible change). */
SPK_API int spk_version(void);
#define SPK_VERSION 1

/* Measurement hook for the attention's gather kernel (the launch that reads the selected K/V
 * rows).  `begin` and `end` are HIP events (hipEvent_t cast to void*, created and owned by the
 * caller).  While both are non-null, every later sparse_decode_attn call records `begin` on its
 * stream immediately before that launch and `end` immediately after it, so
 * hipEventElapsedTime(begin, end) is the kernel's duration; the call's other launches (list
 * assembly, split combine) fall outside the pair.  Pass two nulls to switch it off.
 * Process-wide state: calls that overlap from several host threads while it is set race on the
 * events.  Returns SPK_EINVAL if exactly one of the two is null; SPK_EHIP (from the attention
 * call) if a record fails. */
SPK_API spk_status spk_set_attn_timing_events(void* begin, void* end);

/* Measurement reference: a plain streaming read of `bytes` bytes of device memory at `p`, split
 * into `workgroups` contiguous chunks (each workgroup reads its chunk with 16-byte loads).  It
 * computes nothing of the method; its rate is the HBM read ceiling a kernel of this library
 * reaches on the device at hand, reported beside the vendor's peak.  `sink` is one device
 * uint32 that is written only in the rare case the folded words equal a fixed constant (it keeps
 * the loads live; its value means nothing).  Enqueues on `stream` and returns.  SPK_EINVAL on a
 * null pointer, a pointer or size that is not a multiple of 16 bytes, or workgroups outside
 * [1, 2^20]; bytes = 0 launches nothing. */
SPK_API spk_status spk_stream_read(const void* p, size_t bytes, int workgroups, uint32_t* sink,
                                   void* stream);

/* Measurement reference: spk_stream_read of `bytes` bytes of pinned host memory at `host` (from
 * hipHostMalloc: page-locked and device-mapped), read through the device address HIP reports for
 * it, as the attention reads host-resident rows.  Its rate is the ceiling of kernel reads over
 * the host link, reported beside the link's nominal rate.  The library asks
 * hipPointerGetAttributes and returns SPK_EINVAL unless HIP reports host memory with a device
 * address; that query is its only check, so pass no other memory.  The caller guarantees that
 * [host, host + bytes) lies inside one allocation.  `sink`, errors and bytes = 0 as
 * spk_stream_read (bytes = 0 launches nothing and queries nothing). */
SPK_API spk_status spk_stream_read_host(const void* host, size_t bytes, int workgroups,
                                        uint32_t* sink, void* stream);

/* Measurement reference: reads the K and V rows named by per-group row lists, each listed row
 * once, and computes nothing of the method.  Its rate is the HBM rate a plain gather of exactly
 * that set of rows reaches on the device at hand (the rows of a sparse selection are scattered,
 * which a contiguous streaming read does not capture).  Group g's list is
 * rows[g*rows_ld .. g*rows_ld + rows_ld); entry t names the rows at
 * k + g*group_stride + t*row_stride and v + g*group_stride + t*row_stride (byte offsets), of
 * which the first row_bytes bytes are read; entries < 0 or >= n_rows are skipped.  Each group's
 * list is cut into wg_per_group contiguous parts, one workgroup each.  The caller guarantees
 * that every row of every group lies inside its k and v buffers.  `sink`: as spk_stream_read.
 * Enqueues on `stream` and returns.  SPK_EINVAL on a null pointer, row_bytes not in {64, 128,
 * 256, 512, 1024}, k, v or a stride not a multiple of 16 bytes, row_stride < row_bytes, negative
 * sizes, rows_ld >= 2^31, groups or wg_per_group outside [0, 65535] / [1, 65535]; nothing is
 * launched when groups, rows_ld or n_rows is 0. */
SPK_API spk_status spk_gather_read(const void* k, const void* v, int64_t row_bytes,
                                   int64_t group_stride, int64_t row_stride, int64_t n_rows,
                                   const int32_t* rows, int64_t rows_ld, int groups,
                                   int wg_per_group, uint32_t* sink, void* stream);

/* ------------------------------------------------------------------------------------------
 * sparse_index_score — compact indexer scores, no softmax.
 *
 * Passages: SparDA: Atenção Esparsa Desacoplada, §2 "Indexador de Previsão Compacto" (one
 * predictor head per GQA group, i.e. per KV head, no per-query-head scoring loop, softmax
 * skipped) and "Seleção Esparsa de Lookahead Treinável" (the predictor ranks KV blocks);
 * "Esparsidade de Contexto no Tempo de Inferência", §2 "Oracle Top-K" (exact per-head token
 * scores).  Scores are unscaled dot products in fp32.
 *
 *   q        device; TOKEN_* modes: Q [B,T,Hq,d] contiguous; BLOCK_* modes: predictor
 *            [B,T,Hkv,d] contiguous.  q_dtype SPK_F32 or SPK_BF16.
 *   keys     device; TOKEN_* and BLOCK_RAW: the key cache, row (b,kvh,j) at
 *            keys + b*k_sb + kvh*k_sh + j*k_sn (k_dtype F32 or BF16); BLOCK_POOLED: pooled keys
 *            with the same stride convention, one row per block (F32 or BF16).
 *   n_tokens tokens in the cache.  Candidates: TOKEN_* -> n_tokens tokens; BLOCK_* ->
 *            n_tokens / block_size complete blocks (the partial tail block is not a candidate).
 *   scores   device fp32 [B,T,Hs,s_ld], Hs = Hq for TOKEN_PER_HEAD else Hkv; entries
 *            [0, n_candidates) of each row are written.  s_ld >= n_candidates.
 *   pooled_out  BLOCK_RAW only, optional: device fp32 [B,Hkv,n_tokens/block_size,d]
 *            contiguous, receives the block means; NULL otherwise.
 * ------------------------------------------------------------------------------------------ */
SPK_API spk_status sparse_index_score(spk_index_mode mode,
                                      const void* q, spk_dtype q_dtype,
                                      const void* keys, spk_dtype k_dtype,
                                      int64_t k_sb, int64_t k_sh, int64_t k_sn,
                                      int B, int T, int Hq, int Hkv, int d,
                                      int n_tokens, int block_size,
                                      float* scores, int64_t s_ld,
                                      float* pooled_out,
                                      void* stream);

/* ------------------------------------------------------------------------------------------
 * topk_select — exact top-k of each row of an fp32 score matrix.
 *
 * Passages: SparDA, §2 "Seleção Esparsa de Lookahead Treinável" (top-k blocks) and
 * "Esparsidade de Contexto no Tempo de Inferência", §2 "Oracle Top-K" (exact top-k tokens).
 * Definition: the min(k, n) entries with the largest scores; equal scores go to the lowest
 * index; -0 equals +0; NaN ranks below -inf.  Indices are written in ASCENDING order.
 *
 *   scores   device fp32 [rows, s_ld]; entries [0, n) of each row are read.
 *   idx      device int32 [rows, idx_ld]; entries [0, min(k,n)) written.  idx_ld >= min(k,n).
 *   count    device int32 [rows] or NULL; receives min(k, n).
 *   ws       device workspace of at least topk_select_workspace_size() bytes (may be NULL
 *            when that size is 0).
 * ------------------------------------------------------------------------------------------ */
SPK_API spk_status topk_select_workspace_size(int rows, int n, int k, size_t* bytes);
SPK_API spk_status topk_select(const float* scores, int64_t s_ld, int rows, int n, int k,
                               int32_t* idx, int64_t idx_ld, int32_t* count,
                               void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * topk_select_union — the exact top-k of every score row of each (b, kvh) group's S <= 4
 * selection sets, and the group's union of the S selections with a set mask per row.
 *
 * Passages: "Esparsidade de Contexto no Tempo de Inferência", §2 "Oracle Top-K" and
 * "Implementação de Hardware" (each query head keeps its own top-k tokens); "O Fim do Gargalo
 * de Memória ... Adaptive DHiSparse", "Metodologia e Eficiência de Carga" (queries verified
 * together share the retrieval of their rows: the union is read once).
 *
 *   scores     device fp32 score rows, row stride s_ld >= n: PER_Q_HEAD: rows (b, t, query
 *              head), S = T * G sets per group (set s = t*G + j is head kvh*G + j of token t);
 *              PER_KV_HEAD: rows (b, t, kvh), S = T sets (set s = token t)
 *   n, k       candidates per row (n <= 2^22) and how many to keep (k >= 0; k > n keeps all n)
 *   idx        device int32 [rows][idx_ld], idx_ld >= min(k, n): each row's kept indices in
 *              ascending order (ties to the lowest index), as topk_select
 *   count      device int32 [rows]: min(k, n)
 *   u_list     device int32 [B*Hkv][u_ld], u_ld >= min(n, S * min(k, n)): each group's union,
 *              ascending; u_mask the same shape, uint32, bit s set when set s keeps the row;
 *              u_count device int32 [B*Hkv], the union lengths
 *   ws         device workspace of topk_select_union_workspace_size() bytes, no initial
 *              contents needed
 * Cost: a sample of each row (1/32 of it past 4096 keys) sets a key range expected to hold the
 * k-th key, and one pass over the scores collects the keys above and inside it; the result is
 * the exact top-k whatever the sample says, but a row whose sample misjudges its range (scores
 * ordered against the sampling pattern, or heavy ties) costs a whole-row pass of its own.
 * Errors: SPK_EINVAL (scope not PER_Q_HEAD / PER_KV_HEAD, sizes, null buffers, short leading
 * dims), SPK_EUNSUPPORTED (S > 4), SPK_EWORKSPACE.
 * ---------------------------------------------------------------------------------------- */
SPK_API spk_status topk_select_union_workspace_size(int B, int T, int Hq, int Hkv,
                                                    spk_sel_scope scope, int n, int k,
                                                    size_t* bytes);
SPK_API spk_status topk_select_union(const float* scores, int64_t s_ld,
                                     int B, int T, int Hq, int Hkv, spk_sel_scope scope,
                                     int n, int k, int32_t* idx, int64_t idx_ld, int32_t* count,
                                     int32_t* u_list, uint32_t* u_mask, int32_t* u_count,
                                     int64_t u_ld, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * sparse_index_topk — sparse_index_score followed by topk_select, in one launch, for short
 * candidate rows.
 *
 * Passages: as for sparse_index_score and topk_select (SparDA, §2 "Indexador de Previsão
 * Compacto" and "Seleção Esparsa de Lookahead Treinável").  The scores are those
 * sparse_index_score defines (fp32, possibly differing from it in the last bits, since the
 * dot products are summed in another order); the selection is exactly topk_select of these
 * scores (ties to the lowest index, ascending output).
 *
 *   mode     TOKEN_GROUP_MEAN, TOKEN_PER_HEAD or BLOCK_POOLED (BLOCK_RAW: SPK_EUNSUPPORTED).
 *   q, keys, strides, shapes, n_tokens, block_size: as sparse_index_score.
 *   k        candidates kept per score row (>= 0).
 *   scores   device fp32 [B,T,Hs,s_ld] or NULL (then not written; s_ld ignored).
 *   idx      device int32 [B,T,Hs,idx_ld]; entries [0, min(k, n_candidates)) written.
 *   count    device int32 [B,T,Hs] or NULL; receives min(k, n_candidates).
 * Limits (SPK_EUNSUPPORTED beyond them; use the two calls instead): at most 4 score vectors
 * per KV head (T for TOKEN_GROUP_MEAN and BLOCK_POOLED, T*G for TOKEN_PER_HEAD), at most 8192
 * candidates per row and 16384 scores per KV head.  No workspace.
 * ------------------------------------------------------------------------------------------ */
SPK_API spk_status sparse_index_topk(spk_index_mode mode,
                                     const void* q, spk_dtype q_dtype,
                                     const void* keys, spk_dtype k_dtype,
                                     int64_t k_sb, int64_t k_sh, int64_t k_sn,
                                     int B, int T, int Hq, int Hkv, int d,
                                     int n_tokens, int block_size, int k,
                                     float* scores, int64_t s_ld,
                                     int32_t* idx, int64_t idx_ld, int32_t* count,
                                     void* stream);

/* ------------------------------------------------------------------------------------------
 * sparse_window_pool — mean of the keys of every overlapping compression window.
 *
 * Passage: SparDA, §2 "Estratégia de Treinamento" (at inference the keys are compressed with
 * overlapping windows of kernel 32 and stride 16).  Window w of group (b, kvh) covers tokens
 * [stride*w, stride*w + window); only complete windows exist, nw = (n_tokens - window)/stride + 1
 * of them (0 when n_tokens < window).  kwin[b,kvh,w,:] = mean of those keys (fp32 sum, then
 * one multiply by 1/window).  Done once per cache (or per completed window), off the step.
 *
 *   keys     device cache [B,Hkv,*,d] with row strides k_sb, k_sh, k_sn (elements, multiples
 *            of 8, k_sn >= d), 16-byte aligned; F32 or BF16; rows [0, n_tokens) are read.
 *   window, stride  >= 1, at most 65536.
 *   kwin     device fp32 [B,Hkv,w_cap,d] contiguous, 16-byte aligned, w_cap >= nw; rows
 *            [0, nw) of each group written.
 * Errors: SPK_EINVAL (null pointer, shape, strides, alignment, w_cap < nw), SPK_EUNSUPPORTED
 * (d not 64/128, dtype).  Enqueues one launch on `stream`; nothing when nw = 0.
 * ------------------------------------------------------------------------------------------ */
SPK_API spk_status sparse_window_pool(const void* keys, spk_dtype k_dtype,
                                      int64_t k_sb, int64_t k_sh, int64_t k_sn,
                                      int B, int Hkv, int d, int n_tokens, int window, int stride,
                                      float* kwin, int64_t w_cap, void* stream);

/* ------------------------------------------------------------------------------------------
 * sparse_index_score_windowed — block scores of the predictor from overlapping windows.
 *
 * Passages: SparDA, §2 "Indexador de Previsão Compacto" (one predictor head per GQA group, no
 * softmax) and "Estratégia de Treinamento" (overlapping (32, 16) compression windows; scores
 * of one window grid max-pooled onto another).  Reading taken: the predictor p[b,t,kvh]
 * scores every complete window, p·kwin_w (fp32), and block j — tokens
 * [block_size*j, block_size*j + block_size), complete blocks only — scores the largest of the
 * windows that share at least one token with it (-inf when none does).  With window = stride =
 * block_size this is sparse_index_score in BLOCK_POOLED mode.
 *
 *   pred     device [B,T,Hkv,d] contiguous, F32 or BF16, 16-byte aligned; 1 <= T <= 16.
 *   kwin     device fp32 [B,Hkv,w_cap,d] from sparse_window_pool with the same window/stride.
 *   window, stride, block_size  >= 1, at most 65536; one block may overlap at most 1021
 *            windows ((block_size + window)/stride + 3 <= 1024, else SPK_EUNSUPPORTED).
 *   scores   device fp32 [B,T,Hkv,s_ld], s_ld >= n_tokens / block_size; entries
 *            [0, n_tokens / block_size) of each row written.
 * Errors as sparse_window_pool.  One launch; the scores feed topk_select or
 * sparse_topk_decode_attn exactly like BLOCK_POOLED scores.
 * ------------------------------------------------------------------------------------------ */
SPK_API spk_status sparse_index_score_windowed(const void* pred, spk_dtype p_dtype,
                                               const float* kwin, int64_t w_cap,
                                               int B, int T, int Hkv, int d, int n_tokens,
                                               int window, int stride, int block_size,
                                               float* scores, int64_t s_ld, void* stream);

/* ------------------------------------------------------------------------------------------
 * sparse_decode_attn — gather the selected K/V rows and run exact attention over them only.
 *
 * Passages: "Esparsidade de Contexto no Tempo de Inferência", §3C (decode reads O(k·d) rows
 * instead of O(N·d); irregular per-token, per-query and per-head sparsity, §2 "Implementação
 * de Hardware"); "O Fim do Gargalo de Memória ... Adaptive DHiSparse", "A Inovação" (exact
 * fused retrieval of non-resident rows) and "Metodologia e Eficiência de Carga" (queries
 * verified together share the retrieval of missing rows); "Nem Todos os Pensamentos
 * Necessitam de HBM", §3 Proposition 1 (rows fetched from host memory at full precision give
 * exactly the result of HBM-resident rows: the output here is bit-identical whatever `loc`).
 *
 * For each query vector (b,t,h) the set S(b,t,h) of token ids it reads is the selection list
 * chosen by `scope` (PER_SEQ: row b; PER_KV_HEAD: row (b*T+t)*Hkv + h/G; PER_Q_HEAD: row
 * (b*T+t)*Hq + h), each entry e expanded to tokens [e*gran, e*gran + gran) ∩ [0, n_tokens),
 * united with the sinks [0, n_sink) and the recent window [n_tokens - n_recent, n_tokens).
 * Then out[b,t,h,:] = softmax(sm_scale · q·K_Sᵀ) · V_S with fp32 accumulation, and
 * lse[b,t,h] = log Σ_{i∈S} exp(sm_scale · q·k_i) (natural log; -inf and out = 0 if S is empty).
 * Each (b, kvh) group fetches every row of the union of its query vectors' sets exactly once.
 *
 *   q          device [B,T,Hq,d] contiguous, F32 or BF16.
 *   k, v       device caches, row (b,kvh,slot) at k + b*kv_sb + kvh*kv_sh + slot*kv_sn
 *              (same strides for v), slot < hbm_slots; kv_dtype F32 or BF16.  Without `loc`
 *              n_tokens <= hbm_slots is required.
 *   k_host, v_host  pinned host pools (hipHostMalloc'ed: page-locked and device-mapped).  The
 *              library asks hipPointerGetAttributes and returns SPK_EINVAL unless HIP reports
 *              host memory with a device address; that query is its only check, so pass no
 *              other memory.  Row (b,kvh,slot) at
 *              k_host + b*host_sb + kvh*host_sh + slot*host_sn, slot < host_slots; NULL if unused.
 *   loc        device int32 or NULL.  loc[b*loc_sb + kvh*loc_sh + tok] >= 0: token tok is HBM
 *              slot loc (< hbm_slots); < 0: host slot ~loc (< host_slots; requires k_host and
 *              v_host).  A slot outside its pool is treated as a missing row (not read).
 *              NULL: every token is HBM slot tok.
 *   sel_idx    device int32 [rows, sel_ld], strictly ascending entries (as topk_select and
 *              tier_classify write them; may be NULL when sel_ld is 0); sel_count device int32
 *              [rows] (clamped to sel_ld).
 *   gran       1 for token ids, or the block size for block ids.
 *   out        device fp32 [B,T,Hq,d].  lse: device fp32 [B,T,Hq] or NULL.
 *   logits     device fp32 [B,T,Hq,logits_ld] or NULL: the scaled logit sm_scale·q·k of every
 *              row of the group's fetch list (the ascending union above), -inf for rows the
 *              query vector does not read.  For PER_SEQ with gran 1 and no sinks/recent, the
 *              fetch list is sel_idx itself.  logits_ld >= the fetch-list bound (see below).
 *   ws         device workspace of at least sparse_decode_attn_workspace_size() bytes (no
 *              initial contents needed).  Calls that may run concurrently need separate
 *              workspaces.
 *
 * The fetch-list bound per group is min(n_tokens, sets*sel_ld*gran + n_sink + n_recent) with
 * sets = 1 (PER_SEQ), T (PER_KV_HEAD) or T*G (PER_Q_HEAD); at most 16 sets per group (G*T is
 * at most 16 anyway), and sets*sel_ld*gran must stay below 2^31, else SPK_EUNSUPPORTED.
 * A KV or host-pool row stride of 4 GiB or more returns SPK_EUNSUPPORTED.
 * ------------------------------------------------------------------------------------------ */
SPK_API spk_status sparse_decode_attn_workspace_size(spk_sel_scope scope, int B, int T, int Hq,
                                                     int Hkv, int d, int n_tokens, int64_t sel_ld,
                                                     int gran, int n_sink, int n_recent,
                                                     size_t* bytes);
SPK_API spk_status sparse_decode_attn(const void* q, spk_dtype q_dtype,
                                      const void* k, const void* v, spk_dtype kv_dtype,
                                      int64_t kv_sb, int64_t kv_sh, int64_t kv_sn,
                                      const void* k_host, const void* v_host,
                                      int64_t host_sb, int64_t host_sh, int64_t host_sn,
                                      int64_t host_slots,
                                      const int32_t* loc, int64_t loc_sb, int64_t loc_sh,
                                      int64_t hbm_slots,
                                      const int32_t* sel_idx, const int32_t* sel_count,
                                      int64_t sel_ld, spk_sel_scope scope, int gran,
                                      int n_sink, int n_recent,
                                      int B, int T, int Hq, int Hkv, int d, int n_tokens,
                                      float sm_scale,
                                      float* out, float* lse, float* logits, int64_t logits_ld,
                                      void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * sparse_decode_attn_union — sparse_decode_attn over fetch lists the caller has assembled
 * already (topk_select_union's union), so no assembly runs.
 *
 * Passages: as sparse_decode_attn.
 *
 *   u_list, u_mask, u_count, u_ld   each group's ascending fetch rows (token ids), the mask of
 *              the selection sets holding each row (bit s: set s) and the row count; rows past
 *              n_tokens or past u_ld are never read.  PER_Q_HEAD: query head kvh*G + j of
 *              token t reads the rows with bit t*G + j; PER_KV_HEAD: every head of token t reads
 *              the rows with bit t.
 *   every other argument as sparse_decode_attn (host pools and loc included); logits rows are
 *              indexed by the union position.
 *   ws         device workspace of sparse_decode_attn_union_workspace_size() bytes.
 * Errors: as sparse_decode_attn; SPK_EINVAL for another scope or u_ld <= 0.
 * ---------------------------------------------------------------------------------------- */
SPK_API spk_status sparse_decode_attn_union_workspace_size(spk_sel_scope scope, int B, int T,
                                                           int Hq, int Hkv, int d, int n_tokens,
                                                           int64_t u_ld, size_t* bytes);
SPK_API spk_status sparse_decode_attn_union(const void* q, spk_dtype q_dtype,
                                            const void* k, const void* v, spk_dtype kv_dtype,
                                            int64_t kv_sb, int64_t kv_sh, int64_t kv_sn,
                                            const void* k_host, const void* v_host,
                                            int64_t host_sb, int64_t host_sh, int64_t host_sn,
                                            int64_t host_slots,
                                            const int32_t* loc, int64_t loc_sb, int64_t loc_sh,
                                            int64_t hbm_slots,
                                            const int32_t* u_list, const uint32_t* u_mask,
                                            const int32_t* u_count, int64_t u_ld,
                                            spk_sel_scope scope,
                                            int B, int T, int Hq, int Hkv, int d, int n_tokens,
                                            float sm_scale, float* out, float* lse,
                                            float* logits, int64_t logits_ld,
                                            void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * sparse_decode_attn_noalloc — sparse_decode_attn without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).
 *
 * Arguments, layouts, results and errors are those of sparse_decode_attn, minus ws / ws_bytes:
 * the workspace is a fixed array in device memory owned by the library, one per GPU it runs on,
 * of sparse_decode_attn_noalloc_max_bytes() bytes (32 MiB), held until the process ends.  The
 * call allocates and frees nothing.  A call whose workspace (sparse_decode_attn_workspace_size)
 * exceeds that size returns SPK_EWORKSPACE before any launch.  Every call on one GPU uses the
 * same array and leaves its contents behind (nothing in it needs initial contents): calls that
 * may overlap in time on one GPU (on concurrent streams) race and must not be issued.
 * ---------------------------------------------------------------------------------------- */
SPK_API size_t sparse_decode_attn_noalloc_max_bytes(void);

SPK_API spk_status sparse_decode_attn_noalloc(const void* q, spk_dtype q_dtype,
                                              const void* k, const void* v, spk_dtype kv_dtype,
                                              int64_t kv_sb, int64_t kv_sh, int64_t kv_sn,
                                              const void* k_host, const void* v_host,
                                              int64_t host_sb, int64_t host_sh, int64_t host_sn,
                                              int64_t host_slots,
                                              const int32_t* loc, int64_t loc_sb, int64_t loc_sh,
                                              int64_t hbm_slots,
                                              const int32_t* sel_idx, const int32_t* sel_count,
                                              int64_t sel_ld, spk_sel_scope scope, int gran,
                                              int n_sink, int n_recent,
                                              int B, int T, int Hq, int Hkv, int d, int n_tokens,
                                              float sm_scale,
                                              float* out, float* lse, float* logits,
                                              int64_t logits_ld, void* stream);

/* ------------------------------------------------------------------------------------------
 * lookahead_prefetch — copy the host-resident rows of the blocks a selection names into HBM
 * staging rows, ahead of the attention that will read them, and point the row locations there.
 *
 * Passages: SparDA §2 "Seleção Esparsa de Lookahead Treinável" (layer l+1's blocks are chosen
 * while layer l runs) and "Inovações Principais" (a persistent kernel of a few workgroups copies
 * the missing blocks meanwhile); "Nem Todos os Pensamentos Necessitam de HBM" §3 (Proposition 1:
 * the copy is exact, results do not change).
 *
 *   sel_idx, sel_count, sel_ld   block ids per (b, kvh) group [B*Hkv][sel_ld] and their counts
 *              (topk_select's output of the next layer's block scores); block_size rows each
 *   k_host, v_host, host strides, host_slots   pinned host pools [B,Hkv,host_slots,d]
 *   k, v, kv strides, hbm_slots   the HBM caches [B,Hkv,hbm_slots,d]; rows
 *              [stage_base, stage_base + sel_ld*block_size) are the staging rows (past n_tokens)
 *   loc_home   device int32 [B,Hkv,>=n_tokens] (strides loc_sb, loc_sh): each row's home, >= 0
 *              an HBM row, < 0 the host row ~loc_home (read only)
 *   loc        device int32, same layout: the locations the attention reads; the rows this call
 *              redirects point to staging rows, and the rows the previous call redirected are
 *              first set back to their home
 *   staged, staged_count   device int32 [B*Hkv][sel_ld*block_size] and [B*Hkv]: per group the
 *              tokens a call redirected, as a compact list of staged_count entries, kept for the
 *              next call on the same buffers (which must use the same sel_ld and block_size);
 *              staged_count zero before the first call
 *   workgroups the fixed number of workgroups of the persistent copy kernel (its grid); each
 *              takes whole groups in turn, so more than B*Hkv add nothing
 * Run it on a stream of its own beside the attention of the layer before, and make the
 * attention that reads these rows wait for it.  Errors: SPK_EINVAL (sizes, strides, staging
 * range, pools HIP does not report as device-mapped host memory), SPK_EUNSUPPORTED (d, dtype).
 * ---------------------------------------------------------------------------------------- */
SPK_API spk_status lookahead_prefetch(const int32_t* sel_idx, const int32_t* sel_count,
                                      int64_t sel_ld, int block_size, int B, int Hkv, int d,
                                      spk_dtype kv_dtype, int n_tokens,
                                      const void* k_host, const void* v_host,
                                      int64_t host_sb, int64_t host_sh, int64_t host_sn,
                                      int64_t host_slots, void* k, void* v,
                                      int64_t kv_sb, int64_t kv_sh, int64_t kv_sn,
                                      int64_t hbm_slots, int64_t stage_base,
                                      const int32_t* loc_home, int32_t* loc,
                                      int64_t loc_sb, int64_t loc_sh,
                                      int32_t* staged, int32_t* staged_count, int workgroups,
                                      void* stream);

/* ------------------------------------------------------------------------------------------
 * sparse_topk_decode_attn — topk_select of one score row per (b, kvh) group followed by
 * sparse_decode_attn over the selected ids, in the attention's own launch.
 *
 * Passages: as for topk_select and sparse_decode_attn (SparDA, §2 "Seleção Esparsa de Lookahead
 * Treinável": the predictor's top-k blocks are the ones attention reads).  The selection is
 * exactly topk_select of the score row (ties to the lowest index); the attention is exactly
 * sparse_decode_attn with scope PER_KV_HEAD and T = 1 over that selection, with the same
 * `gran`, sinks and recent window, so out and lse are bit-identical to the two calls.
 *
 *   scores   device fp32, row (b*Hkv + kvh) at scores + row*s_ld, entries [0, n_cand) read.
 *   k        ids kept per row (0 <= k <= 62).  n_cand <= 4096.
 *   q, kc, vc, strides, gran, n_sink, n_recent, shapes, n_tokens, sm_scale, out, lse: as
 *            sparse_decode_attn with T = 1 (bf16 q and caches only; no host pools).
 *   sel_idx  device int32 [B*Hkv, sel_ld] or NULL: receives the ascending selection.
 *   sel_count device int32 [B*Hkv] or NULL: receives min(k, n_cand).
 *   ws       device workspace of sparse_topk_decode_attn_workspace_size() bytes.
 * SPK_EUNSUPPORTED for other dtypes, n_cand > 4096 or k > 62.
 * ------------------------------------------------------------------------------------------ */
SPK_API spk_status sparse_topk_decode_attn_workspace_size(int B, int Hq, int Hkv, int d,
                                                          int n_tokens, int n_cand, int k,
                                                          int gran, int n_sink, int n_recent,
                                                          size_t* bytes);
SPK_API spk_status sparse_topk_decode_attn(const float* scores, int64_t s_ld, int n_cand, int k,
                                           const void* q, spk_dtype q_dtype,
                                           const void* kc, const void* vc, spk_dtype kv_dtype,
                                           int64_t kv_sb, int64_t kv_sh, int64_t kv_sn,
                                           int gran, int n_sink, int n_recent,
                                           int B, int Hq, int Hkv, int d, int n_tokens,
                                           float sm_scale, float* out, float* lse,
                                           int32_t* sel_idx, int32_t* sel_count, int64_t sel_ld,
                                           void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * importance_accumulate — cumulative attention importance, one decode step.
 *
 * Passage: "Nem Todos os Pensamentos Necessitam de HBM", §2 "Pontuação de Importância":
 * s_i += (1/|L|) Σ_ℓ (1/H) Σ_h α_ℓ,h[i], with α the attention probabilities of this step.
 * Here α_ℓ,h[u] = exp(logits[ℓ,b,h,u] - lse[ℓ,b,h]) for position u of sequence b's list;
 * tokens not in the list (evicted or not read) receive nothing.  One query token per
 * sequence (T = 1).
 *
 *   s        device fp32 [B, s_ld], updated in place for tokens sel_idx[b, u], u < count.
 *   sel_idx, sel_count  device int32 [B, sel_ld] / [B]: the per-sequence lists the
 *            attention read (PER_SEQ scope), strictly ascending.
 *   logits   device fp32 [L, B, Hq, logits_ld]: sparse_decode_attn's logits of each layer.
 *   lse      device fp32 [L, B, Hq].
 * ------------------------------------------------------------------------------------------ */
SPK_API spk_status importance_accumulate(float* s, int64_t s_ld, int B, int n_tokens,
                                         const int32_t* sel_idx, const int32_t* sel_count,
                                         int64_t sel_ld,
                                         const float* logits, int64_t logits_ld,
                                         const float* lse, int L, int Hq, void* stream);

/* ------------------------------------------------------------------------------------------
 * tier_classify — tiers by cumulative importance, sinks and recent window protected.
 *
 * Passages: "Nem Todos os Pensamentos Necessitam de HBM", §1 "Classificação de Quatro
 * Níveis" (T0 HBM: protected tokens and the most important; T1 host DDR at full precision,
 * fetched before attention; T2 kept at reduced precision, for instance 8 bits; T3 evicted for
 * good) and §4 (tiers are reassigned periodically; the period is the caller's loop).
 * Definition: protected = tokens [0, n_sink) and [n_tokens - n_recent, n_tokens) -> T0.  The
 * M other tokens are ranked by (live before evicted, s descending, index ascending; NaN ranks
 * with the evicted); rank < floor(M*t0_permille/1000) -> T0, rank < floor(M*t01_permille/1000)
 * -> T1, rank < floor(M*t012_permille/1000) -> T2, the rest -> T3 (t012_permille =
 * t01_permille: no T2).  An evicted token is always T3.
 *
 *   s        device fp32 [B, s_ld].
 *   t0_permille <= t01_permille <= t012_permille <= 1000, else SPK_EINVAL.
 *   evicted  device uint8 [B, ev_ld] or NULL: nonzero = evicted earlier (sticky).  On return,
 *            every token classified T3 has evicted = 1.
 *   tier     device uint8 [B, tier_ld]: 0 (T0), 1 (T1), 2 (T2) or 3 (T3) for tokens
 *            [0, n_tokens).
 *   sel_idx, sel_count  device int32 [B, sel_ld] / [B] or NULL: the ascending list of
 *            T0 ∪ T1 ∪ T2 tokens (the rows attention reads).  sel_ld >= n_tokens.
 *   ws       device workspace of at least tier_classify_workspace_size() bytes (NULL if 0).
 * ------------------------------------------------------------------------------------------ */
SPK_API spk_status tier_classify_workspace_size(int B, int n_tokens, size_t* bytes);
SPK_API spk_status tier_classify(const float* s, int64_t s_ld, int B, int n_tokens,
                                 int n_sink, int n_recent, int t0_permille, int t01_permille,
                                 int t012_permille, uint8_t* evicted, int64_t ev_ld,
                                 uint8_t* tier, int64_t tier_ld,
                                 int32_t* sel_idx, int32_t* sel_count, int64_t sel_ld,
                                 void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * residency_update — which rows of each sequence hold an HBM slot after a tier reassignment,
 * and the list of rows to copy there (differential prefetch).
 *
 * Passages: "Nem Todos os Pensamentos Necessitam de HBM", §1 "Classificação de Quatro Níveis"
 * (T0 stays in HBM; T1 lives in host DDR at full precision and reaches the attention from
 * there) and §4 "Implementação do Sistema" (periodic reassignment; asynchronous differential
 * prefetch: only newly promoted rows cross PCIe); "O Fim do Gargalo de Memória ...", "A
 * Inovação" (optional residency: rows stay in HBM while memory allows).  Reading taken: HBM
 * holds at most `capacity` rows of a sequence, in slots 0..capacity-1 shared by every layer and
 * KV head; every row also lives in host memory at its token index.  The resident set R is the
 * first min(capacity, |T0 ∪ T1|) rows of T0 ∪ T1 ranked by (tier ascending, s descending, index
 * ascending; NaN last in its tier).  A row of R that already holds a slot (0 <= loc < capacity)
 * keeps it; the other rows of R, in ascending token order, take the slots no kept row holds,
 * in ascending slot order, and are listed for the copy.  Afterwards loc[tok] = slot for tok in
 * R and ~tok otherwise, for tok < n_tokens — the form sparse_decode_attn's `loc` reads.
 *
 *   tier       device uint8 [B,tier_ld] from tier_classify (0, 1 or 3).
 *   s          device fp32 [B,s_ld] importance.
 *   loc        device int32 [B,loc_ld], in/out.  On entry the previous residency (start with
 *              ~tok everywhere); the slots held must be distinct (else a row may end up read
 *              from host memory).  Entries >= n_tokens are not touched.
 *   copy_tok, copy_slot  device int32 [B,copy_ld]: the r-th newly resident row and its slot,
 *              r < min(copy_count[b], copy_ld) (copy_ld >= capacity lists every copy).
 *   copy_count device int32 [B]: number of rows listed for the copy (the newly resident rows
 *              that received a slot: all of them when the slots held on entry are distinct).
 * Limits: n_tokens below 2^30 and capacity at most 131072 (SPK_EUNSUPPORTED).  Sequences of up
 * to 16384 tokens (with capacity <= 16384) keep their tokens in registers; longer ones are read
 * from memory chunk by chunk.  One launch, one workgroup per sequence; no workspace.
 * ------------------------------------------------------------------------------------------ */
SPK_API spk_status residency_update(const uint8_t* tier, int64_t tier_ld,
                                    const float* s, int64_t s_ld, int B, int n_tokens,
                                    int capacity, int32_t* loc, int64_t loc_ld,
                                    int32_t* copy_tok, int32_t* copy_slot, int64_t copy_ld,
                                    int32_t* copy_count, void* stream);

/* ------------------------------------------------------------------------------------------
 * residency_append — HBM slots for the rows each sequence gained since the last step.
 *
 * Passages: "Nem Todos os Pensamentos Necessitam de HBM", §1 "Classificação de Quatro Níveis"
 * (the recent window is protected, so a new row is T0, and T0 stays in HBM); "O Fim do Gargalo
 * de Memória ...", "A Inovação" (rows are kept in HBM while memory allows).  Reading taken: a
 * row's K/V are produced on the GPU, so the new rows [n_old, n_new), in ascending token order,
 * take the slots 0..capacity-1 that no row below n_old holds (0 <= loc < capacity), in
 * ascending slot order; rows left without a slot get loc = ~tok (read from host memory until
 * the next reassignment).
 *
 *   loc        device int32 [B, loc_ld] (loc_ld >= n_new), in/out: entries below n_old are read,
 *              entries [n_old, n_new) written.
 *   copy_tok, copy_slot  device int32 [B, copy_ld], copy_ld >= min(n_new - n_old, capacity): the
 *              r-th new row given a slot, and that slot (write its K/V there with
 *              residency_prefetch from the pools that produced it).
 *   copy_count device int32 [B]: the rows given a slot.
 * Limits: capacity <= 131072 (SPK_EUNSUPPORTED).  One launch, one workgroup per sequence.
 * ------------------------------------------------------------------------------------------ */
SPK_API spk_status residency_append(int32_t* loc, int64_t loc_ld, int B, int n_old, int n_new,
                                    int capacity, int32_t* copy_tok, int32_t* copy_slot,
                                    int64_t copy_ld, int32_t* copy_count, void* stream);

/* ------------------------------------------------------------------------------------------
 * residency_prefetch — copy the rows residency_update listed from the host pools into their
 * HBM slots, for every KV head of one layer (the differential prefetch of §4 "Implementação do
 * Sistema", "Nem Todos os Pensamentos Necessitam de HBM": rows cross PCIe only when they newly
 * need HBM; full precision, so the attention result is unchanged — Proposition 1).
 *
 *   k_host, v_host  the source pools: pinned host memory (hipHostMalloc'ed, read through its
 *              device alias) or device memory (rows produced on the GPU, see residency_append);
 *              other memory: SPK_EINVAL.  Row (b,kvh,tok) at k_host + b*host_sb + kvh*host_sh +
 *              tok*host_sn, tok < host_slots.
 *   k_hbm, v_hbm    device pools, row (b,kvh,slot) at k_hbm + b*hbm_sb + kvh*hbm_sh +
 *              slot*hbm_sn, slot < hbm_slots.  Strides in elements; rows 16-byte aligned.
 *   copy_tok, copy_slot, copy_ld, copy_count: as residency_update wrote them.
 *   max_copies upper bound on copy_count (sizes the launch; capacity is always enough).
 * Entries whose token or slot lies outside its pool are skipped.  One launch.
 * ------------------------------------------------------------------------------------------ */
SPK_API spk_status residency_prefetch(const void* k_host, const void* v_host,
                                      int64_t host_sb, int64_t host_sh, int64_t host_sn,
                                      int64_t host_slots, void* k_hbm, void* v_hbm,
                                      int64_t hbm_sb, int64_t hbm_sh, int64_t hbm_sn,
                                      int64_t hbm_slots, spk_dtype kv_dtype, int B, int Hkv, int d,
                                      const int32_t* copy_tok, const int32_t* copy_slot,
                                      int64_t copy_ld, const int32_t* copy_count, int max_copies,
                                      void* stream);

/* ------------------------------------------------------------------------------------------
 * residency_update_tiers — residency_update with the tiers' roles given: tier_classes holds 2
 * bits per tier code t = 0..3 (bits 2t, 2t+1): 0 = ranked first, 1 = ranked second, 2 or 3 =
 * never resident.  residency_update is tier_classes = 0xF4 (T0 first, then T1).  0xCF makes
 * every T2 row resident (T2 alone ranked, the others never): with a capacity of at least the
 * T2 count, the T2 rows hold distinct slots, a row that stays in T2 keeps its slot, and the
 * copy list names the rows new to T2 — the staging of the 8-bit tier (t2_fetch).  Arguments,
 * errors and limits otherwise as residency_update.
 * ------------------------------------------------------------------------------------------ */
SPK_API spk_status residency_update_tiers(const uint8_t* tier, int64_t tier_ld,
                                          const float* s, int64_t s_ld, int B, int n_tokens,
                                          int capacity, int tier_classes, int32_t* loc,
                                          int64_t loc_ld, int32_t* copy_tok, int32_t* copy_slot,
                                          int64_t copy_ld, int32_t* copy_count, void* stream);

/* ------------------------------------------------------------------------------------------
 * kv_quantize_int8 — the 8-bit copy of K or V rows that the T2 tier keeps.
 *
 * Passage: "Nem Todos os Pensamentos Necessitam de HBM", §1 "Classificação de Quatro Níveis"
 * (T2: low-importance rows on the CPU at reduced precision, for instance 8-bit quantization).
 * Reading taken (the pages name no scheme): per row (one token of one KV head), m = the
 * largest |x| over its finite elements; scale = fp32(m / 127); code = rint(fp32(x *
 * fp32(127 / m))), ties to even, clamped to [-127, 127]; non-finite elements get code 0; a row
 * with m = 0 gets codes 0 and scale 0.  IEEE fp32 division and multiplication.
 *
 *   src        rows (b, kvh, tok) at src + b*s_sb + kvh*s_sh + tok*s_sn, bf16 or fp32, device
 *              memory or pinned host memory; 16-byte aligned rows (strides multiples of 8).
 *   row_begin, row_end  the tokens [row_begin, row_end) quantized, for every (b, kvh).
 *   codes      int8 [B, Hkv, >= row_end, d] at codes + b*c_sb + kvh*c_sh + tok*c_sn (strides
 *              multiples of 8), device or pinned host memory.
 *   scales     fp32 [B, Hkv, >= row_end] at scales + b*sc_sb + kvh*sc_sh + tok, device or
 *              pinned host memory.
 * Errors: SPK_EINVAL (sizes, strides, alignment, memory HIP does not know), SPK_EUNSUPPORTED
 * (d, dtype).  One launch.
 * ------------------------------------------------------------------------------------------ */
SPK_API spk_status kv_quantize_int8(const void* src, spk_dtype src_dtype, int64_t s_sb,
                                    int64_t s_sh, int64_t s_sn, int B, int Hkv, int d,
                                    int row_begin, int row_end, int8_t* codes, int64_t c_sb,
                                    int64_t c_sh, int64_t c_sn, float* scales, int64_t sc_sb,
                                    int64_t sc_sh, void* stream);

/* ------------------------------------------------------------------------------------------
 * t2_fetch — bring the listed T2 rows of one layer back to bf16 in HBM staging rows.
 *
 * Passage: "Nem Todos os Pensamentos Necessitam de HBM", §1 (T2 rows are kept at 8 bits on the
 * CPU).  Row copy_tok[b, r] of the code pools (codes_k/codes_v with scale_k/scale_v, as
 * kv_quantize_int8 wrote them; device or pinned host memory, read through the device alias)
 * becomes bf16(fp32(code * scale)), rounded to nearest even, in row stage_base +
 * copy_slot[b, r] of the HBM pools k, v [B, Hkv, hbm_rows, d], for every KV head, for
 * r < min(copy_count[b], copy_ld, max_copies).  The copy list is the one
 * residency_update_tiers (tier_classes 0xCF) wrote.  Entries whose token is outside
 * [0, code_rows) or whose row is outside the pools are skipped.
 * Errors: SPK_EINVAL, SPK_EUNSUPPORTED (d not 64/128, pools not bf16).  One launch.
 * ------------------------------------------------------------------------------------------ */
SPK_API spk_status t2_fetch(const int8_t* codes_k, const int8_t* codes_v, int64_t c_sb,
                            int64_t c_sh, int64_t c_sn, const float* scale_k,
                            const float* scale_v, int64_t sc_sb, int64_t sc_sh, int64_t code_rows,
                            void* k, void* v, spk_dtype kv_dtype, int64_t kv_sb, int64_t kv_sh,
                            int64_t kv_sn, int64_t hbm_rows, int64_t stage_base, int B, int Hkv,
                            int d, const int32_t* copy_tok, const int32_t* copy_slot,
                            int64_t copy_ld, const int32_t* copy_count, int max_copies,
                            void* stream);

/* ------------------------------------------------------------------------------------------
 * t2_locations — the row locations the attention reads under a T2 tier: for tokens
 * [0, n_tokens) of each sequence, loc_out = stage_base + loc_t2 where tier == 2 and loc_t2 >= 0
 * (its staging row), else loc_res (its residency location: an HBM slot, or ~tok for the host
 * pool).  All arrays are device [B, *_ld] (uint8 tier, int32 locations).
 * Errors: SPK_EINVAL (sizes, row strides, stage_base + n_tokens beyond int32).  One launch.
 * ------------------------------------------------------------------------------------------ */
SPK_API spk_status t2_locations(const uint8_t* tier, int64_t tier_ld, const int32_t* loc_res,
                                int64_t res_ld, const int32_t* loc_t2, int64_t t2_ld,
                                int32_t* loc_out, int64_t out_ld, int B, int n_tokens,
                                int64_t stage_base, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SPK_H */
