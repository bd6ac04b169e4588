// sparse_decode_attn: gather the selected K/V rows once per GQA group and run exact softmax
// attention over them only.
//
// "Esparsidade de Contexto no Tempo de Inferência", §3C: decoding over a selection reads O(k·d)
// rows instead of O(N·d), and §2 "Implementação de Hardware": per-token, per-query and per-head
// irregular sparsity.  "O Fim do Gargalo de Memória ... Adaptive DHiSparse": exact fused
// retrieval of non-resident rows; queries verified together share the retrieval of missing rows.
// "Nem Todos os Pensamentos Necessitam de HBM", §3 Proposition 1: rows that come back from host
// memory at full precision contribute exactly what HBM rows would — the reduction order here
// never depends on where a row lives, so the output is bit-identical for any `loc`.
//
// Pipeline (all on one stream):
//  1. assemble  (only when a group has several selection lists, block granularity or forced
//     rows): one workgroup per (b, kvh) sets one bit per token in an LDS bitmap per list, ORs
//     the bitmaps and emits the ascending fetch list with a per-row mask of the lists holding it.
//  2. partial   split-K over the fetch list: workgroup (split, group) walks rows
//     [split*R, split*R + R) and scores every query vector of the group (G heads x T tokens)
//     against each fetched row, so a row is read from HBM (or host memory) once per group.
//     Online softmax in fp32 (exp2 domain); the waves merge at the end and the split's
//     (m, l, acc) go to the workspace.  bf16 caches with bf16 queries run Q·K on MFMA; fp32 on
//     the VALU.
//  3. combine   one wave per query vector merges the group's splits in split order
//     (deterministic, no atomics) into out and lse.  A separate launch: merging inside the
//     partial kernel needs a device-scope release per workgroup, which writes back the XCD's
//     whole L2 and costs far more than this launch.
#include <mutex>
#include <type_traits>

#include "select_common.h"

namespace spk {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kAsmThreads = 1024;
constexpr int kAsmLdsWords = 26624;  // 104 KB of LDS bitmaps; larger ones live in the workspace
constexpr int kAsmStaticLds = 48 * 1024;  // the assembly kernel's static LDS, rounded up
constexpr int kMaxIntervals = 64;   // selection entries + 2 forced ranges, one per lane
constexpr int kScoresMax = 4096;    // candidates per score row selected inside the attention
constexpr int kMaxRows = 8192;      // rows per split (LDS slot table)
constexpr int kTabPad = 512;        // slot-table entries past a split's rows (dead padding)
constexpr int kDead = INT32_MIN;    // row-table entry of a row that is not read

struct Plan {
  int groups = 0, sets = 1, nq = 0, nq_pad = 0, ubound = 0, R = 0, smax = 0, words = 0;
  bool assemble = false, intervals = false, mask = false, bm_lds = true;
  size_t off_list = 0, off_mask = 0, off_count = 0, off_bm = 0, off_ml = 0, off_acc = 0,
         bytes = 0;
};

int pad_nq(int nq) { return nq <= 1 ? 1 : nq <= 2 ? 2 : nq <= 4 ? 4 : nq <= 8 ? 8 : 16; }

// Resources of the bf16 (MFMA) partial kernel of a configuration: resident workgroups per CU
// without dynamic LDS, and its static LDS bytes (queried once per configuration).
struct PartialInfo {
  int occ = 2;
  size_t static_lds = 0;
};
PartialInfo partial_info(int d, int nq_pad, bool mask, int mode);
size_t lds_per_cu();
size_t lds_per_block();

#ifndef SPK_ATTN_WG_ROWS
#define SPK_ATTN_WG_ROWS 128  // fixed cost of a split (set-up, merge), in rows of streaming
#endif

// Dynamic LDS of a partial workgroup: the slot table (and list masks) for R rows plus padding.
inline size_t table_bytes(int R, bool mask) { return (size_t)(R + kTabPad) * 4 * (mask ? 2 : 1); }

// Fetch-list strategy, split size and workspace layout of one call.  A group with one selection
// list expands it in the partial kernel itself (intervals mode) when the list is short; several
// lists per group (per-head or per-token sets) are merged by the assemble kernel first.
//
// Split size: R rows (a multiple of 64) per split, chosen to minimise
// rounds(R) * (R + fixed cost), where rounds(R) is how many times the group's splits fill every
// CU's resident workgroup slots (at the occupancy the slot table's LDS allows).  Workgroups
// then see the same amount of work and the last round is not left half empty.
// pre_ld > 0: the caller hands over each group's fetch list already assembled (ascending rows,
// a set mask per row, at most pre_ld rows); nothing is assembled and the workspace holds only
// the split partials.
Plan make_plan(spk_sel_scope scope, int B, int T, int Hq, int Hkv, int d, int n_tokens,
               int64_t sel_ld, int gran, int n_sink, int n_recent, bool from_scores = false,
               int64_t pre_ld = 0) {
  Plan p;
  const int G = Hq / Hkv;
  p.groups = B * Hkv;
  p.sets = scope == SPK_SEL_PER_SEQ ? 1 : scope == SPK_SEL_PER_KV_HEAD ? T : T * G;
  p.nq = G * T;
  p.nq_pad = pad_nq(p.nq);
  p.mask = p.sets > 1;
  const bool expand = gran > 1 || n_sink > 0 || n_recent > 0;
  // a selection made from scores inside the attention is always expanded there
  p.intervals = pre_ld == 0 && p.sets == 1 && (expand || from_scores) && sel_ld + 2 <= 64;
  p.assemble = pre_ld == 0 && (p.sets > 1 || (expand && !p.intervals));
  int64_t ub = pre_ld > 0 ? pre_ld : (int64_t)p.sets * sel_ld * gran + n_sink + n_recent;
  if (ub > n_tokens) ub = n_tokens;
  p.ubound = (int)ub;
  const PartialInfo info = partial_info(d, p.nq_pad, p.mask, p.intervals ? 1 : 0);
  const int64_t cus = num_cus();
  const size_t lds_cu = lds_per_cu(), lds_wg = lds_per_block();
  const int ubound = p.ubound > 0 ? p.ubound : 1;
  int best_R = 64;
  double best = -1.0;
  for (int R = 64; R <= kMaxRows; R += 64) {
    const size_t lds = info.static_lds + table_bytes(R, p.mask);
    if (lds > lds_wg && R > 64) break;
    int occ = (int)(lds_cu / (lds > 0 ? lds : 1));
    if (occ > info.occ) occ = info.occ;
    if (occ < 1) occ = 1;
    const int64_t wgs = (int64_t)p.groups * ceil_div(ubound, R);
    const int64_t rounds = ceil_div(wgs, (int64_t)occ * cus);
    const double cost = (double)rounds * (double)(R + SPK_ATTN_WG_ROWS);
    if (best < 0 || cost < best) {
      best = cost;
      best_R = R;
    }
    if (R >= ubound) break;
  }
  p.R = best_R;
  p.smax = (int)ceil_div(ubound, p.R);
  p.words = (int)ceil_div(n_tokens > 0 ? n_tokens : 1, 32);
  p.bm_lds = (int64_t)p.sets * p.words <= kAsmLdsWords &&
             (size_t)p.sets * p.words * 4 + kAsmStaticLds <= lds_wg;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  if (p.assemble) {
    p.off_list = take((size_t)p.groups * p.ubound * 4);
    p.off_mask = take(p.mask ? (size_t)p.groups * p.ubound * 4 : 0);
    p.off_bm = take(p.bm_lds ? 0 : (size_t)p.groups * p.sets * p.words * 4);
  }
  if (p.assemble || p.intervals) p.off_count = take((size_t)p.groups * 4);
  p.off_ml = take((size_t)p.groups * p.smax * p.nq_pad * 2 * 4);
  p.off_acc = take((size_t)p.groups * p.smax * p.nq_pad * d * 4);
  p.bytes = off;
  return p;
}

// ------------------------------------------------------------------------------- assemble

struct AsmArgs {
  const int32_t* sel_idx;
  const int32_t* sel_count;
  int64_t sel_ld;
  int scope, gran, n_sink, n_recent, T, Hq, Hkv, G, sets, n_tokens, words, ubound;
  uint32_t* bm_global;
  int32_t* ulist;
  uint32_t* umask;
  int32_t* ucount;
};

// kLds: the bitmaps live in (dynamic) LDS.  The two cases are separate instantiations so the
// LDS case uses LDS instructions: through one generic pointer every bitmap access is a flat
// access whose wait also covers the list stores in flight, which serialises the compaction.
//
// One workgroup per group does all of the group's work, so the kernel is bound by instruction
// issue on a few CUs and every phase keeps its lanes busy: (1) the sets' list lengths; (2) per
// set, kAsmBatch entries per thread are read at once (clamped addresses, one wait) and their
// bits set; (3) forced rows; (4) wave v owns a contiguous run of bitmap words, 64 at a time (lane
// l: word base + l); the lanes' entry offsets, union words and set words go to LDS, and then
// every lane produces one output entry: each word's first entry marks its lane in a 64-slot
// table, a wave prefix maximum gives every entry the lane (word) holding it, and a popcount
// search the bit, so the list is written with full, consecutive stores (per-wave totals give
// each wave its output offset).
constexpr int kAsmBatch = 4;
constexpr int kAsmSets = 16;     // sets per group the kernel handles (G * T <= 16)
constexpr int kAsmRegSets = 8;   // up to this many sets, a word's set bitmaps are staged

// Position of the k-th set bit (k < popcount(u)) of u, by halving popcount search.
__device__ __forceinline__ int nth_set_bit(uint32_t u, int k) {
  int pos = 0;
#pragma unroll
  for (int width = 16; width > 0; width >>= 1) {
    const uint32_t low = u & ((1u << width) - 1u);
    const int c = __popc(low);
    const bool up = k >= c;
    k -= up ? c : 0;
    pos += up ? width : 0;
    u = up ? (u >> width) : low;
  }
  return pos;
}

template <bool kLds>
__global__ __launch_bounds__(kAsmThreads) void assemble_kernel(AsmArgs a) {
  constexpr int NWV = kAsmThreads / kWave;
  extern __shared__ uint32_t bm_dyn[];
  __shared__ int scratch[NWV];
  __shared__ int set_off[kAsmSets + 1];   // first entry of each set in a flat numbering
  __shared__ int64_t set_row[kAsmSets];   // offset of each set's list row in sel_idx
  __shared__ int st_pre[NWV][kWave];      // per lane: first entry of its word in the batch
  __shared__ uint32_t st_u[NWV][kWave];   // per lane: its word of the union
  __shared__ uint32_t st_sw[NWV][kAsmRegSets][kWave];  // per lane: its word of every set
  __shared__ int st_own[NWV][kWave];      // per output slot of a chunk: the lane starting there
  const int g = blockIdx.x;
  const int b = g / a.Hkv, kvh = g % a.Hkv;
  const int W = a.words, S = a.sets;
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  uint32_t* bm;
  if constexpr (kLds) bm = bm_dyn;
  else bm = a.bm_global + (int64_t)g * S * W;
  for (int i = threadIdx.x; i < S * W; i += kAsmThreads) bm[i] = 0u;
  // (1) wave 0: lane r reads set r's count (the host bounds the total below 2^31)
  if (wid == 0) {
    int len = 0;
    if (lane < S) {
      const int r = lane;
      int64_t row;
      if (a.scope == SPK_SEL_PER_SEQ) row = b;
      else if (a.scope == SPK_SEL_PER_KV_HEAD) row = (int64_t)(b * a.T + r) * a.Hkv + kvh;
      else row = (int64_t)(b * a.T + r / a.G) * a.Hq + kvh * a.G + r % a.G;
      const int cnt = max(0, min(a.sel_count[row], (int)a.sel_ld));
      len = cnt * a.gran;
      set_row[r] = row * a.sel_ld;
    }
    const int incl = wave_incl_scan(len);
    if (lane <= S) set_off[lane] = incl - len;
  }
  __syncthreads();
  const int n = a.n_tokens, gran = a.gran;
  // (2) the selected tokens' bits, set by set, kAsmBatch entries per thread in flight
  for (int r = 0; r < S; ++r) {
    const int len = set_off[r + 1] - set_off[r];
    const int32_t* lst = a.sel_idx + set_row[r];
    for (int e0 = threadIdx.x; e0 < len; e0 += kAsmBatch * kAsmThreads) {
      int32_t ent[kAsmBatch];
#pragma unroll
      for (int u = 0; u < kAsmBatch; ++u) {
        const int e = min(e0 + u * kAsmThreads, len - 1);
        ent[u] = lst[gran == 1 ? e : e / gran];
      }
#pragma unroll
      for (int u = 0; u < kAsmBatch; ++u) {
        const int e = e0 + u * kAsmThreads;
        if (e < len) {
          const int64_t tok = (int64_t)ent[u] * gran + (gran == 1 ? 0 : e % gran);
          if (tok >= 0 && tok < n) atomicOr(&bm[r * W + (int)(tok >> 5)], 1u << (tok & 31));
        }
      }
    }
  }
  // (3) forced rows belong to every list
  const int s_end = min(a.n_sink, n);
  const int r_beg = max(0, n - a.n_recent);
  for (int tok = threadIdx.x; tok < s_end + (n - r_beg); tok += kAsmThreads) {
    const int t = tok < s_end ? tok : r_beg + (tok - s_end);
    for (int r = 0; r < S; ++r) atomicOr(&bm[r * W + (t >> 5)], 1u << (t & 31));
  }
  __syncthreads();
  // (4) compaction: wave wid owns words [wb, we), 64 at a time
  const int wpw = (W + NWV * kWave - 1) / (NWV * kWave) * kWave;
  const int wb = min(W, wid * wpw), we = min(W, wb + wpw);
  auto union_word = [&](int w) {
    uint32_t u = 0;
    if (w < we)
      for (int r = 0; r < S; ++r) u |= bm[r * W + w];
    return u;
  };
  int cnt = 0;
  for (int w0 = wb; w0 < we; w0 += kWave) cnt += __popc(union_word(w0 + lane));
  // wave totals -> each wave's first output position
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, kWave);
  if (lane == 0) scratch[wid] = cnt;
  __syncthreads();
  int run = 0, total_u = 0;
  for (int v = 0; v < NWV; ++v) {
    const int c = scratch[v];
    run += v < wid ? c : 0;
    total_u += c;
  }
  int32_t* ul = a.ulist + (int64_t)g * a.ubound;
  uint32_t* um = a.umask ? a.umask + (int64_t)g * a.ubound : nullptr;
  const bool reg_sets = S <= kAsmRegSets;
  for (int w0 = wb; w0 < we; w0 += kWave) {
    const int w = w0 + lane;
    uint32_t sw[kAsmRegSets];
    uint32_t u = 0;
#pragma unroll
    for (int r = 0; r < kAsmRegSets; ++r) sw[r] = 0u;
    if (w < we) {
      if (reg_sets) {
        // every set word read before any is used: one wait
#pragma unroll
        for (int r = 0; r < kAsmRegSets; ++r) sw[r] = r < S ? bm[r * W + w] : 0u;
#pragma unroll
        for (int r = 0; r < kAsmRegSets; ++r) u |= sw[r];
      } else {
        for (int r = 0; r < S; ++r) u |= bm[r * W + w];
      }
    }
    const int c = __popc(u);
    const int incl = wave_incl_scan(c);
    const int btot = __builtin_amdgcn_readlane(incl, kWave - 1);
    const int pre = incl - c;  // this lane's first entry within the batch
    if (reg_sets) {
#pragma unroll
      for (int r = 0; r < kAsmRegSets; ++r)
        if (r < S) st_sw[wid][r][lane] = sw[r];
    }
    st_pre[wid][lane] = pre;
    st_u[wid][lane] = u;
    int carry = 0;  // the lane holding the entry before the current chunk
    for (int i0 = 0; i0 < btot; i0 += kWave) {
      st_own[wid][lane] = -1;
      __builtin_amdgcn_wave_barrier();
      if (c > 0 && pre >= i0 && pre < i0 + kWave) st_own[wid][pre - i0] = lane;
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      const int o = max(wave_incl_max(st_own[wid][lane]), carry);
      carry = __builtin_amdgcn_readlane(o, kWave - 1);
      const int i = i0 + lane;
      if (i < btot) {
        const uint32_t uo = st_u[wid][o];
        const int bit = nth_set_bit(uo, i - st_pre[wid][o]);
        const int pos = run + i;
        if (pos < a.ubound) {
          ul[pos] = (w0 + o) * 32 + bit;
          if (um) {
            uint32_t m = 0;
            if (reg_sets) {
              uint32_t x[kAsmRegSets];
#pragma unroll
              for (int r = 0; r < kAsmRegSets; ++r) x[r] = r < S ? st_sw[wid][r][o] : 0u;
#pragma unroll
              for (int r = 0; r < kAsmRegSets; ++r) m |= ((x[r] >> bit) & 1u) << r;
            } else {
              for (int r = 0; r < S; ++r) m |= ((bm[r * W + w0 + o] >> bit) & 1u) << r;
            }
            um[pos] = m;
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");  // slots read before reuse
      __builtin_amdgcn_wave_barrier();
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    run += btot;
  }
  if (threadIdx.x == 0) a.ucount[g] = min(total_u, a.ubound);
}

// ------------------------------------------------------------------------------- partial

// How a partial workgroup learns the rows of its group's fetch list.
enum ListMode {
  kListExplicit = 0,   // list + count (caller's list, or the assembled one)
  kListIntervals = 1,  // one selection row of ids expanded by `gran`, plus sinks and recent window
  kListScores = 2,     // the ids are the top-k of the group's score row (order as kListVirtual)
  kListVirtual = 3,    // the sinks, then the recent window, then one selection row of ids
                       // expanded by `gran` in list order; rows an earlier part holds are dead
};

struct AttnArgs {
  const void* q;
  int q_bf16;
  const void* k;
  const void* v;
  int64_t kv_sb, kv_sh, kv_sn;
  const void* k_host;
  const void* v_host;
  int64_t host_sb, host_sh, host_sn, host_slots;
  const int32_t* loc;
  int64_t loc_sb, loc_sh, hbm_slots;
  // explicit mode: rows of group g are list[lrow*list_ld + i], i < min(count[lrow], count_clamp)
  // intervals mode: ids sel[lrow*list_ld + i], i < min(count[lrow], list_ld), expanded by gran
  // lrow = b (PER_SEQ) or g
  const int32_t* list;
  const int32_t* count;
  int64_t list_ld;
  int count_clamp;
  int lrow_is_batch;
  int list_mode;
  int gran, n_sink, n_recent;
  int32_t* ucount;       // per-group fetch-list length (written by assemble or intervals mode)
  int ucount_valid;      // ucount holds the lengths (assembled lists)
  int split_bound;       // > 0: rows per split come from this bound, not from the group's count
  const uint32_t* mask;  // per fetch-list row (assembled lists with several sets)
  int mask_div;          // query vector n reads rows whose mask has bit n / mask_div
  int T, Hq, Hkv, G, nq, n_tokens, smax;
  int tab_cap;           // slot-table entries of the dynamic LDS (plan R + padding)
  float scale_log2;
  float* ml;
  float* acc;
  float* logits;
  int64_t logits_ld;
  int logits_vec;        // logits rows are 16-byte aligned (base and row stride)
  // kListScores: score row g at sc_scores + g*sc_ld, sc_n candidates, keep sc_k; the selection
  // is also written to sel_out row g (sel_out_ld) and count_out[g] when those are given
  const float* sc_scores;
  int64_t sc_ld;
  int sc_n, sc_k;
  int32_t* sel_out;
  int32_t* count_out;
  int64_t sel_out_ld;
};

// End of a partial workgroup: merge the 4 waves' (m, l, acc) from `red` and store this split's
// partial for the combine kernel.
template <int D, int NQ, int NW>
__device__ void finish_split(const AttnArgs& a, float (&red)[NW][NQ][D + 2], int g, int split) {
  const int64_t pbase = ((int64_t)g * a.smax + split) * NQ;
  for (int e = threadIdx.x; e < NQ * D; e += kThreads) {
    const int n = e / D, dim = e % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, red[w][n][0]);
    float ls = 0.f, as = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sc = (mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(red[w][n][0] - mx);
      ls += red[w][n][1] * sc;
      as += red[w][n][2 + dim] * sc;
    }
    a.acc[(pbase + n) * D + dim] = as;
    if (dim == 0) {
      a.ml[(pbase + n) * 2] = mx;
      a.ml[(pbase + n) * 2 + 1] = ls;
    }
  }
}

// Where token `tok` of group (b, kvh) lives: HBM slot (>= 0) or host slot (encoded ~slot < 0);
// kDead when the slot lies outside its pool (the row is then not read).
__device__ __forceinline__ int resolve_slot(const AttnArgs& a, int b, int kvh, int tok) {
  if (tok < 0 || tok >= a.n_tokens) return kDead;
  if (!a.loc) return tok;
  const int l = a.loc[(int64_t)b * a.loc_sb + (int64_t)kvh * a.loc_sh + tok];
  const bool ok = l >= 0 ? (int64_t)l < a.hbm_slots : (int64_t)(~l) < a.host_slots;
  return ok ? l : kDead;
}

// A readable, all-zero row: rows that are not read load from here, so every load in the main
// loop is issued unconditionally (no divergent branches between loads and their waits).
__device__ __align__(64) uint32_t g_zero_row[128];

// Rows per split of a group with `cnt` fetch-list rows: the group's rows spread evenly over the
// plan's smax splits (a multiple of 16, at most the plan's R).  Partial and combine kernels agree
// on it.
__device__ __forceinline__ int split_rows(int cnt, int smax) {
  const int r = (cnt + smax - 1) / smax;
  return (r + 15) & ~15;
}

// Byte addresses of a row's K and V from its slot (see resolve_slot): one select of base and
// stride, one 32x32->64-bit multiply-add (row strides are below 4 GiB, checked on the host).
struct RowBase {
  uint64_t k_hbm, k_host, dv_hbm, dv_host, zero;
  uint32_t sn_hbm, sn_host;  // row strides in bytes
};
__device__ __forceinline__ void row_addr(RowBase rb, int slot, uint64_t& ka, uint64_t& va) {
  // selects on values (not on members through a reference, which the compiler may turn into a
  // select of addresses into private memory)
  const uint64_t k_hbm = rb.k_hbm, k_host = rb.k_host, zero = rb.zero;
  const uint64_t dv_hbm = rb.dv_hbm, dv_host = rb.dv_host;
  const uint32_t sn_hbm = rb.sn_hbm, sn_host = rb.sn_host;
  const bool hbm = slot >= 0, dead = slot == kDead;
  const uint32_t idx = hbm ? (uint32_t)slot : (uint32_t)(~slot);
  uint32_t sn = hbm ? sn_hbm : sn_host;
  sn = dead ? 0u : sn;
  uint64_t base = hbm ? k_hbm : k_host;
  base = dead ? zero : base;
  uint64_t dv = hbm ? dv_hbm : dv_host;
  dv = dead ? 0ull : dv;
  ka = base + (uint64_t)idx * sn;
  va = ka + dv;
}

template <typename KT>
__device__ __forceinline__ RowBase make_row_base(const AttnArgs& a, int b, int kvh) {
  RowBase rb;
  rb.k_hbm = reinterpret_cast<uint64_t>(a.k) +
             (uint64_t)(((int64_t)b * a.kv_sb + (int64_t)kvh * a.kv_sh) * (int64_t)sizeof(KT));
  rb.k_host = reinterpret_cast<uint64_t>(a.k_host) +
              (uint64_t)(((int64_t)b * a.host_sb + (int64_t)kvh * a.host_sh) * (int64_t)sizeof(KT));
  rb.dv_hbm = reinterpret_cast<uint64_t>(a.v) - reinterpret_cast<uint64_t>(a.k);
  rb.dv_host = reinterpret_cast<uint64_t>(a.v_host) - reinterpret_cast<uint64_t>(a.k_host);
  rb.zero = reinterpret_cast<uint64_t>(g_zero_row);
  rb.sn_hbm = (uint32_t)(a.kv_sn * (int64_t)sizeof(KT));
  rb.sn_host = (uint32_t)(a.host_sn * (int64_t)sizeof(KT));
  return rb;
}


__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave 0: the ascending union of the selection row's expanded intervals, the sinks [0, s) and
// the recent window [n - r, n) as <= 64 disjoint segments (start, first position); returns the
// union size through *U.  Selection ids must be ascending (as topk_select writes them); ids that
// expand outside [0, n) give empty intervals.
__device__ void build_segments(const AttnArgs& a, const int32_t* sel, const int32_t* count_ptr,
                               int* seg_start, int* seg_pos, int* nseg, int* U) {
  const int lane = lane_id();
  const int n = a.n_tokens;
  const int rs = max(0, n - a.n_recent);
  // the list entries and their count load together (entries past the count are ignored)
  const int cmax = (int)min<int64_t>(a.list_ld, kMaxIntervals - 2);
  int64_t e_sel = -1;
  if (lane >= 1 && lane <= cmax) e_sel = sel[lane - 1];
  const int cnt = max(0, min(*count_ptr, cmax));
  // interval of this lane: 0 = sinks, 1..cnt = selection entries, cnt+1 = recent window
  int lo = n, hi = n;
  bool is_sel = false;
  if (lane == 0) {
    lo = 0;
    hi = min(a.n_sink, n);
  } else if (lane <= cnt) {
    const int64_t e = e_sel;
    const int64_t s0 = e * a.gran;
    lo = (int)min<int64_t>(max<int64_t>(s0, 0), n);
    hi = (int)min<int64_t>(max<int64_t>(s0 + a.gran, 0), n);
    if (e < 0) lo = hi = n;
    is_sel = true;
  } else if (lane == cnt + 1) {
    lo = rs;
    hi = n;
  }
  // order by start: selection entries are ascending; the recent window slots in among them
  const uint64_t before_rs = __ballot(is_sel && lo < rs);
  const int n_before = __popcll(before_rs);
  int rank;
  if (lane == 0) rank = 0;
  else if (is_sel) rank = lane + (lo < rs ? 0 : 1);
  else if (lane == cnt + 1) rank = 1 + n_before;
  else rank = lane;  // unused lanes keep their place (empty intervals at n)
  const int total = cnt + 2;
  int* ord_lo = seg_start;  // reuse the output arrays as sort scratch
  int* ord_hi = seg_pos;
  if (lane < total) {
    ord_lo[rank] = lo;
    ord_hi[rank] = hi;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  int mlo = n, mhi = n;
  if (lane < total) {
    mlo = ord_lo[lane];
    mhi = ord_hi[lane];
  }
  // part of this interval not covered by earlier ones
  int run_end = mhi;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(run_end, o, kWave);
    if (lane >= o) run_end = max(run_end, y);
  }
  int prev_end = __shfl_up(run_end, 1, kWave);
  if (lane == 0) prev_end = 0;
  const int st = max(mlo, prev_end);
  const int len = lane < total ? max(0, mhi - st) : 0;
  const int incl = wave_incl_scan(len);
  __builtin_amdgcn_wave_barrier();
  if (lane < total) {
    seg_start[lane] = st;
    seg_pos[lane] = incl - len;
  }
  if (lane == kWave - 1) {
    *U = incl;
    *nseg = total;
  }
}

// Token at union position p (0 <= p < U): the last segment whose first position is <= p.
__device__ __forceinline__ int token_at(const int* seg_start, const int* seg_pos, int nseg, int p) {
  int lo = 0, hi = nseg;  // find the last index with seg_pos <= p
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (seg_pos[mid] <= p) lo = mid;
    else hi = mid;
  }
  return seg_start[lo] + (p - seg_pos[lo]);
}

// Position layout of a kListVirtual / kListScores fetch list: the forced rows first (the sinks
// [0, ns), then the recent window [rs, n)), then the selection's ids in list order, each expanded
// to `gran` tokens.  With the forced rows in front, a split that holds only them depends on no
// selection and starts reading at once.  A token that an earlier part also holds (recent rows
// inside the sinks, block rows inside the sinks or the recent window) or that lies outside
// [0, n) is dead (-1), so each row is read once.
__device__ __forceinline__ int forced_rows(int ns, int rs, int n) { return ns + (n - rs); }

// Token at position p; `entry` is the list entry covering p (ignored for forced positions).
__device__ __forceinline__ int virtual_token(int p, int gran, int entry, int ns, int rs, int n) {
  if (p < ns) return p;
  const int nf = forced_rows(ns, rs, n);
  if (p < nf) {
    const int tok = rs + (p - ns);
    return tok < ns ? -1 : tok;
  }
  const int64_t tok = (int64_t)entry * gran + (p - nf) % gran;
  return (entry < 0 || tok >= n || tok < ns || tok >= rs) ? -1 : (int)tok;
}

// Rows of a kListVirtual / kListScores fetch list with n_sel ids.
__device__ __forceinline__ int virtual_rows(int n_sel, int gran, int ns, int rs, int n) {
  return forced_rows(ns, rs, n) + n_sel * gran;
}

// Fill the split's slot table (and per-row list masks) in LDS: entries [0, nrows) are the
// split's rows, entries up to tab_rows are dead (they read the zero row).
template <int MODE, bool kMask>
__device__ __forceinline__ void fill_slot_table(const AttnArgs& a, int b, int kvh, int g, int lrow,
                                                int r0, int nrows, int tab_rows, int32_t* slot_s,
                                                uint32_t* mask_s, const int* seg_start,
                                                const int* seg_pos, int nseg,
                                                const int32_t* vlist = nullptr, int n_sel = 0,
                                                const int* pre_e = nullptr, int n_pre = 0) {
  const int32_t* list = a.list + (int64_t)lrow * a.list_ld;
  const uint32_t* mrow = kMask ? a.mask + (int64_t)g * a.list_ld : nullptr;
  const int n = a.n_tokens;
  const int ns = min(a.n_sink, n), rs = max(n - a.n_recent, 0);
  for (int it = 0, i = threadIdx.x; i < tab_rows; ++it, i += kThreads) {
    int slot_v = kDead;
    if (i < nrows) {
      int tok;
      if constexpr (MODE == kListVirtual || MODE == kListScores) {
        const int p = r0 + i;
        const int ps = p - forced_rows(ns, rs, n);  // position in the selection part
        // pre_e[it]: the entry of row r0 + threadIdx.x + it*kThreads, read earlier
        const int e = it < n_pre ? (it == 0 ? pre_e[0] : pre_e[1])
                                 : (ps >= 0 && ps < n_sel * a.gran ? vlist[ps / a.gran] : 0);
        tok = virtual_token(p, a.gran, e, ns, rs, n);
      } else if constexpr (MODE == kListIntervals) {
        tok = token_at(seg_start, seg_pos, nseg, r0 + i);
      } else {
        tok = list[r0 + i];
      }
      slot_v = resolve_slot(a, b, kvh, tok);
    }
    slot_s[i] = slot_v;
    if constexpr (kMask) mask_s[i] = i < nrows ? mrow[r0 + i] : 0u;
  }
}

#ifndef SPK_ATTN_MIN_WAVES
#define SPK_ATTN_MIN_WAVES 2  // register budget: at least this many waves per SIMD
#endif
template <int D, typename KT, int NQ, bool kMask, int MODE, int U>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(SPK_ATTN_MIN_WAVES))) void attn_partial_kernel(AttnArgs a) {
  constexpr int LPR = D / 8;             // lanes per row
  constexpr int SPW = kWave / LPR;       // slots (rows) per wave
  constexpr int NSLOT = SPW * kWaves;    // slots per workgroup
  constexpr int STEP = NSLOT * U;        // rows per workgroup per iteration
  static_assert(3 * STEP <= kTabPad, "slot table padding");
  __shared__ float red[kWaves][NQ][D + 2];
  __shared__ int seg_start[kMaxIntervals], seg_pos[kMaxIntervals], seg_meta[2];
  // row slots (HBM slot, ~host slot, or dead: read the zero row), padded past the last row so
  // every issue in the main loop is unconditional; then the per-row list masks
  extern __shared__ int32_t dyn_s[];
  int32_t* slot_s = dyn_s;
  uint32_t* mask_s = reinterpret_cast<uint32_t*>(dyn_s + a.tab_cap);

  const int g = blockIdx.y;
  const int split = blockIdx.x;
  const int b = g / a.Hkv, kvh = g % a.Hkv;
  const int lrow = a.lrow_is_batch ? b : g;
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  const int sub = lane % LPR, slot = lane / LPR;
  const int sid = wid * SPW + slot;

  int cnt;
  if constexpr (MODE == kListIntervals) {
    if (wid == 0)
      build_segments(a, a.list + (int64_t)lrow * a.list_ld, a.count + lrow, seg_start, seg_pos,
                     &seg_meta[0], &seg_meta[1]);
    __syncthreads();
    cnt = seg_meta[1];
    if (split == 0 && threadIdx.x == 0) a.ucount[g] = cnt;
  } else {
    cnt = a.count[lrow];
    cnt = max(0, min(cnt, a.count_clamp));
  }
  const int rs = split_rows(cnt, a.smax);
  const int r0 = split * rs;
  if (r0 >= cnt) return;
  const int r1 = min(r0 + rs, cnt);
  const int nrows = r1 - r0;

  const int iters = (nrows + STEP - 1) / STEP;
  const int tab_rows = (iters + 2) * STEP;
  const RowBase rbase = make_row_base<KT>(a, b, kvh);
  fill_slot_table<MODE, kMask>(a, b, kvh, g, lrow, r0, nrows, tab_rows, slot_s, mask_s, seg_start,
                               seg_pos, seg_meta[0]);

  // query slices, pre-scaled into the exp2 domain
  float qs[NQ][8];
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    if (n < a.nq) {
      const int t = n / a.G, hl = n % a.G;
      const int64_t off = ((int64_t)(b * a.T + t) * a.Hq + kvh * a.G + hl) * D + sub * 8;
      if (a.q_bf16) load8f(reinterpret_cast<const uint16_t*>(a.q) + off, qs[n]);
      else load8f(reinterpret_cast<const float*>(a.q) + off, qs[n]);
#pragma unroll
      for (int i = 0; i < 8; ++i) qs[n][i] *= a.scale_log2;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) qs[n][i] = 0.f;
    }
  }
  float m[NQ], l[NQ], acc[NQ][8];
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    m[n] = -INFINITY;
    l[n] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[n][i] = 0.f;
  }
  __syncthreads();

  const uint64_t col = (uint64_t)(sub * 8 * (int)sizeof(KT));
  auto issue = [&](int it, Raw8<KT> (&rk)[U], Raw8<KT> (&rv)[U], int (&sl)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) sl[u] = slot_s[it * STEP + u * NSLOT + sid];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint64_t ka, va;
      row_addr(rbase, sl[u], ka, va);
      rk[u].load_addr(ka + col);
      rv[u].load_addr(va + col);
    }
  };
  auto consume = [&](int it, const Raw8<KT> (&rk)[U], const Raw8<KT> (&rv)[U],
                     const int (&sl)[U]) {
    float lg[U][NQ];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = it * STEP + u * NSLOT + sid;
      uint32_t mb = 0xFFFFFFFFu;
      if constexpr (kMask) mb = mask_s[p];
      float x[8];
      rk[u].to_float(x);
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s = fmaf(qs[n][i], x[i], s);
        s = group_sum<LPR>(s);
        const bool reads = sl[u] != kDead && (!kMask || ((mb >> (n / a.mask_div)) & 1u));
        lg[u][n] = reads ? s : -INFINITY;
      }
      if (a.logits) {
        // lane `sub` writes query vector n = sub (and sub + LPR when NQ > LPR)
#pragma unroll
        for (int n0 = 0; n0 < NQ; n0 += LPR) {
          float val = lg[u][n0];
#pragma unroll
          for (int n = n0 + 1; n < n0 + LPR && n < NQ; ++n) val = (sub == n - n0) ? lg[u][n] : val;
          const int n = n0 + sub;
          if (p < nrows && n < a.nq) {
            const int t = n / a.G, hl = n % a.G;
            const int64_t row = (int64_t)(b * a.T + t) * a.Hq + kvh * a.G + hl;
            a.logits[row * a.logits_ld + r0 + p] = val * kLn2;
          }
        }
      }
    }
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      float mx = m[n];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, lg[u][n]);
      const float sc = (mx == -INFINITY) ? 0.f : fast_exp2(m[n] - mx);
      l[n] *= sc;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[n][i] *= sc;
      m[n] = mx;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float y[8];
      rv[u].to_float(y);
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        const float p = (m[n] == -INFINITY) ? 0.f : fast_exp2(lg[u][n] - m[n]);
        l[n] += p;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[n][i] = fmaf(p, y[i], acc[n][i]);
      }
    }
  };

  {
    Raw8<KT> k0[U], v0[U], k1[U], v1[U];
    int s0[U], s1[U];
    // software pipeline: the next batch's loads are in flight while this batch is consumed;
    // scheduling barriers keep the compiler from hoisting consumer work above the loads
    issue(0, k0, v0, s0);
    for (int it = 0; it < iters; it += 2) {
      issue(it + 1, k1, v1, s1);  // rows past the end read the zero row
      __builtin_amdgcn_sched_barrier(0);
      consume(it, k0, v0, s0);
      __builtin_amdgcn_sched_barrier(0);
      if (it + 1 >= iters) break;
      issue(it + 2, k0, v0, s0);
      __builtin_amdgcn_sched_barrier(0);
      consume(it + 1, k1, v1, s1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // merge the slots of this wave (lanes with equal `sub` hold the same dims)
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const float mo = __shfl_xor(m[n], off, kWave);
      const float lo = __shfl_xor(l[n], off, kWave);
      const float mx = fmaxf(m[n], mo);
      const float sa = (mx == -INFINITY) ? 0.f : fast_exp2(m[n] - mx);
      const float sb = (mx == -INFINITY) ? 0.f : fast_exp2(mo - mx);
      l[n] = l[n] * sa + lo * sb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float ao = __shfl_xor(acc[n][i], off, kWave);
        acc[n][i] = acc[n][i] * sa + ao * sb;
      }
      m[n] = mx;
    }
  }
  if (lane < LPR) {
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wid][n][2 + sub * 8 + i] = acc[n][i];
      if (sub == 0) {
        red[wid][n][0] = m[n];
        red[wid][n][1] = l[n];
      }
    }
  }
  __syncthreads();
  finish_split<D, NQ, kWaves>(a, red, g, split);
}

// ------------------------------------------------------------------------------- partial (MFMA)

// bf16 K/V and bf16 queries: both contractions run on the matrix cores.  Each wave owns 16-row
// tiles.
//  * Q·Kᵀ: one v_mfma_f32_16x16x32_bf16 per 32 dims takes A = the tile's K rows (lane l holds
//    16 bytes of row l%16) and B = the group's query vectors (query l%16), giving every lane the
//    logits of rows 4(l/16)..+3 for query l%16.  The online softmax runs in that layout.
//  * P·V: that layout is exactly the A operand of v_mfma_f32_16x16x16_bf16 (query l%16, rows
//    4(l/16)..+3), so the probabilities feed the matrix core where they are.  P is split into a
//    bf16 high part (truncation, exact) and a bf16 low part (the rounded remainder): two MFMAs
//    keep P to about 16 bits, and V is used exactly as stored.  The B operand (4 rows of one V
//    column per lane) comes from the tile staged row-major in LDS through the transposing read
//    ds_read_b64_tr_b16: lane s of each 16-lane group points at 4 consecutive columns of one row
//    and receives, per 16-lane group, the 4x4-transposed elements.
//  The output accumulates in MFMA layout (lane l: queries 4(l/16)..+3, dim l%16 of each
//  16-wide chunk).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#ifndef SPK_MFMA_MIN_WAVES
#define SPK_MFMA_MIN_WAVES 3
#endif

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

#ifndef SPK_MFMA_BATCH
#define SPK_MFMA_BATCH 2
#endif

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int D, int NQ, bool kMask, int MODE>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(SPK_MFMA_MIN_WAVES))) void attn_partial_mfma_kernel(AttnArgs a) {
  constexpr int BATCH = SPK_MFMA_BATCH;   // tiles in flight per wave
  constexpr int TILE = 16;                // rows per wave per step
  constexpr int STEP = TILE * kWaves;     // rows per workgroup per step
  constexpr int KCH = D / 32;             // Q·K MFMA k-chunks per row
  constexpr int DCH = D / 16;             // P·V MFMA output chunks (16 dims each)
  constexpr int LPR = D / 8;              // V load layout: lanes per row (16 bytes each)
  constexpr int RPI = kWave / LPR;        // V load layout: rows per instruction
  constexpr int PVI = TILE / RPI;         // V load instructions per tile
  constexpr int VST = D * 2 + 32;         // LDS row stride of a staged V tile (bytes)
  static_assert(NQ <= 16, "at most 16 query vectors per group");
  static_assert(BATCH <= 4 && 4 * STEP <= kTabPad, "slot table padding covers the last batch");
  // the staged V tiles (main loop) and the wave merge area (end) share one LDS block
  // kListScores: the score row's keys live in the same block before the main loop
  constexpr bool kSc = MODE == kListScores;
  constexpr int kRedBytes = kWaves * NQ * (D + 2) * 4;
  constexpr int kVtBytes = kWaves * TILE * VST;
  constexpr int kScBytes = kSc ? kScoresMax * 4 : 0;
  constexpr int kWorkBytes = kRedBytes > kVtBytes ? (kRedBytes > kScBytes ? kRedBytes : kScBytes)
                                                  : (kVtBytes > kScBytes ? kVtBytes : kScBytes);
  __shared__ __align__(16) unsigned char work_s[kWorkBytes];
  auto& red = *reinterpret_cast<float (*)[kWaves][NQ][D + 2]>(work_s);
  __shared__ int seg_start[kMaxIntervals], seg_pos[kMaxIntervals], seg_meta[2];
  // kListScores: one histogram per radix digit, per-wave counts and the selected ids
  __shared__ __align__(16) uint32_t sc_hist[kSc ? 4 * 256 : 4];
  constexpr int kScRegKeys = 4;  // score rows up to 4*256 candidates select from registers
  __shared__ __align__(16) int sc_wsum[kScRegKeys * kWaves];  // >= 2 * kWaves (LDS path)
  __shared__ int32_t sc_list[kSc ? kMaxIntervals : 1];
  extern __shared__ int32_t dyn_s[];
  int32_t* slot_s = dyn_s;
  uint32_t* mask_s = reinterpret_cast<uint32_t*>(dyn_s + a.tab_cap);

  const int g = blockIdx.y;
  const int split = blockIdx.x;
  const int b = g / a.Hkv, kvh = g % a.Hkv;
  const int lrow = a.lrow_is_batch ? b : g;
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  const int qc = lane % 16, rg = lane / 16;      // MFMA layout: query column, row group
  const int sub = lane % LPR, slot = lane / LPR; // V load layout

  int cnt;
  const int32_t* vlist = nullptr;  // kListVirtual / kListScores: the selection's ids
  int n_sel = 0;
  int pre_e[2] = {0, 0}, n_pre = 0;  // kListVirtual: entries read ahead of the count
  // the split that publishes the group's row count (and, selecting from scores, the selection)
  const int pub_split = MODE == kListScores ? a.smax - 1 : 0;  // the grid is (smax, groups)
  if constexpr (MODE == kListScores) {
    const float* srow = a.sc_scores + (int64_t)g * a.sc_ld;
    const int n = a.sc_n, kk = min(a.sc_k, n);
    const int ns_tok = min(a.n_sink, a.n_tokens), rs_tok = max(a.n_tokens - a.n_recent, 0);
    cnt = virtual_rows(kk, a.gran, ns_tok, rs_tok, a.n_tokens);
    n_sel = kk;
    vlist = sc_list;
    // a split whose rows are all forced needs no selection (the publisher always selects)
    const int rs_ = split_rows(a.split_bound > 0 ? a.split_bound : cnt, a.smax);
    const bool selects = split == pub_split ||
                         min(split * rs_ + rs_, cnt) > forced_rows(ns_tok, rs_tok, a.n_tokens);
    if (selects) {
      // the group's selection: exact top-k of its score row (ties to the lowest index,
      // ascending), as topk_select computes it, kept in LDS
      const int tid = threadIdx.x;
      auto keep = [&](int pos, int i) { sc_list[pos] = i; };
      // the usual case: each thread holds its keys in registers (2 or 4 of them); every load
      // is issued before any is used (clamped in bounds): one wait
      auto reg_path = [&](auto kpt) {
        constexpr int KP = decltype(kpt)::value;
        float sv[KP];
#pragma unroll
        for (int j = 0; j < KP; ++j) sv[j] = 0.f;
        if (n > 0) {
#pragma unroll
          for (int j = 0; j < KP; ++j) sv[j] = srow[min(j * kThreads + tid, n - 1)];
        }
        // the histograms are cleared while the scores are on their way
        for (int i = tid; i < 4 * 256; i += kThreads) sc_hist[i] = 0u;
        uint32_t key[KP];
#pragma unroll
        for (int j = 0; j < KP; ++j) key[j] = j * kThreads + tid < n ? order_key(sv[j]) : 0u;
        if (kk > 0) reg_topk<kThreads, KP, true>(key, n, kk, sc_hist, sc_wsum, keep);
        __syncthreads();
      };
      if (n <= 2 * kThreads) {
        reg_path(std::integral_constant<int, 2>{});
      } else if (n <= kScRegKeys * kThreads) {
        reg_path(std::integral_constant<int, kScRegKeys>{});
      } else {
        uint32_t* keys = reinterpret_cast<uint32_t*>(work_s);
        for (int j0 = 0; j0 < n; j0 += 4 * kThreads) {
          float sv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) sv[u] = srow[min(j0 + u * kThreads + tid, n - 1)];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (j0 + u * kThreads + tid < n) keys[j0 + u * kThreads + tid] = order_key(sv[u]);
        }
        if (kk > 0) lds_topk<kThreads>(keys, n, kk, sc_hist, sc_wsum, keep);
      }
    }
  } else if constexpr (MODE == kListVirtual) {
    vlist = a.list + (int64_t)lrow * a.list_ld;
    const int ns_tok = min(a.n_sink, a.n_tokens), rs_tok = max(a.n_tokens - a.n_recent, 0);
    if (a.split_bound > 0 && a.list_ld > 0) {
      // the list entries of this thread's first two table rows are read together with the
      // count (clamped in bounds; an entry past the selection, or of a forced row, is unused)
      const int p0 = split * split_rows(a.split_bound, a.smax) + (int)threadIdx.x -
                     forced_rows(ns_tok, rs_tok, a.n_tokens);
      const int lmax = (int)a.list_ld - 1;
      pre_e[0] = vlist[min(max(p0, 0) / a.gran, lmax)];
      pre_e[1] = vlist[min(max(p0 + kThreads, 0) / a.gran, lmax)];
      n_pre = 2;
    }
    n_sel = (int)max(0, min(a.count[lrow], (int)a.list_ld));
    cnt = virtual_rows(n_sel, a.gran, ns_tok, rs_tok, a.n_tokens);
  } else if constexpr (MODE == kListIntervals) {
    if (wid == 0)
      build_segments(a, a.list + (int64_t)lrow * a.list_ld, a.count + lrow, seg_start, seg_pos,
                     &seg_meta[0], &seg_meta[1]);
    __syncthreads();
    cnt = seg_meta[1];
  } else {
    cnt = a.count[lrow];
    cnt = max(0, min(cnt, a.count_clamp));
  }
  // the publishing split writes once its work is done: a barrier waits for every earlier global
  // store, so none are issued before it
  auto publish = [&]() {
    if (split != pub_split) return;
    if constexpr (MODE != kListExplicit) {
      if (threadIdx.x == 0) a.ucount[g] = cnt;
    }
    if constexpr (MODE == kListScores) {
      if (a.sel_out)
        for (int i = threadIdx.x; i < n_sel; i += kThreads)
          a.sel_out[(int64_t)g * a.sel_out_ld + i] = sc_list[i];
      if (threadIdx.x == 0 && a.count_out) a.count_out[g] = n_sel;
    }
  };
  const int rs = split_rows(a.split_bound > 0 ? a.split_bound : cnt, a.smax);
  const int r0 = split * rs;
  if (r0 >= cnt) {
    publish();
    return;
  }
  const int r1 = min(r0 + rs, cnt);
  const int nrows = r1 - r0;
  const int iters = (nrows + STEP - 1) / STEP;
  const int tab_rows = (iters + 3) * STEP;
  const RowBase rbase = make_row_base<uint16_t>(a, b, kvh);
  fill_slot_table<MODE, kMask>(a, b, kvh, g, lrow, r0, nrows, tab_rows, slot_s, mask_s, seg_start,
                               seg_pos, seg_meta[0], vlist, n_sel, pre_e, n_pre);

  float m_q = -INFINITY, l_part = 0.f;  // query qc: running max (wave-uniform), own-row denominator
  f32x4 O[DCH];                         // queries 4rg..+3, dims 16c + qc
#pragma unroll
  for (int c = 0; c < DCH; ++c) O[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  // queries as the MFMA B operand: lane holds Q[query qc][32j + 8rg .. +7].  Loaded after the
  // selection list (the list's wait must not include them); they arrive with the first tiles.
  bf16x8 qb[KCH];
  {
    const bool have = qc < a.nq;
    const int t = qc / a.G, hl = qc % a.G;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                         ((int64_t)(b * a.T + t) * a.Hq + kvh * a.G + hl) * D + 8 * rg;
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (have) u = *reinterpret_cast<const uint4*>(qp + 32 * j);
      qb[j] = __builtin_bit_cast(bf16x8, u);
    }
  }
  const uint64_t kcol = (uint64_t)(16 * rg);
  const uint64_t vcol = (uint64_t)(16 * sub);
  const int qd = qc / a.mask_div;
  int64_t lg_row = 0;
  if (a.logits && qc < a.nq) {
    const int t = qc / a.G, hl = qc % a.G;
    lg_row = ((int64_t)(b * a.T + t) * a.Hq + kvh * a.G + hl) * a.logits_ld + r0;
  }
  unsigned char* vt = work_s + wid * TILE * VST;
  // transposing read address: row 4rg + (lane%16)/4, columns 4(lane%4)..+3 of each 16-wide chunk
  const unsigned char* vt_rd = vt + (4 * rg + (lane % 16) / 4) * VST + 8 * (lane % 4);

  // K and V rows: block selections (runs of consecutive rows) stream with nontemporal loads;
  // explicit lists of scattered single rows read faster with plain ones (measured both ways)
  auto kv_load = [](uint64_t addr) {
    if constexpr (MODE == kListExplicit) return gload16(addr);
    else return gload16_nt(addr);
  };
  auto issue = [&](int it, uint4 (&kr)[KCH], uint4 (&vr)[PVI], bool& klive) {
    const int tb = it * STEP + wid * TILE;
    const int sk = slot_s[tb + qc];
    int sv[PVI];
#pragma unroll
    for (int i = 0; i < PVI; ++i) sv[i] = slot_s[tb + i * RPI + slot];
    klive = sk != kDead;
    uint64_t ka, va;
    row_addr(rbase, sk, ka, va);
#pragma unroll
    for (int j = 0; j < KCH; ++j) kr[j] = kv_load(ka + kcol + 64 * j);
#pragma unroll
    for (int i = 0; i < PVI; ++i) {
      row_addr(rbase, sv[i], ka, va);
      vr[i] = kv_load(va + vcol);
    }
  };
  // scaled logits of this lane's 4 rows (query qc)
  auto store_logits = [&](int it, const float (&lg)[4]) {
    if (a.logits && qc < a.nq) {
      // rows 4rg..+3 of query qc are 4 consecutive floats: one 16-byte store when aligned
      const int p0 = it * STEP + wid * TILE + 4 * rg;
      float* dst = a.logits + lg_row + p0;
      if (a.logits_vec && p0 + 3 < nrows) {
        *reinterpret_cast<float4*>(dst) = make_float4(lg[0], lg[1], lg[2], lg[3]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (p0 + i < nrows) dst[i] = lg[i];
      }
    }
  };
  auto consume = [&](int it, const uint4 (&kr)[KCH], const uint4 (&vr)[PVI], bool klive,
                     float (&lgo)[4]) {
    const int tb = it * STEP + wid * TILE;
    // stage the V tile row-major in this wave's LDS slice
#pragma unroll
    for (int i = 0; i < PVI; ++i)
      *reinterpret_cast<uint4*>(vt + (i * RPI + slot) * VST + 16 * sub) = vr[i];
    const uint64_t liveb = __ballot(klive);  // bit r (< 16): row r of the tile is read
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KCH; ++j)
      S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[j]), qb[j], S, 0, 0, 0);
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * rg + i;
      bool rd = ((liveb >> r) & 1ull) && qc < a.nq;
      if constexpr (kMask) rd = rd && ((mask_s[tb + r] >> qd) & 1u);
      sv[i] = rd ? S[i] * a.scale_log2 : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) lgo[i] = sv[i] * kLn2;
    float tmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float m_new = fmaxf(m_q, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_q - m_new);
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = (sv[i] == -INFINITY) ? 0.f : fast_exp2(sv[i] - m_new);
    l_part = l_part * alpha + ((pv[0] + pv[1]) + (pv[2] + pv[3]));
    m_q = m_new;
    if (__ballot(alpha != 1.f)) {
      // output rows are queries 4rg + i; their scale factors live in lanes 4rg + i
      float as[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) as[i] = __shfl(alpha, 4 * rg + i, kWave);
#pragma unroll
      for (int c = 0; c < DCH; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[c][i] *= as[i];
    }
    // P as two bf16 operands: high = truncated bits (exact), low = rounded remainder
    i16x4 ph, pl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = __float_as_uint(pv[i]);
      const float hi = __uint_as_float(u & 0xFFFF0000u);
      ph[i] = (short)(u >> 16);
      pl[i] = (short)bf16_rne_bits(pv[i] - hi);
    }
    wave_lds_fence();
#pragma unroll
    for (int c = 0; c < DCH; ++c) {
      const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vt_rd + 32 * c));
      O[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vb, O[c], 0, 0, 0);
      O[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vb, O[c], 0, 0, 0);
    }
    wave_lds_fence();
  };

  {
    // Each iteration loads BATCH tiles per wave, then consumes them in order; no load is
    // carried across iterations (loop-carried loads make the compiler drain at the loop head).
    // Latency is covered by the other resident waves.
    uint4 kb[BATCH][KCH], vb[BATCH][PVI];
    bool lv[BATCH];
    for (int it = 0; it < iters; it += BATCH) {
#pragma unroll
      for (int t = 0; t < BATCH; ++t) issue(it + t, kb[t], vb[t], lv[t]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < BATCH; ++t) {
        float lg[4];
        consume(it + t, kb[t], vb[t], lv[t], lg);
        store_logits(it + t, lg);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // wave totals: denominators over the 4 row groups; the output rows are already complete
  l_part += __shfl_xor(l_part, 16, kWave);
  l_part += __shfl_xor(l_part, 32, kWave);
  __syncthreads();  // every wave is done with its staged V tiles
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = 4 * rg + i;
    if (q < NQ) {
#pragma unroll
      for (int c = 0; c < DCH; ++c) red[wid][q][2 + 16 * c + qc] = O[c][i];
    }
  }
  if (rg == 0 && qc < NQ) {
    red[wid][qc][0] = m_q;
    red[wid][qc][1] = l_part;
  }
  __syncthreads();
  finish_split<D, NQ, kWaves>(a, red, g, split);
  publish();
}

// ------------------------------------------------------------------------------- combine

// One wave per query vector.  Every load (the group's row count, each split's (m, l) and its
// partial output) is issued up front for up to kCombineMax splits, so the kernel waits on memory
// once; the splits are then merged in split order (deterministic).
constexpr int kCombineMax = 16;

template <int D>
__global__ __launch_bounds__(kWave) void attn_combine_kernel(AttnArgs a, int nq_pad, float* out,
                                                             float* lse) {
  const int g = blockIdx.x / a.nq;
  const int n = blockIdx.x % a.nq;
  const int b = g / a.Hkv, kvh = g % a.Hkv;
  const int lane = lane_id();
  constexpr int PER = D / kWave;
  const int64_t pbase = (int64_t)g * a.smax * nq_pad + n;
  int cnt;
  if (a.list_mode != kListExplicit || a.ucount_valid) {
    cnt = a.ucount[g];
  } else {
    const int lrow = a.lrow_is_batch ? b : g;
    cnt = max(0, min(a.count[lrow], a.count_clamp));
  }
  float o[PER], L = 0.f, mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  for (int s0 = 0; s0 < a.smax; s0 += kCombineMax) {
    // speculative loads of every split slot of the plan (in bounds); slots past the row count
    // are masked out afterwards
    float ms[kCombineMax], ls[kCombineMax], ac[kCombineMax][PER];
#pragma unroll
    for (int j = 0; j < kCombineMax; ++j) {
      const int s = min(s0 + j, a.smax - 1);
      const int64_t pi = pbase + (int64_t)s * nq_pad;
      ms[j] = a.ml[pi * 2];
      ls[j] = a.ml[pi * 2 + 1];
#pragma unroll
      for (int i = 0; i < PER; ++i) ac[j][i] = a.acc[pi * D + lane + i * kWave];
    }
    const int per = cnt > 0 ? split_rows(a.split_bound > 0 ? a.split_bound : cnt, a.smax) : 1;
    const int S = cnt > 0 ? (cnt + per - 1) / per : 0;
    float cmx = mx;
#pragma unroll
    for (int j = 0; j < kCombineMax; ++j)
      if (s0 + j < S) cmx = fmaxf(cmx, ms[j]);
    const float rs = (cmx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mx - cmx);
    L *= rs;
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] *= rs;
    mx = cmx;
#pragma unroll
    for (int j = 0; j < kCombineMax; ++j) {
      if (s0 + j < S && mx != -INFINITY) {
        const float w = __builtin_amdgcn_exp2f(ms[j] - mx);
        L += ls[j] * w;
#pragma unroll
        for (int i = 0; i < PER; ++i) o[i] += ac[j][i] * w;
      }
    }
  }
  const int t = n / a.G, hl = n % a.G;
  const int64_t qrow = (int64_t)(b * a.T + t) * a.Hq + kvh * a.G + hl;
  const bool empty = !(L > 0.f);
  const float inv = empty ? 0.f : 1.0f / L;
#pragma unroll
  for (int i = 0; i < PER; ++i) out[qrow * D + lane + i * kWave] = o[i] * inv;
  if (lse && lane == 0) lse[qrow] = empty ? -INFINITY : (mx + __log2f(L)) * kLn2;
}

#ifndef SPK_ATTN_UNROLL_SMALL
#define SPK_ATTN_UNROLL_SMALL 4
#endif
#ifndef SPK_ATTN_UNROLL_LARGE
#define SPK_ATTN_UNROLL_LARGE 2
#endif
constexpr int attn_unroll(int nq) { return nq <= 4 ? SPK_ATTN_UNROLL_SMALL : SPK_ATTN_UNROLL_LARGE; }

template <int D, typename KT, int NQ, bool kMask, int MODE>
void launch_partial(dim3 grid, hipStream_t st, const AttnArgs& a) {
  constexpr int U = attn_unroll(NQ);
  const size_t dyn = (size_t)a.tab_cap * 4 * (kMask ? 2 : 1);
  hipLaunchKernelGGL((attn_partial_kernel<D, KT, NQ, kMask, MODE, U>), grid, dim3(kThreads), dyn,
                     st, a);
}

template <int D, int NQ, bool kMask, int MODE>
void launch_partial_mfma(dim3 grid, hipStream_t st, const AttnArgs& a) {
  const size_t dyn = (size_t)a.tab_cap * 4 * (kMask ? 2 : 1);
  hipLaunchKernelGGL((attn_partial_mfma_kernel<D, NQ, kMask, MODE>), grid, dim3(kThreads), dyn, st,
                     a);
}

template <int D, typename KT, int NQ>
void dispatch_mode(bool mask, int mode, dim3 grid, hipStream_t st, const AttnArgs& a) {
  if constexpr (std::is_same<KT, uint16_t>::value) {
    if (a.q_bf16) {
      if (mask) launch_partial_mfma<D, NQ, true, kListExplicit>(grid, st, a);
      else if (mode == kListIntervals) launch_partial_mfma<D, NQ, false, kListIntervals>(grid, st, a);
      else if (mode == kListVirtual) launch_partial_mfma<D, NQ, false, kListVirtual>(grid, st, a);
      else launch_partial_mfma<D, NQ, false, kListExplicit>(grid, st, a);
      return;
    }
  }
  if (mask) launch_partial<D, KT, NQ, true, kListExplicit>(grid, st, a);
  else if (mode == kListIntervals) launch_partial<D, KT, NQ, false, kListIntervals>(grid, st, a);
  else launch_partial<D, KT, NQ, false, kListExplicit>(grid, st, a);
}

template <int D>
void dispatch_scores(int nq_pad, dim3 grid, hipStream_t st, const AttnArgs& a) {
  switch (nq_pad) {
    case 1: launch_partial_mfma<D, 1, false, kListScores>(grid, st, a); break;
    case 2: launch_partial_mfma<D, 2, false, kListScores>(grid, st, a); break;
    case 4: launch_partial_mfma<D, 4, false, kListScores>(grid, st, a); break;
    case 8: launch_partial_mfma<D, 8, false, kListScores>(grid, st, a); break;
    default: launch_partial_mfma<D, 16, false, kListScores>(grid, st, a); break;
  }
}

template <int D, typename KT>
void dispatch_nq(int nq_pad, bool mask, int mode, dim3 grid, hipStream_t st, const AttnArgs& a) {
  switch (nq_pad) {
    case 1: dispatch_mode<D, KT, 1>(mask, mode, grid, st, a); break;
    case 2: dispatch_mode<D, KT, 2>(mask, mode, grid, st, a); break;
    case 4: dispatch_mode<D, KT, 4>(mask, mode, grid, st, a); break;
    case 8: dispatch_mode<D, KT, 8>(mask, mode, grid, st, a); break;
    default: dispatch_mode<D, KT, 16>(mask, mode, grid, st, a); break;
  }
}

// Occupancy and static LDS of the bf16 (MFMA) partial kernel of a configuration (queried once).
PartialInfo partial_info(int d, int nq_pad, bool mask, int mode) {
  static PartialInfo cache[2][5][2][2];
  static bool have[2][5][2][2];
  static std::mutex mu;
  const int di = d == 128 ? 0 : 1;
  const int ni = nq_pad == 1 ? 0 : nq_pad == 2 ? 1 : nq_pad == 4 ? 2 : nq_pad == 8 ? 3 : 4;
  std::lock_guard<std::mutex> lock(mu);
  if (have[di][ni][mask ? 1 : 0][mode ? 1 : 0]) return cache[di][ni][mask ? 1 : 0][mode ? 1 : 0];
  const void* fn = nullptr;
#define SPK_FN(D, NQ)                                                                     \
  fn = mask ? (const void*)attn_partial_mfma_kernel<D, NQ, true, kListExplicit>            \
       : mode ? (const void*)attn_partial_mfma_kernel<D, NQ, false, kListIntervals>        \
              : (const void*)attn_partial_mfma_kernel<D, NQ, false, kListExplicit>
#define SPK_FN_D(D)                     \
  switch (nq_pad) {                     \
    case 1: SPK_FN(D, 1); break;        \
    case 2: SPK_FN(D, 2); break;        \
    case 4: SPK_FN(D, 4); break;        \
    case 8: SPK_FN(D, 8); break;        \
    default: SPK_FN(D, 16); break;      \
  }
  if (d == 128) {
    SPK_FN_D(128)
  } else {
    SPK_FN_D(64)
  }
#undef SPK_FN_D
#undef SPK_FN
  PartialInfo info;
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, kThreads, 0) != hipSuccess ||
      blocks <= 0) {
    (void)hipGetLastError();
    blocks = 2;
  }
  info.occ = blocks;
  hipFuncAttributes attr;
  if (hipFuncGetAttributes(&attr, fn) == hipSuccess) info.static_lds = attr.sharedSizeBytes;
  else (void)hipGetLastError();
  cache[di][ni][mask ? 1 : 0][mode ? 1 : 0] = info;
  have[di][ni][mask ? 1 : 0][mode ? 1 : 0] = true;
  return info;
}

static size_t device_attr(hipDeviceAttribute_t attr, size_t fallback) {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&v, attr, dev) != hipSuccess ||
      v <= 0) {
    (void)hipGetLastError();
    return fallback;
  }
  return (size_t)v;
}

size_t lds_per_cu() {
  return device_attr(hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, 65536);
}
size_t lds_per_block() { return device_attr(hipDeviceAttributeMaxSharedMemoryPerBlock, 65536); }

}  // namespace
}  // namespace spk

using spk::Plan;

// Events of spk_set_attn_timing_events (null: timing off).
static hipEvent_t g_timing_begin = nullptr;
static hipEvent_t g_timing_end = nullptr;

extern "C" SPK_API spk_status spk_set_attn_timing_events(void* begin, void* end) {
  using namespace spk;
  clear_error();
  SPK_REQUIRE((begin == nullptr) == (end == nullptr), SPK_EINVAL,
              "spk_set_attn_timing_events: give both events or neither");
  g_timing_begin = static_cast<hipEvent_t>(begin);
  g_timing_end = static_cast<hipEvent_t>(end);
  return SPK_OK;
}

// A host pool must be page-locked, device-mapped host memory; the kernel reads it through the
// device address HIP reports for it.  Pageable memory would fault, so it is refused here.
static spk_status resolve_host_pool(const void* p, const void** dev, const char* name) {
  hipPointerAttribute_t at{};
  const hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return spk::set_error(SPK_EINVAL, "sparse_decode_attn: %s is not memory known to HIP (%s)",
                          name, hipGetErrorString(e));
  }
  if (at.type != hipMemoryTypeHost || at.devicePointer == nullptr)
    return spk::set_error(SPK_EINVAL,
                          "sparse_decode_attn: %s must be pinned, device-mapped host memory", name);
  *dev = at.devicePointer;
  return SPK_OK;
}

static spk_status check_common(spk_sel_scope scope, int B, int T, int Hq, int Hkv, int d,
                               int n_tokens, int64_t sel_ld, int gran, int n_sink, int n_recent) {
  using namespace spk;
  SPK_REQUIRE(scope >= SPK_SEL_PER_SEQ && scope <= SPK_SEL_PER_Q_HEAD, SPK_EINVAL,
              "sparse_decode_attn: unknown scope %d", (int)scope);
  SPK_REQUIRE(B >= 0 && T > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0, SPK_EINVAL,
              "sparse_decode_attn: bad shape B=%d T=%d Hq=%d Hkv=%d (Hq %% Hkv must be 0)", B, T,
              Hq, Hkv);
  SPK_REQUIRE(d == 64 || d == 128, SPK_EUNSUPPORTED, "sparse_decode_attn: d=%d not in {64,128}", d);
  SPK_REQUIRE(n_tokens >= 0 && sel_ld >= 0 && gran >= 1 && n_sink >= 0 && n_recent >= 0,
              SPK_EINVAL, "sparse_decode_attn: negative size or gran < 1");
  SPK_REQUIRE(n_tokens < (1 << 30) && sel_ld < (1 << 30) && gran < (1 << 20), SPK_EINVAL,
              "sparse_decode_attn: size out of range");
  const int G = Hq / Hkv;
  SPK_REQUIRE(G * T <= 16, SPK_EUNSUPPORTED,
              "sparse_decode_attn: %d query vectors per KV head (max 16)", G * T);
  const int sets = scope == SPK_SEL_PER_SEQ ? 1 : scope == SPK_SEL_PER_KV_HEAD ? T : T * G;
  SPK_REQUIRE(sets <= spk::kAsmSets, SPK_EUNSUPPORTED,
              "sparse_decode_attn: %d selection lists per group (max 16)", sets);
  SPK_REQUIRE((int64_t)sets * sel_ld * gran < ((int64_t)1 << 31), SPK_EUNSUPPORTED,
              "sparse_decode_attn: %d lists x %lld entries x granularity %d exceed 2^31 rows",
              sets, (long long)sel_ld, gran);
  return SPK_OK;
}

extern "C" SPK_API spk_status sparse_decode_attn_workspace_size(
    spk_sel_scope scope, int B, int T, int Hq, int Hkv, int d, int n_tokens, int64_t sel_ld,
    int gran, int n_sink, int n_recent, size_t* bytes) {
  using namespace spk;
  SPK_REQUIRE(bytes, SPK_EINVAL, "sparse_decode_attn_workspace_size: null bytes");
  spk_status st = check_common(scope, B, T, Hq, Hkv, d, n_tokens, sel_ld, gran, n_sink, n_recent);
  if (st != SPK_OK) return st;
  *bytes = make_plan(scope, B, T, Hq, Hkv, d, n_tokens, sel_ld, gran, n_sink, n_recent).bytes;
  clear_error();
  return SPK_OK;
}

// The body of sparse_decode_attn and sparse_decode_attn_noalloc: `ws` is the caller's
// workspace or the library's scratch array.  With validate_only, every argument check runs and
// the call returns before the workspace check and any launch.
static spk_status decode_attn_impl(bool validate_only, const uint32_t* pre_mask,
    const void* q, spk_dtype q_dtype, const void* k, const void* v, spk_dtype kv_dtype,
    int64_t kv_sb, int64_t kv_sh, int64_t kv_sn, const void* k_host, const void* v_host,
    int64_t host_sb, int64_t host_sh, int64_t host_sn, int64_t host_slots, const int32_t* loc,
    int64_t loc_sb, int64_t loc_sh, int64_t hbm_slots, const int32_t* sel_idx, const int32_t* sel_count, int64_t sel_ld,
    spk_sel_scope scope, int gran, int n_sink, int n_recent, int B, int T, int Hq, int Hkv, int d,
    int n_tokens, float sm_scale, float* out, float* lse, float* logits, int64_t logits_ld,
    void* ws, size_t ws_bytes, void* stream) {
  using namespace spk;
  spk_status st0 = check_common(scope, B, T, Hq, Hkv, d, n_tokens, sel_ld, gran, n_sink, n_recent);
  if (st0 != SPK_OK) return st0;
  SPK_REQUIRE(dtype_ok(q_dtype) && dtype_ok(kv_dtype), SPK_EUNSUPPORTED,
              "sparse_decode_attn: unsupported dtype");
  SPK_REQUIRE(B == 0 || (q && k && v && out && (sel_idx || sel_ld == 0) && sel_count), SPK_EINVAL,
              "sparse_decode_attn: null q, k, v, out, sel_idx or sel_count");
  SPK_REQUIRE(kv_sn >= d && kv_sb >= 0 && kv_sh >= 0 && kv_sn % 8 == 0 && kv_sh % 8 == 0 &&
                  kv_sb % 8 == 0,
              SPK_EINVAL, "sparse_decode_attn: kv strides must be multiples of 8 with kv_sn >= d");
  SPK_REQUIRE(kv_sn * (int64_t)dtype_size(kv_dtype) < (int64_t)1 << 32, SPK_EUNSUPPORTED,
              "sparse_decode_attn: a KV row stride of 4 GiB or more is not supported");
  SPK_REQUIRE(reinterpret_cast<uintptr_t>(q) % 16 == 0 && reinterpret_cast<uintptr_t>(k) % 16 == 0 &&
                  reinterpret_cast<uintptr_t>(v) % 16 == 0,
              SPK_EINVAL, "sparse_decode_attn: q, k, v must be 16-byte aligned");
  if (loc) {
    SPK_REQUIRE(k_host && v_host, SPK_EINVAL,
                "sparse_decode_attn: loc given without host pools k_host/v_host");
    SPK_REQUIRE(host_sn >= d && host_sb >= 0 && host_sh >= 0 && host_sn % 8 == 0 &&
                    host_sh % 8 == 0 && host_sb % 8 == 0,
                SPK_EINVAL, "sparse_decode_attn: host strides must be multiples of 8");
    SPK_REQUIRE(host_sn * (int64_t)dtype_size(kv_dtype) < (int64_t)1 << 32, SPK_EUNSUPPORTED,
                "sparse_decode_attn: a host row stride of 4 GiB or more is not supported");
    SPK_REQUIRE(reinterpret_cast<uintptr_t>(k_host) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(v_host) % 16 == 0,
                SPK_EINVAL, "sparse_decode_attn: host pools must be 16-byte aligned");
    SPK_REQUIRE(loc_sb >= 0 && loc_sh >= 0 && host_slots >= 0 && host_slots < INT32_MAX &&
                    hbm_slots >= 0,
                SPK_EINVAL,
                "sparse_decode_attn: bad loc strides or slot counts");
    spk_status hs = resolve_host_pool(k_host, &k_host, "k_host");
    if (hs != SPK_OK) return hs;
    hs = resolve_host_pool(v_host, &v_host, "v_host");
    if (hs != SPK_OK) return hs;
  }
  SPK_REQUIRE(loc || n_tokens <= hbm_slots, SPK_EINVAL,
              "sparse_decode_attn: n_tokens %d exceeds the %lld rows of the HBM caches", n_tokens,
              (long long)hbm_slots);
  SPK_REQUIRE(!(sm_scale != sm_scale), SPK_EINVAL, "sparse_decode_attn: sm_scale is NaN");
  const Plan p = make_plan(scope, B, T, Hq, Hkv, d, n_tokens, sel_ld, gran, n_sink, n_recent,
                           false, pre_mask ? sel_ld : 0);
  SPK_REQUIRE(!logits || logits_ld >= p.ubound, SPK_EINVAL,
              "sparse_decode_attn: logits_ld %lld < fetch-list bound %d", (long long)logits_ld,
              p.ubound);
  if (validate_only) {
    clear_error();
    return SPK_OK;
  }
  SPK_REQUIRE(ws_bytes >= p.bytes && (p.bytes == 0 || ws), SPK_EWORKSPACE,
              "sparse_decode_attn: workspace %zu bytes < %zu needed", ws_bytes, p.bytes);
  clear_error();
  if (B == 0) return SPK_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* w = reinterpret_cast<char*>(ws);
  const int G = Hq / Hkv;

  AttnArgs a{};
  a.q = q;
  a.q_bf16 = q_dtype == SPK_BF16;
  a.k = k;
  a.v = v;
  a.kv_sb = kv_sb;
  a.kv_sh = kv_sh;
  a.kv_sn = kv_sn;
  a.k_host = k_host;
  a.v_host = v_host;
  a.host_sb = host_sb;
  a.host_sh = host_sh;
  a.host_sn = host_sn;
  a.host_slots = host_slots;
  a.loc = loc;
  a.loc_sb = loc_sb;
  a.loc_sh = loc_sh;
  a.hbm_slots = hbm_slots;
  a.T = T;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.nq = G * T;
  a.n_tokens = n_tokens;
  a.tab_cap = p.R + kTabPad;
  a.smax = p.smax;
  a.scale_log2 = sm_scale * kLog2e;
  a.ml = reinterpret_cast<float*>(w + p.off_ml);
  a.acc = reinterpret_cast<float*>(w + p.off_acc);
  a.logits = logits;
  a.logits_ld = logits_ld;
  a.logits_vec = reinterpret_cast<uintptr_t>(logits) % 16 == 0 && logits_ld % 4 == 0;
  a.mask = nullptr;
  a.mask_div = scope == SPK_SEL_PER_KV_HEAD ? G : 1;

  a.list_mode = kListExplicit;
  a.gran = gran;
  a.n_sink = n_sink;
  a.n_recent = n_recent;
  a.ucount = p.assemble || p.intervals ? reinterpret_cast<int32_t*>(w + p.off_count) : nullptr;
  // One list per group expanded by gran / sinks / recent window, no logits, on the matrix-core
  // kernel: the forced rows, then the ids' rows in list order (no union to build; rows an earlier
  // part also holds are skipped), and splits are sized from the bound so they are known before
  // the count.
  const bool expand = gran > 1 || n_sink > 0 || n_recent > 0;
  const bool virt = !pre_mask && !logits && kv_dtype == SPK_BF16 && q_dtype == SPK_BF16 &&
                    p.sets == 1 && expand && (int64_t)n_tokens >= sel_ld * gran + n_sink + n_recent;
  if (pre_mask) {
    // the caller's assembled union: rows list[g*sel_ld + i], i < count[g], masks alongside
    a.list = sel_idx;
    a.count = sel_count;
    a.list_ld = sel_ld;
    a.count_clamp = p.ubound;
    a.lrow_is_batch = 0;
    a.mask = pre_mask;
    a.ucount = const_cast<int32_t*>(sel_count);
    a.ucount_valid = 1;
  } else if (virt) {
    a.list_mode = kListVirtual;
    a.list = sel_idx;
    a.count = sel_count;
    a.list_ld = sel_ld;
    a.count_clamp = p.ubound;
    a.split_bound = p.ubound;
    a.lrow_is_batch = scope == SPK_SEL_PER_SEQ;
    a.ucount_valid = 1;
  } else if (p.assemble) {
    AsmArgs as{};
    as.sel_idx = sel_idx;
    as.sel_count = sel_count;
    as.sel_ld = sel_ld;
    as.scope = scope;
    as.gran = gran;
    as.n_sink = n_sink;
    as.n_recent = n_recent;
    as.T = T;
    as.Hq = Hq;
    as.Hkv = Hkv;
    as.G = G;
    as.sets = p.sets;
    as.n_tokens = n_tokens;
    as.words = p.words;
    as.ubound = p.ubound;
    as.bm_global = p.bm_lds ? nullptr : reinterpret_cast<uint32_t*>(w + p.off_bm);
    as.ulist = reinterpret_cast<int32_t*>(w + p.off_list);
    as.umask = p.mask ? reinterpret_cast<uint32_t*>(w + p.off_mask) : nullptr;
    as.ucount = a.ucount;
    if (p.bm_lds)
      hipLaunchKernelGGL(assemble_kernel<true>, dim3(p.groups), dim3(kAsmThreads),
                         (size_t)p.sets * p.words * 4, st, as);
    else hipLaunchKernelGGL(assemble_kernel<false>, dim3(p.groups), dim3(kAsmThreads), 0, st, as);
    spk_status e = check_launch("sparse_decode_attn/assemble");
    if (e != SPK_OK) return e;
    a.list = as.ulist;
    a.count = as.ucount;
    a.list_ld = p.ubound;
    a.count_clamp = p.ubound;
    a.lrow_is_batch = 0;
    a.mask = as.umask;
    a.ucount_valid = 1;
  } else if (p.intervals) {
    a.list_mode = kListIntervals;
    a.list = sel_idx;
    a.count = sel_count;
    a.list_ld = sel_ld;
    a.count_clamp = p.ubound;
    a.lrow_is_batch = scope == SPK_SEL_PER_SEQ;
  } else {
    a.list = sel_idx;
    a.count = sel_count;
    a.list_ld = sel_ld;
    a.count_clamp = (int)(sel_ld < p.ubound ? sel_ld : p.ubound);
    a.lrow_is_batch = scope == SPK_SEL_PER_SEQ;
  }
  dim3 grid(p.smax, p.groups);
  const bool mask = p.mask;
  hipEvent_t ev_begin = g_timing_begin, ev_end = g_timing_end;
  if (ev_begin && hipEventRecord(ev_begin, st) != hipSuccess)
    return set_error(SPK_EHIP, "sparse_decode_attn: recording the timing event failed");
  if (d == 128) {
    if (kv_dtype == SPK_BF16) dispatch_nq<128, uint16_t>(p.nq_pad, mask, a.list_mode, grid, st, a);
    else dispatch_nq<128, float>(p.nq_pad, mask, a.list_mode, grid, st, a);
  } else {
    if (kv_dtype == SPK_BF16) dispatch_nq<64, uint16_t>(p.nq_pad, mask, a.list_mode, grid, st, a);
    else dispatch_nq<64, float>(p.nq_pad, mask, a.list_mode, grid, st, a);
  }
  spk_status e = check_launch("sparse_decode_attn/partial");
  if (e != SPK_OK) return e;
  if (ev_end && hipEventRecord(ev_end, st) != hipSuccess)
    return set_error(SPK_EHIP, "sparse_decode_attn: recording the timing event failed");
  if (d == 128)
    hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(p.groups * a.nq), dim3(kWave), 0, st, a,
                       p.nq_pad, out, lse);
  else
    hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(p.groups * a.nq), dim3(kWave), 0, st, a,
                       p.nq_pad, out, lse);
  return check_launch("sparse_decode_attn/combine");
}

extern "C" SPK_API spk_status sparse_decode_attn(
    const void* q, spk_dtype q_dtype, const void* k, const void* v, spk_dtype kv_dtype,
    int64_t kv_sb, int64_t kv_sh, int64_t kv_sn, const void* k_host, const void* v_host,
    int64_t host_sb, int64_t host_sh, int64_t host_sn, int64_t host_slots, const int32_t* loc,
    int64_t loc_sb, int64_t loc_sh, int64_t hbm_slots, const int32_t* sel_idx, const int32_t* sel_count, int64_t sel_ld,
    spk_sel_scope scope, int gran, int n_sink, int n_recent, int B, int T, int Hq, int Hkv, int d,
    int n_tokens, float sm_scale, float* out, float* lse, float* logits, int64_t logits_ld,
    void* ws, size_t ws_bytes, void* stream) {
  return decode_attn_impl(false, nullptr, q, q_dtype, k, v, kv_dtype, kv_sb, kv_sh, kv_sn, k_host, v_host,
                          host_sb, host_sh, host_sn, host_slots, loc, loc_sb, loc_sh, hbm_slots,
                          sel_idx, sel_count, sel_ld, scope, gran, n_sink, n_recent, B, T, Hq,
                          Hkv, d, n_tokens, sm_scale, out, lse, logits, logits_ld, ws, ws_bytes,
                          stream);
}

extern "C" SPK_API spk_status sparse_decode_attn_union_workspace_size(
    spk_sel_scope scope, int B, int T, int Hq, int Hkv, int d, int n_tokens, int64_t u_ld,
    size_t* bytes) {
  using namespace spk;
  SPK_REQUIRE(bytes, SPK_EINVAL, "sparse_decode_attn_union_workspace_size: null bytes");
  SPK_REQUIRE(scope == SPK_SEL_PER_Q_HEAD || scope == SPK_SEL_PER_KV_HEAD, SPK_EINVAL,
              "sparse_decode_attn_union: scope must be per_q_head or per_kv_head");
  SPK_REQUIRE(u_ld > 0, SPK_EINVAL, "sparse_decode_attn_union: u_ld must be > 0");
  spk_status st = check_common(scope, B, T, Hq, Hkv, d, n_tokens, u_ld, 1, 0, 0);
  if (st != SPK_OK) return st;
  *bytes = make_plan(scope, B, T, Hq, Hkv, d, n_tokens, u_ld, 1, 0, 0, false, u_ld).bytes;
  clear_error();
  return SPK_OK;
}

extern "C" SPK_API spk_status sparse_decode_attn_union(
    const void* q, spk_dtype q_dtype, const void* k, const void* v, spk_dtype kv_dtype,
    int64_t kv_sb, int64_t kv_sh, int64_t kv_sn, const void* k_host, const void* v_host,
    int64_t host_sb, int64_t host_sh, int64_t host_sn, int64_t host_slots, const int32_t* loc,
    int64_t loc_sb, int64_t loc_sh, int64_t hbm_slots, const int32_t* u_list,
    const uint32_t* u_mask, const int32_t* u_count, int64_t u_ld, spk_sel_scope scope, int B,
    int T, int Hq, int Hkv, int d, int n_tokens, float sm_scale, float* out, float* lse,
    float* logits, int64_t logits_ld, void* ws, size_t ws_bytes, void* stream) {
  using namespace spk;
  SPK_REQUIRE(scope == SPK_SEL_PER_Q_HEAD || scope == SPK_SEL_PER_KV_HEAD, SPK_EINVAL,
              "sparse_decode_attn_union: scope must be per_q_head or per_kv_head");
  SPK_REQUIRE(u_ld > 0, SPK_EINVAL, "sparse_decode_attn_union: u_ld must be > 0");
  SPK_REQUIRE(B == 0 || (u_list && u_mask && u_count), SPK_EINVAL,
              "sparse_decode_attn_union: null union list, mask or count");
  const uint32_t* pm = u_mask ? u_mask : reinterpret_cast<const uint32_t*>(u_list);
  return decode_attn_impl(false, pm, q, q_dtype, k, v, kv_dtype, kv_sb, kv_sh, kv_sn, k_host,
                          v_host, host_sb, host_sh, host_sn, host_slots, loc, loc_sb, loc_sh,
                          hbm_slots, u_list, u_count, u_ld, scope, 1, 0, 0, B, T, Hq, Hkv, d,
                          n_tokens, sm_scale, out, lse, logits, logits_ld, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------- allocation-free variant
//
// For callers that cannot allocate (code under HIP graph capture, tight serving loops): the
// attention's workspace is a fixed array in device memory that the library owns.  Each GPU the
// library runs on holds its own copy (kScratchBytes, until the process ends).  The workspace
// needs no initial contents (every call writes what it reads), so nothing is cleared between
// calls; calls on one GPU share the array, so calls that overlap in time on one GPU (concurrent
// streams) race and must not be issued.
namespace spk {
namespace {
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kScratchDevices = 64;
}  // namespace
}  // namespace spk

__device__ __align__(256) unsigned char scratch[spk::kScratchBytes];

namespace spk {
namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// The device address of this GPU's scratch array: resolved once per device, with that device
// current.  The host-side symbol `scratch` is not a device address and is never used directly.
spk_status scratch_for_current_device(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return set_error(SPK_EHIP, "sparse_decode_attn_noalloc: hipGetDevice failed");
  }
  if (dev < 0 || dev >= kScratchDevices)
    return set_error(SPK_EUNSUPPORTED, "sparse_decode_attn_noalloc: device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return set_error(SPK_EHIP, "sparse_decode_attn_noalloc: hipGetSymbolAddress failed (%s)",
                       hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return SPK_OK;
}
}  // namespace
}  // namespace spk

extern "C" SPK_API size_t sparse_decode_attn_noalloc_max_bytes(void) { return spk::kScratchBytes; }

extern "C" SPK_API spk_status sparse_decode_attn_noalloc(
    const void* q, spk_dtype q_dtype, const void* k, const void* v, spk_dtype kv_dtype,
    int64_t kv_sb, int64_t kv_sh, int64_t kv_sn, const void* k_host, const void* v_host,
    int64_t host_sb, int64_t host_sh, int64_t host_sn, int64_t host_slots, const int32_t* loc,
    int64_t loc_sb, int64_t loc_sh, int64_t hbm_slots, const int32_t* sel_idx, const int32_t* sel_count, int64_t sel_ld,
    spk_sel_scope scope, int gran, int n_sink, int n_recent, int B, int T, int Hq, int Hkv, int d,
    int n_tokens, float sm_scale, float* out, float* lse, float* logits, int64_t logits_ld,
    void* stream) {
  using namespace spk;
  size_t need = 0;
  spk_status st = sparse_decode_attn_workspace_size(scope, B, T, Hq, Hkv, d, n_tokens, sel_ld,
                                                    gran, n_sink, n_recent, &need);
  if (st != SPK_OK) return st;
  SPK_REQUIRE(need <= kScratchBytes, SPK_EWORKSPACE,
              "sparse_decode_attn_noalloc: this call needs %zu bytes of workspace, more than the "
              "library's fixed %zu-byte scratch array; use sparse_decode_attn with a workspace",
              need, kScratchBytes);
  st = decode_attn_impl(true, nullptr, q, q_dtype, k, v, kv_dtype, kv_sb, kv_sh, kv_sn, k_host, v_host,
                        host_sb, host_sh, host_sn, host_slots, loc, loc_sb, loc_sh, hbm_slots,
                        sel_idx, sel_count, sel_ld, scope, gran, n_sink, n_recent, B, T, Hq, Hkv,
                        d, n_tokens, sm_scale, out, lse, logits, logits_ld, nullptr, 0, stream);
  if (st != SPK_OK) return st;
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != SPK_OK) return st;
  return decode_attn_impl(false, nullptr, q, q_dtype, k, v, kv_dtype, kv_sb, kv_sh, kv_sn, k_host, v_host,
                          host_sb, host_sh, host_sn, host_slots, loc, loc_sb, loc_sh, hbm_slots,
                          sel_idx, sel_count, sel_ld, scope, gran, n_sink, n_recent, B, T, Hq,
                          Hkv, d, n_tokens, sm_scale, out, lse, logits, logits_ld, ws,
                          kScratchBytes, stream);
}

extern "C" SPK_API spk_status sparse_topk_decode_attn_workspace_size(int B, int Hq, int Hkv,
                                                                     int d, int n_tokens,
                                                                     int n_cand, int k, int gran,
                                                                     int n_sink, int n_recent,
                                                                     size_t* bytes) {
  using namespace spk;
  SPK_REQUIRE(bytes, SPK_EINVAL, "sparse_topk_decode_attn_workspace_size: null bytes");
  spk_status st0 = check_common(SPK_SEL_PER_KV_HEAD, B, 1, Hq, Hkv, d, n_tokens, k, gran, n_sink,
                                n_recent);
  if (st0 != SPK_OK) return st0;
  SPK_REQUIRE(k >= 0 && k + 2 <= kMaxIntervals, SPK_EUNSUPPORTED,
              "sparse_topk_decode_attn_workspace_size: k=%d (at most %d)", k, kMaxIntervals - 2);
  SPK_REQUIRE(n_cand >= 0, SPK_EINVAL, "sparse_topk_decode_attn_workspace_size: n_cand < 0");
  const int kk = k < n_cand ? k : n_cand;
  *bytes = make_plan(SPK_SEL_PER_KV_HEAD, B, 1, Hq, Hkv, d, n_tokens, kk, gran, n_sink, n_recent,
                     true).bytes;
  clear_error();
  return SPK_OK;
}

extern "C" SPK_API spk_status sparse_topk_decode_attn(
    const float* scores, int64_t s_ld, int n_cand, int k, const void* q, spk_dtype q_dtype,
    const void* kc, const void* vc, spk_dtype kv_dtype, int64_t kv_sb, int64_t kv_sh,
    int64_t kv_sn, int gran, int n_sink, int n_recent, int B, int Hq, int Hkv, int d,
    int n_tokens, float sm_scale, float* out, float* lse, int32_t* sel_idx, int32_t* sel_count,
    int64_t sel_ld, void* ws, size_t ws_bytes, void* stream) {
  using namespace spk;
  spk_status st0 = check_common(SPK_SEL_PER_KV_HEAD, B, 1, Hq, Hkv, d, n_tokens, k, gran, n_sink,
                                n_recent);
  if (st0 != SPK_OK) return st0;
  SPK_REQUIRE(q_dtype == SPK_BF16 && kv_dtype == SPK_BF16, SPK_EUNSUPPORTED,
              "sparse_topk_decode_attn: bf16 queries and caches only");
  SPK_REQUIRE(n_cand >= 0 && n_cand <= kScoresMax, SPK_EUNSUPPORTED,
              "sparse_topk_decode_attn: %d candidates per row (max %d)", n_cand, kScoresMax);
  SPK_REQUIRE(k >= 0 && k + 2 <= kMaxIntervals, SPK_EUNSUPPORTED,
              "sparse_topk_decode_attn: k=%d (at most %d)", k, kMaxIntervals - 2);
  SPK_REQUIRE(B == 0 || (scores && q && kc && vc && out), SPK_EINVAL,
              "sparse_topk_decode_attn: null scores, q, k, v or out");
  SPK_REQUIRE(s_ld >= n_cand, SPK_EINVAL, "sparse_topk_decode_attn: s_ld < n_cand");
  const int kk = k < n_cand ? k : n_cand;
  SPK_REQUIRE(!sel_idx || sel_ld >= kk, SPK_EINVAL, "sparse_topk_decode_attn: sel_ld < min(k, n)");
  SPK_REQUIRE(kv_sn >= d && kv_sb >= 0 && kv_sh >= 0 && kv_sn % 8 == 0 && kv_sh % 8 == 0 &&
                  kv_sb % 8 == 0,
              SPK_EINVAL, "sparse_topk_decode_attn: kv strides must be multiples of 8 with kv_sn >= d");
  SPK_REQUIRE(kv_sn * 2 < (int64_t)1 << 32, SPK_EUNSUPPORTED,
              "sparse_topk_decode_attn: a KV row stride of 4 GiB or more is not supported");
  SPK_REQUIRE(reinterpret_cast<uintptr_t>(q) % 16 == 0 && reinterpret_cast<uintptr_t>(kc) % 16 == 0 &&
                  reinterpret_cast<uintptr_t>(vc) % 16 == 0,
              SPK_EINVAL, "sparse_topk_decode_attn: q, k, v must be 16-byte aligned");
  SPK_REQUIRE(!(sm_scale != sm_scale), SPK_EINVAL, "sparse_topk_decode_attn: sm_scale is NaN");
  SPK_REQUIRE((int64_t)n_tokens >= (int64_t)kk * gran + n_sink + n_recent, SPK_EUNSUPPORTED,
              "sparse_topk_decode_attn: n_tokens %d below k*gran + n_sink + n_recent", n_tokens);
  // planned as sparse_decode_attn plans the topk_select output (min(k, n_cand) ids per row),
  // so both paths split the rows, and round, identically
  const Plan p = make_plan(SPK_SEL_PER_KV_HEAD, B, 1, Hq, Hkv, d, n_tokens, kk, gran, n_sink,
                           n_recent, true);
  SPK_REQUIRE(ws_bytes >= p.bytes && (p.bytes == 0 || ws), SPK_EWORKSPACE,
              "sparse_topk_decode_attn: workspace %zu bytes < %zu needed", ws_bytes, p.bytes);
  clear_error();
  if (B == 0) return SPK_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* w = reinterpret_cast<char*>(ws);
  const int G = Hq / Hkv;
  AttnArgs a{};
  a.q = q;
  a.q_bf16 = 1;
  a.k = kc;
  a.v = vc;
  a.kv_sb = kv_sb;
  a.kv_sh = kv_sh;
  a.kv_sn = kv_sn;
  a.hbm_slots = n_tokens;
  a.T = 1;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.nq = G;
  a.n_tokens = n_tokens;
  a.tab_cap = p.R + kTabPad;
  a.smax = p.smax;
  a.scale_log2 = sm_scale * kLog2e;
  a.ml = reinterpret_cast<float*>(w + p.off_ml);
  a.acc = reinterpret_cast<float*>(w + p.off_acc);
  a.mask_div = G;
  a.list_mode = kListScores;
  a.list_ld = kk;
  a.count_clamp = p.ubound;
  a.split_bound = p.ubound;
  a.gran = gran;
  a.n_sink = n_sink;
  a.n_recent = n_recent;
  a.ucount = reinterpret_cast<int32_t*>(w + p.off_count);
  a.ucount_valid = 1;
  a.sc_scores = scores;
  a.sc_ld = s_ld;
  a.sc_n = n_cand;
  a.sc_k = k;
  a.sel_out = sel_idx;
  a.count_out = sel_count;
  a.sel_out_ld = sel_ld;
  dim3 grid(p.smax, p.groups);
  hipEvent_t ev_begin = g_timing_begin, ev_end = g_timing_end;
  if (ev_begin && hipEventRecord(ev_begin, st) != hipSuccess)
    return set_error(SPK_EHIP, "sparse_topk_decode_attn: recording the timing event failed");
  if (d == 128) dispatch_scores<128>(p.nq_pad, grid, st, a);
  else dispatch_scores<64>(p.nq_pad, grid, st, a);
  spk_status e = check_launch("sparse_topk_decode_attn/partial");
  if (e != SPK_OK) return e;
  if (ev_end && hipEventRecord(ev_end, st) != hipSuccess)
    return set_error(SPK_EHIP, "sparse_topk_decode_attn: recording the timing event failed");
  if (d == 128)
    hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(p.groups * a.nq), dim3(kWave), 0, st, a,
                       p.nq_pad, out, lse);
  else
    hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(p.groups * a.nq), dim3(kWave), 0, st, a,
                       p.nq_pad, out, lse);
  return check_launch("sparse_topk_decode_attn/combine");
}
