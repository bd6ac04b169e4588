// tier_classify: T0 / T1 / T2 / T3 tiers by cumulative importance, sinks and recent window
// protected.
//
// "Nem Todos os Pensamentos Necessitam de HBM", §1 "Classificação de Quatro Níveis": protected
// tokens and the most important ones stay in T0 (HBM); the middle goes to T1 (full precision in
// host DDR, fetched before attention); low importance may go to T2 (kept at 8 bits); only the
// least important tail is T3 (evicted for good).  §4: the classification is redone
// periodically; the period is the caller's loop.
//
// One workgroup (1024 threads) per sequence.  The unprotected tokens get order-preserving keys
// (evicted or NaN -> 0, the lowest), radix searches (8-bit digits, one barrier per pass) find
// the keys at ranks floor(M*t0/1000), floor(M*t01/1000) and, with a T2 quota,
// floor(M*t012/1000); ranks in index order (ties at the thresholds to the lower index, then
// positions in the ascending list of attended rows T0 ∪ T1 ∪ T2) come from per-(chunk, wave)
// ballot counts turned into prefixes by one wave scan, so assigning tiers, marking new
// evictions and compacting the list take four barriers, six with T2 (sequences of up to 16384
// tokens, whose keys stay in registers; longer ones rank chunk by chunk with block scans).
#include "select_common.h"

namespace spk {
namespace {

constexpr int kThreads = 1024;
constexpr int kItems = 16;

template <int ITEMS>
__global__ __launch_bounds__(kThreads) void tier_kernel(
    const float* __restrict__ s_all, int64_t s_ld, int n, int n_sink, int n_recent, int p0,
    int p01, int p012, uint8_t* __restrict__ evicted, int64_t ev_ld, uint8_t* __restrict__ tier_all,
    int64_t tier_ld, int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_count,
    int64_t sel_ld) {
  __shared__ __align__(16) uint32_t hist[4 * 256];
  __shared__ int scratch[kThreads / kWave + 1];
  // per-(chunk, wave) counts of the register path, then their prefixes (+ the total)
  __shared__ int cw_eq[(ITEMS > 0 ? ITEMS : 1) * (kThreads / kWave) + 1];
  __shared__ int cw_eq2[(ITEMS > 0 ? ITEMS : 1) * (kThreads / kWave) + 1];
  __shared__ int cw_sel[(ITEMS > 0 ? ITEMS : 1) * (kThreads / kWave) + 1];
  const int b = blockIdx.x;
  if (n <= 0) {
    if (sel_count && threadIdx.x == 0) sel_count[b] = 0;
    return;
  }
  const float* s = s_all + (int64_t)b * s_ld;
  uint8_t* ev = evicted ? evicted + (int64_t)b * ev_ld : nullptr;
  uint8_t* tier = tier_all + (int64_t)b * tier_ld;
  const int lo = min(n_sink, n);
  const int hi = max(lo, n - n_recent);
  const int M = hi - lo;
  const int n0 = (int)(((int64_t)M * p0) / 1000);
  const int n01 = (int)(((int64_t)M * p01) / 1000);
  const int n012 = (int)(((int64_t)M * p012) / 1000);
  const bool has_t2 = n012 > n01;  // uniform: the T2 search and tie counts run only then

  auto key_of = [&](int i) -> uint32_t {
    if (ev && ev[i]) return 0u;
    return order_key(s[i]);
  };
  uint32_t reg[ITEMS > 0 ? ITEMS : 1];
  uint8_t ev_v[ITEMS > 0 ? ITEMS : 1];  // the evicted flags as they were on entry
  if constexpr (ITEMS > 0) {
    // every load issued before any is used (clamped in bounds): one wait for the sequence
    float sv[ITEMS];
#pragma unroll
    for (int c = 0; c < ITEMS; ++c) {
      const int ic = min(c * kThreads + (int)threadIdx.x, n - 1);
      sv[c] = s[ic];
      ev_v[c] = ev ? ev[ic] : (uint8_t)0;
    }
#pragma unroll
    for (int c = 0; c < ITEMS; ++c) {
      const int i = c * kThreads + threadIdx.x;
      reg[c] = (i >= lo && i < hi && !ev_v[c]) ? order_key(sv[c]) : 0u;
    }
  }
  auto for_each = [&](auto&& visit) {
    if constexpr (ITEMS > 0) {
#pragma unroll
      for (int c = 0; c < ITEMS; ++c) {
        const int i = c * kThreads + threadIdx.x;
        if (i >= lo && i < hi) visit(reg[c]);
      }
    } else {
      for (int i = lo + threadIdx.x; i < hi; i += kThreads) visit(key_of(i));
    }
  };
  // thresholds at ranks n0 and n01: one-barrier-per-pass radix searches; when a search ends on
  // a bin that holds exactly the missing keys, every key >= the threshold is kept (need = all)
  uint32_t thr0 = 0xFFFFFFFFu, thr1 = 0xFFFFFFFFu, thr2 = 0xFFFFFFFFu;
  int need0 = 0, need1 = 0, need2 = 0;
  auto search = [&](int rank, uint32_t* thr, int* need) {
    for (int i = threadIdx.x; i < 4 * 256; i += kThreads) hist[i] = 0u;
    __syncthreads();
    bool whole;
    radix_threshold(for_each, rank, hist, thr, need, &whole);
    if (whole) *need = 0x7FFFFFFF;
    __syncthreads();  // every wave is done reading the histograms
  };
  if (n0 > 0) search(n0, &thr0, &need0);
  if (n01 > 0) search(n01, &thr1, &need1);
  if (has_t2) search(n012, &thr2, &need2);

  if constexpr (ITEMS > 0) {
    // ranks in index order (chunk c, then wave, then lane) from per-(chunk, wave) counts: one
    // barrier to publish the counts, one wave scan over them, one barrier to read the prefixes;
    // first for the ties at each threshold, then for the list of attended rows
    constexpr int NWV = kThreads / kWave;
    constexpr int NCW = ITEMS * NWV;
    const int lane = lane_id(), wid = threadIdx.x / kWave;
    const uint64_t lt = (1ull << lane) - 1ull;
    auto prefixes = [&](int* cw) {  // cw[NCW] counts -> exclusive prefixes; returns the total
      __syncthreads();
      if (wid == 0) {
        int carry = 0;
#pragma unroll
        for (int base = 0; base < NCW; base += kWave) {
          const int i = base + lane;
          const int v = i < NCW ? cw[i] : 0;
          const int incl = wave_incl_scan(v);
          if (i < NCW) cw[i] = carry + incl - v;
          carry += __builtin_amdgcn_readlane(incl, kWave - 1);
        }
        if (lane == 0) cw[NCW] = carry;
      }
      __syncthreads();
      return cw[NCW];
    };
    // first sweep: ties at the thresholds (evicted candidates hold ranks too)
#pragma unroll
    for (int c = 0; c < ITEMS; ++c) {
      const int i = c * kThreads + threadIdx.x;
      const bool cand = i >= lo && i < hi;
      const int e0 = __popcll(__ballot(cand && n0 > 0 && reg[c] == thr0));
      const int e1 = __popcll(__ballot(cand && n01 > 0 && reg[c] == thr1));
      const int e2 = __popcll(__ballot(cand && has_t2 && reg[c] == thr2));
      if (lane == 0) {
        cw_eq[c * NWV + wid] = e0 | (e1 << 16);
        cw_eq2[c * NWV + wid] = e2;
      }
    }
    prefixes(cw_eq);
    if (has_t2) prefixes(cw_eq2);
    // second sweep: tiers, evictions, and the per-(chunk, wave) counts of the list
    uint32_t selbits = 0;
#pragma unroll
    for (int c = 0; c < ITEMS; ++c) {
      const int i = c * kThreads + threadIdx.x;
      const bool valid = i < n;
      const bool cand = i >= lo && i < hi;
      const uint32_t key = reg[c];
      const bool eq0 = cand && n0 > 0 && key == thr0;
      const bool eq1 = cand && n01 > 0 && key == thr1;
      const bool eq2 = cand && has_t2 && key == thr2;
      const int pre = cw_eq[c * NWV + wid];
      const int eqrank0 = (pre & 0xFFFF) + __popcll(__ballot(eq0) & lt);
      const int eqrank1 = (pre >> 16) + __popcll(__ballot(eq1) & lt);
      const int eqrank2 = (has_t2 ? cw_eq2[c * NWV + wid] : 0) + __popcll(__ballot(eq2) & lt);
      const bool is_ev = cand && ev_v[c];
      const bool top0 = cand && n0 > 0 && (key > thr0 || (eq0 && eqrank0 < need0));
      const bool top1 = cand && n01 > 0 && (key > thr1 || (eq1 && eqrank1 < need1));
      const bool top2 = cand && has_t2 && (key > thr2 || (eq2 && eqrank2 < need2));
      uint8_t t = 3;
      if (!cand) t = 0;
      else if (is_ev) t = 3;
      else if (top0) t = 0;
      else if (top1) t = 1;
      else if (top2) t = 2;
      const bool sel = valid && t <= 2;
      selbits |= (sel ? 1u : 0u) << c;
      if (valid) {
        tier[i] = t;
        if (ev && t == 3) ev[i] = 1;
      }
      const int nsel = __popcll(__ballot(sel));  // every lane votes: outside the lane-0 branch
      if (lane == 0) cw_sel[c * NWV + wid] = nsel;
    }
    const int total_sel = prefixes(cw_sel);
    if (sel_idx) {
#pragma unroll
      for (int c = 0; c < ITEMS; ++c) {
        const bool sel = (selbits >> c) & 1u;
        const int pos = cw_sel[c * NWV + wid] + __popcll(__ballot(sel) & lt);
        if (sel) sel_idx[(int64_t)b * sel_ld + pos] = c * kThreads + threadIdx.x;
      }
    }
    if (sel_count && threadIdx.x == 0) sel_count[b] = total_sel;
    return;
  }
  int run_eq0 = 0, run_eq1 = 0, run_eq2 = 0, run_sel = 0;
  const int chunks = (n + kThreads - 1) / kThreads;
  for (int c = 0; c < chunks; ++c) {
    const int i = c * kThreads + threadIdx.x;
    const bool valid = i < n;
    const bool cand = i >= lo && i < hi;
    uint32_t key = 0;
    if (cand) {
      if constexpr (ITEMS > 0) {
#pragma unroll
        for (int cc = 0; cc < ITEMS; ++cc)
          if (cc == c) key = reg[cc];
      } else {
        key = key_of(i);
      }
    }
    // ties at each threshold, counted over candidates in index order (evicted ones included:
    // they hold ranks too)
    const int eq0 = cand && n0 > 0 && key == thr0;
    const int eq1 = cand && n01 > 0 && key == thr1;
    const int eq2 = cand && has_t2 && key == thr2;
    int tot, tot2 = 0;
    const int pre = block_excl_scan(eq0 | (eq1 << 16), scratch, &tot);
    const int pre2 = has_t2 ? block_excl_scan(eq2, scratch, &tot2) : 0;
    const int eqrank0 = run_eq0 + (pre & 0xFFFF);
    const int eqrank1 = run_eq1 + (pre >> 16);
    const int eqrank2 = run_eq2 + pre2;
    const bool is_ev = cand && ev && ev[i];
    const bool top0 = cand && n0 > 0 && (key > thr0 || (eq0 && eqrank0 < need0));
    const bool top1 = cand && n01 > 0 && (key > thr1 || (eq1 && eqrank1 < need1));
    const bool top2 = cand && has_t2 && (key > thr2 || (eq2 && eqrank2 < need2));
    uint8_t t = 3;
    if (!cand) t = 0;
    else if (is_ev) t = 3;
    else if (top0) t = 0;
    else if (top1) t = 1;
    else if (top2) t = 2;
    const int sel = valid && t <= 2;
    int tot_sel;
    const int pos = block_excl_scan(sel, scratch, &tot_sel);
    if (valid) {
      tier[i] = t;
      if (ev && t == 3) ev[i] = 1;
      if (sel && sel_idx) sel_idx[(int64_t)b * sel_ld + run_sel + pos] = i;
    }
    run_eq0 += tot & 0xFFFF;
    run_eq1 += tot >> 16;
    run_eq2 += tot2;
    run_sel += tot_sel;
  }
  if (sel_count && threadIdx.x == 0) sel_count[b] = run_sel;
}

}  // namespace
}  // namespace spk

extern "C" SPK_API spk_status tier_classify_workspace_size(int B, int n_tokens, size_t* bytes) {
  using namespace spk;
  SPK_REQUIRE(bytes, SPK_EINVAL, "tier_classify_workspace_size: null bytes");
  SPK_REQUIRE(B >= 0 && n_tokens >= 0, SPK_EINVAL, "tier_classify_workspace_size: negative size");
  *bytes = 0;
  clear_error();
  return SPK_OK;
}

extern "C" SPK_API spk_status tier_classify(const float* s, int64_t s_ld, int B, int n_tokens,
                                            int n_sink, int n_recent, int t0_permille,
                                            int t01_permille, int t012_permille,
                                            uint8_t* evicted, int64_t ev_ld,
                                            uint8_t* tier, int64_t tier_ld, int32_t* sel_idx,
                                            int32_t* sel_count, int64_t sel_ld, void* ws,
                                            size_t ws_bytes, void* stream) {
  using namespace spk;
  (void)ws;
  (void)ws_bytes;
  SPK_REQUIRE(B >= 0 && n_tokens >= 0 && n_sink >= 0 && n_recent >= 0, SPK_EINVAL,
              "tier_classify: negative size");
  SPK_REQUIRE(n_tokens < (1 << 30), SPK_EINVAL, "tier_classify: n_tokens too large");
  SPK_REQUIRE(0 <= t0_permille && t0_permille <= t01_permille && t01_permille <= t012_permille &&
                  t012_permille <= 1000,
              SPK_EINVAL,
              "tier_classify: need 0 <= t0_permille (%d) <= t01_permille (%d) <= t012_permille "
              "(%d) <= 1000",
              t0_permille, t01_permille, t012_permille);
  SPK_REQUIRE(B == 0 || n_tokens == 0 || (s && tier), SPK_EINVAL, "tier_classify: null s or tier");
  SPK_REQUIRE(s_ld >= n_tokens && tier_ld >= n_tokens, SPK_EINVAL,
              "tier_classify: s_ld/tier_ld smaller than n_tokens");
  SPK_REQUIRE(!evicted || ev_ld >= n_tokens, SPK_EINVAL, "tier_classify: ev_ld < n_tokens");
  SPK_REQUIRE(!sel_idx || sel_ld >= n_tokens, SPK_EINVAL, "tier_classify: sel_ld < n_tokens");
  SPK_REQUIRE((sel_idx == nullptr) == (sel_count == nullptr), SPK_EINVAL,
              "tier_classify: sel_idx and sel_count go together");
  clear_error();
  if (B == 0) return SPK_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (n_tokens <= kItems * kThreads) {
    hipLaunchKernelGGL(tier_kernel<kItems>, dim3(B), dim3(kThreads), 0, st, s, s_ld, n_tokens,
                       n_sink, n_recent, t0_permille, t01_permille, t012_permille, evicted, ev_ld,
                       tier, tier_ld, sel_idx, sel_count, sel_ld);
  } else {
    hipLaunchKernelGGL(tier_kernel<0>, dim3(B), dim3(kThreads), 0, st, s, s_ld, n_tokens, n_sink,
                       n_recent, t0_permille, t01_permille, t012_permille, evicted, ev_ld, tier,
                       tier_ld, sel_idx, sel_count, sel_ld);
  }
  return check_launch("tier_classify");
}
