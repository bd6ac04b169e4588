// topk_select: exact top-k of each fp32 score row; ties to the lowest index; indices ascending.
//
// SparDA, §2 "Seleção Esparsa de Lookahead Treinável" (top-k KV blocks) and "Esparsidade de
// Contexto no Tempo de Inferência", §2 "Oracle Top-K" (exact top-k tokens).
//
// One workgroup per row.  Scores map to order-preserving uint32 keys (-0 -> +0, NaN lowest).
//  * n <= 4096: one wave holds the row in registers (up to 64 keys per lane) and needs no
//    barrier at all.
//  * n <= 16384: 256 threads hold the row in registers (up to 64 keys each).  The k-th largest
//    key is found bit by bit from the top: a candidate threshold is kept when at least k keys
//    reach it, the count coming from wave ballots (scalar popcounts) summed across the 4 waves.
//  * larger n: a radix select (4 passes of 8-bit digits, per-wave LDS histograms) over keys
//    re-read from the scores each pass.
// Both finish with one pass in index order that keeps every key above the threshold and the
// first `need` keys equal to it, compacting indices with ballot prefix counts, so the output is
// ascending and ties resolve to the lowest indices.
#include "select_common.h"

namespace spk {
namespace {

constexpr int kSmallThreads = 256;
constexpr int kSmallWaves = kSmallThreads / kWave;
constexpr int kSmallMax = 64 * kSmallThreads;  // 16384
constexpr int kRadixThreads = 1024;

__device__ __forceinline__ uint64_t lanemask_lt() { return (1ull << lane_id()) - 1ull; }

// One wave per row (n <= 4096): item c of lane t is element c*64 + t.  Counting needs only
// ballots and scalar popcounts, so the bit search runs without any barrier.
template <int ITEMS>
__global__ __launch_bounds__(kWave) void topk_wave_kernel(
    const float* __restrict__ scores, int64_t s_ld, int n, int k, int32_t* __restrict__ idx,
    int64_t idx_ld, int32_t* __restrict__ count) {
  const int row = blockIdx.x;
  const float* x = scores + (int64_t)row * s_ld;
  const int kk = min(k, n);
  const int lane = lane_id();
  if (count && lane == 0) count[row] = kk;
  if (kk <= 0) return;
  int32_t* out = idx + (int64_t)row * idx_ld;
  uint32_t key[ITEMS];
#pragma unroll
  for (int c = 0; c < ITEMS; ++c) {
    const int i = c * kWave + lane;
    key[c] = i < n ? order_key(x[i]) : 0u;
  }
  auto count_ge = [&](uint32_t cand) -> int {
    int wc = 0;
#pragma unroll
    for (int c = 0; c < ITEMS; ++c) wc += __popcll(__ballot((c * kWave + lane < n) && key[c] >= cand));
    return wc;
  };
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    if (count_ge(cand) >= kk) thr = cand;
  }
  const int need = kk - (thr == 0xFFFFFFFFu ? 0 : count_ge(thr + 1u));
  int run_gt = 0, run_eq = 0;
  const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int c = 0; c < ITEMS; ++c) {
    const int i = c * kWave + lane;
    const bool valid = i < n;
    const bool gt = valid && key[c] > thr;
    const bool eq = valid && key[c] == thr;
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    const int eq_rank = run_eq + __popcll(be & lt);
    if (gt || (eq && eq_rank < need)) out[run_gt + __popcll(bg & lt) + min(eq_rank, need)] = i;
    run_gt += __popcll(bg);
    run_eq += __popcll(be);
  }
}

// Keys of row `x` held in registers: item c of thread t is element c*256 + t.
template <int ITEMS>
__global__ __launch_bounds__(kSmallThreads) void topk_small_kernel(
    const float* __restrict__ scores, int64_t s_ld, int n, int k, int32_t* __restrict__ idx,
    int64_t idx_ld, int32_t* __restrict__ count) {
  __shared__ int red[2][kSmallWaves][2];
  const int row = blockIdx.x;
  const float* x = scores + (int64_t)row * s_ld;
  const int kk = min(k, n);
  if (count && threadIdx.x == 0) count[row] = kk;
  if (kk <= 0) return;
  int32_t* out = idx + (int64_t)row * idx_ld;
  const int t = threadIdx.x, wid = t / kWave, lane = lane_id();
  uint32_t key[ITEMS];
#pragma unroll
  for (int c = 0; c < ITEMS; ++c) {
    const int i = c * kSmallThreads + t;
    key[c] = i < n ? order_key(x[i]) : 0u;
  }
  // count of valid keys >= cand over the workgroup (one barrier, parity-buffered LDS)
  auto count_ge = [&](uint32_t cand, int parity) -> int {
    int wc = 0;
#pragma unroll
    for (int c = 0; c < ITEMS; ++c) {
      const bool v = (c * kSmallThreads + t < n) && key[c] >= cand;
      wc += __popcll(__ballot(v));
    }
    if (lane == 0) red[parity][wid][0] = wc;
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int w = 0; w < kSmallWaves; ++w) tot += red[parity][w][0];
    return tot;
  };
  uint32_t thr = 0;
  int parity = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    if (count_ge(cand, parity) >= kk) thr = cand;
    parity ^= 1;
  }
  // thr is the kk-th largest key; keys > thr all rank inside the top kk
  const int n_gt = thr == 0xFFFFFFFFu ? 0 : count_ge(thr + 1u, parity);
  parity ^= 1;
  const int need = kk - n_gt;
  int run_gt = 0, run_eq = 0;
#pragma unroll
  for (int c = 0; c < ITEMS; ++c) {
    const int i = c * kSmallThreads + t;
    const bool valid = i < n;
    const bool gt = valid && key[c] > thr;
    const bool eq = valid && key[c] == thr;
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    if (lane == 0) {
      red[parity][wid][0] = __popcll(bg);
      red[parity][wid][1] = __popcll(be);
    }
    __syncthreads();
    int pre_gt = __popcll(bg & lanemask_lt()), pre_eq = __popcll(be & lanemask_lt());
    int tot_gt = 0, tot_eq = 0;
#pragma unroll
    for (int w = 0; w < kSmallWaves; ++w) {
      const int g = red[parity][w][0], e = red[parity][w][1];
      if (w < wid) {
        pre_gt += g;
        pre_eq += e;
      }
      tot_gt += g;
      tot_eq += e;
    }
    const int eq_rank = run_eq + pre_eq;
    if (gt || (eq && eq_rank < need)) out[run_gt + pre_gt + min(eq_rank, need)] = i;
    run_gt += tot_gt;
    run_eq += tot_eq;
    parity ^= 1;
  }
}

template <int ITEMS>
__global__ __launch_bounds__(kRadixThreads) void topk_radix_kernel(
    const float* __restrict__ scores, int64_t s_ld, int n, int k, int32_t* __restrict__ idx,
    int64_t idx_ld, int32_t* __restrict__ count) {
  __shared__ uint32_t hist[kRadixThreads / kWave * 256];
  __shared__ int sh[2];
  __shared__ int scratch[kRadixThreads / kWave + 1];
  const int row = blockIdx.x;
  const float* x = scores + (int64_t)row * s_ld;
  const int kk = min(k, n);
  if (count && threadIdx.x == 0) count[row] = kk;
  if (kk <= 0) return;
  int32_t* out = idx + (int64_t)row * idx_ld;
  if (kk == n) {
    for (int i = threadIdx.x; i < n; i += kRadixThreads) out[i] = i;
    return;
  }
  uint32_t reg[ITEMS > 0 ? ITEMS : 1];
  if constexpr (ITEMS > 0) {
#pragma unroll
    for (int c = 0; c < ITEMS; ++c) {
      const int i = c * kRadixThreads + threadIdx.x;
      reg[c] = i < n ? order_key(x[i]) : 0u;
    }
  }
  auto for_each = [&](auto&& visit) {
    if constexpr (ITEMS > 0) {
#pragma unroll
      for (int c = 0; c < ITEMS; ++c)
        if (c * kRadixThreads + (int)threadIdx.x < n) visit(reg[c]);
    } else {
      for (int i = threadIdx.x; i < n; i += kRadixThreads) visit(order_key(x[i]));
    }
  };
  uint32_t thr;
  int need;
  radix_select<kRadixThreads>(for_each, kk, hist, sh, &thr, &need);

  // Compaction in index order: keep key > thr, and the first `need` keys == thr.
  int run_gt = 0, run_eq = 0;
  const int chunks = (n + kRadixThreads - 1) / kRadixThreads;
  for (int c = 0; c < chunks; ++c) {
    const int i = c * kRadixThreads + threadIdx.x;
    uint32_t key = 0;
    bool valid = i < n;
    if constexpr (ITEMS > 0) {
#pragma unroll
      for (int cc = 0; cc < ITEMS; ++cc)
        if (cc == c) key = reg[cc];
    } else {
      if (valid) key = order_key(x[i]);
    }
    const int gt = valid && key > thr;
    const int eq = valid && key == thr;
    int total;
    const int pre = block_excl_scan(gt | (eq << 16), scratch, &total);
    const int pre_gt = pre & 0xFFFF, pre_eq = pre >> 16;
    if (gt || (eq && run_eq + pre_eq < need))
      out[run_gt + pre_gt + min(run_eq + pre_eq, need)] = i;
    run_gt += total & 0xFFFF;
    run_eq += total >> 16;
  }
}

}  // namespace
}  // namespace spk

extern "C" SPK_API spk_status topk_select_workspace_size(int rows, int n, int k, size_t* bytes) {
  using namespace spk;
  SPK_REQUIRE(bytes, SPK_EINVAL, "topk_select_workspace_size: null bytes");
  SPK_REQUIRE(rows >= 0 && n >= 0, SPK_EINVAL, "topk_select_workspace_size: negative size");
  (void)k;
  *bytes = 0;
  clear_error();
  return SPK_OK;
}

extern "C" SPK_API spk_status topk_select(const float* scores, int64_t s_ld, int rows, int n, int k,
                                          int32_t* idx, int64_t idx_ld, int32_t* count, void* ws,
                                          size_t ws_bytes, void* stream) {
  using namespace spk;
  (void)ws;
  (void)ws_bytes;
  SPK_REQUIRE(rows >= 0 && n >= 0, SPK_EINVAL, "topk_select: rows=%d n=%d", rows, n);
  SPK_REQUIRE(k >= 0, SPK_EINVAL, "topk_select: k=%d < 0", k);
  SPK_REQUIRE(s_ld >= n, SPK_EINVAL, "topk_select: s_ld %lld < n %d", (long long)s_ld, n);
  const int kk = k < n ? k : n;
  SPK_REQUIRE(idx_ld >= kk, SPK_EINVAL, "topk_select: idx_ld %lld < min(k,n) %d",
              (long long)idx_ld, kk);
  SPK_REQUIRE(rows == 0 || ((idx || kk == 0) && (scores || n == 0)), SPK_EINVAL,
              "topk_select: null scores or idx");
  clear_error();
  if (rows == 0) return SPK_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (n <= 64 * kWave) {
    const int items = (n + kWave - 1) / kWave;
#define SPK_WAVE(IT) \
  hipLaunchKernelGGL(topk_wave_kernel<IT>, dim3(rows), dim3(kWave), 0, st, scores, s_ld, n, k, idx, idx_ld, count)
    if (items <= 1) SPK_WAVE(1);
    else if (items <= 2) SPK_WAVE(2);
    else if (items <= 4) SPK_WAVE(4);
    else if (items <= 8) SPK_WAVE(8);
    else if (items <= 16) SPK_WAVE(16);
    else if (items <= 32) SPK_WAVE(32);
    else SPK_WAVE(64);
#undef SPK_WAVE
  } else if (n <= kSmallMax) {
    const int items = (n + kSmallThreads - 1) / kSmallThreads;
#define SPK_SMALL(IT)                                                                          \
  hipLaunchKernelGGL(topk_small_kernel<IT>, dim3(rows), dim3(kSmallThreads), 0, st, scores, s_ld, \
                     n, k, idx, idx_ld, count)
    if (items <= 1) SPK_SMALL(1);
    else if (items <= 2) SPK_SMALL(2);
    else if (items <= 4) SPK_SMALL(4);
    else if (items <= 8) SPK_SMALL(8);
    else if (items <= 16) SPK_SMALL(16);
    else if (items <= 32) SPK_SMALL(32);
    else SPK_SMALL(64);
#undef SPK_SMALL
  } else {
    hipLaunchKernelGGL(topk_radix_kernel<0>, dim3(rows), dim3(kRadixThreads), 0, st, scores, s_ld,
                       n, k, idx, idx_ld, count);
  }
  return check_launch("topk_select");
}
