// topk_select: exact top-k of each fp32 score row; ties to the lowest index; indices ascending.
//
// SparDA, §2 "Seleção Esparsa de Lookahead Treinável" (top-k KV blocks) and "Esparsidade de
// Contexto no Tempo de Inferência", §2 "Oracle Top-K" (exact top-k tokens).
//
// One workgroup per row.  Scores map to order-preserving uint32 keys (-0 -> +0, NaN lowest).
//  * n <= 16384: 256 threads hold the row in registers (up to 64 keys each); a radix search
//    (8-bit digits, one LDS histogram per digit, one barrier per pass, stopping once a digit's
//    bin holds exactly the keys still missing) finds the k-th largest key.
//  * larger n: a 12-bit histogram finds the bin of the k-th key, that bin's keys are gathered
//    into LDS and bit-searched for the exact threshold (a full radix select when ties overflow
//    the store), and each wave compacts its own contiguous segment in index order.
// Both finish with one pass in index order that keeps every key above the threshold and the
// first `need` keys equal to it, compacting indices with ballot prefix counts, so the output is
// ascending and ties resolve to the lowest indices.
#include "select_common.h"

namespace spk {
namespace {

constexpr int kSmallThreads = 256;
constexpr int kSmallWaves = kSmallThreads / kWave;
constexpr int kSmallMax = 64 * kSmallThreads;  // 16384


// Rows of up to 64*256 keys held in registers (KPT per thread); reg_topk selects with one
// barrier per radix pass and one or two for the compaction counts.
template <int KPT>
__global__ __launch_bounds__(kSmallThreads) void topk_reg_kernel(
    const float* __restrict__ scores, int64_t s_ld, int n, int k, int32_t* __restrict__ idx,
    int64_t idx_ld, int32_t* __restrict__ count) {
  __shared__ __align__(16) uint32_t hist[4 * 256];
  __shared__ __align__(16) int wsum[KPT * kSmallWaves];
  const int row = blockIdx.x;
  const int kk = min(k, n);
  if (count && threadIdx.x == 0) count[row] = kk;
  if (kk <= 0) return;
  const float* x = scores + (int64_t)row * s_ld;
  int32_t* out = idx + (int64_t)row * idx_ld;
  // every load issued before any is used (clamped in bounds): one wait for the row
  float v[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) v[j] = x[min(j * kSmallThreads + (int)threadIdx.x, n - 1)];
  uint32_t key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    key[j] = j * kSmallThreads + (int)threadIdx.x < n ? order_key(v[j]) : 0u;
  reg_topk<kSmallThreads>(key, n, kk, hist, wsum, [&](int pos, int i) { out[pos] = i; });
}

// ---------------------------------------------------------------- wide rows (n > 16384)
//
// Two launches.  (1) topk_hist_kernel: the row is cut into C chunks, one workgroup each, and
// every chunk's histogram of the top 12 key bits goes to the workspace.  (2) topk_final_kernel,
// one 1024-thread workgroup per row: sums the C histograms and finds the bin b* holding the k-th
// largest key; one read of the row puts, per wave and in index order, the keys above bin b*
// (all kept) and the keys of bin b* (candidates) into LDS lists; a bit search over the low 20
// bits of the candidates finds the exact threshold; every wave then writes its kept entries
// at offsets from prefix counts over the earlier waves — ascending, ties to the lowest index.
// When bin b* or a wave's list overflows its LDS store (heavy ties, very large k) the row falls
// back to a full radix select and a streaming compaction.
constexpr int kLargeThreads = 1024;
constexpr int kLargeWaves = kLargeThreads / kWave;
constexpr int kBins = 4096;
constexpr int kBinShift = 20;
constexpr int kHistThreads = 256;
constexpr int kListPerWave = 496;  // LDS list entries per wave: two workgroups fit one CU's LDS
constexpr int kCandMax = kLargeWaves * kListPerWave;  // candidates the LDS lists can hold

int hist_chunks(int rows) {
  const int want = (4 * num_cus() + rows - 1) / (rows > 0 ? rows : 1);
  return want < 1 ? 1 : (want > 32 ? 32 : want);
}

// Keys of elements i..i+3 of a row of n >= 4 elements, loaded without branches, so a batch of
// calls issues all its loads before the first wait.  ALIGNED (16-byte aligned rows): one 16-byte
// load from min(i, last), last = the start of the row's last full group of four; the group past
// it (the row's final n % 4 elements) reads that last group back instead, so the caller takes
// those few elements with keys_tail.  Unaligned rows: four clamped 4-byte loads.
template <bool ALIGNED>
__device__ __forceinline__ uint4 keys4_load(const float* x, int i, int n) {
  if constexpr (ALIGNED) {
    const float4 v = *reinterpret_cast<const float4*>(x + min(i, (n - 4) & ~3));
    return make_uint4(order_key(v.x), order_key(v.y), order_key(v.z), order_key(v.w));
  } else {
    return make_uint4(order_key(x[min(i, n - 1)]), order_key(x[min(i + 1, n - 1)]),
                      order_key(x[min(i + 2, n - 1)]), order_key(x[min(i + 3, n - 1)]));
  }
}
// Whether the group at i holds its own elements under keys4_load.
template <bool ALIGNED>
__device__ __forceinline__ bool keys4_own(int i, int n) {
  return !ALIGNED || i <= ((n - 4) & ~3);
}
// First element keys4_load does not deliver (n when it delivers all of them).
template <bool ALIGNED>
__device__ __forceinline__ int keys4_tail(int n) {
  return ALIGNED ? ((n - 4) & ~3) + 4 : n;
}

template <bool ALIGNED>
__global__ __launch_bounds__(kHistThreads) void topk_hist_kernel(const float* __restrict__ scores,
                                                                 int64_t s_ld, int n, int k,
                                                                 int C, uint32_t* __restrict__ ws) {
  __shared__ uint32_t hist[kBins];
  const int row = blockIdx.y, c = blockIdx.x;
  const int kk = min(k, n);
  uint32_t* out = ws + ((int64_t)row * C + c) * kBins;
  if (kk <= 0 || kk == n) return;  // the final kernel needs no histogram then
  const float* x = scores + (int64_t)row * s_ld;
  const int chunk = ((n + C - 1) / C + 1023) / 1024 * 1024;
  const int beg = min(n, c * chunk), end = min(n, beg + chunk);
  for (int i = threadIdx.x; i < kBins; i += kHistThreads) hist[i] = 0u;
  __syncthreads();
  constexpr int UA = 4;
  for (int i0 = beg + 4 * threadIdx.x; i0 < end; i0 += 4 * kHistThreads * UA) {
    uint4 kq[UA];
#pragma unroll
    for (int u = 0; u < UA; ++u) kq[u] = keys4_load<ALIGNED>(x, i0 + u * 4 * kHistThreads, n);
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int i = i0 + u * 4 * kHistThreads;
      if (!keys4_own<ALIGNED>(i, n)) continue;
      if (i < end) atomicAdd(&hist[kq[u].x >> kBinShift], 1u);
      if (i + 1 < end) atomicAdd(&hist[kq[u].y >> kBinShift], 1u);
      if (i + 2 < end) atomicAdd(&hist[kq[u].z >> kBinShift], 1u);
      if (i + 3 < end) atomicAdd(&hist[kq[u].w >> kBinShift], 1u);
    }
  }
  {
    // the row's final n % 4 elements, when keys4_load did not deliver them
    const int t = keys4_tail<ALIGNED>(n) + (int)threadIdx.x;
    if (threadIdx.x < 3 && t < n && t >= beg && t < end)
      atomicAdd(&hist[order_key(x[t]) >> kBinShift], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kBins; i += kHistThreads) out[i] = hist[i];
}

// Sum over the wave of one int per lane (every lane gets the total).
__device__ __forceinline__ int wave_sum(int x) {
  x = (int)group_sum<16>((float)x);  // exact: partial sums stay far below 2^24
  x += __shfl_xor(x, 16, kWave);
  x += __shfl_xor(x, 32, kWave);
  return x;
}

// Two 1024-thread workgroups per CU (at most 64 VGPRs and 80 KB of LDS each), so rows beyond the
// CU count still run in one round.
template <bool ALIGNED>
__global__ __launch_bounds__(kLargeThreads) __attribute__((amdgpu_waves_per_eu(8))) void topk_final_kernel(
    const float* __restrict__ scores, int64_t s_ld, int n, int k, int C,
    const uint32_t* __restrict__ ws, int32_t* __restrict__ idx, int64_t idx_ld,
    int32_t* __restrict__ count) {
  __shared__ __align__(16) uint32_t hist[kBins];
  __shared__ uint32_t lkey[kLargeWaves * kListPerWave];
  __shared__ int32_t lidx[kLargeWaves * kListPerWave];
  __shared__ int wave_n[kLargeWaves], wave_gt[kLargeWaves], wave_eq[kLargeWaves];
  __shared__ int sh[8];
  __shared__ int red[kLargeWaves + 1];
  const int row = blockIdx.x;
  const float* x = scores + (int64_t)row * s_ld;
  const int kk = min(k, n);
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  if (count && tid == 0) count[row] = kk;
  if (kk <= 0) return;
  int32_t* out = idx + (int64_t)row * idx_ld;
  if (kk == n) {
    for (int i = tid; i < n; i += kLargeThreads) out[i] = i;
    return;
  }
  const uint64_t lt = (1ull << lane) - 1ull;
  // wave w's segment of the row: [w*seg, min(n, (w+1)*seg)), seg a multiple of 256
  const int seg = ((n + kLargeWaves - 1) / kLargeWaves + 255) / 256 * 256;
  const int sbeg = min(n, wid * seg), send = min(n, sbeg + seg);

  // ---- sum the chunk histograms (every load of a chunk pair in flight at once), find bin b*
  const uint32_t* hrow = ws + (int64_t)row * C * kBins;
  {
    constexpr int BPT = kBins / kLargeThreads;  // bins per thread
    uint32_t t[BPT];
#pragma unroll
    for (int j = 0; j < BPT; ++j) t[j] = 0u;
    for (int c = 0; c < C; c += 2) {
      uint32_t v[2][BPT];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int j = 0; j < BPT; ++j)
          v[cc][j] = c + cc < C ? hrow[(int64_t)(c + cc) * kBins + j * kLargeThreads + tid] : 0u;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int j = 0; j < BPT; ++j) t[j] += v[cc][j];
    }
#pragma unroll
    for (int j = 0; j < BPT; ++j) hist[j * kLargeThreads + tid] = t[j];
  }
  if (tid == 0) sh[3] = 0;  // overflow flag
  __syncthreads();
  {
    const int top = kBins - 1 - 4 * tid;
    const int c0 = hist[top], c1 = hist[top - 1], c2 = hist[top - 2], c3 = hist[top - 3];
    const int sum = c0 + c1 + c2 + c3;
    int total;
    const int excl = block_excl_scan(sum, red, &total);
    if (excl < kk && kk <= excl + sum) {
      int acc = excl;
      if (acc + c0 >= kk) { sh[0] = top; sh[1] = acc; }
      else if ((acc += c0) + c1 >= kk) { sh[0] = top - 1; sh[1] = acc; }
      else if ((acc += c1) + c2 >= kk) { sh[0] = top - 2; sh[1] = acc; }
      else { acc += c2; sh[0] = top - 3; sh[1] = acc; }
    }
  }
  __syncthreads();
  const uint32_t bstar = (uint32_t)sh[0];
  const int kin = kk - sh[1];  // rank of the threshold inside bin b*
  bool overflow = (int)hist[bstar] > kCandMax;

  // ---- gather: per wave, in index order, keys above b* (flag bit 31 of the index) and keys of b*
  uint32_t* mykey = lkey + wid * kListPerWave;
  int32_t* myidx = lidx + wid * kListPerWave;
  int nl = 0;
  if (!overflow) {
    constexpr int UB = 8;
    for (int c0 = sbeg; c0 < send; c0 += 256 * UB) {
      uint4 kq[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u) kq[u] = keys4_load<ALIGNED>(x, c0 + 256 * u + 4 * lane, n);
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int i = c0 + 256 * u + 4 * lane;
        const bool own = keys4_own<ALIGNED>(i, n);
        const uint32_t kv[4] = {kq[u].x, kq[u].y, kq[u].z, kq[u].w};
        bool take[4];
        int before = 0, tot = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          take[j] = own && i + j < send && (kv[j] >> kBinShift) >= bstar;
          // index order is lane, then j: this lane's entries follow every entry of lower lanes
          const uint64_t bj = __ballot(take[j]);
          before += __popcll(bj & lt);
          tot += __popcll(bj);
        }
        if (tot > 0) {
          if (nl + tot <= kListPerWave) {
            int p = nl + before;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if (take[j]) {
                mykey[p] = kv[j];
                myidx[p] = i + j;
                ++p;
              }
            }
          } else {
            overflow = true;
          }
          nl += tot;
        }
      }
    }
    {
      // the row's final n % 4 elements, when keys4_load did not deliver them (index order: they
      // follow everything this wave took)
      const int t = keys4_tail<ALIGNED>(n) + lane;
      const uint32_t kv = lane < 3 && t < n ? order_key(x[t]) : 0u;
      const bool take = lane < 3 && t < n && t >= sbeg && t < send && (kv >> kBinShift) >= bstar;
      const uint64_t bt = __ballot(take);
      if (bt) {
        const int tot = __popcll(bt);
        if (nl + tot <= kListPerWave) {
          if (take) {
            mykey[nl + __popcll(bt & lt)] = kv;
            myidx[nl + __popcll(bt & lt)] = t;
          }
        } else {
          overflow = true;
        }
        nl += tot;
      }
    }
    if (lane == 0) {
      wave_n[wid] = nl;
      if (overflow) sh[3] = 1;
    }
  }
  __syncthreads();
  overflow = overflow || sh[3] != 0;

  uint32_t thr;
  int need;
  if (!overflow) {
    // ---- threshold inside bin b*: radix search over the candidates' low 20 bits (moved to the
    // top of the key), one LDS histogram per digit and one barrier per pass
    // the bin histogram is no longer read (a barrier followed the gather): reuse it
    for (int i = tid; i < 4 * 256; i += kLargeThreads) hist[i] = 0u;
    __syncthreads();
    bool whole;
    {
      uint32_t tthr;
      int tneed;
      radix_threshold(
          [&](auto visit) {
            for (int j = lane; j < nl; j += kWave) {
              const uint32_t kv = mykey[j];
              if ((kv >> kBinShift) == bstar) visit(kv << (32 - kBinShift));
            }
          },
          kin, hist, &tthr, &tneed, &whole);
      thr = (bstar << kBinShift) | (tthr >> (32 - kBinShift));
      need = tneed;
    }
    // per-wave kept counts: every entry above the threshold, and ties in index order up to need
    // (when the search ended on a bin holding exactly the missing keys, every key >= thr)
    int g = 0, e = 0;
    for (int j = lane; j < nl; j += kWave) {
      const uint32_t kv = mykey[j];
      g += whole ? kv >= thr : kv > thr;
      e += !whole && kv == thr;
    }
    g = wave_sum(g);
    e = wave_sum(e);
    if (lane == 0) {
      wave_gt[wid] = g;
      wave_eq[wid] = e;
    }
    __syncthreads();
    int gt_all = 0, run_gt = 0, run_eq = 0;
#pragma unroll
    for (int w = 0; w < kLargeWaves; ++w) {
      gt_all += wave_gt[w];
      if (w < wid) {
        run_gt += wave_gt[w];
        run_eq += wave_eq[w];
      }
    }
    need = kk - gt_all;
    // ---- write the kept entries of this wave's list, in index order
    for (int j0 = 0; j0 < nl; j0 += kWave) {
      const int j = j0 + lane;
      const uint32_t kv = j < nl ? mykey[j] : 0u;
      const bool gt = j < nl && (whole ? kv >= thr : kv > thr);
      const bool eq = j < nl && !whole && kv == thr;
      const uint64_t bg = __ballot(gt), be = __ballot(eq);
      const int eq_rank = run_eq + __popcll(be & lt);
      if (gt || (eq && eq_rank < need)) out[run_gt + __popcll(bg & lt) + min(eq_rank, need)] = myidx[j];
      run_gt += __popcll(bg);
      run_eq += __popcll(be);
    }
    return;
  }

  // ---- fallback: full radix select over the row and a streaming compaction
  {
    auto for_each = [&](auto&& visit) {
      for (int i = tid; i < n; i += kLargeThreads) visit(order_key(x[i]));
    };
    radix_select<kLargeThreads>(for_each, kk, hist, sh, &thr, &need);
    int g = 0, e = 0;
    for (int c = sbeg; c < send; c += 64) {
      const int i = c + lane;
      const uint32_t kv = i < send ? order_key(x[i]) : 0u;
      g += __popcll(__ballot(i < send && kv > thr));
      e += __popcll(__ballot(i < send && kv == thr));
    }
    if (lane == 0) {
      wave_gt[wid] = g;
      wave_eq[wid] = e;
    }
    __syncthreads();
    int run_gt = 0, run_eq = 0;
    for (int w = 0; w < wid; ++w) {
      run_gt += wave_gt[w];
      run_eq += wave_eq[w];
    }
    for (int c = sbeg; c < send; c += 64) {
      const int i = c + lane;
      const uint32_t kv = i < send ? order_key(x[i]) : 0u;
      const bool gt = i < send && kv > thr, eq = i < send && kv == thr;
      const uint64_t bg = __ballot(gt), be = __ballot(eq);
      const int eq_rank = run_eq + __popcll(be & lt);
      if (gt || (eq && eq_rank < need)) out[run_gt + __popcll(bg & lt) + min(eq_rank, need)] = i;
      run_gt += __popcll(bg);
      run_eq += __popcll(be);
    }
  }
}

}  // namespace
}  // namespace spk

extern "C" SPK_API spk_status topk_select_workspace_size(int rows, int n, int k, size_t* bytes) {
  using namespace spk;
  SPK_REQUIRE(bytes, SPK_EINVAL, "topk_select_workspace_size: null bytes");
  SPK_REQUIRE(rows >= 0 && n >= 0, SPK_EINVAL, "topk_select_workspace_size: negative size");
  (void)k;
  *bytes = n > kSmallMax ? (size_t)rows * hist_chunks(rows) * kBins * sizeof(uint32_t) : 0;
  clear_error();
  return SPK_OK;
}

extern "C" SPK_API spk_status topk_select(const float* scores, int64_t s_ld, int rows, int n, int k,
                                          int32_t* idx, int64_t idx_ld, int32_t* count, void* ws,
                                          size_t ws_bytes, void* stream) {
  using namespace spk;
  SPK_REQUIRE(rows >= 0 && n >= 0, SPK_EINVAL, "topk_select: rows=%d n=%d", rows, n);
  SPK_REQUIRE(k >= 0, SPK_EINVAL, "topk_select: k=%d < 0", k);
  SPK_REQUIRE(s_ld >= n, SPK_EINVAL, "topk_select: s_ld %lld < n %d", (long long)s_ld, n);
  const int kk = k < n ? k : n;
  SPK_REQUIRE(idx_ld >= kk, SPK_EINVAL, "topk_select: idx_ld %lld < min(k,n) %d",
              (long long)idx_ld, kk);
  SPK_REQUIRE(rows == 0 || ((idx || kk == 0) && (scores || n == 0)), SPK_EINVAL,
              "topk_select: null scores or idx");
  const size_t need_ws = n > kSmallMax ? (size_t)rows * hist_chunks(rows) * kBins * sizeof(uint32_t) : 0;
  SPK_REQUIRE(ws_bytes >= need_ws && (need_ws == 0 || ws), SPK_EWORKSPACE,
              "topk_select: workspace %zu bytes < %zu needed", ws_bytes, need_ws);
  clear_error();
  if (rows == 0) return SPK_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (n <= kSmallMax) {
    const int kpt = (n + kSmallThreads - 1) / kSmallThreads;
#define SPK_REG(KPT)                                                                           \
  hipLaunchKernelGGL(topk_reg_kernel<KPT>, dim3(rows), dim3(kSmallThreads), 0, st, scores, s_ld, \
                     n, k, idx, idx_ld, count)
    if (kpt <= 1) SPK_REG(1);
    else if (kpt <= 2) SPK_REG(2);
    else if (kpt <= 4) SPK_REG(4);
    else if (kpt <= 8) SPK_REG(8);
    else if (kpt <= 16) SPK_REG(16);
    else if (kpt <= 32) SPK_REG(32);
    else SPK_REG(64);
#undef SPK_REG
  } else {
    const int C = hist_chunks(rows);
    uint32_t* h = reinterpret_cast<uint32_t*>(ws);
    // rows start 16-byte aligned when the base is and the row stride is a multiple of 4
    const bool aligned = (reinterpret_cast<uintptr_t>(scores) & 15) == 0 && s_ld % 4 == 0;
    if (aligned)
      hipLaunchKernelGGL(topk_hist_kernel<true>, dim3(C, rows), dim3(kHistThreads), 0, st, scores,
                         s_ld, n, k, C, h);
    else
      hipLaunchKernelGGL(topk_hist_kernel<false>, dim3(C, rows), dim3(kHistThreads), 0, st, scores,
                         s_ld, n, k, C, h);
    spk_status e = check_launch("topk_select/histogram");
    if (e != SPK_OK) return e;
    if (aligned)
      hipLaunchKernelGGL(topk_final_kernel<true>, dim3(rows), dim3(kLargeThreads), 0, st, scores,
                         s_ld, n, k, C, h, idx, idx_ld, count);
    else
      hipLaunchKernelGGL(topk_final_kernel<false>, dim3(rows), dim3(kLargeThreads), 0, st, scores,
                         s_ld, n, k, C, h, idx, idx_ld, count);
  }
  return check_launch("topk_select");
}
