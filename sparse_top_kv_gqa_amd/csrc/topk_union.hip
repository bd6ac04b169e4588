// topk_select_union: exact top-k of every score row of a group's S <= 4 selection sets (the
// query heads of a KV head, or the draft tokens verified together), and the group's union of
// the S selections with, per row, the mask of the sets holding it.
//
// "Esparsidade de Contexto no Tempo de Inferência", §2 "Oracle Top-K" (exact top-k tokens) and
// "Implementação de Hardware" (each query head keeps its own tokens); "O Fim do Gargalo de
// Memória ... Adaptive DHiSparse", "Metodologia e Eficiência de Carga" (queries verified
// together share the retrieval of their rows): the union is the group's fetch list, read once.
//
// Order keys and ties as in topk_select: the k largest scores of a row, ties to the lowest
// index, indices ascending.  The union is ascending, each entry with a mask bit per set.
//
// Pipeline for wide rows, every pass spread over the whole chip:
//  (0) union_hist_kernel: the histogram of the top 12 key bits of every row, per chunk of the
//      row (stored whole, so nothing is cleared or added atomically);
//  (1) union_bin_kernel, one workgroup per row: sums the row's chunk histograms; the bin b* of
//      the k-th largest key and the number of keys above it;
//  (2) union_gather_kernel, a wave per contiguous token segment of a group: one read of the
//      S score rows; every token with a key above b* in some set, or in bin b* of some set, is
//      appended, in token order, to the segment's candidate list with an 8-bit mask (4 bits
//      "above", 4 bits "in b*"); every set's in-b* candidates are also appended, with their
//      keys, to a short list of the segment and set;
//  (3) union_thr_kernel, one workgroup per row: its set's short lists are loaded at once (one
//      prefix over the segments' counts places every entry), a radix search over their low 20
//      key bits finds the exact threshold and, for ties, the last tied candidate taken (lowest
//      indices first), and a "taken" bit is or-ed into every taken candidate's entry (a row
//      whose lists overflow falls back to a full radix select over its scores);
//  (4) union_write_kernel, one workgroup per group: a prefix over the segments' counts makes the
//      group's candidates one array, every wave owns a contiguous run of it; the final mask of a
//      candidate is its above bits plus its taken bits; two sweeps (counts, then ballot-ranked
//      stores) write the union list, its masks and count, and every set's ascending index list
//      and count.
//
// A candidate entry is (token offset in its segment) << 8 | mask, with the taken bits at
// 18..21 (segments hold at most 1024 tokens).
#include "select_common.h"

namespace spk {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves4 = kThreads / kWave;
constexpr int kWriteThreads = 1024;
constexpr int kWriteWaves = kWriteThreads / kWave;
constexpr int kMaxSets = 4;
constexpr int kThrCap = 4096;     // in-b* candidates of a row held in LDS by union_thr_kernel
constexpr int kListCap = 128;     // in-b* entries kept per (segment, set) list
constexpr int kGatherU = 8;       // 64-token sub-rows in flight per wave in union_gather_kernel
constexpr int kWriteU = 16;       // candidates per lane in flight in union_write_kernel
constexpr int kTakenShift = 18;   // taken bits of a candidate entry (above the 10-bit offset)
constexpr int kMaxSegLen = 1024;
constexpr int kMaxSegs = 4096;    // segments per group held in LDS prefixes (n <= 2^22)

struct Shape {
  int B, T, Hq, Hkv, G, S, per_head;
};

// Score row of set s of group g: (b, t, head) rows for per-head sets, (b, t, kvh) rows for
// per-token sets.
__host__ __device__ inline int64_t set_row(const Shape& u, int g, int s) {
  const int b = g / u.Hkv, kvh = g % u.Hkv;
  if (u.per_head) {
    const int t = s / u.G, j = s % u.G;
    return (int64_t)(b * u.T + t) * u.Hq + kvh * u.G + j;
  }
  return (int64_t)(b * u.T + s) * u.Hkv + kvh;
}

// Chunks per row of the histogram pass: about four workgroups per CU over the launch, chunks of
// at least 2048 scores.
int hist_chunks(int64_t rows, int n) {
  int64_t c = ceil_div(4LL * num_cus(), rows > 0 ? rows : 1);
  const int64_t most = ceil_div(n > 0 ? n : 1, 2048);
  if (c > most) c = most;
  return (int)(c < 1 ? 1 : c);
}

struct Layout {
  int nseg = 0, seg_len = 0, parts = 0, hist_chunks = 1;
  size_t off_info = 0, off_thr = 0, off_cand = 0, off_ccnt = 0, off_ibl = 0, off_ibc = 0,
         off_hist = 0, bytes = 0;
};

Layout make_layout(int groups, int S, int n) {
  Layout l;
  int seg = kMaxSegLen;
  const int64_t want = 2LL * num_cus();
  while (seg > 256 && (int64_t)groups * ceil_div(n, 4 * seg) < want) seg /= 2;
  l.seg_len = seg;
  l.parts = (int)ceil_div(n > 0 ? n : 1, 4 * seg);
  l.nseg = 4 * l.parts;
  size_t off = 0;
  auto take = [&](size_t b) {
    const size_t o = off;
    off = align_up(off + b, 256);
    return o;
  };
  const int64_t rows = (int64_t)groups * S;
  const int64_t slots = (int64_t)groups * l.nseg * seg;
  l.off_info = take((size_t)rows * 16);
  l.off_thr = take((size_t)rows * 16);
  l.off_cand = take((size_t)slots * 4);
  l.off_ccnt = take((size_t)groups * l.nseg * 4);
  l.off_ibl = take((size_t)groups * l.nseg * kMaxSets * kListCap * 8);
  l.off_ibc = take((size_t)groups * l.nseg * kMaxSets * 4);
  l.hist_chunks = hist_chunks(rows, n);
  l.off_hist = take((size_t)rows * l.hist_chunks * kHistBins * 4);
  l.bytes = off;
  return l;
}

__device__ __forceinline__ int kth_set_bit(uint64_t u, int r) {  // r < popcount(u), 0-based
  for (int i = 0; i < r; ++i) u &= u - 1;
  return (int)__builtin_ctzll(u);
}

// ---------------------------------------------------------------- (0) histogram of the scores

// Histogram of chunk blockIdx.x of score row blockIdx.y, stored whole (no atomics, nothing to
// clear beforehand) at ghist[(row * C + chunk) * kHistBins].
__global__ __launch_bounds__(kThreads) void union_hist_kernel(const float* __restrict__ scores,
                                                              int64_t s_ld, int n, int chunk,
                                                              uint32_t* __restrict__ ghist) {
  __shared__ __align__(16) uint32_t hist[kHistBins];
  const int row = blockIdx.y;
  const int beg = blockIdx.x * chunk, end = min(n, beg + chunk);
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) hist[i] = 0u;
  __syncthreads();
  const float* x = scores + (int64_t)row * s_ld;
  constexpr int U = 8;
  for (int i0 = beg; i0 < end; i0 += kThreads * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = x[min(i0 + u * kThreads + (int)threadIdx.x, end - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i0 + u * kThreads + (int)threadIdx.x < end)
        atomicAdd(&hist[order_key(v[u]) >> kHistShift], 1u);
  }
  __syncthreads();
  uint32_t* gh = ghist + ((int64_t)row * gridDim.x + blockIdx.x) * kHistBins;
  for (int i = threadIdx.x * 4; i < kHistBins; i += kThreads * 4)
    *reinterpret_cast<uint4*>(gh + i) = *reinterpret_cast<const uint4*>(hist + i);
}

// ---------------------------------------------------------------- (1) bin of the k-th key

// info[row] = (b*, keys above b*, rank of the k-th key inside b* (1-based), kk); b* = kHistBins
// when nothing is selected.
// The row's histogram is the sum of its C chunk histograms (C = 1: a whole-row histogram).
__global__ __launch_bounds__(kThreads) void union_bin_kernel(const uint32_t* __restrict__ ghist,
                                                             int C, int n, int k,
                                                             int4* __restrict__ info) {
  __shared__ int red[kWaves4 + 1];
  const int row = blockIdx.x;
  const int kk = min(k, n);
  if (kk <= 0) {
    if (threadIdx.x == 0) info[row] = make_int4(kHistBins, 0, 0, 0);
    return;
  }
  // thread t holds bins [b0, b0 + 16), b0 = kHistBins - 16 (t + 1): thread 0 the largest keys
  constexpr int BPT = kHistBins / kThreads;
  const int b0 = kHistBins - BPT * ((int)threadIdx.x + 1);
  uint32_t c[BPT];
#pragma unroll
  for (int j = 0; j < BPT; ++j) c[j] = 0u;
  for (int ch0 = 0; ch0 < C; ch0 += 4) {
    uint4 v[4][BPT / 4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const uint4* h4 = reinterpret_cast<const uint4*>(
          ghist + ((int64_t)row * C + min(ch0 + cc, C - 1)) * kHistBins + b0);
#pragma unroll
      for (int j = 0; j < BPT / 4; ++j) v[cc][j] = h4[j];
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      if (ch0 + cc >= C) break;
#pragma unroll
      for (int j = 0; j < BPT / 4; ++j) {
        c[4 * j] += v[cc][j].x;
        c[4 * j + 1] += v[cc][j].y;
        c[4 * j + 2] += v[cc][j].z;
        c[4 * j + 3] += v[cc][j].w;
      }
    }
  }
  int sum = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) sum += (int)c[j];
  int total;
  const int excl = block_excl_scan(sum, red, &total);
  if (excl < kk && kk <= excl + sum) {
    int acc = excl;
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      if (acc + (int)c[j] >= kk) {
        info[row] = make_int4(b0 + j, acc, kk - acc, kk);
        break;
      }
      acc += (int)c[j];
    }
  }
}

// ---------------------------------------------------------------- (2) candidates per segment

__global__ __launch_bounds__(kThreads) void union_gather_kernel(
    const float* __restrict__ scores, int64_t s_ld, Shape u, int n, const int4* __restrict__ info,
    int nseg, int seg_len, uint32_t* __restrict__ cand, int32_t* __restrict__ ccnt,
    uint2* __restrict__ ibl, int32_t* __restrict__ ibc) {
  const int g = blockIdx.y;
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  const int seg = blockIdx.x * kWaves4 + wid;
  if (seg >= nseg) return;
  const int beg = min(n, seg * seg_len), end = min(n, beg + seg_len);
  uint32_t bst[kMaxSets];
  const float* xs[kMaxSets];
#pragma unroll
  for (int s = 0; s < kMaxSets; ++s) {
    const int sr = s < u.S ? s : 0;
    const int64_t row = set_row(u, g, sr);
    bst[s] = s < u.S ? (uint32_t)info[row].x : 0xFFFFFFFFu;
    xs[s] = scores + row * s_ld;
  }
  const int64_t gs = (int64_t)g * nseg + seg;
  uint32_t* out = cand + gs * seg_len;
  uint2* lists = ibl + gs * kMaxSets * kListCap;
  const uint64_t lt = (1ull << lane) - 1ull;
  int run = 0, runs[kMaxSets] = {0, 0, 0, 0};
  for (int t0 = beg; t0 < end; t0 += kWave * kGatherU) {
    float v[kGatherU][kMaxSets];
#pragma unroll
    for (int q = 0; q < kGatherU; ++q)
#pragma unroll
      for (int s = 0; s < kMaxSets; ++s) v[q][s] = xs[s][min(t0 + q * kWave + lane, end - 1)];
#pragma unroll
    for (int q = 0; q < kGatherU; ++q) {
      const int t = t0 + q * kWave + lane;
      const bool live = t < end;
      uint32_t m = 0, key[kMaxSets];
#pragma unroll
      for (int s = 0; s < kMaxSets; ++s) {
        key[s] = order_key(v[q][s]);
        const uint32_t bin = key[s] >> kHistShift;
        m |= (uint32_t)(live && bin > bst[s]) << s;
        m |= (uint32_t)(live && bin == bst[s]) << (4 + s);
      }
      const uint64_t bal = __ballot(m != 0);
      const int p = run + __popcll(bal & lt);
      if (m) out[p] = ((uint32_t)(t - beg) << 8) | m;
      run += __popcll(bal);
      if (__ballot(m >> 4)) {  // some lane holds an in-b* key (a few per cent of the tokens)
#pragma unroll
        for (int s = 0; s < kMaxSets; ++s) {
          const bool ib = (m >> (4 + s)) & 1u;
          const uint64_t bs = __ballot(ib);
          const int ps = runs[s] + __popcll(bs & lt);
          if (ib && ps < kListCap)
            lists[s * kListCap + ps] = make_uint2((uint32_t)(seg * seg_len + p), key[s]);
          runs[s] += __popcll(bs);
        }
      }
    }
  }
  if (lane == 0) ccnt[gs] = run;
  if (lane < kMaxSets) ibc[gs * kMaxSets + lane] = runs[0] * (lane == 0) + runs[1] * (lane == 1) +
                                                   runs[2] * (lane == 2) + runs[3] * (lane == 3);
}

// ---------------------------------------------------------------- (3) exact threshold per row

// Exclusive prefix of the per-segment counts cnt[i * stride] (i < nseg) into pre[0..nseg] (LDS),
// by the whole workgroup; returns the total.  `red` holds NT/64 + 1 ints of LDS.
template <int NT>
__device__ int segment_prefix(const int32_t* cnt, int64_t stride, int nseg, int cap, int* pre,
                              int* red, bool* over) {
  int carry = 0;
  bool ov = false;
  for (int i0 = 0; i0 < nseg; i0 += NT) {
    const int i = i0 + (int)threadIdx.x;
    const int c = i < nseg ? cnt[(int64_t)i * stride] : 0;
    ov = ov || c > cap;
    int tot;
    const int ex = block_excl_scan(min(c, cap), red, &tot);
    if (i < nseg) pre[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) pre[nseg] = carry;
  *over = __syncthreads_or(ov);
  return carry;
}

// Segment holding entry e of the concatenation (pre ascending, pre[0] = 0, pre[nseg] = total,
// e < total): the largest i with pre[i] <= e, by a fixed-depth descent with no branches, so the
// lookups of several entries overlap.
__device__ __forceinline__ int segment_of(const int* pre, int nseg, int e) {
  int lo = 0;
#pragma unroll
  for (int step = kMaxSegs / 2; step >= 1; step >>= 1) {
    const int mid = lo + step;
    lo = pre[min(mid, nseg)] <= e ? mid : lo;
  }
  return lo;
}


// thr[row] = (threshold key, position of the last tied candidate taken, whole, 0); every taken
// in-b* candidate of the row's set gets its taken bit in its entry.
__global__ __launch_bounds__(kThreads) void union_thr_kernel(
    const float* __restrict__ scores, int64_t s_ld, Shape u, int n,
    const int4* __restrict__ info, int nseg, int seg_len, uint32_t* __restrict__ cand,
    const int32_t* __restrict__ ccnt, const uint2* __restrict__ ibl,
    const int32_t* __restrict__ ibc, int4* __restrict__ thr_out) {
  __shared__ uint32_t lkey[kThrCap];
  __shared__ int32_t lpos[kThrCap];
  __shared__ int pre[kMaxSegs + 1];
  __shared__ __align__(16) uint32_t hist[4 * 256];
  __shared__ int red[kWaves4 + 1], weq[kWaves4], sh[8];
  const int s = blockIdx.x, g = blockIdx.y;
  const int lane = lane_id(), wid = threadIdx.x / kWave, tid = threadIdx.x;
  const int64_t row = set_row(u, g, s);
  const int4 inf = info[row];
  const int bstar = inf.x, kin = inf.z, kk = inf.w;
  if (kk <= 0) {
    if (tid == 0) thr_out[row] = make_int4(0, -1, 0, 0);
    return;
  }
  const float* x = scores + row * s_ld;
  const uint32_t sbit = 1u << (4 + s);
  const uint32_t tbit = 1u << (kTakenShift + s);
  const int64_t gbase = (int64_t)g * nseg;
  uint32_t* gcand = cand + gbase * seg_len;
  for (int i = tid; i < 4 * 256; i += kThreads) hist[i] = 0u;
  if (tid == 0) {
    sh[1] = -1;
    sh[2] = -1;
  }
  bool over;
  const int total = segment_prefix<kThreads>(ibc + gbase * kMaxSets + s, kMaxSets, nseg, kListCap,
                                             pre, red, &over);
  over = over || total > kThrCap || total < kin;

  if (!over) {
    // ---- this set's in-b* candidates, in token order, into LDS (all loads of a batch at once)
    const uint2* lists = ibl + gbase * kMaxSets * kListCap + s * kListCap;
    constexpr int U = 8;
    for (int e0 = 0; e0 < total; e0 += kThreads * U) {
      uint2 ev[U];
      int ee[U];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int e = min(e0 + q * kThreads + tid, total - 1);
        const int sg = segment_of(pre, nseg, e);
        ee[q] = e;
        ev[q] = lists[(int64_t)sg * kMaxSets * kListCap + (e - pre[sg])];
      }
#pragma unroll
      for (int q = 0; q < U; ++q) {
        if (e0 + q * kThreads + tid < total) {
          lpos[ee[q]] = (int)ev[q].x;
          lkey[ee[q]] = ev[q].y;
        }
      }
    }
    __syncthreads();
    uint32_t tthr;
    int need;
    bool whole;
    radix_threshold(
        [&](auto visit) {
          for (int j = tid; j < total; j += kThreads) visit(lkey[j] << kHistBits);
        },
        kin, hist, &tthr, &need, &whole);
    const uint32_t t_key = ((uint32_t)bstar << kHistShift) | (tthr >> kHistBits);
    int cut = 0x7FFFFFFF;
    if (!whole) {
      // the need-th tie in token order: wave w counts over its contiguous part of the entries
      const int per = ((total + kWaves4 - 1) / kWaves4 + kWave - 1) / kWave * kWave;
      const int lo = min(total, wid * per), hi = min(total, lo + per);
      int e = 0;
      for (int j0 = lo; j0 < hi; j0 += kWave) {
        const int j = j0 + lane;
        e += __popcll(__ballot(j < hi && lkey[j] == t_key));
      }
      if (lane == 0) weq[wid] = e;
      __syncthreads();
      int pr = 0;
      for (int w = 0; w < wid; ++w) pr += weq[w];
      if (pr < need && need <= pr + e) {
        int rem = need - pr;  // 1-based rank inside this wave's ties
        for (int j0 = lo; j0 < hi; j0 += kWave) {
          const int j = j0 + lane;
          const uint64_t bal = __ballot(j < hi && lkey[j] == t_key);
          const int c = __popcll(bal);
          if (rem <= c) {
            if (lane == 0) sh[1] = j0 + kth_set_bit(bal, rem - 1);
            break;
          }
          rem -= c;
        }
      }
      __syncthreads();
      cut = sh[1];
    }
    for (int j = tid; j < total; j += kThreads) {
      const uint32_t kv = lkey[j];
      if (kv > t_key || (kv == t_key && (whole || j <= cut))) atomicOr(&gcand[lpos[j]], tbit);
    }
    if (tid == 0) thr_out[row] = make_int4((int)t_key, cut, whole ? 1 : 0, 0);
    return;
  }

  // ---- fallback (lists overflowed): radix select over the whole row, the cut among the ties
  // by a count in token order, then the taken bit of every in-b* candidate of the set
  {
    uint32_t t_key;
    int need;
    radix_select<kThreads>(
        [&](auto&& visit) {
          for (int i = tid; i < n; i += kThreads) visit(order_key(x[i]));
        },
        kk, hist, sh, &t_key, &need);
    const int seg_r = ((n + kWaves4 - 1) / kWaves4 + kWave - 1) / kWave * kWave;
    const int lo = min(n, wid * seg_r), hi = min(n, lo + seg_r);
    int e = 0;
    for (int i0 = lo; i0 < hi; i0 += kWave) {
      const int i = i0 + lane;
      e += __popcll(__ballot(i < hi && order_key(x[min(i, n - 1)]) == t_key));
    }
    if (lane == 0) weq[wid] = e;
    __syncthreads();
    int pr = 0;
    for (int w = 0; w < wid; ++w) pr += weq[w];
    if (pr < need && need <= pr + e) {
      int rem = need - pr;
      for (int i0 = lo; i0 < hi; i0 += kWave) {
        const int i = i0 + lane;
        const uint64_t bal = __ballot(i < hi && order_key(x[min(i, n - 1)]) == t_key);
        const int c = __popcll(bal);
        if (rem <= c) {
          if (lane == 0) sh[2] = i0 + kth_set_bit(bal, rem - 1);
          break;
        }
        rem -= c;
      }
    }
    __syncthreads();
    const int cut = sh[2];
    for (int sg = wid; sg < nseg; sg += kWaves4) {
      const int cnt = ccnt[gbase + sg];
      for (int i = lane; i < cnt; i += kWave) {
        const uint32_t ev = gcand[(int64_t)sg * seg_len + i];
        if (!(ev & sbit)) continue;
        const int tok = sg * seg_len + (int)((ev >> 8) & (kMaxSegLen - 1));
        const uint32_t kv = order_key(x[tok]);
        if (kv > t_key || (kv == t_key && tok <= cut))
          atomicOr(&gcand[(int64_t)sg * seg_len + i], tbit);
      }
    }
    if (tid == 0) thr_out[row] = make_int4((int)t_key, cut, 0, 0);
  }
}

// ---------------------------------------------------------------- (4) union and index lists

__device__ __forceinline__ uint32_t final_mask(uint32_t e) {
  return (e & 15u) | ((e >> kTakenShift) & 15u);
}

// Workgroup (o, g): o = 0 writes group g's union list, its masks and count; o = 1 + s writes
// set s's index list and count (one output per workgroup, so each entry costs one ballot).  Wave
// w owns the segments [w * nseg / 16, (w + 1) * nseg / 16), 64 at a time: lane l holds the count
// of segment l of the current 64; for a batch of kWave * kWriteU entries the wave first writes,
// into its own LDS map, every entry's address base (segment start minus the segment's first
// entry number), so each lane finds an entry's address with one LDS read; every entry's load is
// issued before the first is used.
__global__ __launch_bounds__(kWriteThreads) void union_write_kernel(
    Shape u, int nseg, int seg_len, const uint32_t* __restrict__ cand,
    const int32_t* __restrict__ ccnt, int32_t* __restrict__ idx, int64_t idx_ld,
    int32_t* __restrict__ count, int32_t* __restrict__ ulist, uint32_t* __restrict__ umask,
    int32_t* __restrict__ ucount, int64_t u_ld) {
  constexpr int kBatch = kWave * kWriteU;
  __shared__ int amap[kWriteWaves][kBatch];
  __shared__ int wc[kWriteWaves];
  const int o = blockIdx.x, g = blockIdx.y;
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  const uint64_t lt = (1ull << lane) - 1ull;
  const int64_t gbase = (int64_t)g * nseg;
  const uint32_t* gcand = cand + gbase * seg_len;
  const int sg_lo = (int)(((int64_t)wid * nseg) / kWriteWaves);
  const int sg_hi = (int)(((int64_t)(wid + 1) * nseg) / kWriteWaves);
  // the output bit this workgroup tracks: any set (union) or set o - 1
  const uint32_t want = o == 0 ? 15u : 1u << (o - 1);
  int* map = amap[wid];

  // body(f[], tok[]) for each batch of this wave's entries, in order (f = 0 past the end)
  auto for_batches = [&](auto&& body) {
    for (int c0 = sg_lo; c0 < sg_hi; c0 += kWave) {
      const int nsw = min(kWave, sg_hi - c0);
      const int c = lane < nsw ? ccnt[gbase + c0 + lane] : 0;
      const int incl = wave_incl_scan(c);
      const int excl = incl - c;
      const int tot = __builtin_amdgcn_readlane(incl, kWave - 1);
      for (int e0 = 0; e0 < tot; e0 += kBatch) {
        for (int j = 0; j < nsw; ++j) {
          const int sj = __builtin_amdgcn_readlane(excl, j), cj = __builtin_amdgcn_readlane(c, j);
          const int a = max(sj, e0), z = min(sj + cj, e0 + kBatch);
          const int base = (c0 + j) * seg_len - sj;
          for (int x = a + lane; x < z; x += kWave) map[x - e0] = base;
        }
        uint32_t e[kWriteU];
        int addr[kWriteU];
#pragma unroll
        for (int q = 0; q < kWriteU; ++q) {
          const int ei = min(e0 + q * kWave + lane, tot - 1);
          addr[q] = map[ei - e0] + ei;
          e[q] = gcand[addr[q]];
        }
        uint32_t f[kWriteU];
        int tok[kWriteU];
#pragma unroll
        for (int q = 0; q < kWriteU; ++q) {
          f[q] = e0 + q * kWave + lane < tot ? final_mask(e[q]) & want : 0u;
          tok[q] = (addr[q] & ~(seg_len - 1)) + (int)((e[q] >> 8) & (kMaxSegLen - 1));
        }
        body(f, tok);
      }
    }
  };

  // sweep 1: this wave's count (per lane, summed over the wave once)
  int cw = 0;
  for_batches([&](const uint32_t (&f)[kWriteU], const int (&tok)[kWriteU]) {
#pragma unroll
    for (int q = 0; q < kWriteU; ++q) cw += f[q] != 0;
  });
  cw = __builtin_amdgcn_readlane(wave_incl_scan(cw), kWave - 1);
  if (lane == 0) wc[wid] = cw;
  __syncthreads();
  int run = 0, total = 0;
  for (int w = 0; w < kWriteWaves; ++w) {
    run += w < wid ? wc[w] : 0;
    total += wc[w];
  }
  int32_t* out;
  int64_t cap;
  if (o == 0) {
    if (threadIdx.x == 0) ucount[g] = (int)min((int64_t)total, u_ld);
    out = ulist + (int64_t)g * u_ld;
    cap = u_ld;
  } else {
    const int64_t row = set_row(u, g, o - 1);
    if (threadIdx.x == 0) count[row] = (int)min((int64_t)total, idx_ld);
    out = idx + row * idx_ld;
    cap = idx_ld;
  }
  uint32_t* om = umask + (int64_t)g * u_ld;

  // sweep 2: the same entries, each stored at its ballot rank
  for_batches([&](const uint32_t (&f)[kWriteU], const int (&tok)[kWriteU]) {
#pragma unroll
    for (int q = 0; q < kWriteU; ++q) {
      const uint64_t bal = __ballot(f[q] != 0);
      const int p = run + __popcll(bal & lt);
      if (f[q] && p < cap) {
        out[p] = tok[q];
        if (o == 0) om[p] = f[q];
      }
      run += __popcll(bal);
    }
  });
}

spk_status check_union_args(int B, int T, int Hq, int Hkv, spk_sel_scope scope, int n, int k,
                            int* S) {
  SPK_REQUIRE(B >= 0 && T > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0, SPK_EINVAL,
              "topk_select_union: bad shape B=%d T=%d Hq=%d Hkv=%d", B, T, Hq, Hkv);
  SPK_REQUIRE(scope == SPK_SEL_PER_Q_HEAD || scope == SPK_SEL_PER_KV_HEAD, SPK_EINVAL,
              "topk_select_union: scope must be per_q_head or per_kv_head");
  SPK_REQUIRE(n >= 0 && n <= kMaxSegs * kMaxSegLen && k >= 0, SPK_EINVAL,
              "topk_select_union: n=%d (0 <= n <= 2^22) or k=%d < 0", n, k);
  *S = scope == SPK_SEL_PER_Q_HEAD ? T * (Hq / Hkv) : T;
  SPK_REQUIRE(*S <= kMaxSets, SPK_EUNSUPPORTED,
              "topk_select_union: %d selection sets per KV head (max %d)", *S, kMaxSets);
  return SPK_OK;
}

}  // namespace
}  // namespace spk

extern "C" SPK_API spk_status topk_select_union_workspace_size(int B, int T, int Hq, int Hkv,
                                                               spk_sel_scope scope, int n, int k,
                                                               size_t* bytes) {
  using namespace spk;
  SPK_REQUIRE(bytes, SPK_EINVAL, "topk_select_union_workspace_size: null bytes");
  int S = 0;
  const spk_status st = check_union_args(B, T, Hq, Hkv, scope, n, k, &S);
  if (st != SPK_OK) return st;
  *bytes = make_layout(B * Hkv, S, n).bytes;
  clear_error();
  return SPK_OK;
}

extern "C" SPK_API spk_status topk_select_union(
    const float* scores, int64_t s_ld, int B, int T, int Hq, int Hkv,
    spk_sel_scope scope, int n, int k, int32_t* idx, int64_t idx_ld, int32_t* count,
    int32_t* u_list, uint32_t* u_mask, int32_t* u_count, int64_t u_ld, void* ws, size_t ws_bytes,
    void* stream) {
  using namespace spk;
  int S = 0;
  spk_status st0 = check_union_args(B, T, Hq, Hkv, scope, n, k, &S);
  if (st0 != SPK_OK) return st0;
  const int kk = k < n ? k : n;
  const int groups = B * Hkv;
  SPK_REQUIRE(B == 0 || (scores && idx && count && u_list && u_mask && u_count), SPK_EINVAL,
              "topk_select_union: null scores, idx, count or union buffers");
  SPK_REQUIRE(s_ld >= n && idx_ld >= kk, SPK_EINVAL,
              "topk_select_union: s_ld %lld < n %d or idx_ld %lld < min(k, n) %d",
              (long long)s_ld, n, (long long)idx_ld, kk);
  const int64_t ub = (int64_t)S * kk < n ? (int64_t)S * kk : n;
  SPK_REQUIRE(u_ld >= ub, SPK_EINVAL, "topk_select_union: u_ld %lld < min(n, sets * k) %lld",
              (long long)u_ld, (long long)ub);
  const Layout l = make_layout(groups, S, n);
  SPK_REQUIRE(ws_bytes >= l.bytes && (l.bytes == 0 || ws), SPK_EWORKSPACE,
              "topk_select_union: workspace %zu bytes < %zu needed", ws_bytes, l.bytes);
  clear_error();
  if (groups == 0) return SPK_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* w = reinterpret_cast<char*>(ws);
  const Shape u{B, T, Hq, Hkv, Hq / Hkv, S, scope == SPK_SEL_PER_Q_HEAD ? 1 : 0};
  const int rows = groups * S;
  // rows are indexed by blockIdx.y over the (b, t, head) rows in memory order; every row
  // belongs to exactly one (group, set).  With n == 0 nothing is selected and the bin pass
  // reads no histogram.
  uint32_t* hist = reinterpret_cast<uint32_t*>(w + l.off_hist);
  const int hc = l.hist_chunks;
  if (n > 0) {
    const int chunk = (int)ceil_div(n, hc);
    hipLaunchKernelGGL(union_hist_kernel, dim3(hc, rows), dim3(kThreads), 0, st, scores, s_ld, n,
                       chunk, hist);
    spk_status e = check_launch("topk_select_union/histogram");
    if (e != SPK_OK) return e;
  }
  int4* info = reinterpret_cast<int4*>(w + l.off_info);
  int4* thr = reinterpret_cast<int4*>(w + l.off_thr);
  uint32_t* cand = reinterpret_cast<uint32_t*>(w + l.off_cand);
  int32_t* ccnt = reinterpret_cast<int32_t*>(w + l.off_ccnt);
  uint2* ibl = reinterpret_cast<uint2*>(w + l.off_ibl);
  int32_t* ibc = reinterpret_cast<int32_t*>(w + l.off_ibc);
  hipLaunchKernelGGL(union_bin_kernel, dim3(rows), dim3(kThreads), 0, st, hist, hc, n, k, info);
  spk_status e = check_launch("topk_select_union/bin");
  if (e != SPK_OK) return e;
  hipLaunchKernelGGL(union_gather_kernel, dim3(l.parts, groups), dim3(kThreads), 0, st, scores,
                     s_ld, u, n, info, l.nseg, l.seg_len, cand, ccnt, ibl, ibc);
  e = check_launch("topk_select_union/gather");
  if (e != SPK_OK) return e;
  hipLaunchKernelGGL(union_thr_kernel, dim3(S, groups), dim3(kThreads), 0, st, scores, s_ld, u, n,
                     info, l.nseg, l.seg_len, cand, ccnt, ibl, ibc, thr);
  e = check_launch("topk_select_union/threshold");
  if (e != SPK_OK) return e;
  hipLaunchKernelGGL(union_write_kernel, dim3(1 + S, groups), dim3(kWriteThreads), 0, st, u, l.nseg,
                     l.seg_len, cand, ccnt, idx, idx_ld, count, u_list, u_mask, u_count, u_ld);
  return check_launch("topk_select_union/write");
}
