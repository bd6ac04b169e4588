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
//  (0) union_range_kernel, two workgroups per row: a key range [lo, hi] expected to hold the
//      row's k-th largest key, from a sample of the row (16-token pieces at 256 evenly spaced
//      offsets, the whole row when it has at most 4096 keys): hi is the sample's key of rank
//      r - delta, lo the key of rank r + delta, r = k * samples / n its expected rank and delta
//      four standard deviations of a sampled count plus two.  Nothing below depends on the
//      range being right: the threshold pass checks it and falls back to exact whole-row work;
//      the range only decides how much work the exact answer takes;
//  (1) union_gather_kernel, a wave per contiguous token segment of a group: one read of the
//      S score rows; every token with a key above hi in some set, or inside [lo, hi] in some
//      set, is appended, in token order, to the segment's candidate list with an 8-bit mask (4
//      bits "above", 4 bits "in range"); every set's in-range candidates are also appended, with
//      their keys, to a short list of the segment and set, and the keys above hi are counted;
//  (2) union_thr_kernel, one workgroup per row: when fewer than k keys lie above hi and the
//      in-range lists hold the rest (none overflowed), the lists are loaded at once (one prefix
//      over the segments' counts places every entry) and a radix search finds the exact
//      threshold and, for ties, the last tied candidate taken (lowest indices first); a "taken"
//      bit is or-ed into every taken candidate's entry.  Otherwise a radix select over the
//      whole row finds the threshold: if no selected key lies below lo, the taken bits are set
//      on the row's candidates (above or in range) and the row's "above" bits are ignored;
//      else the group is marked for direct selection;
//  (3) union_write_kernel, one workgroup per group and output: a prefix over the segments'
//      counts makes the group's candidates one array, every wave owns a contiguous run of it;
//      the final mask of a candidate is its honoured above bits plus its taken bits; two sweeps
//      (counts, then ballot-ranked stores) write the union list, its masks and count, and every
//      set's ascending index list and count.  A group marked for direct selection instead
//      selects from its score rows with every set's exact threshold (the same two sweeps over
//      the tokens).
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
constexpr int kThrCap = 6144;     // in-range candidates of a row held in LDS by union_thr_kernel
constexpr int kListCap = 128;     // in-range entries kept per (segment, set) list
constexpr int kGatherU = 4;       // 64-token sub-rows in flight per wave in union_gather_kernel
constexpr int kWriteU = 16;       // candidates per lane in flight in union_write_kernel
constexpr int kTakenShift = 18;   // taken bits of a candidate entry (above the 10-bit offset)
constexpr int kMaxSegLen = 1024;
constexpr int kMaxSegs = 4096;    // segments per group held in LDS prefixes (n <= 2^22)
constexpr int kSlotBits = 22;     // candidate slots of a group: nseg * seg_len <= 2^22
constexpr uint32_t kSlotMask = (1u << kSlotBits) - 1u;
constexpr int kPieces = 256;      // sample pieces per row
constexpr int kPieceLen = 16;     // consecutive tokens per piece
constexpr int kSampleMax = kPieces * kPieceLen;
constexpr int kRangeThreads = 256;   // 1024 measured slightly slower
constexpr int kSamplePerThread = kSampleMax / kRangeThreads;
// thr_out[row].w: how the write pass treats the row's set
constexpr int kRowRange = 0;      // threshold found inside the range: above bits and taken bits
constexpr int kRowTakenOnly = 1;  // whole-row threshold inside the range: taken bits only
constexpr int kRowDirect = 2;     // a selected key lies below the range: select from the scores

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

struct Layout {
  int nseg = 0, seg_len = 0, parts = 0;
  size_t off_info = 0, off_thr = 0, off_cand = 0, off_ccnt = 0, off_ibl = 0, off_ibc = 0,
         off_iac = 0, bytes = 0;
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
  l.off_iac = take((size_t)groups * l.nseg * kMaxSets * 4);
  l.bytes = off;
  return l;
}

__device__ __forceinline__ int kth_set_bit(uint64_t u, int r) {  // r < popcount(u), 0-based
  for (int i = 0; i < r; ++i) u &= u - 1;
  return (int)__builtin_ctzll(u);
}

// ---------------------------------------------------------------- (0) key range per row

// Token of sample i (< min(n, kSampleMax)) of a row of n: the row itself up to kSampleMax keys,
// else token i % kPieceLen of piece i / kPieceLen, piece j starting at floor(j * n / kPieces)
// (pieces never overlap: n / kPieces >= kPieceLen).
__device__ __forceinline__ int sample_token(int i, int n) {
  if (n <= kSampleMax) return i;
  return (int)(((int64_t)(i / kPieceLen) * n) / kPieces) + i % kPieceLen;
}

// Workgroup (0, row) writes info[row].y = hi, workgroup (1, row) info[row].x = lo and
// info[row].z = min(k, n).  Every row key above hi is meant to be kept, the row's k-th largest
// key is meant to lie in [lo, hi]; hi = 0xFFFFFFFF (no order key is larger) when the sample
// puts fewer than one key above the range, lo = 0 when it puts the range's end past the
// sample.  With the whole row as the sample the range is exact: hi and lo are the k-th
// largest key.  The sample's key of rank q: a 4096-bin histogram of the top 12 key bits names
// its bin, a radix search over the low 20 bits of that bin's keys the key itself.  Both ends
// are keys of sample scores (or the two sentinels).
__global__ __launch_bounds__(kRangeThreads) void union_range_kernel(const float* __restrict__ scores,
                                                               int64_t s_ld, int n, int k,
                                                               int4* __restrict__ info) {
  __shared__ __align__(16) uint32_t bins[kHistBins];
  __shared__ __align__(16) uint32_t hist[4 * 256];
  __shared__ int red[kRangeThreads / kWave + 1], sh[2];
  __shared__ uint32_t kmin;
  const int row = blockIdx.y, upper = blockIdx.x == 0, tid = threadIdx.x;
  int* out = reinterpret_cast<int*>(info + row);
  const int kk = min(k, n);
  if (kk <= 0) {
    if (tid == 0) {
      if (upper) out[1] = -1;
      else {
        out[0] = -1;
        out[2] = 0;
      }
    }
    return;
  }
  const int m = min(n, kSampleMax);
  int q = kk;
  if (n > kSampleMax) {
    const float r = (float)kk * (float)m / (float)n;
    const float delta = 4.f * sqrtf(r) + 2.f;
    q = upper ? (int)floorf(r - delta) : (int)ceilf(r + delta);
  }
  if (upper && q < 1) {
    if (tid == 0) out[1] = -1;
    return;
  }
  if (!upper && q > m) {
    if (tid == 0) {
      out[0] = 0;
      out[2] = kk;
    }
    return;
  }
  const float* x = scores + (int64_t)row * s_ld;
  float v[kSamplePerThread];
#pragma unroll
  for (int u = 0; u < kSamplePerThread; ++u) {
    const int i = u * kRangeThreads + tid;
    v[u] = x[sample_token(min(i, m - 1), n)];
  }
  for (int i = tid * 4; i < kHistBins; i += kRangeThreads * 4)
    *reinterpret_cast<uint4*>(bins + i) = make_uint4(0u, 0u, 0u, 0u);
  for (int i = tid; i < 4 * 256; i += kRangeThreads) hist[i] = 0u;
  if (tid == 0) kmin = 0xFFFFFFFFu;
  uint32_t key[kSamplePerThread];
#pragma unroll
  for (int u = 0; u < kSamplePerThread; ++u) key[u] = order_key(v[u]);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kSamplePerThread; ++u)
    if (u * kRangeThreads + tid < m) atomicAdd(&bins[key[u] >> kHistShift], 1u);
  __syncthreads();
  // thread t holds bins [b0, b0 + 16), b0 = kHistBins - 16 (t + 1): thread 0 the largest keys
  constexpr int BPT = kHistBins / kRangeThreads;
  const int b0 = kHistBins - BPT * (tid + 1);
  uint32_t c[BPT];
#pragma unroll
  for (int j = 0; j < BPT; j += 4) {
    const uint4 w = *reinterpret_cast<const uint4*>(bins + b0 + j);
    c[j] = w.x;
    c[j + 1] = w.y;
    c[j + 2] = w.z;
    c[j + 3] = w.w;
  }
  int sum = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) sum += (int)c[j];
  int total;
  const int excl = block_excl_scan(sum, red, &total);
  if (excl < q && q <= excl + sum) {
    int acc = excl;
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      if (acc + (int)c[j] >= q) {
        sh[0] = b0 + j;
        sh[1] = q - acc;  // rank inside the bin, 1-based
        break;
      }
      acc += (int)c[j];
    }
  }
  __syncthreads();
  const uint32_t bq = (uint32_t)sh[0];
  const int qin = sh[1];
  uint32_t low;
  int need;
  bool whole;
  radix_threshold(
      [&](auto visit) {
#pragma unroll
        for (int u = 0; u < kSamplePerThread; ++u)
          if (u * kRangeThreads + tid < m && (key[u] >> kHistShift) == bq) visit(key[u] << kHistBits);
      },
      qin, hist, &low, &need, &whole);
  uint32_t thr = (bq << kHistShift) | (low >> kHistBits);
  if (whole) {
    // thr is a prefix that exactly the q largest keys reach, not necessarily a key (the gather
    // compares scores with the float of each end): both ends become the smallest of those keys,
    // which the same q sample keys reach
    uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
    for (int u = 0; u < kSamplePerThread; ++u)
      if (u * kRangeThreads + tid < m && key[u] >= thr) mn = min(mn, key[u]);
    atomicMin(&kmin, mn);
    __syncthreads();
    thr = kmin;
  }
  if (tid == 0) {
    if (upper) out[1] = (int)thr;
    else {
      out[0] = (int)thr;
      out[2] = kk;
    }
  }
}

// ---------------------------------------------------------------- (1) candidates per segment

// Number of lanes below this one whose bit is set in the wave mask m.
__device__ __forceinline__ int rank_in_wave(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Float of an order key (the inverse of order_key on the keys it produces; key 0, the key of
// NaN, and the sentinel 0xFFFFFFFF come out as NaN, which compares false).
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// A wave per segment; kGatherU rows of 64 tokens of every set are loaded (one element per lane,
// clamped in bounds) before the first is classified.  A score is compared as a float with the
// range's ends (key order and float order agree on every non-NaN score, and -0 == +0 in both);
// a NaN score (key 0) is in range only when lo is 0.  One end differs: hi = 0 (NaN's key, from a
// sample that is mostly NaN) compares false, so every token is in range and none above (lo is
// then 0 too) — still a valid split for the threshold pass, which lists or re-reads them all.  The classes are wave ballots, so counting
// and compaction run on scalar masks; order keys are formed only for in-range list entries.
// Four 64-token rows per batch: per-wave timestamps put the launch's span at 17.7 us with four,
// 19.0 with two or eight, 22.4 with sixteen (the whole segment's loads at once); a whole segment
// loaded with 16-byte loads measured about 3 us slower still.
__global__ __launch_bounds__(kThreads) void union_gather_kernel(
    const float* __restrict__ scores, int64_t s_ld, Shape u, int n, const int4* __restrict__ info,
    int nseg, int seg_len, uint32_t* __restrict__ cand, int32_t* __restrict__ ccnt,
    uint2* __restrict__ ibl, int32_t* __restrict__ ibc, int32_t* __restrict__ iac) {
  const int g = blockIdx.y;
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  const int seg = blockIdx.x * kWaves4 + wid;
  if (seg >= nseg) return;
  const int beg = min(n, seg * seg_len), end = min(n, beg + seg_len);
  float hf[kMaxSets], lf[kMaxSets];
  uint32_t lo_all[kMaxSets];
  const float* xs[kMaxSets];
#pragma unroll
  for (int s = 0; s < kMaxSets; ++s) {
    const int sr = s < u.S ? s : 0;
    const int64_t row = set_row(u, g, sr);
    const int4 inf = info[row];
    const bool on = s < u.S && inf.z > 0;
    hf[s] = on ? key_float((uint32_t)inf.y) : __uint_as_float(0x7FFFFFFFu);
    lf[s] = on ? key_float((uint32_t)inf.x) : __uint_as_float(0x7FFFFFFFu);
    lo_all[s] = on && inf.x == 0 ? 1u : 0u;
    xs[s] = scores + row * s_ld;
  }
  const int64_t gs = (int64_t)g * nseg + seg;
  uint32_t* out = cand + gs * seg_len;
  uint2* lists = ibl + gs * kMaxSets * kListCap;
  int run = 0, runs[kMaxSets] = {0, 0, 0, 0}, nab[kMaxSets] = {0, 0, 0, 0};
  // kGatherU * 64 tokens from t0; FULL: all of them inside the segment (no clamping)
  auto chunk = [&](int t0, auto full) {
    constexpr bool FULL = decltype(full)::value;
    float v[kGatherU][kMaxSets];
#pragma unroll
    for (int q = 0; q < kGatherU; ++q)
#pragma unroll
      for (int s = 0; s < kMaxSets; ++s)
        v[q][s] = FULL ? xs[s][t0 + q * kWave + lane] : xs[s][min(t0 + q * kWave + lane, end - 1)];
#pragma unroll
    for (int q = 0; q < kGatherU; ++q) {
      const int t = t0 + q * kWave + lane;
      const uint64_t live = FULL ? ~0ull : __ballot(t < end);
      uint64_t A[kMaxSets], R[kMaxSets], any = 0ull, anyr = 0ull;
#pragma unroll
      for (int s = 0; s < kMaxSets; ++s) {
        A[s] = __ballot(v[q][s] > hf[s]) & live;
        R[s] = (lo_all[s] ? live : __ballot(v[q][s] >= lf[s]) & live) & ~A[s];
        nab[s] += __popcll(A[s]);
        any |= A[s] | R[s];
        anyr |= R[s];
      }
      const int p = run + rank_in_wave(any);
      if (__builtin_amdgcn_inverse_ballot_w64(any)) {
        uint32_t m = 0u;
#pragma unroll
        for (int s = 0; s < kMaxSets; ++s)
          m |= (__builtin_amdgcn_inverse_ballot_w64(A[s]) ? 1u << s : 0u) |
               (__builtin_amdgcn_inverse_ballot_w64(R[s]) ? 1u << (4 + s) : 0u);
        out[p] = ((uint32_t)(t - beg) << 8) | m;
      }
      run += __popcll(any);
      if (anyr) {  // some lane holds an in-range key (a few per cent of the tokens)
#pragma unroll
        for (int s = 0; s < kMaxSets; ++s) {
          const int ps = runs[s] + rank_in_wave(R[s]);
          if (__builtin_amdgcn_inverse_ballot_w64(R[s]) && ps < kListCap)
            lists[s * kListCap + ps] =
                make_uint2((uint32_t)(seg * seg_len + p) | ((uint32_t)(t - beg) << kSlotBits),
                           order_key(v[q][s]));
          runs[s] += __popcll(R[s]);
        }
      }
    }
  };
  int t0 = beg;
  for (; t0 + kWave * kGatherU <= end; t0 += kWave * kGatherU) chunk(t0, std::true_type{});
  if (t0 < end) chunk(t0, std::false_type{});
  if (lane == 0) ccnt[gs] = run;
  if (lane < kMaxSets) {
    ibc[gs * kMaxSets + lane] = runs[0] * (lane == 0) + runs[1] * (lane == 1) +
                                runs[2] * (lane == 2) + runs[3] * (lane == 3);
    iac[gs * kMaxSets + lane] = nab[0] * (lane == 0) + nab[1] * (lane == 1) +
                                nab[2] * (lane == 2) + nab[3] * (lane == 3);
  }
}

// ---------------------------------------------------------------- (2) exact threshold per row

// Exclusive prefix of the per-segment counts cnt[i * stride] (i < nseg) into pre[0..nseg] (LDS),
// by the whole workgroup; returns the total and, in *extra_sum, the sum of extra[i * stride]
// (loaded beside the counts, its wave totals published under the barrier of the overflow
// vote).  `red` and `xred` hold NT/64 + 1 ints of LDS each.
template <int NT>
__device__ int segment_prefix(const int32_t* cnt, const int32_t* extra, int64_t stride, int nseg,
                              int cap, int* pre, int* red, int* xred, bool* over, int* extra_sum) {
  int carry = 0, xs = 0;
  bool ov = false;
  for (int i0 = 0; i0 < nseg; i0 += NT) {
    const int i = i0 + (int)threadIdx.x;
    const int c = i < nseg ? cnt[(int64_t)i * stride] : 0;
    xs += i < nseg ? extra[(int64_t)i * stride] : 0;
    ov = ov || c > cap;
    int tot;
    const int ex = block_excl_scan(min(c, cap), red, &tot);
    if (i < nseg) pre[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) pre[nseg] = carry;
  const int xw = __builtin_amdgcn_readlane(wave_incl_scan(xs), kWave - 1);
  if (lane_id() == 0) xred[threadIdx.x / kWave] = xw;
  *over = __syncthreads_or(ov);
  int xsum = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) xsum += xred[w];
  *extra_sum = xsum;
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


// thr[row] = (threshold key, token of the last tied key taken, whole, kind): the row keeps every
// key above the threshold key and, when whole is 0, the keys equal to it up to that token
// (whole = 1: every key equal to it); kind is kRowRange, kRowTakenOnly or kRowDirect (see the
// pipeline above).  Every taken in-range candidate of the row's set (kRowTakenOnly: every
// taken candidate) gets its taken bit in its entry.
__global__ __launch_bounds__(kThreads) void union_thr_kernel(
    const float* __restrict__ scores, int64_t s_ld, Shape u, int n,
    const int4* __restrict__ info, int nseg, int seg_len, uint32_t* __restrict__ cand,
    const int32_t* __restrict__ ccnt, const uint2* __restrict__ ibl,
    const int32_t* __restrict__ ibc, const int32_t* __restrict__ iac, int4* __restrict__ thr_out) {
  __shared__ uint32_t lkey[kThrCap];
  __shared__ int32_t lpos[kThrCap];
  __shared__ int pre[kMaxSegs + 1];
  __shared__ __align__(16) uint32_t hist[4 * 256];
  __shared__ int red[kWaves4 + 1], xred[kWaves4 + 1], weq[kWaves4], sh[8];
  __shared__ uint32_t kand, kor;
  const int s = blockIdx.x, g = blockIdx.y;
  const int lane = lane_id(), wid = threadIdx.x / kWave, tid = threadIdx.x;
  const int64_t row = set_row(u, g, s);
  const int4 inf = info[row];
  const uint32_t lo_key = (uint32_t)inf.x;
  const int kk = inf.z;
  if (kk <= 0) {  // no order key reaches 0xFFFFFFFF: nothing is kept
    if (tid == 0) thr_out[row] = make_int4(-1, -1, 0, kRowRange);
    return;
  }
  const float* x = scores + row * s_ld;
  const uint32_t abit = 1u << s, sbit = 1u << (4 + s);
  const uint32_t tbit = 1u << (kTakenShift + s);
  const int64_t gbase = (int64_t)g * nseg;
  uint32_t* gcand = cand + gbase * seg_len;
  for (int i = tid; i < 4 * 256; i += kThreads) hist[i] = 0u;
  if (tid == 0) {
    sh[1] = -1;
    sh[2] = -1;
    kand = 0xFFFFFFFFu;
    kor = 0u;
  }
  // in-range list lengths and keys above the range, over all segments
  bool over;
  int above;
  const int total = segment_prefix<kThreads>(ibc + gbase * kMaxSets + s, iac + gbase * kMaxSets + s,
                                             kMaxSets, nseg, kListCap, pre, red, xred, &over,
                                             &above);
  const int kin = kk - above;  // keys of the top kk that lie in the range
  over = over || total > kThrCap || kin < 1 || kin > total;

  if (!over) {
    // ---- this set's in-range candidates, in token order, into LDS (all loads of a batch at once)
    const uint2* lists = ibl + gbase * kMaxSets * kListCap + s * kListCap;
    constexpr int U = 12;  // 3072 entries per batch: one batch for the usual 2000-3000
    uint32_t a_and = 0xFFFFFFFFu, a_or = 0u;
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
        a_and &= ev[q].y;  // clamped entries repeat a listed key: harmless to the and / or
        a_or |= ev[q].y;
        if (e0 + q * kThreads + tid < total) {
          lpos[ee[q]] = (int)ev[q].x;  // candidate slot | token offset << kSlotBits
          lkey[ee[q]] = ev[q].y;
        }
      }
    }
    // the bits every listed key shares: the radix search starts below them
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      a_and &= (uint32_t)__shfl_xor((int)a_and, o);
      a_or |= (uint32_t)__shfl_xor((int)a_or, o);
    }
    if (lane == 0) {
      atomicAnd(&kand, a_and);
      atomicOr(&kor, a_or);
    }
    __syncthreads();
    const uint32_t diff = kand ^ kor;
    const int shift = diff ? __builtin_clz(diff) : 0;
    const uint32_t common = shift ? kand & (0xFFFFFFFFu << (32 - shift)) : 0u;
    uint32_t t_key;
    int need;
    bool whole;
    radix_threshold(
        [&](auto visit) {
          for (int j = tid; j < total; j += kThreads) visit(lkey[j] << shift);
        },
        kin, hist, &t_key, &need, &whole);
    t_key = common | (t_key >> shift);
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
      if (kv > t_key || (kv == t_key && (whole || j <= cut)))
        atomicOr(&gcand[lpos[j] & kSlotMask], tbit);
    }
    if (tid == 0) {
      // in whole-row terms: "whole" keeps every key >= max(prefix, lo) (no key below lo is in
      // range); otherwise the cut entry's token
      int cut_tok = -1;
      uint32_t tk = t_key;
      if (whole) {
        tk = t_key > lo_key ? t_key : lo_key;
      } else if (cut >= 0) {
        const uint32_t e = (uint32_t)lpos[cut];
        cut_tok = (int)((e & kSlotMask) / seg_len) * seg_len + (int)(e >> kSlotBits);
      }
      thr_out[row] = make_int4((int)tk, cut_tok, whole ? 1 : 0, kRowRange);
    }
    return;
  }

  // ---- fallback (the range missed the k-th key, or lists overflowed): radix select over the
  // whole row, the cut among the ties by a count in token order
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
  if (t_key < lo_key) {
    // some kept key is not a candidate: the write pass selects this group from its scores
    if (tid == 0) thr_out[row] = make_int4((int)t_key, cut, 0, kRowDirect);
    return;
  }
  // every kept key is a candidate (above or in range) of the set: mark the kept ones
  for (int sg = wid; sg < nseg; sg += kWaves4) {
    const int cnt = ccnt[gbase + sg];
    for (int i = lane; i < cnt; i += kWave) {
      const uint32_t ev = gcand[(int64_t)sg * seg_len + i];
      if (!(ev & (abit | sbit))) continue;
      const int tok = sg * seg_len + (int)((ev >> 8) & (kMaxSegLen - 1));
      const uint32_t kv = order_key(x[tok]);
      if (kv > t_key || (kv == t_key && tok <= cut))
        atomicOr(&gcand[(int64_t)sg * seg_len + i], tbit);
    }
  }
  if (tid == 0) thr_out[row] = make_int4((int)t_key, cut, 0, kRowTakenOnly);
}

// ---------------------------------------------------------------- (3) union and index lists

__device__ __forceinline__ uint32_t final_mask(uint32_t e, uint32_t honoured) {
  return (e & honoured) | ((e >> kTakenShift) & 15u);
}

// Workgroup (o, g): o = 0 writes group g's union list, its masks and count; o = 1 + s writes
// set s's index list and count (one output per workgroup, so each entry costs one ballot).  Wave
// w owns the segments [w * nseg / 16, (w + 1) * nseg / 16), 64 at a time: lane l holds the count
// of segment l of the current 64; for a batch of kWave * kWriteU entries the wave first writes,
// into its own LDS map, every entry's address base (segment start minus the segment's first
// entry number), so each lane finds an entry's address with one LDS read; every entry's load is
// issued before the first is used.  A group with a kRowDirect set is selected from its score
// rows instead: wave w owns the tokens [w * per, (w + 1) * per).
__global__ __launch_bounds__(kWriteThreads) void union_write_kernel(
    const float* __restrict__ scores, int64_t s_ld, Shape u, int n,
    const int4* __restrict__ thr, int nseg, int seg_len,
    const uint32_t* __restrict__ cand, const int32_t* __restrict__ ccnt,
    int32_t* __restrict__ idx, int64_t idx_ld, int32_t* __restrict__ count,
    int32_t* __restrict__ ulist, uint32_t* __restrict__ umask, int32_t* __restrict__ ucount,
    int64_t u_ld) {
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
  // the sets' thresholds: whose above bits count, and whether the group is selected directly
  uint32_t honoured = 0u;
  bool direct = false;
  uint32_t tk[kMaxSets];
  int tcut[kMaxSets];
  bool twhole[kMaxSets], ton[kMaxSets];
  const float* xs[kMaxSets];
#pragma unroll
  for (int s = 0; s < kMaxSets; ++s) {
    const int64_t row = set_row(u, g, s < u.S ? s : 0);
    const int4 th = thr[row];
    ton[s] = s < u.S;
    tk[s] = (uint32_t)th.x;
    tcut[s] = th.y;
    twhole[s] = th.z != 0;
    xs[s] = scores + row * s_ld;
    if (s < u.S && th.w == kRowRange) honoured |= 1u << s;
    direct = direct || (s < u.S && th.w == kRowDirect);
  }

  // body(f[], tok[]) for each batch of this wave's entries, in order (f = 0 past the end); the
  // first batch of the first sweep stays in registers (token | mask << kSlotBits) for the second
  uint32_t keep[kWriteU];
  auto for_batches = [&](bool second, auto&& body) {
    if (direct) {
      const int per = ((n + kWriteWaves - 1) / kWriteWaves + kWave - 1) / kWave * kWave;
      const int t_lo = min(n, wid * per), t_hi = min(n, t_lo + per);
      for (int t0 = t_lo; t0 < t_hi; t0 += kBatch) {
        float v[kWriteU][kMaxSets];
#pragma unroll
        for (int q = 0; q < kWriteU; ++q)
#pragma unroll
          for (int s = 0; s < kMaxSets; ++s)
            v[q][s] = xs[s][min(t0 + q * kWave + lane, t_hi - 1)];
        uint32_t f[kWriteU];
        int tok[kWriteU];
#pragma unroll
        for (int q = 0; q < kWriteU; ++q) {
          const int t = t0 + q * kWave + lane;
          uint32_t m = 0u;
#pragma unroll
          for (int s = 0; s < kMaxSets; ++s) {
            const uint32_t key = order_key(v[q][s]);
            const bool kept =
                key > tk[s] || (key == tk[s] && (twhole[s] || t <= tcut[s]));
            m |= (uint32_t)(ton[s] && kept) << s;
          }
          f[q] = t < t_hi ? m & want : 0u;
          tok[q] = t;
        }
        body(f, tok);
      }
      return;
    }
    for (int c0 = sg_lo; c0 < sg_hi; c0 += kWave) {
      const int nsw = min(kWave, sg_hi - c0);
      const int c = lane < nsw ? ccnt[gbase + c0 + lane] : 0;
      const int incl = wave_incl_scan(c);
      const int excl = incl - c;
      const int tot = __builtin_amdgcn_readlane(incl, kWave - 1);
      for (int e0 = 0; e0 < tot; e0 += kBatch) {
        const bool first_batch = c0 == sg_lo && e0 == 0;
        uint32_t f[kWriteU];
        int tok[kWriteU];
        if (second && first_batch) {
#pragma unroll
          for (int q = 0; q < kWriteU; ++q) {
            f[q] = keep[q] >> kSlotBits;
            tok[q] = (int)(keep[q] & kSlotMask);
          }
        } else {
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
#pragma unroll
          for (int q = 0; q < kWriteU; ++q) {
            f[q] = e0 + q * kWave + lane < tot ? final_mask(e[q], honoured) & want : 0u;
            tok[q] = (addr[q] & ~(seg_len - 1)) + (int)((e[q] >> 8) & (kMaxSegLen - 1));
          }
          if (!second && first_batch) {
#pragma unroll
            for (int q = 0; q < kWriteU; ++q) keep[q] = (uint32_t)tok[q] | (f[q] << kSlotBits);
          }
        }
        body(f, tok);
      }
    }
  };

  // sweep 1: this wave's count (per lane, summed over the wave once)
  int cw = 0;
  for_batches(false, [&](const uint32_t (&f)[kWriteU], const int (&tok)[kWriteU]) {
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
  for_batches(true, [&](const uint32_t (&f)[kWriteU], const int (&tok)[kWriteU]) {
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
  // belongs to exactly one (group, set)
  int4* info = reinterpret_cast<int4*>(w + l.off_info);
  int4* thr = reinterpret_cast<int4*>(w + l.off_thr);
  uint32_t* cand = reinterpret_cast<uint32_t*>(w + l.off_cand);
  int32_t* ccnt = reinterpret_cast<int32_t*>(w + l.off_ccnt);
  uint2* ibl = reinterpret_cast<uint2*>(w + l.off_ibl);
  int32_t* ibc = reinterpret_cast<int32_t*>(w + l.off_ibc);
  int32_t* iac = reinterpret_cast<int32_t*>(w + l.off_iac);
  hipLaunchKernelGGL(union_range_kernel, dim3(2, rows), dim3(kRangeThreads), 0, st, scores, s_ld, n,
                     k, info);
  spk_status e = check_launch("topk_select_union/range");
  if (e != SPK_OK) return e;
  hipLaunchKernelGGL(union_gather_kernel, dim3(l.parts, groups), dim3(kThreads), 0, st, scores,
                     s_ld, u, n, info, l.nseg, l.seg_len, cand, ccnt, ibl, ibc, iac);
  e = check_launch("topk_select_union/gather");
  if (e != SPK_OK) return e;
  hipLaunchKernelGGL(union_thr_kernel, dim3(S, groups), dim3(kThreads), 0, st, scores, s_ld, u, n,
                     info, l.nseg, l.seg_len, cand, ccnt, ibl, ibc, iac, thr);
  e = check_launch("topk_select_union/threshold");
  if (e != SPK_OK) return e;
  hipLaunchKernelGGL(union_write_kernel, dim3(1 + S, groups), dim3(kWriteThreads), 0, st, scores,
                     s_ld, u, n, thr, l.nseg, l.seg_len, cand, ccnt, idx, idx_ld, count,
                     u_list, u_mask, u_count, u_ld);
  return check_launch("topk_select_union/write");
}
