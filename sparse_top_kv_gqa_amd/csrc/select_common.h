// Exact selection primitives on order-preserving uint32 keys (see order_key): a workgroup-wide
// radix select (8-bit digits, most significant first), a one-barrier-per-pass radix search and
// the register and LDS top-k built on it.  Shared by topk_select, tier_classify, the residency
// update and the attention's in-kernel selection.
#pragma once

#include "spk_internal.h"

namespace spk {

// Key histogram of the wide-row selection: the top kHistBits bits of an order key name its bin.
constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kHistShift = 32 - kHistBits;

// Wave 0 finds the digit where the running count (from the largest digit down) reaches kk.
// Writes sh[0] = digit, sh[1] = number of candidates with a larger digit.
__device__ __forceinline__ void find_digit(const uint32_t* h, int kk, int* sh) {
  const int l = lane_id();
  const int d0 = 255 - 4 * l;
  const int c0 = (int)h[d0], c1 = (int)h[d0 - 1], c2 = (int)h[d0 - 2], c3 = (int)h[d0 - 3];
  const int s = c0 + c1 + c2 + c3;
  const int incl = wave_incl_scan(s);
  const int excl = incl - s;
  if (excl < kk && kk <= incl) {
    int acc = excl;
    if (acc + c0 >= kk) {
      sh[0] = d0; sh[1] = acc;
    } else if ((acc += c0) + c1 >= kk) {
      sh[0] = d0 - 1; sh[1] = acc;
    } else if ((acc += c1) + c2 >= kk) {
      sh[0] = d0 - 2; sh[1] = acc;
    } else {
      acc += c2;
      sh[0] = d0 - 3; sh[1] = acc;
    }
  }
}

// Radix select over the candidate keys a workgroup of NT threads visits with `for_each`
// (for_each(visit) calls visit(key) once for every candidate key this thread owns).
// Finds the key `thr` of the kk-th largest candidate (1 <= kk <= #candidates) and `need`, the
// number of candidates equal to thr that rank within the top kk (the rest of the top kk are
// strictly greater).  hist: NT/64*256 uint32 of LDS; sh: 2 ints of LDS.
template <int NT, typename ForEach>
__device__ void radix_select(const ForEach& for_each, int kk, uint32_t* hist, int* sh,
                             uint32_t* thr, int* need) {
  constexpr int NW = NT / kWave;
  uint32_t prefix = 0, pmask = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = threadIdx.x; i < NW * 256; i += NT) hist[i] = 0;
    __syncthreads();
    uint32_t* my = hist + (threadIdx.x / kWave) * 256;
    for_each([&](uint32_t key) {
      if ((key & pmask) == prefix) atomicAdd(&my[(key >> shift) & 255u], 1u);
    });
    __syncthreads();
    if (threadIdx.x < 256) {
      uint32_t s = 0;
      for (int w = 0; w < NW; ++w) s += hist[w * 256 + threadIdx.x];
      hist[threadIdx.x] = s;
    }
    __syncthreads();
    if (threadIdx.x < kWave) find_digit(hist, kk, sh);
    __syncthreads();
    const int dsel = sh[0];
    kk -= sh[1];
    prefix |= (uint32_t)dsel << shift;
    pmask |= 0xFFu << shift;
    __syncthreads();
  }
  *thr = prefix;
  *need = kk;
}

// One radix step, run by every wave on its own: from the 256-bin histogram h of the candidate
// keys' current digit, the digit of the rem-th largest candidate (dsel), the number of candidates
// with a larger digit (above) and with that digit (in_bin); wave-uniform results.
__device__ __forceinline__ void digit_of_rank(const uint32_t* h, int rem, int& dsel, int& above,
                                              int& in_bin) {
  // lane l holds digits 255-4l down to 252-4l; counts run from the largest digit down
  const int lane = lane_id();
  const int d0 = 255 - 4 * lane;
  const uint4 c4 = *reinterpret_cast<const uint4*>(h + d0 - 3);
  const int s = (int)(c4.x + c4.y + c4.z + c4.w);
  const int incl = wave_incl_scan_dpp(s);
  const int excl = incl - s;
  const uint64_t hit = __ballot(excl < rem && rem <= incl);
  int acc = excl, dd, cb;
  if (acc + (int)c4.w >= rem) {
    dd = d0;
    cb = (int)c4.w;
  } else if ((acc += (int)c4.w) + (int)c4.z >= rem) {
    dd = d0 - 1;
    cb = (int)c4.z;
  } else if ((acc += (int)c4.z) + (int)c4.y >= rem) {
    dd = d0 - 2;
    cb = (int)c4.y;
  } else {
    acc += (int)c4.y;
    dd = d0 - 3;
    cb = (int)c4.x;
  }
  const int src = (int)__builtin_ctzll(hit | (1ull << 63));
  dsel = __builtin_amdgcn_readlane(dd, src);
  above = __builtin_amdgcn_readlane(acc, src);
  in_bin = __builtin_amdgcn_readlane(cb, src);
}

// Radix search for the threshold of an exact top-kk (8-bit digits, most significant first).
// Every thread calls it; `for_each(visit)` calls visit(key) for each candidate key the thread
// owns.  hist: 4*256 uint32 of LDS, zero on entry (one histogram per digit, so a pass needs one
// barrier and nothing is cleared between passes).  Returns the kk-th largest key as *thr with
// *need, the number of keys equal to it that are kept (the first ones in index order); or, when
// a digit's bin holds exactly the keys still missing, *whole = true: keep every key >= *thr.
template <typename ForEach>
__device__ __forceinline__ void radix_threshold(const ForEach& for_each, int kk, uint32_t* hist,
                                                uint32_t* thr, int* need, bool* whole) {
  uint32_t prefix = 0, pmask = 0;
  int rem = kk;
  bool wh = false;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    uint32_t* h = hist + pass * 256;
    for_each([&](uint32_t key) {
      if ((key & pmask) == prefix) atomicAdd(&h[(key >> shift) & 255u], 1u);
    });
    __syncthreads();
    int dsel, above, in_bin;
    digit_of_rank(h, rem, dsel, above, in_bin);
    rem -= above;
    prefix |= (uint32_t)dsel << shift;
    pmask |= 0xFFu << shift;
    if (in_bin == rem) {
      wh = true;
      break;
    }
  }
  *thr = prefix;
  *need = rem;
  *whole = wh;
}

__device__ __forceinline__ void keep_class(uint32_t key, bool valid, uint32_t thr, bool whole,
                                           bool& gt, bool& eq) {
  gt = valid && (whole ? key >= thr : key > thr);
  eq = valid && !whole && key == thr;
}

// Exact top-kk of n keys held in registers by a workgroup of NT threads (1 <= kk <= n <= KPT*NT):
// key[j] of thread t is element j*NT + t.  Ties go to the lowest index; calls out(position,
// index) for every kept element, positions 0..kk-1 in ascending index order.  hist: 4*256 uint32
// of LDS; wsum: KPT*NT/64 ints of LDS (KPT*NT/64 <= 256).  Barriers: one to clear, one per radix
// pass, one for the per-(chunk, wave) counts (two above 16 pairs); the caller waits (barrier)
// before reading what out wrote to LDS.
template <int NT, int KPT, bool kCleared = false, typename Out>
__device__ __forceinline__ void reg_topk(const uint32_t (&key)[KPT], int n, int kk, uint32_t* hist, int* wsum,
                         const Out& out) {
  constexpr int NW = NT / kWave;
  constexpr int NC = KPT * NW;  // (chunk, wave) pairs, in index order
  static_assert(NC <= 4 * kWave, "per-(chunk, wave) counts: at most 256");
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  if constexpr (!kCleared)  // kCleared: the caller zeroed hist (no barrier needed after it)
    for (int i = tid; i < 4 * 256; i += NT) hist[i] = 0u;
  __syncthreads();
  uint32_t thr;
  int need;
  bool whole;
  radix_threshold(
      [&](auto visit) {
#pragma unroll
        for (int j = 0; j < KPT; ++j)
          if (j * NT + tid < n) visit(key[j]);
      },
      kk, hist, &thr, &need, &whole);
  // element order: chunk j (indices j*NT ..), inside it wave w (64 indices), inside it the lane.
  // Kept counts per (chunk, wave), packed: greater-than in the low 16 bits, equal in the high
  // 16 (each total <= n <= 16384)
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    bool gt, eq;
    keep_class(key[j], j * NT + tid < n, thr, whole, gt, eq);
    const int c = __popcll(__ballot(gt)) | (__popcll(__ballot(eq)) << 16);
    if (lane == 0) wsum[j * NW + wid] = c;
  }
  __syncthreads();
  int pre[KPT];
  if constexpr (NC <= 16) {
    // few pairs: every thread reads all counts at once and sums its prefixes in registers
    int c[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) c[i] = wsum[i];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      int p = 0;
#pragma unroll
      for (int i = 0; i < NC; ++i) p += i < j * NW + wid ? c[i] : 0;
      pre[j] = p;
    }
  } else {
    // wave 0 turns the counts into exclusive prefixes (one wave scan per 64 pairs)
    if (wid == 0) {
      int carry = 0;
#pragma unroll
      for (int base = 0; base < NC; base += kWave) {
        const int i = base + lane;
        const int c = i < NC ? wsum[i] : 0;
        const int incl = wave_incl_scan(c);
        if (i < NC) wsum[i] = carry + incl - c;
        carry += __builtin_amdgcn_readlane(incl, kWave - 1);
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j) pre[j] = wsum[j * NW + wid];
  }
  const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    bool gt, eq;
    keep_class(key[j], j * NT + tid < n, thr, whole, gt, eq);
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    const int pe = (pre[j] >> 16) + __popcll(be & lt);
    const int pos = (pre[j] & 0xFFFF) + __popcll(bg & lt) + min(pe, need);
    if ((gt || (eq && pe < need)) && pos < kk) out(pos, j * NT + tid);
  }
}

// Exact top-kk of the n order keys keys[0..n) that a workgroup of NT threads holds in LDS
// (1 <= kk <= n), ties to the lowest index: calls out(position, index) once for every kept
// element, positions 0..kk-1 in ascending index order.  hist: 4*256 uint32 of LDS; wsum: 2*NT/64
// ints of LDS.  Every thread calls it after writing its keys; it begins and ends with a barrier.
template <int NT, typename Out>
__device__ __forceinline__ void lds_topk(const uint32_t* keys, int n, int kk, uint32_t* hist, int* wsum,
                         const Out& out) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
  for (int i = tid; i < 4 * 256; i += NT) hist[i] = 0u;
  __syncthreads();
  uint32_t thr;
  int need;
  bool whole;
  radix_threshold(
      [&](auto visit) {
        for (int i = tid; i < n; i += NT) visit(keys[i]);
      },
      kk, hist, &thr, &need, &whole);
  // wave w compacts the contiguous index range [w*seg, w*seg + seg)
  const int seg = ((n + NW - 1) / NW + kWave - 1) / kWave * kWave;
  const int lo = wid * seg, hi = min(n, lo + seg);
  int cg = 0, ce = 0;
  for (int i0 = lo; i0 < hi; i0 += kWave) {
    const int i = i0 + lane;
    bool gt, eq;
    keep_class(i < hi ? keys[i] : 0u, i < hi, thr, whole, gt, eq);
    cg += __popcll(__ballot(gt));
    ce += __popcll(__ballot(eq));
  }
  if (lane == 0) {
    wsum[2 * wid] = cg;
    wsum[2 * wid + 1] = ce;
  }
  __syncthreads();
  int run_g = 0, run_e = 0;
  for (int w = 0; w < wid; ++w) {
    run_g += wsum[2 * w];
    run_e += wsum[2 * w + 1];
  }
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int i0 = lo; i0 < hi; i0 += kWave) {
    const int i = i0 + lane;
    bool gt, eq;
    keep_class(i < hi ? keys[i] : 0u, i < hi, thr, whole, gt, eq);
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    const int pe = run_e + __popcll(be & lt);
    const int pos = run_g + __popcll(bg & lt) + min(pe, need);
    if ((gt || (eq && pe < need)) && pos < kk) out(pos, i);
    run_g += __popcll(bg);
    run_e += __popcll(be);
  }
  __syncthreads();
}

}  // namespace spk
