// Exact selection primitives on order-preserving uint32 keys (see order_key): a workgroup-wide
// radix select (8-bit digits, most significant first) and a small LDS bitonic sort.  Shared by
// topk_select and tier_classify.
#pragma once

#include "spk_internal.h"

namespace spk {

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

// In-place descending bitonic sort of P (a power of two) 64-bit values in LDS.
__device__ __forceinline__ void bitonic_sort_desc(uint64_t* s, int P) {
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < (P >> 1); t += blockDim.x) {
        const int i = 2 * stride * (t / stride) + (t % stride);
        const int j = i + stride;
        const bool desc = (i & size) == 0;
        const uint64_t a = s[i], b = s[j];
        if (desc ? (a < b) : (a > b)) {
          s[i] = b;
          s[j] = a;
        }
      }
      __syncthreads();
    }
  }
}

}  // namespace spk
