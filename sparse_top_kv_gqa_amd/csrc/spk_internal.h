// Internal helpers of libspk: status reporting, argument checks and device primitives
// shared by the kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "spk.h"

namespace spk {

// ---------------------------------------------------------------- status / errors (host)

spk_status set_error(spk_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

#define SPK_REQUIRE(cond, st, ...)                    \
  do {                                                \
    if (!(cond)) return ::spk::set_error((st), __VA_ARGS__); \
  } while (0)

// Check the launch that was just enqueued.
inline spk_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(SPK_EHIP, "%s: %s", what, hipGetErrorString(e));
  return SPK_OK;
}

inline size_t dtype_size(spk_dtype t) { return t == SPK_BF16 ? 2 : 4; }
inline bool dtype_ok(spk_dtype t) { return t == SPK_F32 || t == SPK_BF16; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Number of compute units of the current device (cached per device id).
int num_cus();

// ---------------------------------------------------------------- device primitives

constexpr int kWave = 64;

// bf16 pair packed in a dword -> two floats (exact: a bf16 is the top half of an fp32).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// 16-byte load through the global address space from an integer address (keeps the compiler
// from falling back to flat loads, whose waits also stall on LDS traffic).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 gload16(uint64_t addr) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(1))) const u32x4 global_u32x4;
  const u32x4 v = *reinterpret_cast<global_u32x4*>(addr);
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *reinterpret_cast<const uint4*>(addr);
#endif
}

// 16-byte nontemporal load (streaming: the line is not kept in the caches).  For data read once
// per pass over HBM it streams measurably faster than a plain load.
__device__ __forceinline__ uint4 gload16_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint4 gload16_nt(uint64_t addr) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(1))) const u32x4 global_u32x4;
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<global_u32x4*>(addr));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *reinterpret_cast<const uint4*>(addr);
#endif
}

// Eight consecutive elements of a row, kept raw until they are needed (lets a loop issue
// many loads before the first use).
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> {  // bf16
  uint4 u;
  __device__ __forceinline__ void load(const uint16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void load_addr(uint64_t a) { u = gload16(a); }
  __device__ __forceinline__ void load_nt(const uint16_t* p) { u = gload16_nt(p); }
  __device__ __forceinline__ void to_float(float (&x)[8]) const {
    x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
    x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z); x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
  }
  __device__ __forceinline__ void zero() { u = make_uint4(0, 0, 0, 0); }
};
template <> struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void load_addr(uint64_t x) {
    const uint4 u0 = gload16(x), u1 = gload16(x + 16);
    a = make_float4(__uint_as_float(u0.x), __uint_as_float(u0.y), __uint_as_float(u0.z),
                    __uint_as_float(u0.w));
    b = make_float4(__uint_as_float(u1.x), __uint_as_float(u1.y), __uint_as_float(u1.z),
                    __uint_as_float(u1.w));
  }
  __device__ __forceinline__ void load_nt(const float* p) {
    const uint4 u0 = gload16_nt(p), u1 = gload16_nt(p + 4);
    a = make_float4(__uint_as_float(u0.x), __uint_as_float(u0.y), __uint_as_float(u0.z),
                    __uint_as_float(u0.w));
    b = make_float4(__uint_as_float(u1.x), __uint_as_float(u1.y), __uint_as_float(u1.z),
                    __uint_as_float(u1.w));
  }
  __device__ __forceinline__ void to_float(float (&x)[8]) const {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  __device__ __forceinline__ void zero() { a = make_float4(0, 0, 0, 0); b = a; }
};

template <typename T>
__device__ __forceinline__ void load8f(const T* p, float (&x)[8]) {
  Raw8<T> r;
  r.load(p);
  r.to_float(x);
}

// DPP lane moves inside a row of 16 lanes.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, true));
}
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sum over aligned groups of kLanes (2, 4, 8 or 16) lanes; every lane of the group gets the
// same bits (each step adds a lane's value and its partner's, which commute).
template <int kLanes>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(kLanes == 2 || kLanes == 4 || kLanes == 8 || kLanes == 16, "lanes");
  x += dpp<kDppQuadXor1>(x);
  if constexpr (kLanes >= 4) x += dpp<kDppQuadXor2>(x);
  if constexpr (kLanes >= 8) x += dpp<kDppRowHalfMirror>(x);
  if constexpr (kLanes >= 16) x += dpp<kDppRowMirror>(x);
  return x;
}

// Order-preserving map of an fp32 score to uint32: larger float -> larger key; -0 -> +0; NaN
// -> 0 (below -inf, whose key is 0x007fffff).
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (x != x) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Inclusive prefix sum of an int over the wave with DPP lane moves (no LDS round trips): a
// scan inside each row of 16 lanes (shifts by 1, 2, 4, 8; lanes shifted in from outside the row
// add 0), then the row totals carried forward with the broadcasts of lane 15 (into rows 1 and 3)
// and of lane 31 (into rows 2 and 3).
__device__ __forceinline__ int wave_incl_scan_dpp(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Inclusive prefix maximum over the wave of values >= -1 (the DPP steps of wave_incl_scan_dpp
// with max, and -1 where a lane has no source).
__device__ __forceinline__ int wave_incl_max(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x111, 0xF, 0xF, false));  // row_shr:1
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x112, 0xF, 0xF, false));  // row_shr:2
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x114, 0xF, 0xF, false));  // row_shr:4
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x118, 0xF, 0xF, false));  // row_shr:8
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x142, 0xA, 0xF, false));  // row_bcast:15
  x = max(x, __builtin_amdgcn_update_dpp(-1, x, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return x;
}

// Inclusive prefix sum of an int over the wave.
__device__ __forceinline__ int wave_incl_scan(int x) { return wave_incl_scan_dpp(x); }

// Block-wide exclusive scan of one int per thread; returns the exclusive prefix and writes
// the block total to *total.  `scratch` holds at least blockDim.x/64 + 1 ints of LDS.
__device__ __forceinline__ int block_excl_scan(int x, int* scratch, int* total) {
  const int lane = lane_id();
  const int wid = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  int incl = wave_incl_scan(x);
  if (lane == kWave - 1) scratch[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    int v = lane < nw ? scratch[lane] : 0;
    int vi = wave_incl_scan(v);
    if (lane < nw) scratch[lane] = vi - v;
    if (lane == nw - 1) scratch[nw] = vi;
  }
  __syncthreads();
  int r = scratch[wid] + incl - x;
  *total = scratch[nw];
  __syncthreads();
  return r;
}

}  // namespace spk
