// Bandwidth references: reads that do none of the method's work, against which the sparse
// kernels are measured on the device at hand.
//
// spk_stream_read: a plain streaming read of a device buffer (the HBM roofline as a kernel of
// this library reaches it, beside the vendor's peak).  Each workgroup reads one contiguous
// chunk with 16-byte nontemporal loads, four in flight per lane: of the read shapes measured
// (64 to 1024 threads, 4 to 16 loads in flight, chunks of 8 KB to 512 KB, plain or
// nontemporal loads) the fastest, at about 6.9-7.0 TB/s over 1 GiB against 6.1-6.5 TB/s for
// plain loads.
//
// spk_gather_read: the K and V rows of per-group row lists, read once each and nothing else
// (the rate the HBM allows for that exact set of rows, scattered as the selection scattered
// them).  Each workgroup takes a contiguous part of its group's list; a row is read by
// row_bytes/16 lanes with 16-byte loads, four passes of rows in flight.
//
// Both fold the words into a value that is stored only if it equals an improbable constant, so
// the loads stay live and nothing is written in practice.
#include "spk_internal.h"

namespace spk {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ p,
                                                               uint64_t n16, uint64_t per_wg,
                                                               uint32_t* __restrict__ sink) {
  const uint64_t beg = (uint64_t)blockIdx.x * per_wg;
  const uint64_t end = beg + per_wg < n16 ? beg + per_wg : n16;
  uint32_t acc = 0;
  uint64_t i = beg + threadIdx.x;
  for (; i + 3 * kThreads < end; i += 4 * kThreads) {
    const uint4 a = gload16_nt(p + i), b = gload16_nt(p + i + kThreads),
                c = gload16_nt(p + i + 2 * kThreads), d = gload16_nt(p + i + 3 * kThreads);
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^
           (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < end; i += kThreads) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

constexpr int kGatherPasses = 4;  // passes of rows in flight per lane

template <int LPR>  // lanes per row: row_bytes / 16
__global__ __launch_bounds__(kThreads) void gather_read_kernel(
    uint64_t k, uint64_t v, int64_t sg, int64_t sn, const int32_t* __restrict__ rows,
    int64_t rows_ld, int64_t n_rows, int per_wg, uint32_t* __restrict__ sink) {
  constexpr int RPP = kThreads / LPR;  // rows per pass of the workgroup
  const int g = blockIdx.y;
  const int64_t r0 = (int64_t)blockIdx.x * per_wg;
  const int64_t r1 = r0 + per_wg < rows_ld ? r0 + per_wg : rows_ld;
  const int32_t* lst = rows + (int64_t)g * rows_ld;
  const int sub = (int)threadIdx.x % LPR, slot = (int)threadIdx.x / LPR;
  const uint64_t kb = k + (uint64_t)((int64_t)g * sg) + 16u * (uint64_t)sub;
  const uint64_t vb = v + (uint64_t)((int64_t)g * sg) + 16u * (uint64_t)sub;
  uint32_t acc = 0;
  for (int64_t r = r0; r < r1; r += RPP * kGatherPasses) {
    bool live[kGatherPasses];
    uint64_t off[kGatherPasses];
#pragma unroll
    for (int u = 0; u < kGatherPasses; ++u) {
      const int64_t i = r + u * RPP + slot;
      const int32_t t = i < r1 ? lst[i] : -1;
      live[u] = t >= 0 && t < n_rows;
      off[u] = live[u] ? (uint64_t)((int64_t)t * sn) : 0u;  // a skipped row re-reads row 0
    }
    uint4 a[kGatherPasses], b[kGatherPasses];
#pragma unroll
    for (int u = 0; u < kGatherPasses; ++u) {
      a[u] = gload16(kb + off[u]);
      b[u] = gload16(vb + off[u]);
    }
#pragma unroll
    for (int u = 0; u < kGatherPasses; ++u)
      if (live[u]) acc ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w ^ b[u].x ^ b[u].y ^ b[u].z ^ b[u].w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace
}  // namespace spk

extern "C" SPK_API spk_status spk_gather_read(const void* k, const void* v, int64_t row_bytes,
                                              int64_t group_stride, int64_t row_stride,
                                              int64_t n_rows, const int32_t* rows,
                                              int64_t rows_ld, int groups, int wg_per_group,
                                              uint32_t* sink, void* stream) {
  using namespace spk;
  SPK_REQUIRE(k && v && sink && (rows || rows_ld == 0), SPK_EINVAL,
              "spk_gather_read: null k, v, rows or sink");
  SPK_REQUIRE(row_bytes == 64 || row_bytes == 128 || row_bytes == 256 || row_bytes == 512 ||
                  row_bytes == 1024,
              SPK_EINVAL, "spk_gather_read: row_bytes %lld not one of 64..1024 (powers of two)",
              (long long)row_bytes);
  SPK_REQUIRE(reinterpret_cast<uintptr_t>(k) % 16 == 0 && reinterpret_cast<uintptr_t>(v) % 16 == 0 &&
                  group_stride % 16 == 0 && row_stride % 16 == 0,
              SPK_EINVAL, "spk_gather_read: k, v and strides must be multiples of 16 bytes");
  SPK_REQUIRE(group_stride >= 0 && row_stride >= row_bytes && n_rows >= 0 && rows_ld >= 0 &&
                  rows_ld < (1LL << 31) && groups >= 0 && groups <= 65535,
              SPK_EINVAL, "spk_gather_read: bad strides or sizes");
  SPK_REQUIRE(wg_per_group >= 1 && wg_per_group <= 65535, SPK_EINVAL,
              "spk_gather_read: wg_per_group %d not in [1, 65535]", wg_per_group);
  clear_error();
  if (groups == 0 || rows_ld == 0 || n_rows == 0) return SPK_OK;  // no row can be read
  const int per = (int)((rows_ld + wg_per_group - 1) / wg_per_group);
  const int wgs = (int)((rows_ld + per - 1) / per);
  const dim3 grid(wgs, groups);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint64_t kk = reinterpret_cast<uint64_t>(k), vv = reinterpret_cast<uint64_t>(v);
#define SPK_GATHER(L)                                                                          \
  hipLaunchKernelGGL(gather_read_kernel<L>, grid, dim3(kThreads), 0, st, kk, vv, group_stride, \
                     row_stride, rows, rows_ld, n_rows, per, sink)
  switch (row_bytes / 16) {
    case 4: SPK_GATHER(4); break;
    case 8: SPK_GATHER(8); break;
    case 16: SPK_GATHER(16); break;
    case 32: SPK_GATHER(32); break;
    default: SPK_GATHER(64); break;
  }
#undef SPK_GATHER
  return check_launch("spk_gather_read");
}

extern "C" SPK_API spk_status spk_stream_read_host(const void* host, size_t bytes, int workgroups,
                                                   uint32_t* sink, void* stream) {
  using namespace spk;
  SPK_REQUIRE(host && sink, SPK_EINVAL, "spk_stream_read_host: null buffer or sink");
  SPK_REQUIRE(reinterpret_cast<uintptr_t>(host) % 16 == 0 && bytes % 16 == 0, SPK_EINVAL,
              "spk_stream_read_host: buffer and size must be multiples of 16 bytes");
  SPK_REQUIRE(workgroups >= 1 && workgroups <= (1 << 20), SPK_EINVAL,
              "spk_stream_read_host: workgroups %d not in [1, 2^20]", workgroups);
  clear_error();
  if (bytes == 0) return SPK_OK;
  // the caller states that this is host memory; it is read through the device address HIP
  // reports for it, and only memory HIP reports as host memory with such an address is taken
  // (the check of the attention's host pools)
  hipPointerAttribute_t at{};
  const hipError_t e = hipPointerGetAttributes(&at, host);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return set_error(SPK_EINVAL, "spk_stream_read_host: the buffer is not memory known to HIP (%s)",
                     hipGetErrorString(e));
  }
  SPK_REQUIRE(at.type == hipMemoryTypeHost && at.devicePointer != nullptr, SPK_EINVAL,
              "spk_stream_read_host: the buffer must be pinned, device-mapped host memory");
  const uint64_t n16 = bytes / 16;
  const uint64_t per = (n16 + workgroups - 1) / workgroups;
  const int wgs = (int)((n16 + per - 1) / per);
  hipLaunchKernelGGL(stream_read_kernel, dim3(wgs), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const uint4*>(at.devicePointer), n16, per, sink);
  return check_launch("spk_stream_read_host");
}

extern "C" SPK_API spk_status spk_stream_read(const void* p, size_t bytes, int workgroups,
                                              uint32_t* sink, void* stream) {
  using namespace spk;
  SPK_REQUIRE(p && sink, SPK_EINVAL, "spk_stream_read: null buffer or sink");
  SPK_REQUIRE(reinterpret_cast<uintptr_t>(p) % 16 == 0 && bytes % 16 == 0, SPK_EINVAL,
              "spk_stream_read: buffer and size must be multiples of 16 bytes");
  SPK_REQUIRE(workgroups >= 1 && workgroups <= (1 << 20), SPK_EINVAL,
              "spk_stream_read: workgroups %d not in [1, 2^20]", workgroups);
  clear_error();
  if (bytes == 0) return SPK_OK;
  const uint64_t n16 = bytes / 16;
  const uint64_t per = (n16 + workgroups - 1) / workgroups;
  const int wgs = (int)((n16 + per - 1) / per);
  hipLaunchKernelGGL(stream_read_kernel, dim3(wgs), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint4*>(p), n16,
                     per, sink);
  return check_launch("spk_stream_read");
}
