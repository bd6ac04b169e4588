// spk_stream_read: a plain streaming read of a device buffer.  It does none of the method's
// work; it is the bandwidth reference the sparse kernels are measured against on the device at
// hand (the HBM roofline as a kernel of this library reaches it, beside the vendor's peak).
//
// Each workgroup reads one contiguous chunk with 16-byte loads, four in flight per lane, and
// folds the words into a value that is stored only if it equals an improbable constant, so the
// loads stay live and nothing is written in practice.
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
    const uint4 a = p[i], b = p[i + kThreads], c = p[i + 2 * kThreads], d = p[i + 3 * kThreads];
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^
           (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < end; i += kThreads) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace
}  // namespace spk

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
