// lookahead_prefetch: the host-resident rows of the blocks a selection names are copied into
// HBM staging rows ahead of the attention that reads them, and the row-location table is
// pointed at the copies.
//
// SparDA §2 "Seleção Esparsa de Lookahead Treinável": the blocks layer l+1 needs are chosen
// from that layer's predictor while layer l still runs, so the blocks that are not resident can
// be brought in behind layer l's attention (its "Inovações Principais": a persistent kernel of a
// few workgroups copies the missing blocks while the model computes).  "Nem Todos os
// Pensamentos Necessitam de HBM", §3 (Proposition 1): the copy is exact, so reading a row from
// its copy gives the same result as reading it from host memory.
//
// Persistent: a fixed number of workgroups (the caller's `workgroups`, launched on its own
// stream beside the attention) loop over the (b, kvh) groups.  For its group a workgroup first
// points the rows the previous call redirected back to their home location (the read-only
// loc_home table), then walks the selected blocks in list order: the block at list position t
// owns the staging rows [stage_base + t*bs, stage_base + t*bs + bs); every row of it whose home
// is host memory is copied there and redirected, and the redirected rows are kept, as a compact
// list of tokens, for the next call.  Two passes per group: every home lookup of the selection's rows is issued at once
// and the host rows are listed in LDS (ballot compaction); then 16 lanes per row copy them with
// 16-byte loads through the pinned pool's device alias, four 16-row steps of loads in flight per
// wave.  Nothing the kernel writes to global memory is read back by it, so the only ordering
// needed is the barrier between the restore and the new redirections of a group (the same row
// may be redirected by both calls).
#include "spk_internal.h"

namespace spk {
namespace {

constexpr int kThreads = 256;

constexpr int kRowsPerThread = 8;              // home lookups per thread and pass
constexpr int kListCap = kThreads * kRowsPerThread;  // host rows of a group listed per pass
constexpr int kCopyRows = 4;                   // 16-row copy steps in flight per wave

template <typename KT>
__global__ __launch_bounds__(kThreads) void lookahead_prefetch_kernel(
    const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_count, int64_t sel_ld,
    int bs, int groups, int Hkv, int d, int n_tokens, const KT* __restrict__ k_host,
    const KT* __restrict__ v_host, int64_t h_sb, int64_t h_sh, int64_t h_sn, int64_t host_slots,
    KT* __restrict__ k, KT* __restrict__ v, int64_t kv_sb, int64_t kv_sh, int64_t kv_sn,
    int64_t stage_base, const int32_t* __restrict__ loc_home, int32_t* __restrict__ loc,
    int64_t loc_sb, int64_t loc_sh, int32_t* __restrict__ staged,
    int32_t* __restrict__ staged_count) {
  // host rows of the current pass: (list position in the selection, host slot, token)
  __shared__ int32_t lrow[kListCap], lslot[kListCap], ltok[kListCap];
  __shared__ int wcnt[kThreads / kWave];
  const int64_t cap = sel_ld * bs;  // staging rows (and staged-list entries) per group
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  const uint64_t lt = (1ull << lane) - 1ull;
  constexpr int LPR16 = 16;                     // lanes per row in the copy (16 bytes each)
  const int chunks = d * (int)sizeof(KT) / 16;  // 16-byte pieces of one row (16 or 32)
  for (int g = blockIdx.x; g < groups; g += gridDim.x) {
    const int b = g / Hkv, h = g % Hkv;
    const int32_t* home = loc_home + (int64_t)b * loc_sb + (int64_t)h * loc_sh;
    int32_t* live = loc + (int64_t)b * loc_sb + (int64_t)h * loc_sh;
    int32_t* st = staged + (int64_t)g * cap;
    // ---- the previous call's redirections go back home (a compact list: every load of a
    // thread's entries is issued before the first store)
    const int prev = (int)min((int64_t)max(staged_count[g], 0), cap);
    for (int i0 = 0; i0 < prev; i0 += kThreads * kRowsPerThread) {
      int tok[kRowsPerThread];
#pragma unroll
      for (int j = 0; j < kRowsPerThread; ++j) {
        const int i = i0 + j * kThreads + (int)threadIdx.x;
        tok[j] = i < prev ? st[i] : -1;
      }
      int hv[kRowsPerThread];
#pragma unroll
      for (int j = 0; j < kRowsPerThread; ++j)
        hv[j] = (tok[j] >= 0 && tok[j] < n_tokens) ? home[tok[j]] : 0;
#pragma unroll
      for (int j = 0; j < kRowsPerThread; ++j)
        if (tok[j] >= 0 && tok[j] < n_tokens) live[tok[j]] = hv[j];
    }
    __syncthreads();  // every restore is complete before a row is redirected again
    const int cnt = (int)min((int64_t)max(sel_count[g], 0), sel_ld);
    const int32_t* sel = sel_idx + (int64_t)g * sel_ld;
    const int rows = cnt * bs;
    const KT* kh = k_host + (int64_t)b * h_sb + (int64_t)h * h_sh;
    const KT* vh = v_host + (int64_t)b * h_sb + (int64_t)h * h_sh;
    KT* kd = k + (int64_t)b * kv_sb + (int64_t)h * kv_sh;
    KT* vd = v + (int64_t)b * kv_sb + (int64_t)h * kv_sh;
    int listed = 0;  // host rows redirected so far (the compact staged list)
    for (int p0 = 0; p0 < rows; p0 += kListCap) {
      // ---- pass 1: every home lookup of the pass issued at once; host rows listed in LDS
      int hv[kRowsPerThread], tk[kRowsPerThread];
#pragma unroll
      for (int j = 0; j < kRowsPerThread; ++j) {
        const int i = p0 + j * kThreads + (int)threadIdx.x;
        const int t = min(i, rows - 1) / bs, r = min(i, rows - 1) % bs;
        const int blk = sel[t];
        const int64_t tok64 = (int64_t)blk * bs + r;
        const bool ok = i < rows && blk >= 0 && tok64 < n_tokens;
        tk[j] = ok ? (int)tok64 : -1;
        hv[j] = home[ok ? tok64 : 0];
      }
      int nh = 0;
#pragma unroll
      for (int j = 0; j < kRowsPerThread; ++j) {
        const bool host = tk[j] >= 0 && hv[j] < 0 && (int64_t)(~hv[j]) < host_slots;
        nh += __popcll(__ballot(host));
      }
      if (lane == 0) wcnt[wid] = nh;
      __syncthreads();
      int base = 0;
      for (int w = 0; w < wid; ++w) base += wcnt[w];
      int nhost = 0;
      for (int w = 0; w < kThreads / kWave; ++w) nhost += wcnt[w];
#pragma unroll
      for (int j = 0; j < kRowsPerThread; ++j) {
        const int i = p0 + j * kThreads + (int)threadIdx.x;
        const bool host = tk[j] >= 0 && hv[j] < 0 && (int64_t)(~hv[j]) < host_slots;
        const uint64_t bal = __ballot(host);
        if (host) {
          const int q = base + __popcll(bal & lt);
          lrow[q] = i;
          lslot[q] = ~hv[j];
          ltok[q] = tk[j];
          st[listed + q] = tk[j];
        }
        base += __popcll(bal);
      }
      __syncthreads();
      // ---- pass 2: the listed rows copied, 16 lanes per row, every load of a step in flight
      const int sub = lane % LPR16, slot16 = lane / LPR16;
      const int parts = chunks > LPR16 ? 2 : 1;  // 16-byte pieces per lane and row
      for (int q0 = wid * 4 * kCopyRows; q0 < nhost; q0 += (kThreads / kWave) * 4 * kCopyRows) {
        uint4 kx[kCopyRows][2], vx[kCopyRows][2];
#pragma unroll
        for (int c = 0; c < kCopyRows; ++c) {
          const int q = min(q0 + c * 4 + slot16, nhost - 1);
          const int64_t hs = (int64_t)lslot[q] * h_sn;
#pragma unroll
          for (int part = 0; part < 2; ++part) {
            if (part < parts) {
              const int ch = min(sub + part * LPR16, chunks - 1);
              kx[c][part] = reinterpret_cast<const uint4*>(kh + hs)[ch];
              vx[c][part] = reinterpret_cast<const uint4*>(vh + hs)[ch];
            }
          }
        }
#pragma unroll
        for (int c = 0; c < kCopyRows; ++c) {
          const int q = q0 + c * 4 + slot16;
          if (q < nhost) {
            const int64_t dst = stage_base + lrow[q];
#pragma unroll
            for (int part = 0; part < 2; ++part) {
              const int ch = sub + part * LPR16;
              if (part < parts && ch < chunks) {
                reinterpret_cast<uint4*>(kd + dst * kv_sn)[ch] = kx[c][part];
                reinterpret_cast<uint4*>(vd + dst * kv_sn)[ch] = vx[c][part];
              }
            }
            if (sub == 0) live[ltok[q]] = (int32_t)dst;
          }
        }
      }
      listed += nhost;
      __syncthreads();  // the LDS list is reused by the next pass
    }
    if (threadIdx.x == 0) staged_count[g] = listed;
    __syncthreads();  // the group's entries are settled before the workgroup moves on
  }
}

// A host pool must be page-locked, device-mapped host memory; the kernel reads it through the
// device address HIP reports for it.
spk_status pool_device_ptr(const void* p, const void** dev, const char* name) {
  hipPointerAttribute_t at{};
  const hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return set_error(SPK_EINVAL, "lookahead_prefetch: %s is not memory known to HIP (%s)", name,
                     hipGetErrorString(e));
  }
  if (at.type != hipMemoryTypeHost || at.devicePointer == nullptr)
    return set_error(SPK_EINVAL, "lookahead_prefetch: %s must be pinned, device-mapped host memory",
                     name);
  *dev = at.devicePointer;
  return SPK_OK;
}

}  // namespace
}  // namespace spk

extern "C" SPK_API spk_status lookahead_prefetch(
    const int32_t* sel_idx, const int32_t* sel_count, int64_t sel_ld, int block_size, int B,
    int Hkv, int d, spk_dtype kv_dtype, int n_tokens, const void* k_host, const void* v_host,
    int64_t host_sb, int64_t host_sh, int64_t host_sn, int64_t host_slots, void* k, void* v,
    int64_t kv_sb, int64_t kv_sh, int64_t kv_sn, int64_t hbm_slots, int64_t stage_base,
    const int32_t* loc_home, int32_t* loc, int64_t loc_sb, int64_t loc_sh, int32_t* staged,
    int32_t* staged_count, int workgroups, void* stream) {
  using namespace spk;
  SPK_REQUIRE(B >= 0 && Hkv > 0 && block_size >= 1 && sel_ld >= 0 && n_tokens >= 0, SPK_EINVAL,
              "lookahead_prefetch: bad sizes");
  SPK_REQUIRE(d == 64 || d == 128, SPK_EUNSUPPORTED, "lookahead_prefetch: d=%d not in {64,128}", d);
  SPK_REQUIRE(kv_dtype == SPK_BF16 || kv_dtype == SPK_F32, SPK_EUNSUPPORTED,
              "lookahead_prefetch: unsupported dtype");
  SPK_REQUIRE(workgroups >= 1 && workgroups <= 65535, SPK_EINVAL,
              "lookahead_prefetch: workgroups %d outside [1, 65535]", workgroups);
  SPK_REQUIRE(sel_ld * block_size < ((int64_t)1 << 31), SPK_EINVAL,
              "lookahead_prefetch: sel_ld * block_size too large");
  SPK_REQUIRE(B == 0 || (sel_idx && sel_count && k_host && v_host && k && v && loc_home && loc &&
                         staged && staged_count),
              SPK_EINVAL, "lookahead_prefetch: null pointer");
  SPK_REQUIRE(host_sn >= d && kv_sn >= d && host_sb >= 0 && host_sh >= 0 && kv_sb >= 0 &&
                  kv_sh >= 0 && host_sn % 8 == 0 && host_sh % 8 == 0 && host_sb % 8 == 0 &&
                  kv_sn % 8 == 0 && kv_sh % 8 == 0 && kv_sb % 8 == 0 && loc_sb >= 0 && loc_sh >= 0,
              SPK_EINVAL, "lookahead_prefetch: strides must be multiples of 8 with row strides >= d");
  SPK_REQUIRE(stage_base >= n_tokens && stage_base + sel_ld * block_size <= hbm_slots,
              SPK_EINVAL,
              "lookahead_prefetch: staging rows [%lld, %lld) must lie past the %d tokens and "
              "inside the %lld HBM rows",
              (long long)stage_base, (long long)(stage_base + sel_ld * block_size), n_tokens,
              (long long)hbm_slots);
  SPK_REQUIRE(stage_base + sel_ld * block_size < ((int64_t)1 << 31), SPK_EINVAL,
              "lookahead_prefetch: staging rows beyond int32 locations");
  SPK_REQUIRE(host_slots >= 0, SPK_EINVAL, "lookahead_prefetch: negative host pool");
  SPK_REQUIRE(reinterpret_cast<uintptr_t>(k) % 16 == 0 && reinterpret_cast<uintptr_t>(v) % 16 == 0 &&
                  reinterpret_cast<uintptr_t>(k_host) % 16 == 0 &&
                  reinterpret_cast<uintptr_t>(v_host) % 16 == 0,
              SPK_EINVAL, "lookahead_prefetch: pools must be 16-byte aligned");
  if (B == 0 || sel_ld == 0 || n_tokens == 0) {
    clear_error();
    return SPK_OK;
  }
  const void* khd = nullptr;
  const void* vhd = nullptr;
  spk_status e = pool_device_ptr(k_host, &khd, "k_host");
  if (e != SPK_OK) return e;
  e = pool_device_ptr(v_host, &vhd, "v_host");
  if (e != SPK_OK) return e;
  clear_error();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int groups = B * Hkv;
  const int wg = workgroups < groups ? workgroups : groups;
#define SPK_LA(KTV)                                                                              \
  hipLaunchKernelGGL(lookahead_prefetch_kernel<KTV>, dim3(wg), dim3(kThreads), 0, st, sel_idx,   \
                     sel_count, sel_ld, block_size, groups, Hkv, d, n_tokens,                     \
                     reinterpret_cast<const KTV*>(khd), reinterpret_cast<const KTV*>(vhd), host_sb, \
                     host_sh, host_sn, host_slots, reinterpret_cast<KTV*>(k),                      \
                     reinterpret_cast<KTV*>(v), kv_sb, kv_sh, kv_sn, stage_base, loc_home, loc,     \
                     loc_sb, loc_sh, staged, staged_count)
  if (kv_dtype == SPK_BF16) SPK_LA(uint16_t);
  else SPK_LA(float);
#undef SPK_LA
  return check_launch("lookahead_prefetch");
}
