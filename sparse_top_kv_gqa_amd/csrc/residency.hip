// residency_update and residency_prefetch: which rows of a sequence hold an HBM slot after a
// tier reassignment, and the copy of newly resident rows from host memory into their slots.
//
// "Nem Todos os Pensamentos Necessitam de HBM", §1 "Classificação de Quatro Níveis": T0 stays in
// HBM, T1 lives in host DDR at full precision and reaches the attention from there; §4
// "Implementação do Sistema": tiers are reassigned periodically and the prefetch is
// differential — only rows that newly need HBM cross PCIe.  "O Fim do Gargalo de Memória ...",
// "A Inovação": rows may stay resident in HBM while memory allows (load-adaptive residency).
//
// The resident set of a sequence is the first `capacity` rows of T0 ∪ T1 ranked by (tier
// ascending, importance descending, index ascending).  A resident row that already holds a
// slot keeps it; the other resident rows, in ascending token order, take the free slots in
// ascending order.  Every row also lives in host memory at its token index, so loc[tok] is the
// HBM slot of a resident row and ~tok otherwise — the form sparse_decode_attn reads.  The
// tiers' roles come as a table (2 bits per tier code: ranked first, ranked second, or never
// resident): T0 then T1 for the HBM residency, T2 alone for the staging rows of the 8-bit tier.
#include "select_common.h"

namespace spk {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kItems = 16;                        // register path: n_tokens <= 16384
constexpr int kMaxTokens = kItems * kThreads;
constexpr int kSlotWords = kMaxTokens / 32;       // its slot bitmap: capacity <= 16384
// Longer sequences: tokens are taken chunk by chunk from memory, the slot bitmap covers up to
// 131072 slots (16 KB of LDS, and as much again for the free-slot prefixes).
constexpr int kChunkCap = 131072;
constexpr int kChunkWords = kChunkCap / 32;
constexpr int kWordsPerThread = kChunkWords / kThreads;
constexpr int kMaxTokensChunked = 1 << 30;
constexpr int32_t kNeedsSlot = INT32_MIN;         // loc between the passes: resident, no slot yet

// The k-th zero bit (k counted from 0, least significant first) of w.
__device__ __forceinline__ int nth_zero_bit(uint32_t w, int k) {
  uint32_t z = ~w;
  for (int i = 0; i < k; ++i) z &= z - 1;  // drop the k lowest zero bits
  return __builtin_ctz(z);
}

// The class of a tier for the ranking: 0 and 1 are the two ranked classes (class 0 first),
// any other value is not resident; `classes` holds 2 bits per tier code 0..3.
__device__ __forceinline__ uint8_t tier_class(uint32_t classes, uint8_t t) {
  return (uint8_t)((classes >> (2u * (t & 3u))) & 3u);
}

__global__ __launch_bounds__(kThreads) void residency_kernel(
    const uint8_t* __restrict__ tier_all, int64_t tier_ld, const float* __restrict__ s_all,
    int64_t s_ld, int n, int capacity, uint32_t classes, int32_t* __restrict__ loc_all,
    int64_t loc_ld, int32_t* __restrict__ copy_tok, int32_t* __restrict__ copy_slot,
    int64_t copy_ld, int32_t* __restrict__ copy_count) {
  __shared__ __align__(16) uint32_t hist[4 * 256];
  __shared__ uint32_t held_bits[kSlotWords];
  __shared__ int free_pre[kSlotWords + 1];   // free slots before each bitmap word
  __shared__ int scratch[kWaves + 1];
  __shared__ int counts[2];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const uint8_t* tier = tier_all + (int64_t)b * tier_ld;
  const float* s = s_all + (int64_t)b * s_ld;
  int32_t* loc = loc_all + (int64_t)b * loc_ld;

  // tiers and importance keys of this thread's tokens (NaN -> 0, the lowest key)
  uint8_t tr[kItems];
  uint32_t key[kItems];
  int c0 = 0, c1 = 0;
  {
    // every load issued before any is used (clamped in bounds): one wait for the sequence
    uint8_t tv[kItems];
    float sv[kItems];
#pragma unroll
    for (int c = 0; c < kItems; ++c) {
      tv[c] = 3;
      sv[c] = 0.f;
    }
    if (n > 0) {
#pragma unroll
      for (int c = 0; c < kItems; ++c) {
        const int ic = min(c * kThreads + tid, n - 1);
        tv[c] = tier[ic];
        sv[c] = s[ic];
      }
    }
#pragma unroll
    for (int c = 0; c < kItems; ++c) {
      const bool in = c * kThreads + tid < n;
      tr[c] = in ? tier_class(classes, tv[c]) : (uint8_t)3;
      key[c] = in ? order_key(sv[c]) : 0u;
      c0 += tr[c] == 0;
      c1 += tr[c] == 1;
    }
  }
  for (int i = tid; i < 4 * 256; i += kThreads) hist[i] = 0u;
  for (int i = tid; i < kSlotWords; i += kThreads) held_bits[i] = 0u;
  if (tid == 0) counts[0] = counts[1] = 0;
  __syncthreads();
  atomicAdd(&counts[0], c0);
  atomicAdd(&counts[1], c1);
  __syncthreads();
  const int n0 = counts[0], n1 = counts[1];

  // Which tier is cut by the capacity, and how many of its rows are kept: all of T0 and the
  // top `cut` of T1, or the top `cut` of T0 alone; a tier kept whole needs no threshold.
  const int cut_tier = capacity >= n0 + n1 ? -1 : (capacity >= n0 ? 1 : 0);
  const int cut = cut_tier == 1 ? capacity - n0 : (cut_tier == 0 ? capacity : 0);
  uint32_t thr = 0;
  int need = 0;
  bool whole = false;
  if (cut > 0) {
    radix_threshold(
        [&](auto visit) {
#pragma unroll
          for (int c = 0; c < kItems; ++c)
            if (tr[c] == cut_tier) visit(key[c]);
        },
        cut, hist, &thr, &need, &whole);
  }

  // Pass A, in index order: the resident set, the slots kept rows hold, loc of non-resident
  // rows; `fresh` marks resident rows that need a slot (bit c: item c).
  uint32_t fresh = 0;
  int run_eq = 0;
#pragma unroll
  for (int c = 0; c < kItems; ++c) {
    const int i = c * kThreads + tid;
    const bool in_cut = tr[c] == cut_tier && cut_tier >= 0;
    const bool gt = in_cut && cut > 0 && (whole ? key[c] >= thr : key[c] > thr);
    const bool eq = in_cut && cut > 0 && !whole && key[c] == thr;
    int tot_eq;
    const int pre = block_excl_scan(eq ? 1 : 0, scratch, &tot_eq);
    const bool kept_cut = gt || (eq && run_eq + pre < need);
    run_eq += tot_eq;
    bool res;
    if (cut_tier < 0) res = tr[c] <= 1;
    else if (cut_tier == 1) res = tr[c] == 0 || kept_cut;
    else res = kept_cut;
    if (i < n) {
      const int old = loc[i];
      const bool held = res && old >= 0 && old < capacity;
      if (held) atomicOr(&held_bits[old >> 5], 1u << (old & 31));
      if (!res) loc[i] = ~i;
      if (res && !held) fresh |= 1u << c;
    }
  }
  __syncthreads();
  // free slots per bitmap word (slots >= capacity are not free), then their prefix
  const int words = (capacity + 31) / 32;
  int fz = 0;
  if (tid < words) {
    const int lim = min(32, capacity - tid * 32);
    const uint32_t valid = lim == 32 ? 0xFFFFFFFFu : ((1u << lim) - 1u);
    fz = __popc(~held_bits[tid] & valid);
  }
  int tot_free;
  const int fp = block_excl_scan(tid < kSlotWords ? fz : 0, scratch, &tot_free);
  if (tid < kSlotWords) free_pre[tid] = fp;
  if (tid == 0) free_pre[kSlotWords] = tot_free;
  __syncthreads();

  // Pass B, in index order: the r-th fresh row takes the r-th free slot
  int run = 0;
#pragma unroll
  for (int c = 0; c < kItems; ++c) {
    const int i = c * kThreads + tid;
    const bool f = (fresh >> c) & 1u;
    int tot;
    const int r = run + block_excl_scan(f ? 1 : 0, scratch, &tot);
    run += tot;
    if (f && r < tot_free) {
      // word w with free_pre[w] <= r < free_pre[w + 1]
      int lo = 0, hi = words;  // free_pre[lo] <= r < free_pre[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (free_pre[mid] <= r) lo = mid;
        else hi = mid;
      }
      const int slot = lo * 32 + nth_zero_bit(held_bits[lo], r - free_pre[lo]);
      loc[i] = slot;
      if (r < copy_ld) {
        copy_tok[(int64_t)b * copy_ld + r] = i;
        copy_slot[(int64_t)b * copy_ld + r] = slot;
      }
    } else if (f && i < n) {
      loc[i] = ~i;  // no slot left (only when loc held a slot twice): read from host memory
    }
  }
  if (tid == 0) copy_count[b] = min(run, tot_free);  // the copies listed
}

// Free slots of a bitmap of held slots (up to kChunkCap): free_pre[w] = free slots in words
// below w (slots >= capacity are not free), free_pre[kChunkWords] = the total, which is
// returned.  Each thread owns kWordsPerThread consecutive words; ends with a barrier.
__device__ int free_slot_prefix(const uint32_t* held_bits, int capacity, int* free_pre,
                                int* scratch) {
  const int tid = threadIdx.x;
  const int words = (capacity + 31) / 32;
  int fz[kWordsPerThread];
  int fsum = 0;
#pragma unroll
  for (int j = 0; j < kWordsPerThread; ++j) {
    const int w = tid * kWordsPerThread + j;
    fz[j] = 0;
    if (w < words) {
      const int lim = min(32, capacity - w * 32);
      const uint32_t valid = lim == 32 ? 0xFFFFFFFFu : ((1u << lim) - 1u);
      fz[j] = __popc(~held_bits[w] & valid);
    }
    fsum += fz[j];
  }
  int tot_free;
  int fp = block_excl_scan(fsum, scratch, &tot_free);
#pragma unroll
  for (int j = 0; j < kWordsPerThread; ++j) {
    free_pre[tid * kWordsPerThread + j] = fp;
    fp += fz[j];
  }
  if (tid == 0) free_pre[kChunkWords] = tot_free;
  __syncthreads();
  return tot_free;
}

// The r-th free slot (r < the free total), by binary search over the word prefixes.
__device__ int nth_free_slot(const uint32_t* held_bits, const int* free_pre, int capacity, int r) {
  int lo = 0, hi = (capacity + 31) / 32;  // free_pre[lo] <= r < free_pre[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (free_pre[mid] <= r) lo = mid;
    else hi = mid;
  }
  return lo * 32 + nth_zero_bit(held_bits[lo], r - free_pre[lo]);
}

// The same policy for sequences longer than the register path holds: the tokens' tiers and
// importance are read from memory on every pass (counts, each radix pass, the two index-order
// passes), and between the passes a resident row that still needs a slot is marked in loc
// itself (kNeedsSlot; every other value is a slot >= 0 or ~tok), so no workspace is needed.
// Each thread handles the same tokens in both passes.
__global__ __launch_bounds__(kThreads) void residency_chunked_kernel(
    const uint8_t* __restrict__ tier_all, int64_t tier_ld, const float* __restrict__ s_all,
    int64_t s_ld, int n, int capacity, uint32_t classes, int32_t* __restrict__ loc_all,
    int64_t loc_ld, int32_t* __restrict__ copy_tok, int32_t* __restrict__ copy_slot,
    int64_t copy_ld, int32_t* __restrict__ copy_count) {
  __shared__ __align__(16) uint32_t hist[4 * 256];
  __shared__ uint32_t held_bits[kChunkWords];
  __shared__ int free_pre[kChunkWords + 1];  // free slots before each bitmap word
  __shared__ int scratch[kWaves + 1];
  __shared__ int counts[2];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const uint8_t* tier = tier_all + (int64_t)b * tier_ld;
  const float* s = s_all + (int64_t)b * s_ld;
  int32_t* loc = loc_all + (int64_t)b * loc_ld;

  int c0 = 0, c1 = 0;
  for (int i = tid; i < n; i += kThreads) {
    const uint8_t t = tier_class(classes, tier[i]);
    c0 += t == 0;
    c1 += t == 1;
  }
  for (int i = tid; i < 4 * 256; i += kThreads) hist[i] = 0u;
  for (int i = tid; i < kChunkWords; i += kThreads) held_bits[i] = 0u;
  if (tid == 0) counts[0] = counts[1] = 0;
  __syncthreads();
  atomicAdd(&counts[0], c0);
  atomicAdd(&counts[1], c1);
  __syncthreads();
  const int n0 = counts[0], n1 = counts[1];

  const int cut_tier = capacity >= n0 + n1 ? -1 : (capacity >= n0 ? 1 : 0);
  const int cut = cut_tier == 1 ? capacity - n0 : (cut_tier == 0 ? capacity : 0);
  uint32_t thr = 0;
  int need = 0;
  bool whole = false;
  if (cut > 0) {
    radix_threshold(
        [&](auto visit) {
          for (int i = tid; i < n; i += kThreads)
            if (tier_class(classes, tier[i]) == cut_tier) visit(order_key(s[i]));
        },
        cut, hist, &thr, &need, &whole);
  }

  // Pass A, in index order: the resident set, the slots kept rows hold, loc of non-resident
  // rows, and the mark on resident rows that need a slot
  const int chunks = (n + kThreads - 1) / kThreads;
  int run_eq = 0;
  for (int c = 0; c < chunks; ++c) {
    const int i = c * kThreads + tid;
    const bool valid = i < n;
    const int t = valid ? tier_class(classes, tier[i]) : 3;
    const uint32_t key = valid ? order_key(s[i]) : 0u;
    const bool in_cut = t == cut_tier && cut_tier >= 0;
    const bool gt = in_cut && cut > 0 && (whole ? key >= thr : key > thr);
    const bool eq = in_cut && cut > 0 && !whole && key == thr;
    int tot_eq;
    const int pre = block_excl_scan(eq ? 1 : 0, scratch, &tot_eq);
    const bool kept_cut = gt || (eq && run_eq + pre < need);
    run_eq += tot_eq;
    bool res;
    if (cut_tier < 0) res = t <= 1;
    else if (cut_tier == 1) res = t == 0 || kept_cut;
    else res = kept_cut;
    if (valid) {
      const int old = loc[i];
      const bool held = res && old >= 0 && old < capacity;
      if (held) atomicOr(&held_bits[old >> 5], 1u << (old & 31));
      if (!res) loc[i] = ~i;
      else if (!held) loc[i] = kNeedsSlot;
    }
  }
  __syncthreads();
  const int tot_free = free_slot_prefix(held_bits, capacity, free_pre, scratch);

  // Pass B, in index order: the r-th marked row takes the r-th free slot
  int run = 0;
  for (int c = 0; c < chunks; ++c) {
    const int i = c * kThreads + tid;
    const bool f = i < n && loc[i] == kNeedsSlot;
    int tot;
    const int r = run + block_excl_scan(f ? 1 : 0, scratch, &tot);
    run += tot;
    if (f && r < tot_free) {
      const int slot = nth_free_slot(held_bits, free_pre, capacity, r);
      loc[i] = slot;
      if (r < copy_ld) {
        copy_tok[(int64_t)b * copy_ld + r] = i;
        copy_slot[(int64_t)b * copy_ld + r] = slot;
      }
    } else if (f) {
      loc[i] = ~i;  // no slot left (only when loc held a slot twice): read from host memory
    }
  }
  if (tid == 0) copy_count[b] = min(run, tot_free);  // the copies listed
}

// Rows a sequence gained since the last step, [n_old, n_new): the slots held by the rows below
// n_old (0 <= loc < capacity) are marked in an LDS bitmap, and the r-th new row, in token order,
// takes the r-th free slot (ascending), or stays in host memory (~tok) when none is left.
__global__ __launch_bounds__(kThreads) void residency_append_kernel(
    int32_t* __restrict__ loc_all, int64_t loc_ld, int n_old, int n_new, int capacity,
    int32_t* __restrict__ copy_tok, int32_t* __restrict__ copy_slot, int64_t copy_ld,
    int32_t* __restrict__ copy_count) {
  __shared__ uint32_t held_bits[kChunkWords];
  __shared__ int free_pre[kChunkWords + 1];
  __shared__ int scratch[kWaves + 1];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t* loc = loc_all + (int64_t)b * loc_ld;
  for (int i = tid; i < kChunkWords; i += kThreads) held_bits[i] = 0u;
  __syncthreads();
  for (int i0 = 0; i0 < n_old; i0 += kThreads * 8) {
    int x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // every load of the batch before the first use
      const int i = i0 + j * kThreads + tid;
      x[j] = i < n_old ? loc[i] : -1;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (x[j] >= 0 && x[j] < capacity) atomicOr(&held_bits[x[j] >> 5], 1u << (x[j] & 31));
  }
  __syncthreads();
  const int tot_free = free_slot_prefix(held_bits, capacity, free_pre, scratch);
  const int m = n_new - n_old;
  for (int r = tid; r < m; r += kThreads) {
    const int tok = n_old + r;
    if (r < tot_free) {
      const int slot = nth_free_slot(held_bits, free_pre, capacity, r);
      loc[tok] = slot;
      copy_tok[(int64_t)b * copy_ld + r] = tok;    // r < min(m, capacity) <= copy_ld
      copy_slot[(int64_t)b * copy_ld + r] = slot;
    } else {
      loc[tok] = ~tok;
    }
  }
  if (tid == 0) copy_count[b] = min(m, tot_free);
}

// Copy of newly resident rows: row copy_tok[b, r] of the host pools to slot copy_slot[b, r] of
// the HBM pools, for every KV head; D/8 lanes move one row of K or V with 16-byte accesses.
template <int D, typename KT>
__global__ __launch_bounds__(256) void prefetch_kernel(
    const KT* __restrict__ k_host, const KT* __restrict__ v_host, int64_t h_sb, int64_t h_sh,
    int64_t h_sn, int64_t host_slots, KT* __restrict__ k_hbm, KT* __restrict__ v_hbm,
    int64_t d_sb, int64_t d_sh, int64_t d_sn, int64_t hbm_slots,
    const int32_t* __restrict__ copy_tok, const int32_t* __restrict__ copy_slot, int64_t copy_ld,
    const int32_t* __restrict__ copy_count, int Hkv, int rows_per_wg) {
  constexpr int EPL = 16 / sizeof(KT);        // elements per lane and access
  constexpr int LPR = D / EPL;                // lanes per row
  constexpr int RPI = 256 / LPR;              // rows per workgroup and pass
  const int g = blockIdx.y, b = g / Hkv, kvh = g % Hkv;
  const int cnt = min((int64_t)copy_count[b], copy_ld);
  const int r0 = blockIdx.x * rows_per_wg;
  if (r0 >= cnt) return;
  const int r1 = min(r0 + rows_per_wg, cnt);
  const int sub = threadIdx.x % LPR;
  for (int r = r0 + (int)threadIdx.x / LPR; r < r1; r += RPI) {
    const int tok = copy_tok[(int64_t)b * copy_ld + r];
    const int slot = copy_slot[(int64_t)b * copy_ld + r];
    if (tok < 0 || tok >= host_slots || slot < 0 || slot >= hbm_slots) continue;
    const int64_t hs = (int64_t)b * h_sb + (int64_t)kvh * h_sh + (int64_t)tok * h_sn + sub * EPL;
    const int64_t ds = (int64_t)b * d_sb + (int64_t)kvh * d_sh + (int64_t)slot * d_sn + sub * EPL;
    const uint4 kx = *reinterpret_cast<const uint4*>(k_host + hs);
    const uint4 vx = *reinterpret_cast<const uint4*>(v_host + hs);
    *reinterpret_cast<uint4*>(k_hbm + ds) = kx;
    *reinterpret_cast<uint4*>(v_hbm + ds) = vx;
  }
}

// A source pool is page-locked, device-mapped host memory (read through the device address HIP
// reports for it) or device memory (rows produced on the GPU); anything else is refused.
spk_status source_device_ptr(const void* p, const void** dev, const char* name) {
  hipPointerAttribute_t at{};
  const hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return set_error(SPK_EINVAL, "residency_prefetch: %s is not memory known to HIP (%s)", name,
                     hipGetErrorString(e));
  }
  if (at.type == hipMemoryTypeDevice) {
    *dev = p;
    return SPK_OK;
  }
  if (at.type != hipMemoryTypeHost || at.devicePointer == nullptr)
    return set_error(SPK_EINVAL,
                     "residency_prefetch: %s must be device memory or pinned, device-mapped host "
                     "memory", name);
  *dev = static_cast<const char*>(at.devicePointer) +
         (static_cast<const char*>(p) - static_cast<const char*>(at.hostPointer));
  return SPK_OK;
}

}  // namespace
}  // namespace spk

extern "C" SPK_API spk_status residency_update_tiers(const uint8_t* tier, int64_t tier_ld,
                                                     const float* s, int64_t s_ld, int B,
                                                     int n_tokens, int capacity, int tier_classes,
                                                     int32_t* loc, int64_t loc_ld,
                                                     int32_t* copy_tok, int32_t* copy_slot,
                                                     int64_t copy_ld, int32_t* copy_count,
                                                     void* stream) {
  using namespace spk;
  SPK_REQUIRE(tier_classes >= 0 && tier_classes <= 0xFF, SPK_EINVAL,
              "residency_update: tier_classes 0x%x is not 2 bits per tier code", tier_classes);
  SPK_REQUIRE(B >= 0 && n_tokens >= 0 && capacity >= 0, SPK_EINVAL,
              "residency_update: negative size");
  SPK_REQUIRE(n_tokens < kMaxTokensChunked && capacity <= kChunkCap, SPK_EUNSUPPORTED,
              "residency_update: n_tokens %d / capacity %d: at most %d tokens and %d slots",
              n_tokens, capacity, kMaxTokensChunked - 1, kChunkCap);
  SPK_REQUIRE(B == 0 || (tier && s && loc && copy_count), SPK_EINVAL,
              "residency_update: null tier, s, loc or copy_count");
  SPK_REQUIRE(tier_ld >= n_tokens && s_ld >= n_tokens && loc_ld >= n_tokens, SPK_EINVAL,
              "residency_update: tier_ld / s_ld / loc_ld smaller than n_tokens");
  SPK_REQUIRE(copy_ld >= 0 && (copy_ld == 0 || (copy_tok && copy_slot)), SPK_EINVAL,
              "residency_update: null copy list with copy_ld > 0");
  clear_error();
  if (B == 0) return SPK_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (n_tokens <= kMaxTokens && capacity <= kMaxTokens)
    hipLaunchKernelGGL(residency_kernel, dim3(B), dim3(kThreads), 0, st, tier, tier_ld, s, s_ld,
                       n_tokens, capacity, (uint32_t)tier_classes, loc, loc_ld, copy_tok,
                       copy_slot, copy_ld, copy_count);
  else
    hipLaunchKernelGGL(residency_chunked_kernel, dim3(B), dim3(kThreads), 0, st, tier, tier_ld, s,
                       s_ld, n_tokens, capacity, (uint32_t)tier_classes, loc, loc_ld, copy_tok,
                       copy_slot, copy_ld, copy_count);
  return check_launch("residency_update");
}

extern "C" SPK_API spk_status residency_update(const uint8_t* tier, int64_t tier_ld,
                                               const float* s, int64_t s_ld, int B, int n_tokens,
                                               int capacity, int32_t* loc, int64_t loc_ld,
                                               int32_t* copy_tok, int32_t* copy_slot,
                                               int64_t copy_ld, int32_t* copy_count,
                                               void* stream) {
  // T0 ranks first, T1 second, T2 and T3 are never resident
  return residency_update_tiers(tier, tier_ld, s, s_ld, B, n_tokens, capacity, 0xF4, loc, loc_ld,
                                copy_tok, copy_slot, copy_ld, copy_count, stream);
}

extern "C" SPK_API spk_status residency_append(int32_t* loc, int64_t loc_ld, int B, int n_old,
                                               int n_new, int capacity, int32_t* copy_tok,
                                               int32_t* copy_slot, int64_t copy_ld,
                                               int32_t* copy_count, void* stream) {
  using namespace spk;
  SPK_REQUIRE(B >= 0 && n_old >= 0 && n_new >= n_old && capacity >= 0, SPK_EINVAL,
              "residency_append: need 0 <= n_old <= n_new, capacity >= 0");
  SPK_REQUIRE(capacity <= kChunkCap && n_new < kMaxTokensChunked, SPK_EUNSUPPORTED,
              "residency_append: capacity %d above %d or n_new %d too large", capacity,
              kChunkCap, n_new);
  SPK_REQUIRE(loc_ld >= n_new, SPK_EINVAL, "residency_append: loc_ld %lld < n_new %d",
              (long long)loc_ld, n_new);
  const int m = n_new - n_old;
  const int listed = m < capacity ? m : capacity;
  SPK_REQUIRE(copy_ld >= listed, SPK_EINVAL,
              "residency_append: copy_ld %lld < min(n_new - n_old, capacity) %d",
              (long long)copy_ld, listed);
  SPK_REQUIRE(B == 0 || (loc && copy_count && (listed == 0 || (copy_tok && copy_slot))),
              SPK_EINVAL, "residency_append: null loc, copy list or copy_count");
  clear_error();
  if (B == 0) return SPK_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(residency_append_kernel, dim3(B), dim3(kThreads), 0, st, loc, loc_ld, n_old,
                     n_new, capacity, copy_tok, copy_slot, copy_ld, copy_count);
  return check_launch("residency_append");
}

extern "C" SPK_API spk_status residency_prefetch(
    const void* k_host, const void* v_host, int64_t host_sb, int64_t host_sh, int64_t host_sn,
    int64_t host_slots, void* k_hbm, void* v_hbm, int64_t hbm_sb, int64_t hbm_sh, int64_t hbm_sn,
    int64_t hbm_slots, spk_dtype kv_dtype, int B, int Hkv, int d, const int32_t* copy_tok,
    const int32_t* copy_slot, int64_t copy_ld, const int32_t* copy_count, int max_copies,
    void* stream) {
  using namespace spk;
  SPK_REQUIRE(B >= 0 && Hkv > 0 && max_copies >= 0 && copy_ld >= 0, SPK_EINVAL,
              "residency_prefetch: negative size");
  SPK_REQUIRE(d == 64 || d == 128, SPK_EUNSUPPORTED, "residency_prefetch: d=%d not in {64,128}", d);
  SPK_REQUIRE(kv_dtype == SPK_BF16 || kv_dtype == SPK_F32, SPK_EUNSUPPORTED,
              "residency_prefetch: unsupported dtype");
  SPK_REQUIRE(B == 0 || max_copies == 0 ||
                  (k_host && v_host && k_hbm && v_hbm && copy_tok && copy_slot && copy_count),
              SPK_EINVAL, "residency_prefetch: null pointer");
  const int64_t align = kv_dtype == SPK_BF16 ? 8 : 4;  // elements in 16 bytes
  SPK_REQUIRE(host_sn >= d && hbm_sn >= d && host_sb >= 0 && host_sh >= 0 && hbm_sb >= 0 &&
                  hbm_sh >= 0 && host_sn % align == 0 && host_sh % align == 0 &&
                  host_sb % align == 0 && hbm_sn % align == 0 && hbm_sh % align == 0 &&
                  hbm_sb % align == 0,
              SPK_EINVAL, "residency_prefetch: row strides must cover d and keep 16-byte rows");
  SPK_REQUIRE(host_slots >= 0 && hbm_slots >= 0, SPK_EINVAL, "residency_prefetch: negative pool");
  clear_error();
  if (B == 0 || max_copies == 0) return SPK_OK;
  const void* kh = nullptr;
  const void* vh = nullptr;
  spk_status hs = source_device_ptr(k_host, &kh, "k_host");
  if (hs != SPK_OK) return hs;
  hs = source_device_ptr(v_host, &vh, "v_host");
  if (hs != SPK_OK) return hs;
  SPK_REQUIRE(reinterpret_cast<uintptr_t>(kh) % 16 == 0 && reinterpret_cast<uintptr_t>(vh) % 16 == 0 &&
                  reinterpret_cast<uintptr_t>(k_hbm) % 16 == 0 &&
                  reinterpret_cast<uintptr_t>(v_hbm) % 16 == 0,
              SPK_EINVAL, "residency_prefetch: pools must be 16-byte aligned");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int rows_per_wg = 64;
  const int mc = (int)(max_copies < copy_ld ? max_copies : copy_ld);
  if (mc == 0) return SPK_OK;
  dim3 grid((unsigned)((mc + rows_per_wg - 1) / rows_per_wg), (unsigned)(B * Hkv));
#define SPK_PF(DV, KT)                                                                          \
  hipLaunchKernelGGL((prefetch_kernel<DV, KT>), grid, dim3(256), 0, st,                         \
                     reinterpret_cast<const KT*>(kh), reinterpret_cast<const KT*>(vh), host_sb,    \
                     host_sh, host_sn, host_slots, reinterpret_cast<KT*>(k_hbm),                  \
                     reinterpret_cast<KT*>(v_hbm), hbm_sb, hbm_sh, hbm_sn, hbm_slots, copy_tok,    \
                     copy_slot, copy_ld, copy_count, Hkv, rows_per_wg)
  if (d == 128) {
    if (kv_dtype == SPK_BF16) SPK_PF(128, uint16_t);
    else SPK_PF(128, float);
  } else {
    if (kv_dtype == SPK_BF16) SPK_PF(64, uint16_t);
    else SPK_PF(64, float);
  }
#undef SPK_PF
  return check_launch("residency_prefetch");
}
