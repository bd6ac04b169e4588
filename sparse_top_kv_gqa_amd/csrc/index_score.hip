// sparse_index_score: compact indexer scores (no softmax) for token and block candidates.
//
// SparDA: Atenção Esparsa Desacoplada, §2 "Indexador de Previsão Compacto": one predictor head
// per GQA group (per KV head) scores the cached keys, with no per-query-head loop and no softmax;
// "Seleção Esparsa de Lookahead Treinável": the predictor ranks KV blocks.
// "Esparsidade de Contexto no Tempo de Inferência", §2 "Oracle Top-K": exact per-head scores.
//
// Work layout (HBM-bound streaming of key rows): a workgroup owns a run of candidate rows of one
// (b, kvh) group.  D/8 lanes share a row, each loading 16 B (8 bf16) or 32 B (8 fp32) of it, so a
// wave reads 4 (d=128) or 8 (d=64) rows per load instruction, fully coalesced.  Each lane keeps
// the 8-dim slice of every query vector the group scores (NS <= 16 of them) in registers, forms
// partial dots, and a 16-lane DPP reduction finishes them.  Scores are staged in LDS and written
// back as contiguous runs per output row.
#include <algorithm>
#include <type_traits>

#include "select_common.h"

namespace spk {
namespace {

#ifndef SPK_INDEX_UNROLL
#define SPK_INDEX_UNROLL 4        // key loads in flight per lane
#endif
#ifndef SPK_INDEX_MAX_ROWS
#define SPK_INDEX_MAX_ROWS 256    // candidate rows per workgroup of the block kernels
#endif
constexpr int kThreads = 256;
constexpr int kUnroll = SPK_INDEX_UNROLL;
#ifndef SPK_INDEX_UNROLL_PER_HEAD
#define SPK_INDEX_UNROLL_PER_HEAD 8   // key loads per lane in flight in per-head (dot2) scoring
#endif
constexpr int kUnrollPerHead = SPK_INDEX_UNROLL_PER_HEAD;

constexpr int kMaxRowsPerWg = SPK_INDEX_MAX_ROWS;
// Token scoring: a 16 KB LDS score tile, so a workgroup takes 4096 / NS rows (1024 for four
// score vectors) and writes each score row's part as one run of up to 4 KB: fewer, longer
// write runs than 1 KB ones interleave less with the key reads.
constexpr int kTileFloats = 4096;
constexpr int rows_cap(int ns_pad) { return kTileFloats / ns_pad; }

// Fetch 8 elements [off, off+8) of the query tensor as floats.
__device__ __forceinline__ void load_q8(const void* q, int q_bf16, int64_t off, float (&x)[8]) {
  if (q_bf16) {
    load8f(reinterpret_cast<const uint16_t*>(q) + off, x);
  } else {
    load8f(reinterpret_cast<const float*>(q) + off, x);
  }
}

// The 8-dim slice `sub` of query vector n of group (b, kvh), per indexer mode.
template <int D>
__device__ __forceinline__ void query_slice(int mode, const void* q, int q_bf16, int b, int kvh,
                                            int n, int T, int Hq, int Hkv, int G, int sub,
                                            float (&x)[8]) {
  if (mode == SPK_IDX_TOKEN_GROUP_MEAN) {
    // mean over the G heads of kvh at token t = n
    float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int hl = 0; hl < G; ++hl) {
      float y[8];
      load_q8(q, q_bf16, ((int64_t)(b * T + n) * Hq + kvh * G + hl) * D + sub * 8, y);
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] += y[i];
    }
    const float inv = 1.0f / (float)G;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = s[i] * inv;
  } else if (mode == SPK_IDX_TOKEN_PER_HEAD) {
    const int t = n / G, hl = n % G;
    load_q8(q, q_bf16, ((int64_t)(b * T + t) * Hq + kvh * G + hl) * D + sub * 8, x);
  } else {  // block modes: one predictor per (b, t, kvh)
    load_q8(q, q_bf16, ((int64_t)(b * T + n) * Hkv + kvh) * D + sub * 8, x);
  }
}

// Output row of score vector n of group (b, kvh).
__device__ __forceinline__ int64_t score_row(int mode, int b, int kvh, int n, int T, int Hq,
                                             int Hkv, int G) {
  if (mode == SPK_IDX_TOKEN_PER_HEAD) {
    const int t = n / G, hl = n % G;
    return (int64_t)(b * T + t) * Hq + kvh * G + hl;
  }
  return (int64_t)(b * T + n) * Hkv + kvh;
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Dot product of 8 bf16 keys (four packed pairs) with 8 bf16 query elements: four
// v_dot2c_f32_bf16, whose products of two bf16 values are exact in fp32.
__device__ __forceinline__ float dot8_bf16(const uint4& k, const uint32_t (&qp)[4]) {
  float a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.x),
                                            __builtin_bit_cast(bf16x2_t, qp[0]), 0.f, false);
  a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.y),
                                      __builtin_bit_cast(bf16x2_t, qp[1]), a, false);
  a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.z),
                                      __builtin_bit_cast(bf16x2_t, qp[2]), a, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.w),
                                         __builtin_bit_cast(bf16x2_t, qp[3]), a, false);
}

// DOT2: bf16 keys and bf16 query vectors used as they are (per-head token scores): the query
// slice stays packed and each key load feeds dot2 instructions instead of conversions and FMAs.
// U: key loads per lane in one batch (registers are held for two batches: the next one is
// issued before the current one is used).
template <int D, typename KT, int NS, bool DOT2 = false, int U = kUnroll>
__global__ __launch_bounds__(kThreads) void index_rows_kernel(
    int mode, const void* __restrict__ q, int q_bf16, const KT* __restrict__ keys, int64_t k_sb,
    int64_t k_sh, int64_t k_sn, int T, int Hq, int Hkv, int G, int ns, int n_cand,
    int rows_per_wg, float* __restrict__ scores, int64_t s_ld) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RPS = kWave / LPR;    // rows per wave per load
  constexpr int WAVES = kThreads / kWave;
  constexpr int STEP = WAVES * RPS;   // rows per workgroup per load
  __shared__ float tile[NS][rows_cap(NS)];

  const int group = blockIdx.y;
  const int b = group / Hkv, kvh = group % Hkv;
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  const int sub = lane % LPR, slot = lane / LPR;
  const int row0 = blockIdx.x * rows_per_wg;
  const int row1 = min(row0 + rows_per_wg, n_cand);
  if (row0 >= n_cand) return;

  static_assert(!DOT2 || std::is_same<KT, uint16_t>::value, "the dot2 path takes bf16 keys");
  const KT* base_ptr = keys + (int64_t)b * k_sb + (int64_t)kvh * k_sh + sub * 8;
  // The first batch of key loads goes out before the query slices are fetched, and every later
  // batch before the previous one is used, so the workgroup always has key bytes in flight.
  Raw8<KT> raw[U];
  auto issue = [&](Raw8<KT> (&dst)[U], int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = base + (u * WAVES + wid) * RPS + slot;
      dst[u].load_nt(base_ptr + (int64_t)min(row, row1 - 1) * k_sn);  // past the end: re-read, unused
    }
  };
  issue(raw, row0);
  float qv[DOT2 ? 1 : NS][8];
  uint32_t qp[DOT2 ? NS : 1][4];
  if constexpr (DOT2) {
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      // per-head: score vector n is head n % G of token n / G (vectors past ns load the last
      // one and are zeroed: no branch around the loads)
      const int nn = min(n, ns - 1);
      const int t = nn / G, hl = nn % G;
      uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(q) +
                                                ((int64_t)(b * T + t) * Hq + kvh * G + hl) * D +
                                                sub * 8);
      const bool keep = n < ns;
      qp[n][0] = keep ? u.x : 0u;
      qp[n][1] = keep ? u.y : 0u;
      qp[n][2] = keep ? u.z : 0u;
      qp[n][3] = keep ? u.w : 0u;
    }
  } else {
    // the query slices fetched once per workgroup (a group-mean vector sums G head slices): the
    // first row slot of wave w builds vectors w, w + 4, ... into LDS and every lane reads its
    // slice back after one barrier, instead of every row slot issuing the same loads
    __shared__ uint4 qsh[NS][2 * LPR];
    if (slot == 0) {
      for (int n = wid; n < NS; n += WAVES) {
        float x[8];
        if (n < ns) {
          query_slice<D>(mode, q, q_bf16, b, kvh, n, T, Hq, Hkv, G, sub, x);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = 0.f;
        }
        qsh[n][2 * sub] = make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]),
                                     __float_as_uint(x[2]), __float_as_uint(x[3]));
        qsh[n][2 * sub + 1] = make_uint4(__float_as_uint(x[4]), __float_as_uint(x[5]),
                                         __float_as_uint(x[6]), __float_as_uint(x[7]));
      }
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      const uint4 a0 = qsh[n][2 * sub], a1 = qsh[n][2 * sub + 1];
      qv[n][0] = __uint_as_float(a0.x);
      qv[n][1] = __uint_as_float(a0.y);
      qv[n][2] = __uint_as_float(a0.z);
      qv[n][3] = __uint_as_float(a0.w);
      qv[n][4] = __uint_as_float(a1.x);
      qv[n][5] = __uint_as_float(a1.y);
      qv[n][6] = __uint_as_float(a1.z);
      qv[n][7] = __uint_as_float(a1.w);
    }
  }

  for (int base = row0; base < row1; base += STEP * U) {
    Raw8<KT> nxt[U];
    const bool more = base + STEP * U < row1;   // uniform over the workgroup
    if (more) issue(nxt, base + STEP * U);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = base + (u * WAVES + wid) * RPS + slot;
      float acc[NS];
      if constexpr (DOT2) {
#pragma unroll
        for (int n = 0; n < NS; ++n) acc[n] = group_sum<LPR>(dot8_bf16(raw[u].u, qp[n]));
      } else {
        float x[8];
        raw[u].to_float(x);
#pragma unroll
        for (int n = 0; n < NS; ++n) {
          float a = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) a = fmaf(qv[n][i], x[i], a);
          acc[n] = group_sum<LPR>(a);
        }
      }
      if (row < row1) {
#pragma unroll
        for (int n = 0; n < NS; ++n)
          if (n % LPR == sub && n < ns) tile[n][row - row0] = acc[n];
      }
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) raw[u] = nxt[u];
    }
  }
  __syncthreads();
  const int cnt = row1 - row0;
  for (int i = threadIdx.x; i < ns * cnt; i += kThreads) {
    const int n = i / cnt, r = i % cnt;
    // streamed out: the scores are read once, by the selection that follows
    __builtin_nontemporal_store(tile[n][r],
                                scores + score_row(mode, b, kvh, n, T, Hq, Hkv, G) * s_ld + row0 + r);
  }
}

// Block mode over raw keys: each 16-lane slot pools one block (mean of block_size rows), scores
// it against the predictor(s) and optionally stores the pooled key.
template <int D, typename KT, int NS>
__global__ __launch_bounds__(kThreads) void index_blockraw_kernel(
    const void* __restrict__ q, int q_bf16, const KT* __restrict__ keys, int64_t k_sb,
    int64_t k_sh, int64_t k_sn, int T, int Hkv, int ns, int n_blocks, int bs,
    int blocks_per_wg, float* __restrict__ scores, int64_t s_ld, float* __restrict__ pooled) {
  constexpr int LPR = D / 8;
  constexpr int RPS = kWave / LPR;
  constexpr int WAVES = kThreads / kWave;
  constexpr int STEP = WAVES * RPS;
  __shared__ float tile[NS][kMaxRowsPerWg];

  const int group = blockIdx.y;
  const int b = group / Hkv, kvh = group % Hkv;
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  const int sub = lane % LPR, slot = lane / LPR;
  const int j0 = blockIdx.x * blocks_per_wg;
  const int j1 = min(j0 + blocks_per_wg, n_blocks);
  if (j0 >= n_blocks) return;

  float qv[NS][8];
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    if (n < ns) {
      query_slice<D>(SPK_IDX_BLOCK_RAW, q, q_bf16, b, kvh, n, T, 0, Hkv, 1, sub, qv[n]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[n][i] = 0.f;
    }
  }
  const KT* gbase = keys + (int64_t)b * k_sb + (int64_t)kvh * k_sh + sub * 8;
  for (int jb = j0; jb < j1; jb += STEP) {
    const int j = jb + wid * RPS + slot;
    const bool live = j < j1;
    float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (live) {
      const KT* p = gbase + (int64_t)j * bs * k_sn;
      int r = 0;
      for (; r + kUnroll <= bs; r += kUnroll) {
        Raw8<KT> raw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) raw[u].load(p + (int64_t)(r + u) * k_sn);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          float x[8];
          raw[u].to_float(x);
#pragma unroll
          for (int i = 0; i < 8; ++i) s[i] += x[i];
        }
      }
      for (; r < bs; ++r) {
        float x[8];
        load8f(p + (int64_t)r * k_sn, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] += x[i];
      }
    }
    float mean[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) mean[i] = s[i] / (float)bs;
    if (live && pooled) {
      float* dst = pooled + ((int64_t)group * n_blocks + j) * D + sub * 8;
      *reinterpret_cast<float4*>(dst) = make_float4(mean[0], mean[1], mean[2], mean[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(mean[4], mean[5], mean[6], mean[7]);
    }
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaf(qv[n][i], mean[i], a);
      a = group_sum<LPR>(a);
      if (live && n % LPR == sub && n < ns) tile[n][j - j0] = a;
    }
  }
  __syncthreads();
  const int cnt = j1 - j0;
  for (int i = threadIdx.x; i < ns * cnt; i += kThreads) {
    const int n = i / cnt, r = i % cnt;
    scores[((int64_t)(b * T + n) * Hkv + kvh) * s_ld + j0 + r] = tile[n][r];
  }
}

template <int D, typename KT>
spk_status launch_rows(int ns_pad, dim3 grid, hipStream_t st, int mode, const void* q, int q_bf16,
                       const void* keys, int64_t k_sb, int64_t k_sh, int64_t k_sn, int T, int Hq,
                       int Hkv, int G, int ns, int n_cand, int rpw, float* scores, int64_t s_ld) {
  const KT* kp = reinterpret_cast<const KT*>(keys);
  // bf16 keys scored against bf16 query heads as they are: the dot2 path
  const bool dot2 = std::is_same<KT, uint16_t>::value && q_bf16 && mode == SPK_IDX_TOKEN_PER_HEAD;
#define SPK_ROWS(NSV, DT)                                                                     \
  hipLaunchKernelGGL((index_rows_kernel<D, KT, NSV, DT, DT ? kUnrollPerHead : kUnroll>),        \
                     grid, dim3(kThreads), 0, st, mode, q, q_bf16, kp, k_sb, k_sh, k_sn, T, Hq, \
                     Hkv, G, ns, n_cand, rpw, scores, s_ld)
  if constexpr (std::is_same<KT, uint16_t>::value) {
    if (dot2) {
      switch (ns_pad) {
        case 1: SPK_ROWS(1, true); break;
        case 4: SPK_ROWS(4, true); break;
        case 8: SPK_ROWS(8, true); break;
        default: SPK_ROWS(16, true); break;
      }
      return check_launch("sparse_index_score");
    }
  }
  {
    switch (ns_pad) {
      case 1: SPK_ROWS(1, false); break;
      case 4: SPK_ROWS(4, false); break;
      case 8: SPK_ROWS(8, false); break;
      default: SPK_ROWS(16, false); break;
    }
  }
#undef SPK_ROWS
  return check_launch("sparse_index_score");
}

template <int D, typename KT>
spk_status launch_blockraw(int ns_pad, dim3 grid, hipStream_t st, const void* q, int q_bf16,
                           const void* keys, int64_t k_sb, int64_t k_sh, int64_t k_sn, int T,
                           int Hkv, int ns, int n_blocks, int bs, int bpw, float* scores,
                           int64_t s_ld, float* pooled) {
  const KT* kp = reinterpret_cast<const KT*>(keys);
#define SPK_RAW(NSV)                                                                           \
  hipLaunchKernelGGL((index_blockraw_kernel<D, KT, NSV>), grid, dim3(kThreads), 0, st, q,     \
                     q_bf16, kp, k_sb, k_sh, k_sn, T, Hkv, ns, n_blocks, bs, bpw, scores, s_ld, \
                     pooled)
  switch (ns_pad) {
    case 1: SPK_RAW(1); break;
    case 4: SPK_RAW(4); break;
    case 8: SPK_RAW(8); break;
    default: SPK_RAW(16); break;
  }
#undef SPK_RAW
  return check_launch("sparse_index_score");
}

int pad_ns(int ns) { return ns <= 1 ? 1 : ns <= 4 ? 4 : ns <= 8 ? 8 : 16; }

// ---------------------------------------------------------------- overlapping compression windows
//
// SparDA, "Estratégia de Treinamento": the inference grid compresses the keys with overlapping
// windows (kernel 32, stride 16), and window scores are max-pooled onto another grid.  Window w
// covers tokens [stride*w, stride*w + window) (complete windows only); block j covers
// [bs*j, bs*j + bs) and takes the largest score of the windows that share a token with it.

// Windows overlapping block j: [first, last] (empty when first > last or last < 0).
__host__ __device__ inline int win_first(int j, int bs, int window, int stride) {
  const int64_t t = (int64_t)bs * j - window;  // w must satisfy stride*w > t
  return t < 0 ? 0 : (int)(t / stride + 1);
}
__host__ __device__ inline int win_last(int j, int bs, int stride, int nw) {
  const int64_t w = ((int64_t)bs * (j + 1) - 1) / stride;
  return (int)(w < nw - 1 ? w : nw - 1);
}

constexpr int kWinTile = 1024;  // window scores of one workgroup held in LDS (per score vector)

// Pooling: each D/8-lane slot sums one window's rows (8 dims per lane) and stores the mean.
template <int D, typename KT>
__global__ __launch_bounds__(kThreads) void window_pool_kernel(
    const KT* __restrict__ keys, int64_t k_sb, int64_t k_sh, int64_t k_sn, int Hkv, int nw,
    int window, int stride, int wpw, float* __restrict__ kwin, int64_t w_cap) {
  constexpr int LPR = D / 8;
  constexpr int RPS = kWave / LPR;
  constexpr int STEP = (kThreads / kWave) * RPS;
  const int group = blockIdx.y;
  const int b = group / Hkv, kvh = group % Hkv;
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  const int sub = lane % LPR, slot = lane / LPR;
  const int w0 = blockIdx.x * wpw, w1 = min(w0 + wpw, nw);
  const KT* gbase = keys + (int64_t)b * k_sb + (int64_t)kvh * k_sh + sub * 8;
  const float inv = 1.0f / (float)window;
  for (int wb = w0; wb < w1; wb += STEP) {
    const int w = wb + wid * RPS + slot;
    if (w >= w1) continue;
    const KT* p = gbase + (int64_t)w * stride * k_sn;
    float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int r = 0;
    for (; r + kUnroll <= window; r += kUnroll) {
      Raw8<KT> raw[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) raw[u].load(p + (int64_t)(r + u) * k_sn);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float x[8];
        raw[u].to_float(x);
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] += x[i];
      }
    }
    for (; r < window; ++r) {
      float x[8];
      load8f(p + (int64_t)r * k_sn, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] += x[i];
    }
    float* dst = kwin + ((int64_t)group * w_cap + w) * D + sub * 8;
    *reinterpret_cast<float4*>(dst) = make_float4(s[0] * inv, s[1] * inv, s[2] * inv, s[3] * inv);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(s[4] * inv, s[5] * inv, s[6] * inv, s[7] * inv);
  }
}

// Scoring: a workgroup owns blocks [j0, j1) of one group, scores every window overlapping them
// (fp32 window keys streamed once, all of a pass's loads in flight) into LDS, then writes each
// block's maximum.
template <int D, int NS>
__global__ __launch_bounds__(kThreads) void index_windowed_kernel(
    const void* __restrict__ q, int q_bf16, const float* __restrict__ kwin, int64_t w_cap, int T,
    int Hkv, int ns, int nw, int nb, int window, int stride, int bs, int bpw,
    float* __restrict__ scores, int64_t s_ld) {
  constexpr int LPR = D / 8;
  constexpr int RPS = kWave / LPR;
  constexpr int WAVES = kThreads / kWave;
  constexpr int STEP = WAVES * RPS;
  __shared__ float tile[NS][kWinTile];
  const int group = blockIdx.y;
  const int b = group / Hkv, kvh = group % Hkv;
  const int lane = lane_id(), wid = threadIdx.x / kWave;
  const int sub = lane % LPR, slot = lane / LPR;
  const int j0 = blockIdx.x * bpw, j1 = min(j0 + bpw, nb);
  if (j0 >= nb) return;
  const int W0 = win_first(j0, bs, window, stride);
  const int W1 = win_last(j1 - 1, bs, stride, nw);  // W1 - W0 + 1 <= kWinTile (host sizing)

  float qv[NS][8];
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    if (n < ns) {
      query_slice<D>(SPK_IDX_BLOCK_POOLED, q, q_bf16, b, kvh, n, T, 0, Hkv, 1, sub, qv[n]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[n][i] = 0.f;
    }
  }
  const float* base_ptr = kwin + (int64_t)group * w_cap * D + sub * 8;
  for (int base = W0; base <= W1; base += STEP * kUnroll) {
    Raw8<float> raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int w = base + (u * WAVES + wid) * RPS + slot;
      if (w <= W1) raw[u].load(base_ptr + (int64_t)w * D);
      else raw[u].zero();
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int w = base + (u * WAVES + wid) * RPS + slot;
      float x[8];
      raw[u].to_float(x);
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fmaf(qv[n][i], x[i], a);
        a = group_sum<LPR>(a);
        if (w <= W1 && n % LPR == sub && n < ns) tile[n][w - W0] = a;
      }
    }
  }
  __syncthreads();
  const int cnt = j1 - j0;
  for (int i = threadIdx.x; i < ns * cnt; i += kThreads) {
    const int n = i / cnt, j = j0 + i % cnt;
    const int lo = win_first(j, bs, window, stride), hi = win_last(j, bs, stride, nw);
    float m = -INFINITY;
    for (int w = lo; w <= hi; ++w) m = fmaxf(m, tile[n][w - W0]);
    scores[((int64_t)(b * T + n) * Hkv + kvh) * s_ld + j] = m;
  }
}

// Blocks per workgroup for the windowed scorer: about four workgroups per CU, and the windows
// of a workgroup's blocks fit the LDS tile.
int pick_blocks_per_wg(int nb, int groups, int bs, int window, int stride) {
  int bpw = 64;
  while (bpw > 4 && (int64_t)groups * ceil_div(nb, bpw) < 4LL * num_cus()) bpw /= 2;
  while (bpw > 1 && ((int64_t)bpw * bs + window) / stride + 2 > kWinTile) bpw /= 2;
  return bpw;
}

// ---------------------------------------------------------------- scores + top-k in one launch
//
// For short candidate rows (a block indexer's few hundred blocks, or a few thousand tokens) the
// top-k of a row is worth less than a launch of its own.  One 1024-thread workgroup per (b, kvh)
// group streams the group's candidate keys once (all of a pass's loads in flight), keeps every
// score of its score vectors in LDS, then selects each vector's top-k there with the same radix
// select and index-ordered compaction as topk_select.
constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / kWave;
constexpr int kFusedMaxCand = 8192;    // candidates per score row
constexpr int kFusedLds = 16384;       // score vectors x candidates held in LDS
constexpr int kFusedItems = kFusedMaxCand / kFusedThreads;
constexpr int kFusedMaxVectors = 4;    // score vectors per (b, kvh) group

template <int D, typename KT, int NS>
__global__ __launch_bounds__(kFusedThreads) void index_topk_kernel(
    int mode, const void* __restrict__ q, int q_bf16, const KT* __restrict__ keys, int64_t k_sb,
    int64_t k_sh, int64_t k_sn, int T, int Hq, int Hkv, int G, int ns, int n_cand, int k,
    float* __restrict__ scores, int64_t s_ld, int32_t* __restrict__ idx, int64_t idx_ld,
    int32_t* __restrict__ count) {
  constexpr int LPR = D / 8;          // lanes per key row
  constexpr int RPS = kWave / LPR;    // rows per wave per load
  constexpr int STEP = kFusedWaves * RPS;
  constexpr int U = 8;                // loads in flight per lane
  __shared__ float tile[kFusedLds];   // [ns][n_cand]
  __shared__ uint32_t hist[kFusedWaves * 256];
  __shared__ int sh[2];
  __shared__ int wcnt[kFusedItems][kFusedWaves][2];

  const int group = blockIdx.x;
  const int b = group / Hkv, kvh = group % Hkv;
  const int t = threadIdx.x, lane = lane_id(), wid = t / kWave;
  const int sub = lane % LPR, slot = lane / LPR;

  float qv[NS][8];
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    if (n < ns) {
      query_slice<D>(mode, q, q_bf16, b, kvh, n, T, Hq, Hkv, G, sub, qv[n]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[n][i] = 0.f;
    }
  }
  const KT* base_ptr = keys + (int64_t)b * k_sb + (int64_t)kvh * k_sh + sub * 8;
  for (int base = 0; base < n_cand; base += STEP * U) {
    Raw8<KT> raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = base + (u * kFusedWaves + wid) * RPS + slot;
      if (row < n_cand) raw[u].load(base_ptr + (int64_t)row * k_sn);
      else raw[u].zero();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = base + (u * kFusedWaves + wid) * RPS + slot;
      float x[8];
      raw[u].to_float(x);
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fmaf(qv[n][i], x[i], a);
        a = group_sum<LPR>(a);
        if (row < n_cand && n < ns && n % LPR == sub) tile[n * n_cand + row] = a;
      }
    }
  }
  __syncthreads();
  if (scores) {
    for (int i = t; i < ns * n_cand; i += kFusedThreads) {
      const int n = i / n_cand, j = i % n_cand;
      scores[score_row(mode, b, kvh, n, T, Hq, Hkv, G) * s_ld + j] = tile[i];
    }
  }
  const int kk = min(k, n_cand);
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int n = 0; n < ns; ++n) {
    const int64_t orow = score_row(mode, b, kvh, n, T, Hq, Hkv, G);
    if (count && t == 0) count[orow] = kk;
    if (kk <= 0) continue;
    uint32_t key[kFusedItems];
#pragma unroll
    for (int c = 0; c < kFusedItems; ++c) {
      const int j = c * kFusedThreads + t;
      key[c] = j < n_cand ? order_key(tile[n * n_cand + j]) : 0u;
    }
    uint32_t thr;
    int need;
    radix_select<kFusedThreads>(
        [&](auto visit) {
#pragma unroll
          for (int c = 0; c < kFusedItems; ++c)
            if (c * kFusedThreads + t < n_cand) visit(key[c]);
        },
        kk, hist, sh, &thr, &need);
    // keep every key above thr and the first `need` keys equal to it, in index order
    uint64_t bg[kFusedItems], be[kFusedItems];
#pragma unroll
    for (int c = 0; c < kFusedItems; ++c) {
      const bool valid = c * kFusedThreads + t < n_cand;
      bg[c] = __ballot(valid && key[c] > thr);
      be[c] = __ballot(valid && key[c] == thr);
      if (lane == 0) {
        wcnt[c][wid][0] = __popcll(bg[c]);
        wcnt[c][wid][1] = __popcll(be[c]);
      }
    }
    __syncthreads();
    int32_t* out = idx + orow * idx_ld;
    int run_g = 0, run_e = 0;
#pragma unroll
    for (int c = 0; c < kFusedItems; ++c) {
      if (c * kFusedThreads >= n_cand) break;
      int pre_g = run_g + __popcll(bg[c] & lt), pre_e = run_e + __popcll(be[c] & lt);
      int tot_g = 0, tot_e = 0;
      for (int w = 0; w < kFusedWaves; ++w) {
        const int cg = wcnt[c][w][0], ce = wcnt[c][w][1];
        if (w < wid) {
          pre_g += cg;
          pre_e += ce;
        }
        tot_g += cg;
        tot_e += ce;
      }
      const int j = c * kFusedThreads + t;
      const bool gt = (bg[c] >> lane) & 1ull, eq = (be[c] >> lane) & 1ull;
      if (gt || (eq && pre_e < need)) out[pre_g + min(pre_e, need)] = j;
      run_g += tot_g;
      run_e += tot_e;
    }
    __syncthreads();  // wcnt and hist are reused by the next score vector
  }
}

template <int D, typename KT>
spk_status launch_fused(int ns_pad, int groups, hipStream_t st, int mode, const void* q,
                        int q_bf16, const void* keys, int64_t k_sb, int64_t k_sh, int64_t k_sn,
                        int T, int Hq, int Hkv, int G, int ns, int n_cand, int k, float* scores,
                        int64_t s_ld, int32_t* idx, int64_t idx_ld, int32_t* count) {
  const KT* kp = reinterpret_cast<const KT*>(keys);
#define SPK_FUSED(NSV)                                                                          \
  hipLaunchKernelGGL((index_topk_kernel<D, KT, NSV>), dim3(groups), dim3(kFusedThreads), 0, st, \
                     mode, q, q_bf16, kp, k_sb, k_sh, k_sn, T, Hq, Hkv, G, ns, n_cand, k, scores,  \
                     s_ld, idx, idx_ld, count)
  if (ns_pad == 1) SPK_FUSED(1);
  else SPK_FUSED(4);
#undef SPK_FUSED
  return check_launch("sparse_index_topk");
}

// Rows per workgroup: max_rows, halved (not below `step`) while the launch would have fewer than
// four workgroups per CU.
int pick_rows_per_wg(int64_t rows_total, int step, int max_rows = kMaxRowsPerWg) {
  const int64_t target_wgs = 4LL * num_cus();
  int rpw = max_rows;
  while (rpw > step && rows_total / rpw < target_wgs) rpw /= 2;
  return rpw;
}

}  // namespace
}  // namespace spk

extern "C" SPK_API spk_status sparse_index_score(spk_index_mode mode, const void* q,
                                                 spk_dtype q_dtype, const void* keys,
                                                 spk_dtype k_dtype, int64_t k_sb, int64_t k_sh,
                                                 int64_t k_sn, int B, int T, int Hq, int Hkv,
                                                 int d, int n_tokens, int block_size,
                                                 float* scores, int64_t s_ld, float* pooled_out,
                                                 void* stream) {
  using namespace spk;
  SPK_REQUIRE(mode >= SPK_IDX_TOKEN_GROUP_MEAN && mode <= SPK_IDX_BLOCK_RAW, SPK_EINVAL,
              "sparse_index_score: unknown mode %d", (int)mode);
  SPK_REQUIRE(q && keys && scores, SPK_EINVAL, "sparse_index_score: null q, keys or scores");
  SPK_REQUIRE(B > 0 && T > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0, SPK_EINVAL,
              "sparse_index_score: bad heads/batch B=%d T=%d Hq=%d Hkv=%d", B, T, Hq, Hkv);
  SPK_REQUIRE(dtype_ok(q_dtype) && dtype_ok(k_dtype), SPK_EUNSUPPORTED,
              "sparse_index_score: unsupported dtype");
  SPK_REQUIRE(d == 64 || d == 128, SPK_EUNSUPPORTED, "sparse_index_score: d=%d not in {64,128}", d);
  SPK_REQUIRE(n_tokens >= 0, SPK_EINVAL, "sparse_index_score: n_tokens < 0");
  const bool block = mode == SPK_IDX_BLOCK_POOLED || mode == SPK_IDX_BLOCK_RAW;
  SPK_REQUIRE(!block || block_size >= 1, SPK_EINVAL, "sparse_index_score: block_size < 1");
  SPK_REQUIRE(pooled_out == nullptr || mode == SPK_IDX_BLOCK_RAW, SPK_EINVAL,
              "sparse_index_score: pooled_out is only written in BLOCK_RAW mode");
  SPK_REQUIRE(k_sn >= d && k_sb >= 0 && k_sh >= 0 && k_sn % 8 == 0 && k_sh % 8 == 0 && k_sb % 8 == 0,
              SPK_EINVAL, "sparse_index_score: key strides must be multiples of 8 with k_sn >= d");
  SPK_REQUIRE(reinterpret_cast<uintptr_t>(keys) % 16 == 0 && reinterpret_cast<uintptr_t>(q) % 16 == 0,
              SPK_EINVAL, "sparse_index_score: q and keys must be 16-byte aligned");
  const int G = Hq / Hkv;
  const int ns = mode == SPK_IDX_TOKEN_PER_HEAD ? T * G : T;
  SPK_REQUIRE(ns <= 16, SPK_EUNSUPPORTED,
              "sparse_index_score: %d score vectors per KV head (max 16)", ns);
  const int n_cand = block ? n_tokens / block_size : n_tokens;
  SPK_REQUIRE(s_ld >= n_cand, SPK_EINVAL, "sparse_index_score: s_ld %lld < candidates %d",
              (long long)s_ld, n_cand);
  clear_error();
  if (n_cand == 0) return SPK_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int q_bf16 = q_dtype == SPK_BF16;
  const int ns_pad = pad_ns(ns);
  const int groups = B * Hkv;
  const int step = 4 * (64 / (d / 8));
  if (mode == SPK_IDX_BLOCK_RAW) {
    const int bpw = pick_rows_per_wg((int64_t)n_cand * groups, step);
    dim3 grid(ceil_div(n_cand, bpw), groups);
    if (d == 128)
      return k_dtype == SPK_BF16
                 ? launch_blockraw<128, uint16_t>(ns_pad, grid, st, q, q_bf16, keys, k_sb, k_sh, k_sn, T,
                                                  Hkv, ns, n_cand, block_size, bpw, scores, s_ld, pooled_out)
                 : launch_blockraw<128, float>(ns_pad, grid, st, q, q_bf16, keys, k_sb, k_sh, k_sn, T,
                                               Hkv, ns, n_cand, block_size, bpw, scores, s_ld, pooled_out);
    return k_dtype == SPK_BF16
               ? launch_blockraw<64, uint16_t>(ns_pad, grid, st, q, q_bf16, keys, k_sb, k_sh, k_sn, T,
                                               Hkv, ns, n_cand, block_size, bpw, scores, s_ld, pooled_out)
               : launch_blockraw<64, float>(ns_pad, grid, st, q, q_bf16, keys, k_sb, k_sh, k_sn, T,
                                            Hkv, ns, n_cand, block_size, bpw, scores, s_ld, pooled_out);
  }
  // Rows per workgroup: per-head scoring loads one query slice per score vector and prefers
  // many small workgroups, one batch of key loads each: on the per-head 131072-token workload
  // 128 rows at d = 128 with eight nontemporal loads per lane take 173-177 us, against 182-186
  // at 64 rows with four, 190 at 256 rows with sixteen, and 180-195 for the same 128-row batch
  // at 8 or at 4-7 workgroups per CU (the registers for two batches hold it at five); the
  // group mean builds its vectors once per workgroup in LDS and does best at 256 rows (416 us,
  // against 441 at 1024 and 551 at 64 on the speculative-verify workload); block scores take
  // the whole tile, halved until the launch fills the chip.
  const bool dot2 = k_dtype == SPK_BF16 && q_bf16 && mode == SPK_IDX_TOKEN_PER_HEAD;
  const int batch = step * (dot2 ? kUnrollPerHead : kUnroll);
  const int max_rows = mode == SPK_IDX_TOKEN_PER_HEAD   ? std::min(batch, rows_cap(ns_pad))
                       : mode == SPK_IDX_TOKEN_GROUP_MEAN ? std::min(256, rows_cap(ns_pad))
                                                          : rows_cap(ns_pad);
  const int rpw = pick_rows_per_wg((int64_t)n_cand * groups, std::min(batch, max_rows), max_rows);
  // the score tile holds rows_cap(ns_pad) rows of every vector
  SPK_REQUIRE(rpw >= 1 && rpw <= rows_cap(ns_pad), SPK_EINVAL,
              "sparse_index_score: internal: %d rows per workgroup exceed the tile", rpw);
  dim3 grid(ceil_div(n_cand, rpw), groups);
  if (d == 128)
    return k_dtype == SPK_BF16
               ? launch_rows<128, uint16_t>(ns_pad, grid, st, mode, q, q_bf16, keys, k_sb, k_sh, k_sn, T,
                                            Hq, Hkv, G, ns, n_cand, rpw, scores, s_ld)
               : launch_rows<128, float>(ns_pad, grid, st, mode, q, q_bf16, keys, k_sb, k_sh, k_sn, T, Hq,
                                         Hkv, G, ns, n_cand, rpw, scores, s_ld);
  return k_dtype == SPK_BF16
             ? launch_rows<64, uint16_t>(ns_pad, grid, st, mode, q, q_bf16, keys, k_sb, k_sh, k_sn, T, Hq,
                                         Hkv, G, ns, n_cand, rpw, scores, s_ld)
             : launch_rows<64, float>(ns_pad, grid, st, mode, q, q_bf16, keys, k_sb, k_sh, k_sn, T, Hq,
                                      Hkv, G, ns, n_cand, rpw, scores, s_ld);
}

extern "C" SPK_API spk_status sparse_index_topk(spk_index_mode mode, const void* q,
                                                spk_dtype q_dtype, const void* keys,
                                                spk_dtype k_dtype, int64_t k_sb, int64_t k_sh,
                                                int64_t k_sn, int B, int T, int Hq, int Hkv,
                                                int d, int n_tokens, int block_size, int k,
                                                float* scores, int64_t s_ld, int32_t* idx,
                                                int64_t idx_ld, int32_t* count, void* stream) {
  using namespace spk;
  SPK_REQUIRE(mode >= SPK_IDX_TOKEN_GROUP_MEAN && mode <= SPK_IDX_BLOCK_RAW, SPK_EINVAL,
              "sparse_index_topk: unknown mode %d", (int)mode);
  SPK_REQUIRE(mode != SPK_IDX_BLOCK_RAW, SPK_EUNSUPPORTED,
              "sparse_index_topk: BLOCK_RAW is not fused (pool the keys first)");
  SPK_REQUIRE(q && keys, SPK_EINVAL, "sparse_index_topk: null q or keys");
  SPK_REQUIRE(B > 0 && T > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0, SPK_EINVAL,
              "sparse_index_topk: bad heads/batch B=%d T=%d Hq=%d Hkv=%d", B, T, Hq, Hkv);
  SPK_REQUIRE(dtype_ok(q_dtype) && dtype_ok(k_dtype), SPK_EUNSUPPORTED,
              "sparse_index_topk: unsupported dtype");
  SPK_REQUIRE(d == 64 || d == 128, SPK_EUNSUPPORTED, "sparse_index_topk: d=%d not in {64,128}", d);
  SPK_REQUIRE(n_tokens >= 0 && k >= 0, SPK_EINVAL, "sparse_index_topk: n_tokens or k < 0");
  const bool block = mode == SPK_IDX_BLOCK_POOLED;
  SPK_REQUIRE(!block || block_size >= 1, SPK_EINVAL, "sparse_index_topk: block_size < 1");
  SPK_REQUIRE(k_sn >= d && k_sb >= 0 && k_sh >= 0 && k_sn % 8 == 0 && k_sh % 8 == 0 && k_sb % 8 == 0,
              SPK_EINVAL, "sparse_index_topk: key strides must be multiples of 8 with k_sn >= d");
  SPK_REQUIRE(reinterpret_cast<uintptr_t>(keys) % 16 == 0 && reinterpret_cast<uintptr_t>(q) % 16 == 0,
              SPK_EINVAL, "sparse_index_topk: q and keys must be 16-byte aligned");
  const int G = Hq / Hkv;
  const int ns = mode == SPK_IDX_TOKEN_PER_HEAD ? T * G : T;
  const int n_cand = block ? n_tokens / block_size : n_tokens;
  SPK_REQUIRE(ns <= kFusedMaxVectors && n_cand <= kFusedMaxCand &&
                  (int64_t)ns * n_cand <= kFusedLds,
              SPK_EUNSUPPORTED,
              "sparse_index_topk: %d score vectors x %d candidates per KV head exceed the fused "
              "limits (%d vectors, %d candidates, %d scores); use sparse_index_score + "
              "topk_select",
              ns, n_cand, kFusedMaxVectors, kFusedMaxCand, kFusedLds);
  SPK_REQUIRE(scores == nullptr || s_ld >= n_cand, SPK_EINVAL,
              "sparse_index_topk: s_ld %lld < candidates %d", (long long)s_ld, n_cand);
  const int kk = k < n_cand ? k : n_cand;
  SPK_REQUIRE(kk == 0 || (idx && idx_ld >= kk), SPK_EINVAL,
              "sparse_index_topk: null idx or idx_ld %lld < min(k, candidates) %d",
              (long long)idx_ld, kk);
  clear_error();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int q_bf16 = q_dtype == SPK_BF16;
  const int ns_pad = pad_ns(ns);
  const int groups = B * Hkv;
  if (d == 128)
    return k_dtype == SPK_BF16
               ? launch_fused<128, uint16_t>(ns_pad, groups, st, mode, q, q_bf16, keys, k_sb, k_sh,
                                             k_sn, T, Hq, Hkv, G, ns, n_cand, k, scores, s_ld, idx,
                                             idx_ld, count)
               : launch_fused<128, float>(ns_pad, groups, st, mode, q, q_bf16, keys, k_sb, k_sh, k_sn,
                                          T, Hq, Hkv, G, ns, n_cand, k, scores, s_ld, idx, idx_ld,
                                          count);
  return k_dtype == SPK_BF16
             ? launch_fused<64, uint16_t>(ns_pad, groups, st, mode, q, q_bf16, keys, k_sb, k_sh, k_sn,
                                          T, Hq, Hkv, G, ns, n_cand, k, scores, s_ld, idx, idx_ld,
                                          count)
             : launch_fused<64, float>(ns_pad, groups, st, mode, q, q_bf16, keys, k_sb, k_sh, k_sn, T,
                                       Hq, Hkv, G, ns, n_cand, k, scores, s_ld, idx, idx_ld, count);
}

extern "C" SPK_API spk_status sparse_window_pool(const void* keys, spk_dtype k_dtype, int64_t k_sb,
                                                 int64_t k_sh, int64_t k_sn, int B, int Hkv, int d,
                                                 int n_tokens, int window, int stride,
                                                 float* kwin, int64_t w_cap, void* stream) {
  using namespace spk;
  SPK_REQUIRE(keys && kwin, SPK_EINVAL, "sparse_window_pool: null keys or kwin");
  SPK_REQUIRE(B > 0 && Hkv > 0 && n_tokens >= 0, SPK_EINVAL,
              "sparse_window_pool: bad shape B=%d Hkv=%d n_tokens=%d", B, Hkv, n_tokens);
  SPK_REQUIRE(dtype_ok(k_dtype), SPK_EUNSUPPORTED, "sparse_window_pool: unsupported dtype");
  SPK_REQUIRE(d == 64 || d == 128, SPK_EUNSUPPORTED, "sparse_window_pool: d=%d not in {64,128}", d);
  SPK_REQUIRE(window >= 1 && stride >= 1 && window <= (1 << 16) && stride <= (1 << 16), SPK_EINVAL,
              "sparse_window_pool: window %d / stride %d out of range", window, stride);
  SPK_REQUIRE(k_sn >= d && k_sb >= 0 && k_sh >= 0 && k_sn % 8 == 0 && k_sh % 8 == 0 && k_sb % 8 == 0,
              SPK_EINVAL, "sparse_window_pool: key strides must be multiples of 8 with k_sn >= d");
  SPK_REQUIRE(reinterpret_cast<uintptr_t>(keys) % 16 == 0 && reinterpret_cast<uintptr_t>(kwin) % 16 == 0,
              SPK_EINVAL, "sparse_window_pool: keys and kwin must be 16-byte aligned");
  const int nw = n_tokens < window ? 0 : (n_tokens - window) / stride + 1;
  SPK_REQUIRE(w_cap >= nw, SPK_EINVAL, "sparse_window_pool: w_cap %lld < windows %d",
              (long long)w_cap, nw);
  clear_error();
  if (nw == 0) return SPK_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int groups = B * Hkv;
  const int wpw = pick_rows_per_wg((int64_t)nw * groups, 4 * (64 / (d / 8)));
  dim3 grid(ceil_div(nw, wpw), groups);
#define SPK_POOL(DV, KT)                                                                        \
  hipLaunchKernelGGL((window_pool_kernel<DV, KT>), grid, dim3(kThreads), 0, st,                \
                     reinterpret_cast<const KT*>(keys), k_sb, k_sh, k_sn, Hkv, nw, window, stride, \
                     wpw, kwin, w_cap)
  if (d == 128) {
    if (k_dtype == SPK_BF16) SPK_POOL(128, uint16_t);
    else SPK_POOL(128, float);
  } else {
    if (k_dtype == SPK_BF16) SPK_POOL(64, uint16_t);
    else SPK_POOL(64, float);
  }
#undef SPK_POOL
  return check_launch("sparse_window_pool");
}

extern "C" SPK_API spk_status sparse_index_score_windowed(const void* pred, spk_dtype p_dtype,
                                                          const float* kwin, int64_t w_cap, int B,
                                                          int T, int Hkv, int d, int n_tokens,
                                                          int window, int stride, int block_size,
                                                          float* scores, int64_t s_ld,
                                                          void* stream) {
  using namespace spk;
  SPK_REQUIRE(pred && kwin && scores, SPK_EINVAL,
              "sparse_index_score_windowed: null pred, kwin or scores");
  SPK_REQUIRE(B > 0 && T > 0 && T <= 16 && Hkv > 0 && n_tokens >= 0, SPK_EINVAL,
              "sparse_index_score_windowed: bad shape B=%d T=%d (1..16) Hkv=%d n_tokens=%d", B, T,
              Hkv, n_tokens);
  SPK_REQUIRE(dtype_ok(p_dtype), SPK_EUNSUPPORTED, "sparse_index_score_windowed: unsupported dtype");
  SPK_REQUIRE(d == 64 || d == 128, SPK_EUNSUPPORTED,
              "sparse_index_score_windowed: d=%d not in {64,128}", d);
  SPK_REQUIRE(window >= 1 && stride >= 1 && block_size >= 1 && window <= (1 << 16) &&
                  stride <= (1 << 16) && block_size <= (1 << 16),
              SPK_EINVAL, "sparse_index_score_windowed: window %d / stride %d / block %d out of range",
              window, stride, block_size);
  SPK_REQUIRE(((int64_t)block_size + window) / stride + 3 <= kWinTile, SPK_EUNSUPPORTED,
              "sparse_index_score_windowed: a block overlaps more than %d windows", kWinTile - 3);
  SPK_REQUIRE(reinterpret_cast<uintptr_t>(kwin) % 16 == 0 && reinterpret_cast<uintptr_t>(pred) % 16 == 0,
              SPK_EINVAL, "sparse_index_score_windowed: pred and kwin must be 16-byte aligned");
  const int nw = n_tokens < window ? 0 : (n_tokens - window) / stride + 1;
  const int nb = n_tokens / block_size;
  SPK_REQUIRE(w_cap >= nw, SPK_EINVAL, "sparse_index_score_windowed: w_cap %lld < windows %d",
              (long long)w_cap, nw);
  SPK_REQUIRE(s_ld >= nb, SPK_EINVAL, "sparse_index_score_windowed: s_ld %lld < blocks %d",
              (long long)s_ld, nb);
  clear_error();
  if (nb == 0) return SPK_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int groups = B * Hkv;
  const int bpw = pick_blocks_per_wg(nb, groups, block_size, window, stride);
  dim3 grid(ceil_div(nb, bpw), groups);
  const int q_bf16 = p_dtype == SPK_BF16;
#define SPK_WIN(DV, NSV)                                                                         \
  hipLaunchKernelGGL((index_windowed_kernel<DV, NSV>), grid, dim3(kThreads), 0, st, pred, q_bf16, \
                     kwin, w_cap, T, Hkv, T, nw, nb, window, stride, block_size, bpw, scores, s_ld)
  const int ns_pad = pad_ns(T);
  if (d == 128) {
    switch (ns_pad) {
      case 1: SPK_WIN(128, 1); break;
      case 4: SPK_WIN(128, 4); break;
      case 8: SPK_WIN(128, 8); break;
      default: SPK_WIN(128, 16); break;
    }
  } else {
    switch (ns_pad) {
      case 1: SPK_WIN(64, 1); break;
      case 4: SPK_WIN(64, 4); break;
      case 8: SPK_WIN(64, 8); break;
      default: SPK_WIN(64, 16); break;
    }
  }
#undef SPK_WIN
  return check_launch("sparse_index_score_windowed");
}
