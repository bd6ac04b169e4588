// importance_accumulate: cumulative attention importance, one decode step.
//
// "Nem Todos os Pensamentos Necessitam de HBM", §2 "Pontuação de Importância": at every decode
// step each position's score grows by its attention weight averaged over heads, then over
// layers: s_i += (1/|L|) Σ_ℓ (1/H) Σ_h α_ℓ,h[i].
//
// α_ℓ,h[u] = exp(x - lse) is formed from the scaled logits and the log-sum-exp that
// sparse_decode_attn wrote for each layer, because the normalisation is only known after its
// split-K combine.  One thread per list position: reads of the logits are coalesced along u;
// the L*H terms are summed in a fixed order (no atomics, deterministic).
#include "spk_internal.h"

namespace spk {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxLH = 4096;

__global__ __launch_bounds__(kThreads) void importance_kernel(
    float* __restrict__ s, int64_t s_ld, int B, int n_tokens, const int32_t* __restrict__ sel_idx,
    const int32_t* __restrict__ sel_count, int64_t sel_ld, const float* __restrict__ logits,
    int64_t logits_ld, const float* __restrict__ lse, int L, int Hq, float inv_lh) {
  __shared__ float lse2[kMaxLH];
  const int b = blockIdx.y;
  for (int i = threadIdx.x; i < L * Hq; i += kThreads) {
    const int l = i / Hq, h = i % Hq;
    lse2[i] = lse[((int64_t)l * B + b) * Hq + h] * kLog2e;
  }
  __syncthreads();
  int cnt = sel_count[b];
  if (cnt > sel_ld) cnt = (int)sel_ld;
  const int u = blockIdx.x * kThreads + threadIdx.x;
  if (u >= cnt) return;
  const int tok = sel_idx[(int64_t)b * sel_ld + u];
  if (tok < 0 || tok >= n_tokens) return;
  float acc = 0.f;
  for (int l = 0; l < L; ++l) {
    const float* row = logits + ((int64_t)l * B + b) * Hq * logits_ld + u;
    float part = 0.f;
    for (int h = 0; h < Hq; ++h) {
      const float x = row[(int64_t)h * logits_ld];
      const float m = lse2[l * Hq + h];
      // x = -inf (row not read) or lse = -inf (nothing read) contribute nothing
      if (x != -INFINITY && m != -INFINITY) part += __builtin_amdgcn_exp2f(x * kLog2e - m);
    }
    acc += part;
  }
  float* sp = s + (int64_t)b * s_ld + tok;
  *sp = *sp + acc * inv_lh;
}

}  // namespace
}  // namespace spk

extern "C" SPK_API spk_status importance_accumulate(float* s, int64_t s_ld, int B, int n_tokens,
                                                    const int32_t* sel_idx,
                                                    const int32_t* sel_count, int64_t sel_ld,
                                                    const float* logits, int64_t logits_ld,
                                                    const float* lse, int L, int Hq,
                                                    void* stream) {
  using namespace spk;
  SPK_REQUIRE(B >= 0 && n_tokens >= 0 && L >= 1 && Hq >= 1 && sel_ld >= 0, SPK_EINVAL,
              "importance_accumulate: bad sizes B=%d n_tokens=%d L=%d Hq=%d", B, n_tokens, L, Hq);
  SPK_REQUIRE(L * Hq <= kMaxLH, SPK_EUNSUPPORTED, "importance_accumulate: L*Hq=%d > %d", L * Hq,
              kMaxLH);
  SPK_REQUIRE(s_ld >= n_tokens && logits_ld >= sel_ld, SPK_EINVAL,
              "importance_accumulate: s_ld < n_tokens or logits_ld < sel_ld");
  SPK_REQUIRE(B == 0 || (s && sel_idx && sel_count && logits && lse), SPK_EINVAL,
              "importance_accumulate: null pointer");
  clear_error();
  if (B == 0 || sel_ld == 0) return SPK_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  dim3 grid(ceil_div(sel_ld, kThreads), B);
  hipLaunchKernelGGL(importance_kernel, grid, dim3(kThreads), 0, st, s, s_ld, B, n_tokens, sel_idx,
                     sel_count, sel_ld, logits, logits_ld, lse, L, Hq, 1.0f / (float)(L * Hq));
  return check_launch("importance_accumulate");
}
