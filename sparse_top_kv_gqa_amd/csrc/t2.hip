// The T2 tier: rows kept as 8-bit codes (one fp32 scale per row) in host memory, brought back
// to the cache's bf16 format in HBM staging rows before the attention that reads them.
//
// "Nem Todos os Pensamentos Necessitam de HBM", §1 "Classificação de Quatro Níveis": T2 holds
// low-importance rows on the CPU at reduced precision (for instance 8-bit quantization); its §4
// "Sensibilidade à Precisão" reports what that costs reasoning accuracy.  The pages name no
// scheme; the one taken is symmetric and per row (one token of one KV head, K and V
// separately): m = the largest |x| over the row's finite elements, scale = fp32(m / 127),
// code = rint(fp32(x * fp32(127 / m))) with ties to even, clamped to [-127, 127]; a non-finite
// element gets code 0 and a row with m = 0 codes 0 and scale 0.  A T2 row reaches the
// attention as bf16(fp32(code * scale)), rounded to nearest even.  The quotient, the product
// and the rounding are IEEE fp32 operations (no contraction), so the codes are the ones an fp32
// evaluation of the definition gives.
//
//   kv_quantize_int8  codes and scales of a range of rows (device or pinned host source and
//                     destination)
//   t2_fetch          the listed rows' codes, read through the pool's device address,
//                     dequantized into their staging rows of one layer's HBM pools
//   t2_locations      the locations the attention reads: a T2 row's staging row, every other
//                     row's residency location
#include "spk_internal.h"

namespace spk {
namespace {

constexpr int kThreads = 256;

// Round an fp32 value to bf16, nearest even (the value here is always finite).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Each lane takes 8 consecutive elements of a row; D/8 lanes hold one row.
template <typename KT, int D>
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const KT* __restrict__ src, int64_t s_sb, int64_t s_sh, int64_t s_sn, int Hkv, int row_begin,
    int rows, int8_t* __restrict__ codes, int64_t c_sb, int64_t c_sh, int64_t c_sn,
    float* __restrict__ scales, int64_t sc_sb, int64_t sc_sh) {
  constexpr int LPR = D / 8;                 // lanes per row (8 or 16)
  constexpr int RPW = kThreads / LPR;        // rows per workgroup pass
  const int g = blockIdx.y, b = g / Hkv, h = g % Hkv;
  const int sub = threadIdx.x % LPR;
  const int r = blockIdx.x * RPW + (int)threadIdx.x / LPR;
  const bool live = r < rows;
  const int64_t tok = row_begin + (live ? r : 0);
  Raw8<KT> raw;
  raw.load(src + (int64_t)b * s_sb + (int64_t)h * s_sh + tok * s_sn + sub * 8);
  float x[8];
  raw.to_float(x);
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float a = fabsf(x[j]);
    m = isfinite(x[j]) ? fmaxf(m, a) : m;
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));  // the row's lanes
  const bool pos = m > 0.f;
  const float scale = pos ? __fdiv_rn(m, 127.f) : 0.f;
  const float inv = pos ? __fdiv_rn(127.f, m) : 0.f;
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float c = isfinite(x[j]) ? rintf(__fmul_rn(x[j], inv)) : 0.f;
    c = fminf(127.f, fmaxf(-127.f, c));
    w[j / 4] |= ((uint32_t)(int)c & 0xFFu) << (8 * (j % 4));
  }
  if (live) {
    int8_t* dst = codes + (int64_t)b * c_sb + (int64_t)h * c_sh + tok * c_sn + sub * 8;
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    if (sub == 0) scales[(int64_t)b * sc_sb + (int64_t)h * sc_sh + tok] = scale;
  }
}

// Row copy_tok[b, r] of the code pools, dequantized, into row stage_base + copy_slot[b, r] of
// the HBM pools, for every KV head; D/8 lanes per row, 8 elements (8 code bytes, 16 output
// bytes) per lane.
template <int D>
__global__ __launch_bounds__(kThreads) void t2_fetch_kernel(
    const int8_t* __restrict__ ck, const int8_t* __restrict__ cv, int64_t c_sb, int64_t c_sh,
    int64_t c_sn, const float* __restrict__ sk, const float* __restrict__ sv, int64_t sc_sb,
    int64_t sc_sh, int64_t code_rows, uint16_t* __restrict__ k, uint16_t* __restrict__ v,
    int64_t kv_sb, int64_t kv_sh, int64_t kv_sn, int64_t hbm_rows, int64_t stage_base,
    const int32_t* __restrict__ copy_tok, const int32_t* __restrict__ copy_slot, int64_t copy_ld,
    const int32_t* __restrict__ copy_count, int Hkv, int rows_per_wg) {
  constexpr int LPR = D / 8;
  constexpr int RPW = kThreads / LPR;
  const int g = blockIdx.y, b = g / Hkv, h = g % Hkv;
  const int cnt = (int)min((int64_t)copy_count[b], copy_ld);
  const int r0 = blockIdx.x * rows_per_wg;
  if (r0 >= cnt) return;
  const int r1 = min(r0 + rows_per_wg, cnt);
  const int sub = threadIdx.x % LPR;
  for (int r = r0 + (int)threadIdx.x / LPR; r < r1; r += RPW) {
    const int tok = copy_tok[(int64_t)b * copy_ld + r];
    const int64_t dst = stage_base + copy_slot[(int64_t)b * copy_ld + r];
    if (tok < 0 || tok >= code_rows || copy_slot[(int64_t)b * copy_ld + r] < 0 || dst >= hbm_rows)
      continue;
    const int64_t cs = (int64_t)b * c_sb + (int64_t)h * c_sh + (int64_t)tok * c_sn + sub * 8;
    const int64_t ss = (int64_t)b * sc_sb + (int64_t)h * sc_sh + tok;
    const uint2 qk = *reinterpret_cast<const uint2*>(ck + cs);
    const uint2 qv = *reinterpret_cast<const uint2*>(cv + cs);
    const float fk = sk[ss], fv = sv[ss];
    uint32_t ok[4], ov[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const uint32_t wk = j < 4 ? qk.x : qk.y, wv = j < 4 ? qv.x : qv.y;
      const int sh = 8 * (j % 4);
      const float k0 = (float)(int8_t)((wk >> sh) & 0xFFu), k1 = (float)(int8_t)((wk >> (sh + 8)) & 0xFFu);
      const float v0 = (float)(int8_t)((wv >> sh) & 0xFFu), v1 = (float)(int8_t)((wv >> (sh + 8)) & 0xFFu);
      ok[j / 2] = bf16_rne(__fmul_rn(k0, fk)) | (bf16_rne(__fmul_rn(k1, fk)) << 16);
      ov[j / 2] = bf16_rne(__fmul_rn(v0, fv)) | (bf16_rne(__fmul_rn(v1, fv)) << 16);
    }
    const int64_t ds = (int64_t)b * kv_sb + (int64_t)h * kv_sh + dst * kv_sn + sub * 8;
    *reinterpret_cast<uint4*>(k + ds) = make_uint4(ok[0], ok[1], ok[2], ok[3]);
    *reinterpret_cast<uint4*>(v + ds) = make_uint4(ov[0], ov[1], ov[2], ov[3]);
  }
}

__global__ __launch_bounds__(kThreads) void t2_loc_kernel(
    const uint8_t* __restrict__ tier, int64_t tier_ld, const int32_t* __restrict__ loc_res,
    int64_t res_ld, const int32_t* __restrict__ loc_t2, int64_t t2_ld, int32_t* __restrict__ out,
    int64_t out_ld, int n, int64_t stage_base) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  const int32_t t2 = loc_t2[(int64_t)b * t2_ld + i];
  const bool staged = tier[(int64_t)b * tier_ld + i] == 2 && t2 >= 0;
  out[(int64_t)b * out_ld + i] =
      staged ? (int32_t)(stage_base + t2) : loc_res[(int64_t)b * res_ld + i];
}

// Device address of memory a kernel reads or writes: device memory as is, page-locked host
// memory through the device alias HIP reports for it; anything else is refused.
spk_status kernel_ptr(const void* p, void** dev, const char* where, const char* name) {
  hipPointerAttribute_t at{};
  const hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return set_error(SPK_EINVAL, "%s: %s is not memory known to HIP (%s)", where, name,
                     hipGetErrorString(e));
  }
  if (at.type == hipMemoryTypeDevice) {
    *dev = const_cast<void*>(p);
    return SPK_OK;
  }
  if (at.type == hipMemoryTypeHost && at.devicePointer != nullptr) {
    // the alias of the allocation's base, moved by p's offset inside it
    *dev = static_cast<char*>(at.devicePointer) +
           (static_cast<const char*>(p) - static_cast<const char*>(at.hostPointer));
    return SPK_OK;
  }
  return set_error(SPK_EINVAL, "%s: %s must be device memory or pinned, device-mapped host memory",
                   where, name);
}

}  // namespace
}  // namespace spk

extern "C" SPK_API spk_status kv_quantize_int8(const void* src, spk_dtype src_dtype, int64_t s_sb,
                                               int64_t s_sh, int64_t s_sn, int B, int Hkv, int d,
                                               int row_begin, int row_end, int8_t* codes,
                                               int64_t c_sb, int64_t c_sh, int64_t c_sn,
                                               float* scales, int64_t sc_sb, int64_t sc_sh,
                                               void* stream) {
  using namespace spk;
  SPK_REQUIRE(B >= 0 && Hkv > 0 && row_begin >= 0 && row_end >= row_begin, SPK_EINVAL,
              "kv_quantize_int8: bad sizes");
  SPK_REQUIRE(d == 64 || d == 128, SPK_EUNSUPPORTED, "kv_quantize_int8: d=%d not in {64,128}", d);
  SPK_REQUIRE(dtype_ok(src_dtype), SPK_EUNSUPPORTED, "kv_quantize_int8: unsupported dtype");
  SPK_REQUIRE(s_sn >= d && c_sn >= d && s_sb >= 0 && s_sh >= 0 && c_sb >= 0 && c_sh >= 0 &&
                  sc_sb >= 0 && sc_sh >= 0 && s_sn % 8 == 0 && s_sh % 8 == 0 && s_sb % 8 == 0 &&
                  c_sn % 8 == 0 && c_sh % 8 == 0 && c_sb % 8 == 0,
              SPK_EINVAL, "kv_quantize_int8: strides must be multiples of 8 with row strides >= d");
  const int rows = row_end - row_begin;
  if (B == 0 || rows == 0) {
    clear_error();
    return SPK_OK;
  }
  SPK_REQUIRE(src && codes && scales, SPK_EINVAL, "kv_quantize_int8: null pointer");
  void *sd = nullptr, *cd = nullptr, *scd = nullptr;
  spk_status e = kernel_ptr(src, &sd, "kv_quantize_int8", "src");
  if (e != SPK_OK) return e;
  e = kernel_ptr(codes, &cd, "kv_quantize_int8", "codes");
  if (e != SPK_OK) return e;
  e = kernel_ptr(scales, &scd, "kv_quantize_int8", "scales");
  if (e != SPK_OK) return e;
  SPK_REQUIRE(reinterpret_cast<uintptr_t>(sd) % 16 == 0 && reinterpret_cast<uintptr_t>(cd) % 8 == 0 &&
                  reinterpret_cast<uintptr_t>(scd) % 4 == 0,
              SPK_EINVAL, "kv_quantize_int8: src must be 16-byte, codes 8-byte aligned");
  clear_error();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int rpw = kThreads / (d / 8);
  dim3 grid((unsigned)ceil_div(rows, rpw), (unsigned)(B * Hkv));
#define SPK_Q(KT, DV)                                                                          \
  hipLaunchKernelGGL((quantize_kernel<KT, DV>), grid, dim3(kThreads), 0, st,                    \
                     reinterpret_cast<const KT*>(sd), s_sb, s_sh, s_sn, Hkv, row_begin, rows,    \
                     reinterpret_cast<int8_t*>(cd), c_sb, c_sh, c_sn,                           \
                     reinterpret_cast<float*>(scd), sc_sb, sc_sh)
  if (src_dtype == SPK_BF16) {
    if (d == 128) SPK_Q(uint16_t, 128);
    else SPK_Q(uint16_t, 64);
  } else {
    if (d == 128) SPK_Q(float, 128);
    else SPK_Q(float, 64);
  }
#undef SPK_Q
  return check_launch("kv_quantize_int8");
}

extern "C" SPK_API spk_status t2_fetch(const int8_t* codes_k, const int8_t* codes_v, int64_t c_sb,
                                       int64_t c_sh, int64_t c_sn, const float* scale_k,
                                       const float* scale_v, int64_t sc_sb, int64_t sc_sh,
                                       int64_t code_rows, void* k, void* v, spk_dtype kv_dtype,
                                       int64_t kv_sb, int64_t kv_sh, int64_t kv_sn,
                                       int64_t hbm_rows, int64_t stage_base, int B, int Hkv,
                                       int d, const int32_t* copy_tok, const int32_t* copy_slot,
                                       int64_t copy_ld, const int32_t* copy_count, int max_copies,
                                       void* stream) {
  using namespace spk;
  SPK_REQUIRE(B >= 0 && Hkv > 0 && max_copies >= 0 && copy_ld >= 0 && code_rows >= 0 &&
                  hbm_rows >= 0 && stage_base >= 0,
              SPK_EINVAL, "t2_fetch: negative size");
  SPK_REQUIRE(d == 64 || d == 128, SPK_EUNSUPPORTED, "t2_fetch: d=%d not in {64,128}", d);
  SPK_REQUIRE(kv_dtype == SPK_BF16, SPK_EUNSUPPORTED, "t2_fetch: T2 rows come back as bf16 only");
  SPK_REQUIRE(c_sn >= d && kv_sn >= d && c_sb >= 0 && c_sh >= 0 && sc_sb >= 0 && sc_sh >= 0 &&
                  kv_sb >= 0 && kv_sh >= 0 && c_sn % 8 == 0 && c_sh % 8 == 0 && c_sb % 8 == 0 &&
                  kv_sn % 8 == 0 && kv_sh % 8 == 0 && kv_sb % 8 == 0,
              SPK_EINVAL, "t2_fetch: strides must be multiples of 8 with row strides >= d");
  const int mc = (int)(max_copies < copy_ld ? max_copies : copy_ld);
  if (B == 0 || mc == 0) {
    clear_error();
    return SPK_OK;
  }
  SPK_REQUIRE(codes_k && codes_v && scale_k && scale_v && k && v && copy_tok && copy_slot &&
                  copy_count,
              SPK_EINVAL, "t2_fetch: null pointer");
  void *ckd = nullptr, *cvd = nullptr, *skd = nullptr, *svd = nullptr;
  spk_status e = kernel_ptr(codes_k, &ckd, "t2_fetch", "codes_k");
  if (e == SPK_OK) e = kernel_ptr(codes_v, &cvd, "t2_fetch", "codes_v");
  if (e == SPK_OK) e = kernel_ptr(scale_k, &skd, "t2_fetch", "scale_k");
  if (e == SPK_OK) e = kernel_ptr(scale_v, &svd, "t2_fetch", "scale_v");
  if (e != SPK_OK) return e;
  SPK_REQUIRE(reinterpret_cast<uintptr_t>(ckd) % 8 == 0 && reinterpret_cast<uintptr_t>(cvd) % 8 == 0 &&
                  reinterpret_cast<uintptr_t>(k) % 16 == 0 && reinterpret_cast<uintptr_t>(v) % 16 == 0,
              SPK_EINVAL, "t2_fetch: codes must be 8-byte, HBM pools 16-byte aligned");
  clear_error();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int rows_per_wg = 64;
  dim3 grid((unsigned)ceil_div(mc, rows_per_wg), (unsigned)(B * Hkv));
#define SPK_F(DV)                                                                               \
  hipLaunchKernelGGL((t2_fetch_kernel<DV>), grid, dim3(kThreads), 0, st,                         \
                     reinterpret_cast<const int8_t*>(ckd), reinterpret_cast<const int8_t*>(cvd),  \
                     c_sb, c_sh, c_sn, reinterpret_cast<const float*>(skd),                      \
                     reinterpret_cast<const float*>(svd), sc_sb, sc_sh, code_rows,               \
                     reinterpret_cast<uint16_t*>(k), reinterpret_cast<uint16_t*>(v), kv_sb, kv_sh, \
                     kv_sn, hbm_rows, stage_base, copy_tok, copy_slot, copy_ld, copy_count, Hkv,  \
                     rows_per_wg)
  if (d == 128) SPK_F(128);
  else SPK_F(64);
#undef SPK_F
  return check_launch("t2_fetch");
}

extern "C" SPK_API spk_status t2_locations(const uint8_t* tier, int64_t tier_ld,
                                           const int32_t* loc_res, int64_t res_ld,
                                           const int32_t* loc_t2, int64_t t2_ld, int32_t* loc_out,
                                           int64_t out_ld, int B, int n_tokens,
                                           int64_t stage_base, void* stream) {
  using namespace spk;
  SPK_REQUIRE(B >= 0 && n_tokens >= 0 && stage_base >= 0, SPK_EINVAL, "t2_locations: bad sizes");
  SPK_REQUIRE(tier_ld >= n_tokens && res_ld >= n_tokens && t2_ld >= n_tokens && out_ld >= n_tokens,
              SPK_EINVAL, "t2_locations: row strides smaller than n_tokens");
  SPK_REQUIRE(stage_base + n_tokens < ((int64_t)1 << 31), SPK_EINVAL,
              "t2_locations: staging rows beyond int32 locations");
  if (B == 0 || n_tokens == 0) {
    clear_error();
    return SPK_OK;
  }
  SPK_REQUIRE(tier && loc_res && loc_t2 && loc_out, SPK_EINVAL, "t2_locations: null pointer");
  clear_error();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  dim3 grid((unsigned)ceil_div(n_tokens, kThreads), (unsigned)B);
  hipLaunchKernelGGL(t2_loc_kernel, grid, dim3(kThreads), 0, st, tier, tier_ld, loc_res, res_ld,
                     loc_t2, t2_ld, loc_out, out_ld, n_tokens, stage_base);
  return check_launch("t2_locations");
}
