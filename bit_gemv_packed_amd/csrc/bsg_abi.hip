// C ABI of libbsg: host-side argument validation, launch planning and
// dispatch.  Validation is a pure function of the arguments (no device
// pointer is dereferenced) and runs before any HIP call.
#include <cstdint>
#include <cstdlib>

#include "bsg_internal.h"

namespace bsg {
hipError_t launch_pack(const float* W, int M, int N, int K, bool colscale, uint32_t* bits, float* alpha,
                       uint16_t* cs, void* ws, hipStream_t st);
hipError_t launch_pack_signs(const float* S, int M, int N, uint32_t* bits, hipStream_t st);
hipError_t launch_pack_hybrid(const float* W, int M, int N, int K, int g, int s, const int32_t* idx, bool colscale,
                              uint32_t* bits, uint16_t* alpha, uint16_t* cs, uint32_t* sbits, uint16_t* salpha,
                              uint16_t* scs, void* ws, hipStream_t st);
hipError_t launch_absmean(const float* X, int S, int N, float* xbar, hipStream_t st);
hipError_t launch_salient(const float* W, int M, int N, const float* xbar, int ns, int32_t* rows, int8_t* q,
                          uint16_t* s, float* alpha, int K, void* ws, hipStream_t st);
hipError_t launch_salient_apply(const int32_t* rows, int ns, const int8_t* q, const uint16_t* s, int M, int N,
                                const void* x, int xdt, int B, float* y, hipStream_t st);
hipError_t launch_quantize(const void* x, int xdt, int N, int B, int8_t* xq, float* sx, hipStream_t st);
hipError_t launch_layout(const uint32_t* src, int K, int M, int N, uint32_t* dst, bool to_layout, hipStream_t st);
size_t fit_workspace_bytes(int M, int N, int r);
hipError_t launch_binlr_fit(const float* W, int M, int N, int r, int rounds, const uint32_t* v_init,
                            uint32_t* U_bits, uint32_t* V_bits, uint16_t* alpha_f16, double* alpha_out,
                            double* alpha_greedy_out, double* sse_out, int* solved_out, void* workspace,
                            hipStream_t st);
}  // namespace bsg

using namespace bsg;

namespace {

constexpr int32_t kAbiVersion = 1;

bool misaligned(const void* p, size_t a) { return p && (((uintptr_t)p) % a) != 0; }

bool bad_dtype(int dt) { return dt != BSG_F32 && dt != BSG_F16 && dt != BSG_BF16; }

size_t dtype_size(int dt) { return dt == BSG_F32 ? 4 : 2; }

bool bad_n(int N) { return N <= 0 || (N % 32) != 0; }

// Every operand of one product is addressed with 32-bit byte offsets:
// K*M row scales, N*B activations and K*N column scales below 2^30 elements.
bool too_big(int K, int M, int N, int B) {
  return (size_t)K * M >= (1u << 30) || (size_t)N * B >= (1u << 30) || (size_t)K * N >= (1u << 30);
}

thread_local hipError_t last_hip = hipSuccess;

bsg_status hip_status(hipError_t e) {
  if (e == hipSuccess) return BSG_OK;
  last_hip = e;
  return BSG_ERR_HIP;
}

// binlr workspace: z, fp32 [r][B]
// binlr workspace: z, fp32 [r][B]; for B >= 4 (the matrix-core expansion)
// also the bf16 halves of alpha_r (.) z, [r][B] each
size_t binlr_ws(int r, int B) {
  return align_up((size_t)r * B * 4, 256) + (B >= 4 ? 2 * align_up((size_t)r * B * 2, 256) : 0);
}

bool xvec_ok(const void* x, const void* cs) {
  return (((uintptr_t)x) % 16) == 0 && (((uintptr_t)cs) % 8) == 0;
}

}  // namespace

extern "C" {

int32_t bsg_abi_version(void) { return kAbiVersion; }

int32_t bsg_last_hip_error(void) { return (int32_t)last_hip; }

const char* bsg_last_hip_error_string(void) { return hipGetErrorString(last_hip); }

const char* bsg_status_string(bsg_status s) {
  switch (s) {
    case BSG_OK: return "ok";
    case BSG_ERR_NULL: return "a required pointer is NULL";
    case BSG_ERR_SHAPE: return "invalid size (negative, N not a multiple of 32, or count out of range)";
    case BSG_ERR_DTYPE: return "unknown dtype";
    case BSG_ERR_ALIGN: return "misaligned device pointer";
    case BSG_ERR_UNSUPPORTED: return "unsupported combination";
    case BSG_ERR_WORKSPACE: return "workspace missing or too small";
    case BSG_ERR_HIP: return "HIP runtime or launch failure";
    default: return "unknown status";
  }
}

size_t bsg_layout_words(int K, int M, int N) {
  if (K < 1 || M < 0 || bad_n(N)) return 0;
  return (size_t)K * plane_words(M, N / 32);
}

int64_t bsg_layout_word_offset(int K, int M, int N, int k, int m, int w) {
  if (K < 1 || M < 0 || bad_n(N)) return -1;
  if (k < 0 || k >= K || m < 0 || m >= M || w < 0 || w >= N / 32) return -1;
  return (int64_t)layout_offset(M, N / 32, plane_words(M, N / 32), k, m, w);
}

size_t bsg_binlr_workspace_bytes(int r, int M, int N, int B) {
  if (r <= 0 || (r % 32) != 0 || M < 0 || bad_n(N) || B < 1 || B > kMaxB) return 0;
  return binlr_ws(r, B);
}

size_t bsq_pack_workspace_bytes(int M, int N) {
  if (M < 0 || bad_n(N)) return 0;
  return align_up((size_t)M * N * 8, 256) + 256;
}

size_t bsq_salient_workspace_bytes(int M, int N) {
  if (M < 0 || N <= 0) return 0;
  return align_up((size_t)M * 8, 256) + align_up((size_t)M * 4, 256);
}

bsg_status bsq_pack(const float* W, int M, int N, int K, int flags, uint32_t* bits, float* alpha,
                    uint16_t* colscale, void* workspace, size_t workspace_bytes, void* stream) {
  const bool cs = (flags & BSG_PACK_COLSCALE) != 0;
  if (K < 1 || K > kMaxK || M < 0 || bad_n(N) || (flags & ~BSG_PACK_COLSCALE)) return BSG_ERR_SHAPE;
  if (M == 0) return BSG_OK;
  if (!W || !bits || !alpha || (cs && !colscale)) return BSG_ERR_NULL;
  if (misaligned(W, 4) || misaligned(bits, 16) || misaligned(alpha, 4) || misaligned(colscale, 2) ||
      misaligned(workspace, 16))
    return BSG_ERR_ALIGN;
  if (!workspace || workspace_bytes < bsq_pack_workspace_bytes(M, N)) return BSG_ERR_WORKSPACE;
  return hip_status(launch_pack(W, M, N, K, cs, bits, alpha, cs ? colscale : nullptr, workspace,
                                (hipStream_t)stream));
}

bsg_status bsq_pack_signs(const float* S, int M, int N, uint32_t* bits, void* stream) {
  if (M < 0 || bad_n(N)) return BSG_ERR_SHAPE;
  if (M == 0) return BSG_OK;
  if (!S || !bits) return BSG_ERR_NULL;
  if (misaligned(S, 4) || misaligned(bits, 16)) return BSG_ERR_ALIGN;
  return hip_status(launch_pack_signs(S, M, N, bits, (hipStream_t)stream));
}

bsg_status bsq_absmean(const float* X, int S, int N, float* xbar, void* stream) {
  if (S < 1 || N <= 0) return BSG_ERR_SHAPE;
  if (!X || !xbar) return BSG_ERR_NULL;
  if (misaligned(X, 4) || misaligned(xbar, 4)) return BSG_ERR_ALIGN;
  return hip_status(launch_absmean(X, S, N, xbar, (hipStream_t)stream));
}

bsg_status bsq_salient(const float* W, int M, int N, const float* xbar, int ns, int32_t* rows, int8_t* q,
                       uint16_t* s_f16, float* alpha, int K, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (M < 0 || N <= 0 || ns < 0 || ns > M || K < 0 || K > kMaxK) return BSG_ERR_SHAPE;
  if (M == 0) return BSG_OK;
  if (!W || !xbar || (ns > 0 && (!rows || !q || !s_f16)) || (K > 0 && !alpha)) return BSG_ERR_NULL;
  if (misaligned(W, 4) || misaligned(xbar, 4) || misaligned(rows, 4) || misaligned(s_f16, 2) ||
      misaligned(alpha, 4) || misaligned(workspace, 16))
    return BSG_ERR_ALIGN;
  if (!workspace || workspace_bytes < bsq_salient_workspace_bytes(M, N)) return BSG_ERR_WORKSPACE;
  return hip_status(launch_salient(W, M, N, xbar, ns, rows, q, s_f16, alpha, K, workspace, (hipStream_t)stream));
}

bsg_status bsq_quantize_i8(const void* x, int x_dtype, int N, int B, int8_t* xq, float* sx, void* stream) {
  if (bad_dtype(x_dtype)) return BSG_ERR_DTYPE;
  if (N <= 0 || B < 1) return BSG_ERR_SHAPE;
  if (!x || !xq || !sx) return BSG_ERR_NULL;
  if (misaligned(x, dtype_size(x_dtype)) || misaligned(sx, 4)) return BSG_ERR_ALIGN;
  return hip_status(launch_quantize(x, x_dtype, N, B, xq, sx, (hipStream_t)stream));
}

bsg_status bsg_logical_to_layout(const uint32_t* logical, int K, int M, int N, uint32_t* bits, void* stream) {
  if (K < 1 || M < 0 || bad_n(N)) return BSG_ERR_SHAPE;
  if (M == 0) return BSG_OK;
  if (!logical || !bits) return BSG_ERR_NULL;
  if (misaligned(logical, 4) || misaligned(bits, 16)) return BSG_ERR_ALIGN;
  return hip_status(launch_layout(logical, K, M, N, bits, true, (hipStream_t)stream));
}

bsg_status bsg_layout_to_logical(const uint32_t* bits, int K, int M, int N, uint32_t* logical, void* stream) {
  if (K < 1 || M < 0 || bad_n(N)) return BSG_ERR_SHAPE;
  if (M == 0) return BSG_OK;
  if (!logical || !bits) return BSG_ERR_NULL;
  if (misaligned(logical, 4) || misaligned(bits, 16)) return BSG_ERR_ALIGN;
  return hip_status(launch_layout(bits, K, M, N, logical, false, (hipStream_t)stream));
}

bsg_status bs_gemv(const uint32_t* bits, int K, int M, int N, const float* alpha, const uint16_t* colscale,
                   const void* x, int x_dtype, int B, float* y, int accumulate, void* stream) {
  if (bad_dtype(x_dtype)) return BSG_ERR_DTYPE;
  if (K < 1 || K > kMaxK || M < 0 || bad_n(N) || B < 1 || B > kMaxB || too_big(K, M, N, B)) return BSG_ERR_SHAPE;
  if (M == 0) return BSG_OK;
  if (!bits || !alpha || !x || !y) return BSG_ERR_NULL;
  if (misaligned(bits, 16) || misaligned(alpha, 4) || misaligned(colscale, 2) ||
      misaligned(x, dtype_size(x_dtype)) || misaligned(y, 4))
    return BSG_ERR_ALIGN;
  const ProdPlan p = plan_prod(K, M, N, B, colscale != nullptr, false);
  ProdArgs a{};
  a.bits = bits;
  a.alpha = alpha;
  a.colscale = colscale;
  a.x = x;
  a.y = y;
  a.plane = plane_words(M, N / 32);
  a.K = K;
  a.M = M;
  a.N = N;
  a.ND = N / 32;
  a.B = B;
  a.xdt = x_dtype;
  a.accumulate = accumulate ? 1 : 0;
  a.xvec = xvec_ok(x, colscale);
  // matrix cores for B >= 4 columns of 16-bit x; with column scales for fp16
  // x whose scales are 4-byte aligned (2 scales per load)
  if (mfma_eligible(B, x_dtype, colscale != nullptr) ||
      (colscale && !misaligned(colscale, 4) && mfma_cg_ok(B, x_dtype, x, true, 0, M)))
    return hip_status(launch_prod_mfma(a, (hipStream_t)stream));
  return hip_status(launch_prod_f(a, p, (hipStream_t)stream));
}

bsg_status bs_gemv_multi(const bsg_proj* projs, int P, int K, int N, const void* x, int x_dtype, int B,
                         int accumulate, void* stream) {
  if (bad_dtype(x_dtype)) return BSG_ERR_DTYPE;
  if (!projs) return BSG_ERR_NULL;
  if (P < 1 || P > kMaxProj || K < 1 || K > kMaxK || bad_n(N) || B < 1 || B > kMaxB) return BSG_ERR_SHAPE;
  const bool cs = projs[0].colscale != nullptr;
  for (int i = 0; i < P; ++i) {
    const bsg_proj& d = projs[i];
    if (d.M < 0 || too_big(K, d.M, N, B) || (d.colscale != nullptr) != cs) return BSG_ERR_SHAPE;
  }
  if (!x) return BSG_ERR_NULL;
  if (misaligned(x, dtype_size(x_dtype))) return BSG_ERR_ALIGN;
  for (int i = 0; i < P; ++i) {
    const bsg_proj& d = projs[i];
    if (d.M == 0) continue;
    if (!d.bits || !d.alpha || !d.y) return BSG_ERR_NULL;
    if (misaligned(d.bits, 16) || misaligned(d.alpha, 4) || misaligned(d.colscale, 2) || misaligned(d.y, 4))
      return BSG_ERR_ALIGN;
  }
  hipStream_t st = (hipStream_t)stream;
  ProdArgs a{};
  a.x = x;
  a.K = K;
  a.N = N;
  a.ND = N / 32;
  a.B = B;
  a.xdt = x_dtype;
  a.accumulate = accumulate ? 1 : 0;
  a.xvec = (((uintptr_t)x) % 16) == 0;
  int np = 0;
  for (int i = 0; i < P; ++i) {
    const bsg_proj& d = projs[i];
    if (d.M == 0) continue;
    ProjDesc& e = a.proj[np++];
    e.bits = d.bits;
    e.alpha = d.alpha;
    e.colscale = d.colscale;
    e.y = d.y;
    e.M = d.M;
    if ((((uintptr_t)d.colscale) % 8) != 0) a.xvec = 0;
  }
  if (np == 0) return BSG_OK;
  // several batch columns on the matrix cores: one fused launch per 16
  // columns (and 4 bases)
  if (np > 1 && mfma_eligible(B, x_dtype, cs) && mfma_multi_ok(B, x)) {
    a.np = np;
    return hip_status(launch_prod_mfma(a, st));
  }
  // one projection, or several batch columns off the matrix cores: a launch
  // each
  if (np == 1 || B != 1) {
    for (int i = 0; i < np; ++i) {
      const ProjDesc& e = a.proj[i];
      const bsg_status s = bs_gemv(e.bits, K, e.M, N, e.alpha, e.colscale, x, x_dtype, B, e.y, accumulate, stream);
      if (s != BSG_OK) return s;
    }
    return BSG_OK;
  }
  a.np = np;
  return hip_status(launch_prod_multi(a, st));
}

// group size: a power of two >= 64 dividing N
static bool bad_group(int N, int g) { return g < 64 || (g & (g - 1)) != 0 || N % g != 0; }
// salient columns per group: 8, 16 or 32 (whole groups per sign word)
static bool bad_salient(int s) { return s != 8 && s != 16 && s != 32; }
static int salient_cols(int N, int g, int s) { return s * (N / g); }
static int salient_words(int N, int g, int s) { return (salient_cols(N, g, s) + 31) / 32; }

size_t bsq_pack_hybrid_workspace_bytes(int M, int N, int g, int s) {
  if (M < 0 || bad_n(N) || bad_group(N, g) || (s != 0 && bad_salient(s))) return 0;
  return align_up((size_t)M * N * 8, 256) + align_up((size_t)M * salient_cols(N, g, s) * 8, 256) +
         align_up((size_t)(N / g) * 8, 256);
}

size_t bsq_pack_grouped_workspace_bytes(int M, int N, int g) { return bsq_pack_hybrid_workspace_bytes(M, N, g, 0); }

bsg_status bsq_pack_hybrid(const float* W, int M, int N, int K, int g, int s, const int32_t* idx, int flags,
                           uint32_t* bits, uint16_t* alpha, uint16_t* colscale, uint32_t* sbits, uint16_t* salpha,
                           uint16_t* scolscale, void* workspace, size_t workspace_bytes, void* stream) {
  const bool cs = (flags & BSG_PACK_COLSCALE) != 0;
  if (K < 1 || K > kMaxK || M < 0 || bad_n(N) || bad_group(N, g) || (s != 0 && bad_salient(s)) ||
      (flags & ~BSG_PACK_COLSCALE))
    return BSG_ERR_SHAPE;
  if (M == 0) return BSG_OK;
  if (!W || !bits || !alpha || (cs && !colscale)) return BSG_ERR_NULL;
  if (s && (!idx || !sbits || !salpha || (cs && !scolscale))) return BSG_ERR_NULL;
  if (misaligned(W, 4) || misaligned(bits, 16) || misaligned(alpha, 2) || misaligned(colscale, 2) ||
      misaligned(idx, 16) || misaligned(sbits, 16) || misaligned(salpha, 8) || misaligned(scolscale, 2) ||
      misaligned(workspace, 16))
    return BSG_ERR_ALIGN;
  if (!workspace || workspace_bytes < bsq_pack_hybrid_workspace_bytes(M, N, g, s)) return BSG_ERR_WORKSPACE;
  return hip_status(launch_pack_hybrid(W, M, N, K, g, s, idx, cs, bits, alpha, cs ? colscale : nullptr, sbits,
                                       salpha, cs ? scolscale : nullptr, workspace, (hipStream_t)stream));
}

bsg_status bsq_pack_grouped(const float* W, int M, int N, int K, int g, int flags, uint32_t* bits, uint16_t* alpha,
                            uint16_t* colscale, void* workspace, size_t workspace_bytes, void* stream) {
  return bsq_pack_hybrid(W, M, N, K, g, 0, nullptr, flags, bits, alpha, colscale, nullptr, nullptr, nullptr,
                         workspace, workspace_bytes, stream);
}

bsg_status bs_gemv_hybrid(const uint32_t* bits, int K, int M, int N, int g, const uint16_t* alpha,
                          const uint16_t* colscale, const uint32_t* sbits, int s, const int32_t* idx,
                          const uint16_t* salpha, const uint16_t* scolscale, const void* x, int x_dtype, int B,
                          float* y, int accumulate, void* stream) {
  if (bad_dtype(x_dtype)) return BSG_ERR_DTYPE;
  if (K < 1 || K > 4 || M < 0 || bad_n(N) || bad_group(N, g) || (s != 0 && bad_salient(s)) || B < 1 ||
      B > kMaxB || too_big(K, M, N, B) || (size_t)K * M * (N / g) >= (1u << 30))
    return BSG_ERR_SHAPE;
  // the salient tables share the main tables' space: column scales on both branches or on neither
  if (s && (colscale != nullptr) != (scolscale != nullptr)) return BSG_ERR_SHAPE;
  if (M == 0) return BSG_OK;
  if (!bits || !alpha || !x || !y) return BSG_ERR_NULL;
  if (s && (!sbits || !idx || !salpha)) return BSG_ERR_NULL;
  if (misaligned(bits, 16) || misaligned(alpha, 2) || misaligned(colscale, 2) ||
      misaligned(x, dtype_size(x_dtype)) || misaligned(y, 4) || misaligned(sbits, 16) || misaligned(idx, 16) ||
      misaligned(salpha, 8) || misaligned(scolscale, 8))
    return BSG_ERR_ALIGN;
  ProdArgs a{};
  a.bits = bits;
  a.alpha = (const float*)(const void*)alpha;  // fp16 scales, read as such by the grouped kernels
  a.colscale = colscale;
  a.x = x;
  a.y = y;
  a.plane = plane_words(M, N / 32);
  a.K = K;
  a.M = M;
  a.N = N;
  a.ND = N / 32;
  a.B = B;
  a.xdt = x_dtype;
  a.accumulate = accumulate ? 1 : 0;
  a.xvec = xvec_ok(x, colscale);
  a.gsw = g / 32;
  a.ngrp = N / g;
  if (s) {
    a.vs_bits = sbits;
    a.vs_S = salient_cols(N, g, s);
    a.vs_nd = salient_words(N, g, s);
    a.vs_plane = plane_words(M, a.vs_nd);
    a.vs_idx = idx;
    a.vs_alpha = salpha;
    a.vs_cs = scolscale;
    a.vs_gpw = 32 / s;
  }
  // B >= 4 columns on the matrix cores (g >= 128, M % 4 == 0, fp16 x with column scales, 4-byte
  // aligned scales); the salient columns then with fp16 x, in a second launch that adds onto y
  const bool mc = !misaligned(alpha, 8) && !misaligned(colscale, 4) &&
                  mfma_cg_ok(B, x_dtype, x, colscale != nullptr, a.gsw, M);
  if (mc && !s) return hip_status(launch_prod_mfma(a, (hipStream_t)stream));
  if (mc && vcm_mfma_ok(B, x_dtype, x, K, a.vs_S, scolscale != nullptr)) {
    ProdArgs am = a;
    am.vs_bits = nullptr;
    const hipError_t e = launch_prod_mfma(am, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(launch_vcm_mfma(a, (hipStream_t)stream));
  }
  return hip_status(launch_prod_grouped(a, (hipStream_t)stream));
}

bsg_status bs_gemv_grouped(const uint32_t* bits, int K, int M, int N, int g, const uint16_t* alpha,
                           const uint16_t* colscale, const void* x, int x_dtype, int B, float* y, int accumulate,
                           void* stream) {
  return bs_gemv_hybrid(bits, K, M, N, g, alpha, colscale, nullptr, 0, nullptr, nullptr, nullptr, x, x_dtype, B, y,
                        accumulate, stream);
}

bsg_status bs_gemv_grouped_multi(const bsg_proj_grouped* projs, int P, int K, int N, int g, const void* x,
                                 int x_dtype, int B, int accumulate, void* stream) {
  if (bad_dtype(x_dtype)) return BSG_ERR_DTYPE;
  if (!projs) return BSG_ERR_NULL;
  if (P < 1 || P > kMaxProj || K < 1 || K > 4 || bad_n(N) || bad_group(N, g) || B < 1 || B > kMaxB)
    return BSG_ERR_SHAPE;
  const bool cs = projs[0].colscale != nullptr;
  for (int i = 0; i < P; ++i) {
    const bsg_proj_grouped& d = projs[i];
    if (d.M < 0 || too_big(K, d.M, N, B) || (size_t)K * d.M * (N / g) >= (1u << 30) ||
        (d.colscale != nullptr) != cs)
      return BSG_ERR_SHAPE;
  }
  if (!x) return BSG_ERR_NULL;
  if (misaligned(x, dtype_size(x_dtype))) return BSG_ERR_ALIGN;
  int np = 0;
  for (int i = 0; i < P; ++i) {
    const bsg_proj_grouped& d = projs[i];
    if (d.M == 0) continue;
    if (!d.bits || !d.alpha || !d.y) return BSG_ERR_NULL;
    if (misaligned(d.bits, 16) || misaligned(d.alpha, 2) || misaligned(d.colscale, 2) || misaligned(d.y, 4))
      return BSG_ERR_ALIGN;
    ++np;
  }
  if (np == 0) return BSG_OK;
  if (np == 1 || B != 1) {
    // one projection, or several batch columns: a product each
    for (int i = 0; i < P; ++i) {
      const bsg_proj_grouped& d = projs[i];
      if (d.M == 0) continue;
      const bsg_status r = bs_gemv_grouped(d.bits, K, d.M, N, g, d.alpha, d.colscale, x, x_dtype, B, d.y,
                                           accumulate, stream);
      if (r != BSG_OK) return r;
    }
    return BSG_OK;
  }
  ProdArgs a{};
  a.x = x;
  a.K = K;
  a.N = N;
  a.ND = N / 32;
  a.B = B;
  a.xdt = x_dtype;
  a.accumulate = accumulate ? 1 : 0;
  a.xvec = (((uintptr_t)x) % 16) == 0;
  a.gsw = g / 32;
  a.ngrp = N / g;
  for (int i = 0; i < P; ++i) {
    const bsg_proj_grouped& d = projs[i];
    if (d.M == 0) continue;
    ProjDesc& e = a.proj[a.np++];
    e.bits = d.bits;
    e.alpha = (const float*)(const void*)d.alpha;  // fp16 group scales, read as such
    e.colscale = d.colscale;
    e.y = d.y;
    e.M = d.M;
    if ((((uintptr_t)d.colscale) % 8) != 0) a.xvec = 0;
  }
  return hip_status(launch_prod_grouped(a, (hipStream_t)stream));
}

size_t binlr_fit_workspace_bytes(int M, int N, int r) {
  if (M < 1 || bad_n(N) || r < 1 || r > kMaxFitRank) return 0;
  return fit_workspace_bytes(M, N, r);
}

bsg_status binlr_fit(const float* W, int M, int N, int r, int rounds, const uint32_t* v_init, uint32_t* U_bits,
                     uint32_t* V_bits, uint16_t* alpha_r_f16, double* alpha, double* alpha_greedy, double* sse,
                     int* solved, void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 1 || bad_n(N) || r < 1 || r > kMaxFitRank || rounds < 1 || rounds > 64) return BSG_ERR_SHAPE;
  if (!W || !v_init || !U_bits || !V_bits || !alpha_r_f16) return BSG_ERR_NULL;
  if (misaligned(W, 4) || misaligned(v_init, 4) || misaligned(U_bits, 16) || misaligned(V_bits, 16) ||
      misaligned(alpha_r_f16, 2) || misaligned(workspace, 256))
    return BSG_ERR_ALIGN;
  if (!workspace || workspace_bytes < fit_workspace_bytes(M, N, r)) return BSG_ERR_WORKSPACE;
  return hip_status(launch_binlr_fit(W, M, N, r, rounds, v_init, U_bits, V_bits, alpha_r_f16, alpha, alpha_greedy,
                                     sse, solved, workspace, (hipStream_t)stream));
}

bsg_status bs_gemv_i8(const uint32_t* bits, int K, int M, int N, const float* alpha, const int8_t* xq,
                      const float* sx, int B, int32_t* acc, float* y, int accumulate, void* stream) {
  if (K < 1 || K > kMaxK || M < 0 || bad_n(N) || N > (1 << 24) || B < 1 || B > kMaxB || too_big(K, M, N, B))
    return BSG_ERR_SHAPE;
  if (M == 0) return BSG_OK;
  if (!bits || !xq || (!acc && !y) || (y && (!alpha || !sx))) return BSG_ERR_NULL;
  if (misaligned(bits, 16) || misaligned(alpha, 4) || misaligned(sx, 4) || misaligned(acc, 4) || misaligned(y, 4))
    return BSG_ERR_ALIGN;
  const ProdPlan p = plan_prod(K, M, N, B, false, true);
  ProdArgs a{};
  a.bits = bits;
  a.alpha = alpha;
  a.xq = xq;
  a.sx = sx;
  a.acc = acc;
  a.y = y;
  a.plane = plane_words(M, N / 32);
  a.K = K;
  a.M = M;
  a.N = N;
  a.ND = N / 32;
  a.B = B;
  a.accumulate = accumulate ? 1 : 0;
  return hip_status(launch_prod_i8(a, p, (hipStream_t)stream));
}

// The low-rank correction on the matrix cores (B >= 4 columns of 16-bit x,
// workspace of binlr_ws(r, B) bytes), two launches:
//   z' = V x, written as w_hi = bf16(w), w_lo = bf16(w - w_hi) for
//   w = alpha_r (.) z' (16 significant bits together), then
//   y += U w_hi + U w_lo (two passes over U's tiles in one launch).
// The products with the bf16 halves are exact and the sums fp32: the split's
// 2^-16 relative rounding is the only error beyond fp32 sums.
static hipError_t lowrank_mfma(const uint32_t* U_bits, const uint32_t* V_bits, const uint16_t* alpha_r, int r,
                               int M, int N, const void* x, int xdt, int B, float* y, void* workspace,
                               hipStream_t st) {
  uint16_t* wh = (uint16_t*)((char*)workspace + align_up((size_t)r * B * 4, 256));
  uint16_t* wl = (uint16_t*)((char*)wh + align_up((size_t)r * B * 2, 256));
  ProdArgs v{};
  v.bits = V_bits;
  v.x = x;
  v.plane = plane_words(r, N / 32);
  v.K = 1;
  v.M = r;
  v.N = N;
  v.ND = N / 32;
  v.B = B;
  v.xdt = xdt;
  v.split_hi = wh;
  v.split_lo = wl;
  v.split_scale = alpha_r;
  hipError_t e = launch_prod_mfma(v, st);
  if (e != hipSuccess) return e;
  ProdArgs u{};
  u.bits = U_bits;
  u.x = wh;
  u.x2 = wl;
  u.y = y;
  u.plane = plane_words(M, r / 32);
  u.K = 1;
  u.M = M;
  u.N = r;
  u.ND = r / 32;
  u.B = B;
  u.xdt = BSG_BF16;
  u.accumulate = 1;
  return launch_prod_mfma(u, st);
}

bsg_status binlr_apply(const uint32_t* U_bits, const uint32_t* V_bits, const uint16_t* alpha_r, int r, int M,
                       int N, const void* x, int x_dtype, int B, float* y, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (bad_dtype(x_dtype)) return BSG_ERR_DTYPE;
  if (r <= 0 || (r % 32) != 0 || M < 0 || bad_n(N) || B < 1 || B > kMaxB || too_big(1, M, N, B) ||
      too_big(1, r, r, B))
    return BSG_ERR_SHAPE;
  if (M == 0) return BSG_OK;
  if (!U_bits || !V_bits || !alpha_r || !x || !y) return BSG_ERR_NULL;
  if (misaligned(U_bits, 16) || misaligned(V_bits, 16) || misaligned(alpha_r, 2) ||
      misaligned(x, dtype_size(x_dtype)) || misaligned(y, 4) || misaligned(workspace, 16))
    return BSG_ERR_ALIGN;
  if (!workspace || workspace_bytes < binlr_ws(r, B)) return BSG_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  float* z = (float*)workspace;
  if (mfma_eligible(B, x_dtype, false)) return hip_status(lowrank_mfma(U_bits, V_bits, alpha_r, r, M, N, x, x_dtype, B, y,
                                                                       workspace, st));

  // z' = V x: a one-base sign product with unit row scales
  ProdArgs v{};
  v.bits = V_bits;
  v.x = x;
  v.y = z;
  v.plane = plane_words(r, N / 32);
  v.K = 1;
  v.M = r;
  v.N = N;
  v.ND = N / 32;
  v.B = B;
  v.xdt = x_dtype;
  v.accumulate = 0;
  v.xvec = xvec_ok(x, nullptr);
  hipError_t e = launch_prod_f(v, plan_prod(1, r, N, B, false, false), st);
  if (e != hipSuccess) return BSG_ERR_HIP;

  // y += U (alpha_r (.) z'): a one-base sign product over the r ranks with
  // unit row scales and alpha_r as its column scales (folded into z' when the
  // kernel stages its activations)
  ProdArgs u{};
  u.bits = U_bits;
  u.colscale = alpha_r;
  u.x = z;
  u.y = y;
  u.plane = plane_words(M, r / 32);
  u.K = 1;
  u.M = M;
  u.N = r;
  u.ND = r / 32;
  u.B = B;
  u.xdt = BSG_F32;
  u.accumulate = 1;
  u.xvec = 1;
  return hip_status(launch_prod_f(u, plan_prod(1, M, r, B, true, false), st));
}

size_t bsg_linear_workspace_bytes(int r, int B) {
  if (r < 0 || (r % 32) != 0 || B < 1 || B > kMaxB) return 0;
  return r > 0 ? binlr_ws(r, B) : 0;
}

bsg_status bsg_linear(const uint32_t* bits, int K, int M, int N, const float* alpha, const uint16_t* colscale,
                      const uint32_t* U_bits, const uint32_t* V_bits, const uint16_t* alpha_r, int r,
                      const int32_t* rows, int ns, const int8_t* q, const uint16_t* s_f16, const void* x,
                      int x_dtype, int B, float* y, int accumulate, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (bad_dtype(x_dtype)) return BSG_ERR_DTYPE;
  if (K < 1 || K > kMaxK || M < 0 || bad_n(N) || B < 1 || B > kMaxB || r < 0 || (r % 32) != 0 || ns < 0 ||
      ns > M || too_big(K, M, N, B) || too_big(1, r, r, B) || (size_t)ns * N >= (1u << 30))
    return BSG_ERR_SHAPE;
  if (M == 0) return BSG_OK;
  if (!bits || !alpha || !x || !y) return BSG_ERR_NULL;
  if (r > 0 && (!U_bits || !V_bits || !alpha_r)) return BSG_ERR_NULL;
  if (ns > 0 && (!rows || !q || !s_f16)) return BSG_ERR_NULL;
  if (misaligned(bits, 16) || misaligned(alpha, 4) || misaligned(colscale, 2) ||
      misaligned(x, dtype_size(x_dtype)) || misaligned(y, 4) || misaligned(U_bits, 16) || misaligned(V_bits, 16) ||
      misaligned(alpha_r, 2) || misaligned(rows, 4) || misaligned(q, 16) || misaligned(s_f16, 2) ||
      misaligned(workspace, 16))
    return BSG_ERR_ALIGN;
  if (r > 0 && (!workspace || workspace_bytes < binlr_ws(r, B))) return BSG_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  float* z = (float*)workspace;

  // B >= 4 columns of 16-bit x: the bases, the low-rank correction and the
  // protected rows as separate launches on the matrix cores (the protected
  // rows on their own kernel), each adding onto y
  if (mfma_eligible(B, x_dtype, colscale != nullptr) ||
      (colscale && !misaligned(colscale, 4) && mfma_cg_ok(B, x_dtype, x, true, 0, M))) {
    ProdArgs a{};
    a.bits = bits;
    a.alpha = alpha;
    a.colscale = colscale;
    a.x = x;
    a.y = y;
    a.plane = plane_words(M, N / 32);
    a.K = K;
    a.M = M;
    a.N = N;
    a.ND = N / 32;
    a.B = B;
    a.xdt = x_dtype;
    a.accumulate = accumulate ? 1 : 0;
    hipError_t e = launch_prod_mfma(a, st);
    if (e == hipSuccess && r > 0) e = lowrank_mfma(U_bits, V_bits, alpha_r, r, M, N, x, x_dtype, B, y, workspace, st);
    if (e == hipSuccess && ns > 0) e = launch_salient_apply(rows, ns, q, s_f16, M, N, x, x_dtype, B, y, st);
    return hip_status(e);
  }

  if (r > 0) {  // z' = V x (unit row scales; alpha_r is applied in the expansion)
    ProdArgs v{};
    v.bits = V_bits;
    v.x = x;
    v.y = z;
    v.plane = plane_words(r, N / 32);
    v.K = 1;
    v.M = r;
    v.N = N;
    v.ND = N / 32;
    v.B = B;
    v.xdt = x_dtype;
    v.xvec = xvec_ok(x, nullptr);
    if (launch_prod_f(v, plan_prod(1, r, N, B, false, false), st) != hipSuccess) return BSG_ERR_HIP;
  }
  ProdArgs a{};
  a.bits = bits;
  a.alpha = alpha;
  a.colscale = colscale;
  a.x = x;
  a.y = y;
  a.plane = plane_words(M, N / 32);
  a.K = K;
  a.M = M;
  a.N = N;
  a.ND = N / 32;
  a.B = B;
  a.xdt = x_dtype;
  a.accumulate = accumulate ? 1 : 0;
  a.xvec = xvec_ok(x, colscale);
  if (r > 0) {
    a.lr_bits = U_bits;
    a.lr_plane = plane_words(M, r / 32);
    a.lr_z = z;
    a.lr_scale = alpha_r;
    a.lr_r = r;
  }
  if (ns > 0) {
    a.sal_n = ns;
    a.sal_rows = rows;
    a.sal_q = q;
    a.sal_s = s_f16;
  }
  return hip_status(launch_prod_f(a, plan_prod(K, M, N, B, colscale != nullptr, false), st));
}

bsg_status salient_int8_apply(const int32_t* rows, int ns, const int8_t* q, const uint16_t* s_f16, int M, int N,
                              const void* x, int x_dtype, int B, float* y, void* stream) {
  if (bad_dtype(x_dtype)) return BSG_ERR_DTYPE;
  if (ns < 0 || M < 0 || N <= 0 || B < 1 || B > kMaxB) return BSG_ERR_SHAPE;
  if (M == 0 || ns == 0) return BSG_OK;
  if (!rows || !q || !s_f16 || !x || !y) return BSG_ERR_NULL;
  if (misaligned(rows, 4) || misaligned(s_f16, 2) || misaligned(x, dtype_size(x_dtype)) || misaligned(y, 4))
    return BSG_ERR_ALIGN;
  return hip_status(launch_salient_apply(rows, ns, q, s_f16, M, N, x, x_dtype, B, y, (hipStream_t)stream));
}

}  // extern "C"
