// C ABI of the fused attention forward library: argument checks, kernel
// selection and launch. The operation and the conventions are specified in
// include/attn_fwd.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "attn_fwd.h"
#include "attn_fwd_kernel.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

template <int D, bool CAUSAL>
int launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
           int S, float scale, hipStream_t stream) {
  using namespace attn;
  const int BH = B * H;
  const int n_qtiles = (S + BLOCK_M - 1) / BLOCK_M;
  const int64_t blocks = (int64_t)BH * n_qtiles;
  if (blocks > 0x7fffffff) return fail(ATTN_ERR_SHAPE, "grid of %lld workgroups is too large",
                                       (long long)blocks);
  // Scores are folded in base 2: t = s * |scale| * log2(e). A negative scale
  // is applied by flipping the sign of Q, which is exact in fp16.
  const float c = std::fabs(scale) * 1.4426950408889634f;
  const uint32_t qsign = std::signbit(scale) ? 0x80008000u : 0u;
  hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(THREADS), 0,
                     stream, static_cast<const _Float16*>(q), static_cast<const _Float16*>(k),
                     static_cast<const _Float16*>(v), static_cast<_Float16*>(o), lse, BH, S,
                     n_qtiles, c, qsign);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return fail(ATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int S, int D, float scale, int causal, void* stream) {
  g_last_error[0] = '\0';
  if (!q || !k || !v || !o || !lse)
    return fail(ATTN_ERR_NULL, "null pointer: q=%p k=%p v=%p o=%p lse=%p", q, k, v, o,
                static_cast<void*>(lse));
  if (B < 1 || H < 1 || S < 1)
    return fail(ATTN_ERR_SHAPE, "B, H and S must be >= 1 (got B=%d H=%d S=%d)", B, H, S);
  if (D != 64 && D != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "head dimension D=%d is not supported (64 or 128)", D);
  const double elems = (double)B * H * (double)S * D;
  if (elems >= 1099511627776.0 || (int64_t)B * H > 0x7fffffff)
    return fail(ATTN_ERR_SHAPE, "B*H*S*D = %.0f elements exceeds 2^40", elems);
  if ((int64_t)S * D * 2 > 0x7fffffff)
    return fail(ATTN_ERR_SHAPE, "one head's tensor (S*D*2 = %lld bytes) exceeds 2^31 - 1 bytes",
                (long long)S * D * 2);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(ATTN_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(ATTN_ERR_ALIGN, "lse must be 4-byte aligned");
  if (causal != 0 && causal != 1)
    return fail(ATTN_ERR_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (!std::isfinite(scale)) return fail(ATTN_ERR_ARG, "scale must be finite");

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (D == 64)
    return causal ? launch<64, true>(q, k, v, o, lse, B, H, S, scale, st)
                  : launch<64, false>(q, k, v, o, lse, B, H, S, scale, st);
  return causal ? launch<128, true>(q, k, v, o, lse, B, H, S, scale, st)
                : launch<128, false>(q, k, v, o, lse, B, H, S, scale, st);
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_NULL: return "ATTN_ERR_NULL";
    case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_ALIGN: return "ATTN_ERR_ALIGN";
    case ATTN_ERR_ARG: return "ATTN_ERR_ARG";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    default: return "ATTN_ERR_UNKNOWN";
  }
}

const char* attn_last_error(void) { return g_last_error; }

int attn_version(void) { return ATTN_FWD_ABI_VERSION; }

}  // extern "C"
