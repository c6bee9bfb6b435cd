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

// Bytes of the split-KV partial results: o/d in fp32 [n_splits][B*H][S][D],
// then m + log2(d) in fp32 [n_splits][B*H][S].
int64_t part_o_bytes(int B, int H, int S, int D, int n_splits) {
  return (int64_t)n_splits * B * H * S * D * 4;
}
int64_t workspace_bytes(int B, int H, int S, int D, int n_splits) {
  return part_o_bytes(B, H, S, D, n_splits) + (int64_t)n_splits * B * H * S * 4;
}

// Causal launches are folded (ORDER_FOLDED) from this many workgroups on:
// the CU count of MI355X, one workgroup per CU.
constexpr int64_t FOLD_MIN_WORKGROUPS = 256;

template <int D, bool CAUSAL>
int launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
           int S, float scale, int n_splits, void* workspace, hipStream_t stream) {
  using namespace attn;
  const int BH = B * H;
  const int n_qtiles = (S + BLOCK_M - 1) / BLOCK_M;
  // Single pass: non-causal work is uniform, so the order serves L2 locality
  // alone (head-major per XCD). Causal tiles range from 1 to n_qtiles key
  // tile pairs: folded mirror pairs equalise them when there are enough to
  // fill the CUs, else the heaviest tiles go first.
  int order = ORDER_TILES;
  if (n_splits == 1) {
    if (!CAUSAL)
      order = ORDER_HEADS;
    else if ((int64_t)BH * ((n_qtiles + 1) / 2) >= FOLD_MIN_WORKGROUPS)
      order = ORDER_FOLDED;
  }
  const int64_t blocks = (int64_t)BH * (order == ORDER_FOLDED ? (n_qtiles + 1) / 2 : n_qtiles) *
                         n_splits;
  if (blocks > 0x7fffffff) return fail(ATTN_ERR_SHAPE, "grid of %lld workgroups is too large",
                                       (long long)blocks);
  // Scores are folded in base 2: t = s * |scale| * log2(e). A negative scale
  // is applied by flipping the sign of Q, which is exact in fp16.
  const float c = std::fabs(scale) * 1.4426950408889634f;
  const uint32_t qsign = std::signbit(scale) ? 0x80008000u : 0u;
  const _Float16* qh = static_cast<const _Float16*>(q);
  const _Float16* kh = static_cast<const _Float16*>(k);
  const _Float16* vh = static_cast<const _Float16*>(v);
  _Float16* oh = static_cast<_Float16*>(o);
  if (n_splits == 1) {
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, false>), dim3((unsigned)blocks), dim3(THREADS),
                       0, stream, qh, kh, vh, oh, lse, BH, S, n_qtiles, 1, order, c, qsign,
                       nullptr, nullptr);
  } else {
    float* part_o = static_cast<float*>(workspace);
    float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                               part_o_bytes(B, H, S, D, n_splits));
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, true>), dim3((unsigned)blocks), dim3(THREADS),
                       0, stream, qh, kh, vh, oh, lse, BH, S, n_qtiles, n_splits, order, c,
                       qsign, part_o, part_lse);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
      return fail(ATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    const int64_t rows = (int64_t)BH * S;
    const int64_t cblocks = (rows * (D / 4) + 255) / 256;
    hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((unsigned)cblocks), dim3(256), 0, stream,
                       part_o, part_lse, oh, lse, rows, n_splits);
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return fail(ATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return ATTN_OK;
}

// Checks shared by the entry points; ATTN_OK if the call may proceed.
int check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
               int B, int H, int S, int D, float scale, int causal) {
  if (!q || !k || !v || !o || !lse)
    return fail(ATTN_ERR_NULL, "null pointer: q=%p k=%p v=%p o=%p lse=%p", q, k, v, o,
                static_cast<const void*>(lse));
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
  return ATTN_OK;
}

int dispatch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int S, int D, float scale, int causal, int n_splits, void* workspace,
             void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (D == 64)
    return causal ? launch<64, true>(q, k, v, o, lse, B, H, S, scale, n_splits, workspace, st)
                  : launch<64, false>(q, k, v, o, lse, B, H, S, scale, n_splits, workspace, st);
  return causal ? launch<128, true>(q, k, v, o, lse, B, H, S, scale, n_splits, workspace, st)
                : launch<128, false>(q, k, v, o, lse, B, H, S, scale, n_splits, workspace, st);
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int S, int D, float scale, int causal, void* stream) {
  g_last_error[0] = '\0';
  const int rc = check_args(q, k, v, o, lse, B, H, S, D, scale, causal);
  if (rc != ATTN_OK) return rc;
  return dispatch(q, k, v, o, lse, B, H, S, D, scale, causal, 1, nullptr, stream);
}

size_t attn_fwd_splitkv_workspace_size(int B, int H, int S, int D, int n_splits) {
  if (B < 1 || H < 1 || S < 1 || (D != 64 && D != 128) || n_splits < 1 ||
      n_splits > ATTN_MAX_SPLITS)
    return 0;
  if (n_splits == 1) return 0;
  const double bytes = (double)n_splits * B * H * (double)S * (D + 1) * 4.0;
  if (bytes >= 9.0e18) return 0;
  return (size_t)workspace_bytes(B, H, S, D, n_splits);
}

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int S, int D, float scale, int causal, int n_splits,
                     void* workspace, size_t workspace_size, void* stream) {
  g_last_error[0] = '\0';
  const int rc = check_args(q, k, v, o, lse, B, H, S, D, scale, causal);
  if (rc != ATTN_OK) return rc;
  if (n_splits < 1 || n_splits > ATTN_MAX_SPLITS)
    return fail(ATTN_ERR_ARG, "n_splits must be in [1, %d] (got %d)", ATTN_MAX_SPLITS, n_splits);
  if (n_splits > 1) {
    if (!workspace) return fail(ATTN_ERR_NULL, "workspace is NULL with n_splits=%d", n_splits);
    if (!aligned(workspace, 16)) return fail(ATTN_ERR_ALIGN, "workspace must be 16-byte aligned");
    const size_t need = attn_fwd_splitkv_workspace_size(B, H, S, D, n_splits);
    if (need == 0) return fail(ATTN_ERR_SHAPE, "workspace size overflows");
    if (workspace_size < need)
      return fail(ATTN_ERR_ARG, "workspace of %zu bytes is smaller than the %zu bytes needed",
                  workspace_size, need);
  }
  return dispatch(q, k, v, o, lse, B, H, S, D, scale, causal, n_splits, workspace, stream);
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
