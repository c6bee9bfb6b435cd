// C ABI of the fused attention forward library: argument checks, kernel
// selection and launch. The operation and the conventions are specified in
// include/attn_fwd.h; the host-side checks and launch geometry are in plan.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "attn_fwd.h"
#include "attn_fwd_kernel.h"
#include "plan.h"

static_assert(attn::BLOCK_M == attn::plan::BLOCK_M, "query tile of the kernel and of the plan");
static_assert(attn::THREADS == attn::plan::THREADS, "workgroup size of the kernel and of the plan");
static_assert(attn::COMBINE_THREADS == attn::plan::COMBINE_THREADS, "combine workgroup size");
static_assert(attn::MAX_SPLITS == ATTN_MAX_SPLITS, "split limit of the kernel and of the header");
static_assert(attn::VAR_RING3 == ATTN_VARIANT_RING3 && attn::VAR_EXP_POLY == ATTN_VARIANT_EXP_POLY &&
                  attn::VAR_WIDE == ATTN_VARIANT_WIDE && attn::VAR_SUBPIPE == ATTN_VARIANT_SUBPIPE &&
                  attn::VAR_SYNC == ATTN_VARIANT_SYNC && attn::VAR_BAR2 == ATTN_VARIANT_BAR2 &&
                  attn::VAR_PROD == ATTN_VARIANT_PROD && attn::VAR_TRIO == ATTN_VARIANT_TRIO &&
                  attn::VAR_QUAD == ATTN_VARIANT_QUAD && attn::VAR_ROT == ATTN_VARIANT_ROT &&
                  attn::VAR_M32 == ATTN_VARIANT_M32,
              "variant flags of the kernel and of the header");

namespace {

thread_local char g_last_error[512] = "";

attn::plan::Msg msg() { return attn::plan::Msg{g_last_error, sizeof(g_last_error)}; }

// Keys per head from which a D = 64 launch runs three compute waves per SIMD:
// non-causal, and causal single passes whose tiles are not folded into pairs;
// folded causal single passes from TRIO_MIN_KEYS_FOLDED keys.
constexpr int TRIO_MIN_KEYS = 2048;
constexpr int TRIO_MIN_KEYS_FOLDED = 8192;

// Sq query rows against Sk keys per head (Sq == Sk for self-attention).
template <int D, bool CAUSAL, int VAR = 0>
int launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
           int Sq, int Sk, float scale, int n_splits, void* workspace, hipStream_t stream) {
  using namespace attn;
  // Non-causal launches at D = 64 over at least 2048 keys run three compute
  // waves per SIMD (VAR_TRIO: 1.5-9% faster for a single pass, equal split);
  // shorter ones (3-14% slower there: one or two 192-key intervals, the last
  // partly idle) keep two. Causal single passes run three waves when their
  // tiles are not folded (B1 H8 S4096 3.9% faster) or from 8192 keys when
  // they are (1-2.5% faster; at 4096 keys 1.7% slower, at 1024 13%: a folded
  // pair's two diagonal intervals leave more of a 192-key interval idle);
  // causal split runs keep two (mixed, -8% to +3%). The synchronous-copy
  // check follows the same choice, so that it mirrors the default kernel.
  if constexpr (D == 64 && (VAR == 0 || VAR == VAR_SYNC)) {
    const bool trio =
        !CAUSAL ? Sk >= TRIO_MIN_KEYS
                : n_splits == 1 && Sk >= (plan::folds(B, H, Sq, 1, n_splits) ? TRIO_MIN_KEYS_FOLDED
                                                                             : TRIO_MIN_KEYS);
    if (trio)
      return launch<D, CAUSAL, VAR | VAR_TRIO>(q, k, v, o, lse, B, H, Sq, Sk, scale, n_splits,
                                               workspace, stream);
  }
  plan::Launch L;
  const int rc = plan::make_launch(B, H, Sq, D, CAUSAL ? 1 : 0, n_splits, &L, msg());
  if (rc != ATTN_OK) return rc;
  const int BH = B * H;
  // Scores are folded in base 2: t = s * |scale| * log2(e). A negative scale
  // is applied by flipping the sign of Q, which is exact in fp16.
  const float c = std::fabs(scale) * 1.4426950408889634f;
  const uint32_t qsign = std::signbit(scale) ? 0x80008000u : 0u;
  const _Float16* qh = static_cast<const _Float16*>(q);
  const _Float16* kh = static_cast<const _Float16*>(k);
  const _Float16* vh = static_cast<const _Float16*>(v);
  _Float16* oh = static_cast<_Float16*>(o);
  constexpr int WG_THREADS = Geometry<D, VAR>::WG_THREADS;  // 512, or 768 with producer waves
  if (L.blocks * WG_THREADS > plan::MAX_WORK_ITEMS)
    return plan::fail(msg(), ATTN_ERR_SHAPE, "grid of %lld workgroups x %d threads exceeds 2^32 work-items",
                      (long long)L.blocks, WG_THREADS);
  if (n_splits == 1) {
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, false, VAR>), dim3((unsigned)L.blocks),
                       dim3(WG_THREADS), 0, stream, qh, kh, vh, oh, lse, BH, Sq, Sk, L.n_qtiles, 1,
                       L.order, c, qsign, nullptr, nullptr);
  } else if constexpr (VAR == 0 || (VAR == VAR_TRIO && !CAUSAL)) {
    float* part_o = static_cast<float*>(workspace);
    float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                               plan::part_o_bytes(B, H, Sq, D, n_splits));
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, true, VAR>), dim3((unsigned)L.blocks),
                       dim3(WG_THREADS), 0, stream, qh, kh, vh, oh, lse, BH, Sq, Sk, L.n_qtiles,
                       n_splits, L.order, c, qsign, part_o, part_lse);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
      return plan::fail(msg(), ATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    const int64_t rows = (int64_t)BH * Sq;
    if (L.combine_runs)
      hipLaunchKernelGGL((attn_combine_runs_kernel<D>), dim3((unsigned)L.combine_blocks),
                         dim3(plan::COMBINE_THREADS), 0, stream, part_o, part_lse, oh, lse, rows,
                         n_splits);
    else
      hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((unsigned)L.combine_blocks),
                         dim3(plan::COMBINE_THREADS), 0, stream, part_o, part_lse, oh, lse, rows,
                         n_splits);
  } else {
    return plan::fail(msg(), ATTN_ERR_UNSUPPORTED, "split runs of kernel variant %d are not built", VAR);
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return plan::fail(msg(), ATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return ATTN_OK;
}

int dispatch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int Sq, int Sk, int D, float scale, int causal, int n_splits, void* workspace,
             void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (D == 64)
    return causal ? launch<64, true>(q, k, v, o, lse, B, H, Sq, Sk, scale, n_splits, workspace, st)
                  : launch<64, false>(q, k, v, o, lse, B, H, Sq, Sk, scale, n_splits, workspace, st);
  return causal ? launch<128, true>(q, k, v, o, lse, B, H, Sq, Sk, scale, n_splits, workspace, st)
                : launch<128, false>(q, k, v, o, lse, B, H, Sq, Sk, scale, n_splits, workspace, st);
}

// Single pass of a compiled kernel variant (attn::VAR_* flags), or
// ATTN_ERR_UNSUPPORTED for a combination that is not built.
template <int D, int VAR>
int launch_variant(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int H, int S, float scale, int causal, hipStream_t st) {
  return causal ? launch<D, true, VAR>(q, k, v, o, lse, B, H, S, S, scale, 1, nullptr, st)
                : launch<D, false, VAR>(q, k, v, o, lse, B, H, S, S, scale, 1, nullptr, st);
}

int dispatch_variant(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int S, int D, float scale, int causal, int variant, void* stream) {
  using namespace attn;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (D == 64) {
    switch (variant) {
      case 0: return launch_variant<64, 0>(q, k, v, o, lse, B, H, S, scale, causal, st);
      case VAR_RING3: return launch_variant<64, VAR_RING3>(q, k, v, o, lse, B, H, S, scale, causal, st);
      case VAR_EXP_POLY: return launch_variant<64, VAR_EXP_POLY>(q, k, v, o, lse, B, H, S, scale, causal, st);
      case VAR_WIDE: return launch_variant<64, VAR_WIDE>(q, k, v, o, lse, B, H, S, scale, causal, st);
      case VAR_SUBPIPE: return launch_variant<64, VAR_SUBPIPE>(q, k, v, o, lse, B, H, S, scale, causal, st);
      case VAR_SYNC: return launch_variant<64, VAR_SYNC>(q, k, v, o, lse, B, H, S, scale, causal, st);
      case VAR_BAR2: return launch_variant<64, VAR_BAR2>(q, k, v, o, lse, B, H, S, scale, causal, st);
      case VAR_PROD: return launch_variant<64, VAR_PROD>(q, k, v, o, lse, B, H, S, scale, causal, st);
      case VAR_TRIO: return launch_variant<64, VAR_TRIO>(q, k, v, o, lse, B, H, S, scale, causal, st);
      case VAR_QUAD: return launch_variant<64, VAR_QUAD>(q, k, v, o, lse, B, H, S, scale, causal, st);
      case VAR_ROT: return launch_variant<64, VAR_ROT>(q, k, v, o, lse, B, H, S, scale, causal, st);
      case VAR_M32: return launch_variant<64, VAR_M32>(q, k, v, o, lse, B, H, S, scale, causal, st);
      case VAR_M32 | VAR_TRIO:
        return launch_variant<64, VAR_M32 | VAR_TRIO>(q, k, v, o, lse, B, H, S, scale, causal, st);
      default: break;
    }
  } else {
    switch (variant) {
      case 0: return launch_variant<128, 0>(q, k, v, o, lse, B, H, S, scale, causal, st);
      case VAR_EXP_POLY: return launch_variant<128, VAR_EXP_POLY>(q, k, v, o, lse, B, H, S, scale, causal, st);
      case VAR_SYNC: return launch_variant<128, VAR_SYNC>(q, k, v, o, lse, B, H, S, scale, causal, st);
      default: break;
    }
  }
  return attn::plan::fail(msg(), ATTN_ERR_UNSUPPORTED,
                          "kernel variant %d is not built for D=%d (D=64: 0, %d, %d, %d, %d, %d, %d, %d, %d, "
                          "%d, %d, %d, %d; D=128: 0, %d, %d)", variant, D, ATTN_VARIANT_RING3,
                          ATTN_VARIANT_EXP_POLY, ATTN_VARIANT_WIDE, ATTN_VARIANT_SUBPIPE,
                          ATTN_VARIANT_SYNC, ATTN_VARIANT_BAR2, ATTN_VARIANT_PROD, ATTN_VARIANT_TRIO,
                          ATTN_VARIANT_QUAD, ATTN_VARIANT_ROT, ATTN_VARIANT_M32,
                          ATTN_VARIANT_M32 | ATTN_VARIANT_TRIO, ATTN_VARIANT_EXP_POLY,
                          ATTN_VARIANT_SYNC);
}

// Checks shared by the entry points (Sq query rows against Sk keys).
int check_common(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 int B, int H, int Sq, int Sk, int D, float scale, int causal, int n_splits) {
  const int rc = attn::plan::check_args(q, k, v, o, lse, B, H, Sq, Sk, D, scale, causal, msg());
  if (rc != ATTN_OK) return rc;
  if (n_splits < 1 || n_splits > ATTN_MAX_SPLITS)
    return attn::plan::fail(msg(), ATTN_ERR_ARG, "n_splits must be in [1, %d] (got %d)",
                            ATTN_MAX_SPLITS, n_splits);
  if (n_splits > 1 && attn::plan::workspace_size(B, H, Sq, D, n_splits) == 0)
    return attn::plan::fail(msg(), ATTN_ERR_SHAPE, "workspace size overflows");
  attn::plan::Launch L;  // grid limits, checked before anything is enqueued
  return attn::plan::make_launch(B, H, Sq, D, causal, n_splits, &L, msg());
}

// The workspace checks of the split entry points (n_splits > 1).
int check_workspace(const void* workspace, size_t workspace_size, int B, int H, int Sq, int D,
                    int n_splits) {
  if (n_splits == 1) return ATTN_OK;
  if (!workspace)
    return attn::plan::fail(msg(), ATTN_ERR_NULL, "workspace is NULL with n_splits=%d", n_splits);
  if (!attn::plan::aligned(workspace, 16))
    return attn::plan::fail(msg(), ATTN_ERR_ALIGN, "workspace must be 16-byte aligned");
  const size_t need = attn::plan::workspace_size(B, H, Sq, D, n_splits);
  if (workspace_size < need)
    return attn::plan::fail(msg(), ATTN_ERR_ARG,
                            "workspace of %zu bytes is smaller than the %zu bytes needed",
                            workspace_size, need);
  return ATTN_OK;
}

// ---------------------------------------------------------------------------
// Static scratch of the allocation-free split-KV entry point. Each device
// holds its own copy of this array from the library's load until the process
// ends. Host code must never pass `scratch` itself to a kernel (on the host
// the name is only a stand-in for the symbol): its device address is looked up
// once per device with hipGetSymbolAddress and kept in g_scratch_ptr.
constexpr int MAX_DEVICES = 64;
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];
void* g_scratch_ptr[MAX_DEVICES] = {};
std::mutex g_scratch_mutex;

// Device address of this device's scratch array (looked up on the first call
// on the device, with the device current). ATTN_OK or ATTN_ERR_HIP.
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess)
    return attn::plan::fail(msg(), ATTN_ERR_HIP, "hipGetDevice failed: %s",
                            hipGetErrorString(err));
  if (dev < 0 || dev >= MAX_DEVICES)
    return attn::plan::fail(msg(), ATTN_ERR_HIP, "device %d is outside the %d supported", dev,
                            MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !p)
      return attn::plan::fail(msg(), ATTN_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s",
                              hipGetErrorString(err));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int S, int D, float scale, int causal, void* stream) {
  g_last_error[0] = '\0';
  const int rc = check_common(q, k, v, o, lse, B, H, S, S, D, scale, causal, 1);
  if (rc != ATTN_OK) return rc;
  return dispatch(q, k, v, o, lse, B, H, S, S, D, scale, causal, 1, nullptr, stream);
}

int attn_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int S, int D, float scale, int causal, int variant, void* stream) {
  g_last_error[0] = '\0';
  const int rc = check_common(q, k, v, o, lse, B, H, S, S, D, scale, causal, 1);
  if (rc != ATTN_OK) return rc;
  return dispatch_variant(q, k, v, o, lse, B, H, S, D, scale, causal, variant, stream);
}

size_t attn_fwd_splitkv_workspace_size(int B, int H, int S, int D, int n_splits) {
  return attn::plan::workspace_size(B, H, S, D, n_splits);
}

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int S, int D, float scale, int causal, int n_splits,
                     void* workspace, size_t workspace_size, void* stream) {
  g_last_error[0] = '\0';
  int rc = check_common(q, k, v, o, lse, B, H, S, S, D, scale, causal, n_splits);
  if (rc != ATTN_OK) return rc;
  rc = check_workspace(workspace, workspace_size, B, H, S, D, n_splits);
  if (rc != ATTN_OK) return rc;
  return dispatch(q, k, v, o, lse, B, H, S, S, D, scale, causal, n_splits, workspace, stream);
}

int attn_fwd_kvcache(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int S_q, int S_k, int D, float scale, int causal, int n_splits,
                     void* workspace, size_t workspace_size, void* stream) {
  g_last_error[0] = '\0';
  int rc = check_common(q, k, v, o, lse, B, H, S_q, S_k, D, scale, causal, n_splits);
  if (rc != ATTN_OK) return rc;
  rc = check_workspace(workspace, workspace_size, B, H, S_q, D, n_splits);
  if (rc != ATTN_OK) return rc;
  return dispatch(q, k, v, o, lse, B, H, S_q, S_k, D, scale, causal, n_splits, workspace, stream);
}

int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int S, int D, float scale, int causal, int n_splits,
                             void* stream) {
  g_last_error[0] = '\0';
  const int rc = check_common(q, k, v, o, lse, B, H, S, S, D, scale, causal, n_splits);
  if (rc != ATTN_OK) return rc;
  void* ws = nullptr;
  if (n_splits > 1) {
    const size_t need = attn::plan::workspace_size(B, H, S, D, n_splits);
    if (need > (size_t)ATTN_NOALLOC_SCRATCH_BYTES)
      return attn::plan::fail(msg(), ATTN_ERR_ARG,
                              "n_splits=%d needs %zu bytes of partial results, more than the "
                              "%u-byte static scratch buffer; use attn_fwd_splitkv with a "
                              "workspace, or fewer splits", n_splits, need,
                              (unsigned)ATTN_NOALLOC_SCRATCH_BYTES);
    const int src = scratch_of_current_device(&ws);
    if (src != ATTN_OK) return src;
  }
  // Every partial result the combine kernel reads is written by the split
  // kernel of the same call first, so the scratch needs no clearing.
  return dispatch(q, k, v, o, lse, B, H, S, S, D, scale, causal, n_splits, ws, stream);
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
