// Host side of the attention entry points: argument checks and launch
// geometry (work order, grid sizes, workspace layout). Plain C++ with no HIP
// types, so that host tests can build and run it under AddressSanitizer and
// UndefinedBehaviorSanitizer; attn_fwd.hip uses it before any HIP call.
#pragma once

#include <cmath>
#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <cstdio>

#include "attn_fwd.h"
#include "work_order.h"

namespace attn {
namespace plan {

constexpr int BLOCK_M = 128;          // query rows per workgroup of the attention kernel
constexpr int THREADS = 512;          // threads per workgroup of the attention kernel
constexpr int COMBINE_THREADS = 256;  // threads per workgroup of the combine kernel
constexpr int64_t COMBINE_MAX_BLOCKS = 1 << 16;  // the combine kernel strides over rows
constexpr int64_t COMBINE_FILL_THREADS = 256 * 256;  // threads that fill 256 CUs once
// Causal launches are folded (ORDER_FOLDED) from this many workgroups on:
// the CU count of MI355X, one workgroup per CU.
constexpr int64_t FOLD_MIN_WORKGROUPS = 256;
// A dispatch's work-items (blocks * threads) must fit 32 bits.
constexpr int64_t MAX_WORK_ITEMS = 0xffffffffLL;

// Error message sink: the entry points pass their thread-local buffer.
struct Msg {
  char* buf;
  size_t cap;
};

int fail(Msg m, int status, const char* fmt, ...) __attribute__((format(printf, 3, 4)));

inline int fail(Msg m, int status, const char* fmt, ...) {
  if (m.buf && m.cap) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(m.buf, m.cap, fmt, ap);
    va_end(ap);
  }
  return status;
}

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Checks shared by the entry points (S_q query rows, S_k keys per head);
// ATTN_OK if the call may proceed.
inline int check_args(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, int B, int H, int Sq, int Sk, int D, float scale,
                      int causal, Msg m) {
  if (!q || !k || !v || !o || !lse)
    return fail(m, ATTN_ERR_NULL, "null pointer: q=%p k=%p v=%p o=%p lse=%p", q, k, v, o,
                static_cast<const void*>(lse));
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1)
    return fail(m, ATTN_ERR_SHAPE, "B, H and the sequence lengths must be >= 1 "
                "(got B=%d H=%d S_q=%d S_k=%d)", B, H, Sq, Sk);
  if (D != 64 && D != 128)
    return fail(m, ATTN_ERR_UNSUPPORTED, "head dimension D=%d is not supported (64 or 128)", D);
  const int Smax = Sq > Sk ? Sq : Sk;
  const double elems = (double)B * H * (double)Smax * D;
  if (elems >= 1099511627776.0 || (int64_t)B * H > 0x7fffffff)
    return fail(m, ATTN_ERR_SHAPE, "B*H*S*D = %.0f elements exceeds 2^40", elems);
  if ((int64_t)Smax * D * 2 > 0x7fffffff)
    return fail(m, ATTN_ERR_SHAPE,
                "one head's tensor (S*D*2 = %lld bytes) exceeds 2^31 - 1 bytes",
                (long long)Smax * D * 2);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(m, ATTN_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(m, ATTN_ERR_ALIGN, "lse must be 4-byte aligned");
  if (causal != 0 && causal != 1)
    return fail(m, ATTN_ERR_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (causal && Sq > Sk)
    return fail(m, ATTN_ERR_SHAPE,
                "causal with S_q=%d > S_k=%d leaves the first query rows without keys", Sq, Sk);
  if (!std::isfinite(scale)) return fail(m, ATTN_ERR_ARG, "scale must be finite");
  return ATTN_OK;
}

// Bytes of the split-KV partial results: o/d in fp32 [n_splits][B*H][S_q][D],
// then m + log2(d) in fp32 [n_splits][B*H][S_q].
inline int64_t part_o_bytes(int B, int H, int Sq, int D, int n_splits) {
  return (int64_t)n_splits * B * H * Sq * D * 4;
}
inline int64_t workspace_bytes(int B, int H, int Sq, int D, int n_splits) {
  return part_o_bytes(B, H, Sq, D, n_splits) + (int64_t)n_splits * B * H * Sq * 4;
}

// Workspace bytes for a split launch, 0 for n_splits == 1 or out-of-range
// arguments (the value attn_fwd_splitkv_workspace_size reports).
inline size_t workspace_size(int B, int H, int Sq, int D, int n_splits) {
  if (B < 1 || H < 1 || Sq < 1 || (D != 64 && D != 128) || n_splits < 1 ||
      n_splits > ATTN_MAX_SPLITS)
    return 0;
  if (n_splits == 1) return 0;
  const double bytes = (double)n_splits * B * H * (double)Sq * (D + 1) * 4.0;
  if (bytes >= 9.0e18) return 0;
  return (size_t)workspace_bytes(B, H, Sq, D, n_splits);
}

struct Launch {
  int order;               // work order of the attention kernel (work_order.h)
  int n_qtiles;            // query tiles per head
  int64_t blocks;          // workgroups of the attention kernel
  int64_t combine_blocks;  // workgroups of the combine kernel (n_splits > 1), else 0
  int combine_runs;        // 1: the wave-per-row combine (few rows), 0: thread per row
};

// Whether a single-pass causal launch folds its query tiles into mirror pairs
// (ORDER_FOLDED): when the pairs alone fill the CUs.
inline bool folds(int B, int H, int Sq, int causal, int n_splits) {
  const int64_t n_qtiles = ((int64_t)Sq + BLOCK_M - 1) / BLOCK_M;
  return causal && n_splits == 1 && (int64_t)B * H * ((n_qtiles + 1) / 2) >= FOLD_MIN_WORKGROUPS;
}

// Launch geometry of one call; ATTN_ERR_SHAPE if a grid does not fit a
// dispatch. Arguments are already checked.
inline int make_launch(int B, int H, int Sq, int D, int causal, int n_splits, Launch* out,
                       Msg m) {
  const int64_t BH = (int64_t)B * H;
  const int n_qtiles = (int)(((int64_t)Sq + BLOCK_M - 1) / BLOCK_M);
  // Single pass: non-causal work is uniform, so the order serves L2 locality
  // alone (head-major per XCD). Causal tiles range from 1 to n_qtiles key
  // tile pairs: folded mirror pairs equalise them when there are enough to
  // fill the CUs, else the heaviest tiles go first.
  int order = ORDER_TILES;
  if (n_splits == 1 && !causal)
    order = ORDER_HEADS;
  else if (folds(B, H, Sq, causal, n_splits))
    order = ORDER_FOLDED;
  const int64_t per_head = order == ORDER_FOLDED ? (n_qtiles + 1) / 2 : n_qtiles;
  const int64_t blocks = BH * per_head * n_splits;
  // (This also keeps workgroup ids, which the work order handles as ints,
  // below 2^23.)
  if (blocks * THREADS > MAX_WORK_ITEMS)
    return fail(m, ATTN_ERR_SHAPE, "grid of %lld workgroups x %d threads exceeds 2^32 work-items",
                (long long)blocks, THREADS);
  // Combine: with a thread per row and 4 columns, a launch whose threads do
  // not fill the CUs once (few rows: decode) would merge its runs one after
  // another; it takes a wave per row instead, all runs loaded at once.
  int64_t cblocks = 0;
  int runs = 0;
  if (n_splits > 1) {
    const int64_t rows = BH * Sq;
    const int64_t threads = rows * (D / 4);
    runs = threads < COMBINE_FILL_THREADS ? 1 : 0;
    const int64_t per_block = runs ? COMBINE_THREADS / 64 : COMBINE_THREADS;
    const int64_t items = runs ? rows : threads;
    cblocks = (items + per_block - 1) / per_block;
    if (cblocks > COMBINE_MAX_BLOCKS) cblocks = COMBINE_MAX_BLOCKS;
  }
  out->order = order;
  out->n_qtiles = n_qtiles;
  out->blocks = blocks;
  out->combine_blocks = cblocks;
  out->combine_runs = runs;
  return ATTN_OK;
}

}  // namespace plan
}  // namespace attn
