/*
 * attn_fwd.h -- C ABI of the fused exact-attention forward library
 * (libattn_fwd.so, HIP kernels for AMD Instinct MI355X / gfx950).
 *
 * Operation (scaled dot-product attention, forward only):
 *
 *   O[b,h,i,:] = sum_j softmax_j(scale * Q[b,h,i,:] . K[b,h,j,:]) * V[b,h,j,:]
 *   LSE[b,h,i] = ln sum_j exp(scale * Q[b,h,i,:] . K[b,h,j,:])
 *
 * over the visible keys j: every j < S, or j <= i when causal. This is the
 * attention of "Learning FlashAttention the Hard Way, Part 2" (workload
 * definitions: fp16 Q, K, V of shape [B,H,S,D], default scale 1/sqrt(D)),
 * computed as one streaming kernel that folds K/V tiles into a running
 * (max, denominator, unnormalised output) carrier held in registers (Part 2,
 * introduction and Moves 1-4), so that scores never reach device memory.
 * The causal mask and the LSE output are additions to the pages' problem
 * statement: key j is hidden from query i when j > i (the diagonal is
 * visible), and LSE is in natural-log units of the scaled scores.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers on the current HIP device. The
 *    caller allocates and owns every buffer; the library allocates nothing,
 *    frees nothing, never synchronises and never changes the current device.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *    void*; NULL means the default stream). Buffers must stay valid until
 *    that work completes. Kernel faults surface at the caller's next
 *    synchronisation on the stream, not in the return code.
 *  - Errors are returned as attn_status codes. Argument checks run on the
 *    host before any HIP call, so an invalid call touches no device state.
 *    A thread-local message with details is available from attn_last_error().
 *  - The library keeps no state besides that message and is reentrant.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_FWD_ABI_VERSION 3

/* Largest n_splits accepted by attn_fwd_splitkv. */
#define ATTN_MAX_SPLITS 64

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,         /* a required pointer is NULL                   */
  ATTN_ERR_SHAPE = 2,        /* B, H or S < 1, or the tensors are too large  */
  ATTN_ERR_UNSUPPORTED = 3,  /* head dimension D not in {64, 128}            */
  ATTN_ERR_ALIGN = 4,        /* q/k/v/o not 16-byte or lse not 4-byte aligned*/
  ATTN_ERR_ARG = 5,          /* causal not 0/1, or scale not finite          */
  ATTN_ERR_HIP = 6           /* the HIP launch reported an error             */
} attn_status;

/*
 * attn_fwd -- fused attention forward.
 *
 *  q, k, v : const fp16 (IEEE binary16), contiguous row-major [B, H, S, D];
 *            element (b,h,s,d) at offset ((b*H + h)*S + s)*D + d.
 *            Q, K and V share one shape (self-attention, S_q = S_k = S).
 *  o       : fp16 output, same shape and layout as q. Written with
 *            round-to-nearest-even from the fp32 result.
 *  lse     : fp32 output [B, H, S]; element (b,h,s) at (b*H + h)*S + s.
 *  B, H, S : batch, heads, sequence length; each >= 1, B*H*S*D < 2^40 and
 *            one head's tensor fits 32-bit byte offsets (S*D*2 < 2^31).
 *            S need not be a multiple of any tile size.
 *  D       : head dimension, 64 or 128.
 *  scale   : softmax scale applied to Q.K (finite; any sign; 0 gives uniform
 *            weights). Callers wanting the usual default pass 1/sqrt(D).
 *  causal  : 0 = every key visible, 1 = key j hidden from query i if j > i.
 *  stream  : hipStream_t as void* (NULL = default stream).
 *
 *  o and lse must not alias q, k, v or each other. Non-finite inputs are not
 *  checked and propagate to the outputs. Products are exact and accumulate
 *  in fp32; the softmax runs in fp32 in base 2 with the scale folded in; the
 *  probabilities are rounded to fp16 for the P.V product.
 *
 *  Returns ATTN_OK once the kernel is enqueued, or an error code (nothing is
 *  enqueued on error).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int S, int D, float scale, int causal, void* stream);

/*
 * attn_fwd_splitkv -- the same operation with each query tile's keys cut into
 * n_splits runs (split-KV), folded by separate workgroups and merged by a
 * second kernel: more workgroups where B*H*ceil(S/128) leaves the GPU idle,
 * and shorter critical paths for the long query tiles of a causal mask. The
 * pages name this pairing of a split reduction with a combine kernel ("Learning
 * FlashAttention the Hard Way, Part 2": The Move Stack, its REDUCE knob, and
 * the Flash-Decoding reference, split-KV as split-K of the (m, d, o)
 * carrier), and the merge is the carrier's associative combine.
 *
 *  q ... causal : as attn_fwd (same layouts, same checks, same status codes).
 *  n_splits     : 1 .. ATTN_MAX_SPLITS. Each query tile's key range, in whole
 *                 pairs of 64-key tiles, is cut into n_splits near-equal runs;
 *                 runs may be empty. n_splits = 1 is exactly attn_fwd (the
 *                 workspace is then not used and may be NULL).
 *  workspace    : device buffer of at least workspace_size bytes, 16-byte
 *                 aligned, owned by the caller; its contents on entry do not
 *                 matter and are overwritten (per run and row: o/d in fp32 and
 *                 m + log2 d in fp32). It must not alias any other argument,
 *                 and two calls in flight must not share it.
 *  workspace_size : its size in bytes, >= attn_fwd_splitkv_workspace_size().
 *
 *  Returns ATTN_OK once both kernels are enqueued on `stream`; ATTN_ERR_ARG
 *  for n_splits out of range or a short workspace, ATTN_ERR_NULL for a NULL
 *  workspace with n_splits > 1, ATTN_ERR_ALIGN for a misaligned one. Results
 *  agree with attn_fwd to rounding, not bitwise.
 */
int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int S, int D, float scale, int causal, int n_splits,
                     void* workspace, size_t workspace_size, void* stream);

/* Kernel variants for attn_fwd_variant (measured alternatives of the single
 * pass; results agree with attn_fwd to rounding, not bitwise). */
#define ATTN_VARIANT_DEFAULT 0   /* the kernel attn_fwd runs                    */
#define ATTN_VARIANT_RING3 1     /* D = 64: three-slot K/V ring in LDS, copies   */
                                 /* issued two key intervals ahead of their use  */
#define ATTN_VARIANT_EXP_POLY 2  /* one exponential in four on the FMA path     */
#define ATTN_VARIANT_WIDE 4      /* D = 64: 64-row waves over four 32-key tiles  */
#define ATTN_VARIANT_SUBPIPE 8   /* D = 64: the two 16-row sub-tiles of a wave   */
                                 /* pipelined against each other in one interval */
#define ATTN_VARIANT_SYNC 16     /* every K/V copy waited for and barriered      */
                                 /* right after its issue (ring-protocol check)  */
#define ATTN_VARIANT_BAR2 32     /* D = 64: one workgroup barrier per two key    */
                                 /* intervals, four-slot K/V ring                */
#define ATTN_VARIANT_PROD 64     /* D = 64: four producer waves issue the K/V    */
                                 /* copies (768-thread workgroups)               */
#define ATTN_VARIANT_TRIO 128    /* D = 64: twelve compute waves, three per SIMD, */
                                 /* over 192-key intervals                       */
#define ATTN_VARIANT_QUAD 256    /* D = 64: sixteen compute waves, four per SIMD, */
                                 /* on 32-key tiles                              */
#define ATTN_VARIANT_ROT 512     /* D = 64: three waves per SIMD whose phases are */
                                 /* rotated by a third of an interval            */
#define ATTN_VARIANT_M32 1024    /* D = 64: 32x32x16 MFMAs; alone (two waves per  */
                                 /* SIMD) or with ATTN_VARIANT_TRIO (three)      */

/*
 * attn_fwd_variant -- attn_fwd with a chosen compiled variant of the kernel,
 * for measurement and testing of the alternatives the pages discuss:
 *  - ATTN_VARIANT_RING3: a deeper K/V ring ("Three kernels for a chip the
 *    ecosystem skipped", Kernel one: a third buffer did not fit the 5090's
 *    shared memory; "Learning FlashAttention the Hard Way, Part 2", Refused
 *    Optimizations: deeper rings). Fits MI355X's 160 KB LDS at D = 64.
 *  - ATTN_VARIANT_EXP_POLY: part of the exponentials computed by an FMA
 *    polynomial instead of the transcendental unit (Part 2, Relationship to
 *    FA-3 and FA-4: FlashAttention-4's emulated exponential).
 *  - ATTN_VARIANT_WIDE: each wave owns 64 query rows instead of 32, halving
 *    the LDS operand reads per MFMA (Part 2, Move 4: register tiling).
 *  - ATTN_VARIANT_SUBPIPE: within a wave, the Q.K^T of its second 16-row
 *    sub-tile and the P.V of its first are scheduled beside the softmax of
 *    the other sub-tile, so the matrix and vector units of one wave overlap
 *    (Part 2, Relationship to FA-3 and FA-4: overlapping the softmax with
 *    the matrix products).
 *  - ATTN_VARIANT_BAR2: one workgroup barrier per two key intervals instead
 *    of one per interval, with a four-slot K/V ring and the copies two
 *    intervals ahead (Part 2, Refused Optimizations: deeper rings; fewer
 *    barriers let the two waves of a SIMD drift apart).
 *  - ATTN_VARIANT_PROD: four more waves per workgroup, one per SIMD, issue
 *    every K/V copy and only wait and synchronise, so that the eight compute
 *    waves never touch global memory inside the key loop (Part 2, Refused
 *    Optimizations: the producer warp of warp specialisation).
 *  - ATTN_VARIANT_TRIO: three compute waves per SIMD instead of two (twelve
 *    per workgroup, three 64-key tiles per barrier interval), for more waves
 *    to overlap one another's MFMA and softmax phases. attn_fwd, the split
 *    and the cache entry points run this geometry by default at D = 64 from
 *    2048 keys without the causal mask, and with it for single passes (from
 *    8192 keys when the query tiles are folded into mirror pairs); the
 *    variant runs it for any shape, for comparison.
 *  - ATTN_VARIANT_QUAD: four compute waves per SIMD (sixteen per workgroup,
 *    four 32-key tiles per 128-key interval, at most 128 VGPRs per wave).
 *  - ATTN_VARIANT_ROT: the three-wave geometry with the waves of each SIMD
 *    a third of an interval apart (P.V of the previous tile, Q.K^T and the
 *    softmax of the current one, each wave meeting the barrier after a
 *    different one of the three), so that two waves issue MFMAs while the
 *    third runs its softmax (Part 2, Refused Optimizations: ping-pong
 *    scheduling of two consumer warpgroups, here with three).
 *  - ATTN_VARIANT_M32: both products on 32x32x16 MFMAs, each wave's 32
 *    query rows one MFMA block (the pages' kernels tile with the 5090's
 *    m16n8k16 mma.sync atom: Part 2, the TILE setting of the Emmy knobs;
 *    the Emmy comments, Hybrid FP16/FP32 Accumulation). Alone with two
 *    waves per SIMD, or with ATTN_VARIANT_TRIO (1152) with three.
 *  - ATTN_VARIANT_SYNC: a check of the K/V ring protocol rather than an
 *    optimisation: every copy into LDS is waited for and followed by a
 *    workgroup barrier right after it is issued (and D = 128 runs lock-step,
 *    not ping-pong). Its arithmetic is the default kernel's, so its results
 *    equal attn_fwd's bit for bit unless the default kernel reads a ring slot
 *    before its copy lands or overwrites one still being read.
 *
 *  q ... causal, stream : as attn_fwd (same layouts, checks and status codes).
 *  variant : one of the ATTN_VARIANT_* values; D = 64 builds 0, RING3,
 *            EXP_POLY, WIDE, SUBPIPE, SYNC, BAR2, PROD, TRIO, QUAD and ROT,
 *            D = 128 builds 0, EXP_POLY and SYNC. Any other
 *            value (or combination) returns ATTN_ERR_UNSUPPORTED before
 *            anything is enqueued.
 */
int attn_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int S, int D, float scale, int causal, int variant,
                     void* stream);

/*
 * attn_fwd_kvcache -- S_q queries per head against S_k cached keys and values
 * (decoding, or a chunk of new tokens, against a key/value cache; the Emmy
 * comments page closes on split-KV as what matters when decoding against a
 * large KV cache, and Part 2's references name Flash-Decoding). The queries
 * are the last S_q positions of the sequence: with causal = 1, query row i
 * (position S_k - S_q + i) sees keys 0 .. S_k - S_q + i; with S_q = S_k this
 * is attn_fwd_splitkv exactly.
 *
 *  q    : fp16 [B, H, S_q, D], contiguous; o : fp16 [B, H, S_q, D];
 *  lse  : fp32 [B, H, S_q];
 *  k, v : fp16 [B, H, S_k, D], contiguous (the cache, read only);
 *  S_q, S_k : >= 1; causal = 1 needs S_q <= S_k (else ATTN_ERR_SHAPE);
 *  n_splits, workspace, workspace_size : as attn_fwd_splitkv, with the
 *             workspace sized by attn_fwd_splitkv_workspace_size(B, H, S_q,
 *             D, n_splits) (partials are per query row). Few query rows make
 *             few workgroups, so decoding wants n_splits > 1 (each run of
 *             keys gets its own workgroups).
 *  Other arguments, alignment, ownership and status codes: as attn_fwd.
 */
int attn_fwd_kvcache(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int S_q, int S_k, int D, float scale, int causal,
                     int n_splits, void* workspace, size_t workspace_size, void* stream);

/* Workspace bytes attn_fwd_splitkv needs: n_splits * B * H * S * (D + 1) * 4
 * for n_splits > 1; 0 when n_splits == 1 or an argument is out of range.
 * For attn_fwd_kvcache pass S = S_q. */
size_t attn_fwd_splitkv_workspace_size(int B, int H, int S, int D, int n_splits);

/* Size of the static device scratch buffer of attn_fwd_splitkv_noalloc. */
#define ATTN_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * attn_fwd_splitkv_noalloc -- attn_fwd_splitkv for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the partial results go to a static device
 * array of ATTN_NOALLOC_SCRATCH_BYTES owned by the library instead of a
 * caller workspace. The call allocates nothing; on the first call on a device
 * (with that device current) it looks up the array's device address once.
 *
 *  q ... n_splits : as attn_fwd_splitkv (same layouts, checks and results:
 *                   the same kernels run, so outputs equal attn_fwd_splitkv's
 *                   with the same n_splits bit for bit).
 *  stream         : hipStream_t as void* (NULL = default stream).
 *
 *  Returns ATTN_ERR_ARG when attn_fwd_splitkv_workspace_size(B, H, S, D,
 *  n_splits) exceeds ATTN_NOALLOC_SCRATCH_BYTES (nothing is enqueued), and
 *  ATTN_ERR_HIP if the scratch address cannot be looked up.
 *
 *  Every call on one device shares that device's scratch array, which keeps
 *  the last call's contents (each call writes every partial it reads, so no
 *  clearing is needed): calls with n_splits > 1 that overlap in time on one
 *  device (on different streams, or from different threads) race and must be
 *  serialised by the caller.
 */
int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int S, int D, float scale, int causal, int n_splits,
                             void* stream);

/* Static English name of a status code ("ATTN_OK", ...); never NULL. */
const char* attn_status_string(int status);

/* Thread-local detail of the last error returned on this thread ("" if none).
 * The pointer stays valid until the next call into the library on this
 * thread. */
const char* attn_last_error(void);

/* ATTN_FWD_ABI_VERSION of the loaded library. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */
