// Fused exact-attention forward kernel for gfx950 (CDNA4, wave64, MFMA).
//
// Streaming form of attention from "Learning FlashAttention the Hard Way,
// Part 2": each query row keeps a carrier (running max m, denominator d,
// unnormalised output o) that absorbs key tiles one after another (the FA-1
// update of Move 0, the tensor-core tiles of Moves 1-4), and two carriers
// over disjoint key sets merge by rescaling to the larger max (the split-KV
// remark of the wrap-up). The layout below is designed for CDNA4 rather than
// translated from the page's mma.sync listings.
//
// Work decomposition. A workgroup owns BLOCK_M = 128 query rows of one
// (batch, head) and streams the keys in intervals of NPH tiles of BN keys,
// which arrive in LDS together. Its compute waves form QGROUPS = 4 query
// groups of 32 rows (two 16-row sub-tiles per wave); the NPH waves of a group
// take one tile each per interval (wave phase p folds tiles p, p + NPH, ...).
// Wave w runs on SIMD w % 4, so the waves sharing a SIMD hold different query
// rows and fill each other's stalls. Default: 8 waves, NPH = 2 tiles of 64
// keys (two waves per SIMD); at D = 64 from 2048 keys (non-causal, and causal
// single passes -- folded ones from 8192 keys) VAR_TRIO runs 12 waves,
// NPH = 3 (three per SIMD). Other geometries are variants (see Geometry). At
// the end the NPH carriers of a query group meet in LDS and each wave merges
// them for the output columns it owns.
//
// MFMA: v_mfma_f32_16x16x32_f16 (the VAR_M32 variant: v_mfma_f32_32x32x16_f16,
// its lane layout at Geometry::M32). Lane l = 16*g + i (g = 0..3, i = 0..15):
//   A: row i, contraction slots (g, 0..7); B: column i, slots (g, 0..7);
//   C: column i, rows 4*g + r (r = 0..3).
// A slot (g, e) meets B slot (g, e), so any assignment of the contraction
// index to slots that is the same for both operands gives the same sum.
//
// Transposed products keep one query per lane in every accumulator:
//   S^T = K . Q^T   (A = K rows from LDS, B = Q^T fragments in registers)
//   O^T = V^T . P^T (A = V^T rows from LDS, B = P^T straight from registers)
// MFMA row i of S^T key block kb (0..3) is bound to tile key
//   st_key(kb, i) = 32*(kb/2) + 8*(i/4) + 4*(kb%2) + i%4,
// so lane group g holds keys 32*kc + 8*g + 0..7 of each 32-key chunk kc: the
// eight probabilities, rounded to fp16, are exactly the B slots (g, 0..7) of
// the P.V MFMA, and V^T is read in the same key order. P never touches LDS.
//
// Softmax in base 2 with the scale folded in: t = s * c, c = |scale| log2 e.
// The running max is updated lazily: a tile is first exponentiated against the
// current m; only if some lane's probabilities could overflow (their fp16 sum
// exceeds P_LIMIT, or is not finite) does the wave compute the tile max,
// rescale o and d, and redo the tile, for the 16-row sub-tiles concerned (the
// first step of a tile takes the max up front). Because o and d always share
// one m, the result is the same softmax, and probabilities up to P_LIMIT keep
// fp16's relative precision. The row sum adds the fp16-rounded probabilities (v_dot2 at
// D = 64, v_fma_mix_f32 at D = 128), so d normalises exactly the weights the
// P.V product used.
//
// LDS. K and V tiles arrive by direct global->LDS loads into two-slot rings
// of tile groups, one barrier interval before they are read. K rows are stored in
// MFMA-row order (row 16*kb + i holds key st_key(kb, i)), V rows in key order;
// both are unpadded with XOR-permuted 16-byte chunks so that every operand
// read is free of bank conflicts on the 64-bank LDS. V^T operands come from
// transposing LDS reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "work_order.h"

namespace attn {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BLOCK_M = 128;          // query rows per workgroup
constexpr int WAVES = 8;              // waves per workgroup, two per SIMD
constexpr int THREADS = WAVES * 64;
constexpr int INTERVAL_KEYS = 128;    // keys per barrier interval
constexpr int COMBINE_THREADS = 256;  // combine kernel: four waves, one row each
constexpr int MAX_SPLITS = 64;        // key runs per query tile of a split launch, at most
constexpr float NEG_BIG = -1.0e30f;   // finite stand-in for -infinity
// Lazy-max bound on a lane's tile sum. The sum is taken over the fp16-rounded
// probabilities, so every rounded probability is at most the sum, and a value
// that overflowed to infinity fails the test. 65504 (fp16's largest finite
// value) less a margin of 4064 for the fp32 rounding of the running sum
// against d (d stays below about 2^30 even for a 2^20-key row under this
// bound, where that rounding is a few hundred at most). Against 2^15: 2.5%
// faster on peaked D = 64 rows (Q and K x 3), the same elsewhere.
constexpr float P_LIMIT = 61440.0f;
// A redo sets the running max to the tile's max itself. (Setting it some
// margin h above, so that a row whose max keeps climbing redoes less often,
// shifts every later probability of the row down by 2^-h: with h = 8 those
// more than 17 log2 units below the max round to zero in fp16, and a row
// with one outlying key lost 0.13% of its denominator -- an LSE error of
// 1.3e-3 at S = 8807, scale 0.31, against the 1e-3 budget.)
constexpr uint32_t BUF_FLAGS = 0x00020000u;  // raw buffer, 32-bit data format

// Compile-time variants of the kernel (bit flags), selectable through
// attn_fwd_variant; 0 is the default kernel.
enum : int {
  VAR_RING3 = 1,     // D = 64: three-slot K/V ring, copies two intervals ahead
  VAR_EXP_POLY = 2,  // one exponential in four by an FMA polynomial
  VAR_WIDE = 4,      // D = 64: 64-row waves over four 32-key tiles per interval
  VAR_SUBPIPE = 8,   // D = 64: MFMAs of one sub-tile beside the softmax of the other
  VAR_SYNC = 16,     // every K/V copy waited for and barriered right after its issue
  VAR_BAR2 = 32,     // D = 64: one workgroup barrier per two key intervals (four-slot ring)
  VAR_PROD = 64,     // D = 64: four producer waves issue every K/V copy
  VAR_TRIO = 128,    // D = 64: three waves per SIMD over three 64-key tiles per interval
  VAR_QUAD = 256,    // D = 64: four waves per SIMD over four 32-key tiles per interval
  VAR_ROT = 512,     // D = 64: three waves per SIMD, their phases rotated by a third
  VAR_M32 = 1024,    // D = 64: 32x32x16 MFMAs (one 32-row block per wave)
};

template <int D, int VAR = 0>
struct Geometry {
  // Key tiles per interval, one per wave of a query group (the wave's phase).
  // 64-row waves at D = 64 (VAR_WIDE) halve the LDS operand reads per MFMA
  // but measured no faster than 32-row waves (the path is not bound by
  // them), so they are a variant.
  static constexpr bool WIDE = D == 64 && (VAR & VAR_WIDE) != 0;
  // Three waves per SIMD (VAR_TRIO, D = 64): twelve compute waves, three per
  // query group, each on its own 64-key tile of a 192-key interval (three
  // 159-VGPR allocations fit a SIMD's 512 registers per lane).
  static constexpr bool TRIO = D == 64 && (VAR & (VAR_TRIO | VAR_ROT)) != 0;
  // Rotated order (VAR_ROT, three-wave geometry): the three waves of a SIMD
  // run P.V of interval j-1, Q.K^T of j and the softmax of j in the same
  // order but with their barriers after different parts, so that at any
  // time two of them issue MFMAs and one its softmax. Q.K^T of j runs in
  // interval j for two waves and in j+1 for the third: a three-slot K ring.
  static constexpr bool ROT = D == 64 && (VAR & VAR_ROT) != 0;
  // Four waves per SIMD (VAR_QUAD, D = 64): sixteen compute waves, four per
  // query group on 32-key tiles of a 128-key interval, at most 128 VGPRs.
  static constexpr bool QUAD = D == 64 && (VAR & VAR_QUAD) != 0;
  // 32x32x16 MFMAs (VAR_M32, D = 64, 32-row waves): each wave's 32 query
  // rows are one MFMA block. An MFMA takes one issue slot per 32 cycles
  // instead of one per 16, so the softmax of another wave on the SIMD keeps
  // more of its VALU rate beside it, and each K or V^T fragment read from
  // LDS feeds 32 query columns. Measured: about 3% fewer cycles per launch,
  // but under sustained load the power-limited clock drops from 2.1 to
  // 1.9 GHz (twice the accumulator traffic per FLOP), 7% slower -- a
  // variant. Lane (j, h) = (lane % 32, lane / 32) holds
  // query j: of a 32-key block of S^T, keys 8e' + 4h + r (element 4e' + r);
  // of O^T, rows 8e' + 4h + r of each 32-row block.
  static constexpr bool M32 = D == 64 && (VAR & VAR_M32) != 0;
  static constexpr int NPH = (WIDE || QUAD) ? 4 : TRIO ? 3 : 2;
  static constexpr int CWAVES = TRIO ? 12 : QUAD ? 16 : WAVES;  // compute waves
  static constexpr int QGROUPS = CWAVES / NPH;             // query groups
  static constexpr int ROWS = BLOCK_M / QGROUPS;           // query rows per wave
  // 16-row query sub-tiles per wave (M32: the wave's one 32-row block)
  static constexpr int QSUB = M32 ? 1 : ROWS / 16;
  // Keys per tile: each wave folds one tile per barrier interval. (At D = 64,
  // 64-row waves with 64-key tiles would not fit the 256-register budget of
  // two waves per SIMD; nor would 128-key tiles with 32-row waves.)
  static constexpr int BN = TRIO ? 64 : INTERVAL_KEYS / NPH;
  static constexpr int IKEYS = NPH * BN;                   // keys per barrier interval
  static constexpr int KB = BN / (M32 ? 32 : 16);          // MFMA key blocks of S^T
  static constexpr int KC = BN / (M32 ? 16 : 32);          // key chunks of the P.V contraction
  static constexpr int K_HALVES = BN * D;                  // K rows unpadded, swizzled
  static constexpr int V_HALVES = BN * D;                  // V rows unpadded, swizzled
  // Two-slot rings of tile groups (one tile per phase) for K and for V: one
  // group is read while the next is copied. A three-slot ring (VAR_RING3,
  // D = 64 only: at D = 128 it does not fit next to the Q tile) runs the
  // copies two intervals ahead; it measured no faster.
  // One barrier per two intervals (VAR_BAR2, D = 64): a four-slot ring with
  // the copies two intervals ahead, so that every slot written after a
  // barrier was last read before it, and every slot read before the next
  // barrier was waited for at this one.
  static constexpr bool BAR2 = D == 64 && (VAR & VAR_BAR2) != 0;
  static constexpr int RING = BAR2 ? 4 : (D == 64 && (VAR & VAR_RING3) != 0) ? 3 : 2;
  static constexpr int KRING = ROT ? 3 : RING;  // slots of the K ring (V: RING)
  static constexpr int AHEAD = BAR2 ? 2 : RING - 1;  // intervals between a copy and its use
  static constexpr int SLOT_HALVES = NPH * K_HALVES;        // one interval's tiles
  // Q^T fragments stay in registers for the whole key loop at both head
  // dimensions. (At D = 128 they were staged in LDS and re-read each interval
  // while the kernel needed 250 VGPRs; with them in registers it runs 1-2%
  // faster and reads 64 KB less from LDS per interval and CU.)
  // The second wave of each SIMD (waves 4-7) runs half an interval out of
  // phase with the first (softmax against the other wave's MFMA phase). This
  // pays only where the MFMA phase is long next to the softmax: at D = 128
  // (5% on causal B2 H16 S8192, 4-6% more with dense MFMA phases and row
  // sums without v_dot2), not at D = 64 (2-10% slower, 3-4% with fp32-add
  // row sums in place of the v_dot2 sums that wait for the other wave's
  // MFMAs, and no better with the V operands in registers).
  static constexpr bool PINGPONG = D == 128 && (VAR & VAR_SYNC) == 0;
  // Synchronous copies (VAR_SYNC, a check of the ring protocol): each wave
  // waits for its copies and meets the others at a barrier right after
  // issuing them, in lock-step order. The arithmetic is the default's, so
  // any difference in the results would expose a race on the LDS ring.
  static constexpr bool SYNC = (VAR & VAR_SYNC) != 0;
  // At D = 64 a tile's P.V runs in the same interval as its Q.K^T and
  // softmax (three phases, V copied one interval earlier): the SIMD's two
  // waves then interleave shorter MFMA phases with their softmaxes (1-3%
  // faster). At D = 128 the ping-pong order measured faster than this.
  static constexpr bool PV_SAME = D == 64 && !ROT;
  // Row sums of the rounded fp16 probabilities (the weights P.V uses, so that
  // a row dominated by one key gets exactly that key's V row). At D = 64,
  // dot products with ones (v_dot2). In the D = 128 ping-pong a softmax runs
  // beside the other wave's MFMA phase, and a v_dot2 there waits for the
  // MFMA pipe: one wave issuing MFMAs back to back and one issuing v_dot2
  // take as long as both run one after the other, while adds, FMAs and
  // exponentials beside an MFMA stream lose only 20-35% of their rate
  // (probe of two waves per SIMD). So D = 128 adds each value with
  // v_fma_mix_f32 (fp16 operand, fp32 accumulator; 4-6% faster there, 2-4%
  // slower at D = 64). Sums of the unrounded fp32 values cost the same but
  // let a peaked row's O drift by the fp16 rounding of its dominant weight
  // (3.7e-3 against 2.0e-3 at peaked causal B4 H32 S4096 D128).
  static constexpr bool MIX_SUMS = D == 128;
  // A wave in its softmax raises its issue priority (s_setprio), so that the
  // SIMD's other wave, in its MFMA phase or later in its own softmax, does not
  // starve it (2-3% on every workload).
  static constexpr bool SOFTMAX_PRIO = true;
  // One exponential in four computed on the FMA path (VAR_EXP_POLY).
  static constexpr bool EXP_POLY = (VAR & VAR_EXP_POLY) != 0;
  // Sub-tile pipelined interval (VAR_SUBPIPE, D = 64 with two sub-tiles):
  // Q.K^T of sub-tile 1 runs beside the softmax of sub-tile 0, and P.V of
  // sub-tile 0 beside the softmax of sub-tile 1, each pair in one scheduling
  // region with SIDE_VPER VALU instructions after each MFMA. Measured 2-5%
  // slower than the default order (3 VALU instructions per MFMA was the best
  // of 3, 6, 10 and 16; fp32-add row sums in place of v_dot2 did not help).
  static constexpr bool SUBPIPE = D == 64 && (VAR & VAR_SUBPIPE) != 0 && QSUB == 2;
  static constexpr int SIDE_VPER = 3;
  static constexpr int D_CHUNKS = D / (M32 ? 16 : 32);     // contraction chunks of Q.K
  static constexpr int D_BLOCKS = D / (M32 ? 32 : 16);     // MFMA row blocks of O^T
  using Acc = std::conditional_t<M32, f32x16, f32x4>;     // one MFMA accumulator
  // Producer waves (VAR_PROD, D = 64): the workgroup gets four more waves,
  // one per SIMD, that issue all K/V copies and only wait and synchronise;
  // the eight compute waves never touch global memory inside the key loop.
  // At 159 VGPRs three waves fit a SIMD's 512 registers per lane.
  static constexpr bool PROD = D == 64 && PV_SAME && (VAR & VAR_PROD) != 0;
  static constexpr int PRODUCERS = PROD ? 4 : 0;
  static constexpr int WG_WAVES = CWAVES + PRODUCERS;
  static constexpr int WG_THREADS = 64 * WG_WAVES;
  static constexpr int NCOP = PROD ? PRODUCERS : CWAVES;  // waves that issue the copies
  // per interval, K and V each in 16-byte pieces
  static constexpr int PIECES = NPH * BN * (D / 8);
  static constexpr int LOADS = PIECES / (64 * NCOP);   // copies per copying wave and tensor
  static_assert(D % 64 == 0, "D must be a multiple of 64");
  static_assert(LOADS * 64 * NCOP == PIECES, "tiling");
  static_assert(!PROD || VAR == VAR_PROD, "producer waves run the default two-slot ring alone");
  static_assert(!QUAD || VAR == VAR_QUAD, "four waves per SIMD run the default order alone");
  static_assert(!ROT || VAR == VAR_ROT, "the rotated order runs alone");
  static_assert(!TRIO || ROT || (VAR & ~(VAR_SYNC | VAR_M32)) == VAR_TRIO,
                "three waves per SIMD run the default order (or its synchronous-copy check)");
  static_assert(!M32 || (VAR & ~(VAR_SYNC | VAR_TRIO)) == VAR_M32,
                "32x32 MFMAs run the default two- or three-wave order (or its synchronous-copy check)");
  static_assert(!M32 || ROWS == 32, "32x32 MFMAs need 32-row waves");
  static_assert(ROWS * QGROUPS == BLOCK_M && (M32 || QSUB * 16 == ROWS) && KB >= 2 && KC >= 1,
                "geometry");
  // Carrier hand-off (after the key loop): each wave finalises the output's
  // 16-column blocks it owns (block db belongs to phase db * NPH / D_BLOCKS:
  // an equal share, or at NPH = 3 blocks {0, 1}, {2}, {3}) for its rows. Per
  // wave, 16-byte slots of 64 lanes: {m, d} of two sub-tiles per slot, then
  // one slot per sub-tile and output block.
  // (M32: the unit is a quarter block -- four accumulator elements, rows
  // 8e' + 4h + r of block db for e' = quarter -- owned by phase
  // quarter * NPH / (4 * D_BLOCKS).)
  static constexpr int owner(int db) { return db * NPH / D_BLOCKS; }
  static constexpr int QUARTERS = 4 * D_BLOCKS;
  static constexpr int owner_q(int qd) { return qd * NPH / QUARTERS; }
  static constexpr int MD_SLOTS = (QSUB + 1) / 2;
  static constexpr int HANDOFF_SLOTS = MD_SLOTS + (M32 ? QUARTERS : QSUB * D_BLOCKS);
  static constexpr int HANDOFF_BYTES = CWAVES * HANDOFF_SLOTS * 64 * 16;
  static constexpr int LOOP_BYTES = (KRING + RING) * SLOT_HALVES * 2;
  static constexpr int LDS_BYTES = LOOP_BYTES > HANDOFF_BYTES ? LOOP_BYTES : HANDOFF_BYTES;
  static constexpr int LDS_HALVES = LDS_BYTES / 2;
  static_assert((M32 ? QUARTERS : D_BLOCKS) >= NPH, "every wave of a query group owns an output block");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, BUF_FLAGS);
}

// Key of the tile held in K row `row` of LDS (rows are in MFMA-row order).
__device__ __forceinline__ int st_key(int kb, int i) {
  return 32 * (kb >> 1) + 8 * (i >> 2) + 4 * (kb & 1) + (i & 3);
}
// LDS K row of tile key k (inverse of st_key).
__device__ __forceinline__ int k_row_of(int k) {
  const int kb = 2 * (k >> 5) + ((k >> 2) & 1);
  const int i = 4 * ((k >> 3) & 3) + (k & 3);
  return 16 * kb + i;
}

__device__ __forceinline__ float max4(f32x4 v) {
  return __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), __builtin_fmaxf(v[2], v[3]));
}

// Reduce over the four lanes (i, i+16, i+32, i+48) that hold one query.
__device__ __forceinline__ float group_max(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// LDS tiles are unpadded with their 16-byte chunks permuted per row, so that
// the direct global->LDS copies (which fill LDS in lane order) and every LDS
// read pattern below are free of bank conflicts on the 64-bank LDS.
//
// K: row R = 16*kb + i holds key st_key(kb, i) (MFMA-row order); chunk c sits
// at c ^ k_swizzle(R). The Q.K^T operand read has 16 lanes on 16 consecutive
// rows at one logical chunk; the swizzle spreads them over 16 bank groups.
template <int D>
__device__ __forceinline__ int k_swizzle(int row) {
  return D == 64 ? ((row >> 1) & 7) : (row & 15);
}
// V: row r holds key r (natural order); chunk c sits at c ^ v_swizzle(r). The
// transposing reads of the P.V operand touch 8 rows x 32 bytes per half-wave,
// which this swizzle maps onto distinct bank groups.
template <int D>
__device__ __forceinline__ int v_swizzle(int r) {
  if (D == 64) return 2 * (((r >> 1) & 1) + 2 * ((r >> 3) & 1));
  return 2 * ((r & 3) + 4 * ((r >> 3) & 1));
}

// V with 32x32 MFMAs (M32, D = 64): each half-wave's transposing reads cover 4
// consecutive key rows x 64 bytes; rows 2r and 2r + 1 fall on the two halves
// of the 64 banks, and this swizzle puts rows 4r and 4r + 2 on disjoint
// 64-byte groups of chunks.
__device__ __forceinline__ int v_swizzle_m32(int r) { return 4 * ((r >> 1) & 1); }

// Direct global->LDS copy of one interval's tiles. A buffer load with the LDS
// flag writes lane l's 16 bytes at M0 + 16*l, so each wave instruction fills
// 1 KB of LDS in slot order; each lane therefore fetches the global piece that
// belongs in its slot. Per-lane byte offsets (relative to the first key of the
// interval) are precomputed for K and for V.
template <int D, int VAR>
struct CopyPlan {
  uint32_t k_off[Geometry<D, VAR>::LOADS];
  uint32_t v_off[Geometry<D, VAR>::LOADS];
};

// 1 KB unit of the slot filled by instruction i of copying wave cw
template <int D, int VAR>
__device__ __forceinline__ int copy_unit(int cw, int i) {
  return i * Geometry<D, VAR>::NCOP + cw;
}

template <int D, int VAR>
__device__ __forceinline__ void make_copy_plan(CopyPlan<D, VAR>& cp, int cw, int lane) {
  using G = Geometry<D, VAR>;
  constexpr int CHUNKS = D / 8;                     // 16-byte chunks per row
  constexpr int TILE_SLOTS = G::BN * CHUNKS;
#pragma unroll
  for (int i = 0; i < G::LOADS; ++i) {
    const int slot = copy_unit<D, VAR>(cw, i) * 64 + lane;
    const int t = slot / TILE_SLOTS;                // tile of the interval
    const int w = slot % TILE_SLOTS;
    const int row = w / CHUNKS;
    const int pc = w % CHUNKS;                       // physical chunk in the row
    // (M32: K rows in key order, as the 32x32 operand reads them)
    const int kkey = G::M32 ? row : st_key(row >> 4, row & 15);
    const int vsw = G::M32 ? v_swizzle_m32(row) : v_swizzle<D>(row);
    cp.k_off[i] = (uint32_t)(((t * G::BN + kkey) * D + 8 * (pc ^ k_swizzle<D>(row))) * 2);
    cp.v_off[i] = (uint32_t)(((t * G::BN + row) * D + 8 * (pc ^ vsw)) * 2);
  }
}

// Buffer descriptor over keys [key0, S) of one head's K or V: the hardware
// range check returns zeros for keys >= S.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t keys_from(const _Float16* base, int key0, int S) {
  const uint32_t bytes = key0 < S ? (uint32_t)(S - key0) * D * 2 : 0u;
  return make_rsrc(base + (int64_t)key0 * D, bytes);
}

// Issue the direct copy of the interval starting at key0 into `slot` (its LDS
// area: tile 0, tile 1, ...). Completion is awaited with vmcnt.
template <int D, int VAR>
__device__ __forceinline__ void copy_group(const uint32_t* off, const _Float16* base, int key0,
                                          int S, _Float16* slot, int cw) {
  const __amdgpu_buffer_rsrc_t rs = keys_from<D>(base, key0, S);
#pragma unroll
  for (int i = 0; i < Geometry<D, VAR>::LOADS; ++i) {
    _Float16* dst = slot + copy_unit<D, VAR>(cw, i) * 64 * 8;   // 64 slots of 8 halves
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)dst, 16, off[i], 0, 0, 0);
  }
}

// Wait until this wave's direct copies (vector memory operations) are done.
__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N of this wave's vector memory operations are in flight
// (they complete in order): the N most recent copies may still run.
template <int N>
__device__ __forceinline__ void wait_copies_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // s_waitcnt encoding (gfx9): vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// LDS transposing read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane n supplies the address of 4 consecutive halves X[n][0..3]; lane n
// receives X[4e + n/4][n % 4] for e = 0..3.
__device__ __forceinline__ f16x4 lds_read_tr(const _Float16* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (s16x4 __attribute__((address_space(3)))*)(p));
  return __builtin_bit_cast(f16x4, r);
}

// Per-lane carrier of one query sub-tile (the lane's query is i = lane % 16;
// M32: j = lane % 32).
template <int D, int VAR>
struct Carrier {
  typename Geometry<D, VAR>::Acc o[Geometry<D, VAR>::D_BLOCKS];  // O^T rows of this query:
                                   // 16*db + 4*g + r (M32: 32*db + 8e' + 4h + r)
  float m;                         // running max of t = s*c (base-2 units)
  float d;                         // this lane's share of the denominator
};

// Per-wave register sets: carriers and Q^T fragments of the QSUB sub-tiles, a
// tile's scores, and its fp16 probabilities.
template <int D, int VAR>
using CarrierSet = Carrier<D, VAR>[Geometry<D, VAR>::QSUB];
template <int D, int VAR>
using QSet = f16x8[Geometry<D, VAR>::QSUB][Geometry<D, VAR>::D_CHUNKS];
template <int D, int VAR>
using ScoreSet = std::conditional_t<Geometry<D, VAR>::M32, f32x16[Geometry<D, VAR>::KB],
                                    f32x4[Geometry<D, VAR>::QSUB][Geometry<D, VAR>::KB]>;
template <int D, int VAR>
using ProbSet = f16x8[Geometry<D, VAR>::QSUB][Geometry<D, VAR>::KC];

// Scheduling groups (sched_group_barrier masks): LDS reads and MFMAs.
constexpr int SG_DS_READ = 0x100;
constexpr int SG_MFMA = 0x008;
constexpr int SG_VALU = 0x002;
// LDS read instructions of unit u: two transposing reads for a V^T fragment,
// one 16-byte read for a K fragment.
template <int U, int END, int NPV>
__device__ __forceinline__ void pin_reads() {
  if constexpr (U < END) {
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, U < NPV ? 2 : 1, 0);
    pin_reads<U + 1, END, NPV>();
  }
}
template <int U, int NU, int NPV, int AHEAD, int QSUB>
__device__ __forceinline__ void pin_units() {
  if constexpr (U < NU) {
    if constexpr (U + AHEAD < NU)
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, U + AHEAD < NPV ? 2 : 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, QSUB, 0);
    pin_units<U + 1, NU, NPV, AHEAD, QSUB>();
  }
}

// The MFMA half of an interval with 32x32x16 MFMAs (M32): units as in
// mfma_phase below, one MFMA each.
//  V^T operand (O^T block ob, key chunk cc of 16 keys): lane (i, h) needs
//  V[16cc + 4h + 8x + e][32ob + i] for x = 0, 1 and e = 0..3 -- the keys whose
//  probabilities the lane holds in element 8(cc % 2) + 4x + e of the scores
//  of block cc / 2 -- two transposing reads over 4 key rows x 16 d, source
//  lane n of group g pointing at row 16cc + 4h + 8x + n/4, halves
//  32ob + 16(g % 2) + 4(n % 4).
//  K operand (key block kb, d chunk dc): row 32kb + i, halves 16dc + 8h.
template <int D, int VAR, bool PV, bool QK>
__device__ __forceinline__ void mfma_phase_m32(CarrierSet<D, VAR>& cr,
                                               const ProbSet<D, VAR>& pf,
                                               ScoreSet<D, VAR>& sc,
                                               const QSet<D, VAR>& qf,
                                               const _Float16* __restrict__ vtile,
                                               const _Float16* __restrict__ ktile, int li, int g) {
  using G = Geometry<D, VAR>;
  constexpr int NPV = PV ? G::KC * G::D_BLOCKS : 0;
  constexpr int NQK = QK ? G::KB * G::D_CHUNKS : 0;
  constexpr int NU = NPV + NQK;
  constexpr int AHEAD = 4 < NU ? 4 : NU;
  const int i = 16 * (g & 1) + li;
  const int h = g >> 1;
  // row bit 1 (the swizzle's) is bit 3 of li, for every cc, h and x
  const int vsw = v_swizzle_m32(li >> 2);
  const _Float16* vlane = vtile + (4 * h + (li >> 2)) * D + 4 * (li & 1);
  const int vx = 2 * (g & 1) + ((li & 3) >> 1);  // logical chunk within the block
  const int ksw = k_swizzle<D>(i);  // the swizzle bits of row 32kb + i do not depend on kb
  auto load = [&](int u) -> f16x8 {
    if (u < NPV) {
      const int cc = u / G::D_BLOCKS, ob = u % G::D_BLOCKS;
      const _Float16* vp = vlane + 8 * ((4 * ob + vx) ^ vsw) + (16 * cc) * D;
      const f16x4 lo = lds_read_tr(vp);
      const f16x4 hi = lds_read_tr(vp + 8 * D);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    const int w = u - NPV, dc = w / G::KB, kb = w % G::KB;
    return *reinterpret_cast<const f16x8*>(ktile + (32 * kb + i) * D + 8 * ((2 * dc + h) ^ ksw));
  };
  auto compute = [&](int u, const f16x8& a) {
    if (u < NPV) {
      const int cc = u / G::D_BLOCKS, ob = u % G::D_BLOCKS;
      cr[0].o[ob] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[0][cc], cr[0].o[ob], 0, 0, 0);
    } else {
      const int w = u - NPV, dc = w / G::KB, kb = w % G::KB;
      sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[0][dc], dc == 0 ? f32x16{} : sc[kb],
                                                      0, 0, 0);
    }
  };
  f16x8 fr[NU];
#pragma unroll
  for (int u = 0; u < AHEAD; ++u) fr[u] = load(u);
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (u + AHEAD < NU) fr[u + AHEAD] = load(u + AHEAD);
    compute(u, fr[u]);
  }
  pin_reads<0, AHEAD, NPV>();
  pin_units<0, NU, NPV, AHEAD, 1>();
}

// The MFMA half of an interval: P.V of the previous tile (PV) and Q.K^T of the
// current one (QK), as one software-pipelined stream of units. A unit is one
// A-operand fragment read from LDS (two transposing reads for V^T, one 16-byte
// read for K) and the two MFMAs (both query sub-tiles) that consume it.
// Fragments are read AHEAD units before use, so the LDS latency is covered by
// the MFMAs in between. Units are ordered so that consecutive MFMAs on one
// accumulator are several instructions apart (QSUB MFMAs per unit).
template <int D, int VAR, bool PV, bool QK>
__device__ __forceinline__ void mfma_phase(CarrierSet<D, VAR>& cr,
                                           const ProbSet<D, VAR>& pf,
                                           ScoreSet<D, VAR>& sc,
                                           const QSet<D, VAR>& qf,
                                           const _Float16* __restrict__ vtile,
                                           const _Float16* __restrict__ ktile, int li, int g) {
  using G = Geometry<D, VAR>;
  if constexpr (G::M32) {
    mfma_phase_m32<D, VAR, PV, QK>(cr, pf, sc, qf, vtile, ktile, li, g);
  } else {
  constexpr int QSUB = G::QSUB;
  constexpr int NPV = PV ? G::KC * G::D_BLOCKS : 0;
  constexpr int NQK = QK ? G::KB * G::D_CHUNKS : 0;
  constexpr int NU = NPV + NQK;
  constexpr int AHEAD_MAX = (G::QUAD || G::ROT) ? 4 : D == 64 ? 8 : 4;
  constexpr int AHEAD = AHEAD_MAX < NU ? AHEAD_MAX : NU;
  // V^T operand (d block db, key chunk kc): lane (i, g) needs
  // V[32kc + 8g + e][16db + i], e = 0..7 -- two transposing reads over 4 key
  // rows x 16 d, source lane n of group g pointing at row 32kc + 8g + 4h + n/4,
  // halves 16db + 4(n%4).
  const int vrow = 8 * g + (li >> 2);
  const int vsw = v_swizzle<D>(vrow);  // row bits that matter do not depend on kc or h
  const _Float16* vlane = vtile + vrow * D + 4 * (li & 1);
  const int vx = (li & 3) >> 1;
  // K operand (key block kb, d chunk ch): row 16kb + li, halves 32ch + 8g.
  const int ksw = k_swizzle<D>(li);  // the swizzle bits of row 16*kb + li do not depend on kb
  auto load = [&](int u) -> f16x8 {
    if (u < NPV) {
      const int kc = u / G::D_BLOCKS, db = u % G::D_BLOCKS;
      const _Float16* vp = vlane + 8 * ((2 * db + vx) ^ vsw) + (32 * kc) * D;
      const f16x4 lo = lds_read_tr(vp);
      const f16x4 hi = lds_read_tr(vp + 4 * D);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    const int w = u - NPV, ch = w / G::KB, kb = w % G::KB;
    return *reinterpret_cast<const f16x8*>(ktile + (16 * kb + li) * D + 8 * ((4 * ch + g) ^ ksw));
  };
  auto compute = [&](int u, const f16x8& a) {
    if (u < NPV) {
      const int kc = u / G::D_BLOCKS, db = u % G::D_BLOCKS;
#pragma unroll
      for (int qs = 0; qs < QSUB; ++qs)
        cr[qs].o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pf[qs][kc], cr[qs].o[db], 0, 0, 0);
    } else {
      const int w = u - NPV, ch = w / G::KB, kb = w % G::KB;
#pragma unroll
      for (int qs = 0; qs < QSUB; ++qs)
        sc[qs][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            a, qf[qs][ch], ch == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sc[qs][kb], 0, 0, 0);
    }
  };
  f16x8 fr[NU];
#pragma unroll
  for (int u = 0; u < AHEAD; ++u) fr[u] = load(u);
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (u + AHEAD < NU) fr[u + AHEAD] = load(u + AHEAD);
    compute(u, fr[u]);
  }
  // Pin that order for the scheduler: the reads of the first AHEAD units,
  // then per unit the reads of unit u + AHEAD followed by unit u's two MFMAs.
  // Left to itself at D = 128, the scheduler reads most fragments just
  // before their MFMAs (fewer live registers), so the phase waits on LDS
  // latency unit after unit and the other wave's softmax fills the gaps;
  // pinned, the MFMAs issue back to back (with the mixed-precision row sums
  // 4-6% faster; with v_dot2 sums 2-5% slower, as their softmax then waits).
  pin_reads<0, AHEAD, NPV>();
  pin_units<0, NU, NPV, AHEAD, QSUB>();
  }
}

// Operand fragments of one tile for the sub-tile pipelined interval
// (VAR_SUBPIPE): K fragments (unit ch * KB + kb) and V^T fragments (unit
// kc * D_BLOCKS + db), read from LDS as in mfma_phase, then consumed by the
// MFMAs of one sub-tile at a time.
template <int D, int VAR>
struct TileFrags {
  f16x8 k[Geometry<D, VAR>::KB * Geometry<D, VAR>::D_CHUNKS];
  f16x8 v[Geometry<D, VAR>::KC * Geometry<D, VAR>::D_BLOCKS];
};

template <int D, int VAR>
__device__ __forceinline__ void read_k_frags(TileFrags<D, VAR>& fr,
                                             const _Float16* __restrict__ ktile, int li, int g) {
  using G = Geometry<D, VAR>;
  const int ksw = k_swizzle<D>(li);
#pragma unroll
  for (int ch = 0; ch < G::D_CHUNKS; ++ch)
#pragma unroll
    for (int kb = 0; kb < G::KB; ++kb)
      fr.k[ch * G::KB + kb] =
          *reinterpret_cast<const f16x8*>(ktile + (16 * kb + li) * D + 8 * ((4 * ch + g) ^ ksw));
}

template <int D, int VAR>
__device__ __forceinline__ void read_v_frags(TileFrags<D, VAR>& fr,
                                             const _Float16* __restrict__ vtile, int li, int g) {
  using G = Geometry<D, VAR>;
  const int vrow = 8 * g + (li >> 2);
  const int vsw = v_swizzle<D>(vrow);
  const _Float16* vlane = vtile + vrow * D + 4 * (li & 1);
  const int vx = (li & 3) >> 1;
#pragma unroll
  for (int kc = 0; kc < G::KC; ++kc)
#pragma unroll
    for (int db = 0; db < G::D_BLOCKS; ++db) {
      const _Float16* vp = vlane + 8 * ((2 * db + vx) ^ vsw) + (32 * kc) * D;
      const f16x4 lo = lds_read_tr(vp);
      const f16x4 hi = lds_read_tr(vp + 4 * D);
      fr.v[kc * G::D_BLOCKS + db] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

// S^T of sub-tile QS from the K fragments and its Q^T fragments.
template <int D, int VAR, int QS>
__device__ __forceinline__ void qk_sub(ScoreSet<D, VAR>& sc, const TileFrags<D, VAR>& fr,
                                       const QSet<D, VAR>& qf) {
  using G = Geometry<D, VAR>;
#pragma unroll
  for (int ch = 0; ch < G::D_CHUNKS; ++ch)
#pragma unroll
    for (int kb = 0; kb < G::KB; ++kb)
      sc[QS][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          fr.k[ch * G::KB + kb], qf[QS][ch], ch == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sc[QS][kb],
          0, 0, 0);
}

// O^T += V^T . P^T of sub-tile QS.
template <int D, int VAR, int QS>
__device__ __forceinline__ void pv_sub(CarrierSet<D, VAR>& cr, const TileFrags<D, VAR>& fr,
                                       const ProbSet<D, VAR>& pf) {
  using G = Geometry<D, VAR>;
#pragma unroll
  for (int kc = 0; kc < G::KC; ++kc)
#pragma unroll
    for (int db = 0; db < G::D_BLOCKS; ++db)
      cr[QS].o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fr.v[kc * G::D_BLOCKS + db],
                                                            pf[QS][kc], cr[QS].o[db], 0, 0, 0);
}

// 2^x on the FMA path (the exponential offload of the VAR_EXP_POLY variant,
// after FlashAttention-4's emulated exponential; the coefficients are this
// project's own fit). x is clamped to [-126, 127]: arguments above still
// overflow fp16 after conversion (so the lazy-max test sees them) and those
// below vanish, and the exponent-field add below cannot reach the sign bit.
// n = floor(x), f = x - n in [0, 1), 2^f by the degree-3 polynomial that
// minimises the largest relative error on [0, 1] (Remez exchange,
// csrc/fit_exp2_poly.py: 7.5e-5, below the fp16 rounding of P), and 2^n
// applied by adding n to the exponent field. Eight VALU instructions against
// one v_exp_f32.
__device__ __forceinline__ float exp2_poly(float x) {
  constexpr float C0 = 9.999251962e-01f, C1 = 6.958335638e-01f, C2 = 2.260671556e-01f,
                  C3 = 7.802452147e-02f;
  x = __builtin_amdgcn_fmed3f(x, -126.0f, 127.0f);
  const float fl = __builtin_floorf(x);
  const float f = x - fl;
  const float p = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(C3, f, C2), f, C1), f, C0);
  return __uint_as_float(__float_as_uint(p) + ((uint32_t)(int)fl << 23));
}

// acc + the low (high) fp16 half of hp, exactly converted, in one fp32
// rounding: v_fma_mix_f32 with an fp16 first operand and 1.0, which the
// compiler does not form from C on its own.
__device__ __forceinline__ float add_f16_lo(float acc, uint32_t hp) {
  asm("v_fma_mix_f32 %0, %1, 1.0, %0 op_sel_hi:[1,0,0]" : "+v"(acc) : "v"(hp));
  return acc;
}
__device__ __forceinline__ float add_f16_hi(float acc, uint32_t hp) {
  asm("v_fma_mix_f32 %0, %1, 1.0, %0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(acc) : "v"(hp));
  return acc;
}

// exp2(t - m) of a 4-score accumulator, hidden keys forced to 0 when MASK;
// with POLY the last of the four on the FMA path.
template <bool MASK, bool POLY>
__device__ __forceinline__ f32x4 exp_block(f32x4 s, float c, float m, uint32_t hid) {
  f32x4 p;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float t = __builtin_fmaf(s[r], c, -m);
    float e = POLY && r == 3 ? exp2_poly(t) : __builtin_amdgcn_exp2f(t);
    if (MASK) e = ((hid >> r) & 1u) ? 0.0f : e;
    p[r] = e;
  }
  return p;
}

// Online softmax of one tile with 32x32 MFMAs (M32): the lane's 32 scores
// of query j (element 4e' + r of block kb: key key0 + 32kb + 8e' + 4h + r),
// probabilities packed in that order (chunk 2kb + x: elements 8x .. 8x + 7
// of block kb), the row sum one v_dot2 chain started from the lane's share
// of the denominator, and the lazy-max test and redo as in softmax_tile.
// The two lanes of a query (h = 0, 1) meet by one lane swap.
template <int D, int VAR, bool CAUSAL, bool MASK>
__device__ __forceinline__ void softmax_m32(CarrierSet<D, VAR>& cr, const ScoreSet<D, VAR>& sc,
                                            ProbSet<D, VAR>& pf, float c, int key0, int qpos0,
                                            int S, int li, int g, bool first) {
  using G = Geometry<D, VAR>;
  const int h = g >> 1;
  uint32_t hid[G::KB];
#pragma unroll
  for (int kb = 0; kb < G::KB; ++kb) {
    hid[kb] = 0u;
    if (MASK) {
      const int qpos = qpos0 + 16 * (g & 1) + li;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = key0 + 32 * kb + 8 * (e >> 2) + 4 * h + (e & 3);
        const bool hd = key >= S || (CAUSAL && key > qpos);
        hid[kb] |= (hd ? 1u : 0u) << e;
      }
    }
  }
  Carrier<D, VAR>& cw = cr[0];
  float dnew = 0.0f;
  auto expo = [&]() {
    const float m = cw.m;
    float acc = cw.d;
#pragma unroll
    for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        f16x8 hv;
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) {
          const int e = 8 * x + e8;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][e], c, -m));
          if (MASK) p = ((hid[kb] >> e) & 1u) ? 0.0f : p;
          hv[e8] = (_Float16)p;
        }
        pf[0][2 * kb + x] = hv;
#pragma unroll
        for (int e8 = 0; e8 < 8; e8 += 2)
          acc = __builtin_amdgcn_fdot2(f16x2{hv[e8], hv[e8 + 1]},
                                       f16x2{(_Float16)1.0f, (_Float16)1.0f}, acc, false);
      }
    dnew = acc;
  };
  if (!first) expo();
  const bool over = first || !(dnew <= cw.d + P_LIMIT);
  if (__builtin_amdgcn_ballot_w64(over) != 0) {
    float tmax = NEG_BIG;
#pragma unroll
    for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float sv = (MASK && ((hid[kb] >> e) & 1u)) ? NEG_BIG : sc[kb][e];
        tmax = __builtin_fmaxf(tmax, sv);
      }
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax),
                                              false, false);
    tmax = __builtin_fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const float m_new = __builtin_fmaxf(cw.m, tmax * c);
    const float alpha = __builtin_amdgcn_exp2f(cw.m - m_new);
    cw.d *= alpha;
#pragma unroll
    for (int ob = 0; ob < G::D_BLOCKS; ++ob) cw.o[ob] *= alpha;
    cw.m = m_new;
    expo();
  }
  cw.d = dnew;
}

// Online softmax of one tile's scores: probabilities (fp16, P^T operand
// layout) into pf, denominators and, when the max moves, outputs rescaled.
struct NoSide {
  __device__ __forceinline__ void operator()() const {}
};

// Pins the side work's MFMAs between the softmax's VALU instructions of one
// scheduling region: its LDS reads first, then each MFMA followed by VPER
// VALU instructions.
template <int VPER, int I, int N>
__device__ __forceinline__ void pin_side_mfmas() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_VALU, VPER, 0);
    pin_side_mfmas<VPER, I + 1, N>();
  }
}

// Online softmax of sub-tiles [QS_LO, QS_HI) of a tile. SIDE_MFMAS > 0: the
// `side` work (SIDE_READS LDS reads and SIDE_MFMAS MFMAs that do not touch
// these sub-tiles) is issued in the same scheduling region, before the
// lazy-max branch, and interleaved with the softmax's VALU instructions.
template <int D, int VAR, bool CAUSAL, bool MASK, int QS_LO = 0, int QS_HI = -1,
          int SIDE_MFMAS = 0, int SIDE_READS = 0, class Side = NoSide>
__device__ __forceinline__ void softmax_tile(CarrierSet<D, VAR>& cr,
                                             const ScoreSet<D, VAR>& sc,
                                             ProbSet<D, VAR>& pf, float c, int key0,
                                             int qpos0, int S, int li, int g, bool first,
                                             Side&& side = Side{}) {
  using G = Geometry<D, VAR>;
  if constexpr (G::M32) {
    static_assert(SIDE_MFMAS == 0 && QS_LO == 0, "32x32 MFMAs: whole-tile softmax only");
    side();
    softmax_m32<D, VAR, CAUSAL, MASK>(cr, sc, pf, c, key0, qpos0, S, li, g, first);
  } else {
  constexpr int QSUB = QS_HI < 0 ? G::QSUB : QS_HI;  // one past the last sub-tile
  side();
  // hidden-key bits per sub-tile and key block (bit r: accumulator element
  // r): keys past S, and (causal) keys after the query's sequence position
  // (qpos0 is the position of the wave's first row)
  uint32_t hid[QSUB][G::KB];
#pragma unroll
  for (int qs = QS_LO; qs < QSUB; ++qs)
#pragma unroll
    for (int kb = 0; kb < G::KB; ++kb) {
      hid[qs][kb] = 0u;
      if (MASK) {
        const int qpos = qpos0 + 16 * qs + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + 32 * (kb >> 1) + 8 * g + 4 * (kb & 1) + r;
          const bool h = key >= S || (CAUSAL && key > qpos);
          hid[qs][kb] |= (h ? 1u : 0u) << r;
        }
      }
    }
  // Row sums of the rounded probabilities: dot products with ones, or (with
  // MIX_SUMS) one mixed-precision add per value. With SUM_ONTO_D (D = 64) a
  // sub-tile's sum is one chain started from the lane's denominator (dnew,
  // whose excess over d is the tile's sum); else two chains from zero
  // (tsum), added onto d afterwards. The tile's sum is tested against the
  // lazy-max bound.
  constexpr bool SUM_ONTO_D = G::PV_SAME;
  float dnew[QSUB], tsum[QSUB];
  auto expo = [&](int qs) {
    const float m = cr[qs].m;
    f32x4 p[G::KB];
#pragma unroll
    for (int kb = 0; kb < G::KB; ++kb) p[kb] = exp_block<MASK, G::EXP_POLY>(sc[qs][kb], c, m, hid[qs][kb]);
    float acc[2] = {SUM_ONTO_D ? cr[qs].d : 0.0f, 0.0f};
#pragma unroll
    for (int kc = 0; kc < G::KC; ++kc) {
      f16x8 h;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        h[r] = (_Float16)p[2 * kc][r];
        h[4 + r] = (_Float16)p[2 * kc + 1][r];
      }
      pf[qs][kc] = h;
      if constexpr (G::MIX_SUMS) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const uint32_t hp = __builtin_bit_cast(uint32_t, f16x2{h[e], h[e + 1]});
          acc[0] = add_f16_lo(acc[0], hp);
          acc[1] = add_f16_hi(acc[1], hp);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int a = SUM_ONTO_D ? 0 : (e >> 1) & 1;
          acc[a] = __builtin_amdgcn_fdot2(f16x2{h[e], h[e + 1]},
                                          f16x2{(_Float16)1.0f, (_Float16)1.0f}, acc[a], false);
        }
      }
    }
    static_assert(!(SUM_ONTO_D && G::MIX_SUMS), "one fp32 chain per sub-tile with v_dot2 only");
    if (SUM_ONTO_D)
      dnew[qs] = acc[0];
    else
      tsum[qs] = acc[0] + acc[1];
  };
  // The first step of a tile starts from m = -inf, so its probabilities
  // overflow by construction: there the row max is taken first and the
  // exponentials are computed once, against it (the same arithmetic as the
  // redo below, without the wasted first pass).
  if (!first) {
#pragma unroll
    for (int qs = QS_LO; qs < QSUB; ++qs) expo(qs);
  }
  if constexpr (SIDE_MFMAS > 0) {
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, SIDE_READS, 0);
    pin_side_mfmas<G::SIDE_VPER, 0, SIDE_MFMAS>();
  }
  // Lazy max: refresh m only when this tile's probabilities could overflow,
  // and only for the sub-tiles whose lanes exceed the bound (one test on the
  // common path; with peaked scores one row in 256 often trips it, and every
  // wave of the workgroup then waits for that redo at the barrier).
  auto big = [&](int qs) {
    return SUM_ONTO_D ? !(dnew[qs] <= cr[qs].d + P_LIMIT) : !(tsum[qs] <= P_LIMIT);
  };
  bool over = first;
  if (!first) {
#pragma unroll
    for (int qs = QS_LO; qs < QSUB; ++qs) over = over || big(qs);
  }
  if (__builtin_amdgcn_ballot_w64(over) != 0) {
#pragma unroll
    for (int qs = QS_LO; qs < QSUB; ++qs) {
      if (!first && __builtin_amdgcn_ballot_w64(big(qs)) == 0) continue;
      float tmax = NEG_BIG;
#pragma unroll
      for (int kb = 0; kb < G::KB; ++kb) {
        f32x4 s = sc[qs][kb];
        if (MASK) {
#pragma unroll
          for (int r = 0; r < 4; ++r) s[r] = ((hid[qs][kb] >> r) & 1u) ? NEG_BIG : s[r];
        }
        tmax = __builtin_fmaxf(tmax, max4(s));
      }
      tmax = group_max(tmax);
      const float m_new = __builtin_fmaxf(cr[qs].m, tmax * c);
      const float alpha = __builtin_amdgcn_exp2f(cr[qs].m - m_new);
      cr[qs].d *= alpha;
#pragma unroll
      for (int db = 0; db < G::D_BLOCKS; ++db) cr[qs].o[db] *= alpha;
      cr[qs].m = m_new;
      expo(qs);
    }
  }
#pragma unroll
  for (int qs = QS_LO; qs < QSUB; ++qs) cr[qs].d = SUM_ONTO_D ? dnew[qs] : cr[qs].d + tsum[qs];
  }
}

template <int D, int VAR, bool CAUSAL, int QS_LO = 0, int QS_HI = -1, int SIDE_MFMAS = 0,
          int SIDE_READS = 0, class Side = NoSide>
__device__ __forceinline__ void softmax_any(CarrierSet<D, VAR>& cr,
                                            const ScoreSet<D, VAR>& sc,
                                            ProbSet<D, VAR>& pf, float c, int key0,
                                            int qpos0, int S, int li, int g, bool first,
                                            Side&& side = Side{}) {
  constexpr int BN = Geometry<D, VAR>::BN;
  // Element masks are needed on the sequence tail and on tiles reaching past
  // the position of the wave's first query (causal diagonal).
  const bool needs_mask = (key0 + BN > S) || (CAUSAL && key0 + BN - 1 > qpos0);
  if (needs_mask)
    softmax_tile<D, VAR, CAUSAL, true, QS_LO, QS_HI, SIDE_MFMAS, SIDE_READS>(
        cr, sc, pf, c, key0, qpos0, S, li, g, first, side);
  else
    softmax_tile<D, VAR, CAUSAL, false, QS_LO, QS_HI, SIDE_MFMAS, SIDE_READS>(
        cr, sc, pf, c, key0, qpos0, S, li, g, first, side);
}

// Workgroup id -> (batch*head, query tiles) by `order` (work_order.h).
//
// Schedule. Key interval j holds tiles NPH*j .. NPH*j + NPH - 1; the wave of
// phase p folds tile NPH*j + p, with K and V copied into LDS during the
// interval before they are read.
//  D = 64: interval j is Q.K^T of tile j, the softmax, then P.V of tile j.
//  D = 128: interval j is an MFMA phase (P.V of interval j-1, Q.K^T of
//    interval j) and the softmax of interval j; the second wave of each SIMD
//    (waves 4-7) takes the two halves in the other order (softmax of interval
//    j-1 first), so that one wave's softmax runs against the other's MFMA
//    phase.
//
// SPLIT: the key range of each query tile is cut into n_splits runs of whole
// intervals (split-KV). Workgroup (query tile, head, split) folds its run and
// stores the partial result -- o/d in fp32 and m + log2(d) -- into the
// workspace instead of O and LSE; attn_combine_kernel merges the runs.
template <int D, bool CAUSAL, bool SPLIT, int VAR = 0>
__global__ __launch_bounds__((Geometry<D, VAR>::WG_THREADS)) void attn_fwd_kernel(
    const _Float16* __restrict__ q, const _Float16* __restrict__ k,
    const _Float16* __restrict__ v, _Float16* __restrict__ o, float* __restrict__ lse,
    int BH, int Sq, int Sk, int n_qtiles, int n_splits, int order, float c, uint32_t qsign,
    float* __restrict__ part_o, float* __restrict__ part_lse) {
  using G = Geometry<D, VAR>;
  constexpr int R = G::RING;
  constexpr int QSUB = G::QSUB;
  constexpr int NPH = G::NPH;
  __shared__ __attribute__((aligned(16))) _Float16 smem[G::LDS_HALVES];
  _Float16* kring = smem;                           // [slot][tile] K tiles
  _Float16* vring = smem + G::KRING * G::SLOT_HALVES;  // [slot][tile] V tiles

  const int split = SPLIT ? (int)(blockIdx.x % (unsigned)n_splits) : 0;
  const int bid = SPLIT ? (int)(blockIdx.x / (unsigned)n_splits) : (int)blockIdx.x;
  const TileWork work = work_of(SPLIT ? ORDER_TILES : order, bid, BH, n_qtiles);
  const int bh = work.bh;
  const int64_t qhead = (int64_t)bh * Sq * D;   // Q and O of this head
  const int64_t kvhead = (int64_t)bh * Sk * D;  // K and V of this head
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(q + qhead, (uint32_t)Sq * D * 2);
  const _Float16* kh = k + kvhead;
  const _Float16* vh = v + kvhead;
  // Query row i sits at sequence position i + koff (the queries are the last
  // Sq positions); causal masking hides keys after a query's position.
  const int koff = Sk - Sq;
  const int S = Sk;  // keys per head: the range of the K/V descriptors and masks

  // One query tile: Q load, the key loop and the epilogue.
  auto run_tile = [&](const int qt) __attribute__((always_inline)) {
    // Lane indices are derived afresh for each tile (the empty asm hides
    // the thread id from the optimiser), so that nothing lane-dependent is
    // hoisted out of the tile loop and held in registers across the key loop.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int li = lane & 15;
    const int g = lane >> 4;
    // The NPH waves of a query group are consecutive, so that they run on
    // different SIMDs: when only the first query group has live rows (a few
    // queries against a long cache) its waves do not share a SIMD.
    const int qgrp = wave / NPH;
    const int phase = wave % NPH;
    const bool late = wave >= WAVES / 2;  // second wave of its SIMD
    // With producer waves (waves 8-11) the copies are theirs alone; else
    // every wave copies its share.
    const bool producer = G::PROD && wave >= G::CWAVES;
    const int cw = G::PROD ? wave - G::CWAVES : wave;  // index among the copying waves
    const int q0 = qt * BLOCK_M;
    const int qrow0 = q0 + G::ROWS * qgrp;  // this wave's first query row
    const int qpos0 = qrow0 + koff;         // its sequence position

    // Q^T fragments, loaded once into registers (sign-flipped when the scale
    // is negative); rows past S_q read as zeros (outside the descriptor's
    // range; offsets are unsigned 32-bit, S_q * D * 2 < 2^31).
    f16x8 qf[QSUB][G::D_CHUNKS];
    if (producer) {
      // no query rows
    } else if constexpr (G::M32) {
      // lane (j, h): row qrow0 + j, halves 16dc + 8h of each d chunk dc
      const int row = qrow0 + 16 * (g & 1) + li;
  #pragma unroll
      for (int dc = 0; dc < G::D_CHUNKS; ++dc) {
        u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
            qrs, ((uint32_t)row * D + 16u * dc + 8u * (g >> 1)) * 2u, 0, 0);
        w ^= qsign;
        qf[0][dc] = __builtin_bit_cast(f16x8, w);
      }
    } else {
  #pragma unroll
      for (int qs = 0; qs < QSUB; ++qs) {
        const int row = qrow0 + 16 * qs + li;
  #pragma unroll
        for (int ch = 0; ch < G::D_CHUNKS; ++ch) {
          u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
              qrs, ((uint32_t)row * D + 32u * ch + 8u * g) * 2u, 0, 0);
          w ^= qsign;
          qf[qs][ch] = __builtin_bit_cast(f16x8, w);
        }
      }
    }

    Carrier<D, VAR> cr[QSUB];
  #pragma unroll
    for (int qs = 0; qs < QSUB; ++qs) {
      cr[qs].m = NEG_BIG;
      cr[qs].d = 0.f;
  #pragma unroll
      for (int db = 0; db < G::D_BLOCKS; ++db) cr[qs].o[db] = typename G::Acc{};
    }
    // sc: a tile's scores between Q.K^T and softmax; pf: its fp16
    // probabilities between softmax and P.V (at D = 128 carried across the
    // barrier into the next interval).
    ProbSet<D, VAR> pf;
    ScoreSet<D, VAR> sc;

    const int kend = CAUSAL ? min(S, q0 + BLOCK_M + koff) : S;
    const int n_kt = (kend + G::BN - 1) / G::BN;
    const int n_int_all = (n_kt + NPH - 1) / NPH;
    // This workgroup folds intervals [pb, pb + n_int): all of them, or its
    // split's run.
    const int pb = SPLIT ? (int)((int64_t)split * n_int_all / n_splits) : 0;
    const int n_int = SPLIT ? (int)((int64_t)(split + 1) * n_int_all / n_splits) - pb : n_int_all;
    // Intervals whose tile of this wave's phase holds keys for its rows: a
    // prefix, since tiles past S or past the wave's last query (causal) are
    // skipped. A wave with no query row below Sq (the last query tile of a
    // short query block) only copies and synchronises.
    const int row_end = CAUSAL ? min(kend, qpos0 + G::ROWS) : kend;  // keys < row_end are needed
    const int live_tiles = (row_end + G::BN - 1) / G::BN;
    const int n_live = qrow0 >= Sq ? 0 : min(max((live_tiles - phase + NPH - 1) / NPH - pb, 0), n_int);
    constexpr bool PINGPONG = G::PINGPONG;
    // Only the last live interval of a wave can need element masks: the
    // sequence tail is in the last tile, and the tiles crossing the causal
    // diagonal of the wave's rows are the last ones at or below them, which
    // fall to different phases. (The last live interval of a split run is
    // checked at run time.)

    // Key order. Loop step x folds the keys at interval position pos(x). In
    // a non-causal single pass every wave is live in every interval but
    // possibly the last (the sequence tail, the only one with masks), so the
    // order of the others is free: there, every other round of 32 workgroups
    // per XCD (workgroup ids are dealt round-robin to 8 XCDs) walks them
    // backwards, starting on the K/V that the round before it left in the
    // XCD's L2 (at B1 H8 S16384 D64 the fetched bytes halve), and still ends
    // on the last interval. Elsewhere the order is ascending.
    const bool backwards = !CAUSAL && !SPLIT && ((blockIdx.x >> 8) & 1u) != 0u;
    auto pos = [&](int x) {
      return pb + (backwards && x < n_int - 1 ? n_int - 2 - x : x);
    };

    CopyPlan<D, VAR> cp;
    make_copy_plan<D, VAR>(cp, cw, lane);
    const bool copier = !G::PROD || producer;
    if (copier && n_int > 0)
      copy_group<D, VAR>(cp.k_off, kh, pos(0) * G::IKEYS, S, kring, cw);  // K of step 0
    if constexpr (G::PV_SAME) {
      if (copier && n_int > 0)
        copy_group<D, VAR>(cp.v_off, vh, pos(0) * G::IKEYS, S, vring, cw);  // V of step 0
    }
    if constexpr (G::PV_SAME && G::BAR2) {
      // four-slot ring: steps 0 and 1 land before the first barrier
      if (n_int > 1) {
        copy_group<D, VAR>(cp.k_off, kh, pos(1) * G::IKEYS, S, kring + G::SLOT_HALVES, cw);
        copy_group<D, VAR>(cp.v_off, vh, pos(1) * G::IKEYS, S, vring + G::SLOT_HALVES, cw);
      }
      wait_copies();
    } else if constexpr (G::PV_SAME && R == 3) {
      // three-slot ring: step 1 is in flight from the start
      if (n_int > 1) {
        copy_group<D, VAR>(cp.k_off, kh, pos(1) * G::IKEYS, S, kring + G::SLOT_HALVES, cw);
        copy_group<D, VAR>(cp.v_off, vh, pos(1) * G::IKEYS, S, vring + G::SLOT_HALVES, cw);
        wait_copies_keep<2 * G::LOADS>();
      } else {
        wait_copies();
      }
    } else {
      wait_copies();
    }
    __syncthreads();

    if constexpr (G::PROD) {
      if (producer) {
        // Interval j: right after the barrier that ends interval j - 1 (whose
        // slot the compute waves no longer read), copy K and V of interval
        // j + 1 into that slot; wait; meet the compute waves at the barrier
        // that ends interval j. Then the epilogue's barrier, and done.
        for (int j = 0; j < n_int; ++j) {
          if (j + 1 < n_int) {
            const int sl = (j + 1) % R;
            copy_group<D, VAR>(cp.k_off, kh, pos(j + 1) * G::IKEYS, S,
                               kring + sl * G::SLOT_HALVES, cw);
            copy_group<D, VAR>(cp.v_off, vh, pos(j + 1) * G::IKEYS, S,
                               vring + sl * G::SLOT_HALVES, cw);
          }
          wait_copies();
          __syncthreads();
        }
        __syncthreads();  // the carrier hand-off of the compute waves
        return;
      }
    }

    // Two-phase order (D = 128), barrier interval j (counted from pb): P.V of
    // interval j-1 and Q.K^T of interval j (MFMA), then the copies of K of
    // interval j+1 and V of interval j, then the softmax of interval j
    // (VALU); the probabilities stay in registers for interval j+1. The
    // copies sit between the MFMA phase (whose LDS reads they would slow) and
    // the softmax (which does not touch LDS). K of interval j is read from
    // ring slot j % 2 and V of interval j-1 from slot (j-1) % 2, both copied
    // in interval j-1. Every wave runs all n_int + 1 intervals; the bodies
    // are specialised (compile-time flags) so that the steady state has no
    // branches.
    // K ring slot of interval j (two slots, or three with ROT)
    auto kslot_of = [](int j) { return G::KRING == 2 ? (j & 1) : (int)((unsigned)j % G::KRING); };
    auto copies = [&](int j) __attribute__((always_inline)) {
      if (j + 1 < n_int)
        copy_group<D, VAR>(cp.k_off, kh, pos(j + 1) * G::IKEYS, S,
                      kring + kslot_of(j + 1) * G::SLOT_HALVES, cw);
      if (j < n_int)
        copy_group<D, VAR>(cp.v_off, vh, pos(j) * G::IKEYS, S,
                      vring + (j & 1) * G::SLOT_HALVES, cw);
      if constexpr (G::SYNC) {
        wait_copies();
        __syncthreads();
      }
    };
    // softmax of this wave's tile of interval p (masks possible when EDGE)
    auto softmax_int = [&](int p, auto edge_flag) __attribute__((always_inline)) {
      if constexpr (G::SOFTMAX_PRIO) __builtin_amdgcn_s_setprio(2);
      const int key0 = pos(p) * G::IKEYS + phase * G::BN;
      if constexpr (decltype(edge_flag)::value)
        softmax_any<D, VAR, CAUSAL>(cr, sc, pf, c, key0, qpos0, S, li, g, p == 0);
      else
        softmax_tile<D, VAR, CAUSAL, false>(cr, sc, pf, c, key0, qpos0, S, li, g, p == 0);
      if constexpr (G::SOFTMAX_PRIO) __builtin_amdgcn_s_setprio(0);
    };
    auto mfma = [&](int j, auto pv_flag, auto qk_flag) __attribute__((always_inline)) {
      constexpr bool PV = decltype(pv_flag)::value;
      constexpr bool QK = decltype(qk_flag)::value;
      const _Float16* kslot = kring + kslot_of(j) * G::SLOT_HALVES + phase * G::K_HALVES;
      const _Float16* vslot = vring + ((j + 1) & 1) * G::SLOT_HALVES + phase * G::V_HALVES;
      if constexpr (PV || QK) mfma_phase<D, VAR, PV, QK>(cr, pf, sc, qf, vslot, kslot, li, g);
    };
    auto end_interval = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      wait_copies();
      __syncthreads();
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    int j = 0;
    if constexpr (G::PV_SAME) {
      // Three-phase order (D = 64), interval j: Q.K^T of interval j, copies of
      // K and V of interval j + R - 1 (into the slot of interval j-1, read in
      // interval j-1), softmax of interval j, P.V of interval j. Every wave
      // runs n_int intervals. With a three-slot ring the copies run two
      // intervals ahead of their use, so their latency (about as long as an
      // interval) is off the barrier's critical path.
      constexpr int AH = G::AHEAD;  // intervals between a copy and its use
      auto copies_ahead = [&](int jj) __attribute__((always_inline)) {
        if (!G::PROD && jj + AH < n_int) {
          const int sl = (jj + AH) % R;
          copy_group<D, VAR>(cp.k_off, kh, pos(jj + AH) * G::IKEYS, S,
                        kring + sl * G::SLOT_HALVES, cw);
          copy_group<D, VAR>(cp.v_off, vh, pos(jj + AH) * G::IKEYS, S,
                        vring + sl * G::SLOT_HALVES, cw);
        }
        if constexpr (G::SYNC) {
          wait_copies();
          __syncthreads();
        }
      };
      // End of interval jj: the copies of interval jj + 1 must have landed
      // (those of jj + 2, issued in this interval, may still run).
      auto end_int = [&](int jj) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (G::BAR2) {
          // barrier after odd steps only: copies issued in steps jj - 1 and jj
          // (for jj + 1 and jj + 2, both read before the next barrier) land
          if (jj & 1) {
            wait_copies();
            __syncthreads();
          }
          return;
        }
        if (R > 2 && jj + AH < n_int)
          wait_copies_keep<2 * G::LOADS>();
        else
          wait_copies();
        __syncthreads();
      };
      // Sub-tile pipelined interval (SUBPIPE): Q.K^T of sub-tile 0; then Q.K^T
      // of sub-tile 1 and the V^T reads beside the softmax of sub-tile 0; then
      // P.V of sub-tile 0 beside the softmax of sub-tile 1; then P.V of
      // sub-tile 1. Each softmax ends with its own lazy-max branch, so the
      // MFMAs beside it never depend on a redo.
      auto softmax_sub = [&](int jj, auto edge_flag, auto qs_flag, auto nside, auto nread,
                             auto&& side) __attribute__((always_inline)) {
        constexpr int QS = decltype(qs_flag)::value;
        constexpr int NS = decltype(nside)::value;
        constexpr int NR = decltype(nread)::value;
        const int key0 = pos(jj) * G::IKEYS + phase * G::BN;
        if constexpr (decltype(edge_flag)::value)
          softmax_any<D, VAR, CAUSAL, QS, QS + 1, NS, NR>(cr, sc, pf, c, key0, qpos0, S, li, g,
                                                          jj == 0, side);
        else
          softmax_tile<D, VAR, CAUSAL, false, QS, QS + 1, NS, NR>(cr, sc, pf, c, key0, qpos0, S,
                                                                  li, g, jj == 0, side);
      };
      auto full_sp = [&](int jj, auto edge_flag, auto slot_flag) __attribute__((always_inline)) {
        if constexpr (G::SUBPIPE) {
          constexpr int SL = decltype(slot_flag)::value;
          const int slot = SL >= 0 ? SL : jj % R;
          const _Float16* kslot = kring + slot * G::SLOT_HALVES + phase * G::K_HALVES;
          const _Float16* vslot = vring + slot * G::SLOT_HALVES + phase * G::V_HALVES;
          using I0 = std::integral_constant<int, 0>;
          using I1 = std::integral_constant<int, 1>;
          using NQK = std::integral_constant<int, G::KB * G::D_CHUNKS>;
          using NPV = std::integral_constant<int, G::KC * G::D_BLOCKS>;
          using NVR = std::integral_constant<int, 2 * G::KC * G::D_BLOCKS>;
          TileFrags<D, VAR> fr;
          read_k_frags<D, VAR>(fr, kslot, li, g);
          qk_sub<D, VAR, 0>(sc, fr, qf);
          __builtin_amdgcn_sched_barrier(0);
          copies_ahead(jj);
          __builtin_amdgcn_sched_barrier(0);
          softmax_sub(jj, edge_flag, I0{}, NQK{}, NVR{}, [&]() __attribute__((always_inline)) {
            qk_sub<D, VAR, 1>(sc, fr, qf);
            read_v_frags<D, VAR>(fr, vslot, li, g);
          });
          __builtin_amdgcn_sched_barrier(0);
          softmax_sub(jj, edge_flag, I1{}, NPV{}, I0{}, [&]() __attribute__((always_inline)) {
            pv_sub<D, VAR, 0>(cr, fr, pf);
          });
          __builtin_amdgcn_sched_barrier(0);
          pv_sub<D, VAR, 1>(cr, fr, pf);
          end_int(jj);
        }
      };
      // slot_flag: the ring slot of interval jj as a compile-time constant,
      // or -1 to take it from jj at run time.
      auto full = [&](int jj, auto edge_flag, auto slot_flag) __attribute__((always_inline)) {
        if constexpr (G::SUBPIPE) {
          full_sp(jj, edge_flag, slot_flag);
          return;
        }
        constexpr int SL = decltype(slot_flag)::value;
        const int slot = SL >= 0 ? SL : jj % R;
        const _Float16* kslot = kring + slot * G::SLOT_HALVES + phase * G::K_HALVES;
        const _Float16* vslot = vring + slot * G::SLOT_HALVES + phase * G::V_HALVES;
        mfma_phase<D, VAR, false, true>(cr, pf, sc, qf, vslot, kslot, li, g);
        __builtin_amdgcn_sched_barrier(0);
        copies_ahead(jj);
        __builtin_amdgcn_sched_barrier(0);
        softmax_int(jj, edge_flag);
        __builtin_amdgcn_sched_barrier(0);
        mfma_phase<D, VAR, true, false>(cr, pf, sc, qf, vslot, kslot, li, g);
        end_int(jj);
      };
      using S0 = std::integral_constant<int, 0>;
      using S1 = std::integral_constant<int, 1>;
      using S2 = std::integral_constant<int, 2>;
      using S3 = std::integral_constant<int, 3>;
      using SR = std::integral_constant<int, -1>;
      // Steady state unrolled by the ring depth, so that the ring slots are
      // constant offsets of the LDS reads rather than addresses computed per
      // interval.
      if constexpr (R == 4) {
        for (; j + 4 < n_live; j += 4) {
          full(j, F_{}, S0{});
          full(j + 1, F_{}, S1{});
          full(j + 2, F_{}, S2{});
          full(j + 3, F_{}, S3{});
        }
        for (; j + 1 < n_live; ++j) full(j, F_{}, SR{});
      } else if constexpr (R == 3) {
        for (; j + 3 < n_live; j += 3) {
          full(j, F_{}, S0{});
          full(j + 1, F_{}, S1{});
          full(j + 2, F_{}, S2{});
        }
        for (; j + 1 < n_live; ++j) full(j, F_{}, SR{});
      } else {
        for (; j + 2 < n_live; j += 2) {
          full(j, F_{}, S0{});
          full(j + 1, F_{}, S1{});
        }
        if (j + 1 < n_live) full(j++, F_{}, S0{});  // j is even here
      }
      if (j + 1 == n_live) full(j++, T_{}, SR{});
      for (; j < n_int; ++j) {
        copies_ahead(j);
        end_int(j);
      }
      if constexpr (G::BAR2) {
        // the last step was even: no barrier ended it
        if (n_int > 0 && ((n_int - 1) & 1) == 0) {
          wait_copies();
          __syncthreads();
        }
      }
    } else {
      // Two-phase order as one instruction stream for every wave: interval
      // body j is the MFMA phase (P.V of j-1, Q.K^T of j), then the softmax
      // of j. The first wave of each SIMD ends its interval after the
      // softmax; with PINGPONG the second wave (waves 4-7) ends it right after
      // the MFMA phase, so between two barriers it runs the softmax of j-1
      // and then the MFMA phase of j while its partner runs the MFMA phase
      // and then the softmax of j: one wave's softmax overlaps the other's
      // MFMAs. Only the barrier and the copies move with the role (uniform
      // branches), so both roles share one register allocation. Each wave
      // issues its share of the copies of interval j (K of j+1, V of j)
      // inside interval j: the first role between its MFMA phase and softmax,
      // the second after its softmax. Every wave runs n_int + 1 bodies, each
      // with one barrier.
      const bool second = PINGPONG && late;
      // ROT: role r = wave / 4 (the r-th wave of each SIMD) ends its interval
      // after the softmax (0), after Q.K^T (1) or after P.V (2), and issues
      // the copies of an interval right after the barrier that opens it.
      // Interval k then holds, per role: P.V of k-1, Q.K^T of k, softmax of
      // k (0); softmax of k-1, P.V of k-1, Q.K^T of k (1); Q.K^T of k-1,
      // softmax of k-1, P.V of k-1 (2). K of k-1 and k are read in interval
      // k (a three-slot K ring), V of k-1 only; the copies of interval k
      // (K of k+1, V of k) overwrite K of k-2 and V of k-2, last read in
      // interval k-1.
      const int role = G::ROT ? wave / (G::CWAVES / 3) : 0;
      auto end_interval_rot = [&](int jj) __attribute__((always_inline)) {
        wait_copies();
        __syncthreads();
        copies(jj + 1);
      };
      auto body = [&](int jj, auto pv_flag, auto qk_flag, auto edge_flag) __attribute__((always_inline)) {
        constexpr bool PV = decltype(pv_flag)::value;
        constexpr bool QK = decltype(qk_flag)::value;
        if constexpr (G::ROT) {
          if (role == 0) copies(jj);
          __builtin_amdgcn_sched_barrier(0);
          mfma(jj, pv_flag, F_{});
          __builtin_amdgcn_sched_barrier(0);
          if (role == 2) end_interval_rot(jj);
          __builtin_amdgcn_sched_barrier(0);
          mfma(jj, F_{}, qk_flag);
          __builtin_amdgcn_sched_barrier(0);
          if (role == 1) end_interval_rot(jj);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (QK) softmax_int(jj, edge_flag);
          __builtin_amdgcn_sched_barrier(0);
          if (role == 0) {
            wait_copies();
            __syncthreads();
          }
          (void)PV;
          return;
        }
        mfma(jj, pv_flag, qk_flag);
        __builtin_amdgcn_sched_barrier(0);
        if (second) {
          wait_copies();
          __syncthreads();
        } else {
          copies(jj);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (QK) softmax_int(jj, edge_flag);
        __builtin_amdgcn_sched_barrier(0);
        if (second) {
          copies(jj + 1);
        } else {
          wait_copies();
          __syncthreads();
        }
      };
      if (second || (G::ROT && role != 0)) copies(0);
      if (n_live >= 1)
        body(j++, F_{}, T_{}, T_{});
      else
        body(j++, F_{}, F_{}, F_{});
      for (; j + 1 < n_live; ++j) body(j, T_{}, T_{}, F_{});  // steady state
      if (j + 1 == n_live) body(j++, T_{}, T_{}, T_{});       // last live interval
      if (j == n_live && j >= 1) body(j++, T_{}, F_{}, F_{}); // its P.V
      for (; j <= n_int; ++j) body(j, F_{}, F_{}, F_{});      // idle: copies, barriers
    }

    float* lse_h = lse + (int64_t)bh * Sq;
    _Float16* oh = o + qhead;
    const int64_t part_row0 = ((int64_t)split * BH + bh) * Sq;  // SPLIT: workspace rows
    f32x4* area = reinterpret_cast<f32x4*>(smem) + lane;
    if constexpr (G::M32) {
      // Carrier hand-off with 32x32 MFMAs: per wave one slot {m, d, -, -} and
      // one slot per quarter block it does not finalise (quarter qd: elements
      // 4(qd % 4) .. +3 of block qd / 4, O^T rows 32(qd / 4) + 8(qd % 4) + 4h
      // + r); each wave merges the quarters it owns (owner_q(qd) == phase).
      const int h = g >> 1;
      auto md_slot = [&](int w) { return area + (w * G::HANDOFF_SLOTS) * 64; };
      auto q_slot = [&](int w, int qd) {
        return area + (w * G::HANDOFF_SLOTS + G::MD_SLOTS + qd) * 64;
      };
      auto quarter = [&](int qd) {
        const f32x16& a = cr[0].o[qd / 4];
        const int e0 = 4 * (qd % 4);
        return f32x4{a[e0], a[e0 + 1], a[e0 + 2], a[e0 + 3]};
      };
      *md_slot(wave) = f32x4{cr[0].m, cr[0].d, 0.0f, 0.0f};
  #pragma unroll
      for (int qd = 0; qd < G::QUARTERS; ++qd)
        if (G::owner_q(qd) != phase) *q_slot(wave, qd) = quarter(qd);
      __syncthreads();
      float mp[NPH], dp[NPH], w[NPH];
      float m = NEG_BIG;
  #pragma unroll
      for (int p = 0; p < NPH; ++p) {
        const f32x4 md = *md_slot(qgrp * NPH + p);
        mp[p] = md[0];
        dp[p] = md[1];
        m = __builtin_fmaxf(m, mp[p]);
      }
      float dl = 0.0f;
  #pragma unroll
      for (int p = 0; p < NPH; ++p) {
        w[p] = __builtin_amdgcn_exp2f(mp[p] - m);
        dl += dp[p] * w[p];
      }
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(dl), __float_as_uint(dl), false,
                                                 false);
      const float dsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const int row = qrow0 + 16 * (g & 1) + li;
      const bool empty = SPLIT && !(dsum > 0.0f);
      const float inv = empty ? 0.0f : 1.0f / dsum;
      if (row < Sq) {
  #pragma unroll
        for (int qd = 0; qd < G::QUARTERS; ++qd) {
          if (G::owner_q(qd) != phase) continue;
          f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  #pragma unroll
          for (int p = 0; p < NPH; ++p) {
            if (p == G::owner_q(qd))
              acc += quarter(qd) * w[p];
            else
              acc += *q_slot(qgrp * NPH + p, qd) * w[p];
          }
          const int col = 32 * (qd / 4) + 8 * (qd % 4) + 4 * h;
          if constexpr (SPLIT) {
            float* po = part_o + (part_row0 + row) * D;
            *reinterpret_cast<f32x4*>(po + col) = acc * inv;
          } else {
            f16x4 hv;
  #pragma unroll
            for (int r = 0; r < 4; ++r) hv[r] = (_Float16)(acc[r] * inv);
            *reinterpret_cast<f16x4*>(oh + (int64_t)row * D + col) = hv;
          }
        }
        if (phase == 0 && h == 0) {
          if constexpr (SPLIT)
            part_lse[part_row0 + row] = empty ? NEG_BIG : m + log2f(dsum);
          else
            lse_h[row] = (m + log2f(dsum)) * 0.69314718055994530942f;
        }
      }
    } else {
    // Carrier hand-off. Every wave leaves its carriers in LDS -- per pair of
    // sub-tiles one 16-byte slot {m, d, m, d}, and the output blocks it does
    // not finalise, one slot per block -- each lane at 16 * lane in a slot, so
    // reads and writes are conflict-free. Then each wave merges the NPH
    // carriers of its query group for the blocks it owns (owner(db) ==
    // phase). Block and partner indices are
    // compile-time (unrolled loops with wave-uniform branches on the phase),
    // so no register array is indexed at run time. The last interval ended
    // with a barrier, so the ring is no longer read.
    auto md_slot = [&](int w, int qs) { return area + (w * G::HANDOFF_SLOTS + qs / 2) * 64; };
    auto o_slot = [&](int w, int qs, int db) {
      return area + (w * G::HANDOFF_SLOTS + G::MD_SLOTS + qs * G::D_BLOCKS + db) * 64;
    };
  #pragma unroll
    for (int qs = 0; qs < QSUB; qs += 2) {
      f32x4 md;
      md[0] = cr[qs].m;
      md[1] = cr[qs].d;
      md[2] = qs + 1 < QSUB ? cr[qs + 1].m : 0.0f;
      md[3] = qs + 1 < QSUB ? cr[qs + 1].d : 0.0f;
      *md_slot(wave, qs) = md;
    }
  #pragma unroll
    for (int qs = 0; qs < QSUB; ++qs)
  #pragma unroll
      for (int db = 0; db < G::D_BLOCKS; ++db)
        if (G::owner(db) != phase) *o_slot(wave, qs, db) = cr[qs].o[db];
    __syncthreads();

  #pragma unroll
    for (int qs = 0; qs < QSUB; ++qs) {
      // merged max, each carrier's weight, and the row's denominator
      float mp[NPH], dp[NPH], w[NPH];
      float m = NEG_BIG;
  #pragma unroll
      for (int p = 0; p < NPH; ++p) {
        const f32x4 md = *md_slot(qgrp * NPH + p, qs);
        mp[p] = md[(qs & 1) * 2];
        dp[p] = md[(qs & 1) * 2 + 1];
        m = __builtin_fmaxf(m, mp[p]);
      }
      float dl = 0.0f;
  #pragma unroll
      for (int p = 0; p < NPH; ++p) {
        w[p] = __builtin_amdgcn_exp2f(mp[p] - m);
        dl += dp[p] * w[p];
      }
      const float dsum = group_sum(dl);
      const int row = qrow0 + 16 * qs + li;
      // A run of a split can hold no visible key for a row (empty run, or
      // causal keys above the row): its partial is o = 0 with weight
      // 2^NEG_BIG = 0. A single pass always sees key 0.
      const bool empty = SPLIT && !(dsum > 0.0f);
      const float inv = empty ? 0.0f : 1.0f / dsum;
      if (row < Sq) {
  #pragma unroll
        for (int db = 0; db < G::D_BLOCKS; ++db) {
          if (G::owner(db) != phase) continue;
          f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  #pragma unroll
          for (int p = 0; p < NPH; ++p) {
            if (p == G::owner(db))
              acc += cr[qs].o[db] * w[p];
            else
              acc += *o_slot(qgrp * NPH + p, qs, db) * w[p];
          }
          if constexpr (SPLIT) {
            float* po = part_o + (part_row0 + row) * D;
            *reinterpret_cast<f32x4*>(po + 16 * db + 4 * g) = acc * inv;
          } else {
            f16x4 h;
  #pragma unroll
            for (int r = 0; r < 4; ++r) h[r] = (_Float16)(acc[r] * inv);
            *reinterpret_cast<f16x4*>(oh + (int64_t)row * D + 16 * db + 4 * g) = h;
          }
        }
        if (phase == 0 && g == 0) {
          if constexpr (SPLIT)
            part_lse[part_row0 + row] = empty ? NEG_BIG : m + log2f(dsum);
          else
            lse_h[row] = (m + log2f(dsum)) * 0.69314718055994530942f;
        }
      }
    }
    }
  };
  run_tile(work.qt_first);
  if constexpr (CAUSAL && !SPLIT) {
    if (work.qt_second >= 0) {
      // The second tile's copies overwrite the LDS that the first tile's
      // epilogue reads: all waves meet before it starts.
      __syncthreads();
      run_tile(work.qt_second);
    }
  }
}

// Merge of the split-KV partial results (the carrier merge law, with each
// run's state given as o_s = o/d and l_s = m + log2 d): for every row,
// M = max_s l_s, w_s = 2^(l_s - M), O = sum_s w_s o_s / sum_s w_s and
// LSE = (M + log2 sum_s w_s) ln 2. Two forms, chosen by the launch plan:
//
// attn_combine_kernel: one thread per row and 4 columns, the runs in turn.
// Reads and writes are contiguous along the row; for launches with many rows
// (prefill) it is HBM-bound.
template <int D>
__global__ __launch_bounds__(COMBINE_THREADS) void attn_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse,
    _Float16* __restrict__ o, float* __restrict__ lse, int64_t rows, int n_splits) {
  constexpr int TPR = D / 4;  // threads per row
  const int64_t items = rows * TPR;
  for (int64_t t = (int64_t)blockIdx.x * COMBINE_THREADS + threadIdx.x; t < items;
       t += (int64_t)gridDim.x * COMBINE_THREADS) {
    const int64_t row = t / TPR;
    const int c4 = (int)(t % TPR);
    float M = NEG_BIG;
    for (int s = 0; s < n_splits; ++s) M = __builtin_fmaxf(M, part_lse[s * rows + row]);
    float W = 0.0f;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s = 0; s < n_splits; ++s) {
      const float w = __builtin_amdgcn_exp2f(part_lse[s * rows + row] - M);
      const f32x4 v = *reinterpret_cast<const f32x4*>(part_o + (s * rows + row) * D + 4 * c4);
      W += w;
      acc += w * v;
    }
    const float inv = 1.0f / W;
    f16x4 h;
#pragma unroll
    for (int r = 0; r < 4; ++r) h[r] = (_Float16)(acc[r] * inv);
    *reinterpret_cast<f16x4*>(o + row * D + 4 * c4) = h;
    if (c4 == 0) lse[row] = (M + log2f(W)) * 0.69314718055994530942f;
  }
}

// attn_combine_runs_kernel: one wave per row, for launches with few rows and
// many runs (decode), where the form above would wait on one run after
// another. Lane 16g + i holds
// columns [CW i, CW i + CW) (CW = D / 16) of the runs s = g, g + 4, ..., all
// loaded at once, so that the merge is one round trip of loads; the four lane
// groups' maxima and sums then meet by lane swaps.
//
// Both grids stride over the rows, so any row count fits a bounded grid.
template <int D>
__global__ __launch_bounds__(COMBINE_THREADS) void attn_combine_runs_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse,
    _Float16* __restrict__ o, float* __restrict__ lse, int64_t rows, int n_splits) {
  constexpr int CW = D / 16;  // columns per lane
  constexpr int NV = CW / 4;  // f32x4 loads per lane and run
  constexpr int WPB = COMBINE_THREADS / 64;
  constexpr int RUNS = (MAX_SPLITS + 3) / 4;  // runs per lane group, at most
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int g = lane >> 4;
  const int64_t first = (int64_t)blockIdx.x * WPB + (threadIdx.x >> 6);
  for (int64_t row = first; row < rows; row += (int64_t)gridDim.x * WPB) {
    float l[RUNS];
    f32x4 po[RUNS][NV];
#pragma unroll
    for (int i = 0; i < RUNS; ++i) {
      const int s = g + 4 * i;
      if (s < n_splits) {
        l[i] = part_lse[s * rows + row];
        const float* src = part_o + (s * rows + row) * D + CW * li;
#pragma unroll
        for (int v = 0; v < NV; ++v) po[i][v] = *reinterpret_cast<const f32x4*>(src + 4 * v);
      } else {
        l[i] = NEG_BIG;
#pragma unroll
        for (int v = 0; v < NV; ++v) po[i][v] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
    float M = NEG_BIG;
#pragma unroll
    for (int i = 0; i < RUNS; ++i) M = __builtin_fmaxf(M, l[i]);
    M = group_max(M);
    float W = 0.0f;
    f32x4 acc[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < RUNS; ++i) {
      // runs past n_splits, and runs with no visible key, have l = NEG_BIG:
      // weight 0 against the finite M of a run that saw key 0
      const float w = __builtin_amdgcn_exp2f(l[i] - M);
      W += w;
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[v] += w * po[i][v];
    }
    W = group_sum(W);
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[v][r] = group_sum(acc[v][r]);
    if (g == 0) {
      const float inv = 1.0f / W;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        f16x4 h;
#pragma unroll
        for (int r = 0; r < 4; ++r) h[r] = (_Float16)(acc[v][r] * inv);
        *reinterpret_cast<f16x4*>(o + row * D + CW * li + 4 * v) = h;
      }
    }
    if (lane == 0) lse[row] = (M + log2f(W)) * 0.69314718055994530942f;
  }
}

}  // namespace attn
