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
// Work decomposition. A workgroup of 8 waves owns BLOCK_M = 128 query rows of
// one (batch, head). Waves 0-3 take 32 rows each and fold the even key tiles
// (BLOCK_N = 64 keys); waves 4-7 take the same rows and fold the odd tiles.
// The two waves on one SIMD therefore work on independent data, so the MFMA
// work of one overlaps the softmax VALU work of the other (a single wave
// serialises its own MFMA and VALU instructions on gfx950). At the end each
// odd-tile wave hands its carrier to its partner through LDS and the two are
// merged.
//
// MFMA: v_mfma_f32_16x16x32_f16. Lane l = 16*g + i (g = 0..3, i = 0..15):
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
// rescale o and d, and redo the tile. Because o and d always share one m, the
// result is the same softmax; probabilities up to P_LIMIT keep fp16's
// relative precision. The row sum adds the fp16-rounded probabilities
// (v_dot2), so d normalises exactly the weights the P.V product used.
//
// LDS. Two stages, each holding an even and an odd tile: K as [key][d] with
// rows stored in MFMA-row order (row 16*kb + i holds key st_key(kb, i)) and
// V as V^T [d][key]. Rows are padded by 8 halves, so the 16-byte reads of 16
// consecutive rows hit 16 distinct bank groups of the 64-bank LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BLOCK_M = 128;          // query rows per workgroup
constexpr int BLOCK_N = 64;           // keys per tile
constexpr int QGROUPS = 4;            // waves per key-tile parity (32 rows each)
constexpr int WAVES = 2 * QGROUPS;    // even-tile and odd-tile waves
constexpr int THREADS = WAVES * 64;
constexpr int QSUB = 2;               // 16-row query sub-tiles per wave
constexpr float NEG_BIG = -1.0e30f;   // finite stand-in for -infinity
constexpr float P_LIMIT = 16384.0f;   // lazy-max bound on a lane's fp16 tile sum
constexpr uint32_t BUF_FLAGS = 0x00020000u;  // raw buffer, 32-bit data format

template <int D>
struct Geometry {
  static constexpr int K_HALVES = BLOCK_N * D;             // K rows unpadded, swizzled
  static constexpr int V_HALVES = BLOCK_N * D;             // V rows unpadded, swizzled
  // two-slot rings of tile pairs for K and for V^T
  static constexpr int LDS_BYTES = (4 * K_HALVES + 4 * V_HALVES) * 2;
  static constexpr int D_CHUNKS = D / 32;                  // contraction chunks of Q.K
  static constexpr int D_BLOCKS = D / 16;                  // 16-row blocks of O^T
  // per tile pair, K and V each in 16-byte pieces
  static constexpr int PIECES = 2 * BLOCK_N * (D / 8);
  static constexpr int LOADS = PIECES / THREADS;
  static_assert(D % 64 == 0, "D must be a multiple of 64");
  static_assert(LOADS * THREADS == PIECES, "tiling");
  // carrier hand-off area (after the key loop): per odd wave, per lane
  static constexpr int CARRIER_FLOATS = QSUB * (2 + 4 * D_BLOCKS);
  static_assert(QGROUPS * 64 * CARRIER_FLOATS * 4 <= LDS_BYTES, "hand-off fits in LDS");
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

// Direct global->LDS copy of one tile pair. A buffer load with the LDS flag
// writes lane l's 16 bytes at M0 + 16*l, so each wave instruction fills 1 KB
// of LDS in slot order; each lane therefore fetches the global piece that
// belongs in its slot. Per-lane byte offsets (relative to the first key of the
// pair) are precomputed for K and for V.
template <int D>
struct CopyPlan {
  uint32_t k_off[Geometry<D>::LOADS];
  uint32_t v_off[Geometry<D>::LOADS];
};

template <int D>
__device__ __forceinline__ int copy_unit(int wave, int i) {
  return i * WAVES + wave;  // 1 KB unit of the pair filled by instruction i of a wave
}

template <int D>
__device__ __forceinline__ void make_copy_plan(CopyPlan<D>& cp, int wave, int lane) {
  constexpr int CHUNKS = D / 8;                     // 16-byte chunks per row
  constexpr int TILE_SLOTS = BLOCK_N * CHUNKS;
#pragma unroll
  for (int i = 0; i < Geometry<D>::LOADS; ++i) {
    const int slot = copy_unit<D>(wave, i) * 64 + lane;
    const int t = slot / TILE_SLOTS;                // tile of the pair
    const int w = slot % TILE_SLOTS;
    const int row = w / CHUNKS;
    const int pc = w % CHUNKS;                       // physical chunk in the row
    const int kkey = st_key(row >> 4, row & 15);
    cp.k_off[i] = (uint32_t)(((t * BLOCK_N + kkey) * D + 8 * (pc ^ k_swizzle<D>(row))) * 2);
    cp.v_off[i] = (uint32_t)(((t * BLOCK_N + row) * D + 8 * (pc ^ v_swizzle<D>(row))) * 2);
  }
}

// Buffer descriptor over keys [key0, S) of one head's K or V: the hardware
// range check returns zeros for keys >= S.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t keys_from(const _Float16* base, int key0, int S) {
  const uint32_t bytes = key0 < S ? (uint32_t)(S - key0) * D * 2 : 0u;
  return make_rsrc(base + (int64_t)key0 * D, bytes);
}

// Issue the direct copy of the tile pair starting at key0 into `slot` (the
// pair's LDS area: tile 0 then tile 1). Completion is awaited with vmcnt.
template <int D>
__device__ __forceinline__ void copy_pair(const uint32_t* off, const _Float16* base, int key0,
                                          int S, _Float16* slot, int wave) {
  const __amdgpu_buffer_rsrc_t rs = keys_from<D>(base, key0, S);
#pragma unroll
  for (int i = 0; i < Geometry<D>::LOADS; ++i) {
    _Float16* dst = slot + copy_unit<D>(wave, i) * 64 * 8;   // 64 slots of 8 halves
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)dst, 16, off[i], 0, 0, 0);
  }
}

__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// LDS transposing read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane n supplies the address of 4 consecutive halves X[n][0..3]; lane n
// receives X[4e + n/4][n % 4] for e = 0..3.
__device__ __forceinline__ f16x4 lds_read_tr(const _Float16* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (s16x4 __attribute__((address_space(3)))*)(p));
  return __builtin_bit_cast(f16x4, r);
}

// Per-lane carrier of one query sub-tile (the lane's query is i = lane % 16).
template <int D>
struct Carrier {
  f32x4 o[Geometry<D>::D_BLOCKS];  // O^T rows 16*db + 4*g + r of this query
  float m;                         // running max of t = s*c (base-2 units)
  float d;                         // this lane's share of the denominator
};

// S^T = K . Q^T of one tile: 4 key blocks x 2 query sub-tiles (16 MFMAs).
template <int D>
__device__ __forceinline__ void qk_tile(f32x4 (&sc)[QSUB][4],
                                        const f16x8 (&qf)[QSUB][Geometry<D>::D_CHUNKS],
                                        const _Float16* __restrict__ ktile, int li, int g) {
  using G = Geometry<D>;
  const int sw = k_swizzle<D>(li);  // the swizzle bits of row 16*kb + li do not depend on kb
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    f16x8 a[G::D_CHUNKS];
#pragma unroll
    for (int ch = 0; ch < G::D_CHUNKS; ++ch)
      a[ch] = *reinterpret_cast<const f16x8*>(ktile + (16 * kb + li) * D + 8 * ((4 * ch + g) ^ sw));
#pragma unroll
    for (int qs = 0; qs < QSUB; ++qs) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ch = 0; ch < G::D_CHUNKS; ++ch)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[ch], qf[qs][ch], acc, 0, 0, 0);
      sc[qs][kb] = acc;
    }
  }
}

// O^T += V^T . P^T of one tile (16 MFMAs at D = 64). The A operand of d block
// db and key chunk kc needs, in lane (i, g), V[32kc + 8g + e][16db + i] for
// e = 0..7: two transposing reads, each over 4 key rows x 16 d, where source
// lane n of group g points at row 32kc + 8g + 4h + n/4, halves 16db + 4(n%4).
template <int D>
__device__ __forceinline__ void pv_tile(Carrier<D> (&cr)[QSUB], const f16x8 (&pf)[QSUB][2],
                                        const _Float16* __restrict__ vtile, int li, int g) {
  using G = Geometry<D>;
  const int row = 8 * g + (li >> 2);
  const int sw = v_swizzle<D>(row);  // row bits that matter do not depend on kc or h
  const _Float16* vlane = vtile + row * D + 4 * (li & 1);
  const int x = (li & 3) >> 1;
#pragma unroll
  for (int db = 0; db < G::D_BLOCKS; ++db) {
    const _Float16* vp = vlane + 8 * ((2 * db + x) ^ sw);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const f16x4 lo = lds_read_tr(vp + (32 * kc) * D);
      const f16x4 hi = lds_read_tr(vp + (32 * kc + 4) * D);
      const f16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int qs = 0; qs < QSUB; ++qs)
        cr[qs].o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pf[qs][kc], cr[qs].o[db], 0, 0, 0);
    }
  }
}

// exp2(t - m) of a 4-score accumulator, hidden keys forced to 0 when MASK.
template <bool MASK>
__device__ __forceinline__ f32x4 exp_block(f32x4 s, float c, float m, uint32_t hid) {
  f32x4 p;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -m));
    if (MASK) e = ((hid >> r) & 1u) ? 0.0f : e;
    p[r] = e;
  }
  return p;
}

// Online softmax of one tile's scores: probabilities (fp16, P^T operand
// layout) into pf, denominators and, when the max moves, outputs rescaled.
template <int D, bool CAUSAL, bool MASK>
__device__ __forceinline__ void softmax_tile(Carrier<D> (&cr)[QSUB], const f32x4 (&sc)[QSUB][4],
                                             f16x8 (&pf)[QSUB][2], float c, int key0, int qrow0,
                                             int S, int li, int g) {
  using G = Geometry<D>;
  // hidden-key bits per sub-tile and key block (bit r: accumulator element r)
  uint32_t hid[QSUB][4];
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      hid[qs][kb] = 0u;
      if (MASK) {
        const int qrow = qrow0 + 16 * qs + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + 32 * (kb >> 1) + 8 * g + 4 * (kb & 1) + r;
          const bool h = key >= S || (CAUSAL && key > qrow);
          hid[qs][kb] |= (h ? 1u : 0u) << r;
        }
      }
    }
  float psum[QSUB];
  auto expo = [&](int qs) {
    const float m = cr[qs].m;
    f32x4 p[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) p[kb] = exp_block<MASK>(sc[qs][kb], c, m, hid[qs][kb]);
    float acc[2] = {0.0f, 0.0f};
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      f16x8 h;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        h[r] = (_Float16)p[2 * kc][r];
        h[4 + r] = (_Float16)p[2 * kc + 1][r];
      }
      pf[qs][kc] = h;
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        acc[(e >> 1) & 1] = __builtin_amdgcn_fdot2(
            f16x2{h[e], h[e + 1]}, f16x2{(_Float16)1.0f, (_Float16)1.0f}, acc[(e >> 1) & 1], false);
    }
    psum[qs] = acc[0] + acc[1];
  };
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs) expo(qs);
  // Lazy max: refresh m only when this tile's probabilities could overflow.
  bool over = false;
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs) over = over || !(psum[qs] <= P_LIMIT);
  if (__builtin_amdgcn_ballot_w64(over) != 0) {
#pragma unroll
    for (int qs = 0; qs < QSUB; ++qs) {
      float tmax = NEG_BIG;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
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
  for (int qs = 0; qs < QSUB; ++qs) cr[qs].d += psum[qs];
}

template <int D, bool CAUSAL>
__device__ __forceinline__ void softmax_any(Carrier<D> (&cr)[QSUB], const f32x4 (&sc)[QSUB][4],
                                            f16x8 (&pf)[QSUB][2], float c, int key0, int qrow0,
                                            int S, int li, int g) {
  // Element masks are needed on the sequence tail and on tiles reaching past
  // the wave's first query (causal diagonal).
  const bool needs_mask = (key0 + BLOCK_N > S) || (CAUSAL && key0 + BLOCK_N - 1 > qrow0);
  if (needs_mask)
    softmax_tile<D, CAUSAL, true>(cr, sc, pf, c, key0, qrow0, S, li, g);
  else
    softmax_tile<D, CAUSAL, false>(cr, sc, pf, c, key0, qrow0, S, li, g);
}

// grid.x = BH * n_qtiles; workgroup id -> (query tile, batch*head). The
// heaviest (last) query tiles are issued first, which balances causal work;
// consecutive workgroups take consecutive heads.
//
// Schedule. Key tiles come in pairs (2j, 2j+1); barrier interval j is one
// trip of the main loop. Even waves own tile 2j and odd waves tile 2j+1:
//   even, interval j: P.V of tile 2j-2, S = Q.K^T of tile 2j | softmax of 2j
//   odd,  interval j: softmax of 2j-1 | P.V of 2j-1, S = Q.K^T of 2j+1
// so the two waves of a SIMD alternate between MFMA-heavy and VALU-heavy
// halves in opposite order. K of pair j must be in LDS in interval j and V of
// pair j in interval j+1: interval j copies K of pair j+1 and V of pair j
// (global loads at its start, LDS stores at its end) into two-slot rings.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(THREADS) void attn_fwd_kernel(
    const _Float16* __restrict__ q, const _Float16* __restrict__ k,
    const _Float16* __restrict__ v, _Float16* __restrict__ o, float* __restrict__ lse,
    int BH, int S, int n_qtiles, float c, uint32_t qsign) {
  using G = Geometry<D>;
  __shared__ __attribute__((aligned(16))) _Float16 smem[4 * G::K_HALVES + 4 * G::V_HALVES];
  _Float16* kring = smem;                    // [slot][tile] K tiles
  _Float16* vring = smem + 4 * G::K_HALVES;  // [slot][tile] V^T tiles

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int li = lane & 15;
  const int g = lane >> 4;
  const int qgrp = wave % QGROUPS;
  const int parity = wave / QGROUPS;

  const int bid = blockIdx.x;
  const int qt = n_qtiles - 1 - bid / BH;
  const int bh = bid % BH;
  const int64_t head = (int64_t)bh * S * D;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(q + head, (uint32_t)S * D * 2);
  const _Float16* kh = k + head;
  const _Float16* vh = v + head;

  const int q0 = qt * BLOCK_M;
  const int qrow0 = q0 + 32 * qgrp;  // this wave's first query row

  // Q^T fragments, loaded once (sign-flipped when the scale is negative).
  f16x8 qf[QSUB][G::D_CHUNKS];
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs) {
    const int row = qrow0 + 16 * qs + li;
#pragma unroll
    for (int ch = 0; ch < G::D_CHUNKS; ++ch) {
      u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
          qrs, (uint32_t)((row * D + 32 * ch + 8 * g) * 2), 0, 0);
      w ^= qsign;
      qf[qs][ch] = __builtin_bit_cast(f16x8, w);
    }
  }

  Carrier<D> cr[QSUB];
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs) {
    cr[qs].m = NEG_BIG;
    cr[qs].d = 0.f;
#pragma unroll
    for (int db = 0; db < G::D_BLOCKS; ++db) cr[qs].o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Carried across the barrier: odd waves keep a tile's scores between Q.K^T
  // and softmax; even waves keep its fp16 probabilities between softmax and
  // P.V, packed into the first two blocks of the same registers.
  f32x4 sc[QSUB][4];
  f16x8 pf[QSUB][2];

  const int kend = CAUSAL ? min(S, q0 + BLOCK_M) : S;
  const int n_kt = (kend + BLOCK_N - 1) / BLOCK_N;
  const int n_pairs = (n_kt + 1) / 2;
  // tile t contributes to this wave's rows
  auto live = [&](int t) { return t < n_kt && (!CAUSAL || t * BLOCK_N <= qrow0 + 31); };

  CopyPlan<D> cp;
  make_copy_plan<D>(cp, wave, lane);
  copy_pair<D>(cp.k_off, kh, 0, S, kring, wave);
  wait_copies();
  __syncthreads();

  for (int j = 0; j <= n_pairs; ++j) {
    const bool k_next = j + 1 < n_pairs;
    const bool v_now = j < n_pairs;
    const _Float16* kslot = kring + (j & 1) * 2 * G::K_HALVES + parity * G::K_HALVES;
    const _Float16* vslot = vring + ((j + 1) & 1) * 2 * G::V_HALVES + parity * G::V_HALVES;
    const int tp = 2 * (j - 1) + parity;  // tile whose P.V is due
    const int tc = 2 * j + parity;        // tile whose scores are due
    const bool do_pv = j >= 1 && live(tp);
    const bool do_qk = j < n_pairs && live(tc);
    // MFMA half: P.V of the previous tile, then Q.K^T of this one.
    if (do_pv) {
#pragma unroll
      for (int qs = 0; qs < QSUB; ++qs)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) pf[qs][kc] = __builtin_bit_cast(f16x8, sc[qs][kc]);
      pv_tile<D>(cr, pf, vslot, li, g);
    }
    if (do_qk) qk_tile<D>(sc, qf, kslot, li, g);
    __builtin_amdgcn_sched_barrier(0);
    // Copies for the next interval, issued mid-interval so that the eight
    // waves do not all queue them at once.
    if (k_next) copy_pair<D>(cp.k_off, kh, (j + 1) * 2 * BLOCK_N, S,
                             kring + ((j + 1) & 1) * 2 * G::K_HALVES, wave);
    if (v_now) copy_pair<D>(cp.v_off, vh, j * 2 * BLOCK_N, S, vring + (j & 1) * 2 * G::V_HALVES,
                            wave);
    __builtin_amdgcn_sched_barrier(0);
    // VALU half: softmax of this tile; its probabilities wait in the score
    // registers for the next interval's P.V.
    if (do_qk) {
      softmax_any<D, CAUSAL>(cr, sc, pf, c, tc * BLOCK_N, qrow0, S, li, g);
#pragma unroll
      for (int qs = 0; qs < QSUB; ++qs)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) sc[qs][kc] = __builtin_bit_cast(f32x4, pf[qs][kc]);
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_copies();
    __syncthreads();
  }

  // Odd-tile waves hand their carriers to their even-tile partners.
  float* xfer = reinterpret_cast<float*>(smem) + qgrp * 64 * G::CARRIER_FLOATS + lane;
  if (parity == 1) {
#pragma unroll
    for (int qs = 0; qs < QSUB; ++qs) {
      float* x = xfer + qs * (2 + 4 * G::D_BLOCKS) * 64;
      x[0] = cr[qs].m;
      x[64] = cr[qs].d;
#pragma unroll
      for (int db = 0; db < G::D_BLOCKS; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) x[(2 + 4 * db + r) * 64] = cr[qs].o[db][r];
    }
  }
  __syncthreads();
  if (parity == 1) return;

  float* lse_h = lse + (int64_t)bh * S;
  _Float16* oh = o + head;
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs) {
    const float* x = xfer + qs * (2 + 4 * G::D_BLOCKS) * 64;
    const float m2 = x[0];
    const float m = __builtin_fmaxf(cr[qs].m, m2);
    const float w1 = __builtin_amdgcn_exp2f(cr[qs].m - m);
    const float w2 = __builtin_amdgcn_exp2f(m2 - m);
    const float dsum = group_sum(cr[qs].d * w1 + x[64] * w2);
    const float inv = 1.0f / dsum;
    const int row = qrow0 + 16 * qs + li;
    if (row < S) {
#pragma unroll
      for (int db = 0; db < G::D_BLOCKS; ++db) {
        f16x4 h;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          h[r] = (_Float16)((cr[qs].o[db][r] * w1 + x[(2 + 4 * db + r) * 64] * w2) * inv);
        *reinterpret_cast<f16x4*>(oh + (int64_t)row * D + 16 * db + 4 * g) = h;
      }
      if (g == 0) lse_h[row] = (m + log2f(dsum)) * 0.69314718055994530942f;
    }
  }
}

}  // namespace attn
