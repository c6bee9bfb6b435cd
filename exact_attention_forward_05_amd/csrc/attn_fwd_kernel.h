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
constexpr int PAD = 8;                // halves of padding per LDS row
constexpr float NEG_BIG = -1.0e30f;   // finite stand-in for -infinity
constexpr float P_LIMIT = 16384.0f;   // lazy-max bound on a lane's fp16 tile sum
constexpr uint32_t BUF_FLAGS = 0x00020000u;  // raw buffer, 32-bit data format

template <int D>
struct Geometry {
  static constexpr int K_STRIDE = D + PAD;                 // halves per K row
  static constexpr int V_STRIDE = BLOCK_N + PAD;           // halves per V^T row
  static constexpr int K_HALVES = BLOCK_N * K_STRIDE;
  static constexpr int V_HALVES = D * V_STRIDE;
  static constexpr int TILE_HALVES = K_HALVES + V_HALVES;  // one tile (K + V^T)
  static constexpr int STAGE_HALVES = 2 * TILE_HALVES;     // even + odd tile
  static constexpr int LDS_BYTES = 2 * STAGE_HALVES * 2;   // two stages
  static constexpr int D_CHUNKS = D / 32;                  // contraction chunks of Q.K
  static constexpr int D_BLOCKS = D / 16;                  // 16-row blocks of O^T
  // per tile pair: K in 16-byte pieces, V in (8 keys x 2 d) units
  static constexpr int K_PIECES = 2 * BLOCK_N * (D / 8);
  static constexpr int V_UNITS = 2 * 8 * (D / 2);
  static constexpr int K_LOADS = K_PIECES / THREADS;
  static constexpr int V_LOADS = V_UNITS / THREADS;
  static_assert(D % 64 == 0, "D must be a multiple of 64");
  static_assert(K_LOADS * THREADS == K_PIECES && V_LOADS * THREADS == V_UNITS, "tiling");
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

// Registers holding one prefetched tile pair on its way to LDS.
template <int D>
struct PairRegs {
  u32x4 k[Geometry<D>::K_LOADS];
  uint32_t v[Geometry<D>::V_LOADS][8];
};

// Thread-constant parts of the K/V copy: byte offsets into a head's K/V for
// key tile 0, and LDS destinations within a stage.
template <int D>
struct CopyPlan {
  uint32_t k_goff[Geometry<D>::K_LOADS];
  int k_lds[Geometry<D>::K_LOADS];
  uint32_t v_goff[Geometry<D>::V_LOADS];
  int v_lds[Geometry<D>::V_LOADS];
};

template <int D>
__device__ __forceinline__ void make_copy_plan(CopyPlan<D>& cp, int tid) {
  using G = Geometry<D>;
#pragma unroll
  for (int i = 0; i < G::K_LOADS; ++i) {
    const int u = tid + THREADS * i;
    const int t = u / (BLOCK_N * (D / 8));          // tile of the pair
    const int w = u % (BLOCK_N * (D / 8));
    const int key = w / (D / 8);
    const int col = (w % (D / 8)) * 8;
    cp.k_goff[i] = (uint32_t)(((t * BLOCK_N + key) * D + col) * 2);
    cp.k_lds[i] = t * G::TILE_HALVES + k_row_of(key) * G::K_STRIDE + col;
  }
#pragma unroll
  for (int i = 0; i < G::V_LOADS; ++i) {
    const int u = tid + THREADS * i;
    const int t = u / (8 * (D / 2));
    const int w = u % (8 * (D / 2));
    const int kg = w % 8;                            // keys 8*kg .. 8*kg+7
    const int j = w / 8;
    // d pairs of 16 consecutive lanes land on distinct LDS bank groups
    const int dp = (j & ~7) + ((j & 7) >> 1) + 4 * (j & 1);
    cp.v_goff[i] = (uint32_t)(((t * BLOCK_N + 8 * kg) * D + 2 * dp) * 2);
    cp.v_lds[i] = t * G::TILE_HALVES + G::K_HALVES + (2 * dp) * G::V_STRIDE + 8 * kg;
  }
}

// Global loads of the tile pair starting at key `key0` of one head. The
// buffer descriptors start at that key and end at key S, so the hardware
// range check returns zeros for keys >= S.
template <int D>
__device__ __forceinline__ void load_pair(PairRegs<D>& r, const CopyPlan<D>& cp,
                                          const _Float16* kh, const _Float16* vh, int key0,
                                          int S) {
  using G = Geometry<D>;
  const int64_t off = (int64_t)key0 * D;
  const uint32_t bytes = key0 < S ? (uint32_t)(S - key0) * D * 2 : 0u;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kh + off, bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vh + off, bytes);
#pragma unroll
  for (int i = 0; i < G::K_LOADS; ++i)
    r.k[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, cp.k_goff[i], 0, 0);
#pragma unroll
  for (int i = 0; i < G::V_LOADS; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      r.v[i][j] = __builtin_amdgcn_raw_buffer_load_b32(vrs, cp.v_goff[i] + j * D * 2, 0, 0);
}

template <int D>
__device__ __forceinline__ void store_pair(const PairRegs<D>& r, const CopyPlan<D>& cp,
                                           _Float16* stage) {
  using G = Geometry<D>;
#pragma unroll
  for (int i = 0; i < G::K_LOADS; ++i)
    *reinterpret_cast<u32x4*>(stage + cp.k_lds[i]) = r.k[i];
#pragma unroll
  for (int i = 0; i < G::V_LOADS; ++i) {
    // r.v[i][j] = (V[key j][d0], V[key j][d0+1]); row d0 of V^T takes the low
    // halves of keys 0..7, row d0+1 the high halves.
    u32x4 lo, hi;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t a = r.v[i][2 * j], b = r.v[i][2 * j + 1];
      lo[j] = (a & 0xffffu) | (b << 16);
      hi[j] = (a >> 16) | (b & 0xffff0000u);
    }
    *reinterpret_cast<u32x4*>(stage + cp.v_lds[i]) = lo;
    *reinterpret_cast<u32x4*>(stage + cp.v_lds[i] + G::V_STRIDE) = hi;
  }
}

// Per-lane carrier of one query sub-tile (the lane's query is i = lane % 16).
template <int D>
struct Carrier {
  f32x4 o[Geometry<D>::D_BLOCKS];  // O^T rows 16*db + 4*g + r of this query
  float m;                         // running max of t = s*c (base-2 units)
  float d;                         // this lane's share of the denominator
};

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

// Fold one key tile (in LDS) into the wave's two carriers.
template <int D, bool CAUSAL, bool MASK>
__device__ __forceinline__ void fold_tile(Carrier<D> (&cr)[QSUB],
                                          const f16x8 (&qf)[QSUB][Geometry<D>::D_CHUNKS],
                                          const _Float16* __restrict__ tile, float c, int key0,
                                          int qrow0, int S, int li, int g) {
  using G = Geometry<D>;
  const _Float16* ks = tile;
  const _Float16* vs = tile + G::K_HALVES;

  // S^T = K . Q^T: 4 key blocks x 2 query sub-tiles.
  f32x4 sc[QSUB][4];
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sc[qs][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const _Float16* krow = ks + (16 * kb + li) * G::K_STRIDE + 8 * g;
#pragma unroll
    for (int ch = 0; ch < G::D_CHUNKS; ++ch) {
      const f16x8 a = *reinterpret_cast<const f16x8*>(krow + 32 * ch);
#pragma unroll
      for (int qs = 0; qs < QSUB; ++qs)
        sc[qs][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qf[qs][ch], sc[qs][kb], 0, 0, 0);
    }
  }

  f16x8 pf[QSUB][2];
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs) {
    // hidden-key bits per key block (bit r: accumulator element r)
    uint32_t hid[4] = {0u, 0u, 0u, 0u};
    if (MASK) {
      const int qrow = qrow0 + 16 * qs + li;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + 32 * (kb >> 1) + 8 * g + 4 * (kb & 1) + r;
          const bool h = key >= S || (CAUSAL && key > qrow);
          hid[kb] |= (h ? 1u : 0u) << r;
        }
    }
    float m = cr[qs].m;
    f32x4 p[4];
    float psum;
    auto expo = [&]() {
      psum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) p[kb] = exp_block<MASK>(sc[qs][kb], c, m, hid[kb]);
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
          psum = __builtin_amdgcn_fdot2(f16x2{h[e], h[e + 1]}, f16x2{(_Float16)1.0f, (_Float16)1.0f},
                                        psum, false);
      }
    };
    expo();
    // Lazy max: refresh m only when this tile's probabilities could overflow.
    if (__builtin_amdgcn_ballot_w64(!(psum <= P_LIMIT)) != 0) {
      float tmax = NEG_BIG;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        f32x4 s = sc[qs][kb];
        if (MASK) {
#pragma unroll
          for (int r = 0; r < 4; ++r) s[r] = ((hid[kb] >> r) & 1u) ? NEG_BIG : s[r];
        }
        tmax = __builtin_fmaxf(tmax, max4(s));
      }
      tmax = group_max(tmax);
      const float m_new = __builtin_fmaxf(m, tmax * c);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      cr[qs].d *= alpha;
#pragma unroll
      for (int db = 0; db < G::D_BLOCKS; ++db) cr[qs].o[db] *= alpha;
      m = m_new;
      cr[qs].m = m_new;
      expo();
    }
    cr[qs].d += psum;
  }

  // O^T += V^T . P^T
#pragma unroll
  for (int db = 0; db < G::D_BLOCKS; ++db) {
    const _Float16* vrow = vs + (16 * db + li) * G::V_STRIDE + 8 * g;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const f16x8 a = *reinterpret_cast<const f16x8*>(vrow + 32 * kc);
#pragma unroll
      for (int qs = 0; qs < QSUB; ++qs)
        cr[qs].o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pf[qs][kc], cr[qs].o[db], 0, 0, 0);
    }
  }
}

// grid.x = BH * n_qtiles; workgroup id -> (query tile, batch*head). The
// heaviest (last) query tiles are issued first, which balances causal work;
// consecutive workgroups take consecutive heads.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(THREADS) void attn_fwd_kernel(
    const _Float16* __restrict__ q, const _Float16* __restrict__ k,
    const _Float16* __restrict__ v, _Float16* __restrict__ o, float* __restrict__ lse,
    int BH, int S, int n_qtiles, float c, uint32_t qsign) {
  using G = Geometry<D>;
  __shared__ __attribute__((aligned(16))) _Float16 smem[2 * G::STAGE_HALVES];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int li = lane & 15;
  const int g = lane >> 4;
  const int qgrp = wave % QGROUPS;
  const int parity = wave / QGROUPS;

  const int bid = blockIdx.x;
  const int qt = n_qtiles - 1 - bid / BH;
  const int bh = bid % BH;
  const int64_t head = (int64_t)bh * S * D;
  const uint32_t head_bytes = (uint32_t)S * D * 2;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(q + head, head_bytes);
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

  const int kend = CAUSAL ? min(S, q0 + BLOCK_M) : S;
  const int n_kt = (kend + BLOCK_N - 1) / BLOCK_N;
  const int n_pairs = (n_kt + 1) / 2;

  CopyPlan<D> cp;
  make_copy_plan<D>(cp, tid);
  PairRegs<D> pr;
  load_pair<D>(pr, cp, kh, vh, 0, S);
  store_pair<D>(pr, cp, smem);
  __syncthreads();

  for (int it = 0; it < n_pairs; ++it) {
    const bool more = it + 1 < n_pairs;
    if (more) load_pair<D>(pr, cp, kh, vh, (it + 1) * 2 * BLOCK_N, S);
    const int kt = 2 * it + parity;
    const int key0 = kt * BLOCK_N;
    const _Float16* tile = smem + (it & 1) * G::STAGE_HALVES + parity * G::TILE_HALVES;
    // Tiles past the key range, or entirely after this wave's last query
    // (causal), contribute nothing.
    const bool live = kt < n_kt && (!CAUSAL || key0 <= qrow0 + 31);
    const bool needs_mask = (key0 + BLOCK_N > S) || (CAUSAL && key0 + BLOCK_N - 1 > qrow0);
    if (live) {
      if (needs_mask)
        fold_tile<D, CAUSAL, true>(cr, qf, tile, c, key0, qrow0, S, li, g);
      else
        fold_tile<D, CAUSAL, false>(cr, qf, tile, c, key0, qrow0, S, li, g);
    }
    if (more) store_pair<D>(pr, cp, smem + ((it + 1) & 1) * G::STAGE_HALVES);
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
