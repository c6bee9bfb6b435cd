// Fused exact-attention forward kernel for gfx950 (CDNA4, wave64, MFMA).
//
// One workgroup of 4 waves owns BLOCK_M = 128 query rows of one (batch, head)
// and streams the head's keys in tiles of BLOCK_N = 64. Per tile it computes
// the scores with MFMA, folds them into each row's running carrier
// (max m, denominator d, unnormalised output o) kept in registers, and
// accumulates P.V with MFMA. Scores never leave registers. This is the
// streaming form of attention from "Learning FlashAttention the Hard Way,
// Part 2" (the FA-1 carrier update and its tensor-core Moves 1-4), laid out
// for CDNA4 rather than translated from the page's mma.sync listings.
//
// MFMA used: v_mfma_f32_16x16x32_f16 (A 16x32, B 32x16, C 16x16 fp32).
// Operand layout, lane l = 16*g + i (g = 0..3, i = 0..15):
//   A: row i,   contraction slots (g, e), e = 0..7   -- 8 halves per lane
//   B: column i, contraction slots (g, e)             -- 8 halves per lane
//   C: column i, rows 4*g + r, r = 0..3               -- 4 floats per lane
// A and B pair slot (g, e) with slot (g, e), so any fixed assignment of the
// contraction index to slots, used for both operands, gives the same sum.
//
// Transposed formulation. Both products are computed transposed so that one
// lane's accumulators always belong to one query:
//   S^T = K . Q^T    (A = K rows from LDS, B = Q^T fragments in registers)
//   O^T = V^T . P^T  (A = V^T rows from LDS, B = P^T straight from registers)
// For S^T the MFMA row i of key block kb (0..3) is bound to key
//   32*(kb/2) + 8*(i/4) + 4*(kb%2) + i%4
// so that lane group g ends up holding keys 32*kc + 8*g + 0..7 of each 32-key
// chunk kc in its S^T accumulators. Those 8 probabilities, rounded to fp16,
// are exactly the B operand slots (g, 0..7) of the P.V MFMA, and V^T is read
// with the same key order: the probabilities never pass through LDS.
//
// K/V transport: global -> registers (prefetch of tile t+1 issued before the
// math of tile t) -> LDS double buffer. K is stored as [key][d] and V as
// V^T [d][key]; every row is padded by 8 halves (16 bytes) so that the
// 16-byte reads of 16 consecutive rows fall on distinct bank groups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BLOCK_M = 128;  // query rows per workgroup
constexpr int BLOCK_N = 64;   // keys per tile
constexpr int WAVES = 4;
constexpr int THREADS = WAVES * 64;
constexpr int QSUB = 2;       // 16-row query sub-tiles per wave (32 rows per wave)
constexpr int PAD = 8;        // halves of padding per LDS row
constexpr float NEG_BIG = -1.0e30f;  // finite "minus infinity" for running maxima

template <int D>
struct Geometry {
  static constexpr int K_STRIDE = D + PAD;                 // halves per K row in LDS
  static constexpr int V_STRIDE = BLOCK_N + PAD;           // halves per V^T row in LDS
  static constexpr int K_HALVES = BLOCK_N * K_STRIDE;
  static constexpr int V_HALVES = D * V_STRIDE;
  static constexpr int STAGE_HALVES = K_HALVES + V_HALVES;
  static constexpr int LDS_BYTES = 2 * STAGE_HALVES * 2;   // two stages
  static constexpr int D_CHUNKS = D / 32;                  // contraction chunks of Q.K
  static constexpr int D_BLOCKS = D / 16;                  // 16-row blocks of O^T
  static constexpr int K_LOADS = BLOCK_N * D / 8 / THREADS;  // 16-byte K pieces per thread
  static constexpr int V_UNITS = BLOCK_N * D / 16 / THREADS; // 8-key x 2-d V pieces per thread
  static_assert(D % 64 == 0, "D must be a multiple of 64");
  static_assert(K_LOADS >= 1 && V_UNITS >= 1, "tile too small for the workgroup");
};

// Global fp16 load of 16 bytes, or zeros when the row is out of range.
__device__ __forceinline__ u32x4 load16(const _Float16* p, bool ok) {
  u32x4 z = {0u, 0u, 0u, 0u};
  return ok ? *reinterpret_cast<const u32x4*>(p) : z;
}

__device__ __forceinline__ uint32_t load4(const _Float16* p, bool ok) {
  return ok ? *reinterpret_cast<const uint32_t*>(p) : 0u;
}

__device__ __forceinline__ float wave_max_over_groups(float x) {
  // lanes i, i+16, i+32, i+48 hold the same query; reduce across them
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}

__device__ __forceinline__ float wave_sum_over_groups(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

// Registers holding one prefetched K/V tile on its way to LDS.
template <int D>
struct TileRegs {
  u32x4 k[Geometry<D>::K_LOADS];
  uint32_t v[Geometry<D>::V_UNITS][8];
};

// Issue the global loads of key tile `kt` (rows >= S read as zeros).
template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const _Float16* __restrict__ kh,
                                          const _Float16* __restrict__ vh, int kt, int S,
                                          int tid) {
  using G = Geometry<D>;
  const int key0 = kt * BLOCK_N;
#pragma unroll
  for (int i = 0; i < G::K_LOADS; ++i) {
    const int u = tid + THREADS * i;
    const int key = u / (D / 8);
    const int col = (u % (D / 8)) * 8;
    r.k[i] = load16(kh + (int64_t)(key0 + key) * D + col, key0 + key < S);
  }
#pragma unroll
  for (int i = 0; i < G::V_UNITS; ++i) {
    const int u = tid + THREADS * i;
    const int d0 = (u % (D / 2)) * 2;
    const int kg = u / (D / 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = key0 + 8 * kg + j;
      r.v[i][j] = load4(vh + (int64_t)key * D + d0, key < S);
    }
  }
}

// Write a prefetched tile into one LDS stage: K as [key][d], V as V^T [d][key].
template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, _Float16* stage, int tid) {
  using G = Geometry<D>;
  _Float16* ks = stage;
  _Float16* vs = stage + G::K_HALVES;
#pragma unroll
  for (int i = 0; i < G::K_LOADS; ++i) {
    const int u = tid + THREADS * i;
    const int key = u / (D / 8);
    const int col = (u % (D / 8)) * 8;
    *reinterpret_cast<u32x4*>(ks + key * G::K_STRIDE + col) = r.k[i];
  }
#pragma unroll
  for (int i = 0; i < G::V_UNITS; ++i) {
    const int u = tid + THREADS * i;
    const int d0 = (u % (D / 2)) * 2;
    const int kg = u / (D / 2);
    // r.v[i][j] holds (V[key j][d0], V[key j][d0+1]); gather the low halves
    // into row d0 and the high halves into row d0+1, keys in order.
    u32x4 lo, hi;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t a = r.v[i][2 * j], b = r.v[i][2 * j + 1];
      lo[j] = (a & 0xffffu) | (b << 16);
      hi[j] = (a >> 16) | (b & 0xffff0000u);
    }
    *reinterpret_cast<u32x4*>(vs + d0 * G::V_STRIDE + 8 * kg) = lo;
    *reinterpret_cast<u32x4*>(vs + (d0 + 1) * G::V_STRIDE + 8 * kg) = hi;
  }
}

// Key (within the tile) bound to MFMA row `row` of S^T key block `kb`.
__device__ __forceinline__ int st_key(int kb, int row) {
  return 32 * (kb >> 1) + 8 * (row >> 2) + 4 * (kb & 1) + (row & 3);
}

// One query sub-tile's running carrier, per lane (lane holds query i = lane%16).
template <int D>
struct Carrier {
  f32x4 o[Geometry<D>::D_BLOCKS];  // O^T rows 16*db + 4*g + r for this lane's query
  float m;                         // running max of scale*log2(e)*s (base-2 units)
  float d;                         // this lane's share of the denominator
};

// Fold one key tile (in LDS) into the wave's carriers.
// MASK: apply the causal / sequence-end mask element-wise.
template <int D, bool CAUSAL, bool MASK>
__device__ __forceinline__ void fold_tile(Carrier<D> (&cr)[QSUB], const f16x8 (&qf)[QSUB][Geometry<D>::D_CHUNKS],
                                          const _Float16* __restrict__ stage, float c,
                                          int key0, int qrow0, int S, int li, int g) {
  using G = Geometry<D>;
  const _Float16* ks = stage;
  const _Float16* vs = stage + G::K_HALVES;

  // S^T = K . Q^T for 4 key blocks of 16 keys, both query sub-tiles.
  f32x4 sc[QSUB][4];
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sc[qs][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const _Float16* krow = ks + st_key(kb, li) * G::K_STRIDE + 8 * g;
#pragma unroll
    for (int ch = 0; ch < G::D_CHUNKS; ++ch) {
      const f16x8 a = *reinterpret_cast<const f16x8*>(krow + 32 * ch);
#pragma unroll
      for (int qs = 0; qs < QSUB; ++qs)
        sc[qs][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qf[qs][ch], sc[qs][kb], 0, 0, 0);
    }
  }

  // Online softmax per query sub-tile.
  f16x8 pf[QSUB][2];
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs) {
    const int qrow = qrow0 + 16 * qs + li;
    if (MASK) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + 32 * (kb >> 1) + 8 * g + 4 * (kb & 1) + r;
          const bool hidden = key >= S || (CAUSAL && key > qrow);
          sc[qs][kb][r] = hidden ? -INFINITY : sc[qs][kb][r];
        }
    }
    float mx = NEG_BIG;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[qs][kb][r]);
    mx = wave_max_over_groups(mx);
    const float m_new = fmaxf(cr[qs].m, mx * c);
    const float alpha = __builtin_amdgcn_exp2f(cr[qs].m - m_new);
    float psum = 0.f;
    float p[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qs][kb][r], c, -m_new));
        if (MASK) e = (sc[qs][kb][r] == -INFINITY) ? 0.f : e;
        p[kb][r] = e;
        psum += e;
      }
    cr[qs].d = cr[qs].d * alpha + psum;
    cr[qs].m = m_new;
#pragma unroll
    for (int db = 0; db < G::D_BLOCKS; ++db) cr[qs].o[db] *= alpha;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      f16x8 h;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        h[r] = (_Float16)p[2 * kc][r];
        h[4 + r] = (_Float16)p[2 * kc + 1][r];
      }
      pf[qs][kc] = h;
    }
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

// grid.x = BH * n_qtiles; workgroup id -> (query tile, batch*head).
// Heaviest (last) query tiles are issued first, which balances causal work;
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

  const int bid = blockIdx.x;
  const int qt = n_qtiles - 1 - bid / BH;
  const int bh = bid % BH;
  const int64_t head = (int64_t)bh * S * D;
  const _Float16* qh = q + head;
  const _Float16* kh = k + head;
  const _Float16* vh = v + head;

  const int q0 = qt * BLOCK_M;
  const int qrow0 = q0 + 32 * wave;  // this wave's first query row

  // Q^T fragments, loaded once (sign-flipped when the scale is negative).
  f16x8 qf[QSUB][G::D_CHUNKS];
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs) {
    const int row = qrow0 + 16 * qs + li;
#pragma unroll
    for (int ch = 0; ch < G::D_CHUNKS; ++ch) {
      u32x4 w = load16(qh + (int64_t)row * D + 32 * ch + 8 * g, row < S);
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

  TileRegs<D> tr;
  load_tile<D>(tr, kh, vh, 0, S, tid);
  store_tile<D>(tr, smem, tid);
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const bool more = kt + 1 < n_kt;
    if (more) load_tile<D>(tr, kh, vh, kt + 1, S, tid);
    const _Float16* stage = smem + (kt & 1) * G::STAGE_HALVES;
    const int key0 = kt * BLOCK_N;
    // Tiles entirely after this wave's last query contribute nothing (causal).
    const bool live = !CAUSAL || key0 <= qrow0 + 31;
    // Element masks are needed on the sequence tail and on tiles that reach
    // past this wave's first query (causal diagonal).
    const bool needs_mask = (key0 + BLOCK_N > S) || (CAUSAL && key0 + BLOCK_N - 1 > qrow0);
    if (live) {
      if (needs_mask)
        fold_tile<D, CAUSAL, true>(cr, qf, stage, c, key0, qrow0, S, li, g);
      else
        fold_tile<D, CAUSAL, false>(cr, qf, stage, c, key0, qrow0, S, li, g);
    }
    if (more) store_tile<D>(tr, smem + ((kt + 1) & 1) * G::STAGE_HALVES, tid);
    __syncthreads();
  }

  // Epilogue: O = o / d rounded to fp16; LSE = (m + log2 d) * ln 2.
  float* lse_h = lse + (int64_t)bh * S;
  _Float16* oh = o + head;
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs) {
    const int row = qrow0 + 16 * qs + li;
    const float dsum = wave_sum_over_groups(cr[qs].d);
    const float inv = 1.0f / dsum;
    if (row < S) {
#pragma unroll
      for (int db = 0; db < G::D_BLOCKS; ++db) {
        f16x4 h;
#pragma unroll
        for (int r = 0; r < 4; ++r) h[r] = (_Float16)(cr[qs].o[db][r] * inv);
        *reinterpret_cast<f16x4*>(oh + (int64_t)row * D + 16 * db + 4 * g) = h;
      }
      if (g == 0) lse_h[row] = (cr[qs].m + log2f(dsum)) * 0.69314718055994530942f;
    }
  }
}

}  // namespace attn
