// kla_chunk.h -- the per-chunk triangular solve of the prep kernel.
//
// Paper "Kaczmarz Linear Attention" (arXiv 2605.08587), Proposition 3 (Eq. (7)) and
// Appendix B.2: for one chunk of 64 tokens with step sizes b, chunk-local log-decays G and
// keys K,
//   L = Diag(b) (A^- o K K^T),   A^-_ij = exp(G_i - G_j) for j < i   (strictly lower)
//   T = (I + L)^{-1} Diag(b)
// so that the chunk's U = T (V - Diag(exp G) K S0).  One wavefront computes T by 16 x 16
// blocks: X = (I + L)^{-1} is unit lower triangular; its four diagonal blocks come from
// substitution (lane group kg inverts block kg, one column per lane), its sub-diagonal
// blocks by distance from X_ij = -X_ii sum_{k=j}^{i-1} L_ik X_kj on the matrix cores, and
// T = X Diag(b).
//
// Fragment convention of kla_device.h; lane (r16, kg) = (lane % 16, lane / 16).
#pragma once

#include "kla_device.h"

namespace kla {

// Element (r, c) of a 16 x 16 fp32 block in LDS: rows of 64 bytes, the 16-byte units of
// rows 8..15 XOR-swizzled by 2 so that a half-wavefront reading (row r16, unit kg) hits 32
// distinct 16-byte positions.
__device__ __forceinline__ int bidx(int r, int c) {
  return r * 16 + ((((c >> 2) ^ (((r >> 3) & 1) << 1))) << 2) + (c & 3);
}
// LDS slot of the X block (i, j) that later products read: the diagonal blocks and the
// sub-diagonal blocks of rows 1 and 2.
__host__ __device__ constexpr int xslot(int i, int j) {
  return i == j ? i : (i == 1 ? 4 : (j == 0 ? 5 : 6));
}

// Entries (row, col .. col + 3) of a chunk's 64 x 64 output, col a multiple of 4, straight
// from registers: in the packed layout (tpb_off; entries of the blocks above the diagonal are
// not stored) or row-major.  A lane group (r16, kg) covering one 16 x 16 block writes its
// 256 contiguous packed elements, so a store instruction writes whole lines.
template <typename T>
__device__ __forceinline__ void out_put(T *dst, bool packed, int row, int col, float a, float b,
                                        float c, float d, bool split = false) {
  int off;
  if (packed) {
    const int I = row >> 4, J = col >> 4;
    if (J > I) return;
    off = (I * (I + 1) / 2 + J) * 256 + (row & 15) * 16 + (col & 15);
  } else {
    off = row * kChunk + col;
  }
  if constexpr (sizeof(T) == 2) {
    bf16x4 x4;
    x4[0] = from_f32<T>(a); x4[1] = from_f32<T>(b); x4[2] = from_f32<T>(c); x4[3] = from_f32<T>(d);
    *reinterpret_cast<bf16x4 *>(dst + off) = x4;
    if (split) {  // the rounding residuals, one packed tile further on
      bf16x4 l4;
      l4[0] = from_f32<T>(a - to_f32(x4[0]));
      l4[1] = from_f32<T>(b - to_f32(x4[1]));
      l4[2] = from_f32<T>(c - to_f32(x4[2]));
      l4[3] = from_f32<T>(d - to_f32(x4[3]));
      *reinterpret_cast<bf16x4 *>(dst + kTpbElems + off) = l4;
    }
  } else {
    *reinterpret_cast<f32x4 *>(dst + off) = f32x4{a, b, c, d};
  }
}

// Scratch of one wavefront's solve.
struct PrepSmem {
  alignas(16) float Ld[4][256];  // diagonal blocks of L, row-major
  alignas(16) float XT[7][256];  // X blocks transposed: XT(i, j)[c][r] = X[16 i + r][16 j + c]
  alignas(16) float G2[kChunk];  // G * log2(e)
  alignas(16) float beta[kChunk];
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Product of two 16 x 16 fp32 blocks in the layout of a 16x16x16 matrix-core step (lane
// (r16, kg) supplies A[r16][4 kg + e] in a and B[4 kg + e][r16] in b, e = 0..3), added to
// c.  SPLIT: each operand as a pair of bf16 values, hi = bf16(x) and lo = bf16(x - hi), and
// the product as hi*hi + hi*lo + lo*hi on v_mfma_f32_16x16x16_bf16 (relative error about
// 2^-16 of |A| |B|); otherwise four fp32 16x16x4 steps (exact products).
template <bool SPLIT>
__device__ __forceinline__ f32x4 blk_mma(const f32x4 &a, const f32x4 &b, f32x4 c) {
  if constexpr (SPLIT) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    bf16x4 ah, al, bh, bl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ah[e] = static_cast<__bf16>(a[e]);
      al[e] = static_cast<__bf16>(a[e] - static_cast<float>(ah[e]));
      bh[e] = static_cast<__bf16>(b[e]);
      bl[e] = static_cast<__bf16>(b[e] - static_cast<float>(bh[e]));
    }
    const s16x4 AH = __builtin_bit_cast(s16x4, ah), AL = __builtin_bit_cast(s16x4, al);
    const s16x4 BH = __builtin_bit_cast(s16x4, bh), BL = __builtin_bit_cast(s16x4, bl);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(AL, BH, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(AH, BL, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(AH, BH, c, 0, 0, 0);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
    return c;
  }
}

// The solve proper: X = (I + L)^{-1} and the callbacks put(row, col, x, bv) as for chunk_T,
// from L's sub-diagonal blocks in registers (Lr[i][j], j < i: lane (r16, kg) holds row
// 16 i + r16, columns 16 j + 4 kg + e) and its diagonal blocks in sm.Ld (strictly lower,
// bidx layout), with sm.beta written; both visible to every lane of the wavefront.
template <bool SPLIT, typename Sync, typename Put>
__device__ __forceinline__ void chunk_inverse(const f32x4 (&Lr)[4][3], PrepSmem &sm, Sync sync,
                                              Put put) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, kg = lane >> 4;
  // ---- diagonal blocks: lane group kg inverts I + L_kk by substitution, lane = column r16;
  //      rows of L_kk are read four values at a time (one address per lane group)
  {
    const float *Ld = sm.Ld[kg];
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float lr[16];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (4 * u < i) {
          const f32x4 v4 = *reinterpret_cast<const f32x4 *>(Ld + bidx(i, 4 * u));
          lr[4 * u] = v4[0]; lr[4 * u + 1] = v4[1]; lr[4 * u + 2] = v4[2]; lr[4 * u + 3] = v4[3];
        }
      }
      float a0 = (i == r16) ? 1.f : 0.f, a1 = 0.f;
#pragma unroll
      for (int j = 0; j < i; j += 2) {
        a0 = fmaf(-lr[j], x[j], a0);
        if (j + 1 < i) a1 = fmaf(-lr[j + 1], x[j + 1], a1);
      }
      x[i] = a0 + a1;
    }
    // XT(k, k)[r16][i] = X[16 k + i][16 k + r16]
    float *XTd = sm.XT[xslot(kg, kg)];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<f32x4 *>(XTd + bidx(r16, 4 * u)) =
          f32x4{x[4 * u], x[4 * u + 1], x[4 * u + 2], x[4 * u + 3]};
  }
  sync();

  // ---- T = X Diag(b): lane (r16, kg) stores columns 16 j + 4 kg + e of row 16 i + r16;
  //      diagonal blocks from LDS, the rest as they form
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float *XTi = sm.XT[xslot(i, i)];
    const f32x4 bv = *reinterpret_cast<const f32x4 *>(&sm.beta[16 * i + 4 * kg]);
    float xv[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) xv[s] = XTi[bidx(4 * kg + s, r16)];  // X_ii[r16][4 kg + s]
    put(16 * i + r16, 16 * i + 4 * kg, f32x4{xv[0], xv[1], xv[2], xv[3]}, bv);
  }

  // ---- sub-diagonal blocks, by distance; the blocks of one distance are independent
#pragma unroll
  for (int dist = 1; dist < 4; ++dist) {
#pragma unroll
    for (int i = dist; i < 4; ++i) {
      const int j = i - dist;
      // Y = sum_k L_ik X_kj: A = L_ik (registers), B = X_kj[4 kg + e][r16] from XT(k, j)
      f32x4 Y = zero4();
#pragma unroll
      for (int kb = j; kb < i; ++kb) {
        const f32x4 bx = *reinterpret_cast<const f32x4 *>(&sm.XT[xslot(kb, j)][bidx(r16, 4 * kg)]);
        Y = blk_mma<SPLIT>(Lr[i][kb], bx, Y);
      }
      // X_ij^T = -(Y^T X_ii^T): A = Y^T (Y's accumulator layout), B = X_ii[r16][4 kg + e]
      const float *XTi = sm.XT[xslot(i, i)];
      f32x4 xc;
#pragma unroll
      for (int e = 0; e < 4; ++e) xc[e] = XTi[bidx(4 * kg + e, r16)];
      const f32x4 Zt = blk_mma<SPLIT>(Y, xc, zero4());
      // lane (r16, kg) now holds X_ij[r16][4 kg + e] = -Zt[e]
      const f32x4 bv = *reinterpret_cast<const f32x4 *>(&sm.beta[16 * j + 4 * kg]);
      put(16 * i + r16, 16 * j + 4 * kg, f32x4{-Zt[0], -Zt[1], -Zt[2], -Zt[3]}, bv);
      if (i < 3) {  // read again by the next distances
        float *XTo = sm.XT[xslot(i, j)];
#pragma unroll
        for (int e = 0; e < 4; ++e) XTo[bidx(4 * kg + e, r16)] = -Zt[e];
      }
    }
    sync();
  }
}


// T = (I + L)^{-1} Diag(b) of one chunk from its key rows, by one wavefront.
//   kf[b][ks]  key rows 16 b + r16 as A fragments (elements 32 ks + 8 kg .. + 7)
//   gd[i]      the diagonal Gram tiles K_i K_i^T (fp32 accumulators)
//   bme[i]     b of row 16 i + r16;  G2me[i] its G * log2(e)
//   sm         the wavefront's scratch, with sm.G2 and sm.beta (per token) already written
//              and visible to every lane
//   sync()     makes this wavefront's LDS writes visible to its other lanes
//   put(row, col, x, bv)  gets X[row][col .. col + 3] = x with bv = b[col .. col + 3], so
//              that T[row][col + e] = x[e] bv[e]; called for the ten blocks on and below the
//              diagonal only (blocks above it are zero)
// SPLIT selects the pair-of-bf16 products for the sub-diagonal blocks (see blk_mma).
template <typename Tin, int NKS, bool SPLIT, typename Sync, typename Put>
__device__ __forceinline__ void chunk_T(const typename Frag<Tin>::type (&kf)[4][NKS],
                                        const f32x4 (&gd)[4], const float (&bme)[4],
                                        const float (&G2me)[4], PrepSmem &sm, Sync sync,
                                        Put put) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, kg = lane >> 4;
  // ---- L: diagonal blocks to LDS (row-major), sub-diagonal blocks kept in registers in the
  //      A-operand layout (row r16, columns 4 kg + e); each tile is formed as K_j K_i^T
  f32x4 Lr[4][3];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j <= i; ++j) {
      const int j0 = 16 * j + 4 * kg;
      f32x4 acc = gd[i];
      if (j < i) {
        acc = zero4();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) acc = mma(kf[j][ks], kf[i][ks], acc);
      }
      const f32x4 Gc = *reinterpret_cast<const f32x4 *>(&sm.G2[j0]);
      f32x4 lv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool below = (j < i) || (4 * kg + e < r16);  // column < row
        lv[e] = bme[i] * exp2_fast(below ? G2me[i] - Gc[e] : -INFINITY) * acc[e];
      }
      if (j < i) Lr[i][j] = lv;
      else *reinterpret_cast<f32x4 *>(&sm.Ld[i][bidx(r16, 4 * kg)]) = lv;
    }
  }
  sync();
  chunk_inverse<SPLIT>(Lr, sm, sync, put);
}

}  // namespace kla
