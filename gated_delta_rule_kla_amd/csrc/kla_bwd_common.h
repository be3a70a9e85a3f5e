// kla_bwd_common.h -- tile helpers shared by the backward kernels (the adjoint scans and
// the per-chunk gradient kernels of the scalar and the diagonal gate).
#pragma once
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {

namespace {

constexpr int kAdjBV = 32;          // state columns per adjoint-scan workgroup
constexpr int kAdjThreads = 512;    // eight wavefronts, two to a SIMD
constexpr int kGradThreads = 512;   // eight wavefronts
constexpr int LDB = kAdjBV + 4;     // row stride (elements) of a 32-column block in LDS
constexpr int LDC = kChunk + 4;     // row stride of a 64 x 64 fp32 tile in LDS

// acc[i][j] += sum_{k < KD} A(i, k) B(k, j) over one 16 x 16 tile: lane (r, kq) = (l % 16,
// l / 16) supplies A(r, k0 + kq) and B(k0 + kq, r) and holds D[4 kq + e][r] of the result.
template <int KD, typename FA, typename FB>
__device__ __forceinline__ f32x4 mm_tile(f32x4 acc, int lane, FA fa, FB fb) {
  const int r = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int k0 = 0; k0 < KD; k0 += 4)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa(r, k0 + kq), fb(k0 + kq, r), acc, 0, 0, 0);
  return acc;
}

// The same tile product in the operand precision of the inputs: fp32 inputs keep the fp32
// MFMA; bf16 inputs round both operands to bf16 and contract 32 at a time on
// v_mfma_f32_16x16x32_bf16 (lane (r, kq) supplies A(r, k0 + 8 kq + s) and B(k0 + 8 kq + s, r),
// s = 0..7), accumulating in fp32.  KD is a multiple of 32.
template <typename Tin, int KD, typename FA, typename FB>
__device__ __forceinline__ f32x4 mmt(f32x4 acc, int lane, FA fa, FB fb) {
  if constexpr (sizeof(Tin) == 2) {
    const int r = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < KD; k0 += 32) {
      bf16x8 a, b;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        a[s] = from_f32<__bf16>(fa(r, k0 + 8 * kq + s));
        b[s] = from_f32<__bf16>(fb(k0 + 8 * kq + s, r));
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
    return acc;
  } else {
    return mm_tile<KD>(acc, lane, fa, fb);
  }
}

// The same tile product with each lane's operands read as contiguous runs: pa(r, k) points at
// A(r, k .. k + 7) and pb(r, k) at B(k .. k + 7, r) (a row of B^T), for k = k0 + 8 kq; the
// pointees are float or __bf16 (16-byte aligned).  bf16 inputs: one v_mfma_f32_16x16x32_bf16
// per 32 contraction indices (fp32 pointees rounded to bf16 as read); fp32 inputs: eight
// exact v_mfma_f32_16x16x4_f32 steps, step s contracting the indices k0 + 8 kq + s.
__device__ __forceinline__ void rd8(const float *p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 4);
  x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3]; x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}
__device__ __forceinline__ void rd8(const __bf16 *p, float (&x)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
  for (int s = 0; s < 8; ++s) x[s] = to_f32(v[s]);
}
__device__ __forceinline__ bf16x8 rd8b(const float *p) {
  float x[8];
  rd8(p, x);
  bf16x8 r;
#pragma unroll
  for (int s = 0; s < 8; ++s) r[s] = from_f32<__bf16>(x[s]);
  return r;
}
__device__ __forceinline__ bf16x8 rd8b(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
template <typename Tin, int KD, typename PA, typename PB>
__device__ __forceinline__ f32x4 mmr(f32x4 acc, int lane, PA pa, PB pb) {
  const int r = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int k0 = 0; k0 < KD; k0 += 32) {
    if constexpr (sizeof(Tin) == 2) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rd8b(pa(r, k0 + 8 * kq)), rd8b(pb(r, k0 + 8 * kq)),
                                                    acc, 0, 0, 0);
    } else {
      float a[8], b[8];
      rd8(pa(r, k0 + 8 * kq), a);
      rd8(pb(r, k0 + 8 * kq), b);
#pragma unroll
      for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
    }
  }
  return acc;
}

// Four consecutive elements as loaded (raw), and as fp32.
template <typename T> struct Raw4;
template <> struct Raw4<float> { typedef f32x4 type; };
template <> struct Raw4<__bf16> { typedef bf16x4 type; };
__device__ __forceinline__ f32x4 cvt4(const f32x4 &x) { return x; }
__device__ __forceinline__ f32x4 cvt4(const bf16x4 &x) {
  return f32x4{to_f32(x[0]), to_f32(x[1]), to_f32(x[2]), to_f32(x[3])};
}

// Rows [0, len) of a row-strided tensor, columns 0 .. NC - 1 from src, into an LDS tile with
// row stride LD (fp32, or bf16 rows copied as they are); rows past len are zero.  Every load
// of the thread is issued before the first store.  With sq, also each row's squared norm into
// sq[row] (the NC / 4 consecutive lanes that hold a row reduce it).
template <int NC, int LD, int NT, typename D, typename Src>
__device__ __forceinline__ void stage_rows(D *dst, const Src *src, size_t row_stride, int len,
                                           int tid, float *sq = nullptr) {
  constexpr int N4 = NC / 4;
  static_assert((kChunk * N4) % NT == 0 && 64 % N4 == 0, "whole rounds of pieces");
  static_assert(sizeof(D) == 4 || sizeof(Src) == 2, "bf16 tiles take bf16 rows");
  constexpr int NPER = kChunk * N4 / NT;
  typename Raw4<Src>::type x[NPER];
#pragma unroll
  for (int m = 0; m < NPER; ++m) {
    const int e = tid + NT * m, r = e / N4, c = 4 * (e % N4);
    typename Raw4<Src>::type z = {};
    if (r < len) z = *reinterpret_cast<const typename Raw4<Src>::type *>(src + (size_t)r * row_stride + c);
    x[m] = z;
  }
#pragma unroll
  for (int m = 0; m < NPER; ++m) {
    const int e = tid + NT * m, r = e / N4, c = 4 * (e % N4);
    if constexpr (sizeof(D) == 2)
      *reinterpret_cast<bf16x4 *>(dst + r * LD + c) = x[m];
    else
      *reinterpret_cast<f32x4 *>(dst + r * LD + c) = cvt4(x[m]);
  }
  if (sq) {
#pragma unroll
    for (int m = 0; m < NPER; ++m) {
      const f32x4 v = cvt4(x[m]);
      float ss = v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
#pragma unroll
      for (int off = 1; off < N4; off <<= 1) ss += __shfl_xor(ss, off, N4);
      const int e = tid + NT * m;
      if (e % N4 == 0) sq[e / N4] = ss;
    }
  }
}

// the (I, J) block of the ten blocks on and below the diagonal, in the order (0,0) (1,0) (1,1)
// (2,0) (2,1) (2,2) (3,0) .. (3,3)
__device__ __forceinline__ void lower_block(int b, int &I, int &J) {
  I = b >= 6 ? 3 : b >= 3 ? 2 : b >= 1 ? 1 : 0;
  J = b - I * (I + 1) / 2;
}

// A tile of NR rows x NC columns of a row-strided tensor, held in registers between its
// load (all of a thread's loads issued back to back) and its store into an fp32 LDS tile;
// rows at or past `len` read as zeros.
template <typename T, int NR, int NC, int NT>
struct RegTile {
  static constexpr int NQ = NR * NC / 4, J = (NQ + NT - 1) / NT;
  typename Raw4<T>::type x[J];
  __device__ __forceinline__ void load(const T *src, size_t row_stride, int len, int tid) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = tid + NT * j, r = e / (NC / 4), c = 4 * (e % (NC / 4));
      typename Raw4<T>::type z = {};
      if ((NQ % NT == 0 || e < NQ) && r < len)
        z = *reinterpret_cast<const typename Raw4<T>::type *>(src + (size_t)r * row_stride + c);
      x[j] = z;
    }
  }
  template <int LD, typename D>
  __device__ __forceinline__ void store(D *dst, int tid) const {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = tid + NT * j, r = e / (NC / 4), c = 4 * (e % (NC / 4));
      if (NQ % NT == 0 || e < NQ) {
        const f32x4 v = cvt4(x[j]);
        if constexpr (sizeof(D) == 2) {
          bf16x4 b;
#pragma unroll
          for (int i = 0; i < 4; ++i) b[i] = from_f32<__bf16>(v[i]);
          *reinterpret_cast<bf16x4 *>(dst + r * LD + c) = b;
        } else {
          *reinterpret_cast<f32x4 *>(dst + r * LD + c) = v;
        }
      }
    }
  }
  // each row's squared norm into sq[row] (the NC / 4 consecutive lanes holding a row reduce it)
  __device__ __forceinline__ void sqnorms(float *sq, int tid) const {
    constexpr int N4 = NC / 4;
    static_assert(NQ % NT == 0 && 64 % N4 == 0, "whole rows within a wavefront");
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const f32x4 v = cvt4(x[j]);
      float ss = v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
#pragma unroll
      for (int off = 1; off < N4; off <<= 1) ss += __shfl_xor(ss, off, N4);
      const int e = tid + NT * j;
      if (e % N4 == 0) sq[e / N4] = ss;
    }
  }
};

// A 64 x 64 matrix stored as its ten lower 16 x 16 blocks (the prep kernel's packed T and P),
// in registers; stored into the lower blocks of an fp32 LDS tile (the upper blocks are left
// as they are: zero).
template <typename T, int NT>
struct PackedTile {
  static constexpr int NQ = 10 * 256 / 4, J = (NQ + NT - 1) / NT;
  typename Raw4<T>::type x[J];
  __device__ __forceinline__ void load(const T *src, int tid) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int pq = tid + NT * j;
      typename Raw4<T>::type z = {};
      if (pq < NQ) z = *reinterpret_cast<const typename Raw4<T>::type *>(src + 4 * pq);
      x[j] = z;
    }
  }
  __device__ __forceinline__ void store(float (*dst)[LDC], int tid) const {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int pq = tid + NT * j;
      if (pq < NQ) {
        const int e0 = 4 * pq, w = e0 & 255;
        int I, Jb;
        lower_block(e0 >> 8, I, Jb);
        *reinterpret_cast<f32x4 *>(&dst[16 * I + (w >> 4)][16 * Jb + (w & 15)]) = cvt4(x[j]);
      }
    }
  }
};

// sum over the 16 lanes of a DPP row (lanes with the same l / 16)
__device__ __forceinline__ float row16_sum(float x) {
  x += __shfl_xor(x, 1, 16);
  x += __shfl_xor(x, 2, 16);
  x += __shfl_xor(x, 4, 16);
  x += __shfl_xor(x, 8, 16);
  return x;
}


// gfx950 ds_read_b64_tr_b16: within each group of 16 lanes, lane d receives element d & 3 of
// the 8-byte pieces addressed by lanes (d >> 2) + 4 i, i = 0..3.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
__device__ __forceinline__ bf16x4 tr_read(const __bf16 *p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(p)));
}
// Rows k .. k + 7 of column c0 + (lane & 15) of a row-major bf16 tile with row stride LD:
// lane s of each 16-lane group addresses row k + (s >> 2) (+ 4), columns c0 + 4 (s & 3) .. + 3.
template <int LD>
__device__ __forceinline__ bf16x8 col8(const __bf16 *M, int c0, int k, int lane) {
  const int s = lane & 15;
  const __bf16 *p = M + (k + (s >> 2)) * LD + c0 + 4 * (s & 3);
  const bf16x4 lo = tr_read(p), hi = tr_read(p + 4 * LD);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// Row c0 + (lane & 15), elements k .. k + 7, of a row-major bf16 tile.
template <int LD>
__device__ __forceinline__ bf16x8 row8(const __bf16 *M, int c0, int k, int lane) {
  return *reinterpret_cast<const bf16x8 *>(M + (c0 + (lane & 15)) * LD + k);
}
// acc += the 16 x 16 product with operand fragments fa(k), fb(k) for k = k0 + 8 kq.
template <int KD, typename FA, typename FB>
__device__ __forceinline__ f32x4 mmf(f32x4 acc, int lane, FA fa, FB fb) {
  const int kq = lane >> 4;
#pragma unroll
  for (int k0 = 0; k0 < KD; k0 += 32)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa(k0 + 8 * kq), fb(k0 + 8 * kq), acc, 0, 0, 0);
  return acc;
}


// Row stride of the gradient kernels' d_v-loop tiles, whole 16-byte units: 32 columns (40 bf16
// or 36 fp32).
template <typename LT> constexpr int ldl() { return sizeof(LT) == 2 ? 40 : 36; }

}  // namespace

// The per-chunk gradient kernel under diagonal gating (kla_bwd_diag.hip): Kg, X and A from
// launch_prep_diag, SN from the states-only scan, dS', dU and dR (= dv) from the adjoint scan;
// writes dq, dk (operand type), dg ([n_tok, H, d_k]) and deta (fp32).
hipError_t launch_bwd_grad_diag(Dtype dt, int d_k, int d_v, const void *q, const void *k,
                                const void *v, const void *dO, const float *g, const float *eta,
                                float eps, const CoefOpts &opts, const void *KG, const void *X,
                                const void *A, const void *SN, const void *dSo, const void *dU,
                                const void *dv, void *dq, void *dk, float *dg, float *deta,
                                SeqTables t, int32_t n_seq, int64_t n_chunks_ub, int32_t H,
                                hipStream_t stream);

}  // namespace kla
