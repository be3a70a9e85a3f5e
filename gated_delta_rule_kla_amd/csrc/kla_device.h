// kla_device.h -- device helpers shared by the gfx950 KLA kernels.
//
// Matrix-core convention (CDNA3/CDNA4 16x16 MFMA layouts, 64-lane wavefront):
// a "k-step" contracts 32 values of the inner dimension.  Lane l = r + 16*kg
// (r = l % 16, kg = l / 16) supplies
//   A fragment: A[r][8*kg + s], s = 0..7     (row r of a 16 x 32 tile)
//   B fragment: B[8*kg + s][r], s = 0..7     (column r of a 32 x 16 tile)
// and receives the 16 x 16 fp32 result as
//   D fragment: D[4*kg + i][r], i = 0..3.
// bf16 operands use one v_mfma_f32_16x16x32_bf16 per k-step; fp32 operands use
// eight v_mfma_f32_16x16x4_f32, one per s.  Both sides of a product always use
// the same (kg, s) -> k assignment, so the contraction covers each k exactly once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kla {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int kChunk = 64;
constexpr int kWave = 64;

// ---------------------------------------------------------------- compact T and P tiles
// The per-chunk matrices T and P (64 x 64, lower triangular) in the form the scan stages them
// in LDS.  It leaves out the block of rows 0-31 x columns 32-63 (zero, and outside every
// operand read):
//   region A  rows 0-31, columns 0-31, in tile order: row slot 4 a + i of 16-row tile t
//             (token 8 a + 4 t + i) at row 16 t + 4 a + i, so that a tile's rows are adjacent;
//   region B  rows 32-63, all 64 columns, in token order.
// 16-byte units of a row are XOR-swizzled (twice the amount for fp32 rows) so that the scan's
// 16-byte fragment reads of a tile's rows hit distinct LDS banks.
template <typename T> constexpr int tpc_bytes() { return (32 * 32 + 32 * kChunk) * (int)sizeof(T); }
__device__ __forceinline__ int tpc_sw_a(int rho) { return ((rho >> 3) & 1) << 1; }
__device__ __forceinline__ int tpc_sw_b(int r) {
  return (((r >> 1) & 1) << 2) ^ (((r >> 3) & 1) * 3) ^ (((r >> 4) & 1) << 1);
}
// Byte offset of element e of row r (row < 32 requires e < 32).
template <typename T>
__device__ __forceinline__ int tpc_off(int r, int e) {
  constexpr int ES = sizeof(T);
  const int byte = e * ES;
  if (r < 32) {
    const int rho = 16 * ((r >> 2) & 1) + 4 * ((r >> 3) & 3) + (r & 3);
    const int u = (byte >> 4) ^ (tpc_sw_a(rho) * (ES / 2));
    return rho * 32 * ES + (u << 4) + (byte & 15);
  }
  const int u = (byte >> 4) ^ (tpc_sw_b(r) * (ES / 2));
  return 32 * 32 * ES + (r - 32) * kChunk * ES + (u << 4) + (byte & 15);
}
// In the workspace the tiles keep only their ten 16 x 16 blocks on and below the diagonal,
// each row-major, in the order (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) .. (3,3); the scan
// reads zeros for the two upper blocks the compact tile still holds.
constexpr int kTpbZero = 0x7ffffff0;  // out of range for any tile: a buffer load reads zeros
constexpr int kTpbElems = 10 * 256;  // elements of one packed tile
template <typename T> constexpr int tpb_bytes() { return kTpbElems * (int)sizeof(T); }
// Byte offset of the 16 bytes at (row, col), col a multiple of 16 / sizeof(T); kTpbZero above
// the diagonal blocks.
template <typename T>
__device__ __forceinline__ int tpb_off(int row, int col) {
  constexpr int ES = sizeof(T);
  const int I = row >> 4, J = col >> 4;
  if (J > I) return kTpbZero;
  return ((I * (I + 1) / 2 + J) * 256 + (row & 15) * 16 + (col & 15)) * ES;
}
// The row and column of the 16 bytes at byte offset pb of the packed blocks.
template <typename T>
__device__ __forceinline__ void tpb_piece(int pb, int &row, int &col) {
  constexpr int ES = sizeof(T);
  const int b = pb / (256 * ES), w = (pb % (256 * ES)) / ES;
  const int I = b >= 6 ? 3 : b >= 3 ? 2 : b >= 1 ? 1 : 0, J = b - I * (I + 1) / 2;
  row = 16 * I + w / 16;
  col = 16 * J + w % 16;
}
// The row and first column of the 16 bytes at byte offset pb (a multiple of 16) of a compact
// tile.
template <typename T>
__device__ __forceinline__ void tpc_piece(int pb, int &row, int &col) {
  constexpr int ES = sizeof(T), RA = 32 * ES, RB = kChunk * ES;
  if (pb < 32 * RA) {
    const int rho = pb / RA;
    row = 8 * ((rho >> 2) & 3) + 4 * (rho >> 4) + (rho & 3);
    col = ((((pb % RA) >> 4) ^ (tpc_sw_a(rho) * (ES / 2))) << 4) / ES;
  } else {
    const int qb = pb - 32 * RA;
    row = 32 + qb / RB;
    col = ((((qb % RB) >> 4) ^ (tpc_sw_b(row) * (ES / 2))) << 4) / ES;
  }
}

// ---------------------------------------------------------------- element types
template <typename T> struct Frag;
template <> struct Frag<__bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// float -> bf16 with round-to-nearest-even (NaN stays NaN)
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) {
  return static_cast<__bf16>(x);
}

// ---------------------------------------------------------------- buffer access
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (stride 0, byte-addressed, range checked against `bytes`): loads
// beyond the range return zeros and stores beyond it are dropped.
__device__ __forceinline__ Rsrc make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// 8 consecutive elements at byte offset voff (zeros out of range).
template <typename T> __device__ __forceinline__ typename Frag<T>::type bload8(Rsrc r, int voff);
template <> __device__ __forceinline__ bf16x8 bload8<__bf16>(Rsrc r, int voff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
template <> __device__ __forceinline__ f32x8 bload8<float>(Rsrc r, int voff) {
  const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
  const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, 0, 0);
  const f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
  return f32x8{fa[0], fa[1], fa[2], fa[3], fb[0], fb[1], fb[2], fb[3]};
}
__device__ __forceinline__ float bload1(Rsrc r, int voff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}

// ---------------------------------------------------------------- MFMA k-step
__device__ __forceinline__ f32x4 mma(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const f32x8 &a, const f32x8 &b, f32x4 c) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
  return c;
}

// ---------------------------------------------------------------- fragment loads
// 8 consecutive elements (16 B for bf16, 32 B for fp32) starting at p.
template <typename T> __device__ __forceinline__ typename Frag<T>::type load8(const T *p);
template <> __device__ __forceinline__ bf16x8 load8<__bf16>(const __bf16 *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}
template <> __device__ __forceinline__ f32x8 load8<float>(const float *p) {
  const f32x4 lo = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 hi = *reinterpret_cast<const f32x4 *>(p + 4);
  f32x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// 8 consecutive fp32 values converted to the operand type T.
template <typename T> __device__ __forceinline__ typename Frag<T>::type load8_cvt(const float *p);
template <> __device__ __forceinline__ f32x8 load8_cvt<float>(const float *p) {
  return load8<float>(p);
}
template <> __device__ __forceinline__ bf16x8 load8_cvt<__bf16>(const float *p) {
  const f32x8 x = load8<float>(p);
  bf16x8 r;
#pragma unroll
  for (int s = 0; s < 8; ++s) r[s] = static_cast<__bf16>(x[s]);
  return r;
}

// Convert 8 fp32 values to the operand type T.
template <typename T> __device__ __forceinline__ typename Frag<T>::type cvt8(const f32x8 &x);
template <> __device__ __forceinline__ f32x8 cvt8<float>(const f32x8 &x) { return x; }
template <> __device__ __forceinline__ bf16x8 cvt8<__bf16>(const f32x8 &x) {
  bf16x8 r;
#pragma unroll
  for (int s = 0; s < 8; ++s) r[s] = static_cast<__bf16>(x[s]);
  return r;
}

template <typename T> __device__ __forceinline__ typename Frag<T>::type zero8() {
  typename Frag<T>::type r;
#pragma unroll
  for (int s = 0; s < 8; ++s) r[s] = from_f32<T>(0.0f);
  return r;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------- write coefficient
// Variants of the write coefficient b_t and of the readout (paper section 3.1, Eq. (3) for
// the default; section 2 for the gated delta rule's b_t = eta_t; Appendix D and Table 5 for
// the key-norm-only coefficient and the sequence factors 1/t, 1/sqrt(t), 1/log(t + 1) on
// the Kaczmarz coefficient, t the absolute 1-based position in the sequence; section 3.3
// and Algorithm 1's readout for the readout divided by ||q_t||).
enum BetaMode { kBetaKaczmarz = 0, kBetaGated = 1, kBetaKeyNorm = 2, kBetaInvT = 3,
                kBetaInvSqrtT = 4, kBetaInvLogT = 5 };
struct CoefOpts {
  int beta_mode;            // BetaMode
  int normalize_q;          // nonzero: o_t = q_t S_t / ||q_t||
  const int32_t *pos_offset;  // per sequence (prefill) or batch row (decode); may be null
  int diag_gate = 0;        // nonzero: g holds one log-decay per key channel
};

// b_t from eta_t, den = ||k_t||^2 + eps and the absolute position t >= 1; a zero
// denominator gives b_t = 0 wherever b_t divides by it.
// Reciprocals use the hardware's approximate v_rcp_f32 / v_rsq_f32 (about 1 ulp).
__device__ __forceinline__ float write_coef(int mode, float eta_t, float den, float t) {
  if (mode == kBetaGated) return eta_t;
  const float rden = den != 0.f ? __builtin_amdgcn_rcpf(den) : 0.f;
  if (mode == kBetaKeyNorm) return rden;
  float b = eta_t * rden;
  if (mode == kBetaInvT) b *= __builtin_amdgcn_rcpf(t);
  else if (mode == kBetaInvSqrtT) b *= __builtin_amdgcn_rsqf(t);
  else if (mode == kBetaInvLogT) b *= __builtin_amdgcn_rcpf(logf(t + 1.f));
  return b;
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// LDS-only workgroup barrier: orders LDS traffic without waiting for the global
// loads that are deliberately left in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inclusive prefix sum across the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_inclusive_scan(float x, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

}  // namespace kla
