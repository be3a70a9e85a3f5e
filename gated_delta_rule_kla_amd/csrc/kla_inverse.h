// kla_inverse.h -- X = (I + Diag(b) A)^{-1} for one 64 x 64 chunk in LDS, by 16 x 16 blocks.
//
// Paper "Kaczmarz Linear Attention" (arXiv 2605.08587), Proposition 3 / Eq. (7): the chunk
// solve needs T = (I + L)^{-1} Diag(b) with L = Diag(b) A strictly lower triangular.  With
// X = (I + L)^{-1} split into 16 x 16 blocks X_IJ (J <= I):
//   X_II = (I + L_II)^{-1}                        forward substitution, 16 rows
//   X_IJ = -X_II sum_{K=J}^{I-1} L_IK X_KJ        for I > J, in order of I - J
// which replaces 64 sequential substitution steps by 16 and three rounds of small products.
#pragma once

#include "kla_device.h"

namespace kla {

// x from the lane that the DPP control selects within this lane's row of 16
template <int CTRL>
__device__ __forceinline__ float inv_dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               CTRL, 0xF, 0xF, false));
}

// A: strictly lower 64 x 64 fp32 in LDS (row stride LDA; entries on and above the diagonal
// are never read), b: the 64 row factors, X: the output (row stride LDX), all 64 x 64 entries
// written (zeros above the diagonal).
// Y: LDS scratch of 3 * 256 floats, not aliasing A, b or X.  All NT threads of the
// workgroup call this; it begins and ends with a workgroup barrier.  NT is a multiple of 64.
template <int NT, int LDA, int LDX>
__device__ __forceinline__ void blocked_inverse(const float *A, const float *b, float *X,
                                                float *Y, int tid) {
  __syncthreads();
  for (int e = tid; e < 64 * 64; e += NT) {  // zeros above the diagonal blocks
    const int r = e >> 6, c = e & 63;
    if ((c >> 4) > (r >> 4)) X[r * LDX + c] = 0.f;
  }
  // ---- diagonal blocks: column job j (block I = j / 16, column c = j % 16) on 16 lanes (one
  //      DPP row); lane p keeps X_II[p][c] and adds its term of each row's dot product
  for (int j = tid >> 4; j < 64; j += NT / 16) {
    const int I = j >> 4, c = j & 15, p = tid & 15;
    float xp = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = p < i ? A[(16 * I + i) * LDA + 16 * I + p] * xp : 0.f;
      acc += inv_dpp<0xB1>(acc);   // quad_perm [1,0,3,2]
      acc += inv_dpp<0x4E>(acc);   // quad_perm [2,3,0,1]
      acc += inv_dpp<0x141>(acc);  // row_half_mirror
      acc += inv_dpp<0x140>(acc);  // row_mirror
      const float xi = i == c ? 1.f : (i > c ? -b[16 * I + i] * acc : 0.f);
      if (p == i) xp = xi;
    }
    X[(16 * I + p) * LDX + 16 * I + c] = xp;
  }
  // ---- sub-diagonal blocks by distance d = I - J: Y = sum_K L_IK X_KJ, then X_IJ = -X_II Y
  for (int d = 1; d < 4; ++d) {
    __syncthreads();
    const int nb = 4 - d;  // blocks (J + d, J), J = 0 .. nb - 1
    for (int e = tid; e < nb * 256; e += NT) {
      const int J = e >> 8, I = J + d, r = (e >> 4) & 15, c = e & 15;
      float s = 0.f;
      for (int K = J; K < I; ++K)
#pragma unroll
        for (int m = 0; m < 16; ++m)
          s += A[(16 * I + r) * LDA + 16 * K + m] * X[(16 * K + m) * LDX + 16 * J + c];
      Y[e] = b[16 * I + r] * s;
    }
    __syncthreads();
    for (int e = tid; e < nb * 256; e += NT) {
      const int J = e >> 8, I = J + d, r = (e >> 4) & 15, c = e & 15;
      float z = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) z += X[(16 * I + r) * LDX + 16 * I + m] * Y[J * 256 + m * 16 + c];
      X[(16 * I + r) * LDX + 16 * J + c] = -z;
    }
  }
  __syncthreads();
}

}  // namespace kla
