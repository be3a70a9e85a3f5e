// kla_prep.hip -- sequence planning and the per-chunk stage of the chunkwise solve.
//
// Paper "Kaczmarz Linear Attention" (arXiv 2605.08587), section 4 and
// Algorithm 1 (chunkwise panel): for every chunk of C = 64 tokens of every
// (sequence, head) this stage computes, fully in parallel,
//   b_i = eta_i / (||k_i||^2 + eps)                      Eq. (3)
//   G_i = g_1 + ... + g_i (chunk-local log-decay)        gamma_i = exp(G_i)
//   L   = Diag(b) (A^- o K K^T),  A^-_ij = exp(G_i - G_j), j < i      Appendix B.2
//   T   = (I + L)^{-1} Diag(b)                           so that Eq. (7) reads
//                                                        U = T (V - Diag(gamma) K S0)
// The Gram matrix runs on the matrix cores; (I + L)^{-1} is formed by forward
// substitution out of LDS, one column per lane of a wavefront.
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {

// ---------------------------------------------------------------------------------------------
// Plan: sanitised sequence offsets and chunk offsets, one workgroup of 1024 threads.
// cu_out[n] = running max of clamp(cu_in[n], 0, total) (dense input: n * total / n_seq);
// chunk_off[n] = sum_{m < n} ceil((cu_out[m+1] - cu_out[m]) / 64).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ int block_scan_1024(int x, int *buf, bool is_max) {
  const int tid = threadIdx.x;
  buf[tid] = x;
  __syncthreads();
#pragma unroll 1
  for (int off = 1; off < 1024; off <<= 1) {
    const int y = (tid >= off) ? buf[tid - off] : (is_max ? INT32_MIN : 0);
    __syncthreads();
    x = is_max ? max(x, y) : x + y;
    buf[tid] = x;
    __syncthreads();
  }
  return x;  // inclusive
}

__global__ __launch_bounds__(1024) void kla_plan_kernel(const int32_t *__restrict__ cu_in,
                                                        int32_t n_seq, int32_t total,
                                                        int32_t *__restrict__ cu_out,
                                                        int32_t *__restrict__ chunk_off) {
  __shared__ int buf[1024];
  const int tid = threadIdx.x;
  const int n_ent = n_seq + 1;  // offsets n = 0..n_seq
  const int per = (n_ent + 1023) / 1024;
  const int e0 = min(tid * per, n_ent), e1 = min(e0 + per, n_ent);
  const int dense_len = (cu_in == nullptr && n_seq > 0) ? total / n_seq : 0;
  auto raw = [&](int n) -> int {
    if (cu_in == nullptr) return n * dense_len;
    return min(max(cu_in[n], 0), total);
  };
  // pass 1: running maximum of the clamped offsets
  int local_max = INT32_MIN;
  for (int n = e0; n < e1; ++n) local_max = max(local_max, raw(n));
  int incl = block_scan_1024(local_max, buf, true);
  int run = (tid == 0) ? INT32_MIN : buf[tid - 1];
  __syncthreads();
  for (int n = e0; n < e1; ++n) {
    run = max(run, raw(n));
    cu_out[n] = (n == 0) ? raw(0) : run;
  }
  (void)incl;
  __syncthreads();
  __threadfence_block();
  // pass 2: chunk counts of sequences e0..e1-1 (sequence n spans cu_out[n]..cu_out[n+1])
  int local_sum = 0;
  for (int n = e0; n < e1 && n < n_seq; ++n) local_sum += (cu_out[n + 1] - cu_out[n] + 63) / 64;
  int incl_sum = block_scan_1024(local_sum, buf, false);
  int acc = incl_sum - local_sum;
  for (int n = e0; n < e1; ++n) {
    chunk_off[n] = acc;
    if (n < n_seq) acc += (cu_out[n + 1] - cu_out[n] + 63) / 64;
  }
}

hipError_t launch_plan(const int32_t *cu_in, int32_t n_seq, int32_t total_tokens, SeqTables t,
                       hipStream_t stream) {
  hipLaunchKernelGGL(kla_plan_kernel, dim3(1), dim3(1024), 0, stream, cu_in, n_seq, total_tokens,
                     t.cu, t.chunk_off);
  return hipGetLastError();
}

// Locate the chunk: sequence n with chunk_off[n] <= c < chunk_off[n + 1].
__device__ __forceinline__ int find_sequence(const int32_t *__restrict__ chunk_off, int n_seq,
                                             int c) {
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunk_off[mid] <= c) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------------------------
// Prep / UT kernel: one workgroup (4 wavefronts) per (chunk, head).
//
// (I + L)^{-1} is formed blockwise on 16 x 16 blocks (X = (I + L)^{-1} is unit lower
// triangular): every wavefront inverts one diagonal block by substitution, then the
// sub-diagonal blocks follow level by level,
//   X_ij = -X_ii (sum_{k=j}^{i-1} L_ik X_kj),  i > j,
// with the 16 x 16 x 16 products on the fp32 matrix cores.  T = X Diag(b).
// When q is given the kernel also writes P = (A o Q K^T) (Eq. (8)'s intra-chunk matrix,
// A_ij = exp(G_i - G_j) for j <= i, zero above the diagonal) for the scan.
// ---------------------------------------------------------------------------------------------
template <typename Tin, int DK>
struct PrepSmem {
  static constexpr int PAD = 8;
  alignas(16) Tin K[kChunk][DK + PAD];   // chunk keys, token-major
  alignas(16) Tin Q[kChunk][DK + PAD];   // chunk queries, token-major (only when P is wanted)
  alignas(16) float L[kChunk][kChunk + 4];
  alignas(16) float X[kChunk][kChunk + 4];
  alignas(16) float norm2[kChunk];
  alignas(16) float beta[kChunk];
  alignas(16) float G[kChunk];
};

// D += A B for 16 x 16 fp32 blocks in LDS (row strides lda, ldb), on v_mfma_f32_16x16x4_f32.
__device__ __forceinline__ f32x4 mm16(const float *A, int lda, const float *B, int ldb, f32x4 acc,
                                      int r16, int kg) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[r16 * lda + 4 * s + kg],
                                               B[(4 * s + kg) * ldb + r16], acc, 0, 0, 0);
  return acc;
}
// D += A Y with Y a 16 x 16 block held in accumulator layout (lane (r16, kg) holds rows
// 4 kg + e of column r16): the contraction index is taken in the order the lanes hold it.
__device__ __forceinline__ f32x4 mm16_acc(const float *A, int lda, const f32x4 &Y, f32x4 acc,
                                          int r16, int kg) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[r16 * lda + 4 * kg + s], Y[s], acc, 0, 0, 0);
  return acc;
}

template <typename Tin, int DK, typename TOut>
__global__ __launch_bounds__(256) void kla_prep_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ eta, float eps, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, int n_seq, int H, float *__restrict__ G_out,
    float *__restrict__ beta_out, TOut *__restrict__ T_out, Tin *__restrict__ P_out,
    float *__restrict__ GD_out) {
  __shared__ PrepSmem<Tin, DK> sm;
  const int c = blockIdx.x, h = blockIdx.y;
  if (c >= chunk_off[n_seq]) return;
  const int n = find_sequence(chunk_off, n_seq, c);
  const int t0 = cu[n] + (c - chunk_off[n]) * kChunk;
  const int len = min(kChunk, cu[n + 1] - t0);
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kg = lane >> 4;
  const bool want_p = (q != nullptr) && (P_out != nullptr);
  using FragT = typename Frag<Tin>::type;

  // ---- stage K (and Q) rows (zero past the chunk end); ||k_i||^2 by a lane-group reduction
  constexpr int CPR = DK / 8;       // 8-element groups per key row
  constexpr int RPP = 256 / CPR;    // rows per pass
#pragma unroll
  for (int pass = 0; pass < kChunk / RPP; ++pass) {
    const int row = pass * RPP + tid / CPR, cg = tid % CPR;
    FragT x = zero8<Tin>(), y = zero8<Tin>();
    if (row < len) {
      x = load8<Tin>(k + ((size_t)(t0 + row) * H + h) * DK + cg * 8);
      if (want_p) y = load8<Tin>(q + ((size_t)(t0 + row) * H + h) * DK + cg * 8);
    }
    *reinterpret_cast<FragT *>(&sm.K[row][cg * 8]) = x;
    if (want_p) *reinterpret_cast<FragT *>(&sm.Q[row][cg * 8]) = y;
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float xf = to_f32(x[s]);
      ss = fmaf(xf, xf, ss);
    }
#pragma unroll
    for (int off = CPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, kWave);
    if (cg == 0) sm.norm2[row] = ss;
  }
  __syncthreads();

  // ---- b and chunk-local inclusive log-decay (wavefront scan)
  if (wid == 0) {
    const bool valid = lane < len;
    const size_t th = (size_t)(t0 + lane) * H + h;
    const float gi = valid ? g[th] : 0.f;
    const float Gi = wave_inclusive_scan(gi, lane);
    const float den = sm.norm2[lane] + eps;
    const float bi = (valid && den != 0.f) ? eta[th] / den : 0.f;
    sm.G[lane] = Gi;
    sm.beta[lane] = bi;
    if (valid) {
      if (G_out) G_out[th] = Gi;
      if (beta_out) beta_out[th] = bi;
    }
    // per-chunk decays for the scan: exp(G_i) and exp(G_last - G_i); rows past a ragged
    // end carry G_last (their g is taken as 0), so they read exp(G_last) and 1
    if (GD_out) {
      const float Glast = __shfl(Gi, kChunk - 1, kWave);
      float *gd = GD_out + ((size_t)c * H + h) * (2 * kChunk);
      gd[lane] = __expf(Gi);
      gd[kChunk + lane] = __expf(Glast - Gi);
    }
  }
  __syncthreads();

  const int i0 = 16 * wid;  // this wave's 16 rows
  // ---- Gram K K^T on the matrix cores (causal tiles only), then the strictly lower L
  {
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      f32x4 acc = zero4();
      if (jt <= wid) {
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
          const FragT a = load8<Tin>(&sm.K[i0 + r16][32 * ks + 8 * kg]);
          const FragT b = load8<Tin>(&sm.K[16 * jt + r16][32 * ks + 8 * kg]);
          acc = mma(a, b, acc);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = i0 + 4 * kg + e, col = 16 * jt + r16;
        float val = 0.f;
        if (col < row) val = sm.beta[row] * __expf(sm.G[row] - sm.G[col]) * acc[e];
        sm.L[row][col] = val;
      }
    }
  }
  // ---- P = A o Q K^T, as P^T = K Q^T so each lane holds 4 consecutive columns of a row
  if (want_p) {
    const int i = i0 + r16;
    Tin *Pc = P_out + ((size_t)c * H + h) * (kChunk * kChunk) + (size_t)i * kChunk;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const int j0 = 16 * jt + 4 * kg;
      float pv[4] = {0.f, 0.f, 0.f, 0.f};
      if (jt <= wid) {
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
          const FragT a = load8<Tin>(&sm.K[16 * jt + r16][32 * ks + 8 * kg]);
          const FragT b = load8<Tin>(&sm.Q[i][32 * ks + 8 * kg]);
          acc = mma(a, b, acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pv[e] = (j0 + e <= i) ? __expf(sm.G[i] - sm.G[j0 + e]) * acc[e] : 0.f;
      }
      if constexpr (sizeof(Tin) == 2) {
        bf16x4 x4;
#pragma unroll
        for (int e = 0; e < 4; ++e) x4[e] = from_f32<Tin>(pv[e]);
        *reinterpret_cast<bf16x4 *>(Pc + j0) = x4;
      } else {
        *reinterpret_cast<f32x4 *>(Pc + j0) = f32x4{pv[0], pv[1], pv[2], pv[3]};
      }
    }
  }
  __syncthreads();

  // ---- diagonal blocks: wave w inverts I + L_ww by substitution, lane = column r16
  {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = (i == r16) ? 1.f : 0.f;
      const float *Lrow = &sm.L[i0 + i][i0];
#pragma unroll
      for (int j = 0; j < i; ++j) acc = fmaf(-Lrow[j], x[j], acc);
      x[i] = acc;
    }
    if (kg == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sm.X[i0 + i][i0 + r16] = x[i];
    }
  }
  __syncthreads();
  // ---- sub-diagonal blocks, one level (distance) at a time
  constexpr int LDL = kChunk + 4;
#pragma unroll
  for (int dist = 1; dist < 4; ++dist) {
    const int jb = wid, ib = wid + dist;  // block (ib, jb)
    if (ib < 4) {
      f32x4 Y = zero4();
      for (int kb = jb; kb < ib; ++kb)
        Y = mm16(&sm.L[16 * ib][16 * kb], LDL, &sm.X[16 * kb][16 * jb], LDL, Y, r16, kg);
      f32x4 Z = mm16_acc(&sm.X[16 * ib][16 * ib], LDL, Y, zero4(), r16, kg);
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.X[16 * ib + 4 * kg + e][16 * jb + r16] = -Z[e];
    }
    __syncthreads();
  }

  // ---- T = X Diag(b), zero above the diagonal (blocks above the diagonal were never written)
  {
    TOut *Tc = T_out + ((size_t)c * H + h) * (kChunk * kChunk);
#pragma unroll
    for (int kk = 0; kk < kChunk * kChunk / 256; ++kk) {
      const int e = tid + 256 * kk, row = e >> 6, j = e & 63;
      const float val = (j <= row) ? sm.X[row][j] * sm.beta[j] : 0.f;
      Tc[e] = from_f32<TOut>(val);
    }
  }
}

template <typename Tin, int DK>
static hipError_t launch_prep_t(const void *q, const void *k, const float *g, const float *eta,
                                float eps, SeqTables t, int32_t n_seq, int64_t n_chunks_ub,
                                int32_t H, float *G_out, float *beta_out, void *T_out, bool t_fp32,
                                void *P_out, float *GD_out, hipStream_t stream) {
  if (n_chunks_ub <= 0) return hipSuccess;
  const dim3 grid((unsigned)n_chunks_ub, H);
  const Tin *qq = static_cast<const Tin *>(q);
  Tin *pp = static_cast<Tin *>(P_out);
  if (t_fp32 || sizeof(Tin) == 4)
    hipLaunchKernelGGL((kla_prep_kernel<Tin, DK, float>), grid, dim3(256), 0, stream, qq,
                       static_cast<const Tin *>(k), g, eta, eps, t.cu, t.chunk_off, n_seq, H,
                       G_out, beta_out, static_cast<float *>(T_out), pp, GD_out);
  else
    hipLaunchKernelGGL((kla_prep_kernel<Tin, DK, Tin>), grid, dim3(256), 0, stream, qq,
                       static_cast<const Tin *>(k), g, eta, eps, t.cu, t.chunk_off, n_seq, H,
                       G_out, beta_out, static_cast<Tin *>(T_out), pp, GD_out);
  return hipGetLastError();
}

hipError_t launch_prep(Dtype dt, int d_k, const void *q, const void *k, const float *g,
                       const float *eta, float eps, SeqTables t, int32_t n_seq,
                       int64_t n_chunks_ub, int32_t H, float *G_out, float *beta_out, void *T_out,
                       bool t_fp32, void *P_out, float *GD_out, hipStream_t stream) {
  if (dt == Dtype::BF16) {
    if (d_k == 128)
      return launch_prep_t<__bf16, 128>(q, k, g, eta, eps, t, n_seq, n_chunks_ub, H, G_out,
                                        beta_out, T_out, t_fp32, P_out, GD_out, stream);
    return launch_prep_t<__bf16, 64>(q, k, g, eta, eps, t, n_seq, n_chunks_ub, H, G_out, beta_out,
                                     T_out, t_fp32, P_out, GD_out, stream);
  }
  if (d_k == 128)
    return launch_prep_t<float, 128>(q, k, g, eta, eps, t, n_seq, n_chunks_ub, H, G_out, beta_out,
                                     T_out, t_fp32, P_out, GD_out, stream);
  return launch_prep_t<float, 64>(q, k, g, eta, eps, t, n_seq, n_chunks_ub, H, G_out, beta_out,
                                  T_out, t_fp32, P_out, GD_out, stream);
}

// ---------------------------------------------------------------------------------------------
// WY factors (unit-check path, not used by the prefill): W = T Diag(exp G) K, U~ = T V,
// Appendix B's w and u vectors stacked per chunk.  Plain fp32 loops, one workgroup per
// (chunk, head); rows past the chunk end are not written.
// ---------------------------------------------------------------------------------------------
template <typename Tin>
__global__ __launch_bounds__(256) void kla_wy_kernel(
    const Tin *__restrict__ k, const Tin *__restrict__ v, const float *__restrict__ G,
    const float *__restrict__ T, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, int n_seq, int H, int DK, int DV,
    float *__restrict__ W, float *__restrict__ Ut) {
  __shared__ float sT[kChunk][kChunk + 1];
  __shared__ float sgam[kChunk];
  const int c = blockIdx.x, h = blockIdx.y;
  if (c >= chunk_off[n_seq]) return;
  const int n = find_sequence(chunk_off, n_seq, c);
  const int t0 = cu[n] + (c - chunk_off[n]) * kChunk;
  const int len = min(kChunk, cu[n + 1] - t0);
  const float *Tc = T + ((size_t)c * H + h) * (kChunk * kChunk);
  for (int e = threadIdx.x; e < kChunk * kChunk; e += blockDim.x) sT[e / kChunk][e % kChunk] = Tc[e];
  if (threadIdx.x < kChunk)
    sgam[threadIdx.x] =
        threadIdx.x < len ? __expf(G[(size_t)(t0 + threadIdx.x) * H + h]) : 0.f;
  __syncthreads();
  if (W) {
    for (int e = threadIdx.x; e < len * DK; e += blockDim.x) {
      const int i = e / DK, col = e % DK;
      float acc = 0.f;
      for (int j = 0; j <= i; ++j)
        acc = fmaf(sT[i][j] * sgam[j], to_f32(k[((size_t)(t0 + j) * H + h) * DK + col]), acc);
      W[((size_t)(t0 + i) * H + h) * DK + col] = acc;
    }
  }
  if (Ut) {
    for (int e = threadIdx.x; e < len * DV; e += blockDim.x) {
      const int i = e / DV, col = e % DV;
      float acc = 0.f;
      for (int j = 0; j <= i; ++j)
        acc = fmaf(sT[i][j], to_f32(v[((size_t)(t0 + j) * H + h) * DV + col]), acc);
      Ut[((size_t)(t0 + i) * H + h) * DV + col] = acc;
    }
  }
}

hipError_t launch_wy(Dtype dt, int d_k, int d_v, const void *k, const void *v, const float *G,
                     const float *T, SeqTables t, int32_t n_seq, int64_t n_chunks_ub, int32_t H,
                     float *W, float *Ut, hipStream_t stream) {
  if (n_chunks_ub <= 0 || (!W && !Ut)) return hipSuccess;
  if (dt == Dtype::BF16)
    hipLaunchKernelGGL(kla_wy_kernel<__bf16>, dim3((unsigned)n_chunks_ub, H), dim3(256), 0, stream,
                       static_cast<const __bf16 *>(k), static_cast<const __bf16 *>(v), G, T, t.cu,
                       t.chunk_off, n_seq, H, d_k, d_v, W, Ut);
  else
    hipLaunchKernelGGL(kla_wy_kernel<float>, dim3((unsigned)n_chunks_ub, H), dim3(256), 0, stream,
                       static_cast<const float *>(k), static_cast<const float *>(v), G, T, t.cu,
                       t.chunk_off, n_seq, H, d_k, d_v, W, Ut);
  return hipGetLastError();
}

}  // namespace kla
