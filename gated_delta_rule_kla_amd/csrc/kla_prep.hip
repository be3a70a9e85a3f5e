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
// ---------------------------------------------------------------------------------------------
template <typename Tin, int DK>
struct PrepSmem {
  static constexpr int PAD = 8;
  alignas(16) Tin K[kChunk][DK + PAD];   // chunk keys, token-major
  alignas(16) float L[kChunk][kChunk + 4];
  alignas(16) float norm2[kChunk];
  alignas(16) float beta[kChunk];
  alignas(16) float G[kChunk];
};

template <typename Tin, int DK, typename TOut>
__global__ __launch_bounds__(256) void kla_prep_kernel(
    const Tin *__restrict__ k, const float *__restrict__ g, const float *__restrict__ eta,
    float eps, const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off, int n_seq,
    int H, float *__restrict__ G_out, float *__restrict__ beta_out, TOut *__restrict__ T_out) {
  __shared__ PrepSmem<Tin, DK> sm;
  const int c = blockIdx.x, h = blockIdx.y;
  if (c >= chunk_off[n_seq]) return;
  const int n = find_sequence(chunk_off, n_seq, c);
  const int t0 = cu[n] + (c - chunk_off[n]) * kChunk;
  const int len = min(kChunk, cu[n + 1] - t0);
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kg = lane >> 4;

  // ---- stage K rows (zero past the chunk end) and ||k_i||^2 by a lane-group reduction
  constexpr int CPR = DK / 8;       // 8-element groups per key row
  constexpr int RPP = 256 / CPR;    // rows per pass
#pragma unroll
  for (int pass = 0; pass < kChunk / RPP; ++pass) {
    const int row = pass * RPP + tid / CPR, cg = tid % CPR;
    typename Frag<Tin>::type x = zero8<Tin>();
    if (row < len) x = load8<Tin>(k + ((size_t)(t0 + row) * H + h) * DK + cg * 8);
    *reinterpret_cast<typename Frag<Tin>::type *>(&sm.K[row][cg * 8]) = x;
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
  }
  __syncthreads();

  // ---- Gram K K^T on the matrix cores, rows [16 wid, 16 wid + 16); then L
  {
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      const auto a = load8<Tin>(&sm.K[16 * wid + r16][32 * ks + 8 * kg]);
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const auto b = load8<Tin>(&sm.K[16 * jt + r16][32 * ks + 8 * kg]);
        acc[jt] = mma(a, b, acc[jt]);
      }
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * wid + 4 * kg + i, col = 16 * jt + r16;
        float val = 0.f;
        if (col < row) val = sm.beta[row] * __expf(sm.G[row] - sm.G[col]) * acc[jt][i];
        sm.L[row][col] = val;
      }
    }
  }
  __syncthreads();

  // ---- X = (I + L)^{-1} by forward substitution; lane = column, rows in registers.
  // x_i = delta_ic - sum_{j<i} L_ij x_j  (x_j = 0 for j < c by construction), T_ic = x_i b_c.
  if (wid == 0) {
    float x[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      float acc = (i == lane) ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < (i & ~3); j += 4) {
        const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&sm.L[i][j]);
        acc = fmaf(-l4[0], x[j + 0], acc);
        acc = fmaf(-l4[1], x[j + 1], acc);
        acc = fmaf(-l4[2], x[j + 2], acc);
        acc = fmaf(-l4[3], x[j + 3], acc);
      }
#pragma unroll
      for (int j = (i & ~3); j < i; ++j) acc = fmaf(-sm.L[i][j], x[j], acc);
      x[i] = acc;
    }
    const float bc = sm.beta[lane];
    TOut *Tc = T_out + ((size_t)c * H + h) * (kChunk * kChunk);
#pragma unroll
    for (int i = 0; i < kChunk; ++i) Tc[i * kChunk + lane] = from_f32<TOut>(x[i] * bc);
  }
}

template <typename Tin, int DK>
static hipError_t launch_prep_t(const void *k, const float *g, const float *eta, float eps,
                                SeqTables t, int32_t n_seq, int64_t n_chunks_ub, int32_t H,
                                float *G_out, float *beta_out, void *T_out, bool t_fp32,
                                hipStream_t stream) {
  if (n_chunks_ub <= 0) return hipSuccess;
  const dim3 grid((unsigned)n_chunks_ub, H);
  if (t_fp32 || sizeof(Tin) == 4)
    hipLaunchKernelGGL((kla_prep_kernel<Tin, DK, float>), grid, dim3(256), 0, stream,
                       static_cast<const Tin *>(k), g, eta, eps, t.cu, t.chunk_off, n_seq, H,
                       G_out, beta_out, static_cast<float *>(T_out));
  else
    hipLaunchKernelGGL((kla_prep_kernel<Tin, DK, Tin>), grid, dim3(256), 0, stream,
                       static_cast<const Tin *>(k), g, eta, eps, t.cu, t.chunk_off, n_seq, H,
                       G_out, beta_out, static_cast<Tin *>(T_out));
  return hipGetLastError();
}

hipError_t launch_prep(Dtype dt, int d_k, const void *k, const float *g, const float *eta,
                       float eps, SeqTables t, int32_t n_seq, int64_t n_chunks_ub, int32_t H,
                       float *G_out, float *beta_out, void *T_out, bool t_fp32,
                       hipStream_t stream) {
  if (dt == Dtype::BF16) {
    if (d_k == 128)
      return launch_prep_t<__bf16, 128>(k, g, eta, eps, t, n_seq, n_chunks_ub, H, G_out, beta_out,
                                        T_out, t_fp32, stream);
    return launch_prep_t<__bf16, 64>(k, g, eta, eps, t, n_seq, n_chunks_ub, H, G_out, beta_out,
                                     T_out, t_fp32, stream);
  }
  if (d_k == 128)
    return launch_prep_t<float, 128>(k, g, eta, eps, t, n_seq, n_chunks_ub, H, G_out, beta_out,
                                     T_out, t_fp32, stream);
  return launch_prep_t<float, 64>(k, g, eta, eps, t, n_seq, n_chunks_ub, H, G_out, beta_out,
                                  T_out, t_fp32, stream);
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
