// kla_diag.hip -- the per-chunk stage of the prefill under diagonal gating.
//
// Paper "Kaczmarz Linear Attention" (arXiv 2605.08587), Appendix B.5: with the decay
// Diag(alpha_t), one factor per key channel, the scalar decay products of Propositions 3-4
// act per channel.  Working a chunk of C tokens through as for the scalar gate, with G the
// chunk-local cumulative log-decay per channel (C x d_k) and b the Kaczmarz coefficient
// (unchanged, Eq. (3)):
//   A_ij  = sum_c k_i[c] k_j[c] exp(G_i[c] - G_j[c])     (j < i)
//   T     = (I + Diag(b) A)^{-1} Diag(b)
//   P_ij  = sum_c q_i[c] k_j[c] exp(G_i[c] - G_j[c])     (j <= i)
//   U     = T (V - Kg S),  O = Qg S + P U,  S_out = Diag(exp(G_last)) S + Kd^T U
// with the decayed tiles Kg = K o exp(G), Qg = Q o exp(G) and Kd = K o exp(G_last - G).
// This kernel forms b, G, T, P, Kg, Qg, Kd and exp(G_last) for each (chunk, head); the
// chunk scan then runs as for the scalar gate on Kg, Qg, Kd in place of K, Q (see
// kla_scan.hip), with unit decays and the per-channel state decay exp(G_last).
//
// One 256-lane workgroup per (chunk, head), everything staged in LDS in fp32.  Every decay
// factor is an exponential of a difference G_i - G_j with j <= i (or G_last - G_j), never
// positive, so nothing overflows whatever the decay.
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {

namespace {

constexpr int kDiagThreads = 256;

__device__ __forceinline__ int find_seq(const int32_t *__restrict__ chunk_off, int n_seq, int c) {
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunk_off[mid] <= c) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int DK>
struct DiagSmem {
  // rows of DK + 1 floats: the pair loops read a column of several rows at once
  float K[kChunk][DK + 1], Q[kChunk][DK + 1], G[kChunk][DK + 1];
  float A[kChunk][kChunk + 1], P[kChunk][kChunk + 1], X[kChunk][kChunk + 1];
  float b[kChunk], rq[kChunk];
};

template <typename T>
__device__ __forceinline__ void put(T *dst, size_t i, float x) {
  dst[i] = from_f32<T>(x);
}

}  // namespace

template <typename Tin, int DK>
__global__ __launch_bounds__(kDiagThreads) void kla_prep_diag_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ eta, float eps, CoefOpts opts, SeqTables tabs, int n_seq, int H,
    Tin *__restrict__ T_out, Tin *__restrict__ P_out, float *__restrict__ GD_out,
    Tin *__restrict__ KG_out, Tin *__restrict__ QG_out, Tin *__restrict__ KD_out,
    float *__restrict__ GC_out) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  DiagSmem<DK> &sm = *reinterpret_cast<DiagSmem<DK> *>(smem_raw);
  const int n_chunks = tabs.chunk_off[n_seq];
  const int task = blockIdx.x;  // chunk * H + head
  if (task >= n_chunks * H) return;
  const int c = task / H, h = task - c * H;
  const int n = find_seq(tabs.chunk_off, n_seq, c);
  const int ts = tabs.cu[n];
  const int t0 = ts + (c - tabs.chunk_off[n]) * kChunk;
  const int len = min(kChunk, tabs.cu[n + 1] - t0);
  const int tid = threadIdx.x;

  // ---- the chunk's rows; rows past its end are zero (and add no decay)
  for (int e = tid; e < kChunk * DK; e += kDiagThreads) {
    const int i = e / DK, ch = e % DK;
    const bool in = i < len;
    const size_t idx = ((size_t)(t0 + i) * H + h) * DK + ch;
    sm.K[i][ch] = in ? to_f32(k[idx]) : 0.f;
    sm.Q[i][ch] = in ? to_f32(q[idx]) : 0.f;
    sm.G[i][ch] = in ? g[idx] : 0.f;
  }
  __syncthreads();
  // ---- G: inclusive prefix over the chunk's tokens, per channel
  if (tid < DK) {
    float acc = 0.f;
    for (int i = 0; i < kChunk; ++i) {
      acc += sm.G[i][tid];
      sm.G[i][tid] = acc;
    }
  }
  // ---- b and the readout factor per token
  if (tid < kChunk) {
    const int i = tid;
    float kk = 0.f, qq = 0.f;
    for (int ch = 0; ch < DK; ++ch) {
      kk += sm.K[i][ch] * sm.K[i][ch];
      qq += sm.Q[i][ch] * sm.Q[i][ch];
    }
    float bi = 0.f;
    if (i < len) {
      const size_t th = (size_t)(t0 + i) * H + h;
      const float t_abs = (float)(t0 + i - ts + 1 + (opts.pos_offset ? opts.pos_offset[n] : 0));
      bi = write_coef(opts.beta_mode, eta[th], kk + eps, t_abs);
    }
    sm.b[i] = bi;
    sm.rq[i] = opts.normalize_q ? (qq > 0.f ? 1.f / sqrtf(qq) : 0.f) : 1.f;
  }
  __syncthreads();

  // ---- decayed tiles and the state decay exp(G_last) (row 63 carries G_last)
  const size_t tile0 = (size_t)task * kChunk * DK;
  for (int e = tid; e < kChunk * DK; e += kDiagThreads) {
    const int i = e / DK, ch = e % DK;
    const float Gi = sm.G[i][ch], Gl = sm.G[kChunk - 1][ch];
    const float ei = __expf(Gi);
    put(KG_out, tile0 + e, sm.K[i][ch] * ei);
    put(QG_out, tile0 + e, sm.Q[i][ch] * ei);
    put(KD_out, tile0 + e, sm.K[i][ch] * __expf(Gl - Gi));
  }
  for (int ch = tid; ch < DK; ch += kDiagThreads)
    GC_out[(size_t)task * DK + ch] = __expf(sm.G[kChunk - 1][ch]);

  // ---- A (strictly lower) and P (lower): lane tid owns rows 4 bi .. + 3, columns
  //      4 bj .. + 3 of both
  {
    const int bi = tid >> 4, bj = tid & 15;
    float a[4][4] = {}, p[4][4] = {};
    if (bj <= bi) {
      for (int ch = 0; ch < DK; ++ch) {
        float gi[4], ki[4], qi[4], gj[4], kj[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          gi[r] = sm.G[4 * bi + r][ch];
          ki[r] = sm.K[4 * bi + r][ch];
          qi[r] = sm.Q[4 * bi + r][ch];
          gj[r] = sm.G[4 * bj + r][ch];
          kj[r] = sm.K[4 * bj + r][ch];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int i = 4 * bi + r, j = 4 * bj + s;
            if (j <= i) {
              const float e = __expf(gi[r] - gj[s]) * kj[s];
              p[r][s] += qi[r] * e;
              if (j < i) a[r][s] += ki[r] * e;
            }
          }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sm.A[4 * bi + r][4 * bj + s] = a[r][s];
        sm.P[4 * bi + r][4 * bj + s] = p[r][s] * sm.rq[4 * bi + r];
      }
  }
  __syncthreads();

  // ---- X = (I + Diag(b) A)^{-1}, one column per lane, by forward substitution
  if (tid < kChunk) {
    const int j = tid;
    for (int i = 0; i < kChunk; ++i) {
      float x = (i == j) ? 1.f : 0.f;
      if (i > j) {
        float acc = 0.f;
        for (int l = j; l < i; ++l) acc += sm.A[i][l] * sm.X[l][j];
        x = -sm.b[i] * acc;
      }
      sm.X[i][j] = x;
    }
  }
  __syncthreads();

  // ---- T = X Diag(b) and P, as their ten 16 x 16 blocks on and below the diagonal (tpb_off
  //      layout), in element order of the packed blocks
  const size_t tp0 = (size_t)task * (kChunk * kChunk);
  for (int e = tid; e < 10 * 256; e += kDiagThreads) {
    const int blk = e >> 8, w = e & 255;
    const int I = blk >= 6 ? 3 : blk >= 3 ? 2 : blk >= 1 ? 1 : 0, J = blk - I * (I + 1) / 2;
    const int i = 16 * I + (w >> 4), j = 16 * J + (w & 15);
    const bool low = j <= i;
    put(T_out, tp0 + e, low ? sm.X[i][j] * sm.b[j] : 0.f);
    put(P_out, tp0 + e, low ? sm.P[i][j] : 0.f);
  }
  // ---- decays for the scan: unit gam and dec (the decay sits in Kg, Qg, Kd), the readout
  //      factor as gamO
  if (tid < kChunk) {
    const size_t gd0 = (size_t)task * kGDFloats;
    GD_out[gd0 + tid] = 1.f;
    GD_out[gd0 + kChunk + tid] = 1.f;
    GD_out[gd0 + 2 * kChunk + tid] = sm.rq[tid];
  }
}

template <typename Tin, int DK>
static hipError_t launch_prep_diag_t(const void *q, const void *k, const float *g,
                                     const float *eta, float eps, const CoefOpts &opts,
                                     SeqTables t, int32_t n_seq, int64_t n_chunks_ub, int32_t H,
                                     const DiagTiles &dt, void *T_out, void *P_out,
                                     float *GD_out, hipStream_t stream) {
  const size_t smem = sizeof(DiagSmem<DK>);
  static bool attr_set = false;  // benign race: every thread sets the same value
  if (!attr_set) {
    hipError_t e =
        hipFuncSetAttribute(reinterpret_cast<const void *>(&kla_prep_diag_kernel<Tin, DK>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = n_chunks_ub * H;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((kla_prep_diag_kernel<Tin, DK>), dim3((unsigned)blocks), dim3(kDiagThreads),
                     smem, stream, static_cast<const Tin *>(q), static_cast<const Tin *>(k), g,
                     eta, eps, opts, t, n_seq, H, static_cast<Tin *>(T_out),
                     static_cast<Tin *>(P_out), GD_out,
                     static_cast<Tin *>(const_cast<void *>(dt.kg)),
                     static_cast<Tin *>(const_cast<void *>(dt.qg)),
                     static_cast<Tin *>(const_cast<void *>(dt.kd)), const_cast<float *>(dt.gc));
  return hipGetLastError();
}

hipError_t launch_prep_diag(Dtype dt, int d_k, const void *q, const void *k, const float *g,
                            const float *eta, float eps, const CoefOpts &opts, SeqTables t,
                            int32_t n_seq, int64_t n_chunks_ub, int32_t H, const DiagTiles &tiles,
                            void *T_out, void *P_out, float *GD_out, hipStream_t stream) {
  if (dt == Dtype::BF16) {
    if (d_k == 128)
      return launch_prep_diag_t<__bf16, 128>(q, k, g, eta, eps, opts, t, n_seq, n_chunks_ub, H,
                                             tiles, T_out, P_out, GD_out, stream);
    return launch_prep_diag_t<__bf16, 64>(q, k, g, eta, eps, opts, t, n_seq, n_chunks_ub, H,
                                          tiles, T_out, P_out, GD_out, stream);
  }
  if (d_k == 128)
    return launch_prep_diag_t<float, 128>(q, k, g, eta, eps, opts, t, n_seq, n_chunks_ub, H,
                                          tiles, T_out, P_out, GD_out, stream);
  return launch_prep_diag_t<float, 64>(q, k, g, eta, eps, opts, t, n_seq, n_chunks_ub, H, tiles,
                                       T_out, P_out, GD_out, stream);
}

}  // namespace kla
