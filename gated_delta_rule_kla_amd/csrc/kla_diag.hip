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
// One 1024-lane workgroup per (chunk, head), everything staged in LDS in fp32.  Every decay
// factor is an exponential of a non-positive difference of log-decays (G_i - G_j with j <= i,
// G_last - G_j, or the tile-anchored pieces of the A and P sums), so nothing overflows
// whatever the decay.  X = (I + Diag(b) A)^{-1} comes from kla_inverse.h.
#include "kla_device.h"
#include "kla_inverse.h"
#include "kla_launch.h"

namespace kla {

namespace {

constexpr int kDiagThreads = 1024;

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
  // rows of DK + 4 floats: 16-byte aligned for the pair loops' float4 reads, and offset by
  // one bank group from row to row
  alignas(16) float K[kChunk][DK + 4];
  alignas(16) float Q[kChunk][DK + 4];
  alignas(16) float G[kChunk][DK + 4];
  float A[kChunk][kChunk + 1], P[kChunk][kChunk + 1], X[kChunk][kChunk + 1];
  float b[kChunk], rq[kChunk];
};

// four consecutive values, one 16-byte (fp32) or 8-byte (bf16) store
__device__ __forceinline__ void put4(float *dst, const f32x4 &x) {
  *reinterpret_cast<f32x4 *>(dst) = x;
}
__device__ __forceinline__ void put4(__bf16 *dst, const f32x4 &x) {
  bf16x4 b;
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = from_f32<__bf16>(x[i]);
  *reinterpret_cast<bf16x4 *>(dst) = b;
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

  // ---- the chunk's rows; rows past its end are zero (and add no decay).  Lane tid takes 8
  //      consecutive channels of one row: one 16-byte load of k and of q (bf16), 32 bytes of g
  {
    const int e0 = tid * 8, i = e0 / DK, ch = e0 % DK;
    if (i < kChunk) {
      float kv[8], qv[8], gv[8];
      if (i < len) {
        const size_t idx = ((size_t)(t0 + i) * H + h) * DK + ch;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kv[e] = to_f32(k[idx + e]);
          qv[e] = to_f32(q[idx + e]);
          gv[e] = g[idx + e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kv[e] = qv[e] = gv[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sm.K[i][ch + e] = kv[e];
        sm.Q[i][ch + e] = qv[e];
        sm.G[i][ch + e] = gv[e];
      }
    }
  }
  __syncthreads();
  // ---- G: inclusive prefix over the chunk's tokens, per channel (the column in registers)
  if (tid < DK) {
    float col[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) col[i] = sm.G[i][tid];
#pragma unroll
    for (int i = 1; i < kChunk; ++i) col[i] += col[i - 1];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) sm.G[i][tid] = col[i];
  }
  // ---- b and the readout factor per token: 16 lanes a row, 8 channels at a time
  {
    const int i = tid >> 4, part = tid & 15;
    float kk = 0.f, qq = 0.f;
    if (i < kChunk) {
      for (int ch = 8 * part; ch < DK; ch += 128) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kk += sm.K[i][ch + e] * sm.K[i][ch + e];
          qq += sm.Q[i][ch + e] * sm.Q[i][ch + e];
        }
      }
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
      kk += __shfl_xor(kk, off, 16);
      qq += __shfl_xor(qq, off, 16);
    }
    if (i < kChunk && part == 0) {
      float bi = 0.f;
      if (i < len) {
        const size_t th = (size_t)(t0 + i) * H + h;
        const float t_abs =
            (float)(t0 + i - ts + 1 + (opts.pos_offset ? opts.pos_offset[n] : 0));
        bi = write_coef(opts.beta_mode, eta[th], kk + eps, t_abs);
      }
      sm.b[i] = bi;
      sm.rq[i] = opts.normalize_q ? (qq > 0.f ? 1.f / sqrtf(qq) : 0.f) : 1.f;
    }
  }
  __syncthreads();

  // ---- decayed tiles and the state decay exp(G_last) (row 63 carries G_last)
  //      four consecutive channels per lane and step: 16-byte LDS reads, 8- or 16-byte stores
  const size_t tile0 = (size_t)task * kChunk * DK;
  for (int e = 4 * tid; e < kChunk * DK; e += 4 * kDiagThreads) {
    const int i = e / DK, ch = e % DK;
    const f32x4 Gi = *reinterpret_cast<const f32x4 *>(&sm.G[i][ch]);
    const f32x4 Gl = *reinterpret_cast<const f32x4 *>(&sm.G[kChunk - 1][ch]);
    const f32x4 kv = *reinterpret_cast<const f32x4 *>(&sm.K[i][ch]);
    const f32x4 qv = *reinterpret_cast<const f32x4 *>(&sm.Q[i][ch]);
    f32x4 kg, qg, kd;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float ei = __expf(Gi[x]);
      kg[x] = kv[x] * ei;
      qg[x] = qv[x] * ei;
      kd[x] = kv[x] * __expf(Gl[x] - Gi[x]);
    }
    put4(KG_out + tile0 + e, kg);
    put4(QG_out + tile0 + e, qg);
    put4(KD_out + tile0 + e, kd);
  }
  for (int ch = tid; ch < DK; ch += kDiagThreads)
    GC_out[(size_t)task * DK + ch] = __expf(sm.G[kChunk - 1][ch]);

  // ---- A (strictly lower) and P (lower) in 4 x 4 tiles of (row, column) pairs.  With
  //      l_i = G_i - G_{4 floor(i/4)} (the log-decay since the first row of row i's tile),
  //      a pair in tiles bi > bj factors through the tiles' anchor rows,
  //        exp(G_i - G_j) = exp(l_i) exp(G_{4 bi} - G_{4 bj + 3}) exp(l_{4 bj + 3} - l_j),
  //      three factors that are each at most 1, so the off-diagonal tiles need one exponential
  //      per channel instead of sixteen: with K o exp(l), Q o exp(l) and K o exp(l_last - l)
  //      staged, they are plain sums of products.  The diagonal tiles take exp(l_i - l_j)
  //      directly.
  constexpr int EPL = kChunk * DK / kDiagThreads;  // elements per lane in the elementwise steps
  float *GA = &sm.X[0][0], *GB = GA + 16 * DK;     // G of each tile's first and last row (X is
                                                   // free until the substitution)
  for (int e = tid; e < 16 * DK; e += kDiagThreads) {
    const int t = e / DK, ch = e % DK;
    GA[e] = sm.G[4 * t][ch];
    GB[e] = sm.G[4 * t + 3][ch];
  }
  {
    const int e0 = tid * EPL, i = e0 / DK, ch = e0 % DK;
    float l[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) l[e] = sm.G[i][ch + e] - sm.G[i & ~3][ch + e];
    __syncthreads();  // every read of G (the decayed tiles, the anchors) is done
#pragma unroll
    for (int e = 0; e < EPL; ++e) sm.G[i][ch + e] = l[e];
  }
  __syncthreads();
  // diagonal tiles: wavefront w takes tile w, each lane DK / 64 channels, then wavefront sums
  {
    const int wid = tid >> 6, lane = tid & 63;
    constexpr int CPL = DK / kWave;
    const int t = wid;
    float ad[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, pd[10] = {};
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
      const int ch = lane * CPL + cc;
      float lg[4], kv[4], qv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        lg[r] = sm.G[4 * t + r][ch];
        kv[r] = sm.K[4 * t + r][ch];
        qv[r] = sm.Q[4 * t + r][ch];
      }
      int ia = 0, ip = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c2 = 0; c2 <= r; ++c2) {
          const float x = __expf(lg[r] - lg[c2]) * kv[c2];
          pd[ip++] += qv[r] * x;
          if (c2 < r) ad[ia++] += kv[r] * x;
        }
    }
#pragma unroll
    for (int x = 0; x < 10; ++x) pd[x] = wave_sum(pd[x]);
#pragma unroll
    for (int x = 0; x < 6; ++x) ad[x] = wave_sum(ad[x]);
    if (lane < 16) {
      const int r = lane >> 2, c2 = lane & 3;
      const int ip = r * (r + 1) / 2 + c2, ia = r * (r - 1) / 2 + c2;
      float pv = 0.f, av = 0.f;
#pragma unroll
      for (int x = 0; x < 10; ++x) pv = x == ip && c2 <= r ? pd[x] : pv;
#pragma unroll
      for (int x = 0; x < 6; ++x) av = x == ia && c2 < r ? ad[x] : av;
      sm.P[4 * t + r][4 * t + c2] = pv * sm.rq[4 * t + r];
      sm.A[4 * t + r][4 * t + c2] = av;
    }
  }
  // K -> K o exp(l), Q -> Q o exp(l), l -> K o exp(l_last - l) (l_last: the tile's last row)
  {
    const int e0 = tid * EPL, i = e0 / DK, ch = e0 % DK;
    float kl[EPL], ql[EPL], kr[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float lv = sm.G[i][ch + e], k0 = sm.K[i][ch + e];
      const float el = __expf(lv);
      kl[e] = k0 * el;
      ql[e] = sm.Q[i][ch + e] * el;
      kr[e] = k0 * __expf(sm.G[i | 3][ch + e] - lv);
    }
    __syncthreads();  // the diagonal tiles' reads are done
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      sm.K[i][ch + e] = kl[e];
      sm.Q[i][ch + e] = ql[e];
      sm.G[i][ch + e] = kr[e];
    }
  }
  __syncthreads();
  // off-diagonal tiles (bj < bi): 120 tiles x 8 channel groups on lanes 0..959
  if (tid < 120 * 8) {
    const int t = tid >> 3, g8 = tid & 7;
    const int bi = (int)((1.f + sqrtf(1.f + 8.f * (float)t)) * 0.5f);  // t = bi (bi - 1) / 2 + bj
    const int bj = t - bi * (bi - 1) / 2;
    constexpr int CPG = DK / 8;
    float a[4][4] = {}, p[4][4] = {};
#pragma unroll 1
    for (int c4 = g8 * CPG; c4 < (g8 + 1) * CPG; c4 += 4) {
      const f32x4 ga = *reinterpret_cast<const f32x4 *>(GA + bi * DK + c4);
      const f32x4 gb = *reinterpret_cast<const f32x4 *>(GB + bj * DK + c4);
      f32x4 d;
#pragma unroll
      for (int e = 0; e < 4; ++e) d[e] = __expf(ga[e] - gb[e]);
      f32x4 kl[4], ql[4], kr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        kl[r] = *reinterpret_cast<const f32x4 *>(&sm.K[4 * bi + r][c4]);
        ql[r] = *reinterpret_cast<const f32x4 *>(&sm.Q[4 * bi + r][c4]);
        kr[r] = *reinterpret_cast<const f32x4 *>(&sm.G[4 * bj + r][c4]) * d;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c2 = 0; c2 < 4; ++c2)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[r][c2] += kl[r][e] * kr[c2][e];
            p[r][c2] += ql[r][e] * kr[c2][e];
          }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c2 = 0; c2 < 4; ++c2)
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) {
          a[r][c2] += __shfl_xor(a[r][c2], off, 8);
          p[r][c2] += __shfl_xor(p[r][c2], off, 8);
        }
    if (g8 == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c2 = 0; c2 < 4; ++c2) {
          sm.A[4 * bi + r][4 * bj + c2] = a[r][c2];
          sm.P[4 * bi + r][4 * bj + c2] = p[r][c2] * sm.rq[4 * bi + r];
        }
    }
  }
  __syncthreads();

  // ---- X = (I + Diag(b) A)^{-1} by 16 x 16 blocks (the staged key tile is free scratch now)
  blocked_inverse<kDiagThreads, kChunk + 1, kChunk + 1>(&sm.A[0][0], sm.b, &sm.X[0][0],
                                                        &sm.K[0][0], tid);

  // ---- T = X Diag(b) and P, as their ten 16 x 16 blocks on and below the diagonal (tpb_off
  //      layout), in element order of the packed blocks
  const size_t tp0 = (size_t)task * kTpbElems;
  for (int e = 4 * tid; e < 10 * 256; e += 4 * kDiagThreads) {  // 4 columns of a row per lane
    const int blk = e >> 8, w = e & 255;
    const int I = blk >= 6 ? 3 : blk >= 3 ? 2 : blk >= 1 ? 1 : 0, J = blk - I * (I + 1) / 2;
    const int i = 16 * I + (w >> 4), j0 = 16 * J + (w & 15);
    f32x4 tv, pv;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const bool low = j0 + x <= i;
      tv[x] = low ? sm.X[i][j0 + x] * sm.b[j0 + x] : 0.f;
      pv[x] = low ? sm.P[i][j0 + x] : 0.f;
    }
    put4(T_out + tp0 + e, tv);
    put4(P_out + tp0 + e, pv);
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
