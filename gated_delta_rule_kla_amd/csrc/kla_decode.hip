// kla_decode.hip -- single-token decode step, one HBM read and one HBM write of the state.
//
// Paper "Kaczmarz Linear Attention" (arXiv 2605.08587), Algorithm 1 tokenwise
// panel with the coefficient of Eq. (3).  Substituting the write into the readout
// gives o = a q S + b (q . k) e, so with
//   r = k S,  p = q S  (column reductions over d_k of the OLD state)
//   e = v - a r,  b = eta / (||k||^2 + eps)
//   S' = a S + b k^T e,   o = a p + b (q . k) e
// the state is streamed through registers exactly once.  The coefficient variants and the
// readout divided by ||q|| (see write_coef) only change b and scale o.  The columns of S are
// independent given k, q and the scalars, so a (sequence, head) is split over NS workgroups of
// NT lanes, each taking d_v / NS columns; each lane owns float4 column groups of a few state
// rows, so every load and store is a coalesced 16-byte access.
//
// Diagonal gating (GDIAG; paper Appendix B.5): the decay is Diag(a) with a_i = exp(g_i) per
// key channel, so the forgotten state is Diag(a) S and, with the same substitution,
//   r = (k o a) S,  p = (q o a) S,  e = v - r,  S' = Diag(a) S + b k^T e,  o = p + b (q . k) e.
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {

template <typename Tin, int DK, int DV, int NS, int NT, bool GDIAG>
__global__ __launch_bounds__(NT) void kla_decode_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ eta, float eps, CoefOpts opts,
    int H, const float *S, Tin *__restrict__ o, float *S_new) {
  constexpr int NC4 = DV / NS / 4;  // float4 column groups of this workgroup per state row
  constexpr int RS4 = DV / 4;       // float4 column groups per state row
  constexpr int RPP = NT / NC4;     // state rows per pass
  constexpr int NP = DK / RPP;      // passes (float4 registers per lane)
  constexpr int NW = NT / 64;       // wavefronts
  static_assert(NC4 >= 1 && RPP * NC4 == NT && NP * RPP == DK && NT >= DK, "decode tiling");
  __shared__ float sk[DK], sq[DK];
  __shared__ float sa[GDIAG ? DK : 1], ska[GDIAG ? DK : 1], sqa[GDIAG ? DK : 1];
  __shared__ f32x4 red_r[RPP][NC4], red_p[RPP][NC4];
  __shared__ float sred[3][NW];

  const size_t bh = blockIdx.x / NS;
  const int col0 = (blockIdx.x % NS) * NC4;  // first float4 column group of this workgroup
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int c4 = tid % NC4, rg = tid / NC4;

  // issue the state loads first: they are the only large traffic
  const f32x4 *Sp = reinterpret_cast<const f32x4 *>(S + bh * DK * DV) + col0;
  f32x4 s[NP];
#pragma unroll
  for (int pp = 0; pp < NP; ++pp)
    s[pp] = __builtin_nontemporal_load(&Sp[(pp * RPP + rg) * RS4 + c4]);

  float kf = 0.f, qf = 0.f;
  if (tid < DK) {
    kf = to_f32(k[bh * DK + tid]);
    qf = to_f32(q[bh * DK + tid]);
    sk[tid] = kf;
    sq[tid] = qf;
    if constexpr (GDIAG) {
      const float ai = __expf(g[bh * DK + tid]);
      sa[tid] = ai;
      ska[tid] = kf * ai;
      sqa[tid] = qf * ai;
    }
  }
  const float kk = wave_sum(kf * kf), qk = wave_sum(qf * kf);
  const float qq = opts.normalize_q ? wave_sum(qf * qf) : 0.f;
  if (lane == 0) { sred[0][wid] = kk; sred[1][wid] = qk; sred[2][wid] = qq; }
  __syncthreads();

  f32x4 r = zero4(), p = zero4();
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const int row = pp * RPP + rg;
    if constexpr (GDIAG) {
      r += ska[row] * s[pp];
      p += sqa[row] * s[pp];
    } else {
      r += sk[row] * s[pp];
      p += sq[row] * s[pp];
    }
  }
  red_r[rg][c4] = r;
  red_p[rg][c4] = p;
  __syncthreads();
  f32x4 rt = zero4(), pt = zero4();
#pragma unroll
  for (int gg = 0; gg < RPP; ++gg) { rt += red_r[gg][c4]; pt += red_p[gg][c4]; }

  float kk_all = 0.f, qk_all = 0.f, qq_all = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    kk_all += sred[0][w];
    qk_all += sred[1][w];
    qq_all += sred[2][w];
  }
  const float a = GDIAG ? 1.f : __expf(g[bh]);  // the diagonal decay is inside r, p and sa
  const float den = kk_all + eps;
  const int brow = (int)(bh / H);
  const float t_abs = (float)(1 + (opts.pos_offset ? opts.pos_offset[brow] : 0));
  const float beta = write_coef(opts.beta_mode, eta[bh], den, t_abs);
  // readout factor: 1 / ||q|| under the normalised readout (0 for a zero query), else 1
  const float rq = opts.normalize_q ? (qq_all > 0.f ? 1.f / sqrtf(qq_all) : 0.f) : 1.f;
  f32x4 e;
  const int vc = 4 * (col0 + c4);
#pragma unroll
  for (int j = 0; j < 4; ++j) e[j] = to_f32(v[bh * DV + vc + j]) - a * rt[j];
  if (rg == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[bh * DV + vc + j] = from_f32<Tin>((a * pt[j] + beta * qk_all * e[j]) * rq);
  }
  f32x4 *Sn = reinterpret_cast<f32x4 *>(S_new + bh * DK * DV) + col0;
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const int row = pp * RPP + rg;
    const float bk = beta * sk[row];
    const float ar = GDIAG ? sa[row] : a;
    __builtin_nontemporal_store(ar * s[pp] + bk * e, &Sn[row * RS4 + c4]);
  }
}

// Launch shape.  Where d_k = 128 and d_v >= 128: four 128-lane workgroups per (sequence,
// head) item, each taking a quarter of the columns (128-byte row pieces).  Elsewhere, by the
// number of items: below kDecodeSplitBelow two 128-lane workgroups per item, so that there are
// enough workgroups to keep HBM busy, from there on one 512-lane workgroup per item.  Measured
// at d = 128: 256 x 16 items, four 5.80 TB/s against two 5.64 (5.73 against 5.54 under
// diagonal gating); 512 x 16 and 1024 x 16 items, four 5.74-5.81 against one 5.67-5.74 (two of
// 256 lanes: 5.56-5.66).  Four are slower at d_k = 64 and collapse at d_v = 64 (64-byte pieces).
constexpr int64_t kDecodeSplitBelow = 5120;

template <typename Tin, int DK, int DV, int NS, int NT>
static void launch_decode_shape(int64_t units, const Tin *qt, const Tin *kt, const Tin *vt,
                                const float *g, const float *eta, float eps,
                                const CoefOpts &opts, int32_t H, const float *S, Tin *ot,
                                float *S_new, hipStream_t stream) {
  if (opts.diag_gate)
    hipLaunchKernelGGL((kla_decode_kernel<Tin, DK, DV, NS, NT, true>), dim3((unsigned)units),
                       dim3(NT), 0, stream, qt, kt, vt, g, eta, eps, opts, H, S, ot, S_new);
  else
    hipLaunchKernelGGL((kla_decode_kernel<Tin, DK, DV, NS, NT, false>), dim3((unsigned)units),
                       dim3(NT), 0, stream, qt, kt, vt, g, eta, eps, opts, H, S, ot, S_new);
}

template <typename Tin, int DK, int DV>
static hipError_t launch_decode_t(const void *q, const void *k, const void *v, const float *g,
                                  const float *eta, float eps, const CoefOpts &opts,
                                  const float *S, void *o, float *S_new, int32_t batch,
                                  int32_t H, hipStream_t stream) {
  const int64_t items = (int64_t)batch * H;
  if (items <= 0) return hipSuccess;
  if (items > 0x7fffffff) return hipErrorInvalidValue;  // grid size of the widest shape
  const Tin *qt = static_cast<const Tin *>(q), *kt = static_cast<const Tin *>(k);
  const Tin *vt = static_cast<const Tin *>(v);
  Tin *ot = static_cast<Tin *>(o);
  if constexpr (DK == 128 && DV >= 128) {
    if (4 * items <= 0x7fffffff) {
      launch_decode_shape<Tin, DK, DV, 4, 128>(4 * items, qt, kt, vt, g, eta, eps, opts, H, S,
                                               ot, S_new, stream);
      return hipGetLastError();
    }
  }
  if (items >= kDecodeSplitBelow)
    launch_decode_shape<Tin, DK, DV, 1, 512>(items, qt, kt, vt, g, eta, eps, opts, H, S, ot,
                                             S_new, stream);
  else
    launch_decode_shape<Tin, DK, DV, 2, 128>(2 * items, qt, kt, vt, g, eta, eps, opts, H, S, ot,
                                             S_new, stream);
  return hipGetLastError();
}

template <typename Tin>
static hipError_t launch_decode_dt(int d_k, int d_v, const void *q, const void *k, const void *v,
                                   const float *g, const float *eta, float eps,
                                   const CoefOpts &opts, const float *S, void *o, float *S_new,
                                   int32_t batch, int32_t H, hipStream_t stream) {
#define KLA_DEC(DK_, DV_)                                                                  \
  if (d_k == DK_ && d_v == DV_)                                                            \
    return launch_decode_t<Tin, DK_, DV_>(q, k, v, g, eta, eps, opts, S, o, S_new, batch, H, \
                                          stream);
  KLA_DEC(64, 64)
  KLA_DEC(64, 128)
  KLA_DEC(64, 256)
  KLA_DEC(128, 64)
  KLA_DEC(128, 128)
  KLA_DEC(128, 256)
#undef KLA_DEC
  return hipErrorInvalidValue;
}

hipError_t launch_decode(Dtype dt, int d_k, int d_v, const void *q, const void *k, const void *v,
                         const float *g, const float *eta, float eps, const CoefOpts &opts,
                         const float *S, void *o, float *S_new, int32_t batch, int32_t H,
                         hipStream_t stream) {
  if (dt == Dtype::BF16)
    return launch_decode_dt<__bf16>(d_k, d_v, q, k, v, g, eta, eps, opts, S, o, S_new, batch, H,
                                    stream);
  return launch_decode_dt<float>(d_k, d_v, q, k, v, g, eta, eps, opts, S, o, S_new, batch, H,
                                 stream);
}

}  // namespace kla
