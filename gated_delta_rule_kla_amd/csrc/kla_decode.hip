// kla_decode.hip -- single-token decode step, one HBM read and one HBM write of the state.
//
// Paper "Kaczmarz Linear Attention" (arXiv 2605.08587), Algorithm 1 tokenwise
// panel (steps 2-6) with the coefficient of Eq. (3).  Substituting step 5 into
// step 6 gives o = a q S + b (q . k) e, so with
//   r = k S,  p = q S  (column reductions over d_k of the OLD state)
//   e = v - a r,  b = eta / (||k||^2 + eps)
//   S' = a S + b k^T e,   o = a p + b (q . k) e
// the state is streamed through registers exactly once.  The coefficient variants and the
// readout divided by ||q|| (see write_coef) only change b and scale o.  One workgroup
// (256 lanes) per (sequence, head); each lane owns float4 column groups of a
// few state rows, so every load and store is a coalesced 16-byte access.
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {

template <typename Tin, int DK, int DV>
__global__ __launch_bounds__(256) void kla_decode_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ eta, float eps, CoefOpts opts,
    int H, const float *S, Tin *__restrict__ o, float *S_new) {
  constexpr int NC4 = DV / 4;      // float4 column groups per state row
  constexpr int RPP = 256 / NC4;   // state rows per pass
  constexpr int NP = DK / RPP;     // passes (float4 registers per lane)
  __shared__ float sk[DK], sq[DK];
  __shared__ f32x4 red_r[RPP][NC4], red_p[RPP][NC4];
  __shared__ float sred[3][4];

  const size_t bh = blockIdx.x;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int c4 = tid % NC4, rg = tid / NC4;

  // issue the state loads first: they are the only large traffic
  const f32x4 *Sp = reinterpret_cast<const f32x4 *>(S + bh * DK * DV);
  f32x4 s[NP];
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) s[pp] = __builtin_nontemporal_load(&Sp[(pp * RPP + rg) * NC4 + c4]);

  float kf = 0.f, qf = 0.f;
  if (tid < DK) {
    kf = to_f32(k[bh * DK + tid]);
    qf = to_f32(q[bh * DK + tid]);
    sk[tid] = kf;
    sq[tid] = qf;
  }
  const float kk = wave_sum(kf * kf), qk = wave_sum(qf * kf);
  const float qq = opts.normalize_q ? wave_sum(qf * qf) : 0.f;
  if (lane == 0) { sred[0][wid] = kk; sred[1][wid] = qk; sred[2][wid] = qq; }
  __syncthreads();

  f32x4 r = zero4(), p = zero4();
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const int row = pp * RPP + rg;
    r += sk[row] * s[pp];
    p += sq[row] * s[pp];
  }
  red_r[rg][c4] = r;
  red_p[rg][c4] = p;
  __syncthreads();
  f32x4 rt = zero4(), pt = zero4();
#pragma unroll
  for (int gg = 0; gg < RPP; ++gg) { rt += red_r[gg][c4]; pt += red_p[gg][c4]; }

  const float kk_all = sred[0][0] + sred[0][1] + sred[0][2] + sred[0][3];
  const float qk_all = sred[1][0] + sred[1][1] + sred[1][2] + sred[1][3];
  const float qq_all = sred[2][0] + sred[2][1] + sred[2][2] + sred[2][3];
  const float a = __expf(g[bh]);
  const float den = kk_all + eps;
  const int brow = (int)(bh / H);
  const float t_abs = (float)(1 + (opts.pos_offset ? opts.pos_offset[brow] : 0));
  const float beta = write_coef(opts.beta_mode, eta[bh], den, t_abs);
  // readout factor: 1 / ||q|| under the normalised readout (0 for a zero query), else 1
  const float rq = opts.normalize_q ? (qq_all > 0.f ? 1.f / sqrtf(qq_all) : 0.f) : 1.f;
  f32x4 e;
#pragma unroll
  for (int j = 0; j < 4; ++j) e[j] = to_f32(v[bh * DV + 4 * c4 + j]) - a * rt[j];
  if (rg == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[bh * DV + 4 * c4 + j] = from_f32<Tin>((a * pt[j] + beta * qk_all * e[j]) * rq);
  }
  f32x4 *Sn = reinterpret_cast<f32x4 *>(S_new + bh * DK * DV);
#pragma unroll
  for (int pp = 0; pp < NP; ++pp) {
    const int row = pp * RPP + rg;
    const float bk = beta * sk[row];
    __builtin_nontemporal_store(a * s[pp] + bk * e, &Sn[row * NC4 + c4]);
  }
}

template <typename Tin, int DK, int DV>
static hipError_t launch_decode_t(const void *q, const void *k, const void *v, const float *g,
                                  const float *eta, float eps, const CoefOpts &opts,
                                  const float *S, void *o, float *S_new, int32_t batch,
                                  int32_t H, hipStream_t stream) {
  const int64_t blocks = (int64_t)batch * H;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((kla_decode_kernel<Tin, DK, DV>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const Tin *>(q), static_cast<const Tin *>(k),
                     static_cast<const Tin *>(v), g, eta, eps, opts, H, S, static_cast<Tin *>(o),
                     S_new);
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
