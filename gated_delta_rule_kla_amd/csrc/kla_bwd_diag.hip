// kla_bwd_diag.hip -- the per-chunk gradients of the prefill under diagonal gating.
//
// Paper "Kaczmarz Linear Attention" (arXiv 2605.08587), Appendix B.5: the decay is
// Diag(alpha_t), one factor per key channel.  Per chunk of one (sequence, head), with S the
// chunk's incoming state, G the chunk-local cumulative log-decay per channel (64 x d_k),
// Gamma_ijc = exp(G_ic - G_jc), E = exp(G), D = exp(G_last - G) (elementwise, 64 x d_k),
// q^_i = rq_i q_i (rq_i = 1 / ||q_i|| under the normalised readout of section 3.3, else 1) and
// the decayed tiles Kg = K o E, Q^g = Q^ o E, Kd = K o D that the forward pass used:
//   A_ij = sum_c k_ic k_jc Gamma_ijc (j < i),  P^_ij = sum_c q^_ic k_jc Gamma_ijc (j <= i),
//   X = (I + Diag(b) A)^{-1},  T = X Diag(b),
//   R = V - Kg S,  U = T R,  O = Q^g S + P^ U,  S' = Diag(exp(G_last)) S + Kd^T U.
// The adjoint scan hands over dU, dR (as dV) and dS' per chunk; this kernel forms the rest by
// reverse-mode differentiation of the lines above:
//   qa = dO S^T, ka = dR S^T, kb = U dS'^T (64 x d_k),  sc_c = sum_v S_cv dS'_cv,
//   dP^ = lower(dO U^T),  dT = lower(dU R^T),  dX = dT Diag(b),
//   dL = -strict_lower(X^T dX X^T),  dA = Diag(b) dL,  db = colsum(dT o X) + rowsum(dL o A),
//   F1_ic = sum_j dA_ij k_jc Gamma_ijc,  H1_ic = sum_j dP^_ij k_jc Gamma_ijc,
//   Z_jc  = sum_i Gamma_ijc (dA_ij k_ic + dP^_ij q^_ic),
//   dq^ = E o qa + H1,
//   dk  = -E o ka + D o kb + F1 + Z - Diag(2 b db / den) K   (the last term where b depends on
//         ||k||^2: every coefficient mode but the gated rule's),
//   dG  = q^ o E o qa - K o E o ka - K o D o kb + q^ o H1 + K o F1 - K o Z,
//   dG_last,c += exp(G_last,c) sc_c + sum_i k_ic D_ic kb_ic,
//   dg_t = sum of dG_i over the chunk's positions i >= t (per channel), deta = db (d b / d eta),
//   dq  = dq^ (plain readout) or rq (dq^ - q^ (q^ . dq^)) (normalised readout).
// The products F1, H1 and Z run on the bf16 matrix cores when, on every channel of the
// 16-channel output tile, every row's G lies within 2^64 of row 32's (log2 units): then
// Gamma_ijc = 2^(G_ic - G_32c) 2^(G_32c - G_jc) with both factors normal, the left one scaling
// the output rows and the right one the key / query operand.  Otherwise, and for fp32 inputs,
// each lane sums its outputs' terms directly with one exp2 per term (Gamma <= 1 on every
// term that is kept).
#include "kla_bwd_common.h"
#include "kla_chunk.h"

namespace kla {

namespace {

template <typename LT, int DK>
struct GradDiagSmem {
  static constexpr int LDL = ldl<LT>();
  static constexpr bool TR = sizeof(LT) == 2;
  static constexpr int LK = DK + (TR ? 8 : 4);  // row stride of the key and query tiles
  static constexpr int LG = kChunk + 8;          // row stride of the bf16 64 x 64 tiles
  static constexpr int LGG = DK + 4;             // row stride of the fp32 64 x d_k tiles
  static constexpr int NPART = kGradThreads / DK, RPP = kChunk / NPART;  // G prefix split
  LT K[kChunk][LK];  // Kg rows in the d_v loop, then the key rows
  float X[kChunk][LDC];
  union {
    struct {  // the loop over 32-column blocks of d_v
      LT S[DK][LDL], So[DK][LDL];
      LT R[kChunk][LDL], U[kChunk][LDL], dO[kChunk][LDL], dU[kChunk][LDL], dR[kChunk][LDL];
      LT Rb[TR ? kChunk : 1][TR ? LDL : 4];  // bf16: Diag(b) R
    } lp;
    struct {  // after it
      LT Q[kChunk][LK];          // query rows (not normalised)
      float GT[DK][kChunk + 4];  // G^T: per channel, G in log2 units down the rows
      // dP^ and dT (then W = dT Diag(b) X^T, then dA), adjacent: after the products they
      // hold dG ([64][LGG])
      float dP[kChunk][LDC], dT[kChunk][LDC];
      __bf16 dPb[TR ? kChunk : 1][TR ? LG : 8], dAb[TR ? kChunk : 1][TR ? LG : 8];
      float tot[NPART][DK];      // per-part totals of the G prefix, then of the dg suffix
    } pa;
  } u;
  float b[kChunk], den[kChunk], db[kChunk], db_deta[kChunk], rqn[kChunk];
  float qq[kChunk];            // squared query norms
  float qdot[2][kChunk];       // q^ . dq^, two partial sums
  float zr[4][kChunk];         // row sums of dL o A, one partial per 16-column tile
  float sc[DK];                // <S, dS'> per channel
  float kbs[4][DK];            // sum_i k D kb per channel, one partial per 16-row tile
  int span[DK];                // max_j |G_jc - G_32c| (log2 units, float bits)
};

}  // namespace

template <typename Tin, int DK>
__global__ __launch_bounds__(kGradThreads) void kla_bwd_grad_diag_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const Tin *__restrict__ dO, const float *__restrict__ g, const float *__restrict__ eta,
    float eps, CoefOpts opts, const Tin *__restrict__ KG, const Tin *__restrict__ Xp,
    const Tin *__restrict__ Ap, const Tin *__restrict__ SN, const Tin *__restrict__ dSo,
    const Tin *__restrict__ dUo, const Tin *__restrict__ dvp, Tin *__restrict__ dq,
    Tin *__restrict__ dk, float *__restrict__ dg, float *__restrict__ deta,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off, int n_seq, int H,
    int DV) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  using SMG = GradDiagSmem<Tin, DK>;
  SMG &sm = *reinterpret_cast<SMG *>(smem_raw);
  constexpr int LK = SMG::LK, LG = SMG::LG, LGG = SMG::LGG, LDL = SMG::LDL;
  constexpr bool TR = SMG::TR;
  constexpr int NPART = SMG::NPART, RPP = SMG::RPP;
  constexpr float kLog2e = 1.4426950408889634f;
  const int n_chunks = chunk_off[n_seq];
  const int task = blockIdx.x;  // chunk * H + head
  if (task >= n_chunks * H) return;
  const int c = task / H, h = task - c * H;
  int n = 0;
  {
    int lo = 0, hi = n_seq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (chunk_off[mid] <= c) lo = mid; else hi = mid - 1;
    }
    n = lo;
  }
  const int t0 = cu[n] + (c - chunk_off[n]) * kChunk;
  const int len = min(kChunk, cu[n + 1] - t0);
  const size_t tok = (size_t)t0 * H + h;
  const size_t ch = (size_t)task;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kq = lane >> 4;

  // ---- X (packed fp32 blocks), the key rows (their squared norms now; kept in registers
  //      for after the d_v loop), Kg for the loop, eta, and the first d_v block: all issued
  //      before any is waited for
  constexpr int kXPieces = kTpbElems / 4;
  constexpr int NM = DK / 32;  // 64 x DK tiles per wavefront: rows 16 (wid & 3), columns 16 tj
  const int mti = wid & 3;
  float eta_l = 0.f;
  if (wid == 0 && lane < len) eta_l = eta[tok + (size_t)lane * H];
  typename Raw4<Tin>::type xr[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int e = tid + kGradThreads * x;
    if (e < kXPieces)
      xr[x] = *reinterpret_cast<const typename Raw4<Tin>::type *>(Xp + ch * kTpbElems + 4 * e);
  }
  RegTile<Tin, kChunk, DK, kGradThreads> rkr, rkg, rq;
  rkr.load(k + tok * DK, (size_t)H * DK, len, tid);
  rkg.load(KG + ch * kChunk * DK, DK, kChunk, tid);
  const Tin *Sb = SN + ch * DK * (size_t)DV;
  const Tin *Sob = dSo + ch * DK * (size_t)DV;
  const Tin *dUb = dUo + ch * kChunk * (size_t)DV;
  // dS' and dU as the adjoint scan left them: bf16, each 32-column slice's block contiguous;
  // fp32, row-major over all d_v columns; dR = dV, token rows
  constexpr bool SLM = sizeof(Tin) == 2;
  RegTile<Tin, DK, kAdjBV, kGradThreads> rs, rso;
  RegTile<Tin, kChunk, kAdjBV, kGradThreads> rv, rdo, rdu, rdr;
  auto issue = [&](int v0) {
    rs.load(Sb + v0, (size_t)DV, DK, tid);
    rv.load(v + tok * DV + v0, (size_t)H * DV, len, tid);
    rdo.load(dO + tok * DV + v0, (size_t)H * DV, len, tid);
    rdr.load(dvp + tok * DV + v0, (size_t)H * DV, len, tid);
    if constexpr (SLM) {
      rso.load(Sob + (size_t)v0 * DK, kAdjBV, DK, tid);
      rdu.load(dUb + (size_t)v0 * kChunk, kAdjBV, kChunk, tid);
    } else {
      rso.load(Sob + v0, (size_t)DV, DK, tid);
      rdu.load(dUb + v0, (size_t)DV, kChunk, tid);
    }
  };
  issue(0);
  // what the work after the d_v loop reads, loaded while its last block is computed: the query
  // rows, g at this thread's channel gc and rows gp RPP .., and A at this lane's entries of the
  // dL tiles
  const int gc = tid % DK, gp = tid / DK;
  float Gr[RPP], ar[2][4];
  // (every load unconditional, from a clamped in-range address, and masked afterwards: a load
  // under a branch is waited for inside it)
  auto issue_tail = [&]() {
    rq.load(q + tok * DK, (size_t)H * DK, len, tid);
#pragma unroll
    for (int r = 0; r < RPP; ++r)
      Gr[r] = g[(tok + (size_t)min(gp * RPP + r, len - 1) * H) * DK + gc];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int t = wid + 8 * x, I = t >> 2, J = min(t & 3, I);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        ar[x][e] = to_f32(Ap[ch * kTpbElems + (I * (I + 1) / 2 + J) * 256 + (4 * kq + e) * 16 + r16]);
    }
  };
  rkr.sqnorms(sm.den, tid);
  rkg.template store<LK>(&sm.K[0][0], tid);
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int e = tid + kGradThreads * x;
    if (e < kXPieces) {
      int I, J;
      lower_block(e >> 6, I, J);
      const int r = (e >> 2) & 15, c4 = 4 * (e & 3);
      *reinterpret_cast<f32x4 *>(&sm.X[16 * I + r][16 * J + c4]) = cvt4(xr[x]);
    }
  }
  if (tid < 6 * 64) {  // the six blocks above the diagonal are zero
    const int ub = tid >> 6, I = ub < 3 ? 0 : ub < 5 ? 1 : 2, J = ub < 3 ? ub + 1 : ub < 5 ? ub - 1 : 3;
    const int r = (tid >> 2) & 15, c4 = 4 * (tid & 3);
    *reinterpret_cast<f32x4 *>(&sm.X[16 * I + r][16 * J + c4]) = zero4();
  }
  __syncthreads();
  if (wid == 0) {  // token i = lane; sm.den holds the squared key norms
    const int i = lane;
    const float den = sm.den[i] + eps;
    sm.den[i] = den;
    float bi = 0.f, ci = 0.f;  // b and its derivative in eta
    if (i < len) {
      const float t_abs = (float)(t0 + i - cu[n] + 1 + (opts.pos_offset ? opts.pos_offset[n] : 0));
      bi = write_coef(opts.beta_mode, eta_l, den, t_abs);
      // every mode but key-norm only is linear in eta: db/deta is the coefficient at eta = 1
      ci = opts.beta_mode == kBetaKeyNorm ? 0.f : write_coef(opts.beta_mode, 1.f, den, t_abs);
    }
    sm.b[i] = bi;
    sm.db_deta[i] = ci;
  }

  // ---- the contractions over d_v, 32 columns at a time: Y = Kg S -> R = V - Y, U = T R;
  //      qa = dO S^T, ka = dR S^T, kb = U dS'^T (64 x DK), dP^ = dO U^T and dT = dU R^T (their
  //      lower blocks), and <S, dS'> per channel
  f32x4 qa[NM], ka[NM], kb[NM], pt[3];
#pragma unroll
  for (int m = 0; m < NM; ++m) qa[m] = ka[m] = kb[m] = zero4();
#pragma unroll
  for (int x = 0; x < 3; ++x) pt[x] = zero4();
  constexpr int NSJ = decltype(rs)::J;
  float scp[NSJ];  // this thread's rows of S (piece tid + 512 j, row (tid + 512 j) / 8)
#pragma unroll
  for (int j = 0; j < NSJ; ++j) scp[j] = 0.f;
  auto block = [&](int v0, bool last) __attribute__((always_inline)) {
    __syncthreads();  // the previous block's reads (and the first stores) are done
    rs.template store<LDL>(&sm.u.lp.S[0][0], tid);
    rso.template store<LDL>(&sm.u.lp.So[0][0], tid);
#pragma unroll
    for (int j = 0; j < NSJ; ++j) {
      const f32x4 sv = cvt4(rs.x[j]), so = cvt4(rso.x[j]);
      scp[j] += sv[0] * so[0] + sv[1] * so[1] + sv[2] * so[2] + sv[3] * so[3];
    }
    rv.template store<LDL>(&sm.u.lp.R[0][0], tid);
    rdo.template store<LDL>(&sm.u.lp.dO[0][0], tid);
    rdu.template store<LDL>(&sm.u.lp.dU[0][0], tid);
    rdr.template store<LDL>(&sm.u.lp.dR[0][0], tid);
    __syncthreads();
    if (last) issue_tail(); else issue(v0 + kAdjBV);
    const int yi = wid >> 1, yj = wid & 1;  // this wavefront's 16 x 16 tile of R and U
    {
      f32x4 y;
      if constexpr (TR)
        y = mmf<DK>(
            zero4(), lane, [&](int kk) { return rd8b(&sm.K[16 * yi + r16][kk]); },
            [&](int kk) { return col8<LDL>(&sm.u.lp.S[0][0], 16 * yj, kk, lane); });
      else
        y = mmt<Tin, DK>(
            zero4(), lane, [&](int i, int kk) { return sm.K[16 * yi + i][kk]; },
            [&](int kk, int j) { return to_f32(sm.u.lp.S[kk][16 * yj + j]); });
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * yi + 4 * kq + e;
        Tin &rv_ = sm.u.lp.R[row][16 * yj + r16];
        const Tin rn = from_f32<Tin>(to_f32(rv_) - y[e]);
        rv_ = rn;
        if constexpr (TR) sm.u.lp.Rb[row][16 * yj + r16] = from_f32<Tin>(sm.b[row] * to_f32(rn));
      }
    }
    __syncthreads();
    {
      f32x4 uu;
      if constexpr (TR)
        uu = mmf<kChunk>(
            zero4(), lane, [&](int kk) { return rd8b(&sm.X[16 * yi + r16][kk]); },
            [&](int kk) { return col8<LDL>(&sm.u.lp.Rb[0][0], 16 * yj, kk, lane); });
      else
        uu = mmt<Tin, kChunk>(
            zero4(), lane, [&](int i, int kk) { return sm.X[16 * yi + i][kk]; },
            [&](int kk, int j) { return sm.b[kk] * to_f32(sm.u.lp.R[kk][16 * yj + j]); });
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.u.lp.U[16 * yi + 4 * kq + e][16 * yj + r16] = from_f32<Tin>(uu[e]);
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int tj = (wid >> 2) + 2 * m;  // column tile of 16 key channels
      qa[m] = mmr<Tin, kAdjBV>(
          qa[m], lane, [&](int i, int kk) { return &sm.u.lp.dO[16 * mti + i][kk]; },
          [&](int j, int kk) { return &sm.u.lp.S[16 * tj + j][kk]; });
      ka[m] = mmr<Tin, kAdjBV>(
          ka[m], lane, [&](int i, int kk) { return &sm.u.lp.dR[16 * mti + i][kk]; },
          [&](int j, int kk) { return &sm.u.lp.S[16 * tj + j][kk]; });
      kb[m] = mmr<Tin, kAdjBV>(
          kb[m], lane, [&](int i, int kk) { return &sm.u.lp.U[16 * mti + i][kk]; },
          [&](int j, int kk) { return &sm.u.lp.So[16 * tj + j][kk]; });
    }
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const int jb = wid + 8 * x;  // jobs 0..9: blocks of dP^; 10..19: blocks of dT
      if (jb < 20) {
        int I, J;
        lower_block(jb % 10, I, J);
        if (jb < 10)
          pt[x] = mmr<Tin, kAdjBV>(
              pt[x], lane, [&](int i, int kk) { return &sm.u.lp.dO[16 * I + i][kk]; },
              [&](int j, int kk) { return &sm.u.lp.U[16 * J + j][kk]; });
        else
          pt[x] = mmr<Tin, kAdjBV>(
              pt[x], lane, [&](int i, int kk) { return &sm.u.lp.dU[16 * I + i][kk]; },
              [&](int j, int kk) { return &sm.u.lp.R[16 * J + j][kk]; });
      }
    }
  };
  for (int v0 = 0; v0 + kAdjBV < DV; v0 += kAdjBV) block(v0, false);
  block(DV - kAdjBV, true);  // d_v >= 64: at least two blocks
  // <S, dS'> per channel: the 8 lanes holding a row of S sum their partials
#pragma unroll
  for (int j = 0; j < NSJ; ++j) {
    float x = scp[j];
    x += __shfl_xor(x, 1, 8);
    x += __shfl_xor(x, 2, 8);
    x += __shfl_xor(x, 4, 8);
    if ((tid & 7) == 0) sm.sc[(tid + kGradThreads * j) >> 3] = x;
  }
  __syncthreads();  // the loop's LDS is free

  // ---- the key and query rows (and the squared query norms); G per channel (log2 units),
  //      first within parts of RPP rows; dP^ and dT (lower, zeros above; bf16: also dP^ as a
  //      bf16 tile)
  rkr.template store<LK>(&sm.K[0][0], tid);
  rq.template store<LK>(&sm.u.pa.Q[0][0], tid);
  rq.sqnorms(sm.qq, tid);
#pragma unroll
  for (int r = 0; r < RPP; ++r)
    Gr[r] = (gp * RPP + r < len ? Gr[r] * kLog2e : 0.f) + (r > 0 ? Gr[r - 1] : 0.f);
  sm.u.pa.tot[gp][gc] = Gr[RPP - 1];
  for (int e = tid; e < kChunk * kChunk; e += kGradThreads) {
    const int r = e >> 6, cc = e & 63;
    if ((cc >> 4) > (r >> 4)) {
      sm.u.pa.dP[r][cc] = 0.f;
      sm.u.pa.dT[r][cc] = 0.f;
      if constexpr (TR) sm.u.pa.dPb[r][cc] = from_f32<__bf16>(0.f);
    }
  }
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    const int jb = wid + 8 * x;
    if (jb < 20) {
      int I, J;
      lower_block(jb % 10, I, J);
      float (*dst)[LDC] = jb < 10 ? sm.u.pa.dP : sm.u.pa.dT;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * I + 4 * kq + e, col = 16 * J + r16;
        const float val = col <= row ? pt[x][e] : 0.f;
        dst[row][col] = val;
        if constexpr (TR)
          if (jb < 10) sm.u.pa.dPb[row][col] = from_f32<__bf16>(val);
      }
    }
  }
  if (tid < DK) sm.span[tid] = 0;
  __syncthreads();
  {
    // the carries of the G prefix; rows past a ragged end repeat G_last (their g reads as 0)
    float carry = 0.f;
#pragma unroll
    for (int p = 0; p < NPART - 1; ++p) carry += p < gp ? sm.u.pa.tot[p][gc] : 0.f;
#pragma unroll
    for (int r = 0; r < RPP; ++r) {
      Gr[r] += carry;
      sm.u.pa.GT[gc][gp * RPP + r] = Gr[r];
    }
  }
  if (tid < kChunk) {
    const float qq = sm.qq[tid];
    sm.rqn[tid] = opts.normalize_q ? (qq > 0.f ? 1.f / sqrtf(qq) : 0.f) : 1.f;
  }
  // db from T: column sums of dT o X (8 lanes a column, 8 entries each); W = dT Diag(b) X^T
  // into registers
  const int rc = tid >> 3, part = tid & 7;
  {
    float s1 = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int x = part + 8 * m;
      s1 += sm.u.pa.dT[x][rc] * sm.X[x][rc];
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) s1 += __shfl_xor(s1, off, 8);
    if (part == 0) sm.db[rc] = s1;
  }
  f32x4 w[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int t = wid + 8 * x, I = t >> 2, J = t & 3;
    w[x] = mmt<Tin, kChunk>(
        zero4(), lane, [&](int i, int kk) { return sm.u.pa.dT[16 * I + i][kk] * sm.b[kk]; },
        [&](int kk, int j) { return sm.X[16 * J + j][kk]; });
  }
  __syncthreads();
  // W into dT's place; the span of G around row 32 per channel
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int t = wid + 8 * x, I = t >> 2, J = t & 3;
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.u.pa.dT[16 * I + 4 * kq + e][16 * J + r16] = w[x][e];
  }
  {
    const float g32 = sm.u.pa.GT[gc][32];
    float sp = 0.f;
#pragma unroll
    for (int r = 0; r < RPP; ++r) sp = fmaxf(sp, fabsf(Gr[r] - g32));
    atomicMax(&sm.span[gc], __float_as_int(sp));  // non-negative floats order as integers
  }
  __syncthreads();
  // ---- dL = -strict_lower(X^T W); dA = Diag(b) dL; with A from the prep, the row sums of
  //      dL o A, one partial per tile
  f32x4 dl4[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int t = wid + 8 * x, I = t >> 2, J = t & 3;
    f32x4 acc = zero4();
    if (J <= I)
      acc = mmt<Tin, kChunk>(
          acc, lane, [&](int i, int kk) { return sm.X[kk][16 * I + i]; },
          [&](int kk, int j) { return sm.u.pa.dT[kk][16 * J + j]; });
    float zr4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * I + 4 * kq + e, col = 16 * J + r16;
      const float dl = col < row ? -acc[e] : 0.f;
      zr4[e] = col < row ? dl * ar[x][e] : 0.f;  // (ar holds another block's entry above)
      dl4[x][e] = sm.b[row] * dl;  // dA
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      zr4[e] = row16_sum(zr4[e]);
      if (r16 == 0) sm.zr[J][16 * I + 4 * kq + e] = zr4[e];
    }
  }
  __syncthreads();  // every read of W is done
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int t = wid + 8 * x, I = t >> 2, J = t & 3;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * I + 4 * kq + e, col = 16 * J + r16;
      sm.u.pa.dT[row][col] = dl4[x][e];
      if constexpr (TR) sm.u.pa.dAb[row][col] = from_f32<__bf16>(dl4[x][e]);
    }
  }
  __syncthreads();
  if (tid < kChunk) sm.db[tid] += sm.zr[0][tid] + sm.zr[1][tid] + sm.zr[2][tid] + sm.zr[3][tid];

  // ---- F1, H1 and Z on this wavefront's tiles (rows 16 mti + 4 kq + e, column 16 tj + r16)
  constexpr int LGT = kChunk + 4;
  const float (*GT)[LGT] = sm.u.pa.GT;
  const float (*dAf)[LDC] = sm.u.pa.dT;
  const float (*dPf)[LDC] = sm.u.pa.dP;
  auto g4 = [&](int c, int r) { return *reinterpret_cast<const f32x4 *>(&GT[c][r]); };
  f32x4 F1[NM], H1[NM], Zc[NM];
  // the matrix-core form on tile m (all of its 16 channels within 2^64 of row 32); the left
  // operands (rows of dA and dP^, and their columns for Z) are the same for every tile of the
  // wavefront and read once
  [[maybe_unused]] bf16x8 wfa[2], wfp[2], wfat[2], wfpt[2];
  auto load_w = [&]() {
    if constexpr (TR) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int kk = 32 * x + 8 * kq;
        wfa[x] = row8<LG>(&sm.u.pa.dAb[0][0], 16 * mti, kk, lane);
        wfp[x] = row8<LG>(&sm.u.pa.dPb[0][0], 16 * mti, kk, lane);
        wfat[x] = col8<LG>(&sm.u.pa.dAb[0][0], 16 * mti, kk, lane);
        wfpt[x] = col8<LG>(&sm.u.pa.dPb[0][0], 16 * mti, kk, lane);
      }
    }
  };
  auto prod_fast = [&](int m) __attribute__((always_inline)) {
    if constexpr (TR) {
      const int tj = (wid >> 2) + 2 * m, col = 16 * tj + r16;
      const float g32 = GT[col][32];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int kk = 32 * x + 8 * kq;
        const bf16x8 kc = col8<LK>(&sm.K[0][0], 16 * tj, kk, lane);
        const bf16x8 qc = col8<LK>(&sm.u.pa.Q[0][0], 16 * tj, kk, lane);
        const f32x4 gj0 = g4(col, kk), gj1 = g4(col, kk + 4);
        const f32x4 rq0 = *reinterpret_cast<const f32x4 *>(&sm.rqn[kk]);
        const f32x4 rq1 = *reinterpret_cast<const f32x4 *>(&sm.rqn[kk + 4]);
        bf16x8 kf, ke, qe;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const float d = g32 - (s < 4 ? gj0[s] : gj1[s - 4]);
          const float f = exp2_fast(d), fr = exp2_fast(-d);
          const float kj = to_f32(kc[s]);
          kf[s] = from_f32<__bf16>(kj * f);
          ke[s] = from_f32<__bf16>(kj * fr);
          qe[s] = from_f32<__bf16>(to_f32(qc[s]) * (s < 4 ? rq0[s] : rq1[s - 4]) * fr);
        }
        F1[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfa[x], kf, F1[m], 0, 0, 0);
        H1[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfp[x], kf, H1[m], 0, 0, 0);
        Zc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfat[x], ke, Zc[m], 0, 0, 0);
        Zc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfpt[x], qe, Zc[m], 0, 0, 0);
      }
      const f32x4 gi = g4(col, 16 * mti + 4 * kq);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d = gi[e] - g32;
        const float ef = exp2_fast(d), fr = exp2_fast(-d);
        F1[m][e] *= ef;
        H1[m][e] *= ef;
        Zc[m][e] *= fr;
      }
    }
  };
  // term by term: Gamma = exp2(-|G_i - G_j|), the right value on every term whose dA or dP^
  // entry is not zero (j <= i for F1 and H1, j >= i for Z)
  auto prod_direct = [&](int m) {
    const int tj = (wid >> 2) + 2 * m, col = 16 * tj + r16;
    const f32x4 gi = g4(col, 16 * mti + 4 * kq);
    for (int j = 0; j < kChunk; ++j) {
      const float kj = to_f32(sm.K[j][col]);
      const float qj = to_f32(sm.u.pa.Q[j][col]) * sm.rqn[j];
      const float Gj = GT[col][j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * mti + 4 * kq + e;
        const float t = exp2_fast(-fabsf(gi[e] - Gj));
        F1[m][e] += dAf[i][j] * kj * t;
        H1[m][e] += dPf[i][j] * kj * t;
        Zc[m][e] += t * (dAf[j][i] * kj + dPf[j][i] * qj);
      }
    }
  };
  bool all_fast = false;
#pragma unroll
  for (int m = 0; m < NM; ++m) F1[m] = H1[m] = Zc[m] = zero4();
  if constexpr (TR) {
    bool f = true;
#pragma unroll
    for (int m = 0; m < NM; ++m)
      f = f && __int_as_float(sm.span[16 * ((wid >> 2) + 2 * m) + r16]) <= 64.f;
    all_fast = __all(f);
  }
  if (all_fast) {
    load_w();
#pragma unroll
    for (int m = 0; m < NM; ++m) prod_fast(m);
  } else {
    for (int m = 0; m < NM; ++m) {
      bool fast = false;
      if constexpr (TR) fast = __all(__int_as_float(sm.span[16 * ((wid >> 2) + 2 * m) + r16]) <= 64.f);
      if (fast) {
        load_w();
        prod_fast(m);
      } else {
        prod_direct(m);
      }
    }
  }
  __syncthreads();  // every read of dP^ and dA is done: their place takes dG

  // ---- dq^, dk, dG on this wavefront's tiles; dk out; the column sums of K o D o kb
  float (*dGt)[LGG] = reinterpret_cast<float (*)[LGG]>(&sm.u.pa.dP[0][0]);
  static_assert(sizeof(sm.u.pa.dP) + sizeof(sm.u.pa.dT) >= sizeof(float) * kChunk * LGG,
                "dG fits in the place of dP and dT");
  f32x4 dqh[NM];
  float qd[4] = {0.f, 0.f, 0.f, 0.f};
  // this lane's four rows: the readout factor and the coefficient's key-norm term
  const int row0 = 16 * mti + 4 * kq;
  const f32x4 rq4 = *reinterpret_cast<const f32x4 *>(&sm.rqn[row0]);
  f32x4 cb4;
  {
    const f32x4 den4 = *reinterpret_cast<const f32x4 *>(&sm.den[row0]);
    const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&sm.b[row0]);
    const f32x4 db4 = *reinterpret_cast<const f32x4 *>(&sm.db[row0]);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      cb4[e] = opts.beta_mode != kBetaGated && den4[e] != 0.f
                   ? -2.f * b4[e] * db4[e] * __builtin_amdgcn_rcpf(den4[e])
                   : 0.f;
  }
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int tj = (wid >> 2) + 2 * m, col = 16 * tj + r16;
    const float gl = GT[col][kChunk - 1];
    const f32x4 gi = g4(col, row0);
    float kbs = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = row0 + e;
      const float E = exp2_fast(gi[e]), D = exp2_fast(gl - gi[e]);
      const float kic = to_f32(sm.K[row][col]);
      const float qh = to_f32(sm.u.pa.Q[row][col]) * rq4[e];
      const float ta = E * qa[m][e], tk = E * ka[m][e], tb = D * kb[m][e];
      const float dqv = ta + H1[m][e];
      dqh[m][e] = dqv;
      qd[e] += qh * dqv;
      const float dkv = -tk + tb + F1[m][e] + Zc[m][e] + cb4[e] * kic;
      dGt[row][col] = qh * dqv - kic * (tk + tb - F1[m][e] + Zc[m][e]);
      kbs += kic * tb;
      if (row < len) dk[(tok + (size_t)row * H) * DK + col] = from_f32<Tin>(dkv);
    }
    kbs += __shfl_xor(kbs, 16, kWave);
    kbs += __shfl_xor(kbs, 32, kWave);
    if (kq == 0) sm.kbs[mti][col] = kbs;
  }
  // dq: dq^, or rq (dq^ - q^ (q^ . dq^)) under the normalised readout
  if (opts.normalize_q) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qd[e] = row16_sum(qd[e]);
      if (r16 == 0) sm.qdot[wid >> 2][16 * mti + 4 * kq + e] = qd[e];
    }
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int col = 16 * ((wid >> 2) + 2 * m) + r16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * mti + 4 * kq + e;
      float dqv = dqh[m][e];
      if (opts.normalize_q) {
        const float rq = sm.rqn[row];
        const float qh = to_f32(sm.u.pa.Q[row][col]) * rq;
        dqv = rq * (dqv - qh * (sm.qdot[0][row] + sm.qdot[1][row]));
      }
      if (row < len) dq[(tok + (size_t)row * H) * DK + col] = from_f32<Tin>(dqv);
    }
  }
  // ---- dg: per channel the reverse prefix of dG over the chunk's rows (rows past a ragged
  //      end hold 0), in parts of RPP rows, with the terms of G_last (whose position is
  //      len - 1, so they reach every written row); deta
  float sf[RPP];
#pragma unroll
  for (int r = RPP - 1; r >= 0; --r) sf[r] = dGt[gp * RPP + r][gc] + (r < RPP - 1 ? sf[r + 1] : 0.f);
  sm.u.pa.tot[gp][gc] = sf[0];
  __syncthreads();
  {
    float carry = exp2_fast(GT[gc][kChunk - 1]) * sm.sc[gc] + sm.kbs[0][gc] + sm.kbs[1][gc] +
                  sm.kbs[2][gc] + sm.kbs[3][gc];
#pragma unroll
    for (int p = 1; p < NPART; ++p) carry += p > gp ? sm.u.pa.tot[p][gc] : 0.f;
#pragma unroll
    for (int r = 0; r < RPP; ++r) {
      const int row = gp * RPP + r;
      if (row < len) dg[(tok + (size_t)row * H) * DK + gc] = sf[r] + carry;
    }
  }
  if (tid < len) deta[tok + (size_t)tid * H] = sm.db[tid] * sm.db_deta[tid];
}

template <typename Tin, int DK>
static hipError_t launch_grad_diag_t(int d_v, const void *q, const void *k, const void *v,
                                     const void *dO, const float *g, const float *eta, float eps,
                                     const CoefOpts &opts, const void *KG, const void *X,
                                     const void *A, const void *SN, const void *dSo,
                                     const void *dU, const void *dv, void *dq, void *dk,
                                     float *dg, float *deta, SeqTables t, int32_t n_seq,
                                     int64_t n_chunks_ub, int32_t H, hipStream_t stream) {
  const size_t smG = sizeof(GradDiagSmem<Tin, DK>);
  static_assert(sizeof(GradDiagSmem<Tin, DK>) <= 160 * 1024, "LDS budget");
  static std::atomic<bool> attr_set[kMaxDeviceOrdinals];
  if (hipError_t ea = set_lds_limit_once(
          reinterpret_cast<const void *>(&kla_bwd_grad_diag_kernel<Tin, DK>), (int)smG, attr_set);
      ea != hipSuccess)
    return ea;
  const int64_t blocks = n_chunks_ub * H;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((kla_bwd_grad_diag_kernel<Tin, DK>), dim3((unsigned)blocks),
                     dim3(kGradThreads), smG, stream, static_cast<const Tin *>(q),
                     static_cast<const Tin *>(k), static_cast<const Tin *>(v),
                     static_cast<const Tin *>(dO), g, eta, eps, opts,
                     static_cast<const Tin *>(KG), static_cast<const Tin *>(X),
                     static_cast<const Tin *>(A), static_cast<const Tin *>(SN),
                     static_cast<const Tin *>(dSo), static_cast<const Tin *>(dU),
                     static_cast<const Tin *>(dv), static_cast<Tin *>(dq), static_cast<Tin *>(dk),
                     dg, deta, t.cu, t.chunk_off, n_seq, H, d_v);
  return hipGetLastError();
}

hipError_t launch_bwd_grad_diag(Dtype dt, int d_k, int d_v, const void *q, const void *k,
                                const void *v, const void *dO, const float *g, const float *eta,
                                float eps, const CoefOpts &opts, const void *KG, const void *X,
                                const void *A, const void *SN, const void *dSo, const void *dU,
                                const void *dv, void *dq, void *dk, float *dg, float *deta,
                                SeqTables t, int32_t n_seq, int64_t n_chunks_ub, int32_t H,
                                hipStream_t stream) {
#define KLA_GRAD_DIAG(TIN, DK_)                                                                  \
  return launch_grad_diag_t<TIN, DK_>(d_v, q, k, v, dO, g, eta, eps, opts, KG, X, A, SN, dSo, dU, \
                                      dv, dq, dk, dg, deta, t, n_seq, n_chunks_ub, H, stream);
  if (dt == Dtype::BF16) {
    if (d_k == 128) { KLA_GRAD_DIAG(__bf16, 128) }
    KLA_GRAD_DIAG(__bf16, 64)
  }
  if (d_k == 128) { KLA_GRAD_DIAG(float, 128) }
  KLA_GRAD_DIAG(float, 64)
#undef KLA_GRAD_DIAG
}

}  // namespace kla
