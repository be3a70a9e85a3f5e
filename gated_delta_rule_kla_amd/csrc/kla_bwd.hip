// kla_bwd.hip -- the backward pass of the chunkwise prefill: gradients of q, k, v, g, eta and
// of the incoming state S0 for the cotangents dO of the outputs and dS_T of the final state.
//
// Paper "Kaczmarz Linear Attention" (arXiv 2605.08587) trains with the chunkwise algorithm of
// Propositions 3-4 (Eq. (7)-(9)) but derives no backward pass.  What follows is the
// reverse-mode derivative of that chunk solve, with one scalar gate per token-head and
// o_t = q_t S_t, for the Kaczmarz coefficient of Eq. (3) and its variants (the gated rule's
// b = eta, key-norm only, the sequence factors; b enters only through db below).  Per chunk of one
// (sequence, head), with S the chunk's incoming state, G the chunk-local inclusive prefix of
// g, Gamma_ij = exp(G_i - G_j), gam_i = exp(G_i), dec_i = exp(G_last - G_i),
// A = strict_lower(Gamma o K K^T), P = lower(Gamma o Q K^T), X = (I + Diag(b) A)^{-1},
// T = X Diag(b) and den_i = ||k_i||^2 + eps:
//   forward   R = V - Diag(gam) K S,  U = T R,  O = Diag(gam) Q S + P U,
//             S' = exp(G_last) S + K^T Diag(dec) U
//   backward, given dO and dS' (the next chunk's dS, or dS_T):
//     dU = P^T dO + Diag(dec) K dS',   dR = T^T dU = dV,
//     dS = exp(G_last) dS' + Q^T Diag(gam) dO - K^T Diag(gam) dR    (the previous chunk's dS')
//     dP = lower(dO U^T),  dT = lower(dU R^T),  dX = dT Diag(b),
//     dL = -strict_lower(X^T dX X^T),  dA = Diag(b) dL,
//     db = colsum(dT o X) + rowsum(dL o A),  deta = db (d b / d eta),
//     dQ = Diag(gam) dO S^T + (dP o Gamma) K,
//     dK = Diag(dec) U dS'^T - Diag(gam) dR S^T + (dP o Gamma)^T Q + (dA o Gamma) K
//          + (dA o Gamma)^T K - Diag(2 b db / den) K   (that last term where b depends on
//          ||k||^2: every mode but the gated rule's),
//     dG_i = gam_i q_i.(dO S^T)_i - gam_i k_i.(dR S^T)_i - dec_i k_i.(U dS'^T)_i
//            + rowsum_i(Z) - colsum_i(Z),   Z = dP o P + dA o A,
//     dG_last += exp(G_last) <dS', S> + sum_j dec_j k_j.(U dS'^T)_j,
//     dg_t = sum of dG_i over the chunk's positions i >= t.
// After the forward kernels have run again (the prep, which also stores every chunk's
// X = (I + Diag(b) A)^{-1} in the operand type, then the chunk scan storing every chunk's incoming state
// S), two kernels finish the job:
//   kla_bwd_scan_kernel  the adjoint scan: sequential over the chunks in reverse, parallel over
//                        (sequence, head, 32-column slice) since the columns of dS are
//                        independent given the tiles; stores dS' and dU per chunk, writes
//                        dV (= dR, which the gradient kernel reads back) and dS0.
//   kla_bwd_grad_kernel  one workgroup per (chunk, head): the contractions over d_v with the
//                        stored S and dS', then the chunk-local algebra, dq, dk, dg, deta.
// Tiles sit in LDS in fp32 (the gradient kernel's d_v-loop tiles in the operand type).
// Products run on fp32 MFMA (v_mfma_f32_16x16x4_f32) for fp32 inputs, and on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16, operands rounded to bf16 as they are read, fp32 accumulation)
// for bf16 inputs.
#include "kla_bwd_common.h"

namespace kla {

namespace {

template <int DK>
struct AdjSmem {
  float K[kChunk][DK + 4];
  float Q[kChunk][DK + 4];
  float T[kChunk][LDC];
  float P[kChunk][LDC];
  float dO[kChunk][LDB];
  float dU[kChunk][LDB];
  float dR[kChunk][LDB];
  float dS[DK][LDB];
  float gam[kChunk], dec[kChunk], gamO[kChunk];
  float gC[DK];  // diagonal gating: exp(G_last) per key channel
};

}  // namespace

// The adjoint scan.  Workgroup (sequence n, head h, slice) owns state columns
// 32 slice .. + 31 of dS for the whole sequence, in LDS.
// DIAG (diagonal gating, Appendix B.5): the prep's decayed tiles replace the key and query
// rows: dU = P^T dO + Kd dS' with Kd = K o exp(G_last - G), and
// dS = Diag(exp(G_last)) dS' + Qg^T Diag(gamO) dO - Kg^T dR with Qg = Q o exp(G),
// Kg = K o exp(G), exp(G_last) per key channel (the prep's gam and dec are then 1).  Kd sits
// in the key tile for the dU products and Kg replaces it once they are done.
template <typename Tin, int DK, bool DIAG>
__global__ __launch_bounds__(kAdjThreads) void kla_bwd_scan_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ dO,
    const float *__restrict__ GD, const Tin *__restrict__ Tm, const Tin *__restrict__ Pm,
    const float *__restrict__ dST, float *__restrict__ dS0, float *__restrict__ dSo,
    float *__restrict__ dUo, Tin *__restrict__ dv, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, int H, int DV, DiagTiles dg) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  AdjSmem<DK> &sm = *reinterpret_cast<AdjSmem<DK> *>(smem_raw);
  // the d_v slices of one (sequence, head) read the same K, Q, T and P: give them
  // consecutive logical ids on one XCD (workgroup b runs on XCD b % 8) to share its L2
  const int nsl = DV / kAdjBV;
  const int nblk = gridDim.x, b = blockIdx.x;
  const int pidx = (nblk % 8 == 0) ? (b % 8) * (nblk / 8) + b / 8 : b;
  const int slice = pidx % nsl, sh = pidx / nsl;
  const int h = sh % H, n = sh / H;
  const int v0 = slice * kAdjBV;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int tb = cu[n], te = cu[n + 1], cbase = chunk_off[n];
  const int nchunks = (te - tb + kChunk - 1) / kChunk;
  const size_t sbase = ((size_t)n * H + h) * DK * (size_t)DV + v0;

  // the last chunk's dS' is the cotangent of S_T; T and P keep zeros above their lower blocks
  for (int e = tid; e < DK * kAdjBV; e += kAdjThreads) {
    const int r = e / kAdjBV, c = e % kAdjBV;
    sm.dS[r][c] = dST ? dST[sbase + (size_t)r * DV + c] : 0.f;
  }
  for (int e = tid; e < kChunk * LDC; e += kAdjThreads) {
    (&sm.T[0][0])[e] = 0.f;
    (&sm.P[0][0])[e] = 0.f;
  }
  // every zero is in place before any thread stores a chunk's lower blocks over them
  __syncthreads();
  // a chunk's tiles are loaded into registers while the chunk before it (in this reverse
  // order) is computed, and written to LDS when its turn comes
  RegTile<Tin, kChunk, DK, kAdjThreads> rk, rq;
  RegTile<Tin, DIAG ? kChunk : 4, DIAG ? DK : 4, kAdjThreads> rkg;  // Kg (DIAG)
  RegTile<Tin, kChunk, kAdjBV, kAdjThreads> rdo;
  PackedTile<Tin, kAdjThreads> rt, rp;
  float rgd = 0.f;
  auto issue = [&](int c) {
    const int t0 = tb + c * kChunk, len = min(kChunk, te - t0);
    const size_t ch = (size_t)(cbase + c) * H + h;
    const size_t tok = (size_t)t0 * H + h;
    if constexpr (DIAG) {  // the decayed tiles: all 64 rows, zero past a ragged end
      const size_t t64 = ch * kChunk * DK;
      rk.load(static_cast<const Tin *>(dg.kd) + t64, DK, kChunk, tid);
      rq.load(static_cast<const Tin *>(dg.qg) + t64, DK, kChunk, tid);
    } else {
      rk.load(k + tok * DK, (size_t)H * DK, len, tid);
      rq.load(q + tok * DK, (size_t)H * DK, len, tid);
    }
    rdo.load(dO + tok * DV + v0, (size_t)H * DV, len, tid);
    rt.load(Tm + ch * kTpbElems, tid);
    rp.load(Pm + ch * kTpbElems, tid);
    if (tid < 3 * kChunk) rgd = GD[ch * kGDFloats + tid];  // gam, dec, gamO
    else if (DIAG && tid < 3 * kChunk + DK) rgd = dg.gc[ch * DK + tid - 3 * kChunk];
  };
  auto issue_kg = [&](int c) {
    if constexpr (DIAG)
      rkg.load(static_cast<const Tin *>(dg.kg) + ((size_t)(cbase + c) * H + h) * kChunk * DK, DK,
               kChunk, tid);
  };
  if (nchunks > 0) {
    issue(nchunks - 1);
    issue_kg(nchunks - 1);
  }
  for (int c = nchunks - 1; c >= 0; --c) {
    const int t0 = tb + c * kChunk, len = min(kChunk, te - t0);
    const size_t ch = (size_t)(cbase + c) * H + h;
    const size_t tok = (size_t)t0 * H + h;
    rk.template store<DK + 4>(&sm.K[0][0], tid);
    rq.template store<DK + 4>(&sm.Q[0][0], tid);
    rdo.template store<LDB>(&sm.dO[0][0], tid);
    rt.store(sm.T, tid);
    rp.store(sm.P, tid);
    if (tid < kChunk) sm.gam[tid] = rgd;
    else if (tid < 2 * kChunk) sm.dec[tid - kChunk] = rgd;
    else if (tid < 3 * kChunk) sm.gamO[tid - 2 * kChunk] = rgd;
    else if (DIAG && tid < 3 * kChunk + DK) sm.gC[tid - 3 * kChunk] = rgd;
    __syncthreads();
    if (c > 0) issue(c - 1);

    // this chunk's dS' for the gradient kernel
    {
      float *dst = dSo + ch * DK * (size_t)DV + v0;
      for (int e = tid; e < DK * kAdjBV / 4; e += kAdjThreads) {
        const int r = e / (kAdjBV / 4), c4 = 4 * (e % (kAdjBV / 4));
        *reinterpret_cast<f32x4 *>(dst + (size_t)r * DV + c4) =
            *reinterpret_cast<const f32x4 *>(&sm.dS[r][c4]);
      }
    }
    // dU = P^T dO + Diag(dec) K dS': 4 x 2 tiles, 8 / NW per wavefront
    constexpr int NW = kAdjThreads / 64, NU = 8 / NW;
#pragma unroll
    for (int x = 0; x < NU; ++x) {
      const int t = NU * wid + x, ti = t >> 1, tj = t & 1;
      const f32x4 a = mmt<Tin, kChunk>(
          zero4(), lane, [&](int i, int kk) { return sm.P[kk][16 * ti + i]; },
          [&](int kk, int j) { return sm.dO[kk][16 * tj + j]; });
      const f32x4 y = mmt<Tin, DK>(
          zero4(), lane, [&](int i, int kk) { return sm.K[16 * ti + i][kk]; },
          [&](int kk, int j) { return sm.dS[kk][16 * tj + j]; });
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * ti + 4 * kq + e;
        sm.dU[row][16 * tj + r16] = a[e] + sm.dec[row] * y[e];
      }
    }
    __syncthreads();
    // DIAG: the key tile's readers (the dU products) are done: Kg takes its place for dS
    if constexpr (DIAG) {
      rkg.template store<DK + 4>(&sm.K[0][0], tid);
      if (c > 0) issue_kg(c - 1);
    }
    // dR = T^T dU
#pragma unroll
    for (int x = 0; x < NU; ++x) {
      const int t = NU * wid + x, ti = t >> 1, tj = t & 1;
      const f32x4 rr = mmt<Tin, kChunk>(
          zero4(), lane, [&](int i, int kk) { return sm.T[kk][16 * ti + i]; },
          [&](int kk, int j) { return sm.dU[kk][16 * tj + j]; });
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.dR[16 * ti + 4 * kq + e][16 * tj + r16] = rr[e];
    }
    __syncthreads();
    // dU to the workspace; dV = dR on the chunk's tokens
    {
      float *du = dUo + ch * kChunk * (size_t)DV + v0;
      for (int e = tid; e < kChunk * kAdjBV / 4; e += kAdjThreads) {
        const int r = e / (kAdjBV / 4), c4 = 4 * (e % (kAdjBV / 4));
        const f32x4 u = *reinterpret_cast<const f32x4 *>(&sm.dU[r][c4]);
        const f32x4 x = *reinterpret_cast<const f32x4 *>(&sm.dR[r][c4]);
        *reinterpret_cast<f32x4 *>(du + (size_t)r * DV + c4) = u;
        if (r < len) {
          Tin *o = dv + (tok + (size_t)r * H) * DV + v0 + c4;
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = from_f32<Tin>(x[i]);
        }
      }
    }
    // dS = exp(G_last) dS' + Q^T Diag(gamO) dO - K^T Diag(gam) dR: (DK / 16) x 2 tiles
    //      (gamO = gam, over ||q_i|| under the normalised readout; DIAG: exp(G_last) per key
    //      channel, Qg and Kg in the tiles)
    const float gl = sm.gam[kChunk - 1];  // rows past a ragged end repeat G_last
    constexpr int NX = DK / 8 / NW;       // tiles per wavefront
    f32x4 nd[NX];
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const int t = wid + NW * x, mi = t >> 1, tj = t & 1;
      f32x4 acc = mmt<Tin, kChunk>(
          zero4(), lane, [&](int i, int kk) { return sm.Q[kk][16 * mi + i]; },
          [&](int kk, int j) { return sm.gamO[kk] * sm.dO[kk][16 * tj + j]; });
      acc = mmt<Tin, kChunk>(
          acc, lane, [&](int i, int kk) { return -sm.K[kk][16 * mi + i]; },
          [&](int kk, int j) { return sm.gam[kk] * sm.dR[kk][16 * tj + j]; });
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * mi + 4 * kq + e;
        acc[e] += (DIAG ? sm.gC[row] : gl) * sm.dS[row][16 * tj + r16];
      }
      nd[x] = acc;
    }
    __syncthreads();  // every read of this chunk's tiles and of dS' is done
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const int t = wid + NW * x, mi = t >> 1, tj = t & 1;
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.dS[16 * mi + 4 * kq + e][16 * tj + r16] = nd[x][e];
    }
  }
  __syncthreads();
  if (dS0) {
    for (int e = tid; e < DK * kAdjBV; e += kAdjThreads) {
      const int r = e / kAdjBV, c = e % kAdjBV;
      dS0[sbase + (size_t)r * DV + c] = sm.dS[r][c];
    }
  }
}

namespace {

// The adjoint scan for bf16 inputs.  The tiles sit in LDS in bf16 rows (K, Q, P, T, dO and
// Diag(gamO) dO as staged, dS', dU and Diag(gam) dR transposed, as their producers hold them);
// each product takes each lane's 8 contraction indices either as one 16-byte row read or,
// where it contracts down a column, as two gfx950 transpose reads, and the workgroup's
// 128 x 32 (or 64 x 32) block of dS stays in the registers of the wavefronts that update it,
// as fp32 accumulators.
template <int DK>
struct AdjSmem16 {
  static constexpr int LK = DK + 8, LC = kChunk + 8, LV = kAdjBV + 8;  // bf16 row strides
  __bf16 K[kChunk][LK], Q[kChunk][LK];
  __bf16 P[kChunk][LC], T[kChunk][LC];       // lower blocks; zero above them
  __bf16 dO[kChunk][LV], dOg[kChunk][LV];    // dO and Diag(gamO) dO
  __bf16 dST[kAdjBV][LK];                    // dS'^T
  __bf16 dUT[kAdjBV][LC], dRgT[kAdjBV][LC];  // dU^T, (Diag(gam) dR)^T
  float gam[kChunk], dec[kChunk];
  float gC[DK];  // diagonal gating: exp(G_last) per key channel
};

}  // namespace

// DIAG as for kla_bwd_scan_kernel: Kd in the key tile for dU, then Kg; Qg in the query tile;
// exp(G_last) per key channel.
template <int DK, bool DIAG>
__global__ __launch_bounds__(kAdjThreads) void kla_bwd_scan16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ dO,
    const float *__restrict__ GD, const __bf16 *__restrict__ Tm, const __bf16 *__restrict__ Pm,
    const float *__restrict__ dST, float *__restrict__ dS0, __bf16 *__restrict__ dSo,
    __bf16 *__restrict__ dUo, __bf16 *__restrict__ dv, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, int H, int DV, DiagTiles dg) {
  using SM = AdjSmem16<DK>;
  constexpr int LK = SM::LK, LC = SM::LC, LV = SM::LV;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SM &sm = *reinterpret_cast<SM *>(smem_raw);
  // the d_v slices of one (sequence, head) read the same K, Q, T and P: give them
  // consecutive logical ids on one XCD (workgroup b runs on XCD b % 8) to share its L2
  const int nsl = DV / kAdjBV;
  const int nblk = gridDim.x, b = blockIdx.x;
  const int pidx = (nblk % 8 == 0) ? (b % 8) * (nblk / 8) + b / 8 : b;
  const int slice = pidx % nsl, sh = pidx / nsl;
  const int h = sh % H, n = sh / H;
  const int v0 = slice * kAdjBV;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int tb = cu[n], te = cu[n + 1], cbase = chunk_off[n];
  const int nchunks = (te - tb + kChunk - 1) / kChunk;
  const size_t sbase = ((size_t)n * H + h) * DK * (size_t)DV + v0;
  constexpr int NW = kAdjThreads / 64;
  constexpr int NX = DK / 64;  // dS tiles per wavefront: t = wid + NW x, rows 16 (t >> 1)

  // P and T: zero the blocks above the diagonal blocks, which the packed tiles never write,
  // before any staging
  for (int e = tid; e < kChunk * LC; e += kAdjThreads) {
    (&sm.P[0][0])[e] = from_f32<__bf16>(0.f);
    (&sm.T[0][0])[e] = from_f32<__bf16>(0.f);
  }
  // this wavefront's tiles of dS (initially dS_T): lane (r16, kq) holds rows
  // 16 mi + 4 kq + e, column 16 tj + r16
  f32x4 dS[NX];
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const int t = wid + NW * x, mi = t >> 1, tj = t & 1;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dS[x][e] = dST ? dST[sbase + (size_t)(16 * mi + 4 * kq + e) * DV + 16 * tj + r16] : 0.f;
  }
  __syncthreads();

  // a chunk's inputs are loaded into registers while the chunk before it (in this reverse
  // order) is computed, and staged when its turn comes
  RegTile<__bf16, kChunk, DK, kAdjThreads> rk, rq;
  RegTile<__bf16, DIAG ? kChunk : 4, DIAG ? DK : 4, kAdjThreads> rkg;  // Kg (DIAG)
  RegTile<__bf16, kChunk, kAdjBV, kAdjThreads> rdo;
  PackedTile<__bf16, kAdjThreads> rt, rp;
  static_assert(RegTile<__bf16, kChunk, kAdjBV, kAdjThreads>::J == 1, "one dO quad per thread");
  // gamO of this thread's dO row; gam or dec of token tid (DIAG: exp(G_last) of channel
  // tid - 128 for the next DK threads)
  float rgo = 0.f, rgd = 0.f;
  auto issue = [&](int c) {
    const int t0 = tb + c * kChunk, len = min(kChunk, te - t0);
    const size_t ch = (size_t)(cbase + c) * H + h;
    const size_t tok = (size_t)t0 * H + h;
    if constexpr (DIAG) {  // the decayed tiles: all 64 rows, zero past a ragged end
      const size_t t64 = ch * kChunk * DK;
      rk.load(static_cast<const __bf16 *>(dg.kd) + t64, DK, kChunk, tid);
      rq.load(static_cast<const __bf16 *>(dg.qg) + t64, DK, kChunk, tid);
    } else {
      rk.load(k + tok * DK, (size_t)H * DK, len, tid);
      rq.load(q + tok * DK, (size_t)H * DK, len, tid);
    }
    rdo.load(dO + tok * DV + v0, (size_t)H * DV, len, tid);
    rt.load(Tm + ch * kTpbElems, tid);
    rp.load(Pm + ch * kTpbElems, tid);
    rgo = GD[ch * kGDFloats + 2 * kChunk + tid / (kAdjBV / 4)];
    if (tid < 2 * kChunk) rgd = GD[ch * kGDFloats + tid];  // gam, dec
    else if (DIAG && tid < 2 * kChunk + DK) rgd = dg.gc[ch * DK + tid - 2 * kChunk];
  };
  auto issue_kg = [&](int c) {
    if constexpr (DIAG)
      rkg.load(static_cast<const __bf16 *>(dg.kg) + ((size_t)(cbase + c) * H + h) * kChunk * DK,
               DK, kChunk, tid);
  };
  if (nchunks > 0) {
    issue(nchunks - 1);
    issue_kg(nchunks - 1);
  }
  for (int c = nchunks - 1; c >= 0; --c) {
    const int t0 = tb + c * kChunk, len = min(kChunk, te - t0);
    const size_t ch = (size_t)(cbase + c) * H + h;
    const size_t tok = (size_t)t0 * H + h;
    __syncthreads();  // every read of the previous chunk's tiles is done
    // ---- stage K, Q, P, T, dO and Diag(gamO) dO as rows
    rk.template store<LK>(&sm.K[0][0], tid);
    rq.template store<LK>(&sm.Q[0][0], tid);
#pragma unroll
    for (int j = 0; j < rt.J; ++j) {
      const int pq = tid + kAdjThreads * j;
      if (pq < rt.NQ) {
        const int e0 = 4 * pq, w = e0 & 255;
        int I, Jb;
        lower_block(e0 >> 8, I, Jb);
        const int row = 16 * I + (w >> 4), col = 16 * Jb + (w & 15);
        *reinterpret_cast<bf16x4 *>(&sm.T[row][col]) = rt.x[j];
        *reinterpret_cast<bf16x4 *>(&sm.P[row][col]) = rp.x[j];
      }
    }
    {
      const int r = tid / (kAdjBV / 4), c4 = 4 * (tid % (kAdjBV / 4));
      *reinterpret_cast<bf16x4 *>(&sm.dO[r][c4]) = rdo.x[0];
      bf16x4 g4;
#pragma unroll
      for (int i = 0; i < 4; ++i) g4[i] = from_f32<__bf16>(rgo * to_f32(rdo.x[0][i]));
      *reinterpret_cast<bf16x4 *>(&sm.dOg[r][c4]) = g4;
    }
    if (tid < kChunk) sm.gam[tid] = rgd;
    else if (tid < 2 * kChunk) sm.dec[tid - kChunk] = rgd;
    else if (DIAG && tid < 2 * kChunk + DK) sm.gC[tid - 2 * kChunk] = rgd;
    // dS' (the state in registers) as dS'^T for K dS', and to the workspace for the gradients
    // (bf16, the slice's d_k x 32 block contiguous)
    {
      __bf16 *dst = dSo + ch * DK * (size_t)DV + (size_t)v0 * DK;
#pragma unroll
      for (int x = 0; x < NX; ++x) {
        const int t = wid + NW * x, mi = t >> 1, tj = t & 1;
        bf16x4 b4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          b4[e] = from_f32<__bf16>(dS[x][e]);
          dst[(16 * mi + 4 * kq + e) * kAdjBV + 16 * tj + r16] = b4[e];
        }
        *reinterpret_cast<bf16x4 *>(&sm.dST[16 * tj + r16][16 * mi + 4 * kq]) = b4;
      }
    }
    __syncthreads();
    if (c > 0) issue(c - 1);

    // ---- dU = P^T dO + Diag(dec) K dS': tile (ti, tj) = (wid >> 1, wid & 1)
    const int ti = wid >> 1, tj = wid & 1;
    {
      const f32x4 a = mmf<kChunk>(
          zero4(), lane, [&](int kk) { return col8<LC>(&sm.P[0][0], 16 * ti, kk, lane); },
          [&](int kk) { return col8<LV>(&sm.dO[0][0], 16 * tj, kk, lane); });
      const f32x4 y = mmf<DK>(
          zero4(), lane, [&](int kk) { return row8<LK>(&sm.K[0][0], 16 * ti, kk, lane); },
          [&](int kk) { return row8<LK>(&sm.dST[0][0], 16 * tj, kk, lane); });
      __bf16 *du = dUo + ch * kChunk * (size_t)DV + (size_t)v0 * kChunk;
      bf16x4 b4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * ti + 4 * kq + e;
        b4[e] = from_f32<__bf16>(a[e] + sm.dec[row] * y[e]);
        du[row * kAdjBV + 16 * tj + r16] = b4[e];
      }
      *reinterpret_cast<bf16x4 *>(&sm.dUT[16 * tj + r16][16 * ti + 4 * kq]) = b4;
    }
    __syncthreads();
    // DIAG: the key tile's readers (the dU products) are done: Kg takes its place for dS
    if constexpr (DIAG) {
      rkg.template store<LK>(&sm.K[0][0], tid);
      if (c > 0) issue_kg(c - 1);
    }
    // ---- dR = T^T dU (the same tile); dV = dR on the chunk's tokens
    {
      const f32x4 rr = mmf<kChunk>(
          zero4(), lane, [&](int kk) { return col8<LC>(&sm.T[0][0], 16 * ti, kk, lane); },
          [&](int kk) { return row8<LC>(&sm.dUT[0][0], 16 * tj, kk, lane); });
      bf16x4 b4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * ti + 4 * kq + e, col = 16 * tj + r16;
        const __bf16 rb = from_f32<__bf16>(rr[e]);
        if (row < len) dv[(tok + (size_t)row * H) * DV + v0 + col] = rb;
        b4[e] = from_f32<__bf16>(sm.gam[row] * rr[e]);
      }
      *reinterpret_cast<bf16x4 *>(&sm.dRgT[16 * tj + r16][16 * ti + 4 * kq]) = b4;
    }
    __syncthreads();
    // ---- dS = exp(G_last) dS' + Q^T Diag(gamO) dO - K^T Diag(gam) dR, on this wavefront's
    //      tiles (gamO = gam, over ||q_i|| under the normalised readout; DIAG: exp(G_last)
    //      per key channel, Qg and Kg in the tiles)
    const float gl = sm.gam[kChunk - 1];  // rows past a ragged end repeat G_last
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const int t = wid + NW * x, mi = t >> 1, sj = t & 1;
      f32x4 acc = dS[x] * gl;
      if constexpr (DIAG) acc = dS[x] * *reinterpret_cast<const f32x4 *>(&sm.gC[16 * mi + 4 * kq]);
      acc = mmf<kChunk>(
          acc, lane, [&](int kk) { return col8<LK>(&sm.Q[0][0], 16 * mi, kk, lane); },
          [&](int kk) { return col8<LV>(&sm.dOg[0][0], 16 * sj, kk, lane); });
      const f32x4 kr = mmf<kChunk>(
          zero4(), lane, [&](int kk) { return col8<LK>(&sm.K[0][0], 16 * mi, kk, lane); },
          [&](int kk) { return row8<LC>(&sm.dRgT[0][0], 16 * sj, kk, lane); });
      dS[x] = acc - kr;
    }
  }
  if (dS0) {
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const int t = wid + NW * x, mi = t >> 1, tj = t & 1;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dS0[sbase + (size_t)(16 * mi + 4 * kq + e) * DV + 16 * tj + r16] = dS[x][e];
    }
  }
}

namespace {

// LT: the element type of the d_v-loop tiles: the operand type of the inputs.  Every read of
// them feeds a product in that precision, so bf16 storage loses nothing and halves the LDS
// traffic of those products.

template <typename LT, int DK>
struct GradSmem {
  static constexpr int LDL = ldl<LT>();
  static constexpr bool TR = sizeof(LT) == 2;
  static constexpr int LK = DK + (TR ? 8 : 4);  // row stride of the key and query tiles
  static constexpr int LG = kChunk + 8;          // row stride of the bf16 64 x 64 tiles
  // bf16: the query rows and P sit outside the union (staged and formed before the d_v loop)
  static constexpr bool QO = TR;
  LT K[kChunk][LK];  // key rows in the operand type (exact)
  LT Qo[QO ? kChunk : 1][QO ? LK : 8];
  float X[kChunk][LDC];
  float Po[QO ? kChunk : 1][QO ? LDC : 4];
  union {
    struct {  // the loop over 32-column blocks of d_v
      LT S[DK][LDL], So[DK][LDL];
      LT R[kChunk][LDL], U[kChunk][LDL], dO[kChunk][LDL], dU[kChunk][LDL], dR[kChunk][LDL];
      // bf16: Diag(b) R, whose columns (like those of S) the products K S and X Diag(b) R
      // read by transpose reads (fp32 tiles read their columns element by element)
      LT Rb[TR ? kChunk : 1][TR ? LDL : 4];
    } lp;
    struct {  // the chunk-local algebra after it
      LT Qi[QO ? 1 : kChunk][QO ? 8 : LK];
      float Pi[QO ? 1 : kChunk][QO ? 4 : LDC];
      float dP[kChunk][LDC];  // dP (fp32: then Diag(rqn) (dP o Gamma))
      float dT[kChunk][LDC];  // dT, then dL (fp32: then dA o Gamma)
      // bf16: Diag(rqn) (dP o Gamma) and dA o Gamma + its transpose, for the dq and dk products
      __bf16 dPq[TR ? kChunk : 1][TR ? LG : 8], dAs[TR ? kChunk : 1][TR ? LG : 8];
    } pa;
  } u;
  float gam[kChunk], dec[kChunk], G[kChunk], b[kChunk], den[kChunk], db[kChunk];
  float db_deta[kChunk];  // the derivative of b in eta
  float rqn[kChunk];      // the readout's row factor: 1 / ||q_i|| (normalised readout), else 1
  float qdot[2][kChunk];  // squared query norms, then q^_i . dq^_i as two partial sums
  float rz[kChunk], cz[kChunk];
  float zr[4][kChunk], zc[4][kChunk];  // dL o A row sums and Diag(b) (dL o A) column sums,
                                       // one partial per 16-column (16-row) tile
  // query rows in the operand type (not normalised) and P = Diag(rqn) lower(Gamma o Q K^T),
  // then W = dT Diag(b) X^T in P's place
  __device__ LT *Q() {
    if constexpr (QO) return &Qo[0][0]; else return &u.pa.Qi[0][0];
  }
  __device__ float *P() {
    if constexpr (QO) return &Po[0][0]; else return &u.pa.Pi[0][0];
  }
  float dots[3][2][kChunk];  // row dots of the three d_v contractions, two partial sums each
  float red[kGradThreads / 64];
};

}  // namespace

template <typename Tin, int DK>
__global__ __launch_bounds__(kGradThreads) void kla_bwd_grad_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const Tin *__restrict__ dO, const float *__restrict__ g, const float *__restrict__ eta,
    float eps, CoefOpts opts, const Tin *__restrict__ SN, const Tin *__restrict__ dSo,
    const Tin *__restrict__ dUo, const Tin *__restrict__ dvp, const Tin *__restrict__ Xp,
    Tin *__restrict__ dq, Tin *__restrict__ dk, float *__restrict__ dg, float *__restrict__ deta,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_off, int n_seq, int H,
    int DV) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  using SMG = GradSmem<Tin, DK>;
  SMG &sm = *reinterpret_cast<SMG *>(smem_raw);
  constexpr int LK = SMG::LK, LG = SMG::LG;
  constexpr bool QO = SMG::QO;
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

  // ---- X = (I + Diag(b) A)^{-1}: the prep kernel's packed blocks in the operand type (ten
  //      16 x 16 blocks on and below the diagonal, 640 pieces of four), loaded first, stored
  //      (as fp32) after the key rows
  constexpr int kXPieces = kTpbElems / 4;
  // g and eta of token `lane`, for wavefront 0 (the decays and b), loaded first
  float g_l = 0.f, eta_l = 0.f;
  if (wid == 0 && lane < len) {
    g_l = g[tok + (size_t)lane * H];
    eta_l = eta[tok + (size_t)lane * H];
  }
  typename Raw4<Tin>::type xr[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int e = tid + kGradThreads * x;
    if (e < kXPieces)
      xr[x] = *reinterpret_cast<const typename Raw4<Tin>::type *>(Xp + ch * kTpbElems + 4 * e);
  }
  // ---- K rows (and, bf16, Q rows) with their squared norms; G, b, the decays
  RegTile<Tin, kChunk, DK, kGradThreads> rk;
  RegTile<Tin, QO ? kChunk : 4, QO ? DK : 4, kGradThreads> rq;
  rk.load(k + tok * DK, (size_t)H * DK, len, tid);
  if constexpr (QO) rq.load(q + tok * DK, (size_t)H * DK, len, tid);
  rk.template store<LK>(&sm.K[0][0], tid);
  rk.sqnorms(sm.den, tid);
  if constexpr (QO) {
    rq.template store<LK>(sm.Q(), tid);
    if (opts.normalize_q) rq.sqnorms(&sm.qdot[0][0], tid);
  }
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
  if (wid == 0) {
    const float G = wave_inclusive_scan(g_l, lane);  // rows past the end repeat G_last
    const float Gl = __shfl(G, kChunk - 1, kWave);
    sm.G[lane] = G;
    sm.gam[lane] = __expf(G);
    sm.dec[lane] = __expf(Gl - G);
  }
  __syncthreads();
  if (wid == 0) {  // token i = lane; sm.den holds the squared key norms
    const int i = lane;
    {
      const float den = sm.den[i] + eps;
      sm.den[i] = den;
      float bi = 0.f, ci = 0.f;  // b and its derivative in eta
      if (i < len) {
        const float t_abs =
            (float)(t0 + i - cu[n] + 1 + (opts.pos_offset ? opts.pos_offset[n] : 0));
        bi = write_coef(opts.beta_mode, eta_l, den, t_abs);
        // every mode but key-norm only is linear in eta: db/deta is the coefficient at eta = 1
        ci = opts.beta_mode == kBetaKeyNorm ? 0.f : write_coef(opts.beta_mode, 1.f, den, t_abs);
      }
      sm.b[i] = bi;
      sm.db_deta[i] = ci;
    }
  }
  // the readout's row factor: the chunk solve sees q^_i = rqn_i q_i, rqn_i = 1 / ||q_i|| under
  // the normalised readout (0 for a zero query), else 1; Q stays unscaled in LDS
  auto row_factor = [&](int i) {
    if (!opts.normalize_q) return 1.f;
    const float qq = sm.qdot[0][i];
    return qq > 0.f ? 1.f / sqrtf(qq) : 0.f;
  };
  // P = Diag(rqn) lower(Gamma o Q K^T), two 16 x 16 tiles per wavefront (zeros above the
  // diagonal blocks)
  auto form_P = [&]() {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int t = wid + 8 * x, I = t >> 2, J = t & 3;
      f32x4 acc = zero4();
      if (J <= I)
        acc = mmr<Tin, DK>(
            acc, lane, [&](int i, int kk) { return sm.Q() + (16 * I + i) * LK + kk; },
            [&](int j, int kk) { return &sm.K[16 * J + j][kk]; });
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * I + 4 * kq + e, col = 16 * J + r16;
        sm.P()[row * LDC + col] =
            col <= row ? row_factor(row) * __expf(sm.G[row] - sm.G[col]) * acc[e] : 0.f;
      }
    }
  };
  if constexpr (QO) {
    if (tid < kChunk) sm.rqn[tid] = row_factor(tid);
    form_P();
  }


  // ---- the contractions over d_v, 32 columns at a time:
  //      Y = K S -> R = V - Diag(gam) Y, U = T R; then accumulated in registers
  //      qa = Diag(gam) dO S^T, ka = -Diag(gam) dR S^T, kb = Diag(dec) U dS'^T (64 x DK),
  //      dP = dO U^T, dT = dU R^T (their lower blocks) and <dS', S>
  constexpr int NM = DK / 32;  // 64 x DK tiles per wavefront: t = wid + 8 m, rows 16 (wid & 3)
  const int mti = wid & 3;
  f32x4 qa[NM], ka[NM], kb[NM], pt[3];
#pragma unroll
  for (int m = 0; m < NM; ++m) qa[m] = ka[m] = kb[m] = zero4();
#pragma unroll
  for (int x = 0; x < 3; ++x) pt[x] = zero4();
  float sc = 0.f;
  const Tin *Sb = SN + ch * DK * (size_t)DV;
  const Tin *Sob = dSo + ch * DK * (size_t)DV;
  const Tin *dUb = dUo + ch * kChunk * (size_t)DV;
  // dS' and dU as the adjoint scan left them: bf16, each 32-column slice's block contiguous;
  // fp32, row-major over all d_v columns; dR = dV, token rows
  constexpr bool SLM = sizeof(Tin) == 2;
  // each 32-column block is loaded into registers while the one before it is computed
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
  constexpr int LDL = GradSmem<Tin, DK>::LDL;
  constexpr bool TR = GradSmem<Tin, DK>::TR;
  for (int v0 = 0; v0 < DV; v0 += kAdjBV) {
    __syncthreads();  // the previous block's reads (and X's writes) are done
    rs.template store<LDL>(&sm.u.lp.S[0][0], tid);
    rso.template store<LDL>(&sm.u.lp.So[0][0], tid);
#pragma unroll
    for (int j = 0; j < rs.J; ++j) {
      const f32x4 sv = cvt4(rs.x[j]), so = cvt4(rso.x[j]);
      sc += sv[0] * so[0] + sv[1] * so[1] + sv[2] * so[2] + sv[3] * so[3];
    }
    rv.template store<LDL>(&sm.u.lp.R[0][0], tid);
    rdo.template store<LDL>(&sm.u.lp.dO[0][0], tid);
    rdu.template store<LDL>(&sm.u.lp.dU[0][0], tid);
    rdr.template store<LDL>(&sm.u.lp.dR[0][0], tid);
    __syncthreads();
    if (v0 + kAdjBV < DV) issue(v0 + kAdjBV);
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
        const Tin rn = from_f32<Tin>(to_f32(rv_) - sm.gam[row] * y[e]);
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
    // qa, ka, kb without their row factors gam, -gam and dec (applied after the loop)
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int tj = (wid >> 2) + 2 * m;  // column tile of 16 key dims
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
      const int jb = wid + 8 * x;  // jobs 0..9: blocks of dP; 10..19: blocks of dT
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
  }
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * mti + 4 * kq + e;
      qa[m][e] *= sm.gam[row];
      ka[m][e] *= -sm.gam[row];
      kb[m][e] *= sm.dec[row];
    }
  sc = wave_sum(sc);
  if (lane == 0) sm.red[wid] = sc;
  __syncthreads();  // the loop's LDS is free

  // ---- dP and dT (lower, zeros above); bf16: also Diag(rqn) (dP o Gamma) for the dq products.
  //      fp32: the query rows, then P
  if constexpr (!QO)
    stage_rows<DK, LK, kGradThreads>(sm.Q(), q + tok * DK, (size_t)H * DK, len, tid,
                                     opts.normalize_q ? &sm.qdot[0][0] : nullptr);
  for (int e = tid; e < kChunk * kChunk; e += kGradThreads) {
    const int r = e >> 6, cc = e & 63;
    if ((cc >> 4) > (r >> 4)) {
      sm.u.pa.dP[r][cc] = 0.f;
      sm.u.pa.dT[r][cc] = 0.f;
      if constexpr (TR) sm.u.pa.dPq[r][cc] = from_f32<__bf16>(0.f);
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
        dst[row][col] = col <= row ? pt[x][e] : 0.f;
        if constexpr (TR)
          if (jb < 10)
            sm.u.pa.dPq[row][col] = from_f32<__bf16>(
                col <= row ? sm.rqn[row] * __expf(sm.G[row] - sm.G[col]) * pt[x][e] : 0.f);
      }
    }
  }
  __syncthreads();
  {
    if constexpr (!QO) {
      if (tid < kChunk) sm.rqn[tid] = row_factor(tid);
      form_P();
    }
    // row dots q^_i . qa_i, k_i . ka_i, k_i . kb_i: this wavefront's partial over its column
    // tiles, then its 16-lane row sums
    float dq4[4] = {0.f, 0.f, 0.f, 0.f}, da4[4] = {0.f, 0.f, 0.f, 0.f}, db4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int col = 16 * ((wid >> 2) + 2 * m) + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * mti + 4 * kq + e;
        dq4[e] += qa[m][e] * to_f32(sm.Q()[row * LK + col]);
        da4[e] += ka[m][e] * to_f32(sm.K[row][col]);
        db4[e] += kb[m][e] * to_f32(sm.K[row][col]);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dq4[e] = row16_sum(dq4[e]);
      da4[e] = row16_sum(da4[e]);
      db4[e] = row16_sum(db4[e]);
      if (r16 == 0) {
        const int row = 16 * mti + 4 * kq + e;
        sm.dots[0][wid >> 2][row] = row_factor(row) * dq4[e];
        sm.dots[1][wid >> 2][row] = da4[e];
        sm.dots[2][wid >> 2][row] = db4[e];
      }
    }
  }
  if constexpr (!QO) __syncthreads();  // P formed just above
  // ---- db from T: column sums of dT o X; the dP o P part of Z's row and column sums
  //      (8 lanes a row or column, 8 entries each); W = dT Diag(b) X^T into registers
  const int rc = tid >> 3, part = tid & 7;  // row / column rc, entries part + 8 m
  {
    float s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int x = part + 8 * m;
      s1 += sm.u.pa.dT[x][rc] * sm.X[x][rc];
      s2 += sm.u.pa.dP[rc][x] * sm.P()[rc * LDC + x];
      s3 += sm.u.pa.dP[x][rc] * sm.P()[x * LDC + rc];
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
      s1 += __shfl_xor(s1, off, 8);
      s2 += __shfl_xor(s2, off, 8);
      s3 += __shfl_xor(s3, off, 8);
    }
    if (part == 0) {
      sm.db[rc] = s1;
      sm.rz[rc] = s2;
      sm.cz[rc] = s3;
    }
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
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int t = wid + 8 * x, I = t >> 2, J = t & 3;
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.P()[(16 * I + 4 * kq + e) * LDC + 16 * J + r16] = w[x][e];
  }
  __syncthreads();
  // ---- dL = -strict_lower(X^T W) into dT's place (dT's last readers are past two barriers);
  //      bf16: dA o Gamma + its transpose as a tile (dA = Diag(b) dL); with A =
  //      strict_lower(Gamma o K K^T) formed here tile by tile, the row sums of dL o A and the
  //      column sums of Diag(b) (dL o A), one partial per tile
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int t = wid + 8 * x, I = t >> 2, J = t & 3;
    f32x4 acc = zero4(), kk4 = zero4();
    if (J <= I) {
      acc = mmt<Tin, kChunk>(
          acc, lane, [&](int i, int kk) { return sm.X[kk][16 * I + i]; },
          [&](int kk, int j) { return sm.P()[kk * LDC + 16 * J + j]; });
      kk4 = mmr<Tin, DK>(
          kk4, lane, [&](int i, int kk) { return &sm.K[16 * I + i][kk]; },
          [&](int j, int kk) { return &sm.K[16 * J + j][kk]; });
    }
    float zr4[4], zc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * I + 4 * kq + e, col = 16 * J + r16;
      const bool lower = col < row;
      const float gm = lower ? __expf(sm.G[row] - sm.G[col]) : 0.f;
      const float dl = lower ? -acc[e] : 0.f;
      sm.u.pa.dT[row][col] = dl;
      const float la = dl * gm * kk4[e];  // (dL o A)[row][col]
      zr4[e] = la;
      zc += sm.b[row] * la;
      if constexpr (TR) {
        const __bf16 av = from_f32<__bf16>(sm.b[row] * gm * dl);
        if (lower) {
          sm.u.pa.dAs[row][col] = av;
          sm.u.pa.dAs[col][row] = av;
        } else if (col == row) {
          sm.u.pa.dAs[row][col] = av;  // zero
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      zr4[e] = row16_sum(zr4[e]);
      if (r16 == 0) sm.zr[J][16 * I + 4 * kq + e] = zr4[e];
    }
    zc += __shfl_xor(zc, 16, kWave);
    zc += __shfl_xor(zc, 32, kWave);
    if (kq == 0) sm.zc[I][16 * J + r16] = zc;
  }
  __syncthreads();
  // ---- db += row sums of dL o A; the dA o A part of Z (dA = Diag(b) dL)
  if (tid < kChunk) {
    const int i = tid;
    const float s4 = sm.zr[0][i] + sm.zr[1][i] + sm.zr[2][i] + sm.zr[3][i];
    sm.db[i] += s4;
    sm.rz[i] += sm.b[i] * s4;
    sm.cz[i] += sm.zc[0][i] + sm.zc[1][i] + sm.zc[2][i] + sm.zc[3][i];
  }
  __syncthreads();
  // ---- fp32: Diag(rqn) (dP o Gamma) and dA o Gamma (dA = Diag(b) dL) in place (the bf16 path
  //      formed them as tiles above)
  if constexpr (!TR) {
    for (int e = tid; e < kChunk * kChunk; e += kGradThreads) {
      const int r = e >> 6, cc = e & 63;
      const float gm = cc <= r ? __expf(sm.G[r] - sm.G[cc]) : 0.f;
      sm.u.pa.dP[r][cc] *= gm * sm.rqn[r];
      sm.u.pa.dT[r][cc] *= sm.b[r] * gm;
    }
    __syncthreads();
  }
  // ---- Diag(rqn) dq^ = Diag(rqn) qa + Diag(rqn) (dP o Gamma) K (dq^: the gradient in q^);
  //      dk = ka + kb + (Diag(rqn) (dP o Gamma))^T Q + (dA o Gamma) K + (dA o Gamma)^T K
  //      - Diag(2 b db / den) K
  f32x4 aqs[NM];
  // bf16: this wavefront's 16 rows of the 64-wide left operands, as 16-byte runs (rows of
  // dPq and dAs, columns of dPq by transpose reads), read once for all its column tiles
  [[maybe_unused]] bf16x8 fP[2], fPt[2], fS[2];
  if constexpr (TR) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int kk = 32 * x + 8 * kq;
      fP[x] = row8<LG>(&sm.u.pa.dPq[0][0], 16 * mti, kk, lane);
      fPt[x] = col8<LG>(&sm.u.pa.dPq[0][0], 16 * mti, kk, lane);
      fS[x] = row8<LG>(&sm.u.pa.dAs[0][0], 16 * mti, kk, lane);
    }
  }
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int tj = (wid >> 2) + 2 * m;
    f32x4 aq = qa[m], ak = ka[m] + kb[m];
#pragma unroll
    for (int e = 0; e < 4; ++e) aq[e] *= sm.rqn[16 * mti + 4 * kq + e];
    if constexpr (TR) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int kk = 32 * x + 8 * kq;
        const bf16x8 bk = col8<LK>(&sm.K[0][0], 16 * tj, kk, lane);
        const bf16x8 bq = col8<LK>(sm.Q(), 16 * tj, kk, lane);
        aq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fP[x], bk, aq, 0, 0, 0);
        ak = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fPt[x], bq, ak, 0, 0, 0);
        ak = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fS[x], bk, ak, 0, 0, 0);
      }
    } else {
      aq = mmt<Tin, kChunk>(
          aq, lane, [&](int i, int kk) { return sm.u.pa.dP[16 * mti + i][kk]; },
          [&](int kk, int j) { return sm.K[kk][16 * tj + j]; });
      ak = mmt<Tin, kChunk>(
          ak, lane, [&](int i, int kk) { return sm.u.pa.dP[kk][16 * mti + i]; },
          [&](int kk, int j) { return sm.Q()[kk * LK + 16 * tj + j]; });
      ak = mmt<Tin, kChunk>(
          ak, lane,
          [&](int i, int kk) { return sm.u.pa.dT[16 * mti + i][kk] + sm.u.pa.dT[kk][16 * mti + i]; },
          [&](int kk, int j) { return sm.K[kk][16 * tj + j]; });
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * mti + 4 * kq + e, col = 16 * tj + r16;
      // b depends on k through den = ||k||^2 + eps (all modes but the gated rule's b = eta)
      const float den = sm.den[row];
      const float cb = opts.beta_mode != kBetaGated && den != 0.f
                           ? -2.f * sm.b[row] * sm.db[row] * __builtin_amdgcn_rcpf(den)
                           : 0.f;
      ak[e] += cb * to_f32(sm.K[row][col]);
      if (row < len) {
        const size_t o = (tok + (size_t)row * H) * DK + col;
        if (!opts.normalize_q) dq[o] = from_f32<Tin>(aq[e]);
        dk[o] = from_f32<Tin>(ak[e]);
      }
    }
    aqs[m] = aq;
  }
  // normalised readout: dq = rqn (dq^ - (q^ . dq^) q^) = aq - rqn^2 (q . aq) q with
  // aq = Diag(rqn) dq^ as formed above
  if (opts.normalize_q) {
    float pd[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int col = 16 * ((wid >> 2) + 2 * m) + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) pd[e] += aqs[m][e] * to_f32(sm.Q()[(16 * mti + 4 * kq + e) * LK + col]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pd[e] = row16_sum(pd[e]);
      if (r16 == 0) sm.qdot[wid >> 2][16 * mti + 4 * kq + e] = pd[e];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int col = 16 * ((wid >> 2) + 2 * m) + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * mti + 4 * kq + e;
        const float d = sm.qdot[0][row] + sm.qdot[1][row];
        if (row < len)
          dq[(tok + (size_t)row * H) * DK + col] =
              from_f32<Tin>(aqs[m][e] - sm.rqn[row] * sm.rqn[row] * d * to_f32(sm.Q()[row * LK + col]));
      }
    }
  }
  // ---- dG, its reverse prefix sum dg, and deta (one wavefront, lane = position)
  if (wid == 0) {
    const int i = lane;
    float dGi = sm.dots[0][0][i] + sm.dots[0][1][i] + sm.dots[1][0][i] + sm.dots[1][1][i] -
                sm.dots[2][0][i] - sm.dots[2][1][i] + sm.rz[i] - sm.cz[i];
    const float kb_i = i < len ? sm.dots[2][0][i] + sm.dots[2][1][i] : 0.f;
    const float kb_all = wave_sum(kb_i);
    float scs = 0.f;
#pragma unroll
    for (int x = 0; x < kGradThreads / 64; ++x) scs += sm.red[x];
    if (i == len - 1) dGi += sm.gam[kChunk - 1] * scs + kb_all;
    if (i >= len) dGi = 0.f;
    // reverse inclusive prefix: scan over the reversed lane order
    const float rev = wave_inclusive_scan(__shfl(dGi, kChunk - 1 - i, kWave), lane);
    const float dgi = __shfl(rev, kChunk - 1 - i, kWave);
    if (i < len) {
      dg[tok + (size_t)i * H] = dgi;
      deta[tok + (size_t)i * H] = sm.db[i] * sm.db_deta[i];
    }
  }
}

template <typename Tin, int DK, bool DIAG>
static hipError_t launch_adjoint_t(int d_v, const void *q, const void *k, const void *dO,
                                   const float *GD, const void *T, const void *P,
                                   const float *dST, void *dSo, void *dU, void *dv,
                                   float *dS0, SeqTables t, int32_t n_seq, int32_t H,
                                   const DiagTiles &dg, hipStream_t stream) {
  const Tin *qt = static_cast<const Tin *>(q), *kt = static_cast<const Tin *>(k);
  const int64_t scan_blocks = (int64_t)n_seq * H * (d_v / kAdjBV);
  if (scan_blocks <= 0) return hipSuccess;
  if constexpr (sizeof(Tin) == 2) {
    const size_t sm16 = sizeof(AdjSmem16<DK>);
    static_assert(sizeof(AdjSmem16<DK>) <= 160 * 1024, "LDS budget");
  static std::atomic<bool> attr16[kMaxDeviceOrdinals];
  if (hipError_t ea = set_lds_limit_once(
          reinterpret_cast<const void *>(&kla_bwd_scan16_kernel<DK, DIAG>), (int)sm16, attr16);
      ea != hipSuccess)
    return ea;
    hipLaunchKernelGGL((kla_bwd_scan16_kernel<DK, DIAG>), dim3((unsigned)scan_blocks),
                       dim3(kAdjThreads), sm16, stream, qt, kt, static_cast<const Tin *>(dO), GD,
                       static_cast<const Tin *>(T), static_cast<const Tin *>(P), dST, dS0,
                       static_cast<__bf16 *>(dSo), static_cast<__bf16 *>(dU),
                       static_cast<Tin *>(dv), t.cu, t.chunk_off, H, d_v, dg);
  } else {
    const size_t smA = sizeof(AdjSmem<DK>);
    static_assert(sizeof(AdjSmem<DK>) <= 160 * 1024, "LDS budget");
  static std::atomic<bool> attr[kMaxDeviceOrdinals];
  if (hipError_t ea = set_lds_limit_once(
          reinterpret_cast<const void *>(&kla_bwd_scan_kernel<Tin, DK, DIAG>), (int)smA, attr);
      ea != hipSuccess)
    return ea;
    hipLaunchKernelGGL((kla_bwd_scan_kernel<Tin, DK, DIAG>), dim3((unsigned)scan_blocks),
                       dim3(kAdjThreads), smA, stream, qt, kt, static_cast<const Tin *>(dO), GD,
                       static_cast<const Tin *>(T), static_cast<const Tin *>(P), dST, dS0,
                       static_cast<float *>(dSo), static_cast<float *>(dU),
                       static_cast<Tin *>(dv), t.cu, t.chunk_off, H, d_v, dg);
  }
  return hipGetLastError();
}

template <typename Tin, int DK>
static hipError_t launch_bwd_t(int d_v, const void *q, const void *k, const void *v,
                               const void *dO, const float *g, const float *eta, float eps,
                               const CoefOpts &opts, const float *GD, const void *T,
                               const void *P, const void *X, const float *dST,
                               const void *SN, void *dSo, void *dU, void *dq, void *dk,
                               void *dv, float *dg, float *deta, float *dS0, SeqTables t,
                               int32_t n_seq, int64_t n_chunks_ub, int32_t H,
                               hipStream_t stream, const DiagTiles *diag, const void *A) {
  hipError_t e;
  if (diag) {
    e = launch_adjoint_t<Tin, DK, true>(d_v, q, k, dO, GD, T, P, dST, dSo, dU, dv, dS0, t,
                                        n_seq, H, *diag, stream);
    if (e != hipSuccess) return e;
    return launch_bwd_grad_diag(sizeof(Tin) == 2 ? Dtype::BF16 : Dtype::F32, DK, d_v, q, k, v,
                                dO, g, eta, eps, opts, diag->kg, X, A, SN, dSo, dU, dv, dq, dk,
                                dg, deta, t, n_seq, n_chunks_ub, H, stream);
  }
  e = launch_adjoint_t<Tin, DK, false>(d_v, q, k, dO, GD, T, P, dST, dSo, dU, dv, dS0, t,
                                       n_seq, H, DiagTiles{}, stream);
  if (e != hipSuccess) return e;
  const size_t smG = sizeof(GradSmem<Tin, DK>);
  static_assert(sizeof(GradSmem<Tin, DK>) <= 160 * 1024, "LDS budget");
  static std::atomic<bool> attr_set[kMaxDeviceOrdinals];
  if (hipError_t ea = set_lds_limit_once(
          reinterpret_cast<const void *>(&kla_bwd_grad_kernel<Tin, DK>), (int)smG, attr_set);
      ea != hipSuccess)
    return ea;
  const Tin *qt = static_cast<const Tin *>(q), *kt = static_cast<const Tin *>(k);
  const int64_t grad_blocks = n_chunks_ub * H;
  if (grad_blocks > 0)
    hipLaunchKernelGGL((kla_bwd_grad_kernel<Tin, DK>), dim3((unsigned)grad_blocks),
                       dim3(kGradThreads), smG, stream, qt, kt, static_cast<const Tin *>(v),
                       static_cast<const Tin *>(dO), g, eta, eps, opts,
                       static_cast<const Tin *>(SN), static_cast<const Tin *>(dSo),
                       static_cast<const Tin *>(dU), static_cast<const Tin *>(dv),
                       static_cast<const Tin *>(X), static_cast<Tin *>(dq),
                       static_cast<Tin *>(dk), dg, deta, t.cu, t.chunk_off, n_seq, H, d_v);
  return hipGetLastError();
}

hipError_t launch_bwd(Dtype dt, int d_k, int d_v, const void *q, const void *k, const void *v,
                      const void *dO, const float *g, const float *eta, float eps,
                      const CoefOpts &opts, const float *GD, const void *T, const void *P,
                      const void *X, const float *dST, const void *SN, void *dSo, void *dU,
                      void *dq, void *dk, void *dv, float *dg, float *deta, float *dS0,
                      SeqTables t, int32_t n_seq, int64_t n_chunks_ub, int32_t H,
                      hipStream_t stream, const DiagTiles *diag, const void *A) {
#define KLA_BWD(TIN, DK_)                                                                     \
  return launch_bwd_t<TIN, DK_>(d_v, q, k, v, dO, g, eta, eps, opts, GD, T, P, X, dST, SN, dSo, dU, \
                                dq, dk, dv, dg, deta, dS0, t, n_seq, n_chunks_ub, H, stream, diag, A);
  if (dt == Dtype::BF16) {
    if (d_k == 128) { KLA_BWD(__bf16, 128) }
    KLA_BWD(__bf16, 64)
  }
  if (d_k == 128) { KLA_BWD(float, 128) }
  KLA_BWD(float, 64)
#undef KLA_BWD
}

}  // namespace kla
