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

// Chunk c of the packed input: sequence n, the sequence's first token ts, the chunk's first
// token t0 and its length.  Three ways to get there (PlanMode):
//  - kPlanTables: read the tables the plan kernel wrote;
//  - kPlanDense:  equal-length sequences (no offsets given), pure arithmetic; workgroups of
//                 head 0 also write the tables (entry 256 c + tid) for the scan;
//  - kPlanWave:   at most 63 sequences: every wavefront sanitises the offsets and counts
//                 chunks itself, one sequence per lane, exactly as the plan kernel does;
//                 wavefront 0 of workgroup (0, 0) writes the tables.
// Returns false when c lies past the last chunk.
struct ChunkLoc {
  int n, ts, t0, len;
};

__device__ __forceinline__ int wave_max_scan_i(int x, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x = max(x, y);
  }
  return x;
}
__device__ __forceinline__ int wave_sum_scan_i(int x, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ bool locate_chunk(const PlanArgs &pa, SeqTables tabs, int n_seq, int c,
                                             bool write_tables, ChunkLoc &loc) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (pa.mode == kPlanDense) {
    const int L = pa.total / n_seq, cpc = (L + kChunk - 1) / kChunk;
    if (write_tables) {
      const int e = c * (int)blockDim.x + tid;
      if (e <= n_seq) {
        tabs.cu[e] = e * L;
        tabs.chunk_off[e] = e * cpc;
      }
    }
    if (cpc == 0 || c >= n_seq * cpc) return false;
    loc.n = c / cpc;
    loc.ts = loc.n * L;
    loc.t0 = loc.ts + (c - loc.n * cpc) * kChunk;
    loc.len = min(kChunk, loc.ts + L - loc.t0);
    return true;
  }
  if (pa.mode == kPlanWave) {
    // lane e holds offset e: running maximum of the clamped offsets, then chunk counts
    const int raw = lane <= n_seq ? min(max(pa.cu_in[lane], 0), pa.total) : pa.total;
    const int cs = wave_max_scan_i(raw, lane);
    const int nxt = __shfl(cs, min(lane + 1, kWave - 1), kWave);
    const int cnt = lane < n_seq ? (nxt - cs + kChunk - 1) / kChunk : 0;
    const int co = wave_sum_scan_i(cnt, lane) - cnt;  // exclusive: chunk_off[lane]
    if (write_tables && tid < kWave && lane <= n_seq) {
      tabs.cu[lane] = cs;
      tabs.chunk_off[lane] = co;
    }
    if (c >= __shfl(co, n_seq, kWave)) return false;
    const unsigned long long below = __ballot(lane < n_seq && co <= c);
    loc.n = __popcll(below) - 1;
    loc.ts = __shfl(cs, loc.n, kWave);
    loc.t0 = loc.ts + (c - __shfl(co, loc.n, kWave)) * kChunk;
    loc.len = min(kChunk, __shfl(cs, loc.n + 1, kWave) - loc.t0);
    return true;
  }
  if (c >= tabs.chunk_off[n_seq]) return false;
  loc.n = find_sequence(tabs.chunk_off, n_seq, c);
  loc.ts = tabs.cu[loc.n];
  loc.t0 = loc.ts + (c - tabs.chunk_off[loc.n]) * kChunk;
  loc.len = min(kChunk, tabs.cu[loc.n + 1] - loc.t0);
  return true;
}

// ---------------------------------------------------------------------------------------------
// Prep / UT kernel: one workgroup (4 wavefronts) per (chunk, head); wavefront w owns the
// 16 chunk rows 16 w .. 16 w + 15.
//
// Every wavefront loads its own key (and query) rows straight into MFMA fragments, takes
// their norms from those registers, and scans the chunk's 64 log-decays itself; the key
// rows are shared with the other wavefronts through one swizzled LDS tile for the Gram
// and Q K^T tiles.  (I + L)^{-1} is formed blockwise on 16 x 16 blocks (X = (I + L)^{-1}
// is unit lower triangular): every wavefront inverts its diagonal block by substitution,
// then the sub-diagonal blocks follow level by level,
//   X_ij = -X_ii (sum_{k=j}^{i-1} L_ik X_kj),  i > j,
// with the 16 x 16 x 16 products on the fp32 matrix cores; X reuses the key tile's LDS
// once the Gram stage is done.  T = X Diag(b).
// When q is given the kernel also writes P = (A o Q K^T) (Eq. (8)'s intra-chunk matrix,
// A_ij = exp(G_i - G_j) for j <= i, zero above the diagonal) for the scan.
// ---------------------------------------------------------------------------------------------
constexpr int kLDL = kChunk + 4;  // padded row length of the fp32 L and X tiles

template <typename Tin, int DK>
struct PrepSmem {
  static constexpr int KBYTES = kChunk * DK * (int)sizeof(Tin);
  static constexpr int XBYTES = kChunk * kLDL * (int)sizeof(float);
  // key tile (swizzled 16-byte units) until the Gram stage ends, then X
  alignas(16) unsigned char KX[KBYTES > XBYTES ? KBYTES : XBYTES];
  alignas(16) float XT[kChunk][kLDL];  // X transposed, for 16-byte operand reads
  alignas(16) float L[kChunk][kLDL];
  alignas(16) float beta[kChunk];
  alignas(16) float G[kChunk];
  __device__ float (*X())[kLDL] { return reinterpret_cast<float (*)[kLDL]>(KX); }
};

// Byte offset of the 8-element fragment (row r, k-step ks, lane group kg) in the key tile:
// 16-byte unit 4 ks + kg (two units for fp32) XOR-swizzled by row so that 16 consecutive
// rows at one unit fall into distinct LDS bank groups.
template <typename Tin, int DK>
__device__ __forceinline__ int kfrag_off(int r, int ks, int kg) {
  constexpr int ES = sizeof(Tin), UPF = ES / 2;
  const int f = (DK >= 128 ? ((r >> 1) & 7) : ((r >> 2) & 3)) << 1;
  return r * DK * ES + ((((4 * ks + kg) * UPF) ^ (f * UPF)) << 4);
}

// D += A B for 16 x 16 fp32 blocks in LDS, A row-major (stride lda) and B given as its
// transpose Bt (stride ldbt): with the contraction index k = 4 kg + s in MFMA s, both
// operands are one 16-byte read per lane.
__device__ __forceinline__ f32x4 mm16t(const float *A, int lda, const float *Bt, int ldbt,
                                       f32x4 acc, int r16, int kg) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(A + r16 * lda + 4 * kg);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(Bt + r16 * ldbt + 4 * kg);
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
  return acc;
}
// D += A Y with Y a 16 x 16 block held in accumulator layout (lane (r16, kg) holds rows
// 4 kg + e of column r16): the contraction index is taken in the order the lanes hold it.
__device__ __forceinline__ f32x4 mm16_acc(const float *A, int lda, const f32x4 &Y, f32x4 acc,
                                          int r16, int kg) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(A + r16 * lda + 4 * kg);
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], Y[s], acc, 0, 0, 0);
  return acc;
}

template <typename Tin, int DK, typename TOut>
__global__ __launch_bounds__(256) void kla_prep_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ eta, float eps, int32_t *__restrict__ cu,
    int32_t *__restrict__ chunk_off, int n_seq, int H, float *__restrict__ G_out,
    float *__restrict__ beta_out, TOut *__restrict__ T_out, Tin *__restrict__ P_out,
    float *__restrict__ GD_out, CoefOpts opts, PlanArgs pa) {
  __shared__ PrepSmem<Tin, DK> sm;
  const int c = blockIdx.x, h = blockIdx.y;
  ChunkLoc loc;
  const bool write_tables = pa.mode == kPlanDense ? h == 0 : (c == 0 && h == 0);
  if (!locate_chunk(pa, SeqTables{cu, chunk_off},
                    n_seq, c, write_tables, loc))
    return;
  const int n = loc.n, t0 = loc.t0, len = loc.len;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kg = lane >> 4;
  const int i0 = 16 * wid;  // this wavefront's rows
  const bool want_p = (q != nullptr) && (P_out != nullptr);
  constexpr int NKS = DK / 32;
  using FragT = typename Frag<Tin>::type;

  // ---- loads: own key rows and the query rows of block 3 - w as fragments (zero past the
  //      chunk end), and the chunk's g and eta one token per lane.  Wavefront w forms the
  //      Gram tiles of row block w (w + 1 tiles) and the Q K^T tiles of row block 3 - w
  //      (4 - w tiles), five tiles each.
  const int my_row = i0 + r16;
  const bool row_ok = my_row < len;
  const int p0 = 16 * (3 - wid), p_row = p0 + r16;
  const bool prow_ok = p_row < len;
  FragT kf[NKS], qf[NKS];
  {
    const size_t rbase = ((size_t)(t0 + (row_ok ? my_row : 0)) * H + h) * DK + 8 * kg;
    const size_t qbase = ((size_t)(t0 + (prow_ok ? p_row : 0)) * H + h) * DK + 8 * kg;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kf[ks] = row_ok ? load8<Tin>(k + rbase + 32 * ks) : zero8<Tin>();
      qf[ks] = (want_p && prow_ok) ? load8<Tin>(q + qbase + 32 * ks) : zero8<Tin>();
    }
  }
  const bool tok_ok = lane < len;
  const size_t th = (size_t)(t0 + (tok_ok ? lane : 0)) * H + h;
  const float g_l = tok_ok ? g[th] : 0.f;
  const float eta_l = tok_ok ? eta[th] : 0.f;

  // ---- b for the own rows, G for token `lane` (every wavefront scans all 64)
  float ss = 0.f;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float x = to_f32(kf[ks][s]);
      ss = fmaf(x, x, ss);
    }
  ss += __shfl_xor(ss, 16, kWave);
  ss += __shfl_xor(ss, 32, kWave);
  const float eta_r = __shfl(eta_l, my_row, kWave);
  const float den = ss + eps;
  const float t_abs =
      (float)(t0 - loc.ts + my_row + 1 + (opts.pos_offset ? opts.pos_offset[n] : 0));
  const float b_r = row_ok ? write_coef(opts.beta_mode, eta_r, den, t_abs) : 0.f;
  const float G_l = wave_inclusive_scan(g_l, lane);  // rows past the end carry G_last
  // 1 / ||q|| of query row p_row under the normalised readout (0 for a zero query), else 1
  float rq = 1.f;
  if (opts.normalize_q) {
    float qq = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float x = to_f32(qf[ks][s]);
        qq = fmaf(x, x, qq);
      }
    qq += __shfl_xor(qq, 16, kWave);
    qq += __shfl_xor(qq, 32, kWave);
    rq = qq > 0.f ? 1.f / sqrtf(qq) : 0.f;
  }

#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    *reinterpret_cast<FragT *>(sm.KX + kfrag_off<Tin, DK>(my_row, ks, kg)) = kf[ks];
  if (kg == 0) sm.beta[my_row] = b_r;
  if (wid == 0) {
    sm.G[lane] = G_l;
    if (tok_ok && G_out) G_out[th] = G_l;
    // per-chunk decays for the scan: exp(G_i) and exp(G_last - G_i)
    if (GD_out) {
      const float Glast = __shfl(G_l, kChunk - 1, kWave);
      float *gd = GD_out + ((size_t)c * H + h) * kGDFloats;
      gd[lane] = __expf(G_l);
      gd[kChunk + lane] = __expf(Glast - G_l);
    }
  }
  // the output factor exp(G_i) / ||q_i|| for the query rows this wavefront holds
  {
    const float G_p = __shfl(G_l, p_row, kWave);
    if (GD_out && kg == 0)
      GD_out[((size_t)c * H + h) * kGDFloats + 2 * kChunk + p_row] = __expf(G_p) * rq;
  }
  if (beta_out && kg == 0 && row_ok) beta_out[((size_t)(t0 + my_row)) * H + h] = b_r;
  __syncthreads();

  // ---- Gram K K^T (row block w, column blocks jt <= w) -> strictly lower L
  {
    const f32x4 b_rows = *reinterpret_cast<const f32x4 *>(&sm.beta[i0 + 4 * kg]);
    const f32x4 G_rows = *reinterpret_cast<const f32x4 *>(&sm.G[i0 + 4 * kg]);
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      if (jt > wid) continue;
      FragT bk[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        bk[ks] = *reinterpret_cast<const FragT *>(sm.KX + kfrag_off<Tin, DK>(16 * jt + r16, ks, kg));
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) acc = mma(kf[ks], bk[ks], acc);  // rows i0 + 4 kg + e
      const int col = 16 * jt + r16;
      const float G_col = sm.G[col];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = i0 + 4 * kg + e;
        sm.L[row][col] = (col < row) ? b_rows[e] * __expf(G_rows[e] - G_col) * acc[e] : 0.f;
      }
    }
  }
  // ---- P^T = K Q^T for row block 3 - w, so each lane holds 4 consecutive columns of P row
  //      p_row; P = A o Q K^T is written row-major (zero above the diagonal)
  if (want_p) {
    Tin *Pc = P_out + ((size_t)c * H + h) * (kChunk * kChunk) + (size_t)p_row * kChunk;
    const float G_me = sm.G[p_row];
    const int pb = 3 - wid;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const int j0 = 16 * jt + 4 * kg;
      float pv[4] = {0.f, 0.f, 0.f, 0.f};
      if (jt <= pb) {
        f32x4 accp = zero4();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const FragT bk =
              *reinterpret_cast<const FragT *>(sm.KX + kfrag_off<Tin, DK>(16 * jt + r16, ks, kg));
          accp = mma(bk, qf[ks], accp);  // (Q K^T)[p_row][j0 + e]
        }
        const f32x4 G_cols = *reinterpret_cast<const f32x4 *>(&sm.G[j0]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pv[e] = (j0 + e <= p_row) ? __expf(G_me - G_cols[e]) * accp[e] * rq : 0.f;
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

  // ---- diagonal block: invert I + L_ww by substitution, lane = column r16 (the four lane
  //      groups compute the same column); L rows are read four values at a time
  float x[16];
  {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float lr[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v4 = *reinterpret_cast<const f32x4 *>(&sm.L[i0 + i][i0 + 4 * q4]);
        lr[4 * q4] = v4[0]; lr[4 * q4 + 1] = v4[1]; lr[4 * q4 + 2] = v4[2]; lr[4 * q4 + 3] = v4[3];
      }
      float a0 = (i == r16) ? 1.f : 0.f, a1 = 0.f;
#pragma unroll
      for (int j = 0; j < i; j += 2) {
        a0 = fmaf(-lr[j], x[j], a0);
        if (j + 1 < i) a1 = fmaf(-lr[j + 1], x[j + 1], a1);
      }
      x[i] = a0 + a1;
    }
  }
  __syncthreads();  // every key-tile read and every L row is done; X takes the key tile
  float(*X)[kLDL] = sm.X();
  if (kg == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) X[i0 + i][i0 + r16] = x[i];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<f32x4 *>(&sm.XT[i0 + r16][i0 + 4 * q4]) =
          f32x4{x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]};
  }
  __syncthreads();

  // ---- sub-diagonal blocks, one level (distance) at a time
#pragma unroll
  for (int dist = 1; dist < 4; ++dist) {
    const int jb = wid, ib = wid + dist;  // block (ib, jb)
    if (ib < 4) {
      f32x4 Y = zero4();
      for (int kb = jb; kb < ib; ++kb)
        Y = mm16t(&sm.L[16 * ib][16 * kb], kLDL, &sm.XT[16 * jb][16 * kb], kLDL, Y, r16, kg);
      f32x4 Z = mm16_acc(&X[16 * ib][16 * ib], kLDL, Y, zero4(), r16, kg);
#pragma unroll
      for (int e = 0; e < 4; ++e) X[16 * ib + 4 * kg + e][16 * jb + r16] = -Z[e];
      *reinterpret_cast<f32x4 *>(&sm.XT[16 * jb + r16][16 * ib + 4 * kg]) =
          f32x4{-Z[0], -Z[1], -Z[2], -Z[3]};
    }
    __syncthreads();
  }

  // ---- T = X Diag(b), zero above the diagonal: thread tid writes 16 consecutive entries of
  //      row tid / 4 (blocks above the diagonal of X were never written)
  {
    TOut *Tc = T_out + ((size_t)c * H + h) * (kChunk * kChunk);
    const int row = tid >> 2, j0 = 16 * (tid & 3);
    float tv[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 xv = *reinterpret_cast<const f32x4 *>(&X[row][j0 + 4 * q4]);
      const f32x4 bv = *reinterpret_cast<const f32x4 *>(&sm.beta[j0 + 4 * q4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + 4 * q4 + e;
        tv[4 * q4 + e] = (j <= row) ? xv[e] * bv[e] : 0.f;
      }
    }
    TOut *dst = Tc + (size_t)row * kChunk + j0;
    if constexpr (sizeof(TOut) == 2) {
#pragma unroll
      for (int h8 = 0; h8 < 2; ++h8) {
        bf16x8 o8;
#pragma unroll
        for (int e = 0; e < 8; ++e) o8[e] = from_f32<TOut>(tv[8 * h8 + e]);
        *reinterpret_cast<bf16x8 *>(dst + 8 * h8) = o8;
      }
    } else {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4 *>(dst + 4 * q4) =
            f32x4{tv[4 * q4], tv[4 * q4 + 1], tv[4 * q4 + 2], tv[4 * q4 + 3]};
    }
  }
}

template <typename Tin, int DK>
static hipError_t launch_prep_t(const void *q, const void *k, const float *g, const float *eta,
                                float eps, const CoefOpts &opts, SeqTables t, int32_t n_seq,
                                int64_t n_chunks_ub, int32_t H, float *G_out, float *beta_out,
                                void *T_out, bool t_fp32, void *P_out, float *GD_out,
                                const PlanArgs &pa, hipStream_t stream) {
  if (n_chunks_ub <= 0) return hipSuccess;
  const dim3 grid((unsigned)n_chunks_ub, H);
  const Tin *qq = static_cast<const Tin *>(q);
  Tin *pp = static_cast<Tin *>(P_out);
  if (t_fp32 || sizeof(Tin) == 4)
    hipLaunchKernelGGL((kla_prep_kernel<Tin, DK, float>), grid, dim3(256), 0, stream, qq,
                       static_cast<const Tin *>(k), g, eta, eps, t.cu, t.chunk_off, n_seq, H,
                       G_out, beta_out, static_cast<float *>(T_out), pp, GD_out, opts, pa);
  else
    hipLaunchKernelGGL((kla_prep_kernel<Tin, DK, Tin>), grid, dim3(256), 0, stream, qq,
                       static_cast<const Tin *>(k), g, eta, eps, t.cu, t.chunk_off, n_seq, H,
                       G_out, beta_out, static_cast<Tin *>(T_out), pp, GD_out, opts, pa);
  return hipGetLastError();
}

hipError_t launch_prep(Dtype dt, int d_k, const void *q, const void *k, const float *g,
                       const float *eta, float eps, const CoefOpts &opts, SeqTables t,
                       int32_t n_seq, int64_t n_chunks_ub, int32_t H, float *G_out,
                       float *beta_out, void *T_out, bool t_fp32, void *P_out, float *GD_out,
                       const PlanArgs &pa, hipStream_t stream) {
  if (dt == Dtype::BF16) {
    if (d_k == 128)
      return launch_prep_t<__bf16, 128>(q, k, g, eta, eps, opts, t, n_seq, n_chunks_ub, H, G_out,
                                        beta_out, T_out, t_fp32, P_out, GD_out, pa, stream);
    return launch_prep_t<__bf16, 64>(q, k, g, eta, eps, opts, t, n_seq, n_chunks_ub, H, G_out,
                                     beta_out, T_out, t_fp32, P_out, GD_out, pa, stream);
  }
  if (d_k == 128)
    return launch_prep_t<float, 128>(q, k, g, eta, eps, opts, t, n_seq, n_chunks_ub, H, G_out,
                                     beta_out, T_out, t_fp32, P_out, GD_out, pa, stream);
  return launch_prep_t<float, 64>(q, k, g, eta, eps, opts, t, n_seq, n_chunks_ub, H, G_out,
                                  beta_out, T_out, t_fp32, P_out, GD_out, pa, stream);
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
