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
#include "kla_chunk.h"
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

// Where chunk c of the packed input lies: sequence n, the sequence's first token ts, the
// chunk's first token t0 and its length.  Three ways to get there (PlanMode):
//  - kPlanTables: the tables the plan kernel wrote;
//  - kPlanDense:  equal-length sequences (no offsets given), pure arithmetic;
//  - kPlanWave:   at most 63 sequences: every wavefront sanitises the offsets and counts
//                 chunks itself, one sequence per lane, exactly as the plan kernel does.
// In the last two modes the prep kernel also writes the tables, for the scan.
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

struct Planner {
  int mode, n_seq, n_chunks;
  int L, cpc;   // kPlanDense: sequence length, chunks per sequence
  int cs, co;   // kPlanWave: offset and first chunk of sequence `lane`
  SeqTables tabs;
};

__device__ __forceinline__ Planner make_planner(const PlanArgs &pa, SeqTables tabs, int n_seq) {
  Planner p;
  p.mode = pa.mode;
  p.n_seq = n_seq;
  p.tabs = tabs;
  p.L = p.cpc = p.cs = p.co = 0;
  const int lane = threadIdx.x & 63;
  if (pa.mode == kPlanDense) {
    p.L = pa.total / n_seq;
    p.cpc = (p.L + kChunk - 1) / kChunk;
    p.n_chunks = n_seq * p.cpc;
  } else if (pa.mode == kPlanWave) {
    // lane e holds offset e: running maximum of the clamped offsets, then chunk counts
    const int raw = lane <= n_seq ? min(max(pa.cu_in[lane], 0), pa.total) : pa.total;
    p.cs = wave_max_scan_i(raw, lane);
    const int nxt = __shfl(p.cs, min(lane + 1, kWave - 1), kWave);
    const int cnt = lane < n_seq ? (nxt - p.cs + kChunk - 1) / kChunk : 0;
    p.co = wave_sum_scan_i(cnt, lane) - cnt;  // exclusive: chunk_off[lane]
    p.n_chunks = __shfl(p.co, n_seq, kWave);
  } else {
    p.n_chunks = tabs.chunk_off[n_seq];
  }
  return p;
}

// Tables for the scan, in the modes where no plan kernel ran (every thread of the grid
// takes a share; entries n = 0..n_seq).
__device__ __forceinline__ void write_tables(const Planner &p) {
  const int tid = threadIdx.x;
  if (p.mode == kPlanDense) {
    for (int e = blockIdx.x * (int)blockDim.x + tid; e <= p.n_seq;
         e += gridDim.x * (int)blockDim.x) {
      p.tabs.cu[e] = e * p.L;
      p.tabs.chunk_off[e] = e * p.cpc;
    }
  } else if (p.mode == kPlanWave) {
    if (blockIdx.x == 0 && tid <= p.n_seq) {  // wavefront 0 (n_seq < 64)
      p.tabs.cu[tid] = p.cs;
      p.tabs.chunk_off[tid] = p.co;
    }
  }
}

// Chunk c < n_chunks.
__device__ __forceinline__ ChunkLoc locate(const Planner &p, int c) {
  ChunkLoc loc;
  if (p.mode == kPlanDense) {
    loc.n = c / p.cpc;
    loc.ts = loc.n * p.L;
    loc.t0 = loc.ts + (c - loc.n * p.cpc) * kChunk;
    loc.len = min(kChunk, loc.ts + p.L - loc.t0);
  } else if (p.mode == kPlanWave) {
    const int lane = threadIdx.x & 63;
    const unsigned long long below = __ballot(lane < p.n_seq && p.co <= c);
    loc.n = __popcll(below) - 1;
    loc.ts = __shfl(p.cs, loc.n, kWave);
    loc.t0 = loc.ts + (c - __shfl(p.co, loc.n, kWave)) * kChunk;
    loc.len = min(kChunk, __shfl(p.cs, loc.n + 1, kWave) - loc.t0);
  } else {
    loc.n = find_sequence(p.tabs.chunk_off, p.n_seq, c);
    loc.ts = p.tabs.cu[loc.n];
    loc.t0 = loc.ts + (c - p.tabs.chunk_off[loc.n]) * kChunk;
    loc.len = min(kChunk, p.tabs.cu[loc.n + 1] - loc.t0);
  }
  return loc;
}

// ---------------------------------------------------------------------------------------------
// Prep / UT kernel: one wavefront per (chunk, head), no workgroup barriers.
//
// The wavefront holds the chunk's 64 key rows (and query rows) in registers as MFMA
// fragments, four 16-row blocks.  A row-major key block is both the A fragment of its rows
// and the B fragment of K^T, so every Gram tile and every Q K^T tile is a product of two
// register fragments; taking them as K_j K_i^T (the transpose of the wanted tile) leaves
// lane (r16, kg) with row 16 i + r16, columns 16 j + 4 kg + e -- four consecutive entries
// of one row, which is both the A-operand layout of the fp32 MFMA and a row-contiguous
// store.  With L = Diag(b) (A^- o K K^T) and X = (I + L)^{-1} (unit lower triangular):
//  - the diagonal blocks X_kk by substitution out of LDS (lane group kg inverts block kg,
//    one column per lane);
//  - the sub-diagonal blocks by distance, X_ij = -X_ii Y with Y = sum_{k=j}^{i-1} L_ik X_kj,
//    on the fp32 matrix cores with the L blocks straight from registers, and formed
//    transposed (X_ij^T = Y^T X_ii^T) so that each lane ends with row entries of X_ij;
//  - T = X Diag(b) stored from those registers.
// When q is given the kernel also writes P = (A o Q K^T) (Eq. (8)'s intra-chunk matrix,
// A_ij = exp(G_i - G_j) for j <= i, zero above the diagonal) for the scan.
// ---------------------------------------------------------------------------------------------

// bf16 key or query rows of one chunk as MFMA fragments f[b][ks] (rows 16 b + r16, k-step
// ks), loaded as whole 128-byte lines: for each block and line c, one load covers rows
// 16 b + 0..7 and one rows 16 b + 8..15, lane (r16, kg) taking row r16 % 8 and 16-byte
// unit kg + 4 (r16 / 8) of the line.  Exchanging lanes 8..15 of every 16-lane row between
// the two loads (a row_ror:8 DPP move) leaves the fragments of k-steps 2 c and 2 c + 1.
template <int NKS>
__device__ __forceinline__ void load_rows_bf16(bf16x8 (&f)[4][NKS], Rsrc r, int rowb, int r16,
                                               int kg) {
  const int vrow = (r16 & 7) * rowb + 16 * (kg + 4 * (r16 >> 3));
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int c = 0; c < NKS / 2; ++c) {
      const u32x4 X = __builtin_amdgcn_raw_buffer_load_b128(r, vrow + 16 * b * rowb + 128 * c, 0, 0);
      const u32x4 Y =
          __builtin_amdgcn_raw_buffer_load_b128(r, vrow + (16 * b + 8) * rowb + 128 * c, 0, 0);
      u32x4 F0, F1;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        F0[d] = (unsigned)__builtin_amdgcn_update_dpp((int)X[d], (int)Y[d], 0x128, 0xF, 0xC, false);
        F1[d] = (unsigned)__builtin_amdgcn_update_dpp((int)Y[d], (int)X[d], 0x128, 0xF, 0x3, false);
      }
      f[b][2 * c] = __builtin_bit_cast(bf16x8, F0);
      f[b][2 * c + 1] = __builtin_bit_cast(bf16x8, F1);
    }
}

template <typename Tin, int DK, typename TOut>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(sizeof(Tin) * DK > 256 ? 1 : 2))) void kla_prep_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ eta, float eps, int32_t *__restrict__ cu,
    int32_t *__restrict__ chunk_off, int n_seq, int H, float *__restrict__ G_out,
    float *__restrict__ beta_out, TOut *__restrict__ T_out, Tin *__restrict__ P_out,
    float *__restrict__ GD_out, CoefOpts opts, PlanArgs pa, int tp_split,
    Tin *__restrict__ X_out, float *__restrict__ LC_out) {
  __shared__ PrepSmem sm;
  const Planner pl = make_planner(pa, SeqTables{cu, chunk_off}, n_seq);
  write_tables(pl);
  // task = chunk * H + head, in workgroup order.  (Grouping the heads of a chunk on one XCD
  // fetches each g and eta line once instead of once per XCD, 136 instead of 151 MB read on
  // a 4 x 16 x 4096-token prefill, but made the kernel 8% slower there.)
  const int task = blockIdx.x;
  if (task >= pl.n_chunks * H) return;
  const int c = __builtin_amdgcn_readfirstlane(task / H);
  const int h = __builtin_amdgcn_readfirstlane(task - c * H);
  ChunkLoc loc = locate(pl, c);
  // wave-uniform by construction; said so, so that buffer descriptors stay in SGPRs
  loc.n = __builtin_amdgcn_readfirstlane(loc.n);
  loc.ts = __builtin_amdgcn_readfirstlane(loc.ts);
  loc.t0 = __builtin_amdgcn_readfirstlane(loc.t0);
  loc.len = __builtin_amdgcn_readfirstlane(loc.len);
  const int t0 = loc.t0, len = loc.len;
  const int lane = threadIdx.x, r16 = lane & 15, kg = lane >> 4;
  const bool want_p = (q != nullptr) && (P_out != nullptr);
  constexpr int NKS = DK / 32;
  constexpr float kLog2e = 1.4426950408889634f;
  using FragT = typename Frag<Tin>::type;

  // ---- loads through range-checked buffers (rows past the chunk end read as zeros): key
  //      (and query) rows 16 b + r16 as fragments, g and eta one token per lane
  constexpr int ES = sizeof(Tin);
  const int rowb = H * DK * ES;  // bytes between consecutive tokens
  const size_t off0 = ((size_t)t0 * H + h) * DK;
  const uint32_t kq_bytes = (uint32_t)((len - 1) * rowb + DK * ES);
  FragT kf[4][NKS], qf[4][NKS];
  {
    const Rsrc rk = make_rsrc(k + off0, kq_bytes);
    if constexpr (ES == 2) {
      load_rows_bf16<NKS>(kf, rk, rowb, r16, kg);
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          kf[b][ks] = bload8<Tin>(rk, (16 * b + r16) * rowb + (32 * ks + 8 * kg) * ES);
    }
    if (want_p) {
      const Rsrc rq = make_rsrc(q + off0, kq_bytes);
      if constexpr (ES == 2) {
        load_rows_bf16<NKS>(qf, rq, rowb, r16, kg);
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
            qf[b][ks] = bload8<Tin>(rq, (16 * b + r16) * rowb + (32 * ks + 8 * kg) * ES);
      }
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[b][ks] = zero8<Tin>();
    }
  }
  const bool tok_ok = lane < len;
  const size_t th = (size_t)(t0 + (tok_ok ? lane : 0)) * H + h;
  const uint32_t ge_bytes = (uint32_t)(((len - 1) * H + 1) * 4);
  const float g_l = bload1(make_rsrc(g + (size_t)t0 * H + h, ge_bytes), lane * H * 4);
  const float eta_l = bload1(make_rsrc(eta + (size_t)t0 * H + h, ge_bytes), lane * H * 4);

  // ---- G (token `lane`; rows past the end carry G_last)
  const float G_l = wave_inclusive_scan(g_l, lane);
  const size_t gd0 = (size_t)task * kGDFloats;
  if (GD_out) {
    const float Glast = __shfl(G_l, kChunk - 1, kWave);
    GD_out[gd0 + lane] = __expf(G_l);
    GD_out[gd0 + kChunk + lane] = __expf(Glast - G_l);
  }
  if (tok_ok && G_out) G_out[th] = G_l;
  sm.G2[lane] = G_l * kLog2e;

  // ---- diagonal Gram tiles K_i K_i^T; their diagonals are the squared key norms (and, under
  //      the normalised readout, Q_i Q_i^T gives the squared query norms).  Row 16 i + r16's
  //      diagonal element sits in lane (r16, r16 / 4), entry r16 % 4.
  f32x4 gd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    gd[i] = zero4();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) gd[i] = mma(kf[i][ks], kf[i][ks], gd[i]);
  }
  const int dsrc = r16 + 16 * (r16 >> 2);  // the lane holding row r16's diagonal element
  const int de = r16 & 3;
  const int pos0 = t0 - loc.ts + 1 + (opts.pos_offset ? opts.pos_offset[loc.n] : 0);
  float rqv[4], bme[4], G2me[4];  // per own row 16 i + r16: 1/||q||, b, G log2(e)
  float lexp = 0.f;  // this lane's rows' ln max(1, |1 - b ||k||^2|) (lane group 0)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * i + r16;
    const float ss = de == 0 ? gd[i][0] : de == 1 ? gd[i][1] : de == 2 ? gd[i][2] : gd[i][3];
    const float eta_r = __shfl(eta_l, row, kWave);
    const float G_r = __shfl(G_l, row, kWave);
    float b_r = row < len ? write_coef(opts.beta_mode, eta_r, ss + eps, (float)(pos0 + row)) : 0.f;
    b_r = __shfl(b_r, dsrc, kWave);  // the diagonal lane's value, on all four lane groups
    bme[i] = b_r;
    if (LC_out) {
      const float bk = b_r * __shfl(ss, dsrc, kWave);  // b ||k||^2 of this row
      if (kg == 0) lexp += logf(fmaxf(1.f, fabsf(1.f - bk)));
    }
    G2me[i] = G_r * kLog2e;
    rqv[i] = 1.f;
    if (opts.normalize_q) {  // 1 / ||q|| (0 for a zero query)
      f32x4 qd = zero4();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qd = mma(qf[i][ks], qf[i][ks], qd);
      const float qq = __shfl(de == 0 ? qd[0] : de == 1 ? qd[1] : de == 2 ? qd[2] : qd[3], dsrc,
                              kWave);
      rqv[i] = qq > 0.f ? __builtin_amdgcn_rsqf(qq) : 0.f;
    }
    if (kg == 0) {
      sm.beta[row] = b_r;
      if (GD_out) GD_out[gd0 + 2 * kChunk + row] = __expf(G_r) * rqv[i];
      if (beta_out && row < len) beta_out[(size_t)(t0 + row) * H + h] = b_r;
    }
  }
  // the chunk's contraction bound: the homogeneous map S -> S' of its tokens has spectral norm
  // at most prod_t a_t max(1, |1 - b_t ||k_t||^2|) (each token's map is a_t (I - b_t k_t^T k_t),
  // symmetric); its natural log, for the two-level scan's warm-up test
  if (LC_out) {
    const float lsum = wave_sum(lexp), glast = __shfl(G_l, kChunk - 1, kWave);
    if (lane == 0) LC_out[task] = glast + lsum;
  }
  lds_barrier();

  // ---- P = A o Q K^T from the tiles K_j Q_i^T (row 16 i + r16, columns 16 j + 4 kg + e;
  //      zero above the diagonal)
  if (want_p) {
    Tin *P_task = P_out + (size_t)task * (tp_split ? 2 * kTpbElems : kTpbElems);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int prow = 16 * i + r16;
#pragma unroll
      for (int j = 0; j <= i; ++j) {
        const int j0 = 16 * j + 4 * kg;
        f32x4 accp = zero4();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) accp = mma(kf[j][ks], qf[i][ks], accp);
        const f32x4 Gc = *reinterpret_cast<const f32x4 *>(&sm.G2[j0]);
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool keep = (j < i) || (4 * kg + e <= r16);
          pv[e] = exp2_fast(keep ? G2me[i] - Gc[e] : -INFINITY) * accp[e] * rqv[i];
        }
        out_put<Tin>(P_task, true, prow, j0, pv[0], pv[1], pv[2], pv[3], tp_split != 0);
      }
    }
  }

  // ---- T = (I + L)^{-1} Diag(b), written as the scan's packed blocks (with the decays) or
  //      in full (the unit-check stage, blocks above the diagonal zero)
  const bool t_packed = GD_out != nullptr;
  TOut *T_task =
      T_out + (size_t)task * (t_packed ? (tp_split ? 2 : 1) * kTpbElems : kChunk * kChunk);
  if (!t_packed) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = i + 1; j < 4; ++j)
        out_put<TOut>(T_task, false, 16 * i + r16, 16 * j + 4 * kg, 0.f, 0.f, 0.f, 0.f);
  }
  Tin *X_task = X_out ? X_out + (size_t)task * kTpbElems : nullptr;
  chunk_T<Tin, NKS, false>(
      kf, gd, bme, G2me, sm, [] { lds_barrier(); },
      [&](int row, int col, const f32x4 &x, const f32x4 &bv) {
        out_put<TOut>(T_task, t_packed, row, col, x[0] * bv[0], x[1] * bv[1], x[2] * bv[2],
                      x[3] * bv[3], tp_split != 0);
        if (X_task) out_put<Tin>(X_task, true, row, col, x[0], x[1], x[2], x[3]);
      });
}

template <typename Tin, int DK>
static hipError_t launch_prep_t(const void *q, const void *k, const float *g, const float *eta,
                                float eps, const CoefOpts &opts, SeqTables t, int32_t n_seq,
                                int64_t n_chunks_ub, int32_t H, float *G_out, float *beta_out,
                                void *T_out, bool t_fp32, void *P_out, float *GD_out,
                                const PlanArgs &pa, hipStream_t stream, bool tp_split,
                                void *X_out, float *LC_out) {
  if (n_chunks_ub <= 0 || H <= 0) return hipSuccess;
  if (tp_split && (sizeof(Tin) != 2 || t_fp32 || !GD_out)) return hipErrorInvalidValue;
  const int64_t tasks = n_chunks_ub * H;
  if (tasks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tasks);
  const Tin *qq = static_cast<const Tin *>(q);
  Tin *pp = static_cast<Tin *>(P_out);
  if (t_fp32 || sizeof(Tin) == 4)
    hipLaunchKernelGGL((kla_prep_kernel<Tin, DK, float>), grid, dim3(64), 0, stream, qq,
                       static_cast<const Tin *>(k), g, eta, eps, t.cu, t.chunk_off, n_seq, H,
                       G_out, beta_out, static_cast<float *>(T_out), pp, GD_out, opts, pa, 0,
                       static_cast<Tin *>(X_out), LC_out);
  else
    hipLaunchKernelGGL((kla_prep_kernel<Tin, DK, Tin>), grid, dim3(64), 0, stream, qq,
                       static_cast<const Tin *>(k), g, eta, eps, t.cu, t.chunk_off, n_seq, H,
                       G_out, beta_out, static_cast<Tin *>(T_out), pp, GD_out, opts, pa,
                       tp_split ? 1 : 0, static_cast<Tin *>(X_out), LC_out);
  return hipGetLastError();
}

hipError_t launch_prep(Dtype dt, int d_k, const void *q, const void *k, const float *g,
                       const float *eta, float eps, const CoefOpts &opts, SeqTables t,
                       int32_t n_seq, int64_t n_chunks_ub, int32_t H, float *G_out,
                       float *beta_out, void *T_out, bool t_fp32, void *P_out, float *GD_out,
                       const PlanArgs &pa, hipStream_t stream, bool tp_split, void *X_out,
                       float *LC_out) {
  if (dt == Dtype::BF16) {
    if (d_k == 128)
      return launch_prep_t<__bf16, 128>(q, k, g, eta, eps, opts, t, n_seq, n_chunks_ub, H, G_out,
                                        beta_out, T_out, t_fp32, P_out, GD_out, pa, stream,
                                        tp_split, X_out, LC_out);
    return launch_prep_t<__bf16, 64>(q, k, g, eta, eps, opts, t, n_seq, n_chunks_ub, H, G_out,
                                     beta_out, T_out, t_fp32, P_out, GD_out, pa, stream, tp_split,
                                  X_out, LC_out);
  }
  if (d_k == 128)
    return launch_prep_t<float, 128>(q, k, g, eta, eps, opts, t, n_seq, n_chunks_ub, H, G_out,
                                     beta_out, T_out, t_fp32, P_out, GD_out, pa, stream, tp_split,
                                  X_out, LC_out);
  return launch_prep_t<float, 64>(q, k, g, eta, eps, opts, t, n_seq, n_chunks_ub, H, G_out,
                                  beta_out, T_out, t_fp32, P_out, GD_out, pa, stream, tp_split,
                                  X_out, LC_out);
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
