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
// One workgroup of d_k / 32 wavefronts per (chunk, head); wavefront w owns the 32 key
// channels [32 w, 32 w + 32) and lane (r16, kq) the rows 16 I + r16 (I = 0..3) of channels
// 32 w + 8 kq .. + 7, which is the operand layout of one 16x16x32 matrix-core step.  So the
// sums over channels of A and P become matrix-core products once the decay is split between
// the two operands, with an anchor row a between the rows j < a <= i of every pair:
//   exp(G_i - G_j) = exp(G_i - G_a) exp(G_a - G_j),  both factors at most 1,
// so nothing overflows whatever the decay.  Off the diagonal 16 x 16 blocks the anchor is the
// first row of block I; within a diagonal block, the first row of each 4-row group (one
// product per group, the other rows masked to zero); the pairs within one 4-row group take
// exp(G_i - G_j) directly.  Each wavefront sums its 32 channels; the partial tiles meet in
// LDS.  bf16 operands are split into hi = bf16(x) and lo = bf16(x - hi) and multiplied as
// hi hi + hi lo + lo hi (about 2^-16 relative error, the precision of the fp32 sums they
// replace); fp32 operands use the fp32 matrix core.  Wavefront 0 then solves
// X = (I + Diag(b) A)^{-1} (the prep kernel's blocked solve) and writes T; wavefront 1
// writes P.
#include "kla_chunk.h"
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {

namespace {

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
  static constexpr int NW = DK / 32;
  union {
    // G within each 16-row block (prefix over the block's rows only), for the block totals
    // and the anchor rows; each wavefront reads back its own channels
    float Gb[kChunk][DK + 4];
    // partial tiles (ten 16 x 16 blocks each, one 16-byte piece per lane): A from wavefronts
    // 1 .. NW - 1, P from wavefronts 0, 2 .. NW - 1
    struct {
      f32x4 pa[NW - 1][10][64], pp[NW - 1][10][64];
    } t;
  } u;
  float nk[NW][kChunk], nq[NW][kChunk];  // partial squared norms of the key and query rows
  PrepSmem ps;                           // wavefront 0's solve
};

// one wavefront's LDS writes visible to its other lanes (LDS work of a wavefront is done in
// order; the fences keep the compiler from moving accesses across)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// x from the lane d lanes lower in the same 16-lane row, 0 for the first d lanes
__device__ __forceinline__ float row_shr(float x, int d) {
  const int v = __builtin_bit_cast(int, x);
  int r;
  switch (d) {
    case 1: r = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false); break;
    case 4: r = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false); break;
    default: r = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false); break;
  }
  return __builtin_bit_cast(float, r);
}
// x from lane m of the same group of four lanes
__device__ __forceinline__ float quad_bcast(float x, int m) {
  const int v = __builtin_bit_cast(int, x);
  int r;
  switch (m) {
    case 0: r = __builtin_amdgcn_update_dpp(0, v, 0x00, 0xF, 0xF, false); break;
    case 1: r = __builtin_amdgcn_update_dpp(0, v, 0x55, 0xF, 0xF, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, v, 0xAA, 0xF, 0xF, false); break;
    default: r = __builtin_amdgcn_update_dpp(0, v, 0xFF, 0xF, 0xF, false); break;
  }
  return __builtin_bit_cast(float, r);
}

// An operand of the 16 x 16 products over 32 channels: lane (r16, kq) holds row r16 at
// channels 8 kq .. + 7; bf16 inputs keep it as a hi/lo pair of bf16 fragments, fp32 inputs
// as fp32.
// masked(keep) is the operand or zero.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
template <typename Tin> struct Opnd;
template <> struct Opnd<__bf16> {
  u32x4 hi, lo;  // bf16 pairs
  __device__ __forceinline__ Opnd() {}
  __device__ __forceinline__ explicit Opnd(const float (&x)[8]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const f32x2_t x2 = {x[2 * p], x[2 * p + 1]};
      const unsigned h = __builtin_bit_cast(unsigned, __builtin_convertvector(x2, bf16x2_t));
      const f32x2_t l2 = {x[2 * p] - __builtin_bit_cast(float, h << 16),
                          x[2 * p + 1] - __builtin_bit_cast(float, h & 0xffff0000u)};
      hi[p] = h;
      lo[p] = __builtin_bit_cast(unsigned, __builtin_convertvector(l2, bf16x2_t));
    }
  }
  __device__ __forceinline__ Opnd masked(bool keep) const {
    Opnd r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      r.hi[p] = keep ? hi[p] : 0u;
      r.lo[p] = keep ? lo[p] : 0u;
    }
    return r;
  }
};
template <> struct Opnd<float> {
  float v[8];
  __device__ __forceinline__ Opnd() {}
  __device__ __forceinline__ explicit Opnd(const float (&x)[8]) {
#pragma unroll
    for (int s = 0; s < 8; ++s) v[s] = x[s];
  }
  __device__ __forceinline__ Opnd masked(bool keep) const {
    Opnd r;
#pragma unroll
    for (int s = 0; s < 8; ++s) r.v[s] = keep ? v[s] : 0.f;
    return r;
  }
};
// acc += a^T b in the 16x16 tile sense: D[4 kq + e][r16] = sum_c a[row 4 kq + e][c] b[row r16][c]
// (bf16: hi hi + hi lo + lo hi on 16x16x32 steps; fp32: eight exact 16x16x4 steps)
__device__ __forceinline__ f32x4 dot32(f32x4 acc, const Opnd<__bf16> &a, const Opnd<__bf16> &b) {
  const bf16x8 ah = __builtin_bit_cast(bf16x8, a.hi), al = __builtin_bit_cast(bf16x8, a.lo);
  const bf16x8 bh = __builtin_bit_cast(bf16x8, b.hi), bl = __builtin_bit_cast(bf16x8, b.lo);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 dot32(f32x4 acc, const Opnd<float> &a, const Opnd<float> &b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], acc, 0, 0, 0);
  return acc;
}
__device__ __forceinline__ void ld8(const float *p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 4);
  x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3]; x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}

template <typename T>
__device__ __forceinline__ void load_row8(const T *p, float (&x)[8]) {
  const typename Frag<T>::type v = load8<T>(p);
#pragma unroll
  for (int s = 0; s < 8; ++s) x[s] = to_f32(v[s]);
}
__device__ __forceinline__ void store_row8(float *p, const float (&x)[8]) {
  *reinterpret_cast<f32x4 *>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4 *>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}
__device__ __forceinline__ void store_row8(__bf16 *p, const float (&x)[8]) {
  bf16x8 b;
#pragma unroll
  for (int s = 0; s < 8; ++s) b[s] = from_f32<__bf16>(x[s]);
  *reinterpret_cast<bf16x8 *>(p) = b;
}

}  // namespace

template <typename Tin, int DK>
__global__ __launch_bounds__(DK * 2) __attribute__((amdgpu_waves_per_eu(2))) void kla_prep_diag_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ eta, float eps, CoefOpts opts, SeqTables tabs, int n_seq, int H,
    Tin *__restrict__ T_out, Tin *__restrict__ P_out, float *__restrict__ GD_out,
    Tin *__restrict__ KG_out, Tin *__restrict__ QG_out, Tin *__restrict__ KD_out,
    float *__restrict__ GC_out, Tin *__restrict__ X_out, Tin *__restrict__ A_out) {
  constexpr int NW = DK / 32;
  static_assert(NW >= 2, "wavefronts 0 and 1 finish the chunk");
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
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kq = lane >> 4;
  const int c0 = 32 * wid + 8 * kq;  // this lane's eight channels
  constexpr float kLog2e = 1.4426950408889634f;

  // ---- rows 16 I + r16 of k, q and g at this lane's channels (zeros past the chunk end)
  float kv[4][8], qv[4][8], G[4][8];
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    const int row = 16 * I + r16;
    if (row < len) {
      const size_t idx = ((size_t)(t0 + row) * H + h) * DK + c0;
      load_row8(k + idx, kv[I]);
      load_row8(q + idx, qv[I]);
      load_row8(g + idx, G[I]);
#pragma unroll
      for (int s = 0; s < 8; ++s) G[I][s] *= kLog2e;  // G in log2 units: exp(x) = exp2(x log2 e)
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) kv[I][s] = qv[I][s] = G[I][s] = 0.f;
    }
  }
  // ---- G: inclusive prefix over the tokens per channel, within each 16-row block across the
  //      16 lanes of a row group (parked in LDS: each block's total and anchor rows are read
  //      back from there), then the blocks' carries; rows past the end repeat G_last
#pragma unroll
  for (int I = 0; I < 4; ++I) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      float x = G[I][s];
      x += row_shr(x, 1);
      x += row_shr(x, 2);
      x += row_shr(x, 4);
      x += row_shr(x, 8);
      G[I][s] = x;
    }
    store_row8(&sm.u.Gb[16 * I + r16][c0], G[I]);
  }
  wave_lds_sync();  // a wavefront reads back only its own channels
  float carry[4][8];  // G at the row before each block
  float Gl[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) carry[0][s] = 0.f;
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    float tot[8];
    ld8(&sm.u.Gb[16 * I + 15][c0], tot);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      G[I][s] += carry[I][s];
      const float nx = carry[I][s] + tot[s];
      if (I < 3) carry[I + 1][s] = nx; else Gl[s] = nx;
    }
  }
  // G at row 16 I + a (a within the block) for this lane's channels
  auto anchor = [&](int I, int a, float (&x)[8]) {
    ld8(&sm.u.Gb[16 * I + a][c0], x);
#pragma unroll
    for (int s = 0; s < 8; ++s) x[s] += carry[I][s];
  };
  // ---- decayed tiles (all 64 rows) and exp(G_last)
  const size_t tile0 = (size_t)task * kChunk * DK;
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    float kg[8], qg[8], kd[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float e = exp2_fast(G[I][s]);
      kg[s] = kv[I][s] * e;
      qg[s] = qv[I][s] * e;
      kd[s] = kv[I][s] * exp2_fast(Gl[s] - G[I][s]);
    }
    const size_t off = tile0 + (size_t)(16 * I + r16) * DK + c0;
    store_row8(KG_out + off, kg);
    store_row8(QG_out + off, qg);
    store_row8(KD_out + off, kd);
  }
  if (r16 == 0) {
    float gc[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) gc[s] = exp2_fast(Gl[s]);
    store_row8(GC_out + (size_t)task * DK + c0, gc);
  }
  // ---- squared norms over this wavefront's channels
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      sk += kv[I][s] * kv[I][s];
      sq += qv[I][s] * qv[I][s];
    }
    sk += __shfl_xor(sk, 16, kWave);
    sk += __shfl_xor(sk, 32, kWave);
    sq += __shfl_xor(sq, 16, kWave);
    sq += __shfl_xor(sq, 32, kWave);
    if (kq == 0) {
      sm.nk[wid][16 * I + r16] = sk;
      sm.nq[wid][16 * I + r16] = sq;
    }
  }

  // ---- A and P over this wavefront's channels, ten 16 x 16 blocks each (lower_block order
  //      b = I (I + 1) / 2 + J).  Each product is formed transposed (right factor as the left
  //      operand) so that lane (r16, kq) ends with row 16 I + r16, columns 16 J + 4 kq + e.
  f32x4 Aa[10], Pa[10];
#pragma unroll
  for (int b = 0; b < 10; ++b) Aa[b] = Pa[b] = zero4();
  // One anchor for the whole chunk, row 32, when on every channel of this wavefront every row
  // is within kSpan (log2 units) of row 32: then L_i = k_i 2^(G_i - G_32) and
  // R_j = k_j 2^(G_32 - G_j) stay within 2^-kSpan .. 2^kSpan times k (normal numbers), each
  // tile is one product of them, and the entries above the diagonal are dropped.  Otherwise
  // the blockwise anchors below, whose factors are all at most 1, whatever the decay.
  constexpr float kSpan = 64.f;
  float G32[8];
  bool fast;
  {
    anchor(2, 0, G32);
    float span = 0.f;
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int s = 0; s < 8; ++s) span = fmaxf(span, fabsf(G[I][s] - G32[s]));
    fast = __all(span <= kSpan);
  }
  if (fast) {
    // every operand first (the rows' k, q and G are dead after), then the products
    Opnd<Tin> oR[4], oL[4], oLq[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      float L[8], Lq[8], R[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float d = G[I][s] - G32[s];
        const float e = exp2_fast(d);
        L[s] = kv[I][s] * e;
        Lq[s] = qv[I][s] * e;
        R[s] = kv[I][s] * exp2_fast(-d);
      }
      oR[I] = Opnd<Tin>(R);
      oL[I] = Opnd<Tin>(L);
      oLq[I] = Opnd<Tin>(Lq);
    }
#pragma unroll
    for (int I = 0; I < 4; ++I) {
#pragma unroll
      for (int J = 0; J <= I; ++J) {
        const int b = I * (I + 1) / 2 + J;
        Aa[b] = dot32(Aa[b], oR[J], oL[I]);
        Pa[b] = dot32(Pa[b], oR[J], oLq[I]);
      }
      // the diagonal block: keep column < row for A, column <= row for P
      const int bII = I * (I + 1) / 2 + I;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = 4 * kq + e;
        Aa[bII][e] = col < r16 ? Aa[bII][e] : 0.f;
        Pa[bII][e] = col <= r16 ? Pa[bII][e] : 0.f;
      }
    }
  } else {
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    const int bII = I * (I + 1) / 2 + I;
    // blocks J < I, anchored at row 16 I
    if (I > 0) {
      float Ga[8], L[8], Lq[8];
      anchor(I, 0, Ga);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float e = exp2_fast(G[I][s] - Ga[s]);
        L[s] = kv[I][s] * e;
        Lq[s] = qv[I][s] * e;
      }
      const Opnd<Tin> oL(L), oLq(Lq);
#pragma unroll
      for (int J = 0; J < I; ++J) {
        float R[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) R[s] = kv[J][s] * exp2_fast(Ga[s] - G[J][s]);
        const Opnd<Tin> oR(R);
        const int b = I * (I + 1) / 2 + J;
        Aa[b] = dot32(Aa[b], oR, oL);
        Pa[b] = dot32(Pa[b], oR, oLq);
      }
    }
    // the diagonal block: pairs in different 4-row groups, anchored at the first row of the
    // later group (rows of other groups masked to zero in each product)
    const int grp = r16 >> 2;
    float Lo[8], Lqo[8];  // k_i and q_i times exp(G_i - G at the first row of their group)
    {
      float Go[8];
      ld8(&sm.u.Gb[16 * I + 4 * grp][c0], Go);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float e = exp2_fast(G[I][s] - (Go[s] + carry[I][s]));
        Lo[s] = kv[I][s] * e;
        Lqo[s] = qv[I][s] * e;
      }
    }
    const Opnd<Tin> oLo(Lo), oLqo(Lqo);
#pragma unroll
    for (int s4 = 1; s4 < 4; ++s4) {
      float Gs[8], R[8];
      anchor(I, 4 * s4, Gs);
#pragma unroll
      for (int s = 0; s < 8; ++s) R[s] = kv[I][s] * exp2_fast(Gs[s] - G[I][s]);
      const Opnd<Tin> oR = Opnd<Tin>(R).masked(grp < s4);
      Aa[bII] = dot32(Aa[bII], oR, oLo.masked(grp == s4));
      Pa[bII] = dot32(Pa[bII], oR, oLqo.masked(grp == s4));
    }
    // pairs within one 4-row group, directly: row i = 16 I + r16 against rows
    // 16 I + 4 grp + m of its group (m <= r16 % 4), summed over the lane groups
    float a4[4] = {0.f, 0.f, 0.f, 0.f}, p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float Gj = quad_bcast(G[I][s], m), kj = quad_bcast(kv[I][s], m);
        const float t = m <= (r16 & 3) ? kj * exp2_fast(G[I][s] - Gj) : 0.f;
        if (m < (r16 & 3)) a4[m] += kv[I][s] * t;
        p4[m] += qv[I][s] * t;
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      a4[m] += __shfl_xor(a4[m], 16, kWave);
      a4[m] += __shfl_xor(a4[m], 32, kWave);
      p4[m] += __shfl_xor(p4[m], 16, kWave);
      p4[m] += __shfl_xor(p4[m], 32, kWave);
    }
    if (kq == grp) {  // entry (16 I + r16, 16 I + 4 grp + m) sits in lane (r16, grp), e = m
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        Aa[bII][m] += a4[m];
        Pa[bII][m] += p4[m];
      }
    }
  }
  }

  // ---- the partial tiles meet (in the LDS of the G staging, once every wavefront is past
  //      it): wavefront 0 sums A, wavefront 1 sums P
  __syncthreads();
  if (wid != 0) {
#pragma unroll
    for (int b = 0; b < 10; ++b) sm.u.t.pa[wid - 1][b][lane] = Aa[b];
  }
  if (wid != 1) {
#pragma unroll
    for (int b = 0; b < 10; ++b) sm.u.t.pp[wid == 0 ? 0 : wid - 1][b][lane] = Pa[b];
  }
  __syncthreads();
  if (wid >= 2) return;
  const int i = lane;  // per-token work: token `lane`
  if (wid == 1) {
    // P = Diag(rq) P as ten packed blocks; unit gam and dec for the scan (the decay sits in
    // the tiles) and the readout factor rq as gamO
#pragma unroll
    for (int w = 0; w < NW - 1; ++w)
#pragma unroll
      for (int b = 0; b < 10; ++b) Pa[b] += sm.u.t.pp[w][b][lane];
    float qq = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) qq += sm.nq[w][i];
    const float rq_i = opts.normalize_q ? (qq > 0.f ? 1.f / sqrtf(qq) : 0.f) : 1.f;
    const size_t gd0 = (size_t)task * kGDFloats;
    GD_out[gd0 + i] = 1.f;
    GD_out[gd0 + kChunk + i] = 1.f;
    GD_out[gd0 + 2 * kChunk + i] = rq_i;
    Tin *P_task = P_out + (size_t)task * kTpbElems;
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const float rr = __shfl(rq_i, 16 * I + r16, kWave);
#pragma unroll
      for (int J = 0; J <= I; ++J) {
        const f32x4 pv = Pa[I * (I + 1) / 2 + J];
        out_put<Tin>(P_task, true, 16 * I + r16, 16 * J + 4 * kq, rr * pv[0], rr * pv[1],
                     rr * pv[2], rr * pv[3]);
      }
    }
    return;
  }
  // wavefront 0: b, L = Diag(b) A, and the solve
#pragma unroll
  for (int w = 0; w < NW - 1; ++w)
#pragma unroll
    for (int b = 0; b < 10; ++b) Aa[b] += sm.u.t.pa[w][b][lane];
  if (A_out) {  // the backward pass: A itself (packed blocks, zero on the diagonal)
    Tin *A_task = A_out + (size_t)task * kTpbElems;
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int J = 0; J <= I; ++J) {
        const f32x4 av = Aa[I * (I + 1) / 2 + J];
        out_put<Tin>(A_task, true, 16 * I + r16, 16 * J + 4 * kq, av[0], av[1], av[2], av[3]);
      }
  }
  {
    float kk = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) kk += sm.nk[w][i];
    float bi = 0.f;
    if (i < len) {
      const size_t th = (size_t)(t0 + i) * H + h;
      const float t_abs = (float)(t0 + i - ts + 1 + (opts.pos_offset ? opts.pos_offset[n] : 0));
      bi = write_coef(opts.beta_mode, eta[th], kk + eps, t_abs);
    }
    sm.ps.beta[i] = bi;
  }
  wave_lds_sync();
  f32x4 Lr[4][3];
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    const float bme = sm.ps.beta[16 * I + r16];
#pragma unroll
    for (int J = 0; J < I; ++J) Lr[I][J] = Aa[I * (I + 1) / 2 + J] * bme;
    *reinterpret_cast<f32x4 *>(&sm.ps.Ld[I][bidx(r16, 4 * kq)]) = Aa[I * (I + 1) / 2 + I] * bme;
  }
  wave_lds_sync();
  Tin *T_task = T_out + (size_t)task * kTpbElems;
  Tin *X_task = X_out ? X_out + (size_t)task * kTpbElems : nullptr;
  chunk_inverse<false>(Lr, sm.ps, [] { wave_lds_sync(); },
                       [&](int row, int col, const f32x4 &x, const f32x4 &bv) {
                         out_put<Tin>(T_task, true, row, col, x[0] * bv[0], x[1] * bv[1],
                                      x[2] * bv[2], x[3] * bv[3]);
                         if (X_task) out_put<Tin>(X_task, true, row, col, x[0], x[1], x[2], x[3]);
                       });
}

template <typename Tin, int DK>
static hipError_t launch_prep_diag_t(const void *q, const void *k, const float *g,
                                     const float *eta, float eps, const CoefOpts &opts,
                                     SeqTables t, int32_t n_seq, int64_t n_chunks_ub, int32_t H,
                                     const DiagTiles &dt, void *T_out, void *P_out,
                                     float *GD_out, void *X_out, void *A_out,
                                     hipStream_t stream) {
  const size_t smem = sizeof(DiagSmem<DK>);
  static_assert(sizeof(DiagSmem<DK>) <= 80 * 1024, "two workgroups to a compute unit");
  static std::atomic<bool> attr_set[kMaxDeviceOrdinals];
  if (hipError_t ea = set_lds_limit_once(
          reinterpret_cast<const void *>(&kla_prep_diag_kernel<Tin, DK>), (int)smem, attr_set);
      ea != hipSuccess)
    return ea;
  const int64_t blocks = n_chunks_ub * H;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((kla_prep_diag_kernel<Tin, DK>), dim3((unsigned)blocks), dim3(DK * 2),
                     smem, stream, static_cast<const Tin *>(q), static_cast<const Tin *>(k), g,
                     eta, eps, opts, t, n_seq, H, static_cast<Tin *>(T_out),
                     static_cast<Tin *>(P_out), GD_out,
                     static_cast<Tin *>(const_cast<void *>(dt.kg)),
                     static_cast<Tin *>(const_cast<void *>(dt.qg)),
                     static_cast<Tin *>(const_cast<void *>(dt.kd)), const_cast<float *>(dt.gc),
                     static_cast<Tin *>(X_out), static_cast<Tin *>(A_out));
  return hipGetLastError();
}

hipError_t launch_prep_diag(Dtype dt, int d_k, const void *q, const void *k, const float *g,
                            const float *eta, float eps, const CoefOpts &opts, SeqTables t,
                            int32_t n_seq, int64_t n_chunks_ub, int32_t H, const DiagTiles &tiles,
                            void *T_out, void *P_out, float *GD_out, hipStream_t stream,
                            void *X_out, void *A_out) {
#define KLA_PREP_DIAG(TIN, DK_)                                                                \
  return launch_prep_diag_t<TIN, DK_>(q, k, g, eta, eps, opts, t, n_seq, n_chunks_ub, H, tiles, \
                                      T_out, P_out, GD_out, X_out, A_out, stream);
  if (dt == Dtype::BF16) {
    if (d_k == 128) { KLA_PREP_DIAG(__bf16, 128) }
    KLA_PREP_DIAG(__bf16, 64)
  }
  if (d_k == 128) { KLA_PREP_DIAG(float, 128) }
  KLA_PREP_DIAG(float, 64)
#undef KLA_PREP_DIAG
}

}  // namespace kla
