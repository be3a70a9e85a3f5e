// kla_scan.hip -- inter-chunk state scan with the chunk output fused in.
//
// Paper "Kaczmarz Linear Attention" (arXiv 2605.08587), section 4, Propositions 3
// and 4.  With the per-chunk T = (I + L)^{-1} Diag(b) and chunk-local log-decay G
// from the prep stage, each chunk of a (sequence, head) is, given its incoming
// state S (d_k x d_v, fp32):
//   U     = T (V - Diag(exp G) K S)                      Eq. (7)
//   O     = Diag(exp G) Q S + (A o Q K^T) U              Eq. (8), A_ij = exp(G_i - G_j), j <= i
//   S_out = exp(G_last) S + K^T Diag(exp(G_last - G)) U  Eq. (9)
// and S_out is the next chunk's S.  The chunks of one sequence are processed in
// order by one workgroup; the d_v columns of S are independent given K, G and T,
// so a (sequence, head) is split over d_v / 32 workgroups.
//
// Work split inside the workgroup (4 wavefronts, BV = 32 state columns):
//   wave w owns chunk rows [16 w, 16 w + 16) for K S, Q S, Q K^T, T R and P U,
//   and state rows [w d_k / 4, (w + 1) d_k / 4) for the K^T U update, which it
//   keeps in fp32 accumulator registers for the whole sequence.
// Operands another wave needs go through LDS in the layout its MFMA fragments
// read: keys token-major and transposed, the state / R / U transposed (column-major).
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {

constexpr int kBV = 32;  // state columns per workgroup

// LDS-only workgroup barrier: orders LDS traffic without waiting for the global
// loads that are deliberately left in flight (the next chunk's prefetch).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Chunk operands are double-buffered in LDS unless that would not fit (fp32, d_k = 128).
template <typename Tin, int DK>
constexpr int scan_nbuf() { return (sizeof(Tin) == 4 && DK == 128) ? 1 : 2; }

template <typename Tin, int DK, int NBUF>
struct ScanSmem {
  static constexpr int PAD = 8;
  alignas(16) Tin K[NBUF][kChunk][DK + PAD];     // chunk keys, token-major
  alignas(16) Tin Kt[NBUF][DK][kChunk + PAD];    // chunk keys, transposed
  alignas(16) Tin V[NBUF][kChunk][kBV + PAD];    // value slice
  alignas(16) float G[NBUF][kChunk];             // chunk-local log-decay (tail repeats G[len-1])
  alignas(16) Tin St[kBV][DK + PAD];             // state operand copy, column-major
  alignas(16) Tin Rt[kBV][kChunk + PAD];         // R = V - Diag(gamma) K S, column-major
  alignas(16) Tin Ut[kBV][kChunk + PAD];         // U, column-major
  alignas(16) Tin Udt[kBV][kChunk + PAD];        // Diag(exp(G_last - G)) U, column-major
  alignas(16) Tin P[kChunk][kChunk + PAD];       // A o Q K^T, row-major
};

// Per-thread registers holding one chunk's operands between its global load and its use.
template <typename Tin, int DK>
struct ChunkRegs {
  typename Frag<Tin>::type kr[DK / 32];  // key row `lane`, 8-element groups wid + 4 j
  typename Frag<Tin>::type vr;           // value slice row tid / 4, group tid % 4
  typename Frag<Tin>::type aq[DK / 32];  // this wave's query rows as MFMA A fragments
  f32x8 tr[2];                           // this wave's T rows as fp32 A fragments
  float gr;                              // G of row tid (tid < 64)
};

template <typename Tin, int DK>
__global__ __launch_bounds__(256) void kla_scan_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const float *__restrict__ Gtok, const float *__restrict__ Tm, const float *S0,
    Tin *__restrict__ o, float *S_T, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, int n_seq, int H, int DV) {
  constexpr int NBUF = scan_nbuf<Tin, DK>();
  extern __shared__ __align__(16) unsigned char smem_raw[];
  ScanSmem<Tin, DK, NBUF> &sm = *reinterpret_cast<ScanSmem<Tin, DK, NBUF> *>(smem_raw);
  using FragT = typename Frag<Tin>::type;

  // XCD-aware mapping: workgroup b runs on XCD b % 8; give the d_v slices of one
  // (sequence, head) consecutive logical ids on the same XCD so they share its L2.
  const int nsl = DV / kBV;
  const int nblk = gridDim.x, b = blockIdx.x;
  const int p = (nblk % 8 == 0) ? (b % 8) * (nblk / 8) + b / 8 : b;
  const int slice = p % nsl, sh = p / nsl;
  const int h = sh % H, n = sh / H;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kg = lane >> 4;
  const int v0 = slice * kBV;
  const int tb = cu[n], te = cu[n + 1];
  const int cbase = chunk_off[n];

  constexpr int SROWS = DK / 4;     // state rows per wave
  constexpr int SM = SROWS / 16;    // 16-row tiles per wave
  constexpr int NT = kBV / 16;      // 16-column tiles
  const int srow0 = wid * SROWS;
  const int i0 = wid * 16;          // chunk rows of this wave
  const int nks = (i0 + 16 + 31) / 32;  // k-steps over chunk columns j < i0 + 16

  // ---- one chunk's operands: global -> registers (issued early), registers -> LDS
  // Rows past the chunk end are loaded from the last valid row (always in bounds) and
  // zeroed afterwards, so every load is unconditional and stays in flight.
  auto load_chunk = [&](ChunkRegs<Tin, DK> &R, int c) {
    const int t0 = tb + c * kChunk;
    const int len = min(kChunk, te - t0);
    {
      const int row = min(lane, len - 1);
      const Tin *src = k + ((size_t)(t0 + row) * H + h) * DK + wid * 8;
#pragma unroll
      for (int j = 0; j < DK / 32; ++j) R.kr[j] = load8<Tin>(src + 32 * j);
    }
    {
      const int row = min(tid >> 2, len - 1);
      R.vr = load8<Tin>(v + ((size_t)(t0 + row) * H + h) * DV + v0 + (tid & 3) * 8);
    }
    {
      const int row = min(i0 + r16, len - 1);
      const Tin *src = q + ((size_t)(t0 + row) * H + h) * DK + 8 * kg;
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) R.aq[ks] = load8<Tin>(src + 32 * ks);
    }
    const float *Tc = Tm + ((size_t)(cbase + c) * H + h) * (kChunk * kChunk) + (i0 + r16) * kChunk;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) R.tr[ks] = load8<float>(Tc + 32 * ks + 8 * kg);
    R.gr = Gtok[(size_t)(t0 + min(tid & 63, len - 1)) * H + h];
  };
  // zero the rows past the chunk end (call after the loads have landed)
  auto mask_chunk = [&](ChunkRegs<Tin, DK> &R, int c) {
    const int len = min(kChunk, te - (tb + c * kChunk));
    const FragT z = zero8<Tin>();
    if (lane >= len) {
#pragma unroll
      for (int j = 0; j < DK / 32; ++j) R.kr[j] = z;
    }
    if ((tid >> 2) >= len) R.vr = z;
    if (i0 + r16 >= len) {
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) R.aq[ks] = z;
    }
  };
  auto store_chunk = [&](const ChunkRegs<Tin, DK> &R, int buf) {
#pragma unroll
    for (int j = 0; j < DK / 32; ++j) {
      const int cg = wid + 4 * j;
      *reinterpret_cast<FragT *>(&sm.K[buf][lane][cg * 8]) = R.kr[j];
#pragma unroll
      for (int s = 0; s < 8; ++s) sm.Kt[buf][cg * 8 + s][lane] = R.kr[j][s];
    }
    *reinterpret_cast<FragT *>(&sm.V[buf][tid >> 2][(tid & 3) * 8]) = R.vr;
    if (tid < kChunk) sm.G[buf][tid] = R.gr;
  };

  // ---- state: fp32 accumulator tiles for rows [srow0, srow0 + SROWS) x kBV columns
  const size_t sbase = ((size_t)n * H + h) * DK * (size_t)DV;
  f32x4 Sacc[SM][NT];
#pragma unroll
  for (int mt = 0; mt < SM; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = srow0 + 16 * mt + 4 * kg + i, col = v0 + 16 * nt + r16;
        Sacc[mt][nt][i] = S0 ? S0[sbase + (size_t)row * DV + col] : 0.f;
      }
  auto write_state_operand = [&]() {
#pragma unroll
    for (int mt = 0; mt < SM; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sm.St[16 * nt + r16][srow0 + 16 * mt + 4 * kg + i] = from_f32<Tin>(Sacc[mt][nt][i]);
  };

  const int nchunks = (te - tb + kChunk - 1) / kChunk;
  ChunkRegs<Tin, DK> cur, nxt;
  if (nchunks > 0) {
    load_chunk(cur, 0);
    mask_chunk(cur, 0);
    store_chunk(cur, 0);
  }
  write_state_operand();
  lds_barrier();

  for (int c = 0; c < nchunks; ++c) {
    const int buf = (NBUF == 2) ? (c & 1) : 0;
    const int t0 = tb + c * kChunk;
    const int len = min(kChunk, te - t0);
    const bool has_next = c + 1 < nchunks;
    if (has_next) load_chunk(nxt, c + 1);  // in flight while this chunk computes

    // ---- Y = K S and QS = Q S for this wave's 16 chunk rows; P = Q K^T (causal tiles)
    f32x4 Y[NT], QS[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) { Y[nt] = zero4(); QS[nt] = zero4(); }
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      const FragT ak = load8<Tin>(&sm.K[buf][i0 + r16][32 * ks + 8 * kg]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const FragT bs = load8<Tin>(&sm.St[16 * nt + r16][32 * ks + 8 * kg]);
        Y[nt] = mma(ak, bs, Y[nt]);
        QS[nt] = mma(cur.aq[ks], bs, QS[nt]);
      }
    }
    f32x4 P[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      P[jt] = zero4();
      if (jt <= wid) {
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
          const FragT bk = load8<Tin>(&sm.K[buf][16 * jt + r16][32 * ks + 8 * kg]);
          P[jt] = mma(cur.aq[ks], bk, P[jt]);
        }
      }
    }
    // ---- R = V - Diag(gamma) Y  -> Rt;  P masked by the decay -> sm.P
    const float *Gs = sm.G[buf];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = i0 + 4 * kg + i;
      const float Gr = Gs[row];
      const float gam = __expf(Gr);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int col = 16 * nt + r16;
        sm.Rt[col][row] = from_f32<Tin>(to_f32(sm.V[buf][row][col]) - gam * Y[nt][i]);
      }
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int j = 16 * jt + r16;
        const float val = (j <= row) ? __expf(Gr - Gs[j]) * P[jt][i] : 0.f;
        sm.P[row][j] = from_f32<Tin>(val);
      }
    }
    lds_barrier();

    // ---- U = T R for this wave's rows (T is lower triangular: j < i0 + 16 suffices)
    f32x4 U[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) U[nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (ks < nks) {
        const FragT at = cvt8<Tin>(cur.tr[ks]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const FragT br = load8<Tin>(&sm.Rt[16 * nt + r16][32 * ks + 8 * kg]);
          U[nt] = mma(at, br, U[nt]);
        }
      }
    }
    const float Glast = Gs[kChunk - 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = i0 + 4 * kg + i;
      const float dec = __expf(Glast - Gs[row]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int col = 16 * nt + r16;
        sm.Ut[col][row] = from_f32<Tin>(U[nt][i]);
        sm.Udt[col][row] = from_f32<Tin>(dec * U[nt][i]);
      }
    }
    lds_barrier();

    // ---- O = Diag(gamma) QS + P U
    f32x4 O[NT];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gam = __expf(Gs[i0 + 4 * kg + i]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) O[nt][i] = gam * QS[nt][i];
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (ks < nks) {
        const FragT ap = load8<Tin>(&sm.P[i0 + r16][32 * ks + 8 * kg]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const FragT bu = load8<Tin>(&sm.Ut[16 * nt + r16][32 * ks + 8 * kg]);
          O[nt] = mma(ap, bu, O[nt]);
        }
      }
    }

    // ---- S = exp(G_last) S + K^T Udt for this wave's state rows
    const float dl = __expf(Glast);
#pragma unroll
    for (int mt = 0; mt < SM; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) Sacc[mt][nt] *= dl;
#pragma unroll
    for (int ks = 0; ks < kChunk / 32; ++ks) {
#pragma unroll
      for (int mt = 0; mt < SM; ++mt) {
        const FragT a = load8<Tin>(&sm.Kt[buf][srow0 + 16 * mt + r16][32 * ks + 8 * kg]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const FragT bu = load8<Tin>(&sm.Udt[16 * nt + r16][32 * ks + 8 * kg]);
          Sacc[mt][nt] = mma(a, bu, Sacc[mt][nt]);
        }
      }
    }
    write_state_operand();
    if (has_next) {
      if (NBUF == 1) lds_barrier();  // single buffer: every wave is done with this chunk
      mask_chunk(nxt, c + 1);
      store_chunk(nxt, (NBUF == 2) ? ((c + 1) & 1) : 0);
      cur = nxt;
    }
    // output stores go last so the wait for the prefetched loads above does not also
    // wait for them
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = i0 + 4 * kg + i;
      if (row < len) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          o[((size_t)(t0 + row) * H + h) * DV + v0 + 16 * nt + r16] = from_f32<Tin>(O[nt][i]);
      }
    }
    lds_barrier();
  }

  if (S_T) {
#pragma unroll
    for (int mt = 0; mt < SM; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = srow0 + 16 * mt + 4 * kg + i, col = v0 + 16 * nt + r16;
          S_T[sbase + (size_t)row * DV + col] = Sacc[mt][nt][i];
        }
  }
}

template <typename Tin, int DK>
static hipError_t launch_scan_t(int d_v, const void *q, const void *k, const void *v,
                                const float *G, const float *T, const float *S0, void *o,
                                float *S_T, SeqTables t, int32_t n_seq, int32_t H,
                                hipStream_t stream) {
  const size_t smem = sizeof(ScanSmem<Tin, DK, scan_nbuf<Tin, DK>()>);
  static bool attr_set = false;  // benign race: every thread sets the same value
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&kla_scan_kernel<Tin, DK>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = (int64_t)n_seq * H * (d_v / kBV);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((kla_scan_kernel<Tin, DK>), dim3((unsigned)blocks), dim3(256), smem, stream,
                     static_cast<const Tin *>(q), static_cast<const Tin *>(k),
                     static_cast<const Tin *>(v), G, T, S0, static_cast<Tin *>(o), S_T, t.cu,
                     t.chunk_off, n_seq, H, d_v);
  return hipGetLastError();
}

hipError_t launch_scan(Dtype dt, int d_k, int d_v, const void *q, const void *k, const void *v,
                       const float *G, const float *T, const float *S0, void *o, float *S_T,
                       SeqTables t, int32_t n_seq, int32_t H, hipStream_t stream) {
  if (dt == Dtype::BF16) {
    if (d_k == 128)
      return launch_scan_t<__bf16, 128>(d_v, q, k, v, G, T, S0, o, S_T, t, n_seq, H, stream);
    return launch_scan_t<__bf16, 64>(d_v, q, k, v, G, T, S0, o, S_T, t, n_seq, H, stream);
  }
  if (d_k == 128)
    return launch_scan_t<float, 128>(d_v, q, k, v, G, T, S0, o, S_T, t, n_seq, H, stream);
  return launch_scan_t<float, 64>(d_v, q, k, v, G, T, S0, o, S_T, t, n_seq, H, stream);
}

}  // namespace kla
