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
// Work split inside the workgroup (8 wavefronts, 2 per SIMD, BV = 32 state columns):
// wave w = (mw, nw) with mw = w % 4, nw = w / 4 owns
//   chunk rows [16 mw, 16 mw + 16) x state columns [16 nw, 16 nw + 16) for K S, Q S,
//   T R and P U, every other j-tile of P^T = K Q^T for its chunk rows, and
//   state rows [mw d_k / 4, (mw + 1) d_k / 4) x the same 16 columns for K^T U,
//   which it keeps in fp32 accumulator registers for the whole sequence.
// The next chunk's K, Q, T and V tiles are fetched once per workgroup with 16-byte
// loads while the current chunk computes, and land in the other half of a double
// buffer in LDS.  K^T operands, V in accumulator layout and the output rows are read
// with the LDS transpose read (ds_read_b64_tr_b16) for 16-bit data, so no transposed
// copy of the keys is kept; every other cross-wave operand is written with packed
// 4-element stores because an accumulator fragment holds 4 consecutive rows of a column.
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {

constexpr int kBV = 32;        // state columns per workgroup
constexpr int kScanThreads = 512;

// LDS-only workgroup barrier: orders LDS traffic without waiting for the global
// loads that are deliberately left in flight (the next chunk's prefetch).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 4 consecutive elements of T (packed LDS store of 8 or 16 bytes).
template <typename T> struct Vec4;
template <> struct Vec4<__bf16> { typedef bf16x4 type; };
template <> struct Vec4<float> { typedef f32x4 type; };

template <typename T>
__device__ __forceinline__ void store4(T *p, float a, float b, float c, float d) {
  typename Vec4<T>::type x;
  x[0] = from_f32<T>(a); x[1] = from_f32<T>(b); x[2] = from_f32<T>(c); x[3] = from_f32<T>(d);
  *reinterpret_cast<typename Vec4<T>::type *>(p) = x;
}

// LDS transpose read of 4 x 16-bit values (gfx950).  Within each group of 16 lanes,
// destination lane d receives element (d & 3) of the 8-byte chunks addressed by source
// lanes (d >> 2) + 4 i, i = 0..3.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16 *p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)(reinterpret_cast<const void *>(p)));
  return __builtin_bit_cast(bf16x4, r);
}

// fp32 chunk operands are single-buffered so the tiles fit in LDS.
template <typename Tin>
constexpr int scan_nbuf() { return sizeof(Tin) == 4 ? 1 : 2; }

template <typename Tin, int DK, int NBUF>
struct ScanSmem {
  static constexpr int PAD = 8;
  static constexpr int OT = sizeof(Tin) == 2 ? kBV : 1;  // output staging (16-bit only)
  alignas(16) Tin K[NBUF][kChunk][DK + PAD];     // chunk keys, token-major
  alignas(16) Tin Q[NBUF][kChunk][DK + PAD];     // chunk queries, token-major
  alignas(16) Tin T[NBUF][kChunk][kChunk + PAD]; // T = (I + L)^{-1} Diag(b), row-major
  alignas(16) Tin V[NBUF][kChunk][kBV + PAD];    // value slice, token-major
  alignas(16) float G[NBUF][kChunk];             // chunk-local log-decay (tail repeats G[len-1])
  alignas(16) float gam[NBUF][kChunk];           // exp(G_i)
  alignas(16) float dec[NBUF][kChunk];           // exp(G_last - G_i)
  alignas(16) Tin St[kBV][DK + PAD];             // state operand copy, column-major
  alignas(16) Tin Rt[kBV][kChunk + PAD];         // R = V - Diag(gamma) K S, column-major
  alignas(16) Tin Ut[kBV][kChunk + PAD];         // U, column-major
  alignas(16) Tin Udt[kBV][kChunk + PAD];        // Diag(exp(G_last - G)) U, column-major
  alignas(16) Tin P[kChunk][kChunk + PAD];       // A o Q K^T, row-major
  alignas(16) Tin Ot[OT][kChunk + PAD];          // output staging, column-major
};

// One chunk's K, Q, T, V tiles in flight: 16-byte pieces spread over the 512 threads.
template <typename Tin, int DK>
struct ChunkRegs {
  static constexpr int EP = 16 / sizeof(Tin);                     // elements per piece
  static constexpr int KP = kChunk * DK / EP / kScanThreads;       // K (and Q) pieces per thread
  static constexpr int TP = (kChunk * kChunk / EP + kScanThreads - 1) / kScanThreads;
  static constexpr int VP = (kChunk * kBV / EP + kScanThreads - 1) / kScanThreads;
  typedef u16x8 Piece __attribute__((unused));
  f32x4 k[KP], q[KP], t[TP], v[VP];   // raw 16-byte pieces (bit patterns)
  float gr, glast;                    // G of row lane and of the last row (wave 0)
};

template <typename Tin, int DK>
__global__ __launch_bounds__(kScanThreads) void kla_scan_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const float *__restrict__ Gtok, const Tin *__restrict__ Tm, const float *S0,
    Tin *__restrict__ o, float *S_T, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, int n_seq, int H, int DV) {
  constexpr int NBUF = scan_nbuf<Tin>();
  constexpr bool B16 = sizeof(Tin) == 2;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  ScanSmem<Tin, DK, NBUF> &sm = *reinterpret_cast<ScanSmem<Tin, DK, NBUF> *>(smem_raw);
  using FragT = typename Frag<Tin>::type;
  using CR = ChunkRegs<Tin, DK>;
  constexpr int EP = CR::EP;

  // XCD-aware mapping: workgroup b runs on XCD b % 8; give the d_v slices of one
  // (sequence, head) consecutive logical ids on the same XCD so they share its L2.
  const int nsl = DV / kBV;
  const int nblk = gridDim.x, b = blockIdx.x;
  const int p = (nblk % 8 == 0) ? (b % 8) * (nblk / 8) + b / 8 : b;
  const int slice = p % nsl, sh = p / nsl;
  const int h = sh % H, n = sh / H;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kg = lane >> 4;
  const int mw = wid & 3, nw = wid >> 2;
  const int v0 = slice * kBV;
  const int col = 16 * nw + r16;    // this lane's state column within the slice
  const int tb = cu[n], te = cu[n + 1];
  const int cbase = chunk_off[n];

  constexpr int SROWS = DK / 4;     // state rows per wave
  constexpr int SM = SROWS / 16;    // 16-row tiles per wave
  const int srow0 = mw * SROWS;
  const int i0 = mw * 16;           // chunk rows of this wave
  const int nks = (i0 + 16 + 31) / 32;  // k-steps over chunk columns j < i0 + 16

  // ---- one chunk's tiles: global -> registers (issued early), registers -> LDS.
  // Rows past the chunk end are loaded from the last valid row (always in bounds) and
  // zeroed on the way into LDS.
  constexpr int KPR = DK / EP;      // pieces per key row
  constexpr int TPR = kChunk / EP;  // pieces per T row
  constexpr int VPR = kBV / EP;     // pieces per value-slice row
  auto load_chunk = [&](CR &R, int c) {
    const int t0 = tb + c * kChunk;
    const int len = min(kChunk, te - t0);
#pragma unroll
    for (int j = 0; j < CR::KP; ++j) {
      const int e = tid + kScanThreads * j, row = min(e / KPR, len - 1), pc = e % KPR;
      const size_t off = ((size_t)(t0 + row) * H + h) * DK + pc * EP;
      R.k[j] = *reinterpret_cast<const f32x4 *>(k + off);
      R.q[j] = *reinterpret_cast<const f32x4 *>(q + off);
    }
    const Tin *Tc = Tm + ((size_t)(cbase + c) * H + h) * (kChunk * kChunk);
#pragma unroll
    for (int j = 0; j < CR::TP; ++j) {
      const int e = tid + kScanThreads * j;
      if (e < kChunk * TPR) R.t[j] = *reinterpret_cast<const f32x4 *>(Tc + e * EP);
    }
#pragma unroll
    for (int j = 0; j < CR::VP; ++j) {
      const int e = tid + kScanThreads * j;
      if (e < kChunk * VPR) {
        const int row = min(e / VPR, len - 1), pc = e % VPR;
        R.v[j] = *reinterpret_cast<const f32x4 *>(v + ((size_t)(t0 + row) * H + h) * DV + v0 +
                                                  pc * EP);
      }
    }
    if (wid == 0) {
      R.gr = Gtok[(size_t)(t0 + min(lane, len - 1)) * H + h];
      R.glast = Gtok[(size_t)(t0 + len - 1) * H + h];
    }
  };
  auto store_chunk = [&](const CR &R, int c, int buf) {
    const int len = min(kChunk, te - (tb + c * kChunk));
    const f32x4 z = zero4();
#pragma unroll
    for (int j = 0; j < CR::KP; ++j) {
      const int e = tid + kScanThreads * j, row = e / KPR, pc = e % KPR;
      *reinterpret_cast<f32x4 *>(&sm.K[buf][row][pc * EP]) = row < len ? R.k[j] : z;
      *reinterpret_cast<f32x4 *>(&sm.Q[buf][row][pc * EP]) = row < len ? R.q[j] : z;
    }
#pragma unroll
    for (int j = 0; j < CR::TP; ++j) {
      const int e = tid + kScanThreads * j;
      if (e < kChunk * TPR)
        *reinterpret_cast<f32x4 *>(&sm.T[buf][e / TPR][(e % TPR) * EP]) = R.t[j];
    }
#pragma unroll
    for (int j = 0; j < CR::VP; ++j) {
      const int e = tid + kScanThreads * j;
      if (e < kChunk * VPR) {
        const int row = e / VPR;
        *reinterpret_cast<f32x4 *>(&sm.V[buf][row][(e % VPR) * EP]) = row < len ? R.v[j] : z;
      }
    }
    if (wid == 0) {
      sm.G[buf][lane] = R.gr;
      sm.gam[buf][lane] = __expf(R.gr);
      sm.dec[buf][lane] = __expf(R.glast - R.gr);
    }
  };

  // ---- state: fp32 accumulator tiles for rows [srow0, srow0 + SROWS) x column `col`
  const size_t sbase = ((size_t)n * H + h) * DK * (size_t)DV;
  f32x4 Sacc[SM];
#pragma unroll
  for (int mt = 0; mt < SM; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = srow0 + 16 * mt + 4 * kg + i;
      Sacc[mt][i] = S0 ? S0[sbase + (size_t)row * DV + v0 + col] : 0.f;
    }
  auto write_state_operand = [&]() {
#pragma unroll
    for (int mt = 0; mt < SM; ++mt)
      store4<Tin>(&sm.St[col][srow0 + 16 * mt + 4 * kg], Sacc[mt][0], Sacc[mt][1], Sacc[mt][2],
                  Sacc[mt][3]);
  };
  // output rows of a finished chunk, staged column-major in sm.Ot (16-bit types): each
  // 16-lane group reads 16 rows x 4 columns back row-major and stores 8 bytes per lane
  auto flush_output = [&](int c) {
    if constexpr (B16) {
      const int t0 = tb + c * kChunk;
      const int len = min(kChunk, te - t0);
      const int G4 = 4 * wid + kg;                  // 0..31
      const int rowbase = 16 * (G4 & 3), cb = 4 * (G4 >> 2);
      const bf16x4 x = lds_read_tr(&sm.Ot[cb + (r16 >> 2)][rowbase + 4 * (r16 & 3)]);
      const int row = rowbase + r16;
      if (row < len)
        *reinterpret_cast<bf16x4 *>(o + ((size_t)(t0 + row) * H + h) * DV + v0 + cb) = x;
    }
  };

  const int nchunks = (te - tb + kChunk - 1) / kChunk;
  CR nxt;
  if (nchunks > 0) {
    load_chunk(nxt, 0);
    store_chunk(nxt, 0, 0);
  }
  write_state_operand();
  lds_barrier();

  for (int c = 0; c < nchunks; ++c) {
    const int buf = (NBUF == 2) ? (c & 1) : 0;
    const int t0 = tb + c * kChunk;
    const int len = min(kChunk, te - t0);
    const bool has_next = c + 1 < nchunks;
    if (c > 0) flush_output(c - 1);
    if (has_next) load_chunk(nxt, c + 1);  // in flight while this chunk computes

    // ---- phase A: Y = K S and QS = Q S (16 rows x 16 columns); R = V - Diag(gamma) Y
    f32x4 Y = zero4(), QS = zero4();
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      const FragT ak = load8<Tin>(&sm.K[buf][i0 + r16][32 * ks + 8 * kg]);
      const FragT aq = load8<Tin>(&sm.Q[buf][i0 + r16][32 * ks + 8 * kg]);
      const FragT bs = load8<Tin>(&sm.St[col][32 * ks + 8 * kg]);
      Y = mma(ak, bs, Y);
      QS = mma(aq, bs, QS);
    }
    {
      float vv[4];
      if constexpr (B16) {
        const bf16x4 x = lds_read_tr(&sm.V[buf][i0 + 4 * kg + (r16 >> 2)][16 * nw + 4 * (r16 & 3)]);
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[e] = to_f32(x[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[e] = to_f32(sm.V[buf][i0 + 4 * kg + e][col]);
      }
      const f32x4 g4 = *reinterpret_cast<const f32x4 *>(&sm.gam[buf][i0 + 4 * kg]);
      store4<Tin>(&sm.Rt[col][i0 + 4 * kg], vv[0] - g4[0] * Y[0], vv[1] - g4[1] * Y[1],
                  vv[2] - g4[2] * Y[2], vv[3] - g4[3] * Y[3]);
    }
    lds_barrier();

    // ---- phase B: U = T R; P^T = K Q^T for every other causal j-tile of this wave's rows
    {
      f32x4 U = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks < nks) {
          const FragT at = load8<Tin>(&sm.T[buf][i0 + r16][32 * ks + 8 * kg]);
          const FragT br = load8<Tin>(&sm.Rt[col][32 * ks + 8 * kg]);
          U = mma(at, br, U);
        }
      }
      const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&sm.dec[buf][i0 + 4 * kg]);
      store4<Tin>(&sm.Ut[col][i0 + 4 * kg], U[0], U[1], U[2], U[3]);
      store4<Tin>(&sm.Udt[col][i0 + 4 * kg], d4[0] * U[0], d4[1] * U[1], d4[2] * U[2],
                  d4[3] * U[3]);
    }
    {
      const int i = i0 + r16;  // query row held by this lane in the P^T fragments
      const float Gi = sm.G[buf][i];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        if (jt <= mw && (jt & 1) == nw) {
          f32x4 Pt = zero4();
#pragma unroll
          for (int ks = 0; ks < DK / 32; ++ks) {
            const FragT ak = load8<Tin>(&sm.K[buf][16 * jt + r16][32 * ks + 8 * kg]);
            const FragT bq = load8<Tin>(&sm.Q[buf][i][32 * ks + 8 * kg]);
            Pt = mma(ak, bq, Pt);
          }
          // Pt[e] = (Q K^T)[i][j], j = 16 jt + 4 kg + e; decay mask for j <= i
          const int j0 = 16 * jt + 4 * kg;
          const f32x4 gj = *reinterpret_cast<const f32x4 *>(&sm.G[buf][j0]);
          float pv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[e] = (j0 + e <= i) ? __expf(Gi - gj[e]) * Pt[e] : 0.f;
          store4<Tin>(&sm.P[i][j0], pv[0], pv[1], pv[2], pv[3]);
        } else if (jt > mw && nw == 0) {
          store4<Tin>(&sm.P[i][16 * jt + 4 * kg], 0.f, 0.f, 0.f, 0.f);
        }
      }
    }
    lds_barrier();

    // ---- phase C: O = Diag(gamma) QS + P U;  S = exp(G_last) S + K^T Udt
    {
      f32x4 O;
      const f32x4 g4 = *reinterpret_cast<const f32x4 *>(&sm.gam[buf][i0 + 4 * kg]);
#pragma unroll
      for (int e = 0; e < 4; ++e) O[e] = g4[e] * QS[e];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks < nks) {
          const FragT ap = load8<Tin>(&sm.P[i0 + r16][32 * ks + 8 * kg]);
          const FragT bu = load8<Tin>(&sm.Ut[col][32 * ks + 8 * kg]);
          O = mma(ap, bu, O);
        }
      }
      if constexpr (B16) {
        store4<Tin>(&sm.Ot[col][i0 + 4 * kg], O[0], O[1], O[2], O[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = i0 + 4 * kg + e;
          if (row < len) o[((size_t)(t0 + row) * H + h) * DV + v0 + col] = from_f32<Tin>(O[e]);
        }
      }
    }
    {
      const float dl = sm.gam[buf][kChunk - 1];  // exp(G_last): tail rows repeat G[len-1]
#pragma unroll
      for (int mt = 0; mt < SM; ++mt) Sacc[mt] *= dl;
#pragma unroll
      for (int ks = 0; ks < kChunk / 32; ++ks) {
        const FragT bu = load8<Tin>(&sm.Udt[col][32 * ks + 8 * kg]);
#pragma unroll
        for (int mt = 0; mt < SM; ++mt) {
          const int mb = srow0 + 16 * mt;
          FragT a;
          if constexpr (B16) {
            // K^T fragment: row r16 of the 16 x 32 tile = dimension mb + r16 over 8 tokens
            const int tok = 32 * ks + 8 * kg + (r16 >> 2);
            const bf16x4 lo = lds_read_tr(&sm.K[buf][tok][mb + 4 * (r16 & 3)]);
            const bf16x4 hi = lds_read_tr(&sm.K[buf][tok + 4][mb + 4 * (r16 & 3)]);
#pragma unroll
            for (int e = 0; e < 4; ++e) { a[e] = lo[e]; a[e + 4] = hi[e]; }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = sm.K[buf][32 * ks + 8 * kg + e][mb + r16];
          }
          Sacc[mt] = mma(a, bu, Sacc[mt]);
        }
      }
    }
    if (NBUF == 1) lds_barrier();  // single buffer: every wave is done reading this chunk
    write_state_operand();
    if (has_next) store_chunk(nxt, c + 1, (NBUF == 2) ? ((c + 1) & 1) : 0);
    lds_barrier();
  }
  if (nchunks > 0) flush_output(nchunks - 1);

  if (S_T) {
#pragma unroll
    for (int mt = 0; mt < SM; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = srow0 + 16 * mt + 4 * kg + i;
        S_T[sbase + (size_t)row * DV + v0 + col] = Sacc[mt][i];
      }
  }
}

template <typename Tin, int DK>
static hipError_t launch_scan_t(int d_v, const void *q, const void *k, const void *v,
                                const float *G, const void *T, const float *S0, void *o,
                                float *S_T, SeqTables t, int32_t n_seq, int32_t H,
                                hipStream_t stream) {
  const size_t smem = sizeof(ScanSmem<Tin, DK, scan_nbuf<Tin>()>);
  static bool attr_set = false;  // benign race: every thread sets the same value
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&kla_scan_kernel<Tin, DK>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = (int64_t)n_seq * H * (d_v / kBV);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((kla_scan_kernel<Tin, DK>), dim3((unsigned)blocks), dim3(kScanThreads), smem,
                     stream, static_cast<const Tin *>(q), static_cast<const Tin *>(k),
                     static_cast<const Tin *>(v), G, static_cast<const Tin *>(T), S0,
                     static_cast<Tin *>(o), S_T, t.cu, t.chunk_off, n_seq, H, d_v);
  return hipGetLastError();
}

hipError_t launch_scan(Dtype dt, int d_k, int d_v, const void *q, const void *k, const void *v,
                       const float *G, const void *T, const float *S0, void *o, float *S_T,
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
