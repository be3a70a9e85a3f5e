// kla_scan.hip -- inter-chunk state scan with the chunk output fused in.
//
// Paper "Kaczmarz Linear Attention" (arXiv 2605.08587), section 4, Propositions 3
// and 4.  With the per-chunk T = (I + L)^{-1} Diag(b), the intra-chunk matrix
// P = A o Q K^T, gam_i = exp(G_i) and dec_i = exp(G_last - G_i) from the prep stage, each
// chunk of a (sequence, head) is, given its incoming state S (d_k x d_v, fp32):
//   U     = T (V - Diag(gam) K S)                        Eq. (7)
//   O     = Diag(gam) Q S + P U                          Eq. (8)
//   S_out = exp(G_last) S + K^T Diag(dec) U              Eq. (9)
// and S_out is the next chunk's S.  The chunks of one sequence are processed in order
// by one workgroup; the d_v columns of S are independent given K, T, P and the decays,
// so a (sequence, head) is split over d_v / 64 workgroups.  Each workgroup stages K, Q, T
// and P once for its 64 columns: the staging traffic from L2 into LDS, summed over the
// chip, is what limits the scan when more workgroups share it.
//
// Workgroup = 8 wavefronts with two roles:
//   consumers (waves 0-3) each own 16 state columns and keep them in registers for the
//     whole sequence.  Every product is a 16 x 16 x 32 MFMA whose register operand is an
//     accumulator of the previous product: a D fragment holds rows 4 kg .. 4 kg + 3 of a
//     16-row tile, so two tiles together hold 8 contraction indices per lane, and the
//     tiles are given index maps under which those 8 are consecutive:
//       chunk tile t, row slot 4 a + i  <->  token 32 (t >> 1) + 8 a + 4 (t & 1) + i
//       state tile m, row slot 4 a + i  <->  key dim 32 (m >> 1) + 8 a + 4 (m & 1) + i.
//     The LDS operand of every product is then one 16-byte row piece of K, Q, T or P
//     (or, for K^T, two gfx950 LDS transpose reads).  The output is formed transposed
//     (O^T = S^T Q^T + U^T P^T, the same registers in the other operand slot), so each
//     lane ends with 4 consecutive output columns of one token.
//   producers (waves 4-7) stream the tiles of later chunks into a ring of LDS slots
//     with buffer loads that write LDS directly (no register staging), and write the
//     outputs back.  Each chunk's buffer descriptors end at the sequence's last token, so
//     rows past a ragged end read as zero, and output stores past it are dropped.
// One workgroup barrier per chunk hands a slot from producers to consumers.
//
// LDS tiles are stored in 16-byte units, unit u of row r at u ^ sw(r) (twice sw for fp32
// tiles).  The swizzles follow the gfx950 LDS (64 banks of 4 bytes) as measured: a 16-byte
// read serves together the lanes whose indices differ by an element of span{1, 2, 12, 20}
// (16 lanes: lane bit 5 and the parity of bits 2-4 fixed), and an 8-byte access the lanes
// of one 16-lane block; lanes served together must hit distinct banks.  The fragment reads
// of K, Q, T, P and the output parking are conflict-free under that rule, and among such
// swizzles the ones chosen also time fastest for the transpose reads of K^T and V.
#include <stddef.h>

#include <type_traits>

#include "kla_device.h"
#include "kla_launch.h"

namespace kla {

// Workgroup shape: NC consumer wavefronts (16 state columns each) and NP producers.
template <int NC_, int NP_>
struct ScanShape {
  static constexpr int NC = NC_;
  static constexpr int NP = NP_;
  static constexpr int BV = 16 * NC;              // state columns per workgroup
  static constexpr int THREADS = 64 * (NC + NP);  // consumers first
};
using ScanNarrow = ScanShape<2, 2>;  // 32 columns: the grid fills the chip
using ScanWide = ScanShape<4, 4>;    // 64 columns: K, Q, T, P staged once for twice the columns
constexpr int kLdsBytes = 160 * 1024;

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from buffer offset voff into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(Rsrc r, const void *lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(lds), 16, voff, 0, 0, 0);
}
// Buffer stores of 8 and 16 bytes (dropped beyond the descriptor's range).
__device__ __forceinline__ void store8(u32x2 x, Rsrc r, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b64(x, r, voff, soff, 0);
}
__device__ __forceinline__ void store16(u32x4 x, Rsrc r, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b128(x, r, voff, soff, 0);
}

// Barrier for the producer waves.  They touch LDS only through buffer-to-LDS loads, whose
// completion they establish themselves with wait_vmcnt before arriving; the bare s_barrier
// (a compiler barrier for memory operations) avoids the release fence, which would wait
// for the later chunks' loads as well.
__device__ __forceinline__ void producer_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// ---- swizzles, in 16-byte units of a bf16 row (fp32 rows use twice the value).  Each is
// linear over GF(2): row bits 0, 1, 3 and 4 each flip a fixed set of unit bits.
template <int ROW_ELEMS>
__device__ __forceinline__ int sw_rows(int r) {
  const int b0 = r & 1, b1 = (r >> 1) & 1, b3 = (r >> 3) & 1, b4 = (r >> 4) & 1;
  if constexpr (ROW_ELEMS >= 128)  // 16 units: K, Q with d_k = 128
    return b0 ^ (b1 << 2) ^ (b3 << 3) ^ (b4 << 1);
  else  // 8 units: rows 32-63 of T and P, and K, Q with d_k = 64
    return (b1 << 2) ^ (b3 * 3) ^ (b4 << 1);
}
// value tiles (32 or 64 columns): read by transpose reads, written by the output parking
template <int BV>
__device__ __forceinline__ int sw_val(int r) {
  const int b1 = (r >> 1) & 1, b3 = (r >> 3) & 1, b4 = (r >> 4) & 1;
  if constexpr (BV >= 64)  // 8 units
    return (b1 << 1) ^ (b3 * 3) ^ (b4 << 2);
  else  // 4 units
    return (b3 << 1) ^ (b4 * 3);
}

// Byte offset of element e of row r in a swizzled tile of ROW_ELEMS elements of type T
// (a value tile when VAL).
template <typename T, int ROW_ELEMS, bool VAL = false>
__device__ __forceinline__ int tile_off(int r, int e) {
  constexpr int ES = sizeof(T), ROWB = ROW_ELEMS * ES;
  const int byte = e * ES;
  const int sw = VAL ? sw_val<ROW_ELEMS>(r) : sw_rows<ROW_ELEMS>(r);
  const int u = (byte >> 4) ^ (sw * (ES / 2));
  return r * ROWB + (u << 4) + (byte & 15);
}

// LDS transpose read of 4 x 16-bit values (gfx950 ds_read_b64_tr_b16).  Within each group
// of 16 lanes, destination lane d receives element (d & 3) of the 8-byte chunks addressed
// by source lanes (d >> 2) + 4 i, i = 0..3.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ bf16x4 lds_read_tr(const void *p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// Token (or key dim) of row slot 4 a + i of 16-row tile t.
__device__ __forceinline__ int tmap(int t, int a, int i) {
  return 32 * (t >> 1) + 8 * a + 4 * (t & 1) + i;
}

// ---- LDS layout
template <typename Tin, int DK, int BV, bool DIAG>
struct ScanSlot {
  alignas(16) unsigned char K[kChunk * DK * sizeof(Tin)];  // K, or K o exp(G) (DIAG)
  alignas(16) unsigned char Q[kChunk * DK * sizeof(Tin)];  // Q, or Q o exp(G) (DIAG)
  alignas(16) unsigned char T[tpc_bytes<Tin>()];  // compact tiles (tpc_off)
  alignas(16) unsigned char P[tpc_bytes<Tin>()];
  alignas(16) unsigned char V[kChunk * BV * sizeof(Tin)];
  alignas(16) float gam[kChunk];   // exp(G_i)
  alignas(16) float dec[kChunk];   // exp(G_last - G_i)
  alignas(16) float gamO[kChunk];  // output factor: exp(G_i), over ||q_i|| when normalised
  // diagonal gating: K o exp(G_last - G) for the state update, exp(G_last) per key channel
  alignas(16) unsigned char Kd[DIAG ? kChunk * DK * sizeof(Tin) : 16];
  alignas(16) float gC[DIAG ? DK : 4];
};

template <typename Tin, int DK, int BV, bool DIAG>
constexpr int scan_nslot() {
  constexpr int n = kLdsBytes / (int)sizeof(ScanSlot<Tin, DK, BV, DIAG>);
  return n >= 3 ? 3 : n;
}

template <typename Tin, int DK, int BV, bool DIAG>
struct ScanSmem {
  static constexpr int NSLOT = scan_nslot<Tin, DK, BV, DIAG>();
  ScanSlot<Tin, DK, BV, DIAG> slot[NSLOT];
};

// Buffer-load-to-LDS instructions per chunk (each moves 64 lanes x 16 bytes).
template <typename Tin, int DK, typename SHP, bool DIAG>
struct DmaPlan {
  static constexpr int ES = sizeof(Tin);
  static constexpr int NK = kChunk * DK * ES / 1024;                 // per K (and per Q) tile
  static constexpr int NTC = tpc_bytes<Tin>() / 1024;               // per compact T or P tile
  static constexpr int NV = kChunk * SHP::BV * ES / 1024;            // value slice
  // per producer wave: an equal share of every tile and of the 768-byte decay block, and
  // under diagonal gating of the K o exp(G_last - G) tile and of exp(G_last)
  static constexpr int PER_WAVE =
      (2 * NK + 2 * NTC + NV) / SHP::NP + 1 + (DIAG ? NK / SHP::NP + 1 : 0);
  static_assert(NK % SHP::NP == 0 && (2 * NTC) % SHP::NP == 0 && NV % SHP::NP == 0 &&
                    768 % (16 * SHP::NP) == 0 && (DK * 4) % (16 * SHP::NP) == 0,
                "tiles split over the producer waves");
};

// One workgroup fills a CU's LDS; its waves run at most two to a SIMD.
template <typename Tin, int DK, typename SHP, bool DIAG, bool STATES>
__global__ __launch_bounds__(SHP::THREADS)
__attribute__((amdgpu_waves_per_eu(SHP::THREADS > 256 ? 2 : 1, SHP::THREADS > 256 ? 2 : 1)))
void kla_scan_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const float *__restrict__ GD, const Tin *__restrict__ Tm, const Tin *__restrict__ Pm,
    const float *S0, Tin *__restrict__ o, float *S_T, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, int n_seq, int H, int DV, const Tin *__restrict__ KG,
    const Tin *__restrict__ QG, const Tin *__restrict__ KD, const float *__restrict__ GC,
    Tin *__restrict__ SN) {
  constexpr int kBV = SHP::BV, kConsumers = SHP::NC, kScanThreads = SHP::THREADS;
  using SM = ScanSmem<Tin, DK, kBV, DIAG>;
  using SL = ScanSlot<Tin, DK, kBV, DIAG>;
  using DP = DmaPlan<Tin, DK, SHP, DIAG>;
  using FragT = typename Frag<Tin>::type;
  using KQ = std::integral_constant<int, DK>;
  constexpr bool B16 = sizeof(Tin) == 2;
  constexpr int ES = sizeof(Tin);
  constexpr int NSLOT = SM::NSLOT;
  constexpr int DIST = NSLOT > 1 ? NSLOT - 1 : 1;  // chunks in flight ahead of the consumers
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SM &sm = *reinterpret_cast<SM *>(smem_raw);

  // XCD-aware mapping: workgroup b runs on XCD b % 8; give the d_v slices of one
  // (sequence, head) consecutive logical ids on the same XCD so they share its L2.
  const int nsl = DV / kBV;
  const int nblk = gridDim.x, b = blockIdx.x;
  const int pidx = (nblk % 8 == 0) ? (b % 8) * (nblk / 8) + b / 8 : b;
  const int slice = pidx % nsl, sh = pidx / nsl;
  const int h = sh % H, n = sh / H;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kg = lane >> 4;
  const bool consumer = wid < kConsumers;
  const int v0 = slice * kBV;
  const int tb = cu[n], te = cu[n + 1];
  const int cbase = chunk_off[n];
  const int nchunks = (te - tb + kChunk - 1) / kChunk;

  // Zero the slots once, so a tile row that the range check drops holds zeros or an
  // earlier chunk's finite data whatever the hardware does with dropped lanes.
  for (int i = tid; i < (int)(sizeof(SM) / 16); i += kScanThreads)
    reinterpret_cast<u32x4 *>(smem_raw)[i] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();

  // =========================== producer side ===========================
  // Producer wave pw issues instructions J = NP j + pw of every tile; lane l of instruction
  // J writes tile bytes 1024 J + 16 l, i.e. physical unit pu of row r, which holds logical
  // unit pu ^ sw(r) of that row.
  const int pw = wid - kConsumers;
  constexpr int NP = SHP::NP;
  int offK[DP::NK / NP], offTP[2 * DP::NTC / NP], offV[DP::NV / NP];
  auto dma_off = [&](int J, int row_elems, int gstride_bytes, int sw_of_row) {
    const int pbyte = 1024 * J + 16 * lane, rowb = row_elems * ES;
    const int row = pbyte / rowb, pu = (pbyte % rowb) >> 4;
    return row * gstride_bytes + ((pu ^ sw_of_row) << 4);
  };
  if (!consumer) {
#pragma unroll
    for (int j = 0; j < DP::NK / NP; ++j) {
      const int J = NP * j + pw, row = (1024 * J + 16 * lane) / (DK * ES);
      // K and Q rows: token rows of the inputs, or rows of a chunk's decayed tile (DIAG)
      offK[j] = dma_off(J, DK, (DIAG ? 1 : H) * DK * ES, sw_rows<DK>(row) * (ES / 2));
    }
    // T then P, compact tiles in LDS from packed blocks in memory: item m = NP j + pw is
    // instruction m % NTC of T (m < NTC) or P
#pragma unroll
    for (int j = 0; j < 2 * DP::NTC / NP; ++j) {
      const int m = NP * j + pw;
      int row, col;
      tpc_piece<Tin>(1024 * (m % DP::NTC) + 16 * lane, row, col);
      offTP[j] = tpb_off<Tin>(row, col);
    }
#pragma unroll
    for (int j = 0; j < DP::NV / NP; ++j) {
      const int J = NP * j + pw, row = (1024 * J + 16 * lane) / (kBV * ES);
      offV[j] = dma_off(J, kBV, H * DV * ES, sw_val<kBV>(row) * (ES / 2));
    }
  }
  // issue this wave's half of every load of chunk c into slot s
  auto p_issue = [&](int c, SL &s) {
    const int t0 = tb + c * kChunk;
    const int len = min(kChunk, te - t0);
    const size_t tok = (size_t)t0 * H + h;
    const uint32_t kq_bytes = (uint32_t)(((size_t)(len - 1) * H + 1) * DK * ES);
    const size_t ch = (size_t)(cbase + c) * H + h;
    // the decayed tiles hold all 64 rows, zero past a ragged end
    const Rsrc rk = DIAG ? make_rsrc(KG + ch * (kChunk * DK), kChunk * DK * ES)
                         : make_rsrc(k + tok * DK, kq_bytes);
    const Rsrc rq = DIAG ? make_rsrc(QG + ch * (kChunk * DK), kChunk * DK * ES)
                         : make_rsrc(q + tok * DK, kq_bytes);
    const Rsrc rv =
        make_rsrc(v + tok * DV + v0, (uint32_t)(((size_t)(len - 1) * H * DV + kBV) * ES));
    const Rsrc rt = make_rsrc(Tm + ch * (kChunk * kChunk), tpb_bytes<Tin>());
    const Rsrc rp = make_rsrc(Pm + ch * (kChunk * kChunk), tpb_bytes<Tin>());
    const Rsrc rg = make_rsrc(GD + ch * kGDFloats, kGDFloats * sizeof(float));
#pragma unroll
    for (int j = 0; j < DP::NK / NP; ++j) {
      const int J = NP * j + pw;
      dma16(rk, s.K + 1024 * J, offK[j]);
      dma16(rq, s.Q + 1024 * J, offK[j]);
    }
#pragma unroll
    for (int j = 0; j < 2 * DP::NTC / NP; ++j) {
      const int m = NP * j + pw;
      if (m < DP::NTC) dma16(rt, s.T + 1024 * m, offTP[j]);
      else dma16(rp, s.P + 1024 * (m - DP::NTC), offTP[j]);
    }
#pragma unroll
    for (int j = 0; j < DP::NV / NP; ++j) {
      const int J = NP * j + pw;
      dma16(rv, s.V + 1024 * J, offV[j]);
    }
    // decays (gam, dec, gamO are consecutive in the slot, 768 bytes): producer pw fetches
    // its 768 / NP bytes
    constexpr int GDB = 768 / NP;
    if (lane < GDB / 16)
      dma16(rg, reinterpret_cast<unsigned char *>(s.gam) + GDB * pw, GDB * pw + 16 * lane);
    if constexpr (DIAG) {
      const Rsrc rkd = make_rsrc(KD + ch * (kChunk * DK), kChunk * DK * ES);
#pragma unroll
      for (int j = 0; j < DP::NK / NP; ++j) dma16(rkd, s.Kd + 1024 * (NP * j + pw), offK[j]);
      constexpr int GCB = DK * 4 / NP;  // this wave's bytes of exp(G_last)
      const Rsrc rgc = make_rsrc(GC + ch * DK, DK * sizeof(float));
      if (lane < GCB / 16)
        dma16(rgc, reinterpret_cast<unsigned char *>(s.gC) + GCB * pw, GCB * pw + 16 * lane);
    }
  };

  // chunk c's outputs, parked in slot s's value tile, back to HBM: 16 bytes per lane per
  // piece, whole value-tile rows; rows past a ragged end are dropped.  Producer pw writes
  // back exactly the value-tile bytes its own loads fill (instructions J = NP j + pw).
  constexpr int PPR = kBV * ES / 16;                     // 16-byte pieces per value-tile row
  constexpr int NST = kChunk * PPR / (64 * NP);          // store instructions per producer wave
  auto p_flush = [&](int c, const SL &s) {
    const int t0 = tb + c * kChunk;
    const int len = min(kChunk, te - t0);
    const Rsrc ro = make_rsrc(o + ((size_t)t0 * H + h) * DV + v0,
                              (uint32_t)(((size_t)(len - 1) * H * DV + kBV) * ES));
    u32x4 x[NST];
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      const int e = (tid - 64 * kConsumers) + 64 * NP * j, row = e / PPR, pc = e % PPR;
      x[j] = *reinterpret_cast<const u32x4 *>(s.V + tile_off<Tin, kBV, true>(row, pc * (16 / ES)));
    }
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      const int e = (tid - 64 * kConsumers) + 64 * NP * j, row = e / PPR, pc = e % PPR;
      store16(x[j], ro, (row * H * DV) * ES + pc * 16, 0);
    }
  };

  // =========================== consumer side ===========================
  const int cw = wid;  // consumer wave (producers never use it)
  const int col = 16 * cw + r16;  // this lane's state column within the slice
  constexpr int NM = DK / 16;     // 16-row state tiles
  constexpr int NKS = DK / 32;    // k-steps over d_k
  const size_t sbase = ((size_t)n * H + h) * DK * (size_t)DV;
  f32x4 Sacc[NM];
  if (consumer) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Sacc[m][i] = S0 ? S0[sbase + (size_t)tmap(m, kg, i) * DV + v0 + col] : 0.f;
  }
  // row of this lane's A/B operand fragments in 16-row tile t
  auto frow = [&](int t) { return tmap(t, r16 >> 2, r16 & 3); };
  // elements 32 ks + 8 kg .. + 7 of row r (16 bytes for bf16, 32 for fp32)
  auto rd_frag = [&](const unsigned char *tile, auto row_elems, int r, int ks) {
    constexpr int RE = decltype(row_elems)::value;
    if constexpr (B16) {
      return *reinterpret_cast<const bf16x8 *>(tile + tile_off<Tin, RE>(r, 32 * ks + 8 * kg));
    } else {
      const f32x4 lo =
          *reinterpret_cast<const f32x4 *>(tile + tile_off<Tin, RE>(r, 32 * ks + 8 * kg));
      const f32x4 hi =
          *reinterpret_cast<const f32x4 *>(tile + tile_off<Tin, RE>(r, 32 * ks + 8 * kg + 4));
      return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  // elements 32 ks + 8 kg .. + 7 of row r of a compact T or P tile
  auto rd_tp = [&](const unsigned char *tile, int r, int ks) {
    if constexpr (B16) {
      return *reinterpret_cast<const bf16x8 *>(tile + tpc_off<Tin>(r, 32 * ks + 8 * kg));
    } else {
      const f32x4 lo = *reinterpret_cast<const f32x4 *>(tile + tpc_off<Tin>(r, 32 * ks + 8 * kg));
      const f32x4 hi =
          *reinterpret_cast<const f32x4 *>(tile + tpc_off<Tin>(r, 32 * ks + 8 * kg + 4));
      return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  // accumulator tiles lo (contraction slots 0..3) and hi (4..7) as one operand fragment
  auto accB = [&](const f32x4 &lo, const f32x4 &hi) {
    FragT r;
#pragma unroll
    for (int i = 0; i < 4; ++i) { r[i] = from_f32<Tin>(lo[i]); r[i + 4] = from_f32<Tin>(hi[i]); }
    return r;
  };

  // One chunk.  All LDS operands of a phase are read into registers before the phase's
  // MFMAs, and the next phase's reads are issued while those MFMAs run.
  auto c_step = [&](int c, const SL &s) {
    if constexpr (STATES) {  // the chunk's incoming state in the operand type, for the
                             // backward pass (whose products read it in that precision)
      Tin *dst = SN + ((size_t)(cbase + c) * H + h) * DK * (size_t)DV + v0 + col;
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(size_t)tmap(m, kg, i) * DV] = from_f32<Tin>(Sacc[m][i]);
    }
    FragT Sop[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) Sop[ks] = accB(Sacc[2 * ks], Sacc[2 * ks + 1]);

    // ---- reads for Y = K S and (Q S)^T
    FragT fk[4][NKS], fq[4][NKS];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        fk[t][ks] = rd_frag(s.K, KQ{}, frow(t), ks);
        fq[t][ks] = rd_frag(s.Q, KQ{}, frow(t), ks);
      }
    // ---- reads for R = V - Diag(gam) Y and U = T R
    FragT ft[6];
    ft[0] = rd_tp(s.T, frow(0), 0);
    ft[1] = rd_tp(s.T, frow(1), 0);
    ft[2] = rd_tp(s.T, frow(2), 0);
    ft[3] = rd_tp(s.T, frow(2), 1);
    ft[4] = rd_tp(s.T, frow(3), 0);
    ft[5] = rd_tp(s.T, frow(3), 1);
    f32x4 g4[4], d4[4];
    float vv[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r0 = tmap(t, kg, 0);
      g4[t] = *reinterpret_cast<const f32x4 *>(&s.gam[r0]);
      d4[t] = *reinterpret_cast<const f32x4 *>(&s.dec[r0]);
      if constexpr (B16) {
        const bf16x4 x =
            lds_read_tr(s.V + tile_off<Tin, kBV, true>(r0 + (r16 >> 2), 16 * cw + 4 * (r16 & 3)));
#pragma unroll
        for (int i = 0; i < 4; ++i) vv[t][i] = to_f32(x[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vv[t][i] = *reinterpret_cast<const float *>(s.V + tile_off<Tin, kBV, true>(r0 + i, col));
      }
    }
    const float dl = s.gam[kChunk - 1];  // rows past a ragged end repeat G_last

    // ---- Y = K S first (the dependent chain continues from it)
    f32x4 Y[4], OT[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      Y[t] = zero4();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) Y[t] = mma(fk[t][ks], Sop[ks], Y[t]);
    }
    // the state update's K^T: K, or K o exp(G_last - G) under diagonal gating
    const unsigned char *kt_tile = DIAG ? s.Kd : s.K;
    // ---- reads for the state update: K^T rows = key dims of state tile m, by transpose
    //      reads (source lane r16 of group kg: token 32 ks + 8 kg + (r16 >> 2), + 4 for the
    //      second read; key dims 32 (m >> 1) + 8 (r16 & 3) + 4 (m & 1) .. + 3)
    FragT fkt[NM][2];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if constexpr (B16) {
          const int dk0 = 32 * (m >> 1) + 8 * (r16 & 3) + 4 * (m & 1);
          const int tk = 32 * ks + 8 * kg + (r16 >> 2);
          const bf16x4 lo = lds_read_tr(kt_tile + tile_off<Tin, DK>(tk, dk0));
          const bf16x4 hi = lds_read_tr(kt_tile + tile_off<Tin, DK>(tk + 4, dk0));
#pragma unroll
          for (int i = 0; i < 4; ++i) { fkt[m][ks][i] = lo[i]; fkt[m][ks][i + 4] = hi[i]; }
        } else {
          const int dkr = frow(m);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            fkt[m][ks][e] = *reinterpret_cast<const float *>(
                kt_tile + tile_off<Tin, DK>(32 * ks + 8 * kg + e, dkr));
        }
      }
    // ---- R = V - Diag(gam) Y, U = T R (row tile t needs k-steps ks <= t / 2); (Q S)^T,
    //      which is off the chain, fills the matrix core while R is formed
    FragT Uop[2], Udop[2];
    {
      f32x4 R[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        OT[t] = zero4();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) OT[t] = mma(Sop[ks], fq[t][ks], OT[t]);
#pragma unroll
        for (int i = 0; i < 4; ++i) R[t][i] = vv[t][i] - g4[t][i] * Y[t][i];
      }
      const FragT Rop0 = accB(R[0], R[1]), Rop1 = accB(R[2], R[3]);
      f32x4 U[4];
      U[0] = mma(ft[0], Rop0, zero4());
      U[1] = mma(ft[1], Rop0, zero4());
      U[2] = mma(ft[3], Rop1, mma(ft[2], Rop0, zero4()));
      U[3] = mma(ft[5], Rop1, mma(ft[4], Rop0, zero4()));
      f32x4 Ud[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) Ud[t][i] = d4[t][i] * U[t][i];
      Uop[0] = accB(U[0], U[1]);
      Uop[1] = accB(U[2], U[3]);
      Udop[0] = accB(Ud[0], Ud[1]);
      Udop[1] = accB(Ud[2], Ud[3]);
    }
    // ---- reads for the output: P fragments and this lane's token decays
    FragT fp[6];
    fp[0] = rd_tp(s.P, frow(0), 0);
    fp[1] = rd_tp(s.P, frow(1), 0);
    fp[2] = rd_tp(s.P, frow(2), 0);
    fp[3] = rd_tp(s.P, frow(2), 1);
    fp[4] = rd_tp(s.P, frow(3), 0);
    fp[5] = rd_tp(s.P, frow(3), 1);
    float gt[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) gt[t] = s.gamO[frow(t)];
    // ---- S = exp(G_last) S + K^T Diag(dec) U
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if constexpr (DIAG)  // per key channel: rows tmap(m, kg, 0..3) are consecutive
        Sacc[m] *= *reinterpret_cast<const f32x4 *>(&s.gC[tmap(m, kg, 0)]);
      else
        Sacc[m] *= dl;
      Sacc[m] = mma(fkt[m][0], Udop[0], Sacc[m]);
      Sacc[m] = mma(fkt[m][1], Udop[1], Sacc[m]);
    }
    // ---- O^T = Diag(gam) (Q S)^T + U^T P^T: lane (r16, kg) holds token frow(t), columns
    //      16 cw + 4 kg .. + 3 of this slice.  The block is parked in this wavefront's own
    //      columns of the value tile (read above, and read by no other wavefront); the
    //      producers write whole value-tile rows back to HBM before the slot is refilled.
    {
      unsigned char *vt = const_cast<unsigned char *>(s.V);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 O = OT[t] * gt[t];
        if (t < 2) {
          O = mma(Uop[0], fp[t], O);
        } else {
          O = mma(Uop[0], fp[2 * t - 2], O);
          O = mma(Uop[1], fp[2 * t - 1], O);
        }
        unsigned char *dst = vt + tile_off<Tin, kBV, true>(frow(t), 16 * cw + 4 * kg);
        if constexpr (B16) {
          bf16x4 x4;
#pragma unroll
          for (int i = 0; i < 4; ++i) x4[i] = from_f32<Tin>(O[i]);
          *reinterpret_cast<bf16x4 *>(dst) = x4;
        } else {
          *reinterpret_cast<f32x4 *>(dst) = O;
        }
      }
    }
  };

  // =========================== the chunk loops ===========================
  // The two roles run separate loops that meet at the same number of workgroup barriers.
  if constexpr (NSLOT >= 2) {
    // one barrier before the first chunk and one after each chunk
    if (consumer) {
      lds_barrier();  // chunk 0 staged
      for (int c = 0; c < nchunks; ++c) {
        c_step(c, sm.slot[c % NSLOT]);
        lds_barrier();
      }
    } else {
      const int pro = min(DIST, nchunks);
      for (int c = 0; c < pro; ++c) p_issue(c, sm.slot[c]);
      // chunk 0 complete: only chunk 1's loads (when DIST == 2) may still be in flight
      if (DIST == 2 && pro == 2) wait_vmcnt<DP::PER_WAVE>(); else wait_vmcnt<0>();
      producer_barrier();
      for (int c = 0; c < nchunks; ++c) {
        // slot (c + DIST) % NSLOT held chunk c - 1, released at the barrier just passed:
        // write its outputs back, then refill it
        const bool fl = c >= 1, is = c + DIST < nchunks;
        if (fl) p_flush(c - 1, sm.slot[(c - 1) % NSLOT]);
        if (is) p_issue(c + DIST, sm.slot[(c + DIST) % NSLOT]);
        // chunk c + 1 must be in LDS before the barrier that starts it; what was issued
        // after its loads (this step's stores and loads) may stay in flight
        if (DIST == 2) {
          if (fl && is) wait_vmcnt<NST + DP::PER_WAVE>();
          else if (is) wait_vmcnt<DP::PER_WAVE>();
          else if (fl) wait_vmcnt<NST>();
          else wait_vmcnt<0>();
        } else {
          wait_vmcnt<0>();
        }
        producer_barrier();
      }
      if (nchunks > 0) p_flush(nchunks - 1, sm.slot[(nchunks - 1) % NSLOT]);
    }
  } else {
    // a single slot: one barrier before the loop, then two per chunk (staged, released)
    if (consumer) {
      lds_barrier();
      for (int c = 0; c < nchunks; ++c) {
        lds_barrier();
        c_step(c, sm.slot[0]);
        lds_barrier();
      }
    } else {
      producer_barrier();
      for (int c = 0; c < nchunks; ++c) {
        if (c >= 1) p_flush(c - 1, sm.slot[0]);
        p_issue(c, sm.slot[0]);
        wait_vmcnt<0>();
        producer_barrier();
        producer_barrier();
      }
      if (nchunks > 0) p_flush(nchunks - 1, sm.slot[0]);
    }
  }

  if (consumer && S_T) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S_T[sbase + (size_t)tmap(m, kg, i) * DV + v0 + col] = Sacc[m][i];
  }
}

template <typename Tin, int DK, typename SHP, bool DIAG, bool STATES>
static hipError_t launch_scan_s(int d_v, const void *q, const void *k, const void *v,
                                const float *GD, const void *T, const void *P, const float *S0,
                                void *o, float *S_T, SeqTables t, int32_t n_seq, int32_t H,
                                hipStream_t stream, const DiagTiles *dg, void *SN) {
  using SMT = ScanSmem<Tin, DK, SHP::BV, DIAG>;
  using SLT = ScanSlot<Tin, DK, SHP::BV, DIAG>;
  static_assert(sizeof(SMT) <= kLdsBytes, "LDS budget");
  static_assert(offsetof(SLT, dec) == offsetof(SLT, gam) + 256 &&
                    offsetof(SLT, gamO) == offsetof(SLT, gam) + 512,
                "the decay block is fetched as one contiguous 768-byte piece");
  const size_t smem = sizeof(SMT);
  static bool attr_set = false;  // benign race: every thread sets the same value
  if (!attr_set) {
    hipError_t e =
        hipFuncSetAttribute(reinterpret_cast<const void *>(&kla_scan_kernel<Tin, DK, SHP, DIAG, STATES>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = (int64_t)n_seq * H * (d_v / SHP::BV);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((kla_scan_kernel<Tin, DK, SHP, DIAG, STATES>), dim3((unsigned)blocks),
                     dim3(SHP::THREADS), smem, stream, static_cast<const Tin *>(q),
                     static_cast<const Tin *>(k), static_cast<const Tin *>(v), GD,
                     static_cast<const Tin *>(T), static_cast<const Tin *>(P), S0,
                     static_cast<Tin *>(o), S_T, t.cu, t.chunk_off, n_seq, H, d_v,
                     static_cast<const Tin *>(dg ? dg->kg : nullptr),
                     static_cast<const Tin *>(dg ? dg->qg : nullptr),
                     static_cast<const Tin *>(dg ? dg->kd : nullptr), dg ? dg->gc : nullptr,
                     static_cast<Tin *>(SN));
  return hipGetLastError();
}

// Compute units of the current device (cached per device), 0 if unknown.
static int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

// The narrow shape while its grid fits the chip in one wave of workgroups (more of them
// would only queue behind each other while their staging traffic adds up); the wide shape,
// which stages each tile once for 64 columns, beyond that.
template <typename Tin, int DK, bool DIAG, bool STATES>
static hipError_t launch_scan_t(int d_v, const void *q, const void *k, const void *v,
                                const float *GD, const void *T, const void *P, const float *S0,
                                void *o, float *S_T, SeqTables t, int32_t n_seq, int32_t H,
                                hipStream_t stream, const DiagTiles *dg, void *SN) {
  const int64_t narrow_blocks = (int64_t)n_seq * H * (d_v / ScanNarrow::BV);
  const int cus = device_cus();
  if (cus > 0 && narrow_blocks > cus)
    return launch_scan_s<Tin, DK, ScanWide, DIAG, STATES>(d_v, q, k, v, GD, T, P, S0, o, S_T, t,
                                                          n_seq, H, stream, dg, SN);
  return launch_scan_s<Tin, DK, ScanNarrow, DIAG, STATES>(d_v, q, k, v, GD, T, P, S0, o, S_T, t,
                                                          n_seq, H, stream, dg, SN);
}

template <typename Tin, int DK>
static hipError_t launch_scan_g(int d_v, const void *q, const void *k, const void *v,
                                const float *GD, const void *T, const void *P, const float *S0,
                                void *o, float *S_T, SeqTables t, int32_t n_seq, int32_t H,
                                hipStream_t stream, const DiagTiles *dg, void *SN) {
  if (dg) {
    if (SN) return hipErrorInvalidValue;  // no stored states under diagonal gating
    return launch_scan_t<Tin, DK, true, false>(d_v, q, k, v, GD, T, P, S0, o, S_T, t, n_seq, H,
                                               stream, dg, nullptr);
  }
  if (SN)
    return launch_scan_t<Tin, DK, false, true>(d_v, q, k, v, GD, T, P, S0, o, S_T, t, n_seq, H,
                                               stream, nullptr, SN);
  return launch_scan_t<Tin, DK, false, false>(d_v, q, k, v, GD, T, P, S0, o, S_T, t, n_seq, H,
                                              stream, nullptr, nullptr);
}

hipError_t launch_scan(Dtype dt, int d_k, int d_v, const void *q, const void *k, const void *v,
                       const float *GD, const void *T, const void *P, const float *S0, void *o,
                       float *S_T, SeqTables t, int32_t n_seq, int32_t H, hipStream_t stream,
                       const DiagTiles *dg, void *SN) {
  if (dt == Dtype::BF16) {
    if (d_k == 128)
      return launch_scan_g<__bf16, 128>(d_v, q, k, v, GD, T, P, S0, o, S_T, t, n_seq, H, stream,
                                        dg, SN);
    return launch_scan_g<__bf16, 64>(d_v, q, k, v, GD, T, P, S0, o, S_T, t, n_seq, H, stream,
                                     dg, SN);
  }
  if (d_k == 128)
    return launch_scan_g<float, 128>(d_v, q, k, v, GD, T, P, S0, o, S_T, t, n_seq, H, stream,
                                     dg, SN);
  return launch_scan_g<float, 64>(d_v, q, k, v, GD, T, P, S0, o, S_T, t, n_seq, H, stream, dg,
                                  SN);
}

}  // namespace kla
