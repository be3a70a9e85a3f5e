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
#include "kla_tile.h"

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

// ---- LDS layout
template <typename Tin, int DK, int BV, bool DIAG, bool NOQP = false, bool SPLIT = false>
struct ScanSlot {
  alignas(16) unsigned char K[kChunk * DK * sizeof(Tin)];  // K, or K o exp(G) (DIAG)
  // Q, or Q o exp(G) (DIAG); not staged by the map mode, which forms no outputs
  alignas(16) unsigned char Q[NOQP ? 16 : kChunk * DK * sizeof(Tin)];
  alignas(16) unsigned char T[tpc_bytes<Tin>()];  // compact tiles (tpc_off)
  alignas(16) unsigned char P[NOQP ? 16 : tpc_bytes<Tin>()];
  alignas(16) unsigned char V[kChunk * BV * sizeof(Tin)];
  alignas(16) float gam[kChunk];   // exp(G_i)
  alignas(16) float dec[kChunk];   // exp(G_last - G_i)
  // output factor: exp(G_i), over ||q_i|| when normalised (not staged by the map mode, which
  // then fits three slots in half of a CU's LDS, two workgroups to a CU)
  alignas(16) float gamO[NOQP ? 4 : kChunk];
  // diagonal gating: K o exp(G_last - G) for the state update, exp(G_last) per key channel
  alignas(16) unsigned char Kd[DIAG ? kChunk * DK * sizeof(Tin) : 16];
  alignas(16) float gC[DIAG ? DK : 4];
  // split precision: the low parts of T and P (x - bf16(x), in bf16)
  alignas(16) unsigned char Tl[SPLIT ? tpc_bytes<Tin>() : 16];
  alignas(16) unsigned char Pl[SPLIT ? tpc_bytes<Tin>() : 16];
};

template <typename Tin, int DK, int BV, bool DIAG, bool NOQP, bool SPLIT>
constexpr int scan_nslot() {
  constexpr int n = kLdsBytes / (int)sizeof(ScanSlot<Tin, DK, BV, DIAG, NOQP, SPLIT>);
  return n >= 3 ? 3 : n;
}

template <typename Tin, int DK, int BV, bool DIAG, bool NOQP = false, bool SPLIT = false>
struct ScanSmem {
  static constexpr int NSLOT = scan_nslot<Tin, DK, BV, DIAG, NOQP, SPLIT>();
  ScanSlot<Tin, DK, BV, DIAG, NOQP, SPLIT> slot[NSLOT];
};

// Buffer-load-to-LDS instructions per chunk (each moves 64 lanes x 16 bytes).
template <typename Tin, int DK, typename SHP, bool DIAG, bool NOQP, bool SPLIT = false>
struct DmaPlan {
  static constexpr int ES = sizeof(Tin);
  static constexpr int NK = kChunk * DK * ES / 1024;                 // per K (and per Q) tile
  static constexpr int NTC = tpc_bytes<Tin>() / 1024;               // per compact T or P tile
  static constexpr int NV = kChunk * SHP::BV * ES / 1024;            // value slice
  // per producer wave: an equal share of every tile and of the 768-byte decay block, and
  // under diagonal gating of the K o exp(G_last - G) tile and of exp(G_last); the map mode
  // stages no Q and no P
  // T pieces per wave: the map mode stages T alone, NTC pieces over the producer waves, the
  // last round repeating earlier pieces so that every wave issues the same count; split
  // precision stages T, P and their low parts
  static constexpr int NTW =
      NOQP ? (NTC + SHP::NP - 1) / SHP::NP : (SPLIT ? 4 : 2) * NTC / SHP::NP;
  static constexpr int PER_WAVE =
      ((NOQP ? 1 : 2) * NK + NV) / SHP::NP + NTW + 1 + (DIAG ? NK / SHP::NP + 1 : 0);
  static_assert(NK % SHP::NP == 0 && (2 * NTC) % SHP::NP == 0 && NV % SHP::NP == 0 &&
                    768 % (16 * SHP::NP) == 0 && (DK * 4) % (16 * SHP::NP) == 0,
                "tiles split over the producer waves");
};

// One workgroup fills a CU's LDS; its waves run at most two to a SIMD.
//
// MODE kScanSeq: a workgroup per (sequence, head, column slice), sequences from the tables.
// MODE kScanMap / kScanSeg: the two phases of the two-level scan of equal-length sequences
// (SegArgs): a workgroup per (segment, head, column slice).  kScanMap runs segments
// 0 .. G-2 of each sequence with no outputs on a state of dv + d_k columns: the first dv
// start from zero (segment 0: from S0) and take the values, so they end as the segment's
// N_g = S_out(S_in = 0); the last d_k start from the identity and take zero values, so they
// end as the segment's transition M_g (Eq. (9) makes S_out affine in S_in:
// S_out = M_g S_in + N_g).  kScanSeg runs every segment from its true incoming state (S0
// for segment 0, sa.Sin for the others) with the outputs, and stores S_T from the last one.
//
// SPLIT (bf16, kScanSeq, scalar gate): the products T R, P U and K^T Diag(dec) U take each
// rounded operand other than K as a pair of bf16 values, hi = bf16(x) and lo = bf16(x - hi),
// and sum hi*hi + hi*lo + lo*hi (K is exact in bf16: two terms).  The prep kernel stores T
// and P as such pairs.  S stays one bf16 operand in K S and Q S.
// Whether sequence seq, head h of the two-level scan takes the warm-up start: at every
// segment boundary the W chunks before it either reach back to the sequence start or have a
// contraction bound (the sum of their log bounds) of at most ln 2^-150.  Starting those W
// chunks from a zero state then changes the segment's incoming state by at most 2^-150 times
// the norm of the state W chunks back (the homogeneous map of the W chunks has at most that
// spectral norm).  The same answer in every kernel that asks: it reads only LC.
// Lane l of each wavefront tests boundary 1 + l (+ 64 i); the wavefront's answer is the AND.
__device__ __forceinline__ bool warm_start(const SegArgs &sa, int seq, int h, int H) {
  if (sa.LC == nullptr || sa.W <= 0) return false;
  const int cps = (sa.L + kChunk - 1) / kChunk, cpg = sa.Ls / kChunk;
  const int lane = threadIdx.x & 63;
  bool ok = true;
  for (int g0 = 1; g0 < sa.G; g0 += kWave) {
    const int g = g0 + lane;
    const int c1 = g * cpg, c0 = c1 - sa.W;
    if (g < sa.G && c0 > 0) {  // else past the last boundary, or from S0 at the start: exact
      float s = 0.f;
      for (int c = c0; c < c1; ++c) s += sa.LC[((size_t)seq * cps + c) * H + h];
      ok = ok && (s <= kWarmLog);  // a NaN bound fails too
    }
  }
  return __all(ok);
}

// For at most 64 sequences of mixed lengths, the sequence of rank r when they are ordered
// longest first (ties by index); -1 otherwise (equal lengths, or more sequences).  Lane l
// ranks sequence l against the others; the answer is the lane whose rank is r, the same in
// every lane of the wavefront.
__device__ __forceinline__ int longest_first(const int32_t *__restrict__ cu, int n_seq, int r) {
  if (n_seq > kWave) return -1;
  const int lane = threadIdx.x & (kWave - 1);
  const int len = lane < n_seq ? cu[lane + 1] - cu[lane] : -1;
  if (!__any(lane < n_seq && len != __shfl(len, 0, kWave))) return -1;
  int rank = 0;
  for (int m = 0; m < n_seq; ++m) {
    const int lm = __shfl(len, m, kWave);
    rank += (lm > len || (lm == len && m < lane)) ? 1 : 0;
  }
  const unsigned long long hit = __ballot(lane < n_seq && rank == r);
  return hit ? (int)__builtin_ctzll(hit) : r;  // ranks are a permutation: one lane hits
}

template <typename Tin, int DK, typename SHP, bool DIAG, bool STATES, int MODE,
          bool SPLIT = false>
__global__ __launch_bounds__(SHP::THREADS)
__attribute__((amdgpu_waves_per_eu(SHP::THREADS > 256 || MODE == kScanMap ? 2 : 1,
                                    SHP::THREADS > 256 || MODE == kScanMap ? 2 : 1)))
void kla_scan_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const float *__restrict__ GD, const Tin *__restrict__ Tm, const Tin *__restrict__ Pm,
    const float *S0, Tin *__restrict__ o, float *S_T, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_off, int n_seq, int H, int DV, const Tin *__restrict__ KG,
    const Tin *__restrict__ QG, const Tin *__restrict__ KD, const float *__restrict__ GC,
    Tin *__restrict__ SN, SegArgs sa) {
  constexpr int kBV = SHP::BV, kConsumers = SHP::NC, kScanThreads = SHP::THREADS;
  constexpr bool MAP = MODE == kScanMap;
  // no queries, P or outputs: the map mode, and the states-only pass of the backward
  constexpr bool NOQP = MAP || STATES;
  static_assert(!SPLIT || (sizeof(Tin) == 2 && !DIAG && !STATES && MODE == kScanSeq),
                "split precision: bf16 operands, sequential scalar-gate scan");
  using SM = ScanSmem<Tin, DK, kBV, DIAG, NOQP, SPLIT>;
  using SL = ScanSlot<Tin, DK, kBV, DIAG, NOQP, SPLIT>;
  using DP = DmaPlan<Tin, DK, SHP, DIAG, NOQP, SPLIT>;
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
  // Packed sequences of mixed lengths: the sequential scan takes its units head-major, the
  // sequences longest first within a head, so that one XCD's contiguous share of the units
  // holds every sequence of its heads and the longest start first (they balance over XCDs
  // and CUs).  Otherwise sequence-major.
  int h = sh % H, n = sh / H;  // n: the sequence, or the unit of the two-level scan
  if constexpr (MODE == kScanSeq) {
    const int hm = sh / n_seq, nm = longest_first(cu, n_seq, sh - hm * n_seq);
    if (nm >= 0) {
      h = hm;
      n = nm;
    }
  }
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, kg = lane >> 4;
  const bool consumer = wid < kConsumers;
  const int v0 = slice * kBV;
  // the token range and first global chunk of this workgroup's sequence or segment; VR is the
  // row length of the values and outputs (the state may be wider in the map mode)
  int tb, te, cbase, VR = DV;
  [[maybe_unused]] int seq = n, seg = 0;
  // the warm-up start (segment mode): chunks [0, nwarm) of this workgroup's run precede its
  // segment and write nothing; `zero_start` runs them from a zero state
  int nwarm = 0;
  [[maybe_unused]] bool zero_start = false;
  if constexpr (MODE == kScanSeq) {
    tb = cu[n];
    te = cu[n + 1];
    cbase = chunk_off[n];
  } else {
    const int per = MODE == kScanMap ? sa.G - 1 : sa.G;
    seq = n / per;
    seg = n % per;
    tb = seq * sa.L + seg * sa.Ls;
    te = min(tb + sa.Ls, (seq + 1) * sa.L);
    cbase = seq * ((sa.L + kChunk - 1) / kChunk) + seg * (sa.Ls / kChunk);
    VR = sa.dv;
    // segment 0 starts from S0 and needs no transition: its identity columns have no work
    if (MAP && seg == 0 && v0 >= sa.dv) return;
    const bool warm = warm_start(sa, seq, h, H);
    if (MAP && warm) return;  // the segments start early instead: no transitions needed
    if (MODE == kScanSeg && warm && seg > 0) {
      nwarm = min(sa.W, seg * (sa.Ls / kChunk));
      tb -= nwarm * kChunk;
      cbase -= nwarm;
      zero_start = tb > seq * sa.L;  // else the run starts at the sequence start, from S0
    }
  }
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
  int offK[DP::NK / NP], offTP[DP::NTW], offV[DP::NV / NP];
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
    // T then P (then their low parts), compact tiles in LDS from packed blocks in memory:
    // item m = NP j + pw is instruction m % NTC of tile m / NTC
#pragma unroll
    for (int j = 0; j < DP::NTW; ++j) {
      const int m = NP * j + pw;
      int row, col;
      tpc_piece<Tin>(1024 * (m % DP::NTC) + 16 * lane, row, col);
      offTP[j] = tpb_off<Tin>(row, col);
    }
#pragma unroll
    for (int j = 0; j < DP::NV / NP; ++j) {
      const int J = NP * j + pw, row = (1024 * J + 16 * lane) / (kBV * ES);
      offV[j] = dma_off(J, kBV, H * VR * ES, sw_val<kBV>(row) * (ES / 2));
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
    // value slice (the identity columns of the map mode take zero values: an empty range)
    const bool vcols = !MAP || v0 < VR;
    const Rsrc rv = make_rsrc(v + tok * VR + (vcols ? v0 : 0),
                              vcols ? (uint32_t)(((size_t)(len - 1) * H * VR + kBV) * ES) : 0u);
    // split precision: per chunk-head the hi blocks, then the lo blocks
    constexpr int TS = SPLIT ? 2 : 1;
    const Rsrc rt = make_rsrc(Tm + ch * (TS * kTpbElems), tpb_bytes<Tin>());
    const Rsrc rp = make_rsrc(Pm + ch * (TS * kTpbElems), tpb_bytes<Tin>());
    const Rsrc rg = make_rsrc(GD + ch * kGDFloats, kGDFloats * sizeof(float));
#pragma unroll
    for (int j = 0; j < DP::NK / NP; ++j) {
      const int J = NP * j + pw;
      dma16(rk, s.K + 1024 * J, offK[j]);
      if constexpr (!NOQP) dma16(rq, s.Q + 1024 * J, offK[j]);
    }
#pragma unroll
    for (int j = 0; j < DP::NTW; ++j) {
      const int m = NP * j + pw;
      if (NOQP || m < DP::NTC) {
        dma16(rt, s.T + 1024 * (m % DP::NTC), offTP[j]);
      } else if (m < 2 * DP::NTC) {
        dma16(rp, s.P + 1024 * (m - DP::NTC), offTP[j]);
      } else if constexpr (SPLIT) {
        const Rsrc rtl = make_rsrc(Tm + ch * (2 * kTpbElems) + kTpbElems, tpb_bytes<Tin>());
        const Rsrc rpl = make_rsrc(Pm + ch * (2 * kTpbElems) + kTpbElems, tpb_bytes<Tin>());
        if (m < 3 * DP::NTC) dma16(rtl, s.Tl + 1024 * (m - 2 * DP::NTC), offTP[j]);
        else dma16(rpl, s.Pl + 1024 * (m - 3 * DP::NTC), offTP[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < DP::NV / NP; ++j) {
      const int J = NP * j + pw;
      dma16(rv, s.V + 1024 * J, offV[j]);
    }
    // decays (gam, dec, gamO are consecutive in the slot, 768 bytes; without outputs the
    // first 512): producer pw fetches its share
    constexpr int GDB = (NOQP ? 512 : 768) / NP;
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
    if constexpr (NOQP) return;  // no outputs
    if (c < nwarm) return;       // a warm-up chunk before the segment
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
  const size_t sbase = ((size_t)n * H + h) * DK * (size_t)DV;  // this unit's state (S_T)
  // element (r, cc) of this workgroup's incoming state
  auto initial_state = [&](int r, int cc) -> float {
    if constexpr (MODE == kScanSeq) {
      return S0 ? S0[sbase + (size_t)r * DV + cc] : 0.f;
    } else {
      const size_t seq_base = ((size_t)seq * H + h) * DK * (size_t)VR;
      if (MODE == kScanMap && cc >= VR) return r == cc - VR ? 1.f : 0.f;  // identity columns
      if (seg == 0) return S0 ? S0[seq_base + (size_t)r * VR + cc] : 0.f;
      if (MODE == kScanMap) return 0.f;  // N_g starts from zero
      if (nwarm > 0) return zero_start ? 0.f : (S0 ? S0[seq_base + (size_t)r * VR + cc] : 0.f);
      return sa.Sin[(((size_t)seq * (sa.G - 1) + seg - 1) * H + h) * DK * (size_t)VR +
                    (size_t)r * VR + cc];
    }
  };
  f32x4 Sacc[NM];
  if (consumer) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Sacc[m][i] = initial_state(tmap(m, kg, i), v0 + col);
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
  // the rounding residuals x - bf16(x) of the same operand (split precision)
  auto accB_res = [&](const f32x4 &lo, const f32x4 &hi) {
    FragT r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = from_f32<Tin>(lo[i] - to_f32(from_f32<Tin>(lo[i])));
      r[i + 4] = from_f32<Tin>(hi[i] - to_f32(from_f32<Tin>(hi[i])));
    }
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
        if constexpr (!NOQP) fq[t][ks] = rd_frag(s.Q, KQ{}, frow(t), ks);
      }
    // ---- reads for R = V - Diag(gam) Y and U = T R
    FragT ft[6], ftl[SPLIT ? 6 : 1];
    ft[0] = rd_tp(s.T, frow(0), 0);
    ft[1] = rd_tp(s.T, frow(1), 0);
    ft[2] = rd_tp(s.T, frow(2), 0);
    ft[3] = rd_tp(s.T, frow(2), 1);
    ft[4] = rd_tp(s.T, frow(3), 0);
    ft[5] = rd_tp(s.T, frow(3), 1);
    if constexpr (SPLIT) {
      ftl[0] = rd_tp(s.Tl, frow(0), 0);
      ftl[1] = rd_tp(s.Tl, frow(1), 0);
      ftl[2] = rd_tp(s.Tl, frow(2), 0);
      ftl[3] = rd_tp(s.Tl, frow(2), 1);
      ftl[4] = rd_tp(s.Tl, frow(3), 0);
      ftl[5] = rd_tp(s.Tl, frow(3), 1);
    }
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
    [[maybe_unused]] FragT Uopl[2], Udopl[2];
    {
      f32x4 R[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        OT[t] = zero4();
        if constexpr (!NOQP) {
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) OT[t] = mma(Sop[ks], fq[t][ks], OT[t]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) R[t][i] = vv[t][i] - g4[t][i] * Y[t][i];
      }
      const FragT Rop0 = accB(R[0], R[1]), Rop1 = accB(R[2], R[3]);
      f32x4 U[4];
      U[0] = mma(ft[0], Rop0, zero4());
      U[1] = mma(ft[1], Rop0, zero4());
      U[2] = mma(ft[3], Rop1, mma(ft[2], Rop0, zero4()));
      U[3] = mma(ft[5], Rop1, mma(ft[4], Rop0, zero4()));
      if constexpr (SPLIT) {  // + T_hi R_lo + T_lo R_hi
        const FragT Rl0 = accB_res(R[0], R[1]), Rl1 = accB_res(R[2], R[3]);
        U[0] = mma(ftl[0], Rop0, mma(ft[0], Rl0, U[0]));
        U[1] = mma(ftl[1], Rop0, mma(ft[1], Rl0, U[1]));
        U[2] = mma(ftl[3], Rop1, mma(ft[3], Rl1, mma(ftl[2], Rop0, mma(ft[2], Rl0, U[2]))));
        U[3] = mma(ftl[5], Rop1, mma(ft[5], Rl1, mma(ftl[4], Rop0, mma(ft[4], Rl0, U[3]))));
      }
      f32x4 Ud[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) Ud[t][i] = d4[t][i] * U[t][i];
      Uop[0] = accB(U[0], U[1]);
      Uop[1] = accB(U[2], U[3]);
      Udop[0] = accB(Ud[0], Ud[1]);
      Udop[1] = accB(Ud[2], Ud[3]);
      if constexpr (SPLIT) {
        Uopl[0] = accB_res(U[0], U[1]);
        Uopl[1] = accB_res(U[2], U[3]);
        Udopl[0] = accB_res(Ud[0], Ud[1]);
        Udopl[1] = accB_res(Ud[2], Ud[3]);
      }
    }
    // ---- reads for the output: P fragments and this lane's token decays (none without
    //      outputs)
    FragT fp[6], fpl[SPLIT ? 6 : 1];
    float gt[4];
    if constexpr (!NOQP) {
      fp[0] = rd_tp(s.P, frow(0), 0);
      fp[1] = rd_tp(s.P, frow(1), 0);
      fp[2] = rd_tp(s.P, frow(2), 0);
      fp[3] = rd_tp(s.P, frow(2), 1);
      fp[4] = rd_tp(s.P, frow(3), 0);
      fp[5] = rd_tp(s.P, frow(3), 1);
      if constexpr (SPLIT) {
        fpl[0] = rd_tp(s.Pl, frow(0), 0);
        fpl[1] = rd_tp(s.Pl, frow(1), 0);
        fpl[2] = rd_tp(s.Pl, frow(2), 0);
        fpl[3] = rd_tp(s.Pl, frow(2), 1);
        fpl[4] = rd_tp(s.Pl, frow(3), 0);
        fpl[5] = rd_tp(s.Pl, frow(3), 1);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) gt[t] = s.gamO[frow(t)];
    }
    // ---- S = exp(G_last) S + K^T Diag(dec) U
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if constexpr (DIAG)  // per key channel: rows tmap(m, kg, 0..3) are consecutive
        Sacc[m] *= *reinterpret_cast<const f32x4 *>(&s.gC[tmap(m, kg, 0)]);
      else
        Sacc[m] *= dl;
      Sacc[m] = mma(fkt[m][0], Udop[0], Sacc[m]);
      Sacc[m] = mma(fkt[m][1], Udop[1], Sacc[m]);
      if constexpr (SPLIT) {
        Sacc[m] = mma(fkt[m][0], Udopl[0], Sacc[m]);
        Sacc[m] = mma(fkt[m][1], Udopl[1], Sacc[m]);
      }
    }
    if constexpr (!NOQP) {
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
          if constexpr (SPLIT) O = mma(Uop[0], fpl[t], mma(Uopl[0], fp[t], O));
        } else {
          O = mma(Uop[0], fp[2 * t - 2], O);
          O = mma(Uop[1], fp[2 * t - 1], O);
          if constexpr (SPLIT) {
            O = mma(Uop[0], fpl[2 * t - 2], mma(Uopl[0], fp[2 * t - 2], O));
            O = mma(Uop[1], fpl[2 * t - 1], mma(Uopl[1], fp[2 * t - 1], O));
          }
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
        // chunk c + 1 must be in LDS before the barrier that starts it; this step's chunk
        // c + 2 loads may stay in flight.  The vector-memory counter returns loads in order
        // among themselves but not relative to stores: a store issued after chunk c + 1's
        // loads can complete before them.  So the count left outstanding is the later loads
        // alone (pending stores only make the wait stricter), never loads plus stores.
        if (DIST == 2) {
          if (is) wait_vmcnt<DP::PER_WAVE>();
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

  // the final state: of the sequence, of the map mode's segment ([N_g | M_g]), or of the
  // segment mode's last segment of each sequence
  bool store_st = consumer && S_T;
  size_t st_base = sbase;
  if constexpr (MODE == kScanSeg) {
    store_st = store_st && seg == sa.G - 1;
    st_base = ((size_t)seq * H + h) * DK * (size_t)DV;
  }
  if (store_st) {
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S_T[st_base + (size_t)tmap(m, kg, i) * DV + v0 + col] = Sacc[m][i];
  }
}

// units: sequences (kScanSeq) or segments; DVs: the state's column count (d_v, or
// d_v + d_k in the map mode).
template <typename Tin, int DK, typename SHP, bool DIAG, bool STATES, int MODE,
          bool SPLIT = false>
static hipError_t launch_scan_s(int DVs, int64_t units, const void *q, const void *k,
                                const void *v, const float *GD, const void *T, const void *P,
                                const float *S0, void *o, float *S_T, SeqTables t, int32_t H,
                                hipStream_t stream, const DiagTiles *dg, void *SN,
                                const SegArgs &sa) {
  constexpr bool NOQP = MODE == kScanMap || STATES;
  using SMT = ScanSmem<Tin, DK, SHP::BV, DIAG, NOQP, SPLIT>;
  using SLT = ScanSlot<Tin, DK, SHP::BV, DIAG, NOQP, SPLIT>;
  static_assert(sizeof(SMT) <= kLdsBytes, "LDS budget");
  static_assert(offsetof(SLT, dec) == offsetof(SLT, gam) + 256 &&
                    offsetof(SLT, gamO) == offsetof(SLT, gam) + 512,
                "the decay block is fetched as one contiguous 768-byte piece");
  const size_t smem = sizeof(SMT);
  static std::atomic<bool> attr_set[kMaxDeviceOrdinals];
  if (hipError_t ea = set_lds_limit_once(
          reinterpret_cast<const void *>(&kla_scan_kernel<Tin, DK, SHP, DIAG, STATES, MODE, SPLIT>), (int)smem, attr_set);
      ea != hipSuccess)
    return ea;
  const int64_t blocks = units * H * (DVs / SHP::BV);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((kla_scan_kernel<Tin, DK, SHP, DIAG, STATES, MODE, SPLIT>), dim3((unsigned)blocks),
                     dim3(SHP::THREADS), smem, stream, static_cast<const Tin *>(q),
                     static_cast<const Tin *>(k), static_cast<const Tin *>(v), GD,
                     static_cast<const Tin *>(T), static_cast<const Tin *>(P), S0,
                     static_cast<Tin *>(o), S_T, t.cu, t.chunk_off, (int)units, H, DVs,
                     static_cast<const Tin *>(dg ? dg->kg : nullptr),
                     static_cast<const Tin *>(dg ? dg->qg : nullptr),
                     static_cast<const Tin *>(dg ? dg->kd : nullptr), dg ? dg->gc : nullptr,
                     static_cast<Tin *>(SN), sa);
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
template <typename Tin, int DK, bool DIAG, bool STATES, int MODE = kScanSeq, bool SPLIT = false>
static hipError_t launch_scan_t(int DVs, int64_t units, const void *q, const void *k,
                                const void *v, const float *GD, const void *T, const void *P,
                                const float *S0, void *o, float *S_T, SeqTables t, int32_t H,
                                hipStream_t stream, const DiagTiles *dg, void *SN,
                                const SegArgs &sa = SegArgs{}) {
  const int64_t narrow_blocks = units * H * (DVs / ScanNarrow::BV);
  // workgroups of the narrow shape per CU: one, or in the map mode (two waves per SIMD) as
  // many as the LDS holds, at most two
  constexpr int lds_fit =
      kLdsBytes / (int)sizeof(ScanSmem<Tin, DK, ScanNarrow::BV, DIAG, MODE == kScanMap, SPLIT>);
  constexpr int per_cu = MODE == kScanMap ? (lds_fit >= 2 ? 2 : 1) : 1;
  const int64_t fit = (int64_t)device_cus() * per_cu;
  if (fit > 0 && narrow_blocks > fit)
    return launch_scan_s<Tin, DK, ScanWide, DIAG, STATES, MODE, SPLIT>(
        DVs, units, q, k, v, GD, T, P, S0, o, S_T, t, H, stream, dg, SN, sa);
  return launch_scan_s<Tin, DK, ScanNarrow, DIAG, STATES, MODE, SPLIT>(
      DVs, units, q, k, v, GD, T, P, S0, o, S_T, t, H, stream, dg, SN, sa);
}

template <typename Tin, int DK>
static hipError_t launch_scan_g(int d_v, const void *q, const void *k, const void *v,
                                const float *GD, const void *T, const void *P, const float *S0,
                                void *o, float *S_T, SeqTables t, int32_t n_seq, int32_t H,
                                hipStream_t stream, const DiagTiles *dg, void *SN) {
  if (dg) {
    if (SN)
      return launch_scan_t<Tin, DK, true, true>(d_v, n_seq, q, k, v, GD, T, P, S0, o, S_T, t, H,
                                                stream, dg, SN);
    return launch_scan_t<Tin, DK, true, false>(d_v, n_seq, q, k, v, GD, T, P, S0, o, S_T, t, H,
                                               stream, dg, nullptr);
  }
  if (SN)
    return launch_scan_t<Tin, DK, false, true>(d_v, n_seq, q, k, v, GD, T, P, S0, o, S_T, t, H,
                                               stream, nullptr, SN);
  return launch_scan_t<Tin, DK, false, false>(d_v, n_seq, q, k, v, GD, T, P, S0, o, S_T, t, H,
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

hipError_t launch_scan_split(int d_k, int d_v, const void *q, const void *k, const void *v,
                             const float *GD, const void *T, const void *P, const float *S0,
                             void *o, float *S_T, SeqTables t, int32_t n_seq, int32_t H,
                             hipStream_t stream) {
  if (d_k == 128)
    return launch_scan_t<__bf16, 128, false, false, kScanSeq, true>(
        d_v, n_seq, q, k, v, GD, T, P, S0, o, S_T, t, H, stream, nullptr, nullptr);
  return launch_scan_t<__bf16, 64, false, false, kScanSeq, true>(
      d_v, n_seq, q, k, v, GD, T, P, S0, o, S_T, t, H, stream, nullptr, nullptr);
}

// ---------------------------------------------------------------------------------------------
// The two-level scan's middle phase, sequential over the segments of each sequence: the map
// mode left, per (sequence, segment g < G - 1, head), [N_g | M_g] (d_k x (d_v + d_k)) with
// N_0 = S_out of segment 0 from S0; so the incoming states are S_in(1) = N_0 and
// S_in(g + 1) = M_g S_in(g) + N_g (Eq. (9): S_out is affine in S_in), in fp32 on the matrix
// cores (fp32 16x16x4 steps: exact products).  One workgroup of four wavefronts per
// (sequence, head, 16 state columns); wavefront w forms rows [d_k/4 w, d_k/4 (w + 1)).  The
// contraction over the d_k rows of S_in is ordered so that lane group kg takes the rows
// [d_k/4 kg, d_k/4 (kg + 1)): each lane then reads a contiguous run of M_g's row from memory,
// and S_in sits in LDS with row k at position 4 (k mod d_k/4) + k div d_k/4, so that the
// four lane groups of one step read four consecutive rows.
// ---------------------------------------------------------------------------------------------
template <int DK>
__global__ __launch_bounds__(256) void kla_seg_combine_kernel(const float *__restrict__ NM,
                                                              float *__restrict__ Sin, int G,
                                                              int H, int dv, SegArgs sa) {
  constexpr int KS = DK / 4;   // contraction steps; also rows per wavefront
  constexpr int TW = KS / 16;  // 16-row output tiles per wavefront
  constexpr int NF = KS / 4;   // float4 pieces of a lane's run of M_g's row
  __shared__ __align__(16) float Ss[DK * 16];
  const int nsl = dv / 16;
  const int slice = blockIdx.x % nsl, sh = blockIdx.x / nsl;
  const int h = sh % H, n = sh / H;
  if (warm_start(sa, n, h, H)) return;  // the segments start early instead
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r16 = lane & 15, kg = lane >> 4;
  const int W = dv + DK, c0 = 16 * slice;
  auto nm = [&](int g) { return NM + (((size_t)n * (G - 1) + g) * H + h) * DK * (size_t)W; };
  auto sin_ = [&](int g) { return Sin + (((size_t)n * (G - 1) + g) * H + h) * DK * (size_t)dv; };
  auto pos = [](int k) { return 16 * (4 * (k % KS) + k / KS); };
  {
    const float *N0 = nm(0);
    float *S1 = sin_(0);
    for (int e = tid; e < DK * 16; e += 256) {
      const int r = e >> 4, cc = e & 15;
      const float x = N0[(size_t)r * W + c0 + cc];
      Ss[pos(r) + cc] = x;
      S1[(size_t)r * dv + c0 + cc] = x;
    }
  }
  // this lane's operands of step g: M_g[row][KS kg .. + KS) for the rows of its tiles, and
  // the N_g entries its accumulators start from.  Three register buffers in rotation keep
  // the loads of the next two steps in flight while one step runs.
  struct Ops {
    f32x4 A[TW][NF], N[TW];
  };
  auto load = [&](Ops &o, int g) {
    if (g + 1 >= G) return;  // no such step
    const float *b = nm(g);
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      const int row = KS * w + 16 * t + r16;
#pragma unroll
      for (int j = 0; j < NF; ++j)
        o.A[t][j] = *reinterpret_cast<const f32x4 *>(b + (size_t)row * W + dv + KS * kg + 4 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o.N[t][e] = b[(size_t)(KS * w + 16 * t + 4 * kg + e) * W + c0 + r16];
    }
  };
  auto step = [&](const Ops &o, int g) {
    // two accumulators per tile (even and odd contraction steps) halve the dependent chain
    f32x4 acc[TW][2];
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      acc[t][0] = o.N[t];
      acc[t][1] = zero4();
    }
    __syncthreads();  // Ss holds S_in(g)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const float bv = Ss[16 * (4 * s + kg) + r16];
#pragma unroll
      for (int t = 0; t < TW; ++t)
        acc[t][s & 1] =
            __builtin_amdgcn_mfma_f32_16x16x4f32(o.A[t][s >> 2][s & 3], bv, acc[t][s & 1], 0, 0, 0);
    }
    __syncthreads();  // every read of S_in(g) is done
    float *So = sin_(g);
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = KS * w + 16 * t + 4 * kg + e;
        const float x = acc[t][0][e] + acc[t][1][e];
        Ss[pos(row) + r16] = x;
        So[(size_t)row * dv + c0 + r16] = x;
      }
  };
  Ops o0, o1, o2;
  load(o0, 1);
  load(o1, 2);
  for (int g = 1; g + 1 < G; g += 3) {
    load(o2, g + 2);
    step(o0, g);
    if (g + 2 >= G) break;
    load(o0, g + 3);
    step(o1, g + 1);
    if (g + 3 >= G) break;
    load(o1, g + 4);
    step(o2, g + 2);
  }
}

template <typename Tin, int DK>
static hipError_t launch_two_level_t(int d_v, const void *q, const void *k, const void *v,
                                     const float *GD, const void *T, const void *P,
                                     const float *S0, void *o, float *S_T, int32_t n_seq,
                                     int32_t H, const SegArgs &sa0, float *NM, float *Sin,
                                     hipStream_t stream) {
  const SeqTables none{nullptr, nullptr};
  SegArgs sa = sa0;
  sa.Sin = Sin;
  hipError_t e = launch_scan_t<Tin, DK, false, false, kScanMap>(
      d_v + DK, (int64_t)n_seq * (sa.G - 1), q, k, v, GD, T, P, S0, nullptr, NM, none, H, stream,
      nullptr, nullptr, sa);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kla_seg_combine_kernel<DK>, dim3((unsigned)(n_seq * H * (d_v / 16))),
                     dim3(256), 0, stream, NM, Sin, sa.G, H, d_v, sa);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_scan_t<Tin, DK, false, false, kScanSeg>(d_v, (int64_t)n_seq * sa.G, q, k, v, GD,
                                                        T, P, S0, o, S_T, none, H, stream, nullptr,
                                                        nullptr, sa);
}

hipError_t launch_scan_two_level(Dtype dt, int d_k, int d_v, const void *q, const void *k,
                                 const void *v, const float *GD, const void *T, const void *P,
                                 const float *S0, void *o, float *S_T, int32_t n_seq, int32_t H,
                                 const SegArgs &sa, float *NM, float *Sin, hipStream_t stream) {
  if (sa.G < 2 || sa.Ls <= 0 || sa.Ls % kChunk != 0 || sa.dv != d_v) return hipErrorInvalidValue;
  if (dt == Dtype::BF16) {
    if (d_k == 128)
      return launch_two_level_t<__bf16, 128>(d_v, q, k, v, GD, T, P, S0, o, S_T, n_seq, H, sa, NM,
                                             Sin, stream);
    return launch_two_level_t<__bf16, 64>(d_v, q, k, v, GD, T, P, S0, o, S_T, n_seq, H, sa, NM,
                                          Sin, stream);
  }
  if (d_k == 128)
    return launch_two_level_t<float, 128>(d_v, q, k, v, GD, T, P, S0, o, S_T, n_seq, H, sa, NM,
                                          Sin, stream);
  return launch_two_level_t<float, 64>(d_v, q, k, v, GD, T, P, S0, o, S_T, n_seq, H, sa, NM, Sin,
                                       stream);
}

}  // namespace kla
