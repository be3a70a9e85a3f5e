// kla_launch.h -- host-side launchers of the gfx950 KLA kernels (internal to libkla.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "kla_device.h"

namespace kla {

enum class Dtype { F32 = 0, BF16 = 1 };

// Raises kernel `fn`'s dynamic LDS limit to `bytes` on the current device, once per device
// (the attribute belongs to the device's copy of the kernel).  `done` is the launcher's own
// table of flags, one per device ordinal; concurrent first calls both set the same value.
constexpr int kMaxDeviceOrdinals = 64;
inline hipError_t set_lds_limit_once(const void *fn, int bytes,
                                     std::atomic<bool> (&done)[kMaxDeviceOrdinals]) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDeviceOrdinals && done[dev].load(std::memory_order_acquire))
    return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && dev >= 0 && dev < kMaxDeviceOrdinals)
    done[dev].store(true, std::memory_order_release);
  return e;
}

// Sequence tables the plan kernel writes into the workspace:
//   cu[n]        sanitised token offset of sequence n (n = 0..n_seq)
//   chunk_off[n] index of sequence n's first chunk; chunk_off[n_seq] = chunk count
struct SeqTables {
  int32_t *cu;
  int32_t *chunk_off;
};

// Upper bound on the number of 64-token chunks for any packing of these totals.
inline int64_t chunk_upper_bound(int64_t n_seq, int64_t total_tokens) {
  return (total_tokens + 63) / 64 + n_seq;
}

hipError_t launch_plan(const int32_t *cu_in, int32_t n_seq, int32_t total_tokens, SeqTables t,
                       hipStream_t stream);

// How the prep kernel finds each chunk's sequence.  kPlanTables: from tables launch_plan
// wrote.  kPlanDense (cu_in == NULL, equal lengths) and kPlanWave (n_seq <= kPlanWaveMax):
// computed inside the prep kernel, which then also writes the tables for the scan, so that
// no plan launch is needed.
enum PlanMode { kPlanTables = 0, kPlanDense = 1, kPlanWave = 2 };
constexpr int kPlanWaveMax = 63;
struct PlanArgs {
  int mode;
  const int32_t *cu_in;  // raw offsets (kPlanWave)
  int32_t total;         // total tokens
};

// Decay factors per chunk-head, 3 x 64 fp32: exp(G_i), exp(G_last - G_i), and the output
// factor exp(G_i) (divided by ||q_i|| under the normalised readout).
constexpr int kGDFloats = 3 * 64;

// a1 + a2: b, G, Gram, L, T = (I + L)^{-1} Diag(b) per chunk-head.  T is written in fp32
// when t_fp32 is set, else in the operand type (what the scan kernel reads).  With q and
// P_out given, also P = A o Q K^T per chunk-head (operand type, zero above the diagonal;
// rows divided by ||q_i|| under the normalised readout).  G_out / beta_out (per token) and
// GD_out (per chunk-head decay factors) are each optional.  tp_split (bf16, packed): T and
// P as hi = bf16(x) and lo = bf16(x - hi) blocks, the lo blocks after the hi ones of each
// chunk-head (twice the packed size).  X_out (optional): X = (I + L)^{-1} itself in the
// operand type, packed blocks (kTpbElems elements per chunk-head), for the backward pass.  LC_out (optional):
// per chunk-head the natural log of a bound on the spectral norm of the chunk's homogeneous
// state map, G_last + sum_t ln max(1, |1 - b_t ||k_t||^2|).
hipError_t launch_prep(Dtype dt, int d_k, const void *q, const void *k, const float *g,
                       const float *eta, float eps, const CoefOpts &opts, SeqTables t,
                       int32_t n_seq, int64_t n_chunks_ub, int32_t H, float *G_out,
                       float *beta_out, void *T_out, bool t_fp32, void *P_out, float *GD_out,
                       const PlanArgs &pa, hipStream_t stream, bool tp_split = false,
                       void *X_out = nullptr, float *LC_out = nullptr);

// Diagonal gating: the decayed key and query tiles per chunk-head ([64][d_k] each, operand
// type) K o exp(G), Q o exp(G), K o exp(G_last - G), and exp(G_last) ([d_k] fp32).
struct DiagTiles {
  const void *kg, *qg, *kd;
  const float *gc;
};

// a1 + a2 under diagonal gating (g [n_tok, H, d_k]): b, T and P (packed blocks), unit decays
// with the readout factor in GD, and the decayed tiles.  Reads the tables launch_plan wrote.
// For the backward pass, X_out and A_out (non-null) also receive X = (I + Diag(b) A)^{-1} and
// A itself per chunk-head, in the operand type, as ten packed 16 x 16 blocks like T.
hipError_t launch_prep_diag(Dtype dt, int d_k, const void *q, const void *k, const float *g,
                            const float *eta, float eps, const CoefOpts &opts, SeqTables t,
                            int32_t n_seq, int64_t n_chunks_ub, int32_t H, const DiagTiles &tiles,
                            void *T_out, void *P_out, float *GD_out, hipStream_t stream,
                            void *X_out = nullptr, void *A_out = nullptr);

// Optional WY factors W = T Diag(exp G) K and U~ = T V (unit-check path).
hipError_t launch_wy(Dtype dt, int d_k, int d_v, const void *k, const void *v, const float *G,
                     const float *T, SeqTables t, int32_t n_seq, int64_t n_chunks_ub, int32_t H,
                     float *W, float *Ut, hipStream_t stream);

// a3 + a4: sequential chunk scan with the output fused in; reads T, P and the per-chunk
// decays GD that launch_prep wrote.  With diag (non-null), the diagonal-gated scan: K and Q
// come from the decayed tiles, the state update uses K o exp(G_last - G) and the state decays
// by exp(G_last) per key channel.  With SN (non-null), every chunk's
// incoming state, [chunk][H][d_k][d_v] in the operand type by global chunk number, for the
// backward pass, and no outputs (q, P and o are not read or written and may be null).
hipError_t launch_scan(Dtype dt, int d_k, int d_v, const void *q, const void *k, const void *v,
                       const float *GD, const void *T, const void *P, const float *S0, void *o,
                       float *S_T, SeqTables t, int32_t n_seq, int32_t H, hipStream_t stream,
                       const DiagTiles *diag = nullptr, void *SN = nullptr);

// launch_scan for bf16 operands at split precision (scalar gate): T and P as hi/lo pairs
// (launch_prep with tp_split), and T R, P U, K^T Diag(dec) U on hi/lo operand pairs.
hipError_t launch_scan_split(int d_k, int d_v, const void *q, const void *k, const void *v,
                             const float *GD, const void *T, const void *P, const float *S0,
                             void *o, float *S_T, SeqTables t, int32_t n_seq, int32_t H,
                             hipStream_t stream);

// The two-level scan of equal-length sequences (the chunk scan's map, combine and segment
// phases), for few long sequences: each sequence of L tokens is cut into G segments of Ls
// tokens (a multiple of 64; the last one may be shorter).  NM holds [n_seq][G-1][H][d_k]
// [d_v + d_k] fp32 and Sin [n_seq][G-1][H][d_k][d_v] fp32 (scratch).  Same inputs and
// outputs as launch_scan with equal-length sequence tables.  With sa.LC and sa.W, the
// warm-up start above where it holds.
enum ScanMode { kScanSeq = 0, kScanMap = 1, kScanSeg = 2 };
struct SegArgs {
  int G = 0;                   // segments per sequence
  int L = 0;                   // tokens per sequence
  int Ls = 0;                  // tokens per segment
  int dv = 0;                  // value columns d_v
  const float *Sin = nullptr;  // incoming states of segments 1 .. G-1 (set by the launcher)
  // Warm-up start (optional): per chunk-head the log contraction bound launch_prep writes
  // (LC_out), and the warm-up length W in chunks.  A (sequence, head) whose every segment
  // boundary is preceded by W chunks that contract the state by 2^-150 or more (or that reach
  // back to the sequence start) skips the map and combine phases: each segment starts W
  // chunks early from a zero state (from S0 at the sequence start) and writes outputs from
  // its own first chunk on.
  const float *LC = nullptr;
  int W = 0;
};
// ln(2^-150): the warm-up start's contraction threshold
constexpr float kWarmLog = -103.97207708399179f;
hipError_t launch_scan_two_level(Dtype dt, int d_k, int d_v, const void *q, const void *k,
                                 const void *v, const float *GD, const void *T, const void *P,
                                 const float *S0, void *o, float *S_T, int32_t n_seq, int32_t H,
                                 const SegArgs &sa, float *NM, float *Sin, hipStream_t stream);

// The backward pass after launch_prep (with the same opts, and X_out = X) and launch_scan
// with SN: the adjoint scan (per chunk-head dS' ([d_k][d_v]) and dU ([64][d_v]) in the
// operand type into dSo and dU: fp32 row-major, or bf16 with each 32-column slice's block
// contiguous; dv = dR, and dS0 if non-null), then the per-chunk gradients (which read dR back
// from dv) dq, dk (operand type) and dg, deta (fp32).  dST may be null (a zero cotangent of
// the final state).  Diagonal gating (diag non-null): after launch_prep_diag with X_out = X and
// A_out = A and launch_scan with diag and SN; g and dg are [n_tok, H, d_k].
hipError_t launch_bwd(Dtype dt, int d_k, int d_v, const void *q, const void *k, const void *v,
                      const void *dO, const float *g, const float *eta, float eps,
                      const CoefOpts &opts, const float *GD, const void *T, const void *P,
                      const void *X, const float *dST, const void *SN, void *dSo, void *dU,
                      void *dq, void *dk, void *dv, float *dg, float *deta, float *dS0,
                      SeqTables t, int32_t n_seq, int64_t n_chunks_ub, int32_t H,
                      hipStream_t stream, const DiagTiles *diag = nullptr,
                      const void *A = nullptr);

// a5: one decode step.
hipError_t launch_decode(Dtype dt, int d_k, int d_v, const void *q, const void *k, const void *v,
                         const float *g, const float *eta, float eps, const CoefOpts &opts,
                         const float *S, void *o, float *S_new, int32_t batch, int32_t H,
                         hipStream_t stream);

}  // namespace kla
