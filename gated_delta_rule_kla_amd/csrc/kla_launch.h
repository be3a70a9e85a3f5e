// kla_launch.h -- host-side launchers of the gfx950 KLA kernels (internal to libkla.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kla_device.h"

namespace kla {

enum class Dtype { F32 = 0, BF16 = 1 };

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
// GD_out (per chunk-head decay factors) are each optional.
hipError_t launch_prep(Dtype dt, int d_k, const void *q, const void *k, const float *g,
                       const float *eta, float eps, const CoefOpts &opts, SeqTables t,
                       int32_t n_seq, int64_t n_chunks_ub, int32_t H, float *G_out,
                       float *beta_out, void *T_out, bool t_fp32, void *P_out, float *GD_out,
                       const PlanArgs &pa, hipStream_t stream);

// Diagonal gating: the decayed key and query tiles per chunk-head ([64][d_k] each, operand
// type) K o exp(G), Q o exp(G), K o exp(G_last - G), and exp(G_last) ([d_k] fp32).
struct DiagTiles {
  const void *kg, *qg, *kd;
  const float *gc;
};

// a1 + a2 under diagonal gating (g [n_tok, H, d_k]): b, T and P (packed blocks), unit decays
// with the readout factor in GD, and the decayed tiles.  Reads the tables launch_plan wrote.
hipError_t launch_prep_diag(Dtype dt, int d_k, const void *q, const void *k, const float *g,
                            const float *eta, float eps, const CoefOpts &opts, SeqTables t,
                            int32_t n_seq, int64_t n_chunks_ub, int32_t H, const DiagTiles &tiles,
                            void *T_out, void *P_out, float *GD_out, hipStream_t stream);

// Optional WY factors W = T Diag(exp G) K and U~ = T V (unit-check path).
hipError_t launch_wy(Dtype dt, int d_k, int d_v, const void *k, const void *v, const float *G,
                     const float *T, SeqTables t, int32_t n_seq, int64_t n_chunks_ub, int32_t H,
                     float *W, float *Ut, hipStream_t stream);

// a3 + a4: sequential chunk scan with the output fused in; reads T, P and the per-chunk
// decays GD that launch_prep wrote.  With diag (non-null), the diagonal-gated scan: K and Q
// come from the decayed tiles, the state update uses K o exp(G_last - G) and the state decays
// by exp(G_last) per key channel.  With SN (non-null; scalar gate only), also every chunk's
// incoming state, [chunk][H][d_k][d_v] in the operand type by global chunk number, for the
// backward pass.
hipError_t launch_scan(Dtype dt, int d_k, int d_v, const void *q, const void *k, const void *v,
                       const float *GD, const void *T, const void *P, const float *S0, void *o,
                       float *S_T, SeqTables t, int32_t n_seq, int32_t H, hipStream_t stream,
                       const DiagTiles *diag = nullptr, void *SN = nullptr);

// The backward pass after launch_prep (with the same opts) and launch_scan with SN: the adjoint scan (dS' per
// chunk into dSo, dU and dR into their [chunk][H][64][d_v] fp32 buffers, dv, and dS0 if
// non-null), then the per-chunk gradients dq, dk (operand type) and dg, deta (fp32).  dST
// may be null (a zero cotangent of the final state).
hipError_t launch_bwd(Dtype dt, int d_k, int d_v, const void *q, const void *k, const void *v,
                      const void *dO, const float *g, const float *eta, float eps,
                      const CoefOpts &opts, const float *GD, const void *T, const void *P, const float *dST,
                      const void *SN, float *dSo, float *dU, float *dR, void *dq, void *dk,
                      void *dv, float *dg, float *deta, float *dS0, SeqTables t, int32_t n_seq,
                      int64_t n_chunks_ub, int32_t H, hipStream_t stream);

// a5: one decode step.
hipError_t launch_decode(Dtype dt, int d_k, int d_v, const void *q, const void *k, const void *v,
                         const float *g, const float *eta, float eps, const CoefOpts &opts,
                         const float *S, void *o, float *S_new, int32_t batch, int32_t H,
                         hipStream_t stream);

}  // namespace kla
