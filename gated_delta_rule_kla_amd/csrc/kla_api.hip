// kla_api.hip -- the extern "C" boundary of libkla.so (declared in include/kla.h).
//
// Validates arguments, carves the caller's workspace, and enqueues the kernels
// on the caller's stream.  Nothing here synchronises with the device or
// allocates device memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "kla.h"
#include "kla_launch.h"

namespace {

thread_local char g_last_error[512] = "";

kla_status fail(kla_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

kla_status ok() {
  g_last_error[0] = '\0';
  return KLA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool supported_dk(int32_t d) { return d == 64 || d == 128; }
bool supported_dv(int32_t d) { return d == 64 || d == 128 || d == 256; }

size_t elem_size(kla_dtype dt) { return dt == KLA_DTYPE_BF16 ? 2 : 4; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// Workspace layout, each part 256-byte aligned:
//   [cu: n_seq+1 int32][chunk_off: n_seq+1 int32][G: total*H fp32]
//   [GD: n_chunks_ub * H * 192 fp32][T: n_chunks_ub * H * 10 * 256][P: same]
// T and P are stored by the prep kernel as their ten 16 x 16 blocks on and below the
// diagonal, in the operand type (es bytes per element).
struct WsLayout {
  size_t off_cu, off_co, off_G, off_GD, off_T, off_P;
  // diagonal gating only: per chunk-head the decayed key and query tiles K o exp(G),
  // Q o exp(G), K o exp(G_last - G) ([64][d_k] each, operand type) and exp(G_last) ([d_k])
  size_t off_KG = 0, off_QG = 0, off_KD = 0, off_GC = 0;
  // two-level scan only (G >= 2 segments): [N_g | M_g] per (sequence, segment < G-1, head),
  // [d_k][d_v + d_k] fp32, the chained incoming states, [d_k][d_v] fp32, and per chunk-head
  // the log contraction bound of the warm-up test (fp32)
  size_t off_NM = 0, off_Sin = 0, off_LC = 0;
  size_t total;
};

// The two-level scan's segmentation of a dense problem: G segments of Ls tokens (G = 0: the
// sequential scan).  A function of the shape and the option only, so that the workspace
// size does not depend on the device.  segs_opt: 0 automatic, 1 sequential, >= 2 requested.
struct SegPlan {
  int G = 0, Ls = 0;
};
// Warm-up length of the two-level scan's early segment starts, in chunks (512 tokens).
constexpr int kWarmChunks = 8;
SegPlan seg_plan(int64_t n_seq, int64_t total_tokens, int64_t H, int64_t d_v, bool diag,
                 int32_t segs_opt, bool split = false) {
  SegPlan p;
  if (diag || split || segs_opt == 1 || segs_opt < 0 || n_seq <= 0 || H <= 0 || d_v < 32 ||
      total_tokens <= 0 || total_tokens % n_seq != 0)
    return p;
  const int64_t L = total_tokens / n_seq, cpl = (L + KLA_CHUNK - 1) / KLA_CHUNK;
  int64_t G = segs_opt;
  if (G == 0) {
    const int64_t blocks = n_seq * H * (d_v / 32);  // workgroups of the sequential scan
    if (2 * blocks > 256) return p;
    G = std::min<int64_t>(512 / blocks, cpl / 32);
  }
  G = std::min<int64_t>(G, cpl);
  if (G < 2) return p;
  const int64_t per = (cpl + G - 1) / G;  // chunks per segment
  G = (cpl + per - 1) / per;              // segments that hold tokens
  if (G < 2) return p;
  p.G = (int)G;
  p.Ls = (int)(per * KLA_CHUNK);
  return p;
}

WsLayout ws_layout(int64_t n_seq, int64_t total_tokens, int64_t H, int64_t d_k, size_t es,
                   bool diag = false, int64_t d_v = 0, int segs = 0, bool split = false) {
  WsLayout w;
  w.off_cu = 0;
  w.off_co = align256(w.off_cu + sizeof(int32_t) * (size_t)(n_seq + 1));
  w.off_G = align256(w.off_co + sizeof(int32_t) * (size_t)(n_seq + 1));
  const int64_t nch = kla::chunk_upper_bound(n_seq, total_tokens);
  w.off_GD = align256(w.off_G + sizeof(float) * (size_t)total_tokens * (size_t)H);
  w.off_T = align256(w.off_GD + sizeof(float) * (size_t)nch * (size_t)H * kla::kGDFloats);
  // split precision: hi and lo blocks per chunk-head
  const size_t tile_bytes = es * (size_t)nch * (size_t)H * kla::kTpbElems * (split ? 2 : 1);
  w.off_P = align256(w.off_T + tile_bytes);
  w.total = align256(w.off_P + tile_bytes);
  if (diag) {
    const size_t kt = es * (size_t)nch * (size_t)H * KLA_CHUNK * (size_t)d_k;
    w.off_KG = w.total;
    w.off_QG = align256(w.off_KG + kt);
    w.off_KD = align256(w.off_QG + kt);
    w.off_GC = align256(w.off_KD + kt);
    w.total = align256(w.off_GC + sizeof(float) * (size_t)nch * (size_t)H * (size_t)d_k);
  }
  if (segs >= 2) {
    const size_t units = (size_t)n_seq * (size_t)(segs - 1) * (size_t)H * (size_t)d_k;
    w.off_NM = w.total;
    w.off_Sin = align256(w.off_NM + sizeof(float) * units * (size_t)(d_v + d_k));
    w.off_LC = align256(w.off_Sin + sizeof(float) * units * (size_t)d_v);
    w.total = align256(w.off_LC + sizeof(float) * (size_t)nch * (size_t)H);
  }
  return w;
}

// Checks shared by the prefill entry points.  Returns KLA_OK or an error status.
kla_status check_prefill_shape(const int32_t *cu_seqlens_host, int32_t n_seq, int32_t total_tokens,
                               int32_t n_heads, int32_t d_k, int32_t d_v, kla_dtype dtype,
                               float eps) {
  if (dtype != KLA_DTYPE_F32 && dtype != KLA_DTYPE_BF16)
    return fail(KLA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (n_seq <= 0 || total_tokens < 0 || n_heads <= 0)
    return fail(KLA_ERR_INVALID_ARGUMENT, "need n_seq > 0, total_tokens >= 0, n_heads > 0 (got %d, %d, %d)",
                n_seq, total_tokens, n_heads);
  if (n_heads > 65535) return fail(KLA_ERR_INVALID_ARGUMENT, "n_heads > 65535");
  if (!supported_dk(d_k)) return fail(KLA_ERR_UNSUPPORTED, "d_k = %d not in {64, 128}", d_k);
  if (!supported_dv(d_v)) return fail(KLA_ERR_UNSUPPORTED, "d_v = %d not in {64, 128, 256}", d_v);
  if (!(eps >= 0.f) || !isfinite(eps))
    return fail(KLA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if ((int64_t)n_seq * n_heads * (d_v / 32) > 0x7fffffff)
    return fail(KLA_ERR_INVALID_ARGUMENT, "n_seq * n_heads too large");
  // the scan addresses one 64-token chunk of a tensor with 32-bit buffer offsets
  if ((int64_t)KLA_CHUNK * n_heads * (d_k > d_v ? d_k : d_v) * (int64_t)elem_size(dtype) > 0x7fffffff)
    return fail(KLA_ERR_UNSUPPORTED,
                "64 * n_heads * max(d_k, d_v) * element size must be below 2^31 bytes");
  if (cu_seqlens_host) {
    if (cu_seqlens_host[0] != 0)
      return fail(KLA_ERR_INVALID_ARGUMENT, "cu_seqlens[0] must be 0");
    for (int32_t i = 0; i < n_seq; ++i)
      if (cu_seqlens_host[i + 1] < cu_seqlens_host[i])
        return fail(KLA_ERR_INVALID_ARGUMENT, "cu_seqlens decreases at %d", i);
    if (cu_seqlens_host[n_seq] != total_tokens)
      return fail(KLA_ERR_INVALID_ARGUMENT, "cu_seqlens[n_seq] = %d != total_tokens = %d",
                  cu_seqlens_host[n_seq], total_tokens);
  }
  return KLA_OK;
}

kla_status check_dense(const int32_t *cu_seqlens, int32_t n_seq, int32_t total_tokens) {
  if (!cu_seqlens && total_tokens % n_seq != 0)
    return fail(KLA_ERR_INVALID_ARGUMENT,
                "dense input needs total_tokens (%d) divisible by n_seq (%d); pass cu_seqlens",
                total_tokens, n_seq);
  if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
    return fail(KLA_ERR_INVALID_ARGUMENT, "cu_seqlens must be 4-byte aligned");
  return KLA_OK;
}

kla::Dtype to_dt(kla_dtype d) { return d == KLA_DTYPE_BF16 ? kla::Dtype::BF16 : kla::Dtype::F32; }

// kla_options -> the kernels' CoefOpts (NULL = the defaults), validated.
kla_status to_coef(const kla_options *opts, kla::CoefOpts *out) {
  *out = kla::CoefOpts{kla::kBetaKaczmarz, 0, nullptr};
  if (!opts) return KLA_OK;
  if (opts->beta_mode < KLA_BETA_KACZMARZ || opts->beta_mode > KLA_BETA_INV_LOG_T)
    return fail(KLA_ERR_UNSUPPORTED, "unknown beta_mode %d", (int)opts->beta_mode);
  if (opts->precision != KLA_PRECISION_BF16 && opts->precision != KLA_PRECISION_SPLIT)
    return fail(KLA_ERR_UNSUPPORTED, "unknown precision %d", (int)opts->precision);
  if (opts->pos_offset && !aligned_to(opts->pos_offset, 4))
    return fail(KLA_ERR_INVALID_ARGUMENT, "pos_offset must be 4-byte aligned");
  *out = kla::CoefOpts{opts->beta_mode, opts->normalize_q != 0 ? 1 : 0, opts->pos_offset,
                       opts->diagonal_gate != 0 ? 1 : 0};
  return KLA_OK;
}

kla_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return KLA_OK;
  return fail(KLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

size_t kla_prefill_workspace_bytes_ex(int32_t n_seq, int32_t total_tokens, int32_t n_heads,
                                      int32_t d_k, int32_t d_v, kla_dtype dtype,
                                      const kla_options *opts) {
  if (n_seq <= 0 || total_tokens < 0 || n_heads <= 0 || !supported_dk(d_k) ||
      !supported_dv(d_v) || (dtype != KLA_DTYPE_F32 && dtype != KLA_DTYPE_BF16))
    return 0;
  const bool diag = opts && opts->diagonal_gate != 0;
  const bool split = opts && opts->precision == KLA_PRECISION_SPLIT && dtype == KLA_DTYPE_BF16;
  const SegPlan sp =
      seg_plan(n_seq, total_tokens, n_heads, d_v, diag, opts ? opts->scan_segments : 0, split);
  return ws_layout(n_seq, total_tokens, n_heads, d_k, elem_size(dtype), diag, d_v, sp.G, split)
      .total;
}

size_t kla_prefill_workspace_bytes(int32_t n_seq, int32_t total_tokens, int32_t n_heads,
                                   int32_t d_k, int32_t d_v, kla_dtype dtype) {
  return kla_prefill_workspace_bytes_ex(n_seq, total_tokens, n_heads, d_k, d_v, dtype, nullptr);
}

}  // extern "C"

namespace {

// Backward workspace: the forward layout, then per chunk-head the incoming states S and the
// cotangents dS' of the outgoing ones ([d_k][d_v]), dU ([64][d_v]) and X = (I + L)^{-1}
// (packed blocks, kTpbElems elements), all in the operand type (dR goes to dv, an output).
// Diagonal gating adds the forward's decayed tiles (in the forward layout) and A itself
// (packed blocks like X).
struct BwdLayout {
  WsLayout fw;
  size_t off_SN, off_dSo, off_dU, off_X, off_A = 0, total;
};

BwdLayout bwd_layout(int64_t n_seq, int64_t total_tokens, int64_t H, int64_t d_k, int64_t d_v,
                     size_t es, bool diag = false) {
  BwdLayout b;
  b.fw = ws_layout(n_seq, total_tokens, H, d_k, es, diag);
  const size_t nch = (size_t)kla::chunk_upper_bound(n_seq, total_tokens);
  const size_t st = es * nch * (size_t)H * (size_t)d_k * (size_t)d_v;
  const size_t ut = es * nch * (size_t)H * KLA_CHUNK * (size_t)d_v;
  b.off_SN = b.fw.total;
  b.off_dSo = align256(b.off_SN + es * nch * (size_t)H * (size_t)d_k * (size_t)d_v);
  b.off_dU = align256(b.off_dSo + st);
  b.off_X = align256(b.off_dU + ut);
  b.total = align256(b.off_X + es * nch * (size_t)H * kla::kTpbElems);
  if (diag) {
    b.off_A = b.total;
    b.total = align256(b.off_A + es * nch * (size_t)H * kla::kTpbElems);
  }
  return b;
}

}  // namespace

extern "C" {

size_t kla_prefill_backward_workspace_bytes_ex(int32_t n_seq, int32_t total_tokens,
                                               int32_t n_heads, int32_t d_k, int32_t d_v,
                                               kla_dtype dtype, const kla_options *opts) {
  if (n_seq <= 0 || total_tokens < 0 || n_heads <= 0 || !supported_dk(d_k) ||
      !supported_dv(d_v) || (dtype != KLA_DTYPE_F32 && dtype != KLA_DTYPE_BF16))
    return 0;
  return bwd_layout(n_seq, total_tokens, n_heads, d_k, d_v, elem_size(dtype),
                    opts && opts->diagonal_gate != 0)
      .total;
}

size_t kla_prefill_backward_workspace_bytes(int32_t n_seq, int32_t total_tokens,
                                            int32_t n_heads, int32_t d_k, int32_t d_v,
                                            kla_dtype dtype) {
  return kla_prefill_backward_workspace_bytes_ex(n_seq, total_tokens, n_heads, d_k, d_v, dtype,
                                                 nullptr);
}

}  // extern "C"

namespace {

// Validation of the prefill arguments shared by the three prefill entry points.  Token
// buffers that a given entry point does not use are passed as nullptr with need_* = false.
kla_status check_prefill_args(const void *q, const void *k, const void *v, const float *g,
                              const float *eta, float eps, const float *S0, const void *o,
                              const float *S_T, const int32_t *cu_seqlens,
                              const int32_t *cu_seqlens_host, int32_t n_seq, int32_t total_tokens,
                              int32_t n_heads, int32_t d_k, int32_t d_v, kla_dtype dtype,
                              const void *workspace, size_t workspace_bytes, bool need_prep,
                              bool need_scan, bool check_tables = true, bool diag = false,
                              int segs = 0, bool split = false) {
  kla_status st = check_prefill_shape(cu_seqlens_host, n_seq, total_tokens, n_heads, d_k, d_v,
                                      dtype, eps);
  if (st != KLA_OK) return st;
  if (total_tokens > 0) {
    if (!k || (need_prep && (!g || !eta)) || (need_scan && (!q || !v || !o)))
      return fail(KLA_ERR_INVALID_ARGUMENT, "q, k, v, g, eta and o are required");
  }
  if (check_tables && (st = check_dense(cu_seqlens, n_seq, total_tokens)) != KLA_OK) return st;
  const size_t es = elem_size(dtype);
  // q, k, v are read and o is written with vector accesses; the rest element by element
  for (const void *p : {q, k, v, o})
    if (p && !aligned16(p)) return fail(KLA_ERR_INVALID_ARGUMENT, "q, k, v, o must be 16-byte aligned");
  for (const void *p : {static_cast<const void *>(g), static_cast<const void *>(eta),
                        static_cast<const void *>(S0), static_cast<const void *>(S_T)})
    if (p && !aligned_to(p, 4)) return fail(KLA_ERR_INVALID_ARGUMENT, "g, eta, S0, S_T must be 4-byte aligned");
  const size_t nq = (size_t)total_tokens * n_heads * d_k * es;
  const size_t nv = (size_t)total_tokens * n_heads * d_v * es;
  if (overlap(o, nv, q, nq) || overlap(o, nv, k, nq) || overlap(o, nv, v, nv))
    return fail(KLA_ERR_INVALID_ARGUMENT, "o must not overlap q, k or v");
  const size_t nS = (size_t)n_seq * n_heads * d_k * d_v * sizeof(float);
  if (S_T && S_T != S0 && overlap(S_T, nS, S0, nS))
    return fail(KLA_ERR_INVALID_ARGUMENT, "S_T may equal S0 but must not partially overlap it");
  const size_t need =
      ws_layout(n_seq, total_tokens, n_heads, d_k, es, diag, d_v, segs, split).total;
  if (!workspace || workspace_bytes < need)
    return fail(KLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(KLA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  return KLA_OK;
}

struct WsViews {
  kla::SeqTables tabs;
  float *G, *GD;
  void *T, *P;
  kla::DiagTiles diag;  // diagonal gating only
  float *NM, *Sin, *LC;  // two-level scan only
};

WsViews ws_views(void *workspace, int32_t n_seq, int32_t total_tokens, int32_t n_heads,
                 int32_t d_k, kla_dtype dtype, bool diag = false, int32_t d_v = 0,
                 int segs = 0, bool split = false) {
  const WsLayout w =
      ws_layout(n_seq, total_tokens, n_heads, d_k, elem_size(dtype), diag, d_v, segs, split);
  char *ws = static_cast<char *>(workspace);
  WsViews v{{reinterpret_cast<int32_t *>(ws + w.off_cu),
             reinterpret_cast<int32_t *>(ws + w.off_co)},
            reinterpret_cast<float *>(ws + w.off_G), reinterpret_cast<float *>(ws + w.off_GD),
            ws + w.off_T, ws + w.off_P, {nullptr, nullptr, nullptr, nullptr}, nullptr, nullptr,
            nullptr};
  if (segs >= 2) {
    v.NM = reinterpret_cast<float *>(ws + w.off_NM);
    v.Sin = reinterpret_cast<float *>(ws + w.off_Sin);
    v.LC = reinterpret_cast<float *>(ws + w.off_LC);
  }
  if (diag)
    v.diag = kla::DiagTiles{ws + w.off_KG, ws + w.off_QG, ws + w.off_KD,
                            reinterpret_cast<float *>(ws + w.off_GC)};
  return v;
}

// Diagonal gating: the plan kernel writes the sequence tables, then the per-chunk stage.
kla_status enqueue_prepare_diag(const void *q, const void *k, const float *g, const float *eta,
                                float eps, const kla::CoefOpts &opts, const int32_t *cu_seqlens,
                                int32_t n_seq, int32_t total_tokens, int32_t n_heads, int32_t d_k,
                                kla_dtype dtype, void *workspace, hipStream_t s,
                                void *X_out = nullptr, void *A_out = nullptr) {
  const WsViews wv = ws_views(workspace, n_seq, total_tokens, n_heads, d_k, dtype, true);
  const int64_t nch_ub = kla::chunk_upper_bound(n_seq, total_tokens);
  kla_status st =
      hip_status(kla::launch_plan(cu_seqlens, n_seq, total_tokens, wv.tabs, s), "plan");
  if (st != KLA_OK) return st;
  return hip_status(kla::launch_prep_diag(to_dt(dtype), d_k, q, k, g, eta, eps, opts, wv.tabs,
                                          n_seq, nch_ub, n_heads, wv.diag, wv.T, wv.P, wv.GD, s,
                                          X_out, A_out),
                    "prep (diagonal gate)");
}

kla_status enqueue_prepare(const void *q, const void *k, const float *g, const float *eta, float eps,
                           const kla::CoefOpts &opts, const int32_t *cu_seqlens, int32_t n_seq,
                           int32_t total_tokens, int32_t n_heads, int32_t d_k, kla_dtype dtype,
                           void *workspace, hipStream_t s, bool split = false,
                           void *X_out = nullptr, float *LC_out = nullptr) {
  const WsViews wv =
      ws_views(workspace, n_seq, total_tokens, n_heads, d_k, dtype, false, 0, 0, split);
  const int64_t nch_ub = kla::chunk_upper_bound(n_seq, total_tokens);
  kla::PlanArgs pa{kla::kPlanTables, cu_seqlens, total_tokens};
  if (!cu_seqlens)
    pa.mode = kla::kPlanDense;
  else if (n_seq <= kla::kPlanWaveMax)
    pa.mode = kla::kPlanWave;
  kla_status st;
  if (pa.mode == kla::kPlanTables &&
      (st = hip_status(kla::launch_plan(cu_seqlens, n_seq, total_tokens, wv.tabs, s), "plan")) !=
          KLA_OK)
    return st;
  return hip_status(kla::launch_prep(to_dt(dtype), d_k, q, k, g, eta, eps, opts, wv.tabs, n_seq,
                                     nch_ub, n_heads, nullptr, nullptr, wv.T, false, wv.P, wv.GD,
                                     pa, s, split, X_out, LC_out),
                    "prep");
}

kla_status enqueue_scan(const void *q, const void *k, const void *v, const float *S0, void *o,
                        float *S_T, int32_t n_seq, int32_t total_tokens, int32_t n_heads,
                        int32_t d_k, int32_t d_v, kla_dtype dtype, void *workspace, hipStream_t s,
                        bool diag = false) {
  const WsViews wv = ws_views(workspace, n_seq, total_tokens, n_heads, d_k, dtype, diag);
  return hip_status(kla::launch_scan(to_dt(dtype), d_k, d_v, q, k, v, wv.GD, wv.T, wv.P, S0, o,
                                     S_T, wv.tabs, n_seq, n_heads, s,
                                     diag ? &wv.diag : nullptr),
                    "scan");
}

}  // namespace

extern "C" {

kla_status kla_prefill_chunked_ex(const void *q, const void *k, const void *v, const float *g,
                                  const float *eta, float eps, const float *S0, void *o,
                                  float *S_T, const int32_t *cu_seqlens,
                                  const int32_t *cu_seqlens_host, int32_t n_seq,
                                  int32_t total_tokens, int32_t n_heads, int32_t d_k,
                                  int32_t d_v, kla_dtype dtype, void *workspace,
                                  size_t workspace_bytes, const kla_options *opts, void *stream) {
  kla::CoefOpts co;
  kla_status st = to_coef(opts, &co);
  if (st != KLA_OK) return st;
  const bool diag = co.diag_gate != 0;
  if (opts && opts->scan_segments < 0)
    return fail(KLA_ERR_INVALID_ARGUMENT, "scan_segments must be >= 0");
  // split precision matters for bf16 operands only (fp32 ones take exact products)
  const bool split = opts && opts->precision == KLA_PRECISION_SPLIT && dtype == KLA_DTYPE_BF16;
  if (split && diag)
    return fail(KLA_ERR_UNSUPPORTED, "split precision takes the scalar gate only");
  // the workspace is sized for the shape's segmentation whatever cu_seqlens is; the
  // two-level scan itself runs on dense input only
  const SegPlan sp = seg_plan(n_seq, total_tokens, n_heads, d_v, diag,
                              opts ? opts->scan_segments : 0, split);
  if ((st = check_prefill_args(q, k, v, g, eta, eps, S0, o, S_T, cu_seqlens, cu_seqlens_host,
                               n_seq, total_tokens, n_heads, d_k, d_v, dtype, workspace,
                               workspace_bytes, true, true, true, diag, sp.G, split)) != KLA_OK)
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear any stale error from unrelated work
  const bool two_level = !split && sp.G >= 2 && !cu_seqlens && total_tokens > 0;
  if (diag)
    st = enqueue_prepare_diag(q, k, g, eta, eps, co, cu_seqlens, n_seq, total_tokens, n_heads,
                              d_k, dtype, workspace, s);
  else
    st = enqueue_prepare(
        q, k, g, eta, eps, co, cu_seqlens, n_seq, total_tokens, n_heads, d_k, dtype, workspace,
        s, split, nullptr,
        two_level ? ws_views(workspace, n_seq, total_tokens, n_heads, d_k, dtype, false, d_v,
                             sp.G).LC
                  : nullptr);
  if (st != KLA_OK) return st;
  if (split) {
    const WsViews wv =
        ws_views(workspace, n_seq, total_tokens, n_heads, d_k, dtype, false, 0, 0, true);
    st = hip_status(kla::launch_scan_split(d_k, d_v, q, k, v, wv.GD, wv.T, wv.P, S0, o, S_T,
                                           wv.tabs, n_seq, n_heads, s),
                    "scan (split precision)");
  } else if (two_level) {
    const WsViews wv =
        ws_views(workspace, n_seq, total_tokens, n_heads, d_k, dtype, false, d_v, sp.G);
    kla::SegArgs sa;
    sa.G = sp.G;
    sa.L = total_tokens / n_seq;
    sa.Ls = sp.Ls;
    sa.dv = d_v;
    sa.LC = wv.LC;
    sa.W = kWarmChunks;
    st = hip_status(kla::launch_scan_two_level(to_dt(dtype), d_k, d_v, q, k, v, wv.GD, wv.T, wv.P,
                                               S0, o, S_T, n_seq, n_heads, sa, wv.NM, wv.Sin, s),
                    "two-level scan");
  } else {
    st = enqueue_scan(q, k, v, S0, o, S_T, n_seq, total_tokens, n_heads, d_k, d_v, dtype,
                      workspace, s, diag);
  }
  if (st != KLA_OK) return st;
  return ok();
}

kla_status kla_prefill_chunked(const void *q, const void *k, const void *v, const float *g,
                               const float *eta, float eps, const float *S0, void *o,
                               float *S_T, const int32_t *cu_seqlens,
                               const int32_t *cu_seqlens_host, int32_t n_seq,
                               int32_t total_tokens, int32_t n_heads, int32_t d_k,
                               int32_t d_v, kla_dtype dtype, void *workspace,
                               size_t workspace_bytes, void *stream) {
  return kla_prefill_chunked_ex(q, k, v, g, eta, eps, S0, o, S_T, cu_seqlens, cu_seqlens_host,
                                n_seq, total_tokens, n_heads, d_k, d_v, dtype, workspace,
                                workspace_bytes, nullptr, stream);
}

}  // extern "C"

namespace {

// Scratch of the allocation-free prefill: one array per device, held until the process ends.
// Host code never uses the name itself as an address (on the host it is a stand-in, not the
// device array): scratch_ptr() looks the device address up once per device, with that device
// current, and every launch takes that pointer.
static __device__ __align__(256) unsigned char scratch[KLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

kla_status scratch_ptr(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(KLA_ERR_UNSUPPORTED, "device ordinal %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KLA_OK;
}

}  // namespace

extern "C" {

kla_status kla_prefill_chunked_noalloc(const void *q, const void *k, const void *v,
                                       const float *g, const float *eta, float eps,
                                       const float *S0, void *o, float *S_T,
                                       const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                       int32_t n_seq, int32_t total_tokens, int32_t n_heads,
                                       int32_t d_k, int32_t d_v, kla_dtype dtype,
                                       const kla_options *opts, void *stream) {
  const size_t need =
      kla_prefill_workspace_bytes_ex(n_seq, total_tokens, n_heads, d_k, d_v, dtype, opts);
  if (need > (size_t)KLA_NOALLOC_SCRATCH_BYTES)
    return fail(KLA_ERR_WORKSPACE,
                "this prefill needs %zu bytes of scratch, more than the %zu-byte static "
                "scratch of kla_prefill_chunked_noalloc; use kla_prefill_chunked_ex with a "
                "workspace",
                need, (size_t)KLA_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  kla_status st = scratch_ptr(&ws);
  if (st != KLA_OK) return st;
  // (an unsupported size gives need == 0 and is reported by the shared checks below)
  return kla_prefill_chunked_ex(q, k, v, g, eta, eps, S0, o, S_T, cu_seqlens, cu_seqlens_host,
                                n_seq, total_tokens, n_heads, d_k, d_v, dtype, ws,
                                (size_t)KLA_NOALLOC_SCRATCH_BYTES, opts, stream);
}

kla_status kla_prefill_backward_ex(const void *q, const void *k, const void *v, const float *g,
                                   const float *eta, float eps, const float *S0, const void *dO,
                                   const float *dS_T, void *dq, void *dk, void *dv, float *dg,
                                   float *deta, float *dS0, const int32_t *cu_seqlens,
                                   const int32_t *cu_seqlens_host, int32_t n_seq,
                                   int32_t total_tokens, int32_t n_heads, int32_t d_k,
                                   int32_t d_v, kla_dtype dtype, void *workspace,
                                   size_t workspace_bytes, const kla_options *opts, void *stream) {
  kla::CoefOpts co;
  kla_status st = to_coef(opts, &co);
  if (st != KLA_OK) return st;
  const bool diag = co.diag_gate != 0;
  if (opts && opts->precision != KLA_PRECISION_BF16)
    return fail(KLA_ERR_UNSUPPORTED, "the backward pass takes the bf16 operand precision only");
  if ((st = check_prefill_shape(cu_seqlens_host, n_seq, total_tokens, n_heads, d_k, d_v, dtype,
                                eps)) != KLA_OK)
    return st;
  if (total_tokens > 0 && (!q || !k || !v || !g || !eta || !dO || !dq || !dk || !dv || !dg || !deta))
    return fail(KLA_ERR_INVALID_ARGUMENT,
                "q, k, v, g, eta, dO, dq, dk, dv, dg and deta are required");
  if ((st = check_dense(cu_seqlens, n_seq, total_tokens)) != KLA_OK) return st;
  for (const void *p : {q, k, v, dO, static_cast<const void *>(dq),
                        static_cast<const void *>(dk), static_cast<const void *>(dv)})
    if (p && !aligned16(p))
      return fail(KLA_ERR_INVALID_ARGUMENT, "q, k, v, dO, dq, dk, dv must be 16-byte aligned");
  for (const void *p : {static_cast<const void *>(g), static_cast<const void *>(eta),
                        static_cast<const void *>(S0), static_cast<const void *>(dS_T),
                        static_cast<const void *>(dg), static_cast<const void *>(deta),
                        static_cast<const void *>(dS0)})
    if (p && !aligned_to(p, 4))
      return fail(KLA_ERR_INVALID_ARGUMENT,
                  "g, eta, S0, dS_T, dg, deta, dS0 must be 4-byte aligned");
  const size_t es = elem_size(dtype);
  const size_t nq = (size_t)total_tokens * n_heads * d_k * es;
  const size_t nv = (size_t)total_tokens * n_heads * d_v * es;
  const size_t ns = (size_t)total_tokens * n_heads * sizeof(float);
  const size_t ng = ns * (diag ? (size_t)d_k : 1);  // g and dg: per key channel under diag
  const size_t nS = (size_t)n_seq * n_heads * d_k * d_v * sizeof(float);
  const void *outs[] = {dq, dk, dv, dg, deta, dS0};
  const size_t nouts[] = {nq, nq, nv, ng, ns, nS};
  const void *ins[] = {q, k, v, g, eta, S0, dO, dS_T};
  const size_t nins[] = {nq, nq, nv, ng, ns, nS, nv, nS};
  for (int i = 0; i < 6; ++i) {
    for (int j = 0; j < 8; ++j)
      if (overlap(outs[i], nouts[i], ins[j], nins[j]))
        return fail(KLA_ERR_INVALID_ARGUMENT, "gradient buffers must not overlap the inputs");
    for (int j = i + 1; j < 6; ++j)
      if (overlap(outs[i], nouts[i], outs[j], nouts[j]))
        return fail(KLA_ERR_INVALID_ARGUMENT, "gradient buffers must not overlap each other");
  }
  const BwdLayout bl = bwd_layout(n_seq, total_tokens, n_heads, d_k, d_v, es, diag);
  if (!workspace || workspace_bytes < bl.total)
    return fail(KLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", bl.total,
                workspace ? workspace_bytes : (size_t)0);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(KLA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  for (int i = 0; i < 6; ++i)
    if (overlap(outs[i], nouts[i], workspace, bl.total))
      return fail(KLA_ERR_INVALID_ARGUMENT, "gradient buffers must not overlap the workspace");

  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear any stale error from unrelated work
  char *ws = static_cast<char *>(workspace);
  void *Xbuf = ws + bl.off_X;
  void *Abuf = diag ? ws + bl.off_A : nullptr;
  if (diag)
    st = enqueue_prepare_diag(q, k, g, eta, eps, co, cu_seqlens, n_seq, total_tokens, n_heads,
                              d_k, dtype, workspace, s, Xbuf, Abuf);
  else
    st = enqueue_prepare(q, k, g, eta, eps, co, cu_seqlens, n_seq, total_tokens, n_heads, d_k,
                         dtype, workspace, s, false, Xbuf);
  if (st != KLA_OK) return st;
  const WsViews wv = ws_views(workspace, n_seq, total_tokens, n_heads, d_k, dtype, diag);
  void *SN = ws + bl.off_SN;  // incoming states in the operand type
  if ((st = hip_status(kla::launch_scan(to_dt(dtype), d_k, d_v, nullptr, k, v, wv.GD, wv.T,
                                        nullptr, S0, nullptr, nullptr, wv.tabs, n_seq, n_heads,
                                        s, diag ? &wv.diag : nullptr, SN),
                       "scan (stored states)")) != KLA_OK)
    return st;
  if ((st = hip_status(
           kla::launch_bwd(to_dt(dtype), d_k, d_v, q, k, v, dO, g, eta, eps, co, wv.GD, wv.T, wv.P,
                           Xbuf, dS_T, SN, ws + bl.off_dSo, ws + bl.off_dU, dq,
                           dk, dv, dg, deta, dS0,
                           wv.tabs, n_seq, kla::chunk_upper_bound(n_seq, total_tokens), n_heads,
                           s, diag ? &wv.diag : nullptr, Abuf),
           "backward")) != KLA_OK)
    return st;
  return ok();
}

kla_status kla_prefill_backward(const void *q, const void *k, const void *v, const float *g,
                                const float *eta, float eps, const float *S0, const void *dO,
                                const float *dS_T, void *dq, void *dk, void *dv, float *dg,
                                float *deta, float *dS0, const int32_t *cu_seqlens,
                                const int32_t *cu_seqlens_host, int32_t n_seq,
                                int32_t total_tokens, int32_t n_heads, int32_t d_k, int32_t d_v,
                                kla_dtype dtype, void *workspace, size_t workspace_bytes,
                                void *stream) {
  return kla_prefill_backward_ex(q, k, v, g, eta, eps, S0, dO, dS_T, dq, dk, dv, dg, deta, dS0,
                                 cu_seqlens, cu_seqlens_host, n_seq, total_tokens, n_heads, d_k,
                                 d_v, dtype, workspace, workspace_bytes, nullptr, stream);
}

kla_status kla_prefill_prepare_ex(const void *q, const void *k, const float *g,
                                  const float *eta, float eps, const int32_t *cu_seqlens,
                                  const int32_t *cu_seqlens_host, int32_t n_seq,
                                  int32_t total_tokens, int32_t n_heads, int32_t d_k, int32_t d_v,
                                  kla_dtype dtype, void *workspace, size_t workspace_bytes,
                                  const kla_options *opts, void *stream) {
  kla_status st = check_prefill_args(q, k, nullptr, g, eta, eps, nullptr, nullptr, nullptr,
                                     cu_seqlens, cu_seqlens_host, n_seq, total_tokens, n_heads,
                                     d_k, d_v, dtype, workspace, workspace_bytes, true, false);
  if (st != KLA_OK) return st;
  if (total_tokens > 0 && !q)
    return fail(KLA_ERR_INVALID_ARGUMENT, "q, k, g and eta are required");
  kla::CoefOpts co;
  if ((st = to_coef(opts, &co)) != KLA_OK) return st;
  if (co.diag_gate)
    return fail(KLA_ERR_UNSUPPORTED,
                "a diagonal-gated prefill runs through kla_prefill_chunked_ex only");
  if (opts && opts->precision != KLA_PRECISION_BF16)
    return fail(KLA_ERR_UNSUPPORTED,
                "a split-precision prefill runs through kla_prefill_chunked_ex only");
  (void)hipGetLastError();
  if ((st = enqueue_prepare(q, k, g, eta, eps, co, cu_seqlens, n_seq, total_tokens, n_heads, d_k,
                            dtype, workspace, static_cast<hipStream_t>(stream))) != KLA_OK)
    return st;
  return ok();
}

kla_status kla_prefill_prepare(const void *q, const void *k, const float *g, const float *eta,
                               float eps, const int32_t *cu_seqlens,
                               const int32_t *cu_seqlens_host, int32_t n_seq, int32_t total_tokens,
                               int32_t n_heads, int32_t d_k, int32_t d_v, kla_dtype dtype,
                               void *workspace, size_t workspace_bytes, void *stream) {
  return kla_prefill_prepare_ex(q, k, g, eta, eps, cu_seqlens, cu_seqlens_host, n_seq,
                                total_tokens, n_heads, d_k, d_v, dtype, workspace,
                                workspace_bytes, nullptr, stream);
}

kla_status kla_prefill_scan(const void *q, const void *k, const void *v, const float *S0, void *o,
                            float *S_T, int32_t n_seq, int32_t total_tokens, int32_t n_heads,
                            int32_t d_k, int32_t d_v, kla_dtype dtype, const void *workspace,
                            size_t workspace_bytes, void *stream) {
  // eps only matters to the prepare stage (pass a valid value through the shared checks);
  // the sequence tables come from the workspace the prepare call filled
  kla_status st = check_prefill_args(q, k, v, nullptr, nullptr, 0.f, S0, o, S_T, nullptr, nullptr,
                                     n_seq, total_tokens, n_heads, d_k, d_v, dtype, workspace,
                                     workspace_bytes, false, true, false);
  if (st != KLA_OK) return st;
  (void)hipGetLastError();
  if ((st = enqueue_scan(q, k, v, S0, o, S_T, n_seq, total_tokens, n_heads, d_k, d_v, dtype,
                         const_cast<void *>(workspace), static_cast<hipStream_t>(stream))) != KLA_OK)
    return st;
  return ok();
}

kla_status kla_prefill_chunk_stage(const void *k, const void *v, const float *g,
                                   const float *eta, float eps, float *beta, float *G,
                                   float *T, float *W, float *Ut, const int32_t *cu_seqlens,
                                   const int32_t *cu_seqlens_host, int32_t n_seq,
                                   int32_t total_tokens, int32_t n_heads, int32_t d_k,
                                   int32_t d_v, kla_dtype dtype, void *workspace,
                                   size_t workspace_bytes, void *stream) {
  kla_status st = check_prefill_shape(cu_seqlens_host, n_seq, total_tokens, n_heads, d_k, d_v,
                                      dtype, eps);
  if (st != KLA_OK) return st;
  if (total_tokens > 0 && (!k || !g || !eta || !T || (Ut && !v)))
    return fail(KLA_ERR_INVALID_ARGUMENT, "k, g, eta, T (and v when Ut is requested) are required");
  if ((st = check_dense(cu_seqlens, n_seq, total_tokens)) != KLA_OK) return st;
  for (const void *p : {k, v})
    if (p && !aligned16(p)) return fail(KLA_ERR_INVALID_ARGUMENT, "k, v must be 16-byte aligned");
  for (const void *p : {static_cast<const void *>(g), static_cast<const void *>(eta),
                        static_cast<const void *>(beta), static_cast<const void *>(G),
                        static_cast<const void *>(T), static_cast<const void *>(W),
                        static_cast<const void *>(Ut)})
    if (p && !aligned_to(p, 4)) return fail(KLA_ERR_INVALID_ARGUMENT, "fp32 buffers must be 4-byte aligned");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(KLA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  const WsLayout w = ws_layout(n_seq, total_tokens, n_heads, d_k, elem_size(dtype));
  // this entry point writes G into the caller's buffer when given, else into the workspace
  if (!workspace || workspace_bytes < w.total)
    return fail(KLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.total,
                workspace ? workspace_bytes : (size_t)0);
  char *ws = static_cast<char *>(workspace);
  kla::SeqTables tabs{reinterpret_cast<int32_t *>(ws + w.off_cu),
                      reinterpret_cast<int32_t *>(ws + w.off_co)};
  float *Gbuf = G ? G : reinterpret_cast<float *>(ws + w.off_G);
  const int64_t nch_ub = kla::chunk_upper_bound(n_seq, total_tokens);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const kla::Dtype dt = to_dt(dtype);
  if ((st = hip_status(kla::launch_plan(cu_seqlens, n_seq, total_tokens, tabs, s), "plan")) != KLA_OK)
    return st;
  const kla::CoefOpts co{kla::kBetaKaczmarz, 0, nullptr};
  if ((st = hip_status(kla::launch_prep(dt, d_k, nullptr, k, g, eta, eps, co, tabs, n_seq, nch_ub,
                                        n_heads, Gbuf, beta, T, true, nullptr, nullptr,
                                        kla::PlanArgs{kla::kPlanTables, nullptr, total_tokens}, s),
                       "prep")) != KLA_OK)
    return st;
  if ((st = hip_status(kla::launch_wy(dt, d_k, d_v, k, v, Gbuf, T, tabs, n_seq, nch_ub, n_heads,
                                      W, Ut, s), "wy")) != KLA_OK)
    return st;
  return ok();
}

kla_status kla_decode_step(const void *q, const void *k, const void *v, const float *g,
                           const float *eta, float eps, const float *S, void *o,
                           float *S_new, int32_t batch, int32_t n_heads, int32_t d_k,
                           int32_t d_v, kla_dtype dtype, void *stream) {
  return kla_decode_step_ex(q, k, v, g, eta, eps, S, o, S_new, batch, n_heads, d_k, d_v, dtype,
                            nullptr, stream);
}

kla_status kla_decode_step_ex(const void *q, const void *k, const void *v, const float *g,
                              const float *eta, float eps, const float *S, void *o,
                              float *S_new, int32_t batch, int32_t n_heads, int32_t d_k,
                              int32_t d_v, kla_dtype dtype, const kla_options *opts,
                              void *stream) {
  if (dtype != KLA_DTYPE_F32 && dtype != KLA_DTYPE_BF16)
    return fail(KLA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (batch < 0 || n_heads <= 0)
    return fail(KLA_ERR_INVALID_ARGUMENT, "need batch >= 0 and n_heads > 0");
  if (!supported_dk(d_k)) return fail(KLA_ERR_UNSUPPORTED, "d_k = %d not in {64, 128}", d_k);
  if (!supported_dv(d_v)) return fail(KLA_ERR_UNSUPPORTED, "d_v = %d not in {64, 128, 256}", d_v);
  if (!(eps >= 0.f) || !isfinite(eps))
    return fail(KLA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if ((int64_t)batch * n_heads > 0x7fffffff)
    return fail(KLA_ERR_INVALID_ARGUMENT, "batch * n_heads too large");
  if (!q || !k || !v || !g || !eta || !S || !o || !S_new)
    return fail(KLA_ERR_INVALID_ARGUMENT, "q, k, v, g, eta, S, o and S_new are required");
  // the state streams as float4; the token vectors are read element by element
  if (!aligned16(S) || !aligned16(S_new))
    return fail(KLA_ERR_INVALID_ARGUMENT, "S and S_new must be 16-byte aligned");
  const size_t es = elem_size(dtype);
  for (const void *p : {q, k, v, static_cast<const void *>(o)})
    if (!aligned_to(p, es)) return fail(KLA_ERR_INVALID_ARGUMENT, "q, k, v, o must be element aligned");
  if (!aligned_to(g, 4) || !aligned_to(eta, 4))
    return fail(KLA_ERR_INVALID_ARGUMENT, "g and eta must be 4-byte aligned");
  const size_t nS = (size_t)batch * n_heads * d_k * d_v * sizeof(float);
  if (S_new != S && overlap(S_new, nS, S, nS))
    return fail(KLA_ERR_INVALID_ARGUMENT, "S_new may equal S but must not partially overlap it");
  kla::CoefOpts co;
  kla_status st = to_coef(opts, &co);
  if (st != KLA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  st = hip_status(kla::launch_decode(to_dt(dtype), d_k, d_v, q, k, v, g, eta, eps, co, S, o, S_new,
                                     batch, n_heads, s), "decode");
  if (st != KLA_OK) return st;
  return ok();
}

const char *kla_status_string(kla_status status) {
  switch (status) {
    case KLA_OK: return "KLA_OK";
    case KLA_ERR_INVALID_ARGUMENT: return "KLA_ERR_INVALID_ARGUMENT: invalid argument";
    case KLA_ERR_UNSUPPORTED: return "KLA_ERR_UNSUPPORTED: unsupported size or dtype";
    case KLA_ERR_WORKSPACE: return "KLA_ERR_WORKSPACE: workspace missing or too small";
    case KLA_ERR_HIP: return "KLA_ERR_HIP: HIP launch failed";
    default: break;
  }
  return "unknown kla_status";
}

const char *kla_last_error(void) { return g_last_error; }

int32_t kla_version(void) { return 30100; }

}  // extern "C"
