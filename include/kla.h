/*
 * kla.h -- C ABI of the MI355X (gfx950) Kaczmarz Linear Attention forward pass.
 *
 * The operation (paper "Kaczmarz Linear Attention", arXiv 2605.08587) is the
 * gated delta-rule recurrence that first forgets and then projects, per
 * (sequence, head), in the row-vector convention (state S is d_k x d_v, keys
 * and queries are 1 x d_k rows, values 1 x d_v rows):
 *
 *   a_t = exp(g_t)                                 (g_t is a log-decay, <= 0)
 *   b_t = eta_t / (||k_t||^2 + eps)                Eq. (3); b_t = 0 if the
 *                                                  denominator is exactly 0
 *   S_t = a_t S_{t-1} + b_t k_t^T (v_t - a_t k_t S_{t-1})
 *                                                  Algorithm 1, tokenwise panel
 *   o_t = q_t S_t                                  readout on the q passed in
 *                                                  (the 1/||q_t|| of section 3.3
 *                                                  is left to the caller)
 *
 * kla_prefill_chunked evaluates it with the chunkwise solve of section 4
 * (Proposition 3, Eq. (7); Proposition 4, Eq. (8)-(9)) in chunks of
 * KLA_CHUNK tokens; kla_decode_step applies one tokenwise step.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or retains them.  Tensors are dense, row-major,
 *     with the last named dimension fastest.  Alignment: the prefill's q, k, v, o
 *     and the decode's S, S_new need 16-byte aligned bases (vector accesses); every
 *     other buffer needs its element alignment; the workspace 256 bytes.
 *   - q, k, v, o use the element type `dtype` (fp32 or bf16); g, eta, S0, S_T,
 *     S and S_new are always fp32.  Accumulation and the state are fp32.
 *   - Calls are asynchronous: they validate, enqueue kernels on `stream` (a
 *     hipStream_t; NULL = the legacy default stream) and return.  Buffers must
 *     stay alive until the stream has passed the call.
 *   - On any non-OK status nothing has been enqueued (except KLA_ERR_HIP, which
 *     reports a failed launch).  kla_last_error() gives a human-readable
 *     reason for the last failure on the calling thread.
 *   - Preconditions that are documented but not checked (checking would cost a
 *     pass over the data): g finite and <= 0, eta finite (normally in (0, 1]),
 *     no NaN/Inf in q, k, v, S0 (NaN propagates).
 *   - The library is stateless and thread-safe; concurrent calls on different
 *     streams are independent provided their buffers do not overlap
 *     (kla_prefill_chunked_noalloc aside: its scratch is one static array per GPU).
 *   - A call enqueues kernels only (no allocation, memset, copy or host
 *     synchronisation), so it may be captured into a HIP graph on `stream` and
 *     replayed; the captured pointers, sizes and scalars are fixed, and the
 *     buffers behind them must stay alive while the graph is in use.
 */
#ifndef KLA_H_
#define KLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Tokens per chunk of the chunkwise solve (fixed). */
#define KLA_CHUNK 64

typedef enum kla_status {
  KLA_OK = 0,
  KLA_ERR_INVALID_ARGUMENT = 1, /* NULL required pointer, bad size, eps < 0 or
                                   non-finite, misaligned base, bad cu_seqlens */
  KLA_ERR_UNSUPPORTED = 2,      /* d_k not in {64, 128}, d_v not in {64, 128, 256},
                                   or an unknown dtype */
  KLA_ERR_WORKSPACE = 3,        /* workspace NULL or smaller than required */
  KLA_ERR_HIP = 4,              /* a kernel launch failed */
  /* not a status: makes every int32 value a valid kla_status, so that a caller's
   * unknown value is an ordinary input (kla_status_string says "unknown status") */
  KLA_STATUS_RANGE_ = 0x7fffffff
} kla_status;

typedef enum kla_dtype {
  KLA_DTYPE_F32 = 0,  /* IEEE fp32 */
  KLA_DTYPE_BF16 = 1, /* bfloat16; outputs rounded to nearest even */
  /* not a dtype: makes every int32 value a valid kla_dtype, so that an unknown one is
   * an ordinary input rejected with KLA_ERR_UNSUPPORTED (or a workspace size of 0) */
  KLA_DTYPE_RANGE_ = 0x7fffffff
} kla_dtype;

/* Bytes of device workspace kla_prefill_chunked needs for this problem size and
 * element type (an upper bound valid for any cu_seqlens with these totals).  Per
 * 64-token chunk and head it holds the chunk's T and P (Eq. (7)-(8)) as their ten
 * 16 x 16 blocks on and below the diagonal in the element type, and 768 bytes of
 * decay factors; for dense input of few long sequences, also the scratch of the
 * two-level scan (kla_options.scan_segments).  Returns 0 for an unsupported or
 * invalid size or dtype. */
size_t kla_prefill_workspace_bytes(int32_t n_seq, int32_t total_tokens, int32_t n_heads,
                                   int32_t d_k, int32_t d_v, kla_dtype dtype);

/*
 * Chunkwise prefill: (q, k, v, g, eta, eps, S0) -> (o, S_T).
 * Paper section 4, Algorithm 1 chunkwise panel, Eq. (7)-(9); chunks of
 * KLA_CHUNK tokens restart at every sequence start, the last chunk of a
 * sequence may be short, and the outgoing state of one chunk is the incoming
 * state of the next.
 *
 *   q, k        [total_tokens, n_heads, d_k]   dtype
 *   v           [total_tokens, n_heads, d_v]   dtype
 *   g, eta      [total_tokens, n_heads]        fp32  (log-decay, relaxation)
 *   eps         >= 0 and finite (the pages use 1e-6)
 *   S0          [n_seq, n_heads, d_k, d_v] fp32, or NULL for all-zero states
 *   o           [total_tokens, n_heads, d_v]   dtype (written)
 *   S_T         [n_seq, n_heads, d_k, d_v] fp32, or NULL (not stored);
 *               may be the same pointer as S0 (in-place state update)
 *   cu_seqlens  device int32 [n_seq + 1] token offsets of packed sequences
 *               (cu_seqlens[0] = 0, non-decreasing, cu_seqlens[n_seq] =
 *               total_tokens), or NULL for dense input where every sequence
 *               has total_tokens / n_seq tokens (must divide evenly).
 *               Device offsets are not validated; out-of-range values are
 *               clamped into [0, total_tokens] and made non-decreasing, so a
 *               bad table gives wrong results but no out-of-bounds access.
 *   cu_seqlens_host  optional host copy of cu_seqlens (NULL allowed); when
 *               given it is validated and a bad table is rejected.
 *   workspace   device buffer of at least kla_prefill_workspace_bytes(...)
 *               bytes, 256-byte aligned; contents are scratch.
 * Zero-length sequences are allowed (their S_T is S0, or zeros).  When
 * total_tokens is 0 the token buffers q, k, v, g, eta and o may be NULL.
 * q, k, v, g, eta and o must not overlap each other or the workspace.
 * Sizes: d_k in {64, 128}, d_v in {64, 128, 256}; one chunk of a token tensor,
 * 64 * n_heads * max(d_k, d_v) * element size, must be below 2^31 bytes
 * (KLA_ERR_UNSUPPORTED otherwise).
 */
kla_status kla_prefill_chunked(const void *q, const void *k, const void *v, const float *g,
                               const float *eta, float eps, const float *S0, void *o,
                               float *S_T, const int32_t *cu_seqlens,
                               const int32_t *cu_seqlens_host, int32_t n_seq,
                               int32_t total_tokens, int32_t n_heads, int32_t d_k,
                               int32_t d_v, kla_dtype dtype, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * The two halves of kla_prefill_chunked, for callers that schedule them apart
 * (and for timing each kernel).  kla_prefill_chunked(...) is exactly
 * kla_prefill_prepare(...) followed by kla_prefill_scan(...) on one stream.
 *
 * kla_prefill_prepare: per-chunk stage (paper section 4, Algorithm 1 chunkwise
 *   panel up to the triangular solve): sequence tables, the chunk-local
 *   decays exp(G_i) and exp(G_last - G_i), T = (I + L)^{-1} Diag(b) and the
 *   intra-chunk matrix P = A o Q K^T of Eq. (8) for every chunk, written into
 *   `workspace`.
 *   Arguments as for kla_prefill_chunked.
 * kla_prefill_scan: the sequential chunk scan with the outputs (Eq. (7)-(9)),
 *   reading the workspace a kla_prefill_prepare call with the same q, k, g, eta,
 *   cu_seqlens and sizes filled earlier on the same stream (not checkable: a
 *   workspace from another problem gives wrong results, never out-of-bounds
 *   access as long as the sizes match).  q, k, v, S0, o, S_T as for
 *   kla_prefill_chunked.
 */
kla_status kla_prefill_prepare(const void *q, const void *k, const float *g, const float *eta,
                               float eps, const int32_t *cu_seqlens,
                               const int32_t *cu_seqlens_host, int32_t n_seq, int32_t total_tokens,
                               int32_t n_heads, int32_t d_k, int32_t d_v, kla_dtype dtype,
                               void *workspace, size_t workspace_bytes, void *stream);

kla_status kla_prefill_scan(const void *q, const void *k, const void *v, const float *S0, void *o,
                            float *S_T, int32_t n_seq, int32_t total_tokens, int32_t n_heads,
                            int32_t d_k, int32_t d_v, kla_dtype dtype, const void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * One decode step per sequence: (q, k, v, g, eta, eps, S) -> (o, S').
 * Paper Algorithm 1 tokenwise panel (with Eq. (3)), evaluated with
 * a single read and a single write of S:  r = k S, p = q S,
 * e = v - a r, S' = a S + b k^T e, o = a p + b (q . k) e.
 *
 *   q, k     [batch, n_heads, d_k]  dtype      v, o  [batch, n_heads, d_v]  dtype
 *   g, eta   [batch, n_heads]       fp32       eps   >= 0 and finite
 *   S        [batch, n_heads, d_k, d_v] fp32 (read)
 *   S_new    [batch, n_heads, d_k, d_v] fp32 (written); may equal S
 */
kla_status kla_decode_step(const void *q, const void *k, const void *v, const float *g,
                           const float *eta, float eps, const float *S, void *o,
                           float *S_new, int32_t batch, int32_t n_heads, int32_t d_k,
                           int32_t d_v, kla_dtype dtype, void *stream);

/*
 * Per-chunk stage only (unit checks of the prefill's first kernel): the
 * Kaczmarz step b and chunk-local inclusive log-decay G of every token, and
 * per chunk T = (I + L)^{-1} Diag(b) with L = Diag(b)(A^- o K K^T) strictly
 * lower triangular (Proposition 3 / Appendix B.2), so that the chunk's
 * U = T (V - Diag(exp G) K S0).  Optionally also the WY factors
 * W = T Diag(exp G) K and U~ = T V (then U = U~ - W S0).
 *
 *   beta, G  [total_tokens, n_heads] fp32 (written; either may be NULL)
 *   T        [n_chunks, n_heads, KLA_CHUNK, KLA_CHUNK] fp32 (written), chunks
 *            numbered sequence by sequence; n_chunks = sum_n ceil(T_n / 64).
 *            Rows/columns past a short chunk's end are zero.
 *   W        [total_tokens, n_heads, d_k] fp32 or NULL
 *   Ut       [total_tokens, n_heads, d_v] fp32 or NULL
 * Other arguments as for kla_prefill_chunked (v may be NULL if Ut is NULL).
 */
kla_status kla_prefill_chunk_stage(const void *k, const void *v, const float *g,
                                   const float *eta, float eps, float *beta, float *G,
                                   float *T, float *W, float *Ut, const int32_t *cu_seqlens,
                                   const int32_t *cu_seqlens_host, int32_t n_seq,
                                   int32_t total_tokens, int32_t n_heads, int32_t d_k,
                                   int32_t d_v, kla_dtype dtype, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * Variants of the write coefficient and of the readout (the coverage of the
 * pages' ablations; the default is the method itself):
 *   KLA_BETA_KACZMARZ     b_t = eta_t / (||k_t||^2 + eps)      section 3.1, Eq. (3)
 *   KLA_BETA_GATED        b_t = eta_t, the gated delta rule's learned coefficient
 *                         (section 2; Table 5's "without normalization")
 *   KLA_BETA_KEY_NORM     b_t = 1 / (||k_t||^2 + eps)          Table 5, key-norm only
 *   KLA_BETA_INV_T        Kaczmarz coefficient x 1 / t          Appendix D,
 *   KLA_BETA_INV_SQRT_T   Kaczmarz coefficient x 1 / sqrt(t)    sequence factors, with t
 *   KLA_BETA_INV_LOG_T    Kaczmarz coefficient x 1 / log(t + 1) the absolute 1-based position
 * Wherever b_t divides by ||k_t||^2 + eps, a zero denominator gives b_t = 0.
 * normalize_q != 0 gives the readout o_t = q_t S_t / ||q_t||_2 of section 3.3 and
 * Algorithm 1's readout (o_t = 0 for a zero query); 0 gives o_t = q_t S_t.
 * pos_offset (device int32, [n_seq] for prefill, [batch] for decode, or NULL for
 * all zeros) places a call's tokens in their sequences: the first token of
 * sequence n in a prefill call is at position pos_offset[n] + 1, a decode step
 * of batch row b is at position pos_offset[b] + 1.  Only the sequence-factor
 * modes read it.  diagonal_gate != 0 selects diagonal gating (paper Appendix
 * B.5, "Extension to diagonal gating"): the decay is Diag(alpha_t) with one
 * log-decay per key channel, so g holds d_k values per token-head, laid out
 * like k ([n_tok, n_heads, d_k] for prefill, [batch, n_heads, d_k] for decode),
 * and the forget step scales row i of the state by exp(g_t[i]); the coefficient
 * b_t is unchanged.  A diagonal-gated prefill needs a larger workspace
 * (kla_prefill_workspace_bytes_ex) and runs through kla_prefill_chunked_ex only
 * (kla_prefill_prepare_ex returns KLA_ERR_UNSUPPORTED for it).  A NULL
 * kla_options pointer means the defaults (Kaczmarz coefficient, o_t = q_t S_t,
 * scalar gate).  An unknown mode gives KLA_ERR_UNSUPPORTED.
 */
typedef enum kla_beta_mode {
  KLA_BETA_KACZMARZ = 0,
  KLA_BETA_GATED = 1,
  KLA_BETA_KEY_NORM = 2,
  KLA_BETA_INV_T = 3,
  KLA_BETA_INV_SQRT_T = 4,
  KLA_BETA_INV_LOG_T = 5
} kla_beta_mode;

/* Operand precision of the bf16 prefill's matrix-core products (fp32 state and
 * accumulation either way; fp32 inputs always take exact fp32 products).
 *   KLA_PRECISION_BF16   S, the residual R = V - Diag(gamma) K S, U = T R,
 *                        Diag(dec) U, T and P enter their products rounded to
 *                        bf16 (relative error 2^-9 each).
 *   KLA_PRECISION_SPLIT  T R, P U and K^T Diag(dec) U take R, U, Diag(dec) U, T
 *                        and P as pairs hi = bf16(x), lo = bf16(x - hi) and sum
 *                        hi*hi + hi*lo + lo*hi (K is exact in bf16); T and P are
 *                        stored as such pairs (twice their workspace).  It holds
 *                        o = v of the hard projection (Theorem 1) for keys whose
 *                        norms span 100x, where the bf16 mode's cancellation of
 *                        ||k|| |S|-sized terms loses ~0.1 relative.  Scalar gate,
 *                        kla_prefill_chunked_ex only (sequential chunk scan). */
typedef enum kla_precision {
  KLA_PRECISION_BF16 = 0,
  KLA_PRECISION_SPLIT = 1
} kla_precision;

typedef struct kla_options {
  int32_t beta_mode;          /* a kla_beta_mode value */
  int32_t normalize_q;        /* nonzero: divide each readout by ||q_t||_2 */
  const int32_t *pos_offset;  /* device, 4-byte aligned, or NULL */
  int32_t diagonal_gate;      /* nonzero: g is per key channel, shaped like k */
  /* kla_prefill_chunked_ex's chunk scan over dense input (cu_seqlens NULL) with a
   * scalar gate: 0 picks by shape, 1 forces the sequential scan, G >= 2 the
   * two-level scan with (at most) G segments per sequence.  The two-level scan
   * runs segments 1..G-1 of every sequence from a zero state and from the
   * identity (their outputs unused; only their final states [N_g | M_g], with
   * S_out = M_g S_in + N_g since the chunk update is affine in the state,
   * Eq. (9)), chains the incoming states of the segments in fp32, then runs every
   * segment again from its true incoming state.  It does three times the
   * arithmetic for G-fold parallelism; the shape rule takes it when
   * n_seq * n_heads * d_v / 32 <= 128 (at most half of 256 compute units busy)
   * and each sequence has at least 64 chunks: G = min(512 / (n_seq * n_heads *
   * d_v / 32), chunks per sequence / 32).  Ignored elsewhere. */
  int32_t scan_segments;
  int32_t precision;          /* a kla_precision value */
} kla_options;

/* kla_prefill_workspace_bytes for the variant that opts selects (NULL = the
 * defaults, the same value as kla_prefill_workspace_bytes); 0 for unsupported
 * sizes.  Where total_tokens is a multiple of n_seq and the shape (or
 * scan_segments) selects the two-level scan, the size includes its fp32 scratch:
 * n_seq (G - 1) n_heads d_k (2 d_v + d_k) floats. */
size_t kla_prefill_workspace_bytes_ex(int32_t n_seq, int32_t total_tokens, int32_t n_heads,
                                      int32_t d_k, int32_t d_v, kla_dtype dtype,
                                      const kla_options *opts);

/* kla_prefill_chunked, kla_prefill_prepare and kla_decode_step with options
 * (NULL = the defaults, which is what the calls without _ex use).  The scan
 * half needs no options: kla_prefill_prepare_ex stores everything the variants
 * change (b in T, the readout factor in P and the per-chunk decays) in the
 * workspace. */
kla_status kla_prefill_chunked_ex(const void *q, const void *k, const void *v, const float *g,
                                  const float *eta, float eps, const float *S0, void *o,
                                  float *S_T, const int32_t *cu_seqlens,
                                  const int32_t *cu_seqlens_host, int32_t n_seq,
                                  int32_t total_tokens, int32_t n_heads, int32_t d_k,
                                  int32_t d_v, kla_dtype dtype, void *workspace,
                                  size_t workspace_bytes, const kla_options *opts, void *stream);

kla_status kla_prefill_prepare_ex(const void *q, const void *k, const float *g,
                                  const float *eta, float eps, const int32_t *cu_seqlens,
                                  const int32_t *cu_seqlens_host, int32_t n_seq,
                                  int32_t total_tokens, int32_t n_heads, int32_t d_k, int32_t d_v,
                                  kla_dtype dtype, void *workspace, size_t workspace_bytes,
                                  const kla_options *opts, void *stream);

kla_status kla_decode_step_ex(const void *q, const void *k, const void *v, const float *g,
                              const float *eta, float eps, const float *S, void *o,
                              float *S_new, int32_t batch, int32_t n_heads, int32_t d_k,
                              int32_t d_v, kla_dtype dtype, const kla_options *opts,
                              void *stream);

/*
 * Backward pass of the chunkwise prefill: the gradients (dq, dk, dv, dg, deta,
 * dS0) of the scalar loss <dO, o> + <dS_T, S_T> for the default variant
 * (Kaczmarz coefficient of Eq. (3), one scalar gate per token-head,
 * o_t = q_t S_t; kla_prefill_backward_ex below adds the coefficient modes and
 * the normalised readout).  The paper trains with the chunkwise algorithm (section 4,
 * Propositions 3-4, Eq. (7)-(9)) but derives no backward pass; these are the
 * exact derivatives of that chunk solve, so of the tokenwise recurrence
 * (Algorithm 1), up to rounding.
 *
 *   q, k, v, g, eta, eps, S0, cu_seqlens, cu_seqlens_host, sizes, dtype:
 *               the forward call's arguments, as for kla_prefill_chunked
 *   dO          [total_tokens, n_heads, d_v]   dtype (cotangent of o)
 *   dS_T        [n_seq, n_heads, d_k, d_v] fp32, or NULL for zeros
 *   dq, dk      [total_tokens, n_heads, d_k]   dtype (written)
 *   dv          [total_tokens, n_heads, d_v]   dtype (written)
 *   dg, deta    [total_tokens, n_heads]        fp32 (written)
 *   dS0         [n_seq, n_heads, d_k, d_v] fp32 (written), or NULL
 *   workspace   device buffer of at least kla_prefill_backward_workspace_bytes
 *               bytes, 256-byte aligned; contents are scratch.  It holds the
 *               forward chunk stage run again, and in the element type `dtype`
 *               (bf16 for bf16 inputs) every chunk's (I + L)^{-1}, incoming
 *               state, the cotangent of its outgoing state and its dU (dv,
 *               written first, is read back as the chunks' dR).
 * The gradient buffers must not overlap each other, the inputs or the
 * workspace.  q, k, v, dO, dq, dk and dv must be 16-byte aligned; g, eta, S0,
 * dS_T, dg, deta and dS0 4-byte aligned.  Size limits and errors as for
 * kla_prefill_chunked; zero-length sequences get dS0 = dS_T.
 */
size_t kla_prefill_backward_workspace_bytes(int32_t n_seq, int32_t total_tokens,
                                            int32_t n_heads, int32_t d_k, int32_t d_v,
                                            kla_dtype dtype);
kla_status kla_prefill_backward(const void *q, const void *k, const void *v, const float *g,
                                const float *eta, float eps, const float *S0, const void *dO,
                                const float *dS_T, void *dq, void *dk, void *dv, float *dg,
                                float *deta, float *dS0, const int32_t *cu_seqlens,
                                const int32_t *cu_seqlens_host, int32_t n_seq,
                                int32_t total_tokens, int32_t n_heads, int32_t d_k, int32_t d_v,
                                kla_dtype dtype, void *workspace, size_t workspace_bytes,
                                void *stream);

/* kla_prefill_backward with options (NULL = the defaults): the coefficient
 * modes (beta_mode, pos_offset), the normalised readout (normalize_q; the
 * gradient of a zero query is 0) and diagonal gating (diagonal_gate, paper
 * Appendix B.5: g and dg are then [total_tokens, n_heads, d_k] fp32, the
 * workspace is kla_prefill_backward_workspace_bytes_ex with the same options,
 * and it also holds the decayed key and query tiles of the forward stage and
 * every chunk's A = (K K^T per channel, decayed) in the element type).  precision other
 * than KLA_PRECISION_BF16 gives KLA_ERR_UNSUPPORTED.  The forward arguments and
 * options must be those of the forward call whose gradients are wanted. */
size_t kla_prefill_backward_workspace_bytes_ex(int32_t n_seq, int32_t total_tokens,
                                               int32_t n_heads, int32_t d_k, int32_t d_v,
                                               kla_dtype dtype, const kla_options *opts);
kla_status kla_prefill_backward_ex(const void *q, const void *k, const void *v, const float *g,
                                   const float *eta, float eps, const float *S0, const void *dO,
                                   const float *dS_T, void *dq, void *dk, void *dv, float *dg,
                                   float *deta, float *dS0, const int32_t *cu_seqlens,
                                   const int32_t *cu_seqlens_host, int32_t n_seq,
                                   int32_t total_tokens, int32_t n_heads, int32_t d_k,
                                   int32_t d_v, kla_dtype dtype, void *workspace,
                                   size_t workspace_bytes, const kla_options *opts, void *stream);

/*
 * kla_prefill_chunked_ex without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Its scratch is a static device array of
 * KLA_NOALLOC_SCRATCH_BYTES bytes in libkla.so, one per device the library runs
 * on, held until the process ends; the call allocates nothing.  A problem whose
 * kla_prefill_workspace_bytes_ex exceeds that size returns KLA_ERR_WORKSPACE with
 * nothing enqueued.  Every call on one device shares that device's array, and the
 * scratch keeps the last call's contents (each call writes all it reads, so
 * nothing needs clearing): calls that overlap in time on one device (other
 * streams, other threads) race on it and give wrong results; serialise them.
 * Other arguments, results and errors as for kla_prefill_chunked_ex.
 */
#define KLA_NOALLOC_SCRATCH_BYTES (64u << 20)
kla_status kla_prefill_chunked_noalloc(const void *q, const void *k, const void *v,
                                       const float *g, const float *eta, float eps,
                                       const float *S0, void *o, float *S_T,
                                       const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                       int32_t n_seq, int32_t total_tokens, int32_t n_heads,
                                       int32_t d_k, int32_t d_v, kla_dtype dtype,
                                       const kla_options *opts, void *stream);

/* Static description of a status code. */
const char *kla_status_string(kla_status status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char *kla_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t kla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KLA_H_ */
