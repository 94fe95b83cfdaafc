/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library, libkda.so.
 *
 * The method (miniKimiK3 model card, section "Architecture", Kimi Delta
 * Attention bullet): a linear-attention mixer whose per-head state S
 * (d_k x d_v) takes, for every token, a per-channel decay followed by one
 * gradient-descent step on the squared read-out error of v under key k;
 * it trains through a chunked parallel form and decodes as a fixed-size
 * recurrence.  In matrix form, per head and token t:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t,           alpha_t = exp(g_t),  g_t <= 0 per key channel
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument is DEVICE memory owned by the caller.  The library
 *   never allocates, frees or keeps a pointer after the call returns.
 * - Tensors are dense, contiguous, row-major with the shapes given below
 *   (token-major [B, T, H, D]; states [N, H, Dk, Dv] with Dv contiguous).
 * - Element type of q, k, v, g, beta and o is `dt` (KDA_F32 or KDA_BF16;
 *   KDA_F16 there is KDA_ERR_DTYPE); states (h0, ht, state) are float32,
 *   except a serving pool's, whose type is a knob.  bf16 is bfloat16 with
 *   round-to-nearest-even on output.
 * - Supported head sizes: Dk, Dv in {64, 128}.  g_group in {1, 64} is the
 *   number of consecutive key channels that share one log-decay value
 *   (1 = per-channel KDA decay; 64 = the "decay-g64" ablation of the
 *   Mini-K3-1H-decay-g64 card); it must divide Dk.
 * - All argument checks run on the host BEFORE any HIP call; a failed check
 *   returns its status and launches nothing.  A launch error is reported as
 *   KDA_ERR_HIP (from hipGetLastError, which also clears it).
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = default
 *   stream): no host synchronisation and no library state, so concurrent
 *   calls from several threads are safe as long as their buffers differ.
 * - Results are bitwise deterministic run to run (no atomics).
 * - No query scaling: pre-scale q if a scale is wanted (o is linear in q).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 10

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  KDA_ERR_SHAPE = 2,       /* negative size, mismatched sizes, or size overflow   */
  KDA_ERR_DTYPE = 3,       /* dt is not a kda_dtype value                         */
  KDA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required          */
  KDA_ERR_UNSUPPORTED = 5, /* Dk, Dv or g_group outside the supported set         */
  KDA_ERR_HIP = 6          /* a HIP launch failed                                 */
} kda_status;

/* Element types.  KDA_F16 is accepted only as the state type of the serving
 * pool (kda_recurrent_step_pool*); as an input type it is KDA_ERR_DTYPE. */
typedef enum { KDA_F32 = 0, KDA_BF16 = 1, KDA_F16 = 2 } kda_dtype;

/* Bytes of device workspace kda_chunk_fwd needs for these sizes (0 when no
 * workspace is needed: without cu_seqlens).  num_seqs is the number of
 * documents when cu_seqlens is used, else pass B.  varlen is nonzero when
 * the call will pass cu_seqlens: the workspace then holds the documents'
 * longest-first order (one int each), and only then is it needed.  Returns
 * 0 for invalid sizes (kda_chunk_fwd then reports the error). */
size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int num_seqs, int varlen,
                                     kda_dtype dt);

/* Chunked prefill (the chunked parallel form of the miniKimiK3 card's KDA
 * bullet).  Computes o_t for every token and, optionally, each sequence's
 * final state.  Internally the decay is referenced inside 16-token
 * sub-blocks, the state carried across them in fp32.
 *
 *   H      heads, 1 .. 65535 (a 64-token span of one tensor must stay below
 *          2 GiB: the kernels address a chunk with 32-bit byte offsets);
 *          more heads return KDA_ERR_SHAPE.
 *   q, k   [B, T, H, Dk]        dt
 *   v      [B, T, H, Dv]        dt
 *   g      [B, T, H, Dk/g_group] dt   log(alpha) <= 0
 *   beta   [B, T, H]            dt   write strength, in [0, 1] for a contraction
 *   h0     [N, H, Dk, Dv] f32 or NULL (NULL = zero initial state)
 *   o      [B, T, H, Dv]        dt   output (written for every token)
 *   ht     [N, H, Dk, Dv] f32 or NULL (final states; may alias h0)
 *   cu_seqlens  device int32 [num_seqs + 1] or NULL.  Non-NULL selects packed
 *          documents (Mini-K3-1H-mamba2 README, packed-document paragraph:
 *          state flow resets at every document boundary): B must be 1,
 *          document n is tokens cu[n] .. cu[n+1]-1 and starts from h0[n] (or
 *          zeros).  The caller guarantees cu[0] = 0, non-decreasing, cu[N] = T;
 *          values are clamped into [0, T] on the device so that no access
 *          leaves the buffers even if that is violated.  A zero-length
 *          document gets ht[n] = h0[n] (or zeros).
 *   num_seqs   N: number of documents with cu_seqlens, else must equal B.
 *   workspace  device memory of at least kda_chunk_fwd_workspace_bytes(...)
 *          bytes (may be NULL when that is 0); contents are scratch.
 *
 * Decay domain: the chunked form references decay to the midpoint of each
 * aligned 16-token block of a sequence (tokens 16j .. 16j+15 counted from the
 * sequence's first token), so every factor it forms lies within e^{|s|/2} of
 * 1, s the block's log-decay sum on that channel.  Per key channel, s must
 * stay above -140 (factors within e^{+-70}, inside the float and bf16
 * exponent range with room for the operand magnitudes); the decay over
 * longer spans is unrestricted (chunk sums of -100, -300 and -440 are in the
 * tests).  kda_recurrent_step has no such limit.
 */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                         const float* h0, void* o, float* ht, const int* cu_seqlens, int num_seqs, int B,
                         int T, int H, int Dk, int Dv, int g_group, kda_dtype dt, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Largest num_seqs kda_chunk_fwd_noalloc accepts with cu_seqlens. */
#define KDA_NOALLOC_MAX_SEQS 65536

/* kda_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as kda_chunk_fwd, minus the workspace.
 * The packed-document order table that kda_chunk_fwd keeps in the caller's
 * workspace (one int per document) lives instead in a static device array
 * of the library, 256 KiB, one copy per GPU, held until the process ends;
 * its device address is looked up on the first call on a device.  The call
 * itself allocates nothing (no hipMalloc, no allocating library routine).
 *
 *   cu_seqlens  as for kda_chunk_fwd; with cu_seqlens, num_seqs must be at
 *          most KDA_NOALLOC_MAX_SEQS, else KDA_ERR_WORKSPACE (checked on the
 *          host, nothing launched).  Without cu_seqlens no table is used.
 *   stream the table of the stream's device is used (the current device's
 *          for the NULL stream).
 *
 * Every call on one GPU shares that GPU's table, and each packed call
 * rewrites all of its num_seqs entries before reading them (nothing needs
 * to start at zero).  Packed calls that overlap on one GPU -- on different
 * streams, or from different threads without ordering -- race on the
 * table; the caller serialises them.  KDA_ERR_HIP if the table's address
 * cannot be obtained or a launch fails.
 */
kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                 const float* h0, void* o, float* ht, const int* cu_seqlens, int num_seqs, int B,
                                 int T, int H, int Dk, int Dv, int g_group, kda_dtype dt, void* stream);

/* Bytes of device workspace kda_chunk_bwd needs for these sizes: the
 * per-chunk states and cotangents of the backward pass (64-token chunks of
 * every sequence, dt = KDA_BF16), plus the varlen ordering table.  0 for
 * invalid sizes. */
size_t kda_chunk_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int num_seqs, int varlen,
                                     kda_dtype dt);

/* Backward pass of the chunked prefill (the miniKimiK3 card's KDA bullet:
 * KDA trains through the chunked parallel form).  Returns the gradients of
 * L = <do, o> + <dht, ht> for the forward kda_chunk_fwd(q, k, v, g, beta,
 * h0, cu_seqlens, ...) would compute; the forward's states are recomputed
 * internally, so o is not an input.
 *
 *   q, k, v, g, beta, h0, cu_seqlens, num_seqs, B, T, H, Dk, Dv, g_group:
 *          as for kda_chunk_fwd (same layouts, same head limit, the same
 *          decay domain: factors referenced to the midpoints of 16-token
 *          blocks, each block's log-decay sum above -140 per channel).
 *   dout   [B, T, H, Dv]   bf16  cotangent of o
 *   dht    [N, H, Dk, Dv]  f32 or NULL (NULL = zero)  cotangent of ht
 *   dq, dk [B, T, H, Dk]   bf16  gradients (every token written)
 *   dv     [B, T, H, Dv]   bf16
 *   dg     [B, T, H, Dk/g_group] bf16  (summed over a decay group)
 *   dbeta  [B, T, H]       bf16
 *   dh0    [N, H, Dk, Dv]  f32 or NULL: gradient of h0 (for a zero-length
 *          document it is dht[n])
 *   dt     KDA_BF16 only (KDA_F32 returns KDA_ERR_UNSUPPORTED).
 *   workspace  device memory of at least kda_chunk_bwd_workspace_bytes(...)
 *          bytes, 256-byte aligned; contents are scratch.
 *
 * Gradients of different documents never mix: with cu_seqlens, every
 * gradient of document n depends only on document n's inputs and
 * cotangents.  All pointers are caller-owned device memory; nothing is
 * allocated.  Errors: as for kda_chunk_fwd, plus KDA_ERR_NULL for a missing
 * gradient output when there are tokens.
 */
kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                         const float* h0, const void* dout, const float* dht, void* dq, void* dk, void* dv,
                         void* dg, void* dbeta, float* dh0, const int* cu_seqlens, int num_seqs, int B, int T,
                         int H, int Dk, int Dv, int g_group, kda_dtype dt, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Chunked prefill with the fused gate and normalisation prologue.  The
 * prologue turns a layer's raw projections into KDA's inputs inside the
 * prefill kernel, so there is no separate elementwise pass over q, k and g:
 *   q = q_raw / sqrt(|q_raw|^2 + 1e-6),  k likewise (per token and head);
 *   g = -exp(A_log) * softplus(f + dt_bias)   (per key channel or group);
 *   beta = sigmoid(b_raw).
 * Sources: the configurations' per-token L2-normalised q and k; A_log and
 * dt_bias as KDA's state controls (Kimi-K3-Tiny-L13 card, real weights
 * section; Mini-K3-1H-mamba2 README, optimiser paragraph).  The gate formula
 * itself is not on the pages; this is the Mamba-style reading.
 *
 *   q_raw, k_raw [B, T, H, Dk] dt; v [B, T, H, Dv] dt;
 *   f      [B, T, H, Dk/g_group] dt  gate logits
 *   b_raw  [B, T, H] dt              write-strength logits
 *   A_log, dt_bias  [H, Dk/g_group] f32 (device)
 *   everything else as for kda_chunk_fwd.
 * dt = KDA_BF16 or KDA_F32.  The decay domain of kda_chunk_fwd applies to
 * the g the prologue produces.
 */
kda_status kda_chunk_fwd_prologue(const void* q_raw, const void* k_raw, const void* v, const void* f,
                                  const void* b_raw, const float* A_log, const float* dt_bias, const float* h0,
                                  void* o, float* ht, const int* cu_seqlens, int num_seqs, int B, int T, int H,
                                  int Dk, int Dv, int g_group, kda_dtype dt, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Bytes of device workspace kda_chunk_bwd_prologue needs: the chunked
 * backward's workspace, the prepared inputs and their gradients (bf16), and
 * per 64-token block and head the partial sums of dA_log and d dt_bias.  0
 * for invalid sizes. */
size_t kda_chunk_bwd_prologue_workspace_bytes(int B, int T, int H, int Dk, int Dv, int num_seqs, int varlen,
                                              int g_group, kda_dtype dt);

/* Backward pass through the fused prologue and the chunked form (the
 * miniKimiK3 card's KDA bullet: KDA trains through its chunked form; the
 * Kimi-K3-Tiny-L13 card names A_log and dt_bias as its real parameters).
 * Returns the gradients of L = <do, o> + <dht, ht> for what
 * kda_chunk_fwd_prologue computes, with respect to q_raw, k_raw, v, f, b_raw,
 * A_log, dt_bias and h0.  The prepared q, k, g, beta are formed into the
 * workspace (bf16), kda_chunk_bwd runs on them, and the prologue's chain rule
 * follows: dq_raw = r (dq - q (q . dq)) with r the row's inverse norm,
 * df = dg * (-exp(A_log) sigmoid(f + dt_bias)), db_raw = dbeta beta (1 - beta),
 * dA_log = sum over tokens of dg * g, d dt_bias = sum over tokens of df
 * (summed in a fixed order: bitwise deterministic).
 *
 *   q_raw, k_raw, v, f, b_raw, A_log, dt_bias, h0, cu_seqlens, sizes: as for
 *          kda_chunk_fwd_prologue (dt = KDA_BF16 only, like kda_chunk_bwd).
 *   dout, dht, dv, dh0: as for kda_chunk_bwd.
 *   dq_raw, dk_raw [B, T, H, Dk] bf16; df [B, T, H, Dk/g_group] bf16;
 *   db_raw [B, T, H] bf16; dA_log, ddt_bias [H, Dk/g_group] f32 (always
 *          written; zero without tokens).
 *   workspace  at least kda_chunk_bwd_prologue_workspace_bytes(...) bytes,
 *          256-byte aligned; contents are scratch.
 * q_raw, k_raw, dq_raw, dk_raw (and f, df with g_group = 1) must be 16-byte
 * aligned (KDA_ERR_UNSUPPORTED otherwise).  Other errors as for kda_chunk_bwd.
 */
kda_status kda_chunk_bwd_prologue(const void* q_raw, const void* k_raw, const void* v, const void* f,
                                  const void* b_raw, const float* A_log, const float* dt_bias, const float* h0,
                                  const void* dout, const float* dht, void* dq_raw, void* dk_raw, void* dv, void* df,
                                  void* db_raw, float* dA_log, float* ddt_bias, float* dh0, const int* cu_seqlens,
                                  int num_seqs, int B, int T, int H, int Dk, int Dv, int g_group, kda_dtype dt,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* One decode step with the same fused prologue (q_raw, k_raw [N, H, Dk];
 * v [N, H, Dv]; f [N, H, Dk/g_group]; b_raw [N, H]; A_log, dt_bias
 * [H, Dk/g_group] f32; state [N, H, Dk, Dv] f32 in place; o [N, H, Dv]).
 * dt = KDA_F32 or KDA_BF16.  Errors as for kda_recurrent_step.
 */
kda_status kda_recurrent_step_prologue(const void* q_raw, const void* k_raw, const void* v, const void* f,
                                       const void* b_raw, const float* A_log, const float* dt_bias, float* state,
                                       void* o, int N, int H, int Dk, int Dv, int g_group, kda_dtype dt,
                                       void* stream);

/* Training pair: kda_chunk_fwd_save is kda_chunk_fwd (o, optional ht) that
 * also keeps, in the backward workspace, the state entering every 64-token
 * chunk; kda_chunk_bwd_saved is kda_chunk_bwd without its own recomputation
 * of those states.  The workspace (kda_chunk_bwd_workspace_bytes, 256-byte
 * aligned) must be passed to both, and the backward must see exactly the
 * forward's q, k, v, g, beta, h0, cu_seqlens and sizes; between the two
 * calls the workspace must not be used otherwise.  Gradients are bitwise
 * those of kda_chunk_bwd.  Arguments, dtypes (bf16 only) and errors as for
 * kda_chunk_fwd and kda_chunk_bwd. */
kda_status kda_chunk_fwd_save(const void* q, const void* k, const void* v, const void* g, const void* beta,
                              const float* h0, void* o, float* ht, const int* cu_seqlens, int num_seqs, int B, int T,
                              int H, int Dk, int Dv, int g_group, kda_dtype dt, void* workspace,
                              size_t workspace_bytes, void* stream);
kda_status kda_chunk_bwd_saved(const void* q, const void* k, const void* v, const void* g, const void* beta,
                               const float* h0, const void* dout, const float* dht, void* dq, void* dk, void* dv,
                               void* dg, void* dbeta, float* dh0, const int* cu_seqlens, int num_seqs, int B, int T,
                               int H, int Dk, int Dv, int g_group, kda_dtype dt, void* workspace,
                               size_t workspace_bytes, void* stream);

/* One recurrent decode step for N sequences x H heads (the recurrence of the
 * miniKimiK3 card's KDA bullet: constant cost per token), state in place.
 *
 *   q, k   [N, H, Dk]  dt;   v [N, H, Dv] dt;   g [N, H, Dk/g_group] dt;
 *   beta   [N, H]      dt;
 *   state  [N, H, Dk, Dv] f32, read and overwritten with S_t;
 *   o      [N, H, Dv]  dt.
 * N = 0 is a no-op.  Valid for any g (no chunk-decay domain limit).
 */
kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const void* g, const void* beta,
                              float* state, void* o, int N, int H, int Dk, int Dv, int g_group, kda_dtype dt,
                              void* stream);

/* One recurrent decode step over a serving state pool.  The K3-Tiny-L13 card
 * (serving notes under "Measured on 1x B300") reports decode concurrency
 * capped by the pool of per-sequence KDA states, with the state dtype as a
 * serving knob; this entry point is that pool's step.  Sequence n reads and
 * writes pool slot slots[n]; the step itself is the one of kda_recurrent_step.
 *
 *   q, k, v, g, beta, o   as for kda_recurrent_step ([N, H, ...], dt);
 *   o_gate [N, H, Dv] dt, or NULL: logits z of the output gate.  The
 *          Mini-K3-1H model cards list output gates among the family's
 *          operators without a formula; it is read as the elementwise
 *          logistic gate o <- o * sigmoid(z) on the step's output.  It
 *          never reaches the state; an inactive sequence's row stays zero.
 *   state_pool  [num_slots, H, Dk, Dv] of state_dt, updated in place for the
 *          slots named by active sequences; every other slot is untouched.
 *   slots  device int32 [N]: the pool slot of each sequence.  A value outside
 *          [0, num_slots) marks the sequence inactive: its o row is written
 *          as zeros and no state is read or written.  Two active sequences
 *          must not name the same slot (their updates would race).
 *   num_slots  pool size (>= 0; state_pool may be NULL when it is 0).
 *   state_dt   KDA_F32, KDA_BF16 or KDA_F16.  A bf16 or fp16 state is
 *          widened to fp32 for the step and rounded to nearest even when
 *          written back (fp16: IEEE binary16, overflow to infinity).
 * N = 0 is a no-op.  Errors: KDA_ERR_NULL (q, k, v, g, beta, slots or o NULL,
 * or state_pool NULL with num_slots > 0), KDA_ERR_SHAPE, KDA_ERR_DTYPE (dt
 * or state_dt), KDA_ERR_UNSUPPORTED, KDA_ERR_HIP as elsewhere.
 */
kda_status kda_recurrent_step_pool(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                   void* state_pool, const int* slots, int num_slots, void* o, const void* o_gate,
                                   int N, int H, int Dk, int Dv, int g_group, kda_dtype dt, kda_dtype state_dt,
                                   void* stream);

/* The serving-pool decode step with the fused gate and normalisation
 * prologue: kda_recurrent_step_pool on raw projections, as
 * kda_recurrent_step_prologue is kda_recurrent_step on raw projections.
 *
 *   q_raw, k_raw, v, f, b_raw, A_log, dt_bias   as for
 *          kda_recurrent_step_prologue ([N, H, ...] dt; A_log and dt_bias
 *          f32 [H, Dk/g_group]);
 *   state_pool, slots, num_slots, o, o_gate, state_dt   as for
 *          kda_recurrent_step_pool.
 * N = 0 is a no-op.  Errors as for kda_recurrent_step_pool, plus
 * KDA_ERR_NULL for a NULL A_log or dt_bias when N > 0.
 */
kda_status kda_recurrent_step_pool_prologue(const void* q_raw, const void* k_raw, const void* v, const void* f,
                                            const void* b_raw, const float* A_log, const float* dt_bias,
                                            void* state_pool, const int* slots, int num_slots, void* o,
                                            const void* o_gate, int N, int H, int Dk, int Dv, int g_group,
                                            kda_dtype dt, kda_dtype state_dt, void* stream);

/* Short causal depthwise convolution along the token axis, with document
 * reset.  The miniKimiK3 card ("Limitations") says order information reaches
 * the model only through KDA's decay and short convolutions plus the causal
 * mask; the Mini-K3-1H-mamba2 README (packed-document paragraph) resets
 * convolution history at every document boundary; the Mini-K3-1H cards list
 * convolution length as an ablation axis.  Per channel c and token t of a
 * sequence (or document) that starts at s:
 *
 *   y[t][c] = sum_{w=0}^{W-1} weight[c][w] * x[t - (W-1) + w][c]
 *
 * where a position p < s reads the initial conv state: conv0[n][p - s + W-1][c]
 * (the W-1 inputs that preceded the sequence), or zero when conv0 is NULL.
 * No bias, no activation.  Accumulation is fp32.
 *
 *   x      [B, T, C]   dt        (C: channels, e.g. H * D of one projection)
 *   weight [C, W]      dt
 *   conv0  [N, W-1, C] dt or NULL
 *   y      [B, T, C]   dt        output (may not alias x)
 *   conv_final [N, W-1, C] dt or NULL: each sequence's last W-1 inputs
 *          (positions before its start taken from conv0 / zeros); may not
 *          alias conv0.
 *   cu_seqlens, num_seqs, B, T: as for kda_chunk_fwd (device int32
 *          [num_seqs + 1] or NULL; non-NULL requires B = 1; clamped into
 *          [0, T] on the device).
 * Supported: 1 <= W <= 8, C a positive multiple of 8, and x, y, conv0,
 * conv_final 16-byte aligned.  Errors as for kda_chunk_fwd; KDA_ERR_UNSUPPORTED
 * for W, C or alignment outside that set.
 */
kda_status kda_short_conv_fwd(const void* x, const void* weight, const void* conv0, void* y, void* conv_final,
                              const int* cu_seqlens, int num_seqs, int B, int T, int C, int W, kda_dtype dt,
                              void* stream);

/* Bytes of device workspace kda_short_conv_bwd needs (fp32 partial sums of
 * the weight gradient, one row per 256-token run); 0 for invalid sizes. */
size_t kda_short_conv_bwd_workspace_bytes(int B, int T, int C, int W);

/* Backward of kda_short_conv_fwd: the gradients of L = <dy, y> +
 * <dconv_final, conv_final> (the convolution is linear in x and conv0, and
 * in the weights).  Per channel, for a token t of a sequence [s, e):
 *
 *   dx[t]       = sum_{u=0}^{W-1} weight[W-1-u] dy[t+u]  over t+u < e,
 *                 + dconv_final[t - (e - (W-1))]         for t >= e - (W-1)
 *   dweight[w] += dy[t] x[t - (W-1) + w]   (positions before s: conv0 / zeros)
 *   dconv0[row] = the same sum as dx, at the history position s - (W-1) + row
 *
 *   x, weight, conv0, cu_seqlens, num_seqs, B, T, C, W, dt: as for
 *          kda_short_conv_fwd.
 *   dy [B, T, C] dt; dconv_final [N, W-1, C] dt or NULL (zero).
 *   dx [B, T, C] dt; dweight [C, W] f32 (summed over every token, in a fixed
 *          order: bitwise deterministic); dconv0 [N, W-1, C] dt or NULL.
 *   workspace  at least kda_short_conv_bwd_workspace_bytes(B, T, C, W) bytes,
 *          256-byte aligned; contents are scratch.
 * Supported sizes, alignment and errors as for kda_short_conv_fwd (dy, dx,
 * dconv_final and dconv0 16-byte aligned); KDA_ERR_WORKSPACE for a missing
 * or short workspace.
 */
kda_status kda_short_conv_bwd(const void* x, const void* weight, const void* conv0, const void* dy,
                              const void* dconv_final, void* dx, float* dweight, void* dconv0,
                              const int* cu_seqlens, int num_seqs, int B, int T, int C, int W, kda_dtype dt,
                              void* workspace, size_t workspace_bytes, void* stream);

/* One decode step of the short convolution for N sequences, state in place:
 * with the window [conv_state[n][0..W-2], x[n]], y[n] = sum_w weight[:, w] *
 * window[w] and conv_state[n] <- window[1..W-1].
 *   x [N, C] dt;  weight [C, W] dt;  conv_state [N, W-1, C] dt;  y [N, C] dt.
 * conv_state may be NULL only when W = 1.  N = 0 is a no-op.  Supported W,
 * C and alignment (x, y, conv_state) as for kda_short_conv_fwd.
 */
kda_status kda_short_conv_step(const void* x, const void* weight, void* conv_state, void* y, int N, int C, int W,
                               kda_dtype dt, void* stream);

/* Static description of a status code (never NULL). */
const char* kda_status_str(kda_status s);

/* KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
