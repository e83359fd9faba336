/*
 * kda.h -- C ABI of libkda, the MI355X (gfx950) implementation of the Kimi
 * Delta Attention (KDA) gated delta-rule recurrence.
 *
 * The operation (per batch row b and head h, state S in R^{dk x dv}, row
 * index = key channel):
 *
 *   g_t = g_min * Sigmoid(exp(A_h) * z_t)        lower-bounded log-decay, dk
 *   a_t = exp(g_t)                               channel-wise retention
 *   S_t = (I - beta_t k_t k_t^T) Diag(a_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t = S_t^T q_t
 *
 * Sources: dev.to "Kimi K3 Architecture: Scaling 2.8T Parameters for
 * Long-Context Multimodal MoE", section "The Sequence Bottleneck: Hybrid KDA
 * and Gated MLA" (state shape, retention and delta-strength domains, the gate
 * equation, g_min = -5, 16-token tiles, chunkwise parallel execution);
 * terrencekim.net "Kimi K3 - Sparsity Mechanics ...", section 2, Temporal
 * Sequence card (fixed-size associative memory, Householder-style delta
 * update, channel-wise forget gate).  The pages state the update in words;
 * the algebraic form above is the reading implemented here: decay, then
 * erase-and-write, output from the updated state, no 1/sqrt(d) scale, no
 * output gate or normalisation.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - All tensor arguments are DEVICE pointers, caller-owned; the library never
 *   allocates, frees or synchronises.  Calls enqueue work on `stream`
 *   (a hipStream_t; NULL = the default stream) and return at once.
 * - Layouts are contiguous row-major:
 *     q, k, z   [B, T, H, d_k]      v, o [B, T, H, d_v]
 *     beta      [B, T, H]  fp32     A    [H] fp32
 *     S0, S_T   [B, H, d_k, d_v] fp32 (row = key channel)
 *   Decode uses T = 1: q, k, z [B, H, d_k], v, o [B, H, d_v], beta [B, H].
 * - `dt` gives the element type of q, k, v, z and o (KDA_F32 or KDA_BF16);
 *   beta, A, g_min and the state are always fp32.  Accumulation is fp32.
 * - Supported head sizes: (d_k, d_v) in {(32, 32), (128, 128)}.
 * - Size limits (KDA_ERR_INVALID_SHAPE beyond them): T <= 2^30,
 *   B * H <= 2^26, B * T * H <= 2^40, H * d_k <= 2^24 (the kernels address 32
 *   consecutive tokens of one head with 32-bit byte offsets and count chunks
 *   in 32-bit integers).
 * - beta is used as given (expected in (0, 1)); q and k are used as given
 *   (no normalisation inside).  g_min must lie in [-5, 0]: the chunked form
 *   rescales 16-token tiles by factors up to exp(-16 g_min), which must stay
 *   finite in fp32/bf16 (exp(80) < FLT_MAX).
 * - Alignment: q, k, v, z, o, the decode state S and the workspace must be
 *   16-byte aligned (they are read with 16-byte vector accesses); beta, A,
 *   S0, S_T and the diagnostic outputs need 4-byte alignment.
 * - Every argument is validated on the host BEFORE any HIP call; on error
 *   nothing is enqueued, the status is returned and a detail string is kept
 *   for kda_last_error() (thread-local).  No entry point aborts, exits or
 *   throws across the ABI.  A failed kernel launch returns KDA_ERR_HIP.
 * - Results are bitwise deterministic for identical inputs and launch
 *   (no atomics, fixed reduction orders).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1
/* Tokens per chunk of the chunkwise prefill (the pages' 16-token tiles). */
#define KDA_CHUNK 16

/* Largest token count of one kda_decode_tokens call. */
#define KDA_MAX_DECODE_TOKENS 16

/* Status codes and element types are plain ints in the ABI (any value a
 * caller passes in is well defined; unknown ones are rejected or named
 * "KDA_ERR_UNKNOWN"). */
typedef int kda_status;
enum {
    KDA_OK = 0,
    KDA_ERR_NULL_POINTER = 1,        /* a required pointer is NULL            */
    KDA_ERR_INVALID_SHAPE = 2,       /* B, T or H < 1, or a size limit broken */
    KDA_ERR_INVALID_VALUE = 3,       /* g_min outside [-5, 0] or not finite   */
    KDA_ERR_UNSUPPORTED = 4,         /* head size or dtype not supported      */
    KDA_ERR_MISALIGNED = 5,          /* a pointer is not 16-byte aligned      */
    KDA_ERR_WORKSPACE_TOO_SMALL = 6, /* workspace below the queried size      */
    KDA_ERR_ALIASING = 7,            /* an output overlaps an input illegally */
    KDA_ERR_HIP = 8                  /* the HIP runtime reported an error     */
};

typedef int kda_dtype;
enum { KDA_F32 = 0, KDA_BF16 = 1 };

/* KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);

/* Static, human-readable name of a status code ("KDA_OK", ...). */
const char *kda_status_string(kda_status status);

/* Detail of the last error raised on the calling thread ("" if none).
 * The pointer stays valid until the next libkda call on this thread. */
const char *kda_last_error(void);

/* Bytes of device workspace kda_chunk_prefill needs for these sizes.
 * 0 means the call needs none (workspace may then be NULL).  Returns 0 for
 * arguments kda_chunk_prefill would reject. */
size_t kda_chunk_prefill_workspace_bytes(int B, int T, int H, int d_k, int d_v,
                                         kda_dtype dt);

/* Segments kda_chunk_prefill splits each sequence into for these sizes: 1
 * for a direct plan, R > 1 when it runs the segment scan of
 * kda_chunk_prefill_segmented with n_seg = R (same context parallelism
 * passage as there).  It does so for long sequences of few heads, where the
 * heads' own state chains cannot fill the device: bf16 inputs, d = 128,
 * T >= 65536, B * H <= 32, with B * R * H >= 128 and T / R >= 4096.  Returns
 * 0 for arguments kda_chunk_prefill would reject. */
int kda_chunk_prefill_segments(int B, int T, int H, int d_k, int d_v, kda_dtype dt);

/* The plan kda_chunk_prefill runs for these sizes on the current device, as
 * a static string: "segment scan" (the segment scan above), "ring" (pair
 * producers and state chains in one launch, pairs passed through an XCD's L2:
 * bf16, d = 128, B * H * 8 workgroups fit the device's CUs at one each),
 * "split" (pair blocks through the workspace) or "fused:<columns>" (one
 * launch per 16-token chunk chain, no workspace).  "" for arguments
 * kda_chunk_prefill would reject.  Informational: results do not depend on
 * the plan beyond rounding. */
const char *kda_chunk_prefill_plan(int B, int T, int H, int d_k, int d_v, kda_dtype dt);

/* Chunkwise prefill over T tokens (any T >= 1; chunks of KDA_CHUNK tokens
 * start at t = 0 and the last may be short).  Computes o for every token and,
 * if S_T != NULL, the final state.
 * Source: dev.to "Kimi K3 Architecture ...", section "The Sequence
 * Bottleneck: Hybrid KDA and Gated MLA" -- the gated delta rule run as
 * chunkwise parallel execution over 16-token tiles, the within-tile and
 * state ("diagonal" and "off-diagonal") parts as dense matrix products, the
 * tiles' cumulative log-decay inside (-80, 0) for g_min = -5; terrencekim.net
 * "Kimi K3 - Sparsity Mechanics ...", section 2, Temporal Sequence (KDA)
 * card -- a fixed-size state per head carried from one token to the next.
 *   S0 == NULL      : the initial state is zero.
 *   S_T may alias S0 exactly (in-place continuation); no other overlap of
 *   outputs (o, S_T, workspace) with inputs is allowed.
 *   workspace       : device memory of at least
 *                     kda_chunk_prefill_workspace_bytes(...) bytes, used as
 *                     scratch for this call only (may be NULL if that is 0).
 * The execution plan (one fused kernel, an intra-chunk kernel writing the
 * workspace followed by an inter-chunk kernel, or the segment scan of
 * kda_chunk_prefill_segmented with kda_chunk_prefill_segments(...) segments)
 * is a function of the sizes; the segment scan restarts the chunk grid at
 * every segment start, so results agree with the direct plans up to
 * rounding.  Test and tuning hook only (production callers leave it unset):
 * the environment variable KDA_PREFILL_PLAN overrides the plan (and then no
 * segment scan is chosen): "split" (default inter-chunk variant),
 * "split:<n>:<b>" (n value
 * columns per inter-chunk workgroup, b 16-column blocks per state chain:
 * b = 1 with n in {16, 32} or, for bf16 with d = 128, 64; b = 2 for bf16
 * with d = 128, n in {32, 64}), or "fused:<n>" with n value columns per
 * workgroup (16, 32, 64, or 128 <= d_v; fp32 with d = 128: at most 64).  An
 * override that names no compiled variant is ignored.  The workspace query honours
 * the same variable, so read both under one setting.
 * The chained result of two calls (the second with S0 = the first's S_T)
 * equals one call over the concatenated tokens up to rounding. */
kda_status kda_chunk_prefill(const void *q, const void *k, const void *v,
                             const void *z, const float *beta, const float *A,
                             float g_min, const float *S0, void *o, float *S_T,
                             int B, int T, int H, int d_k, int d_v, kda_dtype dt,
                             void *workspace, size_t workspace_bytes,
                             void *stream);

/* Bytes of the static scratch that kda_chunk_prefill_noalloc uses in place of
 * a workspace (one copy per GPU the library runs on, held until the process
 * ends). */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/* kda_chunk_prefill for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same arguments, results and plan choice as kda_chunk_prefill, but no
 * workspace argument: the workspace kda_chunk_prefill_workspace_bytes(...)
 * names is taken from a static device array of KDA_NOALLOC_SCRATCH_BYTES on
 * the GPU that `stream` runs on.  Sizes needing more than that return
 * KDA_ERR_WORKSPACE_TOO_SMALL (on the host, before any HIP call).  The call
 * allocates nothing; its first call on a device looks up that device's copy
 * of the array (hipGetSymbolAddress).  Every call on one GPU shares that GPU's
 * scratch, so calls that overlap in time on one GPU (different streams, or
 * different host threads without ordering) race and must not be issued; calls
 * in one stream are ordered and safe.  Nothing is expected to be zero in the
 * scratch between calls: every call writes what it reads. */
kda_status kda_chunk_prefill_noalloc(const void *q, const void *k, const void *v,
                                     const void *z, const float *beta, const float *A,
                                     float g_min, const float *S0, void *o, float *S_T,
                                     int B, int T, int H, int d_k, int d_v, kda_dtype dt,
                                     void *stream);

/* Bytes of device workspace kda_chunk_prefill_segmented needs (0 for
 * arguments it would reject): the inner prefill's workspace for B * n_seg
 * rows of T / n_seg tokens, four state tensors [B * n_seg, H, d_k, d_v] fp32,
 * and, unless the map passes are state-only (d = 128 and B * n_seg * H >=
 * 128), a zero value tensor of the size of v. */
size_t kda_chunk_prefill_segmented_workspace_bytes(int B, int T, int H, int d_k,
                                                   int d_v, int n_seg,
                                                   kda_dtype dt);

/* kda_chunk_prefill computed by a scan over n_seg segments of T / n_seg
 * tokens each (n_seg must divide T): the single-GPU form of the pages' KDA
 * context parallelism (dev.to "Kimi K3 Architecture ...", section
 * "Infrastructure and Training/Inference Mechanics": local state updates
 * merged by a prefix scan of fixed-size states).  Each segment's state map
 * S_end = M S_in + N comes from two prefills of all segments side by side (v
 * = 0 from S0 = I; v from S0 = 0); a scan gives every segment's start state
 * and S_T; a last prefill from those start states writes o.  Same arguments,
 * layouts, aliasing rules and results (up to rounding) as kda_chunk_prefill;
 * the chunk grid restarts at every segment start.  It costs three passes
 * over the tokens plus the scan (the two map passes read neither q nor, for
 * M, v and write no o where B * n_seg * H >= 128 and d = 128), and is the
 * building block of a prefill split across devices by sequence position.
 *   workspace : at least kda_chunk_prefill_segmented_workspace_bytes(...)
 *               bytes (never NULL). */
kda_status kda_chunk_prefill_segmented(const void *q, const void *k,
                                       const void *v, const void *z,
                                       const float *beta, const float *A,
                                       float g_min, const float *S0, void *o,
                                       float *S_T, int B, int T, int H,
                                       int d_k, int d_v, int n_seg,
                                       kda_dtype dt, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* Bytes of device workspace kda_chunk_backward needs for these sizes (0 for
 * arguments it would reject).  It holds the state at the start of every
 * 16-token chunk (B * H * ceil(T / 16) * d_k * d_v * 4 bytes) and, when T
 * splits into segments of 256 or more tokens, a segment scan's buffers; for
 * bf16 at d = 128 also the gradient of every chunk's end state (as much
 * again) and the chain's operands (13,824 bytes per chunk and head);
 * otherwise the delta-rule correction v - S'^T k of every token
 * (B * T * H * d_v * 4 bytes), one state per (b, h) carried between launches
 * and partial sums of one segment of the sequence (about 256 MiB, or 128
 * tokens' worth if that is more). */
size_t kda_chunk_backward_workspace_bytes(int B, int T, int H, int d_k, int d_v,
                                          kda_dtype dt);

/* Gradients of kda_chunk_prefill (the pages give no backward pass; this is
 * the exact gradient of the recurrence above, for training; dev.to "Kimi K3
 * Architecture ...", section "The Sequence Bottleneck": chunkwise parallel
 * execution, which training relies on).  For bf16 at d = 128 it runs the
 * chunk equations differentiated: a chain of chunk-end state gradients from
 * dS_T back to dS0, then every chunk's gradients at once, all products on
 * MFMA; other sizes run a token-level reverse sweep.  With dO the
 * gradient of o [B, T, H, d_v] (element type dt) and dS_T that of the final
 * state [B, H, d_k, d_v] fp32 (NULL: zero), it writes the gradients of
 * L = sum(dO * o) + sum(dS_T * S_T):
 *   dq, dk, dz [B, T, H, d_k] and dv [B, T, H, d_v]   element type dt
 *   dbeta [B, T, H], dA [H]                            fp32
 *   dS0 [B, H, d_k, d_v]  fp32, the gradient of the initial state (NULL: not
 *                         written; it is the same whether or not S0 is NULL)
 * q, k, v, z, beta, A, g_min and S0 (NULL: zero) are the forward call's
 * inputs; the forward states are recomputed from them, o is not needed.
 *   S0, dS_T and dS0 must be 16-byte aligned.  No output may overlap an input,
 *   another output or the workspace.
 *   workspace       : device memory of at least
 *                     kda_chunk_backward_workspace_bytes(...) bytes, scratch
 *                     for this call only.
 * The sweep runs in fp32 whatever dt is.  dA and dbeta are summed over
 * value-column blocks and tokens in a fixed order (deterministic).
 * Test and tuning hook only (production callers leave it unset): the
 * environment variable KDA_BACKWARD_PLAN=sweep forces the token-level sweep
 * for bf16 at d = 128 too, and KDA_BACKWARD_PLAN=chain selects the chunk-level plan (a chain of per-chunk state gradients, then
 * every chunk's reverse sweep at once) instead of the default sweep over the
 * whole sequence; the workspace query honours the same variable. */
kda_status kda_chunk_backward(const void *q, const void *k, const void *v,
                              const void *z, const float *beta, const float *A,
                              float g_min, const float *S0, const void *dO,
                              const float *dS_T, void *dq, void *dk, void *dv,
                              void *dz, float *dbeta, float *dA, float *dS0,
                              int B, int T, int H, int d_k, int d_v,
                              kda_dtype dt, void *workspace,
                              size_t workspace_bytes, void *stream);

/* One recurrent decode step: for every (b, h) the state S [B, H, d_k, d_v]
 * (fp32) is read once and overwritten in place with S_t; o receives
 * S_t^T q_t.  o must not overlap S or the inputs.
 * Source: terrencekim.net "Kimi K3 - Sparsity Mechanics ...", section 2,
 * Temporal Sequence (KDA) card -- a fixed-size associative memory in place of
 * a growing KV cache, updated per token by a Householder-style delta rule
 * with channel-wise forget gates; dev.to "Kimi K3 Architecture ...", section
 * "The Sequence Bottleneck: Hybrid KDA and Gated MLA" -- the state shape and
 * the gate equation. */
kda_status kda_decode_step(const void *q, const void *k, const void *v,
                           const void *z, const float *beta, const float *A,
                           float g_min, float *S, void *o, int B, int H,
                           int d_k, int d_v, kda_dtype dt, void *stream);

/* T consecutive decode steps (1 <= T <= KDA_MAX_DECODE_TOKENS) of every
 * sequence from a live state, for checking T drafted tokens at once: the same
 * recurrence as kda_decode_step applied to tokens t = 0 .. T-1 (dev.to page,
 * "The Sequence Bottleneck": the gated delta rule; the podcast page,
 * "Evidence Confidence by Component", names a speculative-decoding use of
 * KDA without describing it -- this is the plain multi-token step it needs).
 *   q, k, v, z, o : [B, T, H, d] like kda_chunk_prefill; beta [B, T, H].
 *   S             : [B, H, d_k, d_v] fp32 state before token 0 (read only).
 *   S_out         : receives the state after token T-1.  S_out == S commits
 *                   in place; a separate buffer leaves S as the snapshot to
 *                   replay the accepted prefix from (call again with the
 *                   accepted count as T).  Partial overlap of S_out and S,
 *                   and any overlap of o or S_out with another argument, is
 *                   KDA_ERR_ALIASING.
 * S is read and S_out written once per call, whatever T.  Returns
 * KDA_ERR_INVALID_SHAPE for T outside [1, KDA_MAX_DECODE_TOKENS]. */
kda_status kda_decode_tokens(const void *q, const void *k, const void *v,
                             const void *z, const float *beta, const float *A,
                             float g_min, const float *S, float *S_out, void *o,
                             int B, int T, int H, int d_k, int d_v, kda_dtype dt,
                             void *stream);

/* Paged states (a serving engine's layout: dev.to page, "Infrastructure and
 * Training/Inference Mechanics", fixed-size KDA states held apart from the
 * attention cache).  The states live in a pool [n_slots, H, d_k, d_v] fp32,
 * and sequence b uses the pool row named by an int32 slot table [B] in
 * device memory; the calls below are the dense calls with S0 / S_T / S
 * replaced by pool rows.  Slot values are read by the kernels only: a
 * sequence whose slot lies outside [0, n_slots) is skipped (none of its
 * outputs and no pool row are written).  Two sequences writing one slot in
 * the same call race; a sequence may read and write the same slot.  The pool
 * may not overlap any other argument, nor o; the slot tables may coincide.
 * Returns KDA_ERR_INVALID_SHAPE for n_slots < 1. */

/* Bytes of device workspace kda_chunk_prefill_paged needs for these sizes
 * (0: none; also 0 for arguments it would reject).  It differs from
 * kda_chunk_prefill_workspace_bytes where the dense call runs the segment
 * scan (which the paged call never does), so query each call with its own
 * function. */
size_t kda_chunk_prefill_paged_workspace_bytes(int B, int T, int H, int d_k, int d_v,
                                               kda_dtype dt);

/* kda_chunk_prefill from pool row slots_in[b] (NULL: zero initial states)
 * into pool row slots_out[b] (NULL: no state written), always by a direct
 * plan (never the segment scan).
 *   workspace : at least kda_chunk_prefill_paged_workspace_bytes(...) bytes
 *               (may be NULL if that is 0). */
kda_status kda_chunk_prefill_paged(const void *q, const void *k, const void *v,
                                   const void *z, const float *beta,
                                   const float *A, float g_min, float *pool,
                                   int n_slots, const int *slots_in,
                                   const int *slots_out, void *o, int B,
                                   int T, int H, int d_k, int d_v,
                                   kda_dtype dt, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* kda_decode_step on pool row slots[b], in place. */
kda_status kda_decode_step_paged(const void *q, const void *k, const void *v,
                                 const void *z, const float *beta,
                                 const float *A, float g_min, float *pool,
                                 int n_slots, const int *slots, void *o, int B,
                                 int H, int d_k, int d_v, kda_dtype dt,
                                 void *stream);

/* kda_decode_tokens from pool row slots_in[b] into pool row slots_out[b]
 * (the same row commits in place; another keeps the snapshot). */
kda_status kda_decode_tokens_paged(const void *q, const void *k, const void *v,
                                   const void *z, const float *beta,
                                   const float *A, float g_min, float *pool,
                                   int n_slots, const int *slots_in,
                                   const int *slots_out, void *o, int B,
                                   int T, int H, int d_k, int d_v,
                                   kda_dtype dt, void *stream);

/* Diagnostic export of the gate stage: G [B, T, H, d_k] fp32 receives the
 * chunk-local inclusive cumulative log-decay
 *   G_t = sum of g_s over s from the start of t's KDA_CHUNK-token chunk to t,
 * (dev.to page, "The Sequence Bottleneck": per-16-token cumulative log-decay
 * in (-80, 0) for g_min = -5).  G must not overlap z. */
kda_status kda_gate_chunk_cumsum(const void *z, const float *A, float g_min,
                                 float *G, int B, int T, int H, int d_k,
                                 kda_dtype dt, void *stream);

/* Diagnostic export of the intra-chunk stage, computed by the same device
 * code the prefill runs.  For chunk n of (b, h), with G the chunk-local
 * cumulative log-decay, Kt = k e^{G}, Kh = k e^{-G}, Qt = q e^{G} (rows =
 * the chunk's tokens, L <= KDA_CHUNK of them; rows past L are zero-padded):
 *   Tm    [B, H, NC, 16, 16] fp32 : (I + tril_{-1}(Diag(beta) Kt Kh^T))^{-1} Diag(beta)
 *   Aqk   [B, H, NC, 16, 16] fp32 : tril_0(Qt Kh^T)
 *   gamma [B, H, NC, d_k]    fp32 : e^{G at the chunk's last token}
 * where NC = ceil(T / KDA_CHUNK).  Tm and Aqk are the products as the MFMA
 * path forms them (operands in the input precision), before any cast. */
kda_status kda_intra_chunk(const void *q, const void *k, const void *z,
                           const float *beta, const float *A, float g_min,
                           float *Tm, float *Aqk, float *gamma, int B, int T,
                           int H, int d_k, kda_dtype dt, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
