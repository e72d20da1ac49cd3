/*
 * deltanet.h -- C ABI of the MI355X (gfx950) delta-rule linear-attention library.
 *
 * The operator (DeltaNet, Gated DeltaNet, KDA) keeps one d_k x d_v fp32 state
 * S per (sequence, head) and, for every token t,
 *     S~ = Diag(alpha_t) S          (decay; alpha_t = exp(g_t): one scalar per
 *                                    token for Gated DeltaNet, one per key
 *                                    channel for KDA, 1 for DeltaNet)
 *     u  = beta_t (v_t - S~^T k_t)  (scaled prediction error)
 *     S  = S~ + k_t u^T             (rank-1 write)
 *     o_t = S^T q_t                 (read-out)
 * Pages: "28. Linear attention and Gated DeltaNet" (sections "Gated DeltaNet",
 * "The recurrent form": the tensor contract below), "DeltaNet: Memory That
 * Edits" (section "The delta rule"), "A walk through of the DeltaNet family of
 * linear attention variants" (KDA recurrence, per-key-channel decay).
 *
 * Common conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or synchronises. Work is enqueued on `stream` (a
 *     hipStream_t; NULL = the default stream) and the call returns after
 *     validation and enqueue. Kernel faults surface at the caller's next sync.
 *   - Tensors are contiguous, row-major, in the layouts given per argument.
 *   - `dtype` (DN_F32 or DN_BF16) is the type of q, k, v, beta, g AND o.
 *     States (S0, S_final, S) are always fp32 [B,H,d_k,d_v] with S^T k as the
 *     read (d_k rows = key channels).
 *   - q is used as given: callers that follow the pages' contract pass q and
 *     k L2-normalised per head and q already scaled by d_k^-1/2. beta is not
 *     clamped (values in [0, 2) are valid: the reflection range).
 *   - Supported head sizes: d_k, d_v in {64, 128} with d_k == d_v.
 *   - q, k, v, o and the fp32 states must be 16-byte aligned; beta and g need
 *     only the alignment of their element type. When T == 0 the per-token
 *     tensors (q, k, v, beta, g, o) are not read and may be NULL.
 *   - All argument checks run before any HIP call, so every error return is
 *     synchronous, touches no device state and is testable without a GPU.
 *   - No global mutable state: calls are thread-safe. Calls that share output
 *     buffers or a workspace must be ordered by the caller (same stream).
 */
#ifndef DELTANET_H
#define DELTANET_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dn_status {
    DN_OK = 0,
    DN_EINVAL = -1,     /* a required pointer is NULL or misaligned, B/H < 1, T < 0,
                           an unknown dtype, or more than 2^24 heads / 2^31-1 chunks */
    DN_ENOTSUP = -2,    /* d_k, d_v outside {64, 128} or d_k != d_v, or no such form
                           (see dn_chunk_fwd_fused) */
    DN_EWORKSPACE = -3, /* workspace NULL or smaller than dn_chunk_fwd_workspace() */
    DN_EHIP = -4,       /* the HIP runtime reported an error at launch */
    DN_EHANDOFF = -5,   /* dn_chunk_fwd_handoff_status only: the latest one-launch
                           prefill on the workspace was recomputed (see there) */
    DN_ESCRATCH = -6    /* dn_chunk_fwd_noalloc only: the sizes need more scratch
                           than its built-in array */
} dn_status;

typedef enum dn_dtype { DN_F32 = 0, DN_BF16 = 1 } dn_dtype;

/* Human-readable text for a status code (static storage, never NULL). */
const char* dn_strerror(int status);

/* Library ABI version (incremented on incompatible changes). */
int dn_version(void);

/*
 * Workspace bytes that dn_chunk_fwd, dn_chunk_fwd_fused and dn_kda_chunk_fwd
 * need for these sizes (0 when T == 0; (size_t)0 also for invalid sizes, which
 * the entry points then reject). The workspace holds one block of per-chunk
 * intermediates of the UT/WY form per (head, chunk), then the hand-off words
 * of the one-launch form and a copy of the start state. It needs no
 * initialisation, its contents between calls are unspecified (apart from what
 * dn_chunk_fwd_handoff_status reads), and calls that overlap in time must not
 * share it.
 */
size_t dn_chunk_fwd_workspace(int B, int H, int T, int dk, int dv, int dtype);

/*
 * Chunkwise-parallel prefill (chunk size 64) of DeltaNet (g == NULL) or Gated
 * DeltaNet (g != NULL). Pages: "28. Linear attention and Gated DeltaNet",
 * section "The chunked form: recurrence as matrix multiplication" (the UT
 * system, outputs and end-of-chunk state); "DeltaNet: Memory That Edits",
 * section "Training it: the WY trick".
 *   q, k     [B,H,T,dk]        v [B,H,T,dv]         (dtype)
 *   beta     [B,H,T]           g [B,H,T] log-decay, or NULL => alpha == 1
 *   S0       [B,H,dk,dv] fp32 start state, or NULL => zeros
 *   o        [B,H,T,dv] (dtype) outputs, written for every t < T
 *   S_final  [B,H,dk,dv] fp32, or NULL => not written. S_final == S0 is
 *            allowed (in-place update of a state buffer).
 *   workspace/workspace_bytes: device scratch of at least
 *            dn_chunk_fwd_workspace(B,H,T,dk,dv,dtype) bytes, 256-byte aligned.
 * T == 0 writes S_final = S0 (or zeros) and nothing else. A last chunk shorter
 * than 64 tokens is handled by masking (identical to zero padding).
 * The result equals the token-by-token recurrence up to rounding.
 */
int dn_chunk_fwd(const void* q, const void* k, const void* v, const void* beta,
                 const void* g, const float* S0, void* o, float* S_final,
                 int B, int H, int T, int dk, int dv, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same prefill as dn_chunk_fwd, always as ONE kernel launch in which the
 * chunk-parallel phase and the sequential scan run concurrently: prep
 * workgroups produce the workspace blocks chunk by chunk while scan
 * workgroups on the same XCD consume them (a block is handed over through
 * 64-bit tags in the workspace, see the hand-off notes in chunk.hip). Same
 * arguments, results bitwise equal to dn_chunk_fwd. Returns DN_ENOTSUP where
 * this form does not exist: dtype other than bf16, or more heads than leave
 * room for the prep workgroups (B*H above about 48 per 8 heads' worth of
 * value tiles; dn_chunk_fwd then runs the two phases). dn_chunk_fwd itself
 * uses this form for long sequences, where it is the faster one: from 128
 * chunks (8,192 tokens) with 16 heads or more, from 512 chunks with fewer.
 *
 * The hand-off relies on two measured facts of the hardware, not guaranteed
 * by any API: workgroup b of a launch runs on XCD b mod 8, and workgroups
 * start in index order. Every wait for a block is bounded; a wait that gives
 * up marks the launch as failed in the workspace. The call also enqueues the
 * two phases behind the launch, guarded on the device: they return at once
 * unless that launch failed, in which case they recompute o and S_final
 * (from a copy of S0 taken before the launch, so in-place calls are covered).
 * The results are therefore correct either way; dn_chunk_fwd_handoff_status
 * tells whether the recomputation ran.
 */
int dn_chunk_fwd_fused(const void* q, const void* k, const void* v, const void* beta,
                       const void* g, const float* S0, void* o, float* S_final,
                       int B, int H, int T, int dk, int dv, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * dn_chunk_fwd without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments (minus the workspace), same results as
 * dn_chunk_fwd, which it calls. Its scratch is a 128 MiB device array built
 * into the library, one per GPU the library runs on, held until the process
 * ends (bf16 at d = 128 that covers about 1,700 (head, 64-token chunk) pairs,
 * e.g. 4 x 8 heads of 2,048 tokens); sizes whose dn_chunk_fwd_workspace()
 * exceeds it return DN_ESCRATCH before any HIP call. The call allocates
 * nothing and frees nothing. Every call on one GPU uses that GPU's array and
 * leaves its contents behind (nothing in it needs clearing between calls):
 * calls that overlap in time on one GPU race, so run them on one stream or
 * serialize them.
 */
int dn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* beta,
                         const void* g, const float* S0, void* o, float* S_final,
                         int B, int H, int T, int dk, int dv, int dtype, void* stream);

/*
 * Whether the latest one-launch prefill (dn_chunk_fwd_fused, or dn_chunk_fwd
 * or dn_kda_chunk_fwd taking that form) that used `workspace` with these sizes had a hand-off
 * wait give up: DN_EHANDOFF if so (its results were recomputed by the two
 * phases and are correct), DN_OK if not or if no one-launch call used the
 * workspace. Reads 16 bytes of the workspace after synchronizing `stream`
 * (blocking the host). DN_EINVAL / DN_ENOTSUP / DN_EWORKSPACE as for
 * dn_chunk_fwd; DN_EHIP if the copy fails.
 */
int dn_chunk_fwd_handoff_status(const void* workspace, size_t workspace_bytes, int B, int H, int T,
                                int dk, int dv, int dtype, void* stream);

/*
 * The chunkwise prefill with a chosen chunk length (page "28. Linear attention
 * and Gated DeltaNet", section "Stretch exercises", item 2: the trade between
 * the work inside a chunk and the number of sequential chunk steps). As
 * dn_chunk_fwd in its two-launch form (DeltaNet with g NULL, Gated DeltaNet
 * otherwise) with chunks of `chunk` tokens: 32, 64 (then bitwise equal to
 * dn_chunk_fwd's two launches) or 128. Supported for bf16 only, at
 * dk = dv = 64 (chunk 32 or 64) and 128 (32, 64, 128); DN_ENOTSUP otherwise.
 * The workspace (dn_chunk_fwd_len_workspace bytes, 256-byte aligned, owned by
 * the caller) holds one block per (head, chunk); contents unspecified
 * between calls. Other arguments, layouts and errors as dn_chunk_fwd.
 */
size_t dn_chunk_fwd_len_workspace(int B, int H, int T, int dk, int dv, int dtype, int chunk);
int dn_chunk_fwd_len(const void* q, const void* k, const void* v, const void* beta, const void* g,
                     const float* S0, void* o, float* S_final, int B, int H, int T, int dk, int dv,
                     int dtype, int chunk, void* workspace, size_t workspace_bytes, void* stream);

/*
 * KDA chunkwise prefill: as dn_chunk_fwd but g is REQUIRED and holds one
 * log-decay per key channel, g [B,H,T,dk] (page "A walk through of the
 * DeltaNet family of linear attention variants", KDA section). Uses the same
 * workspace size function. Like dn_chunk_fwd it takes a one-launch form for
 * bf16 where that is the faster one: from 64 chunks (4,096 tokens) with up to
 * 32 heads, past 512 chunks only with 16 heads or more (the prep of a chunk
 * on four wavefronts, then the same hand-off, the same guarded recomputation
 * and the same status query, dn_chunk_fwd_handoff_status); results are
 * bitwise those of the two phases.
 */
int dn_kda_chunk_fwd(const void* q, const void* k, const void* v, const void* beta,
                     const void* g, const float* S0, void* o, float* S_final,
                     int B, int H, int T, int dk, int dv, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Chunkwise prefill that also returns the state at every chunk boundary, for
 * prefix caching: an engine keeps the state after a shared prefix, at block
 * boundaries, instead of per-position entries (page "28. Linear attention and
 * Gated DeltaNet", section "The state a request carries").
 *   kda      0: DeltaNet / Gated DeltaNet exactly as dn_chunk_fwd (g optional,
 *            [B,H,T]); nonzero: KDA exactly as dn_kda_chunk_fwd (g required,
 *            [B,H,T,dk]).
 *   S_chunks [B,H,n,dk,dv] fp32 with n = ceil(T/64), 16-byte aligned: entry c
 *            is the state after the first min(64(c+1), T) tokens, so the last
 *            one equals S_final. Required when T > 0 (else DN_EINVAL).
 * Every other argument, the workspace and the errors are as for dn_chunk_fwd
 * (always the two-phase form). o and S_final are bitwise the same as
 * dn_chunk_fwd's two-phase form gives.
 */
int dn_chunk_fwd_states(int kda, const void* q, const void* k, const void* v,
                        const void* beta, const void* g, const float* S0, void* o,
                        float* S_final, float* S_chunks, int B, int H, int T, int dk,
                        int dv, int dtype, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * The two phases of the chunkwise prefill, for callers that schedule them
 * separately (for example to overlap one request's chunk-parallel phase with
 * another's sequential phase, or to time them). On one stream,
 *     dn_chunk_prep(kda, ...) then dn_chunk_scan(kda, ...)
 * is exactly dn_chunk_fwd (kda = 0) or dn_kda_chunk_fwd (kda = 1).
 *
 * dn_chunk_prep: every 64-token chunk of every head in parallel. Computes the
 *   running log-decay G, the UT transform T = (I + strict_tril(beta K K^T D))^-1,
 *   W = T (beta e^G K), u = T (beta V), the causal decayed Q K^T, the
 *   decay-scaled K and the decay factors of each chunk (page "28. Linear
 *   attention and Gated DeltaNet", section "The chunked form", the triangular
 *   system and the attention matrix), and writes them to `workspace`; for KDA
 *   also the decay-scaled Q. Arguments as in dn_chunk_fwd; with kda = 0,
 *   g == NULL selects DeltaNet.
 * dn_chunk_scan: the sequential inter-chunk recurrence of every head over the
 *   workspace filled by dn_chunk_prep with the same sizes, dtype and kda: per
 *   chunk U = u - W S, O = (e^G * Q) S + attn U, S = e^{G_C} S + K~^T U (same
 *   section, the chunk loop). q is the tensor given to dn_chunk_prep, read
 *   again here (kda = 0). Writes o and S_final exactly as dn_chunk_fwd;
 *   S0/S_final may alias. q and the workspace are read only.
 */
int dn_chunk_prep(int kda, const void* q, const void* k, const void* v, const void* beta,
                  const void* g, int B, int H, int T, int dk, int dv, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

int dn_chunk_scan(int kda, const void* q, const float* S0, void* o, float* S_final, int B, int H,
                  int T, int dk, int dv, int dtype, const void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * Token-by-token recurrent form over T tokens (page "28. Linear attention and
 * Gated DeltaNet", section "The recurrent form"), same arguments and result as
 * dn_chunk_fwd without a workspace. One wavefront per (sequence, head,
 * 64-column slice of the state) carries the state in registers through all T
 * tokens.
 */
int dn_recurrent_fwd(const void* q, const void* k, const void* v, const void* beta,
                     const void* g, const float* S0, void* o, float* S_final,
                     int B, int H, int T, int dk, int dv, int dtype, void* stream);

/* KDA twin of dn_recurrent_fwd: g REQUIRED, [B,H,T,dk]. */
int dn_kda_recurrent_fwd(const void* q, const void* k, const void* v, const void* beta,
                         const void* g, const float* S0, void* o, float* S_final,
                         int B, int H, int T, int dk, int dv, int dtype, void* stream);

/*
 * One decode step for B sequences (one new token each), updating the state in
 * place and returning the read-out. Decay, predict, correct, write and read are
 * fused; every fp32 state element is read once and written once.
 * (Page "28. Linear attention and Gated DeltaNet", section "The recurrent
 * form", one loop iteration; page "A walk through ...", fused recurrent KDA.)
 *   q, k [B,H,dk]   v [B,H,dv]   beta [B,H]   g [B,H] or NULL (DeltaNet)
 *   S    [B,H,dk,dv] fp32, updated in place     o [B,H,dv] (dtype)
 */
int dn_decode_step(const void* q, const void* k, const void* v, const void* beta,
                   const void* g, float* S, void* o,
                   int B, int H, int dk, int dv, int dtype, void* stream);

/* KDA decode step: g REQUIRED, [B,H,dk] (one log-decay per key channel). */
int dn_kda_decode_step(const void* q, const void* k, const void* v, const void* beta,
                       const void* g, float* S, void* o,
                       int B, int H, int dk, int dv, int dtype, void* stream);

/*
 * Several value heads sharing one key head. The gated layer on page "28.
 * Linear attention and Gated DeltaNet" (section "The full layer")
 * has more value heads than key heads and repeats q and k over the head axis
 * (each key head serving Hv/Hk consecutive value heads) before the rule runs;
 * these entry points read the shared q and k in place instead of a repeated
 * copy. Results equal dn_chunk_fwd / dn_kda_chunk_fwd / dn_decode_step /
 * dn_kda_decode_step on the repeated q and k, bitwise.
 *   kda      0: DeltaNet (g NULL) or Gated DeltaNet; nonzero: KDA (g required)
 *   q, k     [B,Hk,T,dk] (prefill) or [B,Hk,dk] (decode)
 *   v, o     [B,Hv,T,dv] or [B,Hv,dv];  beta [B,Hv,T] or [B,Hv]
 *   g        per value head: [B,Hv,T] / [B,Hv] (gated), [B,Hv,T,dk] / [B,Hv,dk] (KDA)
 *   S0, S_final, S: [B,Hv,dk,dv] fp32
 *   Hk >= 1 and Hv a multiple of Hk, else DN_EINVAL. The workspace is
 *   dn_chunk_fwd_workspace(B, Hv, T, dk, dv, dtype). Every other rule is that
 *   of the matching entry point above.
 */
int dn_chunk_fwd_gqa(int kda, const void* q, const void* k, const void* v,
                     const void* beta, const void* g, const float* S0, void* o,
                     float* S_final, int B, int Hk, int Hv, int T, int dk, int dv,
                     int dtype, void* workspace, size_t workspace_bytes, void* stream);
int dn_decode_step_gqa(int kda, const void* q, const void* k, const void* v,
                       const void* beta, const void* g, float* S, void* o, int B,
                       int Hk, int Hv, int dk, int dv, int dtype, void* stream);

/*
 * Chunkwise prefill over N packed sequences of different lengths, as a serving
 * engine batches requests: one call, every sequence its own recurrence (the
 * pages' model of a request: a state per sequence, page "28. Linear attention
 * and Gated DeltaNet", section "The state a request carries").
 *   kda         0: DeltaNet (g NULL) / Gated DeltaNet; nonzero: KDA (g required)
 *   q, k        [1,H,T,dk], v and o [1,H,T,dv], beta [1,H,T], g [1,H,T] or
 *               [1,H,T,dk]: the sequences back to back along T in every head
 *   cu_seqlens  DEVICE array of N + 1 ints: sequence n holds tokens
 *               cu_seqlens[n] .. cu_seqlens[n+1] - 1; expected cu_seqlens[0] = 0,
 *               nondecreasing, cu_seqlens[N] = T (each bound is clamped to
 *               [0, T] and to its predecessor, so no value reads out of bounds;
 *               an empty sequence passes its state through)
 *   S0, S_final [N,H,dk,dv] fp32 (S0 NULL => zeros; S_final NULL => not written)
 *   workspace   at least dn_chunk_fwd_varlen_workspace(N,H,T,dk,dv,dtype) bytes,
 *               256-byte aligned
 * Each sequence's o and S_final are bitwise what dn_chunk_fwd / dn_kda_chunk_fwd
 * (two-phase form) give for that sequence alone. N < 1, a NULL or misaligned
 * cu_seqlens, and more than 2^24 (sequence, head) rows give DN_EINVAL; the
 * other rules are those of dn_chunk_fwd.
 */
size_t dn_chunk_fwd_varlen_workspace(int N, int H, int T, int dk, int dv, int dtype);
int dn_chunk_fwd_varlen(int kda, const void* q, const void* k, const void* v,
                        const void* beta, const void* g, const float* S0, void* o,
                        float* S_final, const int* cu_seqlens, int N, int H, int T, int dk,
                        int dv, int dtype, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Multi-token decode for speculative decoding: K new tokens of every sequence
 * in one call, with the state after each of them kept, so that an engine that
 * accepts only the first j drafted tokens restores snapshot j - 1 instead of
 * recomputing (a recurrent state cannot forget tokens once mixed in: page
 * "28. Linear attention and Gated DeltaNet", section "The state a request
 * carries"). The tokens run through the token-by-token recurrence.
 *   kda      0: DeltaNet (g NULL) or Gated DeltaNet; nonzero: KDA (g required)
 *   q, k     [B,H,K,dk]; v, o [B,H,K,dv]; beta [B,H,K]; g [B,H,K] or [B,H,K,dk]
 *   S        [B,H,dk,dv] fp32, updated in place to the state after all K tokens
 *   S_snap   [B,H,K,dk,dv] fp32 (16-byte aligned) or NULL: entry j is the state
 *            after token j (the last equals the updated S)
 * K >= 1. o and S are bitwise those of dn_recurrent_fwd / dn_kda_recurrent_fwd
 * over the K tokens from S; errors as for dn_decode_step.
 */
int dn_decode_tokens(int kda, const void* q, const void* k, const void* v,
                     const void* beta, const void* g, float* S, void* o, float* S_snap,
                     int B, int H, int K, int dk, int dv, int dtype, void* stream);

/*
 * The gated layer's work before the rule (page "28. Linear attention and
 * Gated DeltaNet", section "The full layer", steps 2 to 5), in one pass over
 * the projected rows: depthwise causal convolution of width 4 over time with
 * carried history, SiLU, split into key and value heads, L2 normalisation of
 * q and k (q then scaled by dk^-1/2), and the gates beta = sigmoid(b),
 * g = -exp(A_log) * softplus(a + dt_bias). The outputs are exactly the
 * head-major q, k, v, beta, g that dn_chunk_fwd_gqa / dn_decode_step_gqa take.
 *   qkv         [B,T,C] (dtype), C = 2*Hk*dk + Hv*dv: per token, the q channels
 *               of key heads 0..Hk-1, then k, then v of value heads 0..Hv-1
 *   conv_w      [C,4] (dtype) filter taps per channel, tap 3 multiplies the
 *               current token, tap 0 the token three steps back
 *   conv_state  [B,C,3] (dtype) the three inputs before token 0, oldest first,
 *               or NULL => zeros
 *   conv_state_out [B,C,3] (dtype) or NULL => not written: the last three
 *               inputs of (conv_state, qkv) per channel. May equal conv_state
 *               (in-place update; it is written after every read of it); any
 *               other overlap with an input is not allowed.
 *   b, a        [B,T,Hv] (dtype) gate inputs; a is read only when g != NULL
 *   A_log, dt_bias [Hv] fp32 (read only when g != NULL)
 *   q, k        [B,Hk,T,dk] (dtype) out;  v [B,Hv,T,dv] (dtype) out
 *   beta        [B,Hv,T] (dtype) out;     g [B,Hv,T] (dtype) out, or NULL for a
 *               layer without decay (DeltaNet): then a, A_log, dt_bias unused
 *   allow_neg_eigval  nonzero: beta = 2 sigmoid(b) in (0, 2), so the transition
 *               I - beta k k^T may have the negative eigenvalue 1 - beta along k
 *               (page "DeltaNet: Memory That Edits", section "The reflection
 *               hiding in the delta rule"); the rule's kernels never clamp beta
 * Arithmetic is fp32 from the stored inputs, rounded once to dtype at each
 * output. A norm below 1e-12 divides by 1e-12. dk == dv in {64, 128}
 * (DN_ENOTSUP otherwise); Hk, Hv >= 1 with Hv a multiple of Hk, B <= 65535 and
 * 2*Hk + Hv <= 65535 (DN_EINVAL otherwise). qkv, conv_w, the conv states, q, k,
 * v must be 16-byte aligned; b, a, beta, g element-aligned. T == 0 writes only
 * conv_state_out (a copy of conv_state, or zeros); the per-token tensors may be
 * NULL then.
 */
int dn_layer_prologue(const void* qkv, const void* conv_w, const void* conv_state,
                      void* conv_state_out, const void* b, const void* a, const float* A_log,
                      const float* dt_bias, void* q, void* k, void* v, void* beta, void* g,
                      int allow_neg_eigval, int B, int T, int Hk, int Hv, int dk, int dv,
                      int dtype, void* stream);

/*
 * The gated layer's work after the rule (same page and section, step 7):
 * gated RMSNorm of every value head's read-out, written token-major for the
 * output projection,
 *   out[b,t,h*dv + c] = w[c] * n[b,h,t,c] * SiLU(z[b,t,h*dv + c]),
 *   n = o / sqrt(mean_c(o^2) + eps) rounded to dtype (as the page rounds the
 *   normalised value to the activation type before the products).
 *   o      [B,Hv,T,dv] (dtype) the rule's read-out (o of dn_chunk_fwd_gqa)
 *   z      [B,T,Hv*dv] (dtype) the output gate
 *   norm_w [dv] (dtype) the weight vector, shared by all heads
 *   out    [B,T,Hv*dv] (dtype), must not overlap o or z
 * eps >= 0 and finite (the page uses 1e-6). dv in {64, 128} (DN_ENOTSUP
 * otherwise); all four pointers 16-byte aligned; T == 0 does nothing.
 */
int dn_layer_epilogue(const void* o, const void* z, const void* norm_w, void* out, int B, int Hv,
                      int T, int dv, float eps, int dtype, void* stream);

/*
 * The gated layer between its projections for a prefill of T tokens (page "28.
 * Linear attention and Gated DeltaNet", section "The full layer", steps 2-7):
 * the work of dn_layer_prologue, dn_chunk_fwd_gqa and dn_layer_epilogue in
 * order, with the prologue formed inside the prefill's chunk-parallel phase
 * (its load stage) instead of written to memory and read back. Three launches:
 * that phase, the sequential scan, the gated RMSNorm.
 *   qkv, b, a, conv_w, conv_state, conv_state_out, A_log, dt_bias, allow_neg_eigval
 *               as in dn_layer_prologue; a == NULL selects no decay gate. Here
 *               conv_state_out must not overlap conv_state at all (DN_EINVAL),
 *               or may be NULL (not written)
 *   z, norm_w, eps, out  as in dn_layer_epilogue
 *   S0          [B,Hv,d,d] fp32 start state or NULL (zeros); S_final [B,Hv,d,d]
 *               fp32 end state (may be S0)
 *   workspace   at least dn_layer_prefill_workspace(B,T,Hk,Hv,d,dtype) bytes,
 *               256-byte aligned (DN_EWORKSPACE otherwise); it holds the chunk
 *               blocks, the normalised q rows and the read-out
 * The results are bitwise those of the three separate calls (dn_chunk_fwd_gqa
 * in its two-launch form, which its one-launch form equals). bf16 with
 * d = dk = dv = 128 only (DN_ENOTSUP otherwise: the three calls cover the
 * rest); Hv a multiple of Hk; T == 0 only passes the history through and
 * copies the state. Alignment: qkv, conv_w, the conv states, z, norm_w, out,
 * S0, S_final 16 bytes; b, a element; A_log, dt_bias 4 bytes.
 */
size_t dn_layer_prefill_workspace(int B, int T, int Hk, int Hv, int d, int dtype);
int dn_layer_prefill(const void* qkv, const void* conv_w, const void* conv_state, void* conv_state_out,
                     const void* b, const void* a, const float* A_log, const float* dt_bias, const void* z,
                     const void* norm_w, float eps, const float* S0, float* S_final, void* out,
                     int allow_neg_eigval, int B, int T, int Hk, int Hv, int d, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * The whole gated layer between its projections for ONE token per sequence
 * (decode), in a single kernel (page "28. Linear attention and Gated
 * DeltaNet", section "The full layer", steps 2-7, around the recurrent step
 * of section "The recurrent form"): exactly the work of dn_layer_prologue
 * (T = 1), dn_decode_step_gqa and dn_layer_epilogue in order, with q, k, v,
 * beta, g and o kept on chip. One workgroup per (sequence, value head).
 *   qkv, b, a, conv_w, conv_state, conv_state_out, A_log, dt_bias, allow_neg_eigval
 *               as in dn_layer_prologue with T = 1 (qkv [B,1,C], b and a
 *               [B,1,Hv]); a == NULL selects no decay gate (DeltaNet; A_log
 *               and dt_bias unused)
 *   z, norm_w, eps, out  as in dn_layer_epilogue with T = 1 (z, out [B,1,Hv*d])
 *   S           [B,Hv,d,d] fp32, the recurrent state, updated in place
 * d = dk = dv in {64, 128} (DN_ENOTSUP otherwise); Hv a multiple of Hk. The
 * intermediate values are those of the three separate calls: q, k, v, beta
 * and g rounded to dtype, and o rounded to dtype before its norm (the
 * reductions may add in another order: the results agree to rounding, not
 * bit for bit). conv_state_out may be conv_state itself only when Hk == Hv
 * (with shared key heads other workgroups still read a key head's history);
 * any other overlap between the two is DN_EINVAL. The state must not overlap
 * any other argument. Alignment: qkv, conv_w, the conv states, z, norm_w, S,
 * out 16 bytes; b, a element; A_log, dt_bias 4 bytes.
 */
int dn_layer_decode_step(const void* qkv, const void* conv_w, const void* conv_state,
                         void* conv_state_out, const void* b, const void* a, const float* A_log,
                         const float* dt_bias, const void* z, const void* norm_w, float eps, float* S,
                         void* out, int allow_neg_eigval, int B, int Hk, int Hv, int d, int dtype,
                         void* stream);

/*
 * Selective state-space recurrence (decayed linear attention, the form behind
 * RetNet, GLA and Mamba-2): S_t = alpha_t S_{t-1} + k_t v_t^T, o_t = S_t^T q_t,
 * alpha_t = exp(g_t) with one log-decay per head and token. This is Gated
 * DeltaNet with the correction term removed (page "28. Linear attention and
 * Gated DeltaNet", sections "Forget: decay" and "Stretch exercises", item 4),
 * and it runs on the same chunk machinery with the UT solve reduced to the
 * identity. There is no beta. Arguments as for dn_chunk_fwd / dn_recurrent_fwd
 * / dn_decode_step without beta, and g is REQUIRED (pass zeros for plain
 * causal linear attention). The chunked form uses dn_chunk_fwd_workspace()
 * bytes. Each returns DN_EINVAL when g is NULL.
 */
int dn_ssm_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                     const float* S0, void* o, float* S_final, int B, int H, int T, int dk, int dv,
                     int dtype, void* workspace, size_t workspace_bytes, void* stream);
int dn_ssm_recurrent_fwd(const void* q, const void* k, const void* v, const void* g,
                         const float* S0, void* o, float* S_final, int B, int H, int T, int dk,
                         int dv, int dtype, void* stream);
int dn_ssm_decode_step(const void* q, const void* k, const void* v, const void* g, float* S,
                       void* o, int B, int H, int dk, int dv, int dtype, void* stream);

/*
 * The generalized delta rule (page "DeltaNet: Memory That Edits", section "The
 * generalized delta rule"): the roles the delta rule ties together are
 * separated,
 *     S_t = (diag(w_t) - (a_t * kr_t) kr_t^T) S_{t-1} + kw_t v_t^T,  o_t = S_t^T q_t,
 * with w_t = exp(g_t) a per-key-channel decay, kr_t the removal key, kw_t the
 * write key and a_t a per-key-channel removal rate: a diagonal-plus-low-rank
 * key-space transition (page "A walk through of the DeltaNet family of linear
 * attention variants"). kr = k, kw = beta k, a = beta, g = 0 is DeltaNet; the
 * removal term uses the state before the decay, as the transition is written.
 * Token by token (one wavefront per head and 64 value columns); a single
 * token (T == 1, and the decode step) streams each state once instead. The
 * chunked form is dn_gdr_chunk_fwd below.
 *   q, kw, kr, a, g  [B,H,T,dk] (dtype);  v, o  [B,H,T,dv] (dtype)
 *   S0, S_final      [B,H,dk,dv] fp32 (S0 NULL => zeros; S_final NULL => not
 *                    written; S_final == S0 allowed)
 * dn_gdr_decode_step is one token ([B,H,dk] / [B,H,dv] inputs) with S updated
 * in place. dk == dv in {64, 128}. v, o and the states must be 16-byte
 * aligned; q, kw, kr, a, g only element-aligned. Errors as for
 * dn_recurrent_fwd.
 */
int dn_gdr_recurrent_fwd(const void* q, const void* kw, const void* v, const void* kr,
                         const void* a, const void* g, const float* S0, void* o, float* S_final,
                         int B, int H, int T, int dk, int dv, int dtype, void* stream);
int dn_gdr_decode_step(const void* q, const void* kw, const void* v, const void* kr,
                       const void* a, const void* g, float* S, void* o, int B, int H, int dk,
                       int dv, int dtype, void* stream);

/*
 * Chunked form of the generalized delta rule (derived here; the pages give
 * none): every chunk of `chunk` tokens (16, 32 or 64; DN_ENOTSUP otherwise)
 * is reduced to an affine map S <- P S + Sh with
 * read-outs O = Qp S + Oh, where the chunk's removal read-outs solve a unit
 * lower-triangular system whose entries carry the per-channel decay inside
 * their contraction (all exponents <= 0); the maps are then applied chunk
 * after chunk. Arithmetic is fp32 throughout. Same tensors and rules as
 * dn_gdr_recurrent_fwd, except that q, kw, kr, a and g are read as vectors of
 * four elements and must be aligned to 8 bytes (bf16) or 16 bytes (fp32)
 * (DN_EINVAL otherwise), plus a workspace of at least
 * dn_gdr_chunk_workspace(B,H,T,dk,dv,dtype,chunk) bytes (256-byte aligned;
 * 496 KiB per (head, 64-token chunk) at d = 128; contents unspecified between
 * calls; DN_EWORKSPACE if missing or short). The chunk length trades the
 * per-chunk triangular work (quadratic in the length) against the number of
 * sequential chunk steps; the result equals the token-by-token form up to
 * rounding for every length.
 */
size_t dn_gdr_chunk_workspace(int B, int H, int T, int dk, int dv, int dtype, int chunk);
int dn_gdr_chunk_fwd(const void* q, const void* kw, const void* v, const void* kr, const void* a,
                     const void* g, const float* S0, void* o, float* S_final, int B, int H, int T,
                     int dk, int dv, int dtype, int chunk, void* workspace,
                     size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DELTANET_H */
