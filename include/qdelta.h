/*
 * qdelta.h -- C ABI of the MI355X (gfx950) Q-Delta layer library, libqdelta.so.
 *
 * The library computes the forward pass of the gated Q-Delta linear-attention
 * layer, defined per (batch b, head h) on the Q-Delta reading notes page
 * ("Q-Delta: Beyond Key-Value Associative State Evolution"), §2.4, boxed gated
 * update and read-out:
 *
 *     x_t = k_t + lambda_t q_t
 *     S_t = alpha_t S_{t-1} (I - beta_t x_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 *
 * with the state S in R^{d_v x d_k} (§2.1 symbol table).  lambda == 0 gives
 * Gated DeltaNet and lambda == 0, alpha == 1 gives DeltaNet (same section).
 *
 * Memory layouts (all row-major, contiguous, device memory):
 *     q, k      [B][T][H][d_k]   element type per qd_dtype
 *     v, o      [B][T][H][d_v]   element type per qd_dtype
 *     alpha, beta, lambda  [B][T][H]  fp32
 *     S0, S_T   [B][H][d_v][d_k] fp32  (row = value index, column = key index)
 * For the decode step the token axis is absent: q, k [N][H][d_k], v, o
 * [N][H][d_v], gates [N][H], S [N][H][d_v][d_k].
 *
 * Ownership and execution: the caller owns every buffer.  All pointers except
 * `stream` are device pointers.  The library allocates no device memory and
 * enqueues its kernels asynchronously on `stream` (a hipStream_t; NULL means the
 * default stream); nothing synchronises.  Buffers must stay valid until the work on
 * `stream` completes.  Process-wide state: a host-side cache, per device, of the
 * compute-unit count and of the backward gradient kernels' occupancy (each entry filled
 * once, on the first call on that device, with atomic stores, so calls from several
 * host threads are safe); and the device scratch array of qdelta_chunk_fwd_noalloc
 * (see there), the only entry point that uses it.
 *
 * Errors: arguments are checked on the host before anything is enqueued; a
 * failed check returns a status and enqueues nothing.  A launch failure returns
 * QD_ERR_HIP.  Device data are not inspected: NaN/Inf propagate, and alpha <= 0
 * is outside the domain (the kernels take log(alpha)).
 */
#ifndef QDELTA_H_
#define QDELTA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QDELTA_ABI_VERSION 6

typedef enum qd_status {
    QD_OK = 0,
    QD_ERR_INVALID_ARG = 1,   /* null required pointer, negative size, aliasing not allowed */
    QD_ERR_UNSUPPORTED = 2,   /* d_k, d_v, C or dtype outside the supported set            */
    QD_ERR_WORKSPACE = 3,     /* workspace smaller than qdelta_chunk_fwd_workspace_bytes    */
    QD_ERR_HIP = 4,           /* the HIP runtime reported an error at launch                */
    QD_ERR_SCRATCH_LIMIT = 5  /* qdelta_chunk_fwd_noalloc: sizes need more than its scratch */
} qd_status;

typedef enum qd_dtype {
    QD_F32 = 0,               /* q, k, v, o are fp32                                        */
    QD_BF16 = 1               /* q, k, v, o are bf16 (round-to-nearest-even outputs)        */
} qd_dtype;

/* Version of this ABI (QDELTA_ABI_VERSION of the header the library was built with). */
int qdelta_abi_version(void);

/* Static description of a status code; never NULL. */
const char *qdelta_status_string(int status);

/* Bytes of device workspace qdelta_chunk_fwd needs for these sizes, on the current
 * device.  0 for the single-pass schedule, which keeps every chunk intermediate on
 * chip.  Non-zero when the sequence is long and B*H*d_v/64 workgroups would leave
 * most compute units idle (bf16, C = 32 or 64): the forward then cuts the sequence
 * into P segments and composes their affine state maps (S_out = S_in M + G, from the
 * recurrence of the Q-Delta reading notes §2.4 acting on the state from the right).
 * The size is B*P*H*(d_k*d_k + 2*d_v*d_k)*4 bytes, P in {2, 4, 8, 16}.  For a single
 * sequence (B = 1) the first segment, which starts from S0 itself, is walked with its
 * output beside the other segments' maps and needs no map; that schedule uses part of
 * the same buffer.  Callers pass a caller-owned, 16-byte aligned device buffer of at
 * least this size. */
size_t qdelta_chunk_fwd_workspace_bytes(int B, int T, int H, int d_k, int d_v, int C,
                                        int dtype);

/*
 * Layer forward in the chunkwise-parallel WY/UT-transform form (Q-Delta reading
 * notes §2.6: the strictly-lower X K^T interaction, the triangular-solve UT
 * transform, and the entry-state composition of Z, S_out and O).  The result is
 * the recurrence above evaluated over T tokens from S0; C and the schedule (single
 * pass or segmented, see qdelta_chunk_fwd_workspace_bytes) only change rounding.
 *
 *   q, k, v, beta   required when B*T*H > 0.
 *   alpha           NULL means alpha == 1 (selects the no-decay instance).
 *   lambda          NULL means lambda == 0 (selects the Gated DeltaNet instance).
 *   S0              NULL means a zero initial state.
 *   o               required when B*T*H > 0.
 *   S_T             NULL means the final state is not written.  S_T may equal S0
 *                   (in-place state update); no other aliasing is allowed.
 *   B, H, T >= 0 (T == 0 writes S_T = S0, or zeros); d_k, d_v in {64, 128};
 *   C in {16, 32, 64} (chunk length; a short last chunk is handled exactly);
 *   dtype one of qd_dtype.
 *   workspace/ws_bytes: see qdelta_chunk_fwd_workspace_bytes (may be NULL/0
 *                   when that returns 0; otherwise QD_ERR_WORKSPACE if it is NULL
 *                   or smaller).  It must not overlap any other argument, and the
 *                   library overwrites it; its contents are not needed afterwards.
 */
int qdelta_chunk_fwd(const void *q, const void *k, const void *v,
                     const float *alpha, const float *beta, const float *lambda,
                     const float *S0, void *o, float *S_T,
                     int B, int T, int H, int d_k, int d_v, int C, int dtype,
                     void *workspace, size_t ws_bytes, void *stream);

/*
 * One recurrent decode step (Q-Delta reading notes §2.4: the boxed update for a
 * single token, with the read-out expanded as
 * o_t = alpha S_{t-1} q + beta (v - alpha S_{t-1} x)(k^T q)), for N independent
 * sequences x H heads.  S is read and overwritten in place.
 *
 *   q, k, v, beta, S, o   required when N*H > 0.
 *   alpha NULL means 1, lambda NULL means 0.
 *   N, H >= 0; d_k, d_v in {64, 128}; dtype one of qd_dtype.
 */
int qdelta_step(const void *q, const void *k, const void *v,
                const float *alpha, const float *beta, const float *lambda,
                float *S, void *o, int N, int H, int d_k, int d_v, int dtype,
                void *stream);

/*
 * qdelta_chunk_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Arguments, results,
 * layouts, aliasing rules and status codes are those of qdelta_chunk_fwd, without the
 * workspace: where the sizes call for the segmented schedule (qdelta_chunk_fwd_workspace_bytes
 * non-zero), its workspace is a scratch array of QDELTA_NOALLOC_SCRATCH_BYTES that the library
 * holds on every device it runs on until the process ends, set up on the first call on that
 * device.  The call itself allocates nothing.
 *   - Sizes whose workspace would exceed QDELTA_NOALLOC_SCRATCH_BYTES return
 *     QD_ERR_SCRATCH_LIMIT and enqueue nothing (B = 1, T = 65536, H = 16, d = 128 needs 25.2 MB).
 *   - Every call on a GPU uses that GPU's one scratch array: calls that may overlap in time
 *     on one device (different streams, different host threads without ordering) race and
 *     give wrong results; calls ordered on one stream are safe.
 *   - QD_ERR_HIP if the scratch's device address cannot be obtained.
 */
#define QDELTA_NOALLOC_SCRATCH_BYTES (32u << 20)
int qdelta_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                             const float *alpha, const float *beta, const float *lambda,
                             const float *S0, void *o, float *S_T,
                             int B, int T, int H, int d_k, int d_v, int C, int dtype,
                             void *stream);

/*
 * The same two calls with the layer's prologue fused in (the layer of the Q-Delta
 * reading notes §1, trained as in §3.1, feeds the recurrence unit-norm q and k and
 * gates mapped into their ranges).  Arguments, layouts, workspace, aliasing and
 * status codes are those of qdelta_chunk_fwd and qdelta_step, except:
 *
 *   q, k            unnormalised; each (token, head) vector is divided by
 *                   sqrt(|x|^2 + 1e-6) before use (a zero vector stays zero);
 *   alpha_logit     a, alpha = exp(-softplus(a)) = 1 / (1 + exp(a)); NULL means alpha = 1;
 *   beta_logit      b, beta = 1 / (1 + exp(-b)); required;
 *   lambda_logit    l, lambda = 1 / (1 + exp(-l)); NULL means lambda = 0.
 *
 * This replaces a separate pass that would read and rewrite q and k in HBM.
 * qdelta_chunk_fwd_raw supports bf16 with C in {32, 64} (QD_ERR_UNSUPPORTED
 * otherwise); qdelta_step_raw supports every qdelta_step configuration.
 */
int qdelta_chunk_fwd_raw(const void *q, const void *k, const void *v,
                         const float *alpha_logit, const float *beta_logit,
                         const float *lambda_logit, const float *S0, void *o, float *S_T,
                         int B, int T, int H, int d_k, int d_v, int C, int dtype,
                         void *workspace, size_t ws_bytes, void *stream);
int qdelta_step_raw(const void *q, const void *k, const void *v,
                    const float *alpha_logit, const float *beta_logit,
                    const float *lambda_logit, float *S, void *o, int N, int H,
                    int d_k, int d_v, int dtype, void *stream);

/* Bytes of device workspace qdelta_chunk_bwd needs: the entry state of every chunk and
 * the gradient with respect to every chunk's exit state, kept in the input element
 * type (the kernels feed them to the matrix cores in that type):
 * 2*B*H*ceil(T/C)*d_v*d_k*(2 for bf16, 4 for fp32) bytes; 0 when B*H*T == 0 or the
 * sizes are unsupported. */
size_t qdelta_chunk_bwd_workspace_bytes(int B, int T, int H, int d_k, int d_v, int C,
                                        int dtype);

/*
 * Layer backward: the gradients of the scalar sum(o * d_o) + sum(S_T * dS_T) with
 * respect to every input of qdelta_chunk_fwd, o and S_T being that call's results for
 * the same inputs.  The pages give the forward only (Q-Delta reading notes §2.4, the
 * gated update, and §2.6, the chunkwise form); this is its reverse-mode derivative,
 * evaluated in the chunk form in three passes: the forward again, keeping each chunk's
 * entry state; a reverse scan over the chunks for the state gradients and dv; and a
 * parallel pass over the chunks for dq, dk, dalpha, dbeta, dlambda.  C only changes
 * rounding.
 *
 *   q, k, v, alpha, beta, lambda, S0, C, dtype   as for qdelta_chunk_fwd.
 *   d_o       [B][T][H][d_v], dtype elements; required when B*T*H > 0.
 *   dS_T      [B][H][d_v][d_k] fp32, or NULL (zero).
 *   dq, dk    [B][T][H][d_k], dv [B][T][H][d_v], dtype elements; required.
 *   dbeta     [B][T][H] fp32; required.
 *   dalpha    [B][T][H] fp32 or NULL (not written); must be NULL when alpha is NULL.
 *   dlambda   [B][T][H] fp32 or NULL (not written); must be NULL when lambda is NULL.
 *   dS0       [B][H][d_v][d_k] fp32 or NULL (not written).
 *   workspace at least qdelta_chunk_bwd_workspace_bytes, 16-byte aligned; its contents
 *             are overwritten and not needed afterwards.
 *   Supported: d_k, d_v in {64, 128}; C in {16, 32, 64} for bf16 and {16, 32} for fp32.
 *   Every output and the workspace must be disjoint from every input and from one
 *   another (QD_ERR_INVALID_ARG otherwise).
 */
int qdelta_chunk_bwd(const void *q, const void *k, const void *v,
                     const float *alpha, const float *beta, const float *lambda,
                     const float *S0, const void *d_o, const float *dS_T,
                     void *dq, void *dk, void *dv, float *dalpha, float *dbeta,
                     float *dlambda, float *dS0,
                     int B, int T, int H, int d_k, int d_v, int C, int dtype,
                     void *workspace, size_t ws_bytes, void *stream);

/*
 * QED / GDN-2 layer (page "The Query Knows What to Forget", reading notes, §2.1 GDN-2
 * update and §2.2 the boxed QED update), in this header's d_v x d_k state convention
 * (the notes' K x V state transposed; their S^T x is S x here).  Per (b, h), per token:
 *
 *     S_bar = S_{t-1} Diag(exp g_t)                   (per key channel decay)
 *     a_t   = b_t . k_t + lambda_h (u_t - k_t (k_t . u_t)),   u_t = b_t . q_t
 *     S_t   = S_bar + (w_t . v_t - S_bar a_t) k_t^T,   o_t = S_t q_t
 *
 * lambda_h = 0 is GDN-2.  q, k, v, o, S0, S_T, dtype, B, T, H, d_k, d_v, stream as for
 * qdelta_chunk_fwd; additionally (all fp32, device, 16-byte aligned where a row is):
 *   g         [B][T][H][d_k] log decay (<= 0 in the layer; the chunk kernel needs
 *             exp(-(sum of any 8 consecutive g)) within the fp32 range, i.e. per-token
 *             log decays above about -11)
 *   b         [B][T][H][d_k] erase gate
 *   w         [B][T][H][d_v] write gate
 *   lambda_h  [H] strength of the query-derived direction per head.
 * q and k are expected L2-normalised (the projection uses |k| = 1).  C is the chunk
 * length: 16 or 32 for bf16, 16 for fp32 (QD_ERR_UNSUPPORTED otherwise); it changes
 * rounding only.  S_T may equal S0; o must not overlap any input.  No workspace.
 */
int qdelta_qed_chunk_fwd(const void *q, const void *k, const void *v,
                         const float *g, const float *b, const float *w, const float *lambda_h,
                         const float *S0, void *o, float *S_T,
                         int B, int T, int H, int d_k, int d_v, int C, int dtype, void *stream);

/* One QED / GDN-2 decode step for N sequences x H heads (the same update for a single
 * token): q, k [N][H][d_k], v, o [N][H][d_v], g, b [N][H][d_k], w [N][H][d_v],
 * lambda_h [H]; S [N][H][d_v][d_k] fp32 updated in place.  d_k, d_v in {64, 128}. */
int qdelta_qed_step(const void *q, const void *k, const void *v,
                    const float *g, const float *b, const float *w, const float *lambda_h,
                    float *S, void *o, int N, int H, int d_k, int d_v, int dtype, void *stream);

/*
 * Erase-then-Delta (page "Erase-then-Delta Attention" explainer, core method, its
 * two-step pseudo-code), in this header's d_v x d_k convention (the page's K x V memory
 * transposed).  Per (b, h), per token, with a unit erase direction e:
 *
 *     S <- S - (S e) e^T ;   S <- S + (v - S k) k^T ;   o_t = S q
 *
 * (no beta and no decay, as the page writes it).  q, k, e [B][T][H][d_k] and v, o
 * [B][T][H][d_v] in the dtype's elements; S0, S_T, C, dtype and the other sizes as for
 * qdelta_chunk_fwd.  The erase is a delta step with key e, value 0 and beta 1, so the
 * chunked form is DeltaNet over the interleaved sequence e_1, k_1, e_2, k_2, ... read at
 * the k tokens.  In bf16 at C = 32 or 64 the kernel reads that sequence in place and
 * needs no workspace (the size query returns 0; workspace may be NULL).  Otherwise the
 * call writes the sequence into the workspace, runs the chunk forward over it and
 * gathers o; workspace: at least qdelta_eda_chunk_fwd_workspace_bytes
 * (2*B*T*H*((2 d_k + 2 d_v) e + 4) bytes, e = element size), 16-byte aligned, disjoint
 * from every other argument; QD_ERR_WORKSPACE otherwise.
 */
size_t qdelta_eda_chunk_fwd_workspace_bytes(int B, int T, int H, int d_k, int d_v, int C,
                                            int dtype);
int qdelta_eda_chunk_fwd(const void *q, const void *k, const void *v, const void *e,
                         const float *S0, void *o, float *S_T,
                         int B, int T, int H, int d_k, int d_v, int C, int dtype,
                         void *workspace, size_t ws_bytes, void *stream);

/* One Erase-then-Delta decode step for N sequences x H heads: q, k, e [N][H][d_k], v, o
 * [N][H][d_v]; S [N][H][d_v][d_k] fp32 updated in place.  d_k, d_v in {64, 128}. */
int qdelta_eda_step(const void *q, const void *k, const void *v, const void *e, float *S,
                    void *o, int N, int H, int d_k, int d_v, int dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QDELTA_H_ */
