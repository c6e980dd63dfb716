/*
 * lightning_la.h -- C ABI of the Lightning Attention layer for AMD Instinct
 * MI355X (gfx950).
 *
 * The operation.  Lightning Attention is the linear-attention half of the 7:1
 * Lightning-Attention / MLA hybrid described in the Ling & Ring 2.6 Technical
 * Report ("Hybrid Linear Attention: Balancing Long-Context Efficiency and Model
 * Quality": sequence cost O(n) instead of O(n^2), for training and decoding;
 * "Long-Context Training: Context Parallel for Lightning Attention": a
 * recursive hidden state along the sequence).  Per batch row b and head h,
 * with decay lambda_h = exp(-slope[h]):
 *
 *     S_t = lambda_h S_{t-1} + k_t v_t^T          (S_{-1} = state_in, d x d)
 *     o_t = q_t^T S_t                              (o_t[j] = sum_i q_t[i] S_t[i][j])
 *
 * i.e. o_t = sum_{s<=t} lambda^(t-s) (q_t . k_s) v_s + lambda^(t+1) q_t^T S_{-1}.
 * The current token is included with weight lambda^0 = 1.  No softmax, no
 * normalisation, no feature map and no extra 1/sqrt(d) scale are applied.
 *
 * Layouts (row-major, contiguous, no strides):
 *   token tensors q, k, v, o, dout, dq, dk, dv : [B][H][N][d]
 *   state tensors                               : [B][H][d][d] fp32, S[i][j] with
 *                                                 i the key feature, j the value feature
 *   slope                                       : [H] fp32
 *
 * Ownership and threading.  Every pointer argument (except the status
 * strings and the host array cu_seqlens of the packed-batch calls) is a
 * DEVICE pointer owned by the caller.  The library allocates no
 * device memory and keeps no pointer after a call returns; its only mutable
 * global state is the static scratch buffer of la_prefill_noalloc (one per
 * GPU) and the table of its per-device addresses.  Work is enqueued on `stream` (a hipStream_t passed as void*;
 * NULL is the null stream) and the call returns without synchronising.  Calls
 * on different streams that write the same buffers race.
 *
 * Errors.  Arguments are validated before any HIP call; a failed check returns
 * its code and enqueues nothing.  A launch failure returns LA_ERR_HIP.  No C++
 * exception crosses this boundary.
 */
#ifndef LIGHTNING_LA_H
#define LIGHTNING_LA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_ABI_VERSION 4

typedef enum {
  LA_OK = 0,
  LA_ERR_NULL_POINTER = 1, /* a required pointer is NULL                       */
  LA_ERR_BAD_SHAPE = 2,    /* B, H, N < 1, or d / C outside the supported set  */
  LA_ERR_BAD_DTYPE = 3,    /* dtype is not LA_F32 or LA_BF16                   */
  LA_ERR_UNSUPPORTED = 4,  /* valid request this version does not implement    */
  LA_ERR_WORKSPACE = 5,    /* workspace missing or smaller than required       */
  LA_ERR_HIP = 6,          /* a HIP launch or runtime call failed              */
  LA_ERR_ALIGNMENT = 7,    /* a pointer is not 16-byte aligned                 */
  LA_ERR_ALIAS = 8         /* an output aliases an input it must not alias     */
} la_status_t;

typedef enum {
  LA_F32 = 0,  /* fp32 token tensors, fp32 arithmetic                           */
  LA_BF16 = 1  /* bf16 token tensors, fp32 accumulation and fp32 state;
                  bf16 outputs are rounded to nearest-even from fp32            */
} la_dtype_t;

/* ------------------------------------------------------------------------ *
 * la_prefill -- chunked forward over N tokens.
 *
 * Computes o for every token and, if state_out != NULL, the state after the
 * last token.  The sequence is processed in chunks of C tokens: within a
 * chunk the masked scores (Q K^T weighted by lambda^(i-j), j <= i) multiply V,
 * and the chunk reads the d x d state carried from the previous chunks (the
 * evaluation order described on the "Context Parallel for Lightning
 * Attention" section: a local recursion, unfolded into matrix form, plus the
 * carried state).  C changes only the rounding, never the result.  LA_F32
 * rows of at most 256 tokens are evaluated as one masked product over the
 * whole row (the same sum, with no chunk recursion), except an in-place
 * continuation, which runs chunked.
 *
 *   dt        LA_F32 or LA_BF16 (type of q, k, v, o)
 *   B, H, N   >= 1;  d in {64, 128} (LA_F32 also allows 16 and 32)
 *   C         chunk length, one of {16, 32, 64, 128}; N need not be a
 *             multiple of C.  The bf16 kernels run chunks of 32, 64 or 128
 *             tokens: an LA_BF16 request for C = 16 runs in 32-token chunks,
 *             which changes only the rounding.  B*H*N above 2^30, or B*H
 *             above 2^19, gives LA_ERR_UNSUPPORTED, and so does a segment
 *             plan whose pieces would need more than 2^32 work-items (one
 *             workgroup of 2 d threads per piece: only at N near 2^30 with
 *             segments of a prime number of chunks, whose pieces are one
 *             chunk long).
 *   q, k, v   [B][H][N][d] of dt, 16-byte aligned
 *   slope     [H] fp32, the decay is exp(-slope[h]); any finite slope >= 0
 *   state_in  [B][H][d][d] fp32, or NULL for a zero initial state
 *   o         [B][H][N][d] of dt, written; must not overlap q, k or v
 *   state_out [B][H][d][d] fp32 or NULL; may equal state_in (continuation
 *             in place) but must not partially overlap it.  In place is
 *             safe for any plan: when a row is split into segments, the
 *             pre-pass copies its state_in into the workspace and the first
 *             segment reads that copy.
 *   workspace device scratch of at least la_workspace_bytes(0, ...) bytes
 *             (may be NULL when that is 0).  On return it holds the segment
 *             start states and a 256-byte tag naming the sizes, direction and
 *             the k, v, slope and state_in pointers they come from.
 * ------------------------------------------------------------------------ */
la_status_t la_prefill(la_dtype_t dt, int B, int H, int N, int d, int C,
                       const void *q, const void *k, const void *v,
                       const float *slope, const float *state_in, void *o,
                       float *state_out, void *workspace,
                       size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------ *
 * la_prefill_noalloc -- la_prefill without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  It allocates nothing:
 * the segment start states, piece states and their tag go to a static
 * buffer of the library, 64 MiB per GPU, which each GPU the library runs on
 * holds until the process ends (its address is looked up once per device,
 * on the first call with that device current).
 *
 *   arguments, results and errors as for la_prefill, without workspace and
 *   workspace_bytes; the call runs on the current device, and `stream` must
 *   belong to it.
 *   When la_prefill's workspace for these sizes would exceed the buffer, the
 *   same segments are assembled from fewer, longer pieces (this changes only
 *   the rounding of the segment start states); sizes that still do not fit
 *   give LA_ERR_WORKSPACE (with d <= 128 at most 48 MiB is needed, so every
 *   size la_prefill accepts fits).
 *   Every call on one GPU uses that GPU's one buffer: calls that overlap on
 *   a GPU (on different streams, or from different threads) race and give
 *   wrong results; calls on one stream are ordered and safe.  The buffer
 *   keeps the last call's contents; nothing in it has to start at zero,
 *   because a call reads only entries it has written itself.
 * ------------------------------------------------------------------------ */
la_status_t la_prefill_noalloc(la_dtype_t dt, int B, int H, int N, int d,
                               int C, const void *q, const void *k,
                               const void *v, const float *slope,
                               const float *state_in, void *o,
                               float *state_out, void *stream);

/* ------------------------------------------------------------------------ *
 * la_prefill_gated -- la_prefill with the layer's output epilogue fused in:
 * the Group RMSNorm + Sigmoid Gate that the pages fuse for inference
 * ("linghe" section), one group per head.  For every token t and head h,
 * with x = o_t (the d outputs of la_prefill, in fp32, before rounding):
 *
 *     y_t[j] = x[j] / sqrt(mean_j' x[j']^2 + eps) * norm_weight[h][j]
 *              * sigmoid(gate_t[j])
 *
 * and y is written instead of o (rounded once, to dt).  The norm sees the
 * whole head row, so o never makes a round trip through memory.
 *
 *   arguments of la_prefill, with o replaced by y, plus
 *   gate         [B][H][N][d] of dt, 16-byte aligned, must not overlap y
 *   norm_weight  [H][d] fp32
 *   eps          finite, >= 0 (LA_ERR_BAD_SHAPE otherwise)
 *   workspace    at least la_workspace_bytes(0, ...) bytes
 * ------------------------------------------------------------------------ */
la_status_t la_prefill_gated(la_dtype_t dt, int B, int H, int N, int d, int C,
                             const void *q, const void *k, const void *v,
                             const float *slope, const float *state_in,
                             const void *gate, const float *norm_weight,
                             float eps, void *y, float *state_out,
                             void *workspace, size_t workspace_bytes,
                             void *stream);

/* ------------------------------------------------------------------------ *
 * la_prefill_prepass / la_prefill_main -- la_prefill in two calls.
 *
 * When B*H is small, la_prefill cuts each sequence into segments that run in
 * parallel.  la_prefill_prepass computes the state entering every segment
 * from K, V and state_in -- per-piece local states combined by decay, the
 * "local recursion + global correction" of the context-parallel scheme on the
 * "Context Parallel for Lightning Attention" section -- and leaves them in
 * `workspace`.  la_prefill_main then runs all segments from those states.
 * la_prefill is exactly la_prefill_prepass followed by la_prefill_main on the
 * same stream; the split lets a caller time or overlap the two parts.
 *
 * Both calls take the arguments of la_prefill (the prepass only the ones it
 * reads) and must see the same dt, B, H, N, d, C, k, v, slope, state_in and
 * workspace; the workspace must not be modified between the two calls.  When
 * la_workspace_bytes(0, ...) is 0 the prepass enqueues nothing.
 * la_prefill_main checks the workspace tag on the device (the library cannot
 * read device memory without synchronising): if it does not name the same
 * sizes and k, v, slope and state_in pointers, every output and the final
 * state are NaN.  The tag names pointers, not contents: states computed from
 * the same buffers before their contents changed still pass.
 * ------------------------------------------------------------------------ */
la_status_t la_prefill_prepass(la_dtype_t dt, int B, int H, int N, int d, int C,
                               const void *k, const void *v,
                               const float *slope, const float *state_in,
                               void *workspace, size_t workspace_bytes,
                               void *stream);
la_status_t la_prefill_main(la_dtype_t dt, int B, int H, int N, int d, int C,
                            const void *q, const void *k, const void *v,
                            const float *slope, const float *state_in, void *o,
                            float *state_out, void *workspace,
                            size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------ *
 * la_decode_step -- one generated token per (b, h), on a carried state.
 *
 * S <- lambda S + k v^T, then o = q^T S (the update comes first, so the new
 * token contributes with weight 1).  This is the recurrent form of the same
 * operation used for decoding ("Hybrid Linear Attention" section: O(n)
 * training and decoding).
 *
 *   B, H      >= 1, B*H at most 2^21 (LA_ERR_UNSUPPORTED above)
 *   q, k, v   [B][H][d] of dt
 *   slope     [H] fp32
 *   state     [B][H][d][d] fp32, read and written in place: read with
 *             non-temporal loads, written with sc1 stores (so that a state
 *             the Infinity Cache still holds is read from it, and one it
 *             does not hold streams from HBM at the full rate)
 *   o         [B][H][d] of dt, written; must not overlap q, k, v or state
 * ------------------------------------------------------------------------ */
la_status_t la_decode_step(la_dtype_t dt, int B, int H, int d, const void *q,
                           const void *k, const void *v, const float *slope,
                           float *state, void *o, void *stream);

/* ------------------------------------------------------------------------ *
 * la_decode_tokens -- K new tokens per (b, h) on a carried state, in one call:
 * multi-token generation and the verification of K drafted tokens (the pages
 * serve with multi-token generation, "linghe" section).  Equal to K
 * consecutive la_decode_step calls: token j sees tokens 0..j of the call and
 * the state, and the state advances by all K tokens.  Up to 16 tokens run the
 * recurrence step by step on the state held in registers; more tokens run as
 * one chunk of the prefill form (matrix products for the in-call scores).
 * Either way the state is read and written once instead of K times.
 *
 *   dt        LA_F32 or LA_BF16;  B, H >= 1;  1 <= K <= 128 (more gives
 *             LA_ERR_UNSUPPORTED: use la_prefill with state_out = state_in);
 *             B*H at most 2^19, B*H*K at most 2^30 (LA_ERR_UNSUPPORTED above)
 *   d         as for la_prefill
 *   q, k, v   [B][H][K][d] of dt
 *   slope     [H] fp32
 *   state     [B][H][d][d] fp32, read and written in place
 *   o         [B][H][K][d] of dt, written; must not overlap q, k, v or state
 * No workspace.  Errors as for la_decode_step.
 * ------------------------------------------------------------------------ */
la_status_t la_decode_tokens(la_dtype_t dt, int B, int H, int K, int d,
                             const void *q, const void *k, const void *v,
                             const float *slope, float *state, void *o,
                             void *stream);

/* ------------------------------------------------------------------------ *
 * la_prefill_bwd -- gradients of L = sum_t o_t . dout_t with respect to q, k
 * and v (training; the pages train the layer at up to 256K context).
 *
 *   dq_t = S_t dout_t
 *   dk_s = sum_{t>=s} lambda^(t-s) (dout_t . v_s) q_t
 *   dv_s = sum_{t>=s} lambda^(t-s) (q_t . k_s) dout_t
 *
 * No gradient is produced for slope or for an initial state; state_in must be
 * NULL in this version (LA_ERR_UNSUPPORTED otherwise).
 *   dt, B, H, N, d, C, q, k, v, slope : as for la_prefill
 *   dout       [B][H][N][d] of dt
 *   dq, dk, dv [B][H][N][d] of dt, written; must not overlap any input or
 *              each other
 *   workspace  at least la_workspace_bytes(1, ...) bytes
 * ------------------------------------------------------------------------ */
la_status_t la_prefill_bwd(la_dtype_t dt, int B, int H, int N, int d, int C,
                           const void *q, const void *k, const void *v,
                           const void *dout, const float *slope,
                           const float *state_in, void *dq, void *dk,
                           void *dv, void *workspace, size_t workspace_bytes,
                           void *stream);

/* ------------------------------------------------------------------------ *
 * la_prefill_bwd_reuse -- la_prefill_bwd for a caller that keeps the forward's
 * workspace: the dq pass (the causal pass with k and v exchanged, whose states
 * sum v k^T) takes its segment start states as the transposes of those the
 * forward left in the workspace (sums of k v^T) instead of computing them
 * again, which saves its segment pre-pass.
 *
 * Arguments and errors as for la_prefill_bwd.  In addition, workspace must be
 * the workspace of a completed la_prefill (or la_prefill_prepass) call with
 * the same dt, B, H, N, d, C, k, v and slope and a NULL state_in, unmodified
 * since (the forward needs as many bytes as the backward).  The dq pass
 * checks the workspace tag on the device: a workspace whose tag does not name
 * that forward (same sizes, forward direction, the same k, v and slope
 * pointers, NULL state_in) gives an all-NaN dq (dk and dv are unaffected);
 * the status is still LA_OK, since the check runs on the device.  The call
 * overwrites the workspace and its tag, so a second _reuse call on it gives
 * NaN.  fp32 calls, and calls whose rows are not split into segments, need no
 * states and give the same results as la_prefill_bwd.
 * ------------------------------------------------------------------------ */
la_status_t la_prefill_bwd_reuse(la_dtype_t dt, int B, int H, int N, int d,
                                 int C, const void *q, const void *k,
                                 const void *v, const void *dout,
                                 const float *slope, const float *state_in,
                                 void *dq, void *dk, void *dv, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* Device workspace bytes needed by la_prefill (op = 0) or la_prefill_bwd
 * (op = 1) for these sizes: the piece and segment start states of the
 * segment pre-pass plus the 256-byte tag; 0 (no segments) means NULL may be
 * passed.  Returns (size_t)-1 for arguments the corresponding call would
 * reject. */
size_t la_workspace_bytes(int op, la_dtype_t dt, int B, int H, int N, int d,
                          int C);

/* ------------------------------------------------------------------------ *
 * la_prefill_varlen -- la_prefill over a packed batch of sequences of
 * different lengths, each with its own initial and final state.
 *
 * The pages train on variable-length (packed) batches and fold the state
 * correction of several sub-sequences into one kernel ("Context Parallel for
 * Lightning Attention" section), and serve with prefix caching ("linghe"
 * section): a sequence continues from the cached state of its prefix.  Here
 * sequence s is tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 of every head, and
 * is its own recurrence: no token sees a token of another sequence, and its
 * state starts from state_in[s] (zero when state_in is NULL).  Running a
 * sequence in two calls, the second with the first's state_out as state_in,
 * gives the result of one call over the whole sequence.
 *
 *   dt, d, C   as for la_prefill;  1 <= H <= 4096 (more gives LA_ERR_UNSUPPORTED)
 *   nseq       1 .. 256 (more gives LA_ERR_UNSUPPORTED)
 *   cu_seqlens HOST array of nseq + 1 ints, read during the call only:
 *              cu_seqlens[0] = 0, non-decreasing (empty sequences allowed);
 *              T = cu_seqlens[nseq] is the packed length; H*T above 2^30,
 *              or pieces beyond 2^32 work-items (as for la_prefill), gives
 *              LA_ERR_UNSUPPORTED
 *   q, k, v    [H][T][d] of dt (the B = 1 layout of la_prefill with the
 *              sequences back to back), 16-byte aligned
 *   slope      [H] fp32
 *   state_in   [nseq][H][d][d] fp32, or NULL for zero initial states
 *   o          [H][T][d] of dt, written; must not overlap q, k or v
 *   state_out  [nseq][H][d][d] fp32 or NULL; may equal state_in, must not
 *              partially overlap it; an empty sequence's state passes through
 *   workspace  at least la_workspace_bytes_varlen(0, ...) bytes
 * Errors as for la_prefill; a malformed cu_seqlens gives LA_ERR_BAD_SHAPE.
 * ------------------------------------------------------------------------ */
la_status_t la_prefill_varlen(la_dtype_t dt, int H, int d, int C, int nseq,
                              const int *cu_seqlens, const void *q,
                              const void *k, const void *v, const float *slope,
                              const float *state_in, void *o, float *state_out,
                              void *workspace, size_t workspace_bytes,
                              void *stream);

/* ------------------------------------------------------------------------ *
 * la_prefill_bwd_varlen -- la_prefill_bwd over a packed batch (zero initial
 * states): the gradients of L = sum_t o_t . dout_t for o from
 * la_prefill_varlen with state_in = NULL.  Arguments as for
 * la_prefill_varlen and la_prefill_bwd; dout, dq, dk, dv are [H][T][d] of dt,
 * the outputs must not overlap any input or each other; the workspace is at
 * least la_workspace_bytes_varlen(1, ...) bytes.
 * ------------------------------------------------------------------------ */
la_status_t la_prefill_bwd_varlen(la_dtype_t dt, int H, int d, int C, int nseq,
                                  const int *cu_seqlens, const void *q,
                                  const void *k, const void *v,
                                  const void *dout, const float *slope,
                                  void *dq, void *dk, void *dv, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* la_prefill_bwd_varlen_reuse -- la_prefill_bwd_varlen on the workspace of
 * the matching la_prefill_varlen call, as la_prefill_bwd_reuse is to
 * la_prefill_bwd: that call must have had the same dt, H, d, C, nseq,
 * cu_seqlens, k, v and slope and a NULL state_in, and the workspace must be
 * unmodified since; otherwise dq is all NaN (the tag check of
 * la_prefill_bwd_reuse, with the sequence table hashed into the tag). */
la_status_t la_prefill_bwd_varlen_reuse(la_dtype_t dt, int H, int d, int C,
                                        int nseq, const int *cu_seqlens,
                                        const void *q, const void *k,
                                        const void *v, const void *dout,
                                        const float *slope, void *dq, void *dk,
                                        void *dv, void *workspace,
                                        size_t workspace_bytes, void *stream);

/* Device workspace bytes for la_prefill_varlen (op = 0) or
 * la_prefill_bwd_varlen (op = 1); (size_t)-1 for arguments they would
 * reject. */
size_t la_workspace_bytes_varlen(int op, la_dtype_t dt, int H, int d, int C,
                                 int nseq, const int *cu_seqlens);

/* ------------------------------------------------------------------------ *
 * la_probe_stream_rmw -- measurement helper, not part of the layer: x <- a x
 * in place over n floats with 16-byte accesses, each element read once and
 * written once.  It is the decode step's state traffic without its
 * arithmetic, so its rate is the HBM rate that access pattern can reach on
 * the GPU it runs on (the ceiling the decode step is compared with).
 *   x             device pointer, 16-byte aligned
 *   n             a positive multiple of 4, at most 4 * 1024 * (2^24 - 1)
 *                 (LA_ERR_UNSUPPORTED above)
 *   load_policy   cache-policy bits of the loads: 0 or LA_CPOL_NT
 *   store_policy  of the stores: 0, LA_CPOL_NT or LA_CPOL_SC1
 *                 (the decode kernels use LA_CPOL_NT loads, LA_CPOL_SC1
 *                 stores); any other value -> LA_ERR_UNSUPPORTED
 * ------------------------------------------------------------------------ */
#define LA_CPOL_NT 2
#define LA_CPOL_SC1 16
la_status_t la_probe_stream_rmw(float *x, size_t n, float a, int load_policy,
                                int store_policy, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *la_status_string(la_status_t status);

/* LA_ABI_VERSION of the built library. */
int la_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTNING_LA_H */
