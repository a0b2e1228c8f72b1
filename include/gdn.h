/*
 * gdn.h -- C ABI of libgdn: the chunkwise Gated DeltaNet forward and its
 * backward, the input preparation and the single-token decode step, on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation is the gated delta rule of Gated DeltaNet (the December 2024
 * paper by Yang, Kautz and Hatamizadeh that the Qwen FlashQLA article names
 * under "The bottleneck nobody wanted to talk about"), per sequence and per
 * value head, with an fp32 state:
 *
 *     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,     o_t = scale * S_t q_t
 *
 * where a_t = exp(g_t): g is the natural-log decay and b = beta the write
 * strength, the two gate inputs of the jax-linear-attention page's
 * "Quick start", whose call takes q, k, v of shape [B, T, H, D] and returns
 * (o, state) with an fp32 state of shape (B, H, K, V).  The state is exchanged
 * as M = S^T, element (i, j) coupling key dimension i to value dimension j.
 * The call evaluates the recurrence in chunk-parallel form (chunks of 64
 * tokens), the form the same page lists next to the token-by-token
 * reference under "How it works"; the result is the recurrence's, up to
 * rounding.
 *
 * Packed documents: with cu_seqlens the single row of tokens holds N
 * documents, document n being tokens [cu[n], cu[n+1]); the state restarts at
 * every document start (the per-document reset of "How it works" on the
 * jax-linear-attention page; FLA's variable-length inputs on the
 * flash-linear-attention review page, "The library changes shape under
 * you").  Grouped value heads: H_v = G * H_qk and value head j reads q/k head
 * j / G.
 *
 * Conventions for every entry point:
 *   - all tensors are dense, row-major (last index fastest), in device memory
 *     the caller allocated and owns; the library allocates no device memory
 *     and keeps no state between calls other than its compiled kernels;
 *   - work is enqueued on `stream` and nothing synchronises: results are
 *     valid once the stream has reached this point;
 *   - a status other than GDN_OK means nothing was enqueued (except
 *     GDN_ERR_HIP, where a launch failed: outputs are then undefined);
 *   - nothing is thrown across the ABI.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1, /* null required pointer, size out of range, bad cu_seqlens */
    GDN_ERR_UNSUPPORTED = 2, /* a shape or dtype this build has no kernel for */
    GDN_ERR_MISALIGNED = 3,  /* a pointer not aligned to 16 bytes */
    GDN_ERR_WORKSPACE = 4,   /* workspace missing or smaller than the query said */
    GDN_ERR_HIP = 5,         /* a HIP launch failed; see gdn_last_hip_error() */
    GDN_ERR_SCRATCH_LIMIT = 6 /* gdn_chunk_fwd_noalloc: more scratch needed than
                                 GDN_STATIC_SCRATCH_BYTES */
} gdn_status;

/* Bytes of the static device scratch behind gdn_chunk_fwd_noalloc (per GPU). */
#define GDN_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* Option bits of gdn_chunk_fwd, gdn_prepare_inputs and gdn_recurrent_step. */
#define GDN_QK_L2NORM 1u /* divide every q and k row (dk elements) by its L2 norm */
#define GDN_GATE_ACT 2u  /* g and beta arrive raw: g <- logsigmoid(g), beta <- sigmoid(beta) */

typedef enum {
    GDN_F32 = 0,  /* q, k, v and o in IEEE fp32 */
    GDN_BF16 = 1  /* q, k, v and o in bfloat16 (o rounded to nearest even) */
} gdn_dtype;

/*
 * Bytes of device workspace gdn_chunk_fwd can use for these sizes (0 when it
 * uses none).  Only the piece scan uses a workspace: batch-mode bf16 calls
 * with so few rows x heads that compute units would idle are split along the
 * rows into pieces that run in parallel (the exact piece
 * scan the jax-linear-attention page names under "Where we lose": each
 * piece's end state is an affine map of its start state, F + Phi S, so the
 * start states follow from a short scan over the pieces, then every piece
 * is run again from its true start).  The workspace holds, per piece but the
 * last and head, F and Phi (dk x (dv + dk) fp32) and the start state
 * (dk x dv fp32).  The host picks the piece count from the sizes alone (a
 * cost model of workgroup rounds, the scan's serial steps and the extra
 * launches); calls whose whole rows already fill every compute unit, or
 * where pieces would not save a twentieth, return 0.  Returns 0 as well for
 * fp32, and for sizes the forward would reject.
 *
 * Packed calls (cu_seqlens, B = 1) also use the workspace: it holds the
 * order in which the documents are scheduled, longest first (ranked on the
 * device, up to 2,048 documents), and, when the host copy of cu_seqlens is
 * given, the piece scan over long documents: a document longer than the
 * planned piece length is split into pieces exactly as a long row is.  The
 * documents' pieces use at most the piece slots of the single-row plan of
 * T tokens, so the size does not depend on the document lengths.
 *
 * n_seqs: the number of documents when cu_seqlens will be passed, else B.
 */
size_t gdn_chunk_fwd_workspace_size(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk,
                                    int32_t H_v, int32_t dk, int32_t dv, int32_t n_seqs);

/*
 * The plan gdn_chunk_fwd makes for a call given a large enough workspace,
 * without launching anything: *piece_len is the piece length in tokens of
 * the piece scan (0: whole rows or documents), *slots the number of pieces
 * that hand a start state on (the piece arrays' rows), *ordered 1 when the
 * documents of a packed call are scheduled longest first.  Pass
 * cu_seqlens_host (n_seqs documents, B = 1) to plan a packed call, or NULL
 * for B batch rows.  The arguments are validated as gdn_chunk_fwd's are.
 */
gdn_status gdn_chunk_fwd_plan(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk, int32_t H_v,
                              int32_t dk, int32_t dv, const int32_t *cu_seqlens_host,
                              int32_t n_seqs, int64_t *piece_len, int64_t *slots,
                              int32_t *ordered);

/*
 * The chunked forward.
 *
 *   dtype        dtype of q, k, v and o.
 *   B, T         batch rows and tokens per row (T >= 1).  With cu_seqlens,
 *                B must be 1 and T is the total packed length.
 *   H_qk, H_v    q/k heads and value heads; H_v % H_qk == 0.
 *   dk, dv       key and value head dimensions.  Supported: dk, dv in
 *                {64, 128, 256} for both dtypes (dk = 256: the key width
 *                of the Gated DeltaNet 1.3B preset's kernels on the
 *                jax-linear-attention page, "Benchmarks", footnote (d);
 *                those calls walk chunks of 32 tokens).
 *   q, k         [B, T, H_qk, dk]
 *   v            [B, T, H_v, dv]
 *   g            [B, T, H_v] fp32, natural-log decay (a = exp(g)); finite.
 *   beta         [B, T, H_v] fp32, write strength.
 *   scale        multiplies the output (1.0 gives o_t = S_t q_t).
 *   flags        in-op preparation, 0 for none (the inputs are never
 *                modified):
 *                GDN_QK_L2NORM  every q and k row is divided by its L2 norm
 *                               inside the call (use_qk_l2norm of the
 *                               jax-linear-attention page's "Quick start"):
 *                               the inverse norm is taken in fp32 and applied
 *                               as an fp32 factor where the row enters the
 *                               equations, so the normalised row is never
 *                               rounded (gdn_prepare_inputs, which stores
 *                               rows, rounds them to the input dtype); a
 *                               row of zeros stays zero;
 *                GDN_GATE_ACT   g and beta are raw values: the decay is
 *                               logsigmoid(g) and the write strength
 *                               sigmoid(beta).
 *   h0           [N, H_v, dk, dv] fp32 initial states, or NULL for zeros.
 *   cu_seqlens   device int32 [N + 1] document offsets, or NULL (then the
 *                documents are the B rows and N = B).
 *   cu_seqlens_host  optional host copy of cu_seqlens, equal to it.  When
 *                given it is validated (cu[0] = 0, non-decreasing, cu[N] = T)
 *                before anything is enqueued and, with a workspace, lets the
 *                host plan the piece scan over long documents (bf16); when
 *                NULL the device array is trusted and documents run whole.
 *                The kernels read the device array (a host copy that
 *                disagrees with it leaves work undone but never writes
 *                outside the outputs and workspace).  Empty documents are
 *                allowed: their final state is their initial state.
 *   n_seqs       N when cu_seqlens is given (>= 1); ignored otherwise.
 *   o            [B, T, H_v, dv] output, dtype `dtype`.
 *   ht           [N, H_v, dk, dv] fp32 final states, or NULL to skip them.
 *   workspace    device scratch of gdn_chunk_fwd_workspace_size() bytes,
 *                256-byte aligned, owned by the caller and not read after the
 *                call's work completes; or NULL, which runs whole rows and
 *                documents in index order (the same result up to rounding).
 *                A non-NULL workspace smaller than the plan needs returns
 *                GDN_ERR_WORKSPACE.
 *   stream       HIP stream to enqueue on (NULL = the default stream).
 *
 * Every pointer must be 16-byte aligned.  o and ht must not overlap the
 * inputs.
 */
gdn_status gdn_chunk_fwd(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk, int32_t H_v,
                         int32_t dk, int32_t dv, const void *q, const void *k, const void *v,
                         const float *g, const float *beta, float scale, uint32_t flags,
                         const float *h0,
                         const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                         int32_t n_seqs, void *o, float *ht, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * gdn_chunk_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, the same result as
 * gdn_chunk_fwd with a workspace of gdn_chunk_fwd_workspace_size() bytes.
 * The piece scan's arrays go to a static device scratch of
 * GDN_STATIC_SCRATCH_BYTES (64 MiB) that the library holds on every GPU it
 * runs on until the process ends; its address is looked up once per device,
 * on the first call with that device current.  Nothing is allocated and no
 * allocating routine is called.  Returns GDN_ERR_SCRATCH_LIMIT, before
 * anything is enqueued, when the call's piece plan needs more scratch than
 * that (gdn_chunk_fwd with a workspace, or with NULL for whole rows, runs
 * such calls).  Every call on a GPU shares that GPU's scratch: calls that
 * overlap on one GPU (on different streams, or from different threads) race
 * and must be ordered by the caller.  Nothing in the scratch needs to start
 * at zero (each call writes every element it reads).
 */
gdn_status gdn_chunk_fwd_noalloc(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk,
                                 int32_t H_v, int32_t dk, int32_t dv, const void *q,
                                 const void *k, const void *v, const float *g,
                                 const float *beta, float scale, uint32_t flags,
                                 const float *h0, const int32_t *cu_seqlens,
                                 const int32_t *cu_seqlens_host, int32_t n_seqs, void *o,
                                 float *ht, hipStream_t stream);

/*
 * Bytes of device workspace gdn_chunk_bwd needs for these sizes (0 for sizes
 * the backward would reject).  The workspace holds, per chunk and value head,
 * in bf16: the state entering the chunk and the gradient of the state leaving
 * it, and the chunk's Delta and drhs rows (the solved right-hand side of the
 * forward and of its transpose).  At dk = 64 and 128 a chunk is 64 tokens and
 * the states are 128 keys wide: (2 * 128 + 2 * 64) * dv * 2 bytes per chunk
 * and head; at dk = 256 a chunk is 32 tokens: (2 * 256 + 2 * 32) * dv * 2.
 *
 * n_seqs: the number of documents when cu_seqlens will be passed, else B.
 * With cu_seqlens the size covers any split of the T tokens into n_seqs
 * documents.  flags: those gdn_chunk_bwd will get; each option adds room for
 * the prepared copies of the inputs it rewrites (q and k in bf16 for
 * GDN_QK_L2NORM, g and beta in fp32 for GDN_GATE_ACT, each region rounded up
 * to 256 bytes).  Unknown flag bits give 0.
 */
size_t gdn_chunk_bwd_workspace_size(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk,
                                    int32_t H_v, int32_t dk, int32_t dv, int32_t n_seqs,
                                    uint32_t flags);

/*
 * The chunked backward: the gradients of L = sum(do * o) + sum(dht * ht) with
 * respect to q, k, v, g, beta and h0, for the forward gdn_chunk_fwd computes
 * with the same arguments (the follow-on call the problem statement names;
 * the pages give no formulas for it, so it is the reverse mode of the forward
 * recurrence, derived by the chain rule).
 *
 *   dtype, B, T, H_qk, H_v, dk, dv, q, k, v, g, beta, scale, h0, cu_seqlens,
 *   cu_seqlens_host, n_seqs
 *                as for gdn_chunk_fwd.  Supported: bf16 with dk and dv in
 *                {64, 128, 256}; everything else returns
 *                GDN_ERR_UNSUPPORTED.
 *   flags        the in-op preparation of the forward (GDN_QK_L2NORM,
 *                GDN_GATE_ACT, as for gdn_chunk_fwd): q, k, g and beta are
 *                then the raw inputs, and dq, dk_, dg, dbeta come back with
 *                respect to them.  The call prepares copies of the inputs in
 *                the workspace (as gdn_prepare_inputs does), runs the
 *                backward on them, and chains the gradients through the
 *                preparation in place (as gdn_prepare_inputs_bwd does); with
 *                an option set every token of those four outputs is
 *                written.  Unknown bits return GDN_ERR_INVALID_ARG.
 *   dout         [B, T, H_v, dv] upstream gradient of o, dtype `dtype`.
 *   dht          [N, H_v, dk, dv] fp32 upstream gradient of the final state,
 *                or NULL for none.
 *   dq, dk_      [B, T, H_qk, dk] outputs, dtype `dtype`; for grouped value
 *                heads the sum over the value heads sharing the q/k head.
 *   dv_          [B, T, H_v, dv] output, dtype `dtype`.
 *   dg, dbeta    [B, T, H_v] fp32 outputs.
 *   dh0          [N, H_v, dk, dv] fp32 output (the gradient of the initial
 *                state; equal to dht for an empty document), or NULL.
 *   workspace    device scratch of at least gdn_chunk_bwd_workspace_size()
 *                bytes (for the same flags), 256-byte aligned, owned by the
 *                caller; its contents are undefined afterwards.
 *   stream       HIP stream to enqueue on.
 *
 * Every pointer must be 16-byte aligned; outputs must not overlap inputs or
 * the workspace.  Tokens outside every document (none when cu_seqlens is
 * valid) are left untouched in the outputs.
 */
gdn_status gdn_chunk_bwd(gdn_dtype dtype, int64_t B, int64_t T, int32_t H_qk, int32_t H_v,
                         int32_t dk, int32_t dv, const void *q, const void *k, const void *v,
                         const float *g, const float *beta, float scale, uint32_t flags,
                         const float *h0, const int32_t *cu_seqlens,
                         const int32_t *cu_seqlens_host, int32_t n_seqs, const void *dout,
                         const float *dht, void *dq, void *dk_, void *dv_, float *dg,
                         float *dbeta, float *dh0, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * The input preparation the jax-linear-attention page's "Quick start" call
 * offers in-op (use_qk_l2norm: q and k divided by their L2 norms) and the gate
 * activations its example applies to raw gate values (g = logsigmoid(raw) as
 * the natural-log decay, beta = sigmoid(raw) as the write strength).  Run it
 * before gdn_chunk_fwd or gdn_chunk_bwd on the prepared copies.
 *
 *   dtype        dtype of q, k, q_out and k_out.
 *   n_qk_rows    rows of dk elements in q (and in k), e.g. B * T * H_qk.
 *   dk           1 <= dk <= 256.
 *   q, k         inputs; q_out, k_out: outputs of the same size.  With
 *                GDN_QK_L2NORM each row x becomes x / ||x||_2, the norm taken
 *                in fp32 and the result rounded to `dtype` (round to nearest
 *                even); a row of zeros stays zeros.
 *   n_gates      elements of g (and of beta), e.g. B * T * H_v.
 *   g, beta      fp32 inputs; g_out, beta_out: fp32 outputs.  With
 *                GDN_GATE_ACT, g_out = logsigmoid(g), beta_out = sigmoid(beta).
 *   flags        GDN_QK_L2NORM | GDN_GATE_ACT; the pointers of an option not
 *                set, or with no rows or gates, may be NULL and are not read.
 *
 * Outputs may be their own inputs (in place); other overlaps are undefined.
 * Every pointer must be 16-byte aligned.  Unknown flag bits return
 * GDN_ERR_INVALID_ARG.
 */
gdn_status gdn_prepare_inputs(gdn_dtype dtype, int64_t n_qk_rows, int32_t dk, const void *q,
                              const void *k, void *q_out, void *k_out, int64_t n_gates,
                              const float *g, const float *beta, float *g_out,
                              float *beta_out, uint32_t flags, hipStream_t stream);

/*
 * The reverse of gdn_prepare_inputs: from the gradients of a loss with
 * respect to the prepared values, those with respect to the raw inputs.  The
 * pages print no gradients; these are the derivatives of the three maps:
 *
 *   GDN_QK_L2NORM  y = x / n, n = ||x||_2:  dx = (dy - (dy . y) y) / n, per
 *                  row of dk elements (a row of zeros gets zeros), in fp32
 *                  with the norm as gdn_prepare_inputs takes it, the result
 *                  rounded to `dtype` (round to nearest even).
 *   GDN_GATE_ACT   g' = logsigmoid(g):  dg = dg' sigmoid(-g);
 *                  beta' = sigmoid(beta):  dbeta = dbeta' sigmoid(beta) sigmoid(-beta).
 *
 *   dtype, n_qk_rows, dk, n_gates, flags   as for gdn_prepare_inputs.
 *   q, k         the raw rows [n_qk_rows, dk], dtype `dtype`.
 *   dq_in, dk_in gradients with respect to the normalised rows, same shape
 *                and dtype; dq_out, dk_out: the results.
 *   g, beta      the raw gates [n_gates] fp32; dg_in, dbeta_in: gradients
 *                with respect to the activated gates; dg_out, dbeta_out: the
 *                results (fp32).
 *
 * Each output may be its gradient input (in place); other overlaps are
 * undefined.  The pointers of an option not set, or with no rows or gates,
 * may be NULL.  Every pointer must be 16-byte aligned.
 */
gdn_status gdn_prepare_inputs_bwd(gdn_dtype dtype, int64_t n_qk_rows, int32_t dk,
                                  const void *q, const void *k, const void *dq_in,
                                  const void *dk_in, void *dq_out, void *dk_out,
                                  int64_t n_gates, const float *g, const float *beta,
                                  const float *dg_in, const float *dbeta_in, float *dg_out,
                                  float *dbeta_out, uint32_t flags, hipStream_t stream);

/*
 * One token of the recurrence for each of N sequences (decoding), the state
 * kept in a cache of n_slots states and updated in place: the token-by-token
 * form the jax-linear-attention page lists under "How it works", one token
 * per call, with the per-layer recurrent decode state its inference answer
 * describes.  With M the state of the sequence's slot (as in gdn_chunk_fwd,
 * element (i, j) couples key dimension i to value dimension j):
 *
 *     y = M^T k,  delta = beta (v - a y),  M <- a M + k delta^T,  o = scale M^T q
 *
 * with a = exp(g).  The final states of gdn_chunk_fwd ([N, H_v, dk, dv]) are
 * valid cache entries, so a prefill hands over to decoding directly.
 *
 *   dtype        dtype of q, k, v and o.
 *   N            sequences this step (N = 0 enqueues nothing and reads no
 *                pointer).
 *   H_qk, H_v    as for gdn_chunk_fwd (H_v % H_qk == 0).
 *   dk, dv       each 64, 128 or 256.
 *   q, k         [N, H_qk, dk]; v: [N, H_v, dv]; g, beta: [N, H_v] fp32.
 *   scale        multiplies the output.
 *   flags        GDN_QK_L2NORM: q and k are divided by their L2 norms (fp32,
 *                not rounded); GDN_GATE_ACT: g and beta are raw values passed
 *                through logsigmoid and sigmoid.
 *   state        [n_slots, H_v, dk, dv] fp32 cache, read and written.
 *   slots        device int32 [N]: the cache slot of each sequence, or NULL
 *                for slot n (then n_slots >= N).  A slot outside [0, n_slots)
 *                is padding: that sequence starts from a zero state and
 *                nothing is written back.  Two sequences of one call must not
 *                share a slot.
 *   o            [N, H_v, dv] output.
 *
 * Every pointer must be 16-byte aligned; o must not overlap the inputs.
 */
gdn_status gdn_recurrent_step(gdn_dtype dtype, int64_t N, int32_t H_qk, int32_t H_v,
                              int32_t dk, int32_t dv, const void *q, const void *k,
                              const void *v, const float *g, const float *beta, float scale,
                              uint32_t flags, float *state, const int32_t *slots,
                              int64_t n_slots, void *o, hipStream_t stream);

/* A static, human-readable name for a status. */
const char *gdn_status_string(gdn_status status);

/* The HIP error of the last GDN_ERR_HIP returned on this thread. */
hipError_t gdn_last_hip_error(void);

/* Library version, as major * 10000 + minor * 100 + patch. */
int32_t gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
