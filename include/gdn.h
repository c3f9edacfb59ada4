/*
 * gdn.h -- C ABI of the gfx950 (MI355X) gated delta rule library (libgdn.so).
 *
 * The operation (jianyuh.github.io reading notes on Qwen3.8-Next, section 2.1 "Gated
 * DeltaNet", the four-line recurrence and its boxed transition-matrix form): for every
 * sequence n and head h, with a state S in R^{d_k x d_v} (rows over the key dimension),
 * scalar gates alpha_t in (0,1] (decay) and beta_t in [0,1] (write strength),
 *
 *     S_t = alpha_t S_{t-1} + beta_t k_t (v_t - alpha_t S_{t-1}^T k_t)^T
 *         = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *     y_t = S_t^T q_t                       (read from the updated state)
 *
 * The library takes q, k, v and the gates as given: it does not normalise q or k, apply
 * a feature map or a query scale, or derive alpha from log-space parameters.
 *
 * Layouts (all row-major, no padding):
 *   q, k      [rows, H, d_k]       rows = total tokens of the packed batch (prefill)
 *   v, y      [rows, H, d_v]                or the batch size (decode)
 *   alpha,beta[rows, H]            fp32
 *   state     [N, H, d_k, d_v]     fp32, element (i, j) at i * d_v + j
 * q, k, v and y share one dtype (gdn_dtype); the state is always fp32.
 *
 * Ownership and threading: every pointer is a device pointer owned by the caller.  The
 * library never allocates device memory, frees, or synchronises; all work is enqueued on
 * the caller's stream (a hipStream_t passed as void*, NULL = the null stream) and the call
 * returns before it completes.  Device faults surface at the caller's next synchronisation.
 * The library keeps no global state and is safe to call from several threads.
 *
 * Errors: every precondition that can be checked on the host is checked before anything is
 * enqueued; a violation returns a status code and enqueues nothing.  Values inside device
 * buffers (cu_seqlens contents, gate ranges, NaNs) are preconditions that are not checked.
 *
 * Supported shapes: d_k, d_v in {64, 128}; any H >= 1; any lengths (including 0).
 * Alignment: q, k, v, y, the states and the workspace to 16 bytes (the kernels move these
 * in 16-byte units); alpha, beta and cu_seqlens to 4 bytes.  Rows of one token are
 * contiguous, so slicing whole tokens off an aligned tensor keeps the alignment.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARGUMENT = 1,     /* null pointer, bad size, misalignment, bad aliasing */
    GDN_ERR_UNSUPPORTED = 2,          /* head dimension or dtype not built */
    GDN_ERR_WORKSPACE_TOO_SMALL = 3,  /* workspace_bytes < gdn_prefill_workspace_bytes() */
    GDN_ERR_HIP = 4                   /* the HIP runtime refused a launch */
} gdn_status;

typedef enum gdn_dtype {
    GDN_DTYPE_F32 = 0,   /* IEEE binary32 */
    GDN_DTYPE_BF16 = 1   /* bfloat16; y is rounded to nearest even */
} gdn_dtype;

/* Human-readable name of a status code (static storage; never NULL). */
const char *gdn_status_str(int32_t status);

/* Library version string, e.g. "gdn-gfx950 0.1". */
const char *gdn_version(void);

/*
 * Bytes of device workspace gdn_prefill needs for this problem (a pure function of the
 * arguments; 0 on invalid arguments).  The workspace holds, for bf16 inputs, one 8448-byte
 * record per (64-token chunk, head) (the chunk's inverted triangular system and its log-decay
 * prefix, (total_T / 64 + num_seqs) * H records in all) and,
 * for long sequences, the segment table, per-segment transition matrices and start states
 * of the segment-parallel scan.  fp32 inputs without segments need none.
 */
size_t gdn_prefill_workspace_bytes(int32_t num_seqs, int64_t total_T, int32_t H,
                                   int32_t d_k, int32_t d_v, int32_t dtype);

/*
 * Chunked prefill over a packed batch of sequences (the recurrence above, evaluated 64
 * tokens at a time with the exact WY/UT chunk form and an fp32 state).
 *
 *   q, k, v        [total_T, H, d]  dtype           (read only)
 *   alpha, beta    [total_T, H]     fp32            (read only)
 *   initial_state  [num_seqs, H, d_k, d_v] fp32, or NULL for zeros   (read only)
 *   cu_seqlens     device int32 [num_seqs + 1]: 0 = cu[0] <= cu[1] <= ... = total_T,
 *                  or NULL: num_seqs sequences of total_T / num_seqs tokens each
 *                  (total_T must then be a multiple of num_seqs)
 *   y              [total_T, H, d_v] dtype          (written; every element)
 *   final_state    [num_seqs, H, d_k, d_v] fp32 or NULL (not written).  It may be exactly
 *                  initial_state (in-place resume); any other overlap between an output and
 *                  an input, or between the two outputs, is rejected when it can be seen from
 *                  the pointers and sizes.
 *   workspace      device buffer of at least gdn_prefill_workspace_bytes(...) bytes (may be
 *                  NULL when that size is 0); its contents need no initialisation.
 * A zero-length sequence writes no y and returns its initial state.
 */
gdn_status gdn_prefill(const void *q, const void *k, const void *v,
                       const float *alpha, const float *beta,
                       const float *initial_state, const int32_t *cu_seqlens,
                       int32_t num_seqs, int64_t total_T, int32_t H,
                       int32_t d_k, int32_t d_v, int32_t dtype,
                       void *y, float *final_state,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Tuning override of gdn_prefill (same semantics and results up to rounding order):
 * dv_tile in {0 = automatic, 16, 32, 64, 128} columns of the state per workgroup (must divide
 * d_v; fp32 allows at most 64, or 32 when d_k = 128), segment_chunks = 0 (automatic), -1 (never split a sequence) or the number of
 * 64-token chunks per segment of the segment-parallel scan.  The workspace must be sized
 * with gdn_prefill_workspace_bytes_ex for the same options.
 */
size_t gdn_prefill_workspace_bytes_ex(int32_t num_seqs, int64_t total_T, int32_t H,
                                      int32_t d_k, int32_t d_v, int32_t dtype,
                                      int32_t dv_tile, int32_t segment_chunks);
gdn_status gdn_prefill_ex(const void *q, const void *k, const void *v,
                          const float *alpha, const float *beta,
                          const float *initial_state, const int32_t *cu_seqlens,
                          int32_t num_seqs, int64_t total_T, int32_t H,
                          int32_t d_k, int32_t d_v, int32_t dtype,
                          void *y, float *final_state,
                          void *workspace, size_t workspace_bytes, void *stream,
                          int32_t dv_tile, int32_t segment_chunks);

/*
 * gdn_prefill with the gates given as their pre-activations (reading notes, section 2.1
 * "Gating dynamics"): alpha_t = exp(-exp(A_h) softplus(a_t + b_alpha_h)) and
 * beta_t = sigmoid(b_t), formed inside the chunk-record kernel, which takes log2 alpha
 * directly as -exp(A_h) softplus(a_t + b_alpha_h) / ln 2 (no exp and log round trip) and is
 * the only kernel of the bf16 plans that reads the gates.
 *   a, b     [total_T, H] fp32 (4-byte aligned), in place of alpha and beta
 *   A, b_alpha [H] fp32 (4-byte aligned)
 * Every other argument, the workspace (gdn_prefill_workspace_bytes) and the error behaviour
 * are those of gdn_prefill.  bf16 only (GDN_ERR_UNSUPPORTED for fp32); a null A or b_alpha
 * with total_T > 0, or A / b_alpha overlapping an output: GDN_ERR_INVALID_ARGUMENT.
 */
gdn_status gdn_prefill_gated(const void *q, const void *k, const void *v, const float *a,
                             const float *b, const float *A, const float *b_alpha,
                             const float *initial_state, const int32_t *cu_seqlens,
                             int32_t num_seqs, int64_t total_T, int32_t H, int32_t d_k,
                             int32_t d_v, int32_t dtype, void *y, float *final_state,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_prefill followed by the output gate of the layer (reading notes, section 2.1, the output
 * equation; gdn_output_gate below): per (token, head) row of d_v values,
 *   out = sigmoid(z) * y / sqrt(mean(y^2) + eps) * (1 + weight),  y = the rule's output.
 *   z       [total_T, H, d_v] dtype, 16-byte aligned, read only
 *   weight  [d_v] fp32, 4-byte aligned (zero = plain RMSNorm)
 *   eps     finite, >= 0
 *   out     [total_T, H, d_v] dtype, in place of y (y itself is not kept)
 *   dv_tile, segment_chunks: as for gdn_prefill_ex (0, 0 = automatic)
 * The bf16 one-launch plans (d_k = d_v = 128 with dv_tile 128, the plan gdn_prefill_plan
 * reports for long or plentiful work) apply the gate as each row of y leaves the scan, so y
 * never reaches memory; every other plan runs the prefill into out and then the output-gate
 * kernel over out in place.  Workspace: gdn_prefill_workspace_bytes_ex for the same options.
 * Errors: those of gdn_prefill_ex; GDN_ERR_INVALID_ARGUMENT also for a null z or weight with
 * total_T > 0, misalignment, a negative or non-finite eps, or z or weight overlapping an
 * output.
 */
gdn_status gdn_prefill_output_gated(const void *q, const void *k, const void *v,
                                    const float *alpha, const float *beta,
                                    const float *initial_state, const int32_t *cu_seqlens,
                                    int32_t num_seqs, int64_t total_T, int32_t H, int32_t d_k,
                                    int32_t d_v, int32_t dtype, const void *z,
                                    const float *weight, float eps, void *out,
                                    float *final_state, void *workspace,
                                    size_t workspace_bytes, void *stream, int32_t dv_tile,
                                    int32_t segment_chunks);

/*
 * gdn_prefill for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same operation, arguments and
 * results, with no workspace argument.  Its workspace is a fixed array of
 * GDN_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held from the library's
 * load until the process ends; the call allocates nothing (no hipMalloc, no allocating
 * library routine).
 *   Limit: problems whose gdn_prefill_workspace_bytes(...) exceeds
 *   GDN_NOALLOC_SCRATCH_BYTES (= gdn_noalloc_scratch_bytes()) are rejected with
 *   GDN_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.
 *   Concurrency: every call on one GPU shares that GPU's array.  Calls enqueued on one
 *   stream are ordered and safe; calls that may run at the same time on one GPU (several
 *   streams or threads) race on the array and give undefined results.
 *   Errors: those of gdn_prefill; GDN_ERR_HIP also when the array's device address cannot be
 *   obtained on the current device.
 */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)
size_t gdn_noalloc_scratch_bytes(void);
gdn_status gdn_prefill_noalloc(const void *q, const void *k, const void *v,
                               const float *alpha, const float *beta,
                               const float *initial_state, const int32_t *cu_seqlens,
                               int32_t num_seqs, int64_t total_T, int32_t H,
                               int32_t d_k, int32_t d_v, int32_t dtype,
                               void *y, float *final_state, void *stream);

/*
 * The launch plan gdn_prefill would use for this problem: state columns per workgroup and
 * chunks per segment (-1 = sequences are not split).  For reporting.
 */
gdn_status gdn_prefill_plan(int32_t num_seqs, int64_t total_T, int32_t H, int32_t d_k,
                            int32_t d_v, int32_t dtype, int32_t *dv_tile,
                            int32_t *segment_chunks);

/*
 * Channel-wise gated variants of the rule (the reading notes' successors of Gated DeltaNet:
 * Kimi Delta Attention, a gate per feature channel, and Gated DeltaNet-2, separate
 * channel-wise erase and write gates; the notes give no equations, the form below is the
 * library's reading).  Per sequence and head, for every token in order:
 *
 *     S~ = Diag(a_t) S,   e = (w_t .* v_t) - (b_t .* (S~^T k_t)),   S = S~ + k_t e^T,
 *     y_t = S^T q_t
 *
 *   q, k           [total_T, H, d_k] dtype; v, y [total_T, H, d_v] dtype (16-byte aligned)
 *   decay          a: [total_T, H, d_k] fp32 in (0, 1] (16-byte aligned)
 *   erase, write   b, w: [total_T, H, d_v] fp32 in [0, 1]
 *   initial_state  [N, H, d_k, d_v] fp32 or NULL (zeros); final_state the same shape or NULL,
 *                  and may be exactly initial_state (a decode step: one token per sequence,
 *                  state carried in place)
 *   cu_seqlens     as for gdn_prefill
 * Uniform gates (a_t = alpha_t, b_t = w_t = beta_t) give gdn_prefill's rule; b_t = w_t =
 * beta_t with a free a_t is the channel-decay form.  Computed token by token in fp32 with
 * the state in registers (no chunked form); with one token per sequence and no cu_seqlens
 * (a decode step) in one streaming pass over the state.  d_k, d_v in {64, 128}.
 */
gdn_status gdn_channel_gated(const void *q, const void *k, const void *v, const float *decay,
                             const float *erase, const float *write,
                             const float *initial_state, const int32_t *cu_seqlens,
                             int32_t num_seqs, int64_t total_T, int32_t H, int32_t d_k,
                             int32_t d_v, int32_t dtype, void *y, float *final_state,
                             void *stream);

/*
 * The compressed block indexer of the reading notes' sparse attention (QSA, "The compressed
 * lightweight indexer"), for one sequence of n tokens: 4 query heads and one shared key head
 * of 128 dimensions (the projections are done by the caller), key blocks of 4 tokens.
 *   q_i^h = PRoPE(RMSNorm(q_i^h), i),  kb_b = PRoPE(RMSNorm(mean of keys 4b .. 4b+3), 4b)
 *   I_ib  = sum_h ReLU(<q_i^h, kb_b>) over the blocks complete before i (4b + 3 <= i)
 *   the block_budget highest-scoring blocks (ties to the lower index; all complete blocks
 *   when there are fewer), expanded to their tokens and joined with the tail of the current
 *   block, {floor((i+1)/4) 4 .. i}.
 * Readings of what the notes leave open: RMSNorm(x) = x / sqrt(mean(x^2) + 1e-6) without a
 * scale; PRoPE rotates dims (m, m + 32), m < 32, by pos * 10000^(-2m/64) and passes dims
 * 64..127.
 *   q          [n, 4, 128] dtype (16-byte aligned);  k  [n, 128] dtype (16-byte aligned)
 *   blocks     [n, block_budget] int32 or NULL: selected blocks, ascending, -1 padded
 *   tokens     [n, 4 block_budget + 3] int32 or NULL: the selected tokens, ascending (the
 *              blocks' tokens, then the tail), -1 padded.  At least one output is required.
 *   workspace  gdn_qsa_workspace_bytes(n) bytes: the normalised, rotated queries and block
 *              keys in bf16 (about 1 KiB per token; no score matrix is stored)
 * n <= 2^20; block_budget <= 2048, or any budget up to 2^24 that is at least n/4 (every row
 * then takes all its complete blocks): GDN_ERR_UNSUPPORTED beyond.  n <= 0, block_budget
 * <= 0, a null q, k or workspace, no output, misalignment or an output overlapping an input
 * or another output: GDN_ERR_INVALID_ARGUMENT; a short workspace: GDN_ERR_WORKSPACE_TOO_SMALL.
 * The notes' budget is block_budget = 512 (2048 tokens).  The scores use bf16 products of the
 * normalised, rotated vectors with fp32 accumulation; the selection is exact on those scores.
 */
size_t gdn_qsa_workspace_bytes(int64_t n);
gdn_status gdn_qsa_index(const void *q, const void *k, int64_t n, int32_t dtype,
                         int32_t block_budget, int32_t *blocks, int32_t *tokens,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Chunked backward (training) of gdn_prefill.
 *
 * For the scalar L = sum <dy, y> + sum <d_final_state, S_T> of the prefill with the same
 * arguments, writes its derivatives with respect to q, k, v, alpha, beta and the initial
 * state.  The derivative is that of the recurrence of the reading notes (Gated DeltaNet,
 * section 2.1), taken through the chunked WY / UT form: the forward states at every chunk
 * start and the state adjoints at every chunk end are kept in the workspace, then each chunk
 * is differentiated on its own.
 *
 *   q, k, v, alpha, beta, initial_state, cu_seqlens, num_seqs, total_T, H, d_k, d_v:
 *                  as for gdn_prefill (initial_state NULL = zeros)
 *   dtype          GDN_DTYPE_BF16 only (GDN_ERR_UNSUPPORTED otherwise)
 *   dy             [total_T, H, d_v] bf16, the adjoint of y
 *   d_final_state  [N, H, d_k, d_v] fp32, the adjoint of the final state, or NULL (zero)
 *   dq, dk         [total_T, H, d_k] bf16 (written)
 *   dv             [total_T, H, d_v] bf16 (written)
 *   dalpha, dbeta  [total_T, H] fp32 (written); dalpha is zero where alpha < e^-87 (the
 *                  floor of log alpha)
 *   d_initial_state [N, H, d_k, d_v] fp32 (written) or NULL
 *   workspace      gdn_prefill_backward_workspace_bytes(...) bytes, 16-byte aligned
 * Outputs may overlap neither the inputs nor each other.  Pointers as for gdn_prefill (16-
 * byte alignment for tensors, 4 for gates and cu_seqlens).  Invalid arguments are rejected
 * before anything is launched.
 */
size_t gdn_prefill_backward_workspace_bytes(int32_t num_seqs, int64_t total_T, int32_t H,
                                            int32_t d_k, int32_t d_v, int32_t dtype);
gdn_status gdn_prefill_backward(const void *q, const void *k, const void *v, const float *alpha,
                                const float *beta, const float *initial_state,
                                const int32_t *cu_seqlens, int32_t num_seqs, int64_t total_T,
                                int32_t H, int32_t d_k, int32_t d_v, int32_t dtype,
                                const void *dy, const float *d_final_state, void *dq, void *dk,
                                void *dv, float *dalpha, float *dbeta, float *d_initial_state,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step for a batch of B sequences (one token each), state updated in place:
 *
 *   q, k   [B, H, d_k] dtype;  v [B, H, d_v] dtype;  alpha, beta [B, H] fp32  (read only)
 *   state  [B, H, d_k, d_v] fp32, read and then overwritten with S_t
 *   y      [B, H, d_v] dtype, written with S_t^T q_t
 *
 * Each head's state is read once and written once.  state must not overlap any other
 * argument.
 */
gdn_status gdn_decode_step(const void *q, const void *k, const void *v,
                           const float *alpha, const float *beta,
                           float *state, void *y,
                           int32_t B, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype,
                           void *stream);

/*
 * The steps either side of the rule, as the reading notes on Qwen3.8-Next give them
 * (section 2.1 "Gated DeltaNet": "Feature parameterization", "Gating dynamics" and the output
 * equation).  Each is one streaming pass; none allocates, synchronises or keeps state.
 */

/*
 * Short causal depthwise convolution, SiLU and (head_dim > 0) L2 normalisation per head:
 *   out[t, c] = SiLU(sum_j weight[c, j] x[t - (width-1) + j, c])  over t's own sequence,
 *   then, with head_dim > 0, each head's head_dim channels divided by sqrt(sum^2 + 1e-6).
 * The width - 1 inputs before a sequence's first token come from state_in (or are zero).
 *   x, out       [total_T, channels] dtype (token-major, e.g. channels = H * d); 16-byte
 *                aligned; out must not overlap any input
 *   weight       [channels, width] fp32; weight[c, width-1] weighs the current token
 *   cu_seqlens   device int32 [num_seqs + 1] (as for gdn_prefill) or NULL (equal lengths)
 *   state_in     [num_seqs, channels, width - 1] fp32, oldest input first, or NULL (zeros)
 *   state_out    same shape, or NULL: the width - 1 inputs that end each sequence (reaching
 *                into state_in for sequences shorter than width - 1).  It may be exactly
 *                state_in (carried in place); a decode step is a call with num_seqs = B
 *                sequences of one token each.
 * channels: a multiple of 64; width in 1..4; head_dim in {0, 64, 128}, dividing channels.
 */
gdn_status gdn_short_conv(const void *x, const float *weight, const int32_t *cu_seqlens,
                          int32_t num_seqs, int64_t total_T, int32_t channels, int32_t width,
                          int32_t head_dim, int32_t dtype, void *out, const float *state_in,
                          float *state_out, void *stream);

/*
 * Gates:  alpha = exp(-exp(A[h]) * softplus(a + b_alpha[h])),  beta = sigmoid(b).
 *   a, b          [total_T, H] fp32 pre-activations (read only)
 *   A, b_alpha    [H] fp32 per-head time constant and bias
 *   alpha, beta   [total_T, H] fp32 (written), the gates gdn_prefill and gdn_decode_step take
 * Outputs must not overlap the inputs or each other.
 */
gdn_status gdn_gates(const float *a, const float *b, const float *A, const float *b_alpha,
                     int64_t total_T, int32_t H, float *alpha, float *beta, void *stream);

/*
 * Output gate with a zero-centred RMSNorm, per row of d_v values:
 *   out = sigmoid(z) * y / sqrt(mean(y^2) + eps) * (1 + weight)
 *   y, z, out  [rows, d_v] dtype (rows = total_T * H); 16-byte aligned; out may be exactly y
 *   weight     [d_v] fp32, the scale's offset from one (zero = plain RMSNorm)
 * d_v in {64, 128}; eps >= 0 (the binding's default is 1e-6).
 */
gdn_status gdn_output_gate(const void *y, const void *z, const float *weight, int64_t rows,
                           int32_t d_v, float eps, int32_t dtype, void *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
