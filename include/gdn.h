/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet token-mixer library.
 *
 * The operations are those of the Gated DeltaNet mixer in "On the Design of
 * Qwen3.8-Next Architecture" (slinene ai-papers-daily page, Module A; the
 * paper.rainbus.top digest, method step (1)).  Per (batch b, head h) the state
 * S is a d_k x d_v matrix and, token by token,
 *
 *     S_dec = alpha_t S_{t-1}
 *     e_t   = v_t - S_dec^T k_t
 *     S_t   = S_dec + beta_t k_t e_t^T
 *     y_t   = scale * S_t^T q_t
 *
 * and the output epilogue is  o = sigmoid(z) * y / sqrt(mean(y^2) + eps) * (1 + w)
 * (sigmoid output gate, zero-centred RMSNorm weight; slinene page, Module A).
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers, contiguous, in the layouts given
 *    below (row-major, last index fastest), 16-byte aligned.  The caller
 *    allocates and frees all memory; the library never allocates, frees or
 *    keeps pointers after a call returns, and holds no mutable global state,
 *    so calls are reentrant and thread-safe.
 *  - Work is enqueued on `hip_stream` (a hipStream_t passed as void*, NULL =
 *    the null stream); no call synchronises the stream.  Results are ready
 *    once the stream has reached the call.
 *  - Arguments are validated on the host before anything is launched; on any
 *    error nothing is launched and no output is touched.  A launch failure
 *    reported by the runtime returns GDN_ERR_LAUNCH.  Faults inside a kernel
 *    surface at the caller's next synchronisation, as for any HIP kernel.
 *  - No C++ exception crosses this interface.
 *  - Supported head sizes: d_k, d_v in {16, 32, 64, 128}.
 *  - q and k are expected L2-normalised per token (the mixer normalises them
 *    before the recurrence); alpha and beta are expected in [0, 1].  Neither
 *    is checked or clamped.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,        /* a required pointer is NULL                     */
    GDN_ERR_SHAPE = 2,       /* a size is negative / zero where it must not be */
    GDN_ERR_DTYPE = 3,       /* unknown dtype code                             */
    GDN_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned               */
    GDN_ERR_UNSUPPORTED = 5, /* head size outside {16, 32, 64, 128}, or a size
                                whose element count overflows the indexing     */
    GDN_ERR_LAUNCH = 6,      /* the HIP runtime rejected the kernel launch     */
    GDN_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than required        */
    GDN_ERR_DEVICE = 8       /* reported by gdn_prefill_status: the call wrote
                                non-finite y or state values                   */
} gdn_status;

typedef enum {
    GDN_F32 = 0,             /* IEEE float32                                   */
    GDN_BF16 = 1             /* bfloat16                                       */
} gdn_dtype;

/*
 * Chunked prefill over T tokens (slinene page, Module A: the recurrence above,
 * evaluated 64 tokens at a time in its chunkwise form).
 *
 *   q, k          [B, T, H, d_k]  qkv_dtype
 *   v             [B, T, H, d_v]  qkv_dtype
 *   alpha, beta   [B, T, H]       float32, decay and write strength per token
 *   initial_state [B, H, d_k, d_v] float32, or NULL for a zero state
 *   final_state   [B, H, d_k, d_v] float32 out, or NULL to skip; may be the
 *                 same pointer as initial_state (updated in place)
 *   y             [B, T, H, d_v]  float32 out (may be NULL only when T == 0)
 *   scale         multiplies y (1.0: the pages apply no query scaling)
 *   workspace     device scratch of at least gdn_prefill_workspace_bytes(...)
 *                 bytes (may be NULL when that is 0); owned by the caller, its
 *                 contents are overwritten and are meaningless afterwards.  A
 *                 workspace must not be shared by calls that can overlap.
 *
 * With qkv_dtype == GDN_BF16 the dense chunk products run on fp16 MFMA with
 * float32 accumulation and a float32 state; with GDN_F32 they run on float32
 * MFMA.  T may be any value >= 0 (T == 0 copies the initial state).  B * H
 * must not exceed 65535.
 *
 * Range of the bf16 path.  q, k and v are converted to fp16 operands: bf16
 * values of magnitude 2^-14 .. 65504 convert exactly, smaller ones become
 * fp16 subnormals (losing low bits) or zero below 2^-25, larger ones become
 * infinite.  The state S, the residual V - gamma K S, the misses E and the
 * intra-chunk matrices also pass through fp16 operands, so |v|, the state's
 * entries and |y| must stay well below 65504 (of order 10^3 or less keeps the
 * products finite); unit-norm q and k keep the intra-chunk matrices small.
 * The float32 path has no such limit.
 */
gdn_status gdn_prefill_fwd(const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta,
                           const float* initial_state, float* final_state, float* y,
                           int B, int T, int H, int d_k, int d_v,
                           gdn_dtype qkv_dtype, float scale,
                           void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Workspace bytes gdn_prefill_fwd needs for these sizes (0 for GDN_F32 and
 * for T == 0), or 0 with an invalid argument (the call reports the error).
 */
size_t gdn_prefill_workspace_bytes(int B, int T, int H, int d_k, int d_v, gdn_dtype qkv_dtype);

/*
 * gdn_prefill_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The scratch that gdn_prefill_fwd takes as `workspace` lives instead in a
 * static device array of GDN_PREFILL_NOALLOC_SCRATCH_BYTES (128 MiB) that the
 * library holds on each GPU it runs on until the process ends; the call
 * allocates nothing.  Arguments, layouts and results are those of
 * gdn_prefill_fwd (the same kernels run); the caller passes every input and
 * output.  Returns GDN_ERR_WORKSPACE when gdn_prefill_workspace_bytes(...) for
 * these sizes exceeds the array (bf16: 256 bytes plus 7,168 bytes per
 * (sequence, head, 64-token chunk), i.e. B * H * ceil(T / 64) up to 18,724),
 * GDN_ERR_LAUNCH if the array's device address cannot be obtained.  All calls
 * on one GPU share its array, which keeps the last call's contents: calls that
 * can overlap on one GPU (different streams, or host threads) race and must
 * not be issued.
 */
#define GDN_PREFILL_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
gdn_status gdn_prefill_fwd_noalloc(const void* q, const void* k, const void* v,
                                   const float* alpha, const float* beta,
                                   const float* initial_state, float* final_state, float* y,
                                   int B, int T, int H, int d_k, int d_v,
                                   gdn_dtype qkv_dtype, float scale, void* hip_stream);

/*
 * Device status of the last gdn_prefill_fwd call (with qkv_dtype GDN_BF16 and
 * T > 0) that used this workspace.  The chunk walk notes whether it wrote any
 * non-finite y or final-state value in a status word at the start of the
 * workspace (the next call on the workspace clears it).  With finite inputs
 * that only happens when an input or intermediate leaves the fp16 operand
 * range of the bf16 path (see gdn_prefill_fwd), so a caller that cannot bound
 * its inputs can check here instead of scanning the outputs.
 *
 * Synchronises hip_stream, then returns GDN_OK, or GDN_ERR_DEVICE when a
 * non-finite value was written (GDN_ERR_NULL / GDN_ERR_ALIGN for a bad
 * pointer, GDN_ERR_LAUNCH if the runtime fails).
 */
gdn_status gdn_prefill_status(const void* workspace, void* hip_stream);

/*
 * One decode step for N live sequences (slinene page, Module A, one step of the
 * recurrence; the step is bound by moving the state, not by arithmetic, as
 * the rainbus digest notes for decoding).
 *
 *   q, k          [N, H, d_k]  qkv_dtype
 *   v             [N, H, d_v]  qkv_dtype
 *   alpha, beta   [N, H]       float32
 *   state         [N, H, d_k, d_v] float32, read and updated in place
 *   y             [N, H, d_v]  float32 out
 */
gdn_status gdn_decode_step(const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta,
                           float* state, float* y,
                           int N, int H, int d_k, int d_v,
                           gdn_dtype qkv_dtype, float scale, void* hip_stream);

/*
 * Gated zero-centred RMSNorm epilogue (slinene page, Module A: sigmoid gate
 * times RMSNorm of the mixer output, RMSNorm weight stored as an offset w
 * from one), per row of d_v values:
 *
 *     out = sigmoid(z) * y / sqrt(mean(y^2) + eps) * (1 + w)
 *
 *   y       [rows, d_v]  float32 (e.g. the prefill output viewed as B*T*H rows)
 *   z       [rows, d_v]  io_dtype
 *   weight  [d_v]        float32 offsets w, or NULL for w = 0
 *   out     [rows, d_v]  io_dtype
 *   eps     > 0 recommended (1e-6); rows >= 0.
 */
gdn_status gdn_gated_rmsnorm(const float* y, const void* z, const float* weight,
                             float eps, void* out, long rows, int d_v,
                             gdn_dtype io_dtype, void* hip_stream);

/*
 * Front end of the mixer (slinene page, Module A, parameterisation block; the
 * mixer figure of the rainbus digest): the recurrence inputs from the
 * projected streams, per (b, t, h):
 *
 *     q = L2Norm(SiLU(ShortConv(q_proj)))       k = L2Norm(SiLU(ShortConv(k_proj)))
 *     v = SiLU(ShortConv(v_proj))
 *     beta = sigmoid(b_logit)    alpha = exp(-exp(A[h]) * softplus(a_logit + b_alpha[h]))
 *
 * ShortConv is a causal depthwise convolution over time with one filter of
 * conv_width taps per (head, channel) and no bias:
 *     conv_t[c] = sum_{j < W} conv[h][c][j] * x_{t-W+1+j}[c]
 * L2Norm(x) = x / sqrt(sum_c x[c]^2 + norm_eps).  SiLU(x) = x * sigmoid(x).
 *
 *   q_proj, k_proj     [B, T, H, d_k]  io_dtype
 *   v_proj             [B, T, H, d_v]  io_dtype
 *   conv_q, conv_k     [H, d_k, conv_width] float32;  conv_v [H, d_v, conv_width]
 *   a_logit, b_logit   [B, T, H] float32
 *   A, b_alpha         [H] float32
 *   q_hist, k_hist, v_hist  [B, conv_width - 1, H, d] io_dtype: the rows just
 *                      before t = 0 (a previous segment's last rows), or NULL
 *                      for zeros (the sequence starts at t = 0)
 *   q, k, v            outputs, same shapes and dtype as the projections
 *   alpha, beta        [B, T, H] float32 outputs
 *   conv_width in 1..4; norm_eps >= 0 (1e-6 recommended).  The outputs feed
 *   gdn_prefill_fwd / gdn_decode_step directly.
 */
gdn_status gdn_frontend_fwd(const void* q_proj, const void* k_proj, const void* v_proj,
                            const float* conv_q, const float* conv_k, const float* conv_v,
                            const float* a_logit, const float* b_logit, const float* A, const float* b_alpha,
                            const void* q_hist, const void* k_hist, const void* v_hist,
                            void* q, void* k, void* v, float* alpha, float* beta,
                            int B, int T, int H, int d_k, int d_v, int conv_width,
                            gdn_dtype io_dtype, float norm_eps, void* hip_stream);

/*
 * Multi-token decode, both parts in one pass over the state: commit the
 * accepted prefix of the previous verified block (exactly as
 * gdn_decode_mtp_commit with prev_k, prev_alpha, prev_beta, prev_e,
 * prev_accepted and K_prev), then verify the new block from the committed
 * state (exactly as gdn_decode_mtp_verify, without prefix states).  The state
 * is read once and written once (not at all for sequences with nothing
 * accepted), so a draft round costs one state round trip instead of three.
 *
 *   q, k, v, alpha, beta   the new block, [N, K, H, ...] as for verify
 *   state                  [N, H, d_k, d_v] float32, updated in place by the commit
 *   y, e                   the new block's outputs and misses (e may be NULL).
 *                          e may be the same buffer as prev_e only when
 *                          K == K_prev (each workgroup then reads its rows of
 *                          prev_e before writing the same rows of e); that
 *                          aliasing with K != K_prev returns GDN_ERR_SHAPE.
 *                          Otherwise e and prev_e must not overlap.
 *   prev_*                 the previous block, [N, K_prev, H, ...], and its
 *                          accepted counts [N] int32 (clamped to 0..K_prev)
 *   K, K_prev in 1..8.
 */
gdn_status gdn_decode_mtp_commit_verify(const void* q, const void* k, const void* v,
                                        const float* alpha, const float* beta,
                                        float* state, float* y, float* e,
                                        const void* prev_k, const float* prev_alpha, const float* prev_beta,
                                        const float* prev_e, const int* prev_accepted,
                                        int N, int K, int K_prev, int H, int d_k, int d_v,
                                        gdn_dtype qkv_dtype, float scale, void* hip_stream);

/*
 * Backward of gdn_prefill_fwd (the chain rule through the delta form of the
 * slinene page, Module A; the pages mention a backward kernel only as part
 * of the FlashQLA library).  For the loss L = sum <dy, y> + <d_final_state,
 * final_state> it returns the gradients with respect to q, k, v, alpha, beta
 * and the initial state, evaluated in 64-token chunks.
 *
 *   q, k, v, alpha, beta, initial_state   as for gdn_prefill_fwd (initial_state NULL = zeros)
 *   dy             [B, T, H, d_v]  float32, the gradient of y
 *   d_final_state  [B, H, d_k, d_v] float32 or NULL (zero)
 *   dq, dk         [B, T, H, d_k]  float32 out
 *   dv             [B, T, H, d_v]  float32 out
 *   dalpha, dbeta  [B, T, H]       float32 out (dalpha is 0 where log(alpha)
 *                                  is below the forward's floor of -30)
 *   d_initial_state [B, H, d_k, d_v] float32 out, or NULL (not written)
 *   workspace      caller-owned device memory of at least
 *                  gdn_prefill_bwd_workspace_bytes(...) bytes, 16-byte aligned
 *                  (per 64-token chunk and head: the chunk's T, P and M
 *                  matrices, its start state and end-state gradient, and two
 *                  64 x d_v products, each in a float32-sized slot; for bf16
 *                  inputs with d >= 64 the states, products, T and a copy of P
 *                  are kept as fp16 in the first half of their slots)
 *   d_k == d_v in {16, 32, 64, 128}.  With T == 0 only d_initial_state is
 *   written (a copy of d_final_state, or zeros); no workspace is needed.
 */
gdn_status gdn_prefill_bwd(const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, const float* initial_state,
                           const float* dy, const float* d_final_state,
                           float* dq, float* dk, float* dv, float* dalpha, float* dbeta,
                           float* d_initial_state,
                           int B, int T, int H, int d_k, int d_v,
                           gdn_dtype qkv_dtype, float scale,
                           void* workspace, size_t workspace_bytes, void* hip_stream);

/* Workspace bytes gdn_prefill_bwd needs (0 for T == 0 or invalid arguments). */
size_t gdn_prefill_bwd_workspace_bytes(int B, int T, int H, int d_k, int d_v, gdn_dtype qkv_dtype);

/*
 * Multi-token (speculative) decode, part 1: verify a block of K draft tokens
 * per sequence from the live states (rainbus digest, prerequisites section,
 * the paragraph on multi-token prediction and speculative decoding: drafts are
 * verified by the main model; each draft token is one step of the delta form,
 * slinene page, Module A).  For t = 0 .. K-1,
 * starting from S = state:
 *     e_t = v_t - (alpha_t S)^T k_t;   S = alpha_t S + beta_t k_t e_t^T;
 *     y_t = scale * S^T q_t
 * The live state is read once and NOT modified.
 *
 *   q, k           [N, K, H, d_k]  qkv_dtype  (token t of sequence n: row (n K + t) H + h)
 *   v              [N, K, H, d_v]  qkv_dtype
 *   alpha, beta    [N, K, H]       float32
 *   state          [N, H, d_k, d_v] float32, read only
 *   y              [N, K, H, d_v]  float32 out
 *   e              [N, K, H, d_v]  float32 out: the misses e_t, the input of
 *                  gdn_decode_mtp_commit; NULL = not written
 *   prefix_states  [N, K, H, d_k, d_v] float32 out: S after each draft token
 *                  (K state writes: only for callers that keep snapshots);
 *                  NULL = not written
 *   K in 0..8 (K == 0: nothing to do); other sizes as gdn_decode_step.
 */
gdn_status gdn_decode_mtp_verify(const void* q, const void* k, const void* v,
                                 const float* alpha, const float* beta,
                                 const float* state, float* y, float* e, float* prefix_states,
                                 int N, int K, int H, int d_k, int d_v,
                                 gdn_dtype qkv_dtype, float scale, void* hip_stream);

/*
 * Multi-token decode, part 2: advance each live state by the accepted prefix
 * of its verified block, which rolls back the rejected drafts:
 *     for t < accepted[n]:  S = alpha_t S + beta_t k_t e_t^T
 * with the e_t that gdn_decode_mtp_verify wrote for the same block.  The
 * result is exactly that call's prefix state after accepted[n] tokens; one
 * read and one write of the state per sequence with accepted[n] > 0, nothing
 * for sequences with accepted[n] == 0.
 *
 *   k              [N, K, H, d_k]  qkv_dtype (the block's keys)
 *   alpha, beta    [N, K, H]       float32
 *   e              [N, K, H, d_v]  float32 (from gdn_decode_mtp_verify)
 *   accepted       [N] int32 in device memory; values are clamped to 0..K
 *   state          [N, H, d_k, d_v] float32, updated in place
 */
gdn_status gdn_decode_mtp_commit(const void* k, const float* alpha, const float* beta,
                                 const float* e, const int* accepted, float* state,
                                 int N, int K, int H, int d_k, int d_v,
                                 gdn_dtype qkv_dtype, void* hip_stream);

/*
 * QSA indexer, part 1 (slinene page, Module B: the compressed MQA indexer):
 * the indexer operands from the projected streams, per sequence of n tokens
 * with block size r:
 *     q[i][h]  = PRoPE(RMSNorm(q_proj[i][h]), i)
 *     kbar[b]  = PRoPE(RMSNorm(mean(k_proj[b r .. b r + r - 1])), b r),  b < n / r
 * (keys are pooled before the rotation).  RMSNorm(x) = x / sqrt(mean(x^2) + eps)
 * times the weight (NULL = 1).  PRoPE turns the first rope_dims entries in
 * rotate-half pairs (j, j + rope_dims / 2) by pos * rope_base^(-2 j / rope_dims).
 *
 *   q_proj    [B, n, H, D]  io_dtype        k_proj   [B, n, D] io_dtype
 *   q_weight, k_weight  [D] float32 or NULL
 *   q_out     [B, n, H, D]  io_dtype out    kbar_out [B, n / r, D] io_dtype out
 *   D in {32, 64, 128}; 0 <= rope_dims <= D, even; r >= 1; eps >= 0.
 */
gdn_status gdn_qsa_prep(const void* q_proj, const void* k_proj,
                        const float* q_weight, const float* k_weight,
                        void* q_out, void* kbar_out,
                        int B, int n, int H, int D, int r, int rope_dims,
                        float rope_base, float eps, gdn_dtype io_dtype, void* hip_stream);

/*
 * QSA indexer, part 2 (slinene page, Module B: block-causal scoring and
 * top-K block selection): for query i the candidates are the complete blocks
 * b < (i + 1) / r (b r + r - 1 <= i), scored
 *     I[i][b] = sum_h ReLU(<q[i][h], kbar[b]>)
 * and the K_B = ceil(K / r) best are selected (all of them when there are
 * fewer; equal scores are broken towards the later block).  The tail tokens of
 * the current incomplete block are always attended and are not listed.
 *
 *   q            [B, n, H, D]  dtype (the output of gdn_qsa_prep)
 *   kbar         [B, n / r, D] dtype
 *   block_idx    [B, n, K_B]   int32 out: selected blocks in ascending order,
 *                padded with -1
 *   workspace    caller-owned, >= gdn_qsa_select_workspace_bytes(...) bytes,
 *                16-byte aligned.  H = 4 keeps no scores: per query 16
 *                candidate sub-lists of K_B / 16 + 96 (bits, block) pairs
 *                plus a little bookkeeping (B n 16 (K_B / 16 + 96) 8 bytes in
 *                all), and 256 scratch rows of ceil(n / r / 64) 64 floats.
 *                Other H store the fp32 block scores,
 *                B n ceil(n / r / 64) 64 4 bytes.
 *   D in {32, 64, 128}; r >= 1; K >= 1.
 */
gdn_status gdn_qsa_select(const void* q, const void* kbar, int* block_idx,
                          int B, int n, int H, int D, int r, int K,
                          gdn_dtype dtype, void* workspace, size_t workspace_bytes, void* hip_stream);

/* Workspace bytes gdn_qsa_select needs (0 for invalid arguments). */
size_t gdn_qsa_select_workspace_bytes(int B, int n, int H, int D, int r, int K, gdn_dtype dtype);

/* Static, never-NULL description of a status code. */
const char* gdn_status_string(gdn_status status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
