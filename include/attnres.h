/*
 * attnres.h -- C ABI of libattnres.so: the Attention Residuals (AttnRes)
 * depth-routing hot path on AMD Instinct MI355X (gfx950).
 *
 * For every token t and every destination sublayer l, a learned pseudo-query
 * w_l scores each stored depth source v_i as s = w_l . (g * RMSNorm(v_i)); a
 * softmax over depth turns the scores into weights alpha_{i->l}; the output is
 * h_l = sum_i alpha_{i->l} v_i over the UN-normalised sources.
 *   Definitions: b-lab.team summary of "Attention Residuals", §1 (Full) and
 *   §2 (Block); ai-systems-engineering.com "Attention Residuals" explainer,
 *   learned-query section (RMSNorm only on the score side, gain, RMS = root
 *   mean square); chatpaper.ai "Multi-Head Attention Residuals" abstract (H
 *   heads, each with its own depth softmax; H = 1 is AttnRes).
 *
 * Conventions shared by every call
 * --------------------------------
 *  Memory     Every tensor argument is a DEVICE pointer owned by the caller.
 *             The library never allocates, frees, copies between host and
 *             device, or synchronises.  All work is enqueued on `stream`.
 *  Layout     Row-major, contiguous, channel (d) fastest.  A stack of sources
 *             [n, T, d] holds source s at base + s*T*d elements.
 *  dtype      ATTNRES_F32 or ATTNRES_BF16, applied to every activation-shaped
 *             tensor of the call (sources, partials, outputs, dh, source
 *             gradients).  Arithmetic is fp32 throughout.
 *  Parameters w (pseudo-queries), gain, lse, dw, dgain are always fp32.
 *             gain: gain_ld == d -> one [d] vector per destination ([n_dst,d]);
 *                   gain_ld == 0 -> one shared [d] vector;
 *                   gain == NULL -> gain is all ones (gain_ld ignored).
 *  Scalars    eps >= 0 and finite (RMSNorm: x / sqrt(mean(x^2) + eps)).
 *             H >= 1, d % H == 0; head h owns channels [h*d/H, (h+1)*d/H).
 *  Status     0 on success, negative on error (ATTNRES_ERR_*).  Every
 *             argument is checked before any HIP call, so a call that fails
 *             validation enqueues nothing.  attnres_last_error() returns a
 *             thread-local message describing the last failure.
 *  Empty      T == 0 is valid and enqueues nothing, except that the two
 *             backward calls with accumulate == 0 still write zeros to dw and
 *             dgain.
 *  Aliasing   Outputs must not overlap inputs, except where a call says so.
 *  Determinism  Identical inputs, shapes and device give bit-identical
 *             outputs (no floating-point atomics).
 */
#ifndef ATTNRES_H
#define ATTNRES_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* I/O dtypes.  fp32 I/O runs the general kernels at every shape: exact to
 * fp32 rounding, but far slower than bf16 at the large shapes (measured on one
 * MI355X: 11.5 ms for a d = 4096, N = 8, S = 4 block step over 16384 tokens
 * against 0.52 ms in bf16; 16.1 ms for Full over 32 sources and destinations,
 * T = 4096, d = 2048, against 0.26 ms).  attnres_kernel_variant names the
 * kernel a call would run. */
#define ATTNRES_F32 0
#define ATTNRES_BF16 1
/* Phase-1 state format only (o_dtype, with bf16 I/O): fp16 values scaled per
 * token by a power of two, o = stored * o_scale[t].  o_scale[t] = 2^e is
 * chosen from the bound |o| <= max_i ||b_i||_2 so that every stored value is
 * below 32768 in magnitude and the bound sits in [16384, 32768): no fp16
 * overflow for any finite input, and 11 significant bits for the state
 * (bf16 keeps 8).  Requires each rep's sum of squares to be finite in fp32.
 * A bf16 state is refused (ATTNRES_ERR_UNSUPPORTED): its 8 bits, rounded
 * once more by the merge, exceed the bf16 tolerance at full size. */
#define ATTNRES_F16 2

/* Operations named by attnres_kernel_variant. */
#define ATTNRES_OP_PHASE1 0   /* attnres_block_phase1 (N reps, S sublayers)       */
#define ATTNRES_OP_PHASE2 1   /* attnres_block_phase2_merge                       */
#define ATTNRES_OP_BWD 2      /* attnres_bwd (N reps, S sublayers)                */
#define ATTNRES_OP_FULL_FWD 3 /* attnres_full_fwd (N = n_src, S = n_dst)          */
#define ATTNRES_OP_FULL_BWD 4 /* attnres_full_bwd (N = n_src, S = n_dst)          */

#define ATTNRES_OK 0
#define ATTNRES_ERR_INVALID (-1)     /* bad pointer, size, flag, or aliasing   */
#define ATTNRES_ERR_UNSUPPORTED (-2) /* valid request outside built kernels    */
#define ATTNRES_ERR_HIP (-3)         /* HIP launch or runtime error            */
#define ATTNRES_ERR_WORKSPACE (-4)   /* workspace missing or too small         */

/*
 * Full AttnRes forward (b-lab.team summary §1: h_l = sum_{i=0}^{l-1}
 * alpha_{i->l} v_i, v_0 the embedding, v_i the sublayer outputs).
 *
 *  src   [n_src, T, d] dtype   depth sources v_0 .. v_{n_src-1}
 *  w     [n_dst, d] fp32       pseudo-queries of the destinations
 *  gain  see conventions (per-destination rows of length d, shared, or NULL)
 *  out   [n_dst, T, d] dtype   out[j] reads sources 0 .. n_src - n_dst + j
 *
 *  ws    device workspace of at least attnres_full_fwd_workspace_size() bytes
 *        (may be NULL when that size is 0); its contents are scratch
 *
 * With n_dst == n_src == L, destination l = j + 1 reads v_0 .. v_{l-1}; with
 * n_dst == 1 it is the single call a model makes per sublayer.
 * Requires 1 <= n_dst <= n_src <= 64.
 */
int attnres_full_fwd(const void* src, int64_t n_src, int64_t T, int64_t d,
                     const float* w, int64_t n_dst, const float* gain, int64_t gain_ld,
                     float eps, int32_t H, int32_t dtype, void* out, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/*
 * Bytes of device workspace attnres_full_fwd needs.  bf16 calls with n_src <=
 * 32 and either one head or H = 2, 4 or 8 heads with d = 512 .. 2048 in steps
 * of 512 may run the contractions on the matrix cores, which take q = w * gain
 * as a bf16 high part plus a bf16 low part ([2, 32, d] bf16, 128 * d bytes).
 * So may one-head bf16 calls with 33 .. 64 sources and d a multiple of 512:
 * [2, 32, d] for n_dst <= 32, [2, 64, d] (256 * d bytes) above.  Every other
 * request needs none and gets 0.  (One destination over up to 64 sources
 * with d <= 4096, and H = 1, 2, 4 or 8 with d / H a multiple of 512 (or of
 * 256 with d <= 2048), runs a vector kernel that ignores the workspace; the
 * size returned still covers the matrix-core kernels, so a caller need not
 * know which runs.)
 */
size_t attnres_full_fwd_workspace_size(int64_t n_src, int64_t n_dst, int64_t d, int32_t H,
                                       int32_t dtype);

/*
 * Block AttnRes, Phase 1 of two-phase inference (b-lab.team summary §3,
 * Inference; dimensionstp "Attention Residuals Review" §3-2 (4)): the S
 * pseudo-queries of one block against the N cached block representations
 * b_0 .. b_{N-1}, reading each representation once for all S queries.  For
 * sublayer l, o_l = sum_i alpha_{l,i} b_i with alpha the softmax over the reps
 * only (per head).
 *
 *  reps     [N, T, d] dtype
 *  w        [S, d] fp32;  gain as in the conventions (rows per sublayer)
 *  h_first  [T, d] dtype: o_1, already the final input of the block's first
 *           sublayer (its source set has no partial sum)
 *  o_state  [S-1, T, d] in o_dtype: o_2 .. o_S, the state Phase 2 merges
 *           (may be NULL when S == 1)
 *  o_dtype  ATTNRES_F32, or ATTNRES_F16 (bf16 I/O only; see its
 *           definition).  The merge rounds the state once more, so the
 *           state's precision adds to the error: fp32 adds nothing, the scaled
 *           fp16 state about 2^-12 of the value.
 *  lse      [S, H, T] fp32: lse_l = max_i s_i + log sum_i exp(s_i - max_i s_i)
 *  o_scale  [T] fp32, written when o_dtype == ATTNRES_F16 (else may be NULL)
 * Requires 1 <= N <= 63, S >= 1.
 */
int attnres_block_phase1(const void* reps, int64_t N, int64_t T, int64_t d,
                         const float* w, int64_t S, const float* gain, int64_t gain_ld,
                         float eps, int32_t H, int32_t dtype, void* h_first,
                         void* o_state, int32_t o_dtype, float* lse, float* o_scale,
                         hipStream_t stream);

/*
 * Block AttnRes, Phase 2 for sublayer i >= 2 of a block (b-lab.team summary
 * §2 value matrix, §3 Inference; Review §3-2 (4) exact online-softmax merge):
 * score the intra-block partial sum p = b^{(n)}_{i-1} and merge it with
 * Phase 1's state by online softmax, per head:
 *   s_p = w_i . (g_i * RMSNorm(p)),  m = max(lse_i, s_p),
 *   h_i = (exp(lse_i - m) o_i + exp(s_p - m) p) / (exp(lse_i - m) + exp(s_p - m)).
 *
 *  o_i      [T, d] in o_dtype                 Phase 1 state row i
 *  o_scale  [T] fp32 when o_dtype == ATTNRES_F16 (Phase 1's o_scale), else ignored
 *  lse_i    [H, T] fp32                       Phase 1 statistics row i
 *  partial  [T, d] dtype
 *  w_i      [d] fp32;  gain_i [d] fp32 or NULL (ones)
 *  h_i      [T, d] dtype.  h_i may equal o_i when the state's element has
 *           the I/O size (fp32 state with fp32 I/O, scaled fp16 state with
 *           bf16 I/O): every element is read before it is written (in place).
 */
int attnres_block_phase2_merge(const void* o_i, int32_t o_dtype, const float* o_scale,
                               const float* lse_i, const void* partial, int64_t T, int64_t d,
                               const float* w_i, const float* gain_i, float eps, int32_t H,
                               int32_t dtype, void* h_i, hipStream_t stream);

/*
 * Phase 2 fused with the intra-block partial-sum update and the next
 * sublayer's PreNorm statistic (b-lab.team summary §2: the partial sum is the
 * running sum of the block's sublayer outputs; §3 Inference and Review §3-2 (4):
 * the merge is the fused step of two-phase inference).  One pass over the
 * token rows:
 *   p = partial_prev + f_prev  (f_prev alone when partial_prev is NULL, the
 *       block's first update), rounded once to dtype and stored to partial_out;
 *   h_i = attnres_block_phase2_merge(o_i, ..., p, ...) exactly as above, from
 *       the stored p;
 *   h_inv_rms[t] = 1 / sqrt(mean_c h_i[t][c]^2 + norm_eps), over the stored h_i
 *       (the scale an RMSNorm applied to h_i uses; not written when NULL).
 *
 *  partial_prev [T, d] dtype or NULL;  f_prev [T, d] dtype (the output of
 *               sublayer i-1)
 *  partial_out  [T, d] dtype; may equal partial_prev (in place), must not
 *               otherwise overlap an input or another output
 *  h_i          [T, d] dtype; may equal o_i when the state's element has the
 *               I/O size (as attnres_block_phase2_merge)
 *  h_inv_rms    [T] fp32 or NULL;  norm_eps finite and >= 0 when it is used
 * Other arguments as for attnres_block_phase2_merge.
 */
int attnres_block_phase2_merge_update(const void* o_i, int32_t o_dtype, const float* o_scale,
                                      const float* lse_i, const void* partial_prev,
                                      const void* f_prev, int64_t T, int64_t d, const float* w_i,
                                      const float* gain_i, float eps, int32_t H, int32_t dtype,
                                      void* partial_out, void* h_i, float norm_eps,
                                      float* h_inv_rms, hipStream_t stream);

/*
 * Bytes of device workspace mhar_fwd needs: the statistics ([S, H, T] fp32)
 * and the per-token state scale ([T] fp32), each aligned to 256 bytes (the
 * Phase-1 state itself lives in h; see mhar_fwd).  Returns 0 for invalid
 * sizes.
 */
size_t mhar_fwd_workspace_size(int64_t N, int64_t S, int64_t T, int64_t d, int32_t H);

/*
 * One block of multi-head Block AttnRes routing (chatpaper.ai "Multi-Head
 * Attention Residuals" abstract; H = 1 is Block AttnRes): exactly the launches
 * of attnres_block_phase1 (h_first = h[0]; the state of sublayer i >= 2
 * written into h[i-1] itself: the scaled fp16 state ATTNRES_F16 for bf16 I/O,
 * fp32 for fp32 I/O) followed by the S-1 attnres_block_phase2_merge calls for
 * sublayers 2..S, in order, each in place (h_i == o_i = h[i-1]).
 *
 *  reps      [N, T, d] dtype            b_0 .. b_{N-1}
 *  partials  [S-1, T, d] dtype          partials[k] = b^{(n)}_{k+1}, the sum
 *            of the block's first k+1 sublayer outputs (NULL allowed if S == 1)
 *  w         [S, d] fp32;  gain as in the conventions (rows per sublayer)
 *  h         [S, T, d] dtype            h[i-1] is the input of sublayer i
 *  ws        device workspace of at least mhar_fwd_workspace_size() bytes
 * Requires 1 <= N <= 63.
 */
int mhar_fwd(const void* reps, int64_t N, const void* partials, int64_t S, int64_t T, int64_t d,
             const float* w, const float* gain, int64_t gain_ld, float eps, int32_t H,
             int32_t dtype, void* h, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * mhar_fwd over the tokens in chunks of chunk_T (the last chunk may be
 * shorter), for a workspace bounded by the chunk instead of the sequence
 * (b-lab.team summary §3 Inference: prefill may run in chunks; tokens never
 * interact in the routing, so the result is bit-identical to mhar_fwd).
 * Each chunk is one Phase 1 launch and S - 1 merge launches, in token order,
 * on the stream.
 *
 *  ws  device workspace of at least
 *      mhar_fwd_workspace_size(N, S, min(T, chunk_T), d, H) bytes
 * Other arguments as for mhar_fwd; chunk_T >= 1.
 */
int mhar_fwd_chunked(const void* reps, int64_t N, const void* partials, int64_t S, int64_t T,
                     int64_t d, const float* w, const float* gain, int64_t gain_ld, float eps,
                     int32_t H, int32_t dtype, void* h, int64_t chunk_T, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/*
 * mhar_fwd for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same launches as
 * mhar_fwd, with the workspace -- the statistics and per-token scales, the
 * bytes mhar_fwd_workspace_size() reports -- in a static scratch array the
 * library owns on each device (ATTNRES_NOALLOC_SCRATCH_BYTES, held from the
 * device's first use until the process ends).  Allocates nothing: no
 * hipMalloc, hipFree or allocating library call.  A request needing more than
 * the array returns ATTNRES_ERR_UNSUPPORTED before any HIP call (for S = 4,
 * H = 1 the limit is about 400K tokens per call; chunk longer sequences or use
 * mhar_fwd).  Every call on one device shares that device's array: calls that
 * overlap in time on one device (other streams, concurrent graph replays)
 * race and must not be issued.  Nothing in the array needs clearing: each
 * call writes every value it reads.  Other arguments as for mhar_fwd.
 */
#define ATTNRES_NOALLOC_SCRATCH_BYTES (8u << 20)
int mhar_fwd_noalloc(const void* reps, int64_t N, const void* partials, int64_t S, int64_t T, int64_t d,
                     const float* w, const float* gain, int64_t gain_ld, float eps, int32_t H,
                     int32_t dtype, void* h, hipStream_t stream);

/*
 * Bytes of device workspace attnres_bwd needs (fp32 partial sums of the
 * pseudo-query gradient, one [S, d] slab per slot, min(T, 1024) slots).  With
 * S > 4 it also holds the rep gradients of the block's first destinations in
 * fp32 ([N, T, d], 4 N T d bytes): such a block runs as two chunks of at most
 * 4 destinations, and the second adds its rep gradients to the first's before
 * the one rounding to the I/O dtype.
 */
size_t attnres_bwd_workspace_size(int64_t N, int64_t S, int64_t T, int64_t d, int32_t H);

/*
 * Backward of mhar_fwd: gradients of L = sum_j <dh_j, h_j> with respect to the
 * reps, the partial sums, the pseudo-queries and the RMSNorm gain.  The pages
 * give no backward; this is the analytic gradient of the forward definition:
 * with x_i = RMSNorm(v_i), r_i = 1/sqrt(mean v_i^2 + eps), q_j = w_j * g_j,
 *   a = dh_j . v_i (per head), c = alpha (a - sum alpha a),
 *   dv_i = sum_j [alpha dh_j + r_i c q_j] - r_i x_i sum_{j,h} c s / d,
 *   dw_j = g_j * Z_j, dg_j = w_j * Z_j, Z_j = sum_{t,i} c x_i.
 *
 *  dh          [S, T, d] dtype   upstream gradient of h
 *  d_reps      [N, T, d] dtype   d_partials [S-1, T, d] dtype (NULL if S == 1)
 *  dw          [S, d] fp32
 *  dgain       [S, d] fp32 (gain_ld == d) or [d] (gain_ld == 0); ignored and
 *              may be NULL when gain == NULL
 *  accumulate  0: overwrite the four outputs; 1: add into them (reps are read
 *              by later blocks too, so their gradients accumulate)
 *  ws          device workspace of at least attnres_bwd_workspace_size() bytes
 * Requires 1 <= N, N + S - 1 <= 64, S * H * (N + 1) <= 1024 on the general
 * path.  The specialised kernel takes bf16 with N <= 12, S <= 8, d a multiple
 * of 512 up to 4096 and H in {1, 2, 4, 8} dividing d / 512; with S > 4 it runs
 * as two launches over the first ceil(S/2) and the remaining destinations.
 */
int attnres_bwd(const void* reps, int64_t N, const void* partials, int64_t S, int64_t T, int64_t d,
                const float* w, const float* gain, int64_t gain_ld, float eps, int32_t H,
                int32_t dtype, const void* dh, void* d_reps, void* d_partials, float* dw,
                float* dgain, int32_t accumulate, void* ws, size_t ws_bytes, hipStream_t stream);

/* Thread-local message for the last failing call on this thread ("" if none). */
const char* attnres_last_error(void);

/*
 * Bytes of device workspace attnres_full_bwd needs (fp32 partial sums of the
 * query and gain gradients, one [n_dst, d] slab per wavefront, at most 1024
 * slabs), or of the matrix-core path if larger; 0 when T == 0 or on invalid
 * sizes.
 */
size_t attnres_full_bwd_workspace_size(int64_t n_src, int64_t n_dst, int64_t T, int64_t d,
                                       int32_t H);

/*
 * Full AttnRes backward: gradients of L = sum_j <dout_j, out_j> for out =
 * attnres_full_fwd(src, w, gain, ...) with the same arguments.  The pages
 * give no backward; this is the chain rule through the forward definition
 * (b-lab.team summary §1; ai-systems-engineering.com explainer, learned-query
 * section; chatpaper.ai MHAR abstract for heads), with destination j reading
 * the causal prefix of sources 0 .. n_src - n_dst + j.  Per token, with
 * x_i = RMSNorm(v_i), r_i its inverse RMS and q_j = w_j * g_j:
 *   c_{j,i,h} = alpha (dout_j . v_i - sum_m alpha_m dout_j . v_m)    (per head h)
 *   dv_i = sum_j (alpha_{j,i} dout_j + r_i c_{j,i} q_j) - r_i x_i sum_{j,h} c s / d
 *   dw_j = g_j * Z_j,  dgain_j = w_j * Z_j,  Z_j = sum over tokens and sources of c x_i
 *
 *  src, w, gain, eps, H, dtype   as for attnres_full_fwd
 *  dout        [n_dst, T, d] dtype     upstream gradient of out
 *  d_src       [n_src, T, d] dtype
 *  dw          [n_dst, d] fp32
 *  dgain       [n_dst, d] fp32 (gain_ld == d) or [d] (gain_ld == 0); ignored
 *              and may be NULL when gain == NULL
 *  accumulate  0: overwrite d_src, dw and dgain; 1: add into them
 *  ws          device workspace of at least attnres_full_bwd_workspace_size()
 * Requires 1 <= n_dst <= n_src <= 64, and n_dst * H * n_src <= 1024 when the
 * call runs on the general kernel.  The matrix-core kernels have no such
 * limit; they take bf16 with n_src <= 32 and one head, or H = 2, 4 or 8
 * heads of whole 256-channel runs with d = 1024 .. 2048, and bf16 with
 * 33 <= n_src <= 64, n_dst <= 32, one head and d a multiple of 512.  (One
 * destination with d a multiple of 512 runs on a vector kernel: n_src <= 32
 * with d <= 4096, or n_src <= 64 with d <= 2048; H = 1, 2, 4 or 8 with d / H
 * a multiple of 512 channels, or of 256 above 32 sources.)  dw and dgain are fixed-order sums over tokens (no atomics).
 */
int attnres_full_bwd(const void* src, int64_t n_src, int64_t T, int64_t d, const float* w,
                     int64_t n_dst, const float* gain, int64_t gain_ld, float eps, int32_t H,
                     int32_t dtype, const void* dout, void* d_src, float* dw, float* dgain,
                     int32_t accumulate, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Bytes of device workspace attnres_msar_fwd needs (0: none).  The
 * specialised bf16 path for one destination over at most 12 sources with d a
 * multiple of 512 keeps per-token partial sums and the retrieved states
 * (4 d fp32 per token) there: about 16 d + 32 n_src d / 512 + 300 bytes per
 * token.  Returns 0 for invalid sizes and for shapes the general kernel runs.
 */
size_t attnres_msar_fwd_workspace_size(int64_t n_src, int64_t n_dst, int64_t T, int64_t d,
                                       int32_t dtype);

/*
 * MSAR multi-stream depth attention (onedev.kr summary of the MSAR paper,
 * "How it differs"; "How to use it" for the on-demand expansion).  Every
 * source expands into four full-width streams, never written to memory:
 *   v^(0) = v,  v^(r)[t] = sum_{k < K_r} conv_r[k] * v[t - k]  (K = 4, 8, 12
 *   for r = 1, 2, 3; elementwise over channels; zero before the first token).
 * Destination j reads sources 0 .. n_src - n_dst + j; per stream r:
 *   s_i = w_j^(r) . RMSNorm(v_i^(r)),  alpha = softmax_i(s),
 *   Z^(r) = sum_i alpha_i v_i^(r);
 * then the H^pre mixer: beta = sigmoid(RMSNorm([Z^(0) .. Z^(3)]) P_j) and
 *   out_j = sum_r beta_r Z^(r).
 * RMSNorm is x / sqrt(mean x^2 + eps) without gain (a gain folds into w and P).
 *
 *  src   [n_src, T, d] dtype    the T tokens are the sequence from its first
 *                               token (the convolutions see zeros before it)
 *  w     [n_dst, 4, d] fp32     pseudo-queries, stream-major
 *  conv  [24, d] fp32           taps: rows 0-3 stream 1, 4-11 stream 2,
 *                               12-23 stream 3; row k of a stream multiplies
 *                               the source k tokens back; shared by the sources
 *  mix   [n_dst, 4 d, 4] fp32   P_j, row r*d + c is channel c of stream r
 *  out   [n_dst, T, d] dtype
 *  ws    device workspace of attnres_msar_fwd_workspace_size() bytes (may be
 *        NULL when that is 0)
 * Requires 1 <= n_dst <= n_src <= 64.
 */
int attnres_msar_fwd(const void* src, int64_t n_src, int64_t T, int64_t d, const float* w,
                     const float* conv, const float* mix, int64_t n_dst, float eps, int32_t dtype,
                     void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Block MSAR, two-phase ([MSAR] onedev.kr summary, "How to use it": Block MSAR
 * keeps one stream per block and expands on demand, and AttnRes's two-phase
 * computation carries over).  The streams and mixer are those of
 * attnres_msar_fwd.  Sublayer i of a block reads the N reps b_0..b_{N-1} and,
 * for i >= 2, the partial sum b_{i-1}.
 *
 * Phase 1: the S sublayers' per-stream queries against the N reps, each rep's
 * streams expanded once for all of them.  Per sublayer i and stream r:
 *   s_n = w_i^(r) . RMSNorm(v_n^(r)),  o_i^(r) = sum_n softmax_n(s)_n v_n^(r),
 *   lse_i^(r) = log sum_n exp(s_n).
 * Sublayer 1 reads the reps only, so h1 = mixer_1(o_1) is final; sublayers
 * 2..S keep o and lse for Phase 2.
 *
 *  reps     [N, T, d] bf16 (T tokens from the sequence start)
 *  w        [S, 4, d] fp32;  conv [24, d] fp32 (as attnres_msar_fwd)
 *  mix1     [4 d, 4] fp32    sublayer 1's mixer
 *  h1       [T, d] bf16
 *  o_state  [S-1, 4, T, d] fp16 and o_scale [T] fp32: the state is
 *           o_state * o_scale[t], the scale a power of two that bounds every
 *           value of the token (as the Phase-1 state of Block AttnRes)
 *  lse      [S-1, 4, T] fp32 (o_state and lse may be NULL when S == 1)
 *  ws       device workspace of attnres_block_msar_phase1_workspace_size() bytes
 * Requires bf16, 1 <= N <= 12, 1 <= S <= 4, d a multiple of 512 (else
 * ATTNRES_ERR_UNSUPPORTED) and 16-byte-aligned pointers.
 */
size_t attnres_block_msar_phase1_workspace_size(int64_t N, int64_t S, int64_t T, int64_t d);
int attnres_block_msar_phase1(const void* reps, int64_t N, int64_t T, int64_t d, const float* w,
                              int64_t S, const float* conv, const float* mix1, float eps,
                              int32_t dtype, void* h1, void* o_state, float* o_scale, float* lse,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Block MSAR Phase 2 for sublayer i >= 2: the partial's streams are scored
 * with w_i and merged into Phase 1's state by online softmax, per stream
 * (exact: the result equals attnres_msar_fwd over the reps and the partial):
 *   m = max(lse, s_p),  Z^(r) = (e^{lse-m} o^(r) + e^{s_p-m} p^(r)) / (e^{lse-m} + e^{s_p-m}),
 * then h_i = sum_r beta_r Z^(r) with beta = sigmoid(RMSNorm(Flatten(Z)) P_i).
 *
 *  o_i      [4, T, d] fp16, o_scale [T], lse_i [4, T] fp32: Phase 1's
 *           o_state[i-2], o_scale and lse[i-2]
 *  partial  [T, d] bf16 (the block's partial sum before sublayer i)
 *  w_i      [4, d];  conv [24, d];  mix_i [4 d, 4] (fp32)
 *  h_i      [T, d] bf16
 *  ws       device workspace of attnres_block_msar_phase2_workspace_size() bytes
 * Same requirements as Phase 1.
 */
size_t attnres_block_msar_phase2_workspace_size(int64_t T, int64_t d);
int attnres_block_msar_phase2(const void* o_i, const float* o_scale, const float* lse_i,
                              const void* partial, int64_t T, int64_t d, const float* w_i,
                              const float* conv, const float* mix_i, float eps, int32_t dtype,
                              void* h_i, void* ws, size_t ws_bytes, hipStream_t stream);

/* ABI version: (major << 16) | minor.  Major 2 added the Full-forward workspace;
 * minor 1 added the Full backward, minor 2 the fused Phase 2 update, minor 3 the
 * chunked block forward, minor 4 MSAR, minor 5 the two-phase Block MSAR, minor 6
 * attnres_kernel_variant (and mhar_fwd's state moved into h). */
int attnres_version(void);

/*
 * Name of the kernel a call of `op` (ATTNRES_OP_*) with these sizes would run
 * under the current kernel policy, written to buf (len bytes, truncated, NUL
 * terminated): e.g. "phase1_fast<N=8,S=4,CH=2,MH=0> B=256 lds=67712" or
 * "phase1_generic".  N and S are the rep and sublayer counts (n_src and n_dst
 * for the Full ops); o_dtype is the Phase-1 state format (ignored by the other
 * ops); every pointer is taken as 16-byte aligned.  Pure host logic: makes no
 * HIP call, so it can be used (and tested) without a GPU.  Returns 0, or
 * ATTNRES_ERR_INVALID for an unknown op or a NULL or empty buffer.
 */
int attnres_kernel_variant(int32_t op, int64_t N, int64_t S, int64_t T, int64_t d, int32_t H,
                           int32_t dtype, int32_t o_dtype, char* buf, size_t len);

/*
 * Kernel selection, process-wide.  0 (default): the specialised gfx950 kernels
 * wherever the shape allows, the general kernels elsewhere; 1: the general
 * kernels only.  Both give results within the documented tolerance; the
 * setting exists so tests can cross-check the two families on one shape.
 * Returns the previous policy, or ATTNRES_ERR_INVALID for an unknown value.
 */
int attnres_set_kernel_policy(int32_t policy);

#ifdef __cplusplus
}
#endif

#endif /* ATTNRES_H */
