/*
 * ssd.h -- C ABI of libssd.so, a Mamba-2 selective state-space (SSD) layer
 * for AMD Instinct MI355X (gfx950).
 *
 * What the layer computes (page title, then section):
 *  - The recurrence h_t = Abar_t h_{t-1} + Bbar_t x_t with read-out
 *    y_t = C_t h_t + D x_t, whose parameters depend on the input:
 *    "Hybrid Architectures for Language Models: Systematic Analysis and Design
 *    Insights" (Korean summary), section 2 Background.  The same section notes
 *    that Mamba-2's state space duality recasts this as matrix multiplies;
 *    ssd_chunk_scan_fwd computes it in that chunked form.
 *  - A depthwise causal conv (kernel 4) with SiLU in front of the scan, over
 *    the x|B|C channels: "Nemotron-H style Hybrid Mamba-Transformer 3B
 *    feasibility study", tables 1.4 and 1.5 (conv_kernel 4, activation SiLU);
 *    the conv's channel span follows the Mamba cache size
 *    2*N_L*(d_ssm*d_state + N_conv*(2*d_state + d_ssm)) in "Hybrid
 *    Architectures ..." summary, Appendix C.
 *  - Shapes: head_dim P = 64, d_state N = 128, n_groups G, chunk 128
 *    (feasibility study, table 1.4); chunks of 64 and 256 tokens are
 *    compiled too (the chunk length changes the blocking, not the result).
 *  - The decode state is of fixed size, independent of the position
 *    ("Nemotron-H paper explainer", Transformer-vs-Mamba table: O(1) compute
 *    and memory per token).
 *
 * Readings where the pages are silent:
 *  - delta_t = softplus(dt_t + dt_bias_h) if dt_softplus, else dt_t (+ dt_bias_h);
 *    Abar_t = exp(delta_t * A_h) (one scalar per token and head, A_h < 0);
 *    Bbar_t = delta_t * B_t.
 *  - y_t reads the state after x_t has been added.
 *  - out = (y + D_h x) * z * sigmoid(z) when z is given (SiLU gate), else y + D_h x.
 *  - Head h reads group g = floor(h * G / H) of B and C.
 *  - Conv: u[t,c] = bias[c] + sum_{k<K} w[c][k] * xin[t-(K-1)+k, c] (the last tap
 *    meets the current token); xin before the first token comes from the conv
 *    state (oldest row first) or is zero; the activation is SiLU.
 *
 * Conventions for every entry point:
 *  - All tensors are device pointers owned by the caller; the library
 *    allocates no device memory and keeps no state but a thread-local error
 *    string.  Scratch comes from the caller's workspace.
 *  - Activations are token-major: row t of sequence b of a tensor X with
 *    token stride S (in elements) starts at X + (b*L + t)*S; within a row the
 *    innermost index is contiguous.  x, B and C may therefore be views into
 *    one [B, L, Cdim] buffer with channel order x (H*P) | B (G*N) | C (G*N).
 *  - Parameters (conv weights and bias, A, D, dt_bias) are fp32.  SSM states
 *    are fp32 [B, H, P, N], N contiguous.  Conv states are [B, K-1, Cdim] in
 *    the dtype of the raw x|B|C input, oldest row first.
 *  - Every call validates all arguments on the host before anything is
 *    enqueued, so an error status means nothing was written.  Work is
 *    enqueued on `stream` and the call returns without synchronising; a
 *    kernel fault surfaces at the caller's next synchronisation.
 *  - Results are deterministic: no floating-point atomics and a fixed
 *    reduction order, so identical inputs give identical bytes.
 *  - No C++ exception crosses this interface.
 */
#ifndef SSD_H_
#define SSD_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssd_dtype { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype_t;

/* Arithmetic of the scan's matrix products.
 * SSD_MATH_F32: every product and sum in fp32 (vector ALU).
 * SSD_MATH_BF16: the intra-chunk and state products take bf16 operands on the
 *   matrix cores with fp32 accumulation; decays, the state carry between
 *   chunks, the D skip and the gate stay fp32. */
typedef enum ssd_math { SSD_MATH_F32 = 0, SSD_MATH_BF16 = 1 } ssd_math_t;

enum ssd_status {
  SSD_OK = 0,
  SSD_ERR_INVALID_ARG = -1, /* NULL required pointer, bad size/stride/alignment, overlap */
  SSD_ERR_UNSUPPORTED = -2, /* valid, but no compiled kernel for it (e.g. P != 64)     */
  SSD_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the query said        */
  SSD_ERR_HIP = -4          /* a HIP runtime call failed; ssd_last_error() has detail  */
};

/*
 * Depthwise causal conv1d (+ SiLU) over [B, L, Cdim].
 *
 *   x               [B, L, Cdim] x_dtype, token stride x_tok_stride >= cdim
 *   weight          [Cdim, K] fp32;  bias [Cdim] fp32 or NULL
 *   conv_state_in   [B, K-1, Cdim] x_dtype or NULL (zero history)
 *   conv_state_out  [B, K-1, Cdim] x_dtype or NULL: the last K-1 raw inputs
 *                   of each sequence (reaching into conv_state_in when L < K-1);
 *                   must not overlap conv_state_in
 *   out             [B, L, Cdim] out_dtype, token stride out_tok_stride >= cdim;
 *                   must not overlap x
 *   width K in [1, 4]; apply_silu 0/1.
 * batch == 0 or seqlen == 0 is a valid call that only writes conv_state_out.
 */
int ssd_causal_conv1d_fwd(const void* x, int64_t x_tok_stride, ssd_dtype_t x_dtype,
                          const float* weight, const float* bias,
                          const void* conv_state_in, void* conv_state_out, void* out,
                          int64_t out_tok_stride, ssd_dtype_t out_dtype, int batch,
                          int seqlen, int cdim, int width, int apply_silu,
                          hipStream_t stream);

/* Bytes of device workspace ssd_chunk_scan_fwd needs for this shape (0 for
 * SSD_MATH_F32 and for empty inputs); fused_conv is 1 when conv_w will be
 * passed (the size does not depend on it in this version).  The matrix-core
 * path uses the workspace for B and C of every chunk and group, post-conv, in
 * the bf16 layouts its products read, and for the chunk's causal C B^T tiles
 * in fp32 (per sequence and group, 58 KiB per 64-token chunk, 132 KiB per
 * 128-token chunk, 328 KiB per 256-token chunk; all of it is formed once per
 * group rather than once per head), and for per-segment states when it
 * splits a long sequence over more workgroups.  0 for a chunk length the
 * matrix-core path does not support. */
size_t ssd_chunk_scan_workspace_bytes(int batch, int seqlen, int nheads, int headdim,
                                      int ngroups, int dstate, int chunk,
                                      ssd_math_t math, int fused_conv);

/*
 * Chunked selective scan of one Mamba-2 layer (prefill), from x, B, C, dt and z
 * to the gated output, with optional initial and final SSM state.
 *
 *   x   [B, L, H, P]  xbc_dtype, token stride x_tok_stride
 *   Bm  [B, L, G, N]  xbc_dtype, token stride b_tok_stride
 *   Cm  [B, L, G, N]  xbc_dtype, token stride c_tok_stride
 *       post-conv values when conv_w is NULL; raw conv inputs otherwise.
 *   conv_w [Cdim, K] fp32, conv_b [Cdim] fp32 or NULL, conv_width K in [1,4]:
 *       when conv_w is non-NULL the depthwise causal conv + SiLU of
 *       ssd_causal_conv1d_fwd is applied to x, B and C inside the scan
 *       (channel c of x, B, C is row c of conv_w, in the order x | B | C);
 *       conv_state_in / conv_state_out [B, K-1, Cdim] xbc_dtype or NULL as in
 *       ssd_causal_conv1d_fwd.  Both must be NULL when conv_w is NULL.
 *   dt  [B, L, H]     act_dtype, token stride dt_tok_stride (raw, before bias)
 *   z   [B, L, H, P]  act_dtype, token stride z_tok_stride, or NULL (no gate)
 *   A [H] fp32 (< 0 for a decaying state); D [H] fp32 or NULL (no skip);
 *   dt_bias [H] fp32 or NULL; dt_softplus 0/1.
 *   initial_state [B, H, P, N] fp32 or NULL (zero); final_state [B, H, P, N]
 *       fp32 or NULL.  They may be the same buffer.
 *   y   [B, L, H, P]  y_dtype, token stride y_tok_stride; must not overlap any
 *       input.
 *   Supported: P = 64, N = 128, H % G == 0; chunk in {64, 128, 256} for
 *   SSD_MATH_BF16 and in {32, 64, 128, 256} for SSD_MATH_F32; seqlen >= 0 (0 only copies
 *   the states); innermost rows 16-byte aligned.
 *   workspace: at least ssd_chunk_scan_workspace_bytes(...) bytes, 256-byte
 *   aligned, overlapping no tensor (NULL allowed when that is 0).
 */
int ssd_chunk_scan_fwd(const void* x, int64_t x_tok_stride, const void* Bm,
                       int64_t b_tok_stride, const void* Cm, int64_t c_tok_stride,
                       ssd_dtype_t xbc_dtype, const float* conv_w, const float* conv_b,
                       int conv_width, const void* conv_state_in, void* conv_state_out,
                       const void* dt, int64_t dt_tok_stride, const void* z,
                       int64_t z_tok_stride, ssd_dtype_t act_dtype, const float* A,
                       const float* D, const float* dt_bias, int dt_softplus,
                       const float* initial_state, float* final_state, void* y,
                       int64_t y_tok_stride, ssd_dtype_t y_dtype, int batch, int seqlen,
                       int nheads, int headdim, int ngroups, int dstate, int chunk,
                       ssd_math_t math, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * One-token decode step for a batch of sequences: the conv step on the ring of
 * the last K-1 raw inputs, then h <- exp(delta A) h + delta x B^T and
 * y = h C + D x, gated.  The state and the ring are updated in place.  Two
 * launches on the stream, no workspace: one workgroup per (sequence, head)
 * convolves what its head needs from the ring and streams the head's state
 * once; a second, small launch then shifts the ring columns of B and C,
 * which every head of a group reads.
 *
 *   state      [B, H, P, N] fp32, in/out
 *   xbc        [B, Cdim] xbc_dtype: the new token's raw x|B|C when conv_w is
 *              non-NULL, its post-conv values when conv_w is NULL
 *   conv_state [B, K-1, Cdim] xbc_dtype, in/out (required iff conv_w != NULL)
 *   conv_w [Cdim, K] fp32 or NULL, conv_b [Cdim] fp32 or NULL, conv_width K in [1,4]
 *   dt [B, H] act_dtype;  z [B, H*P] act_dtype or NULL
 *   A, D, dt_bias, dt_softplus as in ssd_chunk_scan_fwd
 *   y [B, H*P] y_dtype; must not overlap any input
 *   Supported: P = 64, N = 128, H % G == 0, B <= 65535.
 */
int ssd_state_update(float* state, const void* xbc, ssd_dtype_t xbc_dtype,
                     void* conv_state, const float* conv_w, const float* conv_b,
                     int conv_width, const void* dt, const void* z, ssd_dtype_t act_dtype,
                     const float* A, const float* D, const float* dt_bias, int dt_softplus,
                     void* y, ssd_dtype_t y_dtype, int batch, int nheads, int headdim,
                     int ngroups, int dstate, hipStream_t stream);

/* Bytes of device workspace ssd_state_update_ws needs: the post-conv x|B|C of
 * the step in fp32, 4 * batch * Cdim (0 on bad input or batch 0). */
size_t ssd_state_update_workspace_bytes(int batch, int nheads, int headdim, int ngroups,
                                        int dstate);

/*
 * The same decode step as ssd_state_update, with the same arguments, results
 * and in-place updates, taken in two passes through a caller-provided
 * workspace: the conv step of every channel (writing the post-conv x|B|C to
 * the workspace and shifting the ring), then the state update and readout
 * with one workgroup per 16 state rows of a head.  Both entry points take
 * the same sums in the same fixed order, so their results agree (each is
 * deterministic).
 *
 *   workspace: at least ssd_state_update_workspace_bytes(...) bytes,
 *   256-byte aligned, overlapping no tensor (may be NULL when batch is 0).
 *   Its contents on entry are ignored and on return are unspecified.
 *   Additionally supported: batch * Cdim below 2^31.
 */
int ssd_state_update_ws(float* state, const void* xbc, ssd_dtype_t xbc_dtype, void* conv_state,
                        const float* conv_w, const float* conv_b, int conv_width,
                        const void* dt, const void* z, ssd_dtype_t act_dtype, const float* A,
                        const float* D, const float* dt_bias, int dt_softplus, void* y,
                        ssd_dtype_t y_dtype, int batch, int nheads, int headdim, int ngroups,
                        int dstate, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * ssd_state_update_ws without a workspace argument and without allocating:
 * for callers that cannot call hipMalloc (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments (minus
 * the workspace), results, in-place updates and errors as ssd_state_update_ws,
 * through the same kernels; the post-conv x|B|C goes to a static 16 MiB
 * device array that the library holds on each device it runs on until the
 * process ends.
 *
 *   Limit: batch * Cdim <= 4194304 (Cdim = H*P + 2*G*N; batch 409 at
 *   Cdim 10240); larger calls return SSD_ERR_UNSUPPORTED and touch nothing.
 *   Concurrency: every call on one device shares that device's array (each
 *   call writes all of the part it reads before reading it, so nothing needs
 *   clearing); calls that overlap in time on one device, from different
 *   streams or threads, race on it and must be serialised by the caller.
 *   The first call on a device looks up the array's device address
 *   (hipGetSymbolAddress) and keeps it; SSD_ERR_HIP if that fails.
 */
int ssd_state_update_noalloc(float* state, const void* xbc, ssd_dtype_t xbc_dtype,
                             void* conv_state, const float* conv_w, const float* conv_b,
                             int conv_width, const void* dt, const void* z,
                             ssd_dtype_t act_dtype, const float* A, const float* D,
                             const float* dt_bias, int dt_softplus, void* y, ssd_dtype_t y_dtype,
                             int batch, int nheads, int headdim, int ngroups, int dstate,
                             hipStream_t stream);

/*
 * Measurement aids (not part of the layer): what this GPU reaches on plain
 * streaming and on back-to-back bf16 matrix-core products, for comparing
 * the layer's kernels with measured rates beside the published peaks.
 *
 * ssd_calibrate_stream: one non-temporal pass dst[i] = src[i] over bytes/16
 *   16-byte words.  dst == src streams the buffer in place (every word read
 *   and written back at its own address, as the decode step does with its
 *   state); otherwise a copy (which must not partly overlap).  bytes and both
 *   pointers 16-byte multiples.  Moves 2 * bytes through HBM.
 * ssd_calibrate_mfma_bf16: blocks workgroups of 4 waves; each wave issues
 *   iters * 8 independent-chain 16x16x32 bf16 MFMAs (16384 flops each) on
 *   register operands and writes one float per lane to out (blocks * 256
 *   floats).  Flops per call: blocks * 4 * iters * 8 * 16384.
 */
int ssd_calibrate_stream(void* dst, const void* src, size_t bytes, hipStream_t stream);
int ssd_calibrate_mfma_bf16(float* out, int blocks, int iters, hipStream_t stream);

/* Bytes of decode cache per sequence and layer: the fp32 SSM state
 * (4*H*P*N) plus the conv ring ((K-1) * Cdim elements of conv_dtype).
 * This is the fixed-size Mamba cache of "Hybrid Architectures ..." summary,
 * Appendix C, with an fp32 state and K-1 stored conv rows.  0 on bad input. */
size_t ssd_decode_cache_bytes(int nheads, int headdim, int ngroups, int dstate, int width,
                              ssd_dtype_t conv_dtype);

/* Bytes of device workspace ssd_chunk_scan_bwd needs (0 on bad input;
 * conv_width 0 when no conv is fused): the post-conv x|B|C in fp32, the state
 * entering every 32-token chunk (4*P*N bytes per (sequence, head, chunk)),
 * per-head B and C gradients, and small per-block sums. */
size_t ssd_chunk_scan_bwd_workspace_bytes(int batch, int seqlen, int nheads, int headdim,
                                          int ngroups, int dstate, int conv_width);

/*
 * The layer's backward pass: given the gradient dout of a scalar loss with
 * respect to ssd_chunk_scan_fwd's output (and d_final_state with respect to
 * its final state, or NULL), the loss's gradients with respect to its
 * inputs.  This is reverse-mode differentiation of the recurrence of
 * "Hybrid Architectures ..." summary, section 2 Background, and of the conv
 * and gate in front of and behind it; the pages treat the layer as a
 * trained component ("Nemotron-H style Hybrid Mamba-Transformer 3B
 * feasibility study", section 3).  All arithmetic is fp32.
 *
 *   Inputs: exactly the forward call's (x, Bm, Cm, conv_w/conv_b/
 *   conv_state_in, dt, z, A, D, dt_bias, dt_softplus, initial_state), with
 *   the same layouts and strides.
 *   dout [B, L, H, P] dout_dtype, token stride dout_tok_stride;
 *   d_final_state [B, H, P, N] fp32 or NULL (zero).
 *   Outputs, all dense fp32, overwritten:
 *     dxbc [B, L, Cdim] x|B|C: raw conv inputs when conv_w is given, else the
 *          post-conv values (required);
 *     ddt [B, L, H] with respect to the raw dt (required); dA [H] (required);
 *     dz [B, L, H, P] (NULL, or only when z is given); dD [H], ddt_bias [H],
 *     d_initial_state [B, H, P, N]: each optional (NULL), and defined also
 *     when the forward input was NULL (the gradient at zero);
 *     dconv_w [Cdim, K], dconv_b [Cdim], d_conv_state_in [B, K-1, Cdim]:
 *     optional, only with conv_w.
 *   No output may overlap an input or another output.
 *   Supported: P = 64, N = 128, H % G == 0; any seqlen >= 0.
 *   workspace: at least ssd_chunk_scan_bwd_workspace_bytes(...) bytes,
 *   256-byte aligned, overlapping no tensor.
 * Deterministic: the group sums of the B and C gradients and the parameter
 * sums are taken in a fixed order.
 */
int ssd_chunk_scan_bwd(const void* x, int64_t x_tok_stride, const void* Bm,
                       int64_t b_tok_stride, const void* Cm, int64_t c_tok_stride,
                       ssd_dtype_t xbc_dtype, const float* conv_w, const float* conv_b,
                       int conv_width, const void* conv_state_in, const void* dt,
                       int64_t dt_tok_stride, const void* z, int64_t z_tok_stride,
                       ssd_dtype_t act_dtype, const float* A, const float* D,
                       const float* dt_bias, int dt_softplus, const float* initial_state,
                       const void* dout, int64_t dout_tok_stride, ssd_dtype_t dout_dtype,
                       const float* d_final_state, float* dxbc, float* ddt, float* dz,
                       float* dA, float* dD, float* ddt_bias, float* d_initial_state,
                       float* dconv_w, float* dconv_b, float* d_conv_state_in, int batch,
                       int seqlen, int nheads, int headdim, int ngroups, int dstate,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * The block around the layer: the pre-norm residual block
 *   out = h + out_proj(mixer(rmsnorm(h)))
 * of "Nemotron-H style Hybrid Mamba-Transformer 3B feasibility study",
 * section 3.2 (approach A), whose mixer is in_proj, the layer above (conv +
 * SiLU, scan, D skip, SiLU(z) gate) and out_proj; the two projections hold
 * about 3 * expand * d_model^2 parameters (its section 2.4).
 * Readings where the pages are silent: RMSNorm is x / sqrt(mean(x^2) + eps)
 * times a per-channel fp32 weight; in_proj's output rows are ordered
 * z (H*P) | x (H*P) | B (G*N) | C (G*N) | dt (H); the intermediates (normed
 * h, in_proj output, layer output) are bf16, the projections accumulate in
 * fp32.
 * ------------------------------------------------------------------------ */

/*
 * RMSNorm of ntok rows: out[t][i] = x[t][i] / sqrt(mean_j x[t][j]^2 + eps) * w[i].
 *   x   [ntok, dim] x_dtype, row stride x_tok_stride >= dim
 *   weight [dim] fp32 or NULL (no scale); eps finite, >= 0
 *   out [ntok, dim] out_dtype, row stride out_tok_stride >= dim; out may be x
 *       itself (same dtype and stride) but may not overlap it otherwise
 *   Supported: dim % 8 == 0; rows and weight 16-byte aligned.
 * The sum of squares is fp32 in a fixed order (bitwise reproducible).
 */
int ssd_rmsnorm_fwd(const void* x, int64_t x_tok_stride, ssd_dtype_t x_dtype,
                    const float* weight, float eps, void* out, int64_t out_tok_stride,
                    ssd_dtype_t out_dtype, int64_t ntok, int dim, hipStream_t stream);

/*
 * Projection on the matrix cores: out[m][n] = sum_k a[m][k] * w[n][k]
 * (+ residual[m][n]), bf16 operands, fp32 accumulation, one rounding to
 * out_dtype at the end.
 *   a   [M, K] bf16, row stride lda >= K
 *   w   [N, K] bf16, row stride ldw >= K (the weight of a projection, stored
 *       [out][in])
 *   residual [M, N] res_dtype, row stride ldr >= N, or NULL; out may be the
 *       residual itself (same dtype and stride: an in-place residual add)
 *   out [M, N] out_dtype, row stride ldo >= N; may not overlap a or w
 *   Supported: K % 8 == 0; base pointers and rows 16-byte aligned.
 * M == 0 is a valid call that does nothing.
 */
int ssd_linear_fwd(const void* a, int64_t lda, const void* w, int64_t ldw, const void* residual,
                   int64_t ldr, ssd_dtype_t res_dtype, void* out, int64_t ldo,
                   ssd_dtype_t out_dtype, int64_t M, int N, int K, hipStream_t stream);

/* Bytes of device workspace ssd_block_fwd needs (0 on bad input): the normed
 * input, the in_proj output and the layer output in bf16 (2*d_model +
 * 2*(2*H*P + 2*G*N + H rounded up to 8) + 2*H*P bytes per token), plus the
 * layer's ssd_chunk_scan_workspace_bytes. */
size_t ssd_block_workspace_bytes(int batch, int seqlen, int d_model, int nheads, int headdim,
                                 int ngroups, int dstate);

/*
 * The whole block for a batch of sequences (prefill):
 *   u = rmsnorm(h); [z | x B C | dt] = u in_proj_w^T;
 *   y = the layer (ssd_chunk_scan_fwd with the fused conv, bf16 math) on them;
 *   out = h + y out_proj_w^T.
 *   h   [B, L, d_model] h_dtype, dense
 *   norm_w [d_model] fp32 or NULL; norm_eps finite, >= 0
 *   in_proj_w  [2*H*P + 2*G*N + H, d_model] bf16, dense
 *   conv_w [Cdim, K] fp32, conv_b [Cdim] fp32 or NULL, conv_width K in [1,4],
 *       Cdim = H*P + 2*G*N (the x|B|C channels)
 *   A [H], D [H] or NULL, dt_bias [H] or NULL (fp32); dt_softplus 0/1
 *   out_proj_w [d_model, H*P] bf16, dense
 *   conv_state_in / conv_state_out [B, K-1, Cdim] bf16 or NULL (raw x|B|C
 *       rows of the in_proj output, oldest first), as in ssd_chunk_scan_fwd
 *   initial_state / final_state [B, H, P, N] fp32 or NULL, as in
 *       ssd_chunk_scan_fwd
 *   out [B, L, d_model] out_dtype, dense; may be h itself (same dtype: an
 *       in-place update) but may not overlap it, a parameter or a state
 *       otherwise
 *   workspace: at least ssd_block_workspace_bytes(...) bytes, 256-byte
 *       aligned, overlapping no tensor (NULL allowed when seqlen == 0)
 *   Supported: P = 64, N = 128, H % G == 0, d_model % 8 == 0.
 */
int ssd_block_fwd(const void* h, ssd_dtype_t h_dtype, const float* norm_w, float norm_eps,
                  const void* in_proj_w, const float* conv_w, const float* conv_b,
                  int conv_width, const float* A, const float* D, const float* dt_bias,
                  int dt_softplus, const void* out_proj_w, const void* conv_state_in,
                  void* conv_state_out, const float* initial_state, float* final_state,
                  void* out, ssd_dtype_t out_dtype, int batch, int seqlen, int d_model,
                  int nheads, int headdim, int ngroups, int dstate, void* workspace,
                  size_t workspace_bytes, hipStream_t stream);

/* Static text for a status code. */
const char* ssd_status_string(int status);

/* Detail of the last failing call on this thread ("" if none). */
const char* ssd_last_error(void);

/* Library version string. */
const char* ssd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H_ */
