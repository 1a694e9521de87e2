/*
 * hsq.h -- C ABI of libhsq: the inference-time W4A4 linear layer with a
 * rank-r high-precision branch, for AMD Instinct MI355X (gfx950).
 *
 * The layer (Deflating the Hessian, abstract; thelatestinai.com paper page,
 * Figure 1 caption): every weight is split into a high-precision low-rank
 * component and a low-bit residual, W ~ L1*L2 + Q(R).  Weights and
 * activations are 4-bit with one scale per 64-wide group of the input
 * dimension (same page, Table 1 and Table 8 captions: W4A4, group-64).  A
 * diagonal smoothing moves range from the activations to the weights
 * without changing the full-precision product (H-SVDQuant explainer,
 * rit.work, section on Hessian deflation, last paragraph).  As in the
 * two-branch inference form of DiRotQ (papernotes.org, key design 2), the
 * high-precision branch runs on the unquantized (smoothed) activations:
 *
 *   xh[m,k]  = X[m,k] * fl32(1 / lambda[k])                    smoothing
 *   sx[m,g]  = fp16_rne(fl32(absmax_{k in g} |xh[m,k]| / 7))   (0 if absmax = 0; saturates at 65504)
 *   qx[m,k]  = clamp(rint(xh[m,k] * fl32(1 / sx[m,g])), -8, 7) (all 0 if sx = 0)
 *   U[m,j]   = sum_k xh[m,k] * L1[k,j]                         rank-r down projection
 *   P[m,n,g] = sum_{k in g} qx[m,k] * qw[k,n]                  int32, exact
 *   Y[m,n]   = sum_g P[m,n,g] * sx[m,g] * sw[g,n] + sum_j U[m,j] * L2[j,n] + bias[n]
 *
 * Group g covers input channels [64g, 64g + 64).  The entry points whose
 * names end in _g take the group width as an argument, 64 or 128 (group g
 * then covers [group*g, group*g + group)); the Qwen3-8B experiments of the
 * same page use group-128 (Table 3, 4, 6 and 7 captions).  Rounding is
 * IEEE-754 round-to-nearest-even throughout; rint rounds ties to even.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers (HIP global memory), owned and
 *     allocated by the caller, 16-byte aligned, row-major and densely packed.
 *     The library never allocates or frees memory.
 *   - bf16 and fp16 values travel as uint16_t bit patterns.
 *   - `stream` is a hipStream_t passed as void* (NULL: the null stream).
 *     Work is enqueued asynchronously on it; the call returns once enqueued.
 *   - Arguments are validated before anything is enqueued; on an error the
 *     call returns a negative HSQ_E_* code and enqueues nothing.  Faults that
 *     happen while kernels run surface at the caller's next synchronisation.
 *   - Debugging: with HSQ_DEBUG set in the environment (any value but "0"),
 *     every call that enqueues work waits for its stream before returning
 *     and reports a failure of its own kernels as HSQ_E_HIP, with
 *     hsq_last_hip_error() naming it.  While the stream is being captured
 *     into a graph the call does not wait (waiting is not allowed there).
 *   - The library keeps no state between calls (except the per-device
 *     scratch of hsq_w4a4_lowrank_linear_noalloc) and is thread-safe; no
 *     C++ exception crosses this interface.
 *   - Limits: K % 64 == 0 and K >= 64; M, N >= 1; 0 <= r <= 32;
 *     1 <= batch <= 16; M * K, M * N, K * N < 2^31; and, for the linear,
 *     16*ceil(M/16) * Kp < 2^32 and 16*ceil(N/16) * Kp < 2^32 with
 *     Kp = K rounded up to 128 (the padded int8 activation codes and the
 *     int8 part of the packed residual are addressed through 32-bit buffer
 *     resources).
 */
#ifndef HSQ_H
#define HSQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define HSQ_OK            0
#define HSQ_E_INVAL      -1  /* null pointer, size out of range, bad dtype or kernel choice */
#define HSQ_E_SHAPE      -2  /* K not a positive multiple of 64, or a window outside the matrix */
#define HSQ_E_ALIGN      -3  /* a pointer is not 16-byte aligned */
#define HSQ_E_WORKSPACE  -4  /* workspace missing or smaller than the size function returns */
#define HSQ_E_HIP        -5  /* the HIP runtime refused a launch */
#define HSQ_E_SCRATCH    -6  /* hsq_w4a4_lowrank_linear_noalloc: the sizes need more
                                workspace than its static scratch holds */

/* ---- output dtypes ---- */
#define HSQ_F32   0
#define HSQ_BF16  1

/* ---- kernel choice for the residual contraction ---- */
#define HSQ_KERNEL_AUTO    0  /* SKINNY for M <= 64, TILED otherwise */
#define HSQ_KERNEL_TILED   1  /* LDS-tiled int8-MFMA kernel, one workgroup per output tile */
#define HSQ_GROUP_64     64
#define HSQ_GROUP_128   128

#define HSQ_KERNEL_SKINNY  2  /* weight-streaming kernel for M <= 64: the waves of a
                                 workgroup split K and reduce in a fixed order */

/* Version of the packed-weight layout written by hsq_pack_weights (2:
 * nibbles, then int8 operands; see hsq_packed_weight_bytes). */
int hsq_layout_version(void);

/* Static text for a status code (never NULL). */
const char *hsq_status_string(int status);

/* The HIP runtime's text for the error behind the last HSQ_E_HIP returned
 * on the calling host thread ("no HIP error" if there was none).  Static
 * storage, never NULL. */
const char *hsq_last_hip_error(void);

/* Bytes of one packed residual (K x N int4 codes) as hsq_pack_weights
 * writes it (layout version 2): Np * Kp / 2 bytes of nibbles followed by
 * Np * Kp bytes of the same codes as int8 operands, Np = N rounded up to
 * 16, Kp = K rounded up to 128; 3/2 * Np * Kp in all.  The weight-streaming
 * contraction for few tokens reads the nibbles (half a byte per weight);
 * the tiled contraction for many tokens moves the int8 operands into LDS
 * unchanged, which saves its vector ALU -- the unit that bounds it -- the
 * nibble unpacking.  Returns 0 if K or N is invalid. */
size_t hsq_packed_weight_bytes(int K, int N);

/* Pack residual codes into the layout the contraction kernels read.
 * Operation: the 4-bit residual Q(R) of W ~ L1*L2 + Q(R) (Deflating the
 * Hessian, abstract), group-64 (Table 1 caption).
 *   codes   in : K x N int8 (input channel x output channel), values in [-8, 7]
 *   packed  out: hsq_packed_weight_bytes(K, N) bytes; padding is zero codes
 *   d_status out: one device int; set to 0 (by a kernel: the call enqueues
 *                 kernels only, so it can be captured in a HIP graph),
 *                 then to 1 if any code lies outside [-8, 7] (that code's
 *                 low nibble is stored).  The caller reads it after
 *                 synchronising.
 * Errors: HSQ_E_INVAL, HSQ_E_SHAPE, HSQ_E_ALIGN, HSQ_E_HIP. */
int hsq_pack_weights(const int8_t *codes, int K, int N, uint8_t *packed, int *d_status,
                     void *stream);

/* Inverse of hsq_pack_weights (testing and inspection).
 *   packed in : hsq_packed_weight_bytes(K, N) bytes
 *   codes  out: K x N int8 in [-8, 7]
 * Errors: HSQ_E_INVAL, HSQ_E_SHAPE, HSQ_E_ALIGN, HSQ_E_HIP. */
int hsq_unpack_weights(const uint8_t *packed, int K, int N, int8_t *codes, void *stream);

/* Smooth and quantize activations per token in 64-wide groups, and form the
 * rank-r down projection of the smoothed, unquantized activations (the
 * xh, sx, qx and U lines of the formula block above).
 *   X      in : M x K bf16
 *   lambda in : K fp16 smoothing factors (X is divided by them)
 *   L1     in : K x r bf16 (may be NULL when r == 0)
 *   qx     out: M x K/2 bytes; byte j of a row holds code 2j in its low
 *               nibble and code 2j+1 in its high nibble, two's complement
 *   sx     out: M x K/64 fp16 scales
 *   U      out: M x r fp32 (may be NULL when r == 0)
 * K <= 12288 for this entry point (HSQ_E_INVAL beyond).
 * Errors: HSQ_E_INVAL, HSQ_E_SHAPE, HSQ_E_ALIGN, HSQ_E_HIP. */
int hsq_quantize_act(const uint16_t *X, int M, int K, const uint16_t *lambda,
                     const uint16_t *L1, int r, uint8_t *qx, uint16_t *sx, float *U,
                     void *stream);

/* Workspace bytes hsq_w4a4_lowrank_linear and hsq_w4a4_group_partials need
 * for these sizes (any kernel choice).  Returns 0 if a size is invalid. */
size_t hsq_workspace_bytes(int M, int K, int N, int r, int batch);

/* The fused W4A4 + rank-r linear layer, for `batch` projections that share
 * the input X and the smoothing factors (e.g. Q, K and V).  Computes Y of the
 * formula block above: one pass over X quantizes it and forms U, then the
 * int4 x int4 contraction keeps an int32 partial sum per 64-wide group,
 * rescales it by sx * sw in fp32, and adds U * L2 and the bias.
 *   X        in : M x K bf16
 *   lambda   in : K fp16
 *   packed_w in : batch blobs of hsq_packed_weight_bytes(K, N) bytes, back to back
 *   sw       in : batch x K/64 x N fp16 weight scales
 *   L1       in : batch x K x r bf16   (NULL when r == 0)
 *   L2       in : batch x r x N bf16   (NULL when r == 0)
 *   bias     in : batch x N bf16, or NULL for no bias
 *   Y        out: batch x M x N, fp32 (y_dtype HSQ_F32) or bf16 (HSQ_BF16, RNE)
 *   workspace   : ws_bytes >= hsq_workspace_bytes(M, K, N, r, batch) device
 *                 bytes, scratch owned by the caller; its contents on entry
 *                 do not matter and are clobbered.
 * Errors: HSQ_E_INVAL, HSQ_E_SHAPE, HSQ_E_ALIGN, HSQ_E_WORKSPACE, HSQ_E_HIP. */
int hsq_w4a4_lowrank_linear(const uint16_t *X, int M, int K, int N, int batch,
                            const uint16_t *lambda, const uint8_t *packed_w,
                            const uint16_t *sw, const uint16_t *L1, const uint16_t *L2, int r,
                            const uint16_t *bias, void *Y, int y_dtype, void *workspace,
                            size_t ws_bytes, void *stream);

/* As hsq_w4a4_lowrank_linear, with the contraction kernel chosen by
 * `kernel` (HSQ_KERNEL_*; SKINNY with M > 64 is HSQ_E_INVAL). */
int hsq_w4a4_lowrank_linear_ex(const uint16_t *X, int M, int K, int N, int batch,
                               const uint16_t *lambda, const uint8_t *packed_w,
                               const uint16_t *sw, const uint16_t *L1, const uint16_t *L2,
                               int r, const uint16_t *bias, void *Y, int y_dtype,
                               void *workspace, size_t ws_bytes, int kernel, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer as hsq_w4a4_lowrank_linear (group 64, contraction kernel chosen
 * as for HSQ_KERNEL_AUTO), with its workspace in a static device array of
 * HSQ_NOALLOC_SCRATCH_BYTES (64 MiB) inside the library instead of a caller
 * buffer.  Every GPU the library runs on holds its own array until the
 * process ends; the first call on a device looks up that device's address
 * of it (no allocation).  The call uses the array of the CURRENT device
 * (hipGetDevice); `stream` must belong to that device.  The call allocates
 * and frees nothing.  All calls on one GPU share its array: calls that may
 * overlap in time on one GPU (two streams, two host threads without
 * ordering) race on it and must be serialised by the caller; calls in order
 * on one stream are safe.  No part of the array needs to start zeroed (the
 * quantization pass rewrites everything the contraction reads).
 * Sizes whose workspace (hsq_workspace_bytes(M, K, N, r, batch)) exceeds
 * the array return HSQ_E_SCRATCH before anything is enqueued; every
 * configuration of the diffusion and LLM layers here fits (the largest,
 * 4608 tokens x 12288 channels, needs about 64 MB).
 * Other arguments and errors as for hsq_w4a4_lowrank_linear. */
#define HSQ_NOALLOC_SCRATCH_BYTES (64u << 20)
int hsq_w4a4_lowrank_linear_noalloc(const uint16_t *X, int M, int K, int N, int batch,
                                    const uint16_t *lambda, const uint8_t *packed_w,
                                    const uint16_t *sw, const uint16_t *L1, const uint16_t *L2,
                                    int r, const uint16_t *bias, void *Y, int y_dtype,
                                    void *stream);

/* The same layer in two stages on one stream, for callers that time or
 * schedule them separately, or reuse one quantized input for several
 * contractions with the same (M, K, batch, r).
 *   hsq_w4a4_quantize_stage: the smoothing / quantization / U pass over X
 *     (X, lambda, L1 as for the linear) into `workspace`.
 *   hsq_w4a4_contract_stage: the residual contraction, rescale and U*L2 +
 *     bias epilogue (packed_w, sw, L2, bias, Y as for the linear), reading
 *     the workspace the quantize stage wrote for the same M, K, r and batch.
 * Running both equals hsq_w4a4_lowrank_linear_ex.  The workspace must not
 * be reused by another quantize stage until the contract stages that read it
 * have run (stream order guarantees this on one stream).
 * Errors: as hsq_w4a4_lowrank_linear_ex. */
int hsq_w4a4_quantize_stage(const uint16_t *X, int M, int K, int N, int batch,
                            const uint16_t *lambda, const uint16_t *L1, int r, void *workspace,
                            size_t ws_bytes, void *stream);
int hsq_w4a4_contract_stage(int M, int K, int N, int batch, const uint8_t *packed_w,
                            const uint16_t *sw, const uint16_t *L2, int r, const uint16_t *bias,
                            void *Y, int y_dtype, void *workspace, size_t ws_bytes, int kernel,
                            void *stream);

/* Test export: the per-group int32 partial sums P[m,n,g] (formula block
 * above) of one projection, produced by the same quantization pass and the
 * same contraction loop as hsq_w4a4_lowrank_linear_ex with this `kernel`,
 * with the rescaling epilogue replaced by a store of P.  Only the window
 * m in [m0, m0+mc), n in [n0, n0+nc) is written.
 *   X, lambda, packed_w : as for the linear (one projection)
 *   P        out: mc x nc x K/64 int32
 *   workspace   : as for the linear with batch = 1, r = 0
 * Errors: HSQ_E_INVAL, HSQ_E_SHAPE (window outside M x N), HSQ_E_ALIGN,
 *         HSQ_E_WORKSPACE, HSQ_E_HIP. */
int hsq_w4a4_group_partials(const uint16_t *X, int M, int K, int N, const uint16_t *lambda,
                            const uint8_t *packed_w, int m0, int mc, int n0, int nc,
                            int32_t *P, void *workspace, size_t ws_bytes, int kernel,
                            void *stream);

/* ---- the same layer with the group width as an argument ----
 * group is HSQ_GROUP_64 or HSQ_GROUP_128 (anything else: HSQ_E_INVAL) and
 * must divide K (HSQ_E_SHAPE otherwise).  Every scale array then has K/group
 * groups: sw is batch x K/group x N fp16, P is mc x nc x K/group int32.
 * The packed weights are the same for both widths (hsq_pack_weights).  With
 * group = 64 each function equals its counterpart above.  A group-128
 * scale covers two 64-channel blocks: the contraction accumulates their two
 * int32 block sums before the one rescale by sx * sw. */
size_t hsq_workspace_bytes_g(int M, int K, int N, int r, int batch, int group);
int hsq_w4a4_lowrank_linear_g(const uint16_t *X, int M, int K, int N, int batch, int group,
                              const uint16_t *lambda, const uint8_t *packed_w,
                              const uint16_t *sw, const uint16_t *L1, const uint16_t *L2,
                              int r, const uint16_t *bias, void *Y, int y_dtype,
                              void *workspace, size_t ws_bytes, int kernel, void *stream);
int hsq_w4a4_quantize_stage_g(const uint16_t *X, int M, int K, int N, int batch, int group,
                              const uint16_t *lambda, const uint16_t *L1, int r, void *workspace,
                              size_t ws_bytes, void *stream);
int hsq_w4a4_contract_stage_g(int M, int K, int N, int batch, int group, const uint8_t *packed_w,
                              const uint16_t *sw, const uint16_t *L2, int r, const uint16_t *bias,
                              void *Y, int y_dtype, void *workspace, size_t ws_bytes, int kernel,
                              void *stream);
int hsq_w4a4_group_partials_g(const uint16_t *X, int M, int K, int N, int group,
                              const uint16_t *lambda, const uint8_t *packed_w, int m0, int mc,
                              int n0, int nc, int32_t *P, void *workspace, size_t ws_bytes,
                              int kernel, void *stream);

/* ---- asymmetric activations ----
 * The activation format of the INT W4A4 setting in the DiRotQ notes
 * (papernotes.org, experimental setup): activations quantized per token and
 * group asymmetrically, weights symmetrically as above.  The notes print no
 * formula; this library reads it as the min-max quantizer with 16 levels
 * whose range is widened to contain 0 (so that 0 is a level):
 *   lo[m,g]  = min(0, min_{k in g} xh[m,k]),  hi[m,g] = max(0, max_{k in g} xh[m,k])
 *   sx[m,g]  = fp16_rne(fl32(fl32(hi - lo) / 15))   (0 if hi == lo; saturates at 65504)
 *   z[m,g]   = clamp(rint(fl32(-lo * fl32(1 / sx))), 0, 15)      zero point
 *   q[m,k]   = clamp(rint(fl32(xh * fl32(1 / sx))) + z, 0, 15)  (all 0 if sx = 0)
 *   qx[m,k]  = q[m,k] - z[m,g]                      in [-15, 15]
 * and P, U, Y as in the formula block (with this qx).  qx fits the int8
 * operand of the contraction, so both contraction kernels run unchanged.
 * act_quant is HSQ_AQ_SYMMETRIC (the formula block; each function then
 * equals its _g counterpart) or HSQ_AQ_ASYMMETRIC; anything else is
 * HSQ_E_INVAL.  Arguments, workspace and errors otherwise as for the _g
 * functions. */
#define HSQ_AQ_SYMMETRIC   0
#define HSQ_AQ_ASYMMETRIC  1
int hsq_w4a4_lowrank_linear_aq(const uint16_t *X, int M, int K, int N, int batch, int group,
                               int act_quant, const uint16_t *lambda, const uint8_t *packed_w,
                               const uint16_t *sw, const uint16_t *L1, const uint16_t *L2, int r,
                               const uint16_t *bias, void *Y, int y_dtype, void *workspace,
                               size_t ws_bytes, int kernel, void *stream);
int hsq_w4a4_quantize_stage_aq(const uint16_t *X, int M, int K, int N, int batch, int group,
                               int act_quant, const uint16_t *lambda, const uint16_t *L1, int r,
                               void *workspace, size_t ws_bytes, void *stream);
int hsq_w4a4_group_partials_aq(const uint16_t *X, int M, int K, int N, int group, int act_quant,
                               const uint16_t *lambda, const uint8_t *packed_w, int m0, int mc,
                               int n0, int nc, int32_t *P, void *workspace, size_t ws_bytes,
                               int kernel, void *stream);

/* ---- MX-fp4 format variant of the layer ----
 * The same layer (smoothing, rank-r branch on the smoothed activations,
 * bias) with both 4-bit operands of the residual product in MX-fp4 (OCP
 * Microscaling Formats v1.0) instead of int4 with fp16 group-64 scales: per
 * 32 consecutive values along K one e8m0 scale 2^X, X = floor(log2 amax) - 2
 * (stored as X + 127, clamped to [0, 254]; a zero block stores 127), and
 * e2m1 elements {0, 0.5, 1, 1.5, 2, 3, 4, 6} rounded to nearest (ties to the
 * even mantissa), magnitudes above 6 saturating; the code keeps the value's
 * sign bit, also where the magnitude rounds to 0 (-0, code 8).  The activations are
 * blocked per token, the residual per output column.  The product runs on
 * gfx950's scaled fp4 MFMA, which applies both scales.
 * hsq_mx_pack_weights: R (K x N fp32, the residual, row-major) -> packed
 *   (hsq_mx_packed_weight_bytes(K, N) bytes: codes in MFMA operand order,
 *   then the scales).
 * hsq_mx_lowrank_linear: Y (M x N, HSQ_F32 or HSQ_BF16) = Q(Xh) Q(R) +
 *   (Xh L1) L2 + bias; X, lambda, L1 (K x r), L2 (r x N), bias (N) as for
 *   hsq_w4a4_lowrank_linear with batch 1; workspace of
 *   hsq_mx_workspace_bytes(M, K, r) bytes.
 * Errors: HSQ_E_INVAL, HSQ_E_SHAPE (K not a multiple of 64), HSQ_E_ALIGN,
 * HSQ_E_WORKSPACE, HSQ_E_HIP. */
size_t hsq_mx_packed_weight_bytes(int K, int N);
int hsq_mx_pack_weights(const float *R, int K, int N, uint8_t *packed, void *stream);
size_t hsq_mx_workspace_bytes(int M, int K, int r);
int hsq_mx_lowrank_linear(const uint16_t *X, int M, int K, int N, const uint16_t *lambda,
                          const uint8_t *packed_mx, const uint16_t *L1, const uint16_t *L2, int r,
                          const uint16_t *bias, void *Y, int y_dtype, void *workspace, size_t ws_bytes,
                          void *stream);

/* ---- fused two-layer chain: Y = down(act(up(X))) ----
 * Two linears of the kind above (group 64, one projection each, ranks r_up
 * and r_down) with an elementwise activation between them, as in the MLP
 * of a diffusion transformer block (FLUX.1: an up-projection of width H,
 * GELU, a down-projection; 3072 -> 12288 -> 3072 at its model width).  The
 * up layer's contraction does not write its output:
 * its epilogue applies the activation in fp32 and forms, from that fp32
 * value, the down layer's smoothed input, its group-64 scales and int4
 * codes (the quantizer of the formula block above, applied to
 * a[m,k] = act(Y_up[m,k]) instead of a bf16 X) and the partial sums of the
 * down layer's rank branch U_down = (a * fl32(1/lambda_down)) L1_down.
 * The down layer then runs its contraction on them: the hidden activation
 * never travels through HBM as a bf16 tensor and the down layer has no
 * quantization pass.
 *   act   HSQ_ACT_IDENTITY, or HSQ_ACT_GELU_TANH: the tanh form of GELU,
 *         0.5 y (1 + tanh(z)), z = 0.7978845608 (y + 0.044715 y^3), computed
 *         in fp32 as y / (1 + e(-2z)) with e(x) = p(r) * 2^n, n = rint(x *
 *         1.44269504), r = (x - n * 0.693145751953125) - n *
 *         1.428606765330187e-6, p the degree-6 Taylor polynomial of exp
 *         in Horner form, x clamped to [-87, 88], every operation rounded
 *         once (no fused multiply-add)
 *   Y          out: M x N, HSQ_F32 or HSQ_BF16
 *   Y_hidden   optional out (NULL: not written): M x H fp32, the up
 *              layer's output before the activation (a test export)
 *   r_down     0 .. 8; the up layer runs the tiled contraction unsplit
 * All other arguments as for hsq_w4a4_lowrank_linear, per layer.
 * Performance: on an MI355X this call is SLOWER than the two layers run
 * as separate hsq_w4a4_lowrank_linear calls (FLUX.1 MLP, 4608 tokens:
 * 0.70-0.71 ms fused vs 0.60-0.61 ms separate, the separate path without
 * any activation pass).  The up contraction is bound by its per-group VALU
 * rescale, and the fused epilogue adds about 50 VALU instructions per
 * output element (GELU, smoothing, absmax, codes, rank-r dot product) to
 * it, more than the bf16 round trip and quantization pass it removes.  Use
 * it where the hidden activation must not be materialised, not for speed.
 * Errors: HSQ_E_INVAL, HSQ_E_SHAPE (K or H not a multiple of 64),
 * HSQ_E_ALIGN, HSQ_E_WORKSPACE, HSQ_E_HIP. */
#define HSQ_ACT_IDENTITY   0
#define HSQ_ACT_GELU_TANH  1
size_t hsq_mlp_workspace_bytes(int M, int K, int H, int N, int r_up, int r_down);
int hsq_w4a4_lowrank_mlp(const uint16_t *X, int M, int K, int H, int N, const uint16_t *lambda_up,
                         const uint8_t *packed_up, const uint16_t *sw_up, const uint16_t *L1_up,
                         const uint16_t *L2_up, int r_up, const uint16_t *bias_up, int act,
                         const uint16_t *lambda_down, const uint8_t *packed_down,
                         const uint16_t *sw_down, const uint16_t *L1_down, const uint16_t *L2_down,
                         int r_down, const uint16_t *bias_down, void *Y, int y_dtype, float *Y_hidden,
                         void *workspace, size_t ws_bytes, void *stream);

/* ---- calibration: the Hessian, its deflation, the closed-form L2 ----
 * The steps that produce a layer's factors (Deflating the Hessian, paper
 * page: abstract and Figure 1 caption; H-SVDQuant explainer, rit.work,
 * section on Hessian deflation).  The pages give no formulas; these follow
 * the plainest reading (the activation-noise surrogate term is left out):
 *
 *   H      = Xh^T Xh                     Xh[m,k] = X[m,k] * fl32(1/lambda[k]) (as above)
 *   C      = L1^T H L1                   r x r
 *   Hperp  = H - (H L1) C^-1 (H L1)^T     deflated Hessian: Hperp L1 = 0
 *   E      = W - deq(Q(R))               deq(Q(R))[k,n] = code[k,n] * sw[k/group, n]
 *   L2*    = C^-1 (H L1)^T E             the output-side factor minimising
 *                                        || Xh E - Xh L1 L2 ||_F
 *
 * Sizes: K a multiple of 64 with 64 <= K <= 16384 (HSQ_E_SHAPE / _INVAL),
 * 1 <= r <= 32.  H, Hperp are K x K fp32 row-major.  Pointers are device
 * pointers, 16-byte aligned; buffers are the caller's.  All arithmetic is
 * fp32 except C and its inverse (fp64); results are deterministic. */

/* Workspace of hsq_hessian_accumulate (0: none needed; also 0 for invalid
 * sizes).  Few 128 x 128 blocks of H (small K) split the tokens across
 * workgroups, whose fp32 partial blocks live here. */
size_t hsq_hessian_workspace_bytes(int M, int K);

/* H = Xh^T Xh (accumulate = 0) or H += Xh^T Xh (accumulate = 1), over the
 * M calibration tokens of X (M x K bf16, row-major) with the layer's
 * smoothing lambda (K fp16).  Both triangles of H are written.  Stream the
 * calibration set through several calls with accumulate = 1.
 * M * K < 2^30.  Errors: HSQ_E_INVAL (null pointer, sizes, accumulate not
 * 0/1), HSQ_E_SHAPE, HSQ_E_ALIGN, HSQ_E_WORKSPACE, HSQ_E_HIP. */
int hsq_hessian_accumulate(const uint16_t *X, int M, int K, const uint16_t *lambda, float *H,
                           int accumulate, void *workspace, size_t ws_bytes, void *stream);

/* Workspace of hsq_deflate_hessian (0 for invalid sizes). */
size_t hsq_deflate_workspace_bytes(int K, int r);

/* Deflates H by span(L1) (L1: K x r bf16, the layer's input-side factor):
 *   HL1   out: K x r fp32, H L1
 *   Cinv  out: r x r fp64, (L1^T H L1)^-1 (Gauss-Jordan, partial pivoting;
 *         a singular C gives NaN)
 *   Hperp out: K x K fp32; may be H itself (in place), must not otherwise
 *         overlap it.
 * Errors: HSQ_E_INVAL, HSQ_E_SHAPE, HSQ_E_ALIGN, HSQ_E_WORKSPACE,
 * HSQ_E_HIP. */
int hsq_deflate_hessian(const float *H, int K, const uint16_t *L1, int r, float *Hperp, float *HL1,
                        double *Cinv, void *workspace, size_t ws_bytes, void *stream);

/* Workspace of hsq_closed_form_l2 (0 for invalid sizes). */
size_t hsq_closed_form_l2_workspace_bytes(int K, int N, int r);

/* The closed-form output-side factor L2* = Cinv (HL1)^T E (r x N fp32 out)
 * from the outputs of hsq_deflate_hessian and one projection's weight:
 *   W        K x N bf16, the full-precision (smoothed) weight
 *   packed_w the packed residual codes of its quantized residual
 *            (hsq_pack_weights layout), sw its (K/group) x N fp16 scales
 *   group    HSQ_GROUP_64 or HSQ_GROUP_128 (must divide K)
 * E is decoded on the fly and never stored.  K * N < 2^31.
 * Errors: HSQ_E_INVAL, HSQ_E_SHAPE, HSQ_E_ALIGN, HSQ_E_WORKSPACE,
 * HSQ_E_HIP. */
int hsq_closed_form_l2(const float *HL1, const double *Cinv, int K, int N, int r, int group,
                       const uint16_t *W, const uint8_t *packed_w, const uint16_t *sw, float *L2,
                       void *workspace, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* HSQ_H */
