/*
 * w4a4.h - C ABI of the MI355X (gfx950) W4A4 rotate / quantize / GEMM library.
 *
 * The method: a linear layer Y = X W^T is unchanged when X and W are both
 * multiplied by the same orthogonal Q, so X Q and W Q are quantized instead
 * of X and W; with Q a normalized Hadamard matrix an outlier channel is
 * spread evenly over all channels and 4-bit activations become usable.
 *   Page "Rotations for 4-Bit Activations: QuaRot, SpinQuant, and Friends",
 *   sections "A rotation changes nothing, and that is the point" (invariance,
 *   Q = H / sqrt(n)), "What it buys in 4 bits" (INT4, one scale per token and
 *   one per output channel), "Where the rotations go" (weights rotated
 *   offline, activations rotated online by a fast Hadamard transform fused
 *   with their quantization), "Gotchas" (128-wide blocks vs full width).
 *   Page "SpinQuant (learned rotations + W4A4KV4)", field "Activation scheme"
 *   (per-group asymmetric INT4 for activations and KV cache).
 *   Page "QuaRot (rotation-based outlier removal, W4A4KV4)", field
 *   "Activation scheme" (the KV cache is rotated too).
 *
 * Conventions shared by every call
 *  - All tensor pointers are DEVICE pointers owned by the caller; the
 *    library allocates no device memory and keeps no state besides its code
 *    objects, a per-device architecture check and, per host thread, the
 *    last error message and the events armed by w4a4_time_next_launch.
 *  - Every call is asynchronous and ordered on `stream` (a hipStream_t;
 *    NULL means the null stream).  Buffers must stay alive until the stream
 *    work completes.  Outputs must not alias inputs.
 *  - A call enqueues kernel launches only: no memset, copy, allocation or
 *    host synchronization.  A sequence of calls can therefore be captured
 *    into a HIP graph and replayed (the device must have been used by one
 *    uncaptured call first, for the architecture check).  A replay reads
 *    the captured pointers, so new data goes into the same buffers.
 *  - Arguments are validated on the host before anything is enqueued; on
 *    any error nothing is launched, outputs are untouched, the status says
 *    why and w4a4_last_error() holds a message.  A failed launch returns
 *    W4A4_ERR_DEVICE.  Faults during execution surface at the caller's next
 *    synchronization.
 *  - M == 0 (or B*H*S == 0) returns W4A4_OK and enqueues nothing once the
 *    modes and sizes are valid; pointers are not checked then (may be NULL).
 *  - Matrices are row-major with K contiguous; fp16 inputs are raw IEEE
 *    binary16 bit patterns (uint16_t).  NaN / Inf inputs are outside the
 *    contract: the call does not crash, the values it writes are unspecified.
 *  - Every pointer must be 16-byte aligned; row strides of fp16 inputs must
 *    be multiples of 8 elements (W4A4_ERR_ALIGN otherwise).
 *
 * Hadamard (reading of the pages): the Sylvester matrix in natural order,
 * H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]], no random signs, applied to
 * contiguous aligned blocks of `had_block` elements of every row along K
 * (had_block = 128), or to the whole row (had_block = W4A4_HAD_FULL, K a
 * power of two, 128 <= K <= 16384).  X and W must be rotated with the same
 * had_block; the codes do not record it.
 *
 * Codes (reading): two 4-bit codes per byte, even K index in bits 3:0, odd
 * index in bits 7:4; rows contiguous, K/2 bytes per row.  Symmetric codes
 * are 4-bit two's complement in [-7, 7]; asymmetric codes are unsigned
 * in [0, 15].  Rounding is to nearest, ties to even.
 *
 * Symmetric per row (reading): with z the unnormalized rotated row and
 * a = max|z| (fp32):  scale = a / fl32(7 sqrt(b)),  inv = fl32(7 / a),
 * code = rne(z * inv) (the product exact before rounding), so the
 * dequantized value scale * code approximates z / sqrt(b).  a == 0 gives
 * scale 0 and codes 0.
 * Asymmetric per group of 128 (reading): lo = min(min z, 0), hi = max(max z, 0),
 * r = fl32(hi - lo), scale = r / fl32(15 sqrt(b)), inv = fl32(15 / r),
 * zero = rne(-lo * inv), code = min(rne(z * inv) + zero, 15); dequantized
 * value scale * (code - zero).  r == 0 gives scale 0, zero 0, codes 0.
 */
#ifndef W4A4_H
#define W4A4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef W4A4_API
#define W4A4_API __attribute__((visibility("default")))
#endif

typedef enum {
  W4A4_OK = 0,
  W4A4_ERR_NULL = 1,   /* a required pointer is NULL                        */
  W4A4_ERR_SHAPE = 2,  /* a size or stride is out of range                  */
  W4A4_ERR_ALIGN = 3,  /* a pointer or row stride is misaligned             */
  W4A4_ERR_MODE = 4,   /* unknown mode or unsupported combination of modes  */
  W4A4_ERR_DEVICE = 5  /* no gfx950 device, or the launch failed            */
} w4a4_status;

enum { W4A4_HAD_FULL = 0, W4A4_HAD_128 = 128 };              /* had_block */
enum { W4A4_ACT_SYM_TOKEN = 0, W4A4_ACT_ASYM_G128 = 1 };     /* act_mode  */

#define W4A4_ABI_VERSION 6

/*
 * had_signs (the rotate calls and w4a4_decode_fused): NULL, or a device array of K fp16
 * values (D = 128 for kv_rotate_quant4), each +1.0 or -1.0, 16-byte aligned.
 * Non-NULL turns the rotation into the randomized Hadamard Q = diag(d) H / sqrt(b):
 * element k of every row is multiplied by d[k] (its sign bit is flipped
 * when d[k] carries one) before the per-block transform.  X and W must use
 * the same d (Q stays orthogonal, so X W^T is unchanged); the codes do not
 * record it.  Only the sign bit of each entry is read.
 *   Page "QuaRot (rotation-based outlier removal, W4A4KV4)", field
 *   "Activation scheme" (randomized Hadamard rotations); page "Rotations for
 *   4-Bit Activations: QuaRot, SpinQuant, and Friends", sections "Where the
 *   rotations go" and "The recipe" (random vs fixed Hadamard).  The random
 *   signs are drawn by the caller and passed in.
 */

/*
 * rotate_quant_act - online activation step: per row of X, one fast
 * Walsh-Hadamard transform (per 128-block or full width) fused with INT4
 * quantization and nibble packing.
 *   Page "Rotations for 4-Bit Activations: QuaRot, SpinQuant, and Friends",
 *   section "Where the rotations go" (online Hadamard per token, fused with
 *   activation quantization); section "What it buys in 4 bits" (one scale
 *   per token); page "SpinQuant (learned rotations + W4A4KV4)", field
 *   "Activation scheme" (per-group asymmetric INT4).
 *
 *   x_f16   [M][ldx] fp16, only the first K of each row are read.
 *   M >= 0; K >= 128, K % 128 == 0, K <= 16384; ldx >= K.
 *   had_block  W4A4_HAD_128, or W4A4_HAD_FULL (K a power of two <= 16384;
 *              symmetric mode only).
 *   act_mode   W4A4_ACT_SYM_TOKEN: scales [M] fp32, zeros must be NULL.
 *              W4A4_ACT_ASYM_G128: scales [M][K/128] fp32,
 *              zeros [M][K/128] uint8 (must be non-NULL); had_block 128.
 *   codes   [M][K/2] packed nibbles (written).
 */
W4A4_API w4a4_status rotate_quant_act(const uint16_t* x_f16, int64_t M, int64_t K, int64_t ldx,
                             int32_t had_block, const uint16_t* had_signs, int32_t act_mode,
                             uint8_t* codes, float* scales, uint8_t* zeros, void* stream);

/*
 * quant_weight_offline - offline weight step: rotate each output channel's
 * row of W along K, symmetric INT4 with one scale per output channel, pack;
 * optionally the per-128 group sums of the codes.
 *   Page "Rotations for 4-Bit Activations: QuaRot, SpinQuant, and Friends",
 *   section "Where the rotations go" (weights are rotated offline, free at
 *   run time); section "What it buys in 4 bits" (one scale per output
 *   channel).
 *
 *   w_f16   [N][ldw] fp16; N >= 0 (0: no-op); K as in rotate_quant_act.
 *   codes   [N][K/2] (written), scales [N] fp32 (written),
 *   gsum    NULL, or [N][K/128] int32: sum of the 128 codes of each group.
 */
W4A4_API w4a4_status quant_weight_offline(const uint16_t* w_f16, int64_t N, int64_t K, int64_t ldw,
                                 int32_t had_block, const uint16_t* had_signs,
                                 uint8_t* codes, float* scales, int32_t* gsum, void* stream);

/*
 * w4a4_gemm - Y = dequant(X codes) . dequant(W codes)^T on int8 MFMA with an
 * exact int32 accumulator (CDNA4 has no INT4 matrix instruction; the 4-bit
 * codes are widened to int8 in registers).
 *   Page "Rotations for 4-Bit Activations: QuaRot, SpinQuant, and Friends",
 *   section "A rotation changes nothing, and that is the point" (the product
 *   of the rotated operands is X W^T); section "What it buys in 4 bits".
 *
 *   act_mode W4A4_ACT_SYM_TOKEN:
 *       Y[m][n] = fl32( fl32(x_scales[m] * w_scales[n]) * acc[m][n] ),
 *       acc = sum_k qx[m][k] * qw[n][k]; x_zeros and w_gsum are ignored.
 *   act_mode W4A4_ACT_ASYM_G128 (x_zeros, x_scales [M][K/128]):
 *       Y[m][n] = w_scales[n] * sum_g x_scales[m][g] * A_g[m][n],
 *       A_g = sum_{k in group g} (qx[m][k] - x_zeros[m][g]) * qw[n][k]
 *       (exact integer per group, summed over groups in fp32).
 *       w_gsum is not read (the zero-point is removed from the codes before
 *       the product) and may be NULL.
 *   x_codes [M][K/2], w_codes [N][K/2], y [M][ldy] fp32 (written).
 *   M >= 0, N >= 1, K >= 128, K % 128 == 0, K <= 131072, ldy >= N.
 *   M <= 16 uses a weight-streaming kernel, larger M the tiled MFMA kernel;
 *   both compute the same values.
 */
W4A4_API w4a4_status w4a4_gemm(const uint8_t* x_codes, const float* x_scales, const uint8_t* x_zeros,
                      int32_t act_mode, const uint8_t* w_codes, const float* w_scales,
                      const int32_t* w_gsum, int64_t M, int64_t N, int64_t K,
                      float* y, int64_t ldy, void* stream);

/*
 * w4a4_decode_fused - the decode linear layer in one launch: exactly
 * rotate_quant_act(x, M, K, ldx, W4A4_HAD_128, had_signs, W4A4_ACT_SYM_TOKEN)
 * followed by w4a4_gemm(symmetric) on w_codes / w_scales, with the
 * activation codes and scales kept on chip.  Y equals the two-call result
 * bit for bit.
 *   Page "Rotations for 4-Bit Activations: QuaRot, SpinQuant, and Friends",
 *   section "Where the rotations go" (the online rotation is fused with the
 *   quantization; here also with the product), section "A rotation changes
 *   nothing, and that is the point".
 *
 *   x_f16    [M][ldx] fp16; 1 <= M <= 16; K a multiple of 128 in [128, 8192],
 *            M * K <= 65536; ldx >= K, a multiple of 8, < 2^24.
 *   had_signs  NULL or the fp16 +-1 vector [K] (as in rotate_quant_act).
 *   w_codes  [N][K/2], w_scales [N] fp32, as quant_weight_offline writes them
 *            with had_block 128 and the same had_signs.
 *   y        [M][ldy] fp32 (written); N >= 1, ldy >= N.
 *   Larger M or K: use the two calls.
 */
W4A4_API w4a4_status w4a4_decode_fused(const uint16_t* x_f16, int64_t M, int64_t K, int64_t ldx,
                             const uint16_t* had_signs, const uint8_t* w_codes, const float* w_scales,
                             int64_t N, float* y, int64_t ldy, void* stream);

/*
 * kv_rotate_quant4 - KV-cache step: every (b, h, s) head vector of D = 128
 * fp16 values is rotated by one 128-point Hadamard and quantized to
 * asymmetric INT4 with one (scale, zero) per vector.
 *   Page "QuaRot (rotation-based outlier removal, W4A4KV4)", field
 *   "Activation scheme" (the KV cache is rotated); page "SpinQuant (learned
 *   rotations + W4A4KV4)", field "Activation scheme" (per-group asymmetric
 *   INT4 on the KV cache, 4-bit KV).
 *
 *   kv_f16  element (b,h,s,d) at b*stride_b + h*stride_h + s*stride_s + d
 *           (strides in elements, multiples of 8; d contiguous).
 *   D == 128; B, H, S >= 0; B*H*S < 2^31.
 *   codes  [B][H][S][64], scales [B][H][S] fp32, zeros [B][H][S] uint8 (written,
 *          dense).
 */
W4A4_API w4a4_status kv_rotate_quant4(const uint16_t* kv_f16, int64_t B, int64_t H, int64_t S, int64_t D,
                             int64_t stride_b, int64_t stride_h, int64_t stride_s,
                             const uint16_t* had_signs,
                             uint8_t* codes, float* scales, uint8_t* zeros, void* stream);

/*
 * kv4_attention_decode - single-query attention per (batch, head) over a KV
 * cache that kv_rotate_quant4 stored as rotated asymmetric INT4:
 *   o[b][h] = sum_t p_t v[b][h][t],  p = softmax_t(softmax_scale * q[b][h] . k[b][h][t]),
 * computed without leaving the rotated domain: the query is rotated by the
 * same Q = diag(d) H_128 / sqrt(128) as the cache, scores and the weighted
 * value sum use the dequantized rotated vectors s (code - zero), and the
 * result is rotated back once (o = o_rot Q^T).
 *   Page "QuaRot (rotation-based outlier removal, W4A4KV4)", field
 *   "Activation scheme" (the KV cache and parts of the attention computation
 *   are rotated); page "Rotations for 4-Bit Activations: QuaRot, SpinQuant,
 *   and Friends", section "A rotation changes nothing, and that is the point".
 *
 *   q_f16     [B][H][128] fp16, dense (one decode query per head).
 *   k_codes, v_codes    [B][H][S][64], k_scales, v_scales [B][H][S] fp32,
 *   k_zeros, v_zeros    [B][H][S] uint8: dense, as kv_rotate_quant4 writes them.
 *   D == 128; B, H >= 0 (B*H == 0: no-op); 1 <= S < 2^25.
 *   softmax_scale  finite, > 0 (typically 1/sqrt(128)).
 *   had_signs NULL, or the fp16 +-1 vector [128] the cache was rotated with.
 *   out       [B][H][128] fp32 (written).
 * Arithmetic: the scores take the rotated query in 20-bit fixed point
 * (q ~ sq * qi, |qi| <= 2^19 - 1, sq = max|q| / (2^19 - 1): at most 2^-20 of
 * max|q| per element) on exact integer dot products with the codes; the
 * softmax and the weighted value sum are fp32.
 * One workgroup per (b, h); every token's codes are read once.
 */
W4A4_API w4a4_status kv4_attention_decode(const uint16_t* q_f16, const uint8_t* k_codes,
                             const float* k_scales, const uint8_t* k_zeros,
                             const uint8_t* v_codes, const float* v_scales, const uint8_t* v_zeros,
                             int64_t B, int64_t H, int64_t S, int64_t D, float softmax_scale,
                             const uint16_t* had_signs, float* out, void* stream);

/*
 * kv4_attention_workspace_bytes - bytes of workspace kv4_attention_decode_ws
 * needs for B*H heads of S cached tokens: 0 when it takes the single pass
 * (enough heads to give every compute unit a workgroup), else
 * B * H * ranges * 528 with ranges = min(64, ceil(256 / (B H)), S / 512).
 * Returns -1 (message in w4a4_last_error) when B, H or S is out of the
 * ranges kv4_attention_decode accepts.  Host only; enqueues nothing.
 */
W4A4_API int64_t kv4_attention_workspace_bytes(int64_t B, int64_t H, int64_t S);

/*
 * kv4_attention_decode_ws - kv4_attention_decode for caches with few heads:
 * the same result (same arguments, same rules, same output), computed with
 * the S tokens of every head split into ranges that separate workgroups
 * take, so that B*H heads still spread over the whole GPU.  Each range
 * leaves its online-softmax state (rotated output sum, running maximum and
 * sum) in `workspace`; a second kernel merges a head's states (the split of
 * the softmax sum: o = sum_r 2^(m_r - M) o_r / sum_r 2^(m_r - M) l_r),
 * normalizes and rotates back.  Only the fp32 summation order differs from
 * kv4_attention_decode.
 *   Page "QuaRot (rotation-based outlier removal, W4A4KV4)", field
 *   "Activation scheme"; page "Rotations for 4-Bit Activations: QuaRot,
 *   SpinQuant, and Friends", section "A rotation changes nothing, and that
 *   is the point".
 *
 *   workspace        device buffer owned by the caller, 16-byte aligned, of
 *                    workspace_bytes >= kv4_attention_workspace_bytes(B, H, S)
 *                    bytes (W4A4_ERR_SHAPE if smaller); may be NULL when that
 *                    size is 0.  Its contents on entry do not matter; the
 *                    call overwrites them, and calls that overlap in time
 *                    must not share one workspace.
 * Two kernels are enqueued on `stream` (one when the single pass is taken).
 */
W4A4_API w4a4_status kv4_attention_decode_ws(const uint16_t* q_f16, const uint8_t* k_codes,
                             const float* k_scales, const uint8_t* k_zeros,
                             const uint8_t* v_codes, const float* v_scales, const uint8_t* v_zeros,
                             int64_t B, int64_t H, int64_t S, int64_t D, float softmax_scale,
                             const uint16_t* had_signs, float* out, void* workspace,
                             int64_t workspace_bytes, void* stream);

/*
 * kv4_attention_decode_noalloc - kv4_attention_decode_ws for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same kernels, the same result,
 * with the partial states kept in a static device array of the library
 * instead of a caller's workspace.  The call itself allocates nothing.
 *
 *   Limit: that array holds 524,288 bytes (512 KiB) on each GPU the library
 *   runs on, kept until the process ends; a shape whose
 *   kv4_attention_workspace_bytes(B, H, S) exceeds it is refused with
 *   W4A4_ERR_SHAPE (no valid shape needs more than 269,280 bytes).
 *   Every call on one GPU uses that GPU's one array: calls that overlap in
 *   time on one GPU (two streams, two threads) race and give wrong output;
 *   order them on one stream.  Nothing in the array needs to start at zero:
 *   each call writes every state it later reads.
 * Arguments, rules and output as kv4_attention_decode.
 */
W4A4_API w4a4_status kv4_attention_decode_noalloc(const uint16_t* q_f16, const uint8_t* k_codes,
                             const float* k_scales, const uint8_t* k_zeros,
                             const uint8_t* v_codes, const float* v_scales, const uint8_t* v_zeros,
                             int64_t B, int64_t H, int64_t S, int64_t D, float softmax_scale,
                             const uint16_t* had_signs, float* out, void* stream);

/*
 * rotate_quant_mxfp4 - the rotate step with MXFP4 output: per row, the same
 * normalized Hadamard as rotate_quant_act (per 128-block or full width,
 * optionally randomized), then every 32 consecutive values share one
 * power-of-two scale and become E2M1 codes.  Serves activations online and
 * weights offline alike (both operands of mxfp4_gemm).
 *   Page "Rotations for 4-Bit Activations: QuaRot, SpinQuant, and Friends",
 *   sections "The full model in NVFP4, on vLLM" and "When to rotate"
 *   (rotations help MXFP4: 4-bit values with a power-of-two scale per 32).
 *   The pages give no formulas; the conversion is the usual MX one:
 *     y = fl32(fl32(z) * fl32(1/sqrt(b))), z = the unnormalized transform;
 *     e = floor(log2(max |y| over the 32)) - 2, clamped to [-127, 127]
 *         (a block of zeros: e = -127);
 *     code = E2M1 nearest to y / 2^e (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6
 *            for codes 0..7, bit 3 = sign, ties to the even code,
 *            saturating at 6, no negative zero).
 *
 *   x_f16, M, K, ldx, had_block as in rotate_quant_act (had_block
 *   W4A4_HAD_FULL needs K a power of two).
 *   codes        [M][K/2] packed, element 2i in the low nibble of byte i (written).
 *   scales_e8m0  [M][K/32] uint8 biased exponents e + 127 (written).
 */
W4A4_API w4a4_status rotate_quant_mxfp4(const uint16_t* x_f16, int64_t M, int64_t K, int64_t ldx,
                               int32_t had_block, const uint16_t* had_signs, uint8_t* codes,
                               uint8_t* scales_e8m0, void* stream);

/*
 * mxfp4_gemm - Y = dequant(X) . dequant(W)^T for MXFP4 operands, on
 * gfx950's block-scaled FP4 matrix instruction:
 *   Y[m][n] = sum_j 2^(ex[m][j] + ew[n][j]) * sum_{k in 32-block j} a[m][k] b[n][k],
 * a, b the E2M1 values of the codes, e = scale byte - 127; accumulated in
 * fp32 (the result agrees with the exact sum to fp32 rounding).
 *   Same pages and sections as rotate_quant_mxfp4; page "Rotations for
 *   4-Bit Activations: QuaRot, SpinQuant, and Friends", section "A rotation
 *   changes nothing, and that is the point" (the product of the rotated
 *   operands is X W^T).
 *
 *   x_codes [M][K/2], x_scales_e8m0 [M][K/32]; w_codes [N][K/2],
 *   w_scales_e8m0 [N][K/32], as rotate_quant_mxfp4 writes them; scale
 *   byte 255 (not produced by the quantizer) gives NaN.
 *   y [M][ldy] fp32 (written).
 *   M >= 0, N >= 1, K >= 128, K % 128 == 0, K <= 131072, ldy >= N.
 *   M <= 16 uses a weight-streaming kernel, larger M the tiled kernel.
 */
W4A4_API w4a4_status mxfp4_gemm(const uint8_t* x_codes, const uint8_t* x_scales_e8m0,
                       const uint8_t* w_codes, const uint8_t* w_scales_e8m0,
                       int64_t M, int64_t N, int64_t K, float* y, int64_t ldy, void* stream);

/* Message of the last failed call on this thread ("" after a success). */
W4A4_API const char* w4a4_last_error(void);

/* W4A4_ABI_VERSION of the loaded library. */
W4A4_API int32_t w4a4_abi_version(void);

/* Timing hook, outside the method: arms two HIP events (hipEvent_t values
 * the caller created, e.g. with hipEventCreate, and still owns) for the next
 * entry-point call on this host thread.  The kernel that call enqueues is
 * launched with them attached, so the runtime writes the kernel's own start
 * and end timestamps into them and hipEventElapsedTime(start, stop) is its
 * device duration, without the queue gaps that hipEventRecord markers put
 * between kernels.  The entry point disarms the pair when it returns, also
 * when it fails or enqueues nothing.  Both NULL disarms; exactly one NULL is
 * W4A4_ERR_NULL.  Per host thread; needs no device. */
W4A4_API w4a4_status w4a4_time_next_launch(void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* W4A4_H */
