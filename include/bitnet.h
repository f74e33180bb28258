/*
 * bitnet.h -- C ABI of the MI355X (gfx950) BitNet b1.58 BitLinear hot path.
 *
 * Pages the operations follow (cited by title and section):
 *   [NOTES] "BitNet 1.5技术解析：2比特量化在神经网络中的应用与挑战"
 *           (intelliparadigm.com): 2.1 weight quantization, 2.2 activation
 *           quantization, 3.1 the BitLinear layer, 5.1 graph optimization
 *           (fused quantize / dequantize), 5.2 hardware needs.
 *   [ENG]   "BitNet 三元权重量化训练工程：直通估计器与梯度裁剪实践"
 *           (blog.hotdry.top, 2025-10-04): section on the straight-through
 *           estimator for ternary weights (absmean, absmax per token,
 *           eps = 1e-5); section on gradient clipping (bf16 forward, fp32
 *           gradients).
 *   [WALL]  "1.58-bit量化技术突破AI算力与内存墙限制" (intelliparadigm.com):
 *           1 the memory wall, 2.2 ternary quantization, 3.1 add/subtract
 *           matmul, 3.2 the STE, 4.1 2-bit memory layout, 5.1 deployment
 *           (item 2: packing aligned for the loads).
 *
 * Conventions shared by every call
 *   - Tensors are row-major and contiguous.  Every tensor pointer is a
 *     DEVICE pointer on the current HIP device unless a comment says
 *     otherwise; gamma and scale_x stay on the device (no call copies to
 *     the host).  Pointers must be 16-byte aligned.
 *   - Ownership: the caller allocates and frees every buffer.  The library
 *     never allocates device memory, keeps no pointer after returning and
 *     has no mutable global state, except the fixed device scratch of
 *     bitnet_weight_quant_noalloc (one static array per device, described
 *     there) and the host-side test setting of bitnet_set_gate_polls.
 *   - Asynchrony: a call validates its arguments on the host, enqueues its
 *     kernels on `stream` (a hipStream_t passed as void*; NULL = the null
 *     stream) and returns.  Outputs are valid once the stream reaches that
 *     point.  Calls on one stream run in order.
 *   - Errors: every argument check runs before any launch; on failure the
 *     call returns a negative bitnet_status and enqueues nothing.  A failed
 *     launch returns BITNET_E_HIP.  No C++ exception crosses the ABI.
 *     NaN or Inf inputs give unspecified (but memory-safe) results.
 *   - Determinism: the same inputs give the same output bits (no floating
 *     point atomics; every reduction has a fixed order).
 *   - Sizes: M tokens, K input features, N output features; 1 <= M, N, K
 *     < 2^31.  K % 4 == 0 for the quantizer and packing calls (whole packed
 *     bytes); K % 16 == 0 for the linear calls (whole packed dwords).
 *   - Built for gfx950 only; on any other device a launch fails and the call
 *     returns BITNET_E_HIP.
 *
 * Packed ternary weights ([WALL 4.1]): 2 bits per weight, 00 = 0,
 * 01 = +1, 10 = -1 (11 never written).  Row n of W occupies K/4 bytes
 * starting at byte n*K/4; the code of column k sits in bits 2*(k%4) and
 * 2*(k%4)+1 of byte k/4 of its row.  The bit order is this library's choice
 * (the page fixes only the codes).
 */
#ifndef BITNET_H_
#define BITNET_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BITNET_OK = 0,
    BITNET_E_ARG = -1,       /* null required pointer or bad flag          */
    BITNET_E_SHAPE = -2,     /* M, N or K out of range or K not a multiple  */
    BITNET_E_DTYPE = -3,     /* unknown or unsupported dtype code           */
    BITNET_E_ALIGN = -4,     /* a pointer is not 16-byte aligned            */
    BITNET_E_WORKSPACE = -5, /* workspace missing or smaller than required  */
    BITNET_E_HIP = -6,       /* a HIP launch or runtime call failed         */
    BITNET_E_SCRATCH = -7    /* size beyond a no-allocation call's scratch  */
} bitnet_status;

typedef enum { BITNET_F32 = 0, BITNET_BF16 = 1 } bitnet_dtype;

/* layout of packed weights handed to bitnet_linear_fwd_decode */
typedef enum { BITNET_LAYOUT_ROWS = 0, BITNET_LAYOUT_DECODE = 1 } bitnet_layout;

typedef enum {
    BITNET_OP_WEIGHT_QUANT = 0,
    BITNET_OP_LINEAR_BWD_STE = 1,
    BITNET_OP_LINEAR_FWD = 2,
    BITNET_OP_CODE_COUNTS = 3,
    BITNET_OP_WEIGHT_QUANT_ROWS = 4,
    BITNET_OP_WEIGHT_QUANT_COUNTED = 5
} bitnet_op;

/*
 * Absmean ternary weight quantization and 2-bit packing.
 * [NOTES 2.1], [WALL 2.2], [ENG STE section]:
 *   gamma = max(mean|W|, 1e-5) over the WHOLE matrix,
 *   code  = clamp(round(W / gamma), -1, 1), round = half to even.
 * The mean is evaluated in binary32 in one fixed order: per row a pairwise
 * tree over the row (zero-padded to a power of two), then a pairwise tree
 * over the N row sums, then one division by the binary32 value of N*K.
 * W / gamma is the correctly rounded binary32 quotient.
 *   W        [N][K] fp32 or bf16 (w_dtype)
 *   W_packed [N][K/4] bytes, written
 *   gamma    1 float, written (device)
 *   workspace >= bitnet_workspace_bytes(BITNET_OP_WEIGHT_QUANT, 0, N, K)
 *            bytes of device scratch (row sums); contents on entry ignored.
 * Errors: BITNET_E_ARG, BITNET_E_SHAPE (K % 4), BITNET_E_DTYPE,
 * BITNET_E_ALIGN, BITNET_E_WORKSPACE, BITNET_E_HIP.
 */
int bitnet_weight_quant(const void *W, int w_dtype, int64_t N, int64_t K,
                        uint8_t *W_packed, float *gamma,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * bitnet_weight_quant without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same operation, same kernels and the same output
 * bits as bitnet_weight_quant; its row sums, tree nodes and code threshold live in a
 * fixed device array inside the library instead of the caller's workspace.
 *   W, w_dtype, N, K, W_packed, gamma as bitnet_weight_quant
 *   N <= BITNET_NOALLOC_MAX_N (the scratch holds that many row sums,
 *   1.25 MiB + 256 bytes per device); larger N returns BITNET_E_SCRATCH.
 * The call allocates nothing: no hipMalloc, hipFree or allocating library
 * routine.  Each GPU holds one copy of the scratch from the first call on it
 * until the process ends, and every call on that GPU shares it: calls that
 * overlap on one GPU (on different streams, or from several threads without
 * ordering) race on it and give undefined results.  Calls ordered on one
 * stream are safe; nothing in the scratch needs clearing between calls.
 * Errors: BITNET_E_ARG, BITNET_E_SHAPE (K % 4), BITNET_E_DTYPE,
 * BITNET_E_SCRATCH, BITNET_E_ALIGN, BITNET_E_HIP.
 */
#define BITNET_NOALLOC_MAX_N ((int64_t)1 << 18)
int bitnet_weight_quant_noalloc(const void *W, int w_dtype, int64_t N, int64_t K,
                                uint8_t *W_packed, float *gamma, void *stream);

/*
 * RMSNorm (unit gain) followed by per-token absmax int8 quantization.
 * [NOTES 3.1] (RMSNorm before the quantizer), [NOTES 2.2] and [ENG STE
 * section] (per-row scale 127 / max|x|, max clamped at 1e-5, eps = 1e-5):
 *   d       = sqrt(sum_k x^2 / K + eps)     (pairwise tree over the row)
 *   n_k     = x_k * (1 / d)
 *   scale_x = 127 / max(max_k |n_k|, 1e-5)
 *   q_k     = clamp(round(n_k * scale_x), -128, 127), round half to even
 * every operation a single correctly rounded binary32 operation.
 *   X       [M][K] fp32 or bf16 (x_dtype)
 *   Xq      [M][K] int8, written
 *   scale_x [M] fp32, written
 * Errors: BITNET_E_ARG, BITNET_E_SHAPE, BITNET_E_DTYPE, BITNET_E_ALIGN,
 * BITNET_E_HIP.
 */
int bitnet_act_quant(const void *X, int x_dtype, int64_t M, int64_t K, float eps,
                     int8_t *Xq, float *scale_x, void *stream);

/*
 * Both quantizers of a BitLinear layer in one call: bitnet_act_quant of X and
 * bitnet_weight_quant of W, with one kernel launch fewer ([NOTES 5.1]: fuse
 * the quantization steps).  The first launch reads X and W side by side
 * (activation rows and weight row sums on separate workgroups of one grid);
 * the outputs are bit-identical to the two calls.
 *   X [M][K], W [N][K] fp32 or bf16 (x_dtype, w_dtype; same K)
 *   Xq, scale_x as bitnet_act_quant;  W_packed, gamma as bitnet_weight_quant
 *   workspace >= bitnet_workspace_bytes(BITNET_OP_WEIGHT_QUANT, 0, N, K)
 * K % 4 == 0.  Errors: the union of the two calls' (BITNET_E_ARG,
 * BITNET_E_SHAPE, BITNET_E_DTYPE, BITNET_E_ALIGN, BITNET_E_WORKSPACE,
 * BITNET_E_HIP).
 */
int bitnet_quant_operands(const void *X, int x_dtype, int64_t M, int64_t K, float eps, int8_t *Xq,
                          float *scale_x, const void *W, int w_dtype, int64_t N,
                          uint8_t *W_packed, float *gamma, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * BitLinear forward from the quantized operands.
 * [NOTES 3.1] (linear layer, then multiply back by the scale), [NOTES 5.2]
 * (wide accumulator), [WALL 3.1] (+1 adds, -1 subtracts, 0 skips):
 *   acc[m][n] = sum_k Xq[m][k] * code[n][k]      (exact int32)
 *   Y[m][n]   = acc[m][n] * gamma / scale_x[m]   (fp32)
 * M <= 16 (with K <= 16384) takes the bandwidth-bound packed GEMV (one
 * token with K % 64 == 0 and K <= 8192: a VALU row GEMV, lanes across K),
 * 17 <= M <= 64 the same GEMV once per block of 16 tokens, other shapes
 * the int8 MFMA GEMM.  Every path gives the same bits.
 *   Xq       [M][K] int8;  scale_x [M] fp32;  W_packed [N][K/4];  gamma 1 fp32
 *   Y        [M][N] fp32, written
 *   acc      [M][N] int32, written when non-NULL (for exact checks)
 * |acc| <= 128*K must fit int32, so K < 2^24; K % 16 == 0.  N < 2^23 (the
 * GEMM addresses a 256-row output tile with 32-bit offsets).
 * Errors: BITNET_E_ARG, BITNET_E_SHAPE, BITNET_E_ALIGN, BITNET_E_HIP.
 */
int bitnet_linear_fwd(const int8_t *Xq, const float *scale_x, const uint8_t *W_packed,
                      const float *gamma, int64_t M, int64_t N, int64_t K,
                      float *Y, int32_t *acc, void *stream);

/*
 * Straight-through-estimator backward of the BitLinear forward above.
 * [NOTES 2.1, 2.2] (the detach trick), [WALL 3.2] (the backward passes the
 * incoming gradient through): both quantizers act as the identity, so with
 * W_deq = gamma * code and X_deq = Xq / scale_x
 *   grad_x[m][k] = sum_n grad_y[m][n] * W_deq[n][k]
 *   grad_W[n][k] = sum_m grad_y[m][n] * X_deq[m][k]
 * computed on bf16 matrix cores with fp32 accumulation ([ENG clipping
 * section]: bf16 forward, fp32 gradients).  grad_x is the gradient with
 * respect to the quantizer input (the RMSNorm output).
 *   grad_y  [M][N] bf16 (gy_dtype must be BITNET_BF16)
 *   Xq [M][K] int8, scale_x [M] fp32, W_packed [N][K/4], gamma 1 fp32
 *   grad_x  [M][K] fp32 or bf16 (gx_dtype), written when non-NULL
 *   grad_W  [N][K] fp32, written when non-NULL
 *   workspace >= bitnet_workspace_bytes(BITNET_OP_LINEAR_BWD_STE, M, N, K)
 *            device scratch of grad_W: fp32 partial tiles when its output is
 *            too small to fill the GPU and the token range is split
 *            (splits*N*K*4 bytes), and X_deq transposed (K rows of M rounded
 *            up to 8 tokens, bf16) for a tall output (N >= 8192) on the large
 *            tiles; 0 bytes when neither applies, then NULL is allowed;
 *            contents on entry ignored.
 * K % 16 == 0, K < 2^24, N < 2^23 (tile loads use 32-bit offsets).
 * Errors: BITNET_E_ARG (both outputs NULL), BITNET_E_SHAPE, BITNET_E_DTYPE,
 * BITNET_E_ALIGN, BITNET_E_WORKSPACE, BITNET_E_HIP.
 */
int bitnet_linear_bwd_ste(const void *grad_y, int gy_dtype, const int8_t *Xq,
                          const float *scale_x, const uint8_t *W_packed, const float *gamma,
                          int64_t M, int64_t N, int64_t K,
                          void *grad_x, int gx_dtype, float *grad_W,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Range-gated STE for the master weights: bitnet_linear_bwd_ste, except that
 * grad_W[n][k] is 0 wherever the master weight W[n][k] lies outside
 * [w_lo, w_hi] (both bounds inclusive, decided on the binary32 value of W).
 * "BitNet量化感知训练中的梯度传播优化" (blog.hotdry.top), section on the
 * straight-through estimator: the gradient handed to the full-precision
 * weight is masked by |w| <= 1 (w_lo = -1, w_hi = 1); zyxy.net lecture on
 * STE design, section 7: a quantizer over [a, b] passes the gradient where
 * a <= w <= b.  grad_x is unchanged.
 *   W  [N][K] fp32 or bf16 (w_dtype): the master weights the codes came from
 * Other arguments, sizes, workspace and errors as bitnet_linear_bwd_ste;
 * also BITNET_E_ARG for W NULL or a NaN bound.
 */
int bitnet_linear_bwd_ste_gated(const void *grad_y, int gy_dtype, const int8_t *Xq,
                                const float *scale_x, const uint8_t *W_packed,
                                const float *gamma, const void *W, int w_dtype, float w_lo,
                                float w_hi, int64_t M, int64_t N, int64_t K, void *grad_x,
                                int gx_dtype, float *grad_W, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * Clamp the master weights in place to [lo, hi] after an update (same blog,
 * section on the BitLinear implementation: the weights are kept in [-1, 1]).
 * w < lo -> lo, w > hi -> hi, any other value (NaN included) keeps its bits;
 * for bf16 W a bound that bf16 cannot hold is rounded to nearest even.
 *   W  [N][K] fp32 or bf16 (w_dtype), read and written
 * Errors: BITNET_E_ARG (W NULL, lo > hi or a NaN bound), BITNET_E_SHAPE,
 * BITNET_E_DTYPE, BITNET_E_ALIGN, BITNET_E_HIP.
 */
int bitnet_weight_clamp(void *W, int w_dtype, int64_t N, int64_t K, float lo, float hi,
                        void *stream);

/*
 * Per-output-channel weight scales: one scale per output row instead of one
 * per matrix ("BitNet量化感知训练中的梯度传播优化" (blog.hotdry.top), section
 * on the BitLinear implementation, 1: output = (sign(W) . s) x with
 * s in R^{d_out}; zyxy.net STE lecture: the mean of |w| along each row).
 *
 * bitnet_weight_quant_rows: the absmean rule of bitnet_weight_quant applied
 * to every row on its own,
 *   gamma[n] = max(T(|W[n][:]|) / K, 1e-5)  (T: the row's pairwise tree),
 *   code     = clamp(round(W[n][k] / gamma[n]), -1, 1), half to even,
 * bit-exact like the per-matrix call.  gamma [N] fp32 (device), written;
 * workspace >= bitnet_workspace_bytes(BITNET_OP_WEIGHT_QUANT_ROWS, 0, N, K).
 * Errors as bitnet_weight_quant.
 *
 * bitnet_linear_fwd_channel: bitnet_linear_fwd with a scale per output
 * channel s[N] (the gamma of bitnet_weight_quant_rows, or a learned scale):
 *   y[m][n] = (acc[m][n] * (1 / scale_x[m])) * s[n]   (fp32)
 * Arguments, limits and errors as bitnet_linear_fwd.
 *
 * bitnet_linear_bwd_ste_channel: the STE backward at W_deq[n][k] =
 * s[n] * code[n][k]: grad_x[m][k] = sum_n grad_y[m][n] * s[n] * code[n][k]
 * (s rounded to bf16 once for the bf16 matrix cores); grad_W as
 * bitnet_linear_bwd_ste.  Arguments, workspace and errors as
 * bitnet_linear_bwd_ste with s [N] fp32 (device) in place of gamma.
 */
int bitnet_weight_quant_rows(const void *W, int w_dtype, int64_t N, int64_t K,
                             uint8_t *W_packed, float *gamma, void *workspace,
                             size_t workspace_bytes, void *stream);
int bitnet_linear_fwd_channel(const int8_t *Xq, const float *scale_x, const uint8_t *W_packed,
                              const float *s, int64_t M, int64_t N, int64_t K, float *Y,
                              int32_t *acc, void *stream);

/*
 * Gradient of a LEARNED per-output-channel scale s ("BitNet量化感知训练中的
 * 梯度传播优化" (blog.hotdry.top), section on the BitLinear implementation,
 * 1: output = (sign(W) . s) x, s in R^{d_out x 1} learned by gradient
 * descent).  With the forward of bitnet_linear_fwd_channel,
 *   y[m][n] = s[n] * sum_k X_deq[m][k] * code[n][k],  X_deq = Xq / scale_x,
 * the chain rule gives grad_s[n] = sum_m grad_y[m][n] * sum_k X_deq[m][k] *
 * code[n][k]; exchanging the sums,
 *   grad_s[n] = sum_k code[n][k] * grad_W[n][k]
 * where grad_W = grad_y^T X_deq is the (ungated) grad_W output of
 * bitnet_linear_bwd_ste_channel / bitnet_linear_bwd_ste on the same
 * operands.  Each product is one binary32 multiplication (exact for codes in
 * {-1, 0, +1}); each row is summed in binary32 as a pairwise tree over the
 * row zero-padded to a power of two (the order of bitnet_weight_quant's
 * sums); a zero total is written as +0.  The result follows from grad_W
 * bit for bit.
 *   grad_W   [N][K] fp32, read
 *   W_packed [N][K/4] packed codes ([WALL 4.1] layout)
 *   grad_s   [N] fp32, written
 * K % 16 == 0, K < 2^24.
 * Errors: BITNET_E_ARG, BITNET_E_SHAPE, BITNET_E_ALIGN, BITNET_E_HIP.
 */
int bitnet_channel_scale_grad(const float *grad_W, const uint8_t *W_packed, int64_t N, int64_t K,
                              float *grad_s, void *stream);

/*
 * Decode forward from the unquantized activations in one launch: the
 * activation quantizer of bitnet_act_quant fused into the packed GEMV of
 * bitnet_linear_fwd ([NOTES 5.1]: fuse the quantize and dequantize steps with
 * the product).  Every workgroup quantizes the M <= 16 token rows itself
 * with bitnet_act_quant's arithmetic, operation for operation, so
 *   Y (and Xq, scale_x when requested) are bit-identical to
 *   bitnet_act_quant(X, ..., eps) followed by bitnet_linear_fwd.
 *   X        [M][K] fp32 or bf16 (x_dtype);  gamma 1 fp32
 *   W_packed [N][K/4] packed rows (w_layout BITNET_LAYOUT_ROWS), or the
 *            same weights in the decode layout of bitnet_pack_decode
 *            (BITNET_LAYOUT_DECODE: K == 4096 only; the results are the same
 *            bits, the weight stream reads whole kilobytes)
 *   Y        [M][N] fp32, written
 *   Xq       [M][K] int8, written when non-NULL (16-byte aligned)
 *   scale_x  [M] fp32, written when non-NULL
 * Every workgroup quantizes all M rows itself, so this pays off for a few
 * tokens (measured at K = 4096, N = 11008: 15-20% faster than the two calls
 * at M = 1 and 2, even at M = 8, slower at M = 16).
 * 1 <= M <= 16, K % 16 == 0, K <= 4096 (the quantized rows stay in LDS);
 * fp32 X also M * ceil(K / 256) <= 128 (the raw rows stay in registers: up
 * to 8 rows of 4096); N < 2^23; eps >= 0.  Other shapes: bitnet_act_quant
 * followed by bitnet_linear_fwd.
 * Errors: BITNET_E_ARG (also an unknown w_layout), BITNET_E_SHAPE,
 * BITNET_E_DTYPE, BITNET_E_ALIGN, BITNET_E_HIP.
 */
int bitnet_linear_fwd_decode(const void *X, int x_dtype, const uint8_t *W_packed, int w_layout,
                             const float *gamma, int64_t M, int64_t N, int64_t K, float eps,
                             float *Y, int8_t *Xq, float *scale_x, void *stream);

/*
 * The decode layout: the packed weights of [WALL 4.1] rearranged, once per
 * weight update, into the order in which the decode GEMV's wavefronts load
 * them.  A decode step reads all of W for a few tokens, so it is bound by
 * memory bandwidth ([WALL 1], the memory wall), and [WALL 4.1] and 5.1
 * (item 2) lay the packed weights out for the loads that read them.
 * The GEMV works on row groups of 16 rows, split over 16 waves of 64 lanes;
 * for K = 4096 wave v reads, for row 16 grp + c, packed bytes
 * 64 v + 16 g .. + 15 in lane 16 g + c.  Those 16-byte pieces are stored as
 *   W_decode[((grp * 16 + v) * 64 + 16 g + c) * 16 + b]
 *       = W_packed[16 grp + c][64 v + 16 g + b]    (b = 0..15)
 * with zeros for rows 16 grp + c >= N, so that every load instruction of the
 * GEMV reads one contiguous kilobyte.  Byte values are copied, nothing else.
 *   W_packed [N][K/4] bytes, device, 16-byte aligned, read
 *   W_decode bitnet_decode_layout_bytes(N, K) = ceil(N/16) * 16 * K/4 bytes,
 *            device, 16-byte aligned, written; must not overlap W_packed
 * K == 4096 (the shape bitnet_linear_fwd_decode takes in this layout),
 * 1 <= N < 2^23.  bitnet_decode_layout_bytes returns -1 for other shapes.
 * Errors: BITNET_E_ARG, BITNET_E_SHAPE, BITNET_E_ALIGN, BITNET_E_HIP.
 */
int64_t bitnet_decode_layout_bytes(int64_t N, int64_t K);
int bitnet_pack_decode(const uint8_t *W_packed, int64_t N, int64_t K, uint8_t *W_decode,
                       void *stream);
int bitnet_linear_bwd_ste_channel(const void *grad_y, int gy_dtype, const int8_t *Xq,
                                  const float *scale_x, const uint8_t *W_packed, const float *s,
                                  int64_t M, int64_t N, int64_t K, void *grad_x, int gx_dtype,
                                  float *grad_W, void *workspace, size_t workspace_bytes,
                                  void *stream);

/*
 * Counts of the codes in packed ternary weights, for the monitoring the
 * pages ask for: the share of zero codes ([NOTES 6], practice notes, item 3)
 * and the balance of +1 against -1 ("BitNet量化感知训练中的梯度传播优化",
 * section on convergence monitoring: over-sparse weights, polarity
 * imbalance).  Exact integers:
 *   counts[0] = zeros, counts[1] = +1, counts[2] = -1, counts[3] = fields
 *   holding the unused pattern 11 (0 for anything this library packed)
 *   W_packed [N][K/4] bytes ([WALL 4.1] layout above); K % 4 == 0
 *   counts   4 uint64, DEVICE memory, 8-byte aligned, written
 *   workspace >= bitnet_workspace_bytes(BITNET_OP_CODE_COUNTS, 0, N, K) bytes
 *            of device scratch (per-workgroup partial counts; no atomics,
 *            so the counts need no clearing); contents on entry ignored.
 * Errors: BITNET_E_ARG, BITNET_E_SHAPE, BITNET_E_ALIGN, BITNET_E_WORKSPACE,
 * BITNET_E_HIP.
 */
int bitnet_code_counts(const uint8_t *W_packed, int64_t N, int64_t K, uint64_t *counts,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * bitnet_weight_quant and bitnet_code_counts of its result in one call: the
 * workgroups that write the packed codes also count them, so the counts
 * need no second read of W_packed ([NOTES 6], practice notes, item 3: the
 * zero share; "BitNet量化感知训练中的梯度传播优化", convergence monitoring:
 * polarity balance).  W_packed and gamma are the same bits as
 * bitnet_weight_quant's; counts as bitnet_code_counts's (counts[3], the
 * unused pattern 11, is 0).
 *   W, W_packed, gamma: as bitnet_weight_quant
 *   counts    4 uint64, DEVICE memory, 8-byte aligned, written: zeroed by
 *            the call's first launch and summed into by its last with
 *            64-bit integer atomics (exact in any order)
 *   workspace >= bitnet_workspace_bytes(BITNET_OP_WEIGHT_QUANT_COUNTED, 0, N, K)
 *            device scratch: weight_quant's, then one (+1, -1) pair of
 *            uint32 per pack workgroup (a workgroup packs 4096 to 16384
 *            weights; sized for one pair per 4096), each written once by the
 *            call; contents on entry ignored.
 *            The zeros are the codes minus the nonzero ones: every code the
 *            call writes is 00, 01 or 10.
 * Errors: BITNET_E_ARG, BITNET_E_DTYPE, BITNET_E_SHAPE, BITNET_E_ALIGN,
 * BITNET_E_WORKSPACE, BITNET_E_HIP.
 */
int bitnet_weight_quant_counted(const void *W, int w_dtype, int64_t N, int64_t K,
                                uint8_t *W_packed, float *gamma, uint64_t *counts,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward of the unit-gain RMSNorm in front of the activation quantizer
 * ([NOTES 3.1] places it there; no page derives its backward, so this is the
 * exact derivative of the forward defined under bitnet_act_quant).  Per row,
 * with r = 1/sqrt(sum_k x_k^2 / K + eps) and n = x * r:
 *   grad_X[m][j] = r * (grad_n[m][j] - n_j * (sum_k grad_n[m][k] * n_k) / K)
 * computed in fp32 (a gradient; checked against a float64 reference).
 * grad_n is the gradient w.r.t. the RMSNorm output, i.e. grad_x of
 * bitnet_linear_bwd_ste; composing the two gives the BitLinear input
 * gradient of one QAT step.
 *   X       [M][K] fp32 or bf16 (x_dtype): the forward's RMSNorm input
 *   grad_n  [M][K] fp32 or bf16 (g_dtype)
 *   grad_X  [M][K] fp32 or bf16 (out_dtype, round to nearest even), written
 *   eps     the forward's eps (>= 0)
 * K % 8 == 0.  grad_X must not alias X or grad_n.
 * Errors: BITNET_E_ARG, BITNET_E_SHAPE, BITNET_E_DTYPE, BITNET_E_ALIGN,
 * BITNET_E_HIP.
 */
int bitnet_rmsnorm_bwd(const void *X, int x_dtype, const void *grad_n, int g_dtype,
                       int64_t M, int64_t K, float eps, void *grad_X, int out_dtype,
                       void *stream);

/*
 * Pack pre-quantized ternary codes ([WALL 4.1] code table).
 *   codes    [N][K] int8; a value > 0 packs as +1, < 0 as -1, 0 as 0
 *   W_packed [N][K/4] bytes, written
 * Errors: BITNET_E_ARG, BITNET_E_SHAPE (K % 4), BITNET_E_ALIGN, BITNET_E_HIP.
 */
int bitnet_pack_ternary(const int8_t *codes, int64_t N, int64_t K, uint8_t *W_packed,
                        void *stream);

/* Device scratch bytes `op` needs for these sizes (0 = none). */
size_t bitnet_workspace_bytes(int op, int64_t M, int64_t N, int64_t K);

/* Static, human-readable text for a status code. */
const char *bitnet_status_str(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int bitnet_version(void);

/*
 * For tests of the weight quantizer's fallback path.  With large matrices one
 * pack workgroup evaluates gamma and the code threshold and publishes the
 * threshold; every other workgroup reads it at most `reads` times (default
 * 32) and then evaluates it itself from the same row sums, which gives the
 * same bits.  Setting 0 makes every workgroup take that path in later calls
 * (bitnet_weight_quant, bitnet_weight_quant_counted, bitnet_quant_operands,
 * bitnet_weight_quant_noalloc); outputs are unchanged, only slower.  Host-side
 * setting for the whole process, read when a call launches its kernels; not
 * synchronised with concurrent calls.
 *   reads    0 .. 1024
 * Returns the previous value, or BITNET_E_ARG (nothing changed).
 */
int bitnet_set_gate_polls(int reads);

#ifdef __cplusplus
}
#endif

#endif /* BITNET_H_ */
