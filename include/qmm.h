/*
 * qmm.h -- C ABI of the block-quantized-weight matmul library for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation is the MatMulNBits operator as described on the
 * "onnx-runtime-ep-cpu matmul_nbits.rs" page (module documentation,
 * MatMulNBitsFactory::create and execute):
 *
 *   Y[m, n] = sum_k A[m, k] * w(n, k)  (+ bias[n])
 *   w(n, k) = (code(n, k) - zp(n, b)) * scale[n, b],   b = k / block_size
 *
 * with the weight codes packed least-significant bits first as
 * B[N, kb, block_size*bits/8] bytes, kb = ceil(K / block_size); scales
 * [N, kb]; optional packed zero points [N, ceil(kb*bits/8)] bytes (absent
 * zero points mean 2^(bits-1)).  The dequantized weight is never written to
 * memory: every kernel unpacks codes in registers.
 *
 * Conventions shared by every entry point:
 *  - Every array pointer is a DEVICE pointer owned by the caller.  The
 *    library keeps no pointer after a call returns and never allocates
 *    device memory during a call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued asynchronously on it; nothing synchronizes.
 *  - Arguments are validated on the host before anything is enqueued.  A
 *    negative qmm_status is returned on error and qmm_last_error() gives a
 *    thread-local "what / why / how to fix" message.  A failed launch returns
 *    QMM_ERR_HIP.
 *  - Arrays are dense and row-major with the shapes given below.
 *  - dtypes: A, bias and Y share one float dtype (qmm_dtype); scales may
 *    have any float dtype.  Float results accumulate in fp32.
 */
#ifndef QMM_H_
#define QMM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qmm_dtype {
    QMM_F32 = 0,
    QMM_F16 = 1,
    QMM_BF16 = 2
} qmm_dtype;

typedef enum qmm_layout {
    /* The operator's own layout: B[N, kb, block_size*bits/8], with separate
     * scales and (optional) zero-point tensors. */
    QMM_LAYOUT_ORT = 0,
    /* The tiled layout written by qmm_repack (see there), without / with zero
     * points.  B then points to the whole repacked buffer, which carries the
     * scales and zero points: the scales and zero_points arguments must be
     * NULL and s_dtype names the dtype the scales were repacked from. */
    QMM_LAYOUT_TILED = 1,
    QMM_LAYOUT_TILED_ZP = 2
} qmm_layout;

typedef enum qmm_status {
    QMM_OK = 0,
    QMM_ERR_INVALID_ARG = -1,  /* a shape, dtype, pointer or attribute is wrong */
    QMM_ERR_UNSUPPORTED = -2,  /* valid for the operator, not implemented here  */
    QMM_ERR_WORKSPACE = -3,    /* workspace missing or too small                */
    QMM_ERR_HIP = -4           /* the HIP runtime reported an error             */
} qmm_status;

/* Message of the last failed call on this host thread ("" if none). */
const char *qmm_last_error(void);

/*
 * M = 1 decode GEMV (matmul_nbits.rs: execute, the m == 1 routes).
 *   A      [K]            a_dtype
 *   B      [N, kb, blob]  uint8, 16-byte aligned, layout QMM_LAYOUT_ORT (or the
 *          buffer written by qmm_repack, layout QMM_LAYOUT_TILED[_ZP])
 *   scales [N, kb]        s_dtype
 *   zero_points [N, ceil(kb*bits/8)] uint8 or NULL
 *   g_idx  [g_idx_len]    int32 group indices or NULL (then g_idx_len = 0)
 *   bias   [N]            a_dtype or NULL
 *   Y      [N]            a_dtype (written)
 * bits in {2, 3, 4, 8}; block_size a power of two >= 16 (MatMulNBitsFactory::
 * create).  accuracy_level 0..3 select float compute; the hint can only raise
 * precision and every level computes fp32-accumulated products here.
 * 3-bit weights (MNN ConvInt8TiledExecutor.cpp: the 3-bit reorder splits
 * each code 0..7 into a 2-bit and a 1-bit plane, offset -4): a block's blob
 * of 3 * block_size / 8 bytes is block_size / 4 bytes of the codes' low two
 * bits (code i at bits 2 (i % 4) of byte i / 4) then block_size / 8 bytes of
 * their high bits (code i at bit i % 8 of byte block_size / 4 + i / 8);
 * zero points are one LSB-first 3-bit stream per row of ceil(kb * 3 / 8)
 * bytes (a value may cross a byte), default 4.  3-bit weights take the
 * operator's layout only, block_size <= 8192, and no group indices.
 * accuracy_level 4 (int8 activations) is rejected: use qmm_gemm_compint8.
 *
 * Group indices (act-order; matmul_nbits.rs execute and the group-index
 * branch of dequantize_weight): element k keeps its code from block k / bs
 * but takes the scale and zero point of group g_idx[k]:
 *   w(n, k) = (code(n, k) - zp(n, g_idx[k])) * scale[n, g_idx[k]].
 * g_idx is a device array of g_idx_len = K or kb * block_size int32 values
 * (the first K are read), operator layout only (QMM_ERR_UNSUPPORTED on a
 * tiled B).  Every entry must lie in 0..kb-1: check a host copy once with
 * qmm_check_g_idx.  The kernels clamp an out-of-range entry into that range
 * (it reads in bounds and gives a wrong result, never a fault).
 */
int qmm_gemv(const void *A, int a_dtype, const uint8_t *B, int b_layout,
             const void *scales, int s_dtype, const uint8_t *zero_points,
             const int32_t *g_idx, int64_t g_idx_len, const void *bias,
             void *Y, int64_t K, int64_t N, int block_size, int bits,
             int accuracy_level, void *stream);

/*
 * Range and shape check of group indices held in HOST memory (matmul_nbits.rs
 * execute: shape [K] or [kb * block_size]; dequantize_weight: every entry in
 * 0..kb).  QMM_OK, or QMM_ERR_INVALID_ARG naming the first bad entry.
 */
int qmm_check_g_idx(const int32_t *g_idx, int64_t g_idx_len, int64_t K,
                    int block_size);

/*
 * Batched / prefill matmul, A [M, K] -> Y [M, N]; the other arguments as for
 * qmm_gemv.  M = 0 is a no-op.  bf16 and f16 activations run on the matrix
 * cores with weights dequantized tile by tile to the activation dtype; f32
 * activations are computed in fp32.
 */
int qmm_gemm(const void *A, int a_dtype, const uint8_t *B, int b_layout,
             const void *scales, int s_dtype, const uint8_t *zero_points,
             const int32_t *g_idx, int64_t g_idx_len, const void *bias, void *Y,
             int64_t M, int64_t K, int64_t N, int block_size, int bits,
             int accuracy_level, void *stream);

/*
 * CompInt8 (accuracy_level 4; matmul_nbits.rs: quantize_activation_signed,
 * int4_dot_row_scalar, int8_row).  Each row of A is quantized per K-block of
 * block_size elements to int8 with scale sa = max|x| / 127 (IEEE binary32
 * division, round half to even, clamp to [-127, 127]; a block with sa == 0
 * quantizes to 0).  Then
 *   dot[m, n, b] = sum_{k in b, k < K} qa[m, k] * (code(n, k) - zp(n, b))
 * exactly in int32 and Y[m, n] = sum_b float(dot) * (sa[m, b] * scale[n, b])
 * (+ bias[n]) in fp32.
 * workspace: device memory of at least qmm_compint8_workspace_size(M, K,
 * block_size) bytes, 256-byte aligned, owned by the caller, overwritten (it
 * holds qa and sa between the two launches of the computation; for M = 1 on
 * the tiled layout the quantization runs inside the one launch and the
 * workspace is checked but not written).
 * accuracy_level must be 4.  Arguments otherwise as for qmm_gemm.  B may be
 * the tiled buffer of qmm_repack when block_size >= 32 (the block dots then
 * run on the int8 matrix cores), and for M = 1 also when block_size is at
 * least one 16-byte unit of codes (32, 64 or 16 codes for 4, 2 or 8 bits)
 * and at most 1024; otherwise QMM_ERR_UNSUPPORTED.
 * With group indices (g_idx, as for qmm_gemv) the weight scale changes
 * inside an activation block, so no per-block integer dot exists; as the
 * operator does, the product is then computed with float activations (the
 * result of qmm_gemm) and the workspace is not used.
 */
size_t qmm_compint8_workspace_size(int64_t M, int64_t K, int block_size);

int qmm_gemm_compint8(const void *A, int a_dtype, const uint8_t *B,
                      int b_layout, const void *scales, int s_dtype,
                      const uint8_t *zero_points, const int32_t *g_idx,
                      int64_t g_idx_len, const void *bias, void *Y, int64_t M,
                      int64_t K, int64_t N, int block_size, int bits,
                      int accuracy_level, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * qmm_gemm_compint8 for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops that forbid hipMalloc): the same
 * computation, kernels and results, with the workspace taken from a device
 * array the library holds (one per device, QMM_NOALLOC_SCRATCH_BYTES, kept
 * from library load until the process ends) instead of caller memory.  No
 * call allocates or frees anything.  Arguments as for qmm_gemm_compint8
 * without the workspace.  Errors: QMM_ERR_WORKSPACE when
 * qmm_compint8_workspace_size(M, K, block_size) exceeds
 * QMM_NOALLOC_SCRATCH_BYTES (split A into row batches); QMM_ERR_HIP if the
 * array's device address cannot be found.  The array is found on the device
 * current at the call, which must be the stream's device.  All calls on one
 * device share it: calls that overlap on one device (on different streams,
 * or from threads without ordering) race and give wrong results.
 */
#define QMM_NOALLOC_SCRATCH_BYTES (4 * 1024 * 1024)

int qmm_gemm_compint8_noalloc(const void *A, int a_dtype, const uint8_t *B,
                              int b_layout, const void *scales, int s_dtype,
                              const uint8_t *zero_points, const int32_t *g_idx,
                              int64_t g_idx_len, const void *bias, void *Y,
                              int64_t M, int64_t K, int64_t N, int block_size,
                              int bits, int accuracy_level, void *stream);

/*
 * int16 activations (matmul_nbits.rs execute, the 8-bit route: the
 * activation is quantized to int16 per K-block and reduced against the codes
 * with an integer dot; that page keeps int16 because it matches the fp32
 * result).  Per row m and block b: sa = max|x| / 32767 (IEEE binary32
 * division), qa = clamp(round_half_even(x / sa), -32767, 32767) (0 past K and
 * for sa == 0); dot = sum qa * (code - zp) exactly in int32 and Y[m, n] =
 * sum_b float(dot) * (sa[m, b] * scale[n, b]) (+ bias[n]) in fp32.  Any code
 * width (2, 3, 4, 8), the operator's layout, block_size <= 128 (the int32
 * dot is exact); otherwise QMM_ERR_UNSUPPORTED.  workspace: at least
 * qmm_int16_workspace_size(M, K, block_size) bytes, 256-byte aligned; on
 * return it holds qa [M, kb * block_size] int16 at offset 0 and sa [M, kb]
 * float32 at the next 256-byte boundary.  Arguments otherwise as qmm_gemm.
 * qmm_debug_int16_block_dots writes the int32 block dots [M, N, kb] (same
 * workspace contract; scales are not read).
 */
size_t qmm_int16_workspace_size(int64_t M, int64_t K, int block_size);

int qmm_gemm_int16(const void *A, int a_dtype, const uint8_t *B, int b_layout,
                   const void *scales, int s_dtype, const uint8_t *zero_points,
                   const void *bias, void *Y, int64_t M, int64_t K, int64_t N,
                   int block_size, int bits, void *workspace,
                   size_t workspace_bytes, void *stream);

int qmm_debug_int16_block_dots(const void *A, int a_dtype, const uint8_t *B,
                               const uint8_t *zero_points, int64_t M, int64_t K,
                               int64_t N, int block_size, int bits,
                               int32_t *dots, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * Matmul with block-scaled FP4 weights (rlx-cpu quant.rs: dequant_matmul_nvfp4,
 * lowp_dequantize):
 *   w(n, k) = e2m1(code(n, k)) * scale(n, k / bs) * global_scale
 *   Y[m, n] = sum_k A[m, k] * w(n, k)  (+ bias[n]),  fp32 accumulate
 * QMM_MXFP4: bs = 32, scales are E8M0 bytes (2^(e-127); 255 is nan).
 * QMM_NVFP4: bs = 16, scales are FP8 E4M3 bytes (bias 7; S.1111.111 is nan).
 * E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa bit) codes 0..15 are
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives.
 *   A      [M, K]          a_dtype (f32, f16, bf16)
 *   W      [N, kb, bs/2]   uint8, kb = ceil(K / bs), 16-byte aligned: element
 *                          k of row n in byte k/2 of the row, low nibble for
 *                          even k (rows are K-last; the page's dequantizer
 *                          flattens a [K, N] index the same way)
 *   scales [N, kb]         uint8 scale bytes
 *   global_scale           multiplies every weight (NVFP4's per-tensor f32
 *                          scale; MXFP4 weights pass 1)
 *   bias [N], Y [M, N]     a_dtype (bias may be NULL)
 * M = 1 runs a GEMV; 16-bit activations with M > 16 the matrix cores (each
 * weight is exact in bf16 / f16); the rest an fp32 kernel.  M = 0 is a no-op.
 */
typedef enum qmm_fp4_format { QMM_MXFP4 = 0, QMM_NVFP4 = 1 } qmm_fp4_format;

int qmm_gemm_fp4(const void *A, int a_dtype, const uint8_t *W,
                 const uint8_t *scales, int format, float global_scale,
                 const void *bias, void *Y, int64_t M, int64_t K, int64_t N,
                 void *stream);

/*
 * Low-precision scaled GEMM (rlx-cpu quant.rs: the FP8 / FP6 / FP4
 * scaled-GEMM reference lowp_scaled_matmul and lowp_read_scales), TN:
 *   out[i, j] = sum_p a(i, p) * b(j, p)  (+ bias[j]),  fp32 accumulate
 *   a(i, p) = decode(lhs[i, p]) * lhs_scale(i, p)
 *   b(j, p) = decode(rhs[j, p]) * rhs_scale(j, p)
 *   lhs [m, k], rhs [n, k]   uint8, one code per byte in its low bits
 *                            (rows K-last)
 *   lhs_scales, rhs_scales   by layout:
 *     QMM_LOWP_PER_TENSOR    one f32 each (device memory)
 *     QMM_LOWP_MX            [m, ceil(k/32)] / [n, ceil(k/32)] E8M0 bytes
 *                            (2^(e-127); 255 is nan)
 *     QMM_LOWP_NVFP4         [m, ceil(k/16)] / [n, ceil(k/16)] E4M3 bytes
 *   bias [n] f32 (may be NULL), out [m, n] f32
 * Element formats (OCP FP8 and Microscaling definitions; exponent 0 is
 * subnormal): E4M3 (bias 7, S.1111.111 nan, max 448), E5M2 (bias 15, IEEE
 * inf / nan, max 57344), E2M3 (FP6, bias 1, max 7.5), E3M2 (FP6, bias 3,
 * max 28), E2M1 (FP4, bias 1, max 6).  The two operands may differ in
 * format.  Per tensor and MX run on gfx950's block-scaled matrix-core
 * instruction; NVFP4 decodes to bf16 (exact) for the bf16 one.  Errors:
 * QMM_ERR_INVALID_ARG for an unknown format or layout, null pointers or
 * non-positive n or k; QMM_ERR_UNSUPPORTED when m * k or n * k reaches 2^31.
 * m = 0 is a no-op.
 */
typedef enum qmm_lowp_format {
  QMM_LOWP_E4M3 = 0, QMM_LOWP_E5M2 = 1, QMM_LOWP_E2M3 = 2, QMM_LOWP_E3M2 = 3, QMM_LOWP_E2M1 = 4
} qmm_lowp_format;
typedef enum qmm_lowp_layout {
  QMM_LOWP_PER_TENSOR = 0, QMM_LOWP_MX = 1, QMM_LOWP_NVFP4 = 2
} qmm_lowp_layout;

int qmm_lowp_matmul(const uint8_t *lhs, const uint8_t *rhs, const void *lhs_scales,
                    const void *rhs_scales, const float *bias, float *out, int64_t m,
                    int64_t n, int64_t k, int layout, int lhs_format, int rhs_format,
                    void *stream);

/*
 * The operand producer of qmm_lowp_matmul (rlx-cpu quant.rs:
 * lowp_compute_scales with lowp_snap_scale and the stored forms of
 * ScaledQuantScale, then lowp_quantize), for x [rows, cols] in x_dtype
 * (f32, f16, bf16; 16-bit values are taken exactly as binary32):
 *   scale  per tensor: amax(|x|) / max_finite(format) (1 if amax is 0),
 *          written as one f32; MX / NVFP4: the same per block of 32 / 16
 *          along cols, snapped (E8M0: the binary32 exponent field; NVFP4:
 *          the nearest E4M3) and written as [rows, ceil(cols / bs)] bytes
 *   codes  [rows, cols] uint8: encode(x / scale) with the binary32 quotient
 *          (0 where the scale is 0): the nearest finite value of the format,
 *          ties to the even mantissa, saturating past the largest finite
 *          value, nan to the format's nan (E4M3 / E5M2 0x7F) or 0
 * Maxima skip nan.  Per tensor runs four kernels on `stream` (the scale
 * slot holds amax in between).  Errors: QMM_ERR_INVALID_ARG for an unknown
 * format, layout or dtype, null pointers or non-positive cols;
 * QMM_ERR_UNSUPPORTED when rows * cols reaches 2^31.  rows = 0 is a no-op.
 */
int qmm_lowp_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int format,
                      int layout, uint8_t *codes, void *scales, void *stream);

/*
 * A step: a fixed sequence of matmul calls (say the projections of one
 * decode step) recorded once and replayed as one HIP graph.  The pages find
 * the decode step's cost outside the kernels -- per-operator dispatch and
 * fork/join made decode 2.3x slower, and a persistent pool took it from 6 to
 * 28 tok/s (matmul_nbits.rs, module notes on the decode step and the
 * persistent decode pool); here that cost is the host's validation and
 * enqueue per call, which a small projection's kernel does not cover.
 *   qmm_step_create        a new, empty step (host object; never NULL on QMM_OK)
 *   qmm_step_add_gemv / _gemm / _gemm_compint8
 *                          record one call with the arguments of qmm_gemv /
 *                          qmm_gemm / qmm_gemm_compint8 (no stream); nothing
 *                          is validated or enqueued yet
 *   qmm_step_finalize      validate every recorded call and capture their
 *                          launches into a graph on the current device (an
 *                          internal stream; error: the first failing call's
 *                          status, its position in the message)
 *   qmm_step_launch        enqueue the whole sequence on `stream` with one
 *                          graph launch (the device current at finalize)
 *   qmm_step_size          number of recorded calls
 *   qmm_step_destroy       free the step and its graph (NULL is a no-op)
 * A replay runs exactly the direct calls' kernels with the same arguments:
 * every pointer recorded must stay valid until the step is destroyed, and
 * inputs are changed in place between launches.  The recorded calls enqueue
 * no memory-set operations.  A step is not thread-safe; launches of one step
 * on different streams may overlap and then race on its outputs.
 */
typedef struct qmm_step qmm_step;

int qmm_step_create(qmm_step **step);

int qmm_step_add_gemv(qmm_step *step, const void *A, int a_dtype,
                      const uint8_t *B, int b_layout, const void *scales,
                      int s_dtype, const uint8_t *zero_points,
                      const int32_t *g_idx, int64_t g_idx_len,
                      const void *bias, void *Y, int64_t K, int64_t N,
                      int block_size, int bits, int accuracy_level);

int qmm_step_add_gemm(qmm_step *step, const void *A, int a_dtype,
                      const uint8_t *B, int b_layout, const void *scales,
                      int s_dtype, const uint8_t *zero_points,
                      const int32_t *g_idx, int64_t g_idx_len,
                      const void *bias, void *Y, int64_t M, int64_t K,
                      int64_t N, int block_size, int bits, int accuracy_level);

int qmm_step_add_gemm_compint8(qmm_step *step, const void *A, int a_dtype,
                               const uint8_t *B, int b_layout,
                               const void *scales, int s_dtype,
                               const uint8_t *zero_points,
                               const int32_t *g_idx, int64_t g_idx_len,
                               const void *bias, void *Y, int64_t M,
                               int64_t K, int64_t N, int block_size,
                               int bits, int accuracy_level, void *workspace,
                               size_t workspace_bytes);

int qmm_step_finalize(qmm_step *step);

int qmm_step_launch(const qmm_step *step, void *stream);

int qmm_step_size(const qmm_step *step);

void qmm_step_destroy(qmm_step *step);

/*
 * int8 convolution with requantization (MNN ConvInt8TiledExecutor.cpp:
 * initializeConvInt8QuantInfo, im2col padding with the input zero point,
 * QuanPostTreatParameters clamp; rlx-cpu quant.rs: exec_q_mat_mul).
 *   X  [Nb, H, W, C]        int8 NHWC
 *   Wt [Co, KH, KW, C]      int8 OHWI, symmetric (weight zero point 0)
 *   bias [Co] int32 or NULL; w_scale [Co] float32
 *   Y  [Nb, OH, OW, Co]     int8 NHWC, OH = (H + 2 pad_h - KH) / stride_h + 1
 * acc = bias + sum (x - in_zp) * w, a tap outside the image reading in_zp;
 * mult = (in_scale * w_scale[oc]) / out_scale in binary32;
 * y = clamp(round_half_even(float(acc) * mult) + out_zp, clamp_min, clamp_max).
 * A ReLU is expressed as clamp_min = out_zp.  Groups and dilation are 1.
 * Any C (C % 16 == 0 with 16-byte aligned X and Wt takes 16-byte loads,
 * C % 4 == 0 with 4-byte alignment 4-byte loads, the rest byte gathers).
 * Requires KH*KW*C*2^14 < 2^31 (exact int32 partial sums); the accumulator
 * with the bias is formed in 64 bits and float(acc) is the round-to-nearest
 * conversion.
 */
int qconv_int8(const int8_t *X, const int8_t *Wt, const int32_t *bias,
               const float *w_scale, float in_scale, float out_scale,
               int in_zp, int out_zp, int clamp_min, int clamp_max, int Nb,
               int H, int W, int C, int Co, int KH, int KW, int stride_h,
               int stride_w, int pad_h, int pad_w, int8_t *Y, void *stream);

/*
 * One-time repack of constant weights into the tiled layout (a byte
 * permutation; onnx-runtime-ep-cpu matmul_nbits.rs caches its prepacked
 * weights once per constant input, and the AMX path repacks B into tile
 * order the same way).  Output columns form groups of 32 and K is cut into
 * chunks of 64 codes; the buffer holds three regions, each 256-byte aligned:
 *   codes  [group][chunk][32 columns][64*bits/8 bytes]  (each column chunk
 *          is that column's bytes of B for codes [64c, 64c + 64), zero past
 *          its row)
 *   scales [group][block][32 columns]                  (s_dtype)
 *   zps    [group][block][32 columns], bits per entry packed LSB first
 *          (only when zero_points is non-NULL)
 * Columns past N hold zeros.  qmm_repacked_bytes gives the buffer size.
 * qmm_unrepack restores B and the scales exactly, and the zero points (the
 * unused bits of each zero-point row's last byte are written as zero).
 * Arguments as for qmm_gemv; out / tiled are device buffers of at least
 * qmm_repacked_bytes bytes, 256-byte aligned.
 * The tiled buffer holds no header: every call that takes it locates its
 * regions from K, N, block_size, bits, s_dtype and the layout (with or
 * without zero points).  The caller must pass exactly the values it was
 * repacked with; other values read the wrong bytes (within the buffer's
 * extent only if it is at least qmm_repacked_bytes of those values).  The
 * Python binding records the geometry and rejects a mismatch.
 */
size_t qmm_repacked_bytes(int64_t K, int64_t N, int block_size, int bits, int s_dtype,
                          int has_zero_points);

int qmm_repack(const uint8_t *B, const void *scales, int s_dtype, const uint8_t *zero_points,
               int64_t K, int64_t N, int block_size, int bits, void *out, size_t out_bytes,
               void *stream);

int qmm_unrepack(const void *tiled, int has_zero_points, int64_t K, int64_t N, int block_size,
                 int bits, int s_dtype, uint8_t *B, void *scales, uint8_t *zero_points,
                 void *stream);

/*
 * Test exports: the integer intermediates, for bit-exact comparison.
 *  qmm_debug_unpack: codes [N, K] uint8, zps [N, kb] uint8 (defaults filled
 *    in), w [N, K] float32 = (code - zp) * scale; any output may be NULL.
 *  qmm_debug_quantize_a: qa [M, kb*block_size] int8 (zero past K), sa [M, kb]
 *    float32, exactly as the quantization launch of qmm_gemm_compint8's
 *    two-launch route.
 *  qmm_debug_compint8_block_dots: dots [M, N, kb] int32 computed by the
 *    kernels of the route qmm_gemm_compint8 takes for the same arguments
 *    (same workspace contract).  On return the workspace holds that route's
 *    quantized activations: qa [M, kb*block_size] int8 at offset 0 and sa
 *    [M, kb] float32 at the next 256-byte boundary -- for M = 1 on the tiled
 *    layout, the ones the one-launch kernel computed in LDS.  s_dtype
 *    matters only for a tiled B (it locates the zero-point region).
 */
int qmm_debug_unpack(const uint8_t *B, int b_layout, const void *scales,
                     int s_dtype, const uint8_t *zero_points, int64_t K,
                     int64_t N, int block_size, int bits, uint8_t *codes,
                     uint8_t *zps, float *w, void *stream);

int qmm_debug_quantize_a(const void *A, int a_dtype, int64_t M, int64_t K,
                         int block_size, int8_t *qa, float *sa, void *stream);

int qmm_debug_compint8_block_dots(const void *A, int a_dtype, const uint8_t *B,
                                  int b_layout, int s_dtype,
                                  const uint8_t *zero_points,
                                  int64_t M, int64_t K, int64_t N,
                                  int block_size, int bits, int32_t *dots,
                                  void *workspace, size_t workspace_bytes,
                                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H_ */
