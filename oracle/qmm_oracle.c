/*
 * qmm_oracle.c -- plain, slow CPU oracle for block-quantized-weight matmuls.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header or table with the HIP
 * library: every definition below is written out again from the sources it
 * cites.
 *
 * Sources (web pages, cited by title and section):
 *   [ORT]  onnx-runtime-ep-cpu 0.1.0-dev.5, src/kernels/matmul_nbits.rs
 *          (MatMulNBits: module documentation, dequantize_nbits_value,
 *           dequantize_weight and its group-index branch, execute's g_idx
 *           shape check, prepack_int8_weight, quantize_activation_signed,
 *           int4_dot_row_scalar, int8_row, execute's bias step)
 *   [RLX]  rlx-cpu 0.2.13, src/thunk/ops/quant.rs
 *          (exec_q_mat_mul requantize step, compile_q_conv2d attributes)
 *   [MNN]  MNN ConvInt8TiledExecutor.cpp
 *          (initializeConvInt8QuantInfo defaults, im2col padding with the
 *           input zero point, QuanPostTreatParameters clamp)
 *
 * Precision: float results are accumulated in double; integer results are
 * exact (int32/int64).  Where a floating-point step decides an integer (the
 * activation quantization of CompInt8, the conv requantization), the step is
 * done in IEEE binary32 exactly as written, because the device does the same
 * decision in binary32.  Build with -O2 -fno-fast-math (no contraction).
 *
 * Loops run in natural index order.  OpenMP only splits the outer output
 * loop; each output element is computed by one thread in a fixed order, so
 * results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* O1 codec                                                                  */
/* ------------------------------------------------------------------------ */

/* Number of K blocks: ceil(K / block_size)  ([ORT] module documentation). */
static int64_t n_blocks(int64_t K, int64_t bs) { return (K + bs - 1) / bs; }

/* Bytes per block of packed codes: block_size * bits / 8  ([ORT] execute). */
static int64_t blob_bytes(int64_t bs, int bits) { return bs * bits / 8; }

/* Bytes per row of packed zero points: ceil(k_blocks * bits / 8). */
static int64_t zp_row_bytes(int64_t kb, int bits) { return (kb * bits + 7) / 8; }

/* Code of element k of output row n ([ORT] dequantize_nbits_value): inside
 * block k / bs the element sits at bit offset (k % bs) * bits, counted from
 * the least-significant bit of the block's first byte.
 * 3-bit codes ([MNN] weight reorder for 3 bits: the code 0..7 is split into
 * a 2-bit main plane and a 1-bit aux plane, laid out [main | aux]; offset
 * -4): a block's blob is bs/4 bytes of the low two bits of each code (four
 * per byte, LSB first) followed by bs/8 bytes of the high bits (eight per
 * byte, LSB first); the bit order is the operator's LSB-first one. */
static unsigned code_at(const uint8_t *B, int64_t n, int64_t k, int64_t K,
                        int64_t bs, int bits) {
    int64_t kb = n_blocks(K, bs);
    int64_t blob = blob_bytes(bs, bits);
    const uint8_t *row = B + n * kb * blob;
    int64_t block = k / bs;
    if (bits == 3) {
        const uint8_t *base = row + block * blob;
        int64_t i = k % bs;
        unsigned lo = (base[i / 4] >> (2 * (i % 4))) & 3u;
        unsigned hi = (base[bs / 4 + i / 8] >> (i % 8)) & 1u;
        return lo | (hi << 2);
    }
    int64_t bit = (k % bs) * bits;
    unsigned byte = row[block * blob + bit / 8];
    unsigned mask = (1u << bits) - 1u;
    return (byte >> (bit % 8)) & mask;
}

/* Zero point of block b of row n; the zero-point row packs one bits-wide
 * value per block, LSB first; absent zero points mean 2^(bits-1)
 * ([ORT] dequantize_nbits_value, default_zero_point). */
static unsigned zp_at(const uint8_t *zp, int64_t n, int64_t b, int64_t kb,
                      int bits) {
    if (zp == NULL) return 1u << (bits - 1);
    const uint8_t *row = zp + n * zp_row_bytes(kb, bits);
    int64_t bit = b * bits;
    unsigned mask = (1u << bits) - 1u;
    unsigned v = row[bit / 8] >> (bit % 8);
    /* 3 bits: a value may continue into the next byte (LSB-first stream). */
    if (bit % 8 + bits > 8) v |= (unsigned)row[bit / 8 + 1] << (8 - bit % 8);
    return v & mask;
}

/* codes[n*K + k] for every n < N, k < K. */
EXPORT void oracle_unpack_codes(const uint8_t *B, int64_t N, int64_t K,
                                int64_t bs, int bits, uint8_t *codes) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            codes[n * K + k] = (uint8_t)code_at(B, n, k, K, bs, bits);
}

/* zps[n*kb + b]; zp may be NULL (default value). */
EXPORT void oracle_unpack_zero_points(const uint8_t *zp, int64_t N, int64_t kb,
                                      int bits, uint8_t *zps) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < kb; ++b)
            zps[n * kb + b] = (uint8_t)zp_at(zp, n, b, kb, bits);
}

/* Inverse of oracle_unpack_codes: write codes[n*K + k] into the packed
 * [N, kb, blob] layout.  Bits past K in the last block are left zero. */
EXPORT void oracle_pack_codes(const uint8_t *codes, int64_t N, int64_t K,
                              int64_t bs, int bits, uint8_t *B) {
    int64_t kb = n_blocks(K, bs);
    int64_t blob = blob_bytes(bs, bits);
    memset(B, 0, (size_t)(N * kb * blob));
    unsigned mask = (1u << bits) - 1u;
    for (int64_t n = 0; n < N; ++n) {
        uint8_t *row = B + n * kb * blob;
        for (int64_t k = 0; k < K; ++k) {
            if (bits == 3) {
                uint8_t *base = row + (k / bs) * blob;
                int64_t i = k % bs;
                unsigned c = codes[n * K + k] & mask;
                base[i / 4] |= (uint8_t)((c & 3u) << (2 * (i % 4)));
                base[bs / 4 + i / 8] |= (uint8_t)((c >> 2) << (i % 8));
                continue;
            }
            int64_t bit = (k % bs) * bits;
            row[(k / bs) * blob + bit / 8] |=
                (uint8_t)((codes[n * K + k] & mask) << (bit % 8));
        }
    }
}

/* Inverse of oracle_unpack_zero_points. */
EXPORT void oracle_pack_zero_points(const uint8_t *zps, int64_t N, int64_t kb,
                                    int bits, uint8_t *zp) {
    int64_t rb = zp_row_bytes(kb, bits);
    memset(zp, 0, (size_t)(N * rb));
    unsigned mask = (1u << bits) - 1u;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < kb; ++b) {
            int64_t bit = b * bits;
            unsigned v = (zps[n * kb + b] & mask) << (bit % 8);
            zp[n * rb + bit / 8] |= (uint8_t)(v & 0xFFu);
            if (v >> 8) zp[n * rb + bit / 8 + 1] |= (uint8_t)(v >> 8);
        }
}

/* Group whose scale and zero point apply to element k: its block k / bs,
 * or g_idx[k] when group indices are given ([ORT] dequantize_weight: the
 * code is still read from block k / bs; only the scale and zero point are
 * taken from group g_idx[k]).  The caller has range-checked g_idx. */
static int64_t group_of(const int32_t *g_idx, int64_t k, int64_t bs) {
    return g_idx ? (int64_t)g_idx[k] : k / bs;
}

/* Range check of group indices ([ORT] execute: g_idx has shape [K] or
 * [kb * bs]; dequantize_weight: every entry lies in 0..kb).  Returns -1 if
 * the shape is wrong, the position of the first out-of-range entry, or
 * len (no error). */
EXPORT int64_t oracle_check_g_idx(const int32_t *g_idx, int64_t len, int64_t K,
                                  int64_t bs) {
    int64_t kb = n_blocks(K, bs);
    if (len != K && len != kb * bs) return -1;
    for (int64_t i = 0; i < len; ++i)
        if (g_idx[i] < 0 || (int64_t)g_idx[i] >= kb) return i;
    return len;
}

/* Dequantized weight w[n*K + k] = (code - zp(g)) * scale[n*kb + g] with g the
 * group of k (block k / bs, or g_idx[k]), in double ([ORT]
 * dequantize_nbits_value, dequantize_weight; scales are given already
 * widened; g_idx may be NULL). */
EXPORT void oracle_dequantize(const uint8_t *B, const double *scales,
                              const uint8_t *zp, const int32_t *g_idx,
                              int64_t N, int64_t K, int64_t bs, int bits,
                              double *W) {
    int64_t kb = n_blocks(K, bs);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int64_t g = group_of(g_idx, k, bs);
            double q = (double)code_at(B, n, k, K, bs, bits);
            double z = (double)zp_at(zp, n, g, kb, bits);
            W[n * K + k] = (q - z) * scales[n * kb + g];
        }
}

/* ------------------------------------------------------------------------ */
/* O2 float matmul: Y[m, n] = sum_k A[m, k] * w(n, k)  (+ bias[n])            */
/* ([ORT] module documentation, execute: dequantize then GEMV/GEMM, bias      */
/*  added after the product; with group indices the scale and zero point of  */
/*  element k are those of group g_idx[k], [ORT] dequantize_weight)           */
/* S[m, n] = sum_k |A[m, k] * w(n, k)| + |bias[n]| is the tolerance base.     */
/* g_idx may be NULL; otherwise it has been range-checked.                    */
/* ------------------------------------------------------------------------ */
EXPORT void oracle_matmul_nbits(const double *A, const uint8_t *B,
                                const double *scales, const uint8_t *zp,
                                const int32_t *g_idx, const double *bias,
                                int64_t M, int64_t N, int64_t K, int64_t bs,
                                int bits, double *Y, double *S) {
    int64_t kb = n_blocks(K, bs);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t g = group_of(g_idx, k, bs);
                double q = (double)code_at(B, n, k, K, bs, bits);
                double z = (double)zp_at(zp, n, g, kb, bits);
                double w = (q - z) * scales[n * kb + g];
                double t = A[m * K + k] * w;
                acc += t;
                mag += fabs(t);
            }
            if (bias) {
                acc += bias[n];
                mag += fabs(bias[n]);
            }
            Y[m * N + n] = acc;
            if (S) S[m * N + n] = mag;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* O3 CompInt8 activation quantization ([ORT] quantize_activation_signed:    */
/* per K-block of block_size elements, scale = max|x| / 127, codes rounded    */
/* to nearest; the padded tail past K stays 0).                               */
/* Readings: the block width is the weight block_size; the division is the    */
/* IEEE binary32 quotient x / scale; ties round to even; codes are clamped to */
/* [-127, 127]; a block whose scale is 0 gets all-zero codes.                 */
/* qa is [M, kb*bs] int8, sa is [M, kb] float.                                */
/* ------------------------------------------------------------------------ */
EXPORT void oracle_quantize_a(const float *A, int64_t M, int64_t K, int64_t bs,
                              int8_t *qa, float *sa) {
    int64_t kb = n_blocks(K, bs);
    int64_t padded = kb * bs;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t b = 0; b < kb; ++b) {
            int64_t k0 = b * bs;
            int64_t k1 = k0 + bs < K ? k0 + bs : K;
            float amax = 0.0f;
            for (int64_t k = k0; k < k1; ++k) {
                float a = fabsf(A[m * K + k]);
                if (a > amax) amax = a;
            }
            float scale = amax / 127.0f;
            sa[m * kb + b] = scale;
            for (int64_t k = k0; k < k0 + bs; ++k) {
                int8_t v = 0;
                if (k < K && scale != 0.0f) {
                    float r = rintf(A[m * K + k] / scale);
                    if (r > 127.0f) r = 127.0f;
                    if (r < -127.0f) r = -127.0f;
                    v = (int8_t)r;
                }
                qa[m * padded + k] = v;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* int16 activations ([ORT] execute, the 8-bit route: the activation is        */
/* quantized to int16 per K-block and reduced against the u8 weight with an   */
/* integer dot; the quantizer's body is not on the page).  Reading: the int8   */
/* quantizer with 32767: sa = max|x| / 32767 (binary32), qa = clamp(rne(x /   */
/* sa), -32767, 32767), 0 past K and for an all-zero block.                    */
/* ------------------------------------------------------------------------ */
EXPORT void oracle_quantize_a16(const float *A, int64_t M, int64_t K,
                                int64_t bs, int16_t *qa, float *sa) {
    int64_t kb = n_blocks(K, bs);
    int64_t padded = kb * bs;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t b = 0; b < kb; ++b) {
            int64_t k0 = b * bs, k1 = k0 + bs < K ? k0 + bs : K;
            float amax = 0.0f;
            for (int64_t k = k0; k < k1; ++k) {
                float a = fabsf(A[m * K + k]);
                if (a > amax) amax = a;
            }
            float scale = amax / 32767.0f;
            sa[m * kb + b] = scale;
            for (int64_t k = k0; k < k0 + bs; ++k) {
                int16_t v = 0;
                if (k < K && scale != 0.0f) {
                    float r = rintf(A[m * K + k] / scale);
                    if (r > 32767.0f) r = 32767.0f;
                    if (r < -32767.0f) r = -32767.0f;
                    v = (int16_t)r;
                }
                qa[m * padded + k] = v;
            }
        }
}

/* Y[m, n] = sum_b dot * sa[m, b] * s[n, b] (+ bias), dot = sum over block b */
/* of qa16 * (code - zp), exact in int64; double accumulation; S as for O4. */
EXPORT void oracle_int16_matmul(const int16_t *qa, const float *sa,
                                const uint8_t *B, const double *scales,
                                const uint8_t *zp, const double *bias,
                                int64_t M, int64_t N, int64_t K, int64_t bs,
                                int bits, double *Y, double *S) {
    int64_t kb = n_blocks(K, bs);
    int64_t padded = kb * bs;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, mag = 0.0;
            for (int64_t b = 0; b < kb; ++b) {
                int64_t z = (int64_t)zp_at(zp, n, b, kb, bits);
                int64_t dot = 0, adot = 0;
                for (int64_t k = b * bs; k < (b + 1) * bs && k < K; ++k) {
                    int64_t t = (int64_t)qa[m * padded + k] *
                                ((int64_t)code_at(B, n, k, K, bs, bits) - z);
                    dot += t;
                    adot += t < 0 ? -t : t;
                }
                double f = (double)sa[m * kb + b] * scales[n * kb + b];
                acc += (double)dot * f;
                mag += (double)adot * fabs(f);
            }
            if (bias) {
                acc += bias[n];
                mag += fabs(bias[n]);
            }
            Y[m * N + n] = acc;
            if (S) S[m * N + n] = mag;
        }
}

/* ------------------------------------------------------------------------ */
/* O4 CompInt8 block dot ([ORT] prepack_int8_weight + int4_dot_row_scalar /   */
/* int8_row): dot[m, n, b] = sum over k of block b, k < K, of                 */
/* qa[m, k] * (code(n, k) - zp(n, b)), exact in integers.                     */
/* ------------------------------------------------------------------------ */
EXPORT void oracle_compint8_block_dots(const int8_t *qa, const uint8_t *B,
                                       const uint8_t *zp, int64_t M, int64_t N,
                                       int64_t K, int64_t bs, int bits,
                                       int32_t *dots) {
    int64_t kb = n_blocks(K, bs);
    int64_t padded = kb * bs;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m)
            for (int64_t b = 0; b < kb; ++b) {
                int64_t z = (int64_t)zp_at(zp, n, b, kb, bits);
                int64_t acc = 0;
                for (int64_t k = b * bs; k < (b + 1) * bs && k < K; ++k)
                    acc += (int64_t)qa[m * padded + k] *
                           ((int64_t)code_at(B, n, k, K, bs, bits) - z);
                dots[(m * N + n) * kb + b] = (int32_t)acc;
            }
}

/* CompInt8 output: Y[m, n] = sum_b dot[m,n,b] * sa[m,b] * s[n,b] (+ bias[n])
 * in double ([ORT] int8_row: the signed block dot scaled by the product of the
 * activation and weight scales, summed over blocks, bias added after).
 * S[m, n] = sum_k |qa[m,k] * sa[m,b] * w(n,k)| + |bias[n]|. */
EXPORT void oracle_compint8_matmul(const int8_t *qa, const float *sa,
                                   const uint8_t *B, const double *scales,
                                   const uint8_t *zp, const double *bias,
                                   int64_t M, int64_t N, int64_t K, int64_t bs,
                                   int bits, double *Y, double *S) {
    int64_t kb = n_blocks(K, bs);
    int64_t padded = kb * bs;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, mag = 0.0;
            for (int64_t b = 0; b < kb; ++b) {
                int64_t z = (int64_t)zp_at(zp, n, b, kb, bits);
                int64_t dot = 0, adot = 0;
                for (int64_t k = b * bs; k < (b + 1) * bs && k < K; ++k) {
                    int64_t t = (int64_t)qa[m * padded + k] *
                                ((int64_t)code_at(B, n, k, K, bs, bits) - z);
                    dot += t;
                    adot += t < 0 ? -t : t;
                }
                double f = (double)sa[m * kb + b] * scales[n * kb + b];
                acc += (double)dot * f;
                mag += (double)adot * fabs(f);
            }
            if (bias) {
                acc += bias[n];
                mag += fabs(bias[n]);
            }
            Y[m * N + n] = acc;
            if (S) S[m * N + n] = mag;
        }
}

/* ------------------------------------------------------------------------ */
/* Block-scaled FP4 weights ([RLX] dequant_matmul_nvfp4 and the low-precision */
/* scaled-GEMM reference lowp_scaled_matmul / lowp_dequantize).  Each weight  */
/* is an FP4 E2M1 code times its block's scale, blocks of bs elements along   */
/* K: MXFP4 = E8M0 scale per 32, NVFP4 = E4M3 scale per 16 and one f32 global */
/* scale.  The element formats are decoded from their published definitions  */
/* (OCP Microscaling formats; the NVFP4 scale is OCP FP8 E4M3):              */
/*   E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is the  */
/*         subnormal m * 0.5, else 2^(e-1) * (1 + m/2); no inf or nan.        */
/*   E8M0: 2^(e - 127); e = 255 is nan.                                        */
/*   E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is the */
/*         subnormal m/8 * 2^-6; S.1111.111 is nan; no inf.                   */
/* Layout (reading): weights [N, ceil(K/bs), bs/2] bytes, element k of row n  */
/* in byte k/2 of the row, the low nibble for even k (the nibble order of     */
/* [RLX] dequant_matmul_nvfp4, rows K-last as the rhs of lowp_scaled_matmul); */
/* scales [N, ceil(K/bs)] bytes.                                              */
/* ------------------------------------------------------------------------ */
EXPORT double oracle_e2m1(unsigned code) {
    int sign = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -v : v;
}

EXPORT double oracle_e8m0(unsigned byte) {
    if ((byte & 0xFF) == 0xFF) return NAN;
    return ldexp(1.0, (int)(byte & 0xFF) - 127);
}

EXPORT double oracle_e4m3(unsigned byte) {
    int sign = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp(m / 8.0, -6);
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* fmt 0: MXFP4 (bs 32, E8M0 scales); fmt 1: NVFP4 (bs 16, E4M3 scales).   */
static int fp4_block(int fmt) { return fmt == 0 ? 32 : 16; }

static double fp4_weight(const uint8_t *W, const uint8_t *scales, int fmt,
                         double global_scale, int64_t n, int64_t k, int64_t K) {
    int64_t bs = fp4_block(fmt);
    int64_t kb = n_blocks(K, bs);
    unsigned byte = W[n * kb * (bs / 2) + k / 2];
    unsigned code = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    uint8_t sb = scales[n * kb + k / bs];
    double s = fmt == 0 ? oracle_e8m0(sb) : oracle_e4m3(sb);
    return oracle_e2m1(code) * s * global_scale;
}

/* Dense weight [N, K] in double. */
EXPORT void oracle_fp4_dequantize(const uint8_t *W, const uint8_t *scales, int fmt,
                                  double global_scale, int64_t N, int64_t K,
                                  double *out) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            out[n * K + k] = fp4_weight(W, scales, fmt, global_scale, n, k, K);
}

/* Y[m, n] = sum_k A[m, k] * w(n, k) (+ bias[n]) in double; S as for O2. */
EXPORT void oracle_fp4_matmul(const double *A, const uint8_t *W,
                              const uint8_t *scales, int fmt, double global_scale,
                              const double *bias, int64_t M, int64_t N, int64_t K,
                              double *Y, double *S) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double t = A[m * K + k] *
                           fp4_weight(W, scales, fmt, global_scale, n, k, K);
                acc += t;
                mag += fabs(t);
            }
            if (bias) {
                acc += bias[n];
                mag += fabs(bias[n]);
            }
            Y[m * N + n] = acc;
            if (S) S[m * N + n] = mag;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Low-precision scaled GEMM ([RLX] quant.rs, its FP8/FP6/FP4 scaled-GEMM    */
/* reference: lowp_compute_scales, lowp_quantize, lowp_scaled_matmul,         */
/* lowp_dequantize, lowp_snap_scale, lowp_read_scales).                       */
/* One code per byte (its low bits), rows K-last, out = lhs . rhs^T (TN).     */
/* Element formats (fmt), decoded from their published definitions (OCP 8-bit */
/* floating point and OCP Microscaling formats):                              */
/*   0 E4M3: bias 7, 3 mantissa bits, S.1111.111 nan, no inf, max 448.        */
/*   1 E5M2: bias 15, 2 mantissa bits, exponent 31: inf (m = 0) or nan,       */
/*           max 57344.                                                       */
/*   2 E2M3 (FP6): bias 1, 3 mantissa bits, no inf or nan, max 7.5.           */
/*   3 E3M2 (FP6): bias 3, 2 mantissa bits, no inf or nan, max 28.            */
/*   4 E2M1 (FP4): bias 1, 1 mantissa bit, no inf or nan, max 6.              */
/* Exponent field 0 is subnormal: m / 2^mbits * 2^(1 - bias).                 */
/* Scale layouts (layout): 0 per tensor (one f32 per operand), 1 MX (one E8M0 */
/* byte per 32 elements along K), 2 NVFP4 (one E4M3 byte per 16 along K).     */
/* The codec itself is not printed on the pages; its readings:               */
/*   encode: the finite value of the format nearest to v, ties to the code    */
/*   with the even mantissa; beyond the largest finite value: that value     */
/*   (saturation, inf included); nan: the format's nan (E4M3 0x7F, E5M2      */
/*   0x7F) or 0 where it has none; the sign of v is kept on zero.            */
/*   f32_to_e8m0: the 8 exponent bits of the binary32 value (the power of two */
/*   at or below a normal value; 0 for zero and subnormals; 255 for inf and  */
/*   nan).                                                                    */
/* ------------------------------------------------------------------------ */
static const int LOWP_EBITS[5] = {4, 5, 2, 3, 2};
static const int LOWP_MBITS[5] = {3, 2, 3, 2, 1};
static const int LOWP_BIAS[5] = {7, 15, 1, 3, 1};

static int lowp_bits(int fmt) { return 1 + LOWP_EBITS[fmt] + LOWP_MBITS[fmt]; }

/* Nan or inf code (not a finite value). */
static int lowp_special(int fmt, unsigned c) {
    unsigned e = (c >> LOWP_MBITS[fmt]) & ((1u << LOWP_EBITS[fmt]) - 1);
    unsigned m = c & ((1u << LOWP_MBITS[fmt]) - 1);
    if (fmt == 0) return e == 15 && m == 7;
    if (fmt == 1) return e == 31;
    return 0;
}

EXPORT double oracle_lowp_decode(int fmt, unsigned code) {
    int mb = LOWP_MBITS[fmt], eb = LOWP_EBITS[fmt], bias = LOWP_BIAS[fmt];
    unsigned c = code & ((1u << lowp_bits(fmt)) - 1);
    int sign = (c >> (eb + mb)) & 1;
    int e = (int)((c >> mb) & ((1u << eb) - 1));
    int m = (int)(c & ((1u << mb) - 1));
    double v;
    if (fmt == 0 && e == 15 && m == 7) return NAN;
    if (fmt == 1 && e == 31) v = m == 0 ? INFINITY : NAN;
    else if (e == 0) v = ldexp((double)m / (1 << mb), 1 - bias);
    else v = ldexp(1.0 + (double)m / (1 << mb), e - bias);
    return sign ? -v : v;
}

EXPORT double oracle_lowp_max_finite(int fmt) {
    static const double mx[5] = {448.0, 57344.0, 7.5, 28.0, 6.0};
    return mx[fmt];
}

EXPORT unsigned oracle_lowp_encode(int fmt, double v) {
    int bits = lowp_bits(fmt);
    unsigned signbit = 1u << (bits - 1);
    if (isnan(v)) return (fmt == 0 || fmt == 1) ? 0x7Fu : 0u;
    unsigned sgn = signbit(v) ? signbit : 0u;
    double a = fabs(v);
    if (a > oracle_lowp_max_finite(fmt)) a = oracle_lowp_max_finite(fmt);  /* saturation */
    unsigned best = 0;
    double best_d = INFINITY;
    for (unsigned c = 0; c < signbit; ++c) {          /* the non-negative codes */
        if (lowp_special(fmt, c)) continue;
        double d = fabs(oracle_lowp_decode(fmt, c) - a);
        if (d < best_d || (d == best_d && (c & 1u) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return best | sgn;
}

EXPORT unsigned oracle_f32_to_e8m0(float s) {
    uint32_t u;
    memcpy(&u, &s, 4);
    return (u >> 23) & 0xFFu;
}

static int lowp_block(int layout) { return layout == 1 ? 32 : 16; }

/* lowp_snap_scale: the value the layout can store nearest (by its reading)   */
/* to s.                                                                      */
EXPORT float oracle_lowp_snap_scale(int layout, float s) {
    if (layout == 0) return s;
    if (layout == 1) return (float)oracle_e8m0(oracle_f32_to_e8m0(s));
    return (float)oracle_lowp_decode(0, oracle_lowp_encode(0, (double)s));
}

/* lowp_compute_scales: raw f32 scales of x [rows, cols] (per tensor: one;    */
/* else [rows, nblk]): amax / max_finite (1 where amax is 0), snapped.        */
EXPORT void oracle_lowp_compute_scales(const float *x, int fmt, int layout, int64_t rows,
                                       int64_t cols, float *out) {
    float maxf = (float)oracle_lowp_max_finite(fmt);
    if (layout == 0) {
        float amax = 0.0f;
        for (int64_t i = 0; i < rows * cols; ++i) amax = fmaxf(amax, fabsf(x[i]));
        out[0] = amax > 0.0f ? amax / maxf : 1.0f;
        return;
    }
    int64_t bs = lowp_block(layout), nblk = n_blocks(cols, bs);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nblk; ++b) {
            float amax = 0.0f;
            for (int64_t c = b * bs; c < cols && c < (b + 1) * bs; ++c)
                amax = fmaxf(amax, fabsf(x[r * cols + c]));
            out[r * nblk + b] = oracle_lowp_snap_scale(layout, amax > 0.0f ? amax / maxf : 1.0f);
        }
}

/* Stored scale bytes of raw scales (ScaledQuantScale): per tensor the f32   */
/* itself, MX the E8M0 byte, NVFP4 the E4M3 byte.                             */
EXPORT void oracle_lowp_store_scales(const float *scales, int layout, int64_t n, void *out) {
    if (layout == 0) {
        memcpy(out, scales, 4);
        return;
    }
    uint8_t *o = (uint8_t *)out;
    for (int64_t i = 0; i < n; ++i)
        o[i] = (uint8_t)(layout == 1 ? oracle_f32_to_e8m0(scales[i])
                                     : oracle_lowp_encode(0, (double)scales[i]));
}

/* lowp_read_scales: decoded raw scales from stored bytes. */
EXPORT void oracle_lowp_read_scales(const void *stored, int layout, int64_t n, float *out) {
    if (layout == 0) {
        memcpy(out, stored, 4);
        return;
    }
    const uint8_t *b = (const uint8_t *)stored;
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)(layout == 1 ? oracle_e8m0(b[i]) : oracle_lowp_decode(0, b[i]));
}

static float lowp_scale_at(int layout, const float *scales, int64_t row, int64_t col,
                           int64_t nblk) {
    if (layout == 0) return scales[0];
    return scales[row * nblk + col / lowp_block(layout)];
}

/* lowp_quantize: code = encode(x / s) with the binary32 quotient (0 where s  */
/* is 0).                                                                     */
EXPORT void oracle_lowp_quantize(const float *x, const float *scales, int fmt, int layout,
                                 int64_t rows, int64_t cols, uint8_t *out) {
    int64_t nblk = layout == 0 ? 1 : n_blocks(cols, lowp_block(layout));
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float s = lowp_scale_at(layout, scales, r, c, nblk);
            float v = s != 0.0f ? x[r * cols + c] / s : 0.0f;
            out[r * cols + c] = (uint8_t)oracle_lowp_encode(fmt, (double)v);
        }
}

/* lowp_dequantize: decode(code) * scale, in double. */
EXPORT void oracle_lowp_dequantize(const uint8_t *codes, const float *scales, int fmt,
                                   int layout, int64_t rows, int64_t cols, double *out) {
    int64_t nblk = layout == 0 ? 1 : n_blocks(cols, lowp_block(layout));
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[r * cols + c] = oracle_lowp_decode(fmt, codes[r * cols + c]) *
                                (double)lowp_scale_at(layout, scales, r, c, nblk);
}

/* lowp_scaled_matmul: out[i, j] = sum_p a(i, p) b(j, p) (+ bias[j]) with     */
/* a = decode(lhs) * lhs scale, b = decode(rhs) * rhs scale, in double; S the */
/* sum of |a b| (+ |bias|).                                                   */
EXPORT void oracle_lowp_scaled_matmul(const uint8_t *lhs, const uint8_t *rhs,
                                      const float *ls, const float *rs, const double *bias,
                                      int64_t m, int64_t n, int64_t k, int layout,
                                      int lfmt, int rfmt, double *out, double *S) {
    int64_t nblk = layout == 0 ? 1 : n_blocks(k, lowp_block(layout));
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0, mag = 0.0;
            for (int64_t p = 0; p < k; ++p) {
                double a = oracle_lowp_decode(lfmt, lhs[i * k + p]) *
                           (double)lowp_scale_at(layout, ls, i, p, nblk);
                double b = oracle_lowp_decode(rfmt, rhs[j * k + p]) *
                           (double)lowp_scale_at(layout, rs, j, p, nblk);
                acc += a * b;
                mag += fabs(a * b);
            }
            if (bias) {
                acc += bias[j];
                mag += fabs(bias[j]);
            }
            out[i * n + j] = acc;
            if (S) S[i * n + j] = mag;
        }
}

/* ------------------------------------------------------------------------ */
/* O5 int8 convolution with requantization.                                   */
/* acc = bias[oc] + sum over taps and input channels of                       */
/*       (x - in_zp) * w, an out-of-bounds tap reading x = in_zp             */
/*       ([MNN] im2col padding filled with the input zero point;              */
/*        [RLX] exec_q_mat_mul: bias seeds the int32 accumulator)             */
/* mult[oc] = (in_scale * w_scale[oc]) / out_scale in binary32                */
/* y = clamp(rne(float(acc) * mult[oc]) + out_zp, clamp_min, clamp_max)       */
/*       ([RLX] exec_q_mat_mul requantize; [MNN] clamp bounds; reading:       */
/*        ties to even)                                                        */
/* X is NHWC [Nb, H, W, C], Wt is OHWI [Co, KH, KW, C], Y is NHWC             */
/* [Nb, OH, OW, Co]; groups = dilation = 1; bias may be NULL (zero).          */
/* acc_out (nullable) receives the int32 accumulators, same layout as Y.      */
/* ------------------------------------------------------------------------ */
EXPORT void oracle_conv_int8(const int8_t *X, const int8_t *Wt,
                             const int32_t *bias, const float *w_scale,
                             float in_scale, float out_scale, int in_zp,
                             int out_zp, int clamp_min, int clamp_max, int Nb,
                             int H, int W, int C, int Co, int KH, int KW,
                             int sh, int sw, int ph, int pw, int8_t *Y,
                             int32_t *acc_out) {
    int OH = (H + 2 * ph - KH) / sh + 1;
    int OW = (W + 2 * pw - KW) / sw + 1;
    for (int nb = 0; nb < Nb; ++nb)
        for (int oh = 0; oh < OH; ++oh)
            for (int ow = 0; ow < OW; ++ow)
                for (int oc = 0; oc < Co; ++oc) {
                    int64_t acc = bias ? bias[oc] : 0;
                    for (int kh = 0; kh < KH; ++kh)
                        for (int kw = 0; kw < KW; ++kw) {
                            int ih = oh * sh - ph + kh;
                            int iw = ow * sw - pw + kw;
                            int inside = ih >= 0 && ih < H && iw >= 0 && iw < W;
                            for (int c = 0; c < C; ++c) {
                                int x = inside
                                    ? X[(((int64_t)nb * H + ih) * W + iw) * C + c]
                                    : in_zp;
                                int w = Wt[(((int64_t)oc * KH + kh) * KW + kw) * C + c];
                                acc += (int64_t)(x - in_zp) * w;
                            }
                        }
                    int64_t o = (((int64_t)nb * OH + oh) * OW + ow) * Co + oc;
                    if (acc_out) acc_out[o] = (int32_t)acc;
                    float mult = (in_scale * w_scale[oc]) / out_scale;
                    float r = rintf((float)acc * mult);
                    double v = (double)r + (double)out_zp;
                    if (v < clamp_min) v = clamp_min;
                    if (v > clamp_max) v = clamp_max;
                    Y[o] = (int8_t)v;
                }
}
