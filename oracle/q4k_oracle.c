/*
 * q4k_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU statement of what the fused-dequantize Q4_K
 * matrix-vector product and its ternary sibling compute.  Only the test
 * suite, the package smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code, header, table or constant with the
 * GPU library; it is built with gcc, -O2 -ffp-contract=off, single-threaded.
 *
 * Sources (the pages this follows):
 *   [Q4K]  SKaiNET PR #562, "feat(kernel): SIMD-fused Q4_K matmul kernel +
 *          Q4KMatmulKernel SPI" -- sections "Pipeline" (the canonical
 *          strided qs layout, the lazy-dmin correction) and "Test plan"
 *          (1e-4 parity bar, rejection of inputDim % 256 != 0).
 *          Section "Out of scope" names the follow-ups: Q4_0, the same
 *          algorithm on a simpler block of 32 weights in 18 bytes, and Q6_K,
 *          whose ql + qh layout packs four codes' high bits per qh byte in
 *          two interleaved halves.
 *   [EAG]  SKaiNET docs, "Eager execution: backends and kernels" -- packed
 *          weights reach a kernel by declaring their block order, and a
 *          canonical weight is relayouted into that order once, not per
 *          call.
 *   [TRN]  SKaiNET issue #1138, "[ternary-f32] Phase 2: TernaryF32GemvNative
 *          SPI + reference ViewKernel + TernaryF32KernelPack" -- section
 *          "Tasks" (the gemvPacked contract, the decode formula, the
 *          post-multiplied per-tensor scale, the prefill row loop).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - block_q4_K is 144 bytes: fp16 d at byte 0, fp16 dmin at byte 2 (both
 *     little-endian), 12 bytes of packed 6-bit scales/mins at 4..15 and
 *     128 bytes of qs at 16..143.
 *   - the 12 scale bytes follow the ggml packing (see unpack_scales).
 *   - qs byte 32*j + l holds position l of sub-block 2j (low nibble) and
 *     position l of sub-block 2j+1 (high nibble).
 *   - W is row-major [output][input]: row o holds inputDim/256 blocks.
 *   - weight = d*sc*q - dmin*m ("offset" is subtracted).
 *   - block_q4_0 is 18 bytes: fp16 d at byte 0 (little-endian) and 16
 *     bytes of qs at 2..17; element i < 16 is the low nibble of qs[i],
 *     element 16 + i its high nibble; weight = d * (q - 8) (ggml's
 *     block_q4_0 convention; the page gives only "32 / 18 bytes").
 *   - block_q6_K is 210 bytes: ql[128] at 0, qh[64] at 128, 16 int8
 *     scales at 192, fp16 d at 208 (ggml's block_q6_K; the page names only
 *     ql, qh and the half-interleaved qh packing).  Element e = 128n + 32c
 *     + l (half n, quadrant c, l < 32) has code q = lo | hi << 4 with lo the
 *     low (c < 2) or high (c >= 2) nibble of ql[64n + 32(c & 1) + l] and hi
 *     bits 2c..2c+1 of qh[32n + l]; its sub-block of 16 is 8n + 2c + l/16
 *     and weight = d * scale[sub-block] * (q - 32).
 *   - the tiled block order (see oracle_q4k_relayout_tiled) is this
 *     library's own GPU block order: the docs page fixes only that a
 *     packed weight declares its block order and that a canonical weight is
 *     relayouted into it once.
 *   - ternary element i of a row is bits 2*(i%4)..2*(i%4)+1 of byte i/4;
 *     code 3 decodes to +2 by the formula (never generated).
 *
 * Parity pins for every function live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL_DIM (-1)
#define ORACLE_ENULL (-2)

#define QK 256          /* weights per super-block */
#define BLOCK_BYTES 144 /* bytes per super-block */

/* IEEE-754 binary16 -> binary32, written from the format definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0 is
 * zero/subnormal (fraction * 2^-24), exponent 31 is inf/NaN.  Every
 * binary16 value is exactly representable in binary32. */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return (float)(sign ? -v : v);
}

void oracle_f16_to_f32_array(const uint16_t *h, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f16_to_f32(h[i]);
}

/* The 12 packed bytes S[0..11] carry eight 6-bit scales sc[s] and eight
 * 6-bit mins m[s] (ggml block_q4_K packing):
 *   s < 4 : sc[s] = S[s] & 63,               m[s] = S[s+4] & 63
 *   s >= 4: sc[s] = (S[s+4] & 15) | (S[s-4] >> 6) << 4
 *           m[s]  = (S[s+4] >> 4) | (S[s]   >> 6) << 4            */
void oracle_q4k_unpack_scales(const uint8_t *S, uint8_t *sc, uint8_t *m)
{
    for (int s = 0; s < 8; ++s) {
        if (s < 4) {
            sc[s] = (uint8_t)(S[s] & 63);
            m[s] = (uint8_t)(S[s + 4] & 63);
        } else {
            sc[s] = (uint8_t)((S[s + 4] & 15) | ((S[s - 4] >> 6) << 4));
            m[s] = (uint8_t)((S[s + 4] >> 4) | ((S[s] >> 6) << 4));
        }
    }
}

/* Fully dequantize one 144-byte super-block into 256 fp32 weights.
 * d*sc*q needs at most 11+6+4 = 21 significant bits and dmin*m at most
 * 17, so both products are exact in fp32 and each weight is the
 * correctly rounded value of the exact d*sc*q - dmin*m. */
void oracle_q4k_dequant_block(const uint8_t *blk, float *w)
{
    uint16_t dh = (uint16_t)(blk[0] | (blk[1] << 8));
    uint16_t mh = (uint16_t)(blk[2] | (blk[3] << 8));
    float d = oracle_f16_to_f32(dh);
    float dmin = oracle_f16_to_f32(mh);
    uint8_t sc[8], m[8];
    oracle_q4k_unpack_scales(blk + 4, sc, m);
    const uint8_t *qs = blk + 16;
    for (int j = 0; j < 4; ++j) {
        int s_lo = 2 * j, s_hi = 2 * j + 1;
        for (int l = 0; l < 32; ++l) {
            uint8_t byte = qs[32 * j + l];
            float q_lo = (float)(byte & 15);
            float q_hi = (float)(byte >> 4);
            float a_lo = (d * (float)sc[s_lo]) * q_lo;
            float b_lo = dmin * (float)m[s_lo];
            float a_hi = (d * (float)sc[s_hi]) * q_hi;
            float b_hi = dmin * (float)m[s_hi];
            w[64 * j + l] = a_lo - b_lo;
            w[64 * j + 32 + l] = a_hi - b_hi;
        }
    }
}

static int check_q4k(const void *x, const void *w, const void *y,
                     int64_t K, int64_t N)
{
    if (K <= 0 || N <= 0 || K % QK != 0)
        return ORACLE_EINVAL_DIM;
    if (!x || !w || !y)
        return ORACLE_ENULL;
    return ORACLE_OK;
}

/* y[o] = sum_k W[o,k] * x[k]: dequantize each block to fp32, then a
 * double-precision dot (every fp32*fp32 product is exact in double). */
int oracle_q4k_gemv(const float *x, const uint8_t *w, int64_t K, int64_t N,
                    double *y)
{
    int rc = check_q4k(x, w, y, K, N);
    if (rc)
        return rc;
    int64_t nb = K / QK;
    float wt[QK];
    for (int64_t o = 0; o < N; ++o) {
        double acc = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            oracle_q4k_dequant_block(w + (o * nb + b) * BLOCK_BYTES, wt);
            const float *xb = x + b * QK;
            for (int p = 0; p < QK; ++p)
                acc += (double)wt[p] * (double)xb[p];
        }
        y[o] = acc;
    }
    return ORACLE_OK;
}

/* The same product evaluated in the lazy-dmin form the Q4_K page describes:
 * per sub-block, scale * (sum of code*x) minus offset * (sum of x), with
 * scale = d*sc and offset = dmin*m.  Double precision throughout.  Used only
 * to pin the identity "lazy-dmin == dequantize-then-dot". */
int oracle_q4k_gemv_lazy(const float *x, const uint8_t *w, int64_t K,
                         int64_t N, double *y)
{
    int rc = check_q4k(x, w, y, K, N);
    if (rc)
        return rc;
    int64_t nb = K / QK;
    for (int64_t o = 0; o < N; ++o) {
        double acc = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = w + (o * nb + b) * BLOCK_BYTES;
            double d = oracle_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
            double dmin = oracle_f16_to_f32((uint16_t)(blk[2] | (blk[3] << 8)));
            uint8_t sc[8], m[8];
            oracle_q4k_unpack_scales(blk + 4, sc, m);
            const uint8_t *qs = blk + 16;
            const float *xb = x + b * QK;
            for (int s = 0; s < 8; ++s) {
                int j = s / 2;
                double code_sum = 0.0, input_sum = 0.0;
                for (int l = 0; l < 32; ++l) {
                    uint8_t byte = qs[32 * j + l];
                    int q = (s % 2 == 0) ? (byte & 15) : (byte >> 4);
                    double xv = xb[32 * s + l];
                    code_sum += (double)q * xv;
                    input_sum += xv;
                }
                acc += (d * (double)sc[s]) * code_sum -
                       (dmin * (double)m[s]) * input_sum;
            }
        }
        y[o] = acc;
    }
    return ORACLE_OK;
}

/* Batched: Y[r, :] = W * X[r, :] for each token row r (row r of X at r*K,
 * row r of Y at r*N), the row loop of the ternary page's prefill path. */
int oracle_q4k_matmul(const float *X, const uint8_t *w, int64_t M, int64_t K,
                      int64_t N, double *Y)
{
    if (M <= 0)
        return ORACLE_EINVAL_DIM;
    int rc = check_q4k(X, w, Y, K, N);
    if (rc)
        return rc;
    for (int64_t r = 0; r < M; ++r) {
        rc = oracle_q4k_gemv(X + r * K, w, K, N, Y + r * N);
        if (rc)
            return rc;
    }
    return ORACLE_OK;
}

/* Rows [row_begin, row_end) of the batched product for token rows
 * [tok_begin, tok_end): lets a caller check sampled outputs of a large
 * problem one by one.  Y is indexed with the full N and M layout. */
int oracle_q4k_matmul_part(const float *X, const uint8_t *w, int64_t M,
                           int64_t K, int64_t N, int64_t tok_begin,
                           int64_t tok_end, int64_t row_begin,
                           int64_t row_end, double *Y)
{
    if (M <= 0 || tok_begin < 0 || tok_end > M || tok_begin > tok_end ||
        row_begin < 0 || row_end > N || row_begin > row_end)
        return ORACLE_EINVAL_DIM;
    int rc = check_q4k(X, w, Y, K, N);
    if (rc)
        return rc;
    int64_t nb = K / QK;
    float wt[QK];
    for (int64_t r = tok_begin; r < tok_end; ++r) {
        for (int64_t o = row_begin; o < row_end; ++o) {
            double acc = 0.0;
            for (int64_t b = 0; b < nb; ++b) {
                oracle_q4k_dequant_block(w + (o * nb + b) * BLOCK_BYTES, wt);
                const float *xb = X + r * K + b * QK;
                for (int p = 0; p < QK; ++p)
                    acc += (double)wt[p] * (double)xb[p];
            }
            Y[r * N + o] = acc;
        }
    }
    return ORACLE_OK;
}

#define TILE_ROWS 16     /* rows per row group of the tiled order */
#define TILE_BYTES 2304  /* 16 rows x 144 bytes */

/* [EAG]: the one-time relayout of a canonical Q4_K matrix into the tiled
 * block order.  The same bytes are moved, none is changed:
 *   - rows are taken in groups of 16 (group G holds rows 16G .. 16G+15;
 *     rows at or past N are zero bytes), and super-block b of group G is one
 *     2304-byte tile at byte (G*nb + b)*2304, nb = K/256;
 *   - tile bytes 0..2047 hold the qs bytes of the 16 rows in two halves of
 *     1024: qs byte 32j + 8g + t (sub-block pair j < 4, g < 4, t < 8) of row
 *     16G + n goes to byte 1024*(j/2) + 16*(n + 16g) + 8*(j%2) + t;
 *   - tile bytes 2048..2303 hold the 16 block headers (bytes 0..15: d,
 *     dmin, the 12 scale bytes) of rows 16G .. 16G+15, in row order.
 * The walk below is the plain one: every tile, every row, every byte. */
int oracle_q4k_relayout_tiled(const uint8_t *w, int64_t K, int64_t N,
                              uint8_t *out)
{
    if (K <= 0 || N <= 0 || K % QK != 0)
        return ORACLE_EINVAL_DIM;
    if (!w || !out)
        return ORACLE_ENULL;
    int64_t nb = K / QK;
    int64_t ng = (N + TILE_ROWS - 1) / TILE_ROWS;
    for (int64_t G = 0; G < ng; ++G) {
        for (int64_t b = 0; b < nb; ++b) {
            uint8_t *tile = out + (G * nb + b) * TILE_BYTES;
            for (int n = 0; n < TILE_ROWS; ++n) {
                int64_t row = TILE_ROWS * G + n;
                const uint8_t *blk =
                    row < N ? w + (row * nb + b) * BLOCK_BYTES : NULL;
                for (int c = 0; c < 16; ++c)
                    tile[2048 + 16 * n + c] = blk ? blk[c] : 0;
                for (int j = 0; j < 4; ++j)
                    for (int g = 0; g < 4; ++g)
                        for (int t = 0; t < 8; ++t)
                            tile[1024 * (j / 2) + 16 * (n + 16 * g) +
                                 8 * (j % 2) + t] =
                                blk ? blk[16 + 32 * j + 8 * g + t] : 0;
            }
        }
    }
    return ORACLE_OK;
}

#define QK40 32          /* weights per Q4_0 block */
#define BLOCK40_BYTES 18 /* bytes per Q4_0 block */

/* Dequantize one 18-byte Q4_0 block into 32 fp32 weights.  d has 11
 * significant bits and q - 8 lies in [-8, 7], so every product is exact in
 * fp32. */
void oracle_q4_0_dequant_block(const uint8_t *blk, float *w)
{
    float d = oracle_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
    const uint8_t *qs = blk + 2;
    for (int i = 0; i < 16; ++i) {
        w[i] = d * (float)((int)(qs[i] & 15) - 8);
        w[16 + i] = d * (float)((int)(qs[i] >> 4) - 8);
    }
}

/* y[o] = sum_k W[o,k] * x[k] for a Q4_0 matrix whose row o holds inputDim/32
 * blocks: dequantize each block, then a double-precision dot. */
int oracle_q4_0_gemv(const float *x, const uint8_t *w, int64_t K, int64_t N,
                     double *y)
{
    if (K <= 0 || N <= 0 || K % QK40 != 0)
        return ORACLE_EINVAL_DIM;
    if (!x || !w || !y)
        return ORACLE_ENULL;
    int64_t nb = K / QK40;
    float wt[QK40];
    for (int64_t o = 0; o < N; ++o) {
        double acc = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            oracle_q4_0_dequant_block(w + (o * nb + b) * BLOCK40_BYTES, wt);
            const float *xb = x + b * QK40;
            for (int p = 0; p < QK40; ++p)
                acc += (double)wt[p] * (double)xb[p];
        }
        y[o] = acc;
    }
    return ORACLE_OK;
}

#define QK6 256           /* weights per Q6_K block */
#define BLOCK6_BYTES 210  /* bytes per Q6_K block */

/* Dequantize one 210-byte Q6_K block into 256 fp32 weights.  d has 11
 * significant bits, the scale 7 and q - 32 6, so d * scale * (q - 32) is
 * exact in fp32 (evaluated as (d * scale) * (q - 32), both steps exact). */
void oracle_q6k_dequant_block(const uint8_t *blk, float *w)
{
    const uint8_t *ql = blk;
    const uint8_t *qh = blk + 128;
    const int8_t *sc = (const int8_t *)(blk + 192);
    float d = oracle_f16_to_f32((uint16_t)(blk[208] | (blk[209] << 8)));
    for (int n = 0; n < 2; ++n) {
        for (int c = 0; c < 4; ++c) {
            for (int l = 0; l < 32; ++l) {
                uint8_t lbyte = ql[64 * n + 32 * (c & 1) + l];
                int lo = (c < 2) ? (lbyte & 15) : (lbyte >> 4);
                int hi = (qh[32 * n + l] >> (2 * c)) & 3;
                int q = lo | (hi << 4);
                float s = d * (float)sc[8 * n + 2 * c + l / 16];
                w[128 * n + 32 * c + l] = s * (float)(q - 32);
            }
        }
    }
}

/* y[o] = sum_k W[o,k] * x[k] for a Q6_K matrix whose row o holds
 * inputDim/256 blocks: dequantize each block, then a double-precision dot. */
int oracle_q6k_gemv(const float *x, const uint8_t *w, int64_t K, int64_t N,
                    double *y)
{
    if (K <= 0 || N <= 0 || K % QK6 != 0)
        return ORACLE_EINVAL_DIM;
    if (!x || !w || !y)
        return ORACLE_ENULL;
    int64_t nb = K / QK6;
    float wt[QK6];
    for (int64_t o = 0; o < N; ++o) {
        double acc = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            oracle_q6k_dequant_block(w + (o * nb + b) * BLOCK6_BYTES, wt);
            const float *xb = x + b * QK6;
            for (int p = 0; p < QK6; ++p)
                acc += (double)wt[p] * (double)xb[p];
        }
        y[o] = acc;
    }
    return ORACLE_OK;
}

/* Ternary BitNet b1.58 decode of one byte: element i (0..3) is
 * ((byte >> 2i) & 3) - 1. */
void oracle_ternary_decode_byte(uint8_t byte, int32_t *codes)
{
    for (int i = 0; i < 4; ++i)
        codes[i] = (int32_t)((byte >> (2 * i)) & 3) - 1;
}

static int check_ternary(const void *x, const void *c, const void *y,
                         int64_t K, int64_t N)
{
    if (K <= 0 || N <= 0 || K % 4 != 0)
        return ORACLE_EINVAL_DIM;
    if (!x || !c || !y)
        return ORACLE_ENULL;
    return ORACLE_OK;
}

/* The codes-dot t[o] = sum_i code(o, i) * x[i], scale NOT applied.  Row o
 * holds K/4 bytes. */
int oracle_ternary_gemv_codes(const float *x, const uint8_t *codes, int64_t K,
                              int64_t N, double *t)
{
    int rc = check_ternary(x, codes, t, K, N);
    if (rc)
        return rc;
    int64_t row_bytes = K / 4;
    int32_t c[4];
    for (int64_t o = 0; o < N; ++o) {
        double acc = 0.0;
        for (int64_t i = 0; i < K; ++i) {
            if (i % 4 == 0)
                oracle_ternary_decode_byte(codes[o * row_bytes + i / 4], c);
            acc += (double)c[i % 4] * (double)x[i];
        }
        t[o] = acc;
    }
    return ORACLE_OK;
}

/* Batched ternary product, the row loop of the ternary page's prefill path
 * (section "Tasks"): Y[r, :] = scale * t(X[r, :]) for each token row r, row
 * r of X at r*K and of Y at r*N. */
int oracle_ternary_matmul(const float *X, const uint8_t *codes, float scale,
                          int64_t M, int64_t K, int64_t N, double *Y);

/* y[o] = scale * t[o]: the per-tensor scale is multiplied after the dot. */
int oracle_ternary_gemv(const float *x, const uint8_t *codes, float scale,
                        int64_t K, int64_t N, double *y)
{
    int rc = oracle_ternary_gemv_codes(x, codes, K, N, y);
    if (rc)
        return rc;
    for (int64_t o = 0; o < N; ++o)
        y[o] = (double)scale * y[o];
    return ORACLE_OK;
}

int oracle_ternary_matmul(const float *X, const uint8_t *codes, float scale,
                          int64_t M, int64_t K, int64_t N, double *Y)
{
    if (M <= 0)
        return ORACLE_EINVAL_DIM;
    int rc = check_ternary(X, codes, Y, K, N);
    if (rc)
        return rc;
    for (int64_t r = 0; r < M; ++r) {
        rc = oracle_ternary_gemv(X + r * K, codes, scale, K, N, Y + r * N);
        if (rc)
            return rc;
    }
    return ORACLE_OK;
}
