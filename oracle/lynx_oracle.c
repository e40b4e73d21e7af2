/*
 * Lynx hierarchical split-stream quantizer: CPU ORACLE.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this file's library.  The GPU
 * library never links, includes or calls anything here, and this file shares
 * no code, header, table or constant generator with it.
 *
 * Source: "Lynx: Progressive Speculative Quantization for accelerating KV
 * Transfer in Long-Context Inference" (Han et al.), Section 4.1,
 * Algorithm 1 "Lynx Hierarchical Quantization (Vectorized)", Eq. (3) and
 * Eq. (4); the reading notes "Lynx 阅读笔记" (Zhongzhu Zhou), section
 * "具体算例" (worked example) for the inverse and the anchor-only level.
 *
 * Arithmetic: IEEE-754 binary32 with round-to-nearest-even for every step
 * of Algorithm 1, one rounding per operation (built with -ffp-contract=off,
 * no fast-math).  The compander decision (Eq. 3 followed by Round) is taken
 * in binary64, which decides the real-arithmetic rounding of Y exactly for
 * every binary32 input (the test suite pins the margin).  Attention is
 * evaluated in binary64.
 *
 * Readings of points the pages leave open (each one is listed with its
 * reason in the design notes of the repository):
 *   - axis=1 of X in R^{H x P} is the token axis: statistics are per channel;
 *   - one epsilon for both stages;
 *   - gamma_min, gamma_scale and mu are canonicalised with "+ 0.0f" (turns
 *     -0 into +0), so every stored statistic has one bit pattern;
 *   - the 32-token mean is a balanced pairwise tree sum, then / C;
 *   - S = Sign(X_cent), with +0 and -0 counted as non-negative;
 *   - Round is round-half-up of the real value Y;
 *   - the compander's top code is a parameter (code_scale): 120 by default,
 *     the largest code whose anchor magnitude (I + 7) >> 4 fits a 4-bit
 *     two's-complement nibble; with Eq. (3)'s printed 127 the integer code
 *     is clipped at 120;
 *   - anchor-only reconstruction uses code V << 4;
 *   - the exact inverse of Eq. (3) is ((1 + alpha)^(I / code_scale) - 1) /
 *     alpha;
 *   - denormalisation is the literal inverse of lines "X_final" then
 *     "X <- (X - gamma_min) / (gamma_scale + eps)", four roundings, then
 *     bf16 round-to-nearest-even;
 *   - nibble packing: two channels per byte (channel 2k in the low nibble,
 *     2k+1 in the high nibble), one byte per token; bytes are chunk-tiled,
 *     [chunk j][channel pair k][token i of the chunk], so every chunk of a
 *     page block is one contiguous (H/2) x C byte tile;
 *   - other splits of the 8-bit code (a anchor bits, b = 8 - a residual
 *     bits; the paper's split is 4 + 4): the bias of Stage 4 becomes
 *     2^(b-1) - 1 (the paper's +7 for b = 4), codes are clipped to the
 *     largest one whose anchor magnitude fits a bits, and the fields are
 *     packed as an LSB-first bit stream per (chunk, channel pair): value
 *     2 i + e (token i of the chunk, channel 2k + e) at bit w (2 i + e) of
 *     the pair's C w / 4 bytes.  For a = 4 this is the nibble layout above;
 *   - the single-precision configurations of the paper's evaluation
 *     (Lynx-INT4, Lynx-INT8: Algorithm 1 into one stream, no split) are
 *     one a-bit field per value and no residual (b = 0): the code of
 *     Eq. (3) with code_scale 2^(a-1) - 1 (7 or 127), its magnitude V = I
 *     in the field, one's-complemented for a negative value as the anchor
 *     is; the largest code is 2^(a-1) - 1;
 *   - bfloat16 metadata (meta_bits = 16): every statistic is rounded to a
 *     bfloat16 value where Algorithm 1 produces it and the rounded value is
 *     used from there on, so that the decoder inverts what the encoder did:
 *     gamma_min needs no rounding (a minimum of bfloat16 inputs), gamma_scale
 *     and sigma are rounded up (so X_norm <= 1 and |X_final| <= 1 still
 *     hold), mu to nearest (ties to even).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL -1

/* ---------------------------------------------------------------- bf16 -- */

static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round-to-nearest-even from binary32 to bfloat16 on the bit pattern. */
static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) /* NaN: keep it a quiet NaN */
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* The smallest bfloat16 value >= f, for f >= 0 (bf16 metadata: a scale
 * rounded up never makes a normalised value exceed 1). */
static float bf16_ceil_nonneg(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (u & 0xffffu)
        u = (u & 0xffff0000u) + 0x10000u; /* next bfloat16 above |f| */
    memcpy(&f, &u, sizeof f);
    return f;
}

/* f rounded to the nearest bfloat16 value (ties to even), as binary32. */
static float bf16_nearest(float f)
{
    return bf16_to_f32(f32_to_bf16_rne(f));
}

/* ------------------------------------------------------- Eq. (3), Round -- */

/* Integer code of one magnitude |X_final| (Algorithm 1, Stage 3):
 *   Y = code_scale * ln(1 + alpha*|x|) / ln(1 + alpha),  I = Round(Y),
 * with Round taken as round-half-up of the real value.  alpha*|x| is an
 * exact binary64 product of two binary32 values. */
int oracle_code(float x_abs, float alpha, float code_scale)
{
    double y = (double)code_scale * log1p((double)alpha * (double)x_abs) /
               log1p((double)alpha);
    /* Only non-finite inputs (unspecified codes) leave [0, code_scale]:
     * keep the integer conversion defined for them. */
    if (!(y >= 0.0))
        return 0;
    if (y > 1.0e9)
        return 1000000000;
    double fl = floor(y);
    int i = (int)fl;
    if (y - fl >= 0.5)
        i += 1;
    return i;
}

/* The same Y as a binary64 value, for tests that measure the distance of Y
 * to the rounding boundaries. */
double oracle_code_real(float x_abs, float alpha, float code_scale)
{
    return (double)code_scale * log1p((double)alpha * (double)x_abs) /
           log1p((double)alpha);
}

/* Field widths: a anchor bits and b residual bits, either a split of the
 * 8-bit code (a + b = 8) or a single stream of a-bit codes (b = 0). */
static int valid_bits(int a, int b)
{
    return (a + b == 8 && a >= 2 && a <= 7) || (b == 0 && a >= 2 && a <= 8);
}

/* Largest code whose anchor magnitude (I + bias) >> b still fits an a-bit
 * two's-complement anchor (magnitude <= 2^(a-1) - 1 for either sign):
 * 2^7 - 2^(b-1) for a split (120 for the paper's 4 + 4), 2^(a-1) - 1 for a
 * single stream. */
int oracle_code_max(int anchor_bits, int residual_bits)
{
    if (!valid_bits(anchor_bits, residual_bits))
        return -1;
    if (residual_bits == 0)
        return (1 << (anchor_bits - 1)) - 1;
    return 128 - (1 << (residual_bits - 1));
}

/* Reconstruction level of code k, the inverse of Eq. (3)
 * (|x^| grows as (1 + alpha)^(y / 127), Eq. (4)):
 *   L[k] = ((1 + alpha)^(k / code_scale) - 1) / alpha,
 * evaluated in binary64 and rounded once to binary32. */
float oracle_level(int k, float alpha, float code_scale)
{
    double e = ((double)k / (double)code_scale) * log1p((double)alpha);
    return (float)(expm1(e) / (double)alpha);
}

/* ------------------------------------------------------------ Stage 4 -- */

/* Split-stream construction of one clipped code I with sign S (Algorithm
 * 1, Stage 4), for a anchor bits and b residual bits:
 *   I_bias = I + 2^(b-1) - 1;  V_mag = I_bias >> b;  V_recon = V_mag << b;
 *   Q_res = V_recon - I;  Q_anc = V_mag * S + min(S, 0).
 * The paper's split (a = b = 4) has the bias +7; a single stream (b = 0)
 * has no bias, V_mag = I and Q_res = 0. */
void oracle_split_bits(int code, int sign, int anchor_bits, int residual_bits, int *v_mag,
                       int *q_res, int *q_anc)
{
    (void)anchor_bits;
    int b = residual_bits;
    int i_bias = code + (b > 0 ? (1 << (b - 1)) - 1 : 0);
    int v = i_bias >> b;
    int v_recon = v << b;
    *v_mag = v;
    *q_res = v_recon - code;
    *q_anc = v * sign + (sign < 0 ? sign : 0);
}

void oracle_split(int code, int sign, int *v_mag, int *q_res, int *q_anc)
{
    oracle_split_bits(code, sign, 4, 4, v_mag, q_res, q_anc);
}

/* Inverse of the split: the code that the decoder rebuilds from an anchor
 * nibble alone (V << 4) or from anchor and residual ((V << 4) - Q_res),
 * plus the sign carried by the anchor.  Codes below 0 (only reachable with
 * a residual the quantizer never writes) are clamped to 0. */
static int sext(unsigned field, int w)
{
    field &= (1u << w) - 1u;
    return (field >> (w - 1)) & 1u ? (int)field - (1 << w) : (int)field;
}

int oracle_unsplit_bits(unsigned anc_field, int have_res, unsigned res_field,
                        int anchor_bits, int residual_bits, int *sign)
{
    int b = residual_bits;
    int a = sext(anc_field, anchor_bits);
    int s = a < 0 ? -1 : 1;
    int v = a < 0 ? -a - 1 : a;
    int code = v << b;
    if (have_res && b > 0)
        code -= sext(res_field, b);
    if (code < 0)
        code = 0;
    *sign = s;
    return code;
}

int oracle_unsplit(unsigned anc_nib, int have_res, unsigned res_nib, int *sign)
{
    return oracle_unsplit_bits(anc_nib, have_res, res_nib, 4, 4, sign);
}

/* Bit stream of one (chunk, channel pair) run: field f of width w at bit
 * pos, LSB first, byte by byte (the run starts zeroed). */
static void put_bits(uint8_t *run, int pos, int w, unsigned f)
{
    for (int k = 0; k < w; ++k)
        if ((f >> k) & 1u)
            run[(pos + k) >> 3] |= (uint8_t)(1u << ((pos + k) & 7));
}

static unsigned get_bits(const uint8_t *run, int pos, int w)
{
    unsigned f = 0;
    for (int k = 0; k < w; ++k)
        f |= (unsigned)((run[(pos + k) >> 3] >> ((pos + k) & 7)) & 1u) << k;
    return f;
}

/* Bytes of one (chunk, channel pair) run of w-bit fields: 2 C values. */
static int run_bytes(int C, int w) { return C * w / 4; }

/* ------------------------------------------------------------- Stage 2 -- */

/* Balanced pairwise tree sum of n (a power of two) values:
 * sum(a[0..n)) = sum(a[0..n/2)) + sum(a[n/2..n)). */
static float tree_sum(const float *a, int n)
{
    if (n == 1)
        return a[0];
    return tree_sum(a, n / 2) + tree_sum(a + n / 2, n / 2);
}

static int is_pow2(int n) { return n > 0 && (n & (n - 1)) == 0; }

/* ------------------------------------------------------- one page block -- */

/*
 * Quantize one page block X in R^{H x P} stored token-major: element
 * (channel c, token t) is x[t * row_stride + c] (bfloat16 bits).
 *
 * Outputs (all caller-owned):
 *   anchor, residual : P * H * a / 8 and P * H * (8 - a) / 8 bytes
 *                      (chunk-tiled bit streams, see header; P * H / 2 each
 *                      for the paper's a = 4);
 *   gamma_min, gamma_scale : H floats;
 *   mu, sigma : (P/C) x H floats, chunk-major ([chunk][channel]).
 * Optional intermediates (NULL to skip), each H x P, channel-major
 * ([c * P + t]):
 *   xn (Stage 1 output), xcent, xfinal (Stage 2), code_raw (Round(Y) before
 *   the clip), sign (+1 / -1).
 */
int oracle_quantize_block_bits(const uint16_t *x, int64_t row_stride, int H,
                               int P, int C, float alpha, float eps,
                               float code_scale, int anchor_bits, int residual_bits,
                               int meta_bits, uint8_t *anchor, uint8_t *residual,
                               float *gamma_min, float *gamma_scale, float *mu,
                               float *sigma, float *xn_out, float *xcent_out,
                               float *xfinal_out, int32_t *code_raw_out,
                               int8_t *sign_out)
{
    if (H <= 0 || (H & 1) || P <= 0 || !is_pow2(C) || P % C || C % 4 ||
        !valid_bits(anchor_bits, residual_bits) || (residual_bits > 0 && !residual) ||
        (meta_bits != 32 && meta_bits != 16))
        return ORACLE_EINVAL;
    const int code_max = oracle_code_max(anchor_bits, residual_bits);
    const int m16 = meta_bits == 16;
    const int nchunk = P / C;
    float *xn = (float *)malloc(sizeof(float) * (size_t)P);
    float *xc = (float *)malloc(sizeof(float) * (size_t)P);
    int8_t *qa = (int8_t *)malloc((size_t)H * (size_t)P);
    int8_t *qr = (int8_t *)malloc((size_t)H * (size_t)P);
    if (!xn || !xc || !qa || !qr) {
        free(xn); free(xc); free(qa); free(qr);
        return ORACLE_EINVAL;
    }

    for (int c = 0; c < H; ++c) {
        /* Stage 1: per-channel, page-level normalisation. */
        float mn = bf16_to_f32(x[c]);
        float mx = mn;
        for (int t = 1; t < P; ++t) {
            float v = bf16_to_f32(x[(int64_t)t * row_stride + c]);
            if (v < mn) mn = v;
            if (v > mx) mx = v;
        }
        mn = mn + 0.0f;
        float gscale = (mx - mn) + 0.0f;
        if (m16)
            gscale = bf16_ceil_nonneg(gscale);
        float d1 = gscale + eps;
        gamma_min[c] = mn;
        gamma_scale[c] = gscale;
        for (int t = 0; t < P; ++t) {
            float v = bf16_to_f32(x[(int64_t)t * row_stride + c]);
            float num = v - mn;
            xn[t] = num / d1;
        }

        /* Stage 2: per-channel, chunk-wise isolation. */
        for (int j = 0; j < nchunk; ++j) {
            const float *blk = xn + j * C;
            float m = tree_sum(blk, C) / (float)C + 0.0f;
            if (m16)
                m = bf16_nearest(m);
            float sg = 0.0f;
            for (int i = 0; i < C; ++i) {
                xc[j * C + i] = blk[i] - m;
                float a = fabsf(xc[j * C + i]);
                if (a > sg) sg = a;
            }
            if (m16)
                sg = bf16_ceil_nonneg(sg);
            mu[j * H + c] = m;
            sigma[j * H + c] = sg;
            float d2 = sg + eps;

            /* Stages 3 and 4 for every element of the chunk. */
            for (int i = 0; i < C; ++i) {
                int t = j * C + i;
                float xf = xc[t] / d2;
                int code = oracle_code(fabsf(xf), alpha, code_scale);
                int s = xc[t] < 0.0f ? -1 : 1;
                int code_c = code < code_max ? code : code_max;
                int v, q_res, q_anc;
                oracle_split_bits(code_c, s, anchor_bits, residual_bits, &v, &q_res,
                                  &q_anc);
                qa[(size_t)t * H + c] = (int8_t)q_anc;
                qr[(size_t)t * H + c] = (int8_t)q_res;
                if (xfinal_out) xfinal_out[(size_t)c * P + t] = xf;
                if (code_raw_out) code_raw_out[(size_t)c * P + t] = code;
                if (sign_out) sign_out[(size_t)c * P + t] = (int8_t)s;
            }
        }
        if (xn_out)
            memcpy(xn_out + (size_t)c * P, xn, sizeof(float) * (size_t)P);
        if (xcent_out)
            memcpy(xcent_out + (size_t)c * P, xc, sizeof(float) * (size_t)P);
    }

    /* Packing: two's-complement fields, chunk-tiled bit streams: for chunk
     * j and channel pair k the run of w-bit fields starts at byte
     * (j * (H / 2) + k) * C * w / 4; token i of the chunk and channel
     * 2k + e is field 2 i + e.  (For w = 4: byte i of the run, channel 2k
     * in the low nibble.) */
    const int wa = anchor_bits, wr = residual_bits;
    memset(anchor, 0, (size_t)P * H * wa / 8);
    if (wr > 0)
        memset(residual, 0, (size_t)P * H * wr / 8);
    for (int t = 0; t < P; ++t) {
        const int j = t / C, i = t % C;
        for (int k = 0; k < H / 2; ++k) {
            uint8_t *ra = anchor + ((size_t)j * (H / 2) + k) * run_bytes(C, wa);
            for (int e = 0; e < 2; ++e) {
                const int v = 2 * i + e;
                put_bits(ra, wa * v, wa, (unsigned)qa[(size_t)t * H + 2 * k + e]);
                if (wr > 0)
                    put_bits(residual + ((size_t)j * (H / 2) + k) * run_bytes(C, wr), wr * v,
                             wr, (unsigned)qr[(size_t)t * H + 2 * k + e]);
            }
        }
    }
    free(xn); free(xc); free(qa); free(qr);
    return ORACLE_OK;
}

int oracle_quantize_block_ex(const uint16_t *x, int64_t row_stride, int H,
                             int P, int C, float alpha, float eps,
                             float code_scale, uint8_t *anchor,
                             uint8_t *residual, float *gamma_min,
                             float *gamma_scale, float *mu, float *sigma,
                             float *xn_out, float *xcent_out,
                             float *xfinal_out, int32_t *code_raw_out,
                             int8_t *sign_out)
{
    return oracle_quantize_block_bits(x, row_stride, H, P, C, alpha, eps, code_scale, 4, 4,
                                      32, anchor, residual, gamma_min, gamma_scale, mu, sigma,
                                      xn_out, xcent_out, xfinal_out, code_raw_out, sign_out);
}

/*
 * Dequantize one page block.  residual == NULL gives the anchor-only
 * (draft) reconstruction; otherwise anchor + residual (verification
 * precision).  out is token-major bf16 with row stride out_row_stride.
 *   x^_f = S * L[code];  x^_n = x^_f * (sigma + eps) + mu;
 *   x^ = x^_n * (gamma_scale + eps) + gamma_min;  out = bf16_rne(x^).
 */
int oracle_dequant_block_bits(const uint8_t *anchor, const uint8_t *residual,
                              const float *gamma_min, const float *gamma_scale,
                              const float *mu, const float *sigma, int H, int P,
                              int C, float alpha, float eps, float code_scale,
                              int anchor_bits, int residual_bits, uint16_t *out,
                              int64_t out_row_stride)
{
    if (H <= 0 || (H & 1) || P <= 0 || C <= 0 || P % C || C % 4 ||
        !valid_bits(anchor_bits, residual_bits) || (residual_bits == 0 && residual))
        return ORACLE_EINVAL;
    const int wa = anchor_bits, wr = residual_bits;
    float lut[128];
    for (int k = 0; k < 128; ++k)
        lut[k] = oracle_level(k, alpha, code_scale);
    for (int t = 0; t < P; ++t) {
        int j = t / C;
        for (int c = 0; c < H; ++c) {
            const size_t run = (size_t)j * (H / 2) + c / 2;
            const int v = 2 * (t % C) + (c & 1);
            unsigned an = get_bits(anchor + run * run_bytes(C, wa), wa * v, wa);
            unsigned rn = 0;
            if (residual)
                rn = get_bits(residual + run * run_bytes(C, wr), wr * v, wr);
            int s;
            int code = oracle_unsplit_bits(an, residual != NULL, rn, anchor_bits,
                                           residual_bits, &s);
            float m = lut[code];
            float xf = s < 0 ? -m : m;
            float d2 = sigma[j * H + c] + eps;
            float d1 = gamma_scale[c] + eps;
            float t1 = xf * d2;
            float xnv = t1 + mu[j * H + c];
            float t2 = xnv * d1;
            float xv = t2 + gamma_min[c];
            out[(int64_t)t * out_row_stride + c] = f32_to_bf16_rne(xv);
        }
    }
    return ORACLE_OK;
}

int oracle_dequant_block(const uint8_t *anchor, const uint8_t *residual,
                         const float *gamma_min, const float *gamma_scale,
                         const float *mu, const float *sigma, int H, int P,
                         int C, float alpha, float eps, float code_scale,
                         uint16_t *out, int64_t out_row_stride)
{
    return oracle_dequant_block_bits(anchor, residual, gamma_min, gamma_scale, mu, sigma, H,
                                     P, C, alpha, eps, code_scale, 4, 4, out, out_row_stride);
}

/* ------------------------------------------------------- whole tensors -- */

/*
 * A KV set is num_tensors token-major tensors [T][Ch] (tensor k starts at
 * element k * tensor_stride, token rows row_stride elements apart).  It is
 * cut into page blocks of H channels x P tokens, numbered
 *   b = ((tensor * (T / P)) + page) * (Ch / H) + channel_group.
 * Only blocks [block_begin, block_end) are computed (so several threads
 * can share one call's outputs).  The code and metadata arrays hold blocks
 * from out_first_block on: block b's anchor and residual are bytes
 * [(b - out_first_block) * P * H / 2, ...), its gamma_* floats
 * [(b - out_first_block) * H, ...), its mu / sigma floats
 * [(b - out_first_block) * (P/C) * H, ...).
 */
static int block_geometry(int64_t b, int64_t T, int64_t Ch, int H, int P,
                          int64_t *tensor, int64_t *page, int64_t *group)
{
    int64_t groups = Ch / H, pages = T / P;
    *group = b % groups;
    *page = (b / groups) % pages;
    *tensor = b / (groups * pages);
    return 0;
}

int oracle_quantize_bits(const uint16_t *kv, int64_t num_tensors,
                         int64_t tensor_stride, int64_t T, int64_t Ch,
                         int64_t row_stride, int H, int P, int C, float alpha,
                         float eps, float code_scale, int anchor_bits,
                         int residual_bits, int meta_bits, int64_t block_begin,
                         int64_t block_end, int64_t out_first_block, uint8_t *anchor,
                         uint8_t *residual, float *gamma_min,
                         float *gamma_scale, float *mu, float *sigma)
{
    if (!valid_bits(anchor_bits, residual_bits))
        return ORACLE_EINVAL;
    if (T % P || Ch % H || num_tensors < 0)
        return ORACLE_EINVAL;
    const int64_t nblocks = num_tensors * (T / P) * (Ch / H);
    if (block_begin < 0 || block_end > nblocks || block_begin > block_end ||
        out_first_block > block_begin)
        return ORACLE_EINVAL;
    const int64_t anchor_bytes = (int64_t)P * H * anchor_bits / 8;
    const int64_t residual_bytes = (int64_t)P * H * residual_bits / 8;
    const int64_t chunk_meta = (int64_t)(P / C) * H;
    for (int64_t b = block_begin; b < block_end; ++b) {
        int64_t tensor, page, group;
        block_geometry(b, T, Ch, H, P, &tensor, &page, &group);
        const uint16_t *x = kv + tensor * tensor_stride +
                            page * P * row_stride + group * H;
        const int64_t o = b - out_first_block;
        int rc = oracle_quantize_block_bits(
            x, row_stride, H, P, C, alpha, eps, code_scale, anchor_bits, residual_bits,
            meta_bits, anchor + o * anchor_bytes, residual ? residual + o * residual_bytes : NULL,
            gamma_min + o * H, gamma_scale + o * H, mu + o * chunk_meta,
            sigma + o * chunk_meta, NULL, NULL, NULL, NULL, NULL);
        if (rc)
            return rc;
    }
    return ORACLE_OK;
}

int oracle_quantize(const uint16_t *kv, int64_t num_tensors,
                    int64_t tensor_stride, int64_t T, int64_t Ch,
                    int64_t row_stride, int H, int P, int C, float alpha,
                    float eps, float code_scale, int64_t block_begin,
                    int64_t block_end, int64_t out_first_block,
                    uint8_t *anchor, uint8_t *residual,
                    float *gamma_min, float *gamma_scale, float *mu,
                    float *sigma)
{
    return oracle_quantize_bits(kv, num_tensors, tensor_stride, T, Ch, row_stride, H, P, C,
                                alpha, eps, code_scale, 4, 4, 32, block_begin, block_end,
                                out_first_block, anchor, residual, gamma_min, gamma_scale,
                                mu, sigma);
}

int oracle_dequant_bits(const uint8_t *anchor, const uint8_t *residual,
                        const float *gamma_min, const float *gamma_scale,
                        const float *mu, const float *sigma, int64_t num_tensors,
                        int64_t tensor_stride, int64_t T, int64_t Ch,
                        int64_t row_stride, int H, int P, int C, float alpha,
                        float eps, float code_scale, int anchor_bits,
                        int residual_bits, int64_t block_begin, int64_t block_end,
                        int64_t in_first_block, uint16_t *out)
{
    if (!valid_bits(anchor_bits, residual_bits))
        return ORACLE_EINVAL;
    if (T % P || Ch % H || num_tensors < 0)
        return ORACLE_EINVAL;
    const int64_t nblocks = num_tensors * (T / P) * (Ch / H);
    if (block_begin < 0 || block_end > nblocks || block_begin > block_end ||
        in_first_block > block_begin)
        return ORACLE_EINVAL;
    const int64_t anchor_bytes = (int64_t)P * H * anchor_bits / 8;
    const int64_t residual_bytes = (int64_t)P * H * residual_bits / 8;
    const int64_t chunk_meta = (int64_t)(P / C) * H;
    for (int64_t b = block_begin; b < block_end; ++b) {
        int64_t tensor, page, group;
        block_geometry(b, T, Ch, H, P, &tensor, &page, &group);
        uint16_t *o = out + tensor * tensor_stride + page * P * row_stride +
                      group * H;
        const int64_t i = b - in_first_block;
        int rc = oracle_dequant_block_bits(
            anchor + i * anchor_bytes, residual ? residual + i * residual_bytes : NULL,
            gamma_min + i * H, gamma_scale + i * H, mu + i * chunk_meta,
            sigma + i * chunk_meta, H, P, C, alpha, eps, code_scale, anchor_bits,
            residual_bits, o, row_stride);
        if (rc)
            return rc;
    }
    return ORACLE_OK;
}

int oracle_dequant(const uint8_t *anchor, const uint8_t *residual,
                   const float *gamma_min, const float *gamma_scale,
                   const float *mu, const float *sigma, int64_t num_tensors,
                   int64_t tensor_stride, int64_t T, int64_t Ch,
                   int64_t row_stride, int H, int P, int C, float alpha,
                   float eps, float code_scale, int64_t block_begin,
                   int64_t block_end, int64_t in_first_block, uint16_t *out)
{
    return oracle_dequant_bits(anchor, residual, gamma_min, gamma_scale, mu, sigma,
                               num_tensors, tensor_stride, T, Ch, row_stride, H, P, C, alpha,
                               eps, code_scale, 4, 4, block_begin, block_end, in_first_block,
                               out);
}

/* ----------------------------------------------------------- attention -- */

/*
 * Scaled dot-product attention O = softmax(Q K^T * scale) V (Lynx paper,
 * Section 2.1) over reconstructed bf16 K^, V^, in binary64.
 *   q   : [t_q][n_qh][d] bf16,   k, v : [ctx][n_kvh][d] bf16 (token-major),
 *   out : [t_q][n_qh][d] binary64.
 * Query head h reads KV head h / (n_qh / n_kvh) (grouped-query attention).
 * With causal_tail set, the t_q queries are the last t_q positions of the
 * context and query row r sees positions 0 .. ctx - t_q + r.
 * Only query heads [h_begin, h_end) are computed.
 */
int oracle_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     int t_q, int n_qh, int n_kvh, int d, int64_t ctx,
                     double scale, int causal_tail, int h_begin, int h_end,
                     double *out)
{
    if (t_q <= 0 || n_qh <= 0 || n_kvh <= 0 || n_qh % n_kvh || d <= 0 ||
        ctx <= 0 || (causal_tail && ctx < t_q))
        return ORACLE_EINVAL;
    const int group = n_qh / n_kvh;
    double *s = (double *)malloc(sizeof(double) * (size_t)ctx);
    double *qv = (double *)malloc(sizeof(double) * (size_t)d);
    if (!s || !qv) {
        free(s); free(qv);
        return ORACLE_EINVAL;
    }
    for (int r = 0; r < t_q; ++r) {
        int64_t visible = causal_tail ? ctx - t_q + r + 1 : ctx;
        for (int h = h_begin; h < h_end; ++h) {
            int kh = h / group;
            for (int i = 0; i < d; ++i)
                qv[i] = bf16_to_f32(q[((size_t)r * n_qh + h) * d + i]);
            double mx = -INFINITY;
            for (int64_t p = 0; p < visible; ++p) {
                const uint16_t *kr = k + ((size_t)p * n_kvh + kh) * d;
                double acc = 0.0;
                for (int i = 0; i < d; ++i)
                    acc += qv[i] * (double)bf16_to_f32(kr[i]);
                s[p] = acc * scale;
                if (s[p] > mx) mx = s[p];
            }
            double den = 0.0;
            for (int64_t p = 0; p < visible; ++p) {
                s[p] = exp(s[p] - mx);
                den += s[p];
            }
            double *o = out + ((size_t)r * n_qh + h) * d;
            for (int i = 0; i < d; ++i)
                o[i] = 0.0;
            for (int64_t p = 0; p < visible; ++p) {
                const uint16_t *vr = v + ((size_t)p * n_kvh + kh) * d;
                double w = s[p] / den;
                for (int i = 0; i < d; ++i)
                    o[i] += w * (double)bf16_to_f32(vr[i]);
            }
        }
    }
    free(s);
    free(qv);
    return ORACLE_OK;
}

/* ----------------------------------------------- speculative verification -- */

/*
 * Verification of T draft tokens (Lynx paper, Section 4.3: the drafts made
 * on the Anchor-only cache are checked in one forward pass on the full
 * cache; the notes' "推测验证与无损纠错", Eq. (10) and Eq. (11)).
 *   draft_logits  : [T][V] binary32, the logits the drafts were drawn from
 *                   (q_t = softmax of row t);
 *   target_logits : [T + 1][V] binary32, the full-precision logits (p_t);
 *   tokens        : [T] the draft tokens s_t;
 *   u_accept      : [T] uniforms in [0, 1); u_sample: one uniform in [0, 1).
 * Token t is accepted when u_t < p_t(s_t) / q_t(s_t) (probability
 * min(1, p/q), Eq. 10); the first rejection at position k stops the scan and
 * the next token is drawn from max(0, p_k - q_k) (Eq. 11) by inverse CDF:
 * the smallest x with sum_{y <= x} r(y) > u_sample * sum_y r(y).  If every
 * draft is accepted, the next token is drawn from p_T the same way (the
 * standard speculative sampling step the paper adopts).  Softmaxes, ratios
 * and sums in binary64, sums in increasing token order.
 * Writes *n_accepted (0..T) and *token.
 */
static void softmax_row(const float *l, int V, double *out)
{
    double mx = -INFINITY, den = 0.0;
    for (int i = 0; i < V; ++i)
        if ((double)l[i] > mx) mx = (double)l[i];
    for (int i = 0; i < V; ++i) {
        out[i] = exp((double)l[i] - mx);
        den += out[i];
    }
    for (int i = 0; i < V; ++i)
        out[i] /= den;
}

static int sample_inverse_cdf(const double *w, int V, double u)
{
    double total = 0.0;
    for (int i = 0; i < V; ++i)
        total += w[i];
    const double target = u * total;
    double run = 0.0;
    int last = -1;
    for (int i = 0; i < V; ++i) {
        if (w[i] > 0.0)
            last = i;
        run += w[i];
        if (run > target)
            return i;
    }
    return last;  /* rounding left target at the very top: last positive entry */
}

int oracle_spec_verify(const float *draft_logits, const float *target_logits,
                       const int32_t *tokens, const double *u_accept, double u_sample,
                       int T, int V, int32_t *n_accepted, int32_t *token)
{
    if (T < 0 || V <= 0)
        return ORACLE_EINVAL;
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    double *q = (double *)malloc(sizeof(double) * (size_t)V);
    if (!p || !q) {
        free(p); free(q);
        return ORACLE_EINVAL;
    }
    int k = 0;
    for (; k < T; ++k) {
        const int32_t s = tokens[k];
        if (s < 0 || s >= V) {
            free(p); free(q);
            return ORACLE_EINVAL;
        }
        softmax_row(target_logits + (size_t)k * V, V, p);
        softmax_row(draft_logits + (size_t)k * V, V, q);
        if (!(u_accept[k] < p[s] / q[s]))
            break;
    }
    *n_accepted = k;
    if (k < T) {
        /* p, q hold row k: residual distribution max(0, p - q) */
        for (int i = 0; i < V; ++i)
            p[i] = p[i] > q[i] ? p[i] - q[i] : 0.0;
        *token = sample_inverse_cdf(p, V, u_sample);
    } else {
        softmax_row(target_logits + (size_t)T * V, V, p);
        *token = sample_inverse_cdf(p, V, u_sample);
    }
    free(p);
    free(q);
    return ORACLE_OK;
}
