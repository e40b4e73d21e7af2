/*
 * The library's C ABI used from plain C (no Python, no torch): quantize a
 * small KV set on the GPU, rebuild it from the anchor alone and from anchor +
 * residual, and compare everything with the CPU oracle bit for bit (codes and
 * bf16 outputs byte for byte, metadata by IEEE ==).  Also checks that bad
 * arguments are refused before any launch.
 *
 * TEST INFRASTRUCTURE: links the oracle's library; built by the repository's
 * build step, run by tests/test_gpu_c_abi.py.  Prints "c-abi parity ok" and
 * exits 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lynx.h"

/* oracle/lynx_oracle.c */
int oracle_quantize_bits(const uint16_t *kv, int64_t num_tensors, int64_t tensor_stride,
                         int64_t T, int64_t Ch, int64_t row_stride, int H, int P, int C,
                         float alpha, float eps, float code_scale, int anchor_bits,
                         int residual_bits, int meta_bits, int64_t block_begin,
                         int64_t block_end, int64_t out_first_block, uint8_t *anchor,
                         uint8_t *residual, float *gamma_min, float *gamma_scale, float *mu,
                         float *sigma);
int oracle_dequant_bits(const uint8_t *anchor, const uint8_t *residual,
                        const float *gamma_min, const float *gamma_scale, const float *mu,
                        const float *sigma, int64_t num_tensors, int64_t tensor_stride,
                        int64_t T, int64_t Ch, int64_t row_stride, int H, int P, int C,
                        float alpha, float eps, float code_scale, int anchor_bits,
                        int residual_bits, int64_t block_begin, int64_t block_end,
                        int64_t in_first_block, uint16_t *out);

#define CHECK(cond, ...)                                                                     \
    do {                                                                                     \
        if (!(cond)) {                                                                       \
            fprintf(stderr, "c-abi: " __VA_ARGS__);                                          \
            fprintf(stderr, "\n");                                                           \
            exit(1);                                                                         \
        }                                                                                    \
    } while (0)
#define HIP(x) CHECK((x) == hipSuccess, "%s failed", #x)

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static double uniform(void) /* xorshift64*, (0, 1) */
{
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return ((rng * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0) + 1e-17;
}

static uint16_t bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static void *dev(size_t bytes)
{
    void *p = NULL;
    HIP(hipMalloc(&p, bytes));
    return p;
}

int main(void)
{
    /* 2 tensors x 512 tokens x 256 channels: 8 page blocks; per-channel
     * offset and scale, Laplacian values, one outlier channel x100 */
    const int64_t NT = 2, T = 512, CH = 256;
    const int64_t n = NT * T * CH, nb = n / (256 * 128);
    uint16_t *kv = malloc(n * 2);
    for (int64_t t = 0; t < NT; ++t)
        for (int64_t c = 0; c < CH; ++c) {
            const double off = 4.0 * uniform() - 2.0, sc = exp(0.5 * (uniform() - 0.5));
            for (int64_t i = 0; i < T; ++i) {
                const double u = uniform() - 0.5;
                double x = off + sc * (u < 0 ? log(1 + 2 * u) : -log(1 - 2 * u));
                if (c == 37)
                    x *= 100.0;
                kv[(t * T + i) * CH + c] = bf16_rne((float)x);
            }
        }

    lynx_kv_shape shape = {NT, T * CH, T, CH, CH};
    CHECK(lynx_num_blocks(&shape) == nb, "block count");
    const size_t sb = lynx_stream_bytes(&shape), gf = lynx_gamma_floats(&shape),
                 cf = lynx_chunk_floats(&shape);
    CHECK(sb == (size_t)nb * 16384 && gf == (size_t)nb * 128 && cf == (size_t)nb * 1024,
          "buffer sizes");
    lynx_params p;
    lynx_default_params(&p);

    void *d_kv = dev(n * 2), *d_oa = dev(n * 2), *d_of = dev(n * 2);
    uint8_t *d_anc = dev(sb), *d_res = dev(sb);
    lynx_meta m = {dev(gf * 4), dev(gf * 4), dev(cf * 4), dev(cf * 4)};
    HIP(hipMemcpy(d_kv, kv, n * 2, hipMemcpyHostToDevice));

    /* refused before any launch */
    CHECK(lynx_quantize_pages(NULL, &shape, &p, d_anc, d_res, m, NULL) == LYNX_EINVAL,
          "null input accepted");
    lynx_kv_shape ragged = {NT, T * CH, T - 16, CH, CH};
    CHECK(lynx_quantize_pages(d_kv, &ragged, &p, d_anc, d_res, m, NULL) == LYNX_ESHAPE,
          "ragged page accepted");
    CHECK(lynx_status_string(LYNX_EINVAL) != NULL, "status text");

    CHECK(lynx_quantize_pages(d_kv, &shape, &p, d_anc, d_res, m, NULL) == LYNX_OK, "quantize");
    CHECK(lynx_dequant_anchor(d_anc, m, &shape, &p, d_oa, NULL) == LYNX_OK, "anchor dequant");
    CHECK(lynx_dequant_full(d_anc, d_res, m, &shape, &p, d_of, NULL) == LYNX_OK,
          "full dequant");
    HIP(hipDeviceSynchronize());

    uint8_t *anc = malloc(sb), *res = malloc(sb), *ranc = malloc(sb), *rres = malloc(sb);
    float *meta = malloc((gf * 2 + cf * 2) * 4), *rmeta = malloc((gf * 2 + cf * 2) * 4);
    uint16_t *oa = malloc(n * 2), *of = malloc(n * 2), *roa = calloc(n, 2), *rof = calloc(n, 2);
    HIP(hipMemcpy(anc, d_anc, sb, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(res, d_res, sb, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(meta, m.gamma_min, gf * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(meta + gf, m.gamma_scale, gf * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(meta + 2 * gf, m.mu, cf * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(meta + 2 * gf + cf, m.sigma, cf * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(oa, d_oa, n * 2, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(of, d_of, n * 2, hipMemcpyDeviceToHost));

    CHECK(oracle_quantize_bits(kv, NT, T * CH, T, CH, CH, 128, 256, 32, p.alpha, p.eps,
                               p.code_scale, 4, 4, 32, 0, nb, 0, ranc, rres, rmeta,
                               rmeta + gf, rmeta + 2 * gf, rmeta + 2 * gf + cf) == 0,
          "oracle quantize");
    CHECK(memcmp(anc, ranc, sb) == 0, "anchor stream differs from the oracle");
    CHECK(memcmp(res, rres, sb) == 0, "residual stream differs from the oracle");
    for (size_t i = 0; i < gf * 2 + cf * 2; ++i)
        CHECK(meta[i] == rmeta[i], "metadata %zu differs: %a vs %a", i, meta[i], rmeta[i]);
    CHECK(oracle_dequant_bits(ranc, NULL, rmeta, rmeta + gf, rmeta + 2 * gf,
                              rmeta + 2 * gf + cf, NT, T * CH, T, CH, CH, 128, 256, 32,
                              p.alpha, p.eps, p.code_scale, 4, 4, 0, nb, 0, roa) == 0,
          "oracle anchor dequant");
    CHECK(oracle_dequant_bits(ranc, rres, rmeta, rmeta + gf, rmeta + 2 * gf,
                              rmeta + 2 * gf + cf, NT, T * CH, T, CH, CH, 128, 256, 32,
                              p.alpha, p.eps, p.code_scale, 4, 4, 0, nb, 0, rof) == 0,
          "oracle full dequant");
    CHECK(memcmp(oa, roa, n * 2) == 0, "anchor-only reconstruction differs from the oracle");
    CHECK(memcmp(of, rof, n * 2) == 0, "full reconstruction differs from the oracle");

    HIP(hipFree(d_kv));
    HIP(hipFree(d_oa));
    HIP(hipFree(d_of));
    HIP(hipFree(d_anc));
    HIP(hipFree(d_res));
    HIP(hipFree(m.gamma_min));
    HIP(hipFree(m.gamma_scale));
    HIP(hipFree(m.mu));
    HIP(hipFree(m.sigma));
    printf("c-abi parity ok: %lld page blocks, codes, metadata and both reconstructions\n",
           (long long)nb);
    return 0;
}
