// Host side of liblynx.so: argument validation, the compander and level
// tables of Eq. (3) / Eq. (4), and the extern "C" entry points declared in
// include/lynx.h.  The kernels live in lynx_quant.hip and lynx_dequant.hip.
#include "lynx.h"

#include <math.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "lynx_internal.h"

namespace lynx {
namespace {

thread_local std::string g_hip_error;

// Largest launch (in blocks) of one kernel dispatch: the grid size in
// work-items (blocks x 512) must stay below 2^32.
constexpr int64_t kMaxLaunchBlocks = int64_t(1) << 22;

uint32_t f2u(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}
float u2f(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}

// ---------------------------------------------------------------- tables --

// Y(x) of Eq. (3) in x87 extended precision.
long double eq3(float x, long double alpha, long double cs, long double l1pa) {
    return cs * log1pl(alpha * (long double)x) / l1pa;
}

// Thresholds of the rounding boundaries Y = k - 1/2 as the smallest binary32
// magnitudes that reach them, then the bucket table (at most one threshold
// per bucket of 2^shift consecutive bit patterns).  Returns false if no
// bucket width up to 8 mantissa bits fits kMaxBuckets.
bool build_quant_tab(float alpha, float code_scale, QuantTab *t) {
    memset(t, 0, sizeof *t);
    const long double a = alpha, cs = code_scale, l1pa = log1pl(a);
    t->thr[0] = 0.0f;
    for (int k = 1; k < 128; ++k) {
        if (k > kCodeMax) {
            t->thr[k] = INFINITY;
            continue;
        }
        const long double target = (long double)k - 0.5L;
        long double tau = expm1l(target / cs * l1pa) / a;
        if (!(tau <= 1.0L)) {  // boundary beyond |x| = 1: never reached
            t->thr[k] = INFINITY;
            continue;
        }
        float x = (float)tau;
        while (eq3(x, a, cs, l1pa) < target) x = nextafterf(x, INFINITY);
        while (x > 0.0f && eq3(nextafterf(x, 0.0f), a, cs, l1pa) >= target)
            x = nextafterf(x, 0.0f);
        if (x > 1.0f)
            x = INFINITY;
        t->thr[k] = x;
    }
    auto code_of = [&](uint32_t bits) {
        int c = 0;
        for (int k = 1; k < 128; ++k)
            if (f2u(t->thr[k]) <= bits)
                c = k;
        return c;
    };
    const uint32_t one = f2u(1.0f);
    for (int mbits = 3; mbits <= 8; ++mbits) {
        const int shift = 23 - mbits;
        const uint32_t lo = (f2u(t->thr[1]) - 1u) >> shift;
        const uint32_t hi = one >> shift;
        const uint32_t n = hi - lo + 1u;
        if (n > (uint32_t)kMaxBuckets)
            continue;
        bool ok = true;
        for (uint32_t bk = lo; bk <= hi && ok; ++bk) {
            uint32_t first = bk << shift;
            uint32_t last = ((bk + 1u) << shift) - 1u;
            if (last > one)
                last = one;
            int c0 = code_of(first), c1 = code_of(last);
            if (c1 > c0 + 1)
                ok = false;
            t->bucket_code[bk - lo] = (uint8_t)c0;
        }
        if (ok) {
            t->bucket_lo = (int32_t)lo;
            t->nbuckets = (int32_t)n;
            t->shift = shift;
            return true;
        }
    }
    return false;
}

void build_dequant_tab(float alpha, float code_scale, DequantTab *t) {
    const double l1pa = log1p((double)alpha);
    for (int k = 0; k < 128; ++k)
        t->level[k] = (float)(expm1((double)k / (double)code_scale * l1pa) / (double)alpha);
}

struct Tables {
    QuantTab q;
    DequantTab d;
};

std::mutex g_mu;
std::map<std::pair<uint32_t, uint32_t>, Tables> g_cache;

const Tables *tables_for(const lynx_params &p) {
    std::lock_guard<std::mutex> lock(g_mu);
    auto key = std::make_pair(f2u(p.alpha), f2u(p.code_scale));
    auto it = g_cache.find(key);
    if (it != g_cache.end())
        return &it->second;
    Tables t;
    if (!build_quant_tab(p.alpha, p.code_scale, &t.q))
        return nullptr;
    build_dequant_tab(p.alpha, p.code_scale, &t.d);
    return &g_cache.emplace(key, t).first->second;
}

// ------------------------------------------------------------ validation --

lynx_params resolve(const lynx_params *p) {
    lynx_params d;
    lynx_default_params(&d);
    return p ? *p : d;
}

int check_params(const lynx_params &p) {
    if (p.page_tokens != kPage || p.chunk_tokens != kChunk || p.block_channels != kHead)
        return LYNX_EINVAL;
    if (!(p.alpha > 0.0f) || !(p.alpha <= 1e12f))
        return LYNX_EINVAL;
    if (!(p.eps >= 0x1p-40f) || !(p.eps <= 0x1p-8f))
        return LYNX_EINVAL;
    if (!(p.code_scale >= 1.0f) || !(p.code_scale <= 127.0f))
        return LYNX_EINVAL;
    return LYNX_OK;
}

int check_shape(const lynx_kv_shape *s, int64_t *nblocks) {
    if (!s)
        return LYNX_EINVAL;
    if (s->num_tensors < 0 || s->num_tokens < 0 || s->num_channels < 0 || s->row_stride < 0 ||
        s->tensor_stride < 0)
        return LYNX_EINVAL;
    if (s->num_tokens % kPage || s->num_channels % kHead)
        return LYNX_ESHAPE;
    if (s->row_stride < s->num_channels || s->row_stride % 8)
        return LYNX_ESHAPE;
    if (s->num_tensors > 1 &&
        (s->tensor_stride % 8 || s->tensor_stride < s->num_tokens * s->row_stride))
        return LYNX_ESHAPE;
    const int64_t pages = s->num_tokens / kPage, heads = s->num_channels / kHead;
    if (pages > INT32_MAX || heads > INT32_MAX)
        return LYNX_ESHAPE;
    if (s->num_tensors && pages && heads && s->num_tensors > INT64_MAX / (pages * heads))
        return LYNX_ESHAPE;
    *nblocks = s->num_tensors * pages * heads;
    return LYNX_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

Geometry geometry(const lynx_kv_shape *s, int64_t nblocks) {
    Geometry g;
    g.tensor_stride = s->tensor_stride;
    g.row_stride = s->row_stride;
    g.pages = (int32_t)(s->num_tokens / kPage);
    g.heads = (int32_t)(s->num_channels / kHead);
    g.nblocks = nblocks;
    g.block0 = 0;
    return g;
}

int hip_status(hipError_t e) {
    if (e == hipSuccess)
        return LYNX_OK;
    g_hip_error = hipGetErrorString(e);
    return LYNX_EHIP;
}

int quantize_common(const void *kv, const lynx_kv_shape *shape, const lynx_params *params,
                    uint8_t *anchor, uint8_t *residual, float *gmin, float *gscale, float *mu,
                    float *sigma, int mode, hipStream_t stream) {
    const lynx_params p = resolve(params);
    int rc = check_params(p);
    if (rc)
        return rc;
    int64_t nb = 0;
    if ((rc = check_shape(shape, &nb)))
        return rc;
    if (nb == 0)
        return LYNX_OK;
    if (!kv || !gmin || !gscale)
        return LYNX_EINVAL;
    if (mode != kModePageStats && (!mu || !sigma))
        return LYNX_EINVAL;
    if (mode == kModeQuantize && (!anchor || !residual))
        return LYNX_EINVAL;
    for (const void *ptr : {(const void *)kv, (const void *)gmin, (const void *)gscale,
                            (const void *)mu, (const void *)sigma, (const void *)anchor,
                            (const void *)residual})
        if (ptr && !aligned16(ptr))
            return LYNX_ESHAPE;
    const Tables *t = tables_for(p);
    if (!t)
        return LYNX_EINVAL;
    QuantTab tab = t->q;
    tab.eps = p.eps;
    Geometry g = geometry(shape, nb);
    for (int64_t b0 = 0; b0 < nb; b0 += kMaxLaunchBlocks) {
        g.block0 = b0;
        g.nblocks = (nb - b0) < kMaxLaunchBlocks ? (nb - b0) : kMaxLaunchBlocks;
        rc = hip_status(launch_quantize((const uint16_t *)kv, g, tab, anchor, residual, gmin,
                                        gscale, mu, sigma, mode, stream));
        if (rc)
            return rc;
    }
    return LYNX_OK;
}

int dequant_common(const uint8_t *anchor, const uint8_t *residual, lynx_meta meta,
                   const lynx_kv_shape *shape, const lynx_params *params, void *out,
                   hipStream_t stream) {
    const lynx_params p = resolve(params);
    int rc = check_params(p);
    if (rc)
        return rc;
    int64_t nb = 0;
    if ((rc = check_shape(shape, &nb)))
        return rc;
    if (nb == 0)
        return LYNX_OK;
    if (!anchor || !out || !meta.gamma_min || !meta.gamma_scale || !meta.mu || !meta.sigma)
        return LYNX_EINVAL;
    for (const void *ptr : {(const void *)anchor, (const void *)residual, (const void *)out,
                            (const void *)meta.gamma_min, (const void *)meta.gamma_scale,
                            (const void *)meta.mu, (const void *)meta.sigma})
        if (ptr && !aligned16(ptr))
            return LYNX_ESHAPE;
    const Tables *t = tables_for(p);
    if (!t)
        return LYNX_EINVAL;
    DequantTab tab = t->d;
    tab.eps = p.eps;
    Geometry g = geometry(shape, nb);
    for (int64_t b0 = 0; b0 < nb; b0 += kMaxLaunchBlocks) {
        g.block0 = b0;
        g.nblocks = (nb - b0) < kMaxLaunchBlocks ? (nb - b0) : kMaxLaunchBlocks;
        rc = hip_status(launch_dequant(anchor, residual, meta.gamma_min, meta.gamma_scale,
                                       meta.mu, meta.sigma, g, tab, (uint16_t *)out, stream));
        if (rc)
            return rc;
    }
    return LYNX_OK;
}

}  // namespace
}  // namespace lynx

using namespace lynx;

extern "C" {

void lynx_default_params(lynx_params *p) {
    if (!p)
        return;
    p->alpha = 255.0f;
    p->eps = 1e-6f;
    p->code_scale = 127.0f;
    p->page_tokens = kPage;
    p->chunk_tokens = kChunk;
    p->block_channels = kHead;
}

int64_t lynx_num_blocks(const lynx_kv_shape *shape) {
    int64_t nb = 0;
    int rc = check_shape(shape, &nb);
    return rc ? rc : nb;
}

size_t lynx_stream_bytes(const lynx_kv_shape *shape) {
    int64_t nb = lynx_num_blocks(shape);
    return nb < 0 ? 0 : (size_t)nb * (kPage * kHead / 2);
}

size_t lynx_gamma_floats(const lynx_kv_shape *shape) {
    int64_t nb = lynx_num_blocks(shape);
    return nb < 0 ? 0 : (size_t)nb * kHead;
}

size_t lynx_chunk_floats(const lynx_kv_shape *shape) {
    int64_t nb = lynx_num_blocks(shape);
    return nb < 0 ? 0 : (size_t)nb * kChunks * kHead;
}

uint64_t lynx_kv_bytes(int64_t k_factor, int64_t seq_len, int64_t hidden, int64_t layers,
                       int64_t precision_bytes) {
    const int64_t f[5] = {k_factor, seq_len, hidden, layers, precision_bytes};
    unsigned __int128 acc = 1;
    for (int64_t v : f) {
        if (v < 0)
            return 0;
        acc *= (unsigned __int128)v;
        if (acc > (unsigned __int128)UINT64_MAX)
            return 0;
    }
    return (uint64_t)acc;
}

int lynx_compander_thresholds(const lynx_params *params, float *thr128) {
    const lynx_params p = resolve(params);
    if (!thr128 || check_params(p))
        return LYNX_EINVAL;
    const Tables *t = tables_for(p);
    if (!t)
        return LYNX_EINVAL;
    memcpy(thr128, t->q.thr, sizeof t->q.thr);
    return LYNX_OK;
}

const char *lynx_status_string(int status) {
    switch (status) {
    case LYNX_OK:
        return "ok";
    case LYNX_EINVAL:
        return "invalid argument (null pointer, negative size or unsupported parameter)";
    case LYNX_ESHAPE:
        return "invalid shape (tokens % 256, channels % 128, stride or 16-byte alignment)";
    case LYNX_EHIP:
        return g_hip_error.empty() ? "HIP error" : g_hip_error.c_str();
    default:
        return "unknown status";
    }
}

int lynx_quantize_pages(const void *kv, const lynx_kv_shape *shape, const lynx_params *params,
                        uint8_t *anchor, uint8_t *residual, lynx_meta meta,
                        hipStream_t stream) {
    return quantize_common(kv, shape, params, anchor, residual, meta.gamma_min,
                           meta.gamma_scale, meta.mu, meta.sigma, kModeQuantize, stream);
}

int lynx_dequant_anchor(const uint8_t *anchor, lynx_meta meta, const lynx_kv_shape *shape,
                        const lynx_params *params, void *out, hipStream_t stream) {
    return dequant_common(anchor, nullptr, meta, shape, params, out, stream);
}

int lynx_dequant_full(const uint8_t *anchor, const uint8_t *residual, lynx_meta meta,
                      const lynx_kv_shape *shape, const lynx_params *params, void *out,
                      hipStream_t stream) {
    if (!residual)
        return LYNX_EINVAL;
    return dequant_common(anchor, residual, meta, shape, params, out, stream);
}

int lynx_page_stats(const void *kv, const lynx_kv_shape *shape, const lynx_params *params,
                    float *gamma_min, float *gamma_scale, hipStream_t stream) {
    return quantize_common(kv, shape, params, nullptr, nullptr, gamma_min, gamma_scale, nullptr,
                           nullptr, kModePageStats, stream);
}

int lynx_block_stats(const void *kv, const lynx_kv_shape *shape, const lynx_params *params,
                     const float *gamma_min, const float *gamma_scale, float *mu, float *sigma,
                     hipStream_t stream) {
    return quantize_common(kv, shape, params, nullptr, nullptr, (float *)gamma_min,
                           (float *)gamma_scale, mu, sigma, kModeBlockStats, stream);
}

}  // extern "C"
