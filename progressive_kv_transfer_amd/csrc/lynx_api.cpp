// Host side of liblynx.so: argument validation, the compander and level
// tables of Eq. (3) / Eq. (4), and the extern "C" entry points declared in
// include/lynx.h.  The kernels live in lynx_quant.hip and lynx_dequant.hip.
#include "lynx.h"

#include <math.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <utility>
#include <vector>

#include "lynx_attn_args.h"
#include "lynx_internal.h"

namespace lynx {
namespace {

thread_local std::string g_hip_error;

// Largest launch (in blocks) of one kernel dispatch: the grid size in
// work-items (blocks x 512) must stay below 2^32.
constexpr int64_t kMaxLaunchBlocks = int64_t(1) << 22;

// Largest row stride (elements): the quantize kernel addresses a page
// block's 256 rows through one buffer resource with 32-bit byte offsets
// below 2^31 - 1, up to 255 rows of 2 row_stride bytes plus one 256-byte
// row (4210744 is the largest multiple of 8 below this).
constexpr int64_t kMaxRowStride = (int64_t(0x7fffffff) - 256) / 510;

uint32_t f2u(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
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
bool build_quant_tab(float alpha, float code_scale, int code_max, QuantTab *t) {
    memset(t, 0, sizeof *t);
    const long double a = alpha, cs = code_scale, l1pa = log1pl(a);
    t->thr[0] = 0.0f;
    for (int k = 1; k < 128; ++k) {
        if (k > code_max) {
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
    // 7 mantissa bits first: the bucket is then the upper 16 bits of the
    // magnitude, which the kernel turns into a table address with one
    // instruction; otherwise the coarsest resolution that works.
    static const int kOrder[] = {7, 3, 4, 5, 6, 8};
    for (int mbits : kOrder) {
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

// The quantize kernel's table entries of a 16-bit-shift bucket table (the
// form QuantTab::word describes); bias is the Stage 4 offset of the split.
void build_table_words(int residual_bits, QuantTab *t) {
    if (t->shift != 16)
        return;
    const uint32_t bias = residual_bits > 0 ? (1u << (residual_bits - 1)) - 1u : 0u;
    for (int i = 0; i < t->nbuckets; ++i) {
        const uint32_t c = t->bucket_code[i];
        const uint32_t next = c + 1 < 128 ? f2u(t->thr[c + 1]) : f2u(INFINITY);
        const uint32_t lo =
            (next >> 16) == (uint32_t)(t->bucket_lo + i) ? (next & 0xffffu) : 0x10000u;
        t->word[i] = ((c + bias + 1u) << 24) - lo;
    }
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

// Tables per (alpha, code_scale, field widths), built on first use.  The
// cache is bounded (emptied when full; a caller sweeping parameters rebuilds
// tables, never grows memory) and hands out copies, so no caller holds a
// reference into it.
constexpr size_t kMaxCachedTables = 64;
std::mutex g_mu;
std::map<std::tuple<uint32_t, uint32_t, int, int>, Tables> g_cache;

bool tables_for(const lynx_params &p, Tables *out) {
    std::lock_guard<std::mutex> lock(g_mu);
    auto key = std::make_tuple(f2u(p.alpha), f2u(p.code_scale), (int)p.anchor_bits,
                               (int)p.residual_bits);
    auto it = g_cache.find(key);
    if (it != g_cache.end()) {
        *out = it->second;
        return true;
    }
    Tables t;
    if (!build_quant_tab(p.alpha, p.code_scale, code_max_of(p.anchor_bits, p.residual_bits),
                         &t.q))
        return false;
    build_table_words(p.residual_bits, &t.q);
    build_dequant_tab(p.alpha, p.code_scale, &t.d);
    if (g_cache.size() >= kMaxCachedTables)
        g_cache.clear();
    g_cache.emplace(key, t);
    *out = t;
    return true;
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
    if (!valid_field_bits(p.anchor_bits, p.residual_bits))
        return LYNX_EINVAL;
    // bfloat16 metadata is built for the paper's 4 + 4 split
    if (p.meta_bits != 32 &&
        !(p.meta_bits == 16 && p.anchor_bits == 4 && p.residual_bits == 4))
        return LYNX_EINVAL;
    if (p.layout != LYNX_LAYOUT_SEPARATE && p.layout != LYNX_LAYOUT_PACKED)
        return LYNX_EINVAL;
    return LYNX_OK;
}

// Bytes per page block of the anchor stream, of the metadata, and of the
// anchor-side buffer in the params' layout (the packed record is the anchor
// stream followed by gamma_min, gamma_scale, mu and sigma).
int64_t stream_block_bytes(const lynx_params &p) { return (int64_t)kPage * kHead / 8 * p.anchor_bits; }
int64_t meta_block_bytes(const lynx_params &p) {
    return (int64_t)(2 * kHead + 2 * kChunks * kHead) * (p.meta_bits / 8);
}
int64_t anchor_block_bytes(const lynx_params &p) {
    return stream_block_bytes(p) + (p.layout == LYNX_LAYOUT_PACKED ? meta_block_bytes(p) : 0);
}

// Metadata pointers of a packed anchor-side buffer (block 0's record).
lynx_meta packed_meta(const lynx_params &p, const uint8_t *records) {
    const int64_t e = p.meta_bits / 8;
    uint8_t *g0 = const_cast<uint8_t *>(records) + stream_block_bytes(p);
    lynx_meta m;
    m.gamma_min = (float *)g0;
    m.gamma_scale = (float *)(g0 + kHead * e);
    m.mu = (float *)(g0 + 2 * kHead * e);
    m.sigma = (float *)(g0 + (2 * kHead + kChunks * kHead) * e);
    return m;
}

// The metadata pointers a call works with: as given (separate layout), or
// inside the anchor-side buffer (packed layout, where the caller passes
// NULL metadata pointers).  False if the caller's pointers do not fit the
// layout.
bool resolve_meta(const lynx_params &p, const uint8_t *anchor, lynx_meta in, lynx_meta *out) {
    const bool none = !in.gamma_min && !in.gamma_scale && !in.mu && !in.sigma;
    if (p.layout == LYNX_LAYOUT_PACKED) {
        if (!none || !anchor)
            return false;
        *out = packed_meta(p, anchor);
        return true;
    }
    *out = in;
    return true;
}

int check_shape(const lynx_kv_shape *s, int64_t *nblocks) {
    if (!s)
        return LYNX_EINVAL;
    if (s->num_tensors < 0 || s->num_tokens < 0 || s->num_channels < 0 || s->row_stride < 0 ||
        s->tensor_stride < 0)
        return LYNX_EINVAL;
    if (s->num_tokens % kPage || s->num_channels % kHead)
        return LYNX_ESHAPE;
    if (s->row_stride < s->num_channels || s->row_stride % 8 || s->row_stride > kMaxRowStride)
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

Geometry geometry(const lynx_kv_shape *s, int64_t nblocks, const lynx_params &p) {
    Geometry g;
    g.tensor_stride = s->tensor_stride;
    g.row_stride = s->row_stride;
    g.pages = (int32_t)(s->num_tokens / kPage);
    g.heads = (int32_t)(s->num_channels / kHead);
    g.nblocks = nblocks;
    g.block0 = 0;
    g.grid_wgs = 0;
    g.astride = anchor_block_bytes(p);
    if (p.layout == LYNX_LAYOUT_PACKED) {
        g.gstride = g.cstride = anchor_block_bytes(p) / (p.meta_bits / 8);
    } else {
        g.gstride = kHead;
        g.cstride = kChunks * kHead;
    }
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
    if (mode != kModeQuantize && p.layout != LYNX_LAYOUT_SEPARATE)
        return LYNX_EINVAL;  // the statistics calls write separate arrays
    if (nb == 0)
        return LYNX_OK;
    if (mode == kModeQuantize) {
        lynx_meta m = {gmin, gscale, mu, sigma};
        if (!resolve_meta(p, anchor, m, &m))
            return LYNX_EINVAL;
        gmin = m.gamma_min;
        gscale = m.gamma_scale;
        mu = m.mu;
        sigma = m.sigma;
    }
    if (!kv || !gmin || !gscale)
        return LYNX_EINVAL;
    if (mode != kModePageStats && (!mu || !sigma))
        return LYNX_EINVAL;
    if (mode == kModeQuantize && (!anchor || (p.residual_bits > 0) != (residual != nullptr)))
        return LYNX_EINVAL;
    if (mode != kModeQuantize && p.meta_bits != 32)  // the stats calls write binary32
        return LYNX_EINVAL;
    for (const void *ptr : {(const void *)kv, (const void *)gmin, (const void *)gscale,
                            (const void *)mu, (const void *)sigma, (const void *)anchor,
                            (const void *)residual})
        if (ptr && !aligned16(ptr))
            return LYNX_ESHAPE;
    Tables t;
    if (!tables_for(p, &t))
        return LYNX_EINVAL;
    QuantTab tab = t.q;
    tab.eps = p.eps;
    Geometry g = geometry(shape, nb, p);
    for (int64_t b0 = 0; b0 < nb; b0 += kMaxLaunchBlocks) {
        g.block0 = b0;
        g.nblocks = (nb - b0) < kMaxLaunchBlocks ? (nb - b0) : kMaxLaunchBlocks;
        rc = hip_status(launch_quantize((const uint16_t *)kv, g, tab, anchor, residual, gmin,
                                        gscale, mu, sigma, mode, p.anchor_bits,
                                        p.residual_bits, p.meta_bits, stream));
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
    if (!resolve_meta(p, anchor, meta, &meta))
        return LYNX_EINVAL;
    if (!anchor || !out || !meta.gamma_min || !meta.gamma_scale || !meta.mu || !meta.sigma)
        return LYNX_EINVAL;
    if (residual && p.residual_bits == 0)  // a single stream has no residual phase
        return LYNX_EINVAL;
    for (const void *ptr : {(const void *)anchor, (const void *)residual, (const void *)out,
                            (const void *)meta.gamma_min, (const void *)meta.gamma_scale,
                            (const void *)meta.mu, (const void *)meta.sigma})
        if (ptr && !aligned16(ptr))
            return LYNX_ESHAPE;
    Tables t;
    if (!tables_for(p, &t))
        return LYNX_EINVAL;
    DequantTab tab = t.d;
    tab.eps = p.eps;
    Geometry g = geometry(shape, nb, p);
    for (int64_t b0 = 0; b0 < nb; b0 += kMaxLaunchBlocks) {
        g.block0 = b0;
        g.nblocks = (nb - b0) < kMaxLaunchBlocks ? (nb - b0) : kMaxLaunchBlocks;
        rc = hip_status(launch_dequant(anchor, residual, meta.gamma_min, meta.gamma_scale,
                                       meta.mu, meta.sigma, g, tab, (uint16_t *)out,
                                       p.anchor_bits, p.residual_bits, p.meta_bits, stream));
        if (rc)
            return rc;
    }
    return LYNX_OK;
}

// Split-KV plan of an attention call: query rows per KV head, splits of the
// context (about two resident workgroups per compute unit in total) and the
// workspace of their partials.  Up to 16 rows the decode kernel takes runs
// of 32-token chunks (a multiple of its 8 waves), beyond that the tile
// kernel runs of 128-token steps.
// Launch plan of one attention pass.  The kernels take at most 64 query
// rows (t_q * g) per KV head; more query tokens go through the kernels in
// passes of tq_pass = floor(64 / g) tokens, one after the other on the
// stream, each over the whole context.  The plan below is that of a pass of
// t_q tokens (the first, largest pass when called with the call's t_q: its
// workspace serves every pass).
struct AttnPlan {
    int tq_pass, rows, pages, splits, sps, cps;
    size_t ws_bytes;
};

int attn_plan(int t_q, int n_qh, int n_kvh, int64_t ctx, AttnPlan *pl) {
    if (t_q <= 0 || n_qh <= 0 || n_kvh <= 0 || n_qh % n_kvh || ctx <= 0)
        return LYNX_EINVAL;
    if (ctx % kPage || ctx / kPage > INT32_MAX)
        return LYNX_ESHAPE;
    const int group = n_qh / n_kvh;
    if (group > 64)
        return LYNX_EINVAL;
    pl->tq_pass = t_q < 64 / group ? t_q : 64 / group;
    const int64_t rows = (int64_t)pl->tq_pass * group;
    pl->rows = (int)rows;
    pl->pages = (int)(ctx / kPage);
    const int64_t target_wgs = 512;
    pl->sps = pl->cps = 0;
    if (rows <= 16) {
        const int64_t chunks = ctx / kChunk;
        int64_t cps = (chunks * n_kvh + target_wgs - 1) / target_wgs;
        cps = (cps + 7) / 8 * 8;
        if (cps > chunks)
            cps = chunks;  // a multiple of 8: chunks is
        pl->cps = (int)cps;
        pl->splits = (int)((chunks + cps - 1) / cps);
    } else {
        const int64_t steps = ctx / 128;
        int64_t sps = (steps * n_kvh + target_wgs - 1) / target_wgs;
        if (sps < 1)
            sps = 1;
        if (sps > steps)
            sps = steps;
        pl->sps = (int)sps;
        pl->splits = (int)((steps + sps - 1) / sps);
    }
    pl->ws_bytes = (size_t)pl->splits * n_kvh * pl->rows * (2 + kHead) * sizeof(float);
    return LYNX_OK;
}

}  // namespace
}  // namespace lynx

using namespace lynx;

// ------------------------------------------------- split-stream transfer --

// HIP events owned by one transfer call, destroyed when it returns (after
// every stream has been synchronised).
struct EventSet {
    std::vector<hipEvent_t> ev;
    hipError_t err = hipSuccess;
    hipEvent_t make(bool timing) {
        hipEvent_t e = nullptr;
        const hipError_t r =
            hipEventCreateWithFlags(&e, timing ? hipEventDefault : hipEventDisableTiming);
        if (r != hipSuccess) {
            if (err == hipSuccess)
                err = r;
            return nullptr;
        }
        ev.push_back(e);
        return e;
    }
    ~EventSet() {
        for (hipEvent_t e : ev)
            (void)hipEventDestroy(e);
    }
};

// Anchor stream + metadata (or the residual stream) of blocks [b0, b0 + n)
// from one code set to another: with the packed layout one copy of the
// blocks' records, otherwise the stream and the four metadata arrays.
hipError_t copy_anchor_meta(const lynx_params &p, const lynx_codes &src, const lynx_codes &dst,
                            int64_t b0, int64_t n, hipStream_t s) {
    if (p.layout == LYNX_LAYOUT_PACKED) {
        const size_t rec = (size_t)anchor_block_bytes(p);
        return hipMemcpyAsync(dst.anchor + b0 * rec, src.anchor + b0 * rec, n * rec,
                              hipMemcpyDefault, s);
    }
    const size_t stream_b = (size_t)kPage * kHead / 2, gam = kHead, chk = (size_t)kChunks * kHead;
    hipError_t e = hipMemcpyAsync(dst.anchor + b0 * stream_b, src.anchor + b0 * stream_b,
                                  n * stream_b, hipMemcpyDefault, s);
    const float *sm[4] = {src.meta.gamma_min, src.meta.gamma_scale, src.meta.mu, src.meta.sigma};
    float *dm[4] = {dst.meta.gamma_min, dst.meta.gamma_scale, dst.meta.mu, dst.meta.sigma};
    for (int k = 0; k < 4 && e == hipSuccess; ++k) {
        const size_t per = k < 2 ? gam : chk;
        e = hipMemcpyAsync(dm[k] + b0 * per, sm[k] + b0 * per, n * per * sizeof(float),
                           hipMemcpyDefault, s);
    }
    return e;
}

hipError_t copy_residual(const lynx_codes &src, const lynx_codes &dst, int64_t b0, int64_t n,
                         hipStream_t s) {
    const size_t stream_b = (size_t)kPage * kHead / 2;
    return hipMemcpyAsync(dst.residual + b0 * stream_b, src.residual + b0 * stream_b,
                          n * stream_b, hipMemcpyDefault, s);
}

bool codes_ok(const lynx_params &p, const lynx_codes &c) {
    lynx_meta m;
    if (!resolve_meta(p, c.anchor, c.meta, &m))
        return false;
    const void *ptrs[6] = {c.anchor, c.residual, m.gamma_min, m.gamma_scale, m.mu, m.sigma};
    for (const void *q : ptrs)
        if (!q || !aligned16(q))
            return false;
    return true;
}

constexpr int64_t kMaxTransferObjects = 4096;

extern "C" {

void lynx_default_params(lynx_params *p) {
    if (!p)
        return;
    p->alpha = 255.0f;
    p->eps = 1e-6f;
    p->code_scale = 120.0f;
    p->page_tokens = kPage;
    p->chunk_tokens = kChunk;
    p->block_channels = kHead;
    p->anchor_bits = 4;
    p->residual_bits = 4;
    p->meta_bits = 32;
    p->layout = LYNX_LAYOUT_SEPARATE;
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

size_t lynx_field_stream_bytes(const lynx_kv_shape *shape, int field_bits) {
    int64_t nb = lynx_num_blocks(shape);
    if (nb < 0 || field_bits < 1 || field_bits > 8)
        return 0;
    return (size_t)nb * (kPage * kHead / 8) * (size_t)field_bits;
}

size_t lynx_anchor_block_bytes(const lynx_params *params) {
    const lynx_params p = resolve(params);
    return check_params(p) ? 0 : (size_t)anchor_block_bytes(p);
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
    Tables t;
    if (!tables_for(p, &t))
        return LYNX_EINVAL;
    memcpy(thr128, t.q.thr, sizeof t.q.thr);
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
    case LYNX_ESCRATCH:
        return "the call needs more than the library's fixed device scratch "
               "(LYNX_ATTN_SCRATCH_BYTES); use the entry point that takes a workspace";
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

size_t lynx_attn_workspace_bytes(int t_q, int num_q_heads, int num_kv_heads, int64_t ctx_len) {
    AttnPlan pl;
    return attn_plan(t_q, num_q_heads, num_kv_heads, ctx_len, &pl) ? 0 : pl.ws_bytes;
}

}  // extern "C"

static_assert(kAttnScratchBytes == LYNX_ATTN_SCRATCH_BYTES, "scratch size of lynx.h");

namespace {

// Both attention entry points: the partials go to the caller's workspace,
// or (use_scratch) to the library's fixed device scratch.
int attn_common(const void *q, int t_q, int num_q_heads, const uint8_t *k_anchor,
                const uint8_t *k_residual, lynx_meta k_meta, const uint8_t *v_anchor,
                const uint8_t *v_residual, lynx_meta v_meta, int64_t ctx_len,
                int num_kv_heads, int head_dim, float scale, int causal_tail,
                const lynx_params *params, void *out, int out_dtype, void *workspace,
                size_t workspace_bytes, bool use_scratch, hipStream_t stream) {
    const lynx_params p = resolve(params);
    int rc = check_params(p);
    if (rc)
        return rc;
    if (p.anchor_bits != 4 || p.residual_bits != 4 || p.meta_bits != 32)
        return LYNX_EINVAL;
    if (head_dim != kHead || !(scale > 0.0f) || !(scale < 1e30f) ||
        (out_dtype != LYNX_OUT_BF16 && out_dtype != LYNX_OUT_F32))
        return LYNX_EINVAL;
    AttnPlan pl;
    if ((rc = attn_plan(t_q, num_q_heads, num_kv_heads, ctx_len, &pl)))
        return rc;
    if (causal_tail && ctx_len < t_q)
        return LYNX_EINVAL;
    if (!resolve_meta(p, k_anchor, k_meta, &k_meta) || !resolve_meta(p, v_anchor, v_meta, &v_meta))
        return LYNX_EINVAL;
    if (!q || !out || (!use_scratch && !workspace) || !k_anchor || !v_anchor ||
        !k_meta.gamma_min || !k_meta.gamma_scale || !k_meta.mu || !k_meta.sigma ||
        !v_meta.gamma_min || !v_meta.gamma_scale || !v_meta.mu || !v_meta.sigma)
        return LYNX_EINVAL;
    if (use_scratch ? pl.ws_bytes > kAttnScratchBytes : workspace_bytes < pl.ws_bytes)
        return use_scratch ? LYNX_ESCRATCH : LYNX_EINVAL;
    for (const void *ptr : {(const void *)q, (const void *)out, (const void *)workspace, (const void *)k_anchor,
                            (const void *)k_residual, (const void *)v_anchor,
                            (const void *)v_residual, (const void *)k_meta.gamma_min,
                            (const void *)k_meta.gamma_scale, (const void *)k_meta.mu,
                            (const void *)k_meta.sigma, (const void *)v_meta.gamma_min,
                            (const void *)v_meta.gamma_scale, (const void *)v_meta.mu,
                            (const void *)v_meta.sigma})
        if (ptr && !aligned16(ptr))
            return LYNX_ESHAPE;
    Tables t;
    if (!tables_for(p, &t))
        return LYNX_EINVAL;
    DequantTab tab = t.d;
    tab.eps = p.eps;
    AttnArgs a;
    a.q = (const uint16_t *)q;
    a.k_anc = k_anchor;
    a.k_res = k_residual;
    a.v_anc = v_anchor;
    a.v_res = v_residual;
    a.k_gmin = k_meta.gamma_min;
    a.k_gsc = k_meta.gamma_scale;
    a.k_mu = k_meta.mu;
    a.k_sg = k_meta.sigma;
    a.v_gmin = v_meta.gamma_min;
    a.v_gsc = v_meta.gamma_scale;
    a.v_mu = v_meta.mu;
    a.v_sg = v_meta.sigma;
    if (use_scratch) {
        float *ws = nullptr;
        if ((rc = hip_status(attn_scratch(&ws))))
            return rc;
        a.ws = ws;
    } else {
        a.ws = (float *)workspace;
    }
    a.out = out;
    a.out_f32 = out_dtype == LYNX_OUT_F32 ? 1 : 0;
    {
        const lynx_kv_shape one = {1, 0, ctx_len, (int64_t)num_kv_heads * kHead,
                                   (int64_t)num_kv_heads * kHead};
        const Geometry gs = geometry(&one, 0, p);
        a.astride = gs.astride;
        a.gstride = gs.gstride;
        a.cstride = gs.cstride;
    }
    a.ctx = ctx_len;
    a.n_qh = num_q_heads;
    a.n_kvh = num_kv_heads;
    a.group = num_q_heads / num_kv_heads;
    a.pages = pl.pages;
    a.causal = causal_tail ? 1 : 0;
    a.qk_scale_log2 = (float)((double)scale * 1.4426950408889634);
    // Passes of at most tq_pass query tokens; token r of the call sees keys
    // 0 .. ctx_len - t_q + r under the causal tail.
    const size_t out_elem = a.out_f32 ? sizeof(float) : sizeof(uint16_t);
    for (int tok0 = 0; tok0 < t_q; tok0 += pl.tq_pass) {
        const int n = t_q - tok0 < pl.tq_pass ? t_q - tok0 : pl.tq_pass;
        AttnPlan pp;
        if ((rc = attn_plan(n, num_q_heads, num_kv_heads, ctx_len, &pp)))
            return rc;
        const int64_t row0 = (int64_t)tok0 * num_q_heads * kHead;  // elements of q / out
        a.q = (const uint16_t *)q + row0;
        a.out = (char *)out + row0 * out_elem;
        a.t_q = n;
        a.causal_base = ctx_len - t_q + tok0;
        a.rows = pp.rows;
        a.splits = pp.splits;
        a.steps_per_split = pp.sps;
        a.chunks_per_split = pp.cps;
        if ((rc = hip_status(launch_attention(a, tab, stream))))
            return rc;
    }
    return LYNX_OK;
}

}  // namespace

extern "C" {

int lynx_decode_attn_dequant(const void *q, int t_q, int num_q_heads, const uint8_t *k_anchor,
                             const uint8_t *k_residual, lynx_meta k_meta,
                             const uint8_t *v_anchor, const uint8_t *v_residual,
                             lynx_meta v_meta, int64_t ctx_len, int num_kv_heads, int head_dim,
                             float scale, int causal_tail, const lynx_params *params, void *out,
                             int out_dtype, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    return attn_common(q, t_q, num_q_heads, k_anchor, k_residual, k_meta, v_anchor, v_residual,
                       v_meta, ctx_len, num_kv_heads, head_dim, scale, causal_tail, params, out,
                       out_dtype, workspace, workspace_bytes, false, stream);
}

int lynx_decode_attn_dequant_noalloc(const void *q, int t_q, int num_q_heads,
                                     const uint8_t *k_anchor, const uint8_t *k_residual,
                                     lynx_meta k_meta, const uint8_t *v_anchor,
                                     const uint8_t *v_residual, lynx_meta v_meta,
                                     int64_t ctx_len, int num_kv_heads, int head_dim,
                                     float scale, int causal_tail, const lynx_params *params,
                                     void *out, int out_dtype, hipStream_t stream) {
    return attn_common(q, t_q, num_q_heads, k_anchor, k_residual, k_meta, v_anchor, v_residual,
                       v_meta, ctx_len, num_kv_heads, head_dim, scale, causal_tail, params, out,
                       out_dtype, nullptr, 0, true, stream);
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

// The k-th compute unit a codec stream leaves free, as a bit of the stream's
// CU mask.  On a part of 8 XCDs the driver hands mask bit u to XCD u % 8
// (unit u / 8 there); the k-th reserved unit is unit 4 x + m of XCD x, for
// x = k % 8, m = k / 8, so the reserve is spread evenly over the XCDs, and
// in a numbering of whole XCDs one after another (bit u on XCD u / (ncu / 8))
// it would be spread evenly too.  Distinct for k < ncu; other unit counts
// take every (ncu / reserved)-th bit.
static int reserved_unit(int k, int ncu) {
    constexpr int kXcds = 8;
    const int per = ncu / kXcds;
    if (ncu % kXcds || per % kXcds)
        return k;
    const int x = k % kXcds, m = k / kXcds;
    return x + kXcds * ((per / kXcds * x + m) % per);
}

int lynx_codec_stream_create(int reserved_cus, hipStream_t *stream) {
    if (!stream || reserved_cus < 0)
        return LYNX_EINVAL;
    *stream = nullptr;
    int dev = 0, ncu = 0;
    int rc = hip_status(hipGetDevice(&dev));
    if (rc)
        return rc;
    if ((rc = hip_status(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev))))
        return rc;
    if (reserved_cus >= ncu)
        return LYNX_EINVAL;
    if (reserved_cus == 0)
        return hip_status(hipStreamCreate(stream));
    std::vector<uint32_t> mask((size_t)(ncu + 31) / 32, ~0u);
    if (ncu % 32)
        mask.back() = (1u << (ncu % 32)) - 1u;
    for (int k = 0; k < reserved_cus; ++k) {
        const int u = reserved_unit(k, ncu);
        mask[(size_t)u / 32] &= ~(1u << (u % 32));
    }
    return hip_status(hipExtStreamCreateWithCUMask(stream, (uint32_t)mask.size(), mask.data()));
}

int lynx_stream_destroy(hipStream_t stream) {
    if (!stream)
        return LYNX_EINVAL;
    return hip_status(hipStreamDestroy(stream));
}

int lynx_split_stream_transfer(const void *kv, const lynx_kv_shape *shape,
                               const lynx_params *params, int64_t object_blocks, lynx_codes tx,
                               lynx_codes wire, lynx_codes rx, void *kv_anchor, void *kv_full,
                               int flags, hipStream_t sender, hipStream_t link_out,
                               hipStream_t link_in, hipStream_t receiver,
                               lynx_transfer_times *times) {
    const lynx_params p = resolve(params);
    int rc = check_params(p);
    if (rc)
        return rc;
    if (p.anchor_bits != 4 || p.residual_bits != 4 || p.meta_bits != 32)
        return LYNX_EINVAL;
    int64_t nb = 0;
    if ((rc = check_shape(shape, &nb)))
        return rc;
    // one launch per object: at most kMaxLaunchBlocks blocks each
    if (object_blocks <= 0 || object_blocks > kMaxLaunchBlocks ||
        (flags & ~LYNX_TRANSFER_COPIES_ONLY))
        return LYNX_EINVAL;
    const bool copies_only = (flags & LYNX_TRANSFER_COPIES_ONLY) != 0;
    if (times)
        memset(times, 0, sizeof *times);
    if (nb == 0)
        return LYNX_OK;
    const int64_t nobj = (nb + object_blocks - 1) / object_blocks;
    if (nobj > kMaxTransferObjects)
        return LYNX_EINVAL;
    if (!codes_ok(p, tx) || !codes_ok(p, wire) || !codes_ok(p, rx))
        return LYNX_EINVAL;
    if (p.layout == LYNX_LAYOUT_PACKED) {  // the kernels take the derived pointers
        resolve_meta(p, tx.anchor, tx.meta, &tx.meta);
        resolve_meta(p, rx.anchor, rx.meta, &rx.meta);
    }
    if (!copies_only) {
        if (!kv || !kv_anchor || !kv_full)
            return LYNX_EINVAL;
        if (!aligned16(kv) || !aligned16(kv_anchor) || !aligned16(kv_full))
            return LYNX_ESHAPE;
    }
    Tables t;
    if (!tables_for(p, &t))
        return LYNX_EINVAL;
    QuantTab qt = t.q;
    qt.eps = p.eps;
    DequantTab dt = t.d;
    dt.eps = p.eps;
    const Geometry g0 = geometry(shape, nb, p);

    EventSet es;
    hipEvent_t start = es.make(true), t_q = es.make(true), t_a = es.make(true),
               t_r = es.make(true), t_da0 = es.make(true), t_da = es.make(true),
               t_df = es.make(true);
    // per object: quantized, anchor out of tx, anchor in rx, residual out,
    // residual in rx
    std::vector<hipEvent_t> q(nobj), ao(nobj), a(nobj), ro(nobj), r(nobj);
    for (int64_t i = 0; i < nobj; ++i) {
        q[i] = es.make(false);
        ao[i] = es.make(false);
        a[i] = es.make(false);
        ro[i] = es.make(false);
        r[i] = es.make(false);
    }
    if (es.err != hipSuccess)
        return hip_status(es.err);

    hipError_t err = hipSuccess;
    auto ok = [&](hipError_t e) {
        if (err == hipSuccess && e != hipSuccess)
            err = e;
        return err == hipSuccess;
    };
    auto object = [&](int64_t i, Geometry &g, int64_t &b0, int64_t &n) {
        b0 = i * object_blocks;
        n = (nb - b0) < object_blocks ? (nb - b0) : object_blocks;
        g = g0;
        g.block0 = b0;
        g.nblocks = n;
    };
    ok(hipEventRecord(start, sender));
    for (hipStream_t s : {link_out, link_in, receiver})
        ok(hipStreamWaitEvent(s, start, 0));
    // Anchor queue.  Each link stream carries every anchor + metadata copy
    // before any residual copy (stream order is the strict priority of the
    // anchor queue); the outbound hop (tx -> wire) of object i + 1 overlaps
    // the inbound hop (wire -> rx) of object i, and the quantization of
    // object i + 1 overlaps the sending of object i.
    for (int64_t i = 0; i < nobj && err == hipSuccess; ++i) {
        Geometry g;
        int64_t b0, n;
        object(i, g, b0, n);
        if (!copies_only)
            ok(launch_quantize((const uint16_t *)kv, g, qt, tx.anchor, tx.residual,
                               tx.meta.gamma_min, tx.meta.gamma_scale, tx.meta.mu, tx.meta.sigma,
                               kModeQuantize, 4, 4, 32, sender));
        // the last object's events are the timed milestones themselves, so
        // each milestone is ordered by the same waits as the work it marks
        const bool last = i + 1 == nobj;
        const hipEvent_t qe = last ? t_q : q[i];
        ok(hipEventRecord(qe, sender));
        ok(hipStreamWaitEvent(link_out, qe, 0));
        ok(copy_anchor_meta(p, tx, wire, b0, n, link_out));
        ok(hipEventRecord(ao[i], link_out));
        ok(hipStreamWaitEvent(link_in, ao[i], 0));
        ok(copy_anchor_meta(p, wire, rx, b0, n, link_in));
        const hipEvent_t ae = last ? t_a : a[i];
        ok(hipEventRecord(ae, link_in));
        // deserializer, anchor phase
        ok(hipStreamWaitEvent(receiver, ae, 0));
        if (!copies_only)
            ok(launch_dequant(rx.anchor, nullptr, rx.meta.gamma_min, rx.meta.gamma_scale,
                              rx.meta.mu, rx.meta.sigma, g, dt, (uint16_t *)kv_anchor, 4, 4,
                              32, receiver));
        if (i == 0)
            ok(hipEventRecord(t_da0, receiver));
    }
    ok(hipEventRecord(t_da, receiver));
    // Residual queue: behind the whole anchor queue on both hops.
    for (int64_t i = 0; i < nobj && err == hipSuccess; ++i) {
        Geometry g;
        int64_t b0, n;
        object(i, g, b0, n);
        ok(copy_residual(tx, wire, b0, n, link_out));
        ok(hipEventRecord(ro[i], link_out));
        ok(hipStreamWaitEvent(link_in, ro[i], 0));
        ok(copy_residual(wire, rx, b0, n, link_in));
        ok(hipEventRecord(i + 1 == nobj ? t_r : r[i], link_in));
    }
    // deserializer, residual phase (after the whole anchor phase)
    for (int64_t i = 0; i < nobj && err == hipSuccess; ++i) {
        Geometry g;
        int64_t b0, n;
        object(i, g, b0, n);
        ok(hipStreamWaitEvent(receiver, i + 1 == nobj ? t_r : r[i], 0));
        if (!copies_only)
            ok(launch_dequant(rx.anchor, rx.residual, rx.meta.gamma_min, rx.meta.gamma_scale,
                              rx.meta.mu, rx.meta.sigma, g, dt, (uint16_t *)kv_full, 4, 4,
                              32, receiver));
    }
    ok(hipEventRecord(t_df, receiver));
    // Blocking: every stream drains before the events go away.
    for (hipStream_t s : {sender, link_out, link_in, receiver}) {
        const hipError_t e = hipStreamSynchronize(s);
        if (err == hipSuccess)
            err = e;
    }
    if (err != hipSuccess)
        return hip_status(err);
    if (times) {
        float *out[6] = {&times->quantized,          &times->anchor_arrived,
                         &times->residual_arrived,   &times->first_anchor_ready,
                         &times->anchor_ready,       &times->full_ready};
        hipEvent_t ev[6] = {t_q, t_a, t_r, t_da0, t_da, t_df};
        for (int k = 0; k < 6; ++k)
            if (!ok(hipEventElapsedTime(out[k], start, ev[k])))
                return hip_status(err);
    }
    return LYNX_OK;
}

size_t lynx_spec_verify_workspace_bytes(int t_draft, int vocab) {
    if (t_draft < 0 || t_draft > kVerifyMaxDraft || vocab <= 0)
        return 0;
    const int64_t chunks = (vocab + kVerifyChunk - 1) / kVerifyChunk;
    return verify_workspace_doubles(t_draft, chunks) * sizeof(double);
}

int lynx_spec_verify(const float *draft_logits, const float *target_logits,
                     const int32_t *draft_tokens, const double *u_accept, double u_sample,
                     int t_draft, int vocab, int32_t *out, void *workspace,
                     size_t workspace_bytes, hipStream_t stream) {
    if (t_draft < 0 || t_draft > kVerifyMaxDraft || vocab <= 0 || vocab > (1 << 26))
        return LYNX_EINVAL;
    if (!(u_sample >= 0.0) || !(u_sample < 1.0))
        return LYNX_EINVAL;
    if (!target_logits || !out || !workspace)
        return LYNX_EINVAL;
    if (t_draft > 0 && (!draft_logits || !draft_tokens || !u_accept))
        return LYNX_EINVAL;
    if (workspace_bytes < lynx_spec_verify_workspace_bytes(t_draft, vocab))
        return LYNX_EINVAL;
    if (((uintptr_t)workspace & 7u) || ((uintptr_t)u_accept & 7u) || ((uintptr_t)out & 3u))
        return LYNX_ESHAPE;
    VerifyArgs a;
    a.draft = draft_logits;
    a.target = target_logits;
    a.tokens = draft_tokens;
    a.u_accept = u_accept;
    a.u_sample = u_sample;
    a.t = t_draft;
    a.vocab = vocab;
    a.chunks = (vocab + kVerifyChunk - 1) / kVerifyChunk;
    a.ws = (double *)workspace;
    a.out = out;
    return hip_status(launch_verify(a, stream));
}

}  // extern "C"
