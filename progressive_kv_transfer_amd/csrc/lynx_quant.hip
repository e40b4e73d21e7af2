// gfx950 quantize kernel: Algorithm 1 of "Lynx: Progressive Speculative
// Quantization for accelerating KV Transfer in Long-Context Inference"
// (Section 4.1, Stages 1-4, Eq. (3)) on one 256-token x 128-channel page
// block per workgroup, fused into one pass over HBM:
//   phase 1  page statistics  (Stage 1: per-channel min / max over 256 tokens)
//   phase 2  normalise + chunk statistics (Stage 2: tree mean, max |X - mu|)
//   phase 3  scale, compand, round, split and nibble-pack (Stages 2-4)
// The same kernel body, cut short, gives the Stage 1 and Stage 2
// statistics on their own.
//
// Workgroup = 512 lanes = 8 wave64s.  Wave w owns chunk w (tokens
// 32w..32w+31); inside a wave, lane = 16 s + g owns channels 8g..8g+7 of
// tokens 32w + 8s .. 32w + 8s + 7.  Every token row of the block is 256
// contiguous bytes, so each 16-byte load of a row group is one fully used
// 256-byte segment per 16 lanes.  Reductions over the 4 lanes of a chunk use
// v_permlane16_swap / v_permlane32_swap (no LDS); the 8 waves of a page meet
// once in LDS.
//
// Arithmetic is binary32 with one rounding per operation (built with
// -ffp-contract=off).  The two divisions of Algorithm 1 use
// q = a*r, e = fma(-q, d, a), q' = fma(e, r, q) with r = RN(1/d), which is
// the correctly rounded a/d whenever a = 0 or |a| >= max(2^-100, 2^-125 d)
// and d < 2^125 (Markstein's correction step; checked exhaustively near the
// worst-case significands and on 1.2e10 random operand pairs).  Operands
// outside that range are detected per channel (Stage 1) and per chunk
// (Stage 2) from the statistics and divided with an IEEE division instead.
#include "lynx_internal.h"

namespace lynx {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Correctly rounded a / d in the fast domain (see the file comment).
__device__ __forceinline__ float div_fast(float a, float d, float r) {
    float q = a * r;
    float e = __builtin_fmaf(-q, d, a);
    return __builtin_fmaf(e, r, q);
}

// Pairwise combination across lane rows: after permlane16_swap with both
// operands = v, the pair holds (row 2k, row 2k+1) of v; after
// permlane32_swap it holds (lanes 0-31, lanes 32-63).
struct Pair {
    float a, b;
};
__device__ __forceinline__ Pair swap16(float v) {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return {__uint_as_float(p[0]), __uint_as_float(p[1])};
}
__device__ __forceinline__ Pair swap32(float v) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return {__uint_as_float(p[0]), __uint_as_float(p[1])};
}

constexpr float kTiny100 = 0x1p-100f;
constexpr float kTiny125 = 0x1p-125f;
constexpr float kHuge125 = 0x1p125f;
constexpr float kMuTiny = 0x1p-74f;

template <int MODE>
__global__ __launch_bounds__(512) void quant_kernel(const uint16_t *__restrict__ kv, Geometry g,
                                                    const QuantTab tab,
                                                    uint8_t *__restrict__ anchor,
                                                    uint8_t *__restrict__ residual,
                                                    float *__restrict__ gmin_io,
                                                    float *__restrict__ gscale_io,
                                                    float *__restrict__ mu_out,
                                                    float *__restrict__ sigma_out) {
    __shared__ float s_min[kChunks][kHead];
    __shared__ float s_max[kChunks][kHead];
    __shared__ float4 s_ch[kHead];  // gamma_min, d1, r1, slow flag
    __shared__ uint2 s_tab[MODE == kModeQuantize ? kMaxBuckets : 1];

    const int64_t b = g.block0 + blockIdx.x;
    const int head = (int)(b % g.heads);
    const int64_t tp = b / g.heads;
    const int page = (int)(tp % g.pages);
    const int64_t tensor = tp / g.pages;
    const uint16_t *base =
        kv + tensor * g.tensor_stride + (int64_t)page * kPage * g.row_stride + head * kHead;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int cg = lane & 15;
    const int s = lane >> 4;
    const int tok0 = wave * kChunk + s * 8;

    // ---- load 8 token rows x 8 channels (16 B per row) ------------------
    u32x4 raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        raw[i] = __builtin_nontemporal_load(
            (const u32x4 *)(base + (int64_t)(tok0 + i) * g.row_stride + cg * 8));

    // Compander table into LDS while the loads are in flight.
    if (MODE == kModeQuantize) {
        for (int i = tid; i < tab.nbuckets; i += 512) {
            uint32_t c = tab.bucket_code[i];
            s_tab[i] = make_uint2(__float_as_uint(tab.thr[c + 1]), c + 7u);
        }
    }

    float x[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[i][2 * k] = bf16_lo(raw[i][k]);
            x[i][2 * k + 1] = bf16_hi(raw[i][k]);
        }
    }

    // ---- phase 1: page statistics --------------------------------------
    if (MODE != kModeBlockStats) {
        float mn[8], mx[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            mn[e] = x[0][e];
            mx[e] = x[0][e];
#pragma unroll
            for (int i = 1; i < 8; ++i) {
                mn[e] = fminf(mn[e], x[i][e]);
                mx[e] = fmaxf(mx[e], x[i][e]);
            }
            Pair p = swap16(mn[e]);
            mn[e] = fminf(p.a, p.b);
            p = swap32(mn[e]);
            mn[e] = fminf(p.a, p.b);
            p = swap16(mx[e]);
            mx[e] = fmaxf(p.a, p.b);
            p = swap32(mx[e]);
            mx[e] = fmaxf(p.a, p.b);
        }
        if (s == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                s_min[wave][cg * 8 + e] = mn[e];
                s_max[wave][cg * 8 + e] = mx[e];
            }
        }
        __syncthreads();
    }
    if (tid < kHead) {
        float gmin, gsc;
        if (MODE == kModeBlockStats) {
            gmin = gmin_io[b * kHead + tid];
            gsc = gscale_io[b * kHead + tid];
        } else {
            float a = s_min[0][tid], m = s_max[0][tid];
#pragma unroll
            for (int w = 1; w < kChunks; ++w) {
                a = fminf(a, s_min[w][tid]);
                m = fmaxf(m, s_max[w][tid]);
            }
            gmin = a + 0.0f;  // canonical +0 for a zero minimum
            gsc = m - gmin;
            gmin_io[b * kHead + tid] = gmin;
            gscale_io[b * kHead + tid] = gsc;
        }
        float d1 = gsc + tab.eps;
        float r1 = __fdiv_rn(1.0f, d1);
        // Every nonzero x - gamma_min of a bf16 channel is at least
        // 2^-9 |gamma_min|; the fast division needs it above the bound.
        bool fast = gmin != 0.0f && fabsf(gmin) * 0x1p-9f >= fmaxf(kTiny100, d1 * kTiny125) &&
                    d1 < kHuge125;
        s_ch[tid] = make_float4(gmin, d1, r1, fast ? 0.0f : 1.0f);
    }
    if (MODE == kModePageStats)
        return;
    __syncthreads();

    // ---- phase 2: normalise, chunk mean and max |X - mu| ----------------
    float gmin[8], d1[8], r1[8];
    bool slow1 = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float4 c = s_ch[cg * 8 + e];
        gmin[e] = c.x;
        d1[e] = c.y;
        r1[e] = c.z;
        slow1 |= c.w != 0.0f;
    }
    if (!slow1) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) x[i][e] = div_fast(x[i][e] - gmin[e], d1[e], r1[e]);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) x[i][e] = __fdiv_rn(x[i][e] - gmin[e], d1[e]);
    }

    float mu[8], sg[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        // balanced tree: tokens 8s..8s+7 in-lane, then rows, then halves
        float s8 = ((x[0][e] + x[1][e]) + (x[2][e] + x[3][e])) +
                   ((x[4][e] + x[5][e]) + (x[6][e] + x[7][e]));
        Pair p = swap16(s8);
        float s16 = p.a + p.b;
        p = swap32(s16);
        float s32 = p.a + p.b;
        mu[e] = s32 * 0.03125f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i][e] = x[i][e] - mu[e];
            m = fmaxf(m, fabsf(x[i][e]));
        }
        Pair p = swap16(m);
        m = fmaxf(p.a, p.b);
        p = swap32(m);
        sg[e] = fmaxf(p.a, p.b);
    }
    if (s == 0) {
        float4 *mo = (float4 *)(mu_out + b * (kChunks * kHead) + wave * kHead + cg * 8);
        float4 *so = (float4 *)(sigma_out + b * (kChunks * kHead) + wave * kHead + cg * 8);
        mo[0] = make_float4(mu[0], mu[1], mu[2], mu[3]);
        mo[1] = make_float4(mu[4], mu[5], mu[6], mu[7]);
        so[0] = make_float4(sg[0], sg[1], sg[2], sg[3]);
        so[1] = make_float4(sg[4], sg[5], sg[6], sg[7]);
    }
    if (MODE == kModeBlockStats)
        return;

    // ---- phase 3: scale, compand, split, pack ---------------------------
    float d2[8], r2[8];
    bool slow2 = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        d2[e] = sg[e] + tab.eps;
        r2[e] = __fdiv_rn(1.0f, d2[e]);
        slow2 |= mu[e] > 0.0f && mu[e] < kMuTiny;
    }
    if (slow2) {
        // IEEE quotient; + 0 turns a -0 quotient into +0 so that the sign
        // bit below is exactly [X_cent < 0].
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) x[i][e] = __fdiv_rn(x[i][e], d2[e]) + 0.0f;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) x[i][e] = div_fast(x[i][e], d2[e], r2[e]);
    }
    __syncthreads();  // s_tab complete

    const uint32_t lo = (uint32_t)tab.bucket_lo;
    const uint32_t hi = lo + (uint32_t)tab.nbuckets - 1u;
    const uint32_t sh = (uint32_t)tab.shift;
    uint32_t *anc = (uint32_t *)(anchor + b * (kPage * kHead / 2));
    uint32_t *res = (uint32_t *)(residual + b * (kPage * kHead / 2));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t J[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t mag = __float_as_uint(x[i][e]) & 0x7fffffffu;
            uint32_t idx = mag >> sh;
            idx = idx < lo ? lo : (idx > hi ? hi : idx);
            uint2 ent = s_tab[idx - lo];
            // J = code + 7: high nibble = anchor magnitude (code + 7) >> 4,
            // low nibble ^ 7 = residual (-code) mod 16.
            J[e] = ent.y + (mag >= ent.x ? 1u : 0u);
        }
        uint32_t w_even = J[0] | (J[2] << 8) | (J[4] << 16) | (J[6] << 24);
        uint32_t w_odd = J[1] | (J[3] << 8) | (J[5] << 16) | (J[7] << 24);
        uint32_t a = ((w_even >> 4) & 0x0f0f0f0fu) | (w_odd & 0xf0f0f0f0u);
        uint32_t r = ((w_even & 0x0f0f0f0fu) | ((w_odd << 4) & 0xf0f0f0f0u)) ^ 0x77777777u;
        // Sign bits of the 8 quotients replicated to bytes (v_perm
        // selectors 9 and 11), then to nibbles: anchor of a negative value
        // is the one's complement of its magnitude (-V - 1).
        uint32_t xs[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) xs[e] = __float_as_uint(x[i][e]);
        uint32_t n_even = __builtin_amdgcn_perm(xs[2], xs[0], 0x0c0c0b09u) |
                          __builtin_amdgcn_perm(xs[6], xs[4], 0x0b090c0cu);
        uint32_t n_odd = __builtin_amdgcn_perm(xs[3], xs[1], 0x0c0c0b09u) |
                         __builtin_amdgcn_perm(xs[7], xs[5], 0x0b090c0cu);
        a ^= (n_even & 0x0f0f0f0fu) | (n_odd & 0xf0f0f0f0u);
        const int row = tok0 + i;
        __builtin_nontemporal_store(a, anc + row * (kHead / 8) + cg);
        __builtin_nontemporal_store(r, res + row * (kHead / 8) + cg);
    }
}

}  // namespace

hipError_t launch_quantize(const uint16_t *kv, const Geometry &g, const QuantTab &tab,
                           uint8_t *anchor, uint8_t *residual, float *gmin, float *gscale,
                           float *mu, float *sigma, int mode, hipStream_t stream) {
    if (g.nblocks == 0)
        return hipSuccess;
    dim3 grid((unsigned)g.nblocks), block(512);
    switch (mode) {
    case kModeQuantize:
        hipLaunchKernelGGL(quant_kernel<kModeQuantize>, grid, block, 0, stream, kv, g, tab,
                           anchor, residual, gmin, gscale, mu, sigma);
        break;
    case kModePageStats:
        hipLaunchKernelGGL(quant_kernel<kModePageStats>, grid, block, 0, stream, kv, g, tab,
                           anchor, residual, gmin, gscale, mu, sigma);
        break;
    default:
        hipLaunchKernelGGL(quant_kernel<kModeBlockStats>, grid, block, 0, stream, kv, g, tab,
                           anchor, residual, gmin, gscale, mu, sigma);
        break;
    }
    return hipGetLastError();
}

}  // namespace lynx
