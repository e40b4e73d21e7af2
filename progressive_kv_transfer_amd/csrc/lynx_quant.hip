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
// Each lane owns one whole 32-token chunk of a channel pair (64 values), so
// the chunk mean and max |X - mu| need no cross-lane traffic and every
// per-channel cost is spread over 32 tokens.  A workgroup of 256 lanes
// covers half a page block (64 channels x 256 tokens); its lanes meet once
// in LDS for the page minimum / maximum.  Rows are read with buffer loads
// (scalar row offsets): 32 lanes x 4 bytes = one 128-byte line per row.
// The loads go straight to LDS (buffer_load_dword ... lds), one unit ahead:
// each wave stages the 32 rows of its next unit in its own 8 KiB region
// while it computes the current one, so HBM latency overlaps a whole unit
// of arithmetic without holding registers.
// The anchor and residual bytes of a lane are 32 contiguous bytes of the
// chunk-tiled stream layout, so a workgroup writes whole cache lines that no
// other workgroup touches.  Workgroups are persistent (grid = resident
// workgroups) and build the compander table in LDS once.
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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Correctly rounded a / d in the fast domain (see the file comment).
__device__ __forceinline__ float div_fast(float a, float d, float r) {
    float q = a * r;
    float e = __builtin_fmaf(-q, d, a);
    return __builtin_fmaf(e, r, q);
}

constexpr float kTiny100 = 0x1p-100f;
constexpr float kTiny125 = 0x1p-125f;
constexpr float kHuge125 = 0x1p125f;
constexpr float kMuTiny = 0x1p-74f;

// Lane tile: 2 channels x 32 tokens, i.e. one whole chunk of a channel
// pair.  A work unit is half a page block (64 channels x 256 tokens;
// statistics are per channel, so the halves are independent); unit u is
// half (u & 1) of block block0 + (u >> 1).  A workgroup (4 wave64s) walks
// units u = workgroup, workgroup + grid, ... so the compander table is
// built once per workgroup.
constexpr int kHalf = kHead / 2;        // channels per unit
constexpr int kPairs = kHalf / 2;       // channel pairs per unit (lanes per chunk)
constexpr int kThreads = kPairs * kChunks;  // 256

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff,
                                             0x00020000);
}

// SH16: the compander buckets are the upper 16 bits of the magnitude, so the
// table address is one v_mad_u32_u16 (high half x 8 + base).
template <int MODE, bool SH16>
__global__ __launch_bounds__(kThreads) void quant_kernel(
    const uint16_t *__restrict__ kv, Geometry g, const QuantTab tab,
    uint8_t *__restrict__ anchor, uint8_t *__restrict__ residual, float *__restrict__ gmin_io,
    float *__restrict__ gscale_io, float *__restrict__ mu_out, float *__restrict__ sigma_out) {
    __shared__ float2 s_min[kChunks][kPairs];
    __shared__ float2 s_max[kChunks][kPairs];
    __shared__ float4 s_ch[kHalf];  // gamma_min, d1, r1, slow flag
    __shared__ u32x2 s_tab[MODE == kModeQuantize ? kMaxBuckets : 1];
    // Staged rows of the next unit: [wave][row of chunk][lane].
    __shared__ uint32_t s_stage[kThreads / 64][kChunk][64];

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int p = tid & (kPairs - 1);  // channel pair: channels 2p, 2p+1 of the unit
    const int j = tid / kPairs;        // chunk: tokens 32 j .. 32 j + 31
    const int wave = tid >> 6;
    const int lane = tid & 63;

    // Compander table into LDS, once per workgroup.
    if (MODE == kModeQuantize) {
        for (int i = tid; i < tab.nbuckets; i += kThreads) {
            uint32_t c = tab.bucket_code[i];
            s_tab[i] = u32x2{__float_as_uint(tab.thr[c + 1]), c + 7u};
        }
    }
    typedef __attribute__((address_space(3))) const u32x2 lds_u32x2;
    const float mag_lo = __uint_as_float((uint32_t)tab.bucket_lo << tab.shift);
    const uint32_t sh = (uint32_t)tab.shift;
    const uint32_t tab_base = (uint32_t)(uintptr_t)(lds_u32x2 *)s_tab -
                              (uint32_t)tab.bucket_lo * (uint32_t)sizeof(u32x2);
    const uint32_t row_bytes = (uint32_t)g.row_stride * 2u;
    const int64_t nunits = 2 * g.nblocks;
    const uint32_t voff = (uint32_t)(j * kChunk) * row_bytes + (uint32_t)p * 4u;

    // First element of unit v in the KV set.
    auto unit_base = [&](int64_t v) {
        const int64_t bv = g.block0 + (v >> 1);
        const int64_t tpv = bv / g.heads;
        return kv + (tpv / g.pages) * g.tensor_stride +
               (int64_t)(tpv % g.pages) * kPage * g.row_stride + (bv % g.heads) * kHead +
               (v & 1) * kHalf;
    };
    // Issue the 32 row loads (4 B per lane: channels 2p, 2p+1 of the unit,
    // tokens 32 j + i) of the unit at bp into this wave's staging rows.
    typedef __attribute__((address_space(3))) void lds_void;
    // LDS address of this wave's staging rows, as a wave-uniform scalar.
    const uint32_t stage_lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds_void *)&s_stage[wave][0][0]);
    // The row offsets are stepped with opaque scalar adds so that the 64
    // per-row constants are not hoisted out of the unit loop into SGPRs.
    auto stage = [&](const uint16_t *bp) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(bp);
        uint32_t soff = 0, lds = stage_lds;
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(uintptr_t)lds, 4, voff,
                                                     soff, 0, 0);
            asm volatile("s_add_u32 %0, %0, %1" : "+s"(soff) : "s"(row_bytes));
            asm volatile("s_add_u32 %0, %0, 0x100" : "+s"(lds));
        }
    };
    if ((int64_t)__builtin_amdgcn_workgroup_id_x() < nunits)
        stage(unit_base(__builtin_amdgcn_workgroup_id_x()));

    for (int64_t u = __builtin_amdgcn_workgroup_id_x(); u < nunits;
         u += g.grid_wgs) {
        const int64_t b = g.block0 + (u >> 1);
        const int half = (int)(u & 1);
        const int64_t meta0 = b * kHead + half * kHalf;
        const int64_t cmeta0 = b * (kChunks * kHead) + j * kHead + half * kHalf;
        // Address of the next unit, computed here where few registers are
        // live (the empty asm keeps it from being sunk to its use).
        const bool has_next = u + g.grid_wgs < nunits;
        const uint16_t *next_base = has_next ? unit_base(u + g.grid_wgs) : kv;
        asm volatile("" ::"s"(next_base));

        // ---- 32 token rows x 2 channels (4 B per row) from the stage -----
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        uint32_t raw[kChunk];
#pragma unroll
        for (int i = 0; i < kChunk; ++i) raw[i] = s_stage[wave][i][lane];
        float x[kChunk][2];
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            x[i][0] = bf16_lo(raw[i]);
            x[i][1] = bf16_hi(raw[i]);
        }
        // The staging rows are refilled now: all reads of them have
        // returned (their values are used above).
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (has_next)
            stage(next_base);

        // ---- phase 1: page statistics ------------------------------------
        if (MODE != kModeBlockStats) {
            float mn[2], mx[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                mn[e] = x[0][e];
                mx[e] = x[0][e];
#pragma unroll
                for (int i = 1; i < kChunk; ++i) {
                    mn[e] = fminf(mn[e], x[i][e]);
                    mx[e] = fmaxf(mx[e], x[i][e]);
                }
            }
            s_min[j][p] = make_float2(mn[0], mn[1]);
            s_max[j][p] = make_float2(mx[0], mx[1]);
        }
        __syncthreads();
        if (tid < kHalf) {
            float gmin, gsc;
            if (MODE == kModeBlockStats) {
                gmin = gmin_io[meta0 + tid];
                gsc = gscale_io[meta0 + tid];
            } else {
                const float *mn = (const float *)&s_min[0][0] + tid;
                const float *mx = (const float *)&s_max[0][0] + tid;
                float a = mn[0], m = mx[0];
#pragma unroll
                for (int w = 1; w < kChunks; ++w) {
                    a = fminf(a, mn[w * kHalf]);
                    m = fmaxf(m, mx[w * kHalf]);
                }
                gmin = a + 0.0f;  // canonical +0 for a zero minimum
                gsc = m - gmin;
                gmin_io[meta0 + tid] = gmin;
                gscale_io[meta0 + tid] = gsc;
            }
            float d1 = gsc + tab.eps;
            float r1 = __fdiv_rn(1.0f, d1);
            // Every nonzero x - gamma_min of a bf16 channel is at least
            // 2^-9 |gamma_min|; the fast division needs it above the bound.
            bool fast = gmin != 0.0f &&
                        fabsf(gmin) * 0x1p-9f >= fmaxf(kTiny100, d1 * kTiny125) &&
                        d1 < kHuge125;
            s_ch[tid] = make_float4(gmin, d1, r1, fast ? 0.0f : 1.0f);
        }
        if (MODE == kModePageStats) {
            __syncthreads();  // s_min is rewritten by the next unit
            continue;
        }
        __syncthreads();

        // ---- phase 2: normalise, chunk mean and max |X - mu| -------------
        {
            const float4 c0 = s_ch[2 * p], c1 = s_ch[2 * p + 1];
            const float gm[2] = {c0.x, c1.x}, d1[2] = {c0.y, c1.y}, r1[2] = {c0.z, c1.z};
            if (c0.w == 0.0f && c1.w == 0.0f) {
#pragma unroll
                for (int i = 0; i < kChunk; ++i)
#pragma unroll
                    for (int e = 0; e < 2; ++e) x[i][e] = div_fast(x[i][e] - gm[e], d1[e], r1[e]);
            } else {
                // Rare path; the scheduling barriers keep its register
                // footprint below the fast path's.
#pragma unroll
                for (int i = 0; i < kChunk; ++i)
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        x[i][e] = __fdiv_rn(x[i][e] - gm[e], d1[e]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
            }
        }
        float mu[2], sg[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            // balanced pairwise tree over the 32 tokens of the chunk
            float t16[16], t8[8], t4[4];
#pragma unroll
            for (int k = 0; k < 16; ++k) t16[k] = x[2 * k][e] + x[2 * k + 1][e];
#pragma unroll
            for (int k = 0; k < 8; ++k) t8[k] = t16[2 * k] + t16[2 * k + 1];
#pragma unroll
            for (int k = 0; k < 4; ++k) t4[k] = t8[2 * k] + t8[2 * k + 1];
            float s32 = (t4[0] + t4[1]) + (t4[2] + t4[3]);
            mu[e] = s32 * 0.03125f;
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < kChunk; ++i) {
                x[i][e] = x[i][e] - mu[e];
                m = fmaxf(m, fabsf(x[i][e]));
            }
            sg[e] = m;
        }
        *(float2 *)(mu_out + cmeta0 + 2 * p) = make_float2(mu[0], mu[1]);
        *(float2 *)(sigma_out + cmeta0 + 2 * p) = make_float2(sg[0], sg[1]);
        if (MODE == kModeBlockStats)
            continue;

        // ---- phase 3: scale, compand, split, pack -------------------------
        {
            const float d2[2] = {sg[0] + tab.eps, sg[1] + tab.eps};
            const bool slow2 = (mu[0] > 0.0f && mu[0] < kMuTiny) || (mu[1] > 0.0f && mu[1] < kMuTiny);
            if (slow2) {
                // IEEE quotient; + 0 turns a -0 quotient into +0 so that the
                // sign bit below is exactly [X_cent < 0].
#pragma unroll
                for (int i = 0; i < kChunk; ++i)
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        x[i][e] = __fdiv_rn(x[i][e], d2[e]) + 0.0f;
                        __builtin_amdgcn_sched_barrier(0);
                    }
            } else {
                const float r2[2] = {__fdiv_rn(1.0f, d2[0]), __fdiv_rn(1.0f, d2[1])};
#pragma unroll
                for (int i = 0; i < kChunk; ++i)
#pragma unroll
                    for (int e = 0; e < 2; ++e) x[i][e] = div_fast(x[i][e], d2[e], r2[e]);
            }
        }
        // Magnitudes are clamped into [first value of the lowest bucket, 1]
        // (every finite |X_final| is <= 1; the lower clamp keeps code 0
        // since that bucket starts below the first threshold, and
        // non-finite inputs stay inside the table).  The bucket offset is
        // folded into the LDS base address.
        u32x4 av[2], rv[2];
#pragma unroll
        for (int q = 0; q < 8; ++q) {  // tokens 4q .. 4q+3
            uint32_t J[4][2];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    float m = __builtin_amdgcn_fmed3f(fabsf(x[4 * q + k][e]), mag_lo, 1.0f);
                    uint32_t mb = __float_as_uint(m);
                    uint32_t addr;
                    if (SH16)
                        asm("v_mad_u32_u16 %0, %1, 8, %2 op_sel:[1,0,0,0]"
                            : "=v"(addr) : "v"(mb), "s"(tab_base));
                    else
                        asm("v_lshl_add_u32 %0, %1, 3, %2" : "=v"(addr) : "v"(mb >> sh), "s"(tab_base));
                    u32x2 ent = *(lds_u32x2 *)(uintptr_t)addr;
                    // J = code + 7: high nibble = anchor magnitude
                    // (code + 7) >> 4, low nibble ^ 7 = residual (-code) mod 16.
                    J[k][e] = ent[1] + (mb >= ent[0] ? 1u : 0u);
                }
            }
            // byte k of w0 / w1 = J of channel 2p / 2p+1 at token 4q + k
            uint32_t w0 = J[0][0] | (J[1][0] << 8) | (J[2][0] << 16) | (J[3][0] << 24);
            uint32_t w1 = J[0][1] | (J[1][1] << 8) | (J[2][1] << 16) | (J[3][1] << 24);
            uint32_t a = ((w0 >> 4) & 0x0f0f0f0fu) | (w1 & 0xf0f0f0f0u);
            uint32_t r = ((w0 & 0x0f0f0f0fu) | ((w1 << 4) & 0xf0f0f0f0u)) ^ 0x77777777u;
            // Sign bits of the quotients replicated to bytes (v_perm
            // selectors 9 and 11), then to nibbles: the anchor of a negative
            // value is the one's complement of its magnitude (-V - 1).
            const uint32_t *xa = (const uint32_t *)x[4 * q];
            const uint32_t *xb = (const uint32_t *)x[4 * q + 1];
            const uint32_t *xc = (const uint32_t *)x[4 * q + 2];
            const uint32_t *xd = (const uint32_t *)x[4 * q + 3];
            uint32_t n0 = __builtin_amdgcn_perm(xb[0], xa[0], 0x0c0c0b09u) |
                          __builtin_amdgcn_perm(xd[0], xc[0], 0x0b090c0cu);
            uint32_t n1 = __builtin_amdgcn_perm(xb[1], xa[1], 0x0c0c0b09u) |
                          __builtin_amdgcn_perm(xd[1], xc[1], 0x0b090c0cu);
            a ^= (n0 & 0x0f0f0f0fu) | (n1 & 0xf0f0f0f0u);
            av[q >> 2][q & 3] = a;
            rv[q >> 2][q & 3] = r;
        }
        // 32 contiguous bytes per stream: [chunk j][pair][token of chunk]
        const int64_t coff = b * (kPage * kHead / 2) + j * (kHead / 2 * kChunk) +
                             (half * kPairs + p) * kChunk;
        u32x4 *ao = (u32x4 *)(anchor + coff);
        u32x4 *ro = (u32x4 *)(residual + coff);
        // Ordinary stores: the streams are read again by the dequant kernels.
        ao[0] = av[0];
        ao[1] = av[1];
        ro[0] = rv[0];
        ro[1] = rv[1];
    }
}

}  // namespace

// Workgroups resident on the device (per kernel variant), cached per device.
static int resident_workgroups(const void *kernel, int slot, int threads) {
    static int cache[64][4];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 1024;
    if (cache[dev][slot] == 0) {
        int cus = 0, per_cu = 0;
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0);
        cache[dev][slot] = (cus > 0 ? cus : 256) * (per_cu > 0 ? per_cu : 1);
    }
    return cache[dev][slot];
}

template <int MODE, bool SH16>
static hipError_t launch_variant(int slot, const uint16_t *kv, const Geometry &g,
                                 const QuantTab &tab, uint8_t *anchor, uint8_t *residual,
                                 float *gmin, float *gscale, float *mu, float *sigma,
                                 hipStream_t stream) {
    const int64_t units = 2 * g.nblocks;
    const int64_t res =
        resident_workgroups((const void *)quant_kernel<MODE, SH16>, slot, kThreads);
    Geometry gl = g;
    gl.grid_wgs = units < res ? units : res;
    hipLaunchKernelGGL((quant_kernel<MODE, SH16>), dim3((unsigned)gl.grid_wgs), dim3(kThreads),
                       0, stream, kv, gl, tab, anchor, residual, gmin, gscale, mu, sigma);
    return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t *kv, const Geometry &g, const QuantTab &tab,
                           uint8_t *anchor, uint8_t *residual, float *gmin, float *gscale,
                           float *mu, float *sigma, int mode, hipStream_t stream) {
    if (g.nblocks == 0)
        return hipSuccess;
    switch (mode) {
    case kModeQuantize:
        if (tab.shift == 16)
            return launch_variant<kModeQuantize, true>(0, kv, g, tab, anchor, residual, gmin,
                                                       gscale, mu, sigma, stream);
        return launch_variant<kModeQuantize, false>(1, kv, g, tab, anchor, residual, gmin,
                                                    gscale, mu, sigma, stream);
    case kModePageStats:
        return launch_variant<kModePageStats, false>(2, kv, g, tab, anchor, residual, gmin,
                                                     gscale, mu, sigma, stream);
    default:
        return launch_variant<kModeBlockStats, false>(3, kv, g, tab, anchor, residual, gmin,
                                                      gscale, mu, sigma, stream);
    }
}

}  // namespace lynx
