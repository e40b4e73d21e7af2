// gfx950 dequantize kernels: the anchor phase and the residual phase of the
// Lynx decode workflow ("Lynx: Progressive Speculative Quantization for
// accelerating KV Transfer in Long-Context Inference", Section 4.2,
// Figure 7(b) and 7(c)): page blocks rebuilt from their streams and
// metadata into token-major bf16 rows.
//
// Per element: code from the anchor field (anchor-only: magnitude << b) or
// from anchor and residual fields (full: (magnitude << b) - residual),
// signed level S * L[code] from a 16- or 256-entry LDS table indexed by the
// raw fields, then the literal inverse of Algorithm 1's two scalings,
//   x^ = ((S L[code]) * (sigma + eps) + mu) * (gamma_scale + eps) + gamma_min,
// four binary32 roundings, then bf16 round-to-nearest-even
// (v_cvt_pk_bf16_f32).
//
// Lane mapping: a lane owns one channel pair of one 32-token chunk of one
// page block.  Its codes are the pair's run of the chunk-tiled streams (32
// contiguous bytes per 4-bit stream, 8 w bytes for w-bit fields: a wave
// reads whole tiles), its metadata two floats per array, and every token row
// is one 4-byte store (the 64 lanes of a wave write the block's 256-byte
// piece of the row).  A workgroup of 8 waves takes the same chunk of HW
// neighbouring heads (HW = 8, 4, 2 or 1, the largest dividing the head
// count) times 8 / HW chunks, so it writes whole HW x 256-byte row spans:
// with 8 heads of 128 channels, 32 complete 2 KB rows.  Workgroups go to
// the XCDs in contiguous runs.  Measured on the 16K Qwen-32B-shaped set:
// this layout took the anchor dequant from 1.12 to 1.04 ms and the full one
// from 1.32 to 1.24 ms against the earlier one-block-per-workgroup kernel
// (16-byte row pieces).
#include "lynx_device.h"
#include "lynx_recon.h"

namespace lynx {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Signed level S * L[code] of table entry t for a anchor bits and b residual
// bits: t's low a bits are the anchor field, the next b the residual field
// (full), as signed_level does for a = b = 4.
__device__ __forceinline__ float signed_level_bits(const DequantTab &tab, int t, bool full,
                                                   int abits, int bbits) {
    const int af = t & ((1 << abits) - 1);
    const int av = af >= (1 << (abits - 1)) ? af - (1 << abits) : af;
    const int v = av < 0 ? -av - 1 : av;
    int code = v << bbits;
    if (full) {
        const int rf = (t >> abits) & ((1 << bbits) - 1);
        code -= rf >= (1 << (bbits - 1)) ? rf - (1 << bbits) : rf;
        code = code < 0 ? 0 : code;
    }
    const float m = tab.level[code];
    return av < 0 ? -m : m;
}

// W-bit field v of an LSB-first bit stream held in dwords (v a compile-time
// constant after unrolling).
template <int W>
__device__ __forceinline__ uint32_t get_field(const uint32_t *w, int v) {
    const int pos = W * v, d = pos >> 5, s = pos & 31;
    uint32_t f = w[d] >> s;
    if (s + W > 32)
        f |= w[d + 1] << (32 - s);
    return f & ((1u << W) - 1u);
}

constexpr int kWaves = 8;  // waves per workgroup = (head, chunk) items

// M16: bfloat16 metadata (the four arrays hold bfloat16 bit patterns).
template <bool FULL, int ABITS, int RBITS, bool M16 = false>
__global__ __launch_bounds__(64 * kWaves) void dequant_kernel(
    const uint8_t *__restrict__ anchor, const uint8_t *__restrict__ residual,
    const float *__restrict__ gmin, const float *__restrict__ gscale,
    const float *__restrict__ mu, const float *__restrict__ sigma, Geometry g,
    const DequantTab tab, uint16_t *__restrict__ out) {
    constexpr int kBits = RBITS;
    constexpr bool kNibbles = ABITS == 4 && RBITS == 4;
    static_assert(!FULL || RBITS > 0, "a single stream has no residual phase");
    constexpr int kLut = FULL ? 256 : (1 << ABITS);
    __shared__ float s_lut[kLut];

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int wave = tid >> 6;
    const int p = tid & 63;  // channel pair: channels 2p, 2p + 1 of the block

    // Signed level of every (anchor field, residual field) pair.
    for (int e = tid; e < kLut; e += 64 * kWaves)
        s_lut[e] = kNibbles ? signed_level(tab, e, FULL)
                            : signed_level_bits(tab, e, FULL, ABITS, RBITS);
    __syncthreads();

    // Workgroup shape: HW heads x CW chunks (whole pages only; a launch that
    // starts or ends inside a page takes the 8 chunks of one block).
    const bool pages = g.block0 % g.heads == 0 && g.nblocks % g.heads == 0;
    const int HW = !pages ? 1 : g.heads % 8 == 0 ? 8 : g.heads % 4 == 0 ? 4
                          : g.heads % 2 == 0 ? 2 : 1;
    const int CW = kWaves / HW;
    const int64_t groups = g.heads / HW;
    for (int64_t u = __builtin_amdgcn_workgroup_id_x(); u < g.nblocks; u += g.grid_wgs) {
        // unit v = ((tensor, page), chunk group, head group) (HW > 1) or a
        // block (HW = 1); the launch has one unit per page block
        const int64_t v = xcd_unit(u, g.nblocks);
        int64_t lb;
        int j;
        if (HW == 1) {
            lb = v;
            j = wave;
        } else {
            const int64_t hq = v % groups, rest = v / groups;
            j = CW * (int)(rest % HW) + wave / HW;
            lb = (rest / HW) * g.heads + HW * hq + wave % HW;
        }
        const int64_t b = g.block0 + lb;
        const int head = (int)(b % g.heads);
        const int64_t tp = b / g.heads;
        const int page = (int)(tp % g.pages);
        const int64_t tensor = tp / g.pages;
        uint16_t *obase = out + tensor * g.tensor_stride +
                          (int64_t)(page * kPage + j * kChunk) * g.row_stride + head * kHead +
                          2 * p;

        // The pair's run of 64 fields (token i, channel 2p + e = field 2i + e)
        // in each stream: ABITS (RBITS) x 8 bytes.
        uint32_t aw[2 * ABITS], rw[kBits > 0 ? 2 * kBits : 1];
        {
            const u32x4 *ap = (const u32x4 *)(anchor + b * g.astride +
                                             (int64_t)(j * (kHead / 2) + p) * (8 * ABITS));
#pragma unroll
            for (int d = 0; d < ABITS / 2; ++d) {
                const u32x4 t = ap[d];
#pragma unroll
                for (int k = 0; k < 4; ++k) aw[4 * d + k] = t[k];
            }
            if constexpr (ABITS & 1) {
                const u32x2 t = *(const u32x2 *)(ap + ABITS / 2);
                aw[2 * ABITS - 2] = t[0];
                aw[2 * ABITS - 1] = t[1];
            }
            if constexpr (FULL) {
                const u32x4 *rp = (const u32x4 *)(residual + b * (kPage * kHead / 8 * kBits) +
                                                 (int64_t)(j * (kHead / 2) + p) * (8 * kBits));
#pragma unroll
                for (int d = 0; d < kBits / 2; ++d) {
                    const u32x4 t = rp[d];
#pragma unroll
                    for (int k = 0; k < 4; ++k) rw[4 * d + k] = t[k];
                }
                if constexpr (kBits & 1) {
                    const u32x2 t = *(const u32x2 *)(rp + kBits / 2);
                    rw[2 * kBits - 2] = t[0];
                    rw[2 * kBits - 1] = t[1];
                }
            }
        }
        float gm[2], um[2], d1[2], d2[2];
        {
            const int64_t goff = b * g.gstride + 2 * p;
            const int64_t coff = b * g.cstride + j * kHead + 2 * p;
            if constexpr (M16) {
                auto lo = [](uint32_t w) { return __uint_as_float(w << 16); };
                auto hi = [](uint32_t w) { return __uint_as_float(w & 0xffff0000u); };
                const uint32_t wg = *(const uint32_t *)((const uint16_t *)gmin + goff);
                const uint32_t ws = *(const uint32_t *)((const uint16_t *)gscale + goff);
                const uint32_t wm = *(const uint32_t *)((const uint16_t *)mu + coff);
                const uint32_t wq = *(const uint32_t *)((const uint16_t *)sigma + coff);
                gm[0] = lo(wg);
                gm[1] = hi(wg);
                d1[0] = lo(ws) + tab.eps;
                d1[1] = hi(ws) + tab.eps;
                um[0] = lo(wm);
                um[1] = hi(wm);
                d2[0] = lo(wq) + tab.eps;
                d2[1] = hi(wq) + tab.eps;
            } else {
                const float2 fg = *(const float2 *)(gmin + goff);
                const float2 fs = *(const float2 *)(gscale + goff);
                const float2 fm = *(const float2 *)(mu + coff);
                const float2 fq = *(const float2 *)(sigma + coff);
                gm[0] = fg.x;
                gm[1] = fg.y;
                d1[0] = fs.x + tab.eps;
                d1[1] = fs.y + tab.eps;
                um[0] = fm.x;
                um[1] = fm.y;
                d2[0] = fq.x + tab.eps;
                d2[1] = fq.y + tab.eps;
            }
        }
#pragma unroll
        for (int q = 0; q < kChunk / 4; ++q) {  // tokens 4q .. 4q + 3
            // 4-bit fields: byte i of ev / od = (anchor nibble) | (residual
            // nibble << 4) of channel 2p / 2p + 1 at token 4q + i
            uint32_t ev = 0u, od = 0u;
            if constexpr (kNibbles) {
                const uint32_t A = aw[q];
                if constexpr (FULL) {
                    const uint32_t R = rw[q];
                    ev = (A & 0x0f0f0f0fu) | ((R << 4) & 0xf0f0f0f0u);
                    od = ((A >> 4) & 0x0f0f0f0fu) | (R & 0xf0f0f0f0u);
                } else {
                    ev = A & 0x0f0f0f0fu;
                    od = (A >> 4) & 0x0f0f0f0fu;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float y[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    uint32_t idx;
                    if constexpr (kNibbles) {
                        idx = ((e ? od : ev) >> (8 * i)) & 0xffu;
                    } else {
                        const int fv = 2 * (4 * q + i) + e;
                        idx = get_field<ABITS>(aw, fv);
                        if constexpr (FULL)
                            idx |= get_field<kBits>(rw, fv) << ABITS;
                    }
                    y[e] = reconstruct(s_lut[idx], d2[e], um[e], d1[e], gm[e]);
                }
                __builtin_nontemporal_store(
                    pack_bf16(y[0], y[1]), (uint32_t *)(obase + (int64_t)(4 * q + i) * g.row_stride));
            }
        }
    }
}

}  // namespace

template <bool FULL, int ABITS, int RBITS, bool M16>
static hipError_t launch_one(const uint8_t *anchor, const uint8_t *residual,
                             const float *gmin, const float *gscale, const float *mu,
                             const float *sigma, const Geometry &g, const DequantTab &tab,
                             uint16_t *out, hipStream_t stream) {
    Geometry gl = g;
    gl.grid_wgs = g.nblocks;  // one workgroup per page block's worth of units
    hipLaunchKernelGGL((dequant_kernel<FULL, ABITS, RBITS, M16>), dim3((unsigned)gl.grid_wgs),
                       dim3(64 * kWaves), 0, stream, anchor, residual, gmin, gscale, mu, sigma,
                       gl, tab, out);
    return hipGetLastError();
}

template <int ABITS, int RBITS, bool M16 = false>
static hipError_t launch_split(const uint8_t *anchor, const uint8_t *residual,
                               const float *gmin, const float *gscale, const float *mu,
                               const float *sigma, const Geometry &g, const DequantTab &tab,
                               uint16_t *out, hipStream_t stream) {
    if constexpr (RBITS > 0) {
        if (residual)
            return launch_one<true, ABITS, RBITS, M16>(anchor, residual, gmin, gscale, mu,
                                                       sigma, g, tab, out, stream);
    } else {
        if (residual)
            return hipErrorInvalidValue;
    }
    return launch_one<false, ABITS, RBITS, M16>(anchor, residual, gmin, gscale, mu, sigma, g,
                                                tab, out, stream);
}

hipError_t launch_dequant(const uint8_t *anchor, const uint8_t *residual, const float *gmin,
                          const float *gscale, const float *mu, const float *sigma,
                          const Geometry &g, const DequantTab &tab, uint16_t *out,
                          int anchor_bits, int residual_bits, int meta_bits,
                          hipStream_t stream) {
    if (g.nblocks == 0)
        return hipSuccess;
    if (meta_bits == 16) {
        if (anchor_bits != 4 || residual_bits != 4)
            return hipErrorInvalidValue;
        return launch_split<4, 4, true>(anchor, residual, gmin, gscale, mu, sigma, g, tab, out,
                                        stream);
    }
    switch (anchor_bits * 16 + residual_bits) {
    case 3 * 16 + 5:
        return launch_split<3, 5>(anchor, residual, gmin, gscale, mu, sigma, g, tab, out,
                                  stream);
    case 4 * 16 + 4:
        return launch_split<4, 4>(anchor, residual, gmin, gscale, mu, sigma, g, tab, out,
                                  stream);
    case 5 * 16 + 3:
        return launch_split<5, 3>(anchor, residual, gmin, gscale, mu, sigma, g, tab, out,
                                  stream);
    case 6 * 16 + 2:
        return launch_split<6, 2>(anchor, residual, gmin, gscale, mu, sigma, g, tab, out,
                                  stream);
    case 4 * 16 + 0:
        return launch_split<4, 0>(anchor, residual, gmin, gscale, mu, sigma, g, tab, out,
                                  stream);
    case 8 * 16 + 0:
        return launch_split<8, 0>(anchor, residual, gmin, gscale, mu, sigma, g, tab, out,
                                  stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace lynx
