// gfx950 dequantize kernels: the anchor phase and the residual phase of the
// Lynx decode workflow ("Lynx: Progressive Speculative Quantization for
// accelerating KV Transfer in Long-Context Inference", Section 4.2,
// Figure 7(b) and 7(c)).  Each workgroup rebuilds one 256 x 128 page block
// from its nibble streams and metadata and writes token-major bf16 rows.
//
// Per element: code from the anchor nibble (anchor-only: magnitude << 4) or
// from anchor and residual nibbles (full: (magnitude << 4) - residual),
// signed level S * L[code] from a 16- or 256-entry LDS table indexed by the
// raw nibbles, then the literal inverse of Algorithm 1's two scalings,
//   x^ = ((S L[code]) * (sigma + eps) + mu) * (gamma_scale + eps) + gamma_min,
// four binary32 roundings, then bf16 round-to-nearest-even
// (v_cvt_pk_bf16_f32).
//
// Lane mapping: 256 lanes per page block; lane 16 t + g of wave w owns
// channels 8g..8g+7 of tokens 64w + 16t .. +15 (inside one chunk), so it
// needs the metadata of 8 channels of one chunk only, reads its codes as
// four 16-byte runs of the chunk-tiled streams (one per channel pair) and
// writes 16-byte row pieces that 16 lanes join into one 256-byte row.
// Workgroups are persistent and build the level table in LDS once.
// Other field widths (ABITS anchor bits, RBITS residual bits: the other
// splits of the 8-bit code, or RBITS = 0 for a single stream of whole codes)
// read the lane's fields from the per-(chunk, pair) bit-stream runs: the
// lane's 16 tokens of a pair are ABITS (RBITS) consecutive dwords.
#include "lynx_recon.h"

namespace lynx {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
// Copies of the full (anchor, residual) level table, interleaved word by
// word; lane l reads copy l % kCopies, so lanes of a wave looking up
// different entries spread over the LDS banks.
constexpr int kCopies = 1;

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

// M16: bfloat16 metadata (the four arrays hold bfloat16 bit patterns).
template <bool FULL, int ABITS, int RBITS, bool M16 = false>
__global__ __launch_bounds__(kThreads) void dequant_kernel(
    const uint8_t *__restrict__ anchor, const uint8_t *__restrict__ residual,
    const float *__restrict__ gmin, const float *__restrict__ gscale,
    const float *__restrict__ mu, const float *__restrict__ sigma, Geometry g,
    const DequantTab tab, uint16_t *__restrict__ out) {
    constexpr int kBits = RBITS;
    constexpr bool kNibbles = ABITS == 4 && RBITS == 4;
    static_assert(!FULL || RBITS > 0, "a single stream has no residual phase");
    constexpr int kLut = FULL ? 256 : (1 << ABITS);
    constexpr int kCop = FULL ? kCopies : 1;
    __shared__ float s_lut[kLut * kCop];

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int cg = lane & 15;      // channels 8 cg .. 8 cg + 7
    const int tg = lane >> 4;      // tokens 64 wave + 16 tg .. + 15
    const int j = 2 * wave + (tg >> 1);  // chunk of those tokens
    const int tok0 = 64 * wave + 16 * tg;

    // Signed level of every (anchor nibble, residual nibble) pair.
    for (int e = tid; e < kLut * kCop; e += kThreads)
        s_lut[e] = kNibbles ? signed_level(tab, e / kCop, FULL)
                            : signed_level_bits(tab, e / kCop, FULL, ABITS, RBITS);
    __syncthreads();
    const float *lut = s_lut + (lane % kCop);

    for (int64_t u = __builtin_amdgcn_workgroup_id_x(); u < g.nblocks; u += g.grid_wgs) {
        const int64_t b = g.block0 + u;
        const int head = (int)(b % g.heads);
        const int64_t tp = b / g.heads;
        const int page = (int)(tp % g.pages);
        const int64_t tensor = tp / g.pages;
        uint16_t *obase = out + tensor * g.tensor_stride + (int64_t)page * kPage * g.row_stride +
                          head * kHead + cg * 8;

        // Chunk-tiled streams: the 16 bytes of channel pair 4 cg + k for the
        // lane's 16 tokens sit at [chunk j][pair][16 (tg & 1)].  Each
        // 128-byte line of a tile is read in four 16-byte pieces by
        // successive loads, so these are ordinary (cached) loads.  Other
        // splits: the pair's run of 8 w bytes, dwords w (tg & 1) .. + w - 1.
        u32x4 A[4], R[4];
        uint32_t Aw[4][kNibbles ? 1 : ABITS], Rw[4][kNibbles || kBits == 0 ? 1 : kBits];
        if constexpr (kNibbles) {
            const int64_t coff = b * (kPage * kHead / 2) + j * (kHead / 2 * kChunk) +
                                 (4 * cg) * kChunk + 16 * (tg & 1);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                A[k] = *((const u32x4 *)(anchor + coff + k * kChunk));
                if (FULL)
                    R[k] = *((const u32x4 *)(residual + coff + k * kChunk));
            }
        } else {
            const uint32_t *ar = (const uint32_t *)(anchor + b * (kPage * kHead / 8 * ABITS) +
                                                    (int64_t)(j * (kHead / 2) + 4 * cg) *
                                                        (8 * ABITS)) +
                                 ABITS * (tg & 1);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
#pragma unroll
                for (int d = 0; d < ABITS; ++d) Aw[k][d] = ar[k * 2 * ABITS + d];
            }
            if constexpr (FULL) {
                const uint32_t *rr =
                    (const uint32_t *)(residual + b * (kPage * kHead / 8 * kBits) +
                                       (int64_t)(j * (kHead / 2) + 4 * cg) * (8 * kBits)) +
                    kBits * (tg & 1);
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int d = 0; d < kBits; ++d) Rw[k][d] = rr[k * 2 * kBits + d];
            }
        }
        float4 m0, m1, c0, c1, u0, u1, q0, q1;
        const int64_t goff = b * kHead + cg * 8;
        const int64_t coff8 = b * (kChunks * kHead) + j * kHead + cg * 8;
        if constexpr (M16) {
            // 8 channels = 16 bytes of bfloat16 per array
            auto widen = [](const float *base, int64_t off, float4 &lo, float4 &hi) {
                const u32x4 w = *(const u32x4 *)((const uint16_t *)base + off);
                lo = make_float4(__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                                 __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u));
                hi = make_float4(__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xffff0000u),
                                 __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xffff0000u));
            };
            widen(gmin, goff, m0, m1);
            widen(gscale, goff, c0, c1);
            widen(mu, coff8, u0, u1);
            widen(sigma, coff8, q0, q1);
        } else {
            const float4 *gm4 = (const float4 *)(gmin + goff);
            const float4 *gs4 = (const float4 *)(gscale + goff);
            const float4 *mu4 = (const float4 *)(mu + coff8);
            const float4 *sg4 = (const float4 *)(sigma + coff8);
            m0 = gm4[0], m1 = gm4[1], c0 = gs4[0], c1 = gs4[1];
            u0 = mu4[0], u1 = mu4[1], q0 = sg4[0], q1 = sg4[1];
        }
        const float gm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
        const float um[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
        const float d1[8] = {c0.x + tab.eps, c0.y + tab.eps, c0.z + tab.eps, c0.w + tab.eps,
                             c1.x + tab.eps, c1.y + tab.eps, c1.z + tab.eps, c1.w + tab.eps};
        const float d2[8] = {q0.x + tab.eps, q0.y + tab.eps, q0.z + tab.eps, q0.w + tab.eps,
                             q1.x + tab.eps, q1.y + tab.eps, q1.z + tab.eps, q1.w + tab.eps};

#pragma unroll
        for (int h = 0; h < 4; ++h) {  // tokens 4h .. 4h+3 of the lane's 16
            // byte i of ev[k] / od[k] = (anchor nibble) | (residual nibble << 4)
            // of channel 2k / 2k+1 at token 4h + i.
            uint32_t ev[4], od[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (!kNibbles) {
                    ev[k] = od[k] = 0u;
                } else if (FULL) {
                    ev[k] = (A[k][h] & 0x0f0f0f0fu) | ((R[k][h] << 4) & 0xf0f0f0f0u);
                    od[k] = ((A[k][h] >> 4) & 0x0f0f0f0fu) | (R[k][h] & 0xf0f0f0f0u);
                } else {
                    ev[k] = A[k][h] & 0x0f0f0f0fu;
                    od[k] = (A[k][h] >> 4) & 0x0f0f0f0fu;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float y[8];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
#pragma unroll
                    for (int o = 0; o < 2; ++o) {
                        const int e = 2 * k + o;
                        uint32_t idx;
                        if constexpr (kNibbles) {
                            idx = ((o ? od[k] : ev[k]) >> (8 * i)) & 0xffu;
                        } else {
                            // field of token 4h + i, channel 2k + o of the run
                            const int v = 2 * (4 * h + i) + o;
                            idx = get_field<ABITS>(Aw[k], v);
                            if constexpr (FULL)
                                idx |= get_field<kBits>(Rw[k], v) << ABITS;
                        }
                        y[e] = reconstruct(lut[idx * kCop], d2[e], um[e], d1[e], gm[e]);
                    }
                }
                u32x4 o4;
                o4[0] = pack_bf16(y[0], y[1]);
                o4[1] = pack_bf16(y[2], y[3]);
                o4[2] = pack_bf16(y[4], y[5]);
                o4[3] = pack_bf16(y[6], y[7]);
                __builtin_nontemporal_store(
                    o4, (u32x4 *)(obase + (int64_t)(tok0 + 4 * h + i) * g.row_stride));
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
    gl.grid_wgs = g.nblocks;
    hipLaunchKernelGGL((dequant_kernel<FULL, ABITS, RBITS, M16>), dim3((unsigned)gl.grid_wgs),
                       dim3(kThreads), 0, stream, anchor, residual, gmin, gscale, mu, sigma, gl,
                       tab, out);
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
