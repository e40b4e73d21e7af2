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
// Lane mapping: wave w = chunk w, lane 16 s + g owns channels 8g..8g+7 of
// tokens 32w + 8s .. +7, so every lane needs the metadata of 8 channels of
// one chunk only and writes 16-byte row pieces that 16 lanes join into one
// 256-byte row.  Its codes are four 8-byte runs of the chunk-tiled streams
// (one per channel pair); the 64 lanes of a wave read each 128-byte line of
// the chunk's tile completely.
#include "lynx_internal.h"

namespace lynx {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 h = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

template <bool FULL>
__global__ __launch_bounds__(512) void dequant_kernel(
    const uint8_t *__restrict__ anchor, const uint8_t *__restrict__ residual,
    const float *__restrict__ gmin, const float *__restrict__ gscale,
    const float *__restrict__ mu, const float *__restrict__ sigma, Geometry g,
    const DequantTab tab, uint16_t *__restrict__ out) {
    constexpr int kLut = FULL ? 256 : 16;
    __shared__ float s_lut[kLut];

    const int64_t b = g.block0 + __builtin_amdgcn_workgroup_id_x();
    const int head = (int)(b % g.heads);
    const int64_t tp = b / g.heads;
    const int page = (int)(tp % g.pages);
    const int64_t tensor = tp / g.pages;
    uint16_t *obase =
        out + tensor * g.tensor_stride + (int64_t)page * kPage * g.row_stride + head * kHead;

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int cg = lane & 15;
    const int s = lane >> 4;
    const int tok0 = wave * kChunk + s * 8;

    // Chunk-tiled streams: the 8 bytes of channel pair 4 cg + k for tokens
    // 32 wave + 8 s .. + 7 sit at [chunk wave][pair][8 s].
    const int64_t coff = b * (kPage * kHead / 2) + wave * (kHead / 2 * kChunk) +
                         (4 * cg) * kChunk + 8 * s;
    u32x2 A[4], R[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        A[k] = __builtin_nontemporal_load((const u32x2 *)(anchor + coff + k * kChunk));
        if (FULL)
            R[k] = __builtin_nontemporal_load((const u32x2 *)(residual + coff + k * kChunk));
    }
    const float4 *gm4 = (const float4 *)(gmin + b * kHead + cg * 8);
    const float4 *gs4 = (const float4 *)(gscale + b * kHead + cg * 8);
    const float4 *mu4 = (const float4 *)(mu + b * (kChunks * kHead) + wave * kHead + cg * 8);
    const float4 *sg4 = (const float4 *)(sigma + b * (kChunks * kHead) + wave * kHead + cg * 8);
    float4 m0 = gm4[0], m1 = gm4[1], c0 = gs4[0], c1 = gs4[1];
    float4 u0 = mu4[0], u1 = mu4[1], q0 = sg4[0], q1 = sg4[1];
    const float gm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    const float gs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float um[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    const float sq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};

    // Signed level of every (anchor nibble, residual nibble) pair.
    if (tid < kLut) {
        int a = tid & 15;
        int av = a >= 8 ? a - 16 : a;
        int v = av < 0 ? -av - 1 : av;
        int code = v << 4;
        if (FULL) {
            int r = tid >> 4;
            code -= r >= 8 ? r - 16 : r;
            code = code < 0 ? 0 : code;
        }
        float m = tab.level[code];
        s_lut[tid] = av < 0 ? -m : m;
    }
    float d1[8], d2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        d1[e] = gs[e] + tab.eps;
        d2[e] = sq[e] + tab.eps;
    }
    __syncthreads();

    // idx[i][e]: table index of token i, channel e of the lane's 8.
    uint32_t ev[4][2], od[4][2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // byte i of ev / od = (anchor nibble) | (residual nibble << 4)
            // of channel 2k / 2k+1 at token 4h + i.
            if (FULL) {
                ev[k][h] = (A[k][h] & 0x0f0f0f0fu) | ((R[k][h] << 4) & 0xf0f0f0f0u);
                od[k][h] = ((A[k][h] >> 4) & 0x0f0f0f0fu) | (R[k][h] & 0xf0f0f0f0u);
            } else {
                ev[k][h] = A[k][h] & 0x0f0f0f0fu;
                od[k][h] = (A[k][h] >> 4) & 0x0f0f0f0fu;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t idx[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            idx[2 * k] = (ev[k][i >> 2] >> (8 * (i & 3))) & 0xffu;
            idx[2 * k + 1] = (od[k][i >> 2] >> (8 * (i & 3))) & 0xffu;
        }
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float xf = s_lut[idx[e]];
            float t1 = xf * d2[e];
            float xn = t1 + um[e];
            float t2 = xn * d1[e];
            y[e] = t2 + gm[e];
        }
        u32x4 o;
        o[0] = pack_bf16(y[0], y[1]);
        o[1] = pack_bf16(y[2], y[3]);
        o[2] = pack_bf16(y[4], y[5]);
        o[3] = pack_bf16(y[6], y[7]);
        __builtin_nontemporal_store(o, (u32x4 *)(obase + (int64_t)(tok0 + i) * g.row_stride + cg * 8));
    }
}

}  // namespace

hipError_t launch_dequant(const uint8_t *anchor, const uint8_t *residual, const float *gmin,
                          const float *gscale, const float *mu, const float *sigma,
                          const Geometry &g, const DequantTab &tab, uint16_t *out,
                          hipStream_t stream) {
    if (g.nblocks == 0)
        return hipSuccess;
    dim3 grid((unsigned)g.nblocks), block(512);
    if (residual)
        hipLaunchKernelGGL(dequant_kernel<true>, grid, block, 0, stream, anchor, residual, gmin,
                           gscale, mu, sigma, g, tab, out);
    else
        hipLaunchKernelGGL(dequant_kernel<false>, grid, block, 0, stream, anchor, residual,
                           gmin, gscale, mu, sigma, g, tab, out);
    return hipGetLastError();
}

}  // namespace lynx
