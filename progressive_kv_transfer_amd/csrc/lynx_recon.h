// Reconstruction arithmetic of the dequant kernels: the inverse of
// Algorithm 1 of "Lynx: Progressive Speculative Quantization for
// accelerating KV Transfer in Long-Context Inference" (Eq. (4); the anchor
// level V << 4 of the reading notes' worked example).  The fused attention
// kernels share only the signed level table (signed_level) and the bf16
// rounding (pack_bf16): they fold Eq. (4) into one fused multiply-add per
// element, so their K^ / V^ may differ from lynx_dequant_* by one bf16 unit
// on rare elements (rounding order, not a different level).
#pragma once

#include "lynx_internal.h"

namespace lynx {

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 round-to-nearest-even of two binary32 values (v_cvt_pk_bf16_f32),
// low half = lo.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    f32x2_t v = {lo, hi};
    bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

// Signed level S * L[code] of table entry t: t & 15 = anchor nibble,
// t >> 4 = residual nibble (full) .  Anchor-only uses code = magnitude << 4;
// full uses (magnitude << 4) - residual, clamped at 0 (only streams the
// quantizer never writes reach below 0).
__device__ __forceinline__ float signed_level(const DequantTab &tab, int t, bool full) {
    int a = t & 15;
    int av = a >= 8 ? a - 16 : a;
    int v = av < 0 ? -av - 1 : av;
    int code = v << 4;
    if (full) {
        int r = (t >> 4) & 15;
        code -= r >= 8 ? r - 16 : r;
        code = code < 0 ? 0 : code;
    }
    float m = tab.level[code];
    return av < 0 ? -m : m;
}

// x^ = ((S L) * (sigma + eps) + mu) * (gamma_scale + eps) + gamma_min, four
// binary32 roundings (the file is built with -ffp-contract=off).
__device__ __forceinline__ float reconstruct(float sl, float d2, float mu, float d1, float gmin) {
    float t1 = sl * d2;
    float xn = t1 + mu;
    float t2 = xn * d1;
    return t2 + gmin;
}

}  // namespace lynx
