// Internal declarations shared by the host API and the gfx950 kernels of
// liblynx.so.  Not part of the public ABI (include/lynx.h is).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace lynx {

constexpr int kPage = 256;      // P: tokens per page block
constexpr int kChunk = 32;      // C: tokens per chunk
constexpr int kHead = 128;      // H: channels per page block
constexpr int kChunks = kPage / kChunk;
// Field widths: a anchor bits and b residual bits.  Splits of the 8-bit code
// have a + b = 8 (the paper's split is a = 4, a = 3..6 are built); a single
// stream has b = 0 (a = 4 or 8: the paper's Lynx-INT4 / Lynx-INT8).  The
// largest code whose anchor magnitude (code + bias) >> b fits a
// two's-complement bits is 128 - 2^(b-1) for a split (120 for 4 + 4) and
// 2^(a-1) - 1 for a single stream.
constexpr int kMinAnchorBits = 3, kMaxAnchorBits = 6;
constexpr bool valid_field_bits(int a, int b) {
    return (a + b == 8 && a >= kMinAnchorBits && a <= kMaxAnchorBits) ||
           (b == 0 && (a == 4 || a == 8));
}
constexpr int code_max_of(int a, int b) {
    return b == 0 ? (1 << (a - 1)) - 1 : 128 - (1 << (b - 1));
}
constexpr int kMaxBuckets = 1792;  // 7 KiB of SH16 table words in LDS and in the kernel argument

// Compander tables, built once per (alpha, code_scale, field widths) on the
// host and passed by value as a kernel argument: 9.5 KB, within the kernel
// argument size HIP passes on gfx950 (12 KB launches checked with ROCm 7;
// a runtime that refused it would fail the launch with an error, not
// change a code).
//
// thr[k] (k = 1..120) is the smallest binary32 x >= 0 whose Eq. (3) value
// Y(x) reaches k - 1/2, i.e. the code of |x| is #{k : |x| >= thr[k]};
// thr[0] = 0 and thr[121..127] = +inf (the clip at 120).
//
// Bucket index of a magnitude m is bits(m) >> shift, clamped to
// [bucket_lo, bucket_lo + nbuckets - 1]; every bucket holds at most one
// threshold, so code(m) = bucket_code[i] + (m >= thr[bucket_code[i] + 1]).
//
// word[i] (shift = 16 only): the quantize kernel's table entry of bucket i,
// ((bucket_code[i] + bias + 1) << 24) - t, where bias is the Stage 4 offset
// of the field split and t the low half of thr[bucket_code[i] + 1] if that
// threshold lies in bucket i (the magnitudes of a bucket share their upper
// half), else 0x10000; adding a magnitude's low half to the entry leaves
// code + bias in the top byte.  Entries past nbuckets are zero.
struct QuantTab {
    float thr[128];
    uint8_t bucket_code[kMaxBuckets];
    uint32_t word[kMaxBuckets];
    int32_t bucket_lo;
    int32_t nbuckets;
    int32_t shift;
    float eps;
};

// Reconstruction levels L[k] = ((1 + alpha)^(k / code_scale) - 1) / alpha.
struct DequantTab {
    float level[128];
    float eps;
};

// Geometry of one launch: a KV set cut into page blocks.
struct Geometry {
    int64_t tensor_stride;  // elements
    int64_t row_stride;     // elements
    int32_t pages;          // pages per tensor
    int32_t heads;          // 128-channel groups per tensor
    int64_t nblocks;        // blocks in this launch
    int64_t block0;         // global index of the launch's first block
    int64_t grid_wgs;       // workgroups of a launch whose kernel loops over blocks
    // Per-block strides of the code buffers: bytes of the anchor-side buffer
    // (the anchor stream alone, or with the packed layout the block's whole
    // record: anchor stream then gamma_min, gamma_scale, mu, sigma), and
    // elements of the gamma_min / gamma_scale and mu / sigma arrays.  The
    // residual stream always has 4096 b bytes per block.
    int64_t astride;
    int64_t gstride;
    int64_t cstride;
};

// Block and lane indices come from the amdgcn intrinsics: the kernels are
// built with IEEE mode off, so the device library's index helpers (built
// with it on) would not be inlined.
enum StatsMode : int { kModeQuantize = 0, kModePageStats = 1, kModeBlockStats = 2 };

hipError_t launch_quantize(const uint16_t *kv, const Geometry &g, const QuantTab &tab,
                           uint8_t *anchor, uint8_t *residual, float *gmin, float *gscale,
                           float *mu, float *sigma, int mode, int anchor_bits,
                           int residual_bits, int meta_bits, hipStream_t stream);

hipError_t launch_dequant(const uint8_t *anchor, const uint8_t *residual, const float *gmin,
                          const float *gscale, const float *mu, const float *sigma,
                          const Geometry &g, const DequantTab &tab, uint16_t *out,
                          int anchor_bits, int residual_bits, int meta_bits,
                          hipStream_t stream);

}  // namespace lynx
