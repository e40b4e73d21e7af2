// Argument blocks and launchers of the fused dequant + attention kernels
// (lynx_attn.hip) and of speculative verification (lynx_verify.hip), shared
// with the host code of liblynx.so.  Kept apart from lynx_internal.h, which
// the codec kernels include.  Not part of the public ABI (include/lynx.h is).
#pragma once

#include "lynx_internal.h"

namespace lynx {

// Argument block of the fused dequant + attention kernels.
struct AttnArgs {
    const uint16_t *q;  // [t_q][n_qh][128] bf16
    const uint8_t *k_anc, *k_res, *v_anc, *v_res;
    const float *k_gmin, *k_gsc, *k_mu, *k_sg;
    const float *v_gmin, *v_gsc, *v_mu, *v_sg;
    float *ws;      // partials: [split][kv head][row][128] outputs, then [split][kv head][row][2] (max, sum)
    int64_t astride, gstride, cstride;  // per-block strides of K and V codes
    void *out;      // [t_q][n_qh][128], bf16 or binary32
    int64_t ctx;    // context tokens (multiple of 256)
    int64_t causal_base;  // causal tail: the last key query token 0 of the launch sees
    int n_qh, n_kvh, group, t_q;
    int rows;       // t_q * group
    int pages, splits;
    int steps_per_split;   // tile kernel (more than 16 rows): steps of 128 tokens
    int chunks_per_split;  // decode kernel (at most 16 rows): 32-token chunks
    int causal;
    int out_f32;
    float qk_scale_log2;  // scale * log2(e)
};
int attn_row_tiles(int rows);  // tiles of 16 query rows, -1 if rows > 64
hipError_t launch_attention(const AttnArgs &a, const DequantTab &tab, hipStream_t stream);
// Bytes of the fixed device scratch of lynx_decode_attn_dequant_noalloc
// (LYNX_ATTN_SCRATCH_BYTES of lynx.h) and its device address on the current
// device (looked up once per device).
constexpr size_t kAttnScratchBytes = size_t(24) << 20;
hipError_t attn_scratch(float **ptr);

// Speculative verification (lynx_verify.hip).
constexpr int kVerifyChunk = 2048;    // tokens per statistics workgroup
constexpr int kVerifyMaxDraft = 64;   // draft tokens per call at most
struct VerifyArgs {
    const float *draft;      // [t][vocab] logits the drafts were drawn from
    const float *target;     // [t + 1][vocab] full-precision logits
    const int32_t *tokens;   // [t] draft tokens
    const double *u_accept;  // [t] uniforms
    double u_sample;         // uniform of the correction / bonus draw
    int t, vocab, chunks;    // chunks = ceil(vocab / kVerifyChunk)
    double *ws;              // [2t + 1][chunks][2] chunk max and sum, [chunks]
                             // weight sums, [8] the decision
    int32_t *out;            // [2]: accepted drafts, next token
};
size_t verify_workspace_doubles(int t, int64_t chunks);
hipError_t launch_verify(const VerifyArgs &a, hipStream_t stream);

}  // namespace lynx
