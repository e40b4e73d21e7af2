// gfx950 fused dequant + grouped-query attention over Lynx-coded KV:
// O = softmax(Q K^T * scale) V (the paper's Section 2.1) where K^ and V^ are
// rebuilt on the fly from the Anchor stream alone (the speculative draft,
// Section 4.2 Figure 7(b)) or from Anchor + Residual (the verification
// precision, Figure 7(c)), bit-identical to lynx_dequant_anchor /
// lynx_dequant_full (shared arithmetic in lynx_recon.h).  One query token is
// decode; T query tokens with a causal tail are the single parallel forward
// pass that verifies T drafts (Section 4.3).
//
// Split-KV: workgroup (kv head h, split s) walks pages [s*pps, (s+1)*pps) of
// its head for all M = T * group query rows that read that head (GQA), and
// leaves a partial (running max, running sum, unnormalised output) per row in
// the workspace; attn_combine_kernel merges the splits.
//
// Per 32-token chunk of a page: every lane rebuilds 2 channels x 8 tokens of
// K^ and of V^ into LDS (bf16 pairs, rows padded to 68 dwords so row reads
// spread over the banks); scores come from v_dot2_f32_bf16 with the lane's
// query row kept as 64 packed bf16 pairs in registers (products of bf16 are
// exact in binary32); an online softmax in base 2 (scores pre-multiplied by
// scale * log2 e, v_exp_f32); the P V^ update accumulates binary32.
#include "lynx_recon.h"

namespace lynx {

namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAttnThreads = 256;
constexpr int kRowDw = 68;  // dwords per rebuilt K^ / V^ row in LDS (64 + pad)
constexpr int kPartial = 2 + kHead;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// Rebuild 2 channels (pair p) x 8 tokens (8 qt .. 8 qt + 7) of chunk j of
// page block b into LDS rows dst[token][p] as packed bf16 pairs.
__device__ __forceinline__ void rebuild_pair(const uint8_t *anc, const uint8_t *res,
                                             const float *gmin, const float *gsc,
                                             const float *mu, const float *sg, float eps,
                                             const float *lut, int64_t b, int j, int p, int qt,
                                             uint32_t *dst) {
    const int64_t coff = b * (kPage * kHead / 2) + j * (kHead / 2 * kChunk) + p * kChunk + 8 * qt;
    const u32x2 A = *(const u32x2 *)(anc + coff);
    const u32x2 R = res ? *(const u32x2 *)(res + coff) : u32x2{0u, 0u};
    const float2 gm = *(const float2 *)(gmin + b * kHead + 2 * p);
    const float2 gs = *(const float2 *)(gsc + b * kHead + 2 * p);
    const float2 um = *(const float2 *)(mu + b * (kChunks * kHead) + j * kHead + 2 * p);
    const float2 sq = *(const float2 *)(sg + b * (kChunks * kHead) + j * kHead + 2 * p);
    const float d1a = gs.x + eps, d1b = gs.y + eps, d2a = sq.x + eps, d2b = sq.y + eps;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t ab = (A[i >> 2] >> (8 * (i & 3))) & 0xffu;
        const uint32_t rb = (R[i >> 2] >> (8 * (i & 3))) & 0xffu;
        const uint32_t i0 = (ab & 15u) | ((rb & 15u) << 4);  // channel 2p
        const uint32_t i1 = (ab >> 4) | (rb & 0xf0u);         // channel 2p + 1
        const float y0 = reconstruct(lut[i0], d2a, um.x, d1a, gm.x);
        const float y1 = reconstruct(lut[i1], d2b, um.y, d1b, gm.y);
        dst[(8 * qt + i) * kRowDw + p] = pack_bf16(y0, y1);
    }
}

template <int ROWS>  // padded rows: 8, 16, 32 or 64
__global__ __launch_bounds__(kAttnThreads) void attn_partial_kernel(AttnArgs a,
                                                                    const DequantTab tab) {
    constexpr int kLpr = kAttnThreads / ROWS;  // lanes per query row
    constexpr int kTpl = kChunk / kLpr;        // scores per lane per chunk
    constexpr int kCpl = kHead / kLpr;         // output channels per lane

    __shared__ float s_lut_k[256], s_lut_v[256];
    __shared__ __attribute__((aligned(16))) uint32_t s_k[kChunk * kRowDw];
    __shared__ __attribute__((aligned(16))) uint32_t s_v[kChunk * kRowDw];
    __shared__ float s_s[ROWS][kChunk + 1];

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int wg = (int)__builtin_amdgcn_workgroup_id_x();
    const int kvh = wg % a.n_kvh;
    const int split = wg / a.n_kvh;

    for (int e = tid; e < 256; e += kAttnThreads) {
        s_lut_k[e] = signed_level(tab, a.k_res ? e : (e & 15), a.k_res != nullptr);
        s_lut_v[e] = signed_level(tab, a.v_res ? e : (e & 15), a.v_res != nullptr);
    }

    // This lane's query row (scores and output), rows >= a.rows are padding.
    const int h = tid / kLpr;
    const int sub = tid % kLpr;
    const bool live = h < a.rows;
    const int r = live ? h / a.group : 0;
    const int qh = live ? kvh * a.group + h % a.group : 0;
    const int64_t limit = a.causal ? a.ctx - a.t_q + r : a.ctx - 1;
    uint32_t q2[64];
    {
        const u32x4 *qp = (const u32x4 *)(a.q + ((int64_t)r * a.n_qh + qh) * kHead);
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            u32x4 v = live ? qp[w] : u32x4{0u, 0u, 0u, 0u};
            q2[4 * w] = v[0];
            q2[4 * w + 1] = v[1];
            q2[4 * w + 2] = v[2];
            q2[4 * w + 3] = v[3];
        }
    }
    float m_run = -INFINITY, l_run = 0.0f;
    float o[kCpl];
#pragma unroll
    for (int c = 0; c < kCpl; ++c) o[c] = 0.0f;

    const int p = tid & 63;   // rebuild: channel pair
    const int qt = tid >> 6;  // rebuild: tokens 8 qt .. 8 qt + 7
    const int pg0 = split * a.pages_per_split;
    const int pg1 = min(a.pages, pg0 + a.pages_per_split);
    __syncthreads();
    for (int pg = pg0; pg < pg1; ++pg) {
        const int64_t b = (int64_t)pg * a.n_kvh + kvh;
        for (int j = 0; j < kChunks; ++j) {
            const int64_t pos0 = (int64_t)pg * kPage + j * kChunk;
            rebuild_pair(a.k_anc, a.k_res, a.k_gmin, a.k_gsc, a.k_mu, a.k_sg, tab.eps, s_lut_k,
                         b, j, p, qt, s_k);
            rebuild_pair(a.v_anc, a.v_res, a.v_gmin, a.v_gsc, a.v_mu, a.v_sg, tab.eps, s_lut_v,
                         b, j, p, qt, s_v);
            __syncthreads();
            // scores of row h for tokens sub + k * kLpr
#pragma unroll
            for (int k = 0; k < kTpl; ++k) {
                const int t = sub + k * kLpr;
                const u32x4 *kr = (const u32x4 *)(s_k + t * kRowDw);
                float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
                for (int w = 0; w < 16; ++w) {
                    const u32x4 kv = kr[w];
                    acc0 = dot2(q2[4 * w], kv[0], acc0);
                    acc1 = dot2(q2[4 * w + 1], kv[1], acc1);
                    acc0 = dot2(q2[4 * w + 2], kv[2], acc0);
                    acc1 = dot2(q2[4 * w + 3], kv[3], acc1);
                }
                const float s = (acc0 + acc1) * a.qk_scale_log2;
                s_s[h][t] = (live && pos0 + t <= limit) ? s : -INFINITY;
            }
            __syncthreads();
            // online softmax over the chunk, then O += P V^
            float mc = -INFINITY;
#pragma unroll
            for (int t = 0; t < kChunk; ++t) mc = fmaxf(mc, s_s[h][t]);
            const float m_new = fmaxf(m_run, mc);
            const bool none = m_new == -INFINITY;
            const float corr = none ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= corr;
#pragma unroll
            for (int c = 0; c < kCpl; ++c) o[c] *= corr;
            const int c0 = sub * kCpl;
#pragma unroll 8
            for (int t = 0; t < kChunk; ++t) {
                const float pt = none ? 0.0f : __builtin_amdgcn_exp2f(s_s[h][t] - m_new);
                l_run += pt;
                const uint32_t *vr = s_v + t * kRowDw + c0 / 2;
#pragma unroll
                for (int c = 0; c < kCpl; c += 2) {
                    const uint32_t w = vr[c / 2];
                    o[c] = __builtin_fmaf(pt, __uint_as_float(w << 16), o[c]);
                    o[c + 1] = __builtin_fmaf(pt, __uint_as_float(w & 0xffff0000u), o[c + 1]);
                }
            }
            m_run = m_new;
            __syncthreads();  // s_k, s_v and s_s are rewritten by the next chunk
        }
    }
    float *part = a.ws + (((int64_t)split * a.n_kvh + kvh) * ROWS + h) * kPartial;
    if (sub == 0) {
        part[0] = m_run;
        part[1] = l_run;
    }
#pragma unroll
    for (int c = 0; c < kCpl; ++c) part[2 + sub * kCpl + c] = o[c];
}

// One workgroup of 128 lanes per (kv head, live row): lane c merges channel
// c over the splits and writes the bf16 output.
template <int ROWS>
__global__ __launch_bounds__(kHead) void attn_combine_kernel(AttnArgs a) {
    const int wg = (int)__builtin_amdgcn_workgroup_id_x();
    const int kvh = wg % a.n_kvh;
    const int h = wg / a.n_kvh;
    const int c = (int)__builtin_amdgcn_workitem_id_x();
    float m = -INFINITY;
    for (int s = 0; s < a.splits; ++s)
        m = fmaxf(m, a.ws[(((int64_t)s * a.n_kvh + kvh) * ROWS + h) * kPartial]);
    float l = 0.0f, acc = 0.0f;
    if (m != -INFINITY) {
        for (int s = 0; s < a.splits; ++s) {
            const float *part = a.ws + (((int64_t)s * a.n_kvh + kvh) * ROWS + h) * kPartial;
            const float w = __builtin_amdgcn_exp2f(part[0] - m);
            l = __builtin_fmaf(part[1], w, l);
            acc = __builtin_fmaf(part[2 + c], w, acc);
        }
    }
    const float y = l > 0.0f ? acc / l : 0.0f;
    const int r = h / a.group;
    const int qh = kvh * a.group + h % a.group;
    const int64_t at = ((int64_t)r * a.n_qh + qh) * kHead + c;
    if (a.out_f32)
        ((float *)a.out)[at] = y;
    else
        ((uint16_t *)a.out)[at] = (uint16_t)(pack_bf16(y, 0.0f) & 0xffffu);
}

template <int ROWS>
hipError_t launch_rows(const AttnArgs &a, const DequantTab &tab, hipStream_t stream) {
    hipLaunchKernelGGL(attn_partial_kernel<ROWS>, dim3((unsigned)(a.n_kvh * a.splits)),
                       dim3(kAttnThreads), 0, stream, a, tab);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(attn_combine_kernel<ROWS>, dim3((unsigned)(a.n_kvh * a.rows)), dim3(kHead),
                       0, stream, a);
    return hipGetLastError();
}

}  // namespace

int attn_padded_rows(int rows) {
    return rows <= 8 ? 8 : rows <= 16 ? 16 : rows <= 32 ? 32 : rows <= 64 ? 64 : -1;
}

hipError_t launch_attention(const AttnArgs &a, const DequantTab &tab, hipStream_t stream) {
    switch (attn_padded_rows(a.rows)) {
    case 8:
        return launch_rows<8>(a, tab, stream);
    case 16:
        return launch_rows<16>(a, tab, stream);
    case 32:
        return launch_rows<32>(a, tab, stream);
    case 64:
        return launch_rows<64>(a, tab, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace lynx
