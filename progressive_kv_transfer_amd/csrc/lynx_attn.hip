// gfx950 fused dequant + grouped-query attention over Lynx-coded KV:
// O = softmax(Q K^T * scale) V (the paper's Section 2.1) where K^ and V^ are
// rebuilt on the fly from the Anchor stream alone (the speculative draft,
// Section 4.2 Figure 7(b)) or from Anchor + Residual (the verification
// precision, Figure 7(c)).  Eq. (4) is evaluated as one fused multiply-add
// per element, S L * a + b, with a and b folded per chunk and channel, so
// K^ and V^ equal those of lynx_dequant_anchor / lynx_dequant_full up to
// rounding order (the two can differ by one bf16 unit in the last place
// where a value lies next to a rounding boundary).  One query token is
// decode; T query tokens with a causal tail are the single parallel forward
// pass that verifies T drafts (Section 4.3).
//
// Work split.  The M = T * group query rows that read one KV head form RT
// tiles of 16 rows (M <= 64).  Workgroup (kv head, split) walks a run of
// 128-token steps (half a page) of its head:
//   1. every lane rebuilds 32 tokens x 2 channels of K^ and of V^ of the
//      step from codes prefetched into registers during the previous step,
//      into LDS (K^ as [token][channel], V^ as [channel][token]), then
//      issues the loads of the next step;
//   2. wave w takes row tile w % RT and RT of the step's four 32-token
//      chunks, and per chunk computes S^T = K^ Q^T with
//      v_mfma_f32_16x16x32_bf16 (A = K^ rows from LDS, B = Q^T held in
//      registers; products of bf16 are exact in binary32), an online
//      softmax in base 2 on the 8 scores each lane holds, and
//      O^T += V^T P^T with the same MFMA (A = V^ rows from LDS,
//      B = P^T split into a bf16 high and low part, so P keeps ~16 bits).
// In this orientation every lane owns one query row in both products, so the
// running max, sum and output rescale stay lane-local; the four lanes that
// share a row agree on the max through two lane swaps.  The running max is
// only moved when a chunk exceeds it by more than 2^8 (weights stay <= 256),
// which skips most output rescales.  At the end the waves of a row tile are
// merged in LDS and each live row leaves one partial (max, sum, output) per
// split in the workspace; attn_combine_kernel merges the splits.
#include <mutex>

#include "lynx_attn_args.h"
#include "lynx_recon.h"

namespace lynx {

// Fixed device scratch of the allocation-free attention entry point: the
// split partials live here instead of in a caller's workspace.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// the name is only a stand-in: its device address comes from
// hipGetSymbolAddress, looked up once per device (attn_scratch below).
static __device__ __align__(256) float scratch[kAttnScratchBytes / sizeof(float)];

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAttnThreads = 256;
constexpr int kStep = 128;               // tokens per step (half a page)
constexpr int kRowDw = 68;               // dwords per LDS row: 64 + 4 pad
constexpr int kKDw = kStep * kRowDw;     // K^ [128 tokens][128 channels]
constexpr int kVDw = kHead * kRowDw;     // V^ [128 channel rows][128 tokens]
constexpr int kMergeRow = 132;           // floats per row in the LDS merge area
constexpr float kLazyLog2 = 8.0f;        // move the max only beyond 2^8

// Split partials in the workspace: the 128 outputs of (split, KV head, row)
// as one 512-byte row (whole cache lines), all of them first, then the
// (max, sum) pair of each.
__device__ __forceinline__ float *partial_out(const AttnArgs &a, int64_t split, int kvh, int r) {
    return a.ws + ((split * a.n_kvh + kvh) * a.rows + r) * kHead;
}
__device__ __forceinline__ float *partial_ml(const AttnArgs &a, int64_t split, int kvh, int r) {
    return a.ws + (int64_t)a.splits * a.n_kvh * a.rows * kHead +
           ((split * a.n_kvh + kvh) * a.rows + r) * 2;
}

// Codes and metadata of one tensor for one lane's 32 tokens x channel pair.
struct LaneCodes {
    u32x4 a0, a1, r0, r1;
    float2 gm, gs, mu, sg;
};

// Eq. (4) folded per (chunk, channel): x^ = S L * a + b with
// a = (sigma + eps)(gamma_scale + eps), b = mu (gamma_scale + eps) + gamma_min,
// one fused multiply-add per element (channels 2p in .x, 2p + 1 in .y).
struct Affine {
    float2 a, b;
};

__device__ __forceinline__ Affine fold(const LaneCodes &L, float eps) {
    const float d1x = L.gs.x + eps, d1y = L.gs.y + eps;
    Affine f;
    f.a = make_float2((L.sg.x + eps) * d1x, (L.sg.y + eps) * d1y);
    f.b = make_float2(__builtin_fmaf(L.mu.x, d1x, L.gm.x), __builtin_fmaf(L.mu.y, d1y, L.gm.y));
    return f;
}

__device__ __forceinline__ void load_codes(const uint8_t *anc, const uint8_t *res,
                                           const float *gmin, const float *gsc, const float *mu,
                                           const float *sg, const AttnArgs &a, int64_t b, int j,
                                           int p, LaneCodes &L) {
    const int64_t toff = j * (kHead / 2 * kChunk) + p * kChunk;
    const int64_t aoff = b * a.astride + toff;
    const int64_t roff = b * (kPage * kHead / 2) + toff;
    L.a0 = *(const u32x4 *)(anc + aoff);
    L.a1 = *(const u32x4 *)(anc + aoff + 16);
    if (res) {
        L.r0 = *(const u32x4 *)(res + roff);
        L.r1 = *(const u32x4 *)(res + roff + 16);
    } else {
        L.r0 = u32x4{0u, 0u, 0u, 0u};
        L.r1 = u32x4{0u, 0u, 0u, 0u};
    }
    L.gm = *(const float2 *)(gmin + b * a.gstride + 2 * p);
    L.gs = *(const float2 *)(gsc + b * a.gstride + 2 * p);
    L.mu = *(const float2 *)(mu + b * a.cstride + j * kHead + 2 * p);
    L.sg = *(const float2 *)(sg + b * a.cstride + j * kHead + 2 * p);
}

// Byte i of w shifted left by S (an SDWA byte select: one instruction).
template <int S>
__device__ __forceinline__ uint32_t byte_shl(uint32_t w, int i) {
    uint32_t r;
    switch (i) {
    case 0:
        asm("v_lshlrev_b32_sdwa %0, %2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD "
            "src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(w), "i"(S));
        break;
    case 1:
        asm("v_lshlrev_b32_sdwa %0, %2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD "
            "src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(w), "i"(S));
        break;
    case 2:
        asm("v_lshlrev_b32_sdwa %0, %2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD "
            "src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(w), "i"(S));
        break;
    default:
        asm("v_lshlrev_b32_sdwa %0, %2, %1 dst_sel:DWORD dst_unused:UNUSED_PAD "
            "src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(w), "i"(S));
        break;
    }
    return r;
}

// Signed-level tables at the start of the kernel's LDS (so a table address
// is the shifted code byte itself): lut[residual nibble | anchor nibble << 4]
// for full codes (the residual, the more evenly spread of the two, sits in
// the low bits that pick the LDS bank: fewer conflicts between lanes), and
// lut2[anchor byte] = the levels of both channels of the byte for
// anchor-only codes (one 8-byte read per token).
struct Luts {
    const float *lut;
    const float2 *lut2;
};

// Rebuild 4 tokens of channel pair (2p, 2p+1) from one anchor word and one
// residual word (a byte per token).
template <bool FULL>
__device__ __forceinline__ void rebuild_word(uint32_t A, uint32_t R, const Affine &f,
                                             const Luts &t, float y0[4], float y1[4]) {
    if (FULL) {
        const uint32_t X = ((A << 4) & 0xf0f0f0f0u) | (R & 0x0f0f0f0fu);  // channel 2p
        const uint32_t Y = (A & 0xf0f0f0f0u) | ((R >> 4) & 0x0f0f0f0fu);  // channel 2p + 1
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float s0 = *(const float *)((const char *)t.lut + byte_shl<2>(X, i));
            const float s1 = *(const float *)((const char *)t.lut + byte_shl<2>(Y, i));
            y0[i] = __builtin_fmaf(s0, f.a.x, f.b.x);
            y1[i] = __builtin_fmaf(s1, f.a.y, f.b.y);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float2 sl = *(const float2 *)((const char *)t.lut2 + byte_shl<3>(A, i));
            y0[i] = __builtin_fmaf(sl.x, f.a.x, f.b.x);
            y1[i] = __builtin_fmaf(sl.y, f.a.y, f.b.y);
        }
    }
}

// K^ rows: [token][channel] bf16; the lane writes dword p (channels 2p,
// 2p + 1) of its 32 tokens.
template <bool FULL>
__device__ __forceinline__ void store_k(const LaneCodes &L, float eps, const Luts &t, int p,
                                        int c, uint32_t *sK) {
    const u32x4 a[2] = {L.a0, L.a1}, r[2] = {L.r0, L.r1};
    const Affine f = fold(L, eps);
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        float y0[4], y1[4];
        rebuild_word<FULL>(a[w >> 2][w & 3], r[w >> 2][w & 3], f, t, y0, y1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sK[(32 * c + 4 * w + i) * kRowDw + p] = pack_bf16(y0[i], y1[i]);
    }
}

// V^ rows: row p holds channel 2p, row 64 + p channel 2p + 1, each as 128
// tokens of bf16; the lane writes tokens 32c .. 32c + 31 of both rows.
// Within a chunk's 32 positions the tokens are in the order of the P^T
// operand: positions 8q .. 8q + 7 hold tokens 4q .. 4q + 3 and
// 16 + 4q .. 16 + 4q + 3, so a lane's V^ operand is one 16-byte read.
template <bool FULL>
__device__ __forceinline__ void store_v(const LaneCodes &L, float eps, const Luts &t, int p,
                                        int c, uint32_t *sV) {
    const u32x4 a[2] = {L.a0, L.a1}, r[2] = {L.r0, L.r1};
    const Affine f = fold(L, eps);
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // code word w holds tokens 4w .. 4w + 3
        float y0[8], y1[8];
        rebuild_word<FULL>(a[0][q], r[0][q], f, t, y0, y1);
        rebuild_word<FULL>(a[1][q], r[1][q], f, t, y0 + 4, y1 + 4);
        const u32x4 e = {pack_bf16(y0[0], y0[1]), pack_bf16(y0[2], y0[3]),
                         pack_bf16(y0[4], y0[5]), pack_bf16(y0[6], y0[7])};
        const u32x4 o = {pack_bf16(y1[0], y1[1]), pack_bf16(y1[2], y1[3]),
                         pack_bf16(y1[4], y1[5]), pack_bf16(y1[6], y1[7])};
        *(u32x4 *)(sV + p * kRowDw + 16 * c + 4 * q) = e;
        *(u32x4 *)(sV + (64 + p) * kRowDw + 16 * c + 4 * q) = o;
    }
}

// Max / sum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes of a row).
__device__ __forceinline__ float row_max4(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                              false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                              false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float row_sum4(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                              false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                              false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Step boundary between the rebuild and the products.  With one row tile
// every wave reads back only the chunk it wrote itself, and a wave's LDS
// instructions execute in program order, so the compiler only has to keep
// its LDS accesses on their side of this point; otherwise the waves meet.
template <int RT>
__device__ __forceinline__ void step_sync() {
    if (RT == 1)
        asm volatile("" ::: "memory");
    else
        __syncthreads();
}

template <int RT>  // row tiles of 16: 1, 2 or 4
__global__ __launch_bounds__(kAttnThreads, 2) void attn_partial_kernel(AttnArgs a,
                                                                       const DequantTab tab) {
    constexpr int kWavesPerTile = 4 / RT;

    // One LDS block with the level tables first (address 0 of the
    // workgroup's LDS), then K^ and V^.
    struct Lds {
        float lut[256];
        float2 lut2[256];
        __attribute__((aligned(16))) uint32_t k[kKDw];
        __attribute__((aligned(16))) uint32_t v[kVDw];
    };
    __shared__ Lds lds;
    uint32_t *const sK = lds.k;
    uint32_t *const sV = lds.v;
    float *const s_lut = lds.lut;
    float2 *const s_lut2 = lds.lut2;

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int wg = (int)__builtin_amdgcn_workgroup_id_x();
    const int kvh = wg % a.n_kvh;
    const int split = wg / a.n_kvh;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    s_lut[tid] = signed_level(tab, ((tid & 15) << 4) | (tid >> 4), true);
    s_lut2[tid] = make_float2(signed_level(tab, tid & 15, false),
                              signed_level(tab, tid >> 4, false));
    const Luts luts = {s_lut, s_lut2};

    // Steps [st0, st1) of this split.
    const int steps = a.pages * 2;
    const int st0 = split * a.steps_per_split;
    const int st1 = min(steps, st0 + a.steps_per_split);

    // Rebuild role: channel pair p, chunk (= wave) c_fill of the step.
    const int p = lane;
    const int c_fill = wave;

    // MFMA role: row tile rt, query row h = 16 rt + lane % 16, k-group g.
    const int rt = wave % RT;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int h = 16 * rt + r16;
    const bool live = h < a.rows;
    bf16x8 qreg[4];
    {
        const int r = live ? h / a.group : 0;
        const int qh = live ? kvh * a.group + h % a.group : 0;
        const uint16_t *qp = a.q + ((int64_t)r * a.n_qh + qh) * kHead + 8 * g;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const u32x4 v = live ? *(const u32x4 *)(qp + 32 * kb) : u32x4{0u, 0u, 0u, 0u};
            qreg[kb] = as_bf16x8(v);
        }
    }
    // Last visible position of this lane's row.
    const int64_t limit =
        a.causal ? a.causal_base + (live ? h / a.group : a.t_q - 1) : a.ctx - 1;
    const float cs = a.qk_scale_log2;
    const float lazy = kLazyLog2 / cs;

    float m_run = -INFINITY;  // running max of raw scores q.k
    float l_run = 0.0f;       // this lane's share of the row sum
    f32x4 o[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    LaneCodes ck, cv;
    if (st0 < st1) {
        const int64_t b = (int64_t)(st0 >> 1) * a.n_kvh + kvh;
        const int j = (st0 & 1) * 4 + c_fill;
        load_codes(a.k_anc, a.k_res, a.k_gmin, a.k_gsc, a.k_mu, a.k_sg, a, b, j, p, ck);
        load_codes(a.v_anc, a.v_res, a.v_gmin, a.v_gsc, a.v_mu, a.v_sg, a, b, j, p, cv);
    }
    __syncthreads();  // s_lut

    for (int st = st0; st < st1; ++st) {
        if (a.k_res)
            store_k<true>(ck, tab.eps, luts, p, c_fill, sK);
        else
            store_k<false>(ck, tab.eps, luts, p, c_fill, sK);
        if (a.v_res)
            store_v<true>(cv, tab.eps, luts, p, c_fill, sV);
        else
            store_v<false>(cv, tab.eps, luts, p, c_fill, sV);
        if (st + 1 < st1) {
            const int64_t b = (int64_t)((st + 1) >> 1) * a.n_kvh + kvh;
            const int j = ((st + 1) & 1) * 4 + c_fill;
            load_codes(a.k_anc, a.k_res, a.k_gmin, a.k_gsc, a.k_mu, a.k_sg, a, b, j, p, ck);
            load_codes(a.v_anc, a.v_res, a.v_gmin, a.v_gsc, a.v_mu, a.v_sg, a, b, j, p, cv);
        }
        step_sync<RT>();

        const int64_t tok0 = (int64_t)st * kStep;
        const bool need_mask = tok0 + kStep - 1 > a.causal_base;  // uniform
#pragma unroll
        for (int ci = 0; ci < RT; ++ci) {
            const int c = wave / RT + kWavesPerTile * ci;
            // S^T tiles: s[tt][e] is the score of token 32c + 16 tt + 4g + e.
            f32x4 s[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
            const uint32_t *kr = sK + (32 * c + r16) * kRowDw + 4 * g;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const bf16x8 a0 = as_bf16x8(*(const u32x4 *)(kr + 16 * kb));
                const bf16x8 a1 = as_bf16x8(*(const u32x4 *)(kr + 16 * kRowDw + 16 * kb));
                s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qreg[kb], s[0], 0, 0, 0);
                s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qreg[kb], s[1], 0, 0, 0);
            }
            if (need_mask) {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (tok0 + 32 * c + 16 * tt + 4 * g + e > limit) s[tt][e] = -INFINITY;
            }
            float mc = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                             fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
            mc = row_max4(mc);
            const bool grow = mc > m_run + lazy;
            if (__builtin_amdgcn_ballot_w64(grow)) {
                const float corr = grow ? __builtin_amdgcn_exp2f((m_run - mc) * cs) : 1.0f;
                l_run *= corr;
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) o[mt] *= corr;
                m_run = grow ? mc : m_run;
            }
            const float base = m_run == -INFINITY ? 0.0f : m_run * cs;
            float pr[8];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pr[4 * tt + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tt][e], cs, -base));
                    l_run += pr[4 * tt + e];
                }
            // P^T operands: k-slot 8g + e' <-> token 16 (e' / 4) + 4g + e' % 4.
            u32x4 hi, lo;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t hw = pack_bf16(pr[2 * i], pr[2 * i + 1]);
                hi[i] = hw;
                lo[i] = pack_bf16(pr[2 * i] - __uint_as_float(hw << 16),
                                  pr[2 * i + 1] - __uint_as_float(hw & 0xffff0000u));
            }
            const bf16x8 phi = as_bf16x8(hi), plo = as_bf16x8(lo);
            const uint32_t *vr = sV + r16 * kRowDw + 16 * c + 4 * g;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                const bf16x8 av = as_bf16x8(*(const u32x4 *)(vr + 16 * mt * kRowDw));
                o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, phi, o[mt], 0, 0, 0);
                o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, plo, o[mt], 0, 0, 0);
            }
        }
        step_sync<RT>();  // sK / sV are refilled by the next step
    }
    __syncthreads();  // the merge area overlaps every wave's K^ rows

    // Merge the waves of each row tile in LDS (reusing the K^ area), then
    // write one partial per live row.
    // A lane holds channels 32 m + 8 g .. + 7 of its row in o[m] (the even
    // ones: V^ row rho < 64 is channel 2 rho) and o[m + 4] (the odd ones:
    // row 64 + rho is channel 2 rho + 1): two 16-byte LDS writes per m; a
    // merging lane takes 4 channels of a row.
    const float l_row = row_sum4(l_run);
    float *sm = (float *)sK;  // [wave][16 rows][kMergeRow]: max, sum, -, -, 128 outputs
    if (live) {  // dead rows are never read
        float *row = sm + (wave * 16 + r16) * kMergeRow;
        if (g == 0) {
            row[0] = m_run == -INFINITY ? -INFINITY : m_run * cs;
            row[1] = l_row;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float4 *dst = (float4 *)(row + 4 + 32 * m + 8 * g);
            dst[0] = make_float4(o[m][0], o[m + 4][0], o[m][1], o[m + 4][1]);
            dst[1] = make_float4(o[m][2], o[m + 4][2], o[m][3], o[m + 4][3]);
        }
    }
    __syncthreads();
    for (int idx = tid; idx < a.rows * (kHead / 4); idx += kAttnThreads) {
        const int hr = idx >> 5, c4 = 4 * (idx & (kHead / 4 - 1));
        const int t = hr >> 4, rr = hr & 15;
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < kWavesPerTile; ++k)
            M = fmaxf(M, sm[((t + RT * k) * 16 + rr) * kMergeRow]);
        float l = 0.0f;
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
        for (int k = 0; k < kWavesPerTile; ++k) {
            const float *row = sm + ((t + RT * k) * 16 + rr) * kMergeRow;
            const float w = row[0] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(row[0] - M);
            const float4 v = *(const float4 *)(row + 4 + c4);
            l = __builtin_fmaf(row[1], w, l);
            acc.x = __builtin_fmaf(v.x, w, acc.x);
            acc.y = __builtin_fmaf(v.y, w, acc.y);
            acc.z = __builtin_fmaf(v.z, w, acc.z);
            acc.w = __builtin_fmaf(v.w, w, acc.w);
        }
        if (c4 == 0)
            *(float2 *)partial_ml(a, split, kvh, hr) = make_float2(M, l);
        *(float4 *)(partial_out(a, split, kvh, hr) + c4) = acc;
    }
}

// ---------------------------------------------------------------------------
// Decode kernel (at most 16 query rows per KV head, one row tile): no K^ or
// V^ tiles in LDS.  Each wave walks 32-token chunks on its own; every lane
// loads the 32 code bytes of channel pair `lane` of each stream (two 16-byte
// loads) and the MFMA operands are rebuilt in registers:
//   K^ (A of S^T = K^ Q^T, 8 channels of one token per lane): the codes go
//     through a 2 KiB LDS stage per stream ([pair][8 dwords], the dwords
//     of both token halves of a k-block side by side, the two 16-byte
//     halves of a pair's row swapped for pairs with bit 2 set so that the
//     writes hit distinct banks); lane (r16 = 4 qa + qi, g) reads, per
//     k-block m, one 8-byte pair of dwords of pair 16 m + 4 g + qi: tokens
//     4 qa .. + 3 and 16 + 4 qa .. + 3, and a 4 x 4 byte transpose across the
//     lanes of a quad (two DPP moves, two v_perm) leaves it the 4 pairs
//     16 m + 4 g .. + 3 (channels 32 m + 8 g .. + 7) of token 16 tt + r16.
//   V^ (A of O^T += V^T P^T, 8 tokens of one channel per lane): a 4 x 4
//     dword transpose across the lane quarters (permlane32 / permlane16
//     swaps) gives lane (r16, g) the dwords of pair 16 m + r16 at tokens
//     4 g .. + 3 and 16 + 4 g .. + 3, the token order of the P^T operand;
//     one pair gives the rows of two 16-channel tiles (its even and its odd
//     channel).
// The per-(chunk, channel) affine of Eq. (4) goes through a 2 KiB LDS table
// per wave (one float4 per channel pair), the level tables sit at LDS
// address 0 as in the tile kernel.  At the end the waves merge in LDS and
// one partial per live row and split goes to the workspace for
// attn_combine_kernel (merging the splits inside this kernel, by the last
// workgroups to finish, measured slower: partials visible across the XCDs'
// L2 caches cost either whole-cache write-backs or coherent-level loads,
// more than the second launch).
constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;

// Codes of one chunk (pair `lane`: tokens 0-15 in .0, 16-31 in .1) and the
// metadata of pair `lane`.  With both tensors at full precision the V codes
// are requested after the scores (all four streams at once would spill).
template <bool KF, bool VF>
struct DecCodes {
    u32x4 ka[2], va[2];
    u32x4 kr[KF ? 2 : 1], vr[VF ? 2 : 1];
    float2 kgm, kgs, kmu, ksg, vgm, vgs, vmu, vsg;
};

template <bool KF, bool VF>
__device__ __forceinline__ void dec_load_k(const AttnArgs &a, int64_t b, int j, int lane,
                                           DecCodes<KF, VF> &c) {
    const int64_t go = b * a.gstride + 2 * lane;
    const int64_t co = b * a.cstride + j * kHead + 2 * lane;
    c.kgm = *(const float2 *)(a.k_gmin + go);
    c.kgs = *(const float2 *)(a.k_gsc + go);
    c.kmu = *(const float2 *)(a.k_mu + co);
    c.ksg = *(const float2 *)(a.k_sg + co);
    c.vgm = *(const float2 *)(a.v_gmin + go);
    c.vgs = *(const float2 *)(a.v_gsc + go);
    c.vmu = *(const float2 *)(a.v_mu + co);
    c.vsg = *(const float2 *)(a.v_sg + co);
    const int64_t ab = b * a.astride + j * (kHead / 2 * kChunk) + lane * kChunk;
    const int64_t rb = b * (kPage * kHead / 2) + j * (kHead / 2 * kChunk) + lane * kChunk;
    c.ka[0] = *(const u32x4 *)(a.k_anc + ab);
    c.ka[1] = *(const u32x4 *)(a.k_anc + ab + 16);
    if constexpr (KF) {
        c.kr[0] = *(const u32x4 *)(a.k_res + rb);
        c.kr[1] = *(const u32x4 *)(a.k_res + rb + 16);
    }
}

template <bool KF, bool VF>
__device__ __forceinline__ void dec_load_v(const AttnArgs &a, int64_t b, int j, int lane,
                                           DecCodes<KF, VF> &c) {
    const int64_t ab = b * a.astride + j * (kHead / 2 * kChunk) + lane * kChunk;
    const int64_t rb = b * (kPage * kHead / 2) + j * (kHead / 2 * kChunk) + lane * kChunk;
    c.va[0] = *(const u32x4 *)(a.v_anc + ab);
    c.va[1] = *(const u32x4 *)(a.v_anc + ab + 16);
    if constexpr (VF) {
        c.vr[0] = *(const u32x4 *)(a.v_res + rb);
        c.vr[1] = *(const u32x4 *)(a.v_res + rb + 16);
    }
}

// 4 x 4 byte transpose across the lanes of a quad: lane qi ends with byte
// qi of each lane of its quad (byte k from lane k).  Stage 1 swaps half
// words with lane qi ^ 2, stage 2 bytes with lane qi ^ 1; sel1 / sel2 are
// the lane's v_perm selectors (perm(a, b, s) takes bytes 0-3 from b, 4-7
// from a).
__device__ __forceinline__ uint32_t quad_transpose(uint32_t x, uint32_t sel1, uint32_t sel2) {
    uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4e, 0xf, 0xf, false);
    x = __builtin_amdgcn_perm(y, x, sel1);
    y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xb1, 0xf, 0xf, false);
    return __builtin_amdgcn_perm(y, x, sel2);
}

// 4 x 4 dword transpose across the lane quarters: lane (r16, x) ends with
// d[q] = the d[x] lane (r16, q) held (stage 1 swaps with the other half of
// the wave, stage 2 with the neighbouring quarter).
__device__ __forceinline__ void quarter_transpose(uint32_t d[4]) {
    auto s02 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
    auto s13 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
    auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
    auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
    d[0] = s01[0];
    d[1] = s01[1];
    d[2] = s23[0];
    d[3] = s23[1];
}

// V operand dwords of a stream: out[2 m + h] = pair 16 m + r16, tokens
// 16 h + 4 g .. + 3.
__device__ __forceinline__ void v_operand_words(const u32x4 w[2], uint32_t out[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t d[4] = {w[h][0], w[h][1], w[h][2], w[h][3]};
        quarter_transpose(d);
#pragma unroll
        for (int m = 0; m < 4; ++m) out[2 * m + h] = d[m];
    }
}

// Eq. (4) folded for both channels of a pair: (a_lo, a_hi, b_lo, b_hi).
__device__ __forceinline__ float4 dec_affine(float2 gm, float2 gs, float2 mu, float2 sg,
                                             float eps) {
    const float d1x = gs.x + eps, d1y = gs.y + eps;
    return make_float4((sg.x + eps) * d1x, (sg.y + eps) * d1y, __builtin_fmaf(mu.x, d1x, gm.x),
                       __builtin_fmaf(mu.y, d1y, gm.y));
}

// Levels of the two channels of code byte i of the anchor word A (and, for
// full codes, of the combined words X, Y): .x channel 2P, .y channel 2P + 1.
template <bool FULL>
__device__ __forceinline__ float2 dec_levels(uint32_t X, uint32_t Y, uint32_t A, int i,
                                             const Luts &t) {
    if constexpr (FULL) {
        return make_float2(*(const float *)((const char *)t.lut + byte_shl<2>(X, i)),
                           *(const float *)((const char *)t.lut + byte_shl<2>(Y, i)));
    } else {
        return *(const float2 *)((const char *)t.lut2 + byte_shl<3>(A, i));
    }
}

template <bool KF, bool VF>  // K / V rebuilt from anchor + residual
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(4))) void
attn_decode_kernel(AttnArgs a, const DequantTab tab) {
    constexpr int kMergeFloats = kDecWaves * 16 * kMergeRow;
    struct PerWave {
        float4 affk[64], affv[64];  // affine of each pair, K then V
        uint32_t ka[64 * 8];        // K codes [pair][8 dwords], halves swapped for pair bit 2
        uint32_t kr[KF ? 64 * 8 : 1];
    };
    struct Lds {
        float lut[256];
        float2 lut2[256];
        union {
            PerWave w[kDecWaves];
            float merge[kMergeFloats];  // [wave][16 rows][kMergeRow]
        } u;
    };
    __shared__ Lds lds;

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int wg = (int)__builtin_amdgcn_workgroup_id_x();
    const int kvh = wg % a.n_kvh;
    const int split = wg / a.n_kvh;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int qi = r16 & 3;
    const int qa = r16 >> 2;

    if (tid < 256) {
        lds.lut[tid] = signed_level(tab, ((tid & 15) << 4) | (tid >> 4), true);
        lds.lut2[tid] = make_float2(signed_level(tab, tid & 15, false),
                                    signed_level(tab, tid >> 4, false));
    }
    const Luts luts = {lds.lut, lds.lut2};
    PerWave &pw = lds.u.w[wave];

    // quad-transpose selectors of this lane
    const uint32_t sel1 = qi < 2 ? 0x05040100u : 0x03020706u;
    const uint32_t sel2 = (qi & 1) ? 0x03070105u : 0x06020400u;
    // K stage: this lane's pair row holds dwords 0-7 of the pair's run
    // (tokens 4d .. 4d + 3) in the order 0, 4, 1, 5, 2, 6, 3, 7, so that
    // dwords qa and 4 + qa (token halves tt = 0, 1) are one 8-byte read, with
    // the row's two 16-byte halves swapped for pairs with bit 2 set (the
    // writes then hit distinct banks).  For k-block m the lane reads pair
    // 16 m + 4 g + qi at position 2 qa ^ 4 (g & 1) (pair bit 2 = g & 1).
    const int kw_lo = lane * 8 + 4 * ((lane >> 2) & 1);
    const int kw_hi = lane * 8 + 4 * (((lane >> 2) & 1) ^ 1);
    const int kr_base = (4 * g + qi) * 8 + ((2 * qa) ^ (4 * (g & 1)));

    // Query row h = r16 of this lane (both products), dead rows are zero.
    const int h = r16;
    const bool live = h < a.rows;
    bf16x8 qreg[4];
    {
        const int r = live ? h / a.group : 0;
        const int qh = live ? kvh * a.group + h % a.group : 0;
        const uint16_t *qp = a.q + ((int64_t)r * a.n_qh + qh) * kHead + 8 * g;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const u32x4 v = live ? *(const u32x4 *)(qp + 32 * kb) : u32x4{0u, 0u, 0u, 0u};
            qreg[kb] = as_bf16x8(v);
        }
    }
    const int64_t limit =
        a.causal ? a.causal_base + (live ? h / a.group : a.t_q - 1) : a.ctx - 1;
    const float cs = a.qk_scale_log2;
    const float lazy = kLazyLog2 / cs;

    float m_run = -INFINITY;
    float l_run = 0.0f;
    f32x4 o[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // Chunks of this split: wave w takes c0 + w, c0 + w + 8, ...
    const int64_t chunks = a.ctx / kChunk;
    const int64_t c0 = (int64_t)split * a.chunks_per_split;
    const int64_t c1 = min(chunks, c0 + a.chunks_per_split);
    __syncthreads();  // level tables

    for (int64_t c = c0 + wave; c < c1; c += kDecWaves) {
        const int64_t b = (c >> 3) * a.n_kvh + kvh;
        const int j = (int)(c & 7);
        DecCodes<KF, VF> cd;
        dec_load_k<KF, VF>(a, b, j, lane, cd);
        if constexpr (!(KF && VF))
            dec_load_v<KF, VF>(a, b, j, lane, cd);
        // This wave's own LDS region (a wave's LDS accesses execute in
        // program order): affine tables and the K stage of the chunk.
        pw.affk[lane] = dec_affine(cd.kgm, cd.kgs, cd.kmu, cd.ksg, tab.eps);
        pw.affv[lane] = dec_affine(cd.vgm, cd.vgs, cd.vmu, cd.vsg, tab.eps);
        *(u32x4 *)&pw.ka[kw_lo] = u32x4{cd.ka[0][0], cd.ka[1][0], cd.ka[0][1], cd.ka[1][1]};
        *(u32x4 *)&pw.ka[kw_hi] = u32x4{cd.ka[0][2], cd.ka[1][2], cd.ka[0][3], cd.ka[1][3]};
        if constexpr (KF) {
            *(u32x4 *)&pw.kr[kw_lo] = u32x4{cd.kr[0][0], cd.kr[1][0], cd.kr[0][1], cd.kr[1][1]};
            *(u32x4 *)&pw.kr[kw_hi] = u32x4{cd.kr[0][2], cd.kr[1][2], cd.kr[0][3], cd.kr[1][3]};
        }
        asm volatile("" ::: "memory");

        // ---- S^T = K^ Q^T ------------------------------------------------
        f32x4 s[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            uint32_t A[2], X[2] = {0u, 0u}, Y[2] = {0u, 0u};
            const u32x2 kw = *(const u32x2 *)&pw.ka[m * 128 + kr_base];
            u32x2 rw = {0u, 0u};
            if constexpr (KF)
                rw = *(const u32x2 *)&pw.kr[m * 128 + kr_base];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                A[tt] = quad_transpose(kw[tt], sel1, sel2);
                if constexpr (KF) {
                    const uint32_t R = quad_transpose(rw[tt], sel1, sel2);
                    X[tt] = ((A[tt] << 4) & 0xf0f0f0f0u) | (R & 0x0f0f0f0fu);
                    Y[tt] = (A[tt] & 0xf0f0f0f0u) | ((R >> 4) & 0x0f0f0f0fu);
                }
            }
            u32x4 op[2];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float4 af = pw.affk[16 * m + 4 * g + jj];  // channels 32m + 8g + 2jj, +1
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const float2 lv = dec_levels<KF>(X[tt], Y[tt], A[tt], jj, luts);
                    op[tt][jj] = pack_bf16(__builtin_fmaf(lv.x, af.x, af.z),
                                           __builtin_fmaf(lv.y, af.y, af.w));
                }
            }
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(op[tt]), qreg[m], s[tt],
                                                               0, 0, 0);
        }
        if constexpr (KF && VF)  // both full: V codes after the scores (registers)
            dec_load_v<KF, VF>(a, b, j, lane, cd);
        const int64_t tok0 = c * kChunk;
        if (tok0 + kChunk - 1 > a.causal_base) {  // uniform
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (tok0 + 16 * tt + 4 * g + e > limit) s[tt][e] = -INFINITY;
        }
        float mc = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        mc = row_max4(mc);
        const bool grow = mc > m_run + lazy;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float corr = grow ? __builtin_amdgcn_exp2f((m_run - mc) * cs) : 1.0f;
            l_run *= corr;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) o[mt] *= corr;
            m_run = grow ? mc : m_run;
        }
        const float base = m_run == -INFINITY ? 0.0f : m_run * cs;
        float pr[8];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pr[4 * tt + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tt][e], cs, -base));
                l_run += pr[4 * tt + e];
            }
        // P^T operands: k-slot 8g + e' <-> token 16 (e' / 4) + 4g + e' % 4.
        u32x4 hi, lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t hw = pack_bf16(pr[2 * i], pr[2 * i + 1]);
            hi[i] = hw;
            lo[i] = pack_bf16(pr[2 * i] - __uint_as_float(hw << 16),
                              pr[2 * i + 1] - __uint_as_float(hw & 0xffff0000u));
        }
        const bf16x8 phi = as_bf16x8(hi), plo = as_bf16x8(lo);

        // ---- O^T += V^T P^T ----------------------------------------------
        // Tile 2m: rows = channels 2 (16 m + rho); tile 2m + 1: 2 (16 m + rho) + 1.
        uint32_t va[8], vr[8];
        v_operand_words(cd.va, va);
        if constexpr (VF)
            v_operand_words(cd.vr, vr);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float4 af = pw.affv[16 * m + r16];
            float ve[8], vo[8];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const uint32_t A = va[2 * m + hh];
                uint32_t X = 0, Y = 0;
                if constexpr (VF) {
                    const uint32_t R = vr[2 * m + hh];
                    X = ((A << 4) & 0xf0f0f0f0u) | (R & 0x0f0f0f0fu);
                    Y = (A & 0xf0f0f0f0u) | ((R >> 4) & 0x0f0f0f0fu);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float2 lv = dec_levels<VF>(X, Y, A, e, luts);
                    ve[4 * hh + e] = __builtin_fmaf(lv.x, af.x, af.z);
                    vo[4 * hh + e] = __builtin_fmaf(lv.y, af.y, af.w);
                }
            }
            const bf16x8 aeven = as_bf16x8(u32x4{pack_bf16(ve[0], ve[1]), pack_bf16(ve[2], ve[3]),
                                                 pack_bf16(ve[4], ve[5]), pack_bf16(ve[6], ve[7])});
            const bf16x8 aodd = as_bf16x8(u32x4{pack_bf16(vo[0], vo[1]), pack_bf16(vo[2], vo[3]),
                                                pack_bf16(vo[4], vo[5]), pack_bf16(vo[6], vo[7])});
            o[2 * m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aeven, phi, o[2 * m], 0, 0, 0);
            o[2 * m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aeven, plo, o[2 * m], 0, 0, 0);
            o[2 * m + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aodd, phi, o[2 * m + 1], 0, 0, 0);
            o[2 * m + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aodd, plo, o[2 * m + 1], 0, 0, 0);
        }
        asm volatile("" ::: "memory");  // the wave's LDS region is rewritten by the next chunk
    }
    __syncthreads();  // the merge area overlaps every wave's region

    // Merge the 8 waves in LDS, then one partial per live row.  A lane
    // holds channels 32 m + 8 g .. + 7 of its row in o[2 m] (even) and
    // o[2 m + 1] (odd): two 16-byte LDS writes per m; a merging lane takes 4
    // channels of a row.
    const float l_row = row_sum4(l_run);
    float *sm = lds.u.merge;
    if (r16 < a.rows) {  // dead rows are never read
        float *row = sm + (wave * 16 + r16) * kMergeRow;
        if (g == 0) {
            row[0] = m_run == -INFINITY ? -INFINITY : m_run * cs;
            row[1] = l_row;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float4 *dst = (float4 *)(row + 4 + 32 * m + 8 * g);
            dst[0] = make_float4(o[2 * m][0], o[2 * m + 1][0], o[2 * m][1], o[2 * m + 1][1]);
            dst[1] = make_float4(o[2 * m][2], o[2 * m + 1][2], o[2 * m][3], o[2 * m + 1][3]);
        }
    }
    __syncthreads();
    for (int idx = tid; idx < a.rows * (kHead / 4); idx += kDecThreads) {
        const int hr = idx >> 5, c4 = 4 * (idx & (kHead / 4 - 1));
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < kDecWaves; ++k) M = fmaxf(M, sm[(k * 16 + hr) * kMergeRow]);
        float l = 0.0f;
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
        for (int k = 0; k < kDecWaves; ++k) {
            const float *row = sm + (k * 16 + hr) * kMergeRow;
            const float w = row[0] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(row[0] - M);
            const float4 v = *(const float4 *)(row + 4 + c4);
            l = __builtin_fmaf(row[1], w, l);
            acc.x = __builtin_fmaf(v.x, w, acc.x);
            acc.y = __builtin_fmaf(v.y, w, acc.y);
            acc.z = __builtin_fmaf(v.z, w, acc.z);
            acc.w = __builtin_fmaf(v.w, w, acc.w);
        }
        if (c4 == 0)
            *(float2 *)partial_ml(a, split, kvh, hr) = make_float2(M, l);
        *(float4 *)(partial_out(a, split, kvh, hr) + c4) = acc;
    }

}

// One workgroup of 512 lanes per (KV head, live row) merges the split
// partials in one pass: wave w takes the splits w, w + 8, ... (8 at a time,
// all their loads issued together, so 64 splits cost one round trip; a
// split's max and sum are wave-uniform loads), lane l channel pair l of
// them, with a running maximum per wave; the 8 waves then meet once in LDS,
// where 64 lanes rescale and add their (max, sum, pair) results and write
// the row.
constexpr int kCombineThreads = 512;
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(AttnArgs a) {
    constexpr int kW = kCombineThreads / 64;
    constexpr int kU = 8;
    __shared__ float4 s_part[kW][64];  // pair sums (2), row sum, wave max
    const int wg = (int)__builtin_amdgcn_workgroup_id_x();
    const int kvh = wg % a.n_kvh;
    const int h = wg / a.n_kvh;
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int64_t so = (int64_t)a.n_kvh * a.rows * kHead;  // split strides
    const int64_t sm = (int64_t)a.n_kvh * a.rows * 2;
    const float *ob = partial_out(a, 0, kvh, h);
    const float *mb = partial_ml(a, 0, kvh, h);

    float mw = -INFINITY, l = 0.0f;
    float2 acc = make_float2(0.0f, 0.0f);
    for (int s0 = wave; s0 < a.splits; s0 += kW * kU) {
        float ms[kU], ls[kU];
        float2 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {  // splits past the end re-read the last one, weight 0
            const int sp = min(s0 + kW * u, a.splits - 1);
            ms[u] = mb[sp * sm];
            ls[u] = mb[sp * sm + 1];
            v[u] = *(const float2 *)(ob + sp * so + 2 * lane);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (s0 + kW * u >= a.splits)
                ms[u] = -INFINITY;
        float mn = mw;
#pragma unroll
        for (int u = 0; u < kU; ++u) mn = fmaxf(mn, ms[u]);
        const float c = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - mn);
        l *= c;
        acc.x *= c;
        acc.y *= c;
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const float w = ms[u] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms[u] - mn);
            l = __builtin_fmaf(ls[u], w, l);
            acc.x = __builtin_fmaf(v[u].x, w, acc.x);
            acc.y = __builtin_fmaf(v[u].y, w, acc.y);
        }
        mw = mn;
    }
    s_part[wave][lane] = make_float4(acc.x, acc.y, l, mw);
    __syncthreads();
    if (tid < 64) {
        float M = s_part[0][lane].w;
#pragma unroll
        for (int k = 1; k < kW; ++k) M = fmaxf(M, s_part[k][lane].w);
        float y0 = 0.0f, y1 = 0.0f, lt = 0.0f;
#pragma unroll
        for (int k = 0; k < kW; ++k) {
            const float4 t = s_part[k][lane];
            const float w = t.w == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(t.w - M);
            y0 = __builtin_fmaf(t.x, w, y0);
            y1 = __builtin_fmaf(t.y, w, y1);
            lt = __builtin_fmaf(t.z, w, lt);
        }
        const float o0 = lt > 0.0f ? y0 / lt : 0.0f;
        const float o1 = lt > 0.0f ? y1 / lt : 0.0f;
        const int r = h / a.group;
        const int qh = kvh * a.group + h % a.group;
        const int64_t at = ((int64_t)r * a.n_qh + qh) * kHead + 2 * lane;
        if (a.out_f32)
            *(float2 *)((float *)a.out + at) = make_float2(o0, o1);
        else
            *(uint32_t *)((uint16_t *)a.out + at) = pack_bf16(o0, o1);
    }
}

template <bool KF, bool VF>
hipError_t launch_decode(const AttnArgs &a, const DequantTab &tab, hipStream_t stream) {
    hipLaunchKernelGGL((attn_decode_kernel<KF, VF>), dim3((unsigned)(a.n_kvh * a.splits)),
                       dim3(kDecThreads), 0, stream, a, tab);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(a.n_kvh * a.rows)),
                       dim3(kCombineThreads), 0, stream, a);
    return hipGetLastError();
}

template <int RT>
hipError_t launch_tiles(const AttnArgs &a, const DequantTab &tab, hipStream_t stream) {
    hipLaunchKernelGGL(attn_partial_kernel<RT>, dim3((unsigned)(a.n_kvh * a.splits)),
                       dim3(kAttnThreads), 0, stream, a, tab);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(a.n_kvh * a.rows)),
                       dim3(kCombineThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

int attn_row_tiles(int rows) {
    return rows < 1 ? -1 : rows <= 16 ? 1 : rows <= 32 ? 2 : rows <= 64 ? 4 : -1;
}

hipError_t attn_scratch(float **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static float *per_device[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!per_device[dev]) {
        // the current device is `dev`: the address is that device's copy
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        per_device[dev] = (float *)p;
    }
    *ptr = per_device[dev];
    return hipSuccess;
}

hipError_t launch_attention(const AttnArgs &a, const DequantTab &tab, hipStream_t stream) {
    switch (attn_row_tiles(a.rows)) {
    case 1:
        if (a.k_res)
            return a.v_res ? launch_decode<true, true>(a, tab, stream)
                           : launch_decode<true, false>(a, tab, stream);
        return a.v_res ? launch_decode<false, true>(a, tab, stream)
                       : launch_decode<false, false>(a, tab, stream);
    case 2:
        return launch_tiles<2>(a, tab, stream);
    case 4:
        return launch_tiles<4>(a, tab, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace lynx
