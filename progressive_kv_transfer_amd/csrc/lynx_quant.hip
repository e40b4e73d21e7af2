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
// per-channel cost is spread over 32 tokens.  A workgroup of 512 lanes
// covers a whole page block: wave w takes chunk w, lane l channel pair l;
// the waves meet once in LDS for the page minimum / maximum.
//
// One workgroup per block, grid = blocks, dealt to the 8 XCDs in contiguous
// runs (neighbouring blocks share DRAM rows).  A workgroup first requests
// its block's rows straight into registers: 4 bytes (the lane's channel
// pair) of each of its chunk's 32 rows, one whole 256-byte block row per
// wave instruction.  While they are in flight the compander table arrives
// in LDS by buffer loads into LDS (buffer_load_dwordx4 ... lds): its
// entries are built on the host and travel in the kernel argument, so a
// workgroup copies 7 KiB instead of computing them.  The kernel stays within
// 128 VGPRs and 13 KiB of LDS, so two workgroups (16 waves) share a compute
// unit and one computes while the other's rows stream in: the rare IEEE
// divisions are taken per group of 4 tokens behind a wave-uniform branch (a
// wide unrolled slow path would set the register budget), and the chunk
// minima / maxima meet in LDS as bfloat16 halves (the inputs are bfloat16,
// so this is exact).  Staging the rows through LDS with 16-byte loads
// measured slower (1.41 against 1.36 ms on a 4 GiB set), as did
// nontemporal loads and ordinary code stores.
// The anchor and residual bytes of a lane are 32 contiguous bytes of the
// chunk-tiled stream layout, so a wave writes 2 KiB of each stream that no
// other workgroup touches.
//
// Arithmetic is binary32 with one rounding per operation (built with
// -ffp-contract=off).  The two divisions of Algorithm 1 use
// q = a*r, e = fma(-q, d, a), q' = fma(e, r, q) with r = RN(1/d), which is
// the correctly rounded a/d whenever a = 0 or |a| >= max(2^-100, 2^-125 d)
// and d < 2^125 (Markstein's correction step; checked exhaustively near the
// worst-case significands and on 1.2e10 random operand pairs).  Operands
// outside that range are detected per channel (Stage 1) and per chunk
// (Stage 2) from the statistics and divided with an IEEE division instead.
#include <stddef.h>

#include "lynx_device.h"
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

// bfloat16 metadata: a non-negative scale rounded up to the next bfloat16
// value (a normalised value then stays <= 1), and a value rounded to the
// nearest bfloat16 (ties to even), both returned as binary32.
__device__ __forceinline__ float bf16_up(float x) {
    uint32_t u = __float_as_uint(x);
    u = (u & 0xffffu) ? (u | 0xffffu) + 1u : u;
    return __uint_as_float(u);
}
__device__ __forceinline__ float bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    return __uint_as_float((u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u);
}

constexpr float kTiny100 = 0x1p-100f;
constexpr float kTiny125 = 0x1p-125f;
constexpr float kHuge125 = 0x1p125f;
constexpr float kMuTiny = 0x1p-74f;

// Lane tile: 2 channels x 32 tokens, i.e. one whole chunk of a channel pair.
constexpr int kPairs = kHead / 2;            // channel pairs per block (lanes per chunk)
constexpr int kThreads = kPairs * kChunks;   // 512
constexpr int kWaves = kThreads / 64;        // 8, one per chunk
constexpr int kGroups = kChunk / 4;          // token groups of the division branches

// Workgroup barrier over LDS traffic only: each wave waits for its own LDS
// operations, not for its global stores, which stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until no vector memory operation of this wave is in flight.
__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes,
                                             0x00020000);
}

// A wave-uniform flag the compiler cannot see through: a branch on it stays
// where it is written (inside an unrolled loop) instead of being hoisted
// into one wide copy of the loop per side.
__device__ __forceinline__ uint32_t opaque_uniform(uint32_t f) {
    uint32_t s = __builtin_amdgcn_readfirstlane(f);
    asm volatile("" : "+s"(s));
    return s;
}

// OR a W-bit field into an LSB-first bit stream held in dwords, at field
// index v (bit W v); v is a compile-time constant after unrolling.
template <int W>
__device__ __forceinline__ void put_field(uint32_t *w, int v, uint32_t f) {
    const int pos = W * v, d = pos >> 5, s = pos & 31;
    w[d] |= f << s;
    if (s + W > 32)
        w[d + 1] |= f >> (32 - s);
}

// SH16: the compander buckets are the upper 16 bits of the magnitude, so the
// table address is one v_mad_u32_u16 (high half x 4 + base).  ABITS, RBITS:
// widths of the anchor and residual fields (4 + 4 = the paper's split;
// RBITS = 0 is a single stream of whole codes).  M16: bfloat16 metadata:
// gamma_scale and sigma rounded up and mu to nearest where they are
// produced, the rounded values used from there on and stored as bfloat16
// (the metadata pointers then address uint16 arrays).
//
// Every variant is held to 128 VGPRs (4 waves per SIMD: two workgroups per
// compute unit).  The 3 + 5 and 5 + 3 splits then spill a few registers,
// and still run faster than at one workgroup per CU (1.54 against 2.16 ms
// on a 4 GiB set).
template <int MODE, bool SH16, int ABITS, int RBITS, bool M16 = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void quant_kernel(
    const QuantTab tab, const uint16_t *__restrict__ kv, Geometry g,
    uint8_t *__restrict__ anchor, uint8_t *__restrict__ residual, float *__restrict__ gmin_io,
    float *__restrict__ gscale_io, float *__restrict__ mu_out, float *__restrict__ sigma_out) {
    // Chunk minimum (.x) and maximum (.y) of a lane's two channels as
    // bfloat16 halves (low half = channel 2p).
    __shared__ u32x2 s_mm[kChunks][kPairs];
    __shared__ float4 s_ch[kHead];  // gamma_min, d1, r1, slow flag
    // Compander table, one entry per bucket.  SH16: the host-built word
    // (QuantTab::word).  Otherwise two words: (next threshold, J_base).
    __shared__ __attribute__((aligned(16)))
    uint32_t s_tab[MODE == kModeQuantize ? (SH16 ? kMaxBuckets : 2 * kMaxBuckets) : 1];

    constexpr int kBits = RBITS;  // residual field width
    // Stage 4 bias (+7 at 4 + 4; none for a single stream)
    constexpr uint32_t kBias = kBits > 0 ? (1u << (kBits - 1)) - 1u : 0u;
    constexpr bool kNibbles = ABITS == 4 && RBITS == 4;
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int p = tid & (kPairs - 1);  // channel pair: channels 2p, 2p+1 of the block
    const int j = tid / kPairs;        // chunk: tokens 32 j .. 32 j + 31
    const int wave = tid >> 6;         // = j
    const int lane = tid & 63;

    const int64_t u = xcd_unit((int64_t)__builtin_amdgcn_workgroup_id_x(), g.nblocks);
    const int64_t b = g.block0 + u;
    const int64_t meta0 = b * g.gstride;
    const int64_t cmeta0 = b * g.cstride + j * kHead;
    const uint32_t row_bytes = (uint32_t)g.row_stride * 2u;

    typedef __attribute__((address_space(3))) void lds_void;
    typedef __attribute__((address_space(3))) const u32x2 lds_u32x2;
    typedef __attribute__((address_space(3))) const uint32_t lds_u32;

    // ---- the block's rows into registers ---------------------------------
    // Row i of the lane's chunk: the 4 bytes of its channel pair (one whole
    // 256-byte block row per wave instruction), all 32 requested at once.
    // Buffer loads: the row offset is a scalar (no per-lane address
    // arithmetic); every offset stays below 255 row_bytes + 256 < 2^31.
    uint32_t raw[kChunk];
    {
        const int64_t tp = b / g.heads;
        const uint16_t *bp = kv + (tp / g.pages) * g.tensor_stride +
                             (int64_t)(tp % g.pages) * kPage * g.row_stride +
                             (b % g.heads) * kHead;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(bp, 0x7fffffff);
        const uint32_t voff = (uint32_t)(kChunk * j) * row_bytes + 4u * (uint32_t)p;
#pragma unroll
        for (int i = 0; i < kChunk; ++i)
            raw[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, (uint32_t)i * row_bytes, 0);
    }

    // ---- compander table into LDS ---------------------------------------
    if constexpr (MODE == kModeQuantize && SH16) {
        // 1 KiB of entries per wave from the kernel argument (bounds-checked
        // against the word array; entries past nbuckets are never indexed).
        // The table is the first kernel argument, so its bytes start the
        // kernel argument segment (its address taken from the segment
        // pointer: taking the parameter's own address would copy it).
        static_assert(kMaxBuckets * 4 <= kWaves * 1024, "one load per wave covers the table");
        static_assert(offsetof(QuantTab, word) % 16 == 0, "16-byte loads of the words");
        if (wave * 1024 < kMaxBuckets * 4) {
            const uintptr_t words =
                (uintptr_t)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(QuantTab, word);
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc((const void *)words, (int)sizeof(tab.word));
            const uint32_t lds = __builtin_amdgcn_readfirstlane(
                (uint32_t)(uintptr_t)(lds_void *)&s_tab[wave * 256]);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(uintptr_t)lds, 16,
                                                     (uint32_t)lane * 16u,
                                                     (uint32_t)wave * 1024u, 0, 0);
        }
    } else if constexpr (MODE == kModeQuantize) {
        // Two words per bucket from the thresholds; above code 127 (the top
        // of a single 8-bit stream) there is no next threshold: +inf, which
        // no clamped magnitude reaches.  All of a lane's bucket codes are
        // loaded first, then their thresholds: two dependent loads per lane.
        constexpr int kPer = (kMaxBuckets + kThreads - 1) / kThreads;
        uint32_t code[kPer], next[kPer];
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int i = tid + k * kThreads;
            code[k] = i < tab.nbuckets ? tab.bucket_code[i] : 0u;
        }
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            next[k] = code[k] + 1 < 128 ? __float_as_uint(tab.thr[code[k] + 1]) : 0x7f800000u;
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int i = tid + k * kThreads;
            if (i >= tab.nbuckets)
                break;
            s_tab[2 * i] = next[k];
            s_tab[2 * i + 1] = code[k] + kBias;
        }
    }
    const float mag_lo = __uint_as_float((uint32_t)tab.bucket_lo << tab.shift);
    const uint32_t sh = (uint32_t)tab.shift;
    const uint32_t tab_base = (uint32_t)(uintptr_t)(lds_u32 *)s_tab -
                              (uint32_t)tab.bucket_lo * (SH16 ? 4u : 8u);

    // ---- 32 token rows x 2 channels --------------------------------------
    // The wave's own loads (rows, and table words into LDS) have landed.
    vm_wait_all();
    float x[kChunk][2];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
        x[i][0] = bf16_lo(raw[i]);
        x[i][1] = bf16_hi(raw[i]);
    }

    // ---- phase 1: page statistics ----------------------------------------
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
        s_mm[j][p] = u32x2{(__float_as_uint(mn[0]) >> 16) | (__float_as_uint(mn[1]) & 0xffff0000u),
                           (__float_as_uint(mx[0]) >> 16) | (__float_as_uint(mx[1]) & 0xffff0000u)};
    }
    // Every wave has passed its wait above: the table is complete here.
    lds_barrier();
    if (tid < kHead) {
        float gmin, gsc;
        if (MODE == kModeBlockStats) {
            gmin = gmin_io[meta0 + tid];
            gsc = gscale_io[meta0 + tid];
        } else {
            const int hp = tid >> 1;
            const bool odd = tid & 1;
            auto half = [&](uint32_t w) {
                return __uint_as_float(odd ? (w & 0xffff0000u) : (w << 16));
            };
            float a = half(s_mm[0][hp].x), m = half(s_mm[0][hp].y);
#pragma unroll
            for (int w = 1; w < kChunks; ++w) {
                a = fminf(a, half(s_mm[w][hp].x));
                m = fmaxf(m, half(s_mm[w][hp].y));
            }
            // canonical +0 for a zero minimum (a bf16 value) and scale
            gmin = a + 0.0f;
            gsc = (m - gmin) + 0.0f;
            if (M16) {
                gsc = bf16_up(gsc);
                ((uint16_t *)gmin_io)[meta0 + tid] = (uint16_t)(__float_as_uint(gmin) >> 16);
                ((uint16_t *)gscale_io)[meta0 + tid] = (uint16_t)(__float_as_uint(gsc) >> 16);
            } else {
                gmin_io[meta0 + tid] = gmin;
                gscale_io[meta0 + tid] = gsc;
            }
        }
        float d1 = gsc + tab.eps;
        float r1 = __fdiv_rn(1.0f, d1);
        // Every nonzero x - gamma_min of a bf16 channel is at least
        // 2^-9 |gamma_min|; the fast division needs it above the bound.
        bool fast = gmin != 0.0f &&
                    fabsf(gmin) * 0x1p-9f >= fmaxf(kTiny100, d1 * kTiny125) && d1 < kHuge125;
        s_ch[tid] = make_float4(gmin, d1, r1, fast ? 0.0f : 1.0f);
    }
    if (MODE == kModePageStats)
        return;
    lds_barrier();

    // ---- phase 2: normalise, chunk mean and max |X - mu| -----------------
    // Where a lane needs the IEEE division its whole wave takes it (both
    // give the correctly rounded quotient where the fast one applies).
    {
        const float4 c0 = s_ch[2 * p], c1 = s_ch[2 * p + 1];
        const float gm[2] = {c0.x, c1.x}, d1[2] = {c0.y, c1.y}, r1[2] = {c0.z, c1.z};
        const uint32_t slow =
            __builtin_amdgcn_ballot_w64(c0.w != 0.0f || c1.w != 0.0f) != 0 ? 1u : 0u;
#pragma unroll
        for (int q = 0; q < kGroups; ++q) {
            if (opaque_uniform(slow)) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        x[4 * q + k][e] = __fdiv_rn(x[4 * q + k][e] - gm[e], d1[e]);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        x[4 * q + k][e] = div_fast(x[4 * q + k][e] - gm[e], d1[e], r1[e]);
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
        mu[e] = s32 * 0.03125f + 0.0f;  // canonical +0 for a zero mean
        if (M16)
            mu[e] = bf16_rne(mu[e]);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            x[i][e] = x[i][e] - mu[e];
            m = fmaxf(m, fabsf(x[i][e]));
        }
        sg[e] = M16 ? bf16_up(m) : m;
    }
    if (M16) {
        *(uint32_t *)((uint16_t *)mu_out + cmeta0 + 2 * p) =
            (__float_as_uint(mu[0]) >> 16) | (__float_as_uint(mu[1]) & 0xffff0000u);
        *(uint32_t *)((uint16_t *)sigma_out + cmeta0 + 2 * p) =
            (__float_as_uint(sg[0]) >> 16) | (__float_as_uint(sg[1]) & 0xffff0000u);
    } else {
        *(float2 *)(mu_out + cmeta0 + 2 * p) = make_float2(mu[0], mu[1]);
        *(float2 *)(sigma_out + cmeta0 + 2 * p) = make_float2(sg[0], sg[1]);
    }
    if (MODE == kModeBlockStats)
        return;

    // ---- phase 3: scale, compand, split, pack -----------------------------
    {
        const float d2[2] = {sg[0] + tab.eps, sg[1] + tab.eps};
        const float r2[2] = {__fdiv_rn(1.0f, d2[0]), __fdiv_rn(1.0f, d2[1])};
        const uint32_t slow = __builtin_amdgcn_ballot_w64((mu[0] > 0.0f && mu[0] < kMuTiny) ||
                                                          (mu[1] > 0.0f && mu[1] < kMuTiny)) != 0
                                  ? 1u
                                  : 0u;
#pragma unroll
        for (int q = 0; q < kGroups; ++q) {
            if (opaque_uniform(slow)) {
                // IEEE quotient; + 0 turns a -0 quotient into +0 so that the
                // sign bit below is exactly [X_cent < 0].
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        x[4 * q + k][e] = __fdiv_rn(x[4 * q + k][e], d2[e]) + 0.0f;
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        x[4 * q + k][e] = div_fast(x[4 * q + k][e], d2[e], r2[e]);
            }
        }
    }
    // Magnitudes are clamped into [first value of the lowest bucket, 1]
    // (every finite |X_final| is <= 1; the lower clamp keeps code 0 since
    // that bucket starts below the first threshold, and non-finite inputs
    // stay inside the table).  The bucket offset is folded into the LDS
    // base address.
    // J = code + bias of Stage 4 for one quotient, in the top byte (the low
    // bytes are not part of it): SH16, one v_add of the magnitude's low half
    // (SDWA word select) to the table word; otherwise the threshold compare.
    auto jtop = [&](float xq) -> uint32_t {
        float m = __builtin_amdgcn_fmed3f(fabsf(xq), mag_lo, 1.0f);
        uint32_t mb = __float_as_uint(m);
        uint32_t addr;
        if constexpr (SH16) {
            asm("v_mad_u32_u16 %0, %1, 4, %2 op_sel:[1,0,0,0]"
                : "=v"(addr) : "v"(mb), "s"(tab_base));
            const uint32_t ent = *(lds_u32 *)(uintptr_t)addr;
            uint32_t t;
            asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD "
                "src0_sel:DWORD src1_sel:WORD_0"
                : "=v"(t) : "v"(ent), "v"(mb));
            return t;
        } else {
            asm("v_lshl_add_u32 %0, %1, 3, %2" : "=v"(addr) : "v"(mb >> sh), "s"(tab_base));
            u32x2 ent = *(lds_u32x2 *)(uintptr_t)addr;
            return (ent[1] + (mb >= ent[0] ? 1u : 0u)) << 24;
        }
    };
    auto code_j = [&](float xq) { return jtop(xq) >> 24; };
    if constexpr (kNibbles) {
        u32x4 av[2], rv[2];
#pragma unroll
        for (int q = 0; q < 8; ++q) {  // tokens 4q .. 4q+3
            uint32_t T[4][2];
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    // J = code + 7: high nibble = anchor magnitude
                    // (code + 7) >> 4, low nibble ^ 7 = residual (-code) mod 16.
                    T[k][e] = jtop(x[4 * q + k][e]);
            // byte k of w0 / w1 = J of channel 2p / 2p+1 at token 4q + k
            // (the top bytes gathered by v_perm: 0x0c0c0703 takes byte 3
            // of each source into bytes 0 and 1, 0x05040100 joins two
            // such halves)
            auto gather = [](uint32_t t0, uint32_t t1, uint32_t t2, uint32_t t3) {
                return __builtin_amdgcn_perm(__builtin_amdgcn_perm(t3, t2, 0x0c0c0703u),
                                             __builtin_amdgcn_perm(t1, t0, 0x0c0c0703u),
                                             0x05040100u);
            };
            uint32_t w0 = gather(T[0][0], T[1][0], T[2][0], T[3][0]);
            uint32_t w1 = gather(T[0][1], T[1][1], T[2][1], T[3][1]);
            uint32_t a = ((w0 >> 4) & 0x0f0f0f0fu) | (w1 & 0xf0f0f0f0u);
            uint32_t r = ((w0 & 0x0f0f0f0fu) | ((w1 << 4) & 0xf0f0f0f0u)) ^ 0x77777777u;
            // Sign bits of the quotients replicated to bytes (v_perm
            // selectors 9 and 11), then to nibbles: the anchor of a
            // negative value is the one's complement of its magnitude
            // (-V - 1).
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
        // The chunk's 2 KiB of each stream, [chunk j][pair][token of chunk]:
        // the lane's pair run is 32 bytes, tokens 0-15 in v[0] and 16-31 in
        // v[1].  One permlane32 swap per dword leaves lane l < 32 the first
        // halves of the runs of pairs l and l + 32, and lane l + 32 their
        // second halves, so the first store instruction writes pairs 0-31
        // (1 KiB, whole cache lines) and the second pairs 32-63; storing
        // each lane's run as it is would leave every line half written by
        // each instruction (measured 3% slower on the same access pattern).
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const auto sa = __builtin_amdgcn_permlane32_swap(av[0][k], av[1][k], false, false);
            av[0][k] = sa[0];
            av[1][k] = sa[1];
            const auto sr = __builtin_amdgcn_permlane32_swap(rv[0][k], rv[1][k], false, false);
            rv[0][k] = sr[0];
            rv[1][k] = sr[1];
        }
        const int64_t toff = j * (kHead / 2 * kChunk) + 32 * (lane & 31) + 16 * (lane >> 5);
        u32x4 *ao = (u32x4 *)(anchor + b * g.astride + toff);
        u32x4 *ro = (u32x4 *)(residual + b * (kPage * kHead / 2) + toff);
        // Nontemporal stores (measured faster than ordinary ones here).
        __builtin_nontemporal_store(av[0], ao);
        __builtin_nontemporal_store(av[1], ao + 64);  // + 1 KiB
        __builtin_nontemporal_store(rv[0], ro);
        __builtin_nontemporal_store(rv[1], ro + 64);
    } else {
        // Other widths: field 2 i + e (token i, channel 2p + e) of the lane's
        // run at bit w (2 i + e); the anchor field is the magnitude J >> b,
        // one's-complemented for a negative quotient, the residual
        // (J ^ bias) mod 2^b = (-code) mod 2^b.  A single stream (b = 0)
        // stores the whole code in the anchor field.
        constexpr uint32_t kMaskA = (1u << ABITS) - 1u;
        constexpr uint32_t kMaskR = kBits > 0 ? (1u << kBits) - 1u : 0u;
        uint32_t aw[2 * ABITS], rw[kBits > 0 ? 2 * kBits : 1];
#pragma unroll
        for (int d = 0; d < 2 * ABITS; ++d) aw[d] = 0u;
#pragma unroll
        for (int d = 0; d < 2 * kBits; ++d) rw[d] = 0u;
#pragma unroll
        for (int i = 0; i < kChunk; ++i)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t J = code_j(x[i][e]);
                const uint32_t neg = (uint32_t)((int32_t)__float_as_uint(x[i][e]) >> 31);
                put_field<ABITS>(aw, 2 * i + e, ((J >> kBits) ^ neg) & kMaskA);
                if constexpr (kBits > 0)
                    put_field<kBits>(rw, 2 * i + e, (J ^ kBias) & kMaskR);
            }
        // Run of 8 w bytes per (chunk, pair), 4096 w bytes per block.
        const int64_t aoff = b * g.astride + (int64_t)(j * (kHead / 2) + p) * (8 * ABITS);
        const int64_t roff =
            b * (kPage * kHead / 8 * kBits) + (int64_t)(j * (kHead / 2) + p) * (8 * kBits);
        u32x2 *ao = (u32x2 *)(anchor + aoff);
        u32x2 *ro = (u32x2 *)(residual + roff);
#pragma unroll
        for (int d = 0; d < ABITS; ++d) ao[d] = u32x2{aw[2 * d], aw[2 * d + 1]};
#pragma unroll
        for (int d = 0; d < kBits; ++d) ro[d] = u32x2{rw[2 * d], rw[2 * d + 1]};
    }
}

}  // namespace

template <int MODE, bool SH16, int ABITS, int RBITS, bool M16 = false>
static hipError_t launch_variant(const uint16_t *kv, const Geometry &g, const QuantTab &tab,
                                 uint8_t *anchor, uint8_t *residual, float *gmin, float *gscale,
                                 float *mu, float *sigma, hipStream_t stream) {
    hipLaunchKernelGGL((quant_kernel<MODE, SH16, ABITS, RBITS, M16>), dim3((unsigned)g.nblocks),
                       dim3(kThreads), 0, stream, tab, kv, g, anchor, residual, gmin, gscale, mu,
                       sigma);
    return hipGetLastError();
}

template <int ABITS, int RBITS, bool M16 = false>
static hipError_t launch_split(const uint16_t *kv, const Geometry &g, const QuantTab &tab,
                               uint8_t *anchor, uint8_t *residual, float *gmin, float *gscale,
                               float *mu, float *sigma, hipStream_t stream) {
    if (tab.shift == 16)
        return launch_variant<kModeQuantize, true, ABITS, RBITS, M16>(
            kv, g, tab, anchor, residual, gmin, gscale, mu, sigma, stream);
    return launch_variant<kModeQuantize, false, ABITS, RBITS, M16>(
        kv, g, tab, anchor, residual, gmin, gscale, mu, sigma, stream);
}

// One workgroup per block: the grid is the launch's block count (the host
// cuts a call into launches of at most 2^22 blocks).
hipError_t launch_quantize(const uint16_t *kv, const Geometry &g, const QuantTab &tab,
                           uint8_t *anchor, uint8_t *residual, float *gmin, float *gscale,
                           float *mu, float *sigma, int mode, int anchor_bits,
                           int residual_bits, int meta_bits, hipStream_t stream) {
    if (g.nblocks == 0)
        return hipSuccess;
    if (g.nblocks > (int64_t(1) << 22))
        return hipErrorInvalidValue;
    if (meta_bits == 16) {
        if (mode != kModeQuantize || anchor_bits != 4 || residual_bits != 4)
            return hipErrorInvalidValue;
        return launch_split<4, 4, true>(kv, g, tab, anchor, residual, gmin, gscale, mu, sigma,
                                        stream);
    }
    switch (mode) {
    case kModeQuantize:
        switch (anchor_bits * 16 + residual_bits) {
        case 3 * 16 + 5:
            return launch_split<3, 5>(kv, g, tab, anchor, residual, gmin, gscale, mu, sigma,
                                      stream);
        case 4 * 16 + 4:
            return launch_split<4, 4>(kv, g, tab, anchor, residual, gmin, gscale, mu, sigma,
                                      stream);
        case 5 * 16 + 3:
            return launch_split<5, 3>(kv, g, tab, anchor, residual, gmin, gscale, mu, sigma,
                                      stream);
        case 6 * 16 + 2:
            return launch_split<6, 2>(kv, g, tab, anchor, residual, gmin, gscale, mu, sigma,
                                      stream);
        case 4 * 16 + 0:
            return launch_split<4, 0>(kv, g, tab, anchor, residual, gmin, gscale, mu, sigma,
                                      stream);
        case 8 * 16 + 0:
            return launch_split<8, 0>(kv, g, tab, anchor, residual, gmin, gscale, mu, sigma,
                                      stream);
        default:
            return hipErrorInvalidValue;
        }
    case kModePageStats:
        return launch_variant<kModePageStats, false, 4, 4>(kv, g, tab, anchor, residual, gmin,
                                                           gscale, mu, sigma, stream);
    default:
        return launch_variant<kModeBlockStats, false, 4, 4>(kv, g, tab, anchor, residual, gmin,
                                                            gscale, mu, sigma, stream);
    }
}

}  // namespace lynx
