// gfx950 speculative verification: the step that closes a Lynx decode round
// (paper Section 4.3): drafts generated on the Anchor-only cache are checked
// against the logits of one forward pass on the full cache; the longest
// accepted prefix is kept and the first divergence is corrected (the notes'
// Eq. (10): accept s_t when u_t < p_t(s_t) / q_t(s_t); Eq. (11): draw the
// correction from max(0, p_k - q_k)); after a fully accepted draft the next
// token is drawn from the target distribution.
//
//   verify_stats_kernel   one workgroup per (row, 2048-token chunk) of the
//                         2T + 1 logit rows (T draft rows q, T + 1 target
//                         rows p): chunk max and sum of exp_d(l - max) in
//                         binary64, 8 independent exponentials per lane;
//   verify_chunk_kernel   one workgroup per chunk of the chosen row: each
//                         takes the decision (8 lanes per row merge the
//                         chunk statistics, 32 rows at a time; one lane per
//                         draft tests Eq. (10)), workgroup 0 stores it (the
//                         first rejection k and the statistics of the row to
//                         sample from), and each sums its chunk's weights;
//   verify_select_kernel  one workgroup: the chunk that holds u * total
//                         (lanes over runs of chunks, block scan), then the
//                         8-token run inside it (block scan of the lane
//                         sums), then the token inside the run.
// Ratios and sums are binary64, so a decision can only differ from a
// sequential evaluation within ~1e-15 of its threshold.
#include "lynx_attn_args.h"

namespace lynx {
namespace {

constexpr int kThreads = 256;
constexpr int kPer = kVerifyChunk / kThreads;  // 8 tokens per lane and chunk
static_assert(kVerifyChunk % kThreads == 0, "lanes split a chunk evenly");

// e^x in binary64, inlined (the library exponential is an out-of-line call,
// which serializes a lane's exponentials): Cody and Waite's reduction
// x = k ln 2 + r with ln 2 held as RN(ln 2) + RN(ln 2 - RN(ln 2)) and both
// products by k formed inside an FMA, |r| <= ln 2 / 2, then the Taylor
// polynomial of e^r to degree 13 (truncation below 1e-17 relative, the
// coefficients RN(1/n!)) by Horner's rule, scaled by 2^k.  NaN passes
// through, arguments below -746 (and -inf) give 0.  Within 1 ulp of the C
// library's exp on 2e8 arguments in [-746, 0] (the same steps in C on the
// CPU; a 1e6-argument run of that check is part of the CPU test suite).
__device__ __forceinline__ double exp_d(double x) {
    constexpr double kLog2e = 0x1.71547652b82fep+0;   // RN(1 / ln 2)
    constexpr double kLn2Hi = 0x1.62e42fefa39efp-1;   // RN(ln 2)
    constexpr double kLn2Lo = 0x1.abc9e3b39803fp-56;  // RN(ln 2 - kLn2Hi)
    if (!(x > -746.0))
        return x != x ? x : 0.0;
    const double k = __builtin_rint(x * kLog2e);
    double r = __builtin_fma(-k, kLn2Hi, x);
    r = __builtin_fma(-k, kLn2Lo, r);
    double p = 1.6059043836821613e-10;        // 1/13!
    p = __builtin_fma(p, r, 2.08767569878681e-09);    // 1/12!
    p = __builtin_fma(p, r, 2.505210838544172e-08);   // 1/11!
    p = __builtin_fma(p, r, 2.755731922398589e-07);   // 1/10!
    p = __builtin_fma(p, r, 2.7557319223985893e-06);  // 1/9!
    p = __builtin_fma(p, r, 2.48015873015873e-05);    // 1/8!
    p = __builtin_fma(p, r, 0.0001984126984126984);   // 1/7!
    p = __builtin_fma(p, r, 0.001388888888888889);    // 1/6!
    p = __builtin_fma(p, r, 0.008333333333333333);    // 1/5!
    p = __builtin_fma(p, r, 0.041666666666666664);    // 1/4!
    p = __builtin_fma(p, r, 0.16666666666666666);     // 1/3!
    p = __builtin_fma(p, r, 0.5);
    p = __builtin_fma(p, r, 1.0);
    p = __builtin_fma(p, r, 1.0);
    return __builtin_ldexp(p, (int)k);
}

// Cross-lane moves without LDS round trips: DPP within rows of 16 lanes
// (quad permutes, the mirrored lane of the half row and of the row; row
// shifts for the scan), v_readlane across the four rows.  A binary64 value
// moves as its two halves.
template <int CTRL, bool ZERO_OUT = false>  // ZERO_OUT: lanes without a source read 0
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, ZERO_OUT);
}
template <int CTRL, bool ZERO_OUT = false>
__device__ __forceinline__ double dpp_d(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint64_t lo = dpp_u<CTRL, ZERO_OUT>((uint32_t)u);
    const uint64_t hi = dpp_u<CTRL, ZERO_OUT>((uint32_t)(u >> 32));
    return __builtin_bit_cast(double, (hi << 32) | lo);
}
__device__ __forceinline__ double readlane_d(double x, int l) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, (hi << 32) | lo);
}
constexpr int kQuadSwap1 = 0xb1, kQuadSwap2 = 0x4e, kHalfMirror = 0x141, kRowMirror = 0x140;

// Every lane of a group of 8 (lanes 8 g .. 8 g + 7) gets the group's
// maximum / sum.
__device__ __forceinline__ double group_max8(double x) {
    x = fmax(x, dpp_d<kQuadSwap1>(x));
    x = fmax(x, dpp_d<kQuadSwap2>(x));
    return fmax(x, dpp_d<kHalfMirror>(x));
}
__device__ __forceinline__ double group_sum8(double x) {
    x += dpp_d<kQuadSwap1>(x);
    x += dpp_d<kQuadSwap2>(x);
    return x + dpp_d<kHalfMirror>(x);
}

// Wave reductions, the same value in every lane.
__device__ __forceinline__ double wave_max_d(double x) {
    x = group_max8(x);
    x = fmax(x, dpp_d<kRowMirror>(x));
    return fmax(fmax(readlane_d(x, 0), readlane_d(x, 16)),
                fmax(readlane_d(x, 32), readlane_d(x, 48)));
}
__device__ __forceinline__ double wave_sum_d(double x) {
    x = group_sum8(x);
    x += dpp_d<kRowMirror>(x);
    return (readlane_d(x, 0) + readlane_d(x, 16)) + (readlane_d(x, 32) + readlane_d(x, 48));
}
__device__ __forceinline__ int wave_min_i(int x) {
    x = min(x, (int)dpp_u<kQuadSwap1>((uint32_t)x));
    x = min(x, (int)dpp_u<kQuadSwap2>((uint32_t)x));
    x = min(x, (int)dpp_u<kHalfMirror>((uint32_t)x));
    x = min(x, (int)dpp_u<kRowMirror>((uint32_t)x));
    return min(min(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
               min(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}
__device__ __forceinline__ int wave_max_i(int x) {
    x = max(x, (int)dpp_u<kQuadSwap1>((uint32_t)x));
    x = max(x, (int)dpp_u<kQuadSwap2>((uint32_t)x));
    x = max(x, (int)dpp_u<kHalfMirror>((uint32_t)x));
    x = max(x, (int)dpp_u<kRowMirror>((uint32_t)x));
    return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
               max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// Inclusive prefix sum over the wave in lane order: row shifts by 1, 2, 4
// and 8 (lanes before the row's start read 0), then the totals of the rows
// before.
__device__ __forceinline__ double wave_incl_scan_d(double x, int lane) {
    x += dpp_d<0x111, true>(x);  // row_shr:1
    x += dpp_d<0x112, true>(x);  // row_shr:2
    x += dpp_d<0x114, true>(x);  // row_shr:4
    x += dpp_d<0x118, true>(x);  // row_shr:8
    const double t0 = readlane_d(x, 15), t1 = readlane_d(x, 31), t2 = readlane_d(x, 47);
    const int row = lane >> 4;
    const double off = row == 0 ? 0.0 : row == 1 ? t0 : row == 2 ? t0 + t1 : (t0 + t1) + t2;
    return x + off;
}

// Block-wide (256 lanes = 4 waves) reductions; every lane gets the result.
__device__ double block_max_d(double x, double *s_red) {
    x = wave_max_d(x);
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    __syncthreads();
    if ((tid & 63) == 0) s_red[tid >> 6] = x;
    __syncthreads();
    return fmax(fmax(s_red[0], s_red[1]), fmax(s_red[2], s_red[3]));
}

__device__ double block_sum_d(double x, double *s_red) {
    x = wave_sum_d(x);
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    __syncthreads();
    if ((tid & 63) == 0) s_red[tid >> 6] = x;
    __syncthreads();
    return (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
}

__device__ int block_min_i(int x, int *s_int) {
    x = wave_min_i(x);
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    __syncthreads();
    if ((tid & 63) == 0) s_int[tid >> 6] = x;
    __syncthreads();
    return min(min(s_int[0], s_int[1]), min(s_int[2], s_int[3]));
}

__device__ int block_max_i(int x, int *s_int) {
    x = wave_max_i(x);
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    __syncthreads();
    if ((tid & 63) == 0) s_int[tid >> 6] = x;
    __syncthreads();
    return max(max(s_int[0], s_int[1]), max(s_int[2], s_int[3]));
}

// Lane intervals of one double per lane in lane order: lane l gets
// [lo_l, hi_l) with lo_l the sum of lanes 0 .. l - 1 and hi_l = lo_{l+1}
// (the total for the last lane), so the intervals tile [0, total) without
// gaps.
__device__ void block_intervals(double x, double *s_pre, double *s_wsum, double *lo,
                                double *hi, double *total) {
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63, wave = tid >> 6;
    const double incl = wave_incl_scan_d(x, lane);
    __syncthreads();
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    double off = 0.0;
    for (int w = 0; w < wave; ++w) off += s_wsum[w];
    const double t = (s_wsum[0] + s_wsum[1]) + (s_wsum[2] + s_wsum[3]);
    *lo = off + incl - x;
    s_pre[tid] = *lo;
    __syncthreads();
    *hi = tid + 1 < kThreads ? s_pre[tid + 1] : t;
    *total = t;
}

// Row r < T is draft row r; row T + i is target row i.
__device__ __forceinline__ const float *row_ptr(const VerifyArgs &a, int r) {
    return r < a.t ? a.draft + (int64_t)r * a.vocab : a.target + (int64_t)(r - a.t) * a.vocab;
}

__device__ __forceinline__ double *chunk_sums(const VerifyArgs &a) {
    return a.ws + (int64_t)(2 * a.t + 1) * a.chunks * 2;
}

// The decision: k, then mp, rp, mq, rq.
__device__ __forceinline__ double *choice_slots(const VerifyArgs &a) {
    return chunk_sums(a) + a.chunks;
}

__global__ __launch_bounds__(kThreads) void verify_stats_kernel(VerifyArgs a) {
    __shared__ double s_max[4], s_sum[4];  // one slot per wave, each written once
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int wg = (int)__builtin_amdgcn_workgroup_id_x();
    const int r = wg / a.chunks, c = wg % a.chunks;
    const float *l = row_ptr(a, r);
    const int x0 = c * kVerifyChunk;
    double v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int x = x0 + tid + kThreads * i;
        v[i] = x < a.vocab ? (double)l[x] : -INFINITY;
    }
    double m = v[0];
#pragma unroll
    for (int i = 1; i < kPer; ++i) m = fmax(m, v[i]);
    m = wave_max_d(m);
    if ((tid & 63) == 0) s_max[tid >> 6] = m;
    __syncthreads();
    m = fmax(fmax(s_max[0], s_max[1]), fmax(s_max[2], s_max[3]));
    double s = 0.0;
    if (m != -INFINITY) {  // a chunk of -inf logits holds no mass
        double e[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) e[i] = exp_d(v[i] - m);
#pragma unroll
        for (int i = 0; i < kPer; ++i) s += e[i];
    }
    s = wave_sum_d(s);
    if ((tid & 63) == 0) s_sum[tid >> 6] = s;
    __syncthreads();
    s = (s_sum[0] + s_sum[1]) + (s_sum[2] + s_sum[3]);
    if (tid == 0) {
        a.ws[(int64_t)wg * 2] = m;
        a.ws[(int64_t)wg * 2 + 1] = s;
    }
}

// Accepted prefix k (Eq. 10) and the statistics of the row the next token is
// drawn from: target row k, minus draft row k when k < T (Eq. 11); rp, rq
// are the reciprocals of the row sums.
struct Choice {
    int k;
    double mp, rp, mq, rq;
};

// The decision, computed by every lane of the block: row statistics merged
// from the chunk statistics, then Eq. (10) per draft.
__device__ Choice decide(const VerifyArgs &a, double *s_m, double *s_s, int *s_int) {
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    // The draft lanes' loads go out first, so that they overlap the merge.
    double lp = 0.0, lq = 0.0, ua = 0.0;
    bool in_vocab = false;
    if (tid < a.t) {
        const int s = a.tokens[tid];
        in_vocab = s >= 0 && s < a.vocab;  // not a token: rejected, nothing read
        if (in_vocab) {
            lp = (double)a.target[(int64_t)tid * a.vocab + s];
            lq = (double)a.draft[(int64_t)tid * a.vocab + s];
        }
        ua = a.u_accept[tid];
    }
    // Row statistics (max, sum of exp_d(l - max)) merged from the chunks: a
    // group of 8 lanes per row, 32 rows at a time (the 17 rows of 8 drafts
    // in one pass).  Up to 16 x 8 chunks a lane holds its chunks'
    // statistics in registers (all loads in flight at once, independent
    // exponentials); beyond that it streams them twice.
    constexpr int kG = 8, kHeld = 16;
    const int grp = tid / kG, sub = tid % kG;
    for (int r0 = 0; r0 < 2 * a.t + 1; r0 += kThreads / kG) {
        const int r = r0 + grp;
        const bool live = r < 2 * a.t + 1;
        const double *st = a.ws + (int64_t)(live ? r : 0) * a.chunks * 2;
        double m = -INFINITY, s = 0.0;
        if (a.chunks <= kG * kHeld) {  // uniform
            double mm[kHeld], ss[kHeld];
#pragma unroll
            for (int i = 0; i < kHeld; ++i) {
                const int c = sub + kG * i;
                const bool ok = live && c < a.chunks;
                mm[i] = ok ? st[2 * c] : -INFINITY;
                ss[i] = ok ? st[2 * c + 1] : 0.0;
            }
#pragma unroll
            for (int i = 0; i < kHeld; ++i) m = fmax(m, mm[i]);
            m = group_max8(m);
            double e[kHeld];
#pragma unroll
            for (int i = 0; i < kHeld; ++i)
                e[i] = mm[i] != -INFINITY ? ss[i] * exp_d(mm[i] - m) : 0.0;
#pragma unroll
            for (int i = 0; i < kHeld; ++i) s += e[i];
        } else {
            if (live)
                for (int c = sub; c < a.chunks; c += kG) m = fmax(m, st[2 * c]);
            m = group_max8(m);
            if (live)
                for (int c = sub; c < a.chunks; c += kG) {
                    const double mc = st[2 * c];
                    if (mc != -INFINITY) s += st[2 * c + 1] * exp_d(mc - m);
                }
        }
        s = group_sum8(s);
        if (live && sub == 0) {
            s_m[r] = m;
            s_s[r] = s;
        }
    }
    __syncthreads();
    int rej = a.t;
    if (tid < a.t) {
        bool ok = in_vocab;
        if (ok) {
            const double p = exp_d(lp - s_m[a.t + tid]) / s_s[a.t + tid];
            const double q = exp_d(lq - s_m[tid]) / s_s[tid];
            ok = ua < p / q;
        }
        if (!ok) rej = tid;
    }
    Choice c;
    c.k = block_min_i(rej, s_int);
    c.mp = s_m[a.t + c.k];
    c.rp = 1.0 / s_s[a.t + c.k];
    c.mq = c.k < a.t ? s_m[c.k] : 0.0;
    c.rq = c.k < a.t ? 1.0 / s_s[c.k] : 1.0;
    return c;
}

__device__ __forceinline__ Choice load_choice(const VerifyArgs &a) {
    const double *ch = choice_slots(a);
    Choice c;
    c.k = (int)ch[0];
    c.mp = ch[1];
    c.rp = ch[2];
    c.mq = ch[3];
    c.rq = ch[4];
    return c;
}

// Weights max(0, p_k - q_k) (p_T after a full accept) of the kPer
// consecutive tokens x0 .. x0 + kPer - 1 (0 beyond the vocabulary).
__device__ __forceinline__ void lane_weights(const VerifyArgs &a, const Choice &c, int x0,
                                             double w[kPer]) {
    const float *pr = a.target + (int64_t)c.k * a.vocab;
    const bool two = c.k < a.t;
    const float *qr = two ? a.draft + (int64_t)c.k * a.vocab : pr;
    double lp[kPer], lq[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const bool in = x0 + i < a.vocab;
        lp[i] = in ? (double)pr[x0 + i] : -INFINITY;
        lq[i] = in && two ? (double)qr[x0 + i] : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const double p = exp_d(lp[i] - c.mp) * c.rp;
        if (!two) {
            w[i] = p;
        } else {
            const double q = exp_d(lq[i] - c.mq) * c.rq;
            w[i] = p > q ? p - q : 0.0;
        }
    }
}

// One workgroup per chunk of the chosen row: each takes the decision (a few
// hundred loads of chunk statistics, cheaper than a launch of its own),
// workgroup 0 stores it for the select kernel, and each sums its chunk's
// weights.
__global__ __launch_bounds__(kThreads) void verify_chunk_kernel(VerifyArgs a) {
    __shared__ double s_m[2 * kVerifyMaxDraft + 1], s_s[2 * kVerifyMaxDraft + 1];
    __shared__ double s_red[4];
    __shared__ int s_int[4];
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int c = (int)__builtin_amdgcn_workgroup_id_x();
    const Choice ch = decide(a, s_m, s_s, s_int);
    if (c == 0 && tid == 0) {
        double *slot = choice_slots(a);
        slot[0] = (double)ch.k;
        slot[1] = ch.mp;
        slot[2] = ch.rp;
        slot[3] = ch.mq;
        slot[4] = ch.rq;
    }
    double w[kPer];
    lane_weights(a, ch, c * kVerifyChunk + tid * kPer, w);
    double part = 0.0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) part += w[i];
    part = block_sum_d(part, s_red);
    if (tid == 0) chunk_sums(a)[c] = part;
}

// One workgroup.  Chunk level: lane l sums the chunk sums of its run of
// chunks in order and gets its interval of the running total; the first
// lane whose interval holds u * total walks its run to the chunk (the last
// chunk of the row ends at the total; if rounding leaves the target past
// the walked sums, the run's last chunk is taken).  Token level, inside
// that chunk: the same with 8-token runs and their weights.  Where
// rounding leaves the target at the top, the last token with positive
// weight (of the chunk, or of the row) is taken; -1 when there is no mass
// at all.
__global__ __launch_bounds__(kThreads) void verify_select_kernel(VerifyArgs a) {
    __shared__ double s_pre[kThreads];
    __shared__ double s_wsum[4];
    __shared__ double s_target;
    __shared__ int s_int[4], s_cs, s_tok;
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const Choice ch = load_choice(a);
    const double *sums = chunk_sums(a);

    // ---- chunk level ----
    const int per = (a.chunks + kThreads - 1) / kThreads;
    const int c0 = min(a.chunks, tid * per), c1 = min(a.chunks, c0 + per);
    double run_sum = 0.0;
    int last_pos_chunk = -1;
    for (int c = c0; c < c1; ++c) {
        run_sum += sums[c];
        if (sums[c] > 0.0) last_pos_chunk = c;
    }
    double lo, hi, total;
    block_intervals(run_sum, s_pre, s_wsum, &lo, &hi, &total);
    const double target = a.u_sample * total;
    const bool match = c0 < c1 && lo <= target && target < hi;
    const int first = block_min_i(match ? tid : kThreads, s_int);
    if (tid == 0) {
        s_cs = -1;
        s_target = 0.0;
    }
    __syncthreads();
    if (tid == first) {
        double clo = lo;
        int pick = c1 - 1;
        double pick_lo = clo;
        for (int c = c0; c < c1; ++c) {
            const double chi = c + 1 < a.chunks ? clo + sums[c] : total;
            pick_lo = clo;
            if (clo <= target && target < chi) {
                pick = c;
                break;
            }
            clo = chi;
        }
        s_cs = pick;
        s_target = target - pick_lo;
    }
    __syncthreads();
    int cs = s_cs;
    const bool found = cs >= 0;
    if (!found)  // uniform: the last chunk with mass, for its last positive token
        cs = block_max_i(last_pos_chunk, s_int);

    // ---- token level inside chunk cs ----
    double w[kPer];
    const int x0 = (cs >= 0 ? cs : 0) * kVerifyChunk + tid * kPer;
    if (cs >= 0) {
        lane_weights(a, ch, x0, w);
    } else {
#pragma unroll
        for (int i = 0; i < kPer; ++i) w[i] = 0.0;
    }
    double part = 0.0;
    int last_pos = -1;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        part += w[i];
        if (w[i] > 0.0) last_pos = x0 + i;
    }
    double tlo, thi, ctotal;
    block_intervals(part, s_pre, s_wsum, &tlo, &thi, &ctotal);
    const double ctarget = s_target;
    const bool tmatch = found && cs >= 0 && x0 < a.vocab && tlo <= ctarget && ctarget < thi;
    const int tfirst = block_min_i(tmatch ? tid : kThreads, s_int);
    if (tid == 0) s_tok = -1;
    __syncthreads();
    if (tid == tfirst) {
        double run = tlo;
        int tok = last_pos;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            run += w[i];
            if (run > ctarget) {
                tok = x0 + i;
                break;
            }
        }
        s_tok = tok;
    }
    __syncthreads();
    if (tfirst == kThreads) {  // uniform: no run holds the target
        const int lp = block_max_i(last_pos, s_int);
        if (tid == 0) s_tok = lp;
    }
    __syncthreads();
    if (tid == 0) {
        a.out[0] = ch.k;
        a.out[1] = s_tok;
    }
}

}  // namespace

size_t verify_workspace_doubles(int t, int64_t chunks) {
    // chunk statistics of the 2t + 1 rows, the chosen row's chunk sums, the
    // decision (k, mp, rp, mq, rq)
    return (size_t)(2 * t + 1) * (size_t)chunks * 2 + (size_t)chunks + 8;
}

hipError_t launch_verify(const VerifyArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(verify_stats_kernel, dim3((unsigned)((2 * a.t + 1) * a.chunks)),
                       dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(verify_chunk_kernel, dim3((unsigned)a.chunks), dim3(kThreads), 0,
                       stream, a);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL(verify_select_kernel, dim3(1), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lynx
