// gfx950 speculative verification: the step that closes a Lynx decode round
// (paper Section 4.3): drafts generated on the Anchor-only cache are checked
// against the logits of one forward pass on the full cache; the longest
// accepted prefix is kept and the first divergence is corrected (the notes'
// Eq. (10): accept s_t when u_t < p_t(s_t) / q_t(s_t); Eq. (11): draw the
// correction from max(0, p_k - q_k)); after a fully accepted draft the next
// token is drawn from the target distribution.
//
//   verify_stats_kernel   one workgroup per (row, 8192-token chunk) of the
//                         2T + 1 logit rows (T draft rows q, T + 1 target
//                         rows p): chunk max and sum of exp(l - max) in
//                         binary64;
//   verify_chunk_kernel   one workgroup per chunk of the chosen row: each
//                         merges the statistics and walks the drafts (a few
//                         exponentials), then sums its chunk's weights;
//   verify_select_kernel  one workgroup: the chunk that holds u * total, the
//                         32-token range inside it (wave scan), the token.
// Ratios and sums are binary64, so a decision can only differ from a
// sequential evaluation within ~1e-15 of its threshold.
#include "lynx_internal.h"

namespace lynx {
namespace {

constexpr int kStatThreads = 256;
constexpr int kDecideThreads = 256;
static_assert(kVerifyChunk % kDecideThreads == 0, "lanes split a chunk evenly");

__device__ __forceinline__ double wave_max_d(double x) {
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) x = fmax(x, __shfl_xor(x, d, 64));
    return x;
}

__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) x += __shfl_xor(x, d, 64);
    return x;
}

// Block-wide max / sum of one double per lane (256 lanes = 4 waves).
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

// Row r < T is draft row r; row T + i is target row i.
__device__ __forceinline__ const float *row_ptr(const VerifyArgs &a, int r) {
    return r < a.t ? a.draft + (int64_t)r * a.vocab : a.target + (int64_t)(r - a.t) * a.vocab;
}

__global__ __launch_bounds__(kStatThreads) void verify_stats_kernel(VerifyArgs a) {
    __shared__ double s_red[4];
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int wg = (int)__builtin_amdgcn_workgroup_id_x();
    const int r = wg / a.chunks, c = wg % a.chunks;
    const float *l = row_ptr(a, r);
    const int x0 = c * kVerifyChunk;
    const int x1 = min(a.vocab, x0 + kVerifyChunk);
    double m = -INFINITY;
    for (int x = x0 + tid; x < x1; x += kStatThreads) m = fmax(m, (double)l[x]);
    m = block_max_d(m, s_red);
    double s = 0.0;
    for (int x = x0 + tid; x < x1; x += kStatThreads) s += exp((double)l[x] - m);
    s = block_sum_d(s, s_red);
    if (tid == 0) {
        a.ws[(int64_t)wg * 2] = m;
        a.ws[(int64_t)wg * 2 + 1] = s;
    }
}

// Row statistics (max, sum of exp(l - max)) merged from the chunk partials.
__device__ __forceinline__ void merge_row(const VerifyArgs &a, int r, double &m, double &s) {
    m = -INFINITY;
    for (int c = 0; c < a.chunks; ++c) m = fmax(m, a.ws[((int64_t)r * a.chunks + c) * 2]);
    s = 0.0;
    for (int c = 0; c < a.chunks; ++c) {
        const double mc = a.ws[((int64_t)r * a.chunks + c) * 2];
        s += a.ws[((int64_t)r * a.chunks + c) * 2 + 1] * exp(mc - m);
    }
}

// Smallest / largest value over the block (256 lanes).
__device__ int block_min_i(int x, int *s_int) {
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) x = min(x, __shfl_xor(x, d, 64));
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    __syncthreads();
    if ((tid & 63) == 0) s_int[tid >> 6] = x;
    __syncthreads();
    return min(min(s_int[0], s_int[1]), min(s_int[2], s_int[3]));
}

__device__ int block_max_i(int x, int *s_int) {
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) x = max(x, __shfl_xor(x, d, 64));
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    __syncthreads();
    if ((tid & 63) == 0) s_int[tid >> 6] = x;
    __syncthreads();
    return max(max(s_int[0], s_int[1]), max(s_int[2], s_int[3]));
}

// Accepted prefix k (Eq. 10) and the statistics of the row the next token is
// drawn from: target row k, minus draft row k when k < T (Eq. 11); rp, rq
// are the reciprocals of the row sums.
struct Choice {
    int k;
    double mp, rp, mq, rq;
};

// Block-wide: lane r merges row r, lane t tests draft t, the first rejection
// is a block minimum.  Every lane returns the same choice.
__device__ Choice choose(const VerifyArgs &a, double *s_m, double *s_s, int *s_int) {
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    for (int r = tid; r < 2 * a.t + 1; r += kDecideThreads) {
        double m, sum;
        merge_row(a, r, m, sum);
        s_m[r] = m;
        s_s[r] = sum;
    }
    __syncthreads();
    int rej = a.t;
    for (int t = tid; t < a.t; t += kDecideThreads) {
        const int s = a.tokens[t];
        bool ok = s >= 0 && s < a.vocab;  // not a token: rejected, nothing read
        if (ok) {
            const double p = exp((double)a.target[(int64_t)t * a.vocab + s] - s_m[a.t + t]) /
                             s_s[a.t + t];
            const double q = exp((double)a.draft[(int64_t)t * a.vocab + s] - s_m[t]) / s_s[t];
            ok = a.u_accept[t] < p / q;
        }
        if (!ok) rej = min(rej, t);
    }
    Choice c;
    c.k = block_min_i(rej, s_int);
    c.mp = s_m[a.t + c.k];
    c.rp = 1.0 / s_s[a.t + c.k];
    c.mq = c.k < a.t ? s_m[c.k] : 0.0;
    c.rq = c.k < a.t ? 1.0 / s_s[c.k] : 1.0;
    return c;
}

__device__ __forceinline__ double weight(const VerifyArgs &a, const Choice &c, int x) {
    const double p = exp((double)a.target[(int64_t)c.k * a.vocab + x] - c.mp) * c.rp;
    if (c.k >= a.t)
        return p;
    const double q = exp((double)a.draft[(int64_t)c.k * a.vocab + x] - c.mq) * c.rq;
    return p > q ? p - q : 0.0;
}

// One workgroup per 8192-token chunk of the chosen row: the chunk's weight
// sum into the workspace tail.
__global__ __launch_bounds__(kDecideThreads) void verify_chunk_kernel(VerifyArgs a) {
    __shared__ double s_m[2 * kVerifyMaxDraft + 1], s_s[2 * kVerifyMaxDraft + 1];
    __shared__ double s_red[4];
    __shared__ int s_int[4];
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int c = (int)__builtin_amdgcn_workgroup_id_x();
    const Choice ch = choose(a, s_m, s_s, s_int);
    const int x0 = c * kVerifyChunk, x1 = min(a.vocab, x0 + kVerifyChunk);
    double part = 0.0;
    for (int x = x0 + tid; x < x1; x += kDecideThreads) part += weight(a, ch, x);
    part = block_sum_d(part, s_red);
    if (tid == 0)
        a.ws[(int64_t)(2 * a.t + 1) * a.chunks * 2 + c] = part;
}

// One workgroup: the chunk holding u * total (chunk sums in order), then the
// 32-token lane range inside it (interval j = [prefix_j, prefix_j+1) of one
// computed prefix sequence; the smallest matching lane wins), then the token
// by a sequential rescan.  Where rounding leaves the target at the top, the
// last token with positive weight (of the chunk, or of the row) is taken.
__global__ __launch_bounds__(kDecideThreads) void verify_select_kernel(VerifyArgs a) {
    __shared__ double s_m[2 * kVerifyMaxDraft + 1], s_s[2 * kVerifyMaxDraft + 1];
    __shared__ double s_pre[kDecideThreads];
    __shared__ double s_wsum[4];
    __shared__ double s_target;
    __shared__ int s_found, s_search, s_int[4], s_tok;
    constexpr int kPer = kVerifyChunk / kDecideThreads;  // 32 tokens per lane
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int lane = tid & 63, wave = tid >> 6;
    const double *sums = a.ws + (int64_t)(2 * a.t + 1) * a.chunks * 2;
    const Choice ch = choose(a, s_m, s_s, s_int);
    if (tid == 0) {
        double total = 0.0;
        for (int c = 0; c < a.chunks; ++c) total += sums[c];
        const double target = a.u_sample * total;
        double lo = 0.0;
        int cs = -1, last_pos_chunk = -1;
        s_target = 0.0;
        for (int c = 0; c < a.chunks; ++c) {
            if (sums[c] > 0.0) last_pos_chunk = c;
            const double hi = c + 1 < a.chunks ? lo + sums[c] : total;
            if (cs < 0 && lo <= target && target < hi) {
                cs = c;
                s_target = target - lo;
            }
            lo = hi;
        }
        // No chunk holds the target (rounding at the top, or no mass at
        // all): search the last chunk with mass for its last positive token.
        s_found = cs >= 0 ? 1 : 0;
        s_search = cs >= 0 ? cs : last_pos_chunk;  // -1: no mass anywhere
    }
    __syncthreads();
    const bool found = s_found != 0;
    const int cs = s_search;
    const int x0 = cs >= 0 ? min(a.vocab, cs * kVerifyChunk + tid * kPer) : 0;
    const int x1 = cs >= 0 ? min(a.vocab, min(x0 + kPer, cs * kVerifyChunk + kVerifyChunk)) : 0;
    double part = 0.0;
    int last_pos = -1;
    for (int x = x0; x < x1; ++x) {
        const double w = weight(a, ch, x);
        part += w;
        if (w > 0.0) last_pos = x;
    }
    // exclusive prefix of the lane sums: wave scan, then wave offsets
    double incl = part;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const double y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    double off = 0.0;
    for (int w = 0; w < wave; ++w) off += s_wsum[w];
    const double lo = off + incl - part;
    s_pre[tid] = lo;
    __syncthreads();
    const double hi = tid + 1 < kDecideThreads
                          ? s_pre[tid + 1]
                          : (s_wsum[0] + s_wsum[1]) + (s_wsum[2] + s_wsum[3]);
    const double target = s_target;
    const bool match = found && x0 < x1 && lo <= target && target < hi;
    const int first = block_min_i(match ? tid : kDecideThreads, s_int);
    if (tid == 0) s_tok = -1;
    __syncthreads();
    if (first < kDecideThreads && tid == first) {
        double run = lo;
        int tok = last_pos;
        for (int x = x0; x < x1; ++x) {
            run += weight(a, ch, x);
            if (run > target) {
                tok = x;
                break;
            }
        }
        s_tok = tok;
    }
    __syncthreads();
    if (first == kDecideThreads) {  // uniform: no lane holds the target
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

hipError_t launch_verify(const VerifyArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(verify_stats_kernel, dim3((unsigned)((2 * a.t + 1) * a.chunks)),
                       dim3(kStatThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(verify_chunk_kernel, dim3((unsigned)a.chunks), dim3(kDecideThreads), 0,
                       stream, a);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL(verify_select_kernel, dim3(1), dim3(kDecideThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lynx
