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
//   verify_decide_kernel  one workgroup: merges the chunk statistics, walks
//                         the drafts, then samples by inverse CDF over the
//                         chosen row (per-lane sums of contiguous token
//                         ranges, a block scan, and a rescan of the one range
//                         that holds u * total).
// Ratios and sums are binary64, so a decision can only differ from a
// sequential evaluation within ~1e-15 of its threshold.
#include "lynx_internal.h"

namespace lynx {
namespace {

constexpr int kStatThreads = 256;
constexpr int kDecideThreads = 256;

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

__global__ __launch_bounds__(kDecideThreads) void verify_decide_kernel(VerifyArgs a) {
    __shared__ double s_max[2 * kVerifyMaxDraft + 1], s_sum[2 * kVerifyMaxDraft + 1];
    __shared__ double s_red[4];
    __shared__ double s_part[kDecideThreads];
    __shared__ int s_k, s_tok;
    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int rows = 2 * a.t + 1;

    // Row statistics from the chunk partials.
    for (int r = tid; r < rows; r += kDecideThreads) {
        double m = -INFINITY;
        for (int c = 0; c < a.chunks; ++c) m = fmax(m, a.ws[((int64_t)r * a.chunks + c) * 2]);
        double s = 0.0;
        for (int c = 0; c < a.chunks; ++c) {
            const double mc = a.ws[((int64_t)r * a.chunks + c) * 2];
            s += a.ws[((int64_t)r * a.chunks + c) * 2 + 1] * exp(mc - m);
        }
        s_max[r] = m;
        s_sum[r] = s;
    }
    __syncthreads();

    // Accepted prefix (Eq. 10).
    if (tid == 0) {
        int k = 0;
        for (; k < a.t; ++k) {
            const int s = a.tokens[k];
            if (s < 0 || s >= a.vocab)  // not a token: rejected, nothing read
                break;
            const double p = exp((double)a.target[(int64_t)k * a.vocab + s] - s_max[a.t + k]) /
                             s_sum[a.t + k];
            const double q =
                exp((double)a.draft[(int64_t)k * a.vocab + s] - s_max[k]) / s_sum[k];
            if (!(a.u_accept[k] < p / q))
                break;
        }
        s_k = k;
    }
    __syncthreads();
    const int k = s_k;
    const bool resid = k < a.t;
    const float *lp = a.target + (int64_t)k * a.vocab;
    const float *lq = resid ? a.draft + (int64_t)k * a.vocab : nullptr;
    const double mp = s_max[a.t + k], sp = s_sum[a.t + k];
    const double mq = resid ? s_max[k] : 0.0, sq = resid ? s_sum[k] : 1.0;
    auto weight = [&](int x) {
        const double p = exp((double)lp[x] - mp) / sp;
        if (!resid)
            return p;
        const double q = exp((double)lq[x] - mq) / sq;
        return p > q ? p - q : 0.0;
    };

    // Inverse CDF (Eq. 11): lane j owns tokens [j * per, (j + 1) * per).
    const int per = (a.vocab + kDecideThreads - 1) / kDecideThreads;
    const int x0 = min(a.vocab, tid * per), x1 = min(a.vocab, x0 + per);
    double part = 0.0;
    int last_pos = -1;
    for (int x = x0; x < x1; ++x) {
        const double w = weight(x);
        part += w;
        if (w > 0.0) last_pos = x;
    }
    s_part[tid] = part;
    if (tid == 0) s_tok = -1;
    __syncthreads();
    // Exclusive prefix of the lane sums (serial in lane order: 256 values).
    if (tid == 0) {
        double run = 0.0;
        for (int j = 0; j < kDecideThreads; ++j) {
            const double v = s_part[j];
            s_part[j] = run;
            run += v;
        }
        s_red[0] = run;
    }
    __syncthreads();
    const double total = s_red[0];
    const double target = a.u_sample * total;
    const double lo = s_part[tid];
    if (x0 < x1 && lo <= target && target < lo + part) {
        double run = lo;
        int tok = last_pos;
        for (int x = x0; x < x1; ++x) {
            run += weight(x);
            if (run > target) {
                tok = x;
                break;
            }
        }
        s_tok = tok;  // a single lane matches (ranges are disjoint)
    }
    __syncthreads();
    // Rounding left the target at the very top: the last positive token.
    if (s_tok < 0) {
        const double lp_max = block_max_d(last_pos, s_red);
        if (tid == 0) s_tok = (int)lp_max;
    }
    __syncthreads();
    if (tid == 0) {
        a.out[0] = k;
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
    hipLaunchKernelGGL(verify_decide_kernel, dim3(1), dim3(kDecideThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lynx
