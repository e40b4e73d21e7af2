// Streaming-ceiling probe: a stand-alone program (not part of liblynx.so)
// that times plain HBM streams on the GPU it runs on, so that a kernel's
// fraction of the 8 TB/s peak can be read against what a simple stream of
// the same read / write mix reaches on the same box.
//
// Pattern R : W = each lane reads R and writes W 16-byte words per step
// (four at a time for the read-only and write-only streams), in
// R (W) planes of M words; grid-stride over i < M, indices k * M + i with
// k < R (reads) or k < W (writes), inside buffers of max(R, W) * M words.
// M is chosen so that each direction moves at most 4 GiB, far above the
// 256 MB last-level cache.  Output: one JSON object per line.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define CK(x)                                                                               \
    do {                                                                                    \
        hipError_t e_ = (x);                                                                \
        if (e_ != hipSuccess) {                                                             \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                         \
            exit(1);                                                                        \
        }                                                                                   \
    } while (0)

template <int R, int W, bool NT>
__global__ __launch_bounds__(256) void stream_kernel(const u32x4 *__restrict__ a,
                                                     u32x4 *__restrict__ b, size_t m) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < m; i += stride) {
        u32x4 r[R > 0 ? R : 1];
#pragma unroll
        for (int k = 0; k < R; ++k) r[k] = a[(size_t)k * m + i];
        if constexpr (R == 0) {
            r[0] = u32x4{(unsigned)i, 1u, 2u, 3u};
        }
#pragma unroll
        for (int k = 0; k < W; ++k) {
            const u32x4 v = R > 1 ? r[k % R] ^ r[(k + 1) % R] : r[0];
            if (NT)
                __builtin_nontemporal_store(v, b + (size_t)k * m + i);
            else
                b[(size_t)k * m + i] = v;
        }
        // read-only: a store that never happens (the buffers hold 0x01
        // bytes) keeps every load alive
        if constexpr (W == 0) {
            u32x4 x = r[0];
#pragma unroll
            for (int k = 1; k < R; ++k) x ^= r[k];
            if (x.x == 0x12345678u)
                b[i] = x;
        }
    }
}

constexpr size_t kDirBytes = size_t(1) << 32;  // at most 4 GiB per direction

template <int R, int W, bool NT>
void run(const char *name, const u32x4 *a, u32x4 *b, int reps) {
    const int planes = R > W ? R : W;
    const size_t m = kDirBytes / 16 / planes;
    const double bytes = (double)(R + W) * m * 16;
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));
    double best = 0.0;
    int best_grid = 0;
    for (int grid : {1024, 2048, 4096, 8192, 16384, 32768}) {
        stream_kernel<R, W, NT><<<grid, 256>>>(a, b, m);
        CK(hipGetLastError());
        CK(hipDeviceSynchronize());
        CK(hipEventRecord(e0));
        for (int r = 0; r < reps; ++r)
            stream_kernel<R, W, NT><<<grid, 256>>>(a, b, m);
        CK(hipEventRecord(e1));
        CK(hipEventSynchronize(e1));
        float ms = 0.0f;
        CK(hipEventElapsedTime(&ms, e0, e1));
        const double gbps = bytes / (ms / reps * 1e-3) / 1e9;
        if (gbps > best) {
            best = gbps;
            best_grid = grid;
        }
    }
    printf("{\"pattern\": \"%s\", \"reads\": %d, \"writes\": %d, \"bytes_per_launch\": %.0f, "
           "\"best_GBps\": %.1f, \"of_8TBps\": %.4f, \"grid\": %d, \"threads\": 256}\n",
           name, R, W, bytes, best, best / 8000.0, best_grid);
    fflush(stdout);
    CK(hipEventDestroy(e0));
    CK(hipEventDestroy(e1));
}

}  // namespace

int main() {
    u32x4 *a = nullptr, *b = nullptr;
    CK(hipMalloc(&a, kDirBytes));
    CK(hipMalloc(&b, kDirBytes));
    CK(hipMemset(a, 1, kDirBytes));
    CK(hipMemset(b, 0, kDirBytes));
    const int reps = 10;
    run<4, 0, false>("read only", a, b, reps);
    run<0, 4, false>("write only", a, b, reps);
    run<0, 4, true>("write only, nontemporal", a, b, reps);
    run<1, 1, false>("copy (read 1 : write 1)", a, b, reps);
    run<5, 3, false>("read 5 : write 3 (62.5% reads)", a, b, reps);
    run<2, 1, false>("read 2 : write 1", a, b, reps);
    run<1, 2, false>("read 1 : write 2", a, b, reps);
    CK(hipFree(a));
    CK(hipFree(b));
    return 0;
}
