// Device helpers shared by the gfx950 kernels of liblynx.so (device
// translation units only).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace lynx {

// Workgroup u of a launch of n workgroups, reordered so that the hardware's
// round-robin deal of workgroups to the 8 XCDs (u % 8) gives XCD x the
// contiguous run [x q + min(x, r), ...) (q = n / 8, r = n % 8): the
// workgroups of one XCD work on neighbouring rows.  A bijection of [0, n).
__device__ __forceinline__ int64_t xcd_unit(int64_t u, int64_t n) {
    const int64_t q = n >> 3, r = n & 7, x = u & 7, i = u >> 3;
    return x * q + (x < r ? x : r) + i;
}

}  // namespace lynx
