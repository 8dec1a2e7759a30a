// Measurement helpers, not operations of the method.
// Plain device copy with the data kernels' memory policy, the copy ceiling
// that the dispatch and combine bandwidths are compared with: one 16-byte
// non-temporal load and one non-temporal store per lane, every wave storing
// one 1 KB piece and exiting (the store shape of the row copy), issued over
// ranges within 32-bit work-item ids.
// The empty kernel: one wave that does nothing, whose launches measure the
// floor under the latency-bound kernels (layout, plan).
#include "cgd_device.h"
#include "cgd_launch.h"

namespace cgd {

constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                           int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x;
    if (i < n) store_nt(dst + i, load_nt(src + i));
}

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
    const int64_t n = bytes / 16;
    const int64_t per = kMaxGridWaves * kWave;  // vectors per launch
    for (int64_t i0 = 0; i0 < n; i0 += per) {
        const int64_t m = n - i0 < per ? n - i0 : per;
        hipLaunchKernelGGL(copy_kernel, dim3((unsigned)((m + kCopyThreads - 1) / kCopyThreads)), dim3(kCopyThreads), 0,
                           stream, reinterpret_cast<const uint4*>(src) + i0, reinterpret_cast<uint4*>(dst) + i0, m);
    }
    return hipGetLastError();
}

__global__ __launch_bounds__(kWave) void empty_kernel() {}

hipError_t preload_copy() {
    hipFuncAttributes a;
    return hipFuncGetAttributes(&a, reinterpret_cast<const void*>(&empty_kernel));
}

hipError_t launch_empty(hipStream_t stream) {
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(kWave), 0, stream);
    return hipGetLastError();
}

}  // namespace cgd
