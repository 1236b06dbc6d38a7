// kda_device_copy: the streaming-bandwidth reference of the library's HBM-bound
// kernels.  A plain device-to-device copy in which every lane moves four
// independent 16-byte pieces per iteration with non-temporal loads and stores
// (the cache hint for data touched once), so that a wave keeps 4 KiB of reads
// in flight before it writes.  Timing it gives the bandwidth a streaming kernel
// reaches on the device, and its byte counters calibrate the profiler's
// FETCH_SIZE and WRITE_SIZE readings.
#include "kda_internal.h"

namespace kda {
namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
constexpr int COPY_THREADS = 256, COPY_UNROLL = 4;
constexpr int64_t COPY_SPAN = (int64_t)COPY_THREADS * COPY_UNROLL;  // 16-byte pieces per block step

__global__ void __launch_bounds__(COPY_THREADS)
copy16_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * COPY_SPAN;
    int64_t base = (int64_t)blockIdx.x * COPY_SPAN + threadIdx.x;
    // whole block steps: four loads in flight, then four stores
    for (; base + (COPY_UNROLL - 1) * COPY_THREADS < n16; base += stride) {
        u32x4_t x[COPY_UNROLL];
#pragma unroll
        for (int u = 0; u < COPY_UNROLL; ++u)
            x[u] = __builtin_nontemporal_load(src + base + u * COPY_THREADS);
#pragma unroll
        for (int u = 0; u < COPY_UNROLL; ++u)
            __builtin_nontemporal_store(x[u], dst + base + u * COPY_THREADS);
    }
    // the ragged end (fewer than COPY_SPAN pieces left for this block step)
    for (int u = 0; u < COPY_UNROLL; ++u) {
        const int64_t i = base + u * COPY_THREADS;
        if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
    }
}

}  // namespace

hipError_t launch_device_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
    const int64_t n16 = (int64_t)(bytes / 16);
    if (n16 == 0) return hipSuccess;
    // 32 blocks per CU on a 256-CU device: enough waves to cover HBM latency,
    // few enough that each block streams several consecutive steps
    const int64_t want = (n16 + COPY_SPAN - 1) / COPY_SPAN;
    const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
    hipLaunchKernelGGL(copy16_kernel, dim3(grid), dim3(COPY_THREADS), 0, stream,
                       static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), n16);
    return hipGetLastError();
}

}  // namespace kda
