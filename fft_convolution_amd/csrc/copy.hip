// copy.hip -- a streaming device-to-device copy, the measured ceiling of a
// kernel that reads every byte once and writes it once (the row FFT of a
// batch moves exactly that: one read and one write of each row).  It takes
// no part in any transform; the benchmark times it beside the FFT so that a
// transform's rate can be set against what the memory system delivers to
// this access pattern, not only against the 8 TB/s datasheet peak.
#include "launch.hpp"

namespace fftmi {

typedef float copy_v4 __attribute__((ext_vector_type(4)));

// Each workgroup copies one block of kCopyThreads x kCopyPerLane 16-byte
// vectors: every lane issues all its loads, then all its stores, lanes
// side by side (a 1 KiB run per wave per step), nontemporal both ways, as
// the row kernels stream their rows.
constexpr int kCopyThreads = 256;
constexpr int kCopyPerLane = 8;

__global__ __launch_bounds__(kCopyThreads)
void stream_copy_kernel(const copy_v4* __restrict__ src, copy_v4* __restrict__ dst, int64_t nvec)
{
    const int64_t base = (int64_t)blockIdx.x * (kCopyThreads * kCopyPerLane) + threadIdx.x;
    copy_v4 r[kCopyPerLane];
#pragma unroll
    for (int i = 0; i < kCopyPerLane; ++i) {
        const int64_t k = base + (int64_t)i * kCopyThreads;
        r[i] = k < nvec ? __builtin_nontemporal_load(src + k) : copy_v4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < kCopyPerLane; ++i) {
        const int64_t k = base + (int64_t)i * kCopyThreads;
        if (k < nvec) __builtin_nontemporal_store(r[i], dst + k);
    }
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t nvec, hipStream_t stream)
{
    constexpr int64_t per_block = (int64_t)kCopyThreads * kCopyPerLane;
    const int64_t blocks = (nvec + per_block - 1) / per_block;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, stream,
                       (const copy_v4*)src, (copy_v4*)dst, nvec);
    return hipGetLastError();
}

}  // namespace fftmi
