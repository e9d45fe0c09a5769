// copy.hip -- a streaming device-to-device copy, the measured ceiling of a
// kernel that reads every byte once and writes it once (the row FFT of a
// batch moves exactly that: one read and one write of each row).  It takes
// no part in any transform; the benchmark times it beside the FFT so that a
// transform's rate can be set against what the memory system delivers to
// this access pattern, not only against the 8 TB/s datasheet peak.
#include "launch.hpp"

namespace fftmi {

typedef float copy_v2 __attribute__((ext_vector_type(2)));

// Each workgroup copies one block of kCopyThreads x kCopyPerLane 8-byte
// elements: every lane issues all its loads, then all its stores, lanes side
// by side, nontemporal both ways -- the access pattern of the row kernels
// (256 threads, 16 complex64 elements each).  Measured on MI355X over 512 MiB
// each way: 6.42 TB/s, against 6.31 TB/s for 16-byte lanes (4 or 8 per lane)
// and 5.2 TB/s for 16 16-byte vectors per lane.  Only the last block, if
// partial, checks bounds: a bounds check on every access splits the loads
// into separately waited groups (4.5 TB/s).
constexpr int kCopyThreads = 256;
constexpr int kCopyPerLane = 16;

__global__ __launch_bounds__(kCopyThreads)
void stream_copy_kernel(const copy_v2* __restrict__ src, copy_v2* __restrict__ dst, int64_t nvec)
{
    constexpr int64_t kBlock = (int64_t)kCopyThreads * kCopyPerLane;
    const int64_t b0 = (int64_t)blockIdx.x * kBlock;
    const int64_t base = b0 + threadIdx.x;
    if (b0 + kBlock <= nvec) {
        copy_v2 r[kCopyPerLane];
#pragma unroll
        for (int i = 0; i < kCopyPerLane; ++i) r[i] = __builtin_nontemporal_load(src + base + i * kCopyThreads);
#pragma unroll
        for (int i = 0; i < kCopyPerLane; ++i) __builtin_nontemporal_store(r[i], dst + base + i * kCopyThreads);
    } else {
        for (int i = 0; i < kCopyPerLane; ++i) {
            const int64_t k = base + (int64_t)i * kCopyThreads;
            if (k < nvec) dst[k] = src[k];
        }
    }
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t nvec, hipStream_t stream)
{
    constexpr int64_t per_block = (int64_t)kCopyThreads * kCopyPerLane;
    const int64_t blocks = (nvec + per_block - 1) / per_block;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, stream,
                       (const copy_v2*)src, (copy_v2*)dst, nvec);
    return hipGetLastError();
}

}  // namespace fftmi
