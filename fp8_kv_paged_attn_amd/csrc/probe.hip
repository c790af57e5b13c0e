// probe.hip - streaming HBM read probe.
//
// A plain kernel that reads a buffer once with 16-byte loads, each workgroup a
// contiguous chunk with 16 loads in flight per thread, and keeps nothing: the read bandwidth it reaches on a buffer far
// larger than the Infinity Cache is the practical ceiling against which the
// verify kernel's own bandwidth is read.  A measurement utility: no result of
// the library depends on it.
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kBlocksPerCU = 4;
constexpr int kCUs = 256;
constexpr int kInFlight = 16;             // 16-byte loads in flight per thread

typedef int int4v __attribute__((ext_vector_type(4)));

// Block b reads the contiguous chunk [b * per, min((b + 1) * per, n16)) of
// 16-byte words, kInFlight loads per thread at a time (per is a multiple of
// kThreads * kInFlight).
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const int4v *__restrict__ p,
                                                               int64_t n16, int64_t per,
                                                               uint32_t *__restrict__ sink)
{
    const int64_t begin = (int64_t)blockIdx.x * per;
    const int64_t end = begin + per < n16 ? begin + per : n16;
    int4v x = {0, 0, 0, 0};
    int64_t i = begin + threadIdx.x;
    for (; i + (kInFlight - 1) * kThreads < end; i += kThreads * kInFlight) {
        int4v t[kInFlight];
#pragma unroll
        for (int k = 0; k < kInFlight; ++k)
            t[k] = p[i + k * kThreads];
#pragma unroll
        for (int k = 0; k < kInFlight; ++k)
            x ^= t[k];
    }
    for (; i < end; i += kThreads)
        x ^= p[i];
    // never true for the probe's own buffers (zeros); keeps the loads live
    if ((x.x ^ x.y ^ x.z ^ x.w) == 0x5EED5EED)
        sink[0] = 1u;
}

}  // namespace

hipError_t launch_stream_read(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t stream)
{
    if (bytes == 0)
        return hipSuccess;
    const int64_t n16 = bytes / 16;
    const int blocks = kCUs * kBlocksPerCU;
    const int64_t unit = (int64_t)kThreads * kInFlight;
    const int64_t per = ((n16 + blocks - 1) / blocks + unit - 1) / unit * unit;
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                       static_cast<const int4v *>(buf), n16, per, sink);
    return hipGetLastError();
}

}  // namespace pa
