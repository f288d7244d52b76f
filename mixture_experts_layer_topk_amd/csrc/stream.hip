// Read-only streaming of a byte range: the HBM read ceiling of a footprint.
// A weight-streaming GEMM at the decode shape must read its touched experts'
// weights once; this kernel reads the same number of bytes and does nothing
// else, so its time is what the memory system allows for that footprint
// (start-up and tail included), the yardstick for the GEMM's bandwidth.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kStreamThreads = 256;
constexpr int kStreamPer = 16;          // 16-byte loads per thread, all in flight: 64 KiB per workgroup

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const v4i* __restrict__ src,
                                                                     size_t n16, uint32_t* sink) {
    const size_t base = (size_t)blockIdx.x * (kStreamThreads * kStreamPer) + threadIdx.x;
    v4i v[kStreamPer];
#pragma unroll
    for (int i = 0; i < kStreamPer; ++i) {
        const size_t k = base + (size_t)i * kStreamThreads;
        v[i] = k < n16 ? __builtin_nontemporal_load(src + k) : v4i{0, 0, 0, 0};
    }
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < kStreamPer; ++i) x ^= (uint32_t)(v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3]);
    // the loads feed x; a store taken only on one value keeps them live
    if (x == 0x9E3779B9u) atomicOr(sink, 1u);
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s, hipEvent_t ev0,
                              hipEvent_t ev1) {
    const size_t n16 = bytes / 16;
    const size_t per = (size_t)kStreamThreads * kStreamPer;
    const size_t blocks = (n16 + per - 1) / per;
    if (blocks == 0) return record_pair(ev0, ev1, s);
    if (blocks > 0x7FFFFFFFu) return hipErrorInvalidValue;
    hipExtLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kStreamThreads), 0, s, ev0, ev1,
                          0, static_cast<const v4i*>(src), n16, sink);
    return hipGetLastError();
}

}  // namespace moe
