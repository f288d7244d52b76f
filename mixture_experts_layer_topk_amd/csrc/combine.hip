// Combine: y[t] = BF16(sum over j = 0..k-1 of the float32 values of token t's
// GEMM2 row for slot j), added in slot order ("MegaMoE" notes, "L2 epilogue":
// the source accumulates the top-k BF16 copies in FP32 before storing y;
// "Warp Specialization: DeepEP vs Mega MoE", combine excerpt).  Skipped slots
// add nothing.  Gathering by slot position keeps the sum deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kCombineThreads = 256;
constexpr int kMaxSlots = 16;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const uint16_t* __restrict__ o,
                                                                  const int32_t* __restrict__ slot_of,
                                                                  int64_t tasks, int topk, int H,
                                                                  uint16_t* __restrict__ y) {
    const int cpr = H / 8;   // 8-column chunks per row
    for (int64_t i = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x; i < tasks;
         i += (int64_t)gridDim.x * kCombineThreads) {
        int64_t t = i / cpr;
        int c = (int)(i - t * cpr) * 8;
        // all of the token's slot rows are fetched before any is added
        int pos[kMaxSlots];
#pragma unroll
        for (int j = 0; j < kMaxSlots; ++j) pos[j] = j < topk ? slot_of[t * topk + j] : -1;
        uint4 raw[kMaxSlots];
#pragma unroll
        for (int j = 0; j < kMaxSlots; ++j)
            raw[j] = pos[j] >= 0 ? *reinterpret_cast<const uint4*>(o + (int64_t)pos[j] * H + c)
                                 : make_uint4(0, 0, 0, 0);
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < kMaxSlots; ++j) {
            if (pos[j] < 0) continue;
            acc[0] += bf16_to_f32(raw[j].x & 0xFFFFu); acc[1] += bf16_to_f32(raw[j].x >> 16);
            acc[2] += bf16_to_f32(raw[j].y & 0xFFFFu); acc[3] += bf16_to_f32(raw[j].y >> 16);
            acc[4] += bf16_to_f32(raw[j].z & 0xFFFFu); acc[5] += bf16_to_f32(raw[j].z >> 16);
            acc[6] += bf16_to_f32(raw[j].w & 0xFFFFu); acc[7] += bf16_to_f32(raw[j].w >> 16);
        }
        uint4 out;
        out.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
        out.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
        out.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
        out.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
        *reinterpret_cast<uint4*>(y + t * H + c) = out;
    }
}

hipError_t launch_combine(const uint16_t* o, const int32_t* slot_of, int64_t T, int topk, int H,
                          uint16_t* y, hipStream_t s) {
    int64_t tasks = T * (H / 8);
    if (tasks == 0) return hipSuccess;
    int64_t blocks = std::min<int64_t>((tasks + kCombineThreads - 1) / kCombineThreads, 8192);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(kCombineThreads), 0, s, o,
                       slot_of, tasks, topk, H, y);
    return hipGetLastError();
}

}  // namespace moe
