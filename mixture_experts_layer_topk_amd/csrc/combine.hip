// Combine: y[t] = BF16(sum over j = 0..k-1 of the float32 values of token t's
// GEMM2 row for slot j), added in slot order ("MegaMoE" notes, "L2 epilogue":
// the source accumulates the top-k BF16 copies in FP32 before storing y;
// "Warp Specialization: DeepEP vs Mega MoE", combine excerpt).  Skipped slots
// add nothing.  Gathering by slot position keeps the sum deterministic.
#include "combine_dev.h"
#include "kernels.h"

namespace moe {

// One thread per 8 columns of one token; KS = top-k slots (a template
// argument, so that the slot loads are unrolled without predication).
template <int KS>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const uint16_t* __restrict__ o,
                                                                  const int32_t* __restrict__ slot_of,
                                                                  int64_t tasks, int H,
                                                                  uint16_t* __restrict__ y) {
    const int cpr = H / 8;   // 8-column chunks per row
    const int64_t i = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x;
    if (i >= tasks) return;
    const int64_t t = i / cpr;
    combine_chunk<KS>(o, slot_of, t, (int)(i - t * cpr) * 8, H, y);
}

template <int KS>
static void launch_ks(const uint16_t* o, const int32_t* slot_of, int64_t tasks, int H, uint16_t* y,
                      hipStream_t s) {
    const int64_t blocks = (tasks + kCombineThreads - 1) / kCombineThreads;
    hipLaunchKernelGGL(combine_kernel<KS>, dim3((unsigned)blocks), dim3(kCombineThreads), 0, s, o,
                       slot_of, tasks, H, y);
}

hipError_t launch_combine(const uint16_t* o, const int32_t* slot_of, int64_t T, int topk, int H,
                          uint16_t* y, hipStream_t s) {
    const int64_t tasks = T * (H / 8);
    if (tasks == 0) return hipSuccess;
    switch (topk) {
        case 1: launch_ks<1>(o, slot_of, tasks, H, y, s); break;
        case 2: launch_ks<2>(o, slot_of, tasks, H, y, s); break;
        case 3: launch_ks<3>(o, slot_of, tasks, H, y, s); break;
        case 4: launch_ks<4>(o, slot_of, tasks, H, y, s); break;
        case 5: launch_ks<5>(o, slot_of, tasks, H, y, s); break;
        case 6: launch_ks<6>(o, slot_of, tasks, H, y, s); break;
        case 7: launch_ks<7>(o, slot_of, tasks, H, y, s); break;
        case 8: launch_ks<8>(o, slot_of, tasks, H, y, s); break;
        case 9: launch_ks<9>(o, slot_of, tasks, H, y, s); break;
        case 10: launch_ks<10>(o, slot_of, tasks, H, y, s); break;
        case 11: launch_ks<11>(o, slot_of, tasks, H, y, s); break;
        case 12: launch_ks<12>(o, slot_of, tasks, H, y, s); break;
        case 13: launch_ks<13>(o, slot_of, tasks, H, y, s); break;
        case 14: launch_ks<14>(o, slot_of, tasks, H, y, s); break;
        case 15: launch_ks<15>(o, slot_of, tasks, H, y, s); break;
        default: launch_ks<16>(o, slot_of, tasks, H, y, s); break;
    }
    return hipGetLastError();
}

}  // namespace moe
