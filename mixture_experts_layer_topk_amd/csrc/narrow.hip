// Grouped GEMM1 (+ SwiGLU*w -> E4M3) and GEMM2 (-> BF16) for few rows per
// expert: the decode regime ("MonoMoe kernel — design" §1, phases 3 and 4, at
// up to 8 tokens), where the layer is bound by streaming the touched experts'
// weights from HBM, not by the MFMA rate.
//
// Work unit = (16-row sub-tile of one expert, column chunk):
//   GEMM1  32 I columns: four 16-column MFMA tiles, gate [c, c+16),
//          gate [c+16, c+32), up [c, c+16), up [c+16, c+32);
//   GEMM2  64 H columns: four 16-column tiles.
// The four waves of a workgroup split K into four contiguous ranges and add
// their partial accumulators in LDS, in wave order, at the end of a unit.
//
// The kernel is persistent (two workgroups per CU) and software-pipelined:
// each workgroup takes units blockIdx.x, blockIdx.x + grid, ...; their headers
// (expert, first position, the 16 activation rows and routing weights) are
// fetched into LDS a batch at a time; then the workgroup's (unit, K chunk)
// items flow through a ring of NBUF register buffers.  Every wave loads its
// weight columns straight from global memory into the MFMA B registers (16
// bytes of one weight row per lane, the operand layout of
// v_mfma_scale_f32_16x16x128_f8f6f4) and its activation rows the same way,
// NBUF - 1 items ahead of the MFMAs, so the HBM latency is paid once per batch
// rather than once per dependent step.  A sub-tile's rows past its segment
// repeat its last row and are not stored.
#include "narrow_dev.h"

namespace moe {

template <bool kG1, bool kST>
__global__ __launch_bounds__(kNarrowThreads) void narrow_gemm_kernel(GemmParams p) {
    narrow_gemm<kG1, false, false, kST>(p, blockIdx.x, gridDim.x);
}

template <bool kG1>
static hipError_t launch_narrow(const GemmParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    int cus = 0;
    hipError_t err = device_cus(&cus);
    if (err != hipSuccess) return err;
    const int nch = (kG1 ? p.I : p.H) / NarrowCfg<kG1>::kCols;
    const int64_t units = (int64_t)p.max_subs * nch;
    const int64_t grid = std::min<int64_t>(units, (int64_t)kNarrowBlocksPerCU * cus);
    if (grid <= 0) return record_pair(ev0, ev1, s);
    auto kern = p.w_staged ? narrow_gemm_kernel<kG1, true> : narrow_gemm_kernel<kG1, false>;
    hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kNarrowThreads), 0, s, ev0, ev1, 0, p);
    return hipGetLastError();
}

hipError_t launch_narrow_gemm1(const GemmParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    return launch_narrow<true>(p, s, ev0, ev1);
}
hipError_t launch_narrow_gemm2(const GemmParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    return launch_narrow<false>(p, s, ev0, ev1);
}

// Block-FP8 weights ("MonoMoe kernel — design", fixed-shape paragraph): the same
// units and pipeline with FP8 weight operands and float32 block scales.
template <bool kG1>
__global__ __launch_bounds__(kNarrowThreads) void narrow_w8_gemm_kernel(GemmParams p) {
    narrow_gemm<kG1, false, true>(p, blockIdx.x, gridDim.x);
}

template <bool kG1>
static hipError_t launch_narrow_w8(const GemmParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    int cus = 0;
    hipError_t err = device_cus(&cus);
    if (err != hipSuccess) return err;
    const int nch = (kG1 ? p.I : p.H) / NarrowCfg<kG1, true>::kCols;
    const int64_t units = (int64_t)p.max_subs * nch;
    const int64_t grid = std::min<int64_t>(units, (int64_t)kNarrowBlocksPerCU * cus);
    if (grid <= 0) return record_pair(ev0, ev1, s);
    hipExtLaunchKernelGGL(narrow_w8_gemm_kernel<kG1>, dim3((unsigned)grid), dim3(kNarrowThreads), 0, s, ev0,
                          ev1, 0, p);
    return hipGetLastError();
}

hipError_t launch_narrow_w8_gemm1(const GemmParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    return launch_narrow_w8<true>(p, s, ev0, ev1);
}
hipError_t launch_narrow_w8_gemm2(const GemmParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    return launch_narrow_w8<false>(p, s, ev0, ev1);
}

// GEMM1 -> SwiGLU -> GEMM2 of the narrow kernels in one launch: every
// workgroup runs its GEMM1 units, then its GEMM2 units, whose activation loads
// wait on per-sub-tile ready counters (zeroed by the bucketing stage of the
// call) while their first weight loads are already in flight.  The waits end:
// no workgroup waits before it has finished its own GEMM1 units, and the grid
// is capped at the number of workgroups the GPU holds at once.  A wait longer
// than kNarrowSpinLimit polls sets *p.status and gives up (wrong output, never
// a hang).
template <bool kST>
__global__ __launch_bounds__(kNarrowThreads) void narrow_fused_kernel(GemmParams p) {
    narrow_gemm<true, true, false, kST>(p, blockIdx.x, gridDim.x);
    narrow_gemm<false, true, false, kST>(p, blockIdx.x, gridDim.x);
}

hipError_t launch_narrow_fused(const GemmParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    static DeviceCache occupancy[2];
    int cus = 0, per_cu = 0;
    auto kern = p.w_staged ? narrow_fused_kernel<true> : narrow_fused_kernel<false>;
    hipError_t err = device_cus(&cus);
    if (err == hipSuccess)
        err = per_device(occupancy[p.w_staged ? 1 : 0], [&](int, int* v) {
            return hipOccupancyMaxActiveBlocksPerMultiprocessor(v, kern, kNarrowThreads, 0);
        }, &per_cu);
    if (err != hipSuccess) return err;
    per_cu = std::min(per_cu, kNarrowBlocksPerCU);
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    const int nch = std::max(p.I / NarrowCfg<true>::kCols, p.H / NarrowCfg<false>::kCols);
    const int64_t units = (int64_t)p.max_subs * nch;
    const int64_t grid = std::min<int64_t>(units, (int64_t)per_cu * cus);
    if (grid <= 0) return record_pair(ev0, ev1, s);
    hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kNarrowThreads), 0, s, ev0, ev1, 0, p);
    return hipGetLastError();
}

}  // namespace moe
