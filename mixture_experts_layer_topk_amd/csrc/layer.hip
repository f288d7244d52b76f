// The whole layer in one launch for few routed pairs (T * k <= kSmallPairs,
// the decode regime): routing, bucketing and x quantisation, the narrow
// GEMM1 with its SwiGLU epilogue, the narrow GEMM2 and the combine run as four
// phases of one persistent kernel, separated by grid-wide barriers ("MonoMoe
// kernel — design" §1, phases 1-5 in one launch), instead of four launches
// ordered by the stream.
//
// Grid barriers.  Every workgroup of the launch is resident at once (a
// cooperative launch refuses a grid that does not fit).  Workgroups on
// different XCDs do not share an L2, and those caches are not kept coherent
// with one another within a launch, so a workgroup arriving at a barrier first
// waits for its own stores, then writes back its XCD's dirty L2 lines (a
// device-scope release) before it counts itself in; after the count is
// complete it invalidates its cached lines (a device-scope acquire), so its
// later loads see what every other workgroup stored.  The counter grows by G
// per barrier and is reset by the last workgroup to leave the kernel.  A wait
// that has not ended after kLayerSpinLimit polls sets *status to 2 and goes on
// (wrong output, never a hang).
//
// Measured on one MI355X at the decode shape (T = 8, E = 256, k = 8), this
// launch takes about 0.12 ms against 0.066 ms for the four launches: the
// device-scope release at each barrier (write-back of the XCD's L2) costs
// about 30 us over the three barriers, and even without the fences the
// phases run slower in one kernel than as separate launches, whose
// boundaries the hardware orders more cheaply.  It is therefore opt-in.
#include <hip/hip_runtime.h>

#include "combine_dev.h"
#include "narrow_dev.h"
#include "route_dev.h"

namespace moe {

constexpr int kLayerThreads = 256;
static_assert(kLayerThreads == kRouteThreads && kLayerThreads == kNarrowThreads,
              "the phases share the workgroup shape");
constexpr int kLayerSpinLimit = 1 << 22;

MOE_DEV void grid_barrier(unsigned* count, unsigned target, int* status) {
    __builtin_amdgcn_s_waitcnt(0);                  // this thread's stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int n = 0;
        while (__hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            __builtin_amdgcn_s_sleep(16);      // ~1000 cycles between polls
            if (++n > kLayerSpinLimit) {
                __hip_atomic_store(status, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
}

template <int KS>
MOE_DEV void combine_phase(const GemmParams& gp, const int32_t* slot_of, uint16_t* y, int bid, int G) {
    const int cpr = gp.H / 8;
    const int64_t tasks = gp.T * cpr;
    for (int64_t i = (int64_t)bid * kLayerThreads + threadIdx.x; i < tasks;
         i += (int64_t)G * kLayerThreads) {
        const int64_t t = i / cpr;
        combine_chunk<KS>(gp.o, slot_of, t, (int)(i - t * cpr) * 8, gp.H, y);
    }
}

template <bool kST>
__global__ __launch_bounds__(kLayerThreads) void layer_small_kernel(RouteParams rp, ScatterParams sp,
                                                                    GemmParams gp, LayerParams lp) {
    const int G = gridDim.x, bid = blockIdx.x;
    // phase 1: workgroup 0 routes and buckets, the others quantise x
    if (bid == 0) bucket_small<kLayerThreads>(rp, sp, lp.npl);
    if (rp.x && (bid > 0 || G == 1)) quant_rows<kLayerThreads>(rp, G > 1 ? bid - 1 : 0, G > 1 ? G - 1 : 1);
    grid_barrier(lp.count, (unsigned)G, lp.status);
    narrow_gemm<true, false, false, kST>(gp, bid, G);
    grid_barrier(lp.count, 2u * G, lp.status);
    narrow_gemm<false, false, false, kST>(gp, bid, G);
    grid_barrier(lp.count, 3u * G, lp.status);
    switch (gp.topk) {   // 1 <= topk <= 16
        case 1: combine_phase<1>(gp, sp.slot_of, lp.y, bid, G); break;
        case 2: combine_phase<2>(gp, sp.slot_of, lp.y, bid, G); break;
        case 3: combine_phase<3>(gp, sp.slot_of, lp.y, bid, G); break;
        case 4: combine_phase<4>(gp, sp.slot_of, lp.y, bid, G); break;
        case 5: combine_phase<5>(gp, sp.slot_of, lp.y, bid, G); break;
        case 6: combine_phase<6>(gp, sp.slot_of, lp.y, bid, G); break;
        case 7: combine_phase<7>(gp, sp.slot_of, lp.y, bid, G); break;
        case 8: combine_phase<8>(gp, sp.slot_of, lp.y, bid, G); break;
        case 9: combine_phase<9>(gp, sp.slot_of, lp.y, bid, G); break;
        case 10: combine_phase<10>(gp, sp.slot_of, lp.y, bid, G); break;
        case 11: combine_phase<11>(gp, sp.slot_of, lp.y, bid, G); break;
        case 12: combine_phase<12>(gp, sp.slot_of, lp.y, bid, G); break;
        case 13: combine_phase<13>(gp, sp.slot_of, lp.y, bid, G); break;
        case 14: combine_phase<14>(gp, sp.slot_of, lp.y, bid, G); break;
        case 15: combine_phase<15>(gp, sp.slot_of, lp.y, bid, G); break;
        default: combine_phase<16>(gp, sp.slot_of, lp.y, bid, G); break;
    }
    // every workgroup has passed the last barrier: the last one to leave resets
    // the counters for the next launch
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(lp.exits, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == (unsigned)G - 1) {
            __hip_atomic_store(lp.count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(lp.exits, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

bool layer_small_fits(int64_t T, int topk) { return T > 0 && T * topk <= kSmallPairs; }

hipError_t launch_layer_small(const RouteParams& rp, const ScatterParams& sp, const GemmParams& gp,
                              LayerParams lp, hipStream_t s) {
    static DeviceCache occupancy[2];
    int cus = 0, per_cu = 0;
    const void* kern = gp.w_staged ? (const void*)layer_small_kernel<true> : (const void*)layer_small_kernel<false>;
    hipError_t err = device_cus(&cus);
    if (err == hipSuccess)
        err = per_device(occupancy[gp.w_staged ? 1 : 0], [&](int, int* v) {
            return hipOccupancyMaxActiveBlocksPerMultiprocessor(v, kern, kLayerThreads, 0);
        }, &per_cu);
    if (err != hipSuccess) return err;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    lp.npl = rp.logits ? (rp.E + 63) / 64 : 1;
    // two workgroups per CU, as the narrow GEMM launches use
    const unsigned grid = (unsigned)(std::min(per_cu, kNarrowBlocksPerCU) * cus);
    RouteParams a = rp;
    ScatterParams b = sp;
    GemmParams c = gp;
    void* args[] = {&a, &b, &c, &lp};
    return hipLaunchCooperativeKernel(kern, dim3(grid), dim3(kLayerThreads), args, 0, s);
}

}  // namespace moe
