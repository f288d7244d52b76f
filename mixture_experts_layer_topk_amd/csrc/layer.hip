// The whole layer in one launch for few routed pairs (T * k <= kSmallPairs,
// the decode regime): routing, bucketing and x quantisation, the narrow
// GEMM1 with its SwiGLU epilogue, the narrow GEMM2 and the combine run as
// phases of one persistent kernel ("MonoMoe kernel — design" §1, phases 1-5 in
// one launch) instead of four launches ordered by the stream.  Each phase
// hands its output to the next by arrival counts ("MegaMoE：把通信和计算融合到一个
// Mega Kernel", arrival-count polling), not by grid-wide barriers:
//   routing -> GEMM1   workgroup 0 (the tables) and every workgroup that
//                      quantised rows of x count themselves in once their
//                      stores have completed; GEMM1 starts when all have;
//   GEMM1 -> GEMM2     per 16-row sub-tile: a GEMM2 unit waits until ready[]
//                      counts every GEMM1 unit of its rows (the narrow
//                      one-launch hand-off);
//   GEMM2 -> combine   every workgroup with GEMM2 units counts itself in once
//                      its o rows are stored; the combine starts when all have.
// Only workgroups that stored something count in (one device-scope atomic each
// on one counter; the waits are polls).
// Workgroups on different XCDs do not share an L2, and the caches are not
// coherent with one another within a launch.  Data handed over is therefore
// stored device-coherently (write-through), and stores are complete
// (vmcnt(0)) before the count that publishes them.  A waiting workgroup ends
// its wait with a device-scope acquire (its XCD's stale lines invalidated), so
// no release fence (a write-back of a whole L2) is needed.  Every workgroup
// of the launch is resident at once (a cooperative launch refuses a grid that
// does not fit), and no phase waits for a later one, so every wait ends; one
// that has not after kLayerSpinLimit polls sets *status to 2 and goes on
// (wrong output, never a hang).  The counts grow during the launch and the
// last workgroup to leave resets them.
//
// Measured at the decode shape (T = 8, E = 256, k = 8) on one MI355X: 84 us
// per call against 44 us for the four launches (with grid barriers and their
// release fences it took 120-170 us).  Per-workgroup timestamps: routing 8
// tokens in workgroup 0 takes about 8 us; GEMM1 runs 22 us, GEMM2 14 us; the
// wait for the slowest GEMM2 workgroup another 11 us.  It is therefore opt-in.
#include <hip/hip_runtime.h>

#include "combine_dev.h"
#include "narrow_dev.h"
#include "route_dev.h"

namespace moe {

constexpr int kLayerThreads = 256;
static_assert(kLayerThreads == kRouteThreads && kLayerThreads == kNarrowThreads,
              "the phases share the workgroup shape");
constexpr int kLayerSpinLimit = 1 << 22;

// This workgroup's stores (device-coherent) have completed; thread 0 counts it in.
MOE_DEV void arrive(unsigned* count) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 polls *count until it reaches target (bounded), then acquires at
// device scope; the barrier holds the other threads until then.
MOE_DEV void await_count(unsigned* count, unsigned target, int* status) {
    if (threadIdx.x == 0) {
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
    if (bid == 0) bucket_small<kLayerThreads, true>(rp, sp, lp.npl);
    if (rp.x && (bid > 0 || G == 1))
        quant_rows<kLayerThreads, true>(rp, G > 1 ? bid - 1 : 0, G > 1 ? G - 1 : 1);
    // only the workgroups that stored something count in (one atomic each on one
    // counter): workgroup 0 and the quantising workgroups that had rows
    const int64_t qtasks = rp.x ? rp.T * (rp.H / 8) : 0;
    const int qblocks = G > 1 ? (int)min<int64_t>(G - 1, (qtasks + kLayerThreads - 1) / kLayerThreads) : 0;
    if (bid <= qblocks) arrive(lp.count);
    await_count(lp.count, (unsigned)(1 + qblocks), lp.status);
    // phases 2 and 3: GEMM1 -> GEMM2 through the per-sub-tile ready counts
    narrow_gemm<true, true, false, kST>(gp, bid, G);
    narrow_gemm<false, true, false, kST>(gp, bid, G);
    // phase 4: the combine, once every workgroup with GEMM2 units has stored its
    // rows (workgroup b has units b, b + G, ...: the first min(G, units) have any)
    const int nsub = __hip_atomic_load(const_cast<int32_t*>(gp.nsub), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int units2 = nsub * (gp.H / NarrowCfg<false>::kCols);
    if (bid < units2) arrive(lp.count2);
    await_count(lp.count2, (unsigned)min(G, units2), lp.status);
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
    // every workgroup is past its last wait: the last one to leave resets the
    // counts for the next launch
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(lp.exits, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == (unsigned)G - 1) {
            __hip_atomic_store(lp.count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(lp.count2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    // one workgroup per CU: thread 0 of every workgroup polls the hand-off counts,
    // and at two per CU (the narrow launches' grid) the 512 pollers slowed the
    // counting they wait for (decode: 116 us per call against 84 us)
    const unsigned grid = (unsigned)cus;
    RouteParams a = rp;
    ScatterParams b = sp;
    GemmParams c = gp;
    void* args[] = {&a, &b, &c, &lp};
    return hipLaunchCooperativeKernel(kern, dim3(grid), dim3(kLayerThreads), args, 0, s);
}

}  // namespace moe
