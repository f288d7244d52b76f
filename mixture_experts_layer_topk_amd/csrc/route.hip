// Routing, counting-sort bucketisation and activation quantisation.
//
// Launch A (route_count_quant): each workgroup takes a chunk of tokens and
//   1. routes them: top-k of the float32 logits (softmax and sigmoid are
//      increasing, so the k best scores are the k largest logits), weights from
//      softmax or sigmoid, optionally renormalised ("MonoMoe kernel — design"
//      §1, phase 1); or reads a caller's top-k ids and weights;
//   2. counts its (token, slot) pairs per expert in an LDS histogram, the LDS
//      atomic returning each pair's rank inside the workgroup, then adds the
//      histogram to the global per-expert counters with one atomic per expert,
//      whose return value is this workgroup's base inside the expert
//      ("05.10 Counting Sort / Bucketization" 2.1 COUNT, 2.2 PREFIX SUM); the
//      pair's slot inside its expert is base + rank;
//   3. quantises its tokens' x rows to E4M3 + UE8M0 per 32.
// Launch B (scatter): every workgroup scans the final counts into expert
//   offsets and writes t*k + j to position offsets[e] + slot (2.3 SCATTER) and
//   the inverse map.  The last workgroup to finish zeroes the global counters,
//   so the workspace is ready for the next call without a host memset.
#include "route_dev.h"

namespace moe {

// Blocks [0, route_blocks) route and count one chunk of kRouteTokensPerBlock
// tokens each; the blocks after them quantise their grid-stride share of x
// (the routing blocks, whose work is latency-bound, take no share).
__global__ __launch_bounds__(kRouteThreads) void route_count_quant_kernel(RouteParams p, int npl,
                                                                          int route_blocks) {
    if ((int)blockIdx.x < route_blocks) {
        route_count_block(p, npl);
        return;
    }
    if (p.x) quant_rows<kRouteThreads>(p, (int)blockIdx.x - route_blocks, (int)gridDim.x - route_blocks);
}

__global__ __launch_bounds__(kRouteThreads) void scatter_kernel(ScatterParams p) {
    __shared__ int cnt[kMaxExperts];
    __shared__ int off[kMaxExperts + 1];
    __shared__ int tiles[kMaxExperts];
    __shared__ int toff[kMaxExperts + 1];
    __shared__ BlockScan::storage_type tmp;
    __shared__ int last;
    const int tid = threadIdx.x;
    // this thread's first pair, loaded before the counters so that the two
    // round trips overlap (they do not depend on each other)
    const int64_t npairs = p.T * p.topk;
    const int64_t i0 = (int64_t)blockIdx.x * kRouteThreads + tid;
    int e0 = -1, s0 = -1;
    float w0 = 0.0f;
    if (i0 < npairs) {
        e0 = p.idx[i0];
        s0 = p.slot_in_e[i0];
        w0 = p.wts[i0];
    }
    for (int e = tid; e < p.E; e += kRouteThreads)
        cnt[e] = __hip_atomic_load(&p.cnt[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    // Every counter has been read by this block (the values are in LDS, past
    // the barrier): report it; the last block to report resets them.  No fence:
    // only the block's reads must precede its report, and they have returned.
    if (tid == 0) {
        unsigned prev = atomicAdd(p.arrive, 1u);
        last = prev == gridDim.x - 1;
    }
    block_exclusive_scan(cnt, off, p.E, tmp);
    if (last) {
        for (int e = tid; e < p.E; e += kRouteThreads) p.cnt[e] = 0;
        if (tid == 0) *p.arrive = 0;
    }
    write_tables(p, cnt, off, tiles, toff, tmp, blockIdx.x, gridDim.x);
    for (int64_t i = i0; i < npairs; i += (int64_t)gridDim.x * kRouteThreads) {
        const int e = i == i0 ? e0 : p.idx[i];
        const int s = i == i0 ? s0 : p.slot_in_e[i];
        if (e >= 0 && e < p.E && s >= 0) {
            int pos = off[e] + s;
            p.slot_src[pos] = (int)i;
            p.slot_of[i] = pos;
            p.slot_w[pos] = i == i0 ? w0 : p.wts[i];
        } else {
            p.slot_of[i] = -1;
        }
    }
}

// Few tokens (T <= kSmallTokens, T * k <= kSmallPairs): workgroup 0 routes and
// buckets every pair with no second launch; the other workgroups quantise x
// meanwhile.
__global__ __launch_bounds__(kSmallThreads) void route_small_kernel(RouteParams rp, ScatterParams sp,
                                                                    int npl) {
    if (blockIdx.x == 0) {
        bucket_small<kSmallThreads>(rp, sp, npl);
        if (gridDim.x > 1) return;                    // the other workgroups quantise x
    }
    if (rp.x) {
        const int b = gridDim.x > 1 ? (int)blockIdx.x - 1 : 0;
        quant_rows<kSmallThreads>(rp, b, gridDim.x > 1 ? (int)gridDim.x - 1 : 1);
    }
}

hipError_t launch_route(const RouteParams& rp, const ScatterParams& sp, hipStream_t s) {
    if (rp.T > 0 && rp.T <= kSmallTokens && rp.T * rp.topk <= kSmallPairs) {
        // workgroup 0 routes and buckets; the others quantise x
        int64_t quant_blocks = rp.x ? (rp.T * (rp.H / 8) + kSmallThreads - 1) / kSmallThreads : 0;
        dim3 grid((unsigned)(1 + std::min<int64_t>(quant_blocks, 2048)));
        const int npl = rp.logits ? (rp.E + 63) / 64 : 1;
        hipLaunchKernelGGL(route_small_kernel, grid, dim3(kSmallThreads), 0, s, rp, sp, npl);
        return hipGetLastError();
    }
    if (rp.T > 0) {
        const int64_t route_blocks = (rp.T + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock;
        const int64_t quant_blocks =
            rp.x ? (rp.T * (rp.H / 8) + 4 * kRouteThreads - 1) / (4 * kRouteThreads) : 0;
        if (route_blocks + 2048 > (((int64_t)1 << 31) - 1)) return hipErrorInvalidValue;
        dim3 grid((unsigned)(route_blocks + std::min<int64_t>(quant_blocks, 2048)));
        const int npl = rp.logits ? (rp.E + 63) / 64 : 1;
        hipLaunchKernelGGL(route_count_quant_kernel, grid, dim3(kRouteThreads), 0, s, rp, npl,
                           (int)route_blocks);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // one pair per thread (the scatter is a chain of dependent loads and stores)
    int64_t npairs = sp.T * sp.topk;
    unsigned blocks = (unsigned)std::max<int64_t>(
        1, std::min<int64_t>(2048, (npairs + kRouteThreads - 1) / kRouteThreads));
    hipLaunchKernelGGL(scatter_kernel, dim3(blocks), dim3(kRouteThreads), 0, s, sp);
    return hipGetLastError();
}

}  // namespace moe
