// Host side of the C ABI declared in include/moe.h: argument checks, the
// workspace carve, and the launch sequence of the layer.
#include <atomic>
#include <string>

#include "moe.h"
#include "common.h"
#include "kernels.h"

namespace {

thread_local std::string g_hip_error;

int hip_fail(hipError_t err) {
    g_hip_error = hipGetErrorString(err);
    return MOE_EHIP;
}

constexpr size_t kAlign = 256;
// moe_forward picks the narrow GEMMs when T * topk <= this many rows per expert:
// measured crossover of the two GEMM families at 3 to 4 rows per expert, both at
// H = 7168, I = 2048, E = 32 and at H = 2048, I = 512, E = 256
constexpr int64_t kNarrowRowsPerExpert = 3;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Carve {
    size_t cnt, arrive, status, counts, offsets, mtile_off, mtile_e, mtile_rec, sub_rec, nsub, ready,
        topk_idx, topk_w, slot_in_e, slot_src, slot_of, slot_w;
    size_t xq, xsf, hq, hsf, o, total;
};

// Upper bound of the number of m-tiles: sum over experts of ceil(count / bm)
// <= R / bm + (number of non-empty experts).
int64_t max_mtiles(const moe_dims_t& d) {
    const int64_t R = d.T * d.topk, bm = moe::gemm_bm();
    return (R + bm - 1) / bm + std::min<int64_t>(d.E, R);
}

// The same bound for the 16-row sub-tiles of the narrow GEMMs.
int64_t max_subs(const moe_dims_t& d) {
    const int64_t R = d.T * d.topk;
    return (R + moe::kSubRows - 1) / moe::kSubRows + std::min<int64_t>(d.E, R);
}

Carve carve(const moe_dims_t& d) {
    Carve c{};
    const size_t T = (size_t)d.T, E = (size_t)d.E, k = (size_t)d.topk, R = T * k;
    size_t at = 0;
    auto take = [&](size_t bytes) { size_t off = at; at = align_up(at + bytes); return off; };
    // counters first, at offsets that do not depend on the shape: a workspace can
    // serve calls of different shapes after one moe_workspace_init
    c.cnt = take(moe::kMaxExpertsCap * 4);
    c.arrive = take(64);
    c.status = take(64);
    c.counts = take(E * 4);
    c.offsets = take((E + 1) * 4);
    c.mtile_off = take((E + 1) * 4);
    c.mtile_e = take((max_mtiles(d) + 1) * 4);
    c.mtile_rec = take((max_mtiles(d) + 1) * 16);
    c.sub_rec = take((max_subs(d) + 1) * 16);
    c.nsub = take(4);
    c.ready = take(std::max(max_mtiles(d), max_subs(d)) * 4);
    c.topk_idx = take(R * 4);
    c.topk_w = take(R * 4);
    c.slot_in_e = take(R * 4);
    c.slot_src = take(R * 4);
    c.slot_of = take(R * 4);
    c.slot_w = take(R * 4);
    c.xq = take(T * (size_t)d.H);
    c.xsf = take(T * (size_t)d.H / 32);
    c.hq = take(R * (size_t)d.I);
    c.hsf = take(R * (size_t)d.I / 32);
    // o is BF16 [R, H]; with block-FP8 weights the same bytes first hold GEMM1's
    // float32 h [R, I] (quantised before GEMM2 writes o)
    c.o = take(R * std::max((size_t)d.H * 2, (size_t)d.I * 4));
    c.total = at;
    return c;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15) == 0; }

int check_dims(const moe_dims_t* d) {
    if (!d) return MOE_EINVAL;
    if (d->T < 0 || d->T > (1ll << 24)) return MOE_EINVAL;
    if (d->H <= 0 || d->I <= 0 || d->E <= 0 || d->topk <= 0) return MOE_EINVAL;
    if (d->topk > d->E || d->topk > 16 || d->E > 1024) return MOE_EUNSUPPORTED;
    if (d->H % 128 != 0 || d->I % 128 != 0) return MOE_EUNSUPPORTED;
    if (d->score_fn != MOE_SCORE_SOFTMAX && d->score_fn != MOE_SCORE_SIGMOID) return MOE_EINVAL;
    // the grouped GEMMs address A rows and one expert's weights with 32-bit byte offsets
    const int64_t lim = 1ll << 32;
    if ((int64_t)d->T * d->H >= lim || (int64_t)d->T * d->topk * d->I >= lim ||
        (int64_t)d->H * d->I >= lim)
        return MOE_EUNSUPPORTED;
    return MOE_OK;
}

__global__ void zero_kernel(uint4* p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0, 0, 0, 0);
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off); }

// Regions of the routing step inside a scratch buffer (byte offsets).
struct RouteRegions {
    size_t cnt, arrive, status, mtile_off, mtile_e, mtile_rec, sub_rec, nsub, ready, slot_in_e, slot_w;
};

// Routing and bucketisation of d's logits into the caller's outputs, with the
// counters and tables in `base` at regions r.
hipError_t launch_route_into(const moe_dims_t& d, const float* logits, int32_t* topk_idx, float* topk_w,
                             int32_t* counts, int32_t* offsets, int32_t* slot_src, int32_t* slot_of,
                             uint8_t* base, const RouteRegions& r, hipStream_t s) {
    moe::RouteParams rp{};
    rp.logits = logits;
    rp.idx_out = topk_idx;
    rp.w_out = topk_w;
    rp.cnt = reinterpret_cast<int*>(base + r.cnt);
    rp.slot_in_e = reinterpret_cast<int32_t*>(base + r.slot_in_e);
    rp.T = d.T;
    rp.H = d.H;
    rp.E = d.E;
    rp.topk = d.topk;
    rp.score_fn = d.score_fn;
    rp.renorm = d.renorm;
    moe::ScatterParams sp{};
    sp.idx = topk_idx;
    sp.slot_in_e = rp.slot_in_e;
    sp.cnt = rp.cnt;
    sp.arrive = reinterpret_cast<unsigned*>(base + r.arrive);
    sp.counts_out = counts;
    sp.offsets_out = offsets;
    sp.mtile_off = reinterpret_cast<int32_t*>(base + r.mtile_off);
    sp.mtile_e = reinterpret_cast<int32_t*>(base + r.mtile_e);
    sp.slot_src = slot_src;
    sp.slot_of = slot_of;
    sp.wts = topk_w;
    sp.slot_w = reinterpret_cast<float*>(base + r.slot_w);
    sp.T = d.T;
    sp.E = d.E;
    sp.topk = d.topk;
    sp.bm = moe::gemm_bm();
    sp.mtile_rec = reinterpret_cast<int4*>(base + r.mtile_rec);
    sp.max_mtiles = (int)max_mtiles(d);
    sp.sub_rec = reinterpret_cast<int4*>(base + r.sub_rec);
    sp.nsub = reinterpret_cast<int32_t*>(base + r.nsub);
    sp.max_subs = (int)max_subs(d);
    sp.nready = (int)std::max(max_mtiles(d), max_subs(d));
    sp.ready = reinterpret_cast<int*>(base + r.ready);
    sp.status = reinterpret_cast<int*>(base + r.status);
    return moe::launch_route(rp, sp, s);
}

// ---------------------------------------------------------------- routing without allocation
// moe_route_noalloc keeps the routing step's counters and tables in a file-scope
// device array instead of a caller's workspace, for callers that cannot
// allocate.  Sized for T * topk <= kNoAllocMaxPairs with any E <= 1024.
constexpr int64_t kNoAllocMaxPairs = int64_t(1) << 18;

constexpr size_t align256(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct RouteCarve {
    RouteRegions r;
    size_t total;
};

// The routing regions alone, laid out as carve() lays them out: the counter
// header (cnt, arrive, status) first.
constexpr RouteCarve carve_route(int64_t R, int64_t E) {
    const int64_t nonempty = E < R ? E : R;
    const int64_t mtiles = (R + moe::kTileRows - 1) / moe::kTileRows + nonempty;
    const int64_t subs = (R + moe::kSubRows - 1) / moe::kSubRows + nonempty;
    RouteCarve c{};
    size_t at = 0;
    c.r.cnt = at;       at = align256(at + moe::kMaxExpertsCap * 4);
    c.r.arrive = at;    at = align256(at + 64);
    c.r.status = at;    at = align256(at + 64);
    c.r.mtile_off = at; at = align256(at + (size_t)(E + 1) * 4);
    c.r.mtile_e = at;   at = align256(at + (size_t)(mtiles + 1) * 4);
    c.r.mtile_rec = at; at = align256(at + (size_t)(mtiles + 1) * 16);
    c.r.sub_rec = at;   at = align256(at + (size_t)(subs + 1) * 16);
    c.r.nsub = at;      at = align256(at + 4);
    c.r.ready = at;     at = align256(at + (size_t)(mtiles > subs ? mtiles : subs) * 4);
    c.r.slot_in_e = at; at = align256(at + (size_t)R * 4);
    c.r.slot_w = at;    at = align256(at + (size_t)R * 4);
    c.total = at;
    return c;
}

constexpr size_t kScratchBytes = carve_route(kNoAllocMaxPairs, moe::kMaxExpertsCap).total;   // ~2.4 MiB

}  // namespace

// The no-allocation routing scratch: one copy per device, held until the process
// ends, shared by every moe_route_noalloc call on that device.  Host code never
// uses this name as an address: scratch_address() looks up each device's copy.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::atomic<void*> g_scratch[moe::kMaxDevices];

// Device address of the current device's scratch, looked up once per device
// (hipGetSymbolAddress with that device current) and kept.
hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= moe::kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" {

int moe_workspace_size(const moe_dims_t* d, size_t* bytes) {
    int rc = check_dims(d);
    if (rc) return rc;
    if (!bytes) return MOE_EINVAL;
    *bytes = carve(*d).total;
    return MOE_OK;
}

int moe_workspace_layout(const moe_dims_t* d, moe_layout_t* out) {
    int rc = check_dims(d);
    if (rc) return rc;
    if (!out) return MOE_EINVAL;
    Carve c = carve(*d);
    out->topk_idx = c.topk_idx;
    out->topk_w = c.topk_w;
    out->counts = c.counts;
    out->offsets = c.offsets;
    out->slot_src = c.slot_src;
    out->slot_of = c.slot_of;
    out->xq = c.xq;
    out->xsf = c.xsf;
    out->hq = c.hq;
    out->hsf = c.hsf;
    out->o = c.o;
    out->status = c.status;
    out->total = c.total;
    return MOE_OK;
}

int moe_workspace_init(void* ws, size_t ws_bytes, hipStream_t s) {
    if (!ws || ((uintptr_t)ws % kAlign) != 0 || ws_bytes % 16 != 0) return MOE_EINVAL;
    size_t n16 = ws_bytes / 16;
    if (n16 == 0) return MOE_OK;
    unsigned grid = (unsigned)std::min<size_t>((n16 + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, s, static_cast<uint4*>(ws), n16);
    hipError_t err = hipGetLastError();
    return err == hipSuccess ? MOE_OK : hip_fail(err);
}

int moe_route(const moe_dims_t* d, const float* logits, int32_t* topk_idx, float* topk_w,
              int32_t* counts, int32_t* offsets, int32_t* slot_src, int32_t* slot_of, void* ws,
              size_t ws_bytes, hipStream_t s) {
    int rc = check_dims(d);
    if (rc) return rc;
    if (!logits || !topk_idx || !topk_w || !counts || !offsets || !slot_src || !slot_of || !ws)
        return MOE_EINVAL;
    Carve c = carve(*d);
    if (ws_bytes < c.total || ((uintptr_t)ws % kAlign) != 0) return MOE_EWORKSPACE;
    RouteRegions r{c.cnt, c.arrive, c.status, c.mtile_off, c.mtile_e, c.mtile_rec, c.sub_rec, c.nsub,
                   c.ready, c.slot_in_e, c.slot_w};
    hipError_t err = launch_route_into(*d, logits, topk_idx, topk_w, counts, offsets, slot_src, slot_of,
                                       static_cast<uint8_t*>(ws), r, s);
    return err == hipSuccess ? MOE_OK : hip_fail(err);
}

int moe_route_noalloc(const moe_dims_t* d, const float* logits, int32_t* topk_idx, float* topk_w,
                      int32_t* counts, int32_t* offsets, int32_t* slot_src, int32_t* slot_of,
                      hipStream_t s) {
    int rc = check_dims(d);
    if (rc) return rc;
    if (!logits || !topk_idx || !topk_w || !counts || !offsets || !slot_src || !slot_of)
        return MOE_EINVAL;
    if (d->T * d->topk > kNoAllocMaxPairs) return MOE_ESCRATCH;
    const RouteCarve c = carve_route(d->T * d->topk, d->E);
    if (c.total > kScratchBytes) return MOE_ESCRATCH;
    void* base = nullptr;
    hipError_t err = scratch_address(&base);
    if (err == hipSuccess) {
        // the counter header must be zero on entry: every call clears it with a
        // fill kernel (no memset node, so the call can be captured in a graph)
        const size_t n16 = (c.r.status + 64) / 16;
        hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(256), 0, s, static_cast<uint4*>(base), n16);
        err = hipGetLastError();
    }
    if (err == hipSuccess)
        err = launch_route_into(*d, logits, topk_idx, topk_w, counts, offsets, slot_src, slot_of,
                                static_cast<uint8_t*>(base), c.r, s);
    return err == hipSuccess ? MOE_OK : hip_fail(err);
}

int moe_quant_act(const uint16_t* x, int64_t rows, int32_t cols, uint8_t* q, uint8_t* sf,
                  hipStream_t s) {
    if (rows < 0 || cols <= 0 || cols % 32 != 0) return MOE_EINVAL;
    if (rows == 0) return MOE_OK;
    if (!x || !q || !sf || !aligned16(x) || ((uintptr_t)q & 7) != 0) return MOE_EINVAL;
    hipError_t err = moe::launch_quant_act(x, rows, cols, q, sf, s);
    return err == hipSuccess ? MOE_OK : hip_fail(err);
}

int moe_pack_weights(const uint16_t* w, int64_t rows, int32_t cols, uint8_t* q, uint8_t* sf,
                     hipStream_t s) {
    if (rows < 0 || cols <= 0 || cols % 32 != 0) return MOE_EINVAL;
    if (rows == 0) return MOE_OK;
    if (!w || !q || !sf || !aligned16(w) || ((uintptr_t)q & 3) != 0) return MOE_EINVAL;
    hipError_t err = moe::launch_pack_weights(w, rows, cols, q, sf, s);
    return err == hipSuccess ? MOE_OK : hip_fail(err);
}

int moe_pack_weights_fp8_block128(const uint16_t* w, int64_t rows, int32_t cols, uint8_t* q, float* sf,
                                  hipStream_t s) {
    if (rows < 0 || cols <= 0 || rows % 128 != 0 || cols % 128 != 0) return MOE_EINVAL;
    if (rows == 0) return MOE_OK;
    if (!w || !q || !sf || !aligned16(w) || !aligned16(q) || ((uintptr_t)sf & 3)) return MOE_EINVAL;
    hipError_t err = moe::launch_pack_block128(w, rows, cols, q, sf, s);
    return err == hipSuccess ? MOE_OK : hip_fail(err);
}

int moe_scales_kmajor(const uint8_t* sf, int64_t mats, int32_t rows, int32_t cols, uint8_t* out,
                      hipStream_t s) {
    if (mats < 0 || rows < 0 || cols <= 0 || cols % 128 != 0) return MOE_EINVAL;
    if (mats == 0 || rows == 0) return MOE_OK;
    if (!sf || !out || ((uintptr_t)sf & 3) || ((uintptr_t)out & 3) || sf == out) return MOE_EINVAL;
    hipError_t err = moe::launch_scales_kmajor(sf, mats, rows, cols, out, s);
    return err == hipSuccess ? MOE_OK : hip_fail(err);
}

int moe_stage_weights(const uint8_t* w, int64_t mats, int32_t rows, int32_t cols, int32_t is_w13, uint8_t* out,
                      hipStream_t s) {
    if (mats < 0 || rows < 0 || cols <= 0 || cols % 128 != 0 || rows % 128 != 0) return MOE_EINVAL;
    if (mats == 0 || rows == 0) return MOE_OK;
    const uint64_t bytes = (uint64_t)mats * (uint64_t)rows * (uint64_t)(cols / 2);
    if (!w || !out || !aligned16(w) || !aligned16(out)) return MOE_EINVAL;
    const uintptr_t a0 = (uintptr_t)w, b0 = (uintptr_t)out;
    if (a0 < b0 + bytes && b0 < a0 + bytes) return MOE_EINVAL;
    hipError_t err = moe::launch_stage_weights(w, mats, rows, cols, is_w13 != 0, out, s);
    return err == hipSuccess ? MOE_OK : hip_fail(err);
}

int moe_forward(const moe_args_t* a, hipStream_t s) {
    if (!a) return MOE_EINVAL;
    const moe_dims_t& d = a->dims;
    int rc = check_dims(&d);
    if (rc) return rc;
    if (d.T == 0) return MOE_OK;
    if (!a->x || !a->w13 || !a->w13_sf || !a->w2 || !a->w2_sf || !a->y || !a->ws) return MOE_EINVAL;
    if (!a->logits && (!a->topk_idx || !a->topk_w)) return MOE_EINVAL;
    const uint32_t f = a->flags;
    const uint32_t known = MOE_FLAG_NARROW | MOE_FLAG_TILED | MOE_FLAG_ONE_LAUNCH | MOE_FLAG_ONE_KERNEL |
                           MOE_FLAG_W13_PREINTERLEAVED | MOE_FLAG_W_SCALES_PER_ROW |
                           MOE_FLAG_KEEP_INTERMEDIATES | MOE_FLAG_DEBUG_SPIN_BOUND |
                           MOE_FLAG_WEIGHTS_FP8_BLOCK128 | MOE_FLAG_W_STAGED;
    if ((f & ~known) || ((f & MOE_FLAG_NARROW) && (f & MOE_FLAG_TILED)) ||
        ((f & MOE_FLAG_ONE_KERNEL) &&
         (f & (MOE_FLAG_TILED | MOE_FLAG_ONE_LAUNCH | MOE_FLAG_DEBUG_SPIN_BOUND))))
        return MOE_EINVAL;
    const bool w8 = (f & MOE_FLAG_WEIGHTS_FP8_BLOCK128) != 0;
    if (w8 && (f & (MOE_FLAG_W13_PREINTERLEAVED | MOE_FLAG_W_SCALES_PER_ROW | MOE_FLAG_W_STAGED)))
        return MOE_EINVAL;
    if ((f & MOE_FLAG_W_STAGED) && (f & MOE_FLAG_W13_PREINTERLEAVED)) return MOE_EINVAL;
    if (w8 && (f & (MOE_FLAG_TILED | MOE_FLAG_ONE_LAUNCH | MOE_FLAG_ONE_KERNEL))) return MOE_EUNSUPPORTED;
    if ((f & MOE_FLAG_ONE_KERNEL) && !moe::layer_small_fits(d.T, d.topk)) return MOE_EUNSUPPORTED;
    if (!aligned16(a->x) || !aligned16(a->w13) || !aligned16(a->w2) || !aligned16(a->y) ||
        ((uintptr_t)a->w13_sf & 3) || ((uintptr_t)a->w2_sf & 3))
        return MOE_EINVAL;
    Carve c = carve(d);
    if (a->ws_bytes < c.total || ((uintptr_t)a->ws % kAlign) != 0) return MOE_EWORKSPACE;
    void* ws = a->ws;

    moe::RouteParams rp{};
    rp.logits = a->logits;
    rp.idx_in = a->topk_idx;
    rp.w_in = a->topk_w;
    rp.idx_out = at<int32_t>(ws, c.topk_idx);
    rp.w_out = at<float>(ws, c.topk_w);
    rp.cnt = at<int>(ws, c.cnt);
    rp.slot_in_e = at<int32_t>(ws, c.slot_in_e);
    // block-FP8 weights quantise x per 128 in a launch of their own
    rp.x = w8 ? nullptr : a->x;
    rp.xq = at<uint8_t>(ws, c.xq);
    rp.xsf = at<uint8_t>(ws, c.xsf);
    rp.T = d.T;
    rp.H = d.H;
    rp.E = d.E;
    rp.topk = d.topk;
    rp.score_fn = d.score_fn;
    rp.renorm = d.renorm;
    moe::ScatterParams sp{};
    sp.idx = rp.idx_out;
    sp.slot_in_e = rp.slot_in_e;
    sp.cnt = rp.cnt;
    sp.arrive = at<unsigned>(ws, c.arrive);
    sp.counts_out = at<int32_t>(ws, c.counts);
    sp.offsets_out = at<int32_t>(ws, c.offsets);
    sp.mtile_off = at<int32_t>(ws, c.mtile_off);
    sp.mtile_e = at<int32_t>(ws, c.mtile_e);
    sp.slot_src = at<int32_t>(ws, c.slot_src);
    sp.slot_of = at<int32_t>(ws, c.slot_of);
    sp.wts = rp.w_out;
    sp.slot_w = at<float>(ws, c.slot_w);
    sp.T = d.T;
    sp.E = d.E;
    sp.topk = d.topk;
    sp.bm = moe::gemm_bm();
    sp.mtile_rec = at<int4>(ws, c.mtile_rec);
    sp.max_mtiles = (int)max_mtiles(d);
    sp.sub_rec = at<int4>(ws, c.sub_rec);
    sp.nsub = at<int32_t>(ws, c.nsub);
    sp.max_subs = (int)max_subs(d);
    sp.nready = (int)std::max(max_mtiles(d), max_subs(d));
    sp.ready = at<int>(ws, c.ready);
    sp.status = at<int>(ws, c.status);
    hipEvent_t* ev = a->stage_events;
    hipError_t err = ev ? hipEventRecord(ev[0], s) : hipSuccess;
    const bool one_kernel = (f & MOE_FLAG_ONE_KERNEL) != 0;
    if (err == hipSuccess && !one_kernel) err = moe::launch_route(rp, sp, s);
    if (err != hipSuccess) return hip_fail(err);

    moe::GemmParams gp{};
    gp.offsets = sp.offsets_out;
    gp.mtile_off = sp.mtile_off;
    gp.mtile_e = sp.mtile_e;
    gp.mtile_rec = sp.mtile_rec;
    gp.sub_rec = sp.sub_rec;
    gp.nsub = sp.nsub;
    gp.ready = at<int>(ws, c.ready);
    gp.status = at<int>(ws, c.status);
    gp.slot_src = sp.slot_src;
    gp.slot_w = sp.slot_w;
    gp.topk_w = rp.w_out;
    gp.xq = rp.xq;
    gp.xsf = rp.xsf;
    gp.w13 = a->w13;
    gp.w13sf = a->w13_sf;
    gp.hq = at<uint8_t>(ws, c.hq);
    gp.hsf = at<uint8_t>(ws, c.hsf);
    gp.w2 = a->w2;
    gp.w2sf = a->w2_sf;
    gp.o = at<uint16_t>(ws, c.o);
    gp.hf32 = at<float>(ws, c.o);
    gp.T = d.T;
    gp.H = d.H;
    gp.I = d.I;
    gp.E = d.E;
    gp.topk = d.topk;
    // a bounded wait that gives up after one failed poll (DEBUG_SPIN_BOUND), else the kernels' own
    gp.spin_limit = (f & MOE_FLAG_DEBUG_SPIN_BOUND) ? 1 : 0;
    gp.w13_il = (f & MOE_FLAG_W13_PREINTERLEAVED) ? 1 : 0;
    gp.w_staged = (f & MOE_FLAG_W_STAGED) ? 1 : 0;
    if (f & MOE_FLAG_W_SCALES_PER_ROW) {        // [E, rows, K/32]
        gp.w13sf_rs = d.H / 32;
        gp.w2sf_rs = d.I / 32;
        gp.w13sf_ks = gp.w2sf_ks = 4;
    } else {                                    // [E, K/128, rows, 4]
        gp.w13sf_rs = gp.w2sf_rs = 4;
        gp.w13sf_ks = 4 * 2 * (int64_t)d.I;
        gp.w2sf_ks = 4 * (int64_t)d.H;
    }
    const int64_t R = d.T * d.topk;
    gp.max_mtiles = (int)max_mtiles(d);
    gp.max_subs = (int)max_subs(d);
    if (one_kernel) {
        moe::LayerParams lp{};
        lp.y = a->y;
        lp.count = at<unsigned>(ws, c.arrive) + 4;
        lp.exits = at<unsigned>(ws, c.arrive) + 8;
        lp.count2 = at<unsigned>(ws, c.arrive) + 12;
        lp.status = sp.status;
        err = moe::launch_layer_small(rp, sp, gp, lp, s);
        for (int i = 1; i < MOE_NUM_STAGE_EVENTS && err == hipSuccess && ev; ++i)
            err = hipEventRecord(ev[i], s);
        return err == hipSuccess ? MOE_OK : hip_fail(err);
    }
    // few rows per expert on average: the weight-streaming (narrow) kernels
    bool narrow = R <= kNarrowRowsPerExpert * (int64_t)d.E;
    if (a->flags & MOE_FLAG_NARROW) narrow = true;
    if (a->flags & MOE_FLAG_TILED) narrow = false;
    // ONE_LAUNCH alone keeps its tiled meaning; with NARROW it fuses the narrow GEMMs
    if ((a->flags & MOE_FLAG_ONE_LAUNCH) && !(a->flags & MOE_FLAG_NARROW)) narrow = false;
    const bool fused = (a->flags & MOE_FLAG_ONE_LAUNCH) != 0;
    hipEvent_t* kev = a->kernel_events;
    hipEvent_t k0 = kev ? kev[0] : nullptr, k1 = kev ? kev[1] : nullptr;
    if (w8) {
        // block-FP8 weights: x per 128 -> narrow GEMM1 (float32 h) -> h per 128 -> narrow GEMM2
        err = moe::launch_quant_rows128(a->x, false, d.T, d.H, rp.xq, reinterpret_cast<float*>(rp.xsf), s);
        if (err == hipSuccess && ev) err = hipEventRecord(ev[1], s);
        if (err == hipSuccess) err = moe::launch_narrow_w8_gemm1(gp, s, k0, k1);
        if (err == hipSuccess)
            err = moe::launch_quant_rows128(gp.hf32, true, R, d.I, gp.hq, reinterpret_cast<float*>(gp.hsf), s);
        if (err == hipSuccess && ev) err = hipEventRecord(ev[2], s);
        if (err == hipSuccess) err = moe::launch_narrow_w8_gemm2(gp, s);
        if (err == hipSuccess && ev) err = hipEventRecord(ev[3], s);
        if (err == hipSuccess) err = moe::launch_combine(gp.o, sp.slot_of, d.T, d.topk, d.H, a->y, s);
        if (err == hipSuccess && ev) err = hipEventRecord(ev[4], s);
        return err == hipSuccess ? MOE_OK : hip_fail(err);
    }
    if (ev) err = hipEventRecord(ev[1], s);
    if (fused) {
        // GEMM1 -> SwiGLU -> GEMM2 in one launch: both events after it
        if (err == hipSuccess)
            err = narrow ? moe::launch_narrow_fused(gp, s, k0, k1) : moe::launch_fused_gemm(gp, s, k0, k1);
        if (err == hipSuccess && ev) err = hipEventRecord(ev[2], s);
    } else {
        if (err == hipSuccess)
            err = narrow ? moe::launch_narrow_gemm1(gp, s, k0, k1) : moe::launch_gemm1(gp, s, k0, k1);
        if (err == hipSuccess && ev) err = hipEventRecord(ev[2], s);
        if (err == hipSuccess) err = narrow ? moe::launch_narrow_gemm2(gp, s) : moe::launch_gemm2(gp, s);
    }
    if (err == hipSuccess && ev) err = hipEventRecord(ev[3], s);
    if (err == hipSuccess) err = moe::launch_combine(gp.o, sp.slot_of, d.T, d.topk, d.H, a->y, s);
    if (err == hipSuccess && ev) err = hipEventRecord(ev[4], s);
    return err == hipSuccess ? MOE_OK : hip_fail(err);
}

int moe_stream_read(const void* src, size_t bytes, uint32_t* sink, hipEvent_t start, hipEvent_t stop,
                    hipStream_t s) {
    if (bytes % 16 != 0) return MOE_EINVAL;
    if (bytes && (!src || !sink || !aligned16(src) || ((uintptr_t)sink & 3))) return MOE_EINVAL;
    hipError_t err = moe::launch_stream_read(src, bytes, sink, s, start, stop);
    return err == hipSuccess ? MOE_OK : hip_fail(err);
}

int moe_check_status(const void* ws, hipStream_t s) {
    if (!ws || ((uintptr_t)ws % kAlign) != 0) return MOE_EINVAL;
    // the header's offsets do not depend on the shape: any valid shape gives them
    moe_dims_t one{1, 128, 128, 1, 1, MOE_SCORE_SOFTMAX, 1};
    const Carve c = carve(one);
    int status = 0;
    hipError_t err = hipMemcpyAsync(&status, static_cast<const uint8_t*>(ws) + c.status, sizeof(status),
                                    hipMemcpyDeviceToHost, s);
    if (err == hipSuccess) err = hipStreamSynchronize(s);
    if (err != hipSuccess) return hip_fail(err);
    return status == 0 ? MOE_OK : MOE_ETIMEOUT;
}

const char* moe_error_string(int code) {
    switch (code) {
        case MOE_OK: return "success";
        case MOE_EINVAL: return "invalid argument";
        case MOE_EUNSUPPORTED: return "unsupported shape";
        case MOE_EWORKSPACE: return "workspace too small or misaligned";
        case MOE_ETIMEOUT: return "a bounded wait inside the last call gave up (its output is invalid)";
        case MOE_ESCRATCH: return "T * topk exceeds the 262144 routed pairs the static routing scratch holds";
        case MOE_EHIP: return g_hip_error.empty() ? "HIP error" : g_hip_error.c_str();
        default: return "unknown error";
    }
}

}  // extern "C"
