// Kernel parameter blocks and launchers (internal to the library).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

namespace moe {

constexpr int kRouteTokensPerBlock = 16;
constexpr int kSubRows = 16;            // rows of a sub-tile (the narrow GEMMs' unit of rows)
constexpr int kMaxExpertsCap = 1024;    // largest E the library takes

struct RouteParams {
    const float* logits;        // [T, E] or null
    const int32_t* idx_in;      // [T, k] caller ids (when logits == null)
    const float* w_in;          // [T, k]
    int32_t* idx_out;           // [T, k]
    float* w_out;               // [T, k]
    int* cnt;                   // [E] global counters, zero on entry
    int32_t* slot_in_e;         // [T, k] slot of the pair inside its expert
    const uint16_t* x;          // [T, H] BF16 or null (no quantisation)
    uint8_t* xq;                // [T, H]
    uint8_t* xsf;               // [H/128, T, 4] (K-step major)
    int64_t T;
    int H, E, topk, score_fn, renorm;
};

struct ScatterParams {
    const int32_t* idx;         // [T, k]
    const int32_t* slot_in_e;   // [T, k]
    int* cnt;                   // [E] global counters (reset to zero by the last block)
    unsigned* arrive;           // arrival counter (reset to zero by the last block)
    int32_t* counts_out;        // [E]
    int32_t* offsets_out;       // [E + 1]
    int32_t* mtile_off;         // [E + 1] prefix sum of ceil(count / bm)
    int32_t* mtile_e;           // [sum ceil(count / bm)] expert of each m-tile
    int4* mtile_rec;            // [max_mtiles] {expert, first position, rows, 0}; rows = 0
                                // past the last m-tile
    int4* sub_rec;              // [max_subs] the same for 16-row sub-tiles
    int32_t* nsub;              // [1] number of 16-row sub-tiles
    int* ready;                 // [nready] zeroed here for the one-launch GEMMs
    int* status;                // [1] zeroed here
    int32_t* slot_src;          // [T*k]
    int32_t* slot_of;           // [T, k]
    const float* wts;           // [T, k] routing weights (read by the multi-workgroup scatter)
    float* slot_w;              // [T*k] routing weight of the pair at each position
    int64_t T;
    int E, topk, bm, max_mtiles, max_subs;
    int nready;                 // max(max_mtiles, max_subs)
};

hipError_t launch_route(const RouteParams& rp, const ScatterParams& sp, hipStream_t s);

hipError_t launch_quant_act(const uint16_t* x, int64_t rows, int cols, uint8_t* q, uint8_t* sf,
                            hipStream_t s);
hipError_t launch_pack_weights(const uint16_t* w, int64_t rows, int cols, uint8_t* q,
                               uint8_t* sf, hipStream_t s);
hipError_t launch_scales_kmajor(const uint8_t* sf, int64_t mats, int rows, int cols, uint8_t* out,
                                hipStream_t s);
// packed FP4 codes [mats, rows, cols/2] (canonical row order) -> the staged layout
// (w13: W13 with rows = 2I, else W2)
hipError_t launch_stage_weights(const uint8_t* w, int64_t mats, int rows, int cols, bool w13, uint8_t* out,
                                hipStream_t s);

// Grouped GEMMs.  Positions p index the per-expert segments produced by the
// bucketisation: expert e owns p in [offsets[e], offsets[e+1]).
struct GemmParams {
    const int32_t* offsets;     // [E + 1]
    const int32_t* mtile_off;   // [E + 1] m-tiles per expert, prefix-summed (tile rows = BM)
    const int32_t* mtile_e;     // [max_mtiles] expert of each m-tile
    const int4* mtile_rec;      // [max_mtiles] {expert, first position, rows, 0}
    const int4* sub_rec;        // [max_subs] the same for 16-row sub-tiles
    const int32_t* nsub;        // [1] number of 16-row sub-tiles
    const int32_t* slot_src;    // [R] t*k + j of position p
    const float* slot_w;        // [R] routing weight of the pair at position p
    const float* topk_w;        // [T, k]
    const uint8_t* xq;          // [T, H]    GEMM1 A (gathered rows)
    const uint8_t* xsf;         // [H/128, T, 4]      K-step major scales
    const uint8_t* w13;         // [E, 2I, H/2]
    const uint8_t* w13sf;       // [E, H/128, 2I, 4]
    uint8_t* hq;                // [R, I]    GEMM1 output / GEMM2 A
    uint8_t* hsf;               // [I/128, R, 4]
    const uint8_t* w2;          // [E, H, I/2]
    const uint8_t* w2sf;        // [E, I/128, H, 4]
    uint16_t* o;                // [R, H]    GEMM2 output (BF16)
    float* hf32;                // [R, I]    block-FP8 weights: GEMM1's h in float32 (shares o's bytes)
    int64_t T;
    int H, I, E, topk;
    int max_mtiles;             // upper bound of mtile_off[E]
    int max_subs;               // upper bound of *nsub
    // one-launch GEMM1 -> GEMM2 (both zeroed by the bucketing stage of the call)
    int* ready;                 // [max(max_mtiles, max_subs)] GEMM1 n-tiles of the m-tile (tiled
                                // one-launch) or GEMM1 units of the sub-tile (narrow one-launch)
                                // whose h is stored
    int* status;                // [1] set to 1 if a wait gave up (never in a correct run)
    int wave_experts;           // experts per scheduling wave (set by the launcher)
    int spin_limit;             // polls of a ready counter before a wait gives up; 0: the
                                // kernel's own bound (about 0.5 s)
    int w13_il;                 // W13 rows pre-interleaved: 8 gate rows, then the same 8
                                // columns' up rows (else all gate rows, then all up rows)
    int w_staged;               // W13 and W2 codes in the staged layout (canonical scales)
    // byte strides of the weight scales per weight row and per 128-wide K step:
    // K-step major (4, 4 * rows) or per row (K / 32, 4)
    int64_t w13sf_rs, w13sf_ks, w2sf_rs, w2sf_ks;
};

constexpr int kTileRows = 128;  // rows per m-tile of the tiled grouped GEMMs
int gemm_bm();                  // the same, as the GEMM source defines it (== kTileRows)

// Launch facts cached per device (CU counts, occupancies, "attribute set"):
// the entry for the current device is filled by fill(dev, &value) on first use.
// 0 means "not cached", so a fill that yields 0 runs again next time.  Host
// threads may race on the first fill; they compute the same value.
constexpr int kMaxDevices = 64;
using DeviceCache = std::atomic<int>[kMaxDevices];
template <class F>
hipError_t per_device(DeviceCache& cache, F fill, int* out) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        err = fill(dev, &v);
        if (err != hipSuccess) return err;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    *out = v;
    return hipSuccess;
}
inline hipError_t device_cus(int* cus) {
    static DeviceCache cache;
    return per_device(cache, [](int dev, int* v) {
        return hipDeviceGetAttribute(v, hipDeviceAttributeMultiprocessorCount, dev);
    }, cus);
}

// The GEMM launchers take an optional pair of events that the launch itself
// carries (hipExtLaunchKernel): they take the kernel's start and end times.
// A launcher with nothing to launch records them on the stream instead.
inline hipError_t record_pair(hipEvent_t ev0, hipEvent_t ev1, hipStream_t s) {
    hipError_t err = ev0 ? hipEventRecord(ev0, s) : hipSuccess;
    if (err == hipSuccess && ev1) err = hipEventRecord(ev1, s);
    return err;
}
hipError_t launch_gemm1(const GemmParams& p, hipStream_t s, hipEvent_t ev0 = nullptr,
                        hipEvent_t ev1 = nullptr);
hipError_t launch_gemm2(const GemmParams& p, hipStream_t s, hipEvent_t ev0 = nullptr,
                        hipEvent_t ev1 = nullptr);
// GEMM1 -> SwiGLU -> GEMM2 in one persistent launch with per-m-tile ready counters
hipError_t launch_fused_gemm(const GemmParams& p, hipStream_t s, hipEvent_t ev0 = nullptr,
                             hipEvent_t ev1 = nullptr);
// the same two GEMMs for few rows per expert (decode): N split over many small
// workgroups that stream weights straight into registers
hipError_t launch_narrow_gemm1(const GemmParams& p, hipStream_t s, hipEvent_t ev0 = nullptr,
                               hipEvent_t ev1 = nullptr);
hipError_t launch_narrow_gemm2(const GemmParams& p, hipStream_t s, hipEvent_t ev0 = nullptr,
                               hipEvent_t ev1 = nullptr);
hipError_t launch_narrow_fused(const GemmParams& p, hipStream_t s, hipEvent_t ev0 = nullptr,
                               hipEvent_t ev1 = nullptr);
// the narrow GEMMs with block-FP8 weights (GEMM1 leaves float32 h in p.hf32)
hipError_t launch_narrow_w8_gemm1(const GemmParams& p, hipStream_t s, hipEvent_t ev0 = nullptr,
                                  hipEvent_t ev1 = nullptr);
hipError_t launch_narrow_w8_gemm2(const GemmParams& p, hipStream_t s, hipEvent_t ev0 = nullptr,
                                  hipEvent_t ev1 = nullptr);
// block-FP8 quantisers: rows of BF16 (f32_in false) or float32 values -> E4M3
// codes [rows, cols] + float32 scales [cols/128][rows] (one per row per 128);
// BF16 weights [rows, cols] -> E4M3 codes + float32 scales [rows/128][cols/128]
hipError_t launch_quant_rows128(const void* src, bool f32_in, int64_t rows, int cols, uint8_t* q, float* sf,
                                hipStream_t s);
hipError_t launch_pack_block128(const uint16_t* w, int64_t rows, int cols, uint8_t* q, float* sf,
                                hipStream_t s);

// Read `bytes` (a multiple of 16) from src once, with nothing else to do (the
// HBM read ceiling of a footprint); sink takes a flag no real data sets.
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s,
                              hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

hipError_t launch_combine(const uint16_t* o, const int32_t* slot_of, int64_t T, int topk, int H,
                          uint16_t* y, hipStream_t s);

// The whole layer in one cooperative launch for T * topk <= 1024 (routing and
// bucketing in one workgroup, narrow GEMMs, combine), phases handed over by
// arrival counts that are zero between launches.
struct LayerParams {
    uint16_t* y;                // [T, H] layer output
    unsigned* count;            // workgroups done with the routing phase (zero on entry, reset on exit)
    unsigned* count2;           // workgroups done with GEMM2 (zero on entry, reset on exit)
    unsigned* exits;            // workgroups that have left (zero on entry, reset on exit)
    int* status;                // [1] set to 2 if a hand-off wait gave up
    int npl;                    // logits per lane of the routing waves (set by the launcher)
};
bool layer_small_fits(int64_t T, int topk);
hipError_t launch_layer_small(const RouteParams& rp, const ScatterParams& sp, const GemmParams& gp,
                              LayerParams lp, hipStream_t s);

}  // namespace moe
