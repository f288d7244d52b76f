// Block quantisers: activations BF16 -> E4M3 + UE8M0/32 ("MegaMoE" notes,
// "Dispatch阶段") and weights BF16 -> E2M1 + UE8M0/32 along K ("MegaMoE" notes,
// "Expert矩阵权重量化").  Four lanes share a 32-element group, eight BF16
// (16 bytes) per lane, so a wave reads 1 KiB of contiguous input per step.
#include "common.h"
#include "kernels.h"
#include "mfma.h"

namespace moe {

constexpr int kQuantThreads = 256;

MOE_DEV void load8(const uint16_t* src, float f[8]) {
    const uint4 raw = *reinterpret_cast<const uint4*>(src);
    f[0] = bf16_to_f32(raw.x & 0xFFFFu); f[1] = bf16_to_f32(raw.x >> 16);
    f[2] = bf16_to_f32(raw.y & 0xFFFFu); f[3] = bf16_to_f32(raw.y >> 16);
    f[4] = bf16_to_f32(raw.z & 0xFFFFu); f[5] = bf16_to_f32(raw.z >> 16);
    f[6] = bf16_to_f32(raw.w & 0xFFFFu); f[7] = bf16_to_f32(raw.w >> 16);
}

MOE_DEV float group_amax4(const float f[8]) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, __builtin_fabsf(f[j]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    return fmaxf(amax, __shfl_xor(amax, 2, 64));
}

__global__ __launch_bounds__(kQuantThreads) void quant_act_kernel(const uint16_t* __restrict__ x,
                                                                  int64_t tasks, int cols,
                                                                  uint8_t* __restrict__ q,
                                                                  uint8_t* __restrict__ sf) {
    // task i: 8 elements starting at element 8*i of the flattened [rows, cols] array
    for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < tasks;
         i += (int64_t)gridDim.x * kQuantThreads) {
        float f[8];
        load8(x + i * 8, f);
        float amax = group_amax4(f);
        int e = e4m3_block_exp(amax);
        float inv = exp2_neg(e);
        uint32_t lo = e4m3_pack4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
        uint32_t hi = e4m3_pack4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
        *reinterpret_cast<uint2*>(q + i * 8) = make_uint2(lo, hi);
        if ((i & 3) == 0) sf[i >> 2] = (uint8_t)(e + 127);
    }
}

__global__ __launch_bounds__(kQuantThreads) void pack_weights_kernel(const uint16_t* __restrict__ w,
                                                                     int64_t tasks,
                                                                     uint8_t* __restrict__ q,
                                                                     uint8_t* __restrict__ sf) {
    for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < tasks;
         i += (int64_t)gridDim.x * kQuantThreads) {
        float f[8];
        load8(w + i * 8, f);
        float amax = group_amax4(f);
        int e = e2m1_block_exp(amax);
        float inv = exp2_neg(e);
        uint32_t packed = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) packed |= e2m1_encode(f[j] * inv) << (4 * j);
        reinterpret_cast<uint32_t*>(q)[i] = packed;
        if ((i & 3) == 0) sf[i >> 2] = (uint8_t)(e + 127);
    }
}

// Per-row scales [mats][rows][cols/32] to K-step major [mats][cols/128][rows][4]:
// thread i moves the 4 bytes of one (matrix, K step, row), rows fastest.
__global__ __launch_bounds__(kQuantThreads) void scales_kmajor_kernel(const uint8_t* __restrict__ sf,
                                                                      int64_t tasks, int rows,
                                                                      int steps,
                                                                      uint8_t* __restrict__ out) {
    for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < tasks;
         i += (int64_t)gridDim.x * kQuantThreads) {
        const int64_t r = i % rows, ms = i / rows;
        const int64_t step = ms % steps, mat = ms / steps;
        const uint32_t v = *reinterpret_cast<const uint32_t*>(sf + ((mat * rows + r) * steps + step) * 4);
        reinterpret_cast<uint32_t*>(out)[i] = v;
    }
}

static unsigned grid_for(int64_t tasks) {
    int64_t blocks = (tasks + kQuantThreads - 1) / kQuantThreads;
    return (unsigned)std::min<int64_t>(std::max<int64_t>(blocks, 1), 65536);
}

hipError_t launch_quant_act(const uint16_t* x, int64_t rows, int cols, uint8_t* q, uint8_t* sf,
                            hipStream_t s) {
    int64_t tasks = rows * (cols / 8);
    if (tasks == 0) return hipSuccess;
    hipLaunchKernelGGL(quant_act_kernel, dim3(grid_for(tasks)), dim3(kQuantThreads), 0, s, x,
                       tasks, cols, q, sf);
    return hipGetLastError();
}

hipError_t launch_pack_weights(const uint16_t* w, int64_t rows, int cols, uint8_t* q, uint8_t* sf,
                               hipStream_t s) {
    int64_t tasks = rows * (cols / 8);
    if (tasks == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_weights_kernel, dim3(grid_for(tasks)), dim3(kQuantThreads), 0, s, w,
                       tasks, q, sf);
    return hipGetLastError();
}

}  // namespace moe

namespace moe {

// Packed FP4 codes [mats][rows][cols/2] in canonical row order -> the staged
// layout: thread i writes the 16-byte piece i of the output (matrix, group g,
// K step ks, row c of the group, piece q of its 64 bytes) from row
// staged_w*_row(g, c) of the same matrix.  Writes are contiguous, reads are
// 16-byte pieces of rows.
template <bool kW13>
__global__ __launch_bounds__(kQuantThreads) void stage_weights_kernel(const uint8_t* __restrict__ w,
                                                                      int64_t tasks, int rows, int cols,
                                                                      uint8_t* __restrict__ out) {
    const int nk = cols / 128;
    const int64_t per_mat = (int64_t)rows * nk * 4;     // 16-byte pieces of one matrix
    for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < tasks;
         i += (int64_t)gridDim.x * kQuantThreads) {
        const int64_t mat = i / per_mat;
        const int64_t r = i - mat * per_mat;
        const int q = (int)(r & 3), c = (int)((r >> 2) & 15);
        const int64_t blk = r >> 6;                        // g * nk + ks
        const int g = (int)(blk / nk), ks = (int)(blk - (int64_t)g * nk);
        const int row = kW13 ? staged_w13_row(g, c, rows / 2) : staged_w2_row(g, c);
        const uint8_t* src = w + (mat * rows + row) * (int64_t)(cols / 2) + ks * 64 + q * 16;
        reinterpret_cast<uint4*>(out)[i] = *reinterpret_cast<const uint4*>(src);
    }
}

hipError_t launch_stage_weights(const uint8_t* w, int64_t mats, int rows, int cols, bool w13, uint8_t* out,
                                hipStream_t s) {
    const int64_t tasks = mats * rows * (int64_t)(cols / 32);
    if (tasks == 0) return hipSuccess;
    if (w13)
        hipLaunchKernelGGL(stage_weights_kernel<true>, dim3(grid_for(tasks)), dim3(kQuantThreads), 0, s, w,
                           tasks, rows, cols, out);
    else
        hipLaunchKernelGGL(stage_weights_kernel<false>, dim3(grid_for(tasks)), dim3(kQuantThreads), 0, s, w,
                           tasks, rows, cols, out);
    return hipGetLastError();
}

hipError_t launch_scales_kmajor(const uint8_t* sf, int64_t mats, int rows, int cols, uint8_t* out,
                                hipStream_t s) {
    const int steps = cols / 128;
    const int64_t tasks = mats * rows * (int64_t)steps;
    if (tasks == 0) return hipSuccess;
    hipLaunchKernelGGL(scales_kmajor_kernel, dim3(grid_for(tasks)), dim3(kQuantThreads), 0, s, sf,
                       tasks, rows, steps, out);
    return hipGetLastError();
}
}  // namespace moe
