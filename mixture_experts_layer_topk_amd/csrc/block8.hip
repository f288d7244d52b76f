// Quantisers of the block-FP8 weight variant ("MonoMoe kernel — design", the
// fixed-shape paragraph: block-FP8 128 x 128 weights; §1 phase 2: BF16 -> FP8
// with an activation scale).  A group is 128 consecutive elements of a row
// (activations) or a 128 x 128 block (weights); its float32 scale is
// s = max|v| / 448 (1 for an all-zero group), so its largest element maps to
// +-448, and each code is the E4M3 value nearest to v / s (both divisions
// correctly rounded float32, as the hipcc default compiles `/`), ties to even.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kB8Threads = 256;
constexpr int kB8Block = 128;

MOE_DEV float b8_scale(float amax) { return amax > 0.0f ? amax / 448.0f : 1.0f; }

// v / s rounded to float32, clamped to the E4M3 range (the quotient can exceed
// 448 by a float32 rounding; nearest-even maps it to 448 either way)
MOE_DEV float b8_div(float v, float s) { return fminf(fmaxf(v / s, -448.0f), 448.0f); }

// One 128-element group per 16 lanes (8 elements per lane): rows of BF16 or
// float32 values -> E4M3 codes [rows, cols] and float32 scales K-step major
// [cols/128][rows], the layout the narrow GEMMs read activation scales in.
template <bool kF32>
__global__ __launch_bounds__(kB8Threads) void quant_rows128_kernel(const void* __restrict__ src,
                                                                    int64_t rows, int cols,
                                                                    uint8_t* __restrict__ q,
                                                                    float* __restrict__ sf) {
    const int64_t tasks = rows * (cols / 8);
    // a wave covers 64 consecutive tasks (4 whole groups) and runs while any of
    // them is in range; lanes past the end take part in the reductions with zeros
    const int64_t limit = (tasks + 63) / 64 * 64;
    for (int64_t i = (int64_t)blockIdx.x * kB8Threads + threadIdx.x; i < limit;
         i += (int64_t)gridDim.x * kB8Threads) {
        const bool in = i < tasks;
        float f[8];
        if (kF32) {
            const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + (in ? i : 0) * 8);
            const float4 a = p[0], b = p[1];
            f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
        } else {
            const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + (in ? i : 0) * 8);
            f[0] = bf16_to_f32(raw.x & 0xFFFFu); f[1] = bf16_to_f32(raw.x >> 16);
            f[2] = bf16_to_f32(raw.y & 0xFFFFu); f[3] = bf16_to_f32(raw.y >> 16);
            f[4] = bf16_to_f32(raw.z & 0xFFFFu); f[5] = bf16_to_f32(raw.z >> 16);
            f[6] = bf16_to_f32(raw.w & 0xFFFFu); f[7] = bf16_to_f32(raw.w >> 16);
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, in ? __builtin_fabsf(f[j]) : 0.0f);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        if (in) {
            const float s = b8_scale(amax);
            const uint32_t lo = e4m3_pack4(b8_div(f[0], s), b8_div(f[1], s), b8_div(f[2], s), b8_div(f[3], s));
            const uint32_t hi = e4m3_pack4(b8_div(f[4], s), b8_div(f[5], s), b8_div(f[6], s), b8_div(f[7], s));
            *reinterpret_cast<uint2*>(q + i * 8) = make_uint2(lo, hi);
            if ((i & 15) == 0) {
                const int64_t G = i >> 4, gpr = cols / kB8Block;
                const int64_t r = G / gpr, g = G - r * gpr;
                sf[g * rows + r] = s;
            }
        }
    }
}

// One workgroup per 128 x 128 block of a [rows, cols] BF16 matrix: thread t
// covers row t / 2 and 64 columns.  Codes [rows, cols], scales
// [rows/128][cols/128] row-major.
__global__ __launch_bounds__(kB8Threads) void pack_block128_kernel(const uint16_t* __restrict__ w,
                                                                    int64_t rows, int cols,
                                                                    uint8_t* __restrict__ q,
                                                                    float* __restrict__ sf) {
    __shared__ float s_max[kB8Threads / 64];
    const int nbc = cols / kB8Block;
    const int64_t blk = blockIdx.x;
    const int64_t br = blk / nbc, bc = blk - br * nbc;
    const int t = threadIdx.x;
    const int64_t row = br * kB8Block + t / 2;
    const int64_t col = bc * kB8Block + (t & 1) * 64;
    const uint16_t* src = w + row * cols + col;
    float f[64];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint4 raw = reinterpret_cast<const uint4*>(src)[k];
        f[8 * k + 0] = bf16_to_f32(raw.x & 0xFFFFu); f[8 * k + 1] = bf16_to_f32(raw.x >> 16);
        f[8 * k + 2] = bf16_to_f32(raw.y & 0xFFFFu); f[8 * k + 3] = bf16_to_f32(raw.y >> 16);
        f[8 * k + 4] = bf16_to_f32(raw.z & 0xFFFFu); f[8 * k + 5] = bf16_to_f32(raw.z >> 16);
        f[8 * k + 6] = bf16_to_f32(raw.w & 0xFFFFu); f[8 * k + 7] = bf16_to_f32(raw.w >> 16);
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 64; ++j) amax = fmaxf(amax, __builtin_fabsf(f[j]));
    amax = wave_max(amax);
    if ((t & 63) == 0) s_max[t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    const float s = b8_scale(amax);
    uint8_t* dst = q + row * cols + col;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint4 v;
        v.x = e4m3_pack4(b8_div(f[16 * k + 0], s), b8_div(f[16 * k + 1], s), b8_div(f[16 * k + 2], s),
                         b8_div(f[16 * k + 3], s));
        v.y = e4m3_pack4(b8_div(f[16 * k + 4], s), b8_div(f[16 * k + 5], s), b8_div(f[16 * k + 6], s),
                         b8_div(f[16 * k + 7], s));
        v.z = e4m3_pack4(b8_div(f[16 * k + 8], s), b8_div(f[16 * k + 9], s), b8_div(f[16 * k + 10], s),
                         b8_div(f[16 * k + 11], s));
        v.w = e4m3_pack4(b8_div(f[16 * k + 12], s), b8_div(f[16 * k + 13], s), b8_div(f[16 * k + 14], s),
                         b8_div(f[16 * k + 15], s));
        reinterpret_cast<uint4*>(dst)[k] = v;
    }
    if (t == 0) sf[blk] = s;
}

hipError_t launch_quant_rows128(const void* src, bool f32_in, int64_t rows, int cols, uint8_t* q, float* sf,
                                hipStream_t s) {
    const int64_t tasks = rows * (cols / 8);
    if (tasks == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((tasks + kB8Threads - 1) / kB8Threads, 16384);
    if (f32_in)
        hipLaunchKernelGGL(quant_rows128_kernel<true>, dim3((unsigned)blocks), dim3(kB8Threads), 0, s, src, rows,
                           cols, q, sf);
    else
        hipLaunchKernelGGL(quant_rows128_kernel<false>, dim3((unsigned)blocks), dim3(kB8Threads), 0, s, src,
                           rows, cols, q, sf);
    return hipGetLastError();
}

hipError_t launch_pack_block128(const uint16_t* w, int64_t rows, int cols, uint8_t* q, float* sf,
                                hipStream_t s) {
    const int64_t blocks = (rows / kB8Block) * (cols / kB8Block);
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pack_block128_kernel, dim3((unsigned)blocks), dim3(kB8Threads), 0, s, w, rows, cols, q,
                       sf);
    return hipGetLastError();
}

}  // namespace moe
