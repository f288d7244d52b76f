// Accuracy of the gfx950 matrix instructions the layer uses, against exact sums:
// one wave multiplies random 16 x 128 and 128 x 16 operands of E4M3 (and E2M1)
// codes with unit scales, and the host compares every element with the exact
// dot product.  Prints, per instruction, max |error| / sum_k |a_k b_k| over
// 200 random tiles; the tests take these as the per-instruction accumulation
// error of the parity bounds.
//   fp8xfp4   v_mfma_scale_f32_16x16x128_f8f6f4, A E4M3, B E2M1 (the main path)
//   fp8xfp8   the same instruction with both operands E4M3
//   bf16      four v_mfma_f32_16x16x32_bf16 over the same E4M3 values widened to
//             BF16 (the block-FP8 weight path)
// Buffers are fixed (2 KiB operands, 256 results); one wave of 64 lanes.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <random>
#include <vector>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// operand of lane l for row (column) l % 16: K [16 g, 16 g + 16) and [64 + 16 g, ...), g = l / 16
__device__ v8i fp8_operand(const unsigned char* row, int g) {
    v8i v;
    for (int k = 0; k < 4; ++k) v[k] = *(const int*)(row + 16 * g + 4 * k);
    for (int k = 0; k < 4; ++k) v[4 + k] = *(const int*)(row + 64 + 16 * g + 4 * k);
    return v;
}

// mode 0: E4M3 x E2M1; 1: E4M3 x E4M3; 2: BF16 from E4M3
__global__ void tile_kernel(const unsigned char* A, const unsigned char* B, float* D, int mode) {
    const int l = threadIdx.x, g = l / 16, r = l % 16;
    const v8i a = fp8_operand(A + r * 128, g);
    v4f d = {0.f, 0.f, 0.f, 0.f};
    if (mode == 0) {
        v8i b = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int k = 0; k < 4; ++k) b[k] = *(const int*)(B + r * 64 + 16 * g + 4 * k);   // 32 E2M1 codes
        d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, d, 0, 4, 0, 127, 0, 127);
    } else {
        const v8i b = fp8_operand(B + r * 128, g);
        if (mode == 1) {
            d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, d, 0, 0, 0, 127, 0, 127);
        } else {
            for (int s = 0; s < 4; ++s) {
                v8bf x, y;
                for (int h = 0; h < 2; ++h) {
                    const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a[2 * s + h], 1.0f, false);
                    const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(a[2 * s + h], 1.0f, true);
                    const v2bf q0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b[2 * s + h], 1.0f, false);
                    const v2bf q1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b[2 * s + h], 1.0f, true);
                    x[4 * h] = p0[0]; x[4 * h + 1] = p0[1]; x[4 * h + 2] = p1[0]; x[4 * h + 3] = p1[1];
                    y[4 * h] = q0[0]; y[4 * h + 1] = q0[1]; y[4 * h + 2] = q1[0]; y[4 * h + 3] = q1[1];
                }
                d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, d, 0, 0, 0);
            }
        }
    }
    for (int i = 0; i < 4; ++i) D[(4 * g + i) * 16 + r] = d[i];
}

static double e4m3(unsigned c) {
    const int e = (c >> 3) & 15, m = c & 7;
    const double v = e ? (1 + m / 8.0) * std::ldexp(1.0, e - 7) : (m / 8.0) * std::ldexp(1.0, -6);
    return (c & 0x80) ? -v : v;
}
static double e2m1(unsigned c) {
    static const double mag[8] = {0, 0.5, 1, 1.5, 2, 3, 4, 6};
    return (c & 8) ? -mag[c & 7] : mag[c & 7];
}

int main() {
    std::mt19937 rng(1);
    unsigned char *dA = nullptr, *dB = nullptr;
    float* dD = nullptr;
    if (hipMalloc(&dA, 2048) != hipSuccess || hipMalloc(&dB, 2048) != hipSuccess ||
        hipMalloc(&dD, 256 * sizeof(float)) != hipSuccess) {
        std::printf("hipMalloc failed\n");
        return 1;
    }
    const char* names[3] = {"fp8xfp4", "fp8xfp8", "bf16"};
    for (int mode = 0; mode < 3; ++mode) {
        double worst = 0.0;
        for (int trial = 0; trial < 1000; ++trial) {
            std::vector<unsigned char> A(2048), B(2048);
            // finite E4M3 codes (no NaN), exponent field >= 3: a wide but realistic spread
            auto code8 = [&]() {
                unsigned c;
                do c = rng() & 0xFF; while ((c & 0x7F) == 0x7F || ((c >> 3) & 15) < 3);
                return (unsigned char)c;
            };
            for (auto& v : A) v = code8();
            for (auto& v : B) v = mode == 0 ? (unsigned char)(rng() & 0xFF) : code8();
            if (hipMemcpy(dA, A.data(), 2048, hipMemcpyHostToDevice) != hipSuccess ||
                hipMemcpy(dB, B.data(), 2048, hipMemcpyHostToDevice) != hipSuccess)
                return 1;
            hipLaunchKernelGGL(tile_kernel, dim3(1), dim3(64), 0, 0, dA, dB, dD, mode);
            std::vector<float> D(256);
            if (hipMemcpy(D.data(), dD, 256 * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess) return 1;
            for (int i = 0; i < 16; ++i)
                for (int j = 0; j < 16; ++j) {
                    double s = 0.0, sa = 0.0;
                    for (int k = 0; k < 128; ++k) {
                        const double a = e4m3(A[i * 128 + k]);
                        const double b = mode == 0 ? e2m1((B[j * 64 + k / 2] >> (4 * (k & 1))) & 15)
                                                   : e4m3(B[j * 128 + k]);
                        s += a * b;           // exact: products and partial sums fit a double
                        sa += std::fabs(a * b);
                    }
                    worst = std::fmax(worst, std::fabs(D[i * 16 + j] - s) / sa);
                }
        }
        std::printf("%s max_err_over_sum_abs %.6e log2 %.2f\n", names[mode], worst, std::log2(worst + 1e-300));
    }
    return 0;
}
