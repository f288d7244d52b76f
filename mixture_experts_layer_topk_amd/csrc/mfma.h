// Arithmetic shared by the two grouped-GEMM kernels (the tiled one for many
// rows per expert and the narrow one for few): the same per-step scaled MFMA
// and the same epilogue arithmetic.  The tiled kernel accumulates every K step
// into one accumulator chain in increasing K order; the narrow kernel splits K
// into four ranges, one per wave, and adds the four partial sums in LDS, so the
// two agree within the FP32 summation-order tolerance, not bit for bit.
#pragma once

#include "common.h"

namespace moe {

constexpr int kKStep = 128;             // K per scaled MFMA (FP8 bytes of A per row)

// One 16 x 16 x 128 block-scaled product: A FP8 E4M3 (32 bytes per lane), B FP4
// E2M1 (16 bytes per lane), E8M0 scales in the low byte of sa / sb.
MOE_DEV v4f mfma_fp8_fp4(const v8i& a, const v4i& b, const v4f& c, int sa, int sb) {
    v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b8, c, kFmtFp8, kFmtFp4, 0, sa, 0,
                                                            sb);
}

// Block-FP8 weights: one 128-wide K block of a 16 x 16 tile, FP8 E4M3 A and B
// (32 bytes per lane each, in the 16 x 16 x 128 instruction's operand layout)
// widened to BF16 (exact: E4M3 has 3 mantissa bits) and multiplied by four
// 16 x 16 x 32 BF16 MFMAs into zero accumulators; the caller applies the two
// float32 block scales.  The FP8 instructions are not used here because they do
// not sum in FP32: on gfx950 a 16 x 16 x 128 FP8 x FP8 product errs by up to
// 2^-12.6 of sum |a b| over random E4M3 codes, the BF16 path by 2^-21.8.
// Instruction s takes bytes [8 s, 8 s + 8) of every lane's 32 (K elements
// 16 g + 8 s .. for s < 2, 64 + 16 g + 8 (s - 2) .. else); A and B use the same
// mapping, so the four instructions sum every K of the block exactly once.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
MOE_DEV void fp8x32_to_bf16(const v8i& v, v8bf (&out)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[2 * s], 1.0f, false);
        const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[2 * s], 1.0f, true);
        const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[2 * s + 1], 1.0f, false);
        const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[2 * s + 1], 1.0f, true);
        out[s] = v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
}
MOE_DEV v4f mfma_bf16_block(const v8bf (&a)[4], const v8bf (&b)[4]) {
    v4f c = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], b[s], c, 0, 0, 0);
    return c;
}

// silu(g) = g / (1 + e^-g), with the hardware exp2 and reciprocal (about one
// ulp each; a large negative g gives e^-g = inf and silu = -0).
MOE_DEV float silu(float g) {
    const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// Weight row of W13 that holds projection `up` (0: gate, 1: up) of I column
// icol.  Canonical layout: all gate rows, then all up rows ("MegaMoE" study
// notes, "原始权重布局").  Pre-interleaved (il != 0): groups of 8 gate rows, each
// followed by the up rows of the same 8 columns (the same page's gran = 8
// interleave).
MOE_DEV int w13_row(int icol, int up, int I, int il) {
    return il ? ((icol >> 3) << 4) + (up << 3) + (icol & 7) : up * I + icol;
}

// Staged FP4 weight layout: the packed codes of one expert's matrix (N rows of
// K E2M1 values, K / 2 bytes per row) regrouped so that every global->LDS load
// of the tiled GEMM reads one contiguous KiB.  Rows are taken in groups of 16;
// the 64 bytes of K step ks (128 values) of row c of group g sit at byte
// (g * K / 128 + ks) * 1024 + 64 c.  Group g = 8 b + nt holds the 16 rows that
// one MFMA column tile nt of the tiled kernel's wave slice b stages:
//   W13 (N = 2I, slices of 64 I columns): projection nt & 1 (0 gate, 1 up)
//        of I column 64 b + 4 c + nt / 2;
//   W2  (N = H, slices of 128 H columns): output column 128 b + 8 c + nt.
// The weight scales keep their own layout (canonical row order).
constexpr int kStagedRows = 16;         // rows per group
constexpr int kStagedBlock = 1024;      // bytes of one group for one K step
MOE_DEV int staged_w13_row(int g, int c, int I) { return (g & 1) * I + 64 * (g >> 3) + 4 * c + ((g & 7) >> 1); }
MOE_DEV int staged_w2_row(int g, int c) { return 128 * (g >> 3) + 8 * c + (g & 7); }

// GEMM1 epilogue value of one element: silu(gate) * up * routing weight.
MOE_DEV float swiglu_w(float g, float u, float w) { return silu(g) * u * w; }

}  // namespace moe
