// Device primitives shared by the layer's kernels (gfx950).
//
// Number formats (pages: "MegaMoE" study notes, "Dispatch阶段" and
// "Expert矩阵权重量化"; read as OCP MX v1.0):
//   E4M3 ("FN"): bias 7, largest finite 448, no infinities, subnormals m*2^-9
//   E2M1:        magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}
//   UE8M0:       2^(b - 127)
// A group of 32 values shares the smallest power-of-two scale 2^e with
// max|v| <= Q * 2^e (Q = 448 or 6); codes are v * 2^-e rounded to the nearest
// representable value, ties to the even code, sign kept.  The exponent is read
// off the float32 bit fields of max|v|: with max|v| = m * 2^E, m in [1, 2),
// e = E - 8 + [m > 1.75] for E4M3 and e = E - 2 + [m > 1.5] for E2M1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

#define MOE_DEV static __device__ __forceinline__

namespace moe {

constexpr int kGroup = 32;          // elements per UE8M0 scale
constexpr int kFmtFp8 = 0;          // scaled-MFMA format selector: FP8 E4M3
constexpr int kFmtFp4 = 4;          // scaled-MFMA format selector: FP4 E2M1

MOE_DEV uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
MOE_DEV float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

MOE_DEV float bf16_to_f32(uint32_t b) { return u2f(b << 16); }

// float32 -> BF16, nearest even (inputs are finite).
MOE_DEV uint32_t f32_to_bf16(float f) {
    uint32_t u = f2u(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two floats to BF16, round to nearest even, packed lo | hi << 16 (one
// v_cvt_pk_bf16_f32 on gfx950; the same result as f32_to_bf16 on finite values).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// Block exponent e (clamped to [-127, 127]) for a group whose largest
// magnitude is amax (finite, >= 0).  kMantThresh is the mantissa field of
// Q's significand: 0x600000 (1.75, E4M3) or 0x400000 (1.5, E2M1); kShift is
// log2 of Q's binade (8 for 448, 2 for 6).
template <uint32_t kMantThresh, int kShift>
MOE_DEV int block_exp(float amax) {
    // selects rather than early returns: no divergent branches in the epilogues
    const uint32_t a = f2u(amax) & 0x7FFFFFFFu;
    const int biased = (int)(a >> 23);
    int e = biased - 127 - kShift + ((a & 0x7FFFFFu) > kMantThresh ? 1 : 0);
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    // zero: 0; a float32 subnormal lies below the E8M0 range: -127
    return biased == 0 ? (a == 0 ? 0 : -127) : e;
}
MOE_DEV int e4m3_block_exp(float amax) { return block_exp<0x600000u, 8>(amax); }
MOE_DEV int e2m1_block_exp(float amax) { return block_exp<0x400000u, 2>(amax); }

// 2^-e as a float for e in [-127, 127] (2^-127 is a float32 subnormal).
MOE_DEV float exp2_neg(int e) { return __builtin_ldexpf(1.0f, -e); }

// *p = v, device-coherent when kCoh (a write-through store that other XCDs'
// loads see once it has completed; 16-byte values as four dword stores), for
// data handed to other workgroups inside the same launch.
template <bool kCoh, class T>
MOE_DEV void put(T* p, T v) {
    if constexpr (!kCoh) {
        *p = v;
    } else if constexpr (sizeof(T) == 16) {
        const uint4 u = __builtin_bit_cast(uint4, v);
        uint32_t* q = reinterpret_cast<uint32_t*>(p);
        __hip_atomic_store(q + 0, u.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(q + 1, u.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(q + 2, u.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(q + 3, u.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        static_assert(sizeof(T) == 1 || sizeof(T) == 2 || sizeof(T) == 4 || sizeof(T) == 8, "store size");
        using U = std::conditional_t<sizeof(T) == 1, uint8_t,
                  std::conditional_t<sizeof(T) == 2, uint16_t, std::conditional_t<sizeof(T) == 4, uint32_t, uint64_t>>>;
        __hip_atomic_store(reinterpret_cast<U*>(p), __builtin_bit_cast(U, v), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Two float32 values to E4M3 codes in the low 16 bits (first value in the low
// byte), nearest even, by the gfx950 conversion instruction.  Inputs must be
// finite with |x| <= 448 (the block scale guarantees it); on that range the
// instruction rounds exactly as the format definition requires, which the
// quantiser parity tests check code by code against the CPU reference.
MOE_DEV uint32_t e4m3_pack2(float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}
// Four values to one dword of E4M3 codes (first value in the low byte).
MOE_DEV uint32_t e4m3_pack4(float a, float b, float c, float d) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
}

// |x| <= 6 expected; larger magnitudes clamp to 6.  Nearest, ties to the even
// code: the code is the number of decision thresholds below |x|, a threshold
// being the midpoint between neighbouring magnitudes, counted at equality when
// the upper neighbour has the even code.
MOE_DEV uint32_t e2m1_encode(float x) {
    uint32_t sign = (f2u(x) >> 28) & 0x8u;
    float a = __builtin_fabsf(x);
    uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
                 (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
    return sign | c;
}

MOE_DEV int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Workgroup barrier that orders LDS accesses only: global memory operations
// issued before it need not have completed (for phases in which no wave reads
// back what another wrote to global memory).
MOE_DEV void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Largest x over each row of 16 lanes of a fully active wave, in every lane of
// the row: DPP butterflies (lane pairs 1 apart, 2 apart, then the mirrored
// halves of 8 and of 16).
MOE_DEV uint32_t row_max_u32(uint32_t x) {
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false));
    return max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false));
}

// Wave-level reductions over 64 lanes.
MOE_DEV float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
MOE_DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

}  // namespace moe
