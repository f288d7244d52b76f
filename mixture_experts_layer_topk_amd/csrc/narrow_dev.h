// Device code of the narrow (weight-streaming) grouped GEMMs, shared by their
// launches and the one-kernel layer.
#pragma once

#include "common.h"
#include "kernels.h"
#include "mfma.h"

namespace moe {

constexpr int kNarrowWaves = 4;
constexpr int kNarrowThreads = 64 * kNarrowWaves;
constexpr int kNT = 4;                  // 16-column MFMA tiles per unit
constexpr int kBatch = kNarrowThreads / kSubRows;   // unit headers fetched per batch
constexpr int kNarrowBlocksPerCU = 2;
constexpr int kNarrowSpinLimit = 1 << 14;   // polls of a ready counter before giving up (~20 ms)

template <bool kG1, bool kW8 = false>
struct NarrowCfg {
    static constexpr int kCols = kG1 ? 32 : 64;         // I columns (GEMM1) or H columns
    // K steps per item and wave, items in flight per wave.  GEMM1 loads two
    // K steps per item, so the two 64-byte halves of a weight row's 128-byte
    // line are requested together (6% faster at the decode shape); GEMM2's
    // K = I is too short per wave for that (each wave has I / 512 steps).
    // FP8 weights (kW8) fill a 128-byte line per K step and take twice the
    // registers per item: one K step per item, three items in flight.
    static constexpr int KC = kW8 ? 1 : (kG1 ? 2 : 1);
    static constexpr int NBUF = kW8 ? 3 : (kG1 ? 2 : 4);
};

// LDS of the narrow GEMMs.  One block for every instance of narrow_gemm in a
// kernel: GEMM1 and GEMM2 running one after the other in one launch share it
// (static shared arrays inside the template would be allocated per instance,
// doubling the LDS of such a kernel and halving its occupancy).
struct NarrowLds {
    v4f red2[2][kNarrowWaves][kNT][64];                 // partial accumulators, two buffers
    int hdr[kBatch][4];                                 // expert, first position, rows, chunk
    int arow[kBatch][kSubRows];                         // activation row of each unit row
    __attribute__((aligned(16))) float w[kBatch][kSubRows];    // routing weight (GEMM1)
    __attribute__((aligned(16))) float amax[2][16];
};
__device__ __forceinline__ NarrowLds& narrow_lds() {
    __shared__ NarrowLds s;
    return s;
}

template <int KC, bool kW8>
struct NarrowBuf {
    v4i b[KC][kNT];             // FP4: the lane's 16 bytes; FP8: its first 16 of 32
    v4i b2[kW8 ? KC : 1][kNT];  // FP8: the lane's second 16 bytes (K + 64)
    uint32_t sb[KC][kNT];       // FP4: the step's 4 UE8M0 bytes; FP8: the block's float32 scale
    v4i alo[KC], ahi[KC];
    uint32_t sa[KC];            // MXFP8: the step's 4 UE8M0 bytes; block FP8: the float32 scale
};

// The GEMM of workgroup `bid` of `G` (any G >= 1: the units are dealt out
// persistently).
//
// kCoh: GEMM1 and GEMM2 run in one launch (the GEMM1 part, then the GEMM2
// part, in every workgroup).  The XCDs' L2 caches are not coherent within a
// launch, so GEMM1 stores h with device-coherent stores, waits for them to
// complete and then adds each finished unit to ready[sub-tile]; a GEMM2 batch
// issues its first weight loads, waits until ready[] counts every GEMM1 unit
// of each of its sub-tiles and then reads h with device-coherent loads.
// GEMM2 stores o device-coherently too (the one-kernel layer's combine reads
// it in the same launch).
//
// kW8: block-FP8 weights (E4M3 codes [E, N, K], one float32 scale per 128 x 128
// block) and activations with one float32 scale per row per 128 K ("MonoMoe
// kernel — design", fixed-shape paragraph).  Each K step's 16 x 16 partial
// (mfma_bf16_block: the FP8 values widened to BF16) is added with the row's
// activation scale times the block's weight scale.  GEMM1 then stores h = silu(g) * up * w in
// float32 (p.hf32), to be quantised per 128 columns by the next launch (a
// group spans four units of different workgroups).
//
// kST: FP4 codes in the staged layout (16-row groups, one KiB per group and K
// step).  A unit is then half of a staged column block: GEMM1 unit nc (32 I
// columns) is rows 8 (nc & 1) .. + 7 of groups 8 (nc >> 1) .. + 7, GEMM2 unit
// nc (64 H columns) the same rows of its block's groups, and MFMA tile t takes
// groups 2t and 2t + 1 (lanes l16 < 8 and >= 8), so every tile's loads are two
// contiguous 512-byte runs per K step.  In GEMM1 a tile then holds gate (group
// 2t) and up (group 2t + 1) of the I columns 32 nc + 4 j + t, j < 8.
template <bool kG1, bool kCoh = false, bool kW8 = false, bool kST = false>
MOE_DEV void narrow_gemm(const GemmParams& p, int bid, int G) {
    static_assert(!(kCoh && kW8), "block-FP8 weights run as separate launches");
    static_assert(!(kST && kW8), "the staged layout is one of packed FP4 codes");
    using Cfg = NarrowCfg<kG1, kW8>;
    constexpr int KC = Cfg::KC, NBUF = Cfg::NBUF;
    // partial accumulators, two buffers: unit j writes buffer j % 2, whose
    // previous readers (unit j - 2) finished before unit j - 1's barrier
    NarrowLds& lds = narrow_lds();
    v4f (&s_red2)[2][kNarrowWaves][kNT][64] = lds.red2;
    int (&s_hdr)[kBatch][4] = lds.hdr;
    int (&s_arow)[kBatch][kSubRows] = lds.arow;
    float (&s_w)[kBatch][kSubRows] = lds.w;
    float (&s_amax)[2][16] = lds.amax;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int nch = (kG1 ? p.I : p.H) / Cfg::kCols;
    const int nunits = *p.nsub * nch;

    const int K = kG1 ? p.H : p.I;
    const int nk = K / kKStep;
    const int64_t R = p.T * p.topk;
    const int64_t wrows = kG1 ? 2 * (int64_t)p.I : p.H;  // weight rows of one expert
    const uint8_t* wq = kG1 ? p.w13 : p.w2;
    const uint8_t* wsf = kG1 ? p.w13sf : p.w2sf;
    const uint8_t* aq = kG1 ? p.xq : p.hq;
    const uint8_t* asf = kG1 ? p.xsf : p.hsf;
    const int64_t a_slab = 4 * (kG1 ? p.T : R);          // bytes per K step of activation scales
    // weight-scale byte strides per weight row and per K step (layout-dependent)
    const int64_t w_rs = kG1 ? p.w13sf_rs : p.w2sf_rs;
    const int64_t w_ks = kG1 ? p.w13sf_ks : p.w2sf_ks;
    const int spin_limit = p.spin_limit > 0 ? p.spin_limit : kNarrowSpinLimit;
    // this wave's K range; every wave runs nchunk items per unit
    const int kb = wave * nk / kNarrowWaves, ke = (wave + 1) * nk / kNarrowWaves;
    const int kr = (nk + kNarrowWaves - 1) / kNarrowWaves;
    const int nchunk = (kr + KC - 1) / KC;

    // staged layout: group and row of this lane's weight row in tile t of chunk nc
    auto sgroup = [&](int nc, int t) { return 8 * (nc >> 1) + 2 * t + (l16 >> 3); };
    const int srow_lo = l16 & 7;
    // weight row (= output column) of this lane in tile t of column chunk nc
    auto brow = [&](int nc, int t) -> int {
        if constexpr (kST) {
            const int g = sgroup(nc, t), c = 8 * (nc & 1) + srow_lo;
            return kG1 ? staged_w13_row(g, c, p.I) : staged_w2_row(g, c);
        }
        if (kG1) {
            const int icol = nc * Cfg::kCols + (t & 1) * 16 + l16;
            return w13_row(icol, t >> 1, p.I, p.w13_il);  // tiles 0, 1 gate; 2, 3 up
        }
        return nc * Cfg::kCols + 16 * t + l16;
    };

    for (int u0 = bid; u0 < nunits; u0 += kBatch * G) {
        const int nb = min(kBatch, (nunits - u0 + G - 1) / G);
        const int nitems = nb * nchunk;

        // ---- item q: unit q / nchunk, K steps kb + (q % nchunk) * KC + [0, KC)
        // Items past the end re-read the last one (cached) and K steps past the
        // wave's range re-read one inside it, so every path issues the same loads
        // and the compiler's counted waits keep the later buffers in flight.
        // Weights (expert e, column chunk nc) and activations are issued apart:
        // the first items' weights go out as soon as their expert is known,
        // before the unit headers (rows, routing weights) are resolved.
        auto issue_w = [&](NarrowBuf<KC, kW8>& bf, int q, int e, int nc) {
            q = min(q, nitems - 1);
            const int c = q % nchunk;
            constexpr int kRow = kW8 ? 1 : 2;             // elements per byte of a weight row
            const uint8_t* wq_e = wq + (int64_t)e * wrows * (K / kRow) + lg * 16;
            const uint8_t* wsf_e = wsf + (int64_t)e * wrows * (K / kGroup);
            // block-FP8 scales [E][N/128][K/128] float32
            const float* wsf8_e = reinterpret_cast<const float*>(wsf) + (int64_t)e * (wrows / 128) * nk;
#pragma unroll
            for (int jj = 0; jj < KC; ++jj) {
                const int ks = max(0, min(kb + c * KC + jj, min(ke, nk) - 1));
#pragma unroll
                for (int t = 0; t < kNT; ++t) {
                    const int br = brow(nc, t);
                    const uint8_t* row =
                        kST ? wq_e + ((int64_t)sgroup(nc, t) * nk + ks) * kStagedBlock + (8 * (nc & 1) + srow_lo) * 64
                            : wq_e + (int64_t)br * (K / kRow) + ks * (kKStep / kRow);
                    bf.b[jj][t] = *reinterpret_cast<const v4i*>(row);
                    if constexpr (kW8) {
                        bf.b2[jj][t] = *reinterpret_cast<const v4i*>(row + 64);
                        bf.sb[jj][t] = __builtin_bit_cast(uint32_t, wsf8_e[(br / 128) * nk + ks]);
                    } else {
                        bf.sb[jj][t] = *reinterpret_cast<const uint32_t*>(wsf_e + ks * w_ks + br * w_rs);
                    }
                }
            }
        };
        auto issue_a = [&](NarrowBuf<KC, kW8>& bf, int q) {
            q = min(q, nitems - 1);
            const int j = q / nchunk, c = q - j * nchunk;
            const int64_t arow = s_arow[j][l16];
            const uint8_t* ap = aq + arow * K + lg * 16;
            const uint8_t* asp = asf + arow * 4;
#pragma unroll
            for (int jj = 0; jj < KC; ++jj) {
                const int ks = max(0, min(kb + c * KC + jj, min(ke, nk) - 1));
                if constexpr (kCoh && !kG1) {
                    // h of this launch: device-coherent dword loads
                    auto ld = [](const uint8_t* q) {
                        return (int)__hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(q)),
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    };
                    const uint8_t* a0 = ap + ks * kKStep;
                    bf.alo[jj] = v4i{ld(a0), ld(a0 + 4), ld(a0 + 8), ld(a0 + 12)};
                    bf.ahi[jj] = v4i{ld(a0 + 64), ld(a0 + 68), ld(a0 + 72), ld(a0 + 76)};
                    bf.sa[jj] = (uint32_t)ld(asp + ks * a_slab);
                } else {
                    bf.alo[jj] = *reinterpret_cast<const v4i*>(ap + ks * kKStep);
                    bf.ahi[jj] = *reinterpret_cast<const v4i*>(ap + ks * kKStep + 64);
                    bf.sa[jj] = *reinterpret_cast<const uint32_t*>(asp + ks * a_slab);
                }
            }
        };
        auto issue = [&](NarrowBuf<KC, kW8>& bf, int q) {
            const int j = min(q, nitems - 1) / nchunk;
            issue_w(bf, q, s_hdr[j][0], s_hdr[j][3]);
            issue_a(bf, q);
        };

        // This thread's unit header (16 threads per unit) and the experts of the
        // first items are read before any weight load goes out, and so are the
        // unit rows' pair ids and routing weights (GEMM1): loads complete in
        // issue order, so anything issued after the weights would wait for them.
        const int hj = tid / kSubRows, hr = tid % kSubRows;
        const int hu = u0 + hj * G;
        int4 hrec = make_int4(0, 0, 1, 0);
        if (hu < nunits) hrec = p.sub_rec[hu / nch];    // {expert, first position, rows}
        int early_e[NBUF - 1];
#pragma unroll
        for (int q = 0; q < NBUF - 1; ++q)
            early_e[q] = p.sub_rec[(u0 + (min(q, nitems - 1) / nchunk) * G) / nch].x;
        const int hpos = hrec.y + min(hr, hrec.z - 1);
        int hsrc = 0;
        float hw = 0.0f;
        if (kG1 && hu < nunits) {
            hsrc = p.slot_src[hpos];
            hw = p.slot_w[hpos];
        }

        NarrowBuf<KC, kW8> buf[NBUF];
#pragma unroll
        for (int q = 0; q < NBUF - 1; ++q) {
            const int u = u0 + (min(q, nitems - 1) / nchunk) * G;
            issue_w(buf[q], q, early_e[q], u % nch);
        }

        // ---- headers of units u0 + j * G, j < kBatch, into LDS
        lds_barrier();                                  // the previous batch is done with LDS
        if (hu < nunits) {
            s_arow[hj][hr] = kG1 ? hsrc / p.topk : hpos;
            s_w[hj][hr] = hw;
            if (hr == 0) {
                s_hdr[hj][0] = hrec.x;
                s_hdr[hj][1] = hrec.y;
                s_hdr[hj][2] = hrec.z;
                s_hdr[hj][3] = hu % nch;
            }
        }
        lds_barrier();
        if constexpr (kCoh && !kG1) {
            // every GEMM1 unit of this batch's sub-tiles has stored its h columns
            if (tid == 0) {
                const int need = p.I / NarrowCfg<true>::kCols;
                for (int j = 0; j < nb; ++j) {
                    const int m = (u0 + j * G) / nch;
                    int n = 0;
                    while (__hip_atomic_load(p.ready + m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
                        __builtin_amdgcn_s_sleep(1);
                        if (++n >= spin_limit) {
                            __hip_atomic_store(p.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            break;
                        }
                    }
                }
            }
            __syncthreads();
        }

        v4f acc[kNT];
        auto epilogue = [&](int j) {
            const int p0 = s_hdr[j][1], valid = s_hdr[j][2], nc = s_hdr[j][3];
            v4f (&s_red)[kNarrowWaves][kNT][64] = s_red2[j & 1];
#pragma unroll
            for (int t = 0; t < kNT; ++t) s_red[wave][t][lane] = acc[t];
            __syncthreads();
            // lane holds rows 4 lg + i (i < 4), column l16 of a tile
            if (kG1) {
                // canonical: wave 0 takes I columns [c, c+16) (gate tile 0, up tile 2),
                // wave 1 [c+16, c+32) (tiles 1, 3); staged: wave w takes tiles 2w and
                // 2w + 1, lane l16 < 8 tile 2w, else 2w + 1, gate from the tile's
                // lane j = l16 & 7 and up from its lane 8 + j
                const int gt = kST ? 2 * wave + (l16 >> 3) : wave, ut = kST ? gt : 2 + wave;
                const int gl = kST ? 16 * lg + srow_lo : lane, ul = kST ? gl + 8 : lane;
                const int icol = kST ? 32 * nc + 4 * srow_lo + gt : nc * Cfg::kCols + wave * 16 + l16;
                float h[4] = {0.f, 0.f, 0.f, 0.f};
                if (wave < 2) {
                    v4f g = s_red[0][gt][gl], u = s_red[0][ut][ul];
#pragma unroll
                    for (int w = 1; w < kNarrowWaves; ++w) {
                        g += s_red[w][gt][gl];
                        u += s_red[w][ut][ul];
                    }
                    const v4f wr = *reinterpret_cast<const v4f*>(&s_w[j][4 * lg]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        h[i] = swiglu_w(g[i], u[i], wr[i]);
                        if constexpr (!kW8) {
                            // max |h| over the row's 16 columns (bit patterns of
                            // non-negative floats order like the values)
                            const uint32_t m = row_max_u32(f2u(h[i]) & 0x7FFFFFFFu);
                            if (l16 == 0) s_amax[wave][4 * lg + i] = u2f(m);
                        }
                    }
                }
                if constexpr (kW8) {
                    // h in float32; its 128-column groups are quantised by the next launch
                    if (wave < 2) {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (4 * lg + i < valid) p.hf32[(int64_t)(p0 + 4 * lg + i) * p.I + icol] = h[i];
                    }
                    return;
                }
                // an E4M3 group is the unit's 32 I columns: both waves' maxima
                __syncthreads();
                if (wave < 2) {
                    const v4f m0 = *reinterpret_cast<const v4f*>(&s_amax[0][4 * lg]);
                    const v4f m1 = *reinterpret_cast<const v4f*>(&s_amax[1][4 * lg]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 4 * lg + i;
                        const int ex = e4m3_block_exp(fmaxf(m0[i], m1[i]));
                        if (r < valid) {
                            const int64_t pos = p0 + r;
                            uint8_t* hq = p.hq + pos * p.I + icol;
                            const uint8_t code = (uint8_t)e4m3_pack2(h[i] * exp2_neg(ex), 0.0f);
                            uint8_t* hsf = p.hsf + (int64_t)(icol / (4 * kGroup)) * (R * 4) + pos * 4 +
                                           (icol / kGroup) % 4;
                            const bool sf = wave == 0 && l16 == 0;
                            if constexpr (kCoh) {
                                __hip_atomic_store(hq, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                                if (sf)
                                    __hip_atomic_store(hsf, (uint8_t)(ex + 127), __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
                            } else {
                                *hq = code;
                                if (sf) *hsf = (uint8_t)(ex + 127);
                            }
                        }
                    }
                }
            } else {
                v4f o = s_red[0][wave][lane];
#pragma unroll
                for (int w = 1; w < kNarrowWaves; ++w) o += s_red[w][wave][lane];
                const int col = brow(nc, wave);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * lg + i;
                    if (r < valid) put<kCoh>(p.o + (int64_t)(p0 + r) * p.H + col, (uint16_t)f32_to_bf16(o[i]));
                }
            }
        };
        auto consume = [&](const NarrowBuf<KC, kW8>& bf, int q) {
            const int j = q / nchunk, c = q - j * nchunk;
            if (c == 0) {
#pragma unroll
                for (int t = 0; t < kNT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int jj = 0; jj < KC; ++jj) {
                if (kb + c * KC + jj < ke) {
                    const v8i a = v8i{bf.alo[jj][0], bf.alo[jj][1], bf.alo[jj][2], bf.alo[jj][3],
                                      bf.ahi[jj][0], bf.ahi[jj][1], bf.ahi[jj][2], bf.ahi[jj][3]};
                    if constexpr (kW8) {
                        // scales of this lane's result rows 4 lg + i: row r's sits in lane r
                        const float sa_lane = __builtin_bit_cast(float, bf.sa[jj]);
                        float sa_r[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) sa_r[i] = __shfl(sa_lane, 4 * lg + i, 64);
                        v8bf abf[4];
                        fp8x32_to_bf16(a, abf);
#pragma unroll
                        for (int t = 0; t < kNT; ++t) {
                            const v8i b8 = v8i{bf.b[jj][t][0], bf.b[jj][t][1], bf.b[jj][t][2], bf.b[jj][t][3],
                                               bf.b2[jj][t][0], bf.b2[jj][t][1], bf.b2[jj][t][2],
                                               bf.b2[jj][t][3]};
                            v8bf bbf[4];
                            fp8x32_to_bf16(b8, bbf);
                            const v4f part = mfma_bf16_block(abf, bbf);
                            const float sw = __builtin_bit_cast(float, bf.sb[jj][t]);
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[t][i] = fmaf(part[i], sa_r[i] * sw, acc[t][i]);
                        }
                    } else {
                        // lane group lg supplies the scale of K group lg of the step
                        const int sa = (int)(bf.sa[jj] >> (8 * lg));
#pragma unroll
                        for (int t = 0; t < kNT; ++t)
                            acc[t] = mfma_fp8_fp4(a, bf.b[jj][t], acc[t], sa, (int)(bf.sb[jj][t] >> (8 * lg)));
                    }
                }
            }
            if (c == nchunk - 1) epilogue(j);
        };

#pragma unroll
        for (int q = 0; q < NBUF - 1; ++q) issue_a(buf[q], q);
        for (int q0 = 0; q0 < nitems; q0 += NBUF) {
#pragma unroll
            for (int b = 0; b < NBUF; ++b) {
                issue(buf[(b + NBUF - 1) % NBUF], q0 + b + NBUF - 1);
                if (q0 + b < nitems) consume(buf[b], q0 + b);
            }
        }
        if constexpr (kCoh && kG1) {
            // this batch's h stores have completed (vmcnt(0)); count its units in
            __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8) | (0 << 14));
            __syncthreads();
            if (hr == 0 && hu < nunits)
                __hip_atomic_fetch_add(p.ready + hu / nch, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}


}  // namespace moe
