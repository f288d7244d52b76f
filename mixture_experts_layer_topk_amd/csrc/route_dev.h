// Device functions of routing, counting-sort bucketisation and activation
// quantisation, shared by the routing launches and the one-kernel layer.
#pragma once

#include <rocprim/block/block_scan.hpp>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kMaxTopk = 16;
constexpr int kMaxExperts = kMaxExpertsCap;
constexpr int kSmallPairs = 1024;       // T * k up to which one workgroup buckets every pair

// Unsigned integer with the order of the float value (finite inputs); -0 and
// +0 map to the same integer, as they compare equal.
MOE_DEV uint32_t float_order(float v) {
    const uint32_t u = f2u(v == 0.0f ? 0.0f : v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One token's logits into the lanes (lane l: experts l, l + 64, ...).
template <int NPL>
MOE_DEV void load_logits(const float* __restrict__ lrow, int E, float (&v)[NPL]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? lrow[e] : 0.0f;
    }
}

// Top-k of one token's E logits with one wave.  Lane l owns experts
// l, l + 64, ...; NPL = values per lane.  Writes idx/w for the token.
//
// Every expert gets a unique 42-bit key, its float order in the high bits and
// 1023 - e in the low 10, so a larger key means a larger logit, or an equal
// logit and a smaller index (the tie rule).  The k-th largest key T is found
// bit by bit from the top: a candidate bit is kept when at least k keys are
// >= the candidate, each count a ballot and a popcount per value slot (no LDS
// traffic).  The k keys >= T are then compacted into LDS and each is ranked
// by the number of selected keys above it, which orders the slots.
template <int NPL>
MOE_DEV void route_token(const float (&v)[NPL], int E, int k, int score_fn, int renorm,
                         int32_t* __restrict__ idx_out, float* __restrict__ w_out,
                         float* sel_v, int* sel_i, uint64_t* sel_k, int* lds_idx) {
    const int lane = threadIdx.x & 63;
    uint64_t key[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = e < E ? ((uint64_t)float_order(v[i]) << 10) | (uint64_t)(1023 - e) : 0;
    }
    uint64_t T = 0;
    for (int bit = 41; bit >= 0; --bit) {
        const uint64_t c = T | (1ull << bit);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < NPL; ++i) cnt += __popcll(__ballot(key[i] >= c));
        if (cnt >= k) T = c;
    }
    // compact the k selected keys (and their logits) into LDS
    int base = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const bool sel = key[i] >= T;
        const uint64_t m = __ballot(sel);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (sel) {
            sel_k[base + below] = key[i];
            sel_v[base + below] = v[i];
        }
        base += __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint64_t x = 0;
    float xv = 0.0f;
    int rank = 0;
    if (lane < k) {
        x = sel_k[lane];
        xv = sel_v[lane];
        for (int j = 0; j < k; ++j) rank += sel_k[j] > x;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < k) {
        sel_v[rank] = xv;
        sel_i[rank] = 1023 - (int)(x & 1023);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // weights
    float lmax = sel_v[0];
    float s = 0.0f;
    if (lane < k) {
        float lv = sel_v[lane];
        s = score_fn == 0 ? expf(lv - lmax) : 1.0f / (1.0f + expf(-lv));
    }
    float denom = 1.0f;
    if (renorm) {
        denom = wave_sum(s);
    } else if (score_fn == 0) {
        float z = 0.0f;
#pragma unroll
        for (int i = 0; i < NPL; ++i)
            if (lane + 64 * i < E) z += expf(v[i] - lmax);
        denom = wave_sum(z);
    }
    if (lane < k) {
        idx_out[lane] = sel_i[lane];
        lds_idx[lane] = sel_i[lane];
        w_out[lane] = s / denom;
    }
}

// Quantise x rows [T, H]: task i covers 8 elements of the flattened array.
MOE_DEV void quant_rows(const RouteParams& p, int block, int nblocks) {
    const int64_t tasks = p.T * (p.H / 8);
    const int64_t stride = (int64_t)nblocks * kRouteThreads;
    constexpr int U = 4;
    for (int64_t i0 = (int64_t)block * kRouteThreads + threadIdx.x; i0 < tasks; i0 += U * stride) {
        uint4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t i = i0 + u * stride;
            raw[u] = i < tasks ? *reinterpret_cast<const uint4*>(p.x + i * 8) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t i = i0 + u * stride;
            float f[8];
            f[0] = bf16_to_f32(raw[u].x & 0xFFFFu); f[1] = bf16_to_f32(raw[u].x >> 16);
            f[2] = bf16_to_f32(raw[u].y & 0xFFFFu); f[3] = bf16_to_f32(raw[u].y >> 16);
            f[4] = bf16_to_f32(raw[u].z & 0xFFFFu); f[5] = bf16_to_f32(raw[u].z >> 16);
            f[6] = bf16_to_f32(raw[u].w & 0xFFFFu); f[7] = bf16_to_f32(raw[u].w >> 16);
            float amax = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) amax = fmaxf(amax, __builtin_fabsf(f[j]));
            // the 4 lanes of a group are consecutive and share the predicate i < tasks
            amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
            amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
            if (i < tasks) {
                int e = e4m3_block_exp(amax);
                float inv = exp2_neg(e);
                uint32_t lo = e4m3_pack4(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv);
                uint32_t hi = e4m3_pack4(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv);
                *reinterpret_cast<uint2*>(p.xq + i * 8) = make_uint2(lo, hi);
                if ((i & 3) == 0) {
                    // scales K-step major: xsf[g / 4][t][g % 4] for group g of token t
                    const int64_t G = i >> 2, gpr = p.H / kGroup;
                    const int64_t t = G / gpr, g = G - t * gpr;
                    p.xsf[(g >> 2) * (p.T * 4) + t * 4 + (g & 3)] = (uint8_t)(e + 127);
                }
            }
        }
    }
}

// The tokens [t0, t0 + ntok) of this wave: i = wave, wave + kRouteWaves, ...
template <int NPL>
MOE_DEV void route_tokens(const RouteParams& p, int64_t t0, int ntok, int* pair_exp, float* sel_v,
                          int* sel_i, uint64_t* sel_k) {
    const int k = p.topk;
    int i = threadIdx.x >> 6;
    if (i >= ntok) return;
    float v[NPL];
    for (; i < ntok; i += kRouteWaves) {
        const int64_t t = t0 + i;
        load_logits<NPL>(p.logits + t * p.E, p.E, v);
        route_token<NPL>(v, p.E, k, p.score_fn, p.renorm, p.idx_out + t * k, p.w_out + t * k, sel_v,
                         sel_i, sel_k, pair_exp + i * k);
    }
}

// Route tokens [t0, t0 + ntok) (one wave per token) or take the caller's ids;
// pair i = (t - t0) * k + j of the chunk gets its expert in pair_exp[i].
MOE_DEV void route_chunk(const RouteParams& p, int64_t t0, int ntok, int npl, int* pair_exp,
                         float (*sel_v)[kMaxTopk], int (*sel_i)[kMaxTopk],
                         uint64_t (*sel_k)[kMaxTopk]) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int k = p.topk;
    if (p.logits) {
        if (npl <= 1) route_tokens<1>(p, t0, ntok, pair_exp, sel_v[wave], sel_i[wave], sel_k[wave]);
        else if (npl <= 2) route_tokens<2>(p, t0, ntok, pair_exp, sel_v[wave], sel_i[wave], sel_k[wave]);
        else if (npl <= 4) route_tokens<4>(p, t0, ntok, pair_exp, sel_v[wave], sel_i[wave], sel_k[wave]);
        else if (npl <= 8) route_tokens<8>(p, t0, ntok, pair_exp, sel_v[wave], sel_i[wave], sel_k[wave]);
        else route_tokens<16>(p, t0, ntok, pair_exp, sel_v[wave], sel_i[wave], sel_k[wave]);
    } else {
        for (int i = tid; i < ntok * k; i += kRouteThreads) {
            int e = p.idx_in[t0 * k + i];
            pair_exp[i] = e;
            if (p.idx_in != p.idx_out) {
                p.idx_out[t0 * k + i] = e;
                p.w_out[t0 * k + i] = p.w_in[t0 * k + i];
            }
        }
    }
}

// Routing and counting of one chunk of kRouteTokensPerBlock tokens.
MOE_DEV void route_count_block(const RouteParams& p, int npl) {
    __shared__ int hist[kMaxExperts];
    __shared__ int base[kMaxExperts];
    __shared__ float sel_v[kRouteWaves][kMaxTopk];
    __shared__ int sel_i[kRouteWaves][kMaxTopk];
    __shared__ uint64_t sel_k[kRouteWaves][kMaxTopk];
    __shared__ int pair_rank[kRouteTokensPerBlock * kMaxTopk];
    __shared__ int pair_exp[kRouteTokensPerBlock * kMaxTopk];   // expert of pair i of this block

    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * kRouteTokensPerBlock;
    const int ntok = (int)min<int64_t>(kRouteTokensPerBlock, p.T - t0);
    const int k = p.topk;

    for (int e = tid; e < p.E; e += kRouteThreads) hist[e] = 0;
    // 1. routing (one wave per token) or caller's ids
    route_chunk(p, t0, ntok, npl, pair_exp, sel_v, sel_i, sel_k);
    __syncthreads();

    // 2. count: LDS histogram; the LDS atomic's return is the pair's rank here
    const int npairs = ntok * k;
    for (int i = tid; i < npairs; i += kRouteThreads) {
        int e = pair_exp[i];
        pair_rank[i] = (e >= 0 && e < p.E) ? atomicAdd(&hist[e], 1) : -1;
    }
    __syncthreads();
    for (int e = tid; e < p.E; e += kRouteThreads) {
        int c = hist[e];
        base[e] = c ? atomicAdd(&p.cnt[e], c) : 0;
    }
    __syncthreads();
    for (int i = tid; i < npairs; i += kRouteThreads) {
        int e = pair_exp[i];
        p.slot_in_e[t0 * k + i] = pair_rank[i] >= 0 ? base[e] + pair_rank[i] : -1;
    }
}

using BlockScan = rocprim::block_scan<int, kRouteThreads>;

// Exclusive scan of n <= 1024 ints in LDS by a 256-thread block: out[0..n]
// (out[n] = total).  Ends with a barrier, so st may be reused right away.
MOE_DEV void block_exclusive_scan(const int* in, int* out, int n, BlockScan::storage_type& st) {
    const int tid = threadIdx.x;
    int v[4], o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = tid * 4 + j;
        v[j] = i < n ? in[i] : 0;
    }
    int total;
    BlockScan().exclusive_scan(v, o, 0, total, st);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = tid * 4 + j;
        if (i < n) out[i] = o[j];
    }
    if (tid == 0) out[n] = total;
    __syncthreads();
}

// Per-expert tables of the GEMMs from the final counts cnt[E] and their
// exclusive scan off[E + 1]: counts, offsets, then m-tiles of p.bm rows (tiled
// GEMMs) and sub-tiles of kSubRows rows (narrow GEMMs): per expert
// ceil(count / rows) tiles, prefix-summed, one record per tile {expert, first
// position, rows}, zero records up to the table's size.  Workgroup `part` of
// `nparts` (each holding cnt and off) writes every nparts-th stretch of
// records; part 0 also writes the per-expert arrays.
MOE_DEV void write_tables(const ScatterParams& p, const int* cnt, const int* off, int* tiles,
                          int* toff, BlockScan::storage_type& tmp, int part, int nparts) {
    const int tid = threadIdx.x;
    if (part == 0) {
        for (int e = tid; e < p.E; e += kRouteThreads) p.counts_out[e] = cnt[e];
        for (int e = tid; e <= p.E; e += kRouteThreads) p.offsets_out[e] = off[e];
        // the one-launch GEMMs' per-m-tile counters and status start at zero
        for (int m = tid; m < p.max_mtiles; m += kRouteThreads) p.ready[m] = 0;
        if (tid == 0) *p.status = 0;
    }
    for (int pass = 0; pass < 2; ++pass) {
        const int rows = pass == 0 ? p.bm : kSubRows;
        const int cap = pass == 0 ? p.max_mtiles : p.max_subs;
        int4* rec = pass == 0 ? p.mtile_rec : p.sub_rec;
        for (int e = tid; e < p.E; e += kRouteThreads) tiles[e] = ceil_div(cnt[e], rows);
        __syncthreads();
        block_exclusive_scan(tiles, toff, p.E, tmp);
        const int ntiles = toff[p.E];
        for (int m = part * kRouteThreads + tid; m < cap; m += nparts * kRouteThreads) {
            int4 r = make_int4(0, 0, 0, 0);
            if (m < ntiles) {
                int lo = 0, hi = p.E - 1;          // expert e with toff[e] <= m < toff[e+1]
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (toff[mid] <= m) lo = mid; else hi = mid - 1;
                }
                const int r0 = (m - toff[lo]) * rows;
                r = make_int4(lo, off[lo] + r0, min(rows, cnt[lo] - r0), 0);
                if (pass == 0) p.mtile_e[m] = lo;
            }
            rec[m] = r;
        }
        if (part == 0) {
            if (pass == 0) {
                for (int e = tid; e <= p.E; e += kRouteThreads) p.mtile_off[e] = toff[e];
            } else if (tid == 0) {
                *p.nsub = ntiles;
            }
        }
        __syncthreads();                          // tiles and toff are reused
    }
}


// Few pairs (T * k <= kSmallPairs), one workgroup: route every token, count
// the pairs in an LDS histogram whose atomic returns each pair's rank inside
// its expert, scan the counts, scatter the pairs and write the tables, with no
// global counters ("05.10 Counting Sort / Bucketization" 2.1-2.3 inside one
// workgroup).
MOE_DEV void bucket_small(const RouteParams& rp, const ScatterParams& sp, int npl) {
    __shared__ int hist[kMaxExperts];
    __shared__ int off[kMaxExperts + 1];
    __shared__ int tiles[kMaxExperts];
    __shared__ int toff[kMaxExperts + 1];
    __shared__ BlockScan::storage_type tmp;
    __shared__ float sel_v[kRouteWaves][kMaxTopk];
    __shared__ int sel_i[kRouteWaves][kMaxTopk];
    __shared__ uint64_t sel_k[kRouteWaves][kMaxTopk];
    __shared__ int pair_exp[kSmallPairs];
    __shared__ int pair_rank[kSmallPairs];
    const int tid = threadIdx.x;
    const int k = rp.topk;
    const int npairs = (int)rp.T * k;
    for (int e = tid; e < rp.E; e += kRouteThreads) hist[e] = 0;
    route_chunk(rp, 0, (int)rp.T, npl, pair_exp, sel_v, sel_i, sel_k);
    __syncthreads();
    for (int i = tid; i < npairs; i += kRouteThreads) {
        const int e = pair_exp[i];
        pair_rank[i] = (e >= 0 && e < rp.E) ? atomicAdd(&hist[e], 1) : -1;
    }
    __syncthreads();
    block_exclusive_scan(hist, off, rp.E, tmp);
    for (int i = tid; i < npairs; i += kRouteThreads) {
        const int e = pair_exp[i];
        if (pair_rank[i] >= 0) {
            const int pos = off[e] + pair_rank[i];
            sp.slot_src[pos] = i;
            sp.slot_of[i] = pos;
        } else {
            sp.slot_of[i] = -1;
        }
    }
    write_tables(sp, hist, off, tiles, toff, tmp, 0, 1);
}

}  // namespace moe
