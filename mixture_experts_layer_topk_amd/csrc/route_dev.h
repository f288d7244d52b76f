// Device functions of routing, counting-sort bucketisation and activation
// quantisation, shared by the routing launches and the one-kernel layer.
#pragma once

#include <rocprim/block/block_scan.hpp>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kRouteThreads = 256;
constexpr int kMaxTopk = 16;
constexpr int kMaxExperts = kMaxExpertsCap;
constexpr int kSmallPairs = 1024;       // T * k up to which one workgroup can bucket every pair
constexpr int kSmallThreads = 512;      // that workgroup's size: one wave per token up to 8 tokens
// The routing launch uses that one workgroup for at most this many tokens (4 per
// wave); beyond, its token-serial routing is slower than the two-launch path
// (measured: 12 against 16 us at 32 tokens, 19 against 16 us at 64)
constexpr int kSmallTokens = 32;

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

// Largest (smallest) of x over the 64 lanes of a fully active wave, in every
// lane: row_max_u32 inside each row of 16 lanes, then the four row results
// through scalar registers.
MOE_DEV uint32_t wave_max_u32(uint32_t x) {
    x = row_max_u32(x);
    const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)x, 0),
                           (uint32_t)__builtin_amdgcn_readlane((int)x, 16));
    const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)x, 32),
                           (uint32_t)__builtin_amdgcn_readlane((int)x, 48));
    return max(a, b);
}
MOE_DEV uint32_t wave_min_u32(uint32_t x) { return ~wave_max_u32(~x); }

// Top-k of one token's E logits with one wave.  Lane l owns experts
// l, l + 64, ...; NPL = values per lane.  Writes idx/w for the token.
//
// k rounds of a wave-wide argmax.  Each lane compares its remaining logits
// by float order (the larger logit wins, the smaller index on equal logits),
// the wave takes the largest order value, and of the lanes that hold it the
// one with the smallest expert index wins (a single lane nearly always; a
// second reduction otherwise).  The winner leaves its lane's candidates, and
// lane j keeps round j's expert and logit, so the k slots come out ordered
// by decreasing logit, smaller index first among equal logits.
template <int NPL>
MOE_DEV void route_token(const float (&v)[NPL], int E, int k, int score_fn, int renorm,
                         int32_t* __restrict__ idx_out, float* __restrict__ w_out, int* lds_idx,
                         float* lds_w) {
    const int lane = threadIdx.x & 63;
    uint32_t ord[NPL];                      // 0: no expert here, or already taken
#pragma unroll
    for (int i = 0; i < NPL; ++i) ord[i] = lane + 64 * i < E ? float_order(v[i]) : 0u;
    int my_e = 0;
    float my_v = 0.0f, lmax = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint32_t best = ord[0];
        int bi = 0;
        float bv = v[0];
#pragma unroll
        for (int i = 1; i < NPL; ++i) {
            if (ord[i] > best) {
                best = ord[i];
                bi = i;
                bv = v[i];
            }
        }
        const uint32_t m = wave_max_u32(best);
        const uint64_t tied = __ballot(best == m);
        int e;
        if (__popcll(tied) == 1) {
            const int wl = __builtin_ctzll(tied);
            e = wl + 64 * __builtin_amdgcn_readlane(bi, wl);
        } else {
            e = (int)wave_min_u32(best == m ? (uint32_t)(lane + 64 * bi) : ~0u);
        }
        // expert e is its lane's best candidate, so that lane's bv is its logit
        const float ev = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), e & 63));
        if (j == 0) lmax = ev;
        if (lane == j) {
            my_e = e;
            my_v = ev;
        }
#pragma unroll
        for (int i = 0; i < NPL; ++i)
            if (lane + 64 * i == e) ord[i] = 0u;
    }
    // weights
    float s = 0.0f;
    if (lane < k) s = score_fn == 0 ? expf(my_v - lmax) : 1.0f / (1.0f + expf(-my_v));
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
        const float w = s / denom;
        idx_out[lane] = my_e;
        lds_idx[lane] = my_e;
        w_out[lane] = w;
        if (lds_w) lds_w[lane] = w;
    }
}

// Quantise x rows [T, H]: task i covers 8 elements of the flattened array;
// workgroups of kThreads threads.
template <int kThreads, bool kCoh = false>
MOE_DEV void quant_rows(const RouteParams& p, int block, int nblocks) {
    const int64_t tasks = p.T * (p.H / 8);
    const int64_t stride = (int64_t)nblocks * kThreads;
    constexpr int U = 4;
    for (int64_t i0 = (int64_t)block * kThreads + threadIdx.x; i0 < tasks; i0 += U * stride) {
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
                put<kCoh>(reinterpret_cast<uint64_t*>(p.xq + i * 8), (uint64_t)lo | (uint64_t)hi << 32);
                if ((i & 3) == 0) {
                    // scales K-step major: xsf[g / 4][t][g % 4] for group g of token t
                    const int64_t G = i >> 2, gpr = p.H / kGroup;
                    const int64_t t = G / gpr, g = G - t * gpr;
                    put<kCoh>(p.xsf + (g >> 2) * (p.T * 4) + t * 4 + (g & 3), (uint8_t)(e + 127));
                }
            }
        }
    }
}

// The tokens [t0, t0 + ntok) of this wave: i = wave, wave + W, ... for a
// workgroup of W waves.  Up to 4 logits per lane, the next token's logits are
// loaded while the current one is routed (more would cost registers that the
// quantising workgroups of the same kernel need for occupancy).
template <int NPL, int kThreads>
MOE_DEV void route_tokens(const RouteParams& p, int64_t t0, int ntok, int* pair_exp,
                          float* pair_w) {
    constexpr int W = kThreads / 64;
    constexpr bool kPrefetch = NPL <= 4;
    const int k = p.topk;
    int i = threadIdx.x >> 6;
    if (i >= ntok) return;
    float v[NPL], nv[NPL];
    if (kPrefetch) load_logits<NPL>(p.logits + (t0 + i) * p.E, p.E, v);
    for (; i < ntok; i += W) {
        const int64_t t = t0 + i;
        if (kPrefetch)
            load_logits<NPL>(p.logits + (t0 + min(i + W, ntok - 1)) * p.E, p.E, nv);
        else
            load_logits<NPL>(p.logits + t * p.E, p.E, v);
        route_token<NPL>(v, p.E, k, p.score_fn, p.renorm, p.idx_out + t * k, p.w_out + t * k,
                         pair_exp + i * k, pair_w ? pair_w + i * k : nullptr);
        if (kPrefetch) {
#pragma unroll
            for (int j = 0; j < NPL; ++j) v[j] = nv[j];
        }
    }
}

// Route tokens [t0, t0 + ntok) (one wave per token) or take the caller's ids;
// pair i = (t - t0) * k + j of the chunk gets its expert in pair_exp[i] and, if
// pair_w is given, its weight in pair_w[i].
template <int kThreads>
MOE_DEV void route_chunk(const RouteParams& p, int64_t t0, int ntok, int npl, int* pair_exp,
                         float* pair_w = nullptr) {
    const int tid = threadIdx.x;
    const int k = p.topk;
    if (p.logits) {
        if (npl <= 1) route_tokens<1, kThreads>(p, t0, ntok, pair_exp, pair_w);
        else if (npl <= 2) route_tokens<2, kThreads>(p, t0, ntok, pair_exp, pair_w);
        else if (npl <= 4) route_tokens<4, kThreads>(p, t0, ntok, pair_exp, pair_w);
        else if (npl <= 8) route_tokens<8, kThreads>(p, t0, ntok, pair_exp, pair_w);
        else route_tokens<16, kThreads>(p, t0, ntok, pair_exp, pair_w);
    } else {
        for (int i = tid; i < ntok * k; i += kThreads) {
            int e = p.idx_in[t0 * k + i];
            pair_exp[i] = e;
            if (pair_w) pair_w[i] = p.w_in[t0 * k + i];
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
    __shared__ int pair_rank[kRouteTokensPerBlock * kMaxTopk];
    __shared__ int pair_exp[kRouteTokensPerBlock * kMaxTopk];   // expert of pair i of this block

    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * kRouteTokensPerBlock;
    const int ntok = (int)min<int64_t>(kRouteTokensPerBlock, p.T - t0);
    const int k = p.topk;

    for (int e = tid; e < p.E; e += kRouteThreads) hist[e] = 0;
    // 1. routing (one wave per token) or caller's ids
    route_chunk<kRouteThreads>(p, t0, ntok, npl, pair_exp);
    lds_barrier();

    // 2. count: LDS histogram; the LDS atomic's return is the pair's rank here
    const int npairs = ntok * k;
    for (int i = tid; i < npairs; i += kRouteThreads) {
        int e = pair_exp[i];
        pair_rank[i] = (e >= 0 && e < p.E) ? atomicAdd(&hist[e], 1) : -1;
    }
    lds_barrier();
    for (int e = tid; e < p.E; e += kRouteThreads) {
        int c = hist[e];
        base[e] = c ? atomicAdd(&p.cnt[e], c) : 0;
    }
    lds_barrier();
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
        for (int m = tid; m < p.nready; m += kRouteThreads) p.ready[m] = 0;
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
// workgroup).  One scan serves the pair offsets and both tile tables: each
// expert contributes its pairs, m-tiles and sub-tiles as three 21-bit fields
// of one 64-bit value (none of the sums reaches 2^21 at this size), and the
// thread that owns an expert writes that expert's records itself.  Workgroups
// of kThreads threads.  kCoh: every table is stored device-coherently, for
// workgroups of the same launch that read it after a hand-off.
template <int kThreads, bool kCoh = false>
MOE_DEV void bucket_small(const RouteParams& rp, const ScatterParams& sp, int npl) {
    using Scan = rocprim::block_scan<uint64_t, kThreads>;
    constexpr int kPer = kMaxExperts / kThreads;          // experts per thread
    constexpr uint64_t kField = (1u << 21) - 1;
    __shared__ int hist[kMaxExperts];
    __shared__ int off[kMaxExperts];
    __shared__ typename Scan::storage_type tmp;
    __shared__ int pair_exp[kSmallPairs];
    __shared__ int pair_rank[kSmallPairs];
    __shared__ float pair_w[kSmallPairs];
    const int tid = threadIdx.x;
    const int k = rp.topk, E = rp.E, bm = sp.bm;
    const int npairs = (int)rp.T * k;
    for (int e = tid; e < E; e += kThreads) hist[e] = 0;
    route_chunk<kThreads>(rp, 0, (int)rp.T, npl, pair_exp, pair_w);
    lds_barrier();
    for (int i = tid; i < npairs; i += kThreads) {
        const int e = pair_exp[i];
        pair_rank[i] = (e >= 0 && e < E) ? atomicAdd(&hist[e], 1) : -1;
    }
    lds_barrier();
    int c[kPer];
    uint64_t f[kPer], x[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int e = tid * kPer + j;
        c[j] = e < E ? hist[e] : 0;
        f[j] = (uint64_t)c[j] | (uint64_t)ceil_div(c[j], bm) << 21 |
               (uint64_t)ceil_div(c[j], kSubRows) << 42;
    }
    uint64_t total;
    Scan().exclusive_scan(f, x, (uint64_t)0, total, tmp);
    const int n_mtiles = (int)((total >> 21) & kField), n_subs = (int)(total >> 42);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int e = tid * kPer + j;
        if (e >= E) break;
        const int o = (int)(x[j] & kField);
        int m = (int)((x[j] >> 21) & kField), u = (int)(x[j] >> 42);
        off[e] = o;
        put<kCoh>(sp.counts_out + e, c[j]);
        put<kCoh>(sp.offsets_out + e, o);
        put<kCoh>(sp.mtile_off + e, m);
        for (int r = 0; r < c[j]; r += bm, ++m) {
            put<kCoh>(sp.mtile_rec + m, make_int4(e, o + r, min(bm, c[j] - r), 0));
            put<kCoh>(sp.mtile_e + m, e);
        }
        for (int r = 0; r < c[j]; r += kSubRows, ++u)
            put<kCoh>(sp.sub_rec + u, make_int4(e, o + r, min(kSubRows, c[j] - r), 0));
    }
    if (tid == 0) {
        put<kCoh>(sp.offsets_out + E, (int)(total & kField));
        put<kCoh>(sp.mtile_off + E, n_mtiles);
        put<kCoh>(sp.nsub, n_subs);
        put<kCoh>(sp.status, 0);
    }
    // records past the last tile are zero; the one-launch GEMMs' counters start at zero
    const int4 zero = make_int4(0, 0, 0, 0);
    for (int m = n_mtiles + tid; m < sp.max_mtiles; m += kThreads) put<kCoh>(sp.mtile_rec + m, zero);
    for (int m = n_subs + tid; m < sp.max_subs; m += kThreads) put<kCoh>(sp.sub_rec + m, zero);
    for (int m = tid; m < sp.nready; m += kThreads) put<kCoh>(sp.ready + m, 0);
    lds_barrier();                                        // off[] complete
    for (int i = tid; i < npairs; i += kThreads) {
        const int e = pair_exp[i];
        if (pair_rank[i] >= 0) {
            const int pos = off[e] + pair_rank[i];
            put<kCoh>(sp.slot_src + pos, i);
            put<kCoh>(sp.slot_of + i, pos);
            put<kCoh>(sp.slot_w + pos, pair_w[i]);
        } else {
            put<kCoh>(sp.slot_of + i, -1);
        }
    }
}

}  // namespace moe
