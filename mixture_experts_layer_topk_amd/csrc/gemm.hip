// Grouped block-scaled GEMMs of the expert MLP on gfx950 matrix cores.
//
// GEMM1 ("MegaMoE" notes, "GEMM" and the flow chart; "MegaMoE：把通信和计算融合
// 到一个 Mega Kernel", "L1/L2 交错" table): for every expert e and every position
// p of its segment, acc[n] = sum_K dq(xq[token(p)]) * dq(W13[e, n]) with FP8
// activations and FP4 weights, one UE8M0 scale per 32 K on both sides, FP32
// accumulation.  Epilogue ("L1 epilogue"; "Warp Specialization" L1 epilogue
// excerpt): h = silu(gate) * up * topk_weight on the FP32 accumulators, then
// per 32 columns of I the smallest power-of-two scale and E4M3 codes.
// GEMM2 ("L2 epilogue"): out[p, n] = sum_I dq(hq[p]) * dq(W2[e, n]) in FP32,
// rounded to BF16.
//
// Mapping to the hardware.  One V_MFMA_SCALE_F32_16X16X128_F8F6F4 multiplies a
// 16 x 128 FP8 tile by a 128 x 16 FP4 tile and applies the E8M0 scales itself.
// With g = l / 16, lane l supplies (layout measured on gfx950):
//   A (FP8): row l % 16, K [16 g, 16 g + 16) in bytes 0-15 and
//            K [64 + 16 g, 64 + 16 g + 16) in bytes 16-31;
//   B (FP4): column l % 16, K [32 g, 32 g + 32) in bytes 0-15;
//   scales:  the E8M0 byte of row (column) l % 16 for K group [32 g, 32 g + 32);
// and receives rows 4 g + i, column l % 16 of the 16 x 16 FP32 result.
//
// A workgroup owns a BM x BN output tile and loops over K in steps of 128.
// The waves form a WM x WN grid; each wave computes (BM/WM) x (BN/WN) with
// MT x NT MFMA tiles.
//
// Column permutation.  The B tile's LDS row order is chosen so that a lane's
// NT accumulator columns are contiguous output columns: within a wave's slice,
// LDS row nt*16 + c holds output column c*NT + nt.  For GEMM1 the slice's
// MFMA column tiles alternate gate (even nt) and up (odd nt) for the same
// I columns, so SwiGLU pairs acc[2q] with acc[2q+1] inside one lane and a lane
// owns NT/2 consecutive h columns; an E4M3 group of 32 columns is then
// 32/(NT/2) neighbouring lanes.  The canonical weight layout (gate rows, then
// up rows) is read as is; the pages' offline 8-row gate/up interleave
// ("原始权重布局") is replaced by this in-loader permutation.
//
// Tiles are handed out persistently in a grouped order: tiles are numbered
// in groups of kGM consecutive m-tiles x all n-tiles, m fastest inside a
// group, and workgroup slot q takes tile numbers q, q + grid, ...  Workgroups
// are dealt to the 8 XCDs round-robin (workgroup b runs on XCD b % 8), so
// slots are assigned XCD-contiguously: the grid/8 workgroups of one XCD hold
// consecutive slots, and in each round one XCD works on a rectangle of up to
// kGM m-tiles by a few n-tiles, whose A rows and B columns are shared in its
// own L2, instead of every XCD streaming every m-tile.  An m-tile is BM consecutive
// positions of one expert (the last one ragged), looked up in the per-m-tile
// expert table the bucketisation writes.
//
// Loads go straight from global memory to LDS (global_load_lds_dwordx4): one
// instruction fills 1 KiB of LDS contiguously, lane l landing at byte 16 l, so
// the XOR swizzle of the LDS tiles is applied on the global side by choosing
// which 16-byte chunk each lane fetches.  Three LDS stages rotate: the loads
// of step ks + 2 are issued during step ks into the stage every wave retired
// at the barrier that ended step ks - 1.  In the two-launch kernels the ring
// runs on from one tile of a workgroup to its next: the last two K steps of a
// tile load the next tile's first two, whose row tables and load sources were
// set up during the K loop, so a tile's epilogue overlaps the next tile's
// first loads instead of a drained pipeline.
//
// Eight waves, two per SIMD, each 64 x 128 of the tile.  The SIMD's two waves
// are de-phased (wm = 0 early, wm = 1 late): after the barrier that publishes
// stage ks the early wave reads its fragments and then runs its MFMAs, while
// the late wave first runs the MFMAs of step ks - 1 from registers and then
// reads stage ks, so one wave's LDS reads overlap the other's MFMAs instead of
// both SIMD waves reading, then both computing (measured 5% faster GEMMs).
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "mfma.h"
#define MOE_HD __host__ __device__ __forceinline__
#include "sched.h"

namespace moe {

constexpr int BK = kKStep;              // K per MFMA step (bytes of FP8 A per row)
using sched::grouped_order;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int BM, int BN, int WM, int WN, bool kG1>
struct Cfg {
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int WTM = BM / WM;             // wave tile rows
    static constexpr int WTN = BN / WN;             // wave tile cols
    static constexpr int MT = WTM / 16;
    static constexpr int NT = WTN / 16;
    static constexpr int kABytes = BM * BK;         // FP8
    static constexpr int kBBytes = BN * BK / 2;     // FP4
    static constexpr int kSABytes = BM * 4;
    static constexpr int kSBBytes = BN * 4;
    static constexpr int kStage = kABytes + kBBytes + kSABytes + kSBBytes;
    static constexpr int kStages = 3;
    // LDS: the stages, then two tiles' token rows and topk weights and one
    // staging row of pair indices
    static constexpr int kRowBytes = BM * (2 * 4 + 2 * 4 + 4);
    static constexpr int kLds = kStages * kStage + kRowBytes;
    static constexpr int kAI = kABytes / 1024 / kWaves;   // 1 KiB load instructions per wave
    static constexpr int kBI = kBBytes / 1024 / kWaves;
    // Scale tiles: one dword per lane, 64 rows per load.  Early wave e loads
    // B-scale blocks kSBE e .. kSBE e + kSBE - 1, late wave kEarly + e the
    // A-scale block e if e < kSABlocks.  The late wave's chain sets the end of
    // a K step (its MFMAs, then its loads, fragment reads and the wait for its
    // previous loads), while the early wave has time to spare before the
    // matrix core is free for its MFMAs, so the B scales go to the early
    // waves (GEMM1 -1.1% at the 256-expert shape, no change at 32 experts).
    static constexpr int kEarly = WN;
    static constexpr int kSABlocks = BM / 64, kSBBlocks = BN / 64;
    static constexpr int kSBE = kSBBlocks / kEarly;
    static constexpr int kLoadsEarly = kAI + kBI + kSBE;    // per wave per stage
    static constexpr int kLoadsLate = kAI + kBI;            // + 1 with an A-scale block
    static_assert(kABytes % (1024 * kWaves) == 0 && kBBytes % (1024 * kWaves) == 0, "tile / waves");
    static_assert(BM % 64 == 0 && BN % 64 == 0, "scale tiles in whole 64-row loads");
    static_assert(MT >= 1 && NT >= 2 && NT % 2 == 0, "wave tile");
    static_assert(WM == 2 && kSBBlocks % kEarly == 0 && kSABlocks <= kEarly, "scale loads");
    static_assert(kLoadsLate + 1 < 64, "vmcnt range");
    static_assert(kLds <= 160 * 1024, "LDS of one CU");
};

// LDS swizzles.  An A fragment read touches 16 consecutive rows (128 bytes
// each) at one logical 16-byte chunk; a B fragment read the same for rows of
// 64 bytes.  The XOR patterns below were chosen by timing ds_read_b128 with
// these exact lane patterns on gfx950: they run at the conflict-free rate
// (the same as 64 consecutive 16-byte chunks), where the unswizzled layouts
// take 2.3x as long.  Both depend on the row modulo 8 only, so the fragments
// of different m-tiles (n-tiles) sit at constant offsets from one another.
MOE_DEV int a_swz(int r) { return r & 7; }
MOE_DEV int b_swz(int n) { return (n >> 1) & 3; }
// A: row r, 16-byte chunk c (of 8) -> swizzled byte offset inside the A tile.
MOE_DEV int a_off(int r, int c) { return r * BK + ((c ^ a_swz(r)) << 4); }
// B: row n, 16-byte chunk c (of 4) -> swizzled byte offset inside the B tile.
MOE_DEV int b_off(int n, int c) { return n * (BK / 2) + ((c ^ b_swz(n)) << 4); }

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8], vmcnt[5:4] in bits [15:14]).
template <int N>
MOE_DEV void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without a memory fence: LDS traffic is ordered by the
// explicit vmcnt waits around it; the empty asm keeps the compiler from moving
// memory operations across it.
MOE_DEV void barrier_nofence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Scale tiles are staged so that one lane's scales of four consecutive
// 16-row (16-column) MFMA tiles are one 16-byte run: inside every group of 64
// staged dwords, slot q holds the scales of tile row
//   (q & ~63) | (q & 3) << 4 | (q >> 2) & 15,
// i.e. row 16 t + r of tile t < 4 sits at slot 4 r + t.  A lane (row r)
// then reads tiles 4h .. 4h + 3 with one ds_read_b128 at slot 64 h + 4 r, and
// the 16 lanes of one lane group read 256 consecutive bytes (no conflicts).
MOE_DEV int scale_slot_row(int q) { return (q & ~63) | ((q & 3) << 4) | ((q >> 2) & 15); }

// Largest value over each group of 8 neighbouring lanes (lanes 8j .. 8j + 7),
// with DPP row operations instead of LDS round trips: swap neighbours, swap
// pairs (each quad then holds its maximum), then mirror the 8-lane half-row
// (quad 0 meets quad 1).  The values are bit patterns of non-negative floats,
// which order like the unsigned integers.
MOE_DEV uint32_t max_of_8_lanes(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));  // half mirror
}

// kAux: cache policy bits of the load (kCohAux: device-coherent, sc1)
constexpr int kCohAux = 16;
constexpr int kSpinLimit = 1 << 24;     // polls of a ready counter before giving up (~0.5 s)

template <int kAux>
MOE_DEV void load_lds16(const void* g, uint8_t* lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 16, 0, kAux);
}
template <int kAux>
MOE_DEV void load_lds4(const void* g, uint8_t* lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 4, 0, kAux);
}

// Per-workgroup GEMM state for one output tile at a time: the per-lane global
// sources of the load instructions, the MFMA operands and the accumulators,
// with the pieces of the K-step schedule as members so that the grouped
// kernels (tiles back to back, next tile prefetched) and the one-launch kernel
// (one tile at a time) run the same code.
//
// LDS: kStages stages, then the row tables of two tiles (the one in the K loop
// and the next one): token row per A row (GEMM1), topk weight per A row, and
// a staging row for the position -> pair lookup of the next tile.
// kCoh: the tile runs inside the one-launch kernel, where GEMM2 reads h that
// other XCDs wrote in the same launch; h is then stored and read with
// device-coherent accesses (sc1), which go to the memory-side cache instead of
// an XCD's own L2, while the weights keep the cached path.
// kIL: W13 is in the gran-8 gate/up row interleave (a compile-time choice: a
// run-time select in the row mapping costs the GEMM1 kernel register spills).
// kST: the weight codes are in the staged layout (16-row groups in the order
// the B tile stages them, one contiguous KiB per group and K step), so every
// B load instruction reads one KiB instead of 16 row pieces of 64 bytes; the
// weight scales keep the canonical row order.
template <int BM, int BN, int WM, int WN, bool kG1, bool kCoh, bool kIL = false, bool kST = false>
struct TileEngine {
    using C = Cfg<BM, BN, WM, WN, kG1>;
    static constexpr int kAuxA = (kCoh && !kG1) ? kCohAux : 0;

    const GemmParams& p;
    uint8_t* smem;
    int* s_tok;         // [2][BM] A row source (token row), GEMM1
    float* s_w;         // [2][BM] topk weight of the A row, GEMM1
    int* s_pair;        // [BM]    pair index of the A row, staging for the next tile
    int K, nk;          // reduction length and K steps
    int64_t sa_slab, sb_ks;     // bytes per K step of the activation and the weight scales
    const uint8_t* a_base;
    const uint8_t* sa_base;
    // sources of the next K step to load (A, B, A scales, B scales), advanced
    // by one K step per issue
    const uint8_t* ld_a;
    const uint8_t* ld_w;
    const uint8_t* ld_sa;
    const uint8_t* ld_sw;
    bool late;                  // the second wave of this SIMD (wm == 1)
    int wm_u;                   // wm of this wave (uniform)
    bool rows;                  // this wave's 64 rows of the tile hold rows of the expert
    bool sa_wave;               // a late wave that loads an A-scale block
    int lg;
    int a_lo, a_hi, b_fr, sa_fr, sb_fr;

    uint32_t a_src[C::kAI];
    uint32_t b_src[C::kBI];
    uint32_t sa_src;
    uint32_t sb_src[C::kSBE];
    v4f acc[C::MT][C::NT];
    v8i a[C::MT];
    v4i b[C::NT];
    // scale dwords as read: byte lg of dword t of run h is the scale of K group
    // lg for tile 4h + t; the byte is extracted where the MFMAs use it, so
    // nothing between the fragment reads and the load issue waits for LDS
    v4i sa_run[C::MT / 4];
    v4i sb_run[C::NT / 4];

    // Per-lane indices are re-derived from an opaque copy of the thread id
    // where they are needed, so the compiler recomputes the (cheap) per-lane
    // constants instead of keeping dozens of them alive across the K loop.
    struct Lane {
        int tid, lane, wave, wm, wn, l16, lg;
        __device__ __forceinline__ Lane() {
            int t = threadIdx.x;
            asm volatile("" : "+v"(t));
            tid = t;
            lane = t & 63;
            wave = t >> 6;
            wm = wave / WN;
            wn = wave % WN;
            l16 = lane & 15;
            lg = lane >> 4;
        }
    };

    __device__ __forceinline__ TileEngine(const GemmParams& pp, uint8_t* sm) : p(pp), smem(sm) {
        s_tok = reinterpret_cast<int*>(smem + C::kStages * C::kStage);
        s_w = reinterpret_cast<float*>(s_tok + 2 * BM);
        s_pair = reinterpret_cast<int*>(s_w + 2 * BM);
        K = kG1 ? p.H : p.I;
        nk = K / BK;
        // Scales are stored K-step major: the 4 UE8M0 bytes of one 128-wide K
        // step for row r sit at slab[ks][r][0..3], so a tile's scales for one K
        // step are 4-byte entries of one slab rather than bytes strided across rows.
        sa_slab = 4 * (kG1 ? p.T : p.T * p.topk);
        sb_ks = kG1 ? p.w13sf_ks : p.w2sf_ks;
        a_base = kG1 ? p.xq : p.hq;
        sa_base = kG1 ? p.xsf : p.hsf;
        const Lane L;
        late = __builtin_amdgcn_readfirstlane(L.wm) == 1;
        wm_u = __builtin_amdgcn_readfirstlane(L.wm);
        rows = true;
        sa_wave = late && __builtin_amdgcn_readfirstlane(L.wave) % C::kEarly < C::kSABlocks;
        lg = L.lg;
        // MFMA operands.  Fragment addresses of different tiles differ by
        // constants (the swizzles depend on row % 16 only).
        const int a_row0 = L.wm * C::WTM + L.l16;
        const int b_row0 = L.wn * C::WTN + L.l16;
        a_lo = a_off(a_row0, L.lg);
        a_hi = a_off(a_row0, 4 + L.lg);
        b_fr = C::kABytes + b_off(b_row0, L.lg);
        // scale runs of this lane: tiles 4h .. 4h+3 at slot base + 64 h + 4 l16
        sa_fr = C::kABytes + C::kBBytes + 4 * (L.wm * C::WTM + 4 * L.l16);
        sb_fr = C::kABytes + C::kBBytes + C::kSABytes + 4 * (L.wn * C::WTN + 4 * L.l16);
    }

    // Row tables of a GEMM1 tile {expert, first position, rows} into buffer
    // buf, loaded and published at once (first tile, one-launch tiles).
    __device__ __forceinline__ void load_rows_now(int4 rec, int buf) {
        const int tid = threadIdx.x;
        if (kG1 && tid < BM) {
            const int pair = p.slot_src[rec.y + min(tid, rec.z - 1)];
            s_tok[buf * BM + tid] = pair / p.topk;
            s_w[buf * BM + tid] = p.topk_w[pair];
        }
        __syncthreads();
    }
    // The same for the next tile, spread over two K steps of the current one
    // as loads straight into LDS: part 0 fetches the pair index of every row,
    // part 1 (a step later, after the wait that retires part 0) derives the
    // token row and fetches the topk weight.  Each part is issued before the
    // step's tile loads, so the step's closing vmcnt wait retires it.
    __device__ __forceinline__ void fetch_rows(int4 rec, int buf, int part) {
        const Lane L;
        if (!kG1 || L.wave * 64 >= BM) return;
        if (part == 0) {
            const int* src = p.slot_src + rec.y + min(L.tid, rec.z - 1);
            load_lds4<0>(src, reinterpret_cast<uint8_t*>(s_pair + 64 * L.wave));
        } else {
            const int pair = s_pair[L.tid];
            s_tok[buf * BM + L.tid] = pair / p.topk;
            load_lds4<0>(p.topk_w + pair, reinterpret_cast<uint8_t*>(s_w + buf * BM + 64 * L.wave));
        }
    }

    // Global sources of the loads of tile {rec, ntile}; for GEMM1 the token
    // rows come from row buffer buf, which must be published.
    __device__ __forceinline__ void set_tile(int4 rec, int ntile, int buf) {
        const Lane L;
        const int e = rec.x, p0 = rec.y, valid = rec.z;
        auto row_src = [&](int r) -> uint32_t {
            return kG1 ? (uint32_t)s_tok[buf * BM + r] : (uint32_t)(p0 + min(r, valid - 1));
        };
        // B tile LDS row -> weight row.  Inside a wave's slice, LDS row nt*16 + c
        // holds output column c*NT + nt (GEMM2) or, for GEMM1, I column
        // c*NT/2 + nt/2 of the gate (even nt) or up (odd nt) projection.
        auto b_row = [&](int bq) -> uint32_t {
            const int ws = bq / C::WTN, bl = bq % C::WTN;
            const int nt = bl >> 4, c = bl & 15;
            if (kG1) {
                int icol = ntile * (BN / 2) + ws * (C::WTN / 2) + c * (C::NT / 2) + (nt >> 1);
                icol = min(icol, p.I - 1);          // partial last n-tile: never stored
                return (uint32_t)w13_row(icol, nt & 1, p.I, kIL);
            } else {
                const int n = ntile * BN + ws * C::WTN + c * C::NT + nt;
                return min(n, p.H - 1);
            }
        };
        const int64_t b_stride = K / 2;
        ld_a = a_base;
        ld_w = kG1 ? p.w13 + (int64_t)e * (2 * p.I) * b_stride : p.w2 + (int64_t)e * p.H * b_stride;
        ld_sa = sa_base;
        ld_sw = (kG1 ? p.w13sf : p.w2sf) + (int64_t)e * (kG1 ? 2 * p.I : p.H) * (K / kGroup);
        // per-lane global sources of each load instruction (fixed over K), as
        // 32-bit byte offsets from wave-uniform bases
#pragma unroll
        for (int j = 0; j < C::kAI; ++j) {
            const int r = 8 * (j * C::kWaves + L.wave) + (L.lane >> 3);
            const int c = (L.lane & 7) ^ a_swz(r);
            a_src[j] = row_src(r) * (uint32_t)K + c * 16;
        }
#pragma unroll
        for (int j = 0; j < C::kBI; ++j) {
            const int n = 16 * (j * C::kWaves + L.wave) + (L.lane >> 2);
            const int c = (L.lane & 3) ^ b_swz(n);
            if constexpr (kST) {
                // LDS rows 16 gi .. 16 gi + 15 are MFMA column tile gi % NT of wave
                // slice gi / NT: staged group 8 b + nt of the expert, b the slice's
                // column block (the last one for a partial n-tile: never stored)
                static_assert(C::NT == 8 && C::WTN / (kG1 ? 2 : 1) == (kG1 ? 64 : 128),
                              "staged groups are the wave slices' column tiles");
                const int gi = j * C::kWaves + L.wave;
                const int blk = min(ntile * WN + gi / C::NT, (kG1 ? p.I / 64 : p.H / 128) - 1);
                const int g = 8 * blk + gi % C::NT;
                b_src[j] = (uint32_t)(g * nk) * (uint32_t)kStagedBlock + (L.lane >> 2) * 64 + c * 16;
            } else {
                b_src[j] = b_row(n) * (uint32_t)b_stride + c * 16;
            }
        }
        // scale blocks: B of an early wave, A of a late wave (the other values
        // are not used)
        const int ew = L.wave % C::kEarly;
        sa_src = row_src(scale_slot_row(64 * (ew % C::kSABlocks) + L.lane)) * 4u;
        // B scales are staged in the B tile's LDS row order, regrouped by
        // scale_slot_row: the slots of LDS row q hold weight row b_row(q).
#pragma unroll
        for (int j = 0; j < C::kSBE; ++j)
            sb_src[j] = b_row(scale_slot_row(64 * (C::kSBE * ew + j) + L.lane)) *
                        (uint32_t)(kG1 ? p.w13sf_rs : p.w2sf_rs);
    }

    __device__ __forceinline__ uint8_t* stage_ptr(int stage) const { return smem + stage * C::kStage; }

    // The loads of the next K step into LDS stage `stage`: A tile chunks
    // first, then B, then the two scale tiles.  The LDS destination (M0) is
    // derived from a vector copy of the wave index: measured faster here than
    // the same arithmetic on the scalar unit, which all waves of the CU share.
    __device__ __forceinline__ void issue(int stage) {
        int tv = threadIdx.x;
        asm volatile("" : "+v"(tv));
        const int wave = tv >> 6;
        uint8_t* sA = stage_ptr(stage);
        uint8_t* sB = sA + C::kABytes;
        uint8_t* sSA = sB + C::kBBytes;
        uint8_t* sSB = sSA + C::kSABytes;
#pragma unroll
        for (int j = 0; j < C::kAI; ++j)
            load_lds16<kAuxA>(ld_a + a_src[j], sA + (j * C::kWaves + wave) * 1024);
#pragma unroll
        for (int j = 0; j < C::kBI; ++j)
            load_lds16<0>(ld_w + b_src[j], sB + (j * C::kWaves + wave) * 1024);
        {
            const int ew = wave % C::kEarly;
            if (sa_wave) load_lds4<kAuxA>(ld_sa + sa_src, sSA + ew * 256);
            if (!late) {
#pragma unroll
                for (int j = 0; j < C::kSBE; ++j)
                    load_lds4<0>(ld_sw + sb_src[j], sSB + (C::kSBE * ew + j) * 256);
            }
        }
        ld_a += BK;
        ld_w += kST ? kStagedBlock : BK / 2;
        ld_sa += sa_slab;
        ld_sw += sb_ks;
    }

    // Rows of the tile in the K loop: a wave whose WTM rows all lie past the
    // expert's last row (the late wave in the last m-tile of an expert with
    // at most WTM rows there) skips its MFMAs; its outputs are never stored.
    // (Skipping single 16-row m-tiles instead made the compiler spill the
    // accumulators.)
    __device__ __forceinline__ void set_rows(int valid) { rows = valid > wm_u * C::WTM; }

    __device__ __forceinline__ void zero_acc() {
#pragma unroll
        for (int i = 0; i < C::MT; ++i)
#pragma unroll
            for (int j = 0; j < C::NT; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    }

    __device__ __forceinline__ void read_frags(const uint8_t* st) {
        static_assert(C::MT % 4 == 0 && C::NT % 4 == 0, "scale runs of four tiles");
#pragma unroll
        for (int h = 0; h < C::MT / 4; ++h) sa_run[h] = *reinterpret_cast<const v4i*>(st + sa_fr + 256 * h);
#pragma unroll
        for (int h = 0; h < C::NT / 4; ++h) sb_run[h] = *reinterpret_cast<const v4i*>(st + sb_fr + 256 * h);
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) {
            const v4i lo = *reinterpret_cast<const v4i*>(st + a_lo + mt * 16 * BK);
            const v4i hi = *reinterpret_cast<const v4i*>(st + a_hi + mt * 16 * BK);
            a[mt] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt)
            b[nt] = *reinterpret_cast<const v4i*>(st + b_fr + nt * 16 * (BK / 2));
    }
    // lane group lg supplies the scale of K group lg: byte lg of each dword
    __device__ __forceinline__ void mfmas() {
        int sa[C::MT], sb[C::NT];
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) sa[mt] = (int)((uint32_t)sa_run[mt / 4][mt % 4] >> (8 * lg));
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) sb[nt] = (int)((uint32_t)sb_run[nt / 4][nt % 4] >> (8 * lg));
        if (rows) {
            // m-tile outer: consecutive MFMAs share their A fragment (measured
            // 0.6% faster than sharing B)
#pragma unroll
            for (int mt = 0; mt < C::MT; ++mt) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int nt = 0; nt < C::NT; ++nt)
                    acc[mt][nt] = mfma_fp8_fp4(a[mt], b[nt], acc[mt][nt], sa[mt], sb[nt]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // Steps 0 and 1 of the current tile into stages st and st + 1 (mod
    // kStages) and publish step 0.
    __device__ __forceinline__ void prologue(int st) {
        static_assert(C::kWaves == 8, "the K-step schedule assumes two waves per SIMD");
        wait_vmcnt<0>();
        issue(st);
        if (nk > 1) {
            issue(next_stage(st));
            wait_all_but_last_issue();
        } else {
            wait_vmcnt<0>();
        }
        barrier_nofence();
    }
    __device__ __forceinline__ static int next_stage(int st) { return st == C::kStages - 1 ? 0 : st + 1; }
    // Retire every memory operation of this wave but the loads of its last issue().
    __device__ __forceinline__ void wait_all_but_last_issue() const {
        if (!late)
            wait_vmcnt<C::kLoadsEarly>();
        else if (sa_wave)
            wait_vmcnt<C::kLoadsLate + 1>();
        else
            wait_vmcnt<C::kLoadsLate>();
    }

    // One K step on stage `cur`.  The two waves of a SIMD (wm = 0 and wm = 1)
    // are de-phased: after the barrier that publishes the stage the early wave
    // issues its loads, reads its fragments and then runs its MFMAs; the late
    // wave first runs the MFMAs of the previous step (fragments already in
    // registers), then issues its loads and reads the stage, so one wave's
    // loads and LDS reads overlap the other's MFMAs.  Loads go before the
    // fragment reads: the late wave's wait for its previous loads ends its
    // chain, and the fragments it reads are needed only at the next step
    // (GEMM1 -1.5 to -2.4%).  The late wave runs its MFMAs at raised priority:
    // when the early wave gets to its own MFMAs first, the late wave's still
    // win the SIMD, so it can go on to its loads and reads while the early
    // wave computes (without this the two waves' MFMAs interleave and the
    // late wave's loads and reads end up after every MFMA of the step, with
    // the matrix core idle).
    // `loads()` issues this step's loads (step + 2, or one of the next tile's
    // first two) and returns whether it issued any; `extra()` issues whatever
    // must be retired by this step's wait.  The wait retires everything but
    // this step's loads.
    template <class Extra, class Loads>
    __device__ __forceinline__ void step(const uint8_t* cur, bool first, Extra&& extra, Loads&& loads) {
        if (late && !first) {
            __builtin_amdgcn_s_setprio(2);
            mfmas();
            __builtin_amdgcn_s_setprio(0);
        }
        extra();
        const bool issued = loads();
        __builtin_amdgcn_sched_barrier(0);
        read_frags(cur);
        __builtin_amdgcn_sched_barrier(0);
        if (!late) mfmas();
        if (issued)
            wait_all_but_last_issue();
        else
            wait_vmcnt<0>();
        // the next step's loads overwrite the stage read here: its fragment
        // reads (the late wave's are consumed only by the next step's MFMAs)
        // complete before the barrier
        __builtin_amdgcn_s_waitcnt((63 & 15) | (7 << 4) | (0 << 8) | ((63 >> 4) << 14));  // lgkmcnt(0)
        barrier_nofence();
    }

    // The late wave's last MFMAs.
    __device__ __forceinline__ void finish() {
        if (late) mfmas();
        __builtin_amdgcn_s_waitcnt((63 & 15) | (7 << 4) | (0 << 8) | ((63 >> 4) << 14));  // lgkmcnt(0)
    }

    // ------------------------------------------------------------ epilogue
    __device__ __forceinline__ void epilogue(int4 rec, int ntile, int buf) {
        const Lane L;
        const int p0 = rec.y, valid = rec.z;
        if (kG1) {
            // lane holds, for row 4*lg + i of m-tile mt, the h columns
            // icol0 + l16*(NT/2) + q, q < NT/2 (gate acc[2q], up acc[2q+1])
            constexpr int QN = C::NT / 2;
            static_assert(QN == 4, "a 32-column E4M3 group is 8 neighbouring lanes");
            const int icol0 = ntile * (BN / 2) + L.wn * (C::WTN / 2);
            const int col = icol0 + L.l16 * QN;
            // this lane's first row (m-tile 0, i = 0): the stores of row
            // mt * 16 + i below add (mt * 16 + i) * I (codes) or * 4 (scales)
            const int r0 = L.wm * C::WTM + 4 * L.lg;
            const int64_t pos0 = (int64_t)p0 + r0;
            uint8_t* hq_lane = p.hq + pos0 * p.I + col;
            uint8_t* hsf_lane = p.hsf + (int64_t)(col / (4 * kGroup)) * (p.T * p.topk) * 4 + pos0 * 4 +
                                (col / kGroup) % 4;
#pragma unroll
            for (int mt = 0; mt < C::MT; ++mt) {
                // one m-tile at a time: bounds the registers live in the epilogue
                __builtin_amdgcn_sched_barrier(0);
                // routing weights of this lane's rows 4 lg + i of the m-tile
                const v4f wrow =
                    *reinterpret_cast<const v4f*>(s_w + buf * BM + L.wm * C::WTM + mt * 16 + 4 * L.lg);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = L.wm * C::WTM + mt * 16 + 4 * L.lg + i;
                    const float wr = wrow[i];
                    float h[QN];
                    uint32_t amax = 0;              // bits of max |h| (finite)
#pragma unroll
                    for (int q = 0; q < QN; ++q) {
                        const float g = acc[mt][2 * q][i], u = acc[mt][2 * q + 1][i];
                        h[q] = swiglu_w(g, u, wr);
                        amax = max(amax, f2u(h[q]) & 0x7FFFFFFFu);
                    }
                    const int ex = e4m3_block_exp(u2f(max_of_8_lanes(amax)));
                    const float inv = exp2_neg(ex);
                    if (r < valid && col < p.I) {
                        uint8_t* dst = hq_lane + (int64_t)(mt * 16 + i) * p.I;
                        static_assert(QN % 4 == 0, "whole dwords of E4M3 codes per lane");
#pragma unroll
                        for (int q = 0; q < QN; q += 4) {
                            const uint32_t v = e4m3_pack4(h[q] * inv, h[q + 1] * inv, h[q + 2] * inv,
                                                          h[q + 3] * inv);
                            uint32_t* d = reinterpret_cast<uint32_t*>(dst + q);
                            if constexpr (kCoh)
                                __hip_atomic_store(d, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            else
                                *d = v;
                        }
                        if ((col & (kGroup - 1)) == 0) {
                            uint8_t* d = hsf_lane + (mt * 16 + i) * 4;
                            if constexpr (kCoh)
                                __hip_atomic_store(d, (uint8_t)(ex + 127), __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
                            else
                                *d = (uint8_t)(ex + 127);
                        }
                    }
                }
            }
        } else {
            // lane holds row 4*lg + i, output columns n0 + l16*NT + nt, nt < NT
            const int n0 = ntile * BN + L.wn * C::WTN + L.l16 * C::NT;
#pragma unroll
            for (int mt = 0; mt < C::MT; ++mt) {
                // one m-tile at a time: keeps the accumulators in AGPRs until used
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = L.wm * C::WTM + mt * 16 + 4 * L.lg + i;
                    if (r < valid && n0 < p.H) {
                        uint16_t* dst = p.o + (int64_t)(p0 + r) * p.H + n0;
                        if constexpr (C::NT == 8) {
                            uint4 v;
                            v.x = pack_bf16x2(acc[mt][0][i], acc[mt][1][i]);
                            v.y = pack_bf16x2(acc[mt][2][i], acc[mt][3][i]);
                            v.z = pack_bf16x2(acc[mt][4][i], acc[mt][5][i]);
                            v.w = pack_bf16x2(acc[mt][6][i], acc[mt][7][i]);
                            *reinterpret_cast<uint4*>(dst) = v;
                        } else {
#pragma unroll
                            for (int nt = 0; nt < C::NT; ++nt)
                                dst[nt] = (uint16_t)f32_to_bf16(acc[mt][nt][i]);
                        }
                    }
                }
            }
        }
    }
};

// n-tiles of GEMM1 (BN/2 columns of I, gate and up) or GEMM2 (BN columns of
// H); the last one may be partial (I and H are multiples of 128).
template <int BN>
MOE_DEV int gemm_ntiles(const GemmParams& p, bool g1) {
    return g1 ? (p.I + BN / 2 - 1) / (BN / 2) : (p.H + BN - 1) / BN;
}

// Workgroup slot of this workgroup: consecutive for the workgroups of one XCD.
MOE_DEV int xcd_slot() { return sched::tile_slot(blockIdx.x, gridDim.x); }

// GEMM1 or GEMM2 alone (one launch each, ordered by the stream).  The K
// pipeline of a workgroup runs on across its tiles: while a tile is in its K
// loop the next tile's rows are fetched (GEMM1, steps 1 and 2) and its load
// sources set up (step nk - 2), and the last two steps issue the next tile's
// first two K steps instead of reloading the current tile's last one, so the
// epilogue overlaps those loads and the next tile starts on a full pipeline.
template <int BM, int BN, int WM, int WN, bool kG1, bool kIL, bool kST>
__global__ __launch_bounds__(64 * WM * WN, 1) void grouped_gemm_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    using Eng = TileEngine<BM, BN, WM, WN, kG1, false, kIL, kST>;
    const int NT = gemm_ntiles<BN>(p, kG1);
    const int mtiles = p.mtile_off[p.E];
    const int total = mtiles * NT;
    int tile = xcd_slot();
    if (tile >= total) return;
    Eng eng(p, smem);
    const int nk = eng.nk;
    // rows fetched in steps 1 and 2 are published by the barrier ending step 2
    const bool chain = nk >= (kG1 ? 5 : 2);
    int mt, ntile;
    grouped_order(tile, 0, mtiles, NT, &mt, &ntile);
    int4 rec = p.mtile_rec[mt];                  // {expert, first position, rows}
    int buf = 0, st = 0;                         // row buffer; LDS stage of the next step
    eng.load_rows_now(rec, buf);
    eng.set_tile(rec, ntile, buf);
    eng.prologue(st);
    for (;;) {
        const int nxt = tile + gridDim.x;
        const bool has_next = nxt < total;
        int mt_n = mt, nt_n = ntile;
        if (has_next) grouped_order(nxt, 0, mtiles, NT, &mt_n, &nt_n);
        const int4 rec_n = p.mtile_rec[mt_n];
        const bool pf = has_next && chain;
        eng.set_rows(rec.z);
        eng.zero_acc();
        for (int ks = 0; ks < nk; ++ks) {
            const int st2 = Eng::next_stage(Eng::next_stage(st));
            eng.step(
                eng.stage_ptr(st), ks == 0,
                [&] {
                    if (pf) {
                        if (ks == 1 || ks == 2) eng.fetch_rows(rec_n, buf ^ 1, ks - 1);
                        if (ks == nk - 2) eng.set_tile(rec_n, nt_n, buf ^ 1);
                    }
                },
                [&] {
                    if (ks + 2 >= nk && !pf) return false;
                    eng.issue(st2);
                    return true;
                });
            st = Eng::next_stage(st);
        }
        eng.finish();
        eng.epilogue(rec, ntile, buf);
        if (!has_next) break;
        tile = nxt;
        mt = mt_n;
        ntile = nt_n;
        rec = rec_n;
        buf ^= 1;
        if (!pf) {        // K too short to hide the next tile's set-up: do it here
            eng.load_rows_now(rec, buf);
            eng.set_tile(rec, ntile, buf);
            eng.prologue(st);
        }
    }
}

// Waits until ready[mt] counts every GEMM1 n-tile of m-tile mt.  Every lane
// polls and the loop branches on the first lane's value, so the wait is uniform
// (no divergent loop inside the K pipeline).  Bounded: past the spin limit
// thread 0 sets *p.status and the wait gives up, so the output is wrong but the
// kernel ends.  The bounds are read from p here rather than kept live in the
// caller's K loop.
template <int BN>
MOE_DEV void wait_ready(const GemmParams& p, int mt) {
    const int need = gemm_ntiles<BN>(p, true);
    const int spin_limit = p.spin_limit > 0 ? p.spin_limit : kSpinLimit;
    for (int n = 0;;) {
        const int v = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(p.ready + mt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (v >= need) break;
        __builtin_amdgcn_s_sleep(1);
        if (++n >= spin_limit) {
            if (threadIdx.x == 0) __hip_atomic_store(p.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
    }
}

// A run of one workgroup's consecutive list entries of one family (entries
// tile, tile + grid, ... while they are GEMM1 tiles, or GEMM2 tiles), with the
// two-launch kernel's cross-tile pipeline: the next entry's rows are fetched
// and its first two K steps loaded during the current entry's K loop.  Returns
// the first entry after the run (of the other family, or past the list).
//   GEMM1: h is stored device-coherent; after a tile's epilogue every thread
//          waits for its stores (vmcnt(0)), and after a barrier thread 0 adds
//          one to ready[m-tile].
//   GEMM2: the first tile of the run waits for ready[m] before any load; a
//          pipelined next tile's wait runs at the start of the current tile's
//          K loop, before its loads (at the last two K steps) are issued.
// A GEMM2 entry waits only for GEMM1 entries earlier in the list, GEMM1
// entries never wait, and every workgroup is resident: the waits end.
// List entry -> (family, m-tile, n-tile), seeking from the first segment (a
// few scalar steps per tile, so no cursor stays live across the K loop).
// Returns false past the end of the list.
template <int BN>
MOE_DEV bool fused_entry(const GemmParams& p, int entry, int* g1, int* mt, int* ntile) {
    const int NT1 = gemm_ntiles<BN>(p, true), NT2 = gemm_ntiles<BN>(p, false);
    if (entry >= p.mtile_off[p.E] * (NT1 + NT2)) return false;
    const int nw = (p.E + p.wave_experts - 1) / p.wave_experts;
    sched::FusedCursor cur;
    cur.seek(entry, nw, p.wave_experts, p.E, p.mtile_off, NT1, NT2);
    cur.tile(entry, NT1, NT2, mt, ntile);
    *g1 = cur.sg.g1;
    return true;
}

template <int BM, int BN, int WM, int WN, bool kG1, bool kIL, bool kST>
MOE_DEV int fused_run(const GemmParams& p, int tile, int mt, int ntile, uint8_t* smem) {
    using Eng = TileEngine<BM, BN, WM, WN, kG1, true, kG1 && kIL, kST>;
    Eng eng(p, smem);
    const int nk = eng.nk;
    const bool chain = nk >= (kG1 ? 5 : 2);
    if (!kG1) wait_ready<BN>(p, mt);
    int4 rec = p.mtile_rec[mt];                  // {expert, first position, rows}
    int buf = 0, st = 0;
    eng.load_rows_now(rec, buf);                 // (its barrier also ends the wait above)
    eng.set_tile(rec, ntile, buf);
    eng.prologue(st);
    for (;;) {
        const int nxt = tile + gridDim.x;
        int g1_n = kG1, mt_n = mt, nt_n = ntile;
        const bool has_next = fused_entry<BN>(p, nxt, &g1_n, &mt_n, &nt_n) && (g1_n != 0) == kG1;
        if (!has_next) mt_n = mt, nt_n = ntile;
        const int4 rec_n = p.mtile_rec[mt_n];
        const bool pf = has_next && chain;
        if (!kG1 && pf) wait_ready<BN>(p, mt_n);
        eng.set_rows(rec.z);
        eng.zero_acc();
        for (int ks = 0; ks < nk; ++ks) {
            const int st2 = Eng::next_stage(Eng::next_stage(st));
            eng.step(
                eng.stage_ptr(st), ks == 0,
                [&] {
                    if (pf) {
                        if (ks == 1 || ks == 2) eng.fetch_rows(rec_n, buf ^ 1, ks - 1);
                        if (ks == nk - 2) eng.set_tile(rec_n, nt_n, buf ^ 1);
                    }
                },
                [&] {
                    if (ks + 2 >= nk && !pf) return false;
                    eng.issue(st2);
                    return true;
                });
            st = Eng::next_stage(st);
        }
        eng.finish();
        eng.epilogue(rec, ntile, buf);
        if (kG1) {
            // every thread's coherent h stores have completed (vmcnt(0)) before the barrier
            __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8) | (0 << 14));
            __syncthreads();
            if (threadIdx.x == 0)
                __hip_atomic_fetch_add(p.ready + mt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (!has_next) {
            __syncthreads();                     // LDS free for the next run's engine
            return nxt;
        }
        tile = nxt;
        mt = mt_n;
        ntile = nt_n;
        rec = rec_n;
        buf ^= 1;
        if (!pf) {        // K too short to hide the next tile's set-up: do it here
            if (!kG1) wait_ready<BN>(p, mt);
            eng.load_rows_now(rec, buf);
            eng.set_tile(rec, ntile, buf);
            eng.prologue(st);
        }
    }
}

// GEMM1 -> SwiGLU -> GEMM2 in one persistent launch ("MegaMoE" notes,
// "Scheduler" and "Wave"; "MegaMoE：把通信和计算融合到一个 Mega Kernel", wave-based
// expert processing).  Experts are cut into waves of p.wave_experts; the tile
// list is GEMM1(wave 0), GEMM1(wave 1), GEMM2(wave 0), GEMM1(wave 2),
// GEMM2(wave 1), ..., GEMM2(last wave), each run in the grouped order, and
// workgroup slot q takes list entries q, q + grid, ...  Consecutive entries of
// one family run as one pipelined run (fused_run).  A GEMM1 tile adds one to
// ready[m] once its h columns are stored; a GEMM2 tile of m-tile m starts
// loading when ready[m] counts every GEMM1 n-tile of m (the bucketing stage of
// the call zeroes ready[] before this launch).  A wait longer than kSpinLimit
// polls stops, sets *p.status and lets the tile run (its output is then wrong,
// never a hang).
template <int BM, int BN, int WM, int WN, bool kIL, bool kST>
__global__ __launch_bounds__(64 * WM * WN, 1) void fused_gemm_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    int tile = xcd_slot(), g1, mt, ntile;
    while (fused_entry<BN>(p, tile, &g1, &mt, &ntile)) {
        if (g1)
            tile = fused_run<BM, BN, WM, WN, true, kIL, kST>(p, tile, mt, ntile, smem);
        else
            tile = fused_run<BM, BN, WM, WN, false, kIL, kST>(p, tile, mt, ntile, smem);
    }
}

// Tile configuration: 128 x 512 output tiles over 8 waves, 2 rows x 4 columns
// of 64 x 128 wave tiles (the wave in row 1 is the late one of its SIMD).
// 128-row m-tiles waste fewer padding rows on ragged expert segments than
// 256-row ones, at the MFMA work per K step of a 256 x 256 tile.
constexpr int kBM = 128, kBN = 512, kWM = 2, kWN = 4;
static_assert(kBM == kTileRows, "the workspace tables are sized for kTileRows-row m-tiles");

int gemm_bm() { return kBM; }

// The kernels take more than the default dynamic LDS: raise the limit once per device.
static hipError_t allow_lds(const void* kern, int bytes, DeviceCache& done) {
    int ok = 0;
    return per_device(done, [&](int, int* v) {
        hipError_t err = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        *v = 1;
        return err;
    }, &ok);
}

template <bool kG1, bool kIL, bool kST>
static hipError_t launch_gemm(const GemmParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    using C = Cfg<kBM, kBN, kWM, kWN, kG1>;
    auto kern = grouped_gemm_kernel<kBM, kBN, kWM, kWN, kG1, kIL, kST>;
    const size_t lds = (size_t)C::kLds;
    static DeviceCache lds_set;
    hipError_t err = allow_lds((const void*)kern, (int)lds, lds_set);
    int cus = 0;
    if (err == hipSuccess) err = device_cus(&cus);
    if (err != hipSuccess) return err;
    if (cus <= 0) return hipErrorInvalidDevice;
    const int ntiles = kG1 ? (p.I + kBN / 2 - 1) / (kBN / 2) : (p.H + kBN - 1) / kBN;
    const int64_t upper = (int64_t)p.max_mtiles * ntiles;
    const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(upper, cus));
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(C::kThreads), lds, s, ev0, ev1, 0, p);
    return hipGetLastError();
}

hipError_t launch_gemm1(const GemmParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (p.w_staged) return launch_gemm<true, false, true>(p, s, ev0, ev1);
    return p.w13_il ? launch_gemm<true, true, false>(p, s, ev0, ev1) : launch_gemm<true, false, false>(p, s, ev0, ev1);
}
hipError_t launch_gemm2(const GemmParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    return p.w_staged ? launch_gemm<false, false, true>(p, s, ev0, ev1) : launch_gemm<false, false, false>(p, s, ev0, ev1);
}

template <bool kIL, bool kST>
static hipError_t launch_fused(const GemmParams& p_in, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    using C = Cfg<kBM, kBN, kWM, kWN, true>;
    auto kern = fused_gemm_kernel<kBM, kBN, kWM, kWN, kIL, kST>;
    const size_t lds = (size_t)C::kLds;
    static DeviceCache lds_set;
    hipError_t err = allow_lds((const void*)kern, (int)lds, lds_set);
    int cus = 0;
    if (err == hipSuccess) err = device_cus(&cus);
    if (err != hipSuccess) return err;
    if (cus <= 0) return hipErrorInvalidDevice;
    GemmParams p = p_in;
    const int nt1 = (p.I + kBN / 2 - 1) / (kBN / 2), nt2 = (p.H + kBN - 1) / kBN;
    p.wave_experts = sched::fused_wave_experts(p.T * p.topk, p.E, nt1, cus, kBM);
    // one workgroup per CU, all resident at once: a GEMM2 tile may wait for a GEMM1
    // tile of any other workgroup
    const int64_t upper = (int64_t)p.max_mtiles * (nt1 + nt2);
    const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(upper, cus));
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(C::kThreads), lds, s, ev0, ev1, 0, p);
    return hipGetLastError();
}

hipError_t launch_fused_gemm(const GemmParams& p, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (p.w_staged) return launch_fused<false, true>(p, s, ev0, ev1);
    return p.w13_il ? launch_fused<true, false>(p, s, ev0, ev1) : launch_fused<false, false>(p, s, ev0, ev1);
}

}  // namespace moe
