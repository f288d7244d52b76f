// Tile order of the grouped GEMMs and the tile list of the one-launch GEMM1 ->
// GEMM2 kernel.  Plain integer arithmetic, compiled for the device by the
// kernels and for the host by the schedule model that checks it (every tile
// listed once; every GEMM2 tile after all GEMM1 tiles of its m-tile).  The
// includer defines MOE_HD (the function qualifiers of its compiler).
#pragma once

#include <stdint.h>

#ifndef MOE_HD
#error "define MOE_HD before including sched.h"
#endif

namespace moe {
namespace sched {

constexpr int kGM = 8;                  // m-tiles per tile-order group
constexpr int kXCDs = 8;                // XCDs of the chip, dealt workgroups round-robin

MOE_HD int imin(int a, int b) { return a < b ? a : b; }

// Workgroup slot of workgroup b in a grid of `grid`: workgroup b runs on XCD
// b % 8, so when the grid is a multiple of 8 the grid/8 workgroups of one XCD
// get consecutive slots.  A bijection of [0, grid).
MOE_HD int tile_slot(int b, int grid) {
    return (grid % kXCDs) == 0 ? (b % kXCDs) * (grid / kXCDs) + b / kXCDs : b;
}

// Tile number t of a run of m-tiles [m0, m0 + nm) x nt n-tiles in the grouped
// order: groups of kGM m-tiles x all n-tiles, m fastest inside a group.
MOE_HD void grouped_order(int t, int m0, int nm, int nt, int* mt, int* ntile) {
    const int grp = t / (kGM * nt);
    const int gm = imin(kGM, nm - grp * kGM);
    const int in_grp = t - grp * (kGM * nt);
    *ntile = in_grp / gm;
    *mt = m0 + grp * kGM + (in_grp - *ntile * gm);
}

// Segment s of the one-launch tile list over nw expert waves of ew experts
// ("MegaMoE" study notes, "Scheduler" and "Wave"): GEMM1(wave 0), GEMM1(wave 1),
// GEMM2(wave 0), GEMM1(wave 2), GEMM2(wave 1), ..., GEMM2(last wave).  Segment
// 0 and odd segments are GEMM1 of wave (s + 1) / 2, even segments s > 0 GEMM2
// of wave s / 2 - 1, and the last segment (s = 2 nw - 1) GEMM2 of the last
// wave.  Returns the family (1: GEMM1) and the segment's m-tiles [m0, m0 + nm)
// from the per-expert m-tile prefix sum mtile_off[0..E].
struct Segment {
    int g1, m0, nm;
};
MOE_HD Segment fused_segment(int s, int nw, int ew, int E, const int32_t* mtile_off) {
    int g1, w;
    if (s == 2 * nw - 1) {
        g1 = 0;
        w = nw - 1;
    } else if (s == 0 || (s & 1)) {
        g1 = 1;
        w = (s + 1) / 2;
    } else {
        g1 = 0;
        w = s / 2 - 1;
    }
    const int a = mtile_off[imin(w * ew, E)], b = mtile_off[imin((w + 1) * ew, E)];
    return Segment{g1, a, b - a};
}

// A workgroup's position in the one-launch list: the segment holding its
// current entry.  Entries only move forward (q, q + grid, ...), so seek()
// steps over whole segments, empty ones included.  It stops at the last
// segment, so an entry beyond the list's length (the sum of all segment
// lengths; never asked for) ends with entry >= start + len.
struct FusedCursor {
    int seg, start, len;                // segment index, its first entry and length
    Segment sg;
    MOE_HD FusedCursor() : seg(-1), start(0), len(0), sg{1, 0, 0} {}
    MOE_HD void seek(int entry, int nw, int ew, int E, const int32_t* mtile_off, int nt1, int nt2) {
        while (entry >= start + len && seg + 1 < 2 * nw) {
            start += len;
            ++seg;
            sg = fused_segment(seg, nw, ew, E, mtile_off);
            len = sg.nm * (sg.g1 ? nt1 : nt2);
        }
    }
    // m-tile and n-tile of `entry` (after seek)
    MOE_HD void tile(int entry, int nt1, int nt2, int* mt, int* ntile) const {
        grouped_order(entry - start, sg.m0, sg.nm, sg.g1 ? nt1 : nt2, mt, ntile);
    }
};

// Experts per wave of the one-launch list: enough GEMM1 tiles to give every
// CU about two ("MegaMoE" study notes, "Wave": ceil(2 * SMs / L1 blocks per
// expert)), from the mean rows per expert.
inline int fused_wave_experts(int64_t rows, int E, int ntiles1, int cus, int bm) {
    const int64_t per_expert = rows > E ? (rows + E - 1) / E : 1;
    const int64_t tiles = (per_expert + bm - 1) / bm * ntiles1;
    int64_t ew = (2 * (int64_t)cus + tiles - 1) / tiles;
    ew = ew < 1 ? 1 : (ew > E ? E : ew);
    return (int)ew;
}

}  // namespace sched
}  // namespace moe
