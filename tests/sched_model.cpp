// Host model of the grouped GEMMs' tile order and of the one-launch GEMM1 ->
// GEMM2 tile list, built from the kernels' own header (csrc/sched.h).
//
// For every case (per-expert m-tile counts, n-tiles of both GEMMs, grid, experts
// per wave) it checks:
//   1. tile_slot is a bijection of [0, grid);
//   2. the two-launch order lists every (m-tile, n-tile) exactly once;
//   3. the one-launch list, walked exactly as each workgroup walks it (entries
//      slot, slot + grid, ... through FusedCursor), lists every GEMM1 and every
//      GEMM2 tile exactly once, and every GEMM2 tile of m-tile m comes after all
//      GEMM1 tiles of m in list order;
//   4. progress: workgroups that run their entries in order, a GEMM2 entry only
//      once every GEMM1 n-tile of its m-tile has finished, all finish (no wait
//      that never ends when the whole grid is resident).
// Prints one line per failure and exits nonzero if any check fails.
#include <cstdio>
#include <cstdint>
#include <cstdlib>
#include <vector>

#define MOE_HD inline
#include "sched.h"

using namespace moe::sched;

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(uint32_t n) {        // splitmix64, uniform enough for case generation
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)((z ^ (z >> 31)) % n);
}

static int g_fail = 0;
#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            if (g_fail < 20) {                            \
                std::printf("FAIL %s: ", name);           \
                std::printf(__VA_ARGS__);                 \
                std::printf("\n");                        \
            }                                             \
            ++g_fail;                                     \
            return;                                       \
        }                                                 \
    } while (0)

struct Entry {
    int g1, mt, nt;
};

static void run_case(const char* name, const std::vector<int>& mtiles_per_expert, int nt1, int nt2,
                     int grid, int ew) {
    const int E = (int)mtiles_per_expert.size();
    std::vector<int32_t> off(E + 1, 0);
    for (int e = 0; e < E; ++e) off[e + 1] = off[e] + mtiles_per_expert[e];
    const int M = off[E];
    const int nw = (E + ew - 1) / ew;

    // 1. slots
    std::vector<int> seen(grid, 0);
    for (int b = 0; b < grid; ++b) {
        const int q = tile_slot(b, grid);
        CHECK(q >= 0 && q < grid, "slot %d of workgroup %d outside grid %d", q, b, grid);
        ++seen[q];
    }
    for (int q = 0; q < grid; ++q) CHECK(seen[q] == 1, "slot %d taken %d times", q, seen[q]);

    // 2. two-launch order, both GEMMs
    for (int nt : {nt1, nt2}) {
        std::vector<int> hit((size_t)M * nt, 0);
        for (int t = 0; t < M * nt; ++t) {
            int mt, n;
            grouped_order(t, 0, M, nt, &mt, &n);
            CHECK(mt >= 0 && mt < M && n >= 0 && n < nt, "tile %d -> (%d, %d)", t, mt, n);
            ++hit[(size_t)mt * nt + n];
        }
        for (size_t i = 0; i < hit.size(); ++i) CHECK(hit[i] == 1, "two-launch tile %zu listed %d times", i, hit[i]);
    }

    // 3. one-launch list as each workgroup walks it
    const int total = M * (nt1 + nt2);
    std::vector<Entry> list(total, Entry{-1, -1, -1});
    std::vector<std::vector<int>> mine(grid);
    for (int b = 0; b < grid; ++b) {
        FusedCursor cur;
        for (int t = tile_slot(b, grid); t < total; t += grid) {
            cur.seek(t, nw, ew, E, off.data(), nt1, nt2);
            CHECK(t >= cur.start && t < cur.start + cur.len, "entry %d outside its segment %d [%d, %d)", t,
                  cur.seg, cur.start, cur.start + cur.len);
            int mt, n;
            cur.tile(t, nt1, nt2, &mt, &n);
            list[t] = Entry{cur.sg.g1, mt, n};
            mine[b].push_back(t);
        }
    }
    std::vector<int> g1hit((size_t)M * nt1, 0), g2hit((size_t)M * nt2, 0);
    std::vector<int> last_g1(M, -1), first_g2(M, total);
    for (int t = 0; t < total; ++t) {
        const Entry& x = list[t];
        CHECK(x.mt >= 0 && x.mt < M, "entry %d has m-tile %d (of %d)", t, x.mt, M);
        if (x.g1) {
            CHECK(x.nt >= 0 && x.nt < nt1, "entry %d GEMM1 n-tile %d", t, x.nt);
            ++g1hit[(size_t)x.mt * nt1 + x.nt];
            last_g1[x.mt] = t;
        } else {
            CHECK(x.nt >= 0 && x.nt < nt2, "entry %d GEMM2 n-tile %d", t, x.nt);
            ++g2hit[(size_t)x.mt * nt2 + x.nt];
            if (first_g2[x.mt] == total) first_g2[x.mt] = t;
        }
    }
    for (size_t i = 0; i < g1hit.size(); ++i) CHECK(g1hit[i] == 1, "GEMM1 tile %zu listed %d times", i, g1hit[i]);
    for (size_t i = 0; i < g2hit.size(); ++i) CHECK(g2hit[i] == 1, "GEMM2 tile %zu listed %d times", i, g2hit[i]);
    for (int m = 0; m < M; ++m)
        CHECK(last_g1[m] < first_g2[m], "m-tile %d: GEMM2 entry %d before GEMM1 entry %d", m, first_g2[m],
              last_g1[m]);

    // 4. progress of a resident grid
    std::vector<int> ready(M, 0);
    std::vector<size_t> pos(grid, 0);
    int left = total;
    while (left > 0) {
        bool moved = false;
        for (int b = 0; b < grid; ++b) {
            while (pos[b] < mine[b].size()) {
                const Entry& x = list[mine[b][pos[b]]];
                if (!x.g1 && ready[x.mt] < nt1) break;     // waits on its ready counter
                if (x.g1) ++ready[x.mt];
                ++pos[b];
                --left;
                moved = true;
            }
        }
        CHECK(moved, "no workgroup can proceed with %d entries left", left);
    }
}

int main() {
    int cases = 0;
    // the DeepSeek-V3-like prefill share (1024 rows per expert: 8 or 9 m-tiles),
    // 256 CUs; GEMM1 8 n-tiles (I = 2048), GEMM2 14 (H = 7168)
    {
        std::vector<int> m(32);
        for (int e = 0; e < 32; ++e) m[e] = 8 + (e % 3 == 0);
        run_case("dsv3_prefill", m, 8, 14, 256, fused_wave_experts(32768, 32, 8, 256, 128));
        ++cases;
    }
    // Zipf-skewed routing: one expert at 32 m-tiles, many near-empty or empty
    {
        std::vector<int> m(32);
        for (int e = 0; e < 32; ++e) m[e] = e < 4 ? 32 - 6 * e : (e % 5 == 0 ? 0 : 1 + e % 3);
        run_case("dsv3_skewed", m, 8, 14, 256, fused_wave_experts(32768, 32, 8, 256, 128));
        ++cases;
    }
    // 256 experts of about 256 rows (2 or 3 m-tiles), 8 waves of 32 experts
    {
        std::vector<int> m(256);
        for (int e = 0; e < 256; ++e) m[e] = 2 + (e % 4 == 0);
        run_case("full256", m, 8, 14, 256, fused_wave_experts(65536, 256, 8, 256, 128));
        ++cases;
    }
    // the multi-wave GPU parity shapes: 3072 rows per expert over 8 experts
    {
        std::vector<int> m(8, 24);
        run_case("wave_uniform", m, 8, 2, 256, fused_wave_experts(24576, 8, 8, 256, 128));
        ++cases;
    }
    // random cases: ragged experts, empty experts, grids that are and are not
    // multiples of the XCD count, one expert per wave up to one wave
    for (int i = 0; i < 3000; ++i) {
        const int E = 1 + (int)rnd(40);
        std::vector<int> m(E);
        for (int e = 0; e < E; ++e) m[e] = rnd(4) == 0 ? 0 : (int)rnd(30);
        const int nt1 = 1 + (int)rnd(10), nt2 = 1 + (int)rnd(20);
        const int grids[] = {1, 3, 7, 8, 16, 64, 200, 256};
        const int grid = grids[rnd(8)];
        const int ew = 1 + (int)rnd(E);
        char name[64];
        std::snprintf(name, sizeof name, "random %d (E=%d grid=%d ew=%d)", i, E, grid, ew);
        run_case(name, m, nt1, nt2, grid, ew);
        ++cases;
    }
    std::printf("%d cases, %d failures\n", cases, g_fail);
    return g_fail == 0 ? 0 : 1;
}
