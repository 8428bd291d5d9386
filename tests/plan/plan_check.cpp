// Host-only checks of the launch plan (apexw_plan.hpp) on random tensor
// lists, built with an ordinary C++ compiler under AddressSanitizer and
// UndefinedBehaviorSanitizer: every table read below indexes a std::vector
// sized exactly like the workspace region the engine reserves, so a read
// past it is reported by the sanitizer as well as by the explicit checks.
//
// For every list (including empty tensors, 1-element tensors and lists with
// one dtype pair or all four):
//  1. coverage: the tiles of each launch, through the tile table, cover every
//     element of every tensor exactly once, and a tile never spans tensors;
//  2. table_position maps the launch's logical tiles one-to-one into its
//     padded XCD stripes [table_begin, table_begin + 8*stride), and the
//     entries it never hits are exactly the padding at the stripes' ends;
//  3. read_window: every 4-entry load of a read group lies inside the
//     reserved table (table_entries_reserved), its live entries are the
//     table_position of their tiles, and the groups together visit every
//     tile of the launch exactly once;
//  4. q8_pair_of_workgroup: over the 8-bit kernel's grid of ceil(tiles / 2)
//     workgroups it takes every pair exactly once, its first tile inside the
//     launch, and within each whole window every workgroup of an XCD takes a
//     pair of that XCD's run (checked per launch and for grids of every size
//     up to 4096 and a few large ones).
//
// Usage: plan_check <lists> <seed>; prints "lists N tensors T tiles K ok".
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "apexw_plan.hpp"

using namespace apexw;

static int failures = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            if (failures < 20) {                           \
                fprintf(stderr, "FAIL %s: ", #cond);       \
                fprintf(stderr, __VA_ARGS__);              \
                fputc('\n', stderr);                       \
            }                                              \
            ++failures;                                    \
        }                                                  \
    } while (0)

static void check_pairs(int64_t tiles);

static void check_list(const std::vector<int64_t> &numel, const std::vector<int32_t> &pdt,
                       const std::vector<int32_t> &gdt, int64_t *tiles_seen) {
    const int32_t n = (int32_t)numel.size();
    Plan p;
    CHECK(build_plan(n, numel.data(), pdt.data(), gdt.data(), &p), "build_plan");
    // the table as the workspace holds it: exactly the reserved entries
    std::vector<int32_t> table((size_t)table_entries_reserved(p.n_tiles), -7);
    CHECK(p.tiles.size() <= table.size(), "table %zu > reserved %zu", p.tiles.size(), table.size());
    for (size_t e = 0; e < p.tiles.size() && e < table.size(); ++e) table[e] = p.tiles[e];

    // per tensor: which of its tiles were visited (coverage counts)
    std::vector<std::vector<int>> hits((size_t)n);
    for (int32_t i = 0; i < n; ++i) hits[(size_t)i].assign((size_t)plan_ceil_div(numel[(size_t)i], kTile), 0);

    int64_t logical = 0, table_used = 0;
    std::vector<int> in_list((size_t)n, 0);
    for (const PlanLaunch &L : p.launches) {
        CHECK(L.tile_begin == logical, "launch tile_begin %lld != %lld", (long long)L.tile_begin, (long long)logical);
        CHECK(L.table_begin == table_used, "launch table_begin");
        CHECK(L.table_stride == plan_ceil_div(L.tile_count, kXcds), "stride");
        for (int32_t j = 0; j < L.tensor_count; ++j) {
            const int32_t i = p.tensor_list[(size_t)(L.tensor_begin + j)];
            CHECK(pdt[(size_t)i] == L.pt && gdt[(size_t)i] == L.gt, "tensor %d in the wrong launch", i);
            in_list[(size_t)i] += 1;
        }
        // 1 + 2: positions of the logical tiles
        const int64_t span = (int64_t)kXcds * L.table_stride;
        std::vector<int> pos_hit((size_t)span, 0);
        for (int64_t k = 0; k < L.tile_count; ++k) {
            const int64_t pos = table_position(L.table_begin, L.table_stride, k);
            CHECK(pos >= L.table_begin && pos < L.table_begin + span, "position outside the stripes");
            if (pos < L.table_begin || pos >= L.table_begin + span) continue;
            pos_hit[(size_t)(pos - L.table_begin)] += 1;
            const int32_t i = table[(size_t)pos];
            CHECK(i >= 0 && i < n, "table entry %d", i);
            if (i < 0 || i >= n) continue;
            CHECK(pdt[(size_t)i] == L.pt && gdt[(size_t)i] == L.gt, "tile of another launch");
            const int64_t base = (L.tile_begin + k - p.first_tile[(size_t)i]) * kTile;
            CHECK(base >= 0 && base < numel[(size_t)i], "tile base %lld outside tensor %d of %lld",
                  (long long)base, i, (long long)numel[(size_t)i]);
            if (base < 0 || base >= numel[(size_t)i]) continue;
            CHECK(base % kTile == 0, "tile base");
            hits[(size_t)i][(size_t)(base / kTile)] += 1;
        }
        const int64_t pad = span - L.tile_count;
        CHECK(pad >= 0 && pad < kXcds, "padding %lld", (long long)pad);
        for (int64_t e = 0; e < span; ++e) {
            const int64_t x = e / (L.table_stride ? L.table_stride : 1);
            const int64_t c = e - x * L.table_stride;
            // the padding: the last entry of the stripes x >= tile_count % 8
            const bool padding = c == L.table_stride - 1 && L.tile_count % kXcds != 0 &&
                                 x >= L.tile_count % kXcds;
            CHECK(pos_hit[(size_t)e] == (padding ? 0 : 1), "entry %lld hit %d times (padding %d)",
                  (long long)e, pos_hit[(size_t)e], (int)padding);
        }
        // 3: read groups
        std::vector<int> visited((size_t)L.tile_count, 0);
        const int64_t groups = read_groups(L.table_stride);
        for (int64_t jg = 0; jg < groups; ++jg) {
            const ReadWindow w = read_window(L.table_begin, L.table_stride, jg);
            if (w.k0 >= L.tile_count) continue;                  // a group past the end
            CHECK(w.pos0 >= 0 && w.pos0 + kReadBatch <= (int64_t)table.size(),
                  "read window [%lld, %lld) outside the reserved table of %zu", (long long)w.pos0,
                  (long long)(w.pos0 + kReadBatch), table.size());
            int32_t row[kReadBatch];
            for (int u = 0; u < kReadBatch; ++u) row[u] = table.at((size_t)(w.pos0 + u));
            for (int u = 0; u < kReadBatch; ++u) {
                const int64_t k = w.k0 + (int64_t)kXcds * u;
                if (k >= L.tile_count) continue;
                CHECK(w.pos0 + u == table_position(L.table_begin, L.table_stride, k),
                      "window entry is not the tile's position");
                CHECK(row[u] == table[(size_t)table_position(L.table_begin, L.table_stride, k)],
                      "window entry");
                visited[(size_t)k] += 1;
            }
        }
        for (int64_t k = 0; k < L.tile_count; ++k)
            CHECK(visited[(size_t)k] == 1, "tile %lld visited %d times by the read groups",
                  (long long)k, visited[(size_t)k]);
        // 4: the 8-bit kernel's pairs
        check_pairs(L.tile_count);
        logical += L.tile_count;
        table_used += span;
        *tiles_seen += L.tile_count;
    }
    CHECK(logical == p.n_tiles, "tiles %lld != %lld", (long long)logical, (long long)p.n_tiles);
    CHECK(table_used == (int64_t)p.tiles.size(), "table size");
    for (int32_t i = 0; i < n; ++i) {
        CHECK(in_list[(size_t)i] == 1, "tensor %d in %d launch lists", i, in_list[(size_t)i]);
        for (size_t t = 0; t < hits[(size_t)i].size(); ++t)
            CHECK(hits[(size_t)i][t] == 1, "tensor %d tile %zu covered %d times", i, t,
                  hits[(size_t)i][t]);
    }
}

// Check 4 for a launch of `tiles` tiles: the grid of the 8-bit carried kernel
// (ceil(tiles / 2) workgroups) maps one-to-one onto the pairs, every pair's
// first tile lies in the launch, and in whole windows the pair of workgroup w
// lies in the run of w's XCD.
static void check_pairs(int64_t tiles) {
    const uint32_t P = (uint32_t)((tiles + 1) / 2);
    const uint32_t W = (uint32_t)kXcds * kQ8PairRun;
    std::vector<int> taken((size_t)P, 0);
    for (uint32_t w = 0; w < P; ++w) {
        const uint32_t p = q8_pair_of_workgroup(w, P);
        CHECK(p < P, "pair %u of workgroup %u outside the grid of %u", p, w, P);
        if (p >= P) continue;
        taken[(size_t)p] += 1;
        CHECK(2 * (int64_t)p < tiles, "pair %u starts past the launch's %lld tiles", p,
              (long long)tiles);
        if (w < P / W * W)
            CHECK(p / W == w / W && (p % W) / kQ8PairRun == w % (uint32_t)kXcds,
                  "workgroup %u (XCD %u) takes pair %u outside its run", w, w % (uint32_t)kXcds, p);
    }
    for (uint32_t p = 0; p < P; ++p)
        CHECK(taken[(size_t)p] == 1, "pair %u taken %d times (grid %u)", p, taken[(size_t)p], P);
}

int main(int argc, char **argv) {
    const int lists = argc > 1 ? atoi(argv[1]) : 300;
    std::mt19937_64 rng(argc > 2 ? strtoull(argv[2], nullptr, 10) : 1);
    int64_t tensors = 0, tiles = 0;
    for (int l = 0; l < lists; ++l) {
        const int n = (int)(rng() % 40) + (l % 7 == 0 ? 0 : 1);       // some empty lists
        const int pairs = (int)(rng() % 4) + 1;                        // dtype pairs in use
        std::vector<int64_t> numel((size_t)n);
        std::vector<int32_t> pdt((size_t)n), gdt((size_t)n);
        for (int i = 0; i < n; ++i) {
            const uint64_t r = rng() % 10;
            numel[(size_t)i] = r == 0 ? 0 : r == 1 ? 1 : r == 2 ? 256 * (int64_t)(rng() % 9)
                             : r == 3 ? 256 * (int64_t)(rng() % 9) + 1
                                      : (int64_t)(rng() % 300000);
            const int q = (int)(rng() % pairs);
            pdt[(size_t)i] = q >> 1;
            gdt[(size_t)i] = q & 1;
        }
        check_list(numel, pdt, gdt, &tiles);
        tensors += n;
    }
    // one list of the many-small shape: 20,000 tensors of 64 .. 65,536 elements
    {
        std::vector<int64_t> numel(20000);
        std::vector<int32_t> pdt(20000, kF32), gdt(20000, kF32);
        for (auto &x : numel) x = 64 + (int64_t)(rng() % 65473);
        check_list(numel, pdt, gdt, &tiles);
        tensors += 20000;
    }
    for (int64_t t = 0; t <= 8192; ++t) check_pairs(t);
    for (int64_t t : {94976LL, 94977LL, 2097152LL, 8388611LL}) check_pairs(t);
    printf("lists %d tensors %lld tiles %lld %s\n", lists + 1, (long long)tensors,
           (long long)tiles, failures ? "FAILED" : "ok");
    return failures ? 1 : 0;
}
