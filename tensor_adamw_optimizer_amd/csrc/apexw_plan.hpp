// apexw_plan.hpp -- the launch plan of a tensor list: which tensor each
// 256-element tile belongs to, where each tile's entry sits in the XCD-major
// tile table, and which table entries a read-pass group loads.
//
// Plain C++17 with no HIP dependency: the host engine builds the plan with
// build_plan(), the kernels index it through the constexpr functions below
// (constexpr functions serve host and device code alike), and the host-only
// checks of the tests compile this header with an ordinary C++ compiler.
//
// The plan follows the multi-tensor launch of the "Apex fused optimizers"
// guide (section 三): tensors of one (parameter dtype, grad dtype) pair share
// one launch, cut into fixed chunks; here a chunk is one 256-element tile that
// never spans two tensors.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <new>
#include <vector>

namespace apexw {

constexpr int kThreads = 64;                  // one wave64 per workgroup
constexpr int kVec = 4;                       // contiguous elements per lane
constexpr int kTile = kThreads * kVec;        // 256 elements per tile
constexpr int kXcds = 8;                      // gfx950: 8 XCDs, workgroups dealt round-robin
constexpr int kReadBatch = 4;                 // tiles per read-pass group
constexpr int kMaxLaunches = 4;               // (param, grad) dtype pairs

// dtype codes of parameters and grads (the values of APEXW_F32 / APEXW_BF16)
constexpr int kF32 = 0;
constexpr int kBF16 = 1;

constexpr int64_t plan_ceil_div(int64_t x, int64_t a) { return (x + a - 1) / a; }

// Position of logical tile k (k >= 0) of a launch in its tile table.  The
// table is stored XCD-major: the dispatcher deals workgroups to the XCDs
// round-robin, so the workgroups one XCD runs (k, k+8, k+16, ...) read
// consecutive entries and share the XCD's L2 lines.  Stripe x of the launch
// holds the tiles k = x (mod 8); stride = ceil(tile_count / 8) entries each.
constexpr int64_t table_position(int64_t table_begin, int64_t stride, int64_t k) {
    const uint64_t uk = (uint64_t)k;                  // shifts, not divisions
    return table_begin + (int64_t)(uk % kXcds) * stride + (int64_t)(uk / kXcds);
}

// The 8-bit update kernel takes two consecutive tiles (blocks) per
// workgroup: pair p = tiles 2p, 2p+1 of the launch.  The pair workgroup w of
// P takes: the dispatcher deals consecutive workgroups to the XCDs in turn,
// and each XCD has its own L2, while a block's two scales are 4-byte values
// whose 128-byte lines hold the scales of 16 pairs; taking pair w on
// workgroup w put those 16 pairs on eight XCDs, and each of their L2s
// fetched and wrote back the line.  Here runs of kQ8PairRun consecutive
// pairs go to one XCD: in each window of kXcds * kQ8PairRun workgroups,
// workgroup kXcds*j + x takes pair kQ8PairRun*x + j (a transpose, so every
// pair is taken once); workgroups past the last whole window take their own
// index.  On the LoRA list the kernel's HBM traffic went from 1.0625 to
// 1.0124 times the algorithmic bytes and the step from 43.6-43.8 to
// 42.4-42.5 us (MI355X, three alternating runs each; runs of 8 pairs: 1.019
// times, 42.4-42.6 us).
constexpr uint32_t kQ8PairRun = 16;
constexpr uint32_t q8_pair_of_workgroup(uint32_t w, uint32_t P) {
    constexpr uint32_t W = (uint32_t)kXcds * kQ8PairRun;
    if (w >= P / W * W) return w;
    const uint32_t r = w % W;
    return w - r + (r % (uint32_t)kXcds) * kQ8PairRun + r / (uint32_t)kXcds;
}

// Number of read-pass groups of a launch whose stripes hold `stride` entries.
constexpr int64_t read_groups(int64_t stride) {
    return kXcds * plan_ceil_div(stride, kReadBatch);
}

// Group j of a read pass: XCD stripe x = j % 8, entries 4c .. 4c+3 of it with
// c = j / 8, i.e. the logical tiles k0 + 8u for u = 0..3, k0 = x + 32c, read
// with one 4-entry load starting at table position pos0.
struct ReadWindow {
    int64_t k0;
    int64_t pos0;
};

constexpr ReadWindow read_window(int64_t table_begin, int64_t stride, int64_t j) {
    const int64_t x = j % kXcds, c = j / kXcds;
    return ReadWindow{x + (int64_t)kXcds * kReadBatch * c, table_begin + x * stride + kReadBatch * c};
}

// Tile-table entries the workspace reserves: every launch's stripes padded to
// a multiple of 8, and room for a 4-entry read window that starts at the last
// entry of the last stripe.
constexpr int64_t table_entries_reserved(int64_t n_tiles) {
    return n_tiles + (int64_t)kMaxLaunches * kXcds + kReadBatch;
}

// One launch: the tiles of every tensor of one dtype pair.
struct PlanLaunch {
    int pt, gt;
    int64_t tile_begin, tile_count;     // logical tiles [begin, begin+count) of the list
    int64_t table_begin, table_stride;  // its XCD-major slice of the tile table
    int32_t tensor_begin, tensor_count; // its tensors: tensor_list[begin, begin+count)
};

struct Plan {
    std::vector<PlanLaunch> launches;   // only dtype pairs that hold a tensor
    std::vector<int32_t> tiles;         // the tile table: tensor of each entry
    std::vector<int32_t> tensor_list;   // tensors launch by launch, the largest last
    std::vector<int64_t> first_tile;    // per tensor: its first logical tile
    int64_t n_tiles = 0;
};

// The plan of a list of n tensors: launches in the fixed pair order (fp32,
// fp32), (fp32, bf16), (bf16, fp32), (bf16, bf16); within a launch, tensors in
// list order except that the one with the most tiles (the first such) goes
// last, and each tensor's ceil(numel/256) tiles in order; logical tile k of a
// launch is stored at table_position(table_begin, stride, k), and the padding
// entries of the last column hold 0.  Workgroups are dispatched in logical
// tile order, so the launch ends on full tiles of its largest tensor rather
// than on a small tensor's tile -- which is its first tile (it also forms the
// next step's bias corrections) and often partial, both longer paths.  An
// empty tensor joins its launch's tensor list with no tile.  Returns false if
// memory runs out.
inline bool build_plan(int32_t n, const int64_t *numel, const int32_t *pdt, const int32_t *gdt,
                       Plan *out) {
    try {
        Plan p;
        p.first_tile.assign((size_t)n, 0);
        p.tensor_list.reserve((size_t)n);
        for (int32_t i = 0; i < n; ++i) p.n_tiles += plan_ceil_div(numel[i], kTile);
        p.tiles.reserve((size_t)(p.n_tiles + kMaxLaunches * kXcds));
        const int pairs[kMaxLaunches][2] = {{kF32, kF32}, {kF32, kBF16}, {kBF16, kF32}, {kBF16, kBF16}};
        int64_t logical = 0;
        std::vector<int32_t> order, members;
        for (int q = 0; q < kMaxLaunches; ++q) {
            PlanLaunch L{pairs[q][0], pairs[q][1], logical, 0, (int64_t)p.tiles.size(), 0,
                         (int32_t)p.tensor_list.size(), 0};
            order.clear();
            members.clear();
            for (int32_t i = 0; i < n; ++i)
                if (pdt[i] == L.pt && gdt[i] == L.gt) members.push_back(i);
            if (!members.empty()) {
                size_t big = 0;
                for (size_t u = 1; u < members.size(); ++u)
                    if (numel[members[u]] > numel[members[big]]) big = u;
                std::rotate(members.begin() + (ptrdiff_t)big, members.begin() + (ptrdiff_t)big + 1,
                            members.end());
            }
            for (const int32_t i : members) {
                p.tensor_list.push_back(i);
                p.first_tile[(size_t)i] = logical + (int64_t)order.size();
                order.insert(order.end(), (size_t)plan_ceil_div(numel[i], kTile), i);
            }
            L.tile_count = (int64_t)order.size();
            L.tensor_count = (int32_t)p.tensor_list.size() - L.tensor_begin;
            if (L.tensor_count == 0) continue;
            L.table_stride = plan_ceil_div(L.tile_count, kXcds);
            p.tiles.resize(p.tiles.size() + (size_t)(L.table_stride * kXcds), 0);
            for (int64_t k = 0; k < L.tile_count; ++k)
                p.tiles[(size_t)table_position(L.table_begin, L.table_stride, k)] = order[(size_t)k];
            logical += L.tile_count;
            p.launches.push_back(L);
        }
        *out = std::move(p);
        return true;
    } catch (const std::bad_alloc &) {
        return false;
    }
}

}  // namespace apexw
