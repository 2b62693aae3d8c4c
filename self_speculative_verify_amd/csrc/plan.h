// Host-side planning of the RIPE library: storage geometry of a configuration
// and the launch plan of a verification call.  Plain C++ with no HIP types, so
// the same code is compiled into the library and, on the CPU, into the host
// checks of the test suite (sanitizer builds included).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace ripe {

constexpr int kTile = 32;          // rows (positions or ring slots) per tile
constexpr int kMaxBatchPerLaunch = 64;
constexpr int kMaxRowsPerLaunch = 256;
constexpr int kMaxRowsPerCall = 65535;
constexpr int kMaxSeqArgs = 64;
constexpr int kMaxPairs = 256;     // (sequence, chunk) items listed in a launch's arguments

// Storage geometry derived from a configuration (all counts, no bytes).
struct Geometry {
    int32_t n_layers, R, Hq, Hkv, d, W, B, cap, max_block, anchor;
    int64_t CP;   // deep rows per (layer, seq, head), multiple of 32
    int64_t WR;   // ring slots in use
    int64_t WP;   // ring rows allocated, multiple of 32
    int64_t NR;   // ring planes (R - 1)
    int64_t off_lens, off_deep_k, off_deep_v, off_ring_k, off_ring_v, total;
};

// Fixed plan choices for tuning sweeps and for tests that force every kernel
// variant; 0 in a field leaves that choice to the planner.
struct Tuning {
    int32_t kernel;         // 1 keys kernel, 2 rows kernel
    int32_t keys_waves;     // 4 or 8 waves in a keys workgroup
    int32_t row_tiles;      // row tiles (16 row-heads each) per wave
    int32_t private_waves;  // rows kernel: 1 without, 2 with private waves
    int32_t items_target;   // workgroup slots the chunk split aims to fill
    int32_t min_chunk;      // shortest chunk of committed positions
};

// How one launch covers a call (see make_plan).
struct Plan {
    bool rows_kernel;
    bool priv;         // rows kernel with private waves for the ring and block tiles
    bool wide;         // keys kernel with eight waves
    int rt, nrb, nc, n_groups, M;
    int64_t cl, cx;
    // partial-state bytes this launch writes (0 when every sequence is one chunk)
    size_t need;
    // partial-state bytes that bound `need` over every row set of this row
    // count at these lengths
    size_t bound;
};

// Head sizes and row tiles the kernels are instantiated for.
int keys_max_row_tiles(int d);
int rows_max_row_tiles(int d);
bool rows_private_waves(int d, int rt);

// Plan of one launch of rows_here (<= kMaxRowsPerLaunch) rows at the lengths
// lens[B] of one layer.  rows: the launch's sorted row words (bits 0..7 block
// offset, 8..15 loop); null plans for every row set of that size.  draft: a
// windowed draft call (keys kernel, one chunk, no workspace).
Plan make_plan(const Geometry& g, const int32_t* lens, int rows_here, const uint32_t* rows,
               bool draft, const Tuning& t);

// Workspace bytes that cover every launch of any call of n_rows rows on any
// layer at the lengths lens_all[n_layers][B]: the launches of kMaxRowsPerLaunch
// rows and the one of the remaining n_rows % kMaxRowsPerLaunch.
size_t workspace_bound(const Geometry& g, const int32_t* lens_all, int n_rows, const Tuning& t);

}  // namespace ripe
