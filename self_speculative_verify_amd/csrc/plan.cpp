// Launch planning of a verification call (plain C++; see plan.h).
#include "plan.h"

#include <algorithm>

namespace ripe {

namespace {

int64_t up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Tiles of the ring and draft-block work of the heaviest row block (rows:
// sorted row words of the launch; null for a bound over every row set).
int64_t extra_tiles(const Geometry& g, const uint32_t* rows, int rows_here, int M, int nrb,
                    int rows_per_item, int64_t lmax) {
    const int G = g.Hq / g.Hkv;
    const int64_t ring_tiles = g.R > 1 ? (std::min<int64_t>(g.WR, lmax) + 31) / 32 : 0;
    if (!rows) {
        const int64_t nl = std::min<int64_t>(rows_per_item / G + 1, g.R);
        return nl * ring_tiles + nl * ((g.max_block + 31) / 32);
    }
    int64_t most = 0;
    for (int rb = 0; rb < nrb; ++rb) {
        const int k_lo = rb * rows_per_item / G;
        const int k_hi = std::min(rows_here, (std::min(M, (rb + 1) * rows_per_item) + G - 1) / G);
        int64_t t = 0;
        for (int k = k_lo; k < k_hi; ++k) {
            const int r = (rows[k] >> 8) & 255, i = rows[k] & 255;
            const bool first = k == k_lo || (int)((rows[k - 1] >> 8) & 255) != r;
            const bool last = k + 1 == k_hi || (int)((rows[k + 1] >> 8) & 255) != r;
            if (first && r < g.R) t += ring_tiles;
            if (last) t += i / 32 + 1;     // rows of a loop are sorted by offset
        }
        most = std::max(most, t);
    }
    return most;
}

}  // namespace

int keys_max_row_tiles(int d) { return d == 128 ? 1 : 2; }
int rows_max_row_tiles(int d) { return d == 96 ? 1 : 2; }
// (instantiated at head_dim 64 and 96)
bool rows_private_waves(int d, int rtw) { return d != 128 && d * rtw < 256; }

// Row-heads (query row x query head of a KV group) of a KV head: with 128 or
// more the "rows" kernel gives each wave 16*rt of them and a workgroup 64*rt;
// with fewer the "keys" kernel gives a whole workgroup 16*rt and splits the
// key tiles between its waves.  Committed positions split into chunks of cl (a
// multiple of 32) when the row blocks alone leave workgroup slots of the chip
// empty (one rows workgroup or two four-wave keys workgroups fit on a compute
// unit); the count stops at one round of slots, so no workgroup waits for
// another to finish, and at chunks long enough that their partial states cost
// little next to the keys they read.  Short keys items instead go unsplit to
// an eight-wave workgroup.  The last chunk of a sequence also takes the ring
// and draft-block tiles of its row block, so it reads cx fewer committed
// positions than the others.  When one round of the rows kernel's row blocks
// already fills the chip, sequences far longer than the mean load of a slot
// are split as well (see below).
Plan make_plan(const Geometry& g, const int32_t* lens, int rows_here, const uint32_t* rows,
               bool draft, const Tuning& t) {
    Plan p;
    p.M = rows_here * (g.Hq / g.Hkv);
    int64_t lmax = 0;
    for (int b = 0; b < g.B; ++b) lmax = std::max<int64_t>(lmax, lens[b]);
    // The rows kernel pays off once a KV head carries a hundred row-heads or
    // more, unless most committed positions lie in the window at a head size
    // without private waves: each loop's ring tiles, which only that loop's
    // rows read, then stream past the other row groups of a rows workgroup,
    // while every wave of a keys workgroup works on its one row block (GQA
    // shape, L = 4096: 400 against 560 us at W = 4000, 366 against 448 at
    // W = 3072, equal at W = 2048, the rows kernel ahead at W = 1024).
    const bool ring_heavy = g.R > 1 && lmax > 0 && !rows_private_waves(g.d, rows_max_row_tiles(g.d)) &&
                            5 * std::min<int64_t>(g.WR, lmax) >= 3 * lmax;
    p.rows_kernel = draft ? false : t.kernel ? t.kernel == 2 : p.M >= 128 && !ring_heavy;
    const int64_t heads = (int64_t)g.B * g.Hkv;
    int rows_per_item;
    if (p.rows_kernel) {
        p.rt = rows_max_row_tiles(g.d);
        if (p.rt > 1 && heads * ((p.M + 64 * p.rt - 1) / (64 * p.rt)) < 256) p.rt = 1;
        rows_per_item = 64;
    } else {
        p.rt = std::min(p.M <= 16 ? 1 : 2, keys_max_row_tiles(g.d));
        rows_per_item = 16;
    }
    if (t.row_tiles > 0 && !draft)
        p.rt = std::min<int>(t.row_tiles, p.rows_kernel ? rows_max_row_tiles(g.d) : keys_max_row_tiles(g.d));
    rows_per_item *= p.rt;
    // private waves pay off when the row blocks have ring tiles to read
    p.priv = p.rows_kernel && rows_private_waves(g.d, p.rt) &&
             (t.private_waves ? t.private_waves == 2 : (g.R > 1 && g.WR > 0));
    p.nrb = (p.M + rows_per_item - 1) / rows_per_item;
    // workgroups of one (sequence, chunk) pair, and of the whole call unsplit
    const int64_t units = (int64_t)g.Hkv * p.nrb;
    const int64_t base = g.B * units;
    const int64_t cx = 32 * extra_tiles(g, rows, rows_here, p.M, p.nrb, rows_per_item, lmax);
    // Keys kernel items of at most 32 tiles (four per wave of eight) are read
    // unsplit by one eight-wave workgroup: no partial states and no combine
    // launch, which on such short items costs more than the split saves (a
    // 2-head, 128-position call of 19-tile items: 15.5 against 18.8 us).
    // Longer items split (a Huginn-scale per-loop call, 35 tiles: 15.8 us
    // split, 16.7 unsplit with eight waves, 17.3 with four).
    const bool auto_wide = !p.rows_kernel && !draft && !t.keys_waves && !t.items_target &&
                           (lmax + 31) / 32 + cx / 32 <= 32;
    p.wide = !p.rows_kernel && !draft && (t.keys_waves ? t.keys_waves == 8 : auto_wide);
    // workgroup target: one round of the rows kernel; for the keys kernel
    // (two workgroups per CU) a second round only pays off on long contexts,
    // where the chunks stay long enough to outweigh the extra partial states
    const int64_t slots_max = draft || auto_wide ? 0 : t.items_target ? t.items_target
                                        : (p.rows_kernel || lmax <= 4096 ? 256 : 512);
    const int64_t min_chunk = t.min_chunk ? up(t.min_chunk, 32)
                                          : std::max<int64_t>(256, 8 * rows_per_item);
    // One chunk length for every sequence, from their total: the pairs that
    // fit one round of slots share the work evenly however ragged the
    // lengths are (a sequence gets ceil((L + cx) / cl) chunks).
    int64_t sum = 0;
    for (int b = 0; b < g.B; ++b) sum += lens[b] > 0 ? lens[b] + cx : 0;
    auto chunk_len = [&](int64_t slots) {
        const int64_t pairs = std::max<int64_t>(1, slots / units);
        return std::max<int64_t>(min_chunk, up((sum + pairs - 1) / pairs, 32));
    };
    int64_t slots = slots_max;
    if (slots == 512 && !t.items_target && base < 256) {
        // ... unless one workgroup per CU already holds the call: a split for
        // 256 slots that stays within 256 workgroups beats the two-per-CU one
        // (the wave, 55 heads at L = 8192: 4 chunks, 220 workgroups, 45.7 us
        // against 9 chunks, 495 workgroups, 48.1 us; 5 chunks, 275
        // workgroups: 56.7 us).  Where the ceilings of a ragged batch push
        // that split past 256 workgroups, two per CU stay (a ragged draft
        // pass: 87.6 against 96.2 us per call).
        const int64_t cl1 = chunk_len(256);
        int64_t n = 0;
        for (int b = 0; b < g.B; ++b) n += lens[b] > 0 ? (lens[b] + cx + cl1 - 1) / cl1 : 1;
        if (units * n <= 256) slots = 256;
    }
    int64_t cl = 0, nc_cap = 1;
    if (base < slots) {
        cl = chunk_len(slots);
        // a bound on the chunk count that never falls as rows or lengths grow
        // (taken at the larger target, which the choice above can only lower)
        nc_cap = std::max<int64_t>(1, std::min<int64_t>(std::max<int64_t>(1, slots_max / units),
                                                        (lmax + cx + min_chunk - 1) / min_chunk));
    } else if (p.rows_kernel && !draft && !t.items_target) {
        // One round of row blocks fills the chip, but a sequence much longer
        // than the mean load of a workgroup slot would still finish last (a
        // ragged batch): split the sequences into chunks no longer than that
        // mean, and the launch hands out the longest items first.
        int64_t sum_l = 0;
        for (int b = 0; b < g.B; ++b) sum_l += lens[b] > 0 ? lens[b] : 0;
        const int64_t mean = (units * sum + slots - 1) / slots;
        if (lmax + cx > mean + mean / 8) cl = std::max<int64_t>(min_chunk, up(mean, 32));
        // for any row set of this size (cx at most this one): chunks are never
        // shorter than the mean without cx
        const int64_t cl_lb = std::max<int64_t>(min_chunk, up((units * sum_l + slots - 1) / slots, 32));
        if (lmax + cx > cl_lb + cl_lb / 8) nc_cap = std::max<int64_t>(1, (lmax + cx + cl_lb - 1) / cl_lb);
    }
    if (cl == 0 || cl >= lmax + cx) {
        p.cx = 0;
        p.cl = std::max<int64_t>(32, up(lmax, 32));
        p.nc = 1;
    } else {
        p.cx = cx;
        p.cl = cl;
        p.nc = (int)((lmax + cx + cl - 1) / cl);
    }
    p.n_groups = (int)(heads * p.nc);
    const size_t state = (size_t)p.M * (g.d + 2) * sizeof(float);   // one chunk of a KV head
    p.need = p.nc > 1 ? (size_t)heads * p.nc * state : 0;
    p.bound = nc_cap > 1 ? (size_t)heads * nc_cap * state : 0;
    return p;
}

size_t workspace_bound(const Geometry& g, const int32_t* lens_all, int n_rows, const Tuning& t) {
    if (n_rows <= 0) return 0;
    // every launch but the last takes kMaxRowsPerLaunch rows; the last takes
    // the rest, and a smaller launch may split its keys into more chunks
    int sizes[2] = {std::min(kMaxRowsPerLaunch, n_rows), n_rows % kMaxRowsPerLaunch};
    if (n_rows <= kMaxRowsPerLaunch) sizes[1] = 0;
    size_t ws = 0;
    for (int layer = 0; layer < g.n_layers; ++layer)     // any layer may be verified
        for (int s : sizes)
            if (s > 0)
                ws = std::max(ws, make_plan(g, lens_all + (size_t)layer * g.B, s, nullptr, false, t).bound);
    return ws;
}

}  // namespace ripe
