// Host side of the RIPE C ABI: configuration checks, storage geometry, the
// host copy of the committed lengths, and kernel launches on the caller's
// stream.  See include/ripe.h for the contract of every entry point.
#include "ripe.h"
#include "ripe_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

using ripe::Geometry;

struct ripe_cache {
    uint64_t magic;
    Geometry g;
    uint8_t* storage;
    std::vector<int32_t> lens;   // [n_layers][B], host copy of the lens section
};

namespace {

constexpr uint64_t kMagic = 0x52495045434143ull;   // "RIPECAC"

int64_t up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

bool valid_config(const ripe_config* c) {
    if (!c) return false;
    if (c->n_layers < 1 || c->n_loops < 1 || c->n_loops > 255) return false;
    if (c->n_heads_kv < 1 || c->n_heads_q < 1 || c->n_heads_q % c->n_heads_kv) return false;
    if (c->head_dim != 64 && c->head_dim != 96 && c->head_dim != 128) return false;
    if (c->window < 0 || c->batch < 1 || c->batch > 4096) return false;
    if (c->capacity < 1 || c->max_block < 1 || c->max_block > 256) return false;
    if (c->anchor != RIPE_ANCHOR_QUERY && c->anchor != RIPE_ANCHOR_CACHE) return false;
    // element counts must stay far from int64 overflow
    const double elems = (double)c->n_layers * c->batch * c->n_heads_kv * c->head_dim *
                         ((double)c->capacity + 32.0) * c->n_loops;
    // an append launch indexes its 4-position groups of all planes in one
    // grid dimension
    const double groups = (c->capacity / 4.0 + 2.0) +
                          (c->n_loops - 1) * (std::min<double>(c->window, c->capacity) / 4.0 + 2.0);
    return elems < 4.0e15 && groups < 2147483647.0;
}

Geometry geometry(const ripe_config* c) {
    Geometry g;
    g.n_layers = c->n_layers; g.R = c->n_loops; g.Hq = c->n_heads_q; g.Hkv = c->n_heads_kv;
    g.d = c->head_dim; g.W = c->window; g.B = c->batch; g.cap = c->capacity;
    g.max_block = c->max_block; g.anchor = c->anchor;
    g.CP = up(c->capacity, ripe::kTile);
    g.NR = c->n_loops - 1;
    g.WR = g.NR == 0 ? 0 : std::min<int64_t>(c->window, c->capacity);
    g.WP = up(g.WR, ripe::kTile);
    const int64_t NL = g.n_layers, B = g.B, H = g.Hkv, d = g.d;
    int64_t off = 0;
    g.off_lens = off;   off = up(off + NL * B * 4, 256);
    g.off_deep_k = off; off = up(off + NL * B * H * g.CP * d * 2, 256);
    g.off_deep_v = off; off = up(off + NL * B * H * g.CP * d * 2, 256);
    g.off_ring_k = off; off = up(off + NL * B * H * g.NR * g.WP * d * 2, 256);
    g.off_ring_v = off; off = up(off + NL * B * H * g.NR * g.WP * d * 2, 256);
    g.total = off;
    return g;
}

bool live(const ripe_cache* c) { return c && c->magic == kMagic; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// a view is usable for vectors of d elements: 16-byte aligned pointer, strides
// non-negative multiples of 8 elements
bool view_ok(const ripe_kv_view& v) {
    if (!v.ptr || !aligned(v.ptr, 16)) return false;
    const int64_t s[4] = {v.s_b, v.s_plane, v.s_head, v.s_tok};
    for (int64_t x : s)
        if (x < 0 || x % 8) return false;
    return true;
}

// How one launch covers a call.  Row-heads (query row x query head of a KV
// group) of a KV head: with 128 or more the "rows" kernel gives each wave
// 16*rt of them and a workgroup 64*rt; with fewer the "keys" kernel gives a
// whole workgroup 16*rt and splits the key tiles between its waves.
// Committed positions split into chunks of cl (a multiple of 32) when the row
// blocks alone leave workgroup slots of the chip empty (one rows workgroup or
// two four-wave keys workgroups fit on a compute unit); the count stops at one
// round of slots, so no workgroup waits for another to finish, and at chunks
// long enough that their partial states cost little next to the keys they
// read.  Short keys items instead go unsplit to an eight-wave workgroup.
// The last chunk of a sequence also takes the ring and draft-block tiles of
// its row block, so it reads cx fewer committed positions than the others.
struct Plan {
    bool rows_kernel;
    bool priv;         // rows kernel with private waves for the ring and block tiles
    bool wide;         // keys kernel with eight waves
    int rt, nrb, nc, n_groups, M;
    int64_t cl, cx;
    size_t ws_bytes;
};

int env_int(const char* name, int fallback) {
    const char* e = std::getenv(name);
    const int v = e ? std::atoi(e) : 0;
    return v > 0 ? v : fallback;
}

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

// draft: a windowed draft call (the keys kernel, one chunk: it reads only the
// sinks and a short window, and needs no workspace)
Plan make_plan(const Geometry& g, const int32_t* lens, int rows_here, const uint32_t* rows,
               bool draft = false) {
    // tuning and test overrides: workgroup target, row tiles, kernel (1 keys, 2 rows)
    const int target_env = env_int("RIPE_ITEMS_TARGET", 0);
    const int force_rt = env_int("RIPE_ROW_TILES", 0);
    const int force_kernel = env_int("RIPE_KERNEL", 0);
    const int force_min_chunk = env_int("RIPE_MIN_CHUNK", 0);
    const int force_priv = env_int("RIPE_PRIV", 0);      // 1 off, 2 on
    const int force_waves = env_int("RIPE_KEYS_WAVES", 0);  // 4 or 8
    Plan p;
    p.M = rows_here * (g.Hq / g.Hkv);
    // the rows kernel pays off once a KV head carries a hundred row-heads or more
    p.rows_kernel = draft ? false : force_kernel ? force_kernel == 2 : p.M >= 128;
    const int64_t heads = (int64_t)g.B * g.Hkv;
    int rows_per_item;
    if (p.rows_kernel) {
        p.rt = ripe::rows_max_row_tiles(g.d);
        if (p.rt > 1 && heads * ((p.M + 64 * p.rt - 1) / (64 * p.rt)) < 256) p.rt = 1;
        rows_per_item = 64;
    } else {
        p.rt = std::min(p.M <= 16 ? 1 : 2, ripe::keys_max_row_tiles(g.d));
        rows_per_item = 16;
    }
    if (force_rt > 0 && !draft) p.rt = std::min(force_rt, p.rows_kernel ? ripe::rows_max_row_tiles(g.d)
                                                              : ripe::keys_max_row_tiles(g.d));
    rows_per_item *= p.rt;
    // private waves pay off when the row blocks have ring tiles to read
    p.priv = p.rows_kernel && ripe::rows_private_waves(g.d, p.rt) &&
             (force_priv ? force_priv == 2 : (g.R > 1 && g.WR > 0));
    p.nrb = (p.M + rows_per_item - 1) / rows_per_item;
    int64_t lmax = 0;
    for (int b = 0; b < g.B; ++b) lmax = std::max<int64_t>(lmax, lens[b]);
    // workgroups of one (sequence, chunk) pair, and of the whole call unsplit
    const int64_t units = (int64_t)g.Hkv * p.nrb;
    const int64_t base = g.B * units;
    // workgroup target: one round of the rows kernel; for the keys kernel
    // (two workgroups per CU) a second round only pays off on long contexts,
    // where the chunks stay long enough to outweigh the extra partial states
    const int64_t cx = 32 * extra_tiles(g, rows, rows_here, p.M, p.nrb, rows_per_item, lmax);
    // Keys kernel items of at most 32 tiles (four per wave of eight) are read
    // unsplit by one eight-wave workgroup: no partial states and no combine
    // launch, which on such short items costs more than the split saves (a
    // 2-head, 128-position call of 19-tile items: 15.5 against 18.8 us).
    // Longer items split (a Huginn-scale per-loop call, 35 tiles: 15.8 us
    // split, 16.7 unsplit with eight waves, 17.3 with four).
    const bool auto_wide = !p.rows_kernel && !draft && !force_waves && !target_env &&
                           (lmax + 31) / 32 + cx / 32 <= 32;
    p.wide = !p.rows_kernel && !draft && (force_waves ? force_waves == 8 : auto_wide);
    const int64_t slots = draft || auto_wide ? 0 : target_env ? target_env
                                    : (p.rows_kernel || lmax <= 4096 ? 256 : 512);
    const int64_t min_chunk = force_min_chunk ? force_min_chunk : std::max<int64_t>(256, 8 * rows_per_item);
    // One chunk length for every sequence, from their total: the pairs that
    // fit one round of slots share the work evenly however ragged the
    // lengths are (a sequence gets ceil((L + cx) / cl) chunks).
    int64_t cl = 0, nc_cap = 1;
    if (base < slots) {
        int64_t sum = 0;
        for (int b = 0; b < g.B; ++b) sum += lens[b] > 0 ? lens[b] + cx : 0;
        const int64_t pairs = slots / units;
        cl = std::max<int64_t>(min_chunk, up((sum + pairs - 1) / std::max<int64_t>(pairs, 1), 32));
        // a bound on the chunk count that never falls as rows or lengths grow
        nc_cap = std::max<int64_t>(1, std::min<int64_t>(pairs, (lmax + cx + min_chunk - 1) / min_chunk));
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
    // whenever a split is possible, so a size queried for a row count holds
    // for every row set of that size
    p.ws_bytes = base < slots ? (size_t)heads * nc_cap * p.M * (g.d + 2) * sizeof(float) : 0;
    return p;
}

ripe::View as_view(const ripe_kv_view& v) {
    return ripe::View{static_cast<const uint16_t*>(v.ptr), v.s_b, v.s_plane, v.s_head, v.s_tok};
}

}  // namespace

extern "C" {

size_t ripe_cache_bytes(const ripe_config* cfg) {
    if (!valid_config(cfg)) return 0;
    return (size_t)geometry(cfg).total;
}

int64_t ripe_section_offset(const ripe_config* cfg, int32_t section) {
    if (!valid_config(cfg)) return -1;
    const Geometry g = geometry(cfg);
    switch (section) {
        case RIPE_SECTION_LENS: return g.off_lens;
        case RIPE_SECTION_DEEP_K: return g.off_deep_k;
        case RIPE_SECTION_DEEP_V: return g.off_deep_v;
        case RIPE_SECTION_RING_K: return g.off_ring_k;
        case RIPE_SECTION_RING_V: return g.off_ring_v;
        case RIPE_SECTION_END: return g.total;
    }
    return -1;
}

int32_t ripe_max_batch(const ripe_config* cfg, size_t budget_bytes) {
    if (!cfg) return -1;
    ripe_config c = *cfg;
    c.batch = 1;
    if (!valid_config(&c)) return -1;
    // storage grows with the batch: bisect for the last batch that fits
    int32_t lo = 0, hi = 4096;
    while (lo < hi) {
        const int32_t mid = lo + (hi - lo + 1) / 2;
        c.batch = mid;
        if (valid_config(&c) && (size_t)geometry(&c).total <= budget_bytes) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

ripe_status ripe_cache_create(const ripe_config* cfg, void* d_storage, size_t bytes,
                              hipStream_t stream, ripe_cache** out) {
    if (!out) return RIPE_EINVAL;
    *out = nullptr;
    if (!valid_config(cfg) || !d_storage || !aligned(d_storage, 256)) return RIPE_EINVAL;
    const Geometry g = geometry(cfg);
    if (bytes < (size_t)g.total) return RIPE_EINVAL;
    ripe_cache* c = new (std::nothrow) ripe_cache;
    if (!c) return RIPE_EDEVICE;
    c->magic = kMagic;
    c->g = g;
    c->storage = static_cast<uint8_t*>(d_storage);
    c->lens.assign((size_t)g.n_layers * g.B, 0);
    if (hipMemsetAsync(d_storage, 0, (size_t)g.total, stream) != hipSuccess) {
        c->magic = 0;
        delete c;
        return RIPE_EDEVICE;
    }
    *out = c;
    return RIPE_OK;
}

void ripe_destroy(ripe_cache* cache) {
    if (!live(cache)) return;
    cache->magic = 0;
    delete cache;
}

ripe_status ripe_get_lengths(const ripe_cache* cache, int32_t layer, int32_t* h_lens) {
    if (!live(cache) || !h_lens || layer < 0 || layer >= cache->g.n_layers) return RIPE_EINVAL;
    std::memcpy(h_lens, cache->lens.data() + (size_t)layer * cache->g.B, sizeof(int32_t) * cache->g.B);
    return RIPE_OK;
}

ripe_status ripe_append(ripe_cache* cache, int32_t layer, const int32_t* h_n_new,
                        ripe_kv_view deep_k, ripe_kv_view deep_v, ripe_kv_view win_k,
                        ripe_kv_view win_v, hipStream_t stream) {
    if (!live(cache) || !h_n_new || layer < 0 || layer >= cache->g.n_layers) return RIPE_EINVAL;
    const Geometry& g = cache->g;
    int32_t* lens = cache->lens.data() + (size_t)layer * g.B;
    int64_t n_tok = 0, n_win = 0;
    for (int b = 0; b < g.B; ++b) {
        if (h_n_new[b] < 0) return RIPE_EINVAL;
        n_tok += h_n_new[b];
        n_win += std::min<int64_t>(h_n_new[b], g.WR);
    }
    for (int b = 0; b < g.B; ++b)
        if ((int64_t)lens[b] + h_n_new[b] > g.cap) return RIPE_ECAPACITY;
    if (n_tok == 0) return RIPE_OK;
    if (!view_ok(deep_k) || !view_ok(deep_v)) return RIPE_EINVAL;
    if (n_win > 0 && (!view_ok(win_k) || !view_ok(win_v))) return RIPE_EINVAL;

    ripe::AppendArgs a;
    std::memset(&a, 0, sizeof(a));
    const int64_t lk = (int64_t)layer * g.B * g.Hkv;
    a.deep_k = reinterpret_cast<uint16_t*>(cache->storage + g.off_deep_k) + lk * g.CP * g.d;
    a.deep_v = reinterpret_cast<uint16_t*>(cache->storage + g.off_deep_v) + lk * g.CP * g.d;
    a.ring_k = reinterpret_cast<uint16_t*>(cache->storage + g.off_ring_k) + lk * g.NR * g.WP * g.d;
    a.ring_v = reinterpret_cast<uint16_t*>(cache->storage + g.off_ring_v) + lk * g.NR * g.WP * g.d;
    a.lens = reinterpret_cast<int32_t*>(cache->storage + g.off_lens) + (int64_t)layer * g.B;
    a.dk = as_view(deep_k);
    a.dv = as_view(deep_v);
    if (n_win > 0) {
        a.wk = as_view(win_k);
        a.wv = as_view(win_v);
    }
    a.Hkv = g.Hkv; a.d = g.d; a.NR = (int32_t)g.NR;
    a.CP = g.CP; a.WR = g.WR; a.WP = g.WP;
    const bool ring = g.NR > 0 && g.WR > 0;
    for (int b0 = 0; b0 < g.B; b0 += ripe::kMaxBatchPerLaunch) {
        a.b0 = b0;
        a.nb = std::min(ripe::kMaxBatchPerLaunch, g.B - b0);
        a.gd = 0;
        a.gr = 0;
        for (int s = 0; s < a.nb; ++s) {
            a.n_new[s] = h_n_new[b0 + s];
            a.L0[s] = lens[b0 + s];
            a.n_win[s] = ring ? (int32_t)std::min<int64_t>(a.n_new[s], g.WR) : 0;
            a.gd = std::max(a.gd, ripe::append_groups(a.L0[s], a.n_new[s]));
            a.gr = (int32_t)std::max<int64_t>(
                a.gr, ripe::append_groups((int64_t)a.L0[s] + a.n_new[s] - a.n_win[s], a.n_win[s]));
        }
        if (a.gd == 0) continue;
        if (ripe::launch_append(a, stream) != hipSuccess) return RIPE_EDEVICE;
    }
    for (int b = 0; b < g.B; ++b) lens[b] += h_n_new[b];
    return RIPE_OK;
}

size_t ripe_workspace_bytes(const ripe_cache* cache, int32_t n_rows) {
    if (!live(cache) || n_rows <= 0) return 0;
    const Geometry& g = cache->g;
    const int32_t* lens = cache->lens.data();
    size_t ws = 0;
    for (int layer = 0; layer < g.n_layers; ++layer) {   // any layer may be verified
        const int rows_here = std::min(ripe::kMaxRowsPerLaunch, (int)n_rows);
        ws = std::max(ws, make_plan(g, lens + (size_t)layer * g.B, rows_here, nullptr).ws_bytes);
    }
    return ws;
}

}  // extern "C"

namespace {

// ripe_verify_attn (n_sink = 0, w_draft = -1) and ripe_draft_attn
ripe_status attend(ripe_cache* cache, int32_t layer, int32_t n_rows, const int32_t* h_row_blk,
                   const int32_t* h_row_loop, const void* d_q, ripe_kv_view blk_k,
                   ripe_kv_view blk_v, int32_t n_blk, int32_t n_sink, int32_t w_draft,
                   float* d_out, float* d_lse, void* d_ws, size_t ws_bytes, hipStream_t stream) {
    const bool draft = w_draft >= 0;
    if (!live(cache) || layer < 0 || layer >= cache->g.n_layers) return RIPE_EINVAL;
    const Geometry& g = cache->g;
    if (n_rows < 0 || n_rows > 65535) return RIPE_EINVAL;
    if (n_rows == 0) return RIPE_OK;
    if (!h_row_blk || !h_row_loop || !d_q || !d_out || !d_lse) return RIPE_EINVAL;
    if (n_blk < 1 || n_blk > g.max_block) return RIPE_EINVAL;
    if (!aligned(d_q, 16) || !aligned(d_out, 16) || !aligned(d_lse, 4)) return RIPE_EINVAL;
    if (!view_ok(blk_k) || !view_ok(blk_v)) return RIPE_EINVAL;
    for (int k = 0; k < n_rows; ++k) {
        if (h_row_blk[k] < 0 || h_row_blk[k] >= n_blk) return RIPE_EINVAL;
        if (h_row_loop[k] < 1 || h_row_loop[k] > g.R) return RIPE_EINVAL;
    }
    const size_t need = draft ? 0 : ripe_workspace_bytes(cache, n_rows);
    if (ws_bytes < need || (need > 0 && (!d_ws || !aligned(d_ws, 256)))) return RIPE_EINVAL;

    // rows sorted by (loop, block offset) so that rows reading the same planes
    // are adjacent
    std::vector<uint32_t> rows((size_t)n_rows);
    for (int k = 0; k < n_rows; ++k)
        rows[k] = (uint32_t)h_row_blk[k] | ((uint32_t)h_row_loop[k] << 8) | ((uint32_t)k << 16);
    std::stable_sort(rows.begin(), rows.end(),
                     [](uint32_t x, uint32_t y) { return (x & 0xffffu) < (y & 0xffffu); });

    ripe::VerifyArgs a;
    std::memset(&a, 0, sizeof(a));
    const int64_t lk = (int64_t)layer * g.B * g.Hkv;
    a.deep_k = reinterpret_cast<const uint16_t*>(cache->storage + g.off_deep_k) + lk * g.CP * g.d;
    a.deep_v = reinterpret_cast<const uint16_t*>(cache->storage + g.off_deep_v) + lk * g.CP * g.d;
    a.ring_k = reinterpret_cast<const uint16_t*>(cache->storage + g.off_ring_k) + lk * g.NR * g.WP * g.d;
    a.ring_v = reinterpret_cast<const uint16_t*>(cache->storage + g.off_ring_v) + lk * g.NR * g.WP * g.d;
    a.lens = reinterpret_cast<const int32_t*>(cache->storage + g.off_lens) + (int64_t)layer * g.B;
    a.q = static_cast<const uint16_t*>(d_q);
    a.bk = as_view(blk_k);
    a.bv = as_view(blk_v);
    a.out = d_out;
    a.lse = d_lse;
    a.part = static_cast<float*>(d_ws);
    a.B = g.B; a.n_rows = n_rows; a.Hq = g.Hq; a.Hkv = g.Hkv; a.group = g.Hq / g.Hkv;
    a.R = g.R; a.d = g.d; a.n_blk = n_blk; a.anchor = g.anchor;
    a.W = g.W; a.CP = g.CP; a.WR = g.WR; a.WP = g.WP; a.NR = g.NR;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)g.d));
    a.n_sink = n_sink;
    a.w_draft = w_draft;
    const int32_t* lens = cache->lens.data() + (size_t)layer * g.B;
    for (int k0 = 0; k0 < n_rows; k0 += ripe::kMaxRowsPerLaunch) {
        a.rows_here = std::min(ripe::kMaxRowsPerLaunch, n_rows - k0);
        for (int k = 0; k < a.rows_here; ++k) a.rows[k] = rows[k0 + k];
        const Plan p = make_plan(g, lens, a.rows_here, a.rows, draft);
        a.M = p.M; a.nrb = p.nrb; a.nc = p.nc; a.cl = p.cl; a.cx = p.cx; a.n_groups = p.n_groups;
        for (int b = 0; b < ripe::kMaxSeqArgs; ++b)
            a.snc[b] = b < g.B ? (lens[b] > 0 ? (int32_t)((lens[b] + p.cx + p.cl - 1) / p.cl) : 1) : 0;
        const hipError_t e = p.rows_kernel ? ripe::launch_verify_rows(a, p.rt, p.priv, stream)
                                           : ripe::launch_verify_keys(a, p.rt, p.wide, stream);
        if (e != hipSuccess) return RIPE_EDEVICE;
        if (p.nc > 1 && ripe::launch_combine(a, stream) != hipSuccess) return RIPE_EDEVICE;
    }
    return RIPE_OK;
}

}  // namespace

extern "C" {

ripe_status ripe_verify_attn(ripe_cache* cache, int32_t layer, int32_t n_rows,
                             const int32_t* h_row_blk, const int32_t* h_row_loop,
                             const void* d_q, ripe_kv_view blk_k, ripe_kv_view blk_v,
                             int32_t n_blk, float* d_out, float* d_lse, void* d_ws,
                             size_t ws_bytes, hipStream_t stream) {
    return attend(cache, layer, n_rows, h_row_blk, h_row_loop, d_q, blk_k, blk_v, n_blk, 0, -1,
                  d_out, d_lse, d_ws, ws_bytes, stream);
}

ripe_status ripe_draft_attn(ripe_cache* cache, int32_t layer, int32_t n_rows,
                            const int32_t* h_row_blk, const int32_t* h_row_loop,
                            const void* d_q, ripe_kv_view blk_k, ripe_kv_view blk_v,
                            int32_t n_blk, int32_t n_sink, int32_t w_draft, float* d_out,
                            float* d_lse, hipStream_t stream) {
    if (n_sink < 0 || w_draft < 0) return RIPE_EINVAL;
    return attend(cache, layer, n_rows, h_row_blk, h_row_loop, d_q, blk_k, blk_v, n_blk, n_sink,
                  w_draft, d_out, d_lse, nullptr, 0, stream);
}

const char* ripe_status_string(ripe_status s) {
    switch (s) {
        case RIPE_OK: return "ok";
        case RIPE_EINVAL: return "invalid argument";
        case RIPE_ECAPACITY: return "append exceeds capacity";
        case RIPE_EDEVICE: return "HIP launch or runtime error";
    }
    return "unknown status";
}

}  // extern "C"
