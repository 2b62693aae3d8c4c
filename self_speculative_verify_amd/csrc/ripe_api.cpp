// Host side of the RIPE C ABI: configuration checks, storage geometry, the
// host copy of the committed lengths, and kernel launches on the caller's
// stream.  See include/ripe.h for the contract of every entry point.
//
// Plain host C++ (HIP runtime API only): the test suite also compiles this
// file with a host compiler and sanitizers, against recording stand-ins of
// the kernel launchers, to check every validation path on the CPU.
#include "ripe.h"
#include "ripe_internal.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>
#include <utility>
#include <vector>

using ripe::Geometry;

struct ripe_cache {
    Geometry g;
    uint8_t* storage;
    std::vector<int32_t> lens;   // [n_layers][B], host copy of the lens section
    ripe::Tuning tuning;         // all zero: the planner decides
    int device;                  // device of the storage (-1 until first needed)
    // sorted row words and launch plans of a call, sized once at creation
    // for the largest call, so that a verification call allocates nothing
    std::vector<uint32_t> rows_buf;
    std::vector<ripe::Plan> plans_buf;
};

namespace {

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

// Handles that ripe_cache_create returned and ripe_destroy has not released.
// Every entry point looks its handle up here, so a handle that was already
// destroyed (or never created) is refused instead of read.
std::mutex g_handles_mu;
std::unordered_set<const ripe_cache*>& handles() {
    static std::unordered_set<const ripe_cache*> h;
    return h;
}

bool live(const ripe_cache* c) {
    if (!c) return false;
    std::lock_guard<std::mutex> lock(g_handles_mu);
    return handles().count(c) != 0;
}

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

namespace {

// a registered handle over d_storage with the given committed lengths
ripe_status new_handle(const Geometry& g, void* d_storage, std::vector<int32_t>&& lens, ripe_cache** out) {
    ripe_cache* c = new (std::nothrow) ripe_cache;
    if (!c) return RIPE_EDEVICE;
    c->g = g;
    c->storage = static_cast<uint8_t*>(d_storage);
    c->lens = std::move(lens);
    std::memset(&c->tuning, 0, sizeof(c->tuning));
    c->device = -1;
    c->rows_buf.assign(ripe::kMaxRowsPerCall, 0u);
    c->plans_buf.resize((ripe::kMaxRowsPerCall + ripe::kMaxRowsPerLaunch - 1) / ripe::kMaxRowsPerLaunch);
    {
        std::lock_guard<std::mutex> lock(g_handles_mu);
        handles().insert(c);
    }
    *out = c;
    return RIPE_OK;
}

}  // namespace

ripe_status ripe_cache_create(const ripe_config* cfg, void* d_storage, size_t bytes,
                              hipStream_t stream, ripe_cache** out) {
    if (!out) return RIPE_EINVAL;
    *out = nullptr;
    if (!valid_config(cfg) || !d_storage || !aligned(d_storage, 256)) return RIPE_EINVAL;
    const Geometry g = geometry(cfg);
    if (bytes < (size_t)g.total) return RIPE_EINVAL;
    if (hipMemsetAsync(d_storage, 0, (size_t)g.total, stream) != hipSuccess) return RIPE_EDEVICE;
    return new_handle(g, d_storage, std::vector<int32_t>((size_t)g.n_layers * g.B, 0), out);
}

ripe_status ripe_cache_open(const ripe_config* cfg, void* d_storage, size_t bytes,
                            hipStream_t stream, ripe_cache** out) {
    if (!out) return RIPE_EINVAL;
    *out = nullptr;
    if (!valid_config(cfg) || !d_storage || !aligned(d_storage, 256)) return RIPE_EINVAL;
    const Geometry g = geometry(cfg);
    if (bytes < (size_t)g.total) return RIPE_EINVAL;
    std::vector<int32_t> lens((size_t)g.n_layers * g.B, 0);
    if (hipMemcpyAsync(lens.data(), static_cast<const uint8_t*>(d_storage) + g.off_lens,
                       lens.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return RIPE_EDEVICE;
    for (const int32_t L : lens)
        if (L < 0 || (int64_t)L > g.cap) return RIPE_EINVAL;
    return new_handle(g, d_storage, std::move(lens), out);
}

void ripe_destroy(ripe_cache* cache) {
    if (!cache) return;
    {
        std::lock_guard<std::mutex> lock(g_handles_mu);
        if (handles().erase(cache) == 0) return;   // not a live handle: nothing to release
    }
    delete cache;
}

ripe_status ripe_set_tuning(ripe_cache* cache, const ripe_tuning* t) {
    if (!live(cache)) return RIPE_EINVAL;
    ripe::Tuning n;
    std::memset(&n, 0, sizeof(n));
    if (t) {
        if (t->kernel < 0 || t->kernel > 2) return RIPE_EINVAL;
        if (t->keys_waves != 0 && t->keys_waves != 4 && t->keys_waves != 8) return RIPE_EINVAL;
        if (t->row_tiles < 0 || t->row_tiles > 2) return RIPE_EINVAL;
        if (t->private_waves < 0 || t->private_waves > 2) return RIPE_EINVAL;
        if (t->items_target < 0 || t->items_target > (1 << 24)) return RIPE_EINVAL;
        if (t->min_chunk < 0 || t->min_chunk > (1 << 24)) return RIPE_EINVAL;
        n.kernel = t->kernel;
        n.keys_waves = t->keys_waves;
        n.row_tiles = t->row_tiles;
        n.private_waves = t->private_waves;
        n.items_target = t->items_target;
        n.min_chunk = t->min_chunk;
    }
    cache->tuning = n;
    return RIPE_OK;
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
    if (!live(cache) || n_rows <= 0 || n_rows > ripe::kMaxRowsPerCall) return 0;
    return ripe::workspace_bound(cache->g, cache->lens.data(), n_rows, cache->tuning);
}

}  // extern "C"

namespace ripe {

// The (sequence, chunk) items of a split launch, longest first (stable), in
// the launch's arguments: workgroups start in that order, so the longest items
// do not start last.  Only for at most kMaxSeqArgs sequences and kMaxPairs
// items; otherwise the launch enumerates (sequence, KV head, chunk) in order.
void order_pairs(VerifyArgs& a, const int32_t* lens, int B) {
    a.n_pairs = 0;
    if (a.nc <= 1 || B > kMaxSeqArgs || a.nc > 1024) return;
    int n = 0;
    for (int b = 0; b < B; ++b) n += a.snc[b];
    if (n > kMaxPairs) return;
    int64_t len[kMaxPairs];
    n = 0;
    for (int b = 0; b < B; ++b)
        for (int c = 0; c < a.snc[b]; ++c) {
            // positions of work: a whole chunk, or what the last one holds
            const int64_t work = lens[b] > 0 ? std::min<int64_t>(a.cl, lens[b] + a.cx - (int64_t)c * a.cl) : 0;
            int k = n++;
            while (k > 0 && len[k - 1] < work) {     // insertion: longest first, stable
                len[k] = len[k - 1];
                a.pairs[k] = a.pairs[k - 1];
                --k;
            }
            len[k] = work;
            a.pairs[k] = (uint16_t)(b | (c << 6));
        }
    a.n_pairs = n;
    a.n_groups = n * a.Hkv;
}

// ripe_verify_attn (n_sink = 0, w_draft = -1), ripe_draft_attn and
// ripe_verify_attn_noalloc.  ws_fixed: d_ws is the library's fixed scratch of
// ws_bytes bytes, and a call is refused (RIPE_ESCRATCH) only when one of its
// launches needs more than that; otherwise the caller's workspace must hold
// at least ripe_workspace_bytes for this row count.  Every argument and every
// launch's partial-state size is checked before the first launch.  Uses the
// handle's preallocated row and plan buffers: no allocation of any kind.
ripe_status attend(ripe_cache* cache, int32_t layer, int32_t n_rows, const int32_t* h_row_blk,
                   const int32_t* h_row_loop, const void* d_q, ripe_kv_view blk_k,
                   ripe_kv_view blk_v, int32_t n_blk, int32_t n_sink, int32_t w_draft,
                   float* d_out, float* d_lse, void* d_ws, size_t ws_bytes, bool ws_fixed,
                   hipStream_t stream) {
    const bool draft = w_draft >= 0;
    if (!live(cache) || layer < 0 || layer >= cache->g.n_layers) return RIPE_EINVAL;
    const Geometry& g = cache->g;
    if (n_rows < 0 || n_rows > kMaxRowsPerCall) return RIPE_EINVAL;
    if (n_rows == 0) return RIPE_OK;
    if (!h_row_blk || !h_row_loop || !d_q || !d_out || !d_lse) return RIPE_EINVAL;
    if (n_blk < 1 || n_blk > g.max_block) return RIPE_EINVAL;
    if (!aligned(d_q, 16) || !aligned(d_out, 16) || !aligned(d_lse, 4)) return RIPE_EINVAL;
    if (!view_ok(blk_k) || !view_ok(blk_v)) return RIPE_EINVAL;
    for (int k = 0; k < n_rows; ++k) {
        if (h_row_blk[k] < 0 || h_row_blk[k] >= n_blk) return RIPE_EINVAL;
        if (h_row_loop[k] < 1 || h_row_loop[k] > g.R) return RIPE_EINVAL;
    }
    if (!ws_fixed && !draft) {
        const size_t bound = ripe_workspace_bytes(cache, n_rows);
        if (ws_bytes < bound || (bound > 0 && (!d_ws || !aligned(d_ws, 256)))) return RIPE_EINVAL;
    }

    // rows sorted by (loop, block offset) so that rows reading the same planes
    // are adjacent
    uint32_t* rows = cache->rows_buf.data();
    for (int k = 0; k < n_rows; ++k)
        rows[k] = (uint32_t)h_row_blk[k] | ((uint32_t)h_row_loop[k] << 8) | ((uint32_t)k << 16);
    // (loop and offset first, then the row index in bits 16..31: the order a
    // stable sort would give, without its temporary buffer)
    std::sort(rows, rows + n_rows, [](uint32_t x, uint32_t y) {
        return ((x << 16) | (x >> 16)) < ((y << 16) | (y >> 16));
    });

    // plan every launch first: each one's partial states must fit the workspace
    const int32_t* lens = cache->lens.data() + (size_t)layer * g.B;
    const int n_launch = (n_rows + kMaxRowsPerLaunch - 1) / kMaxRowsPerLaunch;
    Plan* plans = cache->plans_buf.data();
    for (int l = 0; l < n_launch; ++l) {
        const int k0 = l * kMaxRowsPerLaunch;
        const int here = std::min(kMaxRowsPerLaunch, n_rows - k0);
        plans[l] = make_plan(g, lens, here, rows + k0, draft, cache->tuning);
        if (plans[l].need > 0) {
            if (plans[l].need > ws_bytes) return ws_fixed ? RIPE_ESCRATCH : RIPE_EINVAL;
            if (!d_ws || !aligned(d_ws, 256)) return RIPE_EINVAL;
        }
    }

    VerifyArgs a;
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
    for (int l = 0; l < n_launch; ++l) {
        const int k0 = l * kMaxRowsPerLaunch;
        const Plan& p = plans[l];
        a.rows_here = std::min(kMaxRowsPerLaunch, n_rows - k0);
        for (int k = 0; k < a.rows_here; ++k) a.rows[k] = rows[k0 + k];
        a.M = p.M; a.nrb = p.nrb; a.nc = p.nc; a.cl = p.cl; a.cx = p.cx; a.n_groups = p.n_groups;
        for (int b = 0; b < kMaxSeqArgs; ++b)
            a.snc[b] = b < g.B ? (lens[b] > 0 ? (int32_t)((lens[b] + p.cx + p.cl - 1) / p.cl) : 1) : 0;
        order_pairs(a, lens, g.B);
        a.n_split = 0;
        if (p.nc > 1 && g.B <= kMaxSeqArgs)
            for (int b = 0; b < g.B; ++b)
                if (a.snc[b] > 1) a.split_b[a.n_split++] = (uint8_t)b;
        const hipError_t e = p.rows_kernel ? launch_verify_rows(a, p.rt, p.priv, stream)
                                           : launch_verify_keys(a, p.rt, p.wide, stream);
        if (e != hipSuccess) return RIPE_EDEVICE;
        if (p.nc > 1 && launch_combine(a, stream) != hipSuccess) return RIPE_EDEVICE;
    }
    return RIPE_OK;
}

ripe_status cache_device(ripe_cache* cache, int* device) {
    if (!live(cache)) return RIPE_EINVAL;
    if (cache->device < 0) {
        hipPointerAttribute_t attr;
        if (hipPointerGetAttributes(&attr, cache->storage) != hipSuccess) return RIPE_EDEVICE;
        if (attr.device < 0) return RIPE_EDEVICE;
        cache->device = attr.device;
    }
    *device = cache->device;
    return RIPE_OK;
}

}  // namespace ripe

extern "C" {

ripe_status ripe_verify_attn(ripe_cache* cache, int32_t layer, int32_t n_rows,
                             const int32_t* h_row_blk, const int32_t* h_row_loop,
                             const void* d_q, ripe_kv_view blk_k, ripe_kv_view blk_v,
                             int32_t n_blk, float* d_out, float* d_lse, void* d_ws,
                             size_t ws_bytes, hipStream_t stream) {
    return ripe::attend(cache, layer, n_rows, h_row_blk, h_row_loop, d_q, blk_k, blk_v, n_blk, 0,
                        -1, d_out, d_lse, d_ws, ws_bytes, false, stream);
}

ripe_status ripe_draft_attn(ripe_cache* cache, int32_t layer, int32_t n_rows,
                            const int32_t* h_row_blk, const int32_t* h_row_loop,
                            const void* d_q, ripe_kv_view blk_k, ripe_kv_view blk_v,
                            int32_t n_blk, int32_t n_sink, int32_t w_draft, float* d_out,
                            float* d_lse, hipStream_t stream) {
    if (n_sink < 0 || w_draft < 0) return RIPE_EINVAL;
    return ripe::attend(cache, layer, n_rows, h_row_blk, h_row_loop, d_q, blk_k, blk_v, n_blk,
                        n_sink, w_draft, d_out, d_lse, nullptr, 0, false, stream);
}

const char* ripe_status_string(ripe_status s) {
    switch (s) {
        case RIPE_OK: return "ok";
        case RIPE_EINVAL: return "invalid argument";
        case RIPE_ECAPACITY: return "append exceeds capacity";
        case RIPE_EDEVICE: return "HIP launch or runtime error";
        case RIPE_ESCRATCH: return "call needs more scratch than the library's fixed buffer";
    }
    return "unknown status";
}

}  // extern "C"
