// Host checks of the RIPE library's C ABI, built on the CPU with a host
// compiler (and address / undefined-behaviour sanitizers) from the library's
// own host sources, against stand-ins of the HIP calls and kernel launchers
// defined below.  No GPU is involved: "device" buffers are host memory that
// the stand-ins never read, except the lengths section that the append
// stand-in writes as the append kernel does.
//
// Checks: validation paths leave no side effect (nothing launched, lengths
// unchanged); a destroyed handle is refused, and destroying it again is
// harmless; re-opening storage takes its lengths from the image and refuses
// a length outside [0, capacity]; the workspace that ripe_workspace_bytes returns covers the
// partial states every launch of a call writes, over a sweep of shapes, row
// counts (one launch, several launches with a short last one) and forced
// launch choices.  Exit status 0 and a last line "host checks passed" on
// success.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "ripe.h"
#include "ripe_internal.h"

// ----------------------------------------------------------- stand-ins

namespace {
struct Recorder {
    int appends = 0, verifies = 0, combines = 0;
    int last_nc = 0, last_pairs = 0;                 // of the last verify launch
    const void* ws = nullptr;        // workspace the test passed
    size_t ws_bytes = 0;
    const void* real = nullptr;      // host memory behind the fake storage
    size_t real_bytes = 0;
    int failures = 0;
} rec;

#define CHECK(cond, ...)                                                          \
    do {                                                                          \
        if (!(cond)) {                                                            \
            std::fprintf(stderr, "FAILED %s:%d: %s: ", __FILE__, __LINE__, #cond); \
            std::fprintf(stderr, __VA_ARGS__);                                    \
            std::fprintf(stderr, "\n");                                           \
            ++rec.failures;                                                       \
        }                                                                         \
    } while (0)
}  // namespace

extern "C" hipError_t hipMemsetAsync(void* p, int v, size_t n, hipStream_t) {
    // clears the part of the fake storage that exists in host memory
    if (p == rec.real) std::memset(p, v, n < rec.real_bytes ? n : rec.real_bytes);
    return hipSuccess;
}

extern "C" hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
    // only the lengths section exists in host memory
    const uint8_t* s = static_cast<const uint8_t*>(src);
    const uint8_t* r = static_cast<const uint8_t*>(rec.real);
    if (s < r || s + n > r + rec.real_bytes) return hipErrorInvalidValue;
    std::memcpy(dst, src, n);
    return hipSuccess;
}

extern "C" hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

extern "C" hipError_t hipPointerGetAttributes(hipPointerAttribute_t* a, const void*) {
    std::memset(a, 0, sizeof(*a));
    a->device = 0;
    return hipSuccess;
}

namespace ripe {

hipError_t launch_append(const AppendArgs& a, hipStream_t) {
    ++rec.appends;
    for (int i = 0; i < a.nb; ++i) a.lens[a.b0 + i] = a.L0[i] + a.n_new[i];
    return hipSuccess;
}

// What a verify launch's kernels index: every (sequence, KV head, chunk) item
// below n_groups, chunks of every sequence within nc, and, when nc > 1, the
// partial state of every (sequence, KV head, chunk, row-head) inside the
// workspace.
static void check_verify(const VerifyArgs& a, int rt, const char* kind) {
    rec.last_nc = a.nc;
    rec.last_pairs = a.n_pairs;
    CHECK(a.rows_here >= 1 && a.rows_here <= kMaxRowsPerLaunch, "%s rows_here %d", kind, a.rows_here);
    CHECK(a.M == a.rows_here * a.group, "%s M %d", kind, a.M);
    CHECK(a.cl >= 32 && a.cl % 32 == 0, "%s chunk length %lld", kind, (long long)a.cl);
    if (a.n_pairs == 0) {
        CHECK(a.n_groups == a.B * a.Hkv * a.nc, "%s n_groups", kind);
    } else {
        // every (sequence, chunk < its chunk count) exactly once
        CHECK(a.n_groups == a.n_pairs * a.Hkv && a.n_pairs <= kMaxPairs, "%s pair groups", kind);
        std::vector<int> seen((size_t)a.B * a.nc, 0);
        for (int k = 0; k < a.n_pairs; ++k) {
            const int b = a.pairs[k] & 63, c = a.pairs[k] >> 6;
            CHECK(b < a.B && c < a.snc[b], "%s pair %d out of range", kind, k);
            if (b < a.B && c < a.nc) ++seen[(size_t)b * a.nc + c];
        }
        for (int b = 0; b < a.B; ++b)
            for (int c = 0; c < a.snc[b]; ++c) CHECK(seen[(size_t)b * a.nc + c] == 1, "%s pair (%d, %d)", kind, b, c);
    }
    const int per_item = 16 * rt * (std::strcmp(kind, "rows") == 0 ? 4 : 1);
    CHECK(a.nrb == (a.M + per_item - 1) / per_item, "%s nrb %d", kind, a.nrb);
    for (int k = 1; k < a.rows_here; ++k)
        CHECK((a.rows[k - 1] & 0xffffu) <= (a.rows[k] & 0xffffu), "%s rows unsorted", kind);
    for (int b = 0; b < a.B; ++b) {
        const int64_t L = a.lens[b];
        const int64_t nc_b = L > 0 ? (L + a.cx + a.cl - 1) / a.cl : 1;
        CHECK(nc_b <= a.nc, "%s sequence %d needs %lld chunks of %d", kind, b, (long long)nc_b, a.nc);
        if (b < kMaxSeqArgs) CHECK(a.snc[b] == nc_b, "%s snc[%d]", kind, b);
    }
    if (a.nc > 1) {
        const size_t extent = (size_t)a.B * a.Hkv * a.nc * a.M * (a.d + 2) * sizeof(float);
        CHECK(a.part == rec.ws, "%s partials not in the workspace", kind);
        CHECK(extent <= rec.ws_bytes, "%s partials %zu bytes, workspace %zu", kind, extent, rec.ws_bytes);
    }
}

hipError_t launch_verify_keys(const VerifyArgs& a, int rt, bool wide, hipStream_t) {
    ++rec.verifies;
    CHECK(rt >= 1 && rt <= keys_max_row_tiles(a.d), "keys rt %d", rt);
    CHECK(!(wide && a.w_draft >= 0), "eight-wave keys kernel for a windowed draft");
    check_verify(a, rt, "keys");
    return hipSuccess;
}

hipError_t launch_verify_rows(const VerifyArgs& a, int rt, bool priv, hipStream_t) {
    ++rec.verifies;
    CHECK(rt >= 1 && rt <= rows_max_row_tiles(a.d), "rows rt %d", rt);
    CHECK(!priv || rows_private_waves(a.d, rt), "private waves at d %d rt %d", a.d, rt);
    check_verify(a, rt, "rows");
    return hipSuccess;
}

hipError_t launch_combine(const VerifyArgs& a, hipStream_t) {
    ++rec.combines;
    CHECK(a.nc > 1, "combine of a single chunk");
    // the combine's sequence list: every split sequence once, ascending, or
    // none (every sequence enumerated) for larger batches
    if (a.B > kMaxSeqArgs) {
        CHECK(a.n_split == 0, "combine list for %d sequences", a.B);
    } else {
        int k = 0;
        for (int b = 0; b < a.B; ++b)
            if (a.snc[b] > 1) {
                CHECK(k < a.n_split && a.split_b[k] == b, "combine list misses sequence %d", b);
                ++k;
            }
        CHECK(k == a.n_split && k > 0, "combine list of %d sequences, %d split", a.n_split, k);
    }
    return hipSuccess;
}

}  // namespace ripe

// ----------------------------------------------------------- helpers

namespace {

struct Fake {
    ripe_config cfg;
    std::vector<uint8_t> lens_mem;   // the lens section (the only bytes touched)
    ripe_cache* h = nullptr;
};

bool make(Fake& f, ripe_config c) {
    f.cfg = c;
    const size_t bytes = ripe_cache_bytes(&c);
    if (!bytes) return false;
    const int64_t deep = ripe_section_offset(&c, RIPE_SECTION_DEEP_K);
    f.lens_mem.assign((size_t)deep + 256, 0xAB);
    uint8_t* base = f.lens_mem.data() + (256 - (uintptr_t)f.lens_mem.data() % 256) % 256;
    rec.real = base;
    rec.real_bytes = (size_t)deep;
    return ripe_cache_create(&c, base, bytes, nullptr, &f.h) == RIPE_OK;
}

alignas(256) uint16_t g_dummy[1 << 12];   // stands in for every bf16 device operand
alignas(256) float g_out[1 << 12];

ripe_kv_view view() { return ripe_kv_view{g_dummy, 0, 0, 0, 0}; }

ripe_config config(int NL, int R, int Hq, int Hkv, int d, int W, int B, int cap, int Dmax,
                   int anchor = 0) {
    return ripe_config{NL, R, Hq, Hkv, d, W, B, cap, Dmax, anchor};
}

// append n tokens to every sequence of layer 0 (stand-in launch)
ripe_status append_all(Fake& f, const std::vector<int32_t>& n) {
    return ripe_append(f.h, 0, n.data(), view(), view(), view(), view(), nullptr);
}

// verify rows (random block offsets < n_blk and loops) with a workspace of
// ws_bytes bytes at a fake device address (the stand-ins never dereference it)
ripe_status verify(Fake& f, int n_rows, int n_blk, size_t ws_bytes, std::mt19937& rng) {
    std::vector<int32_t> blk(n_rows), loop(n_rows);
    for (int k = 0; k < n_rows; ++k) {
        blk[k] = (int)(rng() % n_blk);
        loop[k] = 1 + (int)(rng() % f.cfg.n_loops);
    }
    void* ws = ws_bytes ? reinterpret_cast<void*>(uintptr_t{1} << 40) : nullptr;
    rec.ws = ws;
    rec.ws_bytes = ws_bytes;
    return ripe_verify_attn(f.h, 0, n_rows, blk.data(), loop.data(), g_dummy, view(), view(),
                            n_blk, g_out, g_out, ws, ws_bytes, nullptr);
}

}  // namespace

// ----------------------------------------------------------- checks

static void check_validation() {
    std::mt19937 rng(1);
    Fake f;
    CHECK(make(f, config(1, 4, 4, 2, 64, 8, 3, 100, 4)), "create");
    // append: negative count, capacity, bad views -- no launch, lengths unchanged
    const int before = rec.appends;
    CHECK(append_all(f, {-1, 0, 0}) == RIPE_EINVAL, "negative count");
    CHECK(append_all(f, {100, 0, 101}) == RIPE_ECAPACITY, "past capacity");
    int32_t lens[3] = {-1, -1, -1};
    CHECK(ripe_get_lengths(f.h, 0, lens) == RIPE_OK && lens[0] == 0 && lens[2] == 0, "lengths after refusal");
    ripe_kv_view bad = view();
    bad.s_tok = 3;
    std::vector<int32_t> one = {1, 1, 1};
    CHECK(ripe_append(f.h, 0, one.data(), bad, view(), view(), view(), nullptr) == RIPE_EINVAL, "bad view");
    ripe_kv_view mis = view();
    mis.ptr = reinterpret_cast<const uint8_t*>(g_dummy) + 2;
    CHECK(ripe_append(f.h, 0, one.data(), mis, view(), view(), view(), nullptr) == RIPE_EINVAL, "misaligned view");
    CHECK(ripe_append(f.h, 1, one.data(), view(), view(), view(), view(), nullptr) == RIPE_EINVAL, "layer");
    CHECK(rec.appends == before, "a refused append launched");
    CHECK(append_all(f, {100, 7, 99}) == RIPE_OK, "append to capacity");
    CHECK(ripe_get_lengths(f.h, 0, lens) == RIPE_OK && lens[0] == 100 && lens[1] == 7 && lens[2] == 99, "lengths");
    const int32_t* dev_lens = reinterpret_cast<const int32_t*>(rec.real);
    CHECK(dev_lens[0] == 100 && dev_lens[1] == 7 && dev_lens[2] == 99, "storage lengths");
    CHECK(append_all(f, {0, 0, 2}) == RIPE_ECAPACITY, "one past capacity");
    CHECK(ripe_get_lengths(f.h, 0, lens) == RIPE_OK && lens[2] == 99, "lengths after capacity refusal");
    CHECK(dev_lens[2] == 99, "storage lengths after capacity refusal");

    // verify: rows, loops, n_blk, pointers, workspace
    const int v0 = rec.verifies;
    std::vector<int32_t> blk = {0, 3}, loop = {1, 4};
    auto call = [&](int n_blk, const int32_t* b, const int32_t* l, const void* q, void* ws, size_t wsb) {
        return ripe_verify_attn(f.h, 0, 2, b, l, q, view(), view(), n_blk, g_out, g_out, ws, wsb, nullptr);
    };
    CHECK(call(4, blk.data(), loop.data(), g_dummy, nullptr, 0) == RIPE_OK ||
          ripe_workspace_bytes(f.h, 2) > 0, "plain call");
    const int v1 = rec.verifies;
    std::vector<int32_t> blk_bad = {0, 4}, loop0 = {0, 1}, loop5 = {1, 5}, blk_neg = {-1, 0};
    CHECK(call(4, blk_bad.data(), loop.data(), g_dummy, nullptr, 0) == RIPE_EINVAL, "block offset >= n_blk");
    CHECK(call(4, blk_neg.data(), loop.data(), g_dummy, nullptr, 0) == RIPE_EINVAL, "negative offset");
    CHECK(call(4, blk.data(), loop0.data(), g_dummy, nullptr, 0) == RIPE_EINVAL, "loop 0");
    CHECK(call(4, blk.data(), loop5.data(), g_dummy, nullptr, 0) == RIPE_EINVAL, "loop R + 1");
    CHECK(call(5, blk.data(), loop.data(), g_dummy, nullptr, 0) == RIPE_EINVAL, "n_blk > max_block");
    CHECK(call(0, blk.data(), loop.data(), g_dummy, nullptr, 0) == RIPE_EINVAL, "n_blk 0");
    CHECK(call(4, blk.data(), loop.data(), reinterpret_cast<const uint8_t*>(g_dummy) + 8, nullptr, 0) ==
              RIPE_EINVAL, "misaligned q");
    CHECK(call(4, blk.data(), loop.data(), nullptr, nullptr, 0) == RIPE_EINVAL, "null q");
    CHECK(ripe_verify_attn(f.h, 0, 2, blk.data(), loop.data(), g_dummy, view(), view(), 4, nullptr,
                           g_out, nullptr, 0, nullptr) == RIPE_EINVAL, "null out");
    CHECK(rec.verifies == v1, "a refused verify launched");
    (void)v0;

    // a workspace one byte short, or null, is refused whenever one is needed
    ripe_tuning split = {1, 0, 0, 0, 100000, 32};
    CHECK(ripe_set_tuning(f.h, &split) == RIPE_OK, "tuning");
    const size_t need = ripe_workspace_bytes(f.h, 2);
    CHECK(need > 0, "forced split needs a workspace");
    alignas(256) static uint8_t ws_buf[1 << 20];
    CHECK(need <= sizeof(ws_buf), "workspace fits the test buffer");
    rec.ws = ws_buf;
    rec.ws_bytes = need;
    CHECK(call(4, blk.data(), loop.data(), g_dummy, ws_buf, need - 1) == RIPE_EINVAL, "short workspace");
    CHECK(call(4, blk.data(), loop.data(), g_dummy, nullptr, need) == RIPE_EINVAL, "null workspace");
    CHECK(call(4, blk.data(), loop.data(), g_dummy, ws_buf + 16, need) == RIPE_EINVAL, "misaligned workspace");
    CHECK(rec.verifies == v1, "a refused verify launched");
    CHECK(call(4, blk.data(), loop.data(), g_dummy, ws_buf, need) == RIPE_OK, "exact workspace");
    CHECK(rec.verifies == v1 + 1 && rec.combines >= 1, "split call launches verify and combine");

    // tuning fields out of range are refused and change nothing
    ripe_tuning t = {3, 0, 0, 0, 0, 0};
    CHECK(ripe_set_tuning(f.h, &t) == RIPE_EINVAL, "kernel 3");
    t = ripe_tuning{0, 6, 0, 0, 0, 0};
    CHECK(ripe_set_tuning(f.h, &t) == RIPE_EINVAL, "6 waves");
    t = ripe_tuning{0, 0, 0, 0, -1, 0};
    CHECK(ripe_set_tuning(f.h, &t) == RIPE_EINVAL, "negative target");
    CHECK(ripe_workspace_bytes(f.h, 2) == need, "refused tuning changed the plan");
    CHECK(ripe_set_tuning(f.h, nullptr) == RIPE_OK, "reset tuning");

    // windowed draft: negative sink or window
    CHECK(ripe_draft_attn(f.h, 0, 2, blk.data(), loop.data(), g_dummy, view(), view(), 4, -1, 8, g_out,
                          g_out, nullptr) == RIPE_EINVAL, "negative sinks");
    CHECK(ripe_draft_attn(f.h, 0, 2, blk.data(), loop.data(), g_dummy, view(), view(), 4, 2, -1, g_out,
                          g_out, nullptr) == RIPE_EINVAL, "negative draft window");

    // destroy: the handle is refused afterwards, and a second destroy is a no-op
    ripe_cache* h = f.h;
    ripe_destroy(h);
    ripe_destroy(h);
    ripe_destroy(nullptr);
    CHECK(ripe_get_lengths(h, 0, lens) == RIPE_EINVAL, "destroyed handle");
    CHECK(append_all(f, {1, 1, 1}) == RIPE_EINVAL, "append on a destroyed handle");
    CHECK(ripe_workspace_bytes(h, 4) == 0, "workspace of a destroyed handle");
    CHECK(ripe_set_tuning(h, nullptr) == RIPE_EINVAL, "tuning of a destroyed handle");
    int fake_handle = 0;
    ripe_destroy(reinterpret_cast<ripe_cache*>(&fake_handle));   // never created: ignored
}

// ripe_workspace_bytes against what every launch of a call writes
static void check_workspace_sweep() {
    std::mt19937 rng(7);
    struct Shape { int R, Hq, Hkv, d, W, B, Dmax; std::vector<int> lens; };
    const int FULL = RIPE_WINDOW_FULL;
    const std::vector<Shape> shapes = {
        {32, 32, 8, 128, 0, 4, 9, {4096, 4096, 4096, 4096}},           // the GQA shape, 9-token block
        {32, 32, 8, 128, 64, 8, 8, {1024, 32768, 5000, 17000, 2048, 9000, 30001, 1100}},
        {32, 55, 55, 96, 64, 1, 9, {16384}},
        {32, 55, 55, 96, 64, 1, 8, {1024}},
        {32, 55, 55, 96, 1024, 1, 8, {1024}},
        {8, 2, 2, 64, 16, 1, 4, {128}},
        {32, 32, 8, 128, FULL, 4, 8, {4096, 100, 0, 4000}},
        {32, 32, 8, 128, 3072, 4, 8, {4096, 4096, 3000, 4096}},   // window over 60%: keys kernel
        {32, 55, 55, 96, 64, 1, 8, {8192}},                        // one keys workgroup per CU
        {4, 4, 2, 64, 8, 70, 3, {}},
        {32, 55, 55, 96, 64, 1, 32, {8192}},
        {1, 8, 2, 128, 0, 3, 40, {3000, 1, 600}},
    };
    const int row_counts[] = {1, 8, 9, 32, 255, 256, 257, 288, 300, 512, 600, 1024};
    const ripe_tuning tunings[] = {
        {0, 0, 0, 0, 0, 0},             // planner
        {1, 0, 0, 0, 0, 0},             // keys kernel
        {2, 0, 0, 0, 0, 0},             // rows kernel
        {1, 8, 0, 0, 0, 0},
        {1, 0, 0, 0, 100000, 32},       // keys kernel, many chunks
        {2, 0, 0, 0, 100000, 32},       // rows kernel, many chunks
        {2, 0, 2, 2, 0, 0},
        {0, 0, 0, 0, 512, 0},
    };
    long calls = 0;
    for (const Shape& s : shapes) {
        std::vector<int> lens = s.lens;
        if (lens.empty())
            for (int b = 0; b < s.B; ++b) lens.push_back((int)(rng() % 300));
        int cap = 1;
        for (int L : lens) cap = std::max(cap, L);
        Fake f;
        if (!make(f, config(1, s.R, s.Hq, s.Hkv, s.d, s.W, s.B, cap + s.Dmax, s.Dmax))) {
            CHECK(false, "create R=%d d=%d", s.R, s.d);
            continue;
        }
        std::vector<int32_t> n(lens.begin(), lens.end());
        CHECK(append_all(f, n) == RIPE_OK, "prefix append");
        for (const ripe_tuning& t : tunings) {
            CHECK(ripe_set_tuning(f.h, &t) == RIPE_OK, "tuning");
            for (int nr : row_counts) {
                const size_t ws = ripe_workspace_bytes(f.h, nr);
                for (int n_blk : {1, s.Dmax}) {
                    const int before = rec.failures;
                    const ripe_status st = verify(f, nr, n_blk, ws, rng);
                    ++calls;
                    CHECK(st == RIPE_OK, "R=%d Hq=%d d=%d W=%d B=%d rows %d n_blk %d kernel %d target %d: "
                          "status %d with the workspace ripe_workspace_bytes gave (%zu)",
                          s.R, s.Hq, s.d, s.W, s.B, nr, n_blk, t.kernel, t.items_target, (int)st, ws);
                    if (rec.failures > before + 3) return;
                }
            }
        }
        ripe_destroy(f.h);
    }
    std::printf("workspace sweep: %ld calls\n", calls);
}

// A batch whose row blocks fill the chip with one sequence ten times longer
// than the others: the planner splits it and orders the items longest first.
static void check_balance_split() {
    std::mt19937 rng(3);
    Fake f;
    CHECK(make(f, config(1, 32, 32, 8, 128, 64, 4, 3008, 8)), "create");
    CHECK(append_all(f, {3000, 200, 310, 150}) == RIPE_OK, "append");
    const size_t ws = ripe_workspace_bytes(f.h, 256);
    CHECK(ws > 0, "no workspace for a call that splits");
    std::vector<int32_t> blk, loop;
    for (int r = 1; r <= 32; ++r)
        for (int i = 0; i < 8; ++i) {
            blk.push_back(i);
            loop.push_back(r);
        }
    rec.ws = reinterpret_cast<void*>(uintptr_t{1} << 40);
    rec.ws_bytes = ws;
    CHECK(ripe_verify_attn(f.h, 0, 256, blk.data(), loop.data(), g_dummy, view(), view(), 8, g_out, g_out,
                           const_cast<void*>(rec.ws), ws, nullptr) == RIPE_OK, "verify");
    CHECK(rec.last_nc == 3 && rec.last_pairs == 6, "split into %d chunks, %d items", rec.last_nc, rec.last_pairs);
    ripe_destroy(f.h);
    (void)rng;
}

static void check_open() {
    Fake f;
    CHECK(make(f, config(2, 4, 4, 2, 64, 8, 3, 100, 4)), "create");
    CHECK(append_all(f, {100, 7, 0}) == RIPE_OK, "append");
    const size_t bytes = ripe_cache_bytes(&f.cfg);
    uint8_t* base = static_cast<uint8_t*>(const_cast<void*>(rec.real));
    const int appends = rec.appends;
    // a second handle over the same image: the lengths come from storage
    ripe_cache* h2 = nullptr;
    CHECK(ripe_cache_open(&f.cfg, base, bytes, nullptr, &h2) == RIPE_OK && h2, "open");
    int32_t lens[3] = {-1, -1, -1};
    CHECK(h2 && ripe_get_lengths(h2, 0, lens) == RIPE_OK && lens[0] == 100 && lens[1] == 7 && lens[2] == 0,
          "lengths of the opened image");
    CHECK(h2 && ripe_get_lengths(h2, 1, lens) == RIPE_OK && lens[0] == 0 && lens[2] == 0, "layer 1");
    CHECK(h2 && ripe_append(h2, 0, std::vector<int32_t>{1, 0, 0}.data(), view(), view(), view(), view(),
                            nullptr) == RIPE_ECAPACITY, "capacity from the image");
    ripe_destroy(h2);
    // a stored length out of range, a short or misaligned storage: refused, no handle
    int32_t* dev_lens = reinterpret_cast<int32_t*>(base);
    for (const int32_t badlen : {101, -1}) {
        const int32_t keep = dev_lens[4];
        dev_lens[4] = badlen;                     // layer 1, sequence 1
        ripe_cache* h3 = reinterpret_cast<ripe_cache*>(&rec);
        CHECK(ripe_cache_open(&f.cfg, base, bytes, nullptr, &h3) == RIPE_EINVAL && !h3, "length %d", badlen);
        dev_lens[4] = keep;
    }
    ripe_cache* h4 = nullptr;
    CHECK(ripe_cache_open(&f.cfg, base, bytes - 1, nullptr, &h4) == RIPE_EINVAL && !h4, "short storage");
    CHECK(ripe_cache_open(&f.cfg, base + 4, bytes, nullptr, &h4) == RIPE_EINVAL && !h4, "misaligned");
    CHECK(ripe_cache_open(&f.cfg, base, bytes, nullptr, nullptr) == RIPE_EINVAL, "null out");
    CHECK(rec.appends == appends, "open launched work");
    ripe_destroy(f.h);
}

int main() {
    check_validation();
    check_open();
    check_balance_split();
    check_workspace_sweep();
    if (rec.failures) {
        std::printf("%d host check(s) failed\n", rec.failures);
        return 1;
    }
    std::printf("host checks passed\n");
    return 0;
}
