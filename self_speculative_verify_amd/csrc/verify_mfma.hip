// Matrix-core verification attention (gfx950, v_mfma_f32_16x16x32_bf16).
//
// The D x R verification grid puts D*R*(Hq/Hkv) query rows on every key tile
// of the shared deepest-plane tail (page "Prefix Keys and Values Matter
// Late", abstract: RIPE keeps loop R of every position, and verification runs
// the block at every loop), so Q.K^T and P.V over the tail are dense
// contractions and run on the matrix cores.
//
// A row-head is one (query row, query head of the KV group).  A work item is
// (sequence b, KV head g, block of row-heads, chunk of committed positions);
// its keys come in 32-row tiles of three kinds:
//   deep tiles  - loop R, positions < e_row of each row-head (every chunk);
//   ring tiles  - the window at loop r < R, one plane per loop present
//                 (last chunk only);
//   block tiles - the draft block at each loop present (last chunk only).
// For one key tile and 16 row-heads a wave computes S^T = K.Q^T (lane =
// row-head, registers = keys), masks, updates the online softmax in the log2
// domain and accumulates O^T += V^T.P^T, with P split into two bf16 terms
// (hi + lo) so the value weights keep ~16 significant bits.  K and V operands
// are 16-byte pieces of the storage tiles, which hold keys as 32x32 blocks and
// values transposed, in exactly the operand order of the instruction.
//
// Two kernels share that tile step:
//   k_verify_rows - many row-heads per KV head (the D x R grid).  Eight
//                   waves: four row groups of 16*RTW row-heads, each split
//                   into two key halves (even and odd tiles).  The tile stream
//                   is staged once per workgroup through a 5-, 6- or 10-stage
//                   LDS pipeline (head_dim 128, 96, 64) fed by direct
//                   global->LDS loads from all eight waves.  With private
//                   waves (four more, one per row group) the ring and block
//                   tiles, which only that row group's loops read, go from
//                   memory into the private wave's registers beside the deep
//                   stream; without them the ring tiles follow the deep tiles
//                   in the stream and the block tiles come after the loop.
//   k_verify_keys - few row-heads (a wave, or a small grid).  The four (or
//                   eight) waves hold the same row-heads, split the key tiles
//                   between them and merge their softmax states through LDS.
// A single-chunk item writes O and LSE; otherwise each chunk writes its
// partial state (m, l, O) and k_combine merges them.
#include "ripe_internal.h"
#include "tile_layout.h"

namespace ripe {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr float kLn2 = 0.69314718055994531f;

__device__ inline f32x4 mfma(const uint4& a, const uint4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two floats -> two bf16 (round to nearest even) in one dword, lo first
__device__ inline uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2_t));
}

// key offset (0..31) inside a tile of the e-th score register of a lane in
// lane group q: registers 0..3 are keys 4q..4q+3, registers 4..7 keys 16+4q..
__device__ inline int key_of(int e, int q) { return 16 * (e >> 2) + 4 * q + (e & 3); }

template <int D>
struct Frags {
    uint4 k[D / 32][2];   // A operand of S^T: 16 keys x 32 dims, two key halves
    uint4 v[D / 16];      // A operand of O^T: 16 value dims x 32 keys
};

// per-lane state of one 16-row-head tile
template <int D>
struct RowTile {
    uint4 q[D / 32];      // B operand of S^T: row-head n, dims 32c + 8q..+8
    float m, l;           // exponent reference (log2 units, at most the running max) and sum of p
    f32x4 o[D / 16];      // O^T: dims 16dt + 4q..+4 of row-head n
    int ri;               // bits 0..7 block offset, 8..15 loop, bit 16 valid
    int e;                // loop-R positions of this row-head end here (e_row)
    int lo;               // windowed draft: committed keys from here on (and sinks)
};
#define RI_OK(x) (((x) >> 16) & 1)
#define RI_R(x) (((x) >> 8) & 255)
#define RI_I(x) ((x) & 255)

// operand pieces of one tile: K at K + c*1024 + key*32 + 8q, V at V + e*32 + 8q
template <int D>
__device__ inline void load_frags(const uint16_t* K, const uint16_t* V, Frags<D>& f, int n, int q) {
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
            f.k[c][hf] = *reinterpret_cast<const uint4*>(K + c * 1024 + (16 * hf + n) * 32 + 8 * q);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        f.v[dt] = *reinterpret_cast<const uint4*>(V + (dt * 16 + n) * 32 + 8 * q);
}

// Maximum that propagates NaN (IEEE maximum): the scores are never NaN, and
// unlike fmaxf it needs no canonicalising moves, so two or three operands take
// one v_maximum3_f32.
__device__ inline float fmaxp(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ inline float max8(const float (&x)[8]) {
    return fmaxp(fmaxp(fmaxp(x[0], x[1]), fmaxp(x[2], x[3])), fmaxp(fmaxp(x[4], x[5]), fmaxp(x[6], x[7])));
}

// max over lanes l, l^16, l^32, l^48 (the four copies of a row-head)
__device__ inline float max_lane_groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxp(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxp(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Scores are kept in log2 units, x = s c with c = log2(e)/sqrt(d), and so is
// a row-head's exponent reference m: p = 2^(x - m).  The reference trails the
// running maximum: it moves only when a tile's maximum passes it by more than
// kLazyLog2, so every p stays below 2^kLazyLog2, and l and O are rescaled only
// then (a row-head's first tile and rare outliers) instead of whenever the
// maximum grows.  O = sum p v / l and LSE = (m + log2 l) ln 2 hold for any
// reference, and fp32 keeps l and O exact enough at that scale.
constexpr float kLazyLog2 = 8.f;
constexpr float kLazyMax = 256.f;       // 2^kLazyLog2
static_assert(kLazyMax == (float)(1 << (int)kLazyLog2), "the margin and its power of two");

// Moves the references that the tile maximum bm passes by more than the margin
// (bm = -inf never does) and rescales l and O there by 2^(m_old - m_new): 0 on
// a row-head's first keys, where l and O are still 0.
template <int D>
__device__ inline void lazy_rescale(RowTile<D>& rt, float bm) {
    const float mo = rt.m;
    const bool up = bm - mo > kLazyLog2;
    if (__any(up)) {
        const float alpha = up ? __builtin_amdgcn_exp2f(mo - bm) : 1.f;
        rt.m = up ? bm : mo;
        rt.l *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            rt.o[dt][0] *= alpha; rt.o[dt][1] *= alpha;
            rt.o[dt][2] *= alpha; rt.o[dt][3] *= alpha;
        }
    }
}

// A lane's 8 weights p added to l, and O += P V with P split into bf16
// hi = round(p) and lo = round(p - hi)
template <int D>
__device__ inline void accumulate_p(RowTile<D>& rt, const Frags<D>& f, const float (&p)[8]) {
    rt.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
        hi[e2] = pack_bf16(p[2 * e2], p[2 * e2 + 1]);
        const float h0 = __uint_as_float(hi[e2] << 16), h1 = __uint_as_float(hi[e2] & 0xffff0000u);
        lo[e2] = pack_bf16(p[2 * e2] - h0, p[2 * e2 + 1] - h1);
    }
    const uint4 phi = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    const uint4 plo = make_uint4(lo[0], lo[1], lo[2], lo[3]);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) rt.o[dt] = mfma(f.v[dt], phi, rt.o[dt]);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) rt.o[dt] = mfma(f.v[dt], plo, rt.o[dt]);
}
// p = 2^(s c - m) of a lane's 8 raw scores s against the finite reference m
// (one fma per score), then accumulate_p
template <int D>
__device__ inline void accumulate(RowTile<D>& rt, const Frags<D>& f, const float (&x)[8], float c, float m) {
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], c, -m));
    accumulate_p<D>(rt, f, p);
}

// S^T = K.Q^T of one key tile against one row tile: lane n, register e holds
// the raw score of key key_of(e, q) for row-head n (the log2-domain scale
// c = log2(e)/sqrt(d) is applied in the exponent's fma).  Returns the
// maximum of the lane's eight scores, computed in the block that runs the
// matrix instructions: the first reader of their results is then never at
// the head of a block that a branch reaches straight from them (the compiler
// left such a path without the wait the results need).
template <int D>
__device__ inline float tile_scores(const RowTile<D>& rt, const Frags<D>& f, float (&x)[8]) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < D / 32; ++k) {
        s0 = mfma(f.k[k][0], rt.q[k], s0);
        s1 = mfma(f.k[k][1], rt.q[k], s1);
    }
    x[0] = s0[0]; x[1] = s0[1]; x[2] = s0[2]; x[3] = s0[3];
    x[4] = s1[0]; x[5] = s1[1]; x[6] = s1[2]; x[7] = s1[3];
    return max8(x);
}
// The rest of a tile for a key tile every row-head of the row tile reads in
// full: no masks, every score finite (so every reference is finite after the
// rescale).  bx: the lane's score maximum from tile_scores.  Uses only f.v.
// (max(s) c is max(s c) exactly: rounding is monotone and c > 0.)
template <int D>
__device__ inline void tile_finish_full(RowTile<D>& rt, const Frags<D>& f, const float (&x)[8], float bx,
                                        float c) {
    lazy_rescale<D>(rt, max_lane_groups(bx) * c);
    accumulate<D>(rt, f, x, c, rt.m);
}

// The fast-phase tile step of the rows kernel for all row tiles of a wave
// (every key valid for every row-head, every score finite).  The weights are
// first taken against the current references; only when one of them passes
// 2^kLazyLog2 (a row-head's first tile, or a tile whose maximum passes the
// reference by more than the margin) are the row-heads' maxima formed across
// their four lane groups, the references moved, l and O rescaled and the
// weights taken again.  The common test reads only the lane's own weights.
template <int D, int RT>
__device__ inline void tiles_fast(RowTile<D> (&rt)[RT], const Frags<D>& f, const float (&x)[RT][8],
                                  const float (&bx)[RT], float c) {
    float p[RT][8];
#pragma unroll
    for (int tr = 0; tr < RT; ++tr)
#pragma unroll
        for (int e = 0; e < 8; ++e) p[tr][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[tr][e], c, -rt[tr].m));
    bool over = false;
#pragma unroll
    for (int tr = 0; tr < RT; ++tr) over = over || __builtin_fmaf(bx[tr], c, -rt[tr].m) > kLazyLog2;
    if (__any(over)) {
        float bm[RT];
        bool up[RT];
#pragma unroll
        for (int tr = 0; tr < RT; ++tr) {
            bm[tr] = max_lane_groups(max8(x[tr])) * c;
            up[tr] = bm[tr] - rt[tr].m > kLazyLog2;
            const float mo = rt[tr].m;
            const float alpha = up[tr] ? __builtin_amdgcn_exp2f(mo - bm[tr]) : 1.f;
            rt[tr].m = up[tr] ? bm[tr] : mo;
            rt[tr].l *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                rt[tr].o[dt][0] *= alpha; rt[tr].o[dt][1] *= alpha;
                rt[tr].o[dt][2] *= alpha; rt[tr].o[dt][3] *= alpha;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) p[tr][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[tr][e], c, -rt[tr].m));
        }
    }
#pragma unroll
    for (int tr = 0; tr < RT; ++tr) accumulate_p<D>(rt[tr], f, p[tr]);
}

// the rest of a tile with masks (invalid keys get -inf; a row-head that has
// seen no valid key keeps m = -inf and takes p = 0); uses only f.v.  The
// maximum of the valid scores is at most bx, the maximum of all eight; taking
// the smaller of the two keeps bx in use on this path too, so its computation
// stays where tile_scores put it (fminf: an invalid key's score may be NaN,
// and then bx is too).
template <int D>
__device__ inline void tile_finish_masked(RowTile<D>& rt, const Frags<D>& f, float (&x)[8],
                                          const bool (&valid)[8], float bx, float c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = valid[e] ? x[e] : -INFINITY;
    lazy_rescale<D>(rt, max_lane_groups(fminf(max8(x), bx)) * c);
    accumulate<D>(rt, f, x, c, rt.m == -INFINITY ? 0.f : rt.m);   // finite reference
}

// One key tile against one row tile.  `full`: every key of the tile is valid
// for every row-head of the tile (no masking needed).
template <int D>
__device__ inline void tile_update(RowTile<D>& rt, const Frags<D>& f, bool full,
                                   const bool (&valid)[8], float c) {
    float x[8];
    float bx = tile_scores<D>(rt, f, x);
    if (!full) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = valid[e] ? x[e] : -INFINITY;
        bx = fminf(max8(x), bx);
    }
    lazy_rescale<D>(rt, max_lane_groups(bx) * c);
    accumulate<D>(rt, f, x, c, rt.m == -INFINITY ? 0.f : rt.m);   // finite reference
}

// ---------------------------------------------------------------- item

struct Item {
    int b, g, c, rb, nc_b;
    bool last;
    int L;
    int nsl, ring_top, ring_base;   // ring slot sl < nsl holds ring_base + sl (- WR past ring_top)
};

// XCD-aware decode: the row blocks of one (b, g, chunk) share blockIdx % 8,
// so they run on one XCD and share its L2.  Groups are dispatched in
// blockIdx order; with a pair list, group k is KV head k % Hkv of the
// (sequence, chunk) pair k / Hkv of the list, which puts the longest first.
__device__ inline bool decode_item(const VerifyArgs& a, Item& it) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int grp = (slot / a.nrb) * 8 + xcd;
    it.rb = slot % a.nrb;
    if (grp >= a.n_groups) return false;
    if (a.n_pairs > 0) {
        const int pr = a.pairs[grp / a.Hkv];
        it.g = grp % a.Hkv;
        it.b = pr & 63;
        it.c = pr >> 6;
    } else {
        it.c = grp % a.nc;
        const int bg = grp / a.nc;
        it.g = bg % a.Hkv;
        it.b = bg / a.Hkv;
    }
    it.L = a.lens[it.b];
    it.nc_b = it.L > 0 ? (int)((it.L + a.cx + a.cl - 1) / a.cl) : 1;
    if (it.c >= it.nc_b) return false;
    it.last = it.c == it.nc_b - 1;
    it.nsl = (int)min(a.WR, (int64_t)it.L);
    it.ring_top = it.nsl > 0 ? (int)((it.L - 1) % a.WR) : 0;
    it.ring_base = it.L - 1 - it.ring_top;
    return true;
}

// e_row: committed positions [0, e_row) are read at loop R
__device__ inline int e_row(const VerifyArgs& a, int L, int i, int r) {
    if (r == a.R) return L;
    const int64_t beta = a.anchor == 0 ? (int64_t)L + i - a.W : (int64_t)L - a.W;
    return (int)(beta < 0 ? 0 : (beta > L ? L : beta));
}

// state of row-head u (query row word `rw`, see VerifyArgs::rows); row-heads
// past M are padding (zero query, never written)
template <int D>
__device__ inline void init_row_word(const VerifyArgs& a, const Item& it, int u, uint32_t rw, int q,
                                     RowTile<D>& rt) {
    const bool ok = u < a.M;
    const int ii = rw & 255, rr = (rw >> 8) & 255;
    rt.ri = ii | (rr << 8) | (ok ? 1 << 16 : 0);
    rt.e = e_row(a, it.L, ii, rr);
    rt.lo = a.w_draft < 0 ? 0 : max(0, it.L + ii - a.w_draft);
    rt.m = -INFINITY;
    rt.l = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) rt.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int orig = (int)(rw >> 16), h = it.g * a.group + (ok ? u % a.group : 0);
    const uint16_t* qp = a.q + (((int64_t)it.b * a.n_rows + orig) * a.Hq + h) * D;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
        rt.q[c] = ok ? *reinterpret_cast<const uint4*>(qp + 32 * c + 8 * q) : make_uint4(0, 0, 0, 0);
}

// masks of one row tile against a deep / ring / block tile; false = the tile
// holds no key of any row-head of this row tile
template <int D>
__device__ inline int mask_deep(const RowTile<D>& rt, int base, int d1, int q, bool (&v)[8]) {
    const int lim = min(rt.e, d1);
    const bool mine = RI_OK(rt.ri) && base < lim;
    if (!__any(mine)) return 0;
    if (__all(!RI_OK(rt.ri) || base + 32 <= lim)) return 2;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = mine && base + key_of(e, q) < lim;
    return 1;
}
template <int D>
__device__ inline int mask_ring(const RowTile<D>& rt, const Item& it, int WR, int r, int base,
                                int q, bool (&v)[8]) {
    const bool mine = RI_OK(rt.ri) && RI_R(rt.ri) == r && rt.e < it.L;
    if (!__any(mine)) return 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int sl = base + key_of(e, q);
        const int pos = it.ring_base + sl - (sl > it.ring_top ? WR : 0);
        v[e] = mine && sl < it.nsl && pos >= rt.e;
    }
    return 1;
}
// windowed draft: of a deep (kind 0) or ring (kind 1) tile's keys that the
// masks above let through (mode 1: v; mode 2: all of them), keep the sinks
// s < n_sink and the window s >= lo
template <int D>
__device__ inline int mask_window(const RowTile<D>& rt, const Item& it, int kind, int base, int n_sink,
                                  int WR, int q, int mode, bool (&v)[8]) {
    bool any = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        int s = base + key_of(e, q);
        if (kind == 1) s = it.ring_base + s - (s > it.ring_top ? WR : 0);   // ring slot -> position
        v[e] = (mode == 2 ? (bool)RI_OK(rt.ri) : v[e]) && (s < n_sink || s >= rt.lo);
        any = any || v[e];
    }
    return __any(any) ? 1 : 0;
}
template <int D>
__device__ inline int mask_block(const RowTile<D>& rt, int r, int base, int q, bool (&v)[8]) {
    const bool mine = RI_OK(rt.ri) && RI_R(rt.ri) == r;
    if (!__any(mine)) return 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = mine && base + key_of(e, q) <= RI_I(rt.ri);
    return 1;
}

// stage 32 draft-block keys/values (caller's [token][dim] layout) into a
// wave-private LDS tile pair in the storage's operand order; keys past n_blk
// are zero.  A lane holds D/16 16-byte pieces of K and of V; they are loaded
// two at a time before any is stored (128 pieces of a wave cover at least
// eight keys), and a group of pieces that lies wholly past n_blk is not
// loaded at all, so a block of up to eight tokens costs one memory round trip.
template <int D>
__device__ inline void stage_block(const VerifyArgs& a, const uint16_t* K, const uint16_t* V,
                                   int base, uint16_t* sk, uint16_t* sv, int lane) {
    constexpr int PK = D / 8;                 // pieces per key row
    constexpr int NI = 32 * PK / 64;          // pieces per lane
    constexpr int GP = 2;                     // pieces loaded before any is stored
    const int n_keys = a.n_blk - base;        // keys of this tile inside the block
    // the value tile is cleared with 16-byte stores and only the keys of the
    // block are scattered into it: its 2-byte stores land in few LDS banks
#pragma unroll
    for (int z = 0; z < D / 16; ++z)
        *reinterpret_cast<uint4*>(sv + (z * 64 + lane) * 8) = make_uint4(0, 0, 0, 0);
#pragma unroll 1
    for (int t0 = 0; t0 < NI; t0 += GP) {
        uint4 kx[GP], vx[GP];
        const bool need = t0 * 64 < n_keys * PK;          // wave-uniform
#pragma unroll
        for (int u = 0; u < GP; ++u) {
            kx[u] = vx[u] = make_uint4(0, 0, 0, 0);
            const int it = lane + 64 * (t0 + u);
            const int key = it / PK, e0 = (it % PK) * 8;
            if (need && t0 + u < NI && key < n_keys) {
                kx[u] = *reinterpret_cast<const uint4*>(K + (base + key) * a.bk.st + e0);
                vx[u] = *reinterpret_cast<const uint4*>(V + (base + key) * a.bv.st + e0);
            }
        }
#pragma unroll
        for (int u = 0; u < GP; ++u) {
            if (t0 + u >= NI) break;
            const int it = lane + 64 * (t0 + u);
            const int key = it / PK, e0 = (it % PK) * 8;
            *reinterpret_cast<uint4*>(sk + key_off(key, e0, D)) = kx[u];
            if (key < n_keys) {
                const uint32_t w[4] = {vx[u].x, vx[u].y, vx[u].z, vx[u].w};
#pragma unroll
                for (int cc = 0; cc < 8; ++cc)
                    sv[val_off(key, e0 + cc, D)] = (uint16_t)(w[cc >> 1] >> (16 * (cc & 1)));
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// final (single chunk) or partial (multi-chunk) result of one row tile whose
// l is already summed over the lane groups
template <int D>
__device__ inline void write_result_word(const VerifyArgs& a, const Item& it, const RowTile<D>& rt,
                                         int u, uint32_t rw, int q) {
    if (!RI_OK(rt.ri)) return;
    const int orig = (int)(rw >> 16), h = it.g * a.group + u % a.group;
    if (it.nc_b == 1) {
        const float inv = 1.f / rt.l;
        float* op = a.out + (((int64_t)it.b * a.n_rows + orig) * a.Hq + h) * D;
        // final rows are not read again by this call: non-temporal stores,
        // so they do not wait in L2 for the write-back at the kernel's end
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            __builtin_nontemporal_store(f32x4{rt.o[dt][0] * inv, rt.o[dt][1] * inv, rt.o[dt][2] * inv,
                                              rt.o[dt][3] * inv},
                                        reinterpret_cast<f32x4*>(op + dt * 16 + 4 * q));
        if (q == 0)
            a.lse[((int64_t)it.b * a.n_rows + orig) * a.Hq + h] = (rt.m + log2f(rt.l)) * kLn2;
    } else {
        const int64_t pidx = (((int64_t)it.b * a.Hkv + it.g) * a.nc + it.c) * a.M + u;
        float* po = a.part + pidx * (D + 2);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            *reinterpret_cast<float2*>(po + dt * 16 + 4 * q) = make_float2(rt.o[dt][0], rt.o[dt][1]);
            *reinterpret_cast<float2*>(po + dt * 16 + 4 * q + 2) = make_float2(rt.o[dt][2], rt.o[dt][3]);
        }
        // partial reference in the log2 domain (-inf stays -inf)
        if (q == 0) *reinterpret_cast<float2*>(po + D) = make_float2(rt.m, rt.l);
    }
}
template <int D>
__device__ inline void sum_lane_groups(RowTile<D>& rt) {
    rt.l += __shfl_xor(rt.l, 16);
    rt.l += __shfl_xor(rt.l, 32);
}

// ---------------------------------------------------------------- many rows

// Workgroup barrier that waits for this wave's LDS operations but leaves its
// global loads in flight (no memory fence, so no vmcnt(0)); the memory clobber
// keeps the compiler from moving memory accesses across it.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wave-wide min / max: rotations within each 16-lane row (DPP row_ror), then
// across the four rows (permlane swaps); every lane ends with the result.
template <bool kMax>
__device__ inline int wave_reduce(int x) {
    auto op = [](int u, int v) { return kMax ? max(u, v) : min(u, v); };
    x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x128, 0xf, 0xf, false));   // row_ror:8
    x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x124, 0xf, 0xf, false));   // row_ror:4
    x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x122, 0xf, 0xf, false));   // row_ror:2
    x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x121, 0xf, 0xf, false));   // row_ror:1
    const auto a = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    x = op((int)a[0], (int)a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    x = op((int)b[0], (int)b[1]);
    return __builtin_amdgcn_readfirstlane(x);
}
__device__ inline int wave_min(int x) { return wave_reduce<false>(x); }
__device__ inline int wave_max(int x) { return wave_reduce<true>(x); }

// Direct global->LDS load of 16 bytes per lane (lane l lands at lds + 16 l),
// written as asm so that the compiler does not treat later LDS accesses as
// possibly aliasing an outstanding load (it would wait for every load in
// flight); the caller waits with explicit s_waitcnt vmcnt.  No register is
// written.
__device__ inline void dma16(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(g), "s"(lds) : "memory");
}
__device__ inline uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// N consecutive 1 KB blocks by direct loads: block i from sbase + voff +
// 1 KB i into lds + 1 KB i + 16 lane (the instruction offset moves the global
// and the LDS address alike).  sbase is wave-uniform (scalar registers), so a
// run costs one scalar move besides its N loads; same contract as dma16.
template <int N>
__device__ inline void dma16_run(const void* sbase, uint32_t voff, uint32_t lds) {
    static_assert(N >= 1 && N <= 4, "one to four blocks");
    if constexpr (N == 1)
        asm volatile("s_mov_b32 m0, %2\n\t"
                     "global_load_lds_dwordx4 %0, %1" :: "v"(voff), "s"(sbase), "s"(lds) : "memory");
    else if constexpr (N == 4)
        asm volatile("s_mov_b32 m0, %2\n\t"
                     "global_load_lds_dwordx4 %0, %1\n\t"
                     "global_load_lds_dwordx4 %0, %1 offset:1024\n\t"
                     "global_load_lds_dwordx4 %0, %1 offset:2048\n\t"
                     "global_load_lds_dwordx4 %0, %1 offset:3072" :: "v"(voff), "s"(sbase), "s"(lds) : "memory");
    else if constexpr (N == 3)
        asm volatile("s_mov_b32 m0, %2\n\t"
                     "global_load_lds_dwordx4 %0, %1\n\t"
                     "global_load_lds_dwordx4 %0, %1 offset:1024\n\t"
                     "global_load_lds_dwordx4 %0, %1 offset:2048" :: "v"(voff), "s"(sbase), "s"(lds) : "memory");
    else
        asm volatile("s_mov_b32 m0, %2\n\t"
                     "global_load_lds_dwordx4 %0, %1\n\t"
                     "global_load_lds_dwordx4 %0, %1 offset:1024" :: "v"(voff), "s"(sbase), "s"(lds) : "memory");
}
// N 4-byte loads (lane l of load i: sbase + 4 l + 256 i into lds + 256 i + 4 l)
template <int N>
__device__ inline void dma4_run(const void* sbase, uint32_t lds, int lane) {
    static_assert(N >= 2 && N <= 4, "two to four loads");
    const uint32_t voff = 4 * lane;
    if constexpr (N == 4)
        asm volatile("s_mov_b32 m0, %2\n\t"
                     "global_load_lds_dword %0, %1\n\t"
                     "global_load_lds_dword %0, %1 offset:256\n\t"
                     "global_load_lds_dword %0, %1 offset:512\n\t"
                     "global_load_lds_dword %0, %1 offset:768" :: "v"(voff), "s"(sbase), "s"(lds) : "memory");
    else if constexpr (N == 3)
        asm volatile("s_mov_b32 m0, %2\n\t"
                     "global_load_lds_dword %0, %1\n\t"
                     "global_load_lds_dword %0, %1 offset:256\n\t"
                     "global_load_lds_dword %0, %1 offset:512" :: "v"(voff), "s"(sbase), "s"(lds) : "memory");
    else
        asm volatile("s_mov_b32 m0, %2\n\t"
                     "global_load_lds_dword %0, %1\n\t"
                     "global_load_lds_dword %0, %1 offset:256" :: "v"(voff), "s"(sbase), "s"(lds) : "memory");
}
// A staged tile pair is D/8 blocks of 1 KB (the key tile's D/16, then the
// value tile's), block b at stage + 1 KB b.  Wave w of the four loading it
// takes the D/32 consecutive blocks from D/32 * w on: waves 0 and 1 the key
// tile, 2 and 3 the value tile.  Its first block within that tile, and the
// lane's 16 bytes in a block (a storage block is the operand piece order of
// the instruction: lane l reads row l % 16, dims 8 (l / 16)..+8), as a byte
// offset from the tile:
template <int D>
__device__ inline uint32_t stage_lane_offset(int wave, int lane) {
    return (uint32_t)(((wave & 1) * (D / 32)) * 1024 + ((lane & 15) * 32 + (lane >> 4) * 8) * 2);
}
// The operand pieces of a staged tile pair as ordinary LDS loads (piece i at
// stage + 1 KB * i, this lane's 16 bytes at + 16 lane): the key half and the
// value half separately.
template <int D>
__device__ inline void lds_keys(const uint16_t* stage, Frags<D>& f, int lane) {
    const uint4* p = reinterpret_cast<const uint4*>(stage) + lane;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
        f.k[c][0] = p[(2 * c) * 64];
        f.k[c][1] = p[(2 * c + 1) * 64];
    }
}
template <int D>
__device__ inline void lds_values(const uint16_t* stage, Frags<D>& f, int lane) {
    const uint4* p = reinterpret_cast<const uint4*>(stage) + lane;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) f.v[dt] = p[(D / 16 + dt) * 64];
}

// LDS stages of the rows kernel's tile stream (one tile pair per key half
// each; the query operands borrow the last stage until the first step):
// 160 / 144 / 160 KB
constexpr int rows_stages(int d) { return d == 128 ? 5 : (d == 96 ? 6 : 10); }
// steps per barrier where the stages allow: K tiles consumed per barrier
// while the next ones load (measured on the Huginn-scale launch: two steps
// 4% and three steps 11% faster than one; at head_dim 128, with four or five
// stages, two steps were 5% slower)
constexpr int rows_barrier_steps(int d) { return rows_stages(d) >= 6 ? 3 : 1; }

// The private wave of row group rw in the rows kernel (PRIV): the ring tiles
// of the row group's loops while the deep tiles stream (spread over the loop,
// each loaded into registers a few steps before it is computed, so its loads
// never hold back a barrier), then its draft-block tiles, staged in a
// wave-private part of the stages once they are free; its state goes to the
// second merge buffer.
// It executes exactly the barriers of the other waves: one before the loop,
// one every rows_barrier_steps steps in it, four after it.
template <int D, int RTW>
__device__ __attribute__((always_inline)) inline void private_wave(const VerifyArgs& a, const Item& it,
        RowTile<D> (&rt)[RTW], int rw, int u_w, int n_iter, int ring_tiles, int64_t rreg0,
        int64_t WPD, float sl2, int lane, uint16_t* stages, const uint4* sq, int merge_slots) {
    constexpr int TILE = 32 * D;
    constexpr int MS = D / 4 + 2;
    const int n = lane & 15, q = lane >> 4;
    asm volatile("s_barrier ; private: queries and tile 0" ::: "memory");
#pragma unroll
    for (int t = 0; t < RTW; ++t)
#pragma unroll
        for (int c = 0; c < D / 32; ++c) rt[t].q[c] = sq[(t * (D / 32) + c) * 64 + lane];
    // the row group's row-heads x = 16t + n in lanes x (x < 16*RTW), sorted by
    // loop then block offset: the first of each loop marks it, the last one
    // carries the loop's largest offset
    // (the shuffle runs in every lane: a lane that is switched off cannot be a source)
    const int ri_hi = __shfl(rt[RTW - 1].ri, (lane + 48) & 63);
    const int ri = lane < 16 ? rt[0].ri : (RTW == 2 && lane < 32 ? ri_hi : 0);
    const int ri_prev = __shfl(ri, (lane + 63) & 63), ri_next = __shfl(ri, (lane + 1) & 63);
    const bool ok = RI_OK(ri), ok_p = lane > 0 && RI_OK(ri_prev), ok_n = lane < 63 && RI_OK(ri_next);
    const bool first = ok && (!ok_p || RI_R(ri_prev) != RI_R(ri));
    const bool last = ok && (!ok_n || RI_R(ri_next) != RI_R(ri));
    const uint64_t fmask = __ballot(first), lmask = __ballot(last);
    (void)u_w;
    // ring jobs: (loop p with r < R, slot tile st), p-major
    int n_ring_loops = 0;
    {
        uint64_t m = fmask;
        while (m) {
            const int k = __builtin_ctzll(m);
            m &= m - 1;
            n_ring_loops += (int)RI_R(__builtin_amdgcn_readlane(ri, k)) < a.R;
        }
    }
    const int n_jobs = it.last ? n_ring_loops * ring_tiles : 0;
    // job j -> ring tile address and loop (wave-uniform)
    auto job = [&](int j, int& r, int& base) -> int64_t {
        const int pl = j / ring_tiles, st = j % ring_tiles;
        uint64_t m = fmask;
        int seen = -1, rr = a.R;
        while (m) {
            const int k = __builtin_ctzll(m);
            m &= m - 1;
            rr = (int)RI_R(__builtin_amdgcn_readlane(ri, k));
            if (rr < a.R && ++seen == pl) break;
        }
        r = rr;
        base = st * 32;
        return rreg0 + (int64_t)(rr - 1) * WPD + (int64_t)st * TILE;
    };
    // One register buffer: a job is loaded, then computed two barriers later
    // (odd steps), and only then is the next one loaded into the same
    // registers; the loads stay in flight across barriers, which do not wait
    // for them.  Jobs left after the loop run one after the other.
    Frags<D> fr;
    int rr = 0, br = 0;
    auto load_job = [&](int j) {
        const int64_t off = job(j, rr, br);
        load_frags<D>(a.ring_k + off, a.ring_v + off, fr, n, q);
    };
    auto run_job = [&]() {
#pragma unroll
        for (int tr = 0; tr < RTW; ++tr) {
            bool v[8];
            if (mask_ring<D>(rt[tr], it, (int)a.WR, rr, br, q, v)) tile_update<D>(rt[tr], fr, false, v, sl2);
        }
    };
    // Draft-block rows: in the common case (at most two loops in the row
    // group, offsets below 8) they are requested into registers now, as
    // pieces pc = (kv*8 + key)*(D/8) + c8 with lane holding pc = lane + 64k,
    // and staged only after the loop; other row sets load them then.
    constexpr int PB = D / 32;
    const int nloops = __popcll(fmask);
    int blk_r[2] = {0, 0}, blk_im[2] = {-1, -1};
    {
        uint64_t m = fmask;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            if (m) {
                const int k = __builtin_ctzll(m);
                m &= m - 1;
                blk_r[p] = (int)RI_R(__builtin_amdgcn_readlane(ri, k));
                blk_im[p] = (int)RI_I(__builtin_amdgcn_readlane(ri, __builtin_ctzll(lmask & (~0ull << k))));
            }
        }
    }
    // (not with two row tiles of 64 dims, whose registers are needed)
    constexpr bool kBlkPf = D * RTW <= 96;
    const bool pf_ok = kBlkPf && it.last && nloops <= 2 && blk_im[0] < 8 && blk_im[1] < 8;
    uint4 pfb[2][PB];
    auto prefetch_block = [&]() {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const uint16_t* pbk = a.bk.p + it.b * a.bk.sb + (int64_t)(max(blk_r[p], 1) - 1) * a.bk.sp + it.g * a.bk.sh;
            const uint16_t* pbv = a.bv.p + it.b * a.bv.sb + (int64_t)(max(blk_r[p], 1) - 1) * a.bv.sp + it.g * a.bv.sh;
#pragma unroll
            for (int k = 0; k < PB; ++k) {
                const int pc = lane + 64 * k;
                const int c8 = pc % (D / 8), rest = pc / (D / 8);
                const int key = rest % 8, kv = rest / 8;
                pfb[p][k] = make_uint4(0, 0, 0, 0);
                if (pf_ok && p < nloops && key < a.n_blk && key <= blk_im[p])
                    pfb[p][k] = *reinterpret_cast<const uint4*>((kv ? pbv + key * a.bv.st : pbk + key * a.bk.st) + c8 * 8);
            }
        }
    };
    // The ring jobs are spread over the loop, sp steps apart: job m is loaded
    // right after job m - 1 is computed (the first after the first barrier,
    // so it does not join the start-up burst of deep tiles) and computed sp
    // steps later; the block rows are requested four steps before the end.
    const int sp = n_jobs > 0 ? min(4, max(2, n_iter / n_jobs)) : 2;
    const int pf_step = max(0, n_iter - 4);
    int done = 0;
    for (int k = 0; k < n_iter; ++k) {
        if (k % rows_barrier_steps(D) == 0) lds_barrier();   // the main waves' barriers
        if (k == 0 && n_jobs > 0) load_job(0);
        if (k % sp == sp - 1 && done < n_jobs) {
            run_job();
            if (++done < n_jobs) load_job(done);
        }
        if (k == pf_step) prefetch_block();
    }
    if (n_iter == 0) {
        if (n_jobs > 0) load_job(0);
        prefetch_block();
    }
    while (done < n_jobs) {
        run_job();
        if (++done < n_jobs) load_job(done);
    }
    // every deep load is done and every wave has left the stages
    lds_barrier();
    if (it.last && pf_ok) {
        // The prefetched rows go row-major into the wave's part of the stages
        // ([kv][key][dim], 16-byte writes), and the operands are read from
        // there: a key operand is key n's 16 bytes at dims 32c + 8q (keys 8 and
        // up, and the second key half, are zero); a value operand holds keys
        // 4q..4q+3 at dim 16dt + n in its first four columns (lane groups 0
        // and 1; its other columns are keys of 16 or more, zero).  Keys past
        // the block were prefetched as zero, so nothing needs clearing.
        uint16_t* rm = stages + rw * 2 * TILE;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            if (p >= nloops) break;
#pragma unroll
            for (int k = 0; k < PB; ++k) {
                const int pc = lane + 64 * k;
                const int c8 = pc % (D / 8), rest = pc / (D / 8);   // rest = kv*8 + key
                *reinterpret_cast<uint4*>(rm + rest * D + c8 * 8) = pfb[p][k];
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            Frags<D> f;
#pragma unroll
            for (int c = 0; c < D / 32; ++c) {
                f.k[c][0] = n < 8 ? *reinterpret_cast<const uint4*>(rm + n * D + 32 * c + 8 * q)
                                  : make_uint4(0, 0, 0, 0);
                f.k[c][1] = make_uint4(0, 0, 0, 0);
            }
            const uint16_t* vr = rm + (8 + 4 * (q & 1)) * D;    // value rows of keys 4q..
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                const uint32_t v0 = vr[16 * dt + n], v1 = vr[D + 16 * dt + n];
                const uint32_t v2 = vr[2 * D + 16 * dt + n], v3 = vr[3 * D + 16 * dt + n];
                f.v[dt] = q < 2 ? make_uint4(v0 | (v1 << 16), v2 | (v3 << 16), 0, 0) : make_uint4(0, 0, 0, 0);
            }
            // every lane has read the rows before the next loop's overwrite them
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int tr = 0; tr < RTW; ++tr) {
                bool v[8];
                if (mask_block<D>(rt[tr], blk_r[p], 0, q, v)) tile_update<D>(rt[tr], f, false, v, sl2);
            }
        }
    } else if (it.last) {
        uint16_t* sk = stages + rw * 2 * TILE;
        uint16_t* sv = sk + TILE;
        uint64_t m = fmask;
        while (m) {
            const int k = __builtin_ctzll(m);
            m &= m - 1;
            const int r = (int)RI_R(__builtin_amdgcn_readlane(ri, k));
            // the loop's last row-head is the first marked last at or after k
            const uint64_t after = lmask & (~0ull << k);
            const int imax = (int)RI_I(__builtin_amdgcn_readlane(ri, __builtin_ctzll(after)));
            const uint16_t* bK = a.bk.p + it.b * a.bk.sb + (int64_t)(r - 1) * a.bk.sp + it.g * a.bk.sh;
            const uint16_t* bV = a.bv.p + it.b * a.bv.sb + (int64_t)(r - 1) * a.bv.sp + it.g * a.bv.sh;
            for (int base = 0; base <= imax; base += 32) {
                stage_block<D>(a, bK, bV, base, sk, sv, lane);
                Frags<D> f;
                load_frags<D>(sk, sv, f, n, q);
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int tr = 0; tr < RTW; ++tr) {
                    bool v[8];
                    if (mask_block<D>(rt[tr], r, base, q, v)) tile_update<D>(rt[tr], f, false, v, sl2);
                }
            }
        }
    }
    lds_barrier();                                 // the merge buffers are free
    // second merge buffer: after the first one's merge_slots lane states
    float* s_m = reinterpret_cast<float*>(stages) + merge_slots * MS;
#pragma unroll
    for (int tr = 0; tr < RTW; ++tr) {
        float* dst = s_m + ((rw * RTW + tr) * 64 + lane) * MS;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[dt * 4 + j] = rt[tr].o[dt][j];
        dst[D / 4] = rt[tr].m;
        dst[D / 4 + 1] = rt[tr].l;
    }
    lds_barrier();                                 // half 0 merges
    lds_barrier();                                 // merge buffers free again
}

// Eight waves: waves w and w+4 own the same 16*RTW row-heads and take the
// even and odd tiles of the stream (key halves kh = 0, 1), so every SIMD runs
// two independent tile steps; their softmax states merge through LDS at the end.
// The stream is the chunk's deep tiles, then the ring tiles of every loop
// r < R present in the workgroup.  All eight waves load each tile pair into an
// LDS stage with direct global->LDS loads, two or more steps ahead (a
// barrier every step, or every third step where the stages allow).  The
// direct loads are asm, which the compiler does not see writing LDS, so its
// own LDS reads of the stages never make it drain the load pipeline; every
// wait on the direct loads is explicit.  Row data goes from the kernel
// arguments into registers.  Deep tiles that every row-head reads in full take
// the unmasked step.
//
// PRIV: four more waves, one per row group, take the ring and draft-block
// tiles of their row group's loops, which no other row group reads, straight
// from memory into registers, while the eight waves stream only the deep tiles
// through LDS; the private waves join every barrier and their softmax state
// joins the merge.  The ring phase then runs beside the deep phase instead of
// after it.
template <int D, int RTW, bool PRIV>
__global__ void __launch_bounds__(PRIV ? 768 : 512, 1) k_verify_rows(VerifyArgs a) {
    constexpr int TILE = 32 * D;                 // elements of one K or V tile
    constexpr int S = rows_stages(D);
    constexpr int K = rows_barrier_steps(D);
    // tiles loaded ahead of the first step: as many as leave the stages of
    // the K tiles consumed before each barrier free for the next K
    constexpr int P = K == 1 ? S - 1 : S - K + 1;
    static_assert(P >= K + 1, "the K tiles after a barrier must be loaded by then");
    static_assert(P <= S - 1, "the last stage holds the queries until the first step");
    constexpr int PT = D / 32;                   // direct loads per thread per tile pair
    constexpr int PF = D / 16;                   // prefetched draft-block pieces per lane
    constexpr int MS = D / 4 + 2;                // floats of one lane's state in the merge
    __shared__ __attribute__((aligned(16))) uint16_t s_tile[S][2][2 * TILE];
    // query operands per row group, in the last stage: the first tiles go to
    // stages 0 .. P - 1 < S - 1, and the last stage's first tile is issued
    // after the first barrier of the loop, when every wave has read them
    static_assert(4 * RTW * (D / 32) * 64 * 16 <= (int)sizeof(s_tile[0]), "queries in a stage");
    uint4 (*const s_q)[RTW * (D / 32)][64] = reinterpret_cast<uint4 (*)[RTW * (D / 32)][64]>(&s_tile[S - 1][0][0]);
    static_assert((PRIV ? 2 : 1) * 4 * RTW * 64 * MS * 4 <= (int)sizeof(s_tile), "merge buffers");
    static_assert(8 * 2 * TILE * 2 <= (int)sizeof(s_tile), "per-wave block scratch");
    static_assert(RTW <= 2, "two row words per lane");

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, n = lane & 15, q = lane >> 4;
    const int rw = wave & 3, kh = wave >> 2;     // row group, key half (2: private wave)
    const int G = a.group;
    // the workgroup's rows k_lo .. k_lo+nk-1 (sorted by loop, then block
    // offset), loaded first since they do not depend on the sequence: row
    // k_lo + lane in w0, row k_lo + 64 + lane in w1
    const int u_blk = (int)((blockIdx.x >> 3) % a.nrb) * 64 * RTW;   // first row-head of the workgroup
    const int k_lo = u_blk / G;
    const int nk = min(a.rows_here, (min(a.M, u_blk + 64 * RTW) + G - 1) / G) - k_lo;
    const uint32_t w0 = lane < nk ? a.rows[k_lo + lane] : 0u;
    const uint32_t w1 = lane + 64 < nk ? a.rows[k_lo + 64 + lane] : 0u;

    Item it;
    if (!decode_item(a, it)) return;
    const int u_w = u_blk + rw * 16 * RTW;       // first row-head of this wave
    const float sl2 = a.scale_log2;
    const int cl = (int)a.cl;
    const int d0 = it.c * cl;
    const int64_t dreg = ((int64_t)it.b * a.Hkv + it.g) * a.CP * D;
    const uint16_t* const gK = a.deep_k + dreg;
    const uint16_t* const gV = a.deep_v + dreg;
    auto row_at = [&](int k) -> uint32_t {       // row word k (wave-uniform k < nk)
        return k < 64 ? (uint32_t)__builtin_amdgcn_readlane(w0, k) : (uint32_t)__builtin_amdgcn_readlane(w1, k - 64);
    };

    RowTile<D> rt[RTW];
    uint32_t rword[RTW];
#pragma unroll
    for (int t = 0; t < RTW; ++t) {
        const int u = u_w + 16 * t + n;
        const int k = (u < a.M ? u / G : k_lo) - k_lo;
        const uint32_t x0 = __shfl(w0, k & 63), x1 = __shfl(w1, k & 63);
        rword[t] = k < 64 ? x0 : x1;
        const bool ok = u < a.M;
        const int ii = rword[t] & 255, rr = (rword[t] >> 8) & 255;
        rt[t].ri = ii | (rr << 8) | (ok ? 1 << 16 : 0);
        rt[t].e = e_row(a, it.L, ii, rr);
        rt[t].m = -INFINITY;
        rt[t].l = 0.f;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) rt[t].o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // query operands into LDS by direct loads (waves of key half 0 load their
    // row group's, both halves read them after the first barrier); padding
    // row-heads load a valid query, their results are never written
    if (kh == 0) {
        const uint32_t qbase = lds_addr(&s_q[rw][0][0]);
#pragma unroll
        for (int t = 0; t < RTW; ++t) {
            const int u = u_w + 16 * t + n;
            const int h = it.g * G + (u < a.M ? u % G : 0);
            const uint16_t* qp = a.q + (((int64_t)it.b * a.n_rows + (int)(rword[t] >> 16)) * a.Hq + h) * D + 8 * q;
#pragma unroll
            for (int c = 0; c < D / 32; ++c) dma16(qp + 32 * c, qbase + (t * (D / 32) + c) * 1024);
        }
    }
    // deep extent of the workgroup: the largest e_row of its rows
    int e_here = lane < nk ? e_row(a, it.L, w0 & 255, (w0 >> 8) & 255) : 0;
    if (lane + 64 < nk) e_here = max(e_here, e_row(a, it.L, w1 & 255, (w1 >> 8) & 255));
    const int E = wave_max(e_here);
    // loops r < R present in the workgroup, ascending: the p-th in lane p of
    // loops_v0 (p < 64) or lane p - 64 of loops_v1
    int loops_v0 = 0, loops_v1 = 0, nl = 0;
    {
        const int r0 = (w0 >> 8) & 255, r1 = (w1 >> 8) & 255;
        const int r0p = __shfl(r0, (lane + 63) & 63), r1p = __shfl(r1, (lane + 63) & 63);
        const int r0_last = __builtin_amdgcn_readlane(r0, 63);
        const bool f0 = lane < nk && r0 < a.R && (lane == 0 || r0 != r0p);
        const bool f1 = lane + 64 < nk && r1 < a.R && r1 != (lane == 0 ? r0_last : r1p);
        uint64_t m = __ballot(f0);
        while (m) {
            const int k = __builtin_ctzll(m);
            m &= m - 1;
            const int r = __builtin_amdgcn_readlane(r0, k);
            loops_v0 = lane == nl ? r : loops_v0;
            ++nl;
        }
        m = __ballot(f1);
        while (m) {
            const int k = __builtin_ctzll(m);
            m &= m - 1;
            const int r = __builtin_amdgcn_readlane(r1, k);
            if (nl < 64) loops_v0 = lane == nl ? r : loops_v0;
            else loops_v1 = lane == nl - 64 ? r : loops_v1;
            ++nl;
        }
    }

    const int d1 = min(d0 + cl, E);
    const int n_deep = d1 > d0 ? (d1 - d0 + 31) / 32 : 0;
    const int ring_tiles = (it.last && a.R > 1 && it.nsl > 0) ? (it.nsl + 31) / 32 : 0;
    const int n_tiles = n_deep + (PRIV ? 0 : nl * ring_tiles);
    const int n_iter = (n_tiles + 1) / 2;
    const int64_t rreg0 = ((int64_t)it.b * a.Hkv + it.g) * a.NR * a.WP * D;
    const int64_t WPD = a.WP * D;

    // per row tile: the deep positions this wave's row-heads read end at
    // lim = min(e_row, d1); tiles below the smallest lim need no mask, tiles at
    // or past the largest are skipped.  Tiles below L - W are full for everyone.
    int full_lim[RTW], any_lim[RTW];
#pragma unroll
    for (int t = 0; t < RTW; ++t) {
        const int lim = min(rt[t].e, d1);
        full_lim[t] = wave_min(RI_OK(rt[t].ri) ? lim : (1 << 30));
        any_lim[t] = wave_max(RI_OK(rt[t].ri) ? lim : -1);
    }
    const int e_lb = (int)max((int64_t)0, min((int64_t)it.L, (int64_t)it.L - a.W));
    const int n_full = min(e_lb, d1) > d0 ? (min(e_lb, d1) - d0) / 32 : 0;
    const int n_fast = min(n_iter, n_full / 2);

    if constexpr (PRIV) {
        if (kh == 2) {
            private_wave<D, RTW>(a, it, rt, rw, u_w, n_iter, ring_tiles, rreg0, WPD, sl2, lane,
                                 &s_tile[0][0][0], &s_q[rw][0][0], 4 * RTW * 64);
            return;
        }
    }

    // issue cursor: the j-th issue of this wave loads tile 2j + kh of the
    // stream; this wave's blocks of it are in the key tile (rw < 2) or the
    // value tile, at iKV (deep tiles), from stage + 1 KB * PT * rw
    int ti = kh, ipl = 0, ist = 0;
    const uint16_t* iKV = (rw < 2 ? gK : gV) + (int64_t)(d0 + 32 * kh) * D;
    const uint32_t voff = stage_lane_offset<D>(rw, lane);
    const uint16_t* ring_kv = rw < 2 ? a.ring_k : a.ring_v;
    auto issue_next = [&](uint16_t* stage) {
        const uint32_t l = lds_addr(stage) + rw * PT * 1024;
        if (PRIV || ti < n_deep) {                // with private waves the stream is deep only
            dma16_run<PT>(iKV, voff, l);
        } else {
            if (ti - 2 < n_deep) { ipl = 0; ist = ti - n_deep; }   // first ring tile of this half
            while (ist >= ring_tiles) { ist -= ring_tiles; ++ipl; }
            const int r = ipl < 64 ? __builtin_amdgcn_readlane(loops_v0, ipl)
                                   : __builtin_amdgcn_readlane(loops_v1, ipl - 64);
            const int64_t off = rreg0 + (int64_t)(r - 1) * WPD + (int64_t)ist * TILE;
            dma16_run<PT>(ring_kv + off, voff, l);
            ist += 2;
        }
        ti += 2;
        iKV += 2 * TILE;
    };
    // Past the end of its tiles a wave still issues one group of PT loads per
    // step: PT 4-byte loads of valid memory into the stage the missing tile
    // would use, which no later tile of this half uses.  Each step thus
    // issues PT loads, and every wait is a constant count: tile j is in LDS
    // when at most the groups issued after it are outstanding (s_waitcnt
    // vmcnt(N); 0xF70 leaves expcnt and lgkmcnt unconstrained).  Constant
    // waits keep the loop free of branches the compiler would thread across
    // its back edge.
    auto issue_dummy = [&](uint16_t* stage) {
        dma4_run<PT>(gK, lds_addr(stage), lane);  // (the first 1 KB of the plane)
        ti += 2;
    };
    static_assert((P - 1) * PT <= 15, "vmcnt field");

    // the first P tile pairs of this half (after the query loads, so the wait
    // for tile 0 covers them)
    for (int j = 0; j < P; ++j) {
        if (ti < n_tiles) issue_next(s_tile[j][kh]);
        else issue_dummy(s_tile[j][kh]);
    }
    int si = P % S;                               // stage of the next issue (tile m in stage m mod S)

    // this wave's loops (ascending, at most two on the fast path) with their
    // largest block offsets, from the sorted row words
    int wl[2] = {0, 0}, wimax[2] = {0, 0}, n_wl = 0;
    bool wl_more = false;                         // more than two loops: slow path
    if (u_w < a.M) {
        const int kw0 = u_w / G - k_lo;
        const int kw1 = (min(a.M, u_w + 16 * RTW) - 1) / G - k_lo;
        const int r_first = (row_at(kw0) >> 8) & 255, r_last = (row_at(kw1) >> 8) & 255;
        // the last row of loop r_first inside [kw0, kw1]
        const bool in0 = lane >= kw0 && lane <= kw1 && (int)((w0 >> 8) & 255) == r_first;
        const bool in1 = lane + 64 >= kw0 && lane + 64 <= kw1 && (int)((w1 >> 8) & 255) == r_first;
        const uint64_t b0 = __ballot(in0), b1 = __ballot(in1);
        const int ka = b1 ? 64 + 63 - __builtin_clzll(b1) : 63 - __builtin_clzll(b0);
        wl[0] = r_first;
        wimax[0] = row_at(ka) & 255;
        n_wl = 1;
        if (r_last != r_first) {
            wl[1] = (row_at(ka + 1) >> 8) & 255;
            wimax[1] = row_at(kw1) & 255;
            n_wl = 2;
            wl_more = r_last != wl[1];
        }
    }
    // Draft-block tiles: the wave's loop slot kh (its first or second loop)
    // is applied by this wave before the halves merge.  Its rows (keys < 8)
    // are prefetched into registers: piece pc = (kv*8 + key)*(D/8) + chunk,
    // lane holds pc = lane + 64k.
    constexpr int PB = D / 32;                   // prefetched pieces per lane
    // (not with 256 dims of row tiles per wave, whose steps need those registers)
    constexpr bool kPf = D * RTW < 256 && !PRIV;
    const bool pf_ok = kPf && it.last && !wl_more && kh < n_wl && (kh ? wimax[1] : wimax[0]) < 8;
    uint4 pf[PB];
    if (kPf) {
        const int my_r = kh ? wl[1] : wl[0];
        const int my_imax = kh ? wimax[1] : wimax[0];
        const uint16_t* pbk = a.bk.p + it.b * a.bk.sb + (int64_t)(my_r - 1) * a.bk.sp + it.g * a.bk.sh;
        const uint16_t* pbv = a.bv.p + it.b * a.bv.sb + (int64_t)(my_r - 1) * a.bv.sp + it.g * a.bv.sh;
#pragma unroll
        for (int k = 0; k < PB; ++k) {
            const int pc = lane + 64 * k;
            const int c8 = pc % (D / 8), rest = pc / (D / 8);
            const int key = rest % 8, kv = rest / 8;
            pf[k] = make_uint4(0, 0, 0, 0);
            if (pf_ok && key < a.n_blk && key <= my_imax)
                pf[k] = *reinterpret_cast<const uint4*>((kv ? pbv + key * a.bv.st : pbk + key * a.bk.st) + c8 * 8);
        }
    }


    // Iteration j computes this half's tile j from registers; the key half of
    // tile j + 1 is read from LDS once the scores of tile j are formed, its
    // value half once O has taken tile j.  Tile j - 1 + S goes into the stage
    // of tile j - 1, whose reads every wave finished before this barrier.
    const int n_mine = kh == 0 ? n_iter : n_tiles / 2;   // tiles of this half
    Frags<D> f;
    // after this barrier the queries and every wave's part of tile 0 are in
    // LDS (the S - 2 groups issued after tile 0 may be outstanding); the asm
    // text differs from the loop's barrier so the two are never merged
    __builtin_amdgcn_s_waitcnt(0xF70 | ((P - 1) * PT));
    asm volatile("s_barrier ; queries and tile 0" ::: "memory");
#pragma unroll
    for (int t = 0; t < RTW; ++t)
#pragma unroll
        for (int c = 0; c < D / 32; ++c) rt[t].q[c] = s_q[rw][t * (D / 32) + c][lane];
    if (n_mine > 0) {
        lds_keys<D>(s_tile[0][kh], f, lane);
        lds_values<D>(s_tile[0][kh], f, lane);
    }
    int sj = 0;                                   // stage of tile j
    int sn = 1;                                   // stage of tile j + 1
    // A barrier every K steps.  At a step j that is a multiple of K every wave
    // waits for its parts of tiles j + 1 .. j + K, the barrier makes them
    // visible (and every wave has read tiles up to j by then), and the next K
    // tiles of the stream go into the stages of tiles j - K + 1 .. j.  Between
    // barriers the waves sharing a SIMD can drift apart.
    auto advance = [&](int j) {
        if (K > 1 && j % K) return;
        // (and no LDS read of this wave in flight: the first barrier of the
        // loop frees the queries' stage)
        __builtin_amdgcn_s_waitcnt(0x070 | ((P - 1 - K) * PT));
        asm volatile("s_barrier" ::: "memory");
        // tile m of the stream lives in stage m mod S; the next K tiles,
        // P + j .. P + j + K - 1, replace tiles consumed by now
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if (ti < n_tiles) issue_next(s_tile[si][kh]);
            else issue_dummy(s_tile[si][kh]);
            si = si == S - 1 ? 0 : si + 1;
        }
    };
    auto next_keys = [&](int j) {
        if (j + 1 < n_mine) lds_keys<D>(s_tile[sn][kh], f, lane);
    };
    auto next_values = [&](int j) {
        if (j + 1 < n_mine) lds_values<D>(s_tile[sn][kh], f, lane);
        sj = sn;
        sn = sn == S - 1 ? 0 : sn + 1;
    };
    // A wave without valid row-heads (the workgroup's last row block, or few
    // rows) only takes its part in the loads and barriers.
    int j = 0;
    if (u_w >= a.M) {
        for (; j < n_iter; ++j) {
            advance(j);
            sj = sn;                              // the stage cursors still move
            sn = sn == S - 1 ? 0 : sn + 1;
        }
    }
    // fast phase: every row-head reads both tiles of the iteration in full.
    // The next tile's operands are read without a test (past this half's
    // last tile the stage holds whatever its dummy loads bring, and no step
    // uses those operands), so the step from the scores' matrix instructions
    // to their first reader is one block.
    // The fast steps whose issues are all deep tiles of the stream (every
    // step before the last few of a long chunk) issue them without the tests
    // of issue_next: j < n_fd, a whole number of barrier groups.  The split
    // point may differ between the halves; both loops pass the same barriers.
    const int n_sdeep = PRIV ? n_tiles : n_deep;  // deep tiles of the stream
    int n_fd = min(n_fast, (n_sdeep - kh + 1) / 2 - P);
    n_fd = n_fd < 0 ? 0 : n_fd / K * K;
    auto fast_step = [&](int j, bool deep_issue) {
        const bool bar = K == 1 || j % K == 0;
        if (bar) {
            __builtin_amdgcn_s_waitcnt(0x070 | ((P - 1 - K) * PT));
            asm volatile("s_barrier" ::: "memory");
        }
        float x[RTW][8], bx[RTW];
#pragma unroll
        for (int tr = 0; tr < RTW; ++tr) bx[tr] = tile_scores<D>(rt[tr], f, x[tr]);
        // (K = 1, deep issue: half the run now, half after the exponentials)
        constexpr bool kSplitRun = K == 1 && PT % 2 == 0;
        const uint32_t l_run = lds_addr(s_tile[si][kh]) + rw * PT * 1024;
        if (bar) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                if (deep_issue && kSplitRun) {
                    dma16_run<PT / 2>(iKV, voff, l_run);
                } else if (deep_issue) {              // (si moves with k)
                    dma16_run<PT>(iKV, voff, lds_addr(s_tile[si][kh]) + rw * PT * 1024);
                    ti += 2;
                    iKV += 2 * TILE;
                            } else if (ti < n_tiles) {
                    issue_next(s_tile[si][kh]);
                } else {
                    issue_dummy(s_tile[si][kh]);
                }
                si = si == S - 1 ? 0 : si + 1;
            }
        }
        lds_keys<D>(s_tile[sn][kh], f, lane);
        tiles_fast<D, RTW>(rt, f, x, bx, sl2);
        if (deep_issue && kSplitRun) {
            dma16_run<PT / 2>(iKV + PT / 2 * 512, voff, l_run + PT / 2 * 1024);
            ti += 2;
            iKV += 2 * TILE;
            }
        lds_values<D>(s_tile[sn][kh], f, lane);
        sj = sn;
        sn = sn == S - 1 ? 0 : sn + 1;
    };
    for (; j < n_fd; ++j) fast_step(j, true);
    for (; j < n_fast; ++j) fast_step(j, false);
    // general phase: deep tiles with masks, then ring tiles
    int cpl = 0, cst = 0;                         // ring cursor of the compute side
    for (; j < n_iter; ++j) {
        advance(j);
        const int t = 2 * j + kh;
        float x[RTW][8];
        int mode[RTW];                            // 0 skip, 1 masked, 2 full
        bool v[RTW][8];
        if (t < n_tiles) {
            if (PRIV || t < n_deep) {
                const int base = d0 + 32 * t;
#pragma unroll
                for (int tr = 0; tr < RTW; ++tr) {
                    mode[tr] = base >= any_lim[tr] ? 0 : (base + 32 <= full_lim[tr] ? 2 : 1);
                    const int lim = min(rt[tr].e, d1);
                    const bool ok = RI_OK(rt[tr].ri);
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[tr][e] = ok && base + key_of(e, q) < lim;
                }
            } else {
                if (t - 2 < n_deep) { cpl = 0; cst = t - n_deep; }
                while (cst >= ring_tiles) { cst -= ring_tiles; ++cpl; }
                const int r = cpl < 64 ? __builtin_amdgcn_readlane(loops_v0, cpl)
                                       : __builtin_amdgcn_readlane(loops_v1, cpl - 64);
                const int base = cst * 32;
                cst += 2;
#pragma unroll
                for (int tr = 0; tr < RTW; ++tr) mode[tr] = mask_ring<D>(rt[tr], it, (int)a.WR, r, base, q, v[tr]);
            }
        } else {
#pragma unroll
            for (int tr = 0; tr < RTW; ++tr) mode[tr] = 0;
        }
        float bx[RTW];
#pragma unroll
        for (int tr = 0; tr < RTW; ++tr)
            if (mode[tr]) bx[tr] = tile_scores<D>(rt[tr], f, x[tr]);
        next_keys(j);
#pragma unroll
        for (int tr = 0; tr < RTW; ++tr) {
            if (mode[tr] == 2) tile_finish_full<D>(rt[tr], f, x[tr], bx[tr], sl2);
            else if (mode[tr] == 1) tile_finish_masked<D>(rt[tr], f, x[tr], v[tr], bx[tr], sl2);
        }
        next_values(j);
    }
    __builtin_amdgcn_s_waitcnt(0xF70);            // no direct load left in flight

    // every wave's loads are done and every wave has left the stages
    lds_barrier();
    // draft-block tiles of the wave's loop slot kh, staged in a wave-private
    // part of the stages (K in storage order, V transposed)
    if (!PRIV && it.last && kh < n_wl) {
        uint16_t* sk = &s_tile[0][0][0] + (rw * 2 + kh) * 2 * TILE;
        uint16_t* sv = sk + TILE;
        const int r = kh ? wl[1] : wl[0];
        const int imax = kh ? wimax[1] : wimax[0];
        const uint16_t* bK = a.bk.p + it.b * a.bk.sb + (int64_t)(r - 1) * a.bk.sp + it.g * a.bk.sh;
        const uint16_t* bV = a.bv.p + it.b * a.bv.sb + (int64_t)(r - 1) * a.bv.sp + it.g * a.bv.sh;
        for (int base = 0; base <= imax; base += 32) {
            if (pf_ok) {
                for (int z = lane; z < 2 * TILE / 8; z += 64)
                    *reinterpret_cast<uint4*>(sk + z * 8) = make_uint4(0, 0, 0, 0);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int k = 0; k < PB; ++k) {
                    const int pc = lane + 64 * k;
                    const int c8 = pc % (D / 8), rest = pc / (D / 8);
                    const int key = rest % 8, kv = rest / 8;
                    if (kv == 0) {
                        *reinterpret_cast<uint4*>(sk + key_off(key, c8 * 8, D)) = pf[k];
                    } else {
                        const uint32_t w[4] = {pf[k].x, pf[k].y, pf[k].z, pf[k].w};
#pragma unroll
                        for (int cc = 0; cc < 8; ++cc)
                            sv[val_off(key, c8 * 8 + cc, D)] = (uint16_t)(w[cc >> 1] >> (16 * (cc & 1)));
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            } else {
                stage_block<D>(a, bK, bV, base, sk, sv, lane);
            }
            Frags<D> f;
            load_frags<D>(sk, sv, f, n, q);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int tr = 0; tr < RTW; ++tr) {
                bool v[8];
                if (mask_block<D>(rt[tr], r, base, q, v)) tile_update<D>(rt[tr], f, false, v, sl2);
            }
        }
    }

    // merge half 1 into half 0 (lane-wise: both hold the same row-heads)
    lds_barrier();
    float* s_m = reinterpret_cast<float*>(&s_tile[0][0][0]);
    if (kh == 1) {
#pragma unroll
        for (int tr = 0; tr < RTW; ++tr) {
            float* dst = s_m + ((rw * RTW + tr) * 64 + lane) * MS;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j) dst[dt * 4 + j] = rt[tr].o[dt][j];
            dst[D / 4] = rt[tr].m;
            dst[D / 4 + 1] = rt[tr].l;
        }
    }
    lds_barrier();
    if (kh == 0) {
#pragma unroll
        for (int tr = 0; tr < RTW; ++tr) {
#pragma unroll
            for (int src_i = 0; src_i < (PRIV ? 2 : 1); ++src_i) {
                const float* src = s_m + (src_i * 4 * RTW * 64 + (rw * RTW + tr) * 64 + lane) * MS;
                const float m2 = src[D / 4], l2 = src[D / 4 + 1];
                const float mn = fmaxf(rt[tr].m, m2);
                const float w1 = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(rt[tr].m - mn);
                const float w2 = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
                rt[tr].m = mn;
                rt[tr].l = rt[tr].l * w1 + l2 * w2;
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) rt[tr].o[dt][j] = rt[tr].o[dt][j] * w1 + src[dt * 4 + j] * w2;
            }
        }
    }
    lds_barrier();                                 // merge buffer free again
    if (kh == 1) return;

    if (!PRIV && it.last) {
        uint16_t* sk = &s_tile[0][0][0] + rw * 2 * TILE;   // per-wave scratch in the stages
        uint16_t* sv = sk + TILE;
        if (wl_more) {
            // loops beyond the first two (unusual row sets): smallest remaining first
            int done = 0;
#pragma unroll
            for (int t = 0; t < RTW; ++t)
                if (RI_OK(rt[t].ri) && ((int)RI_R(rt[t].ri) == wl[0] || (int)RI_R(rt[t].ri) == wl[1]))
                    done |= 1 << t;
            for (;;) {
                int r = 1 << 30;
#pragma unroll
                for (int t = 0; t < RTW; ++t)
                    if (RI_OK(rt[t].ri) && !((done >> t) & 1)) r = min(r, (int)RI_R(rt[t].ri));
                r = wave_min(r);
                if (r == 1 << 30) break;
                int im = 0;
#pragma unroll
                for (int t = 0; t < RTW; ++t)
                    if (RI_OK(rt[t].ri) && RI_R(rt[t].ri) == r) {
                        im = max(im, (int)RI_I(rt[t].ri));
                        done |= 1 << t;
                    }
                im = wave_max(im);
                const uint16_t* bK = a.bk.p + it.b * a.bk.sb + (int64_t)(r - 1) * a.bk.sp + it.g * a.bk.sh;
                const uint16_t* bV = a.bv.p + it.b * a.bv.sb + (int64_t)(r - 1) * a.bv.sp + it.g * a.bv.sh;
                for (int base = 0; base <= im; base += 32) {
                    stage_block<D>(a, bK, bV, base, sk, sv, lane);
                    Frags<D> f;
                    load_frags<D>(sk, sv, f, n, q);
                    __builtin_amdgcn_wave_barrier();
#pragma unroll
                    for (int tr = 0; tr < RTW; ++tr) {
                        bool v[8];
                        if (mask_block<D>(rt[tr], r, base, q, v)) tile_update<D>(rt[tr], f, false, v, sl2);
                    }
                }
            }
        }
    }

#pragma unroll
    for (int tr = 0; tr < RTW; ++tr) {
        sum_lane_groups<D>(rt[tr]);
        write_result_word<D>(a, it, rt[tr], u_w + 16 * tr + n, rword[tr], q);
    }
}

// ---------------------------------------------------------------- few rows

struct Job {
    int kind;              // 0 deep, 1 ring, 2 block
    int r;
    int base;              // first position (deep), slot (ring), block offset (block)
    const uint16_t* K;
    const uint16_t* V;
};

// WIN: windowed draft attention (sinks and a window of committed keys).
// NW waves (4, two workgroups per compute unit, or 8, one): eight halve the
// tiles each wave reads in turn, for items that one workgroup reads unsplit.
template <int D, int RT, bool WIN, int NW>
__global__ void __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) k_verify_keys(VerifyArgs a) {
    static_assert(NW == 4 || NW == 8, "four or eight waves");
    constexpr int kStage = NW * 2 * 32 * D;            // uint16: per-wave block tiles
    constexpr int kMerge = NW / 2 * RT * 16 * (D + 2); // floats: merge buffers
    constexpr int kLds = (kStage * 2 > kMerge * 4) ? kStage * 2 : kMerge * 4;
    __shared__ __attribute__((aligned(16))) unsigned char s_raw[kLds];
    __shared__ int s_lw[NW][64];                       // per wave: loop list

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, q = lane >> 4;
    const int G = a.group;
    // rows of the row block (sorted by loop, then block offset): row k_lo +
    // lane in lane `lane` of w0, at most 16*RT/G + 1 of them; loaded before
    // the sequence is known, so the two loads overlap
    const int u_base = (int)((blockIdx.x >> 3) % a.nrb) * 16 * RT;
    const int k_lo = u_base / G;
    const int nk = min(a.rows_here, (min(a.M, u_base + 16 * RT) + G - 1) / G) - k_lo;
    const uint32_t w0 = lane < nk ? a.rows[k_lo + lane] : 0u;

    Item it;
    if (!decode_item(a, it)) return;
    // A wave's first tile is usually the deep tile at d0 + 32*wave: request it
    // now, before the row-dependent set-up (clamped into the sequence's deep
    // rows; reloaded below if the wave's first job is another tile).
    const int d0 = (int)((int64_t)it.c * a.cl);
    const int64_t dreg = ((int64_t)it.b * a.Hkv + it.g) * a.CP * D;
    const int spec_base = (int)min((int64_t)d0 + 32 * wave, a.CP - 32);
    Frags<D> f;
    load_frags<D>(a.deep_k + dreg + (int64_t)spec_base * D, a.deep_v + dreg + (int64_t)spec_base * D, f, n, q);
    uint16_t* const sk = reinterpret_cast<uint16_t*>(s_raw) + wave * 2 * 32 * D;
    uint16_t* const sv = sk + 32 * D;
    float (*s_st)[RT][16][D + 2] = reinterpret_cast<float (*)[RT][16][D + 2]>(s_raw);

    // deep extent of the workgroup: the largest e_row of its rows
    const int rr = (w0 >> 8) & 255, ii = w0 & 255;
    const int E = wave_max(lane < nk ? e_row(a, it.L, ii, rr) : 0);
    // loops of the row block, ascending: loop p in lane p of lw as r | imax << 8
    // (a loop's rows are sorted by offset, so its last row has the largest);
    // every wave builds the list itself, in its own LDS row
    const int rprev = __shfl(rr, (lane + 63) & 63), rnext = __shfl(rr, (lane + 1) & 63);
    const bool first = lane < nk && (lane == 0 || rprev != rr);
    const bool lastr = lane < nk && (lane + 1 == nk || rnext != rr);
    const uint64_t fmask = __ballot(first);
    const int nloops = __popcll(fmask);
    if (lastr) s_lw[wave][__popcll(fmask & ((2ull << lane) - 1)) - 1] = rr | (ii << 8);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int lw = lane < nloops ? s_lw[wave][lane] : 0;
    const int loop_r = lw & 255;
    // draft-block tiles of loops 0..p (inclusive running sum in lane p)
    int bend = lane < nloops ? (lw >> 8) / 32 + 1 : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int x = __shfl_up(bend, o);
        if (lane >= o) bend += x;
    }
    // loops are ascending and R is the largest, so the loops r < R are the
    // first n_ring_planes of the list
    const bool has_R = nloops > 0 && __builtin_amdgcn_readlane(loop_r, nloops - 1) == a.R;
    const int n_ring_planes = nloops - (has_R ? 1 : 0);

    const int d1 = (int)min((int64_t)d0 + a.cl, (int64_t)E);
    const int n_deep_all = d1 > d0 ? (d1 - d0 + 31) / 32 : 0;
    // a windowed draft skips the deep tiles that lie wholly between the sinks
    // and the lowest window start of the workgroup's rows: tiles gap_at ..
    // gap_at + gap_n - 1 of the chunk
    constexpr bool windowed = WIN;
    int gap_at = n_deep_all, gap_n = 0;
    if (windowed) {
        const int lo_min = wave_min(lane < nk ? max(0, it.L + ii - a.w_draft) : 0x7fffffff);
        const int g0 = max(d0, (a.n_sink + 31) / 32 * 32), g1 = min(d1, lo_min / 32 * 32);
        if (g1 > g0) {
            gap_at = (g0 - d0) / 32;
            gap_n = (g1 - g0) / 32;
        }
    }
    const int n_deep = n_deep_all - gap_n;
    const int ring_tiles = (it.last && a.R > 1 && it.nsl > 0) ? (it.nsl + 31) / 32 : 0;
    const int n_ring = n_ring_planes * ring_tiles;
    const int n_block = it.last ? __builtin_amdgcn_readlane(bend, 63) : 0;
    const int n_jobs = n_deep + n_ring + n_block;
    const int64_t rreg0 = ((int64_t)it.b * a.Hkv + it.g) * a.NR * a.WP * D;
    const float sl2 = a.scale_log2;

    // job j of the workgroup (wave-uniform j): deep tiles, then ring tiles
    // plane by plane, then draft-block tiles loop by loop
    auto job_of = [&](int j) -> Job {
        Job jb;
        if (j < n_deep) {
            jb.kind = 0;
            jb.r = a.R;
            jb.base = d0 + (j < gap_at ? j : j + gap_n) * 32;
            jb.K = a.deep_k + dreg + (int64_t)jb.base * D;
            jb.V = a.deep_v + dreg + (int64_t)jb.base * D;
            return jb;
        }
        j -= n_deep;
        if (j < n_ring) {
            const int pl = j / ring_tiles, st = j % ring_tiles;
            jb.kind = 1;
            jb.r = __builtin_amdgcn_readlane(loop_r, pl);
            jb.base = st * 32;
            const int64_t rreg = rreg0 + (int64_t)(jb.r - 1) * a.WP * D;
            jb.K = a.ring_k + rreg + (int64_t)jb.base * D;
            jb.V = a.ring_v + rreg + (int64_t)jb.base * D;
            return jb;
        }
        j -= n_ring;
        const int p = (int)__builtin_ctzll(__ballot(lane < nloops && bend > j));
        jb.kind = 2;
        jb.r = __builtin_amdgcn_readlane(loop_r, p);
        jb.base = (j - (p > 0 ? __builtin_amdgcn_readlane(bend, p - 1) : 0)) * 32;
        jb.K = a.bk.p + it.b * a.bk.sb + (int64_t)(jb.r - 1) * a.bk.sp + it.g * a.bk.sh;
        jb.V = a.bv.p + it.b * a.bv.sb + (int64_t)(jb.r - 1) * a.bv.sp + it.g * a.bv.sh;
        return jb;
    };

    // Committed tiles (deep, ring) are read from HBM in the operand order
    // straight into registers.  Where the registers allow (kAhead), one tile
    // ahead: a wave loads the operands of its next committed tile before it
    // computes the current one.  Those loads are unconditional (past its last
    // committed tile a wave reloads the first deep tile and ignores it), so
    // the compiler counts them exactly.
    constexpr bool kAhead = WIN ? D * RT < 128 : D * RT <= 128;
    const int n_comm = n_deep + n_ring;
    auto comm_load = [&](int j, Frags<D>& f) {
        const uint16_t* K = a.deep_k + dreg;
        const uint16_t* V = a.deep_v + dreg;
        if (j < n_comm) {
            const Job jb = job_of(j);
            K = jb.K;
            V = jb.V;
        }
        load_frags<D>(K, V, f, n, q);
    };
    if (wave >= n_deep || wave >= gap_at) comm_load(wave, f);   // not the tile requested early
    RowTile<D> rt[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int u = u_base + 16 * t + n;
        init_row_word<D>(a, it, u, __shfl(w0, u < a.M ? u / G - k_lo : 0), q, rt[t]);
    }

    for (int j = wave; j < n_jobs; j += NW) {
        const Job jb = job_of(j);
        const int kind = __builtin_amdgcn_readfirstlane(jb.kind);
        const int jr = __builtin_amdgcn_readfirstlane(jb.r);
        const int base = __builtin_amdgcn_readfirstlane(jb.base);
        Frags<D> fn;
        if (kAhead) comm_load(j + NW, fn);
        else if (kind != 2 && j != wave) comm_load(j, f);
        if (kind == 2) {
            stage_block<D>(a, jb.K, jb.V, base, sk, sv, lane);
            load_frags<D>(sk, sv, f, n, q);
            __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int tr = 0; tr < RT; ++tr) {
            bool v[8];
            int mode;
            if (kind == 0) mode = mask_deep<D>(rt[tr], base, d1, q, v);
            else if (kind == 1) mode = mask_ring<D>(rt[tr], it, (int)a.WR, jr, base, q, v);
            else mode = mask_block<D>(rt[tr], jr, base, q, v);
            if (windowed && kind < 2 && mode)
                mode = mask_window<D>(rt[tr], it, kind, base, a.n_sink, (int)a.WR, q, mode, v);
            if (mode) tile_update<D>(rt[tr], f, mode == 2, v, sl2);
        }
        if (kAhead) f = fn;
    }

    // merge the waves' states pairwise: (NW/2 .. NW-1) -> (0 .. NW/2-1) -> .. -> 0
#pragma unroll
    for (int tr = 0; tr < RT; ++tr) sum_lane_groups<D>(rt[tr]);
    auto put = [&](int buf) {
#pragma unroll
        for (int tr = 0; tr < RT; ++tr) {
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) s_st[buf][tr][n][dt * 16 + 4 * q + jj] = rt[tr].o[dt][jj];
            if (q == 0) {
                s_st[buf][tr][n][D] = rt[tr].m;
                s_st[buf][tr][n][D + 1] = rt[tr].l;
            }
        }
    };
    auto take = [&](int buf) {
#pragma unroll
        for (int tr = 0; tr < RT; ++tr) {
            const float m2 = s_st[buf][tr][n][D], l2 = s_st[buf][tr][n][D + 1];
            const float mn = fmaxf(rt[tr].m, m2);
            const float w1 = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(rt[tr].m - mn);
            const float w2 = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
            rt[tr].m = mn;
            rt[tr].l = rt[tr].l * w1 + l2 * w2;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    rt[tr].o[dt][jj] = rt[tr].o[dt][jj] * w1 + s_st[buf][tr][n][dt * 16 + 4 * q + jj] * w2;
        }
    };
    __syncthreads();            // every wave is done with its staging tile
#pragma unroll
    for (int half = NW / 2; half > 1; half /= 2) {
        if (wave >= half && wave < 2 * half) put(wave - half);
        __syncthreads();
        if (wave < half) take(wave);
        __syncthreads();
    }
    if (wave == 1) put(0);
    __syncthreads();
    if (wave != 0) return;
    take(0);
#pragma unroll
    for (int tr = 0; tr < RT; ++tr) {
        const int u = u_base + 16 * tr + n;
        write_result_word<D>(a, it, rt[tr], u, __shfl(w0, u < a.M ? u / G - k_lo : 0), q);
    }
}

// ---------------------------------------------------------------- combine

// Merge the chunk partials of every row-head of multi-chunk sequences:
// M = max m_c, l = sum l_c 2^(m_c - M), O = sum O_c 2^(m_c - M) / l.
// One wave per row-head.  Lane c reads the (m, l) of chunk c, so the chunk
// states arrive together; the value rows of eight chunks are loaded before
// any is summed, so the loads overlap instead of forming a chain.  With at
// most eight chunks (the usual case) the value rows are requested together
// with the states, and the chunk count comes with the arguments, so the
// merge waits for one round of loads.
template <int D>
__global__ void __launch_bounds__(256) k_combine(VerifyArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    // row-heads of the split sequences only, where the launch lists them
    const int64_t total = (int64_t)(a.n_split > 0 ? a.n_split : a.B) * a.Hkv * a.M;
    if (idx >= total) return;
    const int u = (int)(idx % a.M);
    const int sg = (int)(idx / a.M);
    const int g = sg % a.Hkv, b = a.n_split > 0 ? (int)a.split_b[sg / a.Hkv] : sg / a.Hkv;
    const int bg = b * a.Hkv + g;
    int nc_b = b < kMaxSeqArgs ? a.snc[b] : 0;
    if (nc_b == 0) {
        const int64_t L = a.lens[b];
        nc_b = L > 0 ? (int)((L + a.cx + a.cl - 1) / a.cl) : 1;
    }
    if (nc_b == 1) return;
    const int64_t cs = (int64_t)a.M * (D + 2);                  // chunk stride
    const float* pu = a.part + (int64_t)bg * a.nc * cs + (int64_t)u * (D + 2);
    constexpr int NE = (D + 63) / 64;
    constexpr int CB = 8;                                          // chunks per batch of loads
    float acc[NE], lt = 0.f, mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < NE; ++t) acc[t] = 0.f;
    if (nc_b <= CB) {
        // every load at once: the (m, l) of chunk `lane` and the value rows
        // of all chunks (they do not depend on the maximum)
        float m = -INFINITY, l = 0.f;
        if (lane < nc_b) {
            m = pu[lane * cs + D];
            l = pu[lane * cs + D + 1];
        }
        float v[CB][NE];
#pragma unroll
        for (int j = 0; j < CB; ++j)
#pragma unroll
            for (int t = 0; t < NE; ++t) {
                const int e = lane + 64 * t;
                v[j][t] = (j < nc_b && e < D) ? pu[j * cs + e] : 0.f;
            }
        mx = m;
#pragma unroll
        for (int o = 1; o < CB; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        mx = __shfl(mx, 0);
        const float w = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mx);
        lt = w * l;
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            const float wj = __shfl(w, j);
#pragma unroll
            for (int t = 0; t < NE; ++t) acc[t] += wj * v[j][t];
        }
    } else {
        for (int c = lane; c < nc_b; c += 64) mx = fmaxf(mx, pu[c * cs + D]);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        for (int c0 = 0; c0 < nc_b; c0 += 64) {
            float w = 0.f;
            if (c0 + lane < nc_b) {
                const float* p = pu + (c0 + lane) * cs;
                const float m = p[D];
                w = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mx);
                lt += w * p[D + 1];
            }
            const int n = min(64, nc_b - c0);
            for (int k = 0; k < n; k += CB) {
                float v[CB][NE];
#pragma unroll
                for (int j = 0; j < CB; ++j)
#pragma unroll
                    for (int t = 0; t < NE; ++t) {
                        const int e = lane + 64 * t;
                        v[j][t] = (k + j < n && e < D) ? pu[(c0 + k + j) * cs + e] : 0.f;
                    }
#pragma unroll
                for (int j = 0; j < CB; ++j) {
                    const float wj = __shfl(w, k + j);
#pragma unroll
                    for (int t = 0; t < NE; ++t) acc[t] += wj * v[j][t];
                }
            }
        }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) lt += __shfl_xor(lt, o);
    const uint32_t rw = a.rows[u / a.group];
    const int orig = (int)(rw >> 16), h = g * a.group + u % a.group;
    float* op = a.out + (((int64_t)b * a.n_rows + orig) * a.Hq + h) * D;
    const float inv = 1.f / lt;
#pragma unroll
    for (int t = 0; t < NE; ++t) {
        const int e = lane + 64 * t;
        if (e < D) __builtin_nontemporal_store(acc[t] * inv, op + e);   // (final rows, as above)
    }
    if (lane == 0) a.lse[((int64_t)b * a.n_rows + orig) * a.Hq + h] = (mx + log2f(lt)) * kLn2;
}

template <typename K>
hipError_t launch_items(K kern, const VerifyArgs& a, hipStream_t s, int threads = 256) {
    const int64_t slots = (int64_t)a.nrb * ((a.n_groups + 7) / 8);
    hipLaunchKernelGGL(kern, dim3((unsigned)(8 * slots)), dim3(threads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_verify_keys(const VerifyArgs& a, int rt, bool wide, hipStream_t s) {
    if (rt < 1 || rt > keys_max_row_tiles(a.d)) return hipErrorInvalidValue;
    const bool win = a.w_draft >= 0;
    if (wide && win) return hipErrorInvalidValue;
    if (wide) {
        switch (a.d * 4 + rt) {
            case 64 * 4 + 1: return launch_items(k_verify_keys<64, 1, false, 8>, a, s, 512);
            case 64 * 4 + 2: return launch_items(k_verify_keys<64, 2, false, 8>, a, s, 512);
            case 96 * 4 + 1: return launch_items(k_verify_keys<96, 1, false, 8>, a, s, 512);
            case 96 * 4 + 2: return launch_items(k_verify_keys<96, 2, false, 8>, a, s, 512);
            case 128 * 4 + 1: return launch_items(k_verify_keys<128, 1, false, 8>, a, s, 512);
        }
        return hipErrorInvalidValue;
    }
    switch (a.d * 8 + rt * 2 + (win ? 1 : 0)) {
        case 64 * 8 + 2: return launch_items(k_verify_keys<64, 1, false, 4>, a, s);
        case 64 * 8 + 4: return launch_items(k_verify_keys<64, 2, false, 4>, a, s);
        case 96 * 8 + 2: return launch_items(k_verify_keys<96, 1, false, 4>, a, s);
        case 96 * 8 + 4: return launch_items(k_verify_keys<96, 2, false, 4>, a, s);
        case 128 * 8 + 2: return launch_items(k_verify_keys<128, 1, false, 4>, a, s);
        case 64 * 8 + 3: return launch_items(k_verify_keys<64, 1, true, 4>, a, s);
        case 64 * 8 + 5: return launch_items(k_verify_keys<64, 2, true, 4>, a, s);
        case 96 * 8 + 3: return launch_items(k_verify_keys<96, 1, true, 4>, a, s);
        case 96 * 8 + 5: return launch_items(k_verify_keys<96, 2, true, 4>, a, s);
        case 128 * 8 + 3: return launch_items(k_verify_keys<128, 1, true, 4>, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_verify_rows(const VerifyArgs& a, int rtw, bool priv, hipStream_t s) {
    if (rtw < 1 || rtw > rows_max_row_tiles(a.d)) return hipErrorInvalidValue;
    if (priv && !rows_private_waves(a.d, rtw)) return hipErrorInvalidValue;
    switch (a.d * 4 + rtw) {
        case 64 * 4 + 1:
            return priv ? launch_items(k_verify_rows<64, 1, true>, a, s, 768)
                        : launch_items(k_verify_rows<64, 1, false>, a, s, 512);
        case 64 * 4 + 2:
            return priv ? launch_items(k_verify_rows<64, 2, true>, a, s, 768)
                        : launch_items(k_verify_rows<64, 2, false>, a, s, 512);
        case 96 * 4 + 1:
            return priv ? launch_items(k_verify_rows<96, 1, true>, a, s, 768)
                        : launch_items(k_verify_rows<96, 1, false>, a, s, 512);
        case 128 * 4 + 1: return launch_items(k_verify_rows<128, 1, false>, a, s, 512);
        case 128 * 4 + 2: return launch_items(k_verify_rows<128, 2, false>, a, s, 512);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_combine(const VerifyArgs& a, hipStream_t s) {
    const int64_t units = (int64_t)(a.n_split > 0 ? a.n_split : a.B) * a.Hkv * a.M;
    const unsigned blocks = (unsigned)((units + 3) / 4);
    if (blocks == 0) return hipSuccess;
    switch (a.d) {
        case 64: hipLaunchKernelGGL(k_combine<64>, dim3(blocks), dim3(256), 0, s, a); break;
        case 96: hipLaunchKernelGGL(k_combine<96>, dim3(blocks), dim3(256), 0, s, a); break;
        case 128: hipLaunchKernelGGL(k_combine<128>, dim3(blocks), dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ripe
