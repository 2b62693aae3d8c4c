/*
 * RIPE verification-attention oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct fp64 CPU implementation of what the RIPE
 * verification path computes.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load it; the product library never links or
 * calls it, and the two share no code, header, table or helper.
 *
 * What it follows (page "Prefix Keys and Values Matter Late: RIPE Caching for
 * Self-Speculative Decoding in Looped Language Models", abstract):
 *   - a looped model runs one block of layers R times per token, so each
 *     recurrent layer holds R key/value planes per position, and
 *     self-speculative decoding verifies a draft block with all R loops
 *     (first sentence);
 *   - RIPE stores only the deepest plane (loop R) for positions outside a
 *     window of recent positions, and all R planes inside it (fourth sentence);
 *   - a window at least as long as the draft block makes batched verification
 *     independent of how the block is split (fifth sentence).
 *
 * Readings where the pages are silent (each one is argued in the design notes):
 *   - loops are numbered 1..R; a query at loop r reads loop-r keys/values;
 *   - a committed position s is read at plane r when s >= beta, at plane R
 *     otherwise, with beta = t - W for the query anchor (t = L + i is the
 *     query's own position) and beta = L - W for the cache anchor;
 *   - block keys (positions L..L+i) are read at plane r from the caller's
 *     block buffer; causal: a block offset i sees block offsets 0..i;
 *   - scores are q.k / sqrt(d); LSE is a natural log; GQA head h reads KV
 *     head h / (Hq / Hkv).
 *
 * Storage layout (the byte contract the GPU library must reproduce exactly):
 *   sections, each starting at a multiple of 256 bytes, in this order
 *     lens   int32 [NL][B]
 *     deep_k bf16  [NL][B][Hkv][CP*d]          CP = roundup(capacity, 32)
 *     deep_v bf16  [NL][B][Hkv][CP*d]
 *     ring_k bf16  [NL][B][Hkv][R-1][WP*d]     WR = min(W, capacity), WP = roundup(WR, 32)
 *     ring_v bf16  [NL][B][Hkv][R-1][WP*d]
 *   inside a (layer, seq, head[, plane]) region, row p (a position for deep,
 *   a ring slot p mod WR for the ring) and dimension e live at
 *     K: (p/32)*32*d + (e/32)*1024 + (p%32)*32 + e%32
 *     V: (p/32)*32*d + e*32 + slot(p%32),
 *        slot(k) = 8*((k%16)/4) + 4*(k/16) + k%4
 *   Unwritten bytes stay zero.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORA_OK 0
#define ORA_EINVAL 1
#define ORA_ECAPACITY 2
#define ORA_EMISSING 4   /* a key/value plane the rule needs is not stored */

typedef struct {
    int32_t n_layers, n_loops, n_heads_q, n_heads_kv, head_dim;
    int32_t window, batch, capacity, max_block, anchor;
} ora_config;

typedef struct {
    int64_t lens, deep_k, deep_v, ring_k, ring_v, total;
    int64_t cp, wr, wp, nr;
} ora_layout;

static int64_t up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

static int config_ok(const ora_config* c) {
    if (!c) return 0;
    if (c->n_layers < 1 || c->n_loops < 1 || c->n_heads_kv < 1 || c->n_heads_q < 1) return 0;
    if (c->n_heads_q % c->n_heads_kv) return 0;
    if (c->head_dim < 32 || c->head_dim % 32) return 0;
    if (c->window < 0 || c->batch < 1 || c->capacity < 1 || c->max_block < 1) return 0;
    if (c->anchor != 0 && c->anchor != 1) return 0;
    return 1;
}

static void layout_of(const ora_config* c, ora_layout* o) {
    int64_t NL = c->n_layers, B = c->batch, H = c->n_heads_kv, d = c->head_dim;
    o->cp = up(c->capacity, 32);
    o->wr = c->window < c->capacity ? c->window : c->capacity;
    o->nr = c->n_loops - 1;
    if (o->nr == 0) o->wr = 0;
    o->wp = up(o->wr, 32);
    int64_t off = 0;
    o->lens = off;   off = up(off + NL * B * 4, 256);
    o->deep_k = off; off = up(off + NL * B * H * o->cp * d * 2, 256);
    o->deep_v = off; off = up(off + NL * B * H * o->cp * d * 2, 256);
    o->ring_k = off; off = up(off + NL * B * H * o->nr * o->wp * d * 2, 256);
    o->ring_v = off; off = up(off + NL * B * H * o->nr * o->wp * d * 2, 256);
    o->total = off;
}

/* element offset of row p, dim e inside one tile region */
static int64_t k_index(int64_t p, int64_t e, int64_t d) {
    return (p / 32) * 32 * d + (e / 32) * 1024 + (p % 32) * 32 + e % 32;
}
static int64_t v_slot(int64_t k) { return 8 * ((k % 16) / 4) + 4 * (k / 16) + k % 4; }
static int64_t v_index(int64_t p, int64_t e, int64_t d) {
    return (p / 32) * 32 * d + e * 32 + v_slot(p % 32);
}

static double bf16_to_double(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* ---------------------------------------------------------------- sizes */

int64_t ora_storage_bytes(const ora_config* c) {
    if (!config_ok(c)) return -1;
    ora_layout o;
    layout_of(c, &o);
    return o.total;
}

/* which: 0 lens, 1 deep_k, 2 deep_v, 3 ring_k, 4 ring_v, 5 total,
 *        6 CP, 7 WR, 8 WP */
int64_t ora_layout_value(const ora_config* c, int32_t which) {
    if (!config_ok(c)) return -1;
    ora_layout o;
    layout_of(c, &o);
    switch (which) {
        case 0: return o.lens;
        case 1: return o.deep_k;
        case 2: return o.deep_v;
        case 3: return o.ring_k;
        case 4: return o.ring_v;
        case 5: return o.total;
        case 6: return o.cp;
        case 7: return o.wr;
        case 8: return o.wp;
    }
    return -1;
}

/* ---------------------------------------------------------------- append */

/*
 * Append n_new[b] tokens to every sequence b of one layer.
 *   deep: plane R of the new tokens; element (b, g, t, e) at
 *         dk[b*ds[0] + g*ds[1] + t*ds[2] + e]
 *   win:  planes 1..R-1 of the LAST min(n_new[b], WR) new tokens, oldest
 *         first; element (b, plane r-1, g, u, e) at
 *         wk[b*ws[0] + (r-1)*ws[1] + g*ws[2] + u*ws[3] + e]
 * The ring slot of position p is p mod WR: writing the newest positions into
 * it overwrites the loop-1..R-1 planes of positions that left the window, so
 * only their deepest plane (already in the deep section) remains.
 */
int32_t ora_append(const ora_config* c, void* storage, int32_t layer, const int32_t* n_new,
                   const uint16_t* dk, const uint16_t* dv, const int64_t* ds,
                   const uint16_t* wk, const uint16_t* wv, const int64_t* ws) {
    if (!config_ok(c) || !storage || !n_new || layer < 0 || layer >= c->n_layers) return ORA_EINVAL;
    ora_layout o;
    layout_of(c, &o);
    uint8_t* base = (uint8_t*)storage;
    int32_t* lens = (int32_t*)(base + o.lens) + (int64_t)layer * c->batch;
    const int64_t H = c->n_heads_kv, d = c->head_dim, B = c->batch;
    for (int64_t b = 0; b < B; ++b) {
        if (n_new[b] < 0) return ORA_EINVAL;
        if ((int64_t)lens[b] + n_new[b] > c->capacity) return ORA_ECAPACITY;
    }
    for (int64_t b = 0; b < B; ++b) {
        const int64_t L0 = lens[b], n = n_new[b];
        if (n == 0) continue;
        for (int64_t g = 0; g < H; ++g) {
            const int64_t region = ((layer * B + b) * H + g) * o.cp * d;
            uint16_t* K = (uint16_t*)(base + o.deep_k) + region;
            uint16_t* V = (uint16_t*)(base + o.deep_v) + region;
            for (int64_t t = 0; t < n; ++t)
                for (int64_t e = 0; e < d; ++e) {
                    const int64_t src = b * ds[0] + g * ds[1] + t * ds[2] + e;
                    K[k_index(L0 + t, e, d)] = dk[src];
                    V[v_index(L0 + t, e, d)] = dv[src];
                }
        }
        const int64_t nw = n < o.wr ? n : o.wr;
        for (int64_t r = 1; r <= o.nr; ++r)
            for (int64_t g = 0; g < H; ++g) {
                const int64_t region = (((layer * B + b) * H + g) * o.nr + (r - 1)) * o.wp * d;
                uint16_t* K = (uint16_t*)(base + o.ring_k) + region;
                uint16_t* V = (uint16_t*)(base + o.ring_v) + region;
                for (int64_t u = 0; u < nw; ++u) {
                    const int64_t p = L0 + n - nw + u;
                    const int64_t slot = p % o.wr;
                    for (int64_t e = 0; e < d; ++e) {
                        const int64_t src = b * ws[0] + (r - 1) * ws[1] + g * ws[2] + u * ws[3] + e;
                        K[k_index(slot, e, d)] = wk[src];
                        V[v_index(slot, e, d)] = wv[src];
                    }
                }
            }
        lens[b] = (int32_t)(L0 + n);
    }
    return ORA_OK;
}

/* ---------------------------------------------------------------- verify */

typedef struct {
    const ora_config* c;
    ora_layout o;
    const uint8_t* base;
    int32_t layer;
    const uint16_t* bk;
    const uint16_t* bv;
    const int64_t* bs;   /* block strides: s_b, s_plane, s_head, s_tok */
    int32_t n_blk;
} ctx_t;

/*
 * Fetch the key (kv = 0) or value (kv = 1) vector of position s at loop
 * `plane` for sequence b, KV head g, widened to double.
 */
static int fetch(const ctx_t* x, int64_t b, int64_t g, int64_t L, int64_t s, int64_t plane,
                 int kv, double* out) {
    const ora_config* c = x->c;
    const int64_t d = c->head_dim, H = c->n_heads_kv, B = c->batch, R = c->n_loops;
    if (s >= L) {                       /* a draft-block key, from the caller's buffer */
        const int64_t j = s - L;
        if (j >= x->n_blk) return ORA_EINVAL;
        const uint16_t* p = (kv ? x->bv : x->bk) + b * x->bs[0] + (plane - 1) * x->bs[1] +
                            g * x->bs[2] + j * x->bs[3];
        for (int64_t e = 0; e < d; ++e) out[e] = bf16_to_double(p[e]);
        return ORA_OK;
    }
    if (plane == R) {                   /* the deepest plane is stored for every position */
        const int64_t region = ((x->layer * B + b) * H + g) * x->o.cp * d;
        const uint16_t* p = (const uint16_t*)(x->base + (kv ? x->o.deep_v : x->o.deep_k)) + region;
        for (int64_t e = 0; e < d; ++e)
            out[e] = bf16_to_double(p[kv ? v_index(s, e, d) : k_index(s, e, d)]);
        return ORA_OK;
    }
    /* a shallower plane exists only for the last WR committed positions */
    const int64_t held = L < x->o.wr ? L : x->o.wr;
    if (s < L - held) return ORA_EMISSING;
    const int64_t region = (((x->layer * B + b) * H + g) * x->o.nr + (plane - 1)) * x->o.wp * d;
    const uint16_t* p = (const uint16_t*)(x->base + (kv ? x->o.ring_v : x->o.ring_k)) + region;
    const int64_t slot = s % x->o.wr;
    for (int64_t e = 0; e < d; ++e)
        out[e] = bf16_to_double(p[kv ? v_index(slot, e, d) : k_index(slot, e, d)]);
    return ORA_OK;
}

/* the plane a row at loop r reads for committed or block position s */
static int64_t plane_of(int64_t s, int64_t L, int64_t r, int64_t R, int64_t beta) {
    if (s >= L) return r;     /* block keys: only loop r exists at loop r */
    if (s >= beta) return r;  /* inside the window seen from this query */
    return R;                 /* older positions: the deepest plane */
}

/*
 * Is committed position s (< L) a key of a query at position t?  Every one is
 * for verification (w_win < 0).  A windowed draft (page "Windowed-MTP:
 * Removing the Full-Context Draft-KV Tax at Million-Token Context",
 * abstract: a sliding window plus an attention sink on the draft's attention
 * only) keeps the first n_sink positions and the positions s >= t - w_win.
 */
static int committed_key(int64_t s, int64_t t, int64_t n_sink, int64_t w_win) {
    if (w_win < 0) return 1;
    return s < n_sink || s >= t - w_win;
}

/*
 * Attention for one layer.
 *   rows k = 0..n_rows-1 are (block offset row_blk[k], loop row_loop[k]);
 *   q      bf16 [B][n_rows][Hq][d];
 *   blk_k/blk_v: planes 1..R of the draft block, element (b, r-1, g, j, e)
 *          at b*bs[0] + (r-1)*bs[1] + g*bs[2] + j*bs[3] + e;
 *   n_sink, w_win: the committed keys a query keeps (committed_key above);
 *   want   optional [B][n_rows][Hq] mask of the outputs to compute;
 *   out    double [B][n_rows][Hq][d], lse double [B][n_rows][Hq].
 * For each query: scores q.k/sqrt(d) over its keys among 0..L+i (block keys
 * L..L+i always) at the plane the rule picks, LSE = M + ln sum exp(score -
 * M), O = sum exp(score - LSE) v.
 */
static int32_t attend(const ora_config* c, const void* storage, int32_t layer, int32_t n_rows,
                      const int32_t* row_blk, const int32_t* row_loop, const uint16_t* q,
                      const uint16_t* blk_k, const uint16_t* blk_v, const int64_t* bs,
                      int32_t n_blk, int64_t n_sink, int64_t w_win, const uint8_t* want,
                      double* out, double* lse) {
    if (!config_ok(c) || !storage || layer < 0 || layer >= c->n_layers || n_rows < 0) return ORA_EINVAL;
    if (n_blk < 0 || n_blk > c->max_block) return ORA_EINVAL;
    for (int32_t k = 0; k < n_rows; ++k) {
        if (row_blk[k] < 0 || row_blk[k] >= n_blk) return ORA_EINVAL;
        if (row_loop[k] < 1 || row_loop[k] > c->n_loops) return ORA_EINVAL;
    }
    ctx_t x;
    x.c = c;
    layout_of(c, &x.o);
    x.base = (const uint8_t*)storage;
    x.layer = layer;
    x.bk = blk_k;
    x.bv = blk_v;
    x.bs = bs;
    x.n_blk = n_blk;
    const int32_t* lens = (const int32_t*)(x.base + x.o.lens) + (int64_t)layer * c->batch;
    const int64_t B = c->batch, Hq = c->n_heads_q, d = c->head_dim, R = c->n_loops;
    const int64_t group = c->n_heads_q / c->n_heads_kv;
    const int64_t total = B * n_rows * Hq;
    int32_t status = ORA_OK;

#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t idx = 0; idx < total; ++idx) {
        if (want && !want[idx]) continue;
        const int64_t h = idx % Hq;
        const int64_t k = (idx / Hq) % n_rows;
        const int64_t b = idx / (Hq * n_rows);
        const int64_t L = lens[b], i = row_blk[k], r = row_loop[k];
        const int64_t t = L + i;
        const int64_t beta = c->anchor == 0 ? t - (int64_t)c->window : L - (int64_t)c->window;
        const int64_t g = h / group;
        const int64_t n_keys = t + 1;
        double* qd = (double*)malloc(sizeof(double) * d);
        double* kvec = (double*)malloc(sizeof(double) * d);
        double* sc = (double*)malloc(sizeof(double) * n_keys);
        const uint16_t* qp = q + idx * d;
        for (int64_t e = 0; e < d; ++e) qd[e] = bf16_to_double(qp[e]);
        const double scale = 1.0 / sqrt((double)d);
        int st = ORA_OK;
        double M = -INFINITY;
        for (int64_t s = 0; s < n_keys && st == ORA_OK; ++s) {
            if (s < L && !committed_key(s, t, n_sink, w_win)) {
                sc[s] = -INFINITY;      /* not a key of this query */
                continue;
            }
            st = fetch(&x, b, g, L, s, plane_of(s, L, r, R, beta), 0, kvec);
            double acc = 0.0;
            for (int64_t e = 0; e < d; ++e) acc += qd[e] * kvec[e];
            sc[s] = acc * scale;
            if (sc[s] > M) M = sc[s];
        }
        double sum = 0.0;
        for (int64_t s = 0; s < n_keys; ++s) sum += exp(sc[s] - M);
        const double l = M + log(sum);
        double* o = out + idx * d;
        for (int64_t e = 0; e < d; ++e) o[e] = 0.0;
        for (int64_t s = 0; s < n_keys && st == ORA_OK; ++s) {
            if (sc[s] == -INFINITY) continue;
            st = fetch(&x, b, g, L, s, plane_of(s, L, r, R, beta), 1, kvec);
            const double w = exp(sc[s] - l);
            for (int64_t e = 0; e < d; ++e) o[e] += w * kvec[e];
        }
        lse[idx] = l;
        if (st != ORA_OK) {
#pragma omp atomic write
            status = st;
        }
        free(qd);
        free(kvec);
        free(sc);
    }
    return status;
}

/* Verification attention: every committed position is a key. */
int32_t ora_verify(const ora_config* c, const void* storage, int32_t layer, int32_t n_rows,
                   const int32_t* row_blk, const int32_t* row_loop, const uint16_t* q,
                   const uint16_t* blk_k, const uint16_t* blk_v, const int64_t* bs,
                   int32_t n_blk, const uint8_t* want, double* out, double* lse) {
    return attend(c, storage, layer, n_rows, row_blk, row_loop, q, blk_k, blk_v, bs, n_blk,
                  0, -1, want, out, lse);
}

/* Windowed draft attention: committed keys are the first n_sink positions
 * and the w_draft positions before the query (s >= L + i - w_draft). */
int32_t ora_draft(const ora_config* c, const void* storage, int32_t layer, int32_t n_rows,
                  const int32_t* row_blk, const int32_t* row_loop, const uint16_t* q,
                  const uint16_t* blk_k, const uint16_t* blk_v, const int64_t* bs,
                  int32_t n_blk, int32_t n_sink, int32_t w_draft, const uint8_t* want,
                  double* out, double* lse) {
    if (n_sink < 0 || w_draft < 0) return ORA_EINVAL;
    return attend(c, storage, layer, n_rows, row_blk, row_loop, q, blk_k, blk_v, bs, n_blk,
                  n_sink, w_draft, want, out, lse);
}

/* number of OpenMP threads the oracle will use (for reporting) */
int32_t ora_threads(void) {
    int32_t n = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp single
        n = (int32_t)omp_get_num_threads();
    }
#endif
    return n;
}

/* set the number of OpenMP threads later calls use (n >= 1; for the
 * single-thread CPU baseline) */
void ora_set_threads(int32_t n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
