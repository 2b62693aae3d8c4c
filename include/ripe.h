/*
 * ripe.h -- C ABI of the RIPE verification-attention library for MI355X
 * (gfx950).
 *
 * What it computes.  A looped language model runs one block of layers R times
 * per token, so a recurrent layer holds R key/value planes per position, and
 * self-speculative decoding verifies a draft block with all R loops (page
 * "Prefix Keys and Values Matter Late: RIPE Caching for Self-Speculative
 * Decoding in Looped Language Models", abstract, first sentence).  RIPE keeps
 * the deepest plane (loop R) of every position and all R planes only for a
 * window of the W most recent positions (same abstract, fourth sentence).
 * The library owns the RIPE storage format, appends tokens to it, and
 * evaluates the verification attention of a set of (block offset, loop)
 * query rows -- the D x R grid of a batched verify, or a mixed-depth wave in
 * which each position sits at its own loop (page "WaveFront Decoding" for
 * looped LMs, section on drafting and checking in one pass).
 *
 * Attention rule.  For sequence b with L committed positions, a query row at
 * block offset i and loop r (position t = L + i) attends to keys 0..t:
 *   - block keys L..t at loop r, from the caller's block buffer;
 *   - committed key s at loop r when s >= beta, otherwise at loop R, where
 *     beta = t - W (RIPE_ANCHOR_QUERY) or beta = L - W (RIPE_ANCHOR_CACHE).
 * With the query anchor, W >= D - 1 makes each row's result independent of
 * how the block is split into calls (abstract, fifth sentence); W = 0 is the
 * deepest-plane-only cache and RIPE_WINDOW_FULL the full per-loop cache.
 * Scores are q.k / sqrt(d); out = softmax-weighted values (fp32) and
 * lse = natural-log log-sum-exp of the scores (fp32).  GQA: query head h
 * reads KV head h / (Hq / Hkv).
 *
 * Memory and streams.  Every device buffer belongs to the caller (the
 * Python binding allocates them with PyTorch).  The handle holds only host
 * state: the configuration, the storage pointer and a host copy of the
 * committed lengths.  Calls enqueue kernels on the given HIP stream and
 * return without synchronising; device faults surface at the caller's next
 * synchronisation.  A handle is not thread-safe; calls that use one storage
 * from several streams must be ordered by the caller.
 *
 * Errors.  Every argument is checked before anything is enqueued: a call
 * that returns RIPE_EINVAL or RIPE_ECAPACITY has enqueued nothing and changed
 * no state.  RIPE_EDEVICE means a launch failed part-way; the storage and the
 * lengths are then undefined.
 */
#ifndef RIPE_H
#define RIPE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ripe_cache ripe_cache; /* opaque host handle */

typedef enum {
    RIPE_OK = 0,
    RIPE_EINVAL = 1,    /* bad configuration, pointer, stride, row or size */
    RIPE_ECAPACITY = 2, /* an append would pass the capacity; nothing written */
    RIPE_EDEVICE = 3,   /* a HIP call or kernel launch failed */
    RIPE_ESCRATCH = 4   /* ripe_verify_attn_noalloc: the call needs more than
                           the library's fixed scratch (nothing enqueued) */
} ripe_status;

typedef enum { RIPE_ANCHOR_QUERY = 0, RIPE_ANCHOR_CACHE = 1 } ripe_anchor;

#define RIPE_WINDOW_FULL INT32_MAX /* keep every position at full depth */

typedef struct {
    int32_t n_layers;   /* recurrent layers sharing one storage, >= 1 */
    int32_t n_loops;    /* R, 1..255 */
    int32_t n_heads_q;  /* Hq, a multiple of n_heads_kv */
    int32_t n_heads_kv; /* Hkv >= 1 */
    int32_t head_dim;   /* d: 64, 96 or 128 */
    int32_t window;     /* W >= 0, or RIPE_WINDOW_FULL */
    int32_t batch;      /* B sequences, 1..4096 */
    int32_t capacity;   /* committed positions a sequence may hold, >= 1, with
                           capacity/4 + (R-1)*min(W, capacity)/4 < 2^31 - 2R */
    int32_t max_block;  /* largest draft block (n_blk) a verify call may use, 1..256 */
    int32_t anchor;     /* ripe_anchor */
} ripe_config;

/*
 * A strided bf16 array of key or value vectors.  Element e of the vector at
 * (sequence b, plane p, KV head g, token t) is at
 *     ptr + b*s_b + p*s_plane + g*s_head + t*s_tok + e      (in elements)
 * The d elements of one vector are contiguous.  ptr must be 16-byte aligned
 * and every stride a multiple of 8 elements.  Strides are >= 0.
 */
typedef struct {
    const void* ptr;
    int64_t s_b, s_plane, s_head, s_tok;
} ripe_kv_view;

/*
 * Storage layout (bit-exact; the storage is one caller-owned device buffer).
 * Sections start at multiples of 256 bytes, in this order:
 *   lens   int32 [n_layers][B]                     committed length L
 *   deep_k bf16  [n_layers][B][Hkv][CP * d]         CP = roundup(capacity, 32)
 *   deep_v bf16  [n_layers][B][Hkv][CP * d]
 *   ring_k bf16  [n_layers][B][Hkv][R-1][WP * d]    WR = min(W, capacity)
 *   ring_v bf16  [n_layers][B][Hkv][R-1][WP * d]    (0 when R = 1), WP = roundup(WR, 32)
 * deep_* holds loop R of position p at row p; ring_* holds loop r < R of
 * position p at row (p mod WR) of plane r-1 -- a ring buffer over the W most
 * recent positions, so a position that leaves the window keeps only its
 * deepest plane.  Rows group into tiles of 32 rows x d elements:
 *   key   (row p, dim e): (p/32)*32*d + (e/32)*1024 + (p%32)*32 + e%32
 *   value (row p, dim e): (p/32)*32*d + e*32 + slot(p%32),
 *                         slot(k) = 8*((k%16)/4) + 4*(k/16) + k%4
 * i.e. keys as 32x32 blocks and values transposed, both in the operand order
 * of the gfx950 16x16x32 bf16 matrix instruction.  Unwritten bytes are 0.
 */
typedef enum {
    RIPE_SECTION_LENS = 0,
    RIPE_SECTION_DEEP_K = 1,
    RIPE_SECTION_DEEP_V = 2,
    RIPE_SECTION_RING_K = 3,
    RIPE_SECTION_RING_V = 4,
    RIPE_SECTION_END = 5
} ripe_section;

/* Bytes of storage a configuration needs; 0 if the configuration is invalid. */
size_t ripe_cache_bytes(const ripe_config* cfg);

/* Byte offset of a section inside the storage; -1 if invalid. */
int64_t ripe_section_offset(const ripe_config* cfg, int32_t section);

/*
 * Batch capacity at fixed memory: the largest batch B in [1, 4096] whose
 * storage, ripe_cache_bytes of cfg with its batch field set to B, fits in
 * budget_bytes; 0 if not even one sequence fits; -1 if cfg is invalid (its
 * batch field is ignored).  RIPE's memory saving (abstract, fourth and fifth
 * sentences) read as sequences per budget: with capacity C and the window
 * rounded up to a multiple of 32, a recurrent layer stores C + W(R - 1)
 * vectors per sequence instead of R*C, or C with the deepest plane alone
 * (W = 0).  Host arithmetic only.
 */
int32_t ripe_max_batch(const ripe_config* cfg, size_t budget_bytes);

/*
 * Bind a handle to caller-owned storage of at least ripe_cache_bytes(cfg)
 * bytes (device memory, 256-byte aligned) and zero-fill it on `stream`.
 * All lengths start at 0.  The storage must outlive the handle.  The handle
 * is the host state of one RIPE cache (RIPE abstract, fourth sentence: what
 * the cache stores); no page defines the call itself.
 */
ripe_status ripe_cache_create(const ripe_config* cfg, void* d_storage, size_t bytes,
                              hipStream_t stream, ripe_cache** out);

/*
 * Bind a handle to storage that already holds a cache image of the same
 * configuration (for example a checkpoint of another handle's storage copied
 * back into device memory): nothing is written, and the committed lengths are
 * read from the image's lengths section on `stream` (the call waits for that
 * copy).  Appends and verifies then continue from the image exactly as they
 * would have on the handle that wrote it.  RIPE_EINVAL, with *out NULL, for
 * an invalid configuration or storage, or for a stored length outside
 * [0, capacity]; RIPE_EDEVICE if the copy fails.  No page defines the call
 * (checkpoint and resume of the cache are this library's).
 */
ripe_status ripe_cache_open(const ripe_config* cfg, void* d_storage, size_t bytes,
                            hipStream_t stream, ripe_cache** out);

/*
 * Release the handle (host memory only; the storage stays the caller's).
 * NULL is accepted, and so is a handle that was already destroyed: the
 * library keeps a registry of live handles and ignores any other pointer (a
 * later ripe_cache_create may reuse the address of a destroyed handle, so a
 * destroyed handle must still not be passed to the other calls).  No page
 * defines the call.
 */
void ripe_destroy(ripe_cache* cache);

/*
 * Fixed launch choices for one handle, for tuning sweeps and for tests that
 * run every kernel variant on the same inputs; a zero field leaves that
 * choice to the planner, and a NULL tuning restores the planner for all of
 * them.  Results never depend on these choices beyond float rounding order.
 * No page defines the call; the library reads no environment variable.
 * RIPE_EINVAL for a dead handle or an out-of-range field (nothing changed).
 */
typedef struct {
    int32_t kernel;        /* 1: keys kernel (waves split the key tiles),
                              2: rows kernel (waves own row-heads) */
    int32_t keys_waves;    /* 4 or 8 waves in a keys workgroup */
    int32_t row_tiles;     /* 1 or 2 tiles of 16 row-heads per wave (clamped
                              to what the head size allows) */
    int32_t private_waves; /* rows kernel: 1 without, 2 with the private waves
                              for ring and block tiles (head sizes 64, 96) */
    int32_t items_target;  /* workgroups the split of committed positions aims
                              for (1: never split) */
    int32_t min_chunk;     /* shortest chunk of committed positions (rounded up
                              to 32) */
} ripe_tuning;

ripe_status ripe_set_tuning(ripe_cache* cache, const ripe_tuning* tuning);

/* Host copy of the committed lengths of one layer (B values); no page defines
 * the call. */
ripe_status ripe_get_lengths(const ripe_cache* cache, int32_t layer, int32_t* h_lens);

/*
 * Append h_n_new[b] >= 0 tokens to sequence b of one layer (RIPE abstract,
 * fourth sentence: the deepest plane everywhere, full depth in the window).
 *   deep_k/deep_v: loop R of the new tokens, token t in [0, n_new) of
 *                  sequence b at (b, 0, g, t) of the view (s_plane unused);
 *   win_k/win_v:   loops 1..R-1 of the LAST min(n_new, WR) new tokens,
 *                  oldest first: loop r of window token u at (b, r-1, g, u).
 *                  May be null views when R = 1 or WR = 0.
 * Each new position writes its ring slot (p mod WR), so positions that leave
 * the window are collapsed to their deepest plane without a copy.
 * RIPE_ECAPACITY if any L + n_new > capacity (nothing written).
 * The lengths in storage and the host copy advance in stream order.
 */
ripe_status ripe_append(ripe_cache* cache, int32_t layer, const int32_t* h_n_new,
                        ripe_kv_view deep_k, ripe_kv_view deep_v, ripe_kv_view win_k,
                        ripe_kv_view win_v, hipStream_t stream);

/*
 * Workspace (device bytes) that any ripe_verify_attn call with n_rows rows
 * needs at the handle's current lengths, on any layer and for any set of rows
 * of that size (partial softmax states of split key ranges, for every launch
 * of the call: calls of more than 256 rows run several); may be 0.  0 also
 * for a dead handle or n_rows outside 1..65535.  Takes the handle rather than
 * the configuration because the split depends on the current lengths; after
 * an append the size must be queried again.  No page defines the call (the
 * split of the key range is this library's).
 */
size_t ripe_workspace_bytes(const ripe_cache* cache, int32_t n_rows);

/*
 * Verification attention of one layer.
 *   rows k = 0..n_rows-1: block offset h_row_blk[k] in [0, n_blk) and loop
 *        h_row_loop[k] in [1, R] (host arrays; any order, repeats allowed);
 *   d_q:   bf16 [B][n_rows][Hq][d], contiguous, 16-byte aligned;
 *   blk_k/blk_v: the draft block's own keys/values, loop r of block token j
 *        of sequence b at (b, r-1, g, j) of the view; n_blk in [1, max_block];
 *   d_out: fp32 [B][n_rows][Hq][d]; d_lse: fp32 [B][n_rows][Hq];
 *   d_ws:  at least ripe_workspace_bytes(cache, n_rows) bytes (256-aligned),
 *          or NULL when that is 0.
 * Committed positions come from the storage at the handle's current lengths.
 * Follows the RIPE abstract, first sentence (the draft block verified at
 * every loop over the shared prefix) and fifth sentence (block keys against
 * the window), and the WaveFront page's mixed-depth batched verification
 * (rows at different loops in one call).  RIPE_EINVAL (nothing enqueued) for
 * a dead handle, a layer, row, loop or n_blk out of range, a null or
 * misaligned pointer, a bad view, or a workspace below the size above.
 */
ripe_status ripe_verify_attn(ripe_cache* cache, int32_t layer, int32_t n_rows,
                             const int32_t* h_row_blk, const int32_t* h_row_loop,
                             const void* d_q, ripe_kv_view blk_k, ripe_kv_view blk_v,
                             int32_t n_blk, float* d_out, float* d_lse, void* d_ws,
                             size_t ws_bytes, hipStream_t stream);

/*
 * ripe_verify_attn without a caller workspace and without any allocation, for
 * callers that cannot allocate: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The partial softmax states of split
 * key ranges go to a fixed scratch array inside the library, one per device,
 * of RIPE_NOALLOC_SCRATCH_BYTES; the device holds it until the process ends.
 * A call whose launches need more than that returns RIPE_ESCRATCH with
 * nothing enqueued (ripe_workspace_bytes bounds the need).  Arguments,
 * results and every other error are those of ripe_verify_attn.  Every call on
 * one device shares that device's scratch: calls that overlap on one device
 * (different streams, or different threads without ordering) race and give
 * wrong results; calls ordered on one stream are safe.  Nothing in the
 * scratch needs clearing between calls (every partial state a launch reads
 * was written by the same launch sequence).  The first call on a device looks
 * up that device's scratch address (hipGetSymbolAddress) and keeps it.
 */
#define RIPE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
ripe_status ripe_verify_attn_noalloc(ripe_cache* cache, int32_t layer, int32_t n_rows,
                                     const int32_t* h_row_blk, const int32_t* h_row_loop,
                                     const void* d_q, ripe_kv_view blk_k, ripe_kv_view blk_v,
                                     int32_t n_blk, float* d_out, float* d_lse,
                                     hipStream_t stream);

/*
 * Windowed draft attention of one layer (page "Windowed-MTP: Removing the
 * Full-Context Draft-KV Tax at Million-Token Context", abstract: a sliding
 * window plus an attention sink on the draft's attention only, so a draft
 * reads a bounded set of keys however long the context).  Arguments as for
 * ripe_verify_attn, except that a row (i, r) of sequence b keeps only the
 * committed positions s < n_sink (the sinks) and s >= L_b + i - w_draft (the
 * window) among its keys; its draft-block keys 0..i all stay, and every key
 * is read at the plane the verification rule names (with w_draft <= W the
 * window's positions come from the ring at loop r, the sinks from the deepest
 * plane).  n_sink >= 0 and w_draft >= 0, else RIPE_EINVAL; w_draft >= L + i
 * is the full-context draft.  Needs no workspace; one workgroup reads a KV
 * head's sinks and window, so it is meant for windows of up to a few
 * thousand positions.
 */
ripe_status ripe_draft_attn(ripe_cache* cache, int32_t layer, int32_t n_rows,
                            const int32_t* h_row_blk, const int32_t* h_row_loop,
                            const void* d_q, ripe_kv_view blk_k, ripe_kv_view blk_v,
                            int32_t n_blk, int32_t n_sink, int32_t w_draft, float* d_out,
                            float* d_lse, hipStream_t stream);

/* Static description of a status code. */
const char* ripe_status_string(ripe_status s);

#ifdef __cplusplus
}
#endif

#endif /* RIPE_H */
