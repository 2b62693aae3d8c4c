// Internal declarations shared by the host side of the library and its HIP
// kernels (not part of the public ABI): kernel arguments and launchers.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "plan.h"

namespace ripe {

struct View {            // strided bf16 view, element strides
    const uint16_t* p;
    int64_t sb, sp, sh, st;
};

// ---------------------------------------------------------------- append

struct AppendArgs {
    uint16_t* deep_k;    // layer base of the deep sections: [B][Hkv][CP*d]
    uint16_t* deep_v;
    uint16_t* ring_k;    // layer base of the ring sections: [B][Hkv][NR][WP*d]
    uint16_t* ring_v;
    int32_t* lens;       // layer row of the lens section: [B]
    View dk, dv, wk, wv;
    int32_t Hkv, d, NR;
    int64_t CP, WR, WP;
    int32_t nb;          // sequences in this launch
    int32_t b0;          // first sequence
    // most 4-position groups that any sequence's new positions (gd) and new
    // window positions (gr, 0 when R = 1 or WR = 0) touch
    int64_t gd;
    int32_t gr;
    int32_t n_new[kMaxBatchPerLaunch];
    int32_t L0[kMaxBatchPerLaunch];
    int32_t n_win[kMaxBatchPerLaunch];
};

// groups of 4 positions (aligned to multiples of 4) that the positions
// [first, first + count) touch
inline int64_t append_groups(int64_t first, int64_t count) {
    return count > 0 ? (first + count - 1) / 4 - first / 4 + 1 : 0;
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s);

// ---------------------------------------------------------------- verify

struct VerifyArgs {
    const uint16_t* deep_k;  // layer base: [B][Hkv][CP*d]
    const uint16_t* deep_v;
    const uint16_t* ring_k;  // layer base: [B][Hkv][NR][WP*d]
    const uint16_t* ring_v;
    const int32_t* lens;     // layer row of the lens section
    const uint16_t* q;       // [B][n_rows][Hq][d]
    View bk, bv;             // draft block planes
    float* out;              // [B][n_rows][Hq][d]
    float* lse;              // [B][n_rows][Hq]
    float* part;             // partial softmax states (split key ranges)
    int32_t B, n_rows, Hq, Hkv, group, R, d, n_blk, anchor;
    int64_t W, CP, WR, WP, NR;
    float scale_log2;        // log2(e) / sqrt(d)
    int32_t rows_here;       // rows in this launch
    // matrix-core plan: row-heads of one KV head split into blocks of 16*RT,
    // committed positions split into nc chunks of cl (a multiple of 32)
    int32_t M;               // row-heads per KV head in this launch (rows_here * group)
    int32_t nrb;             // row blocks per KV head
    int32_t nc;              // chunks of the longest sequence
    int64_t cl;              // positions per chunk
    int64_t cx;              // positions' worth of ring and block tiles that the
                             // last chunk of a sequence carries besides its own
    // windowed draft attention: a row (i, r) keeps the committed keys
    // s < n_sink or s >= L + i - w_draft; w_draft < 0: every committed key
    int32_t n_sink, w_draft;
    int32_t n_groups;        // B * Hkv * nc, or n_pairs * Hkv
    // rows of this launch sorted by (loop, block offset):
    // bits 0..7 block offset, 8..15 loop, 16..31 row index in the call
    uint32_t rows[kMaxRowsPerLaunch];
    // chunks of each sequence when the batch has at most kMaxSeqArgs
    // sequences (0: read the length from storage); the host's copy of the
    // lengths advances in stream order with the one in storage
    int32_t snc[kMaxSeqArgs];
    // when n_pairs > 0: the (sequence, chunk) items of a split launch, longest
    // first (bits 0..5 sequence, 6..15 chunk), so the longest start first
    int32_t n_pairs;
    uint16_t pairs[kMaxPairs];
    // for the combine launch: the sequences split into two or more chunks
    // when the batch has at most kMaxSeqArgs sequences (n_split = 0: every
    // sequence is enumerated and the unsplit ones skipped)
    int32_t n_split;
    uint8_t split_b[kMaxSeqArgs];
};

// matrix-core kernels: "keys" (waves split the key tiles of 16*rt row-heads)
// and "rows" (each wave owns 16*rt row-heads; the workgroup 64*rt)
// wide: eight waves instead of four (one workgroup per compute unit; not for
// the windowed draft)
hipError_t launch_verify_keys(const VerifyArgs& a, int rt, bool wide, hipStream_t s);
// priv: four more waves take the ring and draft-block tiles (where rows_private_waves)
hipError_t launch_verify_rows(const VerifyArgs& a, int rt, bool priv, hipStream_t s);
hipError_t launch_combine(const VerifyArgs& a, hipStream_t s);

}  // namespace ripe

// ---------------------------------------------------------------- host side

#include "ripe.h"

namespace ripe {

// Verification attention of one call after full validation (see ripe_api.cpp);
// ws_fixed: d_ws is the library's fixed scratch, refused with RIPE_ESCRATCH
// when a launch needs more than ws_bytes.
ripe_status attend(ripe_cache* cache, int32_t layer, int32_t n_rows, const int32_t* h_row_blk,
                   const int32_t* h_row_loop, const void* d_q, ripe_kv_view blk_k,
                   ripe_kv_view blk_v, int32_t n_blk, int32_t n_sink, int32_t w_draft,
                   float* d_out, float* d_lse, void* d_ws, size_t ws_bytes, bool ws_fixed,
                   hipStream_t stream);
// Device of a live handle's storage (looked up once).
ripe_status cache_device(ripe_cache* cache, int* device);

}  // namespace ripe
