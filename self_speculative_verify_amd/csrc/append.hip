// Append kernels: write new tokens into the RIPE storage.
//
// RIPE keeps the deepest plane of every position and loops 1..R-1 only for a
// window of recent positions (page "Prefix Keys and Values Matter Late",
// abstract, fourth sentence).  Loop R of each new position goes to its deep
// row; loops 1..R-1 of the last min(n_new, WR) new positions go to ring row
// p mod WR, overwriting the shallow planes of the position that just left the
// window (the collapse: that position keeps only its deep row).
//
// One launch writes both the deep rows and the ring rows.  A thread moves 8
// consecutive elements (16 bytes) of one head's vector for up to four
// positions.  Key tiles keep 32 consecutive dimensions of a row together, so
// each position's key is one 16-byte write.  Value tiles are transposed; four
// rows that start at a multiple of 4 are four consecutive value slots, so a
// whole group of four takes one 8-byte write per dimension, and a lone
// position 8 two-byte writes.
#include <algorithm>

#include "ripe_internal.h"
#include "tile_layout.h"

namespace ripe {
namespace {

// bf16 element c (0..7) of 8 packed in x
__device__ inline uint32_t elem(const uint4& x, int c) {
    const uint32_t w = (c >> 1) == 0 ? x.x : (c >> 1) == 1 ? x.y : (c >> 1) == 2 ? x.z : x.w;
    return (w >> ((c & 1) * 16)) & 0xffffu;
}

__device__ inline void store_vec(uint16_t* kreg, uint16_t* vreg, int64_t row, int e0, int d,
                                 const uint16_t* ks, const uint16_t* vs) {
    const uint4 kx = *reinterpret_cast<const uint4*>(ks);
    const uint4 vx = *reinterpret_cast<const uint4*>(vs);
    *reinterpret_cast<uint4*>(kreg + key_off(row, e0, d)) = kx;
#pragma unroll
    for (int c = 0; c < 8; ++c) vreg[val_off(row, e0 + c, d)] = (uint16_t)elem(vx, c);
}

// One thread moves one 8-element chunk (elements e0..e0+7) of one KV head's
// vectors for the new positions of the 4-position group that starts at v0 (a
// multiple of 4).  When all four positions are new and their rows are four
// aligned rows of one tile (always for deep rows; for ring rows when WR is a
// multiple of 4), the transposed value rows take one 8-byte store per
// dimension (the four rows are consecutive value slots); otherwise each new
// position is stored on its own.
//   base_k/base_v: the (sequence, head[, plane]) region;
//   sk/sv:         the source of position `first` (token strides stk/stv);
//   first, count:  the new positions [first, first + count);
//   wr:            ring slots (row = position mod wr), 0 for deep rows.
__device__ inline void store_group(uint16_t* base_k, uint16_t* base_v, const uint16_t* sk,
                                   const uint16_t* sv, int64_t stk, int64_t stv, int first,
                                   int count, int v0, int wr, int e0, int d) {
    const bool full = v0 >= first && (int64_t)v0 + 4 <= (int64_t)first + count && (wr & 3) == 0;
    if (full) {
        const int t0 = v0 - first;
        const int row0 = wr ? v0 % wr : v0;
        const uint4 k0 = *reinterpret_cast<const uint4*>(sk + t0 * stk);
        const uint4 k1 = *reinterpret_cast<const uint4*>(sk + (t0 + 1) * stk);
        const uint4 k2 = *reinterpret_cast<const uint4*>(sk + (t0 + 2) * stk);
        const uint4 k3 = *reinterpret_cast<const uint4*>(sk + (t0 + 3) * stk);
        const uint4 x0 = *reinterpret_cast<const uint4*>(sv + t0 * stv);
        const uint4 x1 = *reinterpret_cast<const uint4*>(sv + (t0 + 1) * stv);
        const uint4 x2 = *reinterpret_cast<const uint4*>(sv + (t0 + 2) * stv);
        const uint4 x3 = *reinterpret_cast<const uint4*>(sv + (t0 + 3) * stv);
        uint16_t* krow = base_k + key_off(row0, e0, d);       // rows row0..row0+3: 32 apart
        *reinterpret_cast<uint4*>(krow) = k0;
        *reinterpret_cast<uint4*>(krow + 32) = k1;
        *reinterpret_cast<uint4*>(krow + 64) = k2;
        *reinterpret_cast<uint4*>(krow + 96) = k3;
        uint16_t* vrow = base_v + val_off(row0, e0, d);       // dims e0..e0+7: 32 apart
#pragma unroll
        for (int c = 0; c < 8; ++c)
            *reinterpret_cast<uint2*>(vrow + c * 32) =
                make_uint2(elem(x0, c) | (elem(x1, c) << 16), elem(x2, c) | (elem(x3, c) << 16));
        return;
    }
    for (int j = 0; j < 4; ++j) {
        const int v = v0 + j;
        if (v < first || (int64_t)v >= (int64_t)first + count) continue;
        const int t = v - first;
        store_vec(base_k, base_v, wr ? v % wr : v, e0, d, sk + t * stk, sv + t * stv);
    }
}

// grid: x = (plane slot, 4-position group): the first gd indexes are the
// groups of the deep rows, then gr for each ring plane in loop order;
// y = block of KV heads; z = sequence.  block: x = 8-element chunk, y = head
// within the block.
__global__ void __launch_bounds__(256) k_append(AppendArgs a) {
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
        for (int i = threadIdx.y * blockDim.x + threadIdx.x; i < a.nb; i += blockDim.x * blockDim.y)
            a.lens[a.b0 + i] = a.L0[i] + a.n_new[i];
    const int sb = (int)blockIdx.z;
    const int g = (int)(blockIdx.y * blockDim.y + threadIdx.y);
    if (g >= a.Hkv) return;
    const int e0 = (int)threadIdx.x * 8;
    const int b = a.b0 + sb;
    const int n_new = a.n_new[sb];
    if ((int64_t)blockIdx.x < a.gd) {
        const int first = a.L0[sb];
        const int v0 = ((first >> 2) + (int)blockIdx.x) * 4;
        if ((int64_t)v0 >= (int64_t)first + n_new) return;
        const int64_t region = ((int64_t)b * a.Hkv + g) * a.CP * a.d;
        const uint16_t* ks = a.dk.p + b * a.dk.sb + g * a.dk.sh + e0;
        const uint16_t* vs = a.dv.p + b * a.dv.sb + g * a.dv.sh + e0;
        store_group(a.deep_k + region, a.deep_v + region, ks, vs, a.dk.st, a.dv.st, first, n_new,
                    v0, 0, e0, a.d);
        return;
    }
    const int x = (int)(blockIdx.x - a.gd);
    const int r = x / a.gr;                 // ring plane (loop r + 1)
    const int q = x - r * a.gr;
    const int n_win = a.n_win[sb];
    const int first = a.L0[sb] + n_new - n_win;
    const int v0 = ((first >> 2) + q) * 4;
    if ((int64_t)v0 >= (int64_t)first + n_win) return;
    const int64_t region = (((int64_t)b * a.Hkv + g) * a.NR + r) * a.WP * a.d;
    const uint16_t* ks = a.wk.p + b * a.wk.sb + r * a.wk.sp + g * a.wk.sh + e0;
    const uint16_t* vs = a.wv.p + b * a.wv.sb + r * a.wv.sp + g * a.wv.sh + e0;
    store_group(a.ring_k + region, a.ring_v + region, ks, vs, a.wk.st, a.wv.st, first, n_win,
                v0, (int)a.WR, e0, a.d);
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
    const int chunks = a.d / 8;
    const int hg = std::max(1, std::min(a.Hkv, 256 / chunks));
    const dim3 grid((unsigned)(a.gd + (int64_t)a.NR * a.gr), (unsigned)((a.Hkv + hg - 1) / hg),
                    (unsigned)a.nb);
    hipLaunchKernelGGL(k_append, grid, dim3((unsigned)chunks, (unsigned)hg), 0, s, a);
    return hipGetLastError();
}

}  // namespace ripe
