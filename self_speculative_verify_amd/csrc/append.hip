// Append kernels: write new tokens into the RIPE storage.
//
// RIPE keeps the deepest plane of every position and loops 1..R-1 only for a
// window of recent positions (page "Prefix Keys and Values Matter Late",
// abstract, fourth sentence).  Loop R of each new position goes to its deep
// row; loops 1..R-1 of the last min(n_new, WR) new positions go to ring row
// p mod WR, overwriting the shallow planes of the position that just left the
// window (the collapse: that position keeps only its deep row).
//
// One thread moves 8 consecutive elements (16 bytes) of one vector.  Key tiles
// keep 32 consecutive dimensions of a row together, so the store is one 16-byte
// write; value tiles are transposed, so it is 8 two-byte writes.
#include "ripe_internal.h"

namespace ripe {
namespace {

__device__ inline int find_seq(const int64_t* prefix, int nb, int64_t idx) {
    int lo = 0, hi = nb;   // prefix[lo] <= idx < prefix[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (prefix[mid] <= idx) lo = mid; else hi = mid;
    }
    return lo;
}

__device__ inline void store_vec(uint16_t* kreg, uint16_t* vreg, int64_t row, int e0, int d,
                                 const uint16_t* ks, const uint16_t* vs) {
    const uint4 kx = *reinterpret_cast<const uint4*>(ks);
    const uint4 vx = *reinterpret_cast<const uint4*>(vs);
    *reinterpret_cast<uint4*>(kreg + key_off(row, e0, d)) = kx;
    const uint32_t w[4] = {vx.x, vx.y, vx.z, vx.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint16_t h = (uint16_t)(w[c >> 1] >> ((c & 1) * 16));
        vreg[val_off(row, e0 + c, d)] = h;
    }
}

// items: (sequence, token t < n_new, kv head g, 8-element chunk)
__global__ void __launch_bounds__(256) k_append_deep(AppendArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blockIdx.x == 0 && threadIdx.x < (unsigned)a.nb)
        a.lens[a.b0 + threadIdx.x] = a.L0[threadIdx.x] + a.n_new[threadIdx.x];
    if (idx >= a.total) return;
    const int sb = find_seq(a.prefix, a.nb, idx);
    int64_t r = idx - a.prefix[sb];
    const int chunks = a.d >> 3;
    const int c = (int)(r % chunks); r /= chunks;
    const int g = (int)(r % a.Hkv); r /= a.Hkv;
    const int64_t t = r;
    const int b = a.b0 + sb;
    const int64_t pos = a.L0[sb] + t;
    const int64_t region = ((int64_t)b * a.Hkv + g) * a.CP * a.d;
    const uint16_t* ks = a.dk.p + b * a.dk.sb + g * a.dk.sh + t * a.dk.st + c * 8;
    const uint16_t* vs = a.dv.p + b * a.dv.sb + g * a.dv.sh + t * a.dv.st + c * 8;
    store_vec(a.deep_k + region, a.deep_v + region, pos, c * 8, a.d, ks, vs);
}

// items: (sequence, window token u < n_win, plane r-1, kv head g, chunk)
__global__ void __launch_bounds__(256) k_append_ring(AppendArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= a.total) return;
    const int sb = find_seq(a.prefix, a.nb, idx);
    int64_t r = idx - a.prefix[sb];
    const int chunks = a.d >> 3;
    const int c = (int)(r % chunks); r /= chunks;
    const int g = (int)(r % a.Hkv); r /= a.Hkv;
    const int pl = (int)(r % a.NR); r /= a.NR;
    const int64_t u = r;
    const int b = a.b0 + sb;
    const int64_t pos = a.L0[sb] + a.n_new[sb] - a.n_win[sb] + u;
    const int64_t slot = pos % a.WR;
    const int64_t region = (((int64_t)b * a.Hkv + g) * a.NR + pl) * a.WP * a.d;
    const uint16_t* ks = a.wk.p + b * a.wk.sb + pl * a.wk.sp + g * a.wk.sh + u * a.wk.st + c * 8;
    const uint16_t* vs = a.wv.p + b * a.wv.sb + pl * a.wv.sp + g * a.wv.sh + u * a.wv.st + c * 8;
    store_vec(a.ring_k + region, a.ring_v + region, slot, c * 8, a.d, ks, vs);
}

}  // namespace

hipError_t launch_append_deep(const AppendArgs& a, hipStream_t s) {
    const int64_t blocks = (a.total + 255) / 256;
    hipLaunchKernelGGL(k_append_deep, dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_append_ring(const AppendArgs& a, hipStream_t s) {
    const int64_t blocks = (a.total + 255) / 256;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_append_ring, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace ripe
