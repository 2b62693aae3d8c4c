// Vector-ALU verification attention: one wavefront per (sequence, query row,
// query head).  For rows that share no key tile with other rows (a
// mixed-depth wave, where each position sits at its own loop), the work is a
// matrix-vector product and belongs on the VALU rather than the matrix cores.
//
// A row (block offset i, loop r) of sequence b with L committed positions
// attends to (page "Prefix Keys and Values Matter Late", abstract, first and
// fourth sentences; the window anchor is the reading beta = t - W or L - W):
//   deep tiles : committed positions s < e_row at loop R, where
//                e_row = L for r = R, else clamp(beta, 0, L);
//   ring tiles : committed positions s >= e_row at loop r (ring slot s mod WR);
//   block keys : positions L..L+i at loop r, from the caller's block buffer.
// Keys are processed 32 per tile with an online softmax in the log2 domain.
//
// Lane layout per tile: lane = 2*key + half; a lane dots 16 dims of each
// 32-dim key column block with the query, a neighbour exchange completes the
// score.  For P.V a lane owns value rows e = lane/4 + 16u and the 8 tile
// columns 8*(lane%4)..+7; the four lanes of a quad are summed at the end.
#include "ripe_internal.h"

namespace ripe {
namespace {

__device__ inline float bf(uint32_t w, int hi) {
    return __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16));
}

__device__ inline float wave_max(float x) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o);
    return x;
}

template <int D>
struct RowState {
    float m, l;
    float acc[D / 16];
};

// One 32-key tile.  Tiled sources (cache) read K at K + j*1024 + key*32 and V
// at V + e*32 + column; the natural source (draft block) reads key rows at
// krow + key*kst and value rows at vrow + key*vst.
template <int D, bool NATURAL>
__device__ inline void tile_step(const float (&qv)[D / 32][16], const uint16_t* K,
                                 const uint16_t* V, int64_t kst, int64_t vst, bool valid,
                                 float sl2, RowState<D>& st, int lane) {
    const int key = lane >> 1, hf = lane & 1;
    float s = 0.f;
    if (!NATURAL || valid) {
#pragma unroll
        for (int j = 0; j < D / 32; ++j) {
            const uint16_t* kp = NATURAL ? K + key * kst + 32 * j + 16 * hf
                                         : K + j * 1024 + key * 32 + 16 * hf;
            const uint4 x0 = *reinterpret_cast<const uint4*>(kp);
            const uint4 x1 = *reinterpret_cast<const uint4*>(kp + 8);
            const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int c = 0; c < 16; ++c) s = fmaf(qv[j][c], bf(w[c >> 1], c & 1), s);
        }
    }
    s += __shfl_xor(s, 1);
    const float x = valid ? s * sl2 : -INFINITY;
    const float mn = fmaxf(st.m, wave_max(x));
    float alpha = 1.f, p = 0.f;
    if (mn != -INFINITY) {
        alpha = exp2f(st.m - mn);
        p = valid ? exp2f(x - mn) : 0.f;
    }
    st.l = st.l * alpha + wave_sum(hf ? 0.f : p);
    st.m = mn;
    const int sg = lane & 3;
    float pk[8];
    bool vk[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int k = 16 * (c >> 2) + 4 * sg + (c & 3);
        pk[c] = __shfl(p, 2 * k);
        vk[c] = __shfl((int)valid, 2 * k) != 0;
    }
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
        const int e = (lane >> 2) + 16 * u;
        float a = st.acc[u] * alpha;
        if (NATURAL) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int k = 16 * (c >> 2) + 4 * sg + (c & 3);
                if (vk[c]) a = fmaf(pk[c], bf(V[k * vst + e], 0), a);
            }
        } else {
            const uint4 x = *reinterpret_cast<const uint4*>(V + e * 32 + 8 * sg);
            const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int c = 0; c < 8; ++c) a = fmaf(pk[c], bf(w[c >> 1], c & 1), a);
        }
        st.acc[u] = a;
    }
}

template <int D>
__global__ void __launch_bounds__(256) k_verify_valu(VerifyArgs a) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + wave;
    const int64_t n_units = (int64_t)a.B * a.rows_here * a.Hq;
    if (unit >= n_units) return;
    const int h = (int)(unit % a.Hq);
    const int k = (int)((unit / a.Hq) % a.rows_here);
    const int b = (int)(unit / ((int64_t)a.Hq * a.rows_here));
    const uint32_t rw = a.rows[k];
    const int i = rw & 255, r = (rw >> 8) & 255, orig = (int)(rw >> 16);
    const int g = h / a.group;
    const int64_t L = a.lens[b];
    const int64_t t = L + i;
    const int64_t beta = a.anchor == 0 ? t - a.W : L - a.W;
    const int64_t e_row = (r == a.R) ? L : (beta < 0 ? 0 : (beta > L ? L : beta));

    const int key = lane >> 1, hf = lane & 1;
    float qv[D / 32][16];
    const uint16_t* qp = a.q + (((int64_t)b * a.n_rows + orig) * a.Hq + h) * D;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
        const uint4 x0 = *reinterpret_cast<const uint4*>(qp + 32 * j + 16 * hf);
        const uint4 x1 = *reinterpret_cast<const uint4*>(qp + 32 * j + 16 * hf + 8);
        const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int c = 0; c < 16; ++c) qv[j][c] = bf(w[c >> 1], c & 1);
    }
    RowState<D> st;
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int u = 0; u < D / 16; ++u) st.acc[u] = 0.f;

    const int64_t dreg = ((int64_t)b * a.Hkv + g) * a.CP * D;
    for (int64_t t0 = 0; t0 < e_row; t0 += kTile)
        tile_step<D, false>(qv, a.deep_k + dreg + t0 * D, a.deep_v + dreg + t0 * D, 0, 0,
                            t0 + key < e_row, a.scale_log2, st, lane);

    if (r < a.R && e_row < L) {
        const int64_t rreg = (((int64_t)b * a.Hkv + g) * a.NR + (r - 1)) * a.WP * D;
        for (int64_t s0 = 0; s0 < a.WR; s0 += kTile) {
            const int64_t sl = s0 + key;
            bool ok = sl < a.WR && sl < L;
            if (ok) {
                const int64_t pos = sl + a.WR * ((L - 1 - sl) / a.WR);   // newest position in slot
                ok = pos >= e_row;
            }
            tile_step<D, false>(qv, a.ring_k + rreg + s0 * D, a.ring_v + rreg + s0 * D, 0, 0, ok,
                                a.scale_log2, st, lane);
        }
    }

    const uint16_t* bk = a.bk.p + b * a.bk.sb + (int64_t)(r - 1) * a.bk.sp + g * a.bk.sh;
    const uint16_t* bv = a.bv.p + b * a.bv.sb + (int64_t)(r - 1) * a.bv.sp + g * a.bv.sh;
    for (int j0 = 0; j0 <= i; j0 += kTile)
        tile_step<D, true>(qv, bk + j0 * a.bk.st, bv + j0 * a.bv.st, a.bk.st, a.bv.st,
                           j0 + key <= i, a.scale_log2, st, lane);

    // sum the four column groups of each value row, normalise, store
    const float inv = 1.f / st.l;
    float* op = a.out + (((int64_t)b * a.n_rows + orig) * a.Hq + h) * D;
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
        float v = st.acc[u];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        if ((lane & 3) == 0) op[(lane >> 2) + 16 * u] = v * inv;
    }
    if (lane == 0)
        a.lse[((int64_t)b * a.n_rows + orig) * a.Hq + h] = (st.m + log2f(st.l)) * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_verify_valu(const VerifyArgs& a, hipStream_t s) {
    const int64_t units = (int64_t)a.B * a.rows_here * a.Hq;
    const unsigned blocks = (unsigned)((units + 3) / 4);
    if (blocks == 0) return hipSuccess;
    switch (a.d) {
        case 64: hipLaunchKernelGGL(k_verify_valu<64>, dim3(blocks), dim3(256), 0, s, a); break;
        case 96: hipLaunchKernelGGL(k_verify_valu<96>, dim3(blocks), dim3(256), 0, s, a); break;
        case 128: hipLaunchKernelGGL(k_verify_valu<128>, dim3(blocks), dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ripe
