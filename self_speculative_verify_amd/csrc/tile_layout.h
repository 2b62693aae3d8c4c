// Tile order of the storage rows (keys as 32x32 blocks, values transposed),
// shared by the append and verification kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace ripe {

// Element offset of (row, dim) inside one tile region, keys and values.
__host__ __device__ inline int64_t key_off(int64_t row, int e, int d) {
    return (row >> 5) * (int64_t)(kTile * d) + (e >> 5) * 1024 + (row & 31) * 32 + (e & 31);
}
// Column of row k (0..31) of a 32-row value tile.  With this order, the two
// 16-row halves of a score tile computed by v_mfma_f32_16x16x32_bf16 (lane
// group q holding rows 4q..4q+3 of each half) feed the value operand of the
// same instruction as 8 consecutive columns 8q..8q+7.
__host__ __device__ inline int v_slot(int k) {
    return 8 * ((k & 15) >> 2) + 4 * (k >> 4) + (k & 3);
}
__host__ __device__ inline int64_t val_off(int64_t row, int e, int d) {
    return (row >> 5) * (int64_t)(kTile * d) + (int64_t)e * 32 + v_slot((int)(row & 31));
}

}  // namespace ripe
