// ripe_verify_attn_noalloc: verification attention whose partial softmax
// states go to a fixed scratch array inside the library instead of a caller
// workspace, so the call allocates nothing (see include/ripe.h).
//
// The array is a file-scope device variable; each device that loads the
// library holds its own copy at its own address.  In host code `scratch`
// names only a host-side stand-in, so its device address is looked up once
// per device (hipGetSymbolAddress, with that device current) and that
// address is what the kernels receive.
#include <mutex>

#include <hip/hip_runtime.h>

#include "ripe.h"
#include "ripe_internal.h"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[RIPE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch`, per device

// Address of the scratch array on `device`, looked up on the first call for
// that device.
ripe_status scratch_on(int device, void** out) {
    if (device < 0 || device >= kMaxDevices) return RIPE_EDEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        int current = -1;
        if (hipGetDevice(&current) != hipSuccess) return RIPE_EDEVICE;
        if (current != device && hipSetDevice(device) != hipSuccess) return RIPE_EDEVICE;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (current != device && hipSetDevice(current) != hipSuccess) return RIPE_EDEVICE;
        if (e != hipSuccess || !p) return RIPE_EDEVICE;
        g_scratch_ptr[device] = p;
    }
    *out = g_scratch_ptr[device];
    return RIPE_OK;
}

}  // namespace

extern "C" ripe_status ripe_verify_attn_noalloc(ripe_cache* cache, int32_t layer, int32_t n_rows,
                                                const int32_t* h_row_blk, const int32_t* h_row_loop,
                                                const void* d_q, ripe_kv_view blk_k,
                                                ripe_kv_view blk_v, int32_t n_blk, float* d_out,
                                                float* d_lse, hipStream_t stream) {
    int device = -1;
    const ripe_status st = ripe::cache_device(cache, &device);
    if (st != RIPE_OK) return st;
    void* ws = nullptr;
    const ripe_status s2 = scratch_on(device, &ws);
    if (s2 != RIPE_OK) return s2;
    return ripe::attend(cache, layer, n_rows, h_row_blk, h_row_loop, d_q, blk_k, blk_v, n_blk, 0,
                        -1, d_out, d_lse, ws, RIPE_NOALLOC_SCRATCH_BYTES, true, stream);
}
