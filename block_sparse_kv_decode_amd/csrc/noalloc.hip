// noalloc.hip -- nosa_decode_step for callers that cannot allocate (HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc): the step's workspace is a fixed device array of this
// library instead of a caller buffer.
//
// The array lives in the library's code object: every GPU the library runs on holds its own copy,
// zero at load, until the process ends.  Host code never names the array in a kernel argument or
// copy (its host-side symbol is only a handle): at a call's first use on a device, with that device
// current, hipGetSymbolAddress yields the device copy's address, kept per device, and only that
// address is handed to the kernels.
#include <hip/hip_runtime.h>
#include <mutex>

#include "nosa.h"
#include "nosa_internal.h"

namespace {

constexpr size_t kScratchBytes = NOSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (resolved once per device).
int scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return nosa::api_fail(NOSA_EHIP, "hipGetDevice: HIP error %d (%s)", (int)e, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return nosa::api_fail(NOSA_EUNSUPPORTED, "device index %d too large", dev);
    std::lock_guard<std::mutex> g(g_lock);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return nosa::api_fail(NOSA_EHIP, "hipGetSymbolAddress(scratch): HIP error %d (%s)", (int)e,
                                  hipGetErrorString(e));
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return NOSA_OK;
}

}  // namespace

extern "C" int nosa_decode_step_noalloc(const nosa_shape *shape, const void *q, const float *pooled_k,
                                        const float *evict, int32_t n_blocks_prev, int32_t *agn_state,
                                        int32_t *selected, const void *k_store, const void *v_store,
                                        int32_t store_blocks, float softmax_scale, void *out, hipStream_t stream) {
    const size_t need = nosa_workspace_bytes(shape);
    if (need == 0)   // an invalid shape: the step reports why, before any HIP call
        return nosa_decode_step(shape, q, pooled_k, evict, n_blocks_prev, agn_state, selected, k_store, v_store,
                                store_blocks, softmax_scale, out, nullptr, stream);
    if (need > kScratchBytes)
        return nosa::api_fail(NOSA_ECAPACITY, "the step needs %zu bytes of workspace; the fixed scratch holds %zu",
                              need, kScratchBytes);
    void *ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc != NOSA_OK) return rc;
    return nosa_decode_step(shape, q, pooled_k, evict, n_blocks_prev, agn_state, selected, k_store, v_store,
                            store_blocks, softmax_scale, out, ws, stream);
}
