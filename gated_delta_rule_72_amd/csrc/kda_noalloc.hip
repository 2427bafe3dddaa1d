// kda_noalloc.hip -- kda_prefill_noalloc: kda_prefill with its workspace in a
// device array of the library instead of a caller buffer, for callers that
// cannot allocate device memory (code under stream capture, serving loops,
// harnesses that forbid hipMalloc).
//
// The array below is a file-scope device global: the module that holds it
// (this file's code object) reserves it on every device it is loaded on, once,
// until the process ends.  Host code never uses the array's name as an
// address (in host code it names a host-side stand-in): the device address
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is handed to kda_prefill.  Nothing here
// allocates: no hipMalloc, no hipFree, no allocating library call.
#include <mutex>

#include "kda.h"
#include "kda_internal.h"

static __device__ __align__(256) unsigned char scratch[KDA_PREFILL_NOALLOC_MAX_WORKSPACE];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` on each device, once known

// The device address of `scratch` on device dev (looked up on first use, with dev current).
hipError_t scratch_on(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" kda_status kda_prefill_noalloc(const void* q, const void* k, const void* v, const float* alpha,
                                          const float* beta, const float* S0, const int32_t* cu_seqlens,
                                          int32_t n_seq, int32_t n_tok, int32_t n_heads, int32_t d_k,
                                          int32_t d_v, kda_dtype dt, void* o, float* S_T, void* stream) {
    // the size check is host arithmetic only: an oversized call is refused before any HIP call
    const size_t need = kda_prefill_workspace_size(n_seq, n_tok, n_heads, d_k, d_v, dt);
    if (need > KDA_PREFILL_NOALLOC_MAX_WORKSPACE) return KDA_ERR_WORKSPACE;
    int dev = 0;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess) return KDA_ERR_DEVICE;
    void* ws = nullptr;
    if (scratch_on(dev, &ws) != hipSuccess) return KDA_ERR_DEVICE;
    return kda_prefill(q, k, v, alpha, beta, S0, cu_seqlens, n_seq, n_tok, n_heads, d_k, d_v, dt, o, S_T, ws,
                       KDA_PREFILL_NOALLOC_MAX_WORKSPACE, stream);
}
