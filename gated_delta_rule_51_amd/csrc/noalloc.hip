// kda_prefill_noalloc: kda_prefill for callers that cannot allocate device memory
// (code under stream capture, tight serving loops, harnesses that forbid hipMalloc).
// The prefill's workspace (the chunk-local operands T' and A_qk per chunk slot and head)
// lives in a file-scope device array instead of a caller-supplied buffer.
//
// Each GPU the library runs on holds its own copy of `scratch` for the life of the
// process.  Host code never uses the array's name as an address: the device address is
// looked up once per device with hipGetSymbolAddress (with that device current) and kept
// in a per-device table; the kernels receive that pointer as their workspace argument.
// Every call on one GPU shares that GPU's array, so calls that overlap on one GPU race
// (serialise them, e.g. on one stream).  Nothing in the array has to start at zero: the
// chunk-local kernel writes every slot the recurrence reads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/kda.h"
#include "kda_launch.hpp"

static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void *g_scratch[MAX_DEVICES] = {};

// Device address of `scratch` on the device that `stream` runs on.
hipError_t scratch_address(void *stream, void **out) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
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

extern "C" {

kda_status kda_prefill_noalloc(const void *q, const void *k, const void *v, const void *log_alpha,
                               const void *beta, const float *init_state, const int32_t *cu_seqlens,
                               int32_t nseq, int64_t total_tokens, int32_t H, int32_t dk, int32_t dv,
                               kda_dtype dt, float *o, float *final_state, void *stream) {
    const size_t need = kda_prefill_workspace_bytes(total_tokens, nseq, H, dk, dv, dt);
    if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_TOO_LARGE;
    void *ws = nullptr;
    const hipError_t e = scratch_address(stream, &ws);
    if (e != hipSuccess) return kda::record_hip_error(e);
    // kda_prefill validates every argument (an invalid shape has need == 0 and is rejected
    // there) and launches the same kernels on the scratch array
    return kda_prefill(q, k, v, log_alpha, beta, init_state, cu_seqlens, nseq, total_tokens, H, dk, dv, dt,
                       o, final_state, ws, (size_t)KDA_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
