// Opt-in validation of a device-resident cu_seqlens (the packed-sequence offsets every
// prefill-family call takes): cu[0] = 0, non-decreasing, cu[nseq] = N.  The calls themselves
// trust it (it lives in device memory, where the host cannot read it without a
// synchronisation); a caller that builds it on the device can check it here first.
//
// One workgroup strides over the nseq + 1 entries, each thread keeps the smallest index that
// breaks the contract, and an LDS minimum gives the first one; thread 0 writes it (or -1) to
// the result word.  No atomics and no memset, so the check records into a HIP graph as well.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {
constexpr int CHECK_THREADS = 1024;
}

__global__ __launch_bounds__(CHECK_THREADS) void check_cu_seqlens_kernel(const int32_t *__restrict__ cu, int32_t nseq,
                                                                         int64_t N, int32_t *__restrict__ result) {
    __shared__ int32_t s_min[CHECK_THREADS];
    int32_t bad = 0x7fffffff;
    for (int32_t i = threadIdx.x; i <= nseq; i += CHECK_THREADS) {
        const int32_t c = cu[i];
        bool ok = c >= 0 && (int64_t)c <= N;
        if (i == 0) ok = ok && c == 0;
        else ok = ok && cu[i - 1] <= c;
        if (i == nseq) ok = ok && (int64_t)c == N;
        if (!ok && i < bad) bad = i;
    }
    s_min[threadIdx.x] = bad;
    __syncthreads();
    for (int s = CHECK_THREADS / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) s_min[threadIdx.x] = min(s_min[threadIdx.x], s_min[threadIdx.x + s]);
        __syncthreads();
    }
    if (threadIdx.x == 0) *result = s_min[0] == 0x7fffffff ? -1 : s_min[0];
}

hipError_t launch_check_cu_seqlens(const int32_t *cu, int32_t nseq, int64_t N, int32_t *result, void *stream) {
    hipLaunchKernelGGL(check_cu_seqlens_kernel, dim3(1), dim3(CHECK_THREADS), 0, (hipStream_t)stream, cu, nseq, N,
                       result);
    return hipGetLastError();
}

}  // namespace kda
