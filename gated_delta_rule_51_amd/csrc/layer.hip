// The KDA layer's passes around the recurrence (gfx950): the decay gate, the
// ShortConv + Swish (+ L2) prologue and the RMSNorm + output-gate epilogue, as
// the Kimi K3 report digest describes the layer (bounded-decay section: g =
// g_min Sigmoid(e^{A_h} z) with g_min = -5; the paragraph after the KDA update
// equation: ShortConv of kernel size 4 and Swish on q, k, v, L2 normalisation
// of q and k; the output-gate section: per-head RMSNorm times a Sigmoid gate).
//
// All three are one streaming pass over [N, H, d] rows: HBM-bound, no matrix
// work.  A thread owns four consecutive channels of one (token, head) row (one
// 8- or 16-byte access per tensor); the d/4 threads of a row sit in one wave,
// so a row sum (L2 or RMS norm) is a few cross-lane adds.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int LAYER_THREADS = 256;
constexpr float GATE_MIN = -5.0f;  // g_min of the bounded gate

__device__ __forceinline__ float sigmoidf(float x) { return 1.f / (1.f + expf(-x)); }

template <typename T>
__device__ __forceinline__ void store_out4(T *p, f32x4 x) {
    if constexpr (sizeof(T) == 4) {
        *reinterpret_cast<f32x4 *>(p) = x;
    } else {
        *reinterpret_cast<bf16x4 *>(p) = to_bf16x4(x);  // round to nearest even
    }
}

// Sum over the R lanes of a row (R a power of two, rows aligned to R lanes).
template <int R>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
    for (int m = 1; m < R; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

// ------------------------------------------------------------------ decay gate
// g = -5 Sigmoid(e^{A_h} z) for every (token, head, channel); the result is
// written in the input dtype, the form the recurrence's entry points take.
template <typename T>
__global__ __launch_bounds__(LAYER_THREADS) void gate_kernel(const T *__restrict__ z,
                                                             const float *__restrict__ A_log,
                                                             T *__restrict__ g, int64_t quads, int32_t H,
                                                             int32_t dk) {
    const int64_t stride = (int64_t)gridDim.x * LAYER_THREADS;
    for (int64_t i = (int64_t)blockIdx.x * LAYER_THREADS + threadIdx.x; i < quads; i += stride) {
        const int64_t e = 4 * i;
        const int h = (int)((e / dk) % H);
        const float s = expf(A_log[h]);
        const f32x4 x = load_in4(z + e);
        f32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = GATE_MIN * sigmoidf(s * x[j]);
        store_out4(g + e, r);
    }
}

// ------------------------------------------------------------------ ShortConv prologue
// y_t = Swish(sum_{j<4} w[j] x_{t-j}) per (head, channel), inputs before the
// sequence's first token from its cache (3 values, oldest first; zeros without
// a cache), then optionally y / sqrt(sum_c y^2 + eps) over the row.
template <typename T, int D>
__global__ __launch_bounds__(LAYER_THREADS) void short_conv_kernel(
    const T *__restrict__ x, const float *__restrict__ w, const float *__restrict__ cache,
    const int32_t *__restrict__ cu, int32_t nseq, int64_t rows, int32_t H, bool l2norm, float eps,
    T *__restrict__ y) {
    constexpr int R = D / 4;  // threads per (token, head) row
    const int64_t stride = (int64_t)gridDim.x * LAYER_THREADS / R;
    const int c0 = 4 * (threadIdx.x % R);
    for (int64_t row = ((int64_t)blockIdx.x * LAYER_THREADS + threadIdx.x) / R; row < rows; row += stride) {
        const int64_t t = row / H;
        const int h = (int)(row - t * H);
        // sequence of token t: the last s with cu[s] <= t
        int lo = 0, hi = nseq - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cu[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        const int64_t bos = cu[lo];
        f32x4 wv[4];  // the 4 taps of channel c0 + m
#pragma unroll
        for (int m = 0; m < 4; ++m) wv[m] = *reinterpret_cast<const f32x4 *>(w + ((int64_t)h * D + c0 + m) * 4);
        f32x4 acc = zero4();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t src = t - j;
            f32x4 xv;
            if (src >= bos) {
                xv = load_in4(x + (src * H + h) * D + c0);
            } else if (cache) {  // position 3 + (src - bos) of the cache, oldest first
                const float *cp = cache + (((int64_t)lo * H + h) * D + c0) * 3 + (3 + (src - bos));
#pragma unroll
                for (int m = 0; m < 4; ++m) xv[m] = cp[3 * m];
            } else {
                xv = zero4();
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[m] += wv[m][j] * xv[m];
        }
        f32x4 r;
#pragma unroll
        for (int m = 0; m < 4; ++m) r[m] = acc[m] * sigmoidf(acc[m]);  // Swish
        if (l2norm) {
            const float ss = row_sum<R>(r[0] * r[0] + r[1] * r[1] + r[2] * r[2] + r[3] * r[3]);
            r = r * (1.f / sqrtf(ss + eps));
        }
        store_out4(y + row * D + c0, r);
    }
}

// The cache after each sequence: its last 3 inputs, oldest first, reaching into
// the incoming cache when the sequence is shorter than 3 tokens.  One thread per
// (sequence, head, channel) reads all three sources before writing, so the
// outgoing cache may be the incoming one.
template <typename T>
__global__ __launch_bounds__(LAYER_THREADS) void conv_cache_kernel(const T *__restrict__ x,
                                                                   const float *cache_in,
                                                                   const int32_t *__restrict__ cu,
                                                                   int64_t items, int32_t H, int32_t d,
                                                                   float *cache_out) {
    const int64_t i = (int64_t)blockIdx.x * LAYER_THREADS + threadIdx.x;
    if (i >= items) return;
    const int64_t s = i / ((int64_t)H * d);
    const int64_t hc = i - s * H * d;
    const int h = (int)(hc / d), c = (int)(hc - (int64_t)h * d);
    const int64_t bos = cu[s], eos = cu[s + 1], len = eos - bos;
    float v[3];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const int64_t src = eos - 3 + m;
        if (src >= bos)
            v[m] = load_in(x + (src * H + h) * d + c);
        else
            v[m] = cache_in ? cache_in[i * 3 + m + len] : 0.f;
    }
#pragma unroll
    for (int m = 0; m < 3; ++m) cache_out[i * 3 + m] = v[m];
}

// ------------------------------------------------------------------ epilogue
// y = Sigmoid(u) * o / sqrt(mean(o^2) + eps) * w over the dv channels of a head.
template <typename T, int D>
__global__ __launch_bounds__(LAYER_THREADS) void out_norm_gate_kernel(const float *__restrict__ o,
                                                                      const T *__restrict__ u,
                                                                      const float *__restrict__ w, float eps,
                                                                      int64_t rows, T *__restrict__ y) {
    constexpr int R = D / 4;
    const int64_t stride = (int64_t)gridDim.x * LAYER_THREADS / R;
    const int c0 = 4 * (threadIdx.x % R);
    const f32x4 wv = *reinterpret_cast<const f32x4 *>(w + c0);
    for (int64_t row = ((int64_t)blockIdx.x * LAYER_THREADS + threadIdx.x) / R; row < rows; row += stride) {
        const f32x4 ov = *reinterpret_cast<const f32x4 *>(o + row * D + c0);
        const f32x4 uv = load_in4(u + row * D + c0);
        const float ms = row_sum<R>(ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3]) * (1.f / D);
        const float inv = 1.f / sqrtf(ms + eps);
        f32x4 r;
#pragma unroll
        for (int m = 0; m < 4; ++m) r[m] = sigmoidf(uv[m]) * ov[m] * inv * wv[m];
        store_out4(y + row * D + c0, r);
    }
}

// ------------------------------------------------------------------ launchers

// Blocks for a grid-stride pass over `threads` threads: enough to fill the chip
// several times over, at most 2^20 threads in flight.
static unsigned layer_blocks(int64_t threads) {
    const int64_t b = (threads + LAYER_THREADS - 1) / LAYER_THREADS;
    const int64_t cap = (int64_t(1) << 20) / LAYER_THREADS;
    return (unsigned)(b < 1 ? 1 : (b < cap ? b : cap));
}

hipError_t launch_gate(const GateArgs &a) {
    const int64_t quads = a.N * a.H * a.dk / 4;
    if (quads == 0) return hipSuccess;
    const hipStream_t st = (hipStream_t)a.stream;
    if (a.bf16)
        hipLaunchKernelGGL(gate_kernel<__bf16>, dim3(layer_blocks(quads)), dim3(LAYER_THREADS), 0, st,
                           (const __bf16 *)a.z, a.A_log, (__bf16 *)a.g, quads, a.H, a.dk);
    else
        hipLaunchKernelGGL(gate_kernel<float>, dim3(layer_blocks(quads)), dim3(LAYER_THREADS), 0, st,
                           (const float *)a.z, a.A_log, (float *)a.g, quads, a.H, a.dk);
    return hipGetLastError();
}

template <typename T, int D>
static void launch_conv_t(const ShortConvArgs &a, int64_t rows) {
    hipLaunchKernelGGL((short_conv_kernel<T, D>), dim3(layer_blocks(rows * (D / 4))), dim3(LAYER_THREADS), 0,
                       (hipStream_t)a.stream, (const T *)a.x, a.w, a.cache_in, a.cu, a.nseq, rows, a.H,
                       a.l2norm, a.eps, (T *)a.y);
}

template <typename T>
static hipError_t launch_conv_dt(const ShortConvArgs &a) {
    const int64_t rows = a.N * a.H;
    if (rows > 0) {
        switch (a.d) {
            case 16: launch_conv_t<T, 16>(a, rows); break;
            case 32: launch_conv_t<T, 32>(a, rows); break;
            case 64: launch_conv_t<T, 64>(a, rows); break;
            case 128: launch_conv_t<T, 128>(a, rows); break;
            default: return hipErrorInvalidValue;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.cache_out) {
        const int64_t items = (int64_t)a.nseq * a.H * a.d;
        hipLaunchKernelGGL(conv_cache_kernel<T>, dim3((unsigned)((items + LAYER_THREADS - 1) / LAYER_THREADS)),
                           dim3(LAYER_THREADS), 0, (hipStream_t)a.stream, (const T *)a.x, a.cache_in, a.cu,
                           items, a.H, a.d, a.cache_out);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_short_conv(const ShortConvArgs &a) {
    return a.bf16 ? launch_conv_dt<__bf16>(a) : launch_conv_dt<float>(a);
}

template <typename T, int D>
static void launch_epi_t(const OutNormGateArgs &a, int64_t rows) {
    hipLaunchKernelGGL((out_norm_gate_kernel<T, D>), dim3(layer_blocks(rows * (D / 4))), dim3(LAYER_THREADS), 0,
                       (hipStream_t)a.stream, a.o, (const T *)a.u, a.w, a.eps, rows, (T *)a.y);
}

template <typename T>
static hipError_t launch_epi_dt(const OutNormGateArgs &a) {
    const int64_t rows = a.N * a.H;
    if (rows == 0) return hipSuccess;
    switch (a.dv) {
        case 16: launch_epi_t<T, 16>(a, rows); break;
        case 32: launch_epi_t<T, 32>(a, rows); break;
        case 64: launch_epi_t<T, 64>(a, rows); break;
        case 128: launch_epi_t<T, 128>(a, rows); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_out_norm_gate(const OutNormGateArgs &a) {
    return a.bf16 ? launch_epi_dt<__bf16>(a) : launch_epi_dt<float>(a);
}

}  // namespace kda
