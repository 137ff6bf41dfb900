// The KDA layer's passes around the recurrence (gfx950): the decay gate, the
// ShortConv + Swish (+ L2) prologue and the RMSNorm + output-gate epilogue, as
// the Kimi K3 report digest describes the layer (bounded-decay section: g =
// g_min Sigmoid(e^{A_h} z) with g_min = -5; the paragraph after the KDA update
// equation: ShortConv of kernel size 4 and Swish on q, k, v, L2 normalisation
// of q and k; the output-gate section: per-head RMSNorm times a Sigmoid gate).
//
// All three are one streaming pass over [N, H, d] rows: HBM-bound, no matrix
// work.  A lane owns eight consecutive channels of one (token, head) row (one
// 16-byte access per bf16 tensor); the d/8 lanes of a row sit in one wave, so
// a row sum (L2 or RMS norm) is a few cross-lane adds.
#include "kda_device.hpp"
#include "kda_launch.hpp"
#include "layer_prologue.hpp"  // the elementwise arithmetic shared with the fused layer prefill

namespace kda {

constexpr int LAYER_THREADS = 256;

__device__ __forceinline__ float sigmoidf(float x) { return layer_sigmoid(x); }

// Eight consecutive elements of one row: one 16-byte access for bf16, two for fp32.
struct V8 {
    f32x4 a, b;
};

template <typename T>
__device__ __forceinline__ V8 load8(const T *p) {
    if constexpr (sizeof(T) == 4) {
        return V8{*reinterpret_cast<const f32x4 *>(p), *reinterpret_cast<const f32x4 *>(p + 4)};
    } else {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(p);
        return V8{f32x4{lo_bf16(w[0]), hi_bf16(w[0]), lo_bf16(w[1]), hi_bf16(w[1])},
                  f32x4{lo_bf16(w[2]), hi_bf16(w[2]), lo_bf16(w[3]), hi_bf16(w[3])}};
    }
}

// The same for data read once (streamed past the caches).
template <typename T>
__device__ __forceinline__ V8 load8_stream(const T *p) {
    if constexpr (sizeof(T) == 4) {
        return V8{__builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p)),
                  __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + 4))};
    } else {
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
        return V8{f32x4{lo_bf16(w[0]), hi_bf16(w[0]), lo_bf16(w[1]), hi_bf16(w[1])},
                  f32x4{lo_bf16(w[2]), hi_bf16(w[2]), lo_bf16(w[3]), hi_bf16(w[3])}};
    }
}

template <typename T>
__device__ __forceinline__ void store8(T *p, const V8 &x) {
    if constexpr (sizeof(T) == 4) {
        __builtin_nontemporal_store(x.a, reinterpret_cast<f32x4 *>(p));
        __builtin_nontemporal_store(x.b, reinterpret_cast<f32x4 *>(p + 4));
    } else {
        // round to nearest even, then one streaming 16-byte store
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, cat(to_bf16x4(x.a), to_bf16x4(x.b))),
                                    reinterpret_cast<u32x4 *>(p));
    }
}

__device__ __forceinline__ float sumsq(const V8 &x) {
    const float c[8] = {x.a[0], x.a[1], x.a[2], x.a[3], x.b[0], x.b[1], x.b[2], x.b[3]};
    return octet_sumsq(c);
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
// Eight channels per lane; dk is a power of two, so the row is a shift.
template <typename T>
__global__ __launch_bounds__(LAYER_THREADS) void gate_kernel(const T *__restrict__ z,
                                                             const float *__restrict__ A_log,
                                                             T *__restrict__ g, int64_t octs, int32_t H,
                                                             int32_t dk_shift) {
    // GATE_UNROLL octets per trip, all loads issued first, so each lane keeps
    // several 16-byte loads in flight
    constexpr int GATE_UNROLL = 4;
    const int64_t stride = (int64_t)gridDim.x * LAYER_THREADS;
    for (int64_t i0 = (int64_t)blockIdx.x * LAYER_THREADS + threadIdx.x; i0 < octs; i0 += GATE_UNROLL * stride) {
        V8 x[GATE_UNROLL];
#pragma unroll
        for (int u = 0; u < GATE_UNROLL; ++u)
            if (i0 + u * stride < octs) x[u] = load8_stream(z + 8 * (i0 + u * stride));
#pragma unroll
        for (int u = 0; u < GATE_UNROLL; ++u) {
            const int64_t i = i0 + u * stride;
            if (i >= octs) break;
            const uint32_t row = (uint32_t)((8 * i) >> dk_shift);  // (token, head) row, < 2^31
            const float s = __expf(A_log[row % (uint32_t)H]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[u].a[j] = gate_of(s, x[u].a[j]);
                x[u].b[j] = gate_of(s, x[u].b[j]);
            }
            store8(g + 8 * i, x[u]);
        }
    }
}

// ------------------------------------------------------------------ ShortConv prologue
// y_t = Swish(sum_{j<4} w[j] x_{t-j}) per (head, channel), inputs before the
// sequence's first token from its cache (3 values, oldest first; zeros without
// a cache), then optionally y / sqrt(sum_c y^2 + eps) over the row.
//
// A work item is a run of RUN consecutive tokens of one head; its D/8 lanes
// (eight channels each) walk the run carrying the last three inputs in
// registers, so each input row is read about once (plus three rows per run),
// and neighbouring items are neighbouring heads of the same tokens (coalesced
// rows).  A run that crosses into the next sequence restarts the window there.
constexpr int CONV_RUN = 16;

template <typename T, int D>
__global__ __launch_bounds__(LAYER_THREADS) void short_conv_kernel(
    const T *__restrict__ x, const float *__restrict__ w, const float *__restrict__ cache,
    const int32_t *__restrict__ cu, int32_t nseq, int64_t N, int32_t H, bool l2norm, float eps,
    T *__restrict__ y) {
    constexpr int R = D / 8;  // lanes per (token, head) row
    const int64_t items = (N + CONV_RUN - 1) / CONV_RUN * H;
    const int64_t stride = (int64_t)gridDim.x * LAYER_THREADS / R;
    const int c0 = 8 * (threadIdx.x % R);
    for (int64_t item = ((int64_t)blockIdx.x * LAYER_THREADS + threadIdx.x) / R; item < items; item += stride) {
        const int64_t run = item / H;
        const int h = (int)(item - run * H);
        const int64_t t0 = run * CONV_RUN;
        const int64_t t1 = t0 + CONV_RUN < N ? t0 + CONV_RUN : N;
        float wv[4][8];  // tap j of channel c0 + m
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const f32x4 wm = *reinterpret_cast<const f32x4 *>(w + ((int64_t)h * D + c0 + m) * 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) wv[j][m] = wm[j];
        }
        // sequence of token t0: the last s with cu[s] <= t0 (without cu_seqlens,
        // every token is a sequence of its own: a decode step)
        int s = 0;
        int64_t bos, eos;
        if (cu) {
            int hi = nseq - 1;
            while (s < hi) {
                const int mid = (s + hi + 1) >> 1;
                if (cu[mid] <= t0) s = mid;
                else hi = mid - 1;
            }
            bos = cu[s];
            eos = cu[s + 1];
        } else {
            s = (int)t0;
            bos = t0;
            eos = t0 + 1;
        }
        // the window x_{t-1}, x_{t-2}, x_{t-3} before token t (cache position 3 + t - j - bos)
        V8 win[3];
        auto fill = [&](int64_t t) {
#pragma unroll
            for (int j = 1; j <= 3; ++j) {
                const int64_t src = t - j;
                if (src >= bos) {
                    win[j - 1] = load8(x + (src * H + h) * D + c0);
                } else if (cache) {
                    const float *cp = cache + (((int64_t)s * H + h) * D + c0) * 3 + (3 + (src - bos));
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        win[j - 1].a[m] = cp[3 * m];
                        win[j - 1].b[m] = cp[3 * (m + 4)];
                    }
                } else {
                    win[j - 1] = V8{zero4(), zero4()};
                }
            }
        };
        fill(t0);
        V8 xn = load8(x + (t0 * H + h) * D + c0);  // the next token's input, one token ahead
        for (int64_t t = t0; t < t1; ++t) {
            if (t == eos) {  // the run enters the next non-empty sequence
                if (cu) {
                    while (cu[s + 1] <= t) ++s;
                    bos = cu[s];
                    eos = cu[s + 1];
                } else {
                    s = (int)t;
                    bos = t;
                    eos = t + 1;
                }
                fill(t);
            }
            const V8 xt = xn;
            if (t + 1 < t1) xn = load8(x + ((t + 1) * H + h) * D + c0);
            V8 r;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                r.a[m] = conv4_swish(f32x4{wv[0][m], wv[1][m], wv[2][m], wv[3][m]}, xt.a[m], win[0].a[m],
                                     win[1].a[m], win[2].a[m]);
                r.b[m] = conv4_swish(f32x4{wv[0][m + 4], wv[1][m + 4], wv[2][m + 4], wv[3][m + 4]}, xt.b[m],
                                     win[0].b[m], win[1].b[m], win[2].b[m]);
            }
            if (l2norm) {
                const float inv = __builtin_amdgcn_rsqf(row_sum<R>(sumsq(r)) + eps);
                r.a = r.a * inv;
                r.b = r.b * inv;
            }
            store8(y + (t * H + h) * D + c0, r);
            win[2] = win[1];
            win[1] = win[0];
            win[0] = xt;
        }
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
    const int64_t bos = cu ? cu[s] : s, eos = cu ? cu[s + 1] : s + 1, len = eos - bos;
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

// The cache after a fused layer prefill (q, k and v read raw by the prefill
// kernels): per (sequence, head), for each channel of the combined q | k | v axis
// (2 dk + dv channels, the layout of the decode layer step's cache), the last 3
// inputs, oldest first, reaching into the incoming cache for short sequences.
// As above, each thread reads its sources before writing, so the caches may alias.
__global__ __launch_bounds__(LAYER_THREADS) void layer_conv_cache_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *cache_in, const int32_t *__restrict__ cu, int64_t items, int32_t H, int32_t dk, int32_t dv,
    float *cache_out) {
    const int64_t i = (int64_t)blockIdx.x * LAYER_THREADS + threadIdx.x;
    if (i >= items) return;
    const int cw = 2 * dk + dv;
    const int64_t s = i / ((int64_t)H * cw);
    const int64_t hc = i - s * H * cw;
    const int h = (int)(hc / cw), c = (int)(hc - (int64_t)h * cw);
    const __bf16 *x = c < dk ? q : (c < 2 * dk ? k : v);
    const int d = c < 2 * dk ? dk : dv;
    const int cc = c < dk ? c : (c < 2 * dk ? c - dk : c - 2 * dk);
    const int64_t bos = cu[s], eos = cu[s + 1], len = eos - bos;
    float r[3];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const int64_t src = eos - 3 + m;
        if (src >= bos)
            r[m] = load_in(x + (src * H + h) * d + cc);
        else
            r[m] = cache_in ? cache_in[i * 3 + m + len] : 0.f;
    }
#pragma unroll
    for (int m = 0; m < 3; ++m) cache_out[i * 3 + m] = r[m];
}

hipError_t launch_layer_conv_cache(const void *q, const void *k, const void *v, const float *cache_in,
                                   float *cache_out, const int32_t *cu, int32_t nseq, int32_t H, int32_t dk,
                                   int32_t dv, void *stream) {
    const int64_t items = (int64_t)nseq * H * (2 * dk + dv);
    hipLaunchKernelGGL(layer_conv_cache_kernel, dim3((unsigned)((items + LAYER_THREADS - 1) / LAYER_THREADS)),
                       dim3(LAYER_THREADS), 0, (hipStream_t)stream, (const __bf16 *)q, (const __bf16 *)k,
                       (const __bf16 *)v, cache_in, cu, items, H, dk, dv, cache_out);
    return hipGetLastError();
}

// ------------------------------------------------------------------ epilogue
// y = Sigmoid(u) * o / sqrt(mean(o^2) + eps) * w over the dv channels of a head.
template <typename T, int D>
__global__ __launch_bounds__(LAYER_THREADS) void out_norm_gate_kernel(const float *__restrict__ o,
                                                                      const T *__restrict__ u,
                                                                      const float *__restrict__ w, float eps,
                                                                      int64_t rows, T *__restrict__ y) {
    constexpr int R = D / 8;
    const int64_t stride = (int64_t)gridDim.x * LAYER_THREADS / R;
    const int c0 = 8 * (threadIdx.x % R);
    const V8 wv = load8(w + c0);
    // two rows per trip, loads first (the lanes of a row stay together: both
    // rows are tested for the whole row group)
    for (int64_t r0 = ((int64_t)blockIdx.x * LAYER_THREADS + threadIdx.x) / R; r0 < rows; r0 += 2 * stride) {
        V8 ov[2], uv[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int64_t row = r0 + k * stride;
            if (row < rows) {
                ov[k] = load8_stream(o + row * D + c0);
                uv[k] = load8_stream(u + row * D + c0);
            }
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int64_t row = r0 + k * stride;
            if (row >= rows) break;
            const float inv = __builtin_amdgcn_rsqf(row_sum<R>(sumsq(ov[k])) * (1.f / D) + eps);
            V8 r;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                r.a[m] = sigmoidf(uv[k].a[m]) * ov[k].a[m] * inv * wv.a[m];
                r.b[m] = sigmoidf(uv[k].b[m]) * ov[k].b[m] * inv * wv.b[m];
            }
            store8(y + row * D + c0, r);
        }
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
    const int64_t octs = a.N * a.H * a.dk / 8;
    if (octs == 0) return hipSuccess;
    const int shift = __builtin_ctz((unsigned)a.dk);
    const hipStream_t st = (hipStream_t)a.stream;
    if (a.bf16)
        hipLaunchKernelGGL(gate_kernel<__bf16>, dim3(layer_blocks(octs)), dim3(LAYER_THREADS), 0, st,
                           (const __bf16 *)a.z, a.A_log, (__bf16 *)a.g, octs, a.H, shift);
    else
        hipLaunchKernelGGL(gate_kernel<float>, dim3(layer_blocks(octs)), dim3(LAYER_THREADS), 0, st,
                           (const float *)a.z, a.A_log, (float *)a.g, octs, a.H, shift);
    return hipGetLastError();
}

template <typename T, int D>
static void launch_conv_t(const ShortConvArgs &a) {
    const int64_t items = (a.N + CONV_RUN - 1) / CONV_RUN * a.H;
    hipLaunchKernelGGL((short_conv_kernel<T, D>), dim3(layer_blocks(items * (D / 8))), dim3(LAYER_THREADS), 0,
                       (hipStream_t)a.stream, (const T *)a.x, a.w, a.cache_in, a.cu, a.nseq, a.N, a.H,
                       a.l2norm, a.eps, (T *)a.y);
}

template <typename T>
static hipError_t launch_conv_dt(const ShortConvArgs &a) {
    const int64_t rows = a.N * a.H;
    if (rows > 0) {
        switch (a.d) {
            case 16: launch_conv_t<T, 16>(a); break;
            case 32: launch_conv_t<T, 32>(a); break;
            case 64: launch_conv_t<T, 64>(a); break;
            case 128: launch_conv_t<T, 128>(a); break;
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
    hipLaunchKernelGGL((out_norm_gate_kernel<T, D>), dim3(layer_blocks(rows * (D / 8))), dim3(LAYER_THREADS), 0,
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
