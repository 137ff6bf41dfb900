// The KDA layer's prologue evaluated where the prefill kernels load their
// inputs (the fused layer prefill).  Kimi K3 report digest, section "Kimi Delta
// Attention", the paragraph after the update equation: q, k and v each pass
// through a causal short convolution of kernel size 4 and Swish, and q and k are
// then L2-normalised; the bounded-decay section gives the gate
// g = -5 Sigmoid(e^{A_h} z).  Both prefill kernels apply it to the raw inputs
// they load, in the same fp32 arithmetic as the stand-alone passes of layer.hip
// (same operation order), and round the results to bf16 -- the values the
// stand-alone passes would have written -- before the recurrence uses them.
//
// Inside a chunk a lane (g4, l16) holds token l16; the convolution's earlier
// tokens come from lanes l16 - 1 .. l16 - 3 of the same 16-lane row (a DPP
// rotation), and for l16 < 3 from lanes 13 .. 15 of a second register that holds
// the three tokens before the chunk (the previous chunk's last rows, or the
// sequence's convolution cache before its first chunk).
#pragma once
#include "kda_device.hpp"
#include "kda_launch.hpp"  // struct LayerPrologue

namespace kda {

constexpr float LAYER_GATE_MIN = -5.0f;  // g_min of the bounded gate

// The elementwise arithmetic below is shared with the stand-alone passes of
// layer.hip and written with explicit fused multiply-adds and a fixed summation
// tree, so a value computed here and there rounds identically: the fused layer
// prefill then hands the recurrence bit for bit the inputs the separate passes
// would have written.

// Sigmoid on the hardware exp and reciprocal (about 1e-6 relative; every use is
// rounded to the input dtype or compared at the fp32 bar).
__device__ __forceinline__ float layer_sigmoid(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// Swish of the 4-tap causal convolution: w[j] multiplies x_{t-j}.
__device__ __forceinline__ float conv4_swish(const f32x4 &w, float x0, float x1, float x2, float x3) {
    const float a = __builtin_fmaf(w[3], x3, __builtin_fmaf(w[2], x2, __builtin_fmaf(w[1], x1, w[0] * x0)));
    return a * layer_sigmoid(a);
}

// Sum of squares of eight consecutive channels c[0..7] (the first step of a row's
// L2 norm; the row sum then adds the octets of a row as a butterfly over the
// octet index, lowest bit first).
__device__ __forceinline__ float octet_sumsq(const float (&c)[8]) {
    float s[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) s[m] = __builtin_fmaf(c[m], c[m], c[m + 4] * c[m + 4]);
    return (s[0] + s[1]) + (s[2] + s[3]);
}

// The decay gate of one logit: -5 Sigmoid(e^{A_h} z), with eA = e^{A_h}.
__device__ __forceinline__ float gate_of(float eA, float z) { return LAYER_GATE_MIN * layer_sigmoid(eA * z); }

// The packed word of token l16 - S (S = 1..3) of the lane's row: lane l16 - S of
// `cur` when l16 >= S, else lane l16 - S + 16 of `prev`.
template <int S>
__device__ __forceinline__ uint32_t conv_tap(uint32_t cur, uint32_t prev, int l16) {
    const uint32_t a = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)cur, 0x120 + S, 0xf, 0xf, false);
    const uint32_t b = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)prev, 0x120 + S, 0xf, 0xf, false);
    return l16 >= S ? a : b;
}

// Swish of the convolution for the 2 W bf16 channels packed in W words (low half
// first); w[c] holds the 4 taps of channel c.
template <int W>
__device__ __forceinline__ void conv_swish(const uint32_t (&cur)[W], const uint32_t (&prev)[W], const f32x4 (&w)[2 * W],
                                           int l16, float (&y)[2 * W]) {
#pragma unroll
    for (int i = 0; i < W; ++i) {
        const uint32_t x0 = cur[i], x1 = conv_tap<1>(cur[i], prev[i], l16), x2 = conv_tap<2>(cur[i], prev[i], l16),
                       x3 = conv_tap<3>(cur[i], prev[i], l16);
        y[2 * i] = conv4_swish(w[2 * i], lo_bf16(x0), lo_bf16(x1), lo_bf16(x2), lo_bf16(x3));
        y[2 * i + 1] = conv4_swish(w[2 * i + 1], hi_bf16(x0), hi_bf16(x1), hi_bf16(x2), hi_bf16(x3));
    }
}

// Round 2 W floats (times s) to bf16 and pack them as W words; rows that are not
// tokens (on == false) become zeros.
template <int W>
__device__ __forceinline__ void pack_scaled(const float (&y)[2 * W], float s, bool on, uint32_t (&out)[W]) {
#pragma unroll
    for (int i = 0; i < W; i += 2) {
        const bf16x4 b = to_bf16x4(f32x4{y[2 * i] * s, y[2 * i + 1] * s, y[2 * i + 2] * s, y[2 * i + 3] * s});
        const u32x2 u = __builtin_bit_cast(u32x2, b);
        out[i] = on ? u[0] : 0u;
        out[i + 1] = on ? u[1] : 0u;
    }
}

// Log-decay from the packed decay logits: g = -5 Sigmoid(e^{A_h} z), rounded to
// bf16; 0 on rows that are not tokens (so they leave the decay unchanged).
template <int W>
__device__ __forceinline__ void gate_words(const uint32_t (&z)[W], float eA, bool on, uint32_t (&out)[W]) {
    float g[2 * W];
#pragma unroll
    for (int i = 0; i < W; ++i) {
        g[2 * i] = gate_of(eA, lo_bf16(z[i]));
        g[2 * i + 1] = gate_of(eA, hi_bf16(z[i]));
    }
    pack_scaled<W>(g, 1.f, on, out);
}

// Three inputs before a sequence from its cache, for the lanes that hold them
// (l16 = 13, 14, 15 <-> cache positions 0, 1, 2), rounded to bf16 and packed:
// 2 W consecutive channels from `ch` of the combined q | k | v channel axis.
template <int W>
__device__ __forceinline__ void cache_halo(const float *cache, int64_t seq_head, int cw, int ch, int l16,
                                           uint32_t (&out)[W]) {
    float x[2 * W];
#pragma unroll
    for (int m = 0; m < 2 * W; ++m)
        x[m] = (cache && l16 >= 13) ? cache[(seq_head * cw + ch + m) * 3 + (l16 - 13)] : 0.f;
    pack_scaled<W>(x, 1.f, true, out);
}

// The 4 taps of 2 W consecutive channels from `ch` of head h.
template <int W>
__device__ __forceinline__ void conv_weights(const float *conv_w, int h, int cw, int ch, f32x4 (&w)[2 * W]) {
#pragma unroll
    for (int m = 0; m < 2 * W; ++m) w[m] = *reinterpret_cast<const f32x4 *>(conv_w + ((int64_t)h * cw + ch + m) * 4);
}

}  // namespace kda
