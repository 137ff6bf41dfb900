// Device building blocks shared by the KDA kernels (gfx950 / CDNA4, wave64).
//
// Fragment convention.  Every matrix operand is cut into 16x16 tiles.  A
// "frag4" of a 16x16 tile X is what one lane of a 64-lane wave holds of it:
//     lane l = 16*g + n  (g = l / 16 in 0..3, n = l % 16) holds X[4g + j][n], j = 0..3.
// This is the accumulator layout of the 16x16 MFMA instructions, so a product's
// result is a frag4.  A product D += A * B over a 16-long contraction takes
//     A as the frag4 of A^T  (lane (g, m) holds A[m][4g + j]) and
//     B as the frag4 of B    (lane (g, n) holds B[4g + j][n]).
// The hardware maps (lane group g, register slot) to the contraction index in
// the same way for A and B, so any consistent packing of two 16-long blocks
// into the 32-long contraction of v_mfma_f32_16x16x32_bf16 is valid; the
// helpers below put block 0 in slots 0..3 and block 1 in slots 4..7.
//
// Precision.  A "split" operand x = hi + lo holds the bf16 rounding of x in hi
// and the bf16 rounding of the residual in lo (about 16 mantissa bits in
// total).  A split product uses hi*hi + lo*hi + hi*lo (and lo*lo where it costs
// nothing), all accumulated in fp32 by the matrix cores.  For fp32 inputs the products use
// v_mfma_f32_16x16x4_f32, which multiplies in full fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int CHUNK = 16;
constexpr int WAVE = 64;

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ float bf16_to_f32(__bf16 x) {
    return bf16_bits_to_f32(__builtin_bit_cast(uint16_t, x));
}

// Round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return static_cast<__bf16>(x); }

// Vector conversion: lowers to two packed v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Widen four bf16 by moving each into the high half of a 32-bit word (explicit
// bit operations on the packed pairs, so no element is converted twice).
__device__ __forceinline__ f32x4 from_bf16x4(bf16x4 x) {
    const u32x2_t w = __builtin_bit_cast(u32x2_t, x);
    return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                 __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
}

struct Split4 {
    bf16x4 hi, lo;
};

// x = hi + lo: hi = bf16(x), lo = bf16(x - hi); 3 VALU operations per element.
__device__ __forceinline__ Split4 split4(f32x4 x) {
    Split4 s;
    s.hi = to_bf16x4(x);
    s.lo = to_bf16x4(x - from_bf16x4(s.hi));
    return s;
}

// Input element loads: T is float or __bf16; the value is widened exactly.
template <typename T>
__device__ __forceinline__ float load_in(const T *p) {
    if constexpr (sizeof(T) == 4) {
        return *p;
    } else {
        return bf16_bits_to_f32(*reinterpret_cast<const uint16_t *>(p));
    }
}

// Four consecutive input elements (8-byte aligned for bf16, 16-byte for fp32).
template <typename T>
__device__ __forceinline__ f32x4 load_in4(const T *p) {
    if constexpr (sizeof(T) == 4) {
        return *reinterpret_cast<const f32x4 *>(p);
    } else {
        const u16x4 b = *reinterpret_cast<const u16x4 *>(p);
        f32x4 r;
        r[0] = bf16_bits_to_f32(b[0]);
        r[1] = bf16_bits_to_f32(b[1]);
        r[2] = bf16_bits_to_f32(b[2]);
        r[3] = bf16_bits_to_f32(b[3]);
        return r;
    }
}

// ---------------------------------------------------------------- MFMA wrappers

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A single 16-long contraction runs on the 32-long instruction with the upper
// half zero, so every bf16 product in the library uses one instruction form and
// one operand layout.  (An earlier version that mixed in the 16x16x16 form gave
// wrong results for some workgroup shapes; the cause was not established -- an
// operand-layout assumption or a missing wait in that code are as likely as the
// instruction itself -- and the single-form code passes every test.)
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    const bf16x4 z = {};
    return mma32(cat(a, z), cat(b, z), c);
}

// fp32 product over one 16-long block: four 16x16x4 fp32 MFMAs; MFMA j uses
// contraction index 4g + j from lane group g.
__device__ __forceinline__ f32x4 mma_f32_k16(f32x4 a, f32x4 b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
}

// Split product over one 16-long block, as two K=32 MFMAs sharing the A
// operand [a.hi | a.lo]: against [b.hi | b.hi] (hi*hi + lo*hi) and against
// [b.lo | b.lo] (hi*lo + lo*lo), i.e. the full product of the split values.
__device__ __forceinline__ f32x4 mma_split_k16(const Split4 &a, const Split4 &b, f32x4 c) {
    const bf16x8 aa = cat(a.hi, a.lo);
    c = mma32(aa, cat(b.hi, b.hi), c);
    return mma32(aa, cat(b.lo, b.lo), c);
}

// Split A against an exactly representable bf16 B: hi*B + lo*B, one K=32 MFMA.
__device__ __forceinline__ f32x4 mma_splitA_k16(const Split4 &a, bf16x4 b, f32x4 c) {
    return mma32(cat(a.hi, a.lo), cat(b, b), c);
}

// Split product over two 16-long blocks (0 and 1): three K=32 MFMAs.
__device__ __forceinline__ f32x4 mma_split_k32(const Split4 &a0, const Split4 &a1,
                                               const Split4 &b0, const Split4 &b1, f32x4 c) {
    c = mma32(cat(a0.hi, a1.hi), cat(b0.hi, b1.hi), c);
    c = mma32(cat(a0.lo, a1.lo), cat(b0.hi, b1.hi), c);
    return mma32(cat(a0.hi, a1.hi), cat(b0.lo, b1.lo), c);
}

// Single-bf16 product over two 16-long blocks: one K=32 MFMA.
__device__ __forceinline__ f32x4 mma_single_k32(bf16x4 a0, bf16x4 a1, bf16x4 b0, bf16x4 b1, f32x4 c) {
    return mma32(cat(a0, a1), cat(b0, b1), c);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// exp for the decay factors: ROCm's device expf (full-accuracy path).
__device__ __forceinline__ float decay_exp(float x) { return expf(x); }

// exp through the hardware 2^x (v_exp_f32) on x * log2(e).  For the gate range
// [-5, 0] the rounding of the product costs at most ~4e-7 relative, far below
// the bf16 operand rounding it feeds; used for bf16 inputs only.
__device__ __forceinline__ float decay_exp_fast(float x) { return __expf(x); }

// ---------------------------------------------------------------- buffer access
//
// Raw buffer resources (gfx9 family word 3 = 0x00020000): the base address is
// uniform (SGPRs), the per-lane byte offset is a VGPR.  A lane whose offset is at
// or beyond num_records reads zeros and its stores are dropped by the hardware;
// OOB is used to park padding lanes of a ragged chunk.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t BUF_WORD3 = 0x00020000u;
constexpr uint32_t OOB = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, (int)BUF_WORD3);
}

__device__ __forceinline__ uint16_t buf_load_u16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

__device__ __forceinline__ uint32_t buf_load_u32(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 buf_load_u32x2(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}

__device__ __forceinline__ u32x4 buf_load_u32x4(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ void buf_store_f32(float x, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
}

// Widen packed input elements held in 32-bit words.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------- matrix-core layout helpers

__device__ __forceinline__ f32x4 unpack_bf16x4(u32x2 w) {
    return f32x4{lo_bf16(w[0]), hi_bf16(w[0]), lo_bf16(w[1]), hi_bf16(w[1])};
}

// B operand of the 16x16 identity (lane (g4, n) holds I[4 g4 + j][n]).  A 16x16
// bf16 tile held as the A operand of a product -- row m in lane group m, four
// consecutive columns per lane -- times this returns the same tile in the
// accumulator layout (four consecutive rows per lane, one column per lane):
// a transpose of the register layout on the matrix cores, exact for bf16 data.
__device__ __forceinline__ bf16x4 identity_operand(int g4, int l16) {
    u16x4 bits;
#pragma unroll
    for (int j = 0; j < 4; ++j) bits[j] = (4 * g4 + j == l16) ? 0x3f80 : 0;
    return __builtin_bit_cast(bf16x4, bits);
}

// A operands of -I in one half of the 32-long contraction and 0 in the other:
// with B = cat(hi_a, hi_b) (two bf16 tiles in the layout of the accumulator),
// mma32(neg_identity_operand<0>, B, x) = x - hi_a and <1> gives x - hi_b.
// With hi = x rounded to bf16 that difference is exactly representable, and
// the matrix core forms it exactly (one nonzero product, fp32 accumulation):
// the residual of a hi/lo bf16 split without vector-ALU unpacking.
template <int HALF>
__device__ __forceinline__ bf16x8 neg_identity_operand(int g4, int l16) {
    u16x4 bits;
#pragma unroll
    for (int j = 0; j < 4; ++j) bits[j] = (4 * g4 + j == l16) ? 0xbf80 : 0;
    const bf16x4 m = __builtin_bit_cast(bf16x4, bits), z = {};
    return HALF == 0 ? cat(m, z) : cat(z, m);
}
// x = hi + lo in bf16, x in the accumulator layout; returns lo, sets hh = cat(hi, hi).
__device__ __forceinline__ bf16x4 split_lo(f32x4 x, const bf16x8 &nil, bf16x8 &hh) {
    const bf16x4 hi = to_bf16x4(x);
    hh = cat(hi, hi);
    return to_bf16x4(mma32(nil, hh, x));
}

// Longest chains first.  A chain is one (sequence, head) recurrence, and its cost
// grows with its sequence's length; workgroups go to compute units in blockIdx
// order as units free up, so in index order a long sequence that comes late ends
// the launch well after the average.  With the sequences ranked by length,
// longest first (ties in index order), dispatch slot p runs head p % H of the
// sequence of rank p / H: greedy list scheduling with the longest jobs first,
// which ends within about one short chain of the average.  Every thread of the
// workgroup calls it (two barriers); nsort is the number of sequences when it is
// in [2, LPT_MAX_SEQS], else 0 and the slot is the chain.
constexpr int LPT_MAX_SEQS = 128;
__device__ __forceinline__ int lpt_chain(const int32_t *__restrict__ cu, int nsort, int H, int slot) {
    if (nsort < 2 || nsort > LPT_MAX_SEQS) return slot;
    __shared__ int32_t s_len[LPT_MAX_SEQS];
    __shared__ int32_t s_pick;
    const int nt = (int)blockDim.x;
    for (int t = (int)threadIdx.x; t < nsort; t += nt) s_len[t] = cu[t + 1] - cu[t];
    __syncthreads();
    const int r = slot / H;
    for (int t = (int)threadIdx.x; t < nsort; t += nt) {
        const int lt = s_len[t];
        int rank = 0;
        for (int u = 0; u < nsort; ++u) {
            const int lu = s_len[u];
            rank += (lu > lt) | ((lu == lt) & (u < t));
        }
        if (rank == r) s_pick = t;
    }
    __syncthreads();
    return s_pick * H + slot % H;
}

}  // namespace kda
