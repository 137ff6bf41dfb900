// Backward pass of the KDA prefill (gfx950): the gradients of a loss with
// respect to q, k, v, the log-decay, beta and the initial state, given dL/do and
// dL/d(final state).  Differentiates the recurrence of the Kimi K3 report digest
// ("Kimi Delta Attention": S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T,
// o_t = S_t^T q_t) in the chunk form the prefill uses.  Per 16-token chunk with
// incoming state S0, its Delta = T'(V - K+ S0) and the adjoint S^ of the state
// after the chunk:
//     X  = A_qk^T dO + K~ S^,   E = T^T X  (rows eps_r = S^_r^T k_r),   dV = diag(beta) E
//     S^ <- Diag(e^{G_n}) S^ + Q+^T dO - K+^T dV                (the adjoint recurrence)
//     dQ = e^{G} (.) (dO S0^T + tril(dO Delta^T) K-)
//     a  = e^{-G} (.) (triu(Delta dO^T) Q+ - striu(Delta dV^T) K+ + e^{G_n} (.) (Delta S^^T))
//     b  = diag(beta) e^{G} (.) (E S0^T + stril(E Delta^T) K-),   dK = a - b
//     U  = K+ S0 + stril(K+ K-^T) Delta,   dbeta_r = eps_r . (v_r - u_r)
//     dlog_alpha_t = rowsum(dS_final (.) S_final) + sum_{s >= t} (q_s (.) dq_s - k_s (.) (a_s + b_s))
// (the last because raising g_t[c] only rescales row c of S_{t-1}).  T = (I + A_kk)^-1
// itself is needed (E), not only T' = T diag(beta).
//
// Four kernels, all in fp32 (the products on the fp32 matrix cores where they are dense):
//   0. mats      per (chunk, head): T', T^T, A_qk^T and stril(K+ K-^T);
//   1. fwd sweep per (sequence, head, groups of 16-column dv slices): the forward chunk
//      recurrence, writing S at every chunk start and every chunk's Delta;
//   2. adjoint   the same grid, chunks in reverse: dV, S^ after every chunk, E, dinit;
//   3. grads     per (chunk, head), all dv columns in 16-column blocks: dq, dk, dbeta and
//      dlog_alpha (its part from the later tokens read off the chunk's checkpoints).
// The column slices of 1 and 2 are independent (the state's columns evolve
// separately), the chunks of 0 and 3 too, so only the recurrences in 1 and 2 are serial.
#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

// Chunk c of sequence s occupies slot cu[s]/16 + s + c (the prefill workspace's map).
__device__ __forceinline__ int64_t slot_of(const int32_t *cu, int s, int c) {
    return (int64_t)cu[s] / 16 + s + c;
}

// ------------------------------------------------------------------ row-layout chunk operands
// Lane l = 16 g + m of a wave holds, of key-channel block b, token m and the four
// channels 16b + 4g + j (j = 0..3): the A-operand layout of a product contracting
// over the key channels (and, for the second factor of such a product, its B-operand
// layout).  The cumulative decay e^{G} of a channel over the chunk is then a prefix
// product across the 16 lanes of a DPP row, and its value at the last token sits in
// lane 15 of the row.  (A running product of the per-token e^{g} keeps a few ulps of
// relative error however far G falls; the exp of an fp32 cumulative sum would carry the
// sum's absolute rounding, ~1e-5 at |G| = 80, into every factor.)

template <int N>
__device__ __forceinline__ float row_shr_or1(float x) {  // lane m reads lane m - N of its row, 1 before it
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(x), 0x110 | N, 0xF, 0xF, false));
}

__device__ __forceinline__ f32x4 row_prefix_prod(f32x4 x) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[j] *= row_shr_or1<1>(x[j]);
        x[j] *= row_shr_or1<2>(x[j]);
        x[j] *= row_shr_or1<4>(x[j]);
        x[j] *= row_shr_or1<8>(x[j]);
    }
    return x;
}

// Inputs of one chunk are read through a buffer resource based at the chunk's first
// token row of the head and as long as its n rows: reads of rows past n return zeros
// without a branch (a guarded load would make the compiler wait for it at the join).
template <typename T>
__device__ __forceinline__ rsrc_t chunk_rsrc(const T *base, int64_t t0, int n, int32_t H, int h, int D) {
    return make_rsrc(base + (t0 * H + h) * (int64_t)D, (uint32_t)n * (uint32_t)H * (uint32_t)D * sizeof(T));
}

// Four consecutive input elements at byte offset off.
template <typename T>
__device__ __forceinline__ f32x4 buf_in4(rsrc_t r, uint32_t off) {
    if constexpr (sizeof(T) == 4) {
        const u32x4 w = buf_load_u32x4(r, off);
        return f32x4{__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]), __uint_as_float(w[3])};
    } else {
        return unpack_bf16x4(buf_load_u32x2(r, off));
    }
}

template <typename T>
__device__ __forceinline__ float buf_in(rsrc_t r, uint32_t off) {
    if constexpr (sizeof(T) == 4) return __uint_as_float(buf_load_u32(r, off));
    else return bf16_bits_to_f32(buf_load_u16(r, off));
}

// Four channels c0.. of token m of a chunk seen through chunk_rsrc (row layout).
template <typename T>
__device__ __forceinline__ f32x4 load_row4(rsrc_t r, int m, int32_t H, int D, int c0) {
    return buf_in4<T>(r, ((uint32_t)m * (uint32_t)H * (uint32_t)D + (uint32_t)c0) * sizeof(T));
}

// Raw words of four consecutive input elements (row layout) and their widening.  The
// sweeps carry raw words from one iteration to the next and widen them where they are
// used: a conversion right after a load would make the compiler wait for it there.
template <typename T>
using Row4Raw = std::conditional_t<sizeof(T) == 4, u32x4, u32x2>;

template <typename T>
__device__ __forceinline__ Row4Raw<T> load_row4_raw(rsrc_t r, int m, int32_t H, int D, int c0) {
    const uint32_t off = ((uint32_t)m * (uint32_t)H * (uint32_t)D + (uint32_t)c0) * sizeof(T);
    if constexpr (sizeof(T) == 4) return buf_load_u32x4(r, off);
    else return buf_load_u32x2(r, off);
}

template <typename T>
__device__ __forceinline__ f32x4 widen_row4(Row4Raw<T> w) {
    if constexpr (sizeof(T) == 4) return __builtin_bit_cast(f32x4, w);
    else return unpack_bf16x4(w);
}

// Column col of the four tokens 4g + j (the accumulator layout), through chunk_rsrc, as
// raw 32-bit words.  A bf16 element is read as the aligned word that holds it (its pair
// partner lies in the same row, so the word never leaves the resource); widen_col4 takes
// the right half.
template <typename T>
__device__ __forceinline__ uint32_t col_off(int gq, int j, int32_t H, int D, int col) {
    return ((uint32_t)(4 * gq + j) * (uint32_t)H * (uint32_t)D + (uint32_t)col) * sizeof(T);
}

template <typename T>
__device__ __forceinline__ u32x4 load_col4_raw(rsrc_t r, int gq, int32_t H, int D, int col) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = buf_load_u32(r, col_off<T>(gq, j, H, D, col) & ~3u);
    return w;
}

template <typename T>
__device__ __forceinline__ f32x4 widen_col4(u32x4 w, int gq, int32_t H, int D, int col) {
    f32x4 x;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (sizeof(T) == 4) x[j] = __uint_as_float(w[j]);
        else x[j] = (col_off<T>(gq, j, H, D, col) & 2u) ? hi_bf16(w[j]) : lo_bf16(w[j]);
    }
    return x;
}

template <typename T>
__device__ __forceinline__ f32x4 load_col4(rsrc_t r, int gq, int32_t H, int D, int col) {
    return widen_col4<T>(load_col4_raw<T>(r, gq, H, D, col), gq, H, D, col);
}

// Tokens in chunk c of a sequence of len tokens (0 outside it), wave-uniform.
__device__ __forceinline__ int chunk_len(int64_t len, int c) {
    const int64_t r = len - 16 * (int64_t)c;
    return __builtin_amdgcn_readfirstlane(c < 0 || r <= 0 ? 0 : (r < 16 ? (int)r : 16));
}

// The decay-weighted operands of one block from its raw g, k (and q): e^{G}, e^{-G} and
// e^{G_n - G} per element, G the inclusive cumulative log-decay.
struct RowOps {
    f32x4 kp, km, kt, qp, egn;  // K e^{G}, K e^{-G}, K e^{G_n - G}, Q e^{G}, e^{G_n}
};

__device__ __forceinline__ RowOps row_ops(f32x4 g, f32x4 k, f32x4 q, int lane) {
    f32x4 a;
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = expf(g[j]);
    const f32x4 P = row_prefix_prod(a);
    RowOps o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float ep = P[j], em = __builtin_amdgcn_rcpf(ep);
        const float en = __shfl(ep, lane | 15);
        o.kp[j] = k[j] * ep;
        o.km[j] = k[j] * em;
        o.kt[j] = k[j] * (en * em);
        o.qp[j] = q[j] * ep;
        o.egn[j] = en;
    }
    return o;
}

// The sequence owning chunk slot `slot`: the last s with cu[s]/16 + s <= slot.
__device__ __forceinline__ int seq_of_slot(const int32_t *cu, int32_t nseq, int64_t slot) {
    int s = 0, hi = nseq - 1;
    while (s < hi) {
        const int mid = (s + hi + 1) >> 1;
        if (slot_of(cu, mid, 0) <= slot) s = mid;
        else hi = mid - 1;
    }
    return s;
}

// ------------------------------------------------------------------ 0. chunk matrices
// Per (chunk slot, head), four 16x16 fp32 matrices stored row-major, each the matrix
// whose row m lane (g, m) reads as an MFMA A operand (columns 4g..4g+3):
constexpr int MAT_TP = 0;    // T' = T diag(beta)            (Delta = T'(V - K+ S))
constexpr int MAT_TT = 1;    // T^T                          (E = T^T X)
constexpr int MAT_AQKT = 2;  // A_qk^T, A_qk = tril(Q+ K-^T)  (A_qk^T dO)
constexpr int MAT_AP = 3;    // stril(K+ K-^T)                (U = K+ S0 + Ap Delta)
constexpr int NMAT = 4;
constexpr int MATS_WAVES = 4;

__device__ __forceinline__ f32x4 plus_identity(f32x4 x, int g4, int l16, float s) {
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = (4 * g4 + j == l16 ? s : 0.f) + x[j];
    return x;
}

// One wave per (slot, head).  K+ K-^T and Q+ K-^T on the fp32 matrix cores straight from
// the row layout; A = diag(beta) stril(K+ K-^T) is nilpotent (A^16 = 0), so
// T = (I + A)^-1 = (I - A)(I + A^2)(I + A^4)(I + A^8): eight 16x16 products.  A matrix
// X held in the accumulator layout (lane (g, n): X[4g + j][n]) is the B operand of X and
// the A operand of X^T, so each power is formed together with its transpose.
template <int DK, typename T>
__global__ __launch_bounds__(64 * MATS_WAVES) void bwd_mats_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ g, const T *__restrict__ beta,
    const int32_t *__restrict__ cu, int32_t nseq, int32_t H, int64_t items, float *__restrict__ mats) {
    constexpr int NB = DK / 16;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int lane = threadIdx.x % 64, gq = lane / 16, m = lane % 16;
    __shared__ float tr[MATS_WAVES][16][20];
    int64_t item = (int64_t)blockIdx.x * MATS_WAVES + wave;
    const bool in_grid = item < items;
    if (!in_grid) item = items - 1;  // every wave reaches the barrier below
    const int64_t slot = item / H;
    const int h = (int)(item % H);
    const int s = seq_of_slot(cu, nseq, slot);
    const int64_t bos = cu[s], len = cu[s + 1] - bos;
    const int c = (int)(slot - slot_of(cu, s, 0));
    const int n = chunk_len(len, c);
    const int64_t t0 = bos + 16 * (int64_t)c;
    const rsrc_t rq = chunk_rsrc(q, t0, n, H, h, DK), rk = chunk_rsrc(k, t0, n, H, h, DK);
    const rsrc_t rg = chunk_rsrc(g, t0, n, H, h, DK), rb = chunk_rsrc(beta, t0, n, H, h, 1);

    f32x4 akk = zero4(), aqk = zero4();
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int c0 = 16 * b + 4 * gq;
        const RowOps o = row_ops(load_row4<T>(rg, m, H, DK, c0), load_row4<T>(rk, m, H, DK, c0),
                                 load_row4<T>(rq, m, H, DK, c0), lane);
        akk = mma_f32_k16(o.kp, o.km, akk);
        aqk = mma_f32_k16(o.qp, o.km, aqk);
    }
    const f32x4 br = load_col4<T>(rb, gq, H, 1, 0);                             // beta of rows 4g + j
    const float bc = buf_in<T>(rb, (uint32_t)m * (uint32_t)H * sizeof(T));   // beta of column m
    f32x4 ac;  // A = diag(beta) stril(K+ K-^T), accumulator layout
#pragma unroll
    for (int j = 0; j < 4; ++j) ac[j] = m < 4 * gq + j ? br[j] * akk[j] : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) tr[wave][4 * gq + j][m] = ac[j];
    __syncthreads();
    const f32x4 at = *reinterpret_cast<const f32x4 *>(&tr[wave][m][4 * gq]);  // A^T, accumulator layout
    const f32x4 z = zero4();
    const f32x4 a2 = mma_f32_k16(at, ac, z), a2t = mma_f32_k16(ac, at, z);
    const f32x4 a4 = mma_f32_k16(a2t, a2, z), a4t = mma_f32_k16(a2, a2t, z);
    const f32x4 a8 = mma_f32_k16(a4t, a4, z);
    const f32x4 r1 = mma_f32_k16(plus_identity(a4t, gq, m, 1.f), plus_identity(a8, gq, m, 1.f), z);
    const f32x4 r2 = mma_f32_k16(plus_identity(a2t, gq, m, 1.f), r1, z);
    const f32x4 tc = mma_f32_k16(plus_identity(-at, gq, m, 1.f), r2, z);  // T, accumulator layout
    if (!in_grid || n == 0) return;
    float *out = mats + item * (NMAT * 256);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 4 * gq + j;
        out[MAT_TP * 256 + r * 16 + m] = tc[j] * bc;
        out[MAT_AP * 256 + r * 16 + m] = m < r ? akk[j] : 0.f;
    }
    f32x4 qt;
#pragma unroll
    for (int j = 0; j < 4; ++j) qt[j] = m <= 4 * gq + j ? aqk[j] : 0.f;
    *reinterpret_cast<f32x4 *>(out + MAT_TT * 256 + m * 16 + 4 * gq) = tc;
    *reinterpret_cast<f32x4 *>(out + MAT_AQKT * 256 + m * 16 + 4 * gq) = qt;
}


// ------------------------------------------------------------------ 1/2. the two sweeps
// A workgroup serves one (sequence, head) and NS 16-column slices of dv with two kinds
// of waves:
//   * NS slice waves keep their dk x 16 slice of the state (or of the adjoint) in
//     registers as NB accumulator tiles (tile b, lane (g, n): row 16b + 4g + j, column n
//     of the slice) and advance it with fp32 MFMAs;
//   * NP producer waves build the decay operands of the next chunk (channel block b by
//     producer b mod NP) into the other half of a double-buffered LDS set.
// One barrier per chunk hands a set over.  Both roles hold their inputs for two chunks
// in registers and load three chunks ahead (the loop is unrolled by two so that the
// register sets are fixed); a look-ahead past either end of the sequence reads empty
// resources, so the loop body has no branch.  The forward sweep walks the chunks in
// order, the adjoint sweep in reverse; both count iterations i = 0, 1, ...
template <int DK, bool ADJ, bool TRA = true>
struct SweepSet {
    float rows[16][DK + 4];       // forward: K+ rows;  adjoint: K~ rows
    float trA[TRA ? DK : 1][20];  // forward: K~^T;     adjoint: Q+^T (when the slice waves form Q+^T dO)
    float trB[ADJ ? DK : 1][20];  // adjoint: K+^T
    float gam[DK];                // e^{G_n}
};

// Adjoint sweep with NQ <= 2 slice waves: the producers also form Q+^T dO for every slice
// (it does not depend on the adjoint, so it is off the slice waves' chain) and hand it over
// as accumulator-layout tiles: t[slice][block][lane].
template <int DK, int NQ>
struct QoSet {
    f32x4 t[NQ][DK / 16][64];
};

template <int DK, int NP, bool ADJ, typename T, int NQ = 0>
struct RawBlocks {
    // producer w builds channel blocks w, w + NP, ... (a block index past NB reads an
    // empty resource and writes nothing); with NQ > 0 it also forms Q+^T dO of its blocks
    // for the NQ slices of the workgroup (dO slices loaded with the rest)
    static constexpr int NB = DK / 16, NBW = (NB + NP - 1) / NP;
    Row4Raw<T> rg[NBW], rk[NBW], rq[NBW];
    u32x4 ro[NQ > 0 ? NQ : 1];

    __device__ __forceinline__ void load(const T *q, const T *k, const T *g, int64_t t0, int n, int32_t H, int h,
                                         int wave, int lane, const float *dO = nullptr, int DV = 0, int col0 = 0) {
        const int m = lane % 16, gq = lane / 16;
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            const int b = wave + NP * i;
            const int nb = b < NB ? n : 0;
            const int c0 = (b < NB ? 16 * b : 0) + 4 * gq;
            rg[i] = load_row4_raw<T>(chunk_rsrc(g, t0, nb, H, h, DK), m, H, DK, c0);
            rk[i] = load_row4_raw<T>(chunk_rsrc(k, t0, nb, H, h, DK), m, H, DK, c0);
            if (ADJ) rq[i] = load_row4_raw<T>(chunk_rsrc(q, t0, nb, H, h, DK), m, H, DK, c0);
        }
        if constexpr (NQ > 0) {
            const rsrc_t rO = chunk_rsrc(dO, t0, n, H, h, DV);
#pragma unroll
            for (int sl = 0; sl < NQ; ++sl) ro[sl] = load_col4_raw<float>(rO, gq, H, DV, col0 + 16 * sl + m);
        }
    }

    // tsc: this producer's 16 x 20 LDS scratch (NQ > 0: the transpose of its Q+ block)
    template <bool TRA>
    __device__ __forceinline__ void build(SweepSet<DK, ADJ, TRA> &P, int wave, int lane, QoSet<DK, (NQ > 0 ? NQ : 1)> *Qo,
                                          float (*tsc)[20], int32_t H, int DV, int col0) const {
        const int m = lane % 16, gq = lane / 16;
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            const int b = wave + NP * i;
            const f32x4 kw = widen_row4<T>(rk[i]);
            const RowOps o = row_ops(widen_row4<T>(rg[i]), kw, ADJ ? widen_row4<T>(rq[i]) : kw, lane);
            if (NB % NP != 0 && b >= NB) continue;
            const int c0 = 16 * b + 4 * gq;
            *reinterpret_cast<f32x4 *>(&P.rows[m][c0]) = ADJ ? o.kt : o.kp;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (TRA) P.trA[c0 + j][m] = ADJ ? o.qp[j] : o.kt[j];
                if (ADJ) P.trB[c0 + j][m] = o.kp[j];
            }
            if (m == 15) *reinterpret_cast<f32x4 *>(&P.gam[c0]) = o.egn;
            if constexpr (NQ > 0) {
                // Q+ of this block transposed through the scratch (this wave's own writes and
                // reads, which the LDS performs in order), then one 16-long product per slice:
                // (Q+^T dO)[16b + r][col] = sum_t Q+[t][16b + r] dO[t][col]
#pragma unroll
                for (int j = 0; j < 4; ++j) tsc[4 * gq + j][m] = o.qp[j];
                const f32x4 qa = *reinterpret_cast<const f32x4 *>(&tsc[m][4 * gq]);
#pragma unroll
                for (int sl = 0; sl < NQ; ++sl)
                    Qo->t[sl][b][lane] = mma_f32_k16(qa, widen_col4<float>(ro[sl], gq, H, DV, col0 + 16 * sl + m),
                                                     zero4());
            }
        }
    }
};

// The 16x16 matrix `which` of chunk c as an A operand, through a resource that is empty
// for chunks outside the sequence (so look-ahead reads there return zeros).
__device__ __forceinline__ f32x4 load_mat(const float *mats, const int32_t *cu, int s, int c, int nc, int32_t H,
                                          int h, int which, int lane) {
    const bool in = c >= 0 && c < nc;
    const int64_t slot = in ? slot_of(cu, s, c) : 0;
    const rsrc_t r = make_rsrc(mats + ((slot * H + h) * NMAT + which) * 256, in ? 1024u : 0u);
    const u32x4 w = buf_load_u32x4(r, ((uint32_t)(lane % 16) * 16u + 4u * (uint32_t)(lane / 16)) * 4u);
    return f32x4{__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]), __uint_as_float(w[3])};
}

// vmcnt(0) with expcnt and lgkmcnt left free: used once after the prologue's state loads,
// so the loop that follows carries no pending load into its first iteration.
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// A per-wave LDS stage turns a tile held in the accumulator layout (lane (g, n): rows
// 4g + j, column n) into row-major order, which the wave then stores as one contiguous
// 1 KiB piece (lane l: row l / 4, columns 4 (l % 4) .. +3) instead of four scattered
// pieces per row group.  Row groups are 80 floats apart, so the four lane groups' writes
// fall on distinct banks.  The wave's LDS operations run in order, so no barrier is needed
// between its writes and its reads.
constexpr int STAGE_TILE = 320;

__device__ __forceinline__ void stage_put(float *st, f32x4 x, int gq, int m) {
#pragma unroll
    for (int j = 0; j < 4; ++j) st[gq * 80 + j * 16 + m] = x[j];
}

__device__ __forceinline__ f32x4 stage_get(const float *st, int lane) {
    const int r = lane / 4;
    return *reinterpret_cast<const f32x4 *>(st + (r / 4) * 80 + (r % 4) * 16 + 4 * (lane % 4));
}

__device__ __forceinline__ void buf_store_f32x4(f32x4 x, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, 0);
}

// Producer waves per workgroup of the sweeps: every SIMD gets work (a lone slice wave
// has three helpers), at most one producer per SIMD.
template <int NS>
struct SweepShape {
    static constexpr int NP = NS == 1 ? 3 : (NS == 2 ? 2 : 4);
    static constexpr int THREADS = 64 * (NS + NP);
};

template <int P>
using Par = std::integral_constant<int, P>;

// Runs body(i, Par<i & 1>) for i = 0 .. nc - 1, two iterations per trip.
template <typename F>
__device__ __forceinline__ void unrolled_chunks(int nc, F &&body) {
    int i = 0;
    for (; i + 1 < nc; i += 2) {
        body(i, Par<0>{});
        body(i + 1, Par<1>{});
    }
    if (i < nc) body(i, Par<0>{});
}

template <int DK, int NP, bool ADJ, typename T, int NQ = 0, bool TRA = true>
__device__ __forceinline__ void sweep_producer(SweepSet<DK, ADJ, TRA> (&L)[2], const T *q, const T *k, const T *g,
                                               int64_t bos, int64_t len, int nc, int32_t H, int h, int pw,
                                               int lane, QoSet<DK, (NQ > 0 ? NQ : 1)> *Qo = nullptr,
                                               float (*tsc)[20] = nullptr, const float *dO = nullptr, int DV = 0,
                                               int col0 = 0) {
    RawBlocks<DK, NP, ADJ, T, NQ> raw[2];
    auto chunk = [&](int i) { return ADJ ? nc - 1 - i : i; };
    auto load = [&](RawBlocks<DK, NP, ADJ, T, NQ> &r, int i) {
        const int c = chunk(i);
        r.load(q, k, g, bos + 16 * (int64_t)c, chunk_len(len, c), H, h, pw, lane, dO, DV, col0);
    };
    load(raw[0], 0);
    load(raw[1], 1);
    raw[0].build(L[0], pw, lane, Qo, tsc, H, DV, col0);
    load(raw[0], 2);
    __syncthreads();
    unrolled_chunks(nc, [&](int i, auto par) {
        constexpr int p = 1 - decltype(par)::value;  // the set of iteration i + 1
        raw[p].build(L[p], pw, lane, Qo ? Qo + p : Qo, tsc, H, DV, col0);
        load(raw[p], i + 3);
        __syncthreads();
    });
}

// fin != NULL: the state after each sequence's last chunk is also written there ([nseq, H,
// dk, dv]; the boundary pass of a slabbed backward).
template <int DK, int DV, int NS, typename T>
__global__ __launch_bounds__(SweepShape<NS>::THREADS) void bwd_fwd_sweep_kernel(
    const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ g, const float *__restrict__ init,
    const int32_t *__restrict__ cu, int32_t H, const float *__restrict__ mats, float *__restrict__ sck,
    float *__restrict__ dbuf, float *__restrict__ fin) {
    constexpr int NB = DK / 16, NCB = DV / 16, NG = NCB / NS, NP = SweepShape<NS>::NP;
    const int chain = blockIdx.x / NG, sg = blockIdx.x % NG;
    const int s = chain / H, h = chain % H;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int lane = threadIdx.x % 64, gq = lane / 16, m = lane % 16;
    __shared__ SweepSet<DK, false> L[2];
    __shared__ __attribute__((aligned(16))) float stage_all[NS][NB][STAGE_TILE];
    const int64_t hd = (int64_t)s * H + h;
    const int64_t bos = cu[s], len = cu[s + 1] - bos;
    const int nc = (int)((len + 15) / 16);

    if (wave >= NS) {
        sweep_producer<DK, NP, false, T>(L, k, k, g, bos, len, nc, H, h, wave - NS, lane);
        return;
    }
    // -------------------------------------------------------------------- slice wave
    const int cb = sg * NS + wave, col0 = 16 * cb;
    float *stage = stage_all[wave][0];
    f32x4 S[NB];
    {  // (an empty resource without an initial state: its loads return 0)
        const rsrc_t ri = make_rsrc(init ? init + hd * DK * DV : init, init ? DK * DV * 4u : 0u);
#pragma unroll
        for (int b = 0; b < NB; ++b) S[b] = load_col4<float>(ri, 4 * b + gq, 1, DV, col0 + m);
        wait_vm0();
    }
    u32x4 vn[2];  // v slice (raw words) and T' of the chunks two iterations ahead
    f32x4 tpn[2];
    auto load_slice = [&](int p, int c) {
        vn[p] = load_col4_raw<T>(chunk_rsrc(v, bos + 16 * (int64_t)c, chunk_len(len, c), H, h, DV), gq, H, DV,
                                 col0 + m);
        tpn[p] = load_mat(mats, cu, s, c, nc, H, h, MAT_TP, lane);
    };
    load_slice(0, 0);
    load_slice(1, 1);
    __syncthreads();
    unrolled_chunks(nc, [&](int c, auto par) {
        constexpr int p = decltype(par)::value;
        const SweepSet<DK, false> &P = L[p];
        const u32x4 vraw = vn[p];
        const f32x4 tp = tpn[p];
        load_slice(p, c + 2);
        const int64_t item = slot_of(cu, s, c) * H + h;
        // this chunk's operands; with one or two slice waves per workgroup all read from LDS
        // before anything waits for one of them (the scheduling barrier keeps the compiler
        // from moving the reads down next to their uses, where each would stall the product
        // chain for a full LDS latency); with four or more, reading them at their uses
        // measured faster (and with three waves per SIMD the early reads' registers spill)
        f32x4 kr[NB], tr[NB], gm[NB];
        constexpr bool EARLY = NS <= 2;
        auto read_rows = [&](int b) { kr[b] = *reinterpret_cast<const f32x4 *>(&P.rows[m][16 * b + 4 * gq]); };
        auto read_upd = [&](int b) {
            tr[b] = *reinterpret_cast<const f32x4 *>(&P.trA[16 * b + m][4 * gq]);
            gm[b] = *reinterpret_cast<const f32x4 *>(&P.gam[16 * b + 4 * gq]);
        };
        if constexpr (EARLY) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                read_rows(b);
                read_upd(b);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // the state at the chunk's start, staged to row-major tiles
#pragma unroll
        for (int b = 0; b < NB; ++b) stage_put(stage + b * STAGE_TILE, S[b], gq, m);
        f32x4 x = zero4();  // K+ S
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if constexpr (!EARLY) read_rows(b);
            x = mma_f32_k16(kr[b], S[b], x);
        }
        float *ck = sck + item * DK * DV + cb * 256 + 4 * lane;
#pragma unroll
        for (int b = 0; b < NB; ++b)
            *reinterpret_cast<f32x4 *>(ck + b * NCB * 256) = stage_get(stage + b * STAGE_TILE, lane);
        const f32x4 vc = widen_col4<T>(vraw, gq, H, DV, col0 + m);
        const f32x4 d = mma_f32_k16(tp, vc - x, zero4());  // Delta = T'(V - K+ S)
        stage_put(stage, d, gq, m);
        *reinterpret_cast<f32x4 *>(dbuf + item * 16 * DV + cb * 256 + 4 * lane) = stage_get(stage, lane);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if constexpr (!EARLY) read_upd(b);
            S[b] = mma_f32_k16(tr[b], d, S[b] * gm[b]);
        }
        __syncthreads();
    });
    if (fin) {  // accumulator layout: rows 16 b + 4 gq + j, column col0 + m
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) fin[(hd * DK + 16 * b + 4 * gq + j) * DV + col0 + m] = S[b][j];
    }
}

template <int DK, int DV, int NS, typename T>
__global__ __launch_bounds__(SweepShape<NS>::THREADS) void bwd_adjoint_sweep_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ g, const T *__restrict__ beta,
    const float *__restrict__ dO, const float *__restrict__ dfinal, const int32_t *__restrict__ cu, int32_t H,
    const float *__restrict__ mats, float *__restrict__ hck, float *__restrict__ ebuf, float *__restrict__ dv,
    float *__restrict__ dinit) {
    constexpr int NB = DK / 16, NCB = DV / 16, NG = NCB / NS, NP = SweepShape<NS>::NP;
    const int chain = blockIdx.x / NG, sg = blockIdx.x % NG;
    const int s = chain / H, h = chain % H;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int lane = threadIdx.x % 64, gq = lane / 16, m = lane % 16;
    // with one or two slice waves the producers (then on SIMDs of their own) form Q+^T dO
    // (QO); with four, a producer shares each slice wave's SIMD and matrix core, and moving
    // the products there measured slower (K3 layer 12.6 -> 13.5 ms); with eight the LDS
    // would not hold the tiles
    constexpr bool QO = NS <= 2;
    constexpr int NQ = QO ? NS : 1;
    __shared__ SweepSet<DK, true, !QO> L[2];
    __shared__ QoSet<DK, NQ> Qo[QO ? 2 : 1];
    __shared__ float tsc_all[QO ? NP : 1][16][20];
    __shared__ __attribute__((aligned(16))) float stage_all[NS][NB < 2 ? 2 : NB][STAGE_TILE];
    const int64_t hd = (int64_t)s * H + h;
    const int64_t bos = cu[s], len = cu[s + 1] - bos;
    const int nc = (int)((len + 15) / 16);

    if (wave >= NS) {
        if constexpr (QO)
            sweep_producer<DK, NP, true, T, NS, false>(L, q, k, g, bos, len, nc, H, h, wave - NS, lane, Qo,
                                                       tsc_all[wave - NS], dO, DV, sg * NS * 16);
        else
            sweep_producer<DK, NP, true, T, 0, true>(L, q, k, g, bos, len, nc, H, h, wave - NS, lane);
        return;
    }
    // -------------------------------------------------------------------- slice wave
    const int cb = sg * NS + wave, col0 = 16 * cb;
    float *stage = stage_all[wave][0];
    f32x4 Sh[NB];
    {
        const rsrc_t rf = make_rsrc(dfinal ? dfinal + hd * DK * DV : dfinal, dfinal ? DK * DV * 4u : 0u);
#pragma unroll
        for (int b = 0; b < NB; ++b) Sh[b] = load_col4<float>(rf, 4 * b + gq, 1, DV, col0 + m);
        wait_vm0();
    }
    u32x4 on[2], bn[2];  // dO slice and beta (raw words), A_qk^T, T^T two iterations ahead
    f32x4 aqn[2], ttn[2];
    auto load_slice = [&](int p, int c) {
        const int64_t t0 = bos + 16 * (int64_t)c;
        const int n = chunk_len(len, c);
        on[p] = load_col4_raw<float>(chunk_rsrc(dO, t0, n, H, h, DV), gq, H, DV, col0 + m);
        bn[p] = load_col4_raw<T>(chunk_rsrc(beta, t0, n, H, h, 1), gq, H, 1, 0);
        aqn[p] = load_mat(mats, cu, s, c, nc, H, h, MAT_AQKT, lane);
        ttn[p] = load_mat(mats, cu, s, c, nc, H, h, MAT_TT, lane);
    };
    load_slice(0, nc - 1);
    load_slice(1, nc - 2);
    __syncthreads();
    unrolled_chunks(nc, [&](int i, auto par) {
        constexpr int p = decltype(par)::value;
        const int c = nc - 1 - i;
        const SweepSet<DK, true, !QO> &P = L[p];
        const f32x4 ob = widen_col4<float>(on[p], gq, H, DV, col0 + m);
        const f32x4 bt = widen_col4<T>(bn[p], gq, H, 1, 0);
        const f32x4 aq = aqn[p], tt = ttn[p];
        load_slice(p, c - 2);
        const int64_t item = slot_of(cu, s, c) * H + h;
        const int64_t t0 = bos + 16 * (int64_t)c;
        const int n = chunk_len(len, c);
        // this chunk's operands read from LDS ahead of their uses: the K~ rows first, the rest
        // while the first product runs
        f32x4 kr[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) kr[b] = *reinterpret_cast<const f32x4 *>(&P.rows[m][16 * b + 4 * gq]);
        // the adjoint of the state after the chunk, staged to row-major tiles
#pragma unroll
        for (int b = 0; b < NB; ++b) stage_put(stage + b * STAGE_TILE, Sh[b], gq, m);
        f32x4 qr[NB], pr[NB], gm[NB];  // qr: Q+^T rows, or with QO the producers' Q+^T dO tile
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if constexpr (QO) qr[b] = Qo[p].t[wave][b][lane];
            else qr[b] = *reinterpret_cast<const f32x4 *>(&P.trA[16 * b + m][4 * gq]);
            pr[b] = *reinterpret_cast<const f32x4 *>(&P.trB[16 * b + m][4 * gq]);
            gm[b] = *reinterpret_cast<const f32x4 *>(&P.gam[16 * b + 4 * gq]);
        }
        if constexpr (NS <= 4) __builtin_amdgcn_sched_barrier(0);  // (the reads stay ahead of the products)
        f32x4 x = mma_f32_k16(aq, ob, zero4());  // A_qk^T dO + K~ S^
#pragma unroll
        for (int b = 0; b < NB; ++b) x = mma_f32_k16(kr[b], Sh[b], x);
        float *hk = hck + item * DK * DV + cb * 256 + 4 * lane;
#pragma unroll
        for (int b = 0; b < NB; ++b)
            *reinterpret_cast<f32x4 *>(hk + b * NCB * 256) = stage_get(stage + b * STAGE_TILE, lane);
        const f32x4 e = mma_f32_k16(tt, x, zero4());  // E = T^T X
        const f32x4 dvv = bt * e;
        stage_put(stage, e, gq, m);
        stage_put(stage + STAGE_TILE, dvv, gq, m);
        *reinterpret_cast<f32x4 *>(ebuf + item * 16 * DV + cb * 256 + 4 * lane) = stage_get(stage, lane);
        // dV rows past n are dropped by the resource
        buf_store_f32x4(stage_get(stage + STAGE_TILE, lane), chunk_rsrc(dv, t0, n, H, h, DV),
                        ((uint32_t)(lane / 4) * (uint32_t)H * DV + col0 + 4 * (lane % 4)) * 4u);
        const f32x4 nd = -dvv;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if constexpr (QO) Sh[b] = mma_f32_k16(pr[b], nd, Sh[b] * gm[b] + qr[b]);
            else Sh[b] = mma_f32_k16(pr[b], nd, mma_f32_k16(qr[b], ob, Sh[b] * gm[b]));
        }
        __syncthreads();
    });
    if (dinit)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int j = 0; j < 4; ++j) dinit[(hd * DK + 16 * b + 4 * gq + j) * DV + col0 + m] = Sh[b][j];
}

// ------------------------------------------------------------------ 3. per-chunk gradients
// GW waves per (chunk slot, head), on the fp32 matrix cores.  Contracting over the dv
// columns in 16-column blocks cb, with the chunk's dO, Delta, E rows in the row layout
// (lane (g, m): row m, columns 16cb + 4g + j) and the checkpoint tiles read the same way
// (lane (g, n): state row 16b + n, the same columns), wave w forms, for its channel
// blocks b = w, w + GW, ...,
//     dO S0^T, Delta S^^T, E S0^T   (16 x 16 tiles)
// and its share of the four 16x16 Gram matrices
//     M1 = Delta dO^T, M4 = dO Delta^T = M1^T, M3 = E Delta^T, M3^T,
// which it passes to the others through LDS.  A 16x16 result held in the accumulator
// layout is the A operand of its transpose, which is why both of each pair are formed.
// Per channel block the triangular terms then come from 16-long products with K-, Q+, K+
// in the accumulator layout (lane (g, n): token 4g + j, channel 16b + n), built in
// registers from q, k, g.  dbeta_r uses
//     sum_col E (.) (K+ S0 + Ap Delta) = sum_ch K+ (.) (E S0^T) + sum_i Ap (.) M3   (row r),
// so U itself is never formed.  The sweeps store the checkpoints as row-major 16x16 tiles
// (tile (b, cb) of a dk x dv state, tile cb of a 16 x dv block), so each of these loads
// is 1 KiB contiguous.
// The log-decay gradient is dg_t = rowsum(dS_T (.) S_T) + sum_{s >= t} incr_s with
// incr_s = q_s (.) dq_s - k_s (.) (a_s + b_s).  Within the chunk this kernel sums the
// increments itself; the rest, everything after the chunk's last token tau, is exactly
// rowsum(S^ (.) S_tau): raising row c of S_tau by a factor is the same as raising the next
// token's decay of channel c, and S^ (the adjoint of S_tau through the later tokens) is the
// checkpoint this chunk reads.  With S_tau = Diag(e^{G_n}) S0 + K~^T Delta,
//     rowsum(S^ (.) S_tau) = e^{G_n} (.) rowsum(S^ (.) S0) + sum_r K~_r (.) (Delta S^^T)_r,
// both from quantities formed here anyway, so no sum runs over the whole sequence (whose
// fp32 rounding would grow with its length).
template <int N>
__device__ __forceinline__ float row_ror(float x) {  // lane m reads lane (m + N) mod 16 of its row
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 | N, 0xF, 0xF, false));
}

__device__ __forceinline__ float row_sum(float x) {  // the sum over the 16 lanes of the row, in every lane
    x += row_ror<1>(x);
    x += row_ror<2>(x);
    x += row_ror<4>(x);
    x += row_ror<8>(x);
    return x;
}

template <int DK>
struct GradShape {
    static constexpr int NB = DK / 16;
    static constexpr int GW = NB < 4 ? NB : 4;  // waves per (chunk, head)
    static constexpr int NBW = NB / GW;         // channel blocks per wave
};

template <int DK, int DV, typename T>
__global__ __launch_bounds__(64 * GradShape<DK>::GW) __attribute__((amdgpu_waves_per_eu(2, 8))) void bwd_grads_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ g,
    const T *__restrict__ beta, const float *__restrict__ dO, const int32_t *__restrict__ cu, int32_t nseq,
    int32_t H, const float *__restrict__ sck, const float *__restrict__ hck, const float *__restrict__ dbuf,
    const float *__restrict__ ebuf, const float *__restrict__ mats, float *__restrict__ dq, float *__restrict__ dk,
    float *__restrict__ dgs, float *__restrict__ dbeta) {
    constexpr int NCB = DV / 16, GW = GradShape<DK>::GW, NBW = GradShape<DK>::NBW;
    const int64_t item = blockIdx.x;
    const int64_t slot = item / H;
    const int h = (int)(item % H);
    const int wave = GW == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int lane = threadIdx.x % 64, gq = lane / 16, m = lane % 16;
    __shared__ __attribute__((aligned(16))) float Ms[4][256];  // M1, M4, M3, M3^T (accumulator layout)
    __shared__ float dbp[GW][16];
    const int s = seq_of_slot(cu, nseq, slot);
    const int64_t bos = cu[s], len = cu[s + 1] - bos;
    const int c = (int)(slot - slot_of(cu, s, 0));
    const int n = chunk_len(len, c);
    if (n == 0) return;  // a slot no chunk uses (uniform over the workgroup)
    const int64_t t0 = bos + 16 * (int64_t)c;
    const uint32_t ro = (uint32_t)(m * 16 + 4 * gq);  // this lane's place in a row-major tile
    const float *S0 = sck + item * DK * DV + ro, *Sh = hck + item * DK * DV + ro;
    const float *Dl = dbuf + item * 16 * DV + ro, *El = ebuf + item * 16 * DV + ro;
    const rsrc_t rO = chunk_rsrc(dO, t0, n, H, h, DV), rV = chunk_rsrc(v, t0, n, H, h, DV);

    struct Ops {
        f32x4 o, d, e, s0[NBW], sh[NBW];
        Row4Raw<T> vv;
    };
    auto load_ops = [&](Ops &x, int cb) {
        x.o = widen_row4<float>(load_row4_raw<float>(rO, m, H, DV, 16 * cb + 4 * gq));
        x.vv = load_row4_raw<T>(rV, m, H, DV, 16 * cb + 4 * gq);
        x.d = *reinterpret_cast<const f32x4 *>(Dl + cb * 256);
        x.e = *reinterpret_cast<const f32x4 *>(El + cb * 256);
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            const int b = wave + GW * i;
            x.s0[i] = *reinterpret_cast<const f32x4 *>(S0 + (b * NCB + cb) * 256);
            x.sh[i] = *reinterpret_cast<const f32x4 *>(Sh + (b * NCB + cb) * 256);
        }
    };
    // the epilogue's inputs, loaded now (raw words) so that their latency hides under the
    // contraction
    const rsrc_t rq = chunk_rsrc(q, t0, n, H, h, DK), rk = chunk_rsrc(k, t0, n, H, h, DK);
    const rsrc_t rg = chunk_rsrc(g, t0, n, H, h, DK), rb = chunk_rsrc(beta, t0, n, H, h, 1);
    u32x4 qraw[NBW], kraw[NBW], graw[NBW];
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
        const int ch = 16 * (wave + GW * i) + m;
        qraw[i] = load_col4_raw<T>(rq, gq, H, DK, ch);
        kraw[i] = load_col4_raw<T>(rk, gq, H, DK, ch);
        graw[i] = load_col4_raw<T>(rg, gq, H, DK, ch);
    }
    const u32x4 braw = load_col4_raw<T>(rb, gq, H, 1, 0);
    const float *ap = mats + (item * NMAT + MAT_AP) * 256;
    f32x4 apv;  // stril(K+ K-^T) at rows 4g + j, column m
#pragma unroll
    for (int j = 0; j < 4; ++j) apv[j] = ap[(4 * gq + j) * 16 + m];

    f32x4 QS[NBW], DS[NBW], ES[NBW];
#pragma unroll
    for (int i = 0; i < NBW; ++i) QS[i] = DS[i] = ES[i] = zero4();
    constexpr int NM = 4 / GW;  // Gram matrices per wave: wave w forms M_w, M_{w + GW}, ...
    f32x4 mm[NM];
#pragma unroll
    for (int t = 0; t < NM; ++t) mm[t] = zero4();
    float ev = 0.f;  // sum over this lane's columns of E (.) V, row m
    f32x4 SH[NBW];   // S0 S^^T of each channel block (its diagonal is rowsum(S^ (.) S0))
#pragma unroll
    for (int i = 0; i < NBW; ++i) SH[i] = zero4();
    auto step = [&](const Ops &x) {
#pragma unroll
        for (int t = 0; t < NM; ++t) {
            // M_0 = Delta dO^T, M_1 = dO Delta^T, M_2 = E Delta^T, M_3 = Delta E^T, chosen by
            // vector selects (with the wave index in a scalar register the compiler would
            // branch, splitting the unrolled loop into small blocks)
            const int id = (int)(threadIdx.x / 64) + GW * t;
            f32x4 a, b;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                a[j] = id == 1 ? x.o[j] : (id == 2 ? x.e[j] : x.d[j]);
                b[j] = id == 0 ? x.o[j] : (id == 3 ? x.e[j] : x.d[j]);
            }
            mm[t] = mma_f32_k16(a, b, mm[t]);
        }
        const f32x4 vv = widen_row4<T>(x.vv);
#pragma unroll
        for (int j = 0; j < 4; ++j) ev += x.e[j] * vv[j];
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            QS[i] = mma_f32_k16(x.o, x.s0[i], QS[i]);
            ES[i] = mma_f32_k16(x.e, x.s0[i], ES[i]);
            DS[i] = mma_f32_k16(x.d, x.sh[i], DS[i]);
            SH[i] = mma_f32_k16(x.s0[i], x.sh[i], SH[i]);
        }
    };
    // the column blocks fully unrolled over two operand sets: the loads of block cb + 1 are
    // in flight while block cb is used
    Ops buf[2];
    load_ops(buf[0], 0);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        if (cb + 1 < NCB) load_ops(buf[(cb + 1) % 2], cb + 1);
        step(buf[cb % 2]);
    }
#pragma unroll
    for (int t = 0; t < NM; ++t) *reinterpret_cast<f32x4 *>(&Ms[wave + GW * t][4 * lane]) = mm[t];
    __syncthreads();
    const f32x4 m1 = *reinterpret_cast<const f32x4 *>(&Ms[0][4 * lane]);
    const f32x4 m4 = *reinterpret_cast<const f32x4 *>(&Ms[1][4 * lane]);
    const f32x4 m3 = *reinterpret_cast<const f32x4 *>(&Ms[2][4 * lane]);
    const f32x4 m3t = *reinterpret_cast<const f32x4 *>(&Ms[3][4 * lane]);

    // A operands of the masked 16x16 factors (lane (g, m), slot j: row m, column 4g + j).
    const f32x4 br = widen_col4<T>(braw, gq, H, 1, 0);  // beta of tokens 4g + j
    f32x4 aq, aa1, aa2, ab;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = 4 * gq + j;
        aq[j] = col <= m ? m1[j] : 0.f;            // tril(M4)
        aa1[j] = col >= m ? m4[j] : 0.f;           // triu(M1)
        aa2[j] = col > m ? -br[j] * m3[j] : 0.f;   // -striu(M2), M2 = Delta dV^T = M3^T diag(beta)
        ab[j] = col < m ? m3t[j] : 0.f;            // stril(M3)
    }
    const rsrc_t rdq = chunk_rsrc(dq, t0, n, H, h, DK), rdk = chunk_rsrc(dk, t0, n, H, h, DK);
    const rsrc_t rin = chunk_rsrc(dgs, t0, n, H, h, DK);
    f32x4 kes = zero4();  // sum over channels of K+ (.) E S0^T, rows 4g + j
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
        const int ch = 16 * (wave + GW * i) + m;
        const f32x4 qv = widen_col4<T>(qraw[i], gq, H, DK, ch), kv = widen_col4<T>(kraw[i], gq, H, DK, ch);
        const f32x4 gv = widen_col4<T>(graw[i], gq, H, DK, ch);
        // e^{G} over the chunk's tokens: a running product within the lane, then across groups
        f32x4 P;
#pragma unroll
        for (int j = 0; j < 4; ++j) P[j] = expf(gv[j]);
#pragma unroll
        for (int j = 1; j < 4; ++j) P[j] *= P[j - 1];
        const float T0 = __shfl(P[3], m), T1 = __shfl(P[3], 16 + m), T2 = __shfl(P[3], 32 + m);
        const float before = gq == 0 ? 1.f : (gq == 1 ? T0 : (gq == 2 ? T0 * T1 : (T0 * T1) * T2));
        f32x4 ep, em, kp, km, qp;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ep[j] = before * P[j];
            em[j] = __builtin_amdgcn_rcpf(ep[j]);
            kp[j] = kv[j] * ep[j];
            km[j] = kv[j] * em[j];
            qp[j] = qv[j] * ep[j];
        }
        const float egn = __shfl(ep[3], 48 + m);  // e^{G_n} of channel ch
        const f32x4 tq = mma_f32_k16(aq, km, QS[i]);
        const f32x4 ta = mma_f32_k16(aa2, kp, mma_f32_k16(aa1, qp, DS[i] * egn));
        const f32x4 tb = mma_f32_k16(ab, km, ES[i]);
        f32x4 inc;
        float kd = 0.f;  // sum over this lane's tokens of K~ (.) Delta S^^T, channel ch
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float dqv = ep[j] * tq[j], av = em[j] * ta[j], bv = br[j] * ep[j] * tb[j];
            const uint32_t off = ((uint32_t)(4 * gq + j) * (uint32_t)H * DK + (uint32_t)ch) * 4u;
            buf_store_f32(dqv, rdq, off);
            buf_store_f32(av - bv, rdk, off);
            inc[j] = qv[j] * dqv - kv[j] * (av + bv);
            kes[j] += kp[j] * ES[i][j];
            kd += kv[j] * (egn * em[j]) * DS[i][j];
        }
        // everything after the chunk: e^{G_n} rowsum(S^ (.) S0) + sum_r K~ (.) Delta S^^T; the
        // diagonal entry of channel m sits in lane group m / 4, slot m % 4
        float dg0 = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) dg0 = 4 * gq + j == m ? SH[i][j] : dg0;
        const float s0sh = __shfl(dg0, 16 * (m / 4) + m);
        kd += __shfl_xor(kd, 16);
        kd += __shfl_xor(kd, 32);
        const float carry = egn * s0sh + kd;
        // reverse cumulative sum over the chunk's tokens: within the lane, then the later groups
#pragma unroll
        for (int j = 2; j >= 0; --j) inc[j] += inc[j + 1];
        const float U1 = __shfl(inc[0], 16 + m), U2 = __shfl(inc[0], 32 + m), U3 = __shfl(inc[0], 48 + m);
        const float after = gq == 3 ? 0.f : (gq == 2 ? U3 : (gq == 1 ? U3 + U2 : (U3 + U2) + U1));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            buf_store_f32((inc[j] + after) + carry, rin,
                          ((uint32_t)(4 * gq + j) * (uint32_t)H * DK + (uint32_t)ch) * 4u);
    }
    // dbeta_r = sum_col E V - sum_ch K+ (.) E S0^T - sum_i Ap (.) M3
    f32x4 red;
#pragma unroll
    for (int j = 0; j < 4; ++j) red[j] = row_sum(kes[j] + (wave == 0 ? apv[j] * m3[j] : 0.f));
    // row m's reduced term sits in lane group m / 4, slot m % 4
    const int src = 16 * (m / 4);
    const float r0 = __shfl(red[0], src), r1 = __shfl(red[1], src), r2 = __shfl(red[2], src);
    const float r3 = __shfl(red[3], src);
    const int jm = m % 4;
    const float rr = jm == 0 ? r0 : (jm == 1 ? r1 : (jm == 2 ? r2 : r3));
    ev += __shfl_xor(ev, 16);
    ev += __shfl_xor(ev, 32);
    if (gq == 0) dbp[wave][m] = (wave == 0 ? ev : 0.f) - rr;
    __syncthreads();
    if (wave == 0 && gq == 0) {
        float x = 0.f;
#pragma unroll
        for (int w = 0; w < GW; ++w) x += dbp[w][m];
        buf_store_f32(x, chunk_rsrc(dbeta, t0, n, H, h, 1), (uint32_t)m * (uint32_t)H * 4u);
    }
}

// ------------------------------------------------------------------ launch

// Column slices per workgroup of the sweeps: as few as fill the chip (each slice gets a
// SIMD to itself while there are fewer than about 256 workgroups), so the chunk's
// operands are built by several waves only where the grid is large anyway.
static int sweep_slices(int64_t chains, int nsl) {
    int ns = 1;
    while (ns < nsl && chains * (nsl / ns) > 256) ns *= 2;
    return ns;
}

template <int DK, int DV, int NS, typename T>
static hipError_t launch_sweeps(const BackwardArgs &a, const float *mats, float *sck, float *hck, float *dbuf,
                                float *ebuf, float *fin_only) {
    const hipStream_t st = (hipStream_t)a.stream;
    const unsigned grid = (unsigned)((int64_t)a.nseq * a.H * (DV / 16 / NS));
    const dim3 block(SweepShape<NS>::THREADS);
    hipLaunchKernelGGL((bwd_fwd_sweep_kernel<DK, DV, NS, T>), dim3(grid), block, 0, st, (const T *)a.k,
                       (const T *)a.v, (const T *)a.g, a.init, a.cu, a.H, mats, sck, dbuf, fin_only);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || fin_only) return e;
    hipLaunchKernelGGL((bwd_adjoint_sweep_kernel<DK, DV, NS, T>), dim3(grid), block, 0, st, (const T *)a.q,
                       (const T *)a.k, (const T *)a.g, (const T *)a.beta, a.dO, a.dfinal, a.cu, a.H, mats, hck, ebuf,
                       a.dv, a.dinit);
    return hipGetLastError();
}

// fin_only != NULL: only the chunk matrices and the forward sweep, which also writes the
// final states there (the boundary pass of a slabbed backward).
template <int DK, int DV, typename T>
static hipError_t launch_bwd_t(const BackwardArgs &a, float *fin_only = nullptr) {
    const int64_t slots = chunk_slots(a.N, a.nseq);
    const int64_t blk = slots * a.H * (int64_t)DK * DV;  // floats of one per-chunk state array
    float *sck = a.ws, *hck = sck + blk;
    float *dbuf = hck + blk, *ebuf = dbuf + slots * a.H * 16 * (int64_t)DV;
    float *mats = ebuf + slots * a.H * 16 * (int64_t)DV;
    const hipStream_t st = (hipStream_t)a.stream;
    hipError_t e = hipSuccess;
    const int64_t items = slots * a.H;
    if (a.N > 0) {
        hipLaunchKernelGGL((bwd_mats_kernel<DK, T>), dim3((unsigned)((items + MATS_WAVES - 1) / MATS_WAVES)),
                           dim3(64 * MATS_WAVES), 0, st, (const T *)a.q, (const T *)a.k, (const T *)a.g,
                           (const T *)a.beta, a.cu, a.nseq, a.H, items, mats);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    constexpr int NSL = DV / 16;
    switch (sweep_slices((int64_t)a.nseq * a.H, NSL)) {
    case 1: e = launch_sweeps<DK, DV, 1, T>(a, mats, sck, hck, dbuf, ebuf, fin_only); break;
    case 2: if constexpr (NSL >= 2) e = launch_sweeps<DK, DV, 2, T>(a, mats, sck, hck, dbuf, ebuf, fin_only); break;
    case 4: if constexpr (NSL >= 4) e = launch_sweeps<DK, DV, 4, T>(a, mats, sck, hck, dbuf, ebuf, fin_only); break;
    default: if constexpr (NSL >= 8) e = launch_sweeps<DK, DV, 8, T>(a, mats, sck, hck, dbuf, ebuf, fin_only); break;
    }
    if (e != hipSuccess || fin_only) return e;
    if (a.N > 0) {
        hipLaunchKernelGGL((bwd_grads_kernel<DK, DV, T>), dim3((unsigned)items), dim3(64 * GradShape<DK>::GW), 0, st,
                           (const T *)a.q, (const T *)a.k, (const T *)a.v, (const T *)a.g, (const T *)a.beta, a.dO,
                           a.cu, a.nseq, a.H, sck, hck, dbuf, ebuf, mats, a.dq, a.dk, a.dg, a.dbeta);
        e = hipGetLastError();
    }
    return e;
}

template <typename T>
static hipError_t launch_bwd_dt(const BackwardArgs &a, float *fin_only) {
#define KDA_BWD_CASE(DKV, DVV) \
    if (a.dk_ == DKV && a.dv_ == DVV) return launch_bwd_t<DKV, DVV, T>(a, fin_only);
#define KDA_BWD_ROW(DKV) KDA_BWD_CASE(DKV, 16) KDA_BWD_CASE(DKV, 32) KDA_BWD_CASE(DKV, 64) KDA_BWD_CASE(DKV, 128)
    KDA_BWD_ROW(16) KDA_BWD_ROW(32) KDA_BWD_ROW(64) KDA_BWD_ROW(128)
#undef KDA_BWD_ROW
#undef KDA_BWD_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_backward(const BackwardArgs &a) {
    return a.bf16 ? launch_bwd_dt<__bf16>(a, nullptr) : launch_bwd_dt<float>(a, nullptr);
}

hipError_t launch_backward_states(const BackwardArgs &a, float *fin) {
    return a.bf16 ? launch_bwd_dt<__bf16>(a, fin) : launch_bwd_dt<float>(a, fin);
}

// Per-slab sequence lists of a slabbed backward over one sequence of N tokens: slab s covers
// tokens [s L, min(N, (s+1) L)), and its list is {0, its length}.
__global__ void bwd_slab_cu_kernel(int32_t *cu, int64_t N, int64_t L, int32_t nslab) {
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= nslab) return;
    const int64_t a = (int64_t)s * L, b = a + L < N ? a + L : N;
    cu[2 * s] = 0;
    cu[2 * s + 1] = (int32_t)(b - a);
}

hipError_t launch_backward_slab_cu(int32_t *cu, int64_t N, int64_t L, int32_t nslab, void *stream) {
    hipLaunchKernelGGL(bwd_slab_cu_kernel, dim3((unsigned)((nslab + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, cu, N, L, nslab);
    return hipGetLastError();
}

int64_t backward_workspace_floats(int64_t N, int32_t nseq, int32_t H, int32_t dk, int32_t dv) {
    const int64_t slots = chunk_slots(N, nseq);
    // S and S^ checkpoints, Delta and E, chunk matrices
    return 2 * slots * H * (int64_t)dk * dv + 2 * slots * H * 16 * (int64_t)dv + slots * H * 4 * 256;
}

}  // namespace kda
