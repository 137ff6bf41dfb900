// Single-pass KDA prefill for bf16 inputs (gfx950): the chunk-local work and the
// inter-chunk recurrence in one kernel, so q, k, log-decay and beta are read from HBM
// once and nothing goes through a workspace.
//
// Chunked form (Kimi K3 report digest, "Kimi Delta Attention": the chunk output is the
// inter-chunk term (Gamma (.) Q) S plus an intra-chunk term A V~; bounded-decay section:
// with g >= -5 the 16-token cumulative decay stays in [-80, 0], so the decayed key/query
// blocks are dense products in fp32/bf16 range).  Per 16-token chunk, with G the
// inclusive cumulative log-decay per key channel:
//     K+ = K (.) e^{G},  K- = K (.) e^{-G},  Q+ = Q (.) e^{G},  K~ = K (.) e^{G_n - G}
//     A    = diag(beta) strictly_lower(K+ K-^T),     T = (I + A)^-1,   T' = T diag(beta)
//     Aqk  = lower_incl_diag(Q+ K-^T)
//     Delta = T' (V - K+ S),   O = Q+ S + Aqk Delta,   S <- Diag(e^{G_n}) S + K~^T Delta
//
// A workgroup serves one (sequence, head) and NC*SL 16-column slices of dv, with two
// kinds of waves (the overlap of the token-parallel and the serial work that the
// digest's "chunkwise kernel" paragraph describes, laid out for 64-lane wavefronts):
//   * NC consumer waves keep SL fp32 state slices (128 x 16 each) in registers and
//     advance them chunk by chunk on the matrix cores (the serial part);
//   * NP = 4 producer waves build everything that does not depend on the state, three
//     chunks ahead: per chunk they stage q, k, g through LDS, form G (0/1-triangle
//     products on the matrix cores), e^{+-G}, Q+, K+, K~, Gamma and, over their own key
//     channels, partial sums of A, A^T and Aqk^T; one producer per chunk (in turn) then
//     adds the partials and inverts I + A as the product (I - B)(I + B^2)(I + B^4)(I + B^8)
//     (B = A^T is strictly upper triangular, so B^16 = 0) on the matrix cores, in two
//     halves over two intervals (the solve is a chain of dependent products; done whole
//     beside a build it made that wave the last at every barrier).
// One barrier per chunk.  In interval c the consumers advance chunk c (operand set c % 4),
// producer (c + 1) % 4 finishes the solve of chunk c + 1 (T' and Aqk into set (c + 1) % 4),
// producer (c + 2) % 4 begins that of chunk c + 2 (partials from buffer c % 2) and the
// producers build chunk c + 3 (set (c + 3) % 4, partials into buffer (c + 1) % 2).
//
// Precision (as in the two-kernel path): every product split bf16 (hi*hi + lo*hi + hi*lo,
// and lo*lo where it is free) with fp32 accumulation; the products of the inverse use both
// halves of both factors.  State and output fp32.  (K+ S and A in single bf16 were enough
// for mild decay, not for a gate at its -5 floor with heavy-tailed values.)
//
// Layout conventions and the key-channel relabelling inside block pairs are those of the
// warp-specialised inter-chunk kernel: internal channel 16 (2P + h) + 4 g4 + j is memory
// channel 32 P + 8 g4 + 4 h + j, so one lane's part of a block pair is one 16-byte piece.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

// Waves of a workgroup: wave w and wave w + 4 share a SIMD.  With one or two consumers
// the slots that would share a SIMD with a consumer hold idle waves (barriers only).
template <int NC, int NP>
struct FusedLayout {
    static constexpr int NIDLE = (NC + NP > 4 && NC <= 2) ? NC : 0;
    static constexpr int NW = NC + NP + NIDLE;
    // consumer index (>= 0), producer index - NP (in [-NP, 0)), or -NP - 1 (idle)
    static __device__ __forceinline__ int role(int w) {
        if (w < NC) return w;
        if (w < 4 || NIDLE == 0) return w - NC - NP;
        if (w < 4 + NIDLE) return -NP - 1;
        return w - NC - NIDLE - NP;
    }
};

template <int DK>
struct FusedOps {
    static constexpr int NB = DK / 16, NPAIR = NB / 2;
    bf16x8 qp_hi[NPAIR][64];  // Q+ A-operand fragments, block pairs packed
    bf16x8 qp_lo[NPAIR][64];
    bf16x8 kp[NPAIR][64];     // K+ as hi + lo
    bf16x8 kp_lo[NPAIR][64];
    Split4 kt[NB][64];        // K~^T (channel rows, 4 tokens per lane), {hi, lo}
    Split4 tp[64];            // T' as the A operand of Delta = T' Y: lane (g4, m) holds T'[m][4 g4 + j]
    Split4 aq[64];            // Aqk as the A operand of Aqk Delta
    float gam[DK];            // e^{G_n} per (internal) channel
    float beta[16];           // beta of the chunk's tokens (0 past a ragged end)
};

// x = hi + lo split of a tile held in the accumulator layout.
struct SplitT {
    bf16x4 hi, lo;
};

}  // namespace

template <int DK, int DV, int NC, int SL>
__global__ __launch_bounds__((64 * FusedLayout<NC, 4>::NW)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_fused_kernel(const __bf16 *__restrict__ q, const __bf16 *__restrict__ k,
                          const __bf16 *__restrict__ v, const __bf16 *__restrict__ g,
                          const __bf16 *__restrict__ beta, const float *__restrict__ init,
                          const int32_t *__restrict__ cu, int32_t H, float *__restrict__ o,
                          float *__restrict__ fin, int32_t nsplit, int32_t nchains, int32_t nsort) {
    constexpr int NP = 4;
    constexpr int NSETS = 4;  // operand sets: chunks c .. c + 3 are in flight in interval c
    constexpr int NB = DK / 16, NPAIR = NB / 2, BPW = NB / NP;
    constexpr uint32_t EB = 2;
    static_assert(DK == 128, "the fused kernel is built for 128 key channels (one block pair per producer)");
    static_assert(BPW == 2, "one block pair per producer");
    static_assert(DV % (16 * NC * SL) == 0, "column slices");
    using Layout = FusedLayout<NC, NP>;

    // XCD-aware order: all column groups of one chain share an XCD (blockIdx mod 8);
    // the chains in dispatch order go longest first.
    const int L = blockIdx.x;
    const int xcd = L & 7;
    const int sx = L >> 3;
    const int split = sx % nsplit;
    const int slot = (sx / nsplit) * 8 + xcd;
    if (slot >= nchains) return;
    const int chain = lpt_chain(cu, nsort, H, slot);
    const int s = chain / H, h = chain % H;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int role = Layout::role(tid >> 6);
    const int g4 = lane >> 4, l16 = lane & 15;

    __shared__ __attribute__((aligned(16))) FusedOps<DK> ops[NSETS];
    // partial sums per producer: A, A^T, Aqk^T in the accumulator layout
    __shared__ __attribute__((aligned(16))) f32x4 part[2][NP][3][64];

    const int64_t bos = cu[s], eos = cu[s + 1];
    const int nc = (int)((eos - bos + 15) / 16);
    const int64_t hd = (int64_t)s * H + h;
    const uint32_t rowK = (uint32_t)H * DK * EB;   // bytes between tokens in q, k, g
    const uint32_t rowV = (uint32_t)H * DV * EB;   // ... in v
    const uint32_t rowO = (uint32_t)H * DV * 4;    // ... in o
    const int len = (int)(eos - bos);
    // Rows of chunk c (0 past the end); readfirstlane keeps it scalar so the buffer
    // resources built from it stay uniform.
    auto chunk_len = [&](int c) -> int {
        const int left = len - 16 * c;
        return __builtin_amdgcn_readfirstlane(left <= 0 ? 0 : (left < 16 ? left : 16));
    };
    auto rsrc_in = [&](const __bf16 *base, int c, int d) {
        const int64_t t0 = bos + 16 * (int64_t)c;
        return make_rsrc(base + (t0 * H + h) * d, (uint32_t)chunk_len(c) * (uint32_t)H * d * EB);
    };
    auto rsrc_beta = [&](int c) {
        const int64_t t0 = bos + 16 * (int64_t)c;
        return make_rsrc(beta + t0 * H + h, (uint32_t)chunk_len(c) * (uint32_t)H * EB);
    };
    auto rsrc_out = [&](int c) {
        const int64_t t0 = bos + 16 * (int64_t)c;
        return make_rsrc(o + (t0 * H + h) * DV, (uint32_t)chunk_len(c) * rowO);
    };

    if (role == -NP - 1) {
        // idle wave: the same barriers as the others (two before the chunk loop)
        if (nc > 0)
            for (int c = 0; c < nc + 3; ++c) __syncthreads();
    } else if (role >= 0) {
        // ============================================================ consumer
        const int wave = role;
        // State slices: internal rows 16 b + 4 g4 + jj, column col0 + l16; internal row
        // 16 b + 4 g4 + jj is memory key channel mrow(b, jj).
        int col0[SL];
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) col0[sl] = ((split * NC + wave) * SL + sl) * 16;
        auto mrow = [&](int b, int jj) { return 32 * (b >> 1) + 8 * g4 + 4 * (b & 1) + jj; };
        const rsrc_t rinit = make_rsrc(init ? init + hd * DK * DV : init, init ? DK * DV * 4u : 0u);
        f32x4 S[SL][NB];
#pragma unroll
        for (int sl = 0; sl < SL; ++sl)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    S[sl][b][jj] = __builtin_bit_cast(
                        float, buf_load_u32(rinit, (mrow(b, jj) * DV + col0[sl] + l16) * 4u));

        if (nc > 0) {
            // v of token l16, columns col0 + 4 g4 .. +3 of each slice (the identity product
            // below turns it into the state's layout), loaded three chunks ahead
            struct CIn {
                u32x2 v[SL];
            };
            const bf16x4 ID = identity_operand(g4, l16);
            const bf16x8 NIL = neg_identity_operand<0>(g4, l16), NIH = neg_identity_operand<1>(g4, l16);
            auto cload = [&](CIn &X, int c) {
                const rsrc_t rv = rsrc_in(v, c, DV);
#pragma unroll
                for (int sl = 0; sl < SL; ++sl)
                    X.v[sl] = buf_load_u32x2(rv, l16 * rowV + (col0[sl] + 4 * g4) * EB);
            };
            auto advance = [&](const FusedOps<DK> &P, const CIn &X, int c) {
                // K+ (hi, lo) read first, so its LDS latency overlaps the state split
                bf16x8 kpa[NPAIR], kla[NPAIR];
#pragma unroll
                for (int p = 0; p < NPAIR; ++p) {
                    kpa[p] = P.kp[p][lane];
                    kla[p] = P.kp_lo[p][lane];
                }
                const Split4 Tp = P.tp[lane];
                const Split4 Aq = P.aq[lane];
                __builtin_amdgcn_sched_barrier(0);
                const bf16x8 tpp = cat(Tp.hi, Tp.lo);
                // Per block pair and slice: the state's bf16 split, then every product that
                // reads it (X = K+ S and Q+ S, each as hi*hi, lo*hi, hi*lo), so a split lives
                // only briefly and the slices' independent chains interleave.
                f32x4 Xa[SL], Xb[SL], Oa[SL], Ob[SL], Oc[SL];
#pragma unroll
                for (int sl = 0; sl < SL; ++sl) Xa[sl] = Xb[sl] = Oa[sl] = Ob[sl] = Oc[sl] = zero4();
#pragma unroll
                for (int p = 0; p < NPAIR; ++p) {
                    const bf16x8 kpr = kpa[p], kplr = kla[p];
                    const bf16x8 qhr = P.qp_hi[p][lane], qlr = P.qp_lo[p][lane];
#pragma unroll
                    for (int sl = 0; sl < SL; ++sl) {
                        const bf16x8 Shi = cat(to_bf16x4(S[sl][2 * p]), to_bf16x4(S[sl][2 * p + 1]));
                        const bf16x8 Slo = cat(to_bf16x4(mma32(NIL, Shi, S[sl][2 * p])),
                                               to_bf16x4(mma32(NIH, Shi, S[sl][2 * p + 1])));
                        Xa[sl] = mma32(kpr, Shi, Xa[sl]);
                        Xb[sl] = mma32(kplr, Shi, Xb[sl]);
                        Xb[sl] = mma32(kpr, Slo, Xb[sl]);
                        Oa[sl] = mma32(qhr, Shi, Oa[sl]);
                        Ob[sl] = mma32(qlr, Shi, Ob[sl]);
                        Oc[sl] = mma32(qhr, Slo, Oc[sl]);
                    }
                }
                // Diag(Gamma) S now: it does not depend on Delta and fills the Delta chain's gaps
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const f32x4 gm = *reinterpret_cast<const f32x4 *>(&P.gam[16 * b + 4 * g4]);
#pragma unroll
                    for (int sl = 0; sl < SL; ++sl) S[sl][b] *= gm;
                }
                // Delta = T' (V - X), per slice
                f32x4 Op[SL];
                bf16x8 dhh[SL], dll[SL];
#pragma unroll
                for (int sl = 0; sl < SL; ++sl) {
                    const f32x4 vc = mma16(__builtin_bit_cast(bf16x4, X.v[sl]), ID, zero4());
                    bf16x8 yhh;
                    const bf16x4 ylo = split_lo(vc - (Xa[sl] + Xb[sl]), NIL, yhh);
                    f32x4 D = mma32(tpp, yhh, zero4());
                    D = mma32(tpp, cat(ylo, ylo), D);
                    const bf16x4 dlo = split_lo(D, NIL, dhh[sl]);
                    dll[sl] = cat(dlo, dlo);
                    Op[sl] = Oa[sl] + (Ob[sl] + Oc[sl]);
                }
                // S <- (Diag(Gamma) S, formed above) + K~^T Delta, one key block at a time for every slice
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const Split4 kt = P.kt[b][lane];
                    const bf16x8 ktt = cat(kt.hi, kt.lo);
#pragma unroll
                    for (int sl = 0; sl < SL; ++sl) {
                        const f32x4 acc = mma32(ktt, dhh[sl], S[sl][b]);
                        S[sl][b] = mma32(ktt, dll[sl], acc);
                    }
                }
                // O = Q+ S + Aqk Delta
                const bf16x8 aqq = cat(Aq.hi, Aq.lo);
                const rsrc_t ro = rsrc_out(c);
#pragma unroll
                for (int sl = 0; sl < SL; ++sl) {
                    f32x4 O = mma32(aqq, dhh[sl], Op[sl]);
                    O = mma32(aqq, dll[sl], O);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        buf_store_f32(O[jj], ro, (4 * g4 + jj) * rowO + (col0[sl] + l16) * 4u);
                }
            };

            CIn X0, X1, X2;
            cload(X0, 0);
            cload(X1, 1);
            cload(X2, 2);
            __syncthreads();  // chunk 0 built (partials)
            __syncthreads();  // chunk 0 complete (T', Aqk); chunk 1 built
            __syncthreads();  // chunk 1 half solved; chunk 2 built
            // Everything loaded so far (state, first inputs) has arrived before the loop: the
            // wait-count pass otherwise merges these loads, issued with few others after them,
            // into the loop header and makes the first chunks of every unrolled trip wait for
            // the loads and stores of the chunk just before.
            __builtin_amdgcn_s_waitcnt(0);
            auto citer = [&](int c, CIn &X) {
                advance(ops[c & (NSETS - 1)], X, c);
                cload(X, c + 3);
                __syncthreads();
            };
            // whole groups of three in the loop, the remainder after it (an exit inside the
            // body made the compiler wait for every load in flight at the loop head)
            int c = 0;
            for (; c + 3 <= nc; c += 3) {
                citer(c, X0);
                citer(c + 1, X1);
                citer(c + 2, X2);
            }
            if (c < nc) citer(c, X0);
            if (c + 1 < nc) citer(c + 1, X1);
        }
        if (fin) {
#pragma unroll
            for (int sl = 0; sl < SL; ++sl)
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        fin[(hd * DK + mrow(b, jj)) * DV + col0[sl] + l16] = S[sl][b][jj];
        }
    } else if (nc > 0) {
        // ============================================================ producer
        const int pw = role + NP;  // channel blocks 2 pw, 2 pw + 1 (block pair pw)
        // 0/1 triangles: LT (B of G^T = g^T L^T): lane (g4, n) holds [4 g4 + j <= n];
        // UT (A of Gs = U g): lane (g4, i) holds [4 g4 + j > i]
        u16x4 lt_bits, ut_bits;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lt_bits[j] = (4 * g4 + j <= l16) ? 0x3f80 : 0;
            ut_bits[j] = (4 * g4 + j > l16) ? 0x3f80 : 0;
        }
        const bf16x4 LT = __builtin_bit_cast(bf16x4, lt_bits);
        const bf16x4 UT = __builtin_bit_cast(bf16x4, ut_bits);
        const bf16x4 ID = identity_operand(g4, l16);
        const bf16x4 z4 = {};
        const bf16x8 IDL = cat(ID, z4), IDH = cat(z4, ID), LTL = cat(LT, z4), LTH = cat(z4, LT);
        const bf16x8 UTL = cat(UT, z4), UTH = cat(z4, UT);
        const bf16x8 NIL = neg_identity_operand<0>(g4, l16), NIH = neg_identity_operand<1>(g4, l16);

        // Raw q, k, g of a chunk: whole 64-byte row pieces of block pair pw with four
        // consecutive lanes per token row, and beta of token l16.
        struct PIn {
            u32x4 d[3];
            uint32_t b;
        };
        auto pload = [&](PIn &R, int c) {
            const rsrc_t rq = rsrc_in(q, c, DK), rk = rsrc_in(k, c, DK), rg = rsrc_in(g, c, DK);
            const uint32_t off = (lane >> 2) * rowK + 64u * pw + 16u * (lane & 3);
            R.d[0] = buf_load_u32x4(rq, off);
            R.d[1] = buf_load_u32x4(rk, off);
            R.d[2] = buf_load_u32x4(rg, off);
            R.b = buf_load_u16(rsrc_beta(c), (uint32_t)l16 * (uint32_t)H * EB);
        };
        // Per-wave stage: 16 token rows of 64 bytes per tensor, rows padded to 80 bytes so
        // the operand-layout reads hit distinct banks.
        __shared__ __attribute__((aligned(16))) u32x4 stage[NP][3][16][5];
        struct AIn {
            u32x4 d[3];
            float b;
        };
        auto stage_put = [&](const PIn &R) {
#pragma unroll
            for (int t = 0; t < 3; ++t) stage[pw][t][lane >> 2][lane & 3] = R.d[t];
        };
        auto stage_get = [&](AIn &A, const PIn &R) {
#pragma unroll
            for (int t = 0; t < 3; ++t) A.d[t] = stage[pw][t][l16][g4];
            A.b = bf16_bits_to_f32((uint16_t)R.b);
        };
        auto half = [](const u32x4 &x, int hh) { return hh ? u32x2{x[2], x[3]} : u32x2{x[0], x[1]}; };

        // Build the state-independent operands of a chunk into operand set P and this
        // wave's partial sums of A, A^T and Aqk^T into pp.
        auto build = [&](const AIn &A, FusedOps<DK> &P, f32x4 (&pp)[3][64]) {
            const int b0 = 2 * pw, b1 = b0 + 1;
            const u32x2 Rq[2] = {half(A.d[0], 0), half(A.d[0], 1)};
            const u32x2 Rk[2] = {half(A.d[1], 0), half(A.d[1], 1)};
            const bf16x8 ga = __builtin_bit_cast(bf16x8, A.d[2]);
            const bf16x8 ka = __builtin_bit_cast(bf16x8, A.d[1]);
            // g and k as tokens 4 g4 + jj of channel 16 b + l16 (exact: bf16 values)
            const bf16x8 gf = cat(to_bf16x4(mma32(ga, IDL, zero4())), to_bf16x4(mma32(ga, IDH, zero4())));
            const f32x4 kc[2] = {mma32(ka, IDL, zero4()), mma32(ka, IDH, zero4())};
            // G at token l16, channels 16 b + 4 g4 + jj; Gs at tokens 4 g4 + jj, channel 16 b + l16
            const f32x4 GT[2] = {mma32(gf, LTL, zero4()), mma32(gf, LTH, zero4())};
            const f32x4 GS[2] = {mma32(UTL, gf, zero4()), mma32(UTH, gf, zero4())};
            f32x4 Pp[2], Pm[2], qv[2], ktv[2], kmv[2], kpv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                f32x4 F;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    Pp[u][j] = decay_exp_fast(GT[u][j]);    // e^{G_r}
                    Pm[u][j] = decay_exp_fast(-GT[u][j]);   // e^{-G_r}
                    F[j] = decay_exp_fast(GS[u][j]);        // e^{G_n - G_r}
                }
                const f32x4 kk = unpack_bf16x4(Rk[u]);
                qv[u] = unpack_bf16x4(Rq[u]) * Pp[u];
                kpv[u] = kk * Pp[u];
                kmv[u] = kk * Pm[u];
                ktv[u] = kc[u] * F;
            }
            // Q+, K+, K~ and K- as hi + lo (residuals from the matrix core)
            const bf16x8 qh = cat(to_bf16x4(qv[0]), to_bf16x4(qv[1]));
            const bf16x8 kth = cat(to_bf16x4(ktv[0]), to_bf16x4(ktv[1]));
            const bf16x8 kmh = cat(to_bf16x4(kmv[0]), to_bf16x4(kmv[1]));
            const bf16x8 kpp = cat(to_bf16x4(kpv[0]), to_bf16x4(kpv[1]));
            const bf16x8 ql = cat(to_bf16x4(mma32(NIL, qh, qv[0])), to_bf16x4(mma32(NIH, qh, qv[1])));
            const bf16x4 ktl[2] = {to_bf16x4(mma32(NIL, kth, ktv[0])), to_bf16x4(mma32(NIH, kth, ktv[1]))};
            const bf16x8 kml = cat(to_bf16x4(mma32(NIL, kmh, kmv[0])), to_bf16x4(mma32(NIH, kmh, kmv[1])));
            const bf16x8 kpl = cat(to_bf16x4(mma32(NIL, kpp, kpv[0])), to_bf16x4(mma32(NIH, kpp, kpv[1])));
            P.qp_hi[pw][lane] = qh;
            P.qp_lo[pw][lane] = ql;
            P.kp[pw][lane] = kpp;
            P.kp_lo[pw][lane] = kpl;
            P.kt[b0][lane] = Split4{__builtin_shufflevector(kth, kth, 0, 1, 2, 3), ktl[0]};
            P.kt[b1][lane] = Split4{__builtin_shufflevector(kth, kth, 4, 5, 6, 7), ktl[1]};
            if (l16 == 15) {
                *reinterpret_cast<f32x4 *>(&P.gam[16 * b0 + 4 * g4]) = Pp[0];
                *reinterpret_cast<f32x4 *>(&P.gam[16 * b1 + 4 * g4]) = Pp[1];
            }
            if (pw == 0 && lane < 16) P.beta[lane] = A.b;
            // partial sums over this wave's 32 key channels (split bf16, hi*hi + lo*hi + hi*lo):
            // A = K+ K-^T, A^T = K- K+^T, Aqk^T = K- Q+^T, all in the accumulator layout
            f32x4 at = mma32(kpp, kmh, zero4());
            at = mma32(kpl, kmh, at);
            pp[0][lane] = mma32(kpp, kml, at);
            f32x4 bt = mma32(kmh, kpp, zero4());
            bt = mma32(kml, kpp, bt);
            pp[1][lane] = mma32(kmh, kpl, bt);
            f32x4 aqt = mma32(kmh, qh, zero4());
            aqt = mma32(kml, qh, aqt);
            pp[2][lane] = mma32(kmh, ql, aqt);
        };

        // Complete a chunk: add the partials, apply beta and the triangular masks, invert
        // I + A and write T' and Aqk as A-operand fragments (split bf16) into P.
        auto splitT = [&](const f32x4 &x) {
            bf16x8 hh;
            const bf16x4 lo = split_lo(x, NIL, hh);
            return SplitT{__builtin_shufflevector(hh, hh, 0, 1, 2, 3), lo};
        };
        // X Y for X, Y given by the splits of the accumulator layouts of X^T (left) and Y
        // (right); all four half products, fp32 accumulation onto c.
        auto prod = [&](const SplitT &xt, const SplitT &y, f32x4 c) {
            const bf16x8 a = cat(xt.hi, xt.lo);
            c = mma32(a, cat(y.hi, y.hi), c);
            return mma32(a, cat(y.lo, y.lo), c);
        };
        // The solve in two halves, run in consecutive intervals by the same wave: the first
        // adds the partials and forms B^2, B^4 and (I - B)(I + B^2); the second finishes the
        // product and writes T' and Aqk.
        struct SolveMid {
            f32x4 A4, B4, R1, Qm, brow;
        };
        auto solve1 = [&](const FusedOps<DK> &P, const f32x4 (&pp)[NP][3][64]) {
            f32x4 Am = pp[0][0][lane], Bm = pp[0][1][lane], Qm = pp[0][2][lane];
#pragma unroll
            for (int w = 1; w < NP; ++w) {
                Am += pp[w][0][lane];
                Bm += pp[w][1][lane];
                Qm += pp[w][2][lane];
            }
            const f32x4 brow = *reinterpret_cast<const f32x4 *>(&P.beta[4 * g4]);  // beta of rows 4 g4 + j
            const float bcol = P.beta[l16];                                       // beta of column l16
            f32x4 R0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * g4 + j;
                Am[j] = (r > l16) ? Am[j] * brow[j] : 0.f;   // A   = diag(beta) strictly_lower
                Bm[j] = (l16 > r) ? Bm[j] * bcol : 0.f;      // A^T
                Qm[j] = (l16 >= r) ? Qm[j] : 0.f;            // Aqk^T (lower incl. diagonal of Aqk)
                R0[j] = (r == l16 ? 1.f : 0.f) - Bm[j];      // I - B, B = A^T
            }
            const SplitT sA = splitT(Am), sB = splitT(Bm);
            // powers: A^2 = A A (left A: accumulator layout of A^T = B), B^2 = B B, ...
            const f32x4 A2 = prod(sB, sA, zero4()), B2 = prod(sA, sB, zero4());
            const SplitT sA2 = splitT(A2), sB2 = splitT(B2), sR0 = splitT(R0);
            SolveMid m;
            m.A4 = prod(sB2, sA2, zero4());
            m.B4 = prod(sA2, sB2, zero4());
            // T^T = (I + B)^-1 = (I - B)(I + B^2)(I + B^4)(I + B^8): R <- R + B^(2^k) R, the left
            // factor B^(2^k) given by the accumulator layout of its transpose A^(2^k)
            m.R1 = prod(sA2, sR0, R0);
            m.Qm = Qm;
            m.brow = brow;
            return m;
        };
        auto solve2 = [&](FusedOps<DK> &P, const SolveMid &m) {
            const SplitT sA4 = splitT(m.A4), sB4 = splitT(m.B4), sR1 = splitT(m.R1);
            const f32x4 A8 = prod(sB4, sA4, zero4());
            const f32x4 R2 = prod(sA4, sR1, m.R1);
            const SplitT sA8 = splitT(A8), sR2 = splitT(R2);
            f32x4 Tt = prod(sA8, sR2, R2);
            // T'^T = diag(beta) T^T: the accumulator layout of T'^T is the A operand of T'
            Tt *= m.brow;
            const SplitT st = splitT(Tt), sq = splitT(m.Qm);
            P.tp[lane] = Split4{st.hi, st.lo};
            P.aq[lane] = Split4{sq.hi, sq.lo};
        };

        // Interval c: the wave pw == (c + 1) % NP finishes the solve of chunk c + 1 (begun in
        // interval c - 1), the wave pw == (c + 2) % NP begins that of chunk c + 2, and every
        // producer builds its part of chunk c + 3 (staged in the interval before), stages
        // chunk c + 4 and loads chunk c + 7; register sets rotate R1 -> R2 -> R0.  Priority
        // goes to the solve, whose chain the consumers wait for at the next barrier.
        PIn R0, R1, R2;
        AIn A;
        SolveMid mid;
        pload(R0, 0);
        pload(R1, 1);
        pload(R2, 2);
        stage_put(R0);
        stage_get(A, R0);  // (the wave's own LDS accesses stay in order)
        pload(R0, 3);
        build(A, ops[0], part[0][pw]);
        stage_put(R1);
        stage_get(A, R1);
        pload(R1, 4);
        __syncthreads();  // partials of chunk 0 complete
        if (pw == 0) solve2(ops[0], solve1(ops[0], part[0]));
        build(A, ops[1], part[1][pw]);
        stage_put(R2);
        stage_get(A, R2);
        pload(R2, 5);
        __syncthreads();  // chunk 0 complete; partials of chunk 1 complete
        if (pw == 1) mid = solve1(ops[1], part[1]);
        build(A, ops[2], part[0][pw]);
        stage_put(R0);
        stage_get(A, R0);
        pload(R0, 6);
        __syncthreads();  // chunk 1 half solved, chunk 2 built
        __builtin_amdgcn_s_waitcnt(0);  // (as for the consumers: no merged waits in the loop)
        auto piter = [&](int c, PIn &R) {
            if (pw == (c + 1) % NP) {
                __builtin_amdgcn_s_setprio(3);
                solve2(ops[(c + 1) & (NSETS - 1)], mid);
                __builtin_amdgcn_s_setprio(0);
            }
            if (pw == (c + 2) % NP) {
                __builtin_amdgcn_s_setprio(3);
                mid = solve1(ops[(c + 2) & (NSETS - 1)], part[c & 1]);
                __builtin_amdgcn_s_setprio(0);
            }
            build(A, ops[(c + 3) & (NSETS - 1)], part[(c + 1) & 1][pw]);
            stage_put(R);
            stage_get(A, R);
            pload(R, c + 7);
            __syncthreads();
        };
        int c = 0;
        for (; c + 3 <= nc; c += 3) {
            piter(c, R1);
            piter(c + 1, R2);
            piter(c + 2, R0);
        }
        if (c < nc) piter(c, R1);
        if (c + 1 < nc) piter(c + 1, R2);
    }
}

template <int DK, int DV, int NC, int SL>
static hipError_t launch_fused_t(const PrefillFusedArgs &a) {
    const int nchains = a.nseq * a.H;
    const int nsplit = DV / (16 * NC * SL);
    const int64_t grid = ((int64_t)nchains + 7) / 8 * 8 * nsplit;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((prefill_fused_kernel<DK, DV, NC, SL>), dim3((unsigned)grid),
                       dim3(64 * FusedLayout<NC, 4>::NW), 0, (hipStream_t)a.stream, (const __bf16 *)a.q,
                       (const __bf16 *)a.k, (const __bf16 *)a.v, (const __bf16 *)a.g, (const __bf16 *)a.beta,
                       a.init, a.cu, a.H, a.o, a.fin, nsplit, nchains, a.nseq <= LPT_MAX_SEQS ? a.nseq : 0);
    return hipGetLastError();
}

// The single-pass kernel serves bf16 inputs with dk = dv = 128 when the (sequence, head) chains
// fill the chip with one workgroup each; with fewer chains the two-kernel path (whose producers
// carry no chunk-local work) keeps the serial step shorter.
bool prefill_fused_supported(int dk, int dv, bool bf16, int64_t chains) {
    return bf16 && dk == 128 && dv == 128 && chains >= 256;
}

// Shape: consumers per workgroup and 16-column slices per consumer; (0, 0) chooses from the
// number of (sequence, head) chains: one workgroup per chain (four consumers of two slices)
// when the chains fill the chip, else column groups spread over more workgroups.
bool prefill_fused_shape_built(int nc, int sl) {
    return (nc == 0 && sl == 0) || (nc == 4 && (sl == 1 || sl == 2)) || (nc == 2 && sl == 1);
}

hipError_t launch_prefill_fused(const PrefillFusedArgs &a, int nc, int sl) {
    const int64_t chains = (int64_t)a.nseq * a.H;
    if (!(a.bf16 && a.dk == 128 && a.dv == 128)) return hipErrorInvalidValue;
    if (nc == 0) {
        if (chains >= 256) {
            nc = 4;
            sl = 2;
        } else if (chains >= 64) {
            nc = 4;
            sl = 1;
        } else {
            nc = 2;
            sl = 1;
        }
    }
    if (nc == 4 && sl == 2) return launch_fused_t<128, 128, 4, 2>(a);
    if (nc == 4 && sl == 1) return launch_fused_t<128, 128, 4, 1>(a);
    if (nc == 2 && sl == 1) return launch_fused_t<128, 128, 2, 1>(a);
    return hipErrorInvalidValue;
}

}  // namespace kda
