// Decode windows as one chunk on the matrix cores (bf16 inputs, dk = dv = 128).
//
// A window of at most 16 tokens per (sequence, head) -- its drafts and, with a
// replay, the previous window's accepted prefix in front of them -- is one chunk
// of the chunked form (Kimi K3 report digest, "Kimi Delta Attention": the chunk
// output is the inter-chunk term (Gamma (.) Q) S plus an intra-chunk term; serving
// section: verification windows and the replay of accepted drafts).  With G the
// inclusive cumulative log-decay per key channel over the chunk's tokens and a the
// number of tokens whose state is committed:
//     K+ = K (.) e^{G},  K- = K (.) e^{-G},  Q+ = Q (.) e^{G}
//     A = diag(beta) strictly_lower(K+ K-^T),  T' = (I + A)^-1 diag(beta)
//     Aqk = lower_incl_diag(Q+ K-^T)
//     Delta = T' (V - K+ S),   O = Q+ S + Aqk Delta                    (every token)
//     S_a = Diag(e^{G_{a-1}}) S + K~_a^T Delta,   K~_a[r] = k_r (.) e^{G_{a-1} - G_r}, r < a
// The per-token window kernel (decode.hip) carries the state through the window
// on the vector ALUs, four multiply-adds per state element and token, which beyond
// a few tokens sets its time rather than HBM.  Here the state is read once,
// multiplied on the matrix cores as in the prefill (split bf16 operands, fp32
// accumulation) and written once, so the arithmetic per state element does not
// grow with the window and the state's HBM traffic stays the bound.
//
// Rows of the chunk past a head's tokens read as zeros (k = 0, g = 0, beta = 0),
// which leaves every product of the real rows unchanged.  A and T are lower
// triangular and K~_a is zero from row a on, so the entries that reach S_a are
// the ones a chunk of only the first a tokens would hold, with the other entries
// exact zeros: the committed state is the same, bit for bit, as this kernel gives
// for the accepted prefix alone, whatever drafts follow it.
//
// A workgroup of four waves serves one (sequence, head) at a time and loops over
// heads (a persistent grid of two workgroups per compute unit, so that one
// workgroup's loads overlap the others' arithmetic).  Wave w builds the operands
// of key-channel block pair w, as the single-pass prefill's producers do; wave 0
// then inverts I + A while every wave forms K+ S and Q+ S for its 32 state columns
// (two 16-column slices), and after a barrier every wave finishes Delta, O and the
// committed state of its columns.  The next head's inputs are loaded during the
// current head's build, its state after the current state is written.
//
// Layout conventions and the key-channel relabelling inside block pairs are those
// of the prefill kernels: internal channel 16 (2P + h) + 4 g4 + j is memory channel
// 32 P + 8 g4 + 4 h + j, so one lane's part of a block pair is one 16-byte piece.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int WC_D = 128;               // dk = dv
constexpr int WC_NB = WC_D / 16;        // 16-channel blocks
constexpr int WC_NPAIR = WC_NB / 2;     // block pairs = waves
constexpr int WC_SL = 2;                // 16-column state slices per wave
constexpr int WC_WAVES = 4;
constexpr int WC_BLOCKS_PER_CU = 2;

static_assert(WC_NPAIR == WC_WAVES && WC_WAVES * WC_SL * 16 == WC_D, "one block pair and 32 columns per wave");

// The state-independent operands of a head's chunk (A-operand fragments; block
// pairs packed as in the prefill kernels).
struct WcOps {
    bf16x8 qp_hi[WC_NPAIR][64];
    bf16x8 qp_lo[WC_NPAIR][64];
    bf16x8 kp[WC_NPAIR][64];
    bf16x8 kp_lo[WC_NPAIR][64];
    Split4 kt[WC_NB][64];  // K~_a^T (channel rows, 4 tokens per lane), {hi, lo}
    Split4 tp[64];         // T' as the A operand of Delta = T' Y
    Split4 aq[64];         // Aqk as the A operand of Aqk Delta
    float gam[WC_D];       // e^{G_{a-1}} per (internal) channel
    float beta[16];
};

// Per wave: the raw q, k, g rows of the head (16 token rows of 64 bytes, padded to
// 80 so the operand-layout reads hit distinct banks), and once they are read, the
// wave's partial sums of A, A^T and Aqk^T.
union WcStage {
    u32x4 rows[3][16][5];
    f32x4 part[3][64];
};

struct WcSplitT {
    bf16x4 hi, lo;
};

// One (sequence, head) of the window: scalars, uniform over the workgroup.
struct WcHead {
    uint32_t b, h;
    int rp;   // replayed tokens in front of the window's (rows 0 .. rp - 1)
    int n;    // tokens of the chunk: rp + Tw
    int acc;  // tokens whose state is committed (0: none)
};

}  // namespace

template <bool REPLAY>
__global__ __launch_bounds__(64 * WC_WAVES) __attribute__((amdgpu_waves_per_eu(WC_BLOCKS_PER_CU, WC_BLOCKS_PER_CU)))
void window_chunk_kernel(const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
                         const __bf16 *__restrict__ g, const __bf16 *__restrict__ beta, float *__restrict__ state,
                         float *__restrict__ o, const int32_t *__restrict__ accept, uint32_t heads, uint32_t H,
                         int32_t Tw, const __bf16 *__restrict__ pq, const __bf16 *__restrict__ pk,
                         const __bf16 *__restrict__ pv, const __bf16 *__restrict__ pg,
                         const __bf16 *__restrict__ pb, const int32_t *__restrict__ replay, int32_t Tp,
                         int32_t acc_default) {
    constexpr uint32_t EB = 2;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g4 = lane >> 4, l16 = lane & 15;
    const uint32_t rowK = H * WC_D * EB;  // bytes between tokens in q, k, g, v
    const uint32_t rowO = H * WC_D * 4;   // ... in o
    const uint32_t rowB = H * EB;         // ... in beta

    __shared__ __attribute__((aligned(16))) WcOps ops;
    __shared__ __attribute__((aligned(16))) WcStage stage[WC_WAVES];

    auto head_of = [&](uint32_t hd) {
        WcHead x;
        x.b = hd / H;
        x.h = hd - x.b * H;
        int rp = 0;
        if constexpr (REPLAY) {
            rp = replay[x.b];
            rp = rp < 0 ? 0 : (rp > Tp ? Tp : rp);
        }
        int a = acc_default;
        if (accept) {
            a = accept[x.b];
            a = a < 0 ? 0 : (a > Tw ? Tw : a);
        }
        x.rp = __builtin_amdgcn_readfirstlane(rp);
        x.n = x.rp + Tw;
        x.acc = __builtin_amdgcn_readfirstlane(a) + x.rp;
        return x;
    };
    // Token rows of the chunk: row r < rp is token r of the previous window, row r >= rp
    // token r - rp of this one; rows past n and every unused source read as zeros.
    auto cur_rsrc = [&](const __bf16 *base, const WcHead &x, uint32_t row, uint32_t d) {
        return make_rsrc(base + ((int64_t)x.b * Tw * H + x.h) * d, (uint32_t)Tw * row);
    };
    auto prev_rsrc = [&](const __bf16 *base, const WcHead &x, uint32_t row, uint32_t d) {
        return make_rsrc(base + ((int64_t)x.b * Tp * H + x.h) * d, (uint32_t)x.rp * row);
    };
    auto cur_off = [&](const WcHead &x, int r, uint32_t row, uint32_t inrow) {
        return r >= x.rp ? (uint32_t)(r - x.rp) * row + inrow : OOB;
    };

    // ---------------------------------------------------------------- operand build (wave w: block pair w)
    u16x4 lt_bits;
#pragma unroll
    for (int j = 0; j < 4; ++j) lt_bits[j] = (4 * g4 + j <= l16) ? 0x3f80 : 0;
    const bf16x4 LT = __builtin_bit_cast(bf16x4, lt_bits);
    const bf16x4 ID = identity_operand(g4, l16);
    const bf16x4 z4 = {};
    const bf16x8 IDL = cat(ID, z4), IDH = cat(z4, ID), LTL = cat(LT, z4), LTH = cat(z4, LT);
    const bf16x8 NIL = neg_identity_operand<0>(g4, l16), NIH = neg_identity_operand<1>(g4, l16);

    struct PIn {
        u32x4 d[3];
        uint32_t b;
    };
    // q, k, g rows of block pair w (four consecutive lanes per token row) and beta of token l16
    auto pload = [&](PIn &R, const WcHead &x) {
        const int r = lane >> 2;
        const uint32_t inrow = 64u * w + 16u * (lane & 3);
        const uint32_t oc = cur_off(x, r, rowK, inrow);
        const uint32_t ob = cur_off(x, l16, rowB, 0);
        R.d[0] = buf_load_u32x4(cur_rsrc(q, x, rowK, WC_D), oc);
        R.d[1] = buf_load_u32x4(cur_rsrc(k, x, rowK, WC_D), oc);
        R.d[2] = buf_load_u32x4(cur_rsrc(g, x, rowK, WC_D), oc);
        R.b = buf_load_u16(cur_rsrc(beta, x, rowB, 1), ob);
        if constexpr (REPLAY) {
            const uint32_t op = (uint32_t)r * rowK + inrow;
            R.d[0] |= buf_load_u32x4(prev_rsrc(pq, x, rowK, WC_D), op);
            R.d[1] |= buf_load_u32x4(prev_rsrc(pk, x, rowK, WC_D), op);
            R.d[2] |= buf_load_u32x4(prev_rsrc(pg, x, rowK, WC_D), op);
            R.b |= buf_load_u16(prev_rsrc(pb, x, rowB, 1), (uint32_t)l16 * rowB);
        }
    };
    struct AIn {
        u32x4 d[3];
        float b;
    };
    auto stage_put = [&](const PIn &R) {
#pragma unroll
        for (int t = 0; t < 3; ++t) stage[w].rows[t][lane >> 2][lane & 3] = R.d[t];
    };
    auto stage_get = [&](AIn &A, const PIn &R) {
#pragma unroll
        for (int t = 0; t < 3; ++t) A.d[t] = stage[w].rows[t][l16][g4];
        A.b = bf16_bits_to_f32((uint16_t)R.b);
    };
    auto half = [](const u32x4 &x, int hh) { return hh ? u32x2{x[2], x[3]} : u32x2{x[0], x[1]}; };

    // Operands of block pair w into ops, this wave's partial sums of A, A^T and Aqk^T
    // into its stage (after its rows have been read from there).
    auto build = [&](const AIn &A, const WcHead &x) {
        const int b0 = 2 * w, b1 = b0 + 1;
        // 0/1 triangle of the committed decay, as the A operand of Gs = U g: lane (g4, i)
        // holds [i < t < a] for t = 4 g4 + j, so Gs_i = G_{a-1} - G_i for i < a
        u16x4 ut_bits;
#pragma unroll
        for (int j = 0; j < 4; ++j) ut_bits[j] = (4 * g4 + j > l16 && 4 * g4 + j < x.acc) ? 0x3f80 : 0;
        const bf16x4 UT = __builtin_bit_cast(bf16x4, ut_bits);
        const bf16x8 UTL = cat(UT, z4), UTH = cat(z4, UT);
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
        f32x4 Pp[2], qv[2], ktv[2], kmv[2], kpv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x4 Pm, F;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                Pp[u][j] = decay_exp_fast(GT[u][j]);   // e^{G_r}
                Pm[j] = decay_exp_fast(-GT[u][j]);     // e^{-G_r}
                F[j] = decay_exp_fast(GS[u][j]);       // e^{G_{a-1} - G_r}
            }
            const f32x4 kk = unpack_bf16x4(Rk[u]);
            qv[u] = unpack_bf16x4(Rq[u]) * Pp[u];
            kpv[u] = kk * Pp[u];
            kmv[u] = kk * Pm;
#pragma unroll
            for (int j = 0; j < 4; ++j) ktv[u][j] = (4 * g4 + j < x.acc) ? kc[u][j] * F[j] : 0.f;
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
        ops.qp_hi[w][lane] = qh;
        ops.qp_lo[w][lane] = ql;
        ops.kp[w][lane] = kpp;
        ops.kp_lo[w][lane] = kpl;
        ops.kt[b0][lane] = Split4{__builtin_shufflevector(kth, kth, 0, 1, 2, 3), ktl[0]};
        ops.kt[b1][lane] = Split4{__builtin_shufflevector(kth, kth, 4, 5, 6, 7), ktl[1]};
        if (l16 == x.acc - 1) {
            *reinterpret_cast<f32x4 *>(&ops.gam[16 * b0 + 4 * g4]) = Pp[0];
            *reinterpret_cast<f32x4 *>(&ops.gam[16 * b1 + 4 * g4]) = Pp[1];
        }
        if (w == 0 && lane < 16) ops.beta[lane] = A.b;
        // partial sums over this wave's 32 key channels (split bf16, hi*hi + lo*hi + hi*lo):
        // A = K+ K-^T, A^T = K- K+^T, Aqk^T = K- Q+^T, all in the accumulator layout
        f32x4 at = mma32(kpp, kmh, zero4());
        at = mma32(kpl, kmh, at);
        at = mma32(kpp, kml, at);
        f32x4 bt = mma32(kmh, kpp, zero4());
        bt = mma32(kml, kpp, bt);
        bt = mma32(kmh, kpl, bt);
        f32x4 aqt = mma32(kmh, qh, zero4());
        aqt = mma32(kml, qh, aqt);
        aqt = mma32(kmh, ql, aqt);
        stage[w].part[0][lane] = at;
        stage[w].part[1][lane] = bt;
        stage[w].part[2][lane] = aqt;
    };

    // ---------------------------------------------------------------- inverse (wave 0)
    auto splitT = [&](const f32x4 &x) {
        bf16x8 hh;
        const bf16x4 lo = split_lo(x, NIL, hh);
        return WcSplitT{__builtin_shufflevector(hh, hh, 0, 1, 2, 3), lo};
    };
    // X Y for X, Y given by the splits of the accumulator layouts of X^T (left) and Y
    // (right); all four half products, fp32 accumulation onto c.
    auto prod = [&](const WcSplitT &xt, const WcSplitT &y, f32x4 c) {
        const bf16x8 a = cat(xt.hi, xt.lo);
        c = mma32(a, cat(y.hi, y.hi), c);
        return mma32(a, cat(y.lo, y.lo), c);
    };
    // Add the partials, apply beta and the triangular masks, invert I + A as
    // (I - B)(I + B^2)(I + B^4)(I + B^8) with B = A^T (strictly upper triangular, B^16 = 0),
    // and write T' and Aqk as A-operand fragments (split bf16).
    auto solve = [&]() {
        f32x4 Am = stage[0].part[0][lane], Bm = stage[0].part[1][lane], Qm = stage[0].part[2][lane];
#pragma unroll
        for (int u = 1; u < WC_WAVES; ++u) {
            Am += stage[u].part[0][lane];
            Bm += stage[u].part[1][lane];
            Qm += stage[u].part[2][lane];
        }
        const f32x4 brow = *reinterpret_cast<const f32x4 *>(&ops.beta[4 * g4]);  // beta of rows 4 g4 + j
        const float bcol = ops.beta[l16];                                        // beta of column l16
        f32x4 R0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * g4 + j;
            Am[j] = (r > l16) ? Am[j] * brow[j] : 0.f;   // A   = diag(beta) strictly_lower
            Bm[j] = (l16 > r) ? Bm[j] * bcol : 0.f;      // A^T
            Qm[j] = (l16 >= r) ? Qm[j] : 0.f;            // Aqk^T (lower incl. diagonal of Aqk)
            R0[j] = (r == l16 ? 1.f : 0.f) - Bm[j];      // I - B
        }
        const WcSplitT sA = splitT(Am), sB = splitT(Bm);
        const f32x4 A2 = prod(sB, sA, zero4()), B2 = prod(sA, sB, zero4());
        const WcSplitT sA2 = splitT(A2), sB2 = splitT(B2), sR0 = splitT(R0);
        const f32x4 A4 = prod(sB2, sA2, zero4()), B4 = prod(sA2, sB2, zero4());
        const f32x4 R1 = prod(sA2, sR0, R0);
        const WcSplitT sA4 = splitT(A4), sB4 = splitT(B4), sR1 = splitT(R1);
        const f32x4 A8 = prod(sB4, sA4, zero4());
        const f32x4 R2 = prod(sA4, sR1, R1);
        const WcSplitT sA8 = splitT(A8), sR2 = splitT(R2);
        f32x4 Tt = prod(sA8, sR2, R2);
        Tt *= brow;  // T'^T = diag(beta) T^T: its accumulator layout is the A operand of T'
        const WcSplitT st = splitT(Tt), sq = splitT(Qm);
        ops.tp[lane] = Split4{st.hi, st.lo};
        ops.aq[lane] = Split4{sq.hi, sq.lo};
    };

    // ---------------------------------------------------------------- state columns (every wave)
    // State slices: internal rows 16 b + 4 g4 + jj, column col0 + l16; internal row
    // 16 b + 4 g4 + jj is memory key channel mrow(b, jj).
    int col0[WC_SL];
#pragma unroll
    for (int sl = 0; sl < WC_SL; ++sl) col0[sl] = (w * WC_SL + sl) * 16;
    auto state_rsrc = [&](const WcHead &x) {
        return make_rsrc(state + ((int64_t)x.b * H + x.h) * (WC_D * WC_D), WC_D * WC_D * 4u);
    };
    // Byte offset of state element (mrow(b, jj), col0[sl] + l16): a per-lane part (one
    // register for all 64 elements) plus a constant that goes into the scalar offset.
    const uint32_t s_voff = ((8 * g4) * WC_D + col0[0] + l16) * 4u;
    auto s_soff = [](int sl, int b, int jj) {
        return (uint32_t)(((32 * (b >> 1) + 4 * (b & 1) + jj) * WC_D + 16 * sl) * 4);
    };
    auto load_state = [&](f32x4 (&S)[WC_SL][WC_NB], const WcHead &x) {
        const rsrc_t rs = state_rsrc(x);
#pragma unroll
        for (int sl = 0; sl < WC_SL; ++sl)
#pragma unroll
            for (int b = 0; b < WC_NB; ++b)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    S[sl][b][jj] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(rs, s_voff, s_soff(sl, b, jj), 0));
    };
    // v of token l16, columns col0 + 4 g4 .. +3 of each slice
    struct CIn {
        u32x2 v[WC_SL];
    };
    auto cload = [&](CIn &X, const WcHead &x) {
        const rsrc_t rv = cur_rsrc(v, x, rowK, WC_D);
#pragma unroll
        for (int sl = 0; sl < WC_SL; ++sl) {
            const uint32_t in = (col0[sl] + 4 * g4) * EB;
            X.v[sl] = buf_load_u32x2(rv, cur_off(x, l16, rowK, in));
            if constexpr (REPLAY) X.v[sl] |= buf_load_u32x2(prev_rsrc(pv, x, rowK, WC_D), (uint32_t)l16 * rowK + in);
        }
    };

    uint32_t hd = blockIdx.x;
    if (hd >= heads) return;
    WcHead cur = head_of(hd);
    PIn R;
    CIn X;
    f32x4 S[WC_SL][WC_NB];
    pload(R, cur);
    cload(X, cur);
    load_state(S, cur);
    for (;;) {
        AIn A;
        stage_put(R);
        stage_get(A, R);  // (the wave's own LDS accesses stay in order)
        const uint32_t nh = hd + gridDim.x;
        const bool more = nh < heads;
        WcHead nxt = cur;
        if (more) {
            nxt = head_of(nh);
            pload(R, nxt);
        }
        build(A, cur);
        __syncthreads();  // operands and partials of this head
        if (w == 0) solve();
        // X = K+ S and Q+ S per slice, each as hi*hi, lo*hi, hi*lo
        f32x4 Xa[WC_SL], Xb[WC_SL], Oa[WC_SL], Ob[WC_SL], Oc[WC_SL];
#pragma unroll
        for (int sl = 0; sl < WC_SL; ++sl) Xa[sl] = Xb[sl] = Oa[sl] = Ob[sl] = Oc[sl] = zero4();
#pragma unroll
        for (int p = 0; p < WC_NPAIR; ++p) {
            const bf16x8 kpr = ops.kp[p][lane], kplr = ops.kp_lo[p][lane];
            const bf16x8 qhr = ops.qp_hi[p][lane], qlr = ops.qp_lo[p][lane];
#pragma unroll
            for (int sl = 0; sl < WC_SL; ++sl) {
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
        __syncthreads();  // T' and Aqk of this head
        const Split4 Tp4 = ops.tp[lane], Aq = ops.aq[lane];
        const bf16x8 tpp = cat(Tp4.hi, Tp4.lo), aqq = cat(Aq.hi, Aq.lo);
        const rsrc_t ro = make_rsrc(o ? o + ((int64_t)cur.b * Tw * H + cur.h) * WC_D : o, o ? (uint32_t)Tw * rowO : 0u);
        // output rows 4 g4 + jj of this window (rows of the replay and past the window dropped)
        uint32_t o_voff[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) o_voff[jj] = cur_off(cur, 4 * g4 + jj, rowO, (col0[0] + l16) * 4u);
        bf16x8 dhh[WC_SL], dll[WC_SL];
#pragma unroll
        for (int sl = 0; sl < WC_SL; ++sl) {
            // Delta = T' (V - X); O = Q+ S + Aqk Delta for the rows of this window
            const f32x4 vc = mma16(__builtin_bit_cast(bf16x4, X.v[sl]), ID, zero4());
            bf16x8 yhh;
            const bf16x4 ylo = split_lo(vc - (Xa[sl] + Xb[sl]), NIL, yhh);
            f32x4 D = mma32(tpp, yhh, zero4());
            D = mma32(tpp, cat(ylo, ylo), D);
            const bf16x4 dlo = split_lo(D, NIL, dhh[sl]);
            dll[sl] = cat(dlo, dlo);
            f32x4 O = mma32(aqq, dhh[sl], Oa[sl] + (Ob[sl] + Oc[sl]));
            O = mma32(aqq, dll[sl], O);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(O[jj]), ro, o_voff[jj], 64u * sl, 0);
        }
        if (cur.acc > 0) {
            // S_a = Diag(e^{G_{a-1}}) S + K~_a^T Delta, written back
            const rsrc_t rs = state_rsrc(cur);
#pragma unroll
            for (int b = 0; b < WC_NB; ++b) {
                const Split4 kt = ops.kt[b][lane];
                const f32x4 gm = *reinterpret_cast<const f32x4 *>(&ops.gam[16 * b + 4 * g4]);
                const bf16x8 ktt = cat(kt.hi, kt.lo);
#pragma unroll
                for (int sl = 0; sl < WC_SL; ++sl) {
                    const f32x4 acc = mma32(ktt, dhh[sl], S[sl][b] * gm);
                    const f32x4 Sn = mma32(ktt, dll[sl], acc);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Sn[jj]), rs, s_voff, s_soff(sl, b, jj), 0);
                }
            }
        }
        if (more) {
            cload(X, nxt);
            load_state(S, nxt);
        }
        __syncthreads();  // operands of this head read by every wave
        if (!more) break;
        hd = nh;
        cur = nxt;
    }
}

hipError_t launch_window_chunk(const DecodeWindowArgs &a) {
    if (!window_chunk_supported(a)) return hipErrorInvalidValue;
    const int64_t heads = (int64_t)a.B * a.H;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int64_t cap = (int64_t)cus * WC_BLOCKS_PER_CU;
    const int64_t grid = heads < cap ? heads : cap;
    const int acc_default = a.acc_default < 0 ? a.T : a.acc_default;
    auto kern = a.replay ? window_chunk_kernel<true> : window_chunk_kernel<false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * WC_WAVES), 0, (hipStream_t)a.stream,
                       (const __bf16 *)a.q, (const __bf16 *)a.k, (const __bf16 *)a.v, (const __bf16 *)a.g,
                       (const __bf16 *)a.beta, a.state, a.o, a.accept, (uint32_t)heads, (uint32_t)a.H, a.T,
                       (const __bf16 *)a.pq, (const __bf16 *)a.pk, (const __bf16 *)a.pv, (const __bf16 *)a.pg,
                       (const __bf16 *)a.pbeta, a.replay, a.Tp, acc_default);
    e = hipGetLastError();
    if (e != hipSuccess || !a.fx.u) return e;
    const OutNormGateArgs ep{a.o, a.fx.u, a.fx.w, a.fx.eps, (int64_t)a.B * a.T, a.H, a.dv, a.bf16, a.fx.y, a.stream};
    return launch_out_norm_gate(ep);
}

}  // namespace kda
