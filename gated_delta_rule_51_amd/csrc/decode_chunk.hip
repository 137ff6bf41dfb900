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
// A workgroup of eight waves serves one (sequence, head) at a time and loops over
// heads (a persistent grid, one workgroup per compute unit).  Waves 0..3 build the
// operands of key-channel block pairs 0..3, as the single-pass prefill's producers
// do; wave 4 then inverts I + A while every wave forms K+ S and Q+ S for its 16
// state columns, and after a barrier every wave finishes Delta, O and the committed
// state of its columns.  The head's state is the bound: its rows are loaded one head
// ahead (a state load is in flight through the whole of the previous head, 64 KB
// per compute unit at all times) and pass through an LDS copy in both directions
// (below); the next head's inputs are loaded during the current head's build.
//
// Layout conventions and the key-channel relabelling inside block pairs are those
// of the prefill kernels: internal channel 16 (2P + h) + 4 g4 + j is memory channel
// 32 P + 8 g4 + 4 h + j, so one lane's part of a block pair is one 16-byte piece.
#include "kda_device.hpp"
#include "kda_launch.hpp"
#include "layer_prologue.hpp"

namespace kda {

namespace {

constexpr int WC_D = 128;               // dk = dv
constexpr int WC_NB = WC_D / 16;        // 16-channel blocks
constexpr int WC_NPAIR = WC_NB / 2;     // block pairs = waves
constexpr int WC_SL = 1;                // 16-column state slices per wave
constexpr int WC_WAVES = 8;
constexpr int WC_BUILDERS = 4;          // waves that build the operands, one block pair each
constexpr int WC_SOLVER = 4;            // the wave that inverts I + A (shares a SIMD with builder 0)
constexpr int WC_LP = WC_D + 4;         // padded row of the state's LDS copy (16-byte aligned rows)

static_assert(WC_NPAIR == WC_BUILDERS && WC_WAVES * WC_SL * 16 == WC_D, "one block pair per builder, 16 columns per wave");

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
    uint32_t on;  // 1; 0 makes every load of the head read zeros without touching memory
    float eA;     // e^{A_h} of the gate from logits (0 without)
};

}  // namespace

template <bool REPLAY>
__global__ __launch_bounds__(64 * WC_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void window_chunk_kernel(const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
                         const __bf16 *__restrict__ g, const __bf16 *__restrict__ beta, float *__restrict__ state,
                         float *__restrict__ o, const int32_t *__restrict__ accept, uint32_t heads, uint32_t H,
                         int32_t Tw, const __bf16 *__restrict__ pq, const __bf16 *__restrict__ pk,
                         const __bf16 *__restrict__ pv, const __bf16 *__restrict__ pg,
                         const __bf16 *__restrict__ pb, const int32_t *__restrict__ replay, int32_t Tp,
                         int32_t acc_default, const float *__restrict__ A_log) {
    constexpr uint32_t EB = 2;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g4 = lane >> 4, l16 = lane & 15;
    const uint32_t rowK = H * WC_D * EB;  // bytes between tokens in q, k, g, v
    const uint32_t rowO = H * WC_D * 4;   // ... in o
    const uint32_t rowB = H * EB;         // ... in beta

    __shared__ __attribute__((aligned(16))) WcOps ops;
    __shared__ __attribute__((aligned(16))) WcStage stage[WC_BUILDERS];
    __shared__ __attribute__((aligned(16))) float lst[WC_D * WC_LP];  // the head's state

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
        x.on = 1;
        x.eA = A_log ? __expf(A_log[x.h]) : 0.f;
        return x;
    };
    // Token rows of the chunk: row r < rp is token r of the previous window, row r >= rp
    // token r - rp of this one; rows past n and every unused source read as zeros.
    auto cur_rsrc = [&](const __bf16 *base, const WcHead &x, uint32_t row, uint32_t d, uint32_t on = 1) {
        return make_rsrc(base + ((int64_t)x.b * Tw * H + x.h) * d, (uint32_t)Tw * row * (x.on & on));
    };
    auto prev_rsrc = [&](const __bf16 *base, const WcHead &x, uint32_t row, uint32_t d, uint32_t on = 1) {
        return make_rsrc(base + ((int64_t)x.b * Tp * H + x.h) * d, (uint32_t)x.rp * row * (x.on & on));
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

    // (with a replay the rows of both windows load into registers of their own and are
    // combined where they are used: a combination right after the loads would make the
    // compiler wait there for every load in flight)
    struct PIn {
        u32x4 d[3], pd[3];
        uint32_t b, pb;
    };
    // q, k, g rows of block pair w (four consecutive lanes per token row) and beta of token l16
    // (every wave issues these loads, so the wait counts are the same on every path; only
    // the builders' read memory)
    const uint32_t builder = w < WC_BUILDERS ? 1u : 0u;
    auto pload = [&](PIn &R, const WcHead &x) {
        const int r = lane >> 2;
        const uint32_t inrow = 64u * (w & 3) + 16u * (lane & 3);
        const uint32_t oc = cur_off(x, r, rowK, inrow);
        const uint32_t ob = cur_off(x, l16, rowB, 0);
        R.d[0] = buf_load_u32x4(cur_rsrc(q, x, rowK, WC_D, builder), oc);
        R.d[1] = buf_load_u32x4(cur_rsrc(k, x, rowK, WC_D, builder), oc);
        R.d[2] = buf_load_u32x4(cur_rsrc(g, x, rowK, WC_D, builder), oc);
        R.b = buf_load_u16(cur_rsrc(beta, x, rowB, 1, builder), ob);
        if constexpr (REPLAY) {
            const uint32_t op = (uint32_t)r * rowK + inrow;
            R.pd[0] = buf_load_u32x4(prev_rsrc(pq, x, rowK, WC_D, builder), op);
            R.pd[1] = buf_load_u32x4(prev_rsrc(pk, x, rowK, WC_D, builder), op);
            R.pd[2] = buf_load_u32x4(prev_rsrc(pg, x, rowK, WC_D, builder), op);
            R.pb = buf_load_u16(prev_rsrc(pb, x, rowB, 1, builder), (uint32_t)l16 * rowB);
        }
    };
    struct AIn {
        u32x4 d[3];
        float b;
    };
    auto stage_put = [&](const PIn &R) {
#pragma unroll
        for (int t = 0; t < 3; ++t) stage[w].rows[t][lane >> 2][lane & 3] = REPLAY ? (R.d[t] | R.pd[t]) : R.d[t];
    };
    auto stage_get = [&](AIn &A, const PIn &R) {
#pragma unroll
        for (int t = 0; t < 3; ++t) A.d[t] = stage[w].rows[t][l16][g4];
        A.b = bf16_bits_to_f32((uint16_t)(REPLAY ? (R.b | R.pb) : R.b));
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
        const bf16x8 ka = __builtin_bit_cast(bf16x8, A.d[1]);
        const f32x4 kc[2] = {mma32(ka, IDL, zero4()), mma32(ka, IDH, zero4())};
        // g and k as tokens 4 g4 + jj of channel 16 b + l16 (exact for bf16 values); G at token
        // l16, channels 16 b + 4 g4 + jj; Gs at tokens 4 g4 + jj, channel 16 b + l16
        f32x4 GT[2], GS[2];
        if (A_log) {
            // the gate from logits, -5 Sigmoid(e^{A_h} z), in fp32 and split hi + lo for the
            // transposes and the triangle sums (rows past the head's tokens: g = 0)
            const bf16x8 za = __builtin_bit_cast(bf16x8, A.d[2]);
            const bool row = l16 < x.n;
            f32x4 gv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int j = 0; j < 4; ++j) gv[u][j] = row ? gate_of(x.eA, (float)za[4 * u + j]) : 0.f;
            const bf16x4 gh0 = to_bf16x4(gv[0]), gh1 = to_bf16x4(gv[1]);
            const bf16x8 gah = cat(gh0, gh1);
            const bf16x8 gal = cat(to_bf16x4(gv[0] - from_bf16x4(gh0)), to_bf16x4(gv[1] - from_bf16x4(gh1)));
            const bf16x8 gfh = cat(to_bf16x4(mma32(gah, IDL, zero4())), to_bf16x4(mma32(gah, IDH, zero4())));
            const bf16x8 gfl = cat(to_bf16x4(mma32(gal, IDL, zero4())), to_bf16x4(mma32(gal, IDH, zero4())));
            GT[0] = mma32(gfl, LTL, mma32(gfh, LTL, zero4()));
            GT[1] = mma32(gfl, LTH, mma32(gfh, LTH, zero4()));
            GS[0] = mma32(UTL, gfl, mma32(UTL, gfh, zero4()));
            GS[1] = mma32(UTH, gfl, mma32(UTH, gfh, zero4()));
        } else {
            const bf16x8 ga = __builtin_bit_cast(bf16x8, A.d[2]);
            const bf16x8 gf = cat(to_bf16x4(mma32(ga, IDL, zero4())), to_bf16x4(mma32(ga, IDH, zero4())));
            GT[0] = mma32(gf, LTL, zero4());
            GT[1] = mma32(gf, LTH, zero4());
            GS[0] = mma32(UTL, gf, zero4());
            GS[1] = mma32(UTH, gf, zero4());
        }
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
        for (int u = 1; u < WC_BUILDERS; ++u) {
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
    // The state moves between HBM and the waves through an LDS copy of the head's 128 x 128
    // matrix (rows padded to WC_LP floats): HBM sees whole 512-byte rows in 16-byte pieces
    // (wave w, lane l: rows 16 w + 2 i + l / 32, columns 4 (l % 32) .. +3, i = 0..7), eight
    // loads and eight stores per wave and head -- few enough that the compiler's wait
    // counters track the next head's loads across the current head instead of draining
    // them -- and each wave reads its 16 columns in the accumulator layout from LDS.
    // Wave w's slice: internal rows 16 b + 4 g4 + jj, column 16 w + l16; internal row
    // 16 b + 4 g4 + jj is memory key channel mrow(b, jj).
    const int col0 = 16 * w;
    auto mrow = [&](int b, int jj) { return 32 * (b >> 1) + 8 * g4 + 4 * (b & 1) + jj; };
    auto state_rsrc = [&](const WcHead &x) {
        return make_rsrc(state + ((int64_t)x.b * H + x.h) * (WC_D * WC_D), WC_D * WC_D * 4u * x.on);
    };
    const int row0 = 16 * w + (lane >> 5), c4 = 4 * (lane & 31);
    const uint32_t row_voff = (uint32_t)(row0 * WC_D + c4) * 4u;
    typedef u32x4 Rows[8];
    auto load_rows = [&](Rows &P, const WcHead &x) {
        const rsrc_t rs = state_rsrc(x);
#pragma unroll
        for (int i = 0; i < 8; ++i) P[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, row_voff, i * 2u * WC_D * 4u, 0);
    };
    auto rows_to_lds = [&](const Rows &P) {
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4 *>(&lst[(row0 + 2 * i) * WC_LP + c4]) = P[i];
    };
    // v of token l16, columns col0 + 4 g4 .. +3
    struct VIn {
        u32x2 c, p;  // this window's and (with a replay) the previous window's rows
    };
    auto cload = [&](VIn &X, const WcHead &x) {
        const uint32_t in = (col0 + 4 * g4) * EB;
        X.c = buf_load_u32x2(cur_rsrc(v, x, rowK, WC_D), cur_off(x, l16, rowK, in));
        if constexpr (REPLAY) X.p = buf_load_u32x2(prev_rsrc(pv, x, rowK, WC_D), (uint32_t)l16 * rowK + in);
    };

    // One head: its state rows in P (loaded one head earlier) and its v in X; the next
    // head's rows go into P once these are in LDS, its v into Xn, its q/k/g into R.
    PIn R;
    Rows P;
    // (The next head's loads are issued in the order q/k/g, state rows, v, each into the
    // registers its own data came in, so no load result is copied and the waits for one
    // never include the ones issued after it.)
    auto process = [&](const VIn &X, VIn &Xn, const WcHead &cur, bool more, const WcHead &nxt) {
        rows_to_lds(P);
        AIn A;
        if (w < WC_BUILDERS) {
            stage_put(R);
            stage_get(A, R);  // (the wave's own LDS accesses stay in order)
        }
        __builtin_amdgcn_sched_barrier(0);  // R read before it is reloaded
        WcHead ld = nxt;  // past the last head: loads that read zeros
        ld.on = more ? 1u : 0u;
        pload(R, ld);
        load_rows(P, ld);
        cload(Xn, ld);
        if (w < WC_BUILDERS) build(A, cur);
        __syncthreads();  // operands, partials and the state copy of this head
        if (w == WC_SOLVER) solve();
        f32x4 S[WC_NB];
#pragma unroll
        for (int b = 0; b < WC_NB; ++b)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) S[b][jj] = lst[mrow(b, jj) * WC_LP + col0 + l16];
        // X = K+ S and Q+ S, each as hi*hi, lo*hi, hi*lo
        f32x4 Xa = zero4(), Xb = zero4(), Oa = zero4(), Ob = zero4(), Oc = zero4();
#pragma unroll
        for (int p = 0; p < WC_NPAIR; ++p) {
            const bf16x8 kpr = ops.kp[p][lane], kplr = ops.kp_lo[p][lane];
            const bf16x8 qhr = ops.qp_hi[p][lane], qlr = ops.qp_lo[p][lane];
            const bf16x8 Shi = cat(to_bf16x4(S[2 * p]), to_bf16x4(S[2 * p + 1]));
            const bf16x8 Slo = cat(to_bf16x4(mma32(NIL, Shi, S[2 * p])), to_bf16x4(mma32(NIH, Shi, S[2 * p + 1])));
            Xa = mma32(kpr, Shi, Xa);
            Xb = mma32(kplr, Shi, Xb);
            Xb = mma32(kpr, Slo, Xb);
            Oa = mma32(qhr, Shi, Oa);
            Ob = mma32(qlr, Shi, Ob);
            Oc = mma32(qhr, Slo, Oc);
        }
        __syncthreads();  // T' and Aqk of this head; every wave's state copy read
        const Split4 Tp4 = ops.tp[lane], Aq = ops.aq[lane];
        const bf16x8 tpp = cat(Tp4.hi, Tp4.lo), aqq = cat(Aq.hi, Aq.lo);
        const rsrc_t ro = make_rsrc(o ? o + ((int64_t)cur.b * Tw * H + cur.h) * WC_D : o, o ? (uint32_t)Tw * rowO : 0u);
        // Delta = T' (V - X); O = Q+ S + Aqk Delta for the rows of this window (rows of the
        // replay and past the window dropped)
        const f32x4 vc = mma16(__builtin_bit_cast(bf16x4, REPLAY ? (X.c | X.p) : X.c), ID, zero4());
        bf16x8 yhh, dhh;
        const bf16x4 ylo = split_lo(vc - (Xa + Xb), NIL, yhh);
        f32x4 D = mma32(tpp, yhh, zero4());
        D = mma32(tpp, cat(ylo, ylo), D);
        const bf16x4 dlo = split_lo(D, NIL, dhh);
        const bf16x8 dll = cat(dlo, dlo);
        f32x4 O = mma32(aqq, dhh, Oa + (Ob + Oc));
        O = mma32(aqq, dll, O);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            buf_store_f32(O[jj], ro, cur_off(cur, 4 * g4 + jj, rowO, (col0 + l16) * 4u));
        {
            // S_a = Diag(e^{G_{a-1}}) S + K~_a^T Delta, through the LDS copy back to HBM; with
            // a = 0 the stores go to an empty buffer (dropped) rather than behind a branch, so
            // the wait counts of the next head's loads are the same on every path
#pragma unroll
            for (int b = 0; b < WC_NB; ++b) {
                const Split4 kt = ops.kt[b][lane];
                const f32x4 gm = *reinterpret_cast<const f32x4 *>(&ops.gam[16 * b + 4 * g4]);
                const bf16x8 ktt = cat(kt.hi, kt.lo);
                const f32x4 Sn = mma32(ktt, dll, mma32(ktt, dhh, S[b] * gm));
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) lst[mrow(b, jj) * WC_LP + col0 + l16] = Sn[jj];
            }
            __syncthreads();  // the committed state in LDS
            WcHead st = cur;
            st.on = cur.acc > 0 ? 1u : 0u;
            const rsrc_t rs = state_rsrc(st);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4 *>(&lst[(row0 + 2 * i) * WC_LP + c4]),
                                                       rs, row_voff, i * 2u * WC_D * 4u, 0);
        }
        __syncthreads();  // operands and the state copy of this head no longer read
    };

    const uint32_t G = gridDim.x;
    uint32_t hd = blockIdx.x;
    if (hd >= heads) return;
    VIn XA, XB;
    WcHead cur = head_of(hd);
    pload(R, cur);
    load_rows(P, cur);
    cload(XA, cur);
    // Two heads per trip, so the two v registers swap roles without a copy; the first head
    // is peeled off, so the loop is entered where it loops back (same loads in flight on
    // both edges, and the wait counts at its head stay exact).
    bool more = hd + G < heads;
    WcHead nxt = more ? head_of(hd + G) : cur;
    process(XA, XB, cur, more, nxt);
    while (more) {
        hd += G;
        cur = nxt;
        more = hd + G < heads;
        nxt = more ? head_of(hd + G) : cur;
        process(XB, XA, cur, more, nxt);
        if (!more) break;
        hd += G;
        cur = nxt;
        more = hd + G < heads;
        nxt = more ? head_of(hd + G) : cur;
        process(XA, XB, cur, more, nxt);
    }
}

hipError_t launch_window_chunk(const DecodeWindowArgs &a) {
    if (!window_chunk_supported(a)) return hipErrorInvalidValue;
    const int64_t heads = (int64_t)a.B * a.H;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int64_t cap = cus;  // one workgroup per compute unit
    const int64_t grid = heads < cap ? heads : cap;
    const int acc_default = a.acc_default < 0 ? a.T : a.acc_default;
    auto kern = a.replay ? window_chunk_kernel<true> : window_chunk_kernel<false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * WC_WAVES), 0, (hipStream_t)a.stream,
                       (const __bf16 *)a.q, (const __bf16 *)a.k, (const __bf16 *)a.v, (const __bf16 *)a.g,
                       (const __bf16 *)a.beta, a.state, a.o, a.accept, (uint32_t)heads, (uint32_t)a.H, a.T,
                       (const __bf16 *)a.pq, (const __bf16 *)a.pk, (const __bf16 *)a.pv, (const __bf16 *)a.pg,
                       (const __bf16 *)a.pbeta, a.replay, a.Tp, acc_default, a.fx.A_log);
    e = hipGetLastError();
    if (e != hipSuccess || !a.fx.u) return e;
    const OutNormGateArgs ep{a.o, a.fx.u, a.fx.w, a.fx.eps, (int64_t)a.B * a.T, a.H, a.dv, a.bf16, a.fx.y, a.stream};
    return launch_out_norm_gate(ep);
}

// ------------------------------------------------------------------ the layer's window
// The layer's decode window (ShortConv + Swish on q, k, v, L2 norms of q and k, the gate
// from logits; Kimi K3 report digest, "Kimi Delta Attention", the paragraph after the
// update equation, and the bounded-decay section) in the one-chunk form: a prologue pass
// runs each (sequence, head) through its replayed prefix and the window's tokens in order,
// from the sequence's convolution cache, and writes the chunk kernel's bf16 inputs -- the
// normalised q and k, Swish(conv(v)) and the log-decay -- to a workspace; it commits the
// cache after the prefix (where the chunk kernel commits the state).  The chunk kernel then
// runs on those rows, and the output epilogue on o.
//
// One wave per (sequence, head); lane l holds channels 2 l and 2 l + 1 of q, k, v and the
// gate, carries the convolution's three earlier inputs of each in registers, and the row
// norms are butterfly sums over the wave.
constexpr int WP_WAVES = 4;

__global__ __launch_bounds__(64 * WP_WAVES) void window_prologue_kernel(
    const __bf16 *__restrict__ qkv, const __bf16 *__restrict__ gate, const __bf16 *__restrict__ pqkv,
    const __bf16 *__restrict__ pgate, const int32_t *__restrict__ replay, int32_t Tp, int32_t Tw, int32_t H,
    int64_t heads, const float *__restrict__ conv_w, float *__restrict__ conv_cache, float l2eps,
    const float *__restrict__ A_log, __bf16 *__restrict__ ws) {
    constexpr int D = WC_D, C = 3 * WC_D;
    const int lane = threadIdx.x & 63;
    const int64_t head = (int64_t)blockIdx.x * WP_WAVES + (threadIdx.x >> 6);
    if (head >= heads) return;  // (whole waves)
    const int64_t b = head / H;
    const int h = (int)(head - b * H);
    int rp = 0;
    if (Tp > 0) {
        rp = replay[b];
        rp = rp < 0 ? 0 : (rp > Tp ? Tp : rp);
    }
    const int n = rp + Tw;
    // workspace: q, k, v, g rows of the window ([B, Tw, H, D] each), then of the prefix
    // ([B, Tp, H, D] each)
    const int64_t cur_sz = heads * Tw * D, pre_sz = heads * Tp * D;
    float x1[3][2], x2[3][2], x3[3][2];  // inputs t - 1, t - 2, t - 3 of q, k, v
    f32x4 w[3][2];
    float *cc = conv_cache + head * (int64_t)C * 3;
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int ch = t * D + 2 * lane + m;
            x3[t][m] = cc[ch * 3 + 0];
            x2[t][m] = cc[ch * 3 + 1];
            x1[t][m] = cc[ch * 3 + 2];
            w[t][m] = *reinterpret_cast<const f32x4 *>(conv_w + ((int64_t)h * C + ch) * 4);
        }
    const float eA = A_log ? __expf(A_log[h]) : 0.f;
    for (int j = 0; j < n; ++j) {
        const bool pre = j < rp;
        const int64_t row = pre ? ((b * Tp + j) * H + h) : ((b * Tw + (j - rp)) * H + h);
        const __bf16 *src = (pre ? pqkv : qkv) + row * C;
        const uint32_t gw = *reinterpret_cast<const uint32_t *>((pre ? pgate : gate) + row * D + 2 * lane);
        float x0[3][2], y[3][2];
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const uint32_t xw = *reinterpret_cast<const uint32_t *>(src + t * D + 2 * lane);
            x0[t][0] = lo_bf16(xw);
            x0[t][1] = hi_bf16(xw);
#pragma unroll
            for (int m = 0; m < 2; ++m) y[t][m] = conv4_swish(w[t][m], x0[t][m], x1[t][m], x2[t][m], x3[t][m]);
        }
        float sq = __builtin_fmaf(y[0][0], y[0][0], y[0][1] * y[0][1]);
        float sk = __builtin_fmaf(y[1][0], y[1][0], y[1][1] * y[1][1]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            sq += __shfl_xor(sq, m);
            sk += __shfl_xor(sk, m);
        }
        const float iq = __builtin_amdgcn_rsqf(sq + l2eps), ik = __builtin_amdgcn_rsqf(sk + l2eps);
        float g0 = lo_bf16(gw), g1 = hi_bf16(gw);
        if (A_log) {
            g0 = gate_of(eA, g0);
            g1 = gate_of(eA, g1);
        }
        const bf16x4 qk = to_bf16x4(f32x4{y[0][0] * iq, y[0][1] * iq, y[1][0] * ik, y[1][1] * ik});
        const bf16x4 vg = to_bf16x4(f32x4{y[2][0], y[2][1], g0, g1});
        const u32x2 qkw = __builtin_bit_cast(u32x2, qk), vgw = __builtin_bit_cast(u32x2, vg);
        __bf16 *dst = ws + (pre ? 4 * cur_sz : 0) + row * D + 2 * lane;
        const int64_t step = pre ? pre_sz : cur_sz;
        *reinterpret_cast<uint32_t *>(dst) = qkw[0];
        *reinterpret_cast<uint32_t *>(dst + step) = qkw[1];
        *reinterpret_cast<uint32_t *>(dst + 2 * step) = vgw[0];
        *reinterpret_cast<uint32_t *>(dst + 3 * step) = vgw[1];
#pragma unroll
        for (int t = 0; t < 3; ++t)
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                x3[t][m] = x2[t][m];
                x2[t][m] = x1[t][m];
                x1[t][m] = x0[t][m];
            }
        if (j + 1 == rp) {  // the commit point: the cache holds the three inputs before it
#pragma unroll
            for (int t = 0; t < 3; ++t)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int ch = t * D + 2 * lane + m;
                    cc[ch * 3 + 0] = x3[t][m];
                    cc[ch * 3 + 1] = x2[t][m];
                    cc[ch * 3 + 2] = x1[t][m];
                }
        }
    }
}

size_t layer_window_chunk_bytes(int64_t B, int64_t T, int64_t Tp, int64_t H) {
    return (size_t)(4 * WC_D * 2) * (size_t)(B * H * (T + Tp));
}

hipError_t launch_layer_window_chunk(const DecodeWindowArgs &a, void *ws) {
    if (!layer_window_chunk_supported(a) || !ws) return hipErrorInvalidValue;
    const int64_t heads = (int64_t)a.B * a.H;
    const int64_t blocks = (heads + WP_WAVES - 1) / WP_WAVES;
    const int32_t Tp = a.replay ? a.Tp : 0;
    __bf16 *w = static_cast<__bf16 *>(ws);
    hipLaunchKernelGGL(window_prologue_kernel, dim3((unsigned)blocks), dim3(64 * WP_WAVES), 0, (hipStream_t)a.stream,
                       (const __bf16 *)a.q, (const __bf16 *)a.g, (const __bf16 *)a.pq, (const __bf16 *)a.pg,
                       a.replay, Tp, a.T, a.H, heads, a.fx.conv_w, a.fx.conv_cache, a.fx.l2eps, a.fx.A_log, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t cur_sz = heads * a.T * WC_D, pre_sz = heads * Tp * WC_D;
    DecodeWindowArgs c = a;
    c.q = w;
    c.k = w + cur_sz;
    c.v = w + 2 * cur_sz;
    c.g = w + 3 * cur_sz;
    if (Tp > 0) {
        __bf16 *p = w + 4 * cur_sz;
        c.pq = p;
        c.pk = p + pre_sz;
        c.pv = p + 2 * pre_sz;
        c.pg = p + 3 * pre_sz;
    }
    c.fx.A_log = nullptr;
    c.fx.conv_w = nullptr;
    c.fx.conv_cache = nullptr;
    c.form = 2;
    return launch_window_chunk(c);
}

}  // namespace kda
