// Inter-chunk phase of the KDA prefill, warp-specialised form for bf16 inputs
// (gfx950).  Same algebra as inter_chunk.hip (Kimi K3 report digest, "Kimi
// Delta Attention": the chunk output is the inter-chunk term (Gamma (.) Q) S
// plus the intra-chunk term; the state advances as Diag(Gamma) S + K~^T Delta):
//     K+ = K (.) e^{G},  Q+ = Q (.) e^{G},  K~ = K (.) e^{G_n - G},  Gamma = e^{G_n}
//     Delta = T' (V - K+ S),   O = Q+ S + A_qk Delta,   S <- Diag(Gamma) S + K~^T Delta
//
// A workgroup serves one (sequence, head) and NC 16-column slices of dv.  Its
// waves have two roles:
//   * NC consumer waves each keep a 16-column fp32 state slice in registers
//     and advance it chunk by chunk (matrix cores; the serial part);
//   * NP producer waves build the state-independent operands of the next
//     chunk (Q+, K+, K~, Gamma) into LDS while the consumers work.
// One barrier per chunk hands a finished operand set from producers to
// consumers (two sets in LDS, used alternately).  Splitting the roles takes
// the token-parallel work off the consumers' critical path and lets the two
// kinds of work share each SIMD.
//
// Producers hold q, k and g of a chunk as token rows with four consecutive
// channels per block per lane (the operand layout of Q+ and K+; they arrive
// through a per-wave LDS stage, see pload below).  A product with the identity
// turns g and k into four consecutive tokens of one channel per lane, and the
// cumulative log-decay G of the chunk is then a product with a 0/1 triangle,
// G^T = g^T L^T and Gs = U g (Gs_r = sum over later tokens = G_n - G_r).  The
// first lands in the operand layout of Q+ and K+, the second in that of K~^T
// (channel rows, four consecutive tokens per lane), so every operand is formed
// where it is needed and written with one vector store.  g is bf16 and the
// triangles are 0/1, so the sums are exact up to fp32 accumulation.
// Each role loads its own inputs straight from HBM ahead of use (past the last
// chunk through empty buffer resources, which return zeros): producers q/k/g,
// consumers T', A_qk (workspace fragments) and their v columns (transposed on
// the matrix cores like the producers' g and k).  Padding tokens of a ragged
// last chunk load as zeros (g = 0 keeps the decay unchanged, k = 0 removes
// them from every product).
//
// Precision: every product split bf16 (hi*hi + lo*hi + hi*lo) with fp32
// accumulation, fp32 state.  (K+ S in single bf16, enough for mild decay,
// became the largest output error with strong decay -- a gate at its -5 floor
// on every channel and heavy-tailed values, as the layer's ShortConv produces
// -- where the emulated error of a 65,536-token head dropped from 3e-3 to
// 4e-4 of RMS with the split; the classic kernel in inter_chunk.hip keeps the
// single form.)  The
// residuals lo = x - hi of those splits are formed on the matrix cores (an
// exact product with -I), which keeps the vector ALUs -- the busiest unit
// here -- for the rest.

#include "kda_device.hpp"
#include "kda_launch.hpp"
#include "layer_prologue.hpp"

namespace kda {

// Waves of a workgroup and their roles.  Wave w and wave w + 4 run on the same
// SIMD (waves 0..3 on four different ones).  With one or two consumers and more
// than four waves, the waves that would share a SIMD with a consumer stay idle
// (they only take part in the barriers), so each consumer has its SIMD to itself
// and the producers pair up on the others.
template <int NC, int NP>
struct WsLayout {
    static constexpr int NIDLE = (NC + NP > 4 && NC <= 2) ? NC : 0;
    static constexpr int NW = NC + NP + NIDLE;
    // role of wave w: consumer index (>= 0), producer index - NP (in [-NP, 0)), or
    // -NP - 1 for an idle wave
    static __device__ __forceinline__ int role(int w) {
        if (w < NC) return w;
        if (w < 4 || NIDLE == 0) return w - NC - NP;
        if (w < 4 + NIDLE) return -NP - 1;
        return w - NC - NIDLE - NP;
    }
};

template <int DK>
struct WsOps {
    static constexpr int NB = DK / 16, NPAIR = NB / 2;
    bf16x8 qp_hi[NPAIR][64];  // Q+ A-fragments, block pairs packed (one K=32 MFMA operand)
    bf16x8 qp_lo[NPAIR][64];
    bf16x8 kp[NPAIR][64];     // K+ as hi + lo, same packing
    bf16x8 kp_lo[NPAIR][64];
    Split4 kt[NB][64];        // K~^T A-fragments (channel rows, 4 tokens per lane), {hi, lo}
    float gam[DK];            // e^{G_n} per channel
};

// With LAYER the kernel is the second pass of the fused layer prefill: q, k and g
// are the normalised q, k and the log-decay the chunk-local pass computed, and v
// is the raw projection, to which the consumers apply the layer prologue
// (layer_prologue.hpp: ShortConv + Swish) as they load it.  The convolution's
// three earlier tokens are the previous chunk's raw rows, or the sequence's cache
// before its first chunk.  (Recomputing the q and k prologue here as well, from
// row norms the first pass stored, doubled this kernel's time: the producer waves
// have no vector-ALU time to spare for it.)
template <int DK, int DV, int NC, int NP, bool LAYER>
__global__ __launch_bounds__((64 * WsLayout<NC, NP>::NW)) __attribute__((amdgpu_waves_per_eu(2, 2))) void inter_chunk_ws_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const __bf16 *__restrict__ g, const float *__restrict__ init, const int32_t *__restrict__ cu,
    int32_t H, const float *__restrict__ ws, float *__restrict__ o, float *__restrict__ fin,
    int32_t nsplit, int32_t nchains, LayerPrologue lp, const int32_t *__restrict__ skip, int32_t nsort) {
    static_assert(!LAYER || (DK == 128 && DV == 128), "the fused layer prologue is built for dk = dv = 128");
    constexpr int NB = DK / 16, NPAIR = NB / 2, BPW = NB / NP;
    constexpr uint32_t EB = 2;
    static_assert(NB % 2 == 0 && NB % NP == 0, "channel blocks split evenly over producers");
    static_assert(DV % (16 * NC) == 0, "column slices");

    // XCD-aware order (as in inter_chunk.hip): all slices of one chain share an XCD.
    const int L = blockIdx.x;
    const int xcd = L & 7;
    const int sx = L >> 3;
    const int split = sx % nsplit;
    const int slot = (sx / nsplit) * 8 + xcd;
    if (slot >= nchains) return;
    const int chain = lpt_chain(cu, nsort, H, slot);
    if (skip && skip[chain]) return;  // (context parallelism: a transition known to be negligible)
    const int s = chain / H, h = chain % H;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int role = WsLayout<NC, NP>::role(tid >> 6);
    const int g4 = lane >> 4, l16 = lane & 15;

    __shared__ __attribute__((aligned(16))) WsOps<DK> ops[2];

    const int64_t bos = cu[s], eos = cu[s + 1];
    const int nc = (int)((eos - bos + 15) / 16);
    const int64_t slot0 = bos / 16 + s;
    const int64_t hd = (int64_t)s * H + h;
    const uint32_t rowK = (uint32_t)H * DK * EB;   // bytes between tokens in q, k, g
    const uint32_t rowV = (uint32_t)H * DV * EB;   // ... in v
    const uint32_t rowO = (uint32_t)H * DV * 4;    // ... in o

    // Chunks at or past the end get an empty buffer resource, so look-ahead loads
    // there return zeros without touching memory.
    const int len = (int)(eos - bos);
    // (The clamp compiles to a vector instruction; readfirstlane keeps the result
    // -- the same in every lane -- scalar, so the buffer resources built from it
    // stay uniform and their loads need no per-lane loop.)
    auto chunk_len = [&](int c) -> int {
        const int left = len - 16 * c;
        return __builtin_amdgcn_readfirstlane(left <= 0 ? 0 : (left < 16 ? left : 16));
    };
    // Buffer resource over chunk c of this head: base = the chunk's first token,
    // length = its rows (an empty resource past the end).  A NULL v reads as zeros and a
    // NULL o is not written: their resources get length 0 (on q as a stand-in base),
    // decided once here -- a null test at each resource would compile to branches that
    // split the chunk loop.
    const uint32_t v_on = v ? 1u : 0u, o_on = o ? 1u : 0u;
    const __bf16 *vb = v ? v : q;
    float *ob = o ? o : reinterpret_cast<float *>(const_cast<__bf16 *>(q));
    auto rsrc_in = [&](const __bf16 *base, int c, int d, uint32_t on) {
        const int64_t t0 = bos + 16 * (int64_t)c;
        return make_rsrc(base + (t0 * H + h) * d, (uint32_t)chunk_len(c) * (uint32_t)H * d * EB * on);
    };
    auto rsrc_out = [&](int c) {
        const int64_t t0 = bos + 16 * (int64_t)c;
        return make_rsrc(ob + (t0 * H + h) * DV, (uint32_t)chunk_len(c) * rowO * o_on);
    };
    auto rsrc_ws = [&](int c) {
        return make_rsrc(ws + ((slot0 + c) * H + h) * (int64_t)WS_FLOATS_PER_CHUNK_HEAD,
                         c < nc ? WS_FLOATS_PER_CHUNK_HEAD * 4u : 0u);
    };

    if (role == -NP - 1) {
        // idle wave: the same barriers as the others
        if (nc > 0)
            for (int c = 0; c <= nc; ++c) __syncthreads();
    } else if (role >= 0) {
        const int wave = role;
        // ============================================================ consumer
        // State slice: internal rows 16 b + 4 g4 + jj, column col0 + l16 (accumulator
        // layout); internal row 16 b + 4 g4 + jj is key channel mrow(b, jj) of the
        // state in memory (the relabelling the producers' loads use).
        const int col0 = (split * NC + wave) * 16;
        auto mrow = [&](int b, int jj) { return 32 * (b >> 1) + 8 * g4 + 4 * (b & 1) + jj; };
        // (an empty buffer resource without an initial state: the loads return 0)
        const rsrc_t rinit = make_rsrc(init ? init + hd * DK * DV : init, init ? DK * DV * 4u : 0u);
        f32x4 S[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                S[b][jj] = __builtin_bit_cast(float, buf_load_u32(rinit, (mrow(b, jj) * DV + col0 + l16) * 4u));

        if (nc > 0) {
            // Per-chunk consumer inputs: T' and A_qk fragments (workspace), and
            // v of token l16, columns col0 + 4 g4 .. +3 (one 8-byte load; the
            // identity product below turns it into rows 4 g4 + jj, column
            // col0 + l16, the layout of the state slice).
            struct CIn {
                u32x4 tp, aq;
                u32x2 v;
            };
            const bf16x4 ID = identity_operand(g4, l16);
            const bf16x8 NIL = neg_identity_operand<0>(g4, l16), NIH = neg_identity_operand<1>(g4, l16);
            // layer prologue of v: the 4 taps of this lane's columns and the raw v of the
            // chunk before (lanes l16 = 13..15 hold its last rows; first the sequence's
            // cache).  Both live in LDS, where each lane reads back what it wrote itself:
            // registers are short here.
            __shared__ f32x4 wv_lds[LAYER ? NC : 1][4][4];
            __shared__ u32x2 vprev_lds[LAYER ? NC : 1][64];
            if constexpr (LAYER) {
                f32x4 w[4];
                conv_weights<2>(lp.conv_w, h, lp.cw, 2 * DK + col0 + 4 * g4, w);
#pragma unroll
                for (int m = 0; m < 4; ++m) wv_lds[wave][g4][m] = w[m];
                uint32_t hv[2];
                cache_halo<2>(lp.cache, hd, lp.cw, 2 * DK + col0 + 4 * g4, l16, hv);
                vprev_lds[wave][lane] = u32x2{hv[0], hv[1]};
            }
            auto cload = [&](CIn &X, int c) {
                const rsrc_t rw = rsrc_ws(c);
                X.tp = buf_load_u32x4(rw, lane * 16u);
                X.aq = buf_load_u32x4(rw, (64 + lane) * 16u);
                const rsrc_t rv = rsrc_in(vb, c, DV, v_on);
                X.v = buf_load_u32x2(rv, l16 * rowV + (col0 + 4 * g4) * EB);
            };
            auto advance = [&](int ob, const CIn &X, int c) {
                const WsOps<DK> &P = ops[ob];
                // (layer: ShortConv + Swish of v first, while few registers are live)
                u32x2 vin = X.v;
                if constexpr (LAYER) {
                    const uint32_t cur[2] = {X.v[0], X.v[1]};
                    const u32x2 pv = vprev_lds[wave][lane];
                    const uint32_t prev[2] = {pv[0], pv[1]};
                    const f32x4 wv[4] = {wv_lds[wave][g4][0], wv_lds[wave][g4][1], wv_lds[wave][g4][2],
                                         wv_lds[wave][g4][3]};
                    float y[4];
                    uint32_t vh[2];
                    conv_swish<2>(cur, prev, wv, l16, y);
                    pack_scaled<2>(y, 1.f, true, vh);
                    vprev_lds[wave][lane] = X.v;
                    vin = u32x2{vh[0], vh[1]};
                }
                // Operand reads go out first, in two batches (K+ for X; then Q+, K~ and
                // Gamma), so their LDS latency overlaps the state split and the K+ S
                // products instead of stalling each matrix-core instruction that
                // consumes them.
                bf16x8 kpr[NPAIR], kplr[NPAIR];
#pragma unroll
                for (int p = 0; p < NPAIR; ++p) {
                    kpr[p] = P.kp[p][lane];
                    kplr[p] = P.kp_lo[p][lane];
                }
                __builtin_amdgcn_sched_barrier(0);
                const Split4 Tp = __builtin_bit_cast(Split4, X.tp);
                const Split4 Aq = __builtin_bit_cast(Split4, X.aq);
                const f32x4 vc = mma16(__builtin_bit_cast(bf16x4, vin), ID, zero4());
                // S = Shi + Slo (bf16), residuals on the matrix cores
                bf16x8 Shi[NPAIR], Slo[NPAIR];
#pragma unroll
                for (int p = 0; p < NPAIR; ++p) {
                    Shi[p] = cat(to_bf16x4(S[2 * p]), to_bf16x4(S[2 * p + 1]));
                    Slo[p] = cat(to_bf16x4(mma32(NIL, Shi[p], S[2 * p])),
                                 to_bf16x4(mma32(NIH, Shi[p], S[2 * p + 1])));
                }
                // X = K+ S (hi*hi + lo*hi + hi*lo, in three independent sums)
                f32x4 Xa = zero4(), Xb = zero4(), Xc = zero4();
#pragma unroll
                for (int p = 0; p < NPAIR; ++p) {
                    Xa = mma32(kpr[p], Shi[p], Xa);
                    Xb = mma32(kplr[p], Shi[p], Xb);
                    Xc = mma32(kpr[p], Slo[p], Xc);
                }
                bf16x8 qhr[NPAIR], qlr[NPAIR];
#pragma unroll
                for (int p = 0; p < NPAIR; ++p) {
                    qhr[p] = P.qp_hi[p][lane];
                    qlr[p] = P.qp_lo[p][lane];
                }
                Split4 ktr[NB];
                f32x4 gmr[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    ktr[b] = P.kt[b][lane];
                    gmr[b] = *reinterpret_cast<const f32x4 *>(&P.gam[16 * b + 4 * g4]);
                }
                __builtin_amdgcn_sched_barrier(0);
                // Q+ S for the output (hi*hi, lo*hi, hi*lo in three independent
                // sums); it does not depend on Delta and fills the gaps of the
                // Delta chain below.
                f32x4 Oa = zero4(), Ob = zero4(), Oc = zero4();
#pragma unroll
                for (int p = 0; p < NPAIR; ++p) {
                    Oa = mma32(qhr[p], Shi[p], Oa);
                    Ob = mma32(qlr[p], Shi[p], Ob);
                    Oc = mma32(qhr[p], Slo[p], Oc);
                }
                // Diag(Gamma) S now: it does not depend on Delta and fills the Delta chain's gaps
#pragma unroll
                for (int b = 0; b < NB; ++b) S[b] *= gmr[b];
                // Delta = T' (V - X)
                bf16x8 yhh, dhh;
                const bf16x4 ylo = split_lo(vc - (Xa + (Xb + Xc)), NIL, yhh);
                const bf16x8 tpp = cat(Tp.hi, Tp.lo);
                f32x4 D = mma32(tpp, yhh, zero4());
                D = mma32(tpp, cat(ylo, ylo), D);
                const bf16x4 dlo = split_lo(D, NIL, dhh);
                const bf16x8 dll = cat(dlo, dlo);
                // S <- (Diag(Gamma) S, formed above) + K~^T Delta
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const bf16x8 ktt = cat(ktr[b].hi, ktr[b].lo);
                    const f32x4 acc = mma32(ktt, dhh, S[b]);
                    S[b] = mma32(ktt, dll, acc);
                }
                // O = Q+ S + A_qk Delta
                const bf16x8 aqq = cat(Aq.hi, Aq.lo);
                f32x4 O = mma32(aqq, dhh, Oa);
                O = mma32(aqq, dll, O);
                O += Ob + Oc;
                const rsrc_t ro = rsrc_out(c);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    buf_store_f32(O[jj], ro, (4 * g4 + jj) * rowO + (col0 + l16) * 4u);
            };

            // Chunk c uses operand set c & 1 and the inputs loaded three chunks
            // earlier; the register sets rotate X0 -> X1 -> X2.
            CIn X0, X1, X2;
            cload(X0, 0);
            cload(X1, 1);
            cload(X2, 2);
            __syncthreads();  // operand set 0 ready
            // Everything loaded so far (state, first inputs) has arrived before the loop: the
            // wait-count pass otherwise merges these loads, issued with few others after them,
            // into the loop header and makes the first chunks of every unrolled trip wait for
            // the loads and stores of the chunk just before.
            __builtin_amdgcn_s_waitcnt(0);
            auto citer = [&](int c, CIn &X) {
                advance(c & 1, X, c);
                cload(X, c + 3);
                __syncthreads();  // set c+1 ready; set c free
            };
            // Whole groups of three in the loop and the remainder after it: with
            // an exit inside the loop body the compiler merged the loop's entry
            // and back edge conservatively and waited there for every load in
            // flight, including the ones issued just before.
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
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    fin[(hd * DK + mrow(b, jj)) * DV + col0 + l16] = S[b][jj];
        }
    } else if (nc > 0) {
        // ============================================================ producer
        // Producer pw builds the operands of channel blocks pw * BPW .. + BPW - 1.
        const int pw = role + NP;
        // Constant 0/1 triangles as matrix-core operands (bf16 1.0 = 0x3f80):
        //   LT, B operand of G^T = g^T L^T: lane (g4, n) holds L[n][4 g4 + j] = [4 g4 + j <= n];
        //   UT, A operand of Gs  = U g:     lane (g4, i) holds U[i][4 g4 + j] = [4 g4 + j >  i].
        // G_r = sum_{t <= r} g_t is the cumulative log-decay, Gs_r = sum_{t > r} g_t = G_n - G_r.
        u16x4 lt_bits, ut_bits;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lt_bits[j] = (4 * g4 + j <= l16) ? 0x3f80 : 0;
            ut_bits[j] = (4 * g4 + j > l16) ? 0x3f80 : 0;
        }
        const bf16x4 LT = __builtin_bit_cast(bf16x4, lt_bits);
        const bf16x4 UT = __builtin_bit_cast(bf16x4, ut_bits);
        const bf16x4 ID = identity_operand(g4, l16);
        // Raw q, k, g.  Inside the kernel the 32 channels of block pair P are
        // ordered so that what one lane needs of the pair -- channels 4 g4 .. +3 of
        // block 2P and of block 2P+1 -- are the eight consecutive memory channels
        // 32 P + 8 g4 .. +7:
        //     internal channel 16 (2P + h) + 4 g4 + j  <->  memory channel 32 P + 8 g4 + 4 h + j
        // (a relabelling of the key channels; the state rows follow it).  Loads then
        // read whole 64-byte pieces of a pair's token row with four consecutive lanes
        // per row (lane L: row L / 4, bytes 16 (L % 4)), so the address unit sees
        // one cache line per four lanes instead of one per lane, and a round trip
        // through the wave's own LDS stage gives the operand layout (lane (g4, l16):
        // token l16, the 16 bytes at 16 g4).
        constexpr int NPW = (BPW + 1) / 2;  // block pairs this wave touches
        const int pair0 = (pw * BPW) / 2;
        struct PIn {
            u32x4 d[3][NPW];  // q, k, g
        };
        auto pload = [&](PIn &R, int c) {
            const rsrc_t rq = rsrc_in(q, c, DK, 1u), rk = rsrc_in(k, c, DK, 1u), rg = rsrc_in(g, c, DK, 1u);
#pragma unroll
            for (int pp = 0; pp < NPW; ++pp) {
                const uint32_t off = (lane >> 2) * rowK + 64u * (pair0 + pp) + 16u * (lane & 3);
                R.d[0][pp] = buf_load_u32x4(rq, off);
                R.d[1][pp] = buf_load_u32x4(rk, off);
                R.d[2][pp] = buf_load_u32x4(rg, off);
            }
        };
        // Per-wave stage: 16 token rows of 64 bytes per (tensor, pair), rows padded to
        // 80 bytes so the operand-layout reads (16 rows, one 16-byte piece each) hit
        // distinct banks.
        __shared__ __attribute__((aligned(16))) u32x4 stage[NP][3][NPW][16][5];
        auto stage_put = [&](const PIn &R) {
#pragma unroll
            for (int t = 0; t < 3; ++t)
#pragma unroll
                for (int pp = 0; pp < NPW; ++pp) stage[pw][t][pp][lane >> 2][lane & 3] = R.d[t][pp];
        };
        auto stage_get = [&](PIn &A) {
#pragma unroll
            for (int t = 0; t < 3; ++t)
#pragma unroll
                for (int pp = 0; pp < NPW; ++pp) A.d[t][pp] = stage[pw][t][pp][l16][g4];
        };
        // The 8 bytes of block half h (0: block 2P, 1: block 2P+1) in a staged piece.
        auto half = [](const u32x4 &x, int h) { return h ? u32x2{x[2], x[3]} : u32x2{x[0], x[1]}; };
        // The wave's channel blocks are handled in pairs, so every 32-long operand
        // carries two blocks' data and a constant operand with the wanted matrix in
        // one half (0 in the other) selects the block: no operand is padded.
        const bf16x4 z4 = {};
        const bf16x8 IDL = cat(ID, z4), IDH = cat(z4, ID), LTL = cat(LT, z4), LTH = cat(z4, LT);
        const bf16x8 UTL = cat(UT, z4), UTH = cat(z4, UT);
        const bf16x8 NIL = neg_identity_operand<0>(g4, l16), NIH = neg_identity_operand<1>(g4, l16);
        auto produce = [&](const PIn &A, int ob) {
            WsOps<DK> &P = ops[ob];
#pragma unroll
            for (int pp = 0; pp < NPW; ++pp) {
                // blocks b0, b1 of this pair; a wave with one block (BPW = 1) pairs it with itself
                const int hb = (BPW == 1) ? (pw & 1) : 0;
                const int b0 = (BPW == 1) ? pw : pw * BPW + 2 * pp, b1 = (BPW == 1) ? pw : b0 + 1;
                const u32x2 Rq[2] = {half(A.d[0][pp], hb), half(A.d[0][pp], BPW == 1 ? hb : 1)};
                const u32x2 Rk[2] = {half(A.d[1][pp], hb), half(A.d[1][pp], BPW == 1 ? hb : 1)};
                const u32x2 Rg[2] = {half(A.d[2][pp], hb), half(A.d[2][pp], BPW == 1 ? hb : 1)};
                const bf16x8 ga = cat(__builtin_bit_cast(bf16x4, Rg[0]), __builtin_bit_cast(bf16x4, Rg[1]));
                const bf16x8 ka = cat(__builtin_bit_cast(bf16x4, Rk[0]), __builtin_bit_cast(bf16x4, Rk[1]));
                // g and k as tokens 4 g4 + jj of channel 16 b + l16 (exact: bf16 values)
                const bf16x8 gf = cat(to_bf16x4(mma32(ga, IDL, zero4())), to_bf16x4(mma32(ga, IDH, zero4())));
                const f32x4 kc[2] = {mma32(ka, IDL, zero4()), mma32(ka, IDH, zero4())};
                // G at token l16, channels 16 b + 4 g4 + jj; Gs at tokens 4 g4 + jj, channel 16 b + l16
                const f32x4 GT[2] = {mma32(gf, LTL, zero4()), mma32(gf, LTH, zero4())};
                const f32x4 GS[2] = {mma32(UTL, gf, zero4()), mma32(UTH, gf, zero4())};
                f32x4 Pp[2], qv[2], ktv[2], kpv[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    f32x4 F;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        Pp[u][j] = decay_exp_fast(GT[u][j]);   // e^{G_r}
                        F[j] = decay_exp_fast(GS[u][j]);       // e^{G_n - G_r}
                    }
                    qv[u] = unpack_bf16x4(Rq[u]) * Pp[u];
                    kpv[u] = unpack_bf16x4(Rk[u]) * Pp[u];
                    ktv[u] = kc[u] * F;
                }
                // Q+, K+ and K~ as hi + lo (all held in the accumulator layout of a tile:
                // Q+^T, K+^T and K~), residuals from the matrix core
                const bf16x8 qh = cat(to_bf16x4(qv[0]), to_bf16x4(qv[1]));
                const bf16x8 kph = cat(to_bf16x4(kpv[0]), to_bf16x4(kpv[1]));
                const bf16x8 kth = cat(to_bf16x4(ktv[0]), to_bf16x4(ktv[1]));
                const bf16x4 ql[2] = {to_bf16x4(mma32(NIL, qh, qv[0])), to_bf16x4(mma32(NIH, qh, qv[1]))};
                const bf16x4 kpl[2] = {to_bf16x4(mma32(NIL, kph, kpv[0])), to_bf16x4(mma32(NIH, kph, kpv[1]))};
                const bf16x4 ktl[2] = {to_bf16x4(mma32(NIL, kth, ktv[0])), to_bf16x4(mma32(NIH, kth, ktv[1]))};
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    if (u == 1 && b1 == b0) break;
                    const int b = u ? b1 : b0;
                    bf16x4 *qhp = reinterpret_cast<bf16x4 *>(&P.qp_hi[b >> 1][lane]) + (b & 1);
                    bf16x4 *qlp = reinterpret_cast<bf16x4 *>(&P.qp_lo[b >> 1][lane]) + (b & 1);
                    bf16x4 *kpp = reinterpret_cast<bf16x4 *>(&P.kp[b >> 1][lane]) + (b & 1);
                    bf16x4 *kplp = reinterpret_cast<bf16x4 *>(&P.kp_lo[b >> 1][lane]) + (b & 1);
                    *qhp = u ? __builtin_shufflevector(qh, qh, 4, 5, 6, 7) : __builtin_shufflevector(qh, qh, 0, 1, 2, 3);
                    *qlp = ql[u];
                    *kpp = u ? __builtin_shufflevector(kph, kph, 4, 5, 6, 7) : __builtin_shufflevector(kph, kph, 0, 1, 2, 3);
                    *kplp = kpl[u];
                    P.kt[b][lane] = Split4{u ? __builtin_shufflevector(kth, kth, 4, 5, 6, 7)
                                             : __builtin_shufflevector(kth, kth, 0, 1, 2, 3),
                                           ktl[u]};
                    if (l16 == 15) *reinterpret_cast<f32x4 *>(&P.gam[16 * b + 4 * g4]) = Pp[u];
                }
            }
        };

        // Iteration c builds the operands of chunk c+1 into set (c+1) & 1, then
        // passes chunk c+2 (registers loaded three iterations earlier) through the
        // stage, so its LDS latency falls in the barrier wait, and reuses those
        // registers for chunk c+5; register sets rotate R2 -> R0 -> R1.
        PIn R0, R1, R2, A;
        pload(R0, 0);
        pload(R1, 1);
        pload(R2, 2);
        stage_put(R0);
        stage_get(A);  // (the wave's own LDS accesses stay in order)
        produce(A, 0);
        stage_put(R1);
        stage_get(A);
        pload(R0, 3);
        pload(R1, 4);
        __syncthreads();  // operand set 0 ready
        auto piter = [&](int c, PIn &R) {
            produce(A, (c + 1) & 1);
            stage_put(R);
            stage_get(A);
            pload(R, c + 5);
            __syncthreads();
        };
        int c = 0;  // (loop form as for the consumers)
        for (; c + 3 <= nc; c += 3) {
            piter(c, R2);
            piter(c + 1, R0);
            piter(c + 2, R1);
        }
        if (c < nc) piter(c, R2);
        if (c + 1 < nc) piter(c + 1, R0);
    }
}

template <int DK, int DV, int NC, int NP>
static hipError_t launch_ws_t(const InterChunkArgs &a) {
    const int nchains = a.nseq * a.H;
    const int nsplit = DV / (16 * NC);
    const int64_t grid = ((int64_t)nchains + 7) / 8 * 8 * nsplit;
    const int nsort = a.nseq <= LPT_MAX_SEQS ? a.nseq : 0;
    if (a.layer) {
        if constexpr (DK == 128 && DV == 128) {
            hipLaunchKernelGGL((inter_chunk_ws_kernel<DK, DV, NC, NP, true>), dim3((unsigned)grid),
                               dim3(64 * WsLayout<NC, NP>::NW), 0, (hipStream_t)a.stream, (const __bf16 *)a.q,
                               (const __bf16 *)a.k, (const __bf16 *)a.v, (const __bf16 *)a.g, a.init, a.cu,
                               a.H, a.ws, a.o, a.fin, nsplit, nchains, *a.layer, a.skip, nsort);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL((inter_chunk_ws_kernel<DK, DV, NC, NP, false>), dim3((unsigned)grid),
                       dim3(64 * WsLayout<NC, NP>::NW), 0, (hipStream_t)a.stream, (const __bf16 *)a.q,
                       (const __bf16 *)a.k, (const __bf16 *)a.v, (const __bf16 *)a.g, a.init, a.cu,
                       a.H, a.ws, a.o, a.fin, nsplit, nchains, LayerPrologue{}, a.skip, nsort);
    return hipGetLastError();
}

// Shapes: consumers NC (16 columns each), producers NP.  Returns
// hipErrorInvalidValue for a shape that is not instantiated.
// Shapes built: for dk = dv = 128 four or two consumers with four producers; for the other
// head sizes min(dv/16, 4) or min(dv/16, 2) consumers with min(dk/16, 4) producers.
#define KDA_WS_SHAPES(CASE) \
    CASE(128, 128, 4, 4) CASE(128, 128, 2, 4) \
    KDA_WS_ROW(CASE, 32) KDA_WS_ROW(CASE, 64) KDA_WS_ROW(CASE, 128)
#define KDA_WS_DEF(CASE, DKV, DVV) CASE(DKV, DVV, ((DVV / 16) < 4 ? (DVV / 16) : 4), ((DKV / 16) < 4 ? (DKV / 16) : 4))
#define KDA_WS_DEF2(CASE, DKV, DVV) CASE(DKV, DVV, ((DVV / 16) < 2 ? (DVV / 16) : 2), ((DKV / 16) < 4 ? (DKV / 16) : 4))
#define KDA_WS_ROW(CASE, DKV) KDA_WS_DEF(CASE, DKV, 16) KDA_WS_DEF(CASE, DKV, 32) KDA_WS_DEF(CASE, DKV, 64) \
    KDA_WS_DEF(CASE, DKV, 128) KDA_WS_DEF2(CASE, DKV, 64) KDA_WS_DEF2(CASE, DKV, 128)

bool inter_chunk_ws_shape_built(int dk, int dv, int ncw, int npw) {
#define KDA_WS_HAS(DKV, DVV, NCV, NPV) if (dk == DKV && dv == DVV && ncw == NCV && npw == NPV) return true;
    KDA_WS_SHAPES(KDA_WS_HAS)
#undef KDA_WS_HAS
    return false;
}

hipError_t launch_inter_chunk_ws(const InterChunkArgs &a, int ncw, int npw) {
#define KDA_WS_CASE(DKV, DVV, NCV, NPV) \
    if (a.dk == DKV && a.dv == DVV && ncw == NCV && npw == NPV) return launch_ws_t<DKV, DVV, NCV, NPV>(a);
    KDA_WS_SHAPES(KDA_WS_CASE)
#undef KDA_WS_CASE
    return hipErrorInvalidValue;
}
#undef KDA_WS_ROW
#undef KDA_WS_DEF2
#undef KDA_WS_DEF
#undef KDA_WS_SHAPES

}  // namespace kda
