// Inter-chunk phase of the KDA prefill (gfx950): the sequential state
// propagation over the 16-token chunks of each sequence.
//
// For a chunk with incoming state S (dk x dv), per-channel prefix products
// P_r = e^{G_r}, Gamma = P_n, and F_r = e^{G_n - G_r}:
//     K+ = K (.) P,   Q+ = Q (.) P,   K~ = K (.) F
//     Delta = T' (V - K+ S)            (= U - W S with W = T' K+, U = T' V)
//     O     = Q+ S + A_qk Delta
//     S    <- Diag(Gamma) S + K~^T Delta
// (Kimi K3 report digest, "Kimi Delta Attention": chunk output = inter-chunk
// term (Gamma (.) Q) S + intra-chunk term A V~; T' and A_qk come from the
// chunk-local phase.)
//
// Work split: the columns of S evolve independently once T', A_qk, K+, Q+, K~
// are known (the transition multiplies S from the left), so each wave owns a
// 16-column slice of dv and keeps its 16 x dk x fp32 state slice in registers
// for the whole sequence.  A workgroup of NW waves covers NW slices of one
// (sequence, head) and shares the chunk-dependent operands through LDS:
//   * prep1: per key channel, one "prefix" job (e^{G_r}, Gamma) and one
//     "suffix" job (K~ = K (.) e^{G_15 - G_r}), spread over all threads; T' and
//     A_qk fragments from the workspace;
//   * prep2 (one item per (token, 4 channels)): Q+ and K+ fragments.
// The prep of chunk c+1 runs while the waves advance the state through chunk
// c (double-buffered LDS, two barriers per chunk), and the raw inputs of
// chunk c+2 are loaded into registers meanwhile.  Inputs are read through
// buffer resources whose base is the chunk's first token (uniform, in SGPRs):
// per-lane offsets stay constant from chunk to chunk, and the rows of a ragged
// last chunk are parked out of bounds so the hardware returns zeros.  This overlaps the
// token-parallel work with the serial recurrence, as the page's KDA systems
// section describes for its own chunkwise kernel.
//
// Precision: K+ S uses single-bf16 operands; T'(V - K+S), Q+ S, A_qk Delta and
// K~^T Delta use split-bf16 (hi*hi + lo*hi + hi*lo) with fp32 accumulation;
// the state stays fp32.  fp32 inputs use fp32 MFMAs throughout.
#include <stdio.h>

#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int DK, int DV, typename T, int NW>
struct IC {
    static constexpr bool F32 = sizeof(T) == 4;
    static constexpr uint32_t EB = sizeof(T);               // input element bytes
    static constexpr int NT = 64 * NW;
    static constexpr int NB = DK / 16;                       // 16-channel key blocks
    static constexpr int NPAIR = (NB + 1) / 2;               // block pairs (one K=32 MFMA each)
    static constexpr int UNITS = 4 * DK;                     // (token, 4-channel group) units of a chunk tile
    static constexpr int UPT = (UNITS + NT - 1) / NT;
    // prep1 splits each key channel's 16 tokens into NPART parts (1, 2 or 4) held
    // by lanes of one wave, CPW channels per wave, TP tokens per part; with fewer
    // threads than channels each thread takes CPT channels.
    static constexpr int NPART = (NT / DK) >= 4 ? 4 : ((NT / DK) >= 2 ? 2 : 1);
    static constexpr int CPW = 64 / NPART;
    static constexpr int TP = 16 / NPART;
    static constexpr int CPT = DK > NT ? DK / NT : 1;
    static constexpr bool PREP1_FULL = NW * CPW * CPT == DK;   // every thread owns a real channel
    static constexpr bool UNITS_FULL = (UNITS % NT) == 0;
    static constexpr int VW = 16 * NW;                       // v columns of this workgroup
    static constexpr int MU = 2 * 16 * 16 * 4 / 8;           // T' + A_qk fragments in 8-byte units (256)
    static constexpr int MPT = (MU + NT - 1) / NT;
    static constexpr int LDT = DK + (F32 ? 4 : 8);           // padded stage row (elements)
    using OpT = std::conditional_t<F32, f32x4, Split4>;     // split operand fragment (K~, T', A_qk)
    using Raw4 = std::conditional_t<F32, u32x4, u32x2>;     // four raw input elements
};

// LDS operand set of one chunk.
//   qp_hi/qp_lo[p][lane]: Q+ for block pair p in the A-fragment layout, the two
//     blocks' four-element halves packed back to back (one K=32 MFMA operand);
//   kp[p][lane]: K+ (single bf16), same packing;
//   kt[b][lane]: K~ for block b in the K-side layout, {hi, lo};
//   gam: e^{G_n} per channel.
// (T' and A_qk arrive from the chunk-local phase already in fragment form and
// are loaded by each wave straight into registers.)
template <int DK, typename T>
struct OpsBF16 {
    static constexpr int NB = DK / 16, NPAIR = (NB + 1) / 2;
    bf16x8 qp_hi[NPAIR][64];
    bf16x8 qp_lo[NPAIR][64];
    bf16x8 kp[NPAIR][64];
    Split4 kt[NB][64];
    float gam[DK];
};

template <int DK, typename T>
struct OpsF32 {
    static constexpr int NB = DK / 16;
    f32x4 qp[NB][64];
    f32x4 kp[NB][64];
    f32x4 kt[NB][64];
    float gam[DK];
};

template <typename O>
__device__ __forceinline__ O make_op(f32x4 x) {
    if constexpr (std::is_same_v<O, f32x4>) return x;
    else return split4(x);
}

template <typename O>
__device__ __forceinline__ void set_op_elem(O &dst, int slot, float x) {
    if constexpr (std::is_same_v<O, f32x4>) {
        dst[slot] = x;
    } else {
        const __bf16 h = f32_to_bf16(x);
        dst.hi[slot] = h;
        dst.lo[slot] = f32_to_bf16(x - bf16_to_f32(h));
    }
}

template <bool F32>
__device__ __forceinline__ float gate_exp(float x) {
    if constexpr (F32) return decay_exp(x);
    else return decay_exp_fast(x);
}

// Split a pair of state tiles into pair-packed bf16 operands.
__device__ __forceinline__ void split_pair(const f32x4 &a, const f32x4 &b, bf16x8 &hi, bf16x8 &lo) {
    const bf16x4 ah = to_bf16x4(a), bh = to_bf16x4(b);
    const bf16x4 al = to_bf16x4(a - from_bf16x4(ah)), bl = to_bf16x4(b - from_bf16x4(bh));
    hi = cat(ah, bh);
    lo = cat(al, bl);
}

template <int DK, int DV, typename T, int NW>
__global__ __launch_bounds__(64 * NW, (NW >= 4 ? 2 : 1)) void inter_chunk_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ g, const float *__restrict__ init, const int32_t *__restrict__ cu,
    int32_t nseq, int32_t H, const float *__restrict__ ws, float *__restrict__ o,
    float *__restrict__ fin, int32_t nsplit, int32_t nchains, const int32_t *__restrict__ skip) {
    using C = IC<DK, DV, T, NW>;
    using OpT = typename C::OpT;
    using Raw4 = typename C::Raw4;
    using Ops = std::conditional_t<C::F32, OpsF32<DK, T>, OpsBF16<DK, T>>;
    constexpr bool F32 = C::F32;
    constexpr uint32_t EB = C::EB;
    constexpr int NT = C::NT, NB = C::NB, NPAIR = C::NPAIR, UPT = C::UPT;
    constexpr int NPART = C::NPART, CPW = C::CPW, TP = C::TP, CPT = C::CPT;
    constexpr int LDT = C::LDT;

    // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin by
    // linear id, so all slices of one (sequence, head) get the same id mod 8
    // and share that XCD's L2 for the q/k/g/workspace reads.
    const int L = blockIdx.x;
    const int xcd = L & 7;
    const int sx = L >> 3;
    const int split = sx % nsplit;
    const int chain = (sx / nsplit) * 8 + xcd;
    if (chain >= nchains) return;
    if (skip && skip[chain]) return;  // (context parallelism: a transition known to be negligible)
    const int s = chain / H, h = chain % H;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int g4 = lane >> 4, n16 = lane & 15;
    const int col0 = (split * NW + wave) * 16;

    constexpr int VW = C::VW, MPT = C::MPT;
    // (vector loads/stores of 8 and 16 bytes address these arrays: 16-byte aligned)
    __shared__ __attribute__((aligned(16))) Ops ops[2];
    __shared__ __attribute__((aligned(16))) T stq[2][16][LDT];   // raw chunk tiles, token-major
    __shared__ __attribute__((aligned(16))) T stk[2][16][LDT];
    __shared__ __attribute__((aligned(16))) T stg[2][16][LDT];
    __shared__ __attribute__((aligned(16))) T stv[2][16][VW + 4];         // this workgroup's v columns
    __shared__ __attribute__((aligned(16))) uint32_t stm[2][2 * 16 * 16]; // T', A_qk fragments (workspace copy)
    __shared__ __attribute__((aligned(16))) float sP[16][DK + 4];

    const int64_t bos = cu[s], eos = cu[s + 1];
    const int nc = (int)((eos - bos + 15) / 16);
    const int64_t slot0 = bos / 16 + s;
    const int64_t hd = (int64_t)s * H + h;
    const uint32_t rowK = (uint32_t)H * DK * EB;   // bytes between tokens in q, k, g
    const uint32_t rowV = (uint32_t)H * DV * EB;   // ... in v
    const uint32_t rowO = (uint32_t)H * DV * 4;    // ... in o

    // ---- state slice: rows 16b + 4*g4 + jj, column col0 + n16 (frag4 layout)
    f32x4 S[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            S[b][jj] = init ? init[(hd * DK + 16 * b + 4 * g4 + jj) * DV + col0 + n16] : 0.f;

    auto chunk_len = [&](int c) -> int {
        const int64_t left = eos - (bos + 16 * (int64_t)c);
        return left < 16 ? (int)left : 16;
    };
    // Buffer resource of chunk c for this head: base = the head's slice of the
    // chunk's first token.  Rows at or past the chunk length are parked at an
    // out-of-bounds offset, so their loads return zeros and stores are dropped.
    // A NULL v (a pass that only propagates the state's transition) reads as zeros and a
    // NULL o is not written: their resources get length 0 (on q as a stand-in base),
    // decided once here rather than by a null test at each resource.
    const uint32_t v_on = v ? 1u : 0u, o_on = o ? 1u : 0u;
    const T *vb = v ? v : q;
    float *obase = o ? o : reinterpret_cast<float *>(const_cast<T *>(q));
    auto rsrc_in = [&](const T *base, int c, int d, uint32_t on) {
        const int64_t t0 = bos + 16 * (int64_t)c;
        const int n = chunk_len(c);
        return make_rsrc(base + (t0 * H + h) * d, (uint32_t)(n > 0 ? n : 0) * (uint32_t)H * d * EB * on);
    };
    // Look-ahead loads past the last chunk re-read the last chunk (results unused).
    auto clampc = [&](int c) { return c < nc ? c : nc - 1; };

    // ---- raw loads of one chunk, all issued together three chunks ahead and
    // parked in the LDS stage one chunk ahead:
    //   q, k, g tiles: unit u = (token u / (DK/4), channels 4 (u % (DK/4)) .. +3);
    //   v: unit = (token, 4 of this workgroup's columns) -- one per thread;
    //   T' and A_qk fragments: 2 KiB copied in 8-byte units.
    struct Units {
        Raw4 q[UPT], k[UPT], g[UPT];
        Raw4 v;
        u32x2 m[MPT];
    };
    auto load_units = [&](Units &U, int c) {
        const int n = chunk_len(c);
        const rsrc_t rq = rsrc_in(q, c, DK, 1u), rk = rsrc_in(k, c, DK, 1u), rg = rsrc_in(g, c, DK, 1u);
#pragma unroll
        for (int ui = 0; ui < UPT; ++ui) {
            const int u = tid + ui * NT;
            const int t = u / (DK / 4), a = u % (DK / 4);
            const uint32_t off = (u < C::UNITS && t < n) ? t * rowK + 4 * a * EB : OOB;
            if constexpr (F32) {
                U.q[ui] = buf_load_u32x4(rq, off);
                U.k[ui] = buf_load_u32x4(rk, off);
                U.g[ui] = buf_load_u32x4(rg, off);
            } else {
                U.q[ui] = buf_load_u32x2(rq, off);
                U.k[ui] = buf_load_u32x2(rk, off);
                U.g[ui] = buf_load_u32x2(rg, off);
            }
        }
        {
            const rsrc_t rv = rsrc_in(vb, c, DV, v_on);
            const int t = tid / (VW / 4), a = tid % (VW / 4);
            const uint32_t off = t < n ? t * rowV + (split * VW + 4 * a) * EB : OOB;
            if constexpr (F32) U.v = buf_load_u32x4(rv, off);
            else U.v = buf_load_u32x2(rv, off);
        }
        const u32x2 *w = reinterpret_cast<const u32x2 *>(ws + ((slot0 + c) * H + h) * (int64_t)WS_FLOATS_PER_CHUNK_HEAD);
#pragma unroll
        for (int mi = 0; mi < MPT; ++mi) {
            const int e = tid + mi * NT;
            U.m[mi] = w[e < C::MU ? e : C::MU - 1];
        }
    };
    auto store_units = [&](const Units &U, int sb) {
#pragma unroll
        for (int ui = 0; ui < UPT; ++ui) {
            const int u = tid + ui * NT;
            if (C::UNITS_FULL || u < C::UNITS) {
                const int t = u / (DK / 4), a = u % (DK / 4);
                *reinterpret_cast<Raw4 *>(&stq[sb][t][4 * a]) = U.q[ui];
                *reinterpret_cast<Raw4 *>(&stk[sb][t][4 * a]) = U.k[ui];
                *reinterpret_cast<Raw4 *>(&stg[sb][t][4 * a]) = U.g[ui];
            }
        }
        {
            const int t = tid / (VW / 4), a = tid % (VW / 4);
            *reinterpret_cast<Raw4 *>(&stv[sb][t][4 * a]) = U.v;
        }
#pragma unroll
        for (int mi = 0; mi < MPT; ++mi) {
            const int e = tid + mi * NT;
            if (e < C::MU) *reinterpret_cast<u32x2 *>(&stm[sb][2 * e]) = U.m[mi];
        }
    };

    // ---- per-wave operands of the chunk in stage buffer sb: T' and A_qk
    // fragments, and the v fragment (rows 4*g4 + jj, column col0 + n16).
    struct Frags {
        OpT tp, aq;
    };
    auto stage_frags = [&](int sb) {
        Frags F;
        F.tp = reinterpret_cast<const OpT *>(&stm[sb][0])[lane];
        F.aq = reinterpret_cast<const OpT *>(&stm[sb][0])[64 + lane];
        return F;
    };
    auto stage_v = [&](int sb) {
        f32x4 r;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) r[jj] = load_in(&stv[sb][4 * g4 + jj][wave * 16 + n16]);
        return r;
    };

    // ---- prep1 (chunk in stage buffer sb -> operand set ob): per key channel, the
    // running products of alpha = e^{g} over the chunk's tokens (padding tokens
    // hold g = 0, i.e. alpha = 1): P_r = e^{G_r} (to LDS for prep2), Gamma = P_15,
    // and K~_r = k_r e^{G_15 - G_r}.  A thread takes TP consecutive tokens of one
    // channel, forms local prefix / suffix products, and combines them with the
    // other parts of the channel through two lane shuffles at most; every thread
    // runs the same instruction stream.
    auto prep1 = [&](int sb, int ob) {
        const int part = lane / CPW;
        const int r0 = part * TP;
#pragma unroll
        for (int ci = 0; ci < CPT; ++ci) {
            const int ch = wave * CPW + (lane % CPW) + ci * NT;
            const bool valid = ch < DK;
            const int chc = valid ? ch : 0;
            float a[TP], kk[TP], lp[TP], ls[TP];
#pragma unroll
            for (int i = 0; i < TP; ++i) {
                a[i] = gate_exp<F32>(load_in(&stg[sb][r0 + i][chc]));
                kk[i] = load_in(&stk[sb][r0 + i][chc]);
            }
            float p = 1.f;
#pragma unroll
            for (int i = 0; i < TP; ++i) {
                p *= a[i];
                lp[i] = p;
            }
            float f = 1.f;
#pragma unroll
            for (int i = TP - 1; i >= 0; --i) {
                ls[i] = f;
                f *= a[i];
            }
            // combine the parts: pre = product of earlier parts, suf = of later parts
            float pre = 1.f, suf = 1.f, tot = p;
            if constexpr (NPART == 2) {
                const float o1 = __shfl_xor(p, 32);
                pre = part ? o1 : 1.f;
                suf = part ? 1.f : o1;
                tot = p * o1;
            } else if constexpr (NPART == 4) {
                const float o1 = __shfl_xor(p, 16);
                const float pp = p * o1;
                const bool low = (part & 1) == 0;
                const float o2 = __shfl_xor(pp, 32);
                const bool lowpair = part < 2;
                pre = (low ? 1.f : o1) * (lowpair ? 1.f : o2);
                suf = (low ? o1 : 1.f) * (lowpair ? o2 : 1.f);
                tot = pp * o2;
            }
            if (C::PREP1_FULL || valid) {
#pragma unroll
                for (int i = 0; i < TP; ++i) sP[r0 + i][ch] = pre * lp[i];
                if (part == 0) ops[ob].gam[ch] = tot;
#pragma unroll
                for (int qi = 0; qi < TP / 4; ++qi) {
                    const int tq = r0 / 4 + qi;
                    f32x4 kt;
#pragma unroll
                    for (int j = 0; j < 4; ++j) kt[j] = kk[4 * qi + j] * (ls[4 * qi + j] * suf);
                    ops[ob].kt[ch >> 4][tq * 16 + (ch & 15)] = make_op<OpT>(kt);
                }
            }
        }
    };

    // ---- prep2: per unit (token, 4 channels), Q+ and K+ fragments from P.
    auto prep2 = [&](int sb, int ob) {
#pragma unroll
        for (int ui = 0; ui < UPT; ++ui) {
            const int u = tid + ui * NT;
            if (C::UNITS_FULL || u < C::UNITS) {
                const int t = u / (DK / 4), a = u % (DK / 4);
                const int c = 4 * a;
                const f32x4 P = *reinterpret_cast<const f32x4 *>(&sP[t][c]);
                const f32x4 qv = load_in4(&stq[sb][t][c]) * P;
                const f32x4 kv = load_in4(&stk[sb][t][c]) * P;
                const int b = c >> 4;
                const int ln = ((c & 15) >> 2) * 16 + t;
                if constexpr (F32) {
                    ops[ob].qp[b][ln] = qv;
                    ops[ob].kp[b][ln] = kv;
                } else {
                    const Split4 qs = split4(qv);
                    bf16x4 *qh = reinterpret_cast<bf16x4 *>(&ops[ob].qp_hi[b >> 1][ln]) + (b & 1);
                    bf16x4 *ql = reinterpret_cast<bf16x4 *>(&ops[ob].qp_lo[b >> 1][ln]) + (b & 1);
                    bf16x4 *kh = reinterpret_cast<bf16x4 *>(&ops[ob].kp[b >> 1][ln]) + (b & 1);
                    *qh = qs.hi;
                    *ql = qs.lo;
                    *kh = to_bf16x4(kv);
                    if constexpr (NB == 1) {  // a lone block: the pair's upper half must be zero
                        const bf16x4 z = {};
                        qh[1] = z;
                        ql[1] = z;
                        kh[1] = z;
                    }
                }
            }
        }
    };

    // ---- one chunk of the recurrence for this wave's 16 columns (operand set ob)
    auto advance = [&](int ob, f32x4 vc, const Frags &F, int c) {
        const Ops &P = ops[ob];
        f32x4 O;
        if constexpr (F32) {
            f32x4 X = zero4();
#pragma unroll
            for (int b = 0; b < NB; ++b) X = mma_f32_k16(P.kp[b][lane], S[b], X);
            const f32x4 D = mma_f32_k16(F.tp, vc - X, zero4());
            O = mma_f32_k16(F.aq, D, zero4());
#pragma unroll
            for (int b = 0; b < NB; ++b) O = mma_f32_k16(P.qp[b][lane], S[b], O);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const f32x4 gam = *reinterpret_cast<const f32x4 *>(&P.gam[16 * b + 4 * g4]);
                S[b] = mma_f32_k16(P.kt[b][lane], D, S[b] * gam);
            }
        } else {
            bf16x8 Shi[NPAIR], Slo[NPAIR];
            const bf16x4 z = {};
#pragma unroll
            for (int p = 0; p < NPAIR; ++p) {
                if constexpr (NB == 1) {
                    const Split4 s0 = split4(S[0]);
                    Shi[p] = cat(s0.hi, z);
                    Slo[p] = cat(s0.lo, z);
                } else {
                    split_pair(S[2 * p], S[2 * p + 1], Shi[p], Slo[p]);
                }
            }
            // X = K+ S (single bf16), Delta = T' (V - X) (split), O = A_qk Delta + Q+ S (split)
            f32x4 X = zero4();
#pragma unroll
            for (int p = 0; p < NPAIR; ++p) X = mma32(P.kp[p][lane], Shi[p], X);
            const Split4 Ys = split4(vc - X);
            const Split4 &Tp = F.tp;
            const bf16x8 tpp = cat(Tp.hi, Tp.lo);
            f32x4 D = mma32(tpp, cat(Ys.hi, Ys.hi), zero4());
            D = mma32(tpp, cat(Ys.lo, Ys.lo), D);
            const Split4 Ds = split4(D);
            const bf16x8 dhh = cat(Ds.hi, Ds.hi), dll = cat(Ds.lo, Ds.lo);
            const Split4 &Aq = F.aq;
            const bf16x8 aqq = cat(Aq.hi, Aq.lo);
            O = mma32(aqq, dhh, zero4());
            O = mma32(aqq, dll, O);
#pragma unroll
            for (int p = 0; p < NPAIR; ++p) {
                O = mma32(P.qp_hi[p][lane], Shi[p], O);
                O = mma32(P.qp_lo[p][lane], Shi[p], O);
                O = mma32(P.qp_hi[p][lane], Slo[p], O);
            }
            // S <- Diag(Gamma) S + K~^T Delta
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const f32x4 gam = *reinterpret_cast<const f32x4 *>(&P.gam[16 * b + 4 * g4]);
                const Split4 kt = P.kt[b][lane];
                const bf16x8 ktt = cat(kt.hi, kt.lo);
                f32x4 acc = mma32(ktt, dhh, S[b] * gam);
                S[b] = mma32(ktt, dll, acc);
            }
        }
        const int64_t t0 = bos + 16 * (int64_t)c;
        const int n = chunk_len(c);
        const rsrc_t ro = make_rsrc(obase + (t0 * H + h) * DV, (uint32_t)n * rowO * o_on);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int t = 4 * g4 + jj;
            buf_store_f32(O[jj], ro, t < n ? t * rowO + (col0 + n16) * 4u : OOB);
        }
    };

    // Pipeline (iteration c): [barrier] advance(c) || prep1(c+1) [barrier]
    // prep2(c+1); park the raw loads of chunk c+2 (issued one iteration earlier)
    // in the stage buffer chunk c just vacated; issue the loads of chunk c+3.
    // The body is branch-free: look-ahead past the last chunk re-reads the last
    // chunk and fills buffers nobody reads, so the compiler can interleave the
    // recurrence with the prep, and the only wait on global loads sits one full
    // iteration after their issue.
    if (nc > 0) {
        Units U;
        load_units(U, 0);
        store_units(U, 0);
        load_units(U, clampc(1));
        store_units(U, 1);
        load_units(U, clampc(2));
        __syncthreads();
        prep1(0, 0);
        __syncthreads();
        prep2(0, 0);
        for (int c = 0; c < nc; ++c) {
            __syncthreads();
            advance(c & 1, stage_v(c & 1), stage_frags(c & 1), c);
            prep1((c + 1) & 1, (c + 1) & 1);
            __syncthreads();
            prep2((c + 1) & 1, (c + 1) & 1);
            store_units(U, c & 1);
            load_units(U, clampc(c + 3));
        }
    }

    if (fin) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                fin[(hd * DK + 16 * b + 4 * g4 + jj) * DV + col0 + n16] = S[b][jj];
    }
}

template <int DK, int DV, typename T, int NW>
static hipError_t launch_ic_t(const InterChunkArgs &a) {
    const int nchains = a.nseq * a.H;
    const int nsplit = DV / (16 * NW);
    const int64_t groups = ((int64_t)nchains + 7) / 8;
    const int64_t grid = groups * 8 * nsplit;
    hipLaunchKernelGGL((inter_chunk_kernel<DK, DV, T, NW>), dim3((unsigned)grid), dim3(64 * NW), 0,
                       (hipStream_t)a.stream, (const T *)a.q, (const T *)a.k, (const T *)a.v,
                       (const T *)a.g, a.init, a.cu, a.nseq, a.H, a.ws, a.o, a.fin, nsplit, nchains, a.skip);
    return hipGetLastError();
}

// Default waves per workgroup: up to 4 slices per workgroup (fewer when dv is small).
static int default_waves(int dk, int dv) {
    (void)dk;
    const int slices = dv / 16;
    return slices < 4 ? slices : 4;
}

template <typename T>
static hipError_t launch_ic_dt(const InterChunkArgs &a, int nw) {
#define KDA_IC_CASE(DKV, DVV, NWV) \
    if (a.dk == DKV && a.dv == DVV && nw == NWV) return launch_ic_t<DKV, DVV, T, NWV>(a);
    KDA_IC_CASE(128, 128, 2) KDA_IC_CASE(128, 128, 4) KDA_IC_CASE(128, 128, 8)
#define KDA_IC_DEF(DKV, DVV) KDA_IC_CASE(DKV, DVV, ((DVV / 16) < 4 ? (DVV / 16) : 4))
#define KDA_IC_ROW(DKV) KDA_IC_DEF(DKV, 16) KDA_IC_DEF(DKV, 32) KDA_IC_DEF(DKV, 64) KDA_IC_DEF(DKV, 128)
    KDA_IC_ROW(16) KDA_IC_ROW(32) KDA_IC_ROW(64) KDA_IC_ROW(128)
#undef KDA_IC_ROW
#undef KDA_IC_DEF
#undef KDA_IC_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_inter_chunk(const InterChunkArgs &a) {
    // Kernel choice.  bf16 inputs with dk >= 32 run the warp-specialised kernel
    // (inter_chunk_ws.hip), whose producer waves take the token-parallel work
    // off the consumers' critical path; it is the faster one both while the
    // serial recurrence is latency-bound (few (sequence, head) chains) and when
    // thousands of chains make the work throughput-bound.  This file's kernel
    // serves fp32 inputs and dk = 16.
    const int64_t nchains = (int64_t)a.nseq * a.H;
    if (a.bf16 && a.dk >= 32) {
        int ncw = a.ws_consumers, npw = a.ws_producers;
        if (ncw == 0 && npw == 0) {
            ncw = nchains < 64 ? 2 : 4;
            if (ncw > a.dv / 16) ncw = a.dv / 16;
            npw = a.dk / 16 < 4 ? a.dk / 16 : 4;
        }
        return launch_inter_chunk_ws(a, ncw, npw);
    }
    int nw = default_waves(a.dk, a.dv);
    // dk = dv = 128: one 8-wave workgroup per (sequence, head) when there are enough
    // chains to give every CU one; otherwise two 4-wave workgroups per chain so that
    // twice as many CUs work on the serial recurrence.
    if (a.dk == 128 && a.dv == 128) nw = nchains >= 256 ? 8 : 4;
    return a.bf16 ? launch_ic_dt<__bf16>(a, nw) : launch_ic_dt<float>(a, nw);
}

}  // namespace kda
