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
//   * prep1 (one thread per key channel): e^{g}, running prefix/suffix
//     products, Gamma, K~ fragments; T' and A_qk fragments from the workspace;
//   * prep2 (one thread per (token, 4 channels)): Q+ and K+ fragments.
// The prep of chunk c+1 runs while the waves advance the state through chunk
// c (double-buffered LDS, two barriers per chunk), and the raw inputs of
// chunk c+2 are loaded into registers meanwhile.  This overlaps the
// token-parallel work with the serial recurrence, as the page's KDA systems
// section describes for its own chunkwise kernel.
//
// Precision: K+ S uses single-bf16 operands; T'(V - K+S), Q+ S, A_qk Delta and
// K~^T Delta use split-bf16 (hi*hi + lo*hi + hi*lo) with fp32 accumulation;
// the state stays fp32.  fp32 inputs use fp32 MFMAs throughout.
#include <stdlib.h>

#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int DK, int DV, typename T, int NW>
struct IC {
    static constexpr bool F32 = sizeof(T) == 4;
    static constexpr int NT = 64 * NW;
    static constexpr int NB = DK / 16;
    static constexpr int CPT = (DK + NT - 1) / NT;        // channels per thread (prep1)
    static constexpr int IPT = (4 * DK + NT - 1) / NT;    // (token, quad) items per thread (prep2)
    static constexpr int EPT = (256 + NT - 1) / NT;       // T' / A_qk elements per thread
    using OpT = std::conditional_t<F32, f32x4, Split4>;   // split operand fragment
    using KpT = std::conditional_t<F32, f32x4, bf16x4>;   // single operand fragment
};

template <int DK, int DV, typename T, int NW>
struct Raw {
    using C = IC<DK, DV, T, NW>;
    float g[C::CPT][16];
    float k[C::CPT][16];
    f32x4 q4[C::IPT];
    f32x4 k4[C::IPT];
    float tp[C::EPT];
    float aq[C::EPT];
};

template <typename O>
__device__ __forceinline__ O make_op(f32x4 x) {
    if constexpr (std::is_same_v<O, f32x4>) return x;
    else return split4(x);
}

template <typename O>
__device__ __forceinline__ O make_kp(f32x4 x) {
    if constexpr (std::is_same_v<O, f32x4>) return x;
    else return to_bf16x4(x);
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

template <int DK, int DV, typename T, int NW>
__global__ __launch_bounds__(64 * NW) void inter_chunk_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ g, const float *__restrict__ init, const int32_t *__restrict__ cu,
    int32_t nseq, int32_t H, const float *__restrict__ ws, float *__restrict__ o,
    float *__restrict__ fin, int32_t nsplit, int32_t nchains) {
    using C = IC<DK, DV, T, NW>;
    using OpT = typename C::OpT;
    using KpT = typename C::KpT;
    constexpr int NT = C::NT, NB = C::NB, CPT = C::CPT, IPT = C::IPT, EPT = C::EPT;

    // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin by
    // linear id, so all slices of one (sequence, head) get the same id mod 8
    // and share that XCD's L2 for the q/k/g/workspace reads.
    const int L = blockIdx.x;
    const int xcd = L & 7;
    const int sx = L >> 3;
    const int split = sx % nsplit;
    const int chain = (sx / nsplit) * 8 + xcd;
    if (chain >= nchains) return;
    const int s = chain / H, h = chain % H;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int g4 = lane >> 4, n16 = lane & 15;
    const int col0 = (split * NW + wave) * 16;

    __shared__ OpT sQp[2][NB][64];
    __shared__ KpT sKp[2][NB][64];
    __shared__ OpT sKt[2][NB][64];
    __shared__ OpT sTp[2][64];
    __shared__ OpT sAq[2][64];
    __shared__ float sGam[2][DK];
    __shared__ float sP[16][DK + 4];

    const int64_t bos = cu[s], eos = cu[s + 1];
    const int nc = (int)((eos - bos + 15) / 16);
    const int64_t slot0 = bos / 16 + s;
    const int64_t hd = (int64_t)s * H + h;

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

    // Loads are unconditional (addresses clamped to a valid token row / channel,
    // padding zeroed by a select afterwards) so the compiler issues them back to
    // back instead of branching and waiting on each one.  A chunk that exists has
    // n >= 1 tokens, so row t0 + min(t, n-1) is always inside the sequence.
    auto load_raw = [&](Raw<DK, DV, T, NW> &R, int c) {
        const int64_t t0 = bos + 16 * (int64_t)c;
        const int n = chunk_len(c);
#pragma unroll
        for (int ci = 0; ci < CPT; ++ci) {
            const int ch = tid + ci * NT;
            const int chc = ch < DK ? ch : DK - 1;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const bool ok = ch < DK && r < n;
                const int rr = r < n ? r : n - 1;
                const int64_t off = ((t0 + rr) * H + h) * DK + chc;
                const float gv = load_in(g + off);
                const float kv = load_in(k + off);
                R.g[ci][r] = ok ? gv : 0.f;
                R.k[ci][r] = ok ? kv : 0.f;
            }
        }
#pragma unroll
        for (int ii = 0; ii < IPT; ++ii) {
            const int item = tid + ii * NT;
            const int itc = item < 4 * DK ? item : 4 * DK - 1;
            const int t = itc / (DK / 4), a = itc % (DK / 4);
            const bool ok = item < 4 * DK && t < n;
            const int tt = t < n ? t : n - 1;
            const int64_t off = ((t0 + tt) * H + h) * DK + 4 * a;
            const f32x4 qv = load_in4(q + off);
            const f32x4 kv = load_in4(k + off);
            R.q4[ii] = ok ? qv : zero4();
            R.k4[ii] = ok ? kv : zero4();
        }
        const float *w = ws + ((slot0 + c) * H + h) * (int64_t)WS_FLOATS_PER_CHUNK_HEAD;
#pragma unroll
        for (int ei = 0; ei < EPT; ++ei) {
            const int e = (NT - 1 - tid) + ei * NT;
            const int ec = e < 256 ? e : 255;
            const float tv = w[ec], av = w[256 + ec];
            R.tp[ei] = e < 256 ? tv : 0.f;
            R.aq[ei] = e < 256 ? av : 0.f;
        }
    };

    auto prep1 = [&](const Raw<DK, DV, T, NW> &R, int buf) {
#pragma unroll
        for (int ci = 0; ci < CPT; ++ci) {
            const int ch = tid + ci * NT;
            if (ch < DK) {
                float a[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) a[r] = decay_exp(R.g[ci][r]);
                float p = 1.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    p *= a[r];
                    sP[r][ch] = p;
                }
                sGam[buf][ch] = p;
                float kt[16];
                float f = 1.f;  // product of alpha over tokens after r
#pragma unroll
                for (int r = 15; r >= 0; --r) {
                    kt[r] = R.k[ci][r] * f;
                    f *= a[r];
                }
#pragma unroll
                for (int tq = 0; tq < 4; ++tq)
                    sKt[buf][ch >> 4][tq * 16 + (ch & 15)] =
                        make_op<OpT>(f32x4{kt[4 * tq], kt[4 * tq + 1], kt[4 * tq + 2], kt[4 * tq + 3]});
            }
        }
#pragma unroll
        for (int ei = 0; ei < EPT; ++ei) {
            const int e = (NT - 1 - tid) + ei * NT;
            if (e < 256) {
                const int r = e >> 4, col = e & 15;
                const int ln = (col >> 2) * 16 + r;
                set_op_elem(sTp[buf][ln], col & 3, R.tp[ei]);
                set_op_elem(sAq[buf][ln], col & 3, R.aq[ei]);
            }
        }
    };

    auto prep2 = [&](const Raw<DK, DV, T, NW> &R, int buf) {
#pragma unroll
        for (int ii = 0; ii < IPT; ++ii) {
            const int item = tid + ii * NT;
            if (item < 4 * DK) {
                const int t = item / (DK / 4), a = item % (DK / 4);
                const int c = 4 * a;
                const f32x4 P = *reinterpret_cast<const f32x4 *>(&sP[t][c]);
                const int ln = ((c & 15) >> 2) * 16 + t;
                sQp[buf][c >> 4][ln] = make_op<OpT>(R.q4[ii] * P);
                sKp[buf][c >> 4][ln] = make_kp<KpT>(R.k4[ii] * P);
            }
        }
    };

    auto load_v = [&](int c) -> f32x4 {
        const int64_t t0 = bos + 16 * (int64_t)c;
        const int n = chunk_len(c);
        f32x4 r;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int t = 4 * g4 + jj;
            const int tt = t < n ? t : n - 1;
            const float x = load_in(v + ((t0 + tt) * H + h) * DV + col0 + n16);
            r[jj] = t < n ? x : 0.f;
        }
        return r;
    };

    // One chunk of the recurrence for this wave's 16 columns.
    auto advance = [&](int buf, f32x4 vc, int c) {
        f32x4 O;
        if constexpr (C::F32) {
            f32x4 X = zero4();
#pragma unroll
            for (int b = 0; b < NB; ++b) X = mma_f32_k16(sKp[buf][b][lane], S[b], X);
            const f32x4 D = mma_f32_k16(sTp[buf][lane], vc - X, zero4());
            O = mma_f32_k16(sAq[buf][lane], D, zero4());
#pragma unroll
            for (int b = 0; b < NB; ++b) O = mma_f32_k16(sQp[buf][b][lane], S[b], O);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const f32x4 gam = *reinterpret_cast<const f32x4 *>(&sGam[buf][16 * b + 4 * g4]);
                S[b] = mma_f32_k16(sKt[buf][b][lane], D, S[b] * gam);
            }
        } else {
            Split4 Ss[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) Ss[b] = split4(S[b]);
            f32x4 X = zero4();
            if constexpr (NB == 1) {
                X = mma16(sKp[buf][0][lane], Ss[0].hi, X);
            } else {
#pragma unroll
                for (int b = 0; b < NB; b += 2)
                    X = mma_single_k32(sKp[buf][b][lane], sKp[buf][b + 1][lane], Ss[b].hi, Ss[b + 1].hi, X);
            }
            const f32x4 D = mma_split_k16(sTp[buf][lane], split4(vc - X), zero4());
            const Split4 Ds = split4(D);
            O = mma_split_k16(sAq[buf][lane], Ds, zero4());
            if constexpr (NB == 1) {
                O = mma_split_k16(sQp[buf][0][lane], Ss[0], O);
            } else {
#pragma unroll
                for (int b = 0; b < NB; b += 2)
                    O = mma_split_k32(sQp[buf][b][lane], sQp[buf][b + 1][lane], Ss[b], Ss[b + 1], O);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const f32x4 gam = *reinterpret_cast<const f32x4 *>(&sGam[buf][16 * b + 4 * g4]);
                S[b] = mma_split_k16(sKt[buf][b][lane], Ds, S[b] * gam);
            }
        }
        const int64_t t0 = bos + 16 * (int64_t)c;
        const int n = chunk_len(c);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int t = 4 * g4 + jj;
            if (t < n) o[((t0 + t) * H + h) * DV + col0 + n16] = O[jj];
        }
    };

    if (nc > 0) {
        Raw<DK, DV, T, NW> R;
        load_raw(R, 0);
        prep1(R, 0);
        __syncthreads();
        prep2(R, 0);
        f32x4 vcur = load_v(0);
        if (nc > 1) load_raw(R, 1);
        __syncthreads();
        for (int c = 0; c < nc; ++c) {
            const int buf = c & 1;
            const f32x4 vnext = (c + 1 < nc) ? load_v(c + 1) : zero4();
            advance(buf, vcur, c);
            if (c + 1 < nc) prep1(R, buf ^ 1);
            __syncthreads();
            if (c + 1 < nc) {
                prep2(R, buf ^ 1);
                if (c + 2 < nc) load_raw(R, c + 2);
            }
            __syncthreads();
            vcur = vnext;
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
                       (const T *)a.g, a.init, a.cu, a.nseq, a.H, a.ws, a.o, a.fin, nsplit, nchains);
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
    int nw = a.waves_per_group;
    if (nw <= 0) {
        nw = default_waves(a.dk, a.dv);
        // Tuning knob: KDA_WAVES in {2, 4, 8} for dk = dv = 128.
        if (a.dk == 128 && a.dv == 128) {
            if (const char *e = getenv("KDA_WAVES")) {
                const int w = atoi(e);
                if (w == 2 || w == 4 || w == 8) nw = w;
            }
        }
    }
    return a.bf16 ? launch_ic_dt<__bf16>(a, nw) : launch_ic_dt<float>(a, nw);
}

}  // namespace kda
