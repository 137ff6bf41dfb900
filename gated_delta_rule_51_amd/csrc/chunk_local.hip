// Chunk-local phase of the KDA prefill (gfx950): one wave per (16-token
// chunk, head), fully parallel.  Two kernels with the same outputs: one for
// fp32 inputs (fp32 matrix cores, running products of e^{+-g}), and one for
// bf16 inputs laid out for the bf16 matrix cores (described above it).
//
// Chunked form (Kimi K3 report digest, "Kimi Delta Attention": the output of
// chunk t is an inter-chunk term (Gamma (.) Q) S plus an intra-chunk term
// A V~).  With G_r the inclusive cumulative log-decay of token r inside the
// chunk (per key channel), K+ = K (.) e^{G}, K- = K (.) e^{-G}, Q+ = Q (.) e^{G}:
//     A_kk = diag(beta) * strictly_lower(K+ K-^T)      (16 x 16)
//     T    = (I + A_kk)^{-1}                            (unit lower triangular)
//     A_qk = lower_incl_diag(Q+ K-^T)                   (16 x 16)
// This kernel writes T' = T diag(beta) and A_qk to the workspace, as MFMA
// A-operand fragments (split bf16 for bf16 inputs, fp32 for fp32 inputs).  The
// pseudo-keys W = T' K+ and pseudo-values U = T' V are applied by the
// inter-chunk phase in the factored form Delta = T' (V - K+ S) = U - W S.
//
// Bounded decay (same page, "bounded decay" section): g >= -5, so over a
// 16-token chunk G lies in [-80, 0] and e^{-G} <= e^80 stays inside fp32/bf16
// range.  The decayed key-key and query-key blocks are therefore dense
// 16x16xdk matrix products on the matrix cores; e^{+-G} are formed as running
// products of e^{+-g} (no exp of a large argument).
//
// Precision: A_kk and A_qk use split-bf16 operands (hi*hi + lo*hi + hi*lo,
// ~16-bit mantissas).  A single-bf16 A_kk is enough for mild decay, but with
// strong decay and heavy-tailed values (the layer's ShortConv outputs under a
// gate near its -5 floor) its rounding became the largest error term of the
// output in an fp64 emulation (5e-3 of RMS on one 8192-token head, growing with
// the number of samples), and this kernel has matrix-core time to spare.  fp32
// inputs use fp32 MFMAs throughout.
#include "kda_device.hpp"
#include "kda_launch.hpp"
#include "layer_prologue.hpp"

namespace kda {

template <int DK, typename T>
__global__ __launch_bounds__(64) void chunk_local_f32_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ g,
    const T *__restrict__ beta, const int32_t *__restrict__ cu, int32_t nseq, int32_t H,
    float *__restrict__ ws) {
    constexpr bool F32 = sizeof(T) == 4;
    constexpr int NB = DK / 16;
    constexpr int LD = DK + 4;  // padded LDS row (floats)
    const int64_t slot = blockIdx.x;
    const int h = blockIdx.y;
    const int lane = threadIdx.x;

    // Which sequence owns this slot: the largest s with floor(cu[s]/16) + s <= slot.
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)(cu[mid] / 16) + mid <= slot) lo = mid;
        else hi = mid - 1;
    }
    const int s = lo;
    const int64_t bos = cu[s], eos = cu[s + 1];
    const int64_t j = slot - ((int64_t)(bos / 16) + s);
    if (j < 0 || 16 * j >= eos - bos) return;  // slot not used by any chunk
    const int64_t t0 = bos + 16 * j;
    const int n = (int)((eos - t0) < 16 ? (eos - t0) : 16);

    __shared__ float sP[16][LD];     // e^{G_r}   (running product of alpha)
    __shared__ float sPi[16][LD];    // e^{-G_r}
    __shared__ float sA[16][17];
    __shared__ float sBeta[16];

    // Per key channel: running products over the chunk's tokens (pads: g = 0).
    // Unconditional loads from clamped rows (n >= 1), padding zeroed by a select.
    for (int c = lane; c < DK; c += 64) {
        float gv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float x = load_in(g + ((t0 + (r < n ? r : n - 1)) * H + h) * DK + c);
            gv[r] = (r < n) ? x : 0.f;
        }
        float p = 1.f, pi = 1.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if constexpr (F32) {
                p *= decay_exp(gv[r]);
                pi *= decay_exp(-gv[r]);
            } else {
                p *= decay_exp_fast(gv[r]);
                pi *= decay_exp_fast(-gv[r]);
            }
            sP[r][c] = p;
            sPi[r][c] = pi;
        }
    }
    if (lane < 16) {
        const float b = load_in(beta + (t0 + (lane < n ? lane : n - 1)) * H + h);
        sBeta[lane] = (lane < n) ? b : 0.f;
    }
    __syncthreads();

    // Operands in the A/B fragment layout: lane (g4, m) holds token m, channels
    // 16b + 4*g4 + 0..3 of K+, K-, Q+.
    const int m = lane & 15, g4 = lane >> 4;
    const bool valid = m < n;
    const int64_t mrow = t0 + (valid ? m : n - 1);
    const T *krow = k + (mrow * H + h) * DK;
    const T *qrow = q + (mrow * H + h) * DK;
    f32x4 akk = zero4(), aqk = zero4();
    auto operands = [&](int b, f32x4 &kp, f32x4 &km, f32x4 &qp) {
        const int c = 16 * b + 4 * g4;
        const f32x4 kl = load_in4(krow + c);
        const f32x4 ql = load_in4(qrow + c);
        const f32x4 kk = valid ? kl : zero4();
        const f32x4 qq = valid ? ql : zero4();
        const f32x4 P = *reinterpret_cast<const f32x4 *>(&sP[m][c]);
        const f32x4 Pi = *reinterpret_cast<const f32x4 *>(&sPi[m][c]);
        kp = kk * P;
        km = kk * Pi;
        qp = qq * P;
    };
    if constexpr (F32) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            f32x4 kp, km, qp;
            operands(b, kp, km, qp);
            akk = mma_f32_k16(kp, km, akk);
            aqk = mma_f32_k16(qp, km, aqk);
        }
    } else if constexpr (NB == 1) {
        f32x4 kp, km, qp;
        operands(0, kp, km, qp);
        akk = mma16(to_bf16x4(kp), to_bf16x4(km), akk);
        aqk = mma_split_k16(split4(qp), split4(km), aqk);
    } else {
#pragma unroll
        for (int b = 0; b < NB; b += 2) {
            f32x4 kp0, km0, qp0, kp1, km1, qp1;
            operands(b, kp0, km0, qp0);
            operands(b + 1, kp1, km1, qp1);
            akk = mma_single_k32(to_bf16x4(kp0), to_bf16x4(kp1), to_bf16x4(km0), to_bf16x4(km1), akk);
            aqk = mma_split_k32(split4(qp0), split4(qp1), split4(km0), split4(km1), aqk);
        }
    }

    // Accumulator lane (g4, i) holds rows r = 4*g4 + jj of column i.
    __shared__ float sAq[16][17];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int r = 4 * g4 + jj, i = m;
        sA[r][i] = (r > i) ? sBeta[r] * akk[jj] : 0.f;
        sAq[r][i] = (r >= i) ? aqk[jj] : 0.f;
    }
    __syncthreads();

    // T = (I + A_kk)^{-1} by forward substitution; lane c builds column c:
    // T[r][c] = [r == c] - sum_{i < r} A[r][i] T[i][c]  (T[i][c] = 0 for i < c).
    // T' = T diag(beta) overwrites A_kk in LDS (every lane has read it by then).
    float t[16];
    if (lane < 16) {
        const int c = lane;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) acc += sA[r][i] * t[i];
            t[r] = ((r == c) ? 1.f : 0.f) - acc;
        }
    }
    __syncthreads();
    if (lane < 16) {
        const float bc = sBeta[lane];
#pragma unroll
        for (int r = 0; r < 16; ++r) sA[r][lane] = t[r] * bc;
    }
    __syncthreads();

    // Store T' and A_qk as A-operand fragments of the 16x16 MFMA: lane (g4, m)
    // holds M[m][4*g4 + 0..3] -- split {hi, lo} bf16 for bf16 inputs, fp32 for
    // fp32 inputs -- so the inter-chunk phase loads them with one 16-byte read
    // per lane.
    const f32x4 tv = {sA[m][4 * g4], sA[m][4 * g4 + 1], sA[m][4 * g4 + 2], sA[m][4 * g4 + 3]};
    const f32x4 av = {sAq[m][4 * g4], sAq[m][4 * g4 + 1], sAq[m][4 * g4 + 2], sAq[m][4 * g4 + 3]};
    float *w = ws + (slot * H + h) * (int64_t)WS_FLOATS_PER_CHUNK_HEAD;
    if constexpr (F32) {
        reinterpret_cast<f32x4 *>(w)[lane] = tv;
        reinterpret_cast<f32x4 *>(w + 256)[lane] = av;
    } else {
        reinterpret_cast<Split4 *>(w)[lane] = split4(tv);
        reinterpret_cast<Split4 *>(w + 256)[lane] = split4(av);
    }
}


// bf16 inputs.  Same outputs; the work is laid out for the matrix cores:
//   * q, k, g of the chunk are read through buffer resources based at the
//     chunk's first token (4 channels of one token per lane and block -- the
//     A-operand layout of K+, K-, Q+; padding rows read as zeros);
//   * the cumulative log-decay G is a product with the 0/1 lower triangle,
//     G^T = g^T L^T, after an identity product turns g into 4 tokens of one
//     channel per lane (both exact: g is bf16), so e^{+-G} = exp(+-G) need no
//     per-token running products and no LDS round trip (|G| <= 80);
//   * the hi/lo splits of Q+ and K- take their residuals from the matrix core
//     (an exact product with -I) instead of vector-ALU unpacking;
//   * the triangular solve reads the rows of A_kk as 16-byte vectors.
//
// With LAYER the kernel is the first pass of the fused layer prefill: q, k and g
// are the raw q and k projections and the decay logits z, and the layer
// prologue (layer_prologue.hpp) turns them into the normalised q, k and the
// log-decay in registers, which the kernel also writes (bf16, lp.qkg) for the
// inter-chunk pass: computing the prologue once and storing its results costs
// less than recomputing it in both passes (it is a vector-ALU load comparable
// to the chunk-local work itself).
template <int DK, bool LAYER>
__global__ __launch_bounds__(64) void chunk_local_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ g,
    const __bf16 *__restrict__ beta, const int32_t *__restrict__ cu, int32_t nseq, int32_t H,
    float *__restrict__ ws, int64_t base, LayerPrologue lp) {
    static_assert(!LAYER || DK == 128, "the fused layer prologue is built for dk = 128");
    constexpr int NB = DK / 16;
    constexpr uint32_t EB = 2;
    // Item id = slot * H + head: the heads of one chunk are neighbours, so the
    // waves in flight read neighbouring pieces of the same token rows.
    const int64_t id = base + blockIdx.x;
    const int64_t slot = id / H;
    const int h = (int)(id - slot * H);
    const int lane = threadIdx.x;

    // Which sequence owns this slot: the largest s with floor(cu[s]/16) + s <= slot.
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)(cu[mid] / 16) + mid <= slot) lo = mid;
        else hi = mid - 1;
    }
    const int s = lo;
    const int64_t bos = cu[s], eos = cu[s + 1];
    const int64_t j = slot - ((int64_t)(bos / 16) + s);
    if (j < 0 || 16 * j >= eos - bos) return;  // slot not used by any chunk
    const int64_t t0 = bos + 16 * j;
    const int n = (int)((eos - t0) < 16 ? (eos - t0) : 16);

    const int g4 = lane >> 4, l16 = lane & 15;
    const uint32_t rowK = (uint32_t)H * DK * EB;
    const rsrc_t rq = make_rsrc(q + (t0 * H + h) * DK, (uint32_t)n * rowK);
    const rsrc_t rk = make_rsrc(k + (t0 * H + h) * DK, (uint32_t)n * rowK);
    const rsrc_t rg = make_rsrc(g + (t0 * H + h) * DK, (uint32_t)n * rowK);
    const rsrc_t rb = make_rsrc(beta + t0 * H + h, (uint32_t)n * (uint32_t)H * EB);

    __shared__ __attribute__((aligned(16))) float sA[16][20];   // A_kk, then T'
    __shared__ __attribute__((aligned(16))) float sAq[16][20];  // A_qk
    __shared__ float sBeta[16];

    // All loads first: token l16, channels 16 b + 4 g4 .. +3 of q, k, g (block b
    // in the kernel's own channel order).  The products below contract over the
    // channels, so any consistent order will do; with two or more blocks the
    // kernel takes, in block pair P, internal channel 16 (2P + h) + 4 g4 + j to be
    // memory channel 32 P + 8 g4 + 4 h + j, which makes what a lane needs of the
    // pair one 16-byte piece (half the load instructions, each touching the same
    // 16 token rows).
    const uint32_t row = l16 < n ? l16 * rowK : OOB;
    u32x2 gr[NB], kr[NB], qr[NB];
    if constexpr (NB % 2 == 0) {
        uint32_t gx[NB / 2][4], kx[NB / 2][4], qx[NB / 2][4];
#pragma unroll
        for (int p = 0; p < NB / 2; ++p) {
            const uint32_t o = row == OOB ? OOB : row + (32 * p + 8 * g4) * EB;
            const u32x4 gv = buf_load_u32x4(rg, o), kv = buf_load_u32x4(rk, o), qv = buf_load_u32x4(rq, o);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gx[p][i] = gv[i];
                kx[p][i] = kv[i];
                qx[p][i] = qv[i];
            }
        }
        if constexpr (LAYER) {
            // The three tokens before the chunk (lanes l16 = 13..15): packed rows of the same
            // sequence, or its cache before the first chunk.
            uint32_t hq[NB / 2][4], hk[NB / 2][4];
            if (j > 0) {
                const rsrc_t hq_r = make_rsrc(q + ((t0 - 3) * H + h) * DK, 3u * rowK);
                const rsrc_t hk_r = make_rsrc(k + ((t0 - 3) * H + h) * DK, 3u * rowK);
#pragma unroll
                for (int p = 0; p < NB / 2; ++p) {
                    const uint32_t o = l16 >= 13 ? (l16 - 13) * rowK + (32 * p + 8 * g4) * EB : OOB;
                    const u32x4 a = buf_load_u32x4(hq_r, o), b = buf_load_u32x4(hk_r, o);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        hq[p][i] = a[i];
                        hk[p][i] = b[i];
                    }
                }
            } else {
#pragma unroll
                for (int p = 0; p < NB / 2; ++p) {
                    cache_halo<4>(lp.cache, (int64_t)s * H + h, lp.cw, 32 * p + 8 * g4, l16, hq[p]);
                    cache_halo<4>(lp.cache, (int64_t)s * H + h, lp.cw, DK + 32 * p + 8 * g4, l16, hk[p]);
                }
            }
            // The head's q and k taps (2 x 128 channels x 4, contiguous in conv_w) pass through
            // LDS: four coalesced 16-byte loads per lane instead of 64 row-broadcast ones.
            __shared__ __attribute__((aligned(16))) f32x4 sW[2 * DK];
            {
                const f32x4 *src = reinterpret_cast<const f32x4 *>(lp.conv_w + (int64_t)h * lp.cw * 4);
#pragma unroll
                for (int i = 0; i < 2 * DK / 64; ++i) sW[64 * i + lane] = src[64 * i + lane];
            }
            // ShortConv + Swish of q and k, then the L2 norms of the rows.  The 128 channels
            // of token l16 sit in lanes l16 + 16 g4, octet 4 p + g4 in pair p; the octets are
            // added in the order of the stand-alone pass's butterfly over the octet index
            // (bits 0, 1 of it are g4: across lanes; bits 2, 3 are p: in the lane).
            float yq[NB / 2][8], yk[NB / 2][8];
            float oq[NB / 2], ok[NB / 2];
#pragma unroll
            for (int p = 0; p < NB / 2; ++p) {
                f32x4 w[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) w[m] = sW[32 * p + 8 * g4 + m];
                conv_swish<4>(qx[p], hq[p], w, l16, yq[p]);
#pragma unroll
                for (int m = 0; m < 8; ++m) w[m] = sW[DK + 32 * p + 8 * g4 + m];
                conv_swish<4>(kx[p], hk[p], w, l16, yk[p]);
                oq[p] = octet_sumsq(yq[p]);
                ok[p] = octet_sumsq(yk[p]);
                oq[p] += __shfl_xor(oq[p], 16);
                ok[p] += __shfl_xor(ok[p], 16);
                oq[p] += __shfl_xor(oq[p], 32);
                ok[p] += __shfl_xor(ok[p], 32);
            }
            const float sq = (oq[0] + oq[1]) + (oq[2] + oq[3]), sk = (ok[0] + ok[1]) + (ok[2] + ok[3]);
            const float iq = __builtin_amdgcn_rsqf(sq + lp.l2_eps), ik = __builtin_amdgcn_rsqf(sk + lp.l2_eps);
            const bool valid = l16 < n;
            const float eA = __expf(lp.A_log[h]);
#pragma unroll
            for (int p = 0; p < NB / 2; ++p) {
                pack_scaled<4>(yq[p], iq, valid, qx[p]);
                pack_scaled<4>(yk[p], ik, valid, kx[p]);
                gate_words<4>(gx[p], eA, valid, gx[p]);
            }
            // the prologue's outputs for the inter-chunk pass (token rows of this chunk only)
            if (valid) {
                __bf16 *qo = static_cast<__bf16 *>(lp.qkg);
                const int64_t plane = (int64_t)lp.n_tokens * H * DK;
                const int64_t rowo = ((t0 + l16) * H + h) * DK;
#pragma unroll
                for (int p = 0; p < NB / 2; ++p) {
                    const int64_t e = rowo + 32 * p + 8 * g4;
                    *reinterpret_cast<u32x4 *>(qo + e) = u32x4{qx[p][0], qx[p][1], qx[p][2], qx[p][3]};
                    *reinterpret_cast<u32x4 *>(qo + plane + e) = u32x4{kx[p][0], kx[p][1], kx[p][2], kx[p][3]};
                    *reinterpret_cast<u32x4 *>(qo + 2 * plane + e) = u32x4{gx[p][0], gx[p][1], gx[p][2], gx[p][3]};
                }
            }
        }
#pragma unroll
        for (int p = 0; p < NB / 2; ++p) {
            gr[2 * p] = u32x2{gx[p][0], gx[p][1]};
            gr[2 * p + 1] = u32x2{gx[p][2], gx[p][3]};
            kr[2 * p] = u32x2{kx[p][0], kx[p][1]};
            kr[2 * p + 1] = u32x2{kx[p][2], kx[p][3]};
            qr[2 * p] = u32x2{qx[p][0], qx[p][1]};
            qr[2 * p + 1] = u32x2{qx[p][2], qx[p][3]};
        }
    } else {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint32_t o = row == OOB ? OOB : row + (16 * b + 4 * g4) * EB;
            gr[b] = buf_load_u32x2(rg, o);
            kr[b] = buf_load_u32x2(rk, o);
            qr[b] = buf_load_u32x2(rq, o);
        }
    }
    if (lane < 16) sBeta[lane] = bf16_bits_to_f32(buf_load_u16(rb, lane < n ? lane * (uint32_t)H * EB : OOB));

    // Constant operands.  Channel blocks are handled in pairs, so every 32-long
    // operand carries two blocks' data; a constant B with the wanted matrix in
    // one half and 0 in the other (or -I in one half of A) selects the block.
    const bf16x4 z4 = {};
    const bf16x4 ID = identity_operand(g4, l16);
    u16x4 lt_bits;  // L^T: lane (g4, n) holds L[n][4 g4 + j] = [4 g4 + j <= n]
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) lt_bits[jj] = (4 * g4 + jj <= l16) ? 0x3f80 : 0;
    const bf16x4 LT = __builtin_bit_cast(bf16x4, lt_bits);
    const bf16x8 IDL = cat(ID, z4), IDH = cat(z4, ID), LTL = cat(LT, z4), LTH = cat(z4, LT);
    const bf16x8 NIL = neg_identity_operand<0>(g4, l16), NIH = neg_identity_operand<1>(g4, l16);

    // Operands of blocks b0, b1 (token l16, channels 16 b + 4 g4 + jj):
    // K+ = K e^{G}, K- = K e^{-G}, Q+ = Q e^{G}.
    struct Pair {
        f32x4 kp[2], km[2], qp[2];
    };
    auto operands = [&](int b0, int b1) {
        const bf16x8 ga = cat(__builtin_bit_cast(bf16x4, gr[b0]), __builtin_bit_cast(bf16x4, gr[b1]));
        // g as 4 tokens of one channel per lane, then G^T = g^T L^T (both exact)
        const bf16x8 gf = cat(to_bf16x4(mma32(ga, IDL, zero4())), to_bf16x4(mma32(ga, IDH, zero4())));
        const f32x4 G[2] = {mma32(gf, LTL, zero4()), mma32(gf, LTH, zero4())};
        Pair r;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x4 P, Pi;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                P[jj] = decay_exp_fast(G[u][jj]);
                Pi[jj] = decay_exp_fast(-G[u][jj]);
            }
            const f32x4 kk = unpack_bf16x4(kr[u ? b1 : b0]);
            r.kp[u] = kk * P;
            r.km[u] = kk * Pi;
            r.qp[u] = unpack_bf16x4(qr[u ? b1 : b0]) * P;
        }
        return r;
    };
    // hi (pair-packed) and the two lo halves of a pair of values held in the
    // accumulator layout of their transposes; residuals from the matrix core.
    struct SplitPair {
        bf16x8 hi, lo;
    };
    auto split_pair = [&](const f32x4 &x0, const f32x4 &x1) {
        const bf16x8 hh = cat(to_bf16x4(x0), to_bf16x4(x1));
        return SplitPair{hh, cat(to_bf16x4(mma32(NIL, hh, x0)), to_bf16x4(mma32(NIH, hh, x1)))};
    };
    f32x4 akk = zero4(), aqk = zero4();
    constexpr int NP2 = (NB + 1) / 2;
#pragma unroll
    for (int pi = 0; pi < NP2; ++pi) {
        const int b0 = 2 * pi, b1 = (2 * pi + 1 < NB) ? 2 * pi + 1 : 2 * pi;
        Pair r = operands(b0, b1);
        if (b1 == b0) {  // a lone block (dk = 16): the second half must not contribute
            r.kp[1] = zero4();
            r.qp[1] = zero4();
        }
        const SplitPair qs = split_pair(r.qp[0], r.qp[1]);
        const SplitPair ms = split_pair(r.km[0], r.km[1]);
        const SplitPair ps = split_pair(r.kp[0], r.kp[1]);
        // A_kk and A_qk: hi*hi + lo*hi + hi*lo
        akk = mma32(ps.hi, ms.hi, akk);
        akk = mma32(ps.lo, ms.hi, akk);
        akk = mma32(ps.hi, ms.lo, akk);
        aqk = mma32(qs.hi, ms.hi, aqk);
        aqk = mma32(qs.lo, ms.hi, aqk);
        aqk = mma32(qs.hi, ms.lo, aqk);
    }
    __syncthreads();  // sBeta visible

    // Accumulator lane (g4, i) holds rows r = 4*g4 + jj of column i.
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int r = 4 * g4 + jj, i = l16;
        sA[r][i] = (r > i) ? sBeta[r] * akk[jj] : 0.f;
        sAq[r][i] = (r >= i) ? aqk[jj] : 0.f;
    }
    __syncthreads();

    // T = (I + A_kk)^{-1} by forward substitution; lane c builds column c:
    // T[r][c] = [r == c] - sum_{i < r} A[r][i] T[i][c]; rows of A come as four
    // 16-byte reads (the same address for every lane).
    float t[16];
    if (lane < 16) {
        const int c = lane;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int q4 = 0; q4 < (r + 3) / 4; ++q4) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(&sA[r][4 * q4]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * q4 + e < r) acc += a[e] * t[4 * q4 + e];
            }
            t[r] = ((r == c) ? 1.f : 0.f) - acc;
        }
    }
    __syncthreads();
    if (lane < 16) {
        const float bc = sBeta[lane];
#pragma unroll
        for (int r = 0; r < 16; ++r) sA[r][lane] = t[r] * bc;
    }
    __syncthreads();

    // T' and A_qk as A-operand fragments: lane (g4, m) holds M[m][4*g4 + 0..3], {hi, lo}.
    const f32x4 tv = *reinterpret_cast<const f32x4 *>(&sA[l16][4 * g4]);
    const f32x4 av = *reinterpret_cast<const f32x4 *>(&sAq[l16][4 * g4]);
    float *w = ws + (slot * H + h) * (int64_t)WS_FLOATS_PER_CHUNK_HEAD;
    const SplitPair ts = split_pair(tv, av);
    reinterpret_cast<Split4 *>(w)[lane] = Split4{__builtin_shufflevector(ts.hi, ts.hi, 0, 1, 2, 3),
                                                 __builtin_shufflevector(ts.lo, ts.lo, 0, 1, 2, 3)};
    reinterpret_cast<Split4 *>(w + 256)[lane] = Split4{__builtin_shufflevector(ts.hi, ts.hi, 4, 5, 6, 7),
                                                       __builtin_shufflevector(ts.lo, ts.lo, 4, 5, 6, 7)};
}

template <int DK, typename T>
static hipError_t launch_cl_t(const ChunkLocalArgs &a) {
    const int64_t slots = chunk_slots(a.total_tokens, a.nseq);
    const dim3 grid((unsigned)slots, (unsigned)a.H);
    if constexpr (sizeof(T) == 2) {
        // one wave per (slot, head) item, in launches of at most 2^25 workgroups
        const int64_t items = slots * a.H, per_launch = int64_t(1) << 25;
        for (int64_t base = 0; base < items; base += per_launch) {
            const int64_t n = items - base < per_launch ? items - base : per_launch;
            if constexpr (DK == 128) {
                if (a.layer) {
                    hipLaunchKernelGGL((chunk_local_bf16_kernel<DK, true>), dim3((unsigned)n), dim3(64), 0,
                                       (hipStream_t)a.stream, (const __bf16 *)a.q, (const __bf16 *)a.k,
                                       (const __bf16 *)a.g, (const __bf16 *)a.beta, a.cu, a.nseq, a.H, a.ws, base,
                                       *a.layer);
                    const hipError_t e = hipGetLastError();
                    if (e != hipSuccess) return e;
                    continue;
                }
            }
            if (a.layer) return hipErrorInvalidValue;
            hipLaunchKernelGGL((chunk_local_bf16_kernel<DK, false>), dim3((unsigned)n), dim3(64), 0,
                               (hipStream_t)a.stream, (const __bf16 *)a.q, (const __bf16 *)a.k,
                               (const __bf16 *)a.g, (const __bf16 *)a.beta, a.cu, a.nseq, a.H, a.ws, base,
                               LayerPrologue{});
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    } else {
        if (a.layer) return hipErrorInvalidValue;
        hipLaunchKernelGGL((chunk_local_f32_kernel<DK, T>), grid, dim3(64), 0, (hipStream_t)a.stream,
                           (const T *)a.q, (const T *)a.k, (const T *)a.g, (const T *)a.beta, a.cu,
                           a.nseq, a.H, a.ws);
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_cl_dt(const ChunkLocalArgs &a) {
    switch (a.dk) {
        case 16: return launch_cl_t<16, T>(a);
        case 32: return launch_cl_t<32, T>(a);
        case 64: return launch_cl_t<64, T>(a);
        case 128: return launch_cl_t<128, T>(a);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_chunk_local(const ChunkLocalArgs &a) {
    return a.bf16 ? launch_cl_dt<__bf16>(a) : launch_cl_dt<float>(a);
}

}  // namespace kda
