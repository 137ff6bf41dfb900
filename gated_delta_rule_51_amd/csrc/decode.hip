// Recurrent single-token KDA decode (gfx950).
//
// Per head (Kimi K3 report digest, "Kimi Delta Attention", update equation):
//     S' = Diag(alpha) S                      forget
//     S  = (I - beta k k^T) S' + beta k v^T   erase + write
//     o  = S^T q
// rewritten for a single pass over S:
//     vhat = S'^T k,  r = S'^T q,  delta = beta (v - vhat)
//     S    = S' + k delta^T,       o = r + delta (k^T q)
// Each state element is read once and written once, in place.  The serving
// section of the same page names this in-place state traffic as the decode
// bottleneck, so the kernel is built around streaming the fp32 state at HBM
// rate.  No matrix cores are used (about one flop per byte).
//
// Shape of the launch: a persistent grid of at most GRID_THREADS / NT
// workgroups walks the heads with stride gridDim.x, so at any moment the
// resident workgroups stream neighbouring 64 KiB state blocks (DRAM-page
// friendly), and each workgroup issues the loads of its next head's state
// before it reduces and writes back the current one, keeping reads and
// writes in flight together.  Thread (rg, c4) holds column quad c4 of rows
// rg, rg + RP, ... in registers.
//
// Column sums S'^T k and S'^T q go through LDS in two stages: every row
// group writes its partial quads, then P = RP/8 neighbouring lanes own one
// output column, each adds 8 partials (rows part, part + P, ...; the row
// stride is padded so the lanes of a wave hit distinct banks) and the P
// lanes combine by cross-lane shuffles.  Every thread then reads back only
// the two quads it needs.
#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int DK, int DV, int MAXT = 1024>
struct DecodeShape {
    static constexpr int NC4 = DV / 4;                       // column quads per row
    static constexpr int RP_CAP = MAXT / NC4 < 64 ? MAXT / NC4 : 64;
    static constexpr int RP = DK < RP_CAP ? DK : RP_CAP;     // row groups (>= 16)
    static constexpr int NT = NC4 * RP;                      // threads per workgroup
    static constexpr int NR = DK / RP;                       // rows per thread
    static constexpr int P = RP / 8;                         // lanes per output column
    static constexpr int STRIDE = DV + ((64 / P - DV % 64) + 64) % 64;  // floats per partial row
    static constexpr int NKW = (DK + 63) / 64;               // waves that reduce k.q
    static_assert(RP >= 16 && RP % 8 == 0 && NT % 64 == 0 && NT >= 64 * NKW, "decode shape");
    static_assert(NT / P == 2 * DV, "one output column per P lanes");
    static_assert(STRIDE % 4 == 0, "partial rows hold aligned quads");
};

// Total threads of the persistent grid (4 Mi state floats in flight at most).
constexpr int64_t GRID_THREADS = 1 << 20;

// Fused layer work (Kimi K3 report digest: the bounded-decay section's gate
// g = g_min Sigmoid(e^{A_h} z) with g_min = -5, and the output-gate section's
// per-head RMSNorm times a Sigmoid gate), evaluated in fp32 where the decode
// kernels already hold the operands: the gate on the key channels before the
// forget step (both kernels); the epilogue on the output row in the
// single-token kernel (the NC4 lanes that hold it sit in the first wave, so its
// mean square is a few cross-lane adds) -- the window runs it as a second pass.
// (hardware exp and reciprocal, about 1e-6 relative: these sit on the serial
// path of each head, between barriers)
__device__ __forceinline__ float gate_from_logit(float z, float scale) {
    return -5.0f * __builtin_amdgcn_rcpf(1.0f + __expf(-scale * z));
}

// The output-gate logits of row `row`, columns 4 c4 .. +3, loaded ahead of use
// and kept as loaded (two registers for bf16) until the epilogue widens them.
template <typename T>
using GateRaw = typename std::conditional<sizeof(T) == 4, f32x4, u32x2>::type;

template <int NC4, typename T>
__device__ __forceinline__ GateRaw<T> epilogue_gate(const DecodeFusion &fx, int64_t row, int c4) {
    return *reinterpret_cast<const GateRaw<T> *>(reinterpret_cast<const T *>(fx.u) + row * (4 * NC4) + 4 * c4);
}

template <typename T>
__device__ __forceinline__ f32x4 widen_gate(GateRaw<T> x) {
    if constexpr (sizeof(T) == 4)
        return x;
    else
        return unpack_bf16x4(x);
}

template <int NC4, typename T>
__device__ __forceinline__ void epilogue_store(const DecodeFusion &fx, int64_t row, int c4, f32x4 ov, f32x4 uv,
                                               f32x4 wv) {
    float ss = ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3];
#pragma unroll
    for (int m = 1; m < NC4; m <<= 1) ss += __shfl_xor(ss, m);
    const float inv = __builtin_amdgcn_rsqf(ss * (1.f / (4 * NC4)) + fx.eps);
    f32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = ov[j] * inv * wv[j] * __builtin_amdgcn_rcpf(1.f + __expf(-uv[j]));
    T *y = reinterpret_cast<T *>(fx.y) + row * (4 * NC4) + 4 * c4;
    if constexpr (sizeof(T) == 4)
        *reinterpret_cast<f32x4 *>(y) = r;
    else
        *reinterpret_cast<bf16x4 *>(y) = to_bf16x4(r);
}

template <int DK, int DV, typename T, bool FX, bool CONV>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NT)) void decode_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ g, const T *__restrict__ beta, float *__restrict__ state,
    float *__restrict__ o, int64_t heads, int32_t H, DecodeFusion fx) {
    using Sh = DecodeShape<DK, DV>;
    constexpr int NC4 = Sh::NC4, RP = Sh::RP, NR = Sh::NR, P = Sh::P, NKW = Sh::NKW;
    const int tid = threadIdx.x;
    const int c4 = tid % NC4;
    const int rg = tid / NC4;
    const int64_t stride = gridDim.x;

    __shared__ float s_k[DK], s_q[DK], s_a[DK];
    __shared__ __attribute__((aligned(16))) float s_red[2][RP][Sh::STRIDE];
    __shared__ __attribute__((aligned(16))) float s_fin[2][DV];
    __shared__ float s_kq[2][NKW];
    // prologue: squared norms of q and k per wave, the convolved v (double-buffered)
    __shared__ float s_nq[CONV ? NKW : 1], s_nk[CONV ? NKW : 1];
    __shared__ __attribute__((aligned(16))) float s_vv[CONV ? 2 : 1][CONV ? DV : 4];
    constexpr int RS = 2 * DK + DV;  // pre-convolution row (q | k | v channels)

    // the RMSNorm weight of this lane's columns (epilogue lanes: rg == 0)
    f32x4 ep_w = zero4();
    if (FX && fx.u && rg == 0) ep_w = *reinterpret_cast<const f32x4 *>(fx.w + 4 * c4);

    auto load_rows = [&](f32x4 (&rows)[NR], int64_t head) {
        const float *S = state + head * (int64_t)(DK * DV);
#pragma unroll
        for (int r = 0; r < NR; ++r)
            rows[r] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4 *>(S + (int64_t)(rg + r * RP) * DV) + c4);
    };

    // One head.  LDS reuse across heads: s_k/s_q/s_a are last read before the
    // second barrier, s_red before the third, s_fin after the third (rewritten
    // only after the next head's second barrier), s_kq is double-buffered.
    auto step = [&](f32x4 (&rows)[NR], f32x4 (&nxt)[NR], int64_t head, int par) {
        float kk = 0.f, qq = 0.f;
        // prologue: y = Swish(w0 x_t + w1 x_{t-1} + w2 x_{t-2} + w3 x_{t-3}) per
        // channel from the 3-input cache, which then shifts in x_t (each channel
        // is read and written by one thread)
        const T *xr = q + head * RS;
        float *cc = CONV ? fx.conv_cache + head * RS * 3 : nullptr;
        const float *wr = CONV ? fx.conv_w + (head % H) * RS * 4 : nullptr;
        auto conv1 = [&](float x, int ch) -> float {
            float *c = cc + ch * 3;
            const float c0 = c[0], c1 = c[1], c2 = c[2];
            const f32x4 w4 = *reinterpret_cast<const f32x4 *>(wr + ch * 4);
            const float a = w4[0] * x + w4[1] * c2 + w4[2] * c1 + w4[3] * c0;
            c[0] = c1;
            c[1] = c2;
            c[2] = x;
            return a * __builtin_amdgcn_rcpf(1.f + __expf(-a));
        };
        if (tid < DK) {
            if constexpr (CONV) {
                qq = conv1(load_in(xr + tid), tid);
                kk = conv1(load_in(xr + DK + tid), DK + tid);
            } else {
                kk = load_in(k + head * DK + tid);
                qq = load_in(q + head * DK + tid);
            }
            s_k[tid] = kk;
            s_q[tid] = qq;
            const float gz = load_in(g + head * DK + tid);
            s_a[tid] = decay_exp(FX && fx.A_log ? gate_from_logit(gz, __expf(fx.A_log[head % H])) : gz);
        }
        if (tid < 64 * NKW) {  // whole waves: k.q (and the norms) by cross-lane sums
            float kq = kk * qq, nq = qq * qq, nk = kk * kk;
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) {
                kq += __shfl_xor(kq, m);
                if (CONV) {
                    nq += __shfl_xor(nq, m);
                    nk += __shfl_xor(nk, m);
                }
            }
            if ((tid & 63) == 0) {
                s_kq[par][tid >> 6] = kq;
                if (CONV) {
                    s_nq[tid >> 6] = nq;
                    s_nk[tid >> 6] = nk;
                }
            }
        }
        f32x4 vv;
        if constexpr (CONV) {
            // v's columns, each convolved once (row groups 0..3 take one column of
            // every quad) and shared through LDS
            if (rg < 4) {
                const int col = 4 * c4 + rg;
                s_vv[par][col] = conv1(load_in(xr + 2 * DK + col), 2 * DK + col);
            }
            vv = zero4();
        } else {
            vv = load_in4(v + head * DV + 4 * c4);
        }
        const float b = load_in(beta + head);
        GateRaw<T> ep_u = {};
        if (FX && fx.u && rg == 0) ep_u = epilogue_gate<NC4, T>(fx, head, c4);
        if (head + stride < heads) load_rows(nxt, head + stride);
        __syncthreads();

        // L2 normalisation of q and k (prologue): applied where they are read
        float inv_q = 1.f, inv_k = 1.f;
        if constexpr (CONV) {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int w = 0; w < NKW; ++w) {
                sq += s_nq[w];
                sk += s_nk[w];
            }
            inv_q = __builtin_amdgcn_rsqf(sq + fx.l2eps);
            inv_k = __builtin_amdgcn_rsqf(sk + fx.l2eps);
        }
        f32x4 pv = zero4(), pq = zero4();
        float kr[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int row = rg + r * RP;
            kr[r] = CONV ? s_k[row] * inv_k : s_k[row];
            rows[r] = rows[r] * s_a[row];                     // forget
            pv += kr[r] * rows[r];                            // partial S'^T k
            pq += (CONV ? s_q[row] * inv_q : s_q[row]) * rows[r];  // partial S'^T q
        }
        *reinterpret_cast<f32x4 *>(&s_red[0][rg][4 * c4]) = pv;
        *reinterpret_cast<f32x4 *>(&s_red[1][rg][4 * c4]) = pq;
        __syncthreads();

        {
            const int out = tid / P, part = tid % P;
            const int arr = out / DV, col = out % DV;
            float x = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) x += s_red[arr][part + P * j][col];
#pragma unroll
            for (int m = 1; m < P; m <<= 1) x += __shfl_xor(x, m);
            if (part == 0) s_fin[arr][col] = x;
        }
        __syncthreads();

        const f32x4 vhat = *reinterpret_cast<const f32x4 *>(&s_fin[0][4 * c4]);
        const f32x4 rq = *reinterpret_cast<const f32x4 *>(&s_fin[1][4 * c4]);
        float kq = 0.f;
#pragma unroll
        for (int w = 0; w < NKW; ++w) kq += s_kq[par][w];
        if constexpr (CONV) {
            kq *= inv_k * inv_q;
            vv = *reinterpret_cast<const f32x4 *>(&s_vv[par][4 * c4]);
        }
        const f32x4 delta = b * (vv - vhat);
        if (rg == 0) {
            const f32x4 ov = rq + kq * delta;
            if (o) reinterpret_cast<f32x4 *>(o + head * DV)[c4] = ov;
            if (FX && fx.u) epilogue_store<NC4, T>(fx, head, c4, ov, widen_gate<T>(ep_u), ep_w);
        }

        float *S = state + head * (int64_t)(DK * DV);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int row = rg + r * RP;
            __builtin_nontemporal_store(rows[r] + kr[r] * delta,  // erase + write
                                        reinterpret_cast<f32x4 *>(S + (int64_t)row * DV) + c4);
        }
    };

    int64_t head = blockIdx.x;
    if (head >= heads) return;
    f32x4 ra[NR], rb[NR];
    load_rows(ra, head);
    for (;;) {  // two heads per trip so the register sets swap roles without copies
        step(ra, rb, head, 0);
        head += stride;
        if (head >= heads) break;
        step(rb, ra, head, 1);
        head += stride;
        if (head >= heads) break;
    }
}

// A window of Tw consecutive tokens per sequence (speculative-decoding
// verification and replay; Kimi K3 report digest, serving section): the state
// of each (sequence, head) is read once, carried through the window in
// registers, and written back once -- the state after the first acc tokens,
// acc = accept[b] clamped to [0, Tw] (all Tw without accept; no write when 0) --
// while o gets the output of every token of the window.  Per token the work is
// the single-token step above; the next token's inputs are loaded while the
// current token is reduced, and the next head's state during the window's first
// token, so its latency hides behind the whole window.  With Tw tokens per state
// pass the kernel does Tw times the arithmetic per byte of the single step, so
// beyond a few tokens it is bound by the vector ALUs, not HBM: the workgroups
// are half as large (two per compute unit, at most 128 registers per lane) so
// that one's barrier waits are filled by the other's arithmetic.  Inputs are
// [B, Tw, H, ...] (token-major within a sequence).
//
// With a replay (the serving form of the same page's scheme: the verifier's
// accepted count for a window is known only after the window ran), the tokens
// of a (sequence, head) are first rp = replay[b] tokens of the previous window
// (inputs [B, Tp, H, ...], no outputs), then the Tw tokens of this window; the
// state is written back after token rp + acc, acc = accept[b] (or acc_default),
// so with no accept the committed state is the one after the accepted prefix
// of the previous window and this window's drafts stay uncommitted.
//
// With CONV (the layer's decode window, same page's layer paragraph: ShortConv of
// size 4 + Swish on q, k, v, L2 norms of q and k) q points at pre-convolution rows
// q | k | v of 2 dk + dv channels ([B, Tw, H, .], the replay's at pq): each token
// is convolved in order from a three-input window per channel that starts as the
// sequence's cache (fx.conv_cache) and slides through the replayed and the new
// tokens; at the commit point the cache receives the window as it stands, so
// cache and state are committed together.  q and k channel c sit with thread
// c < dk, v column 4 c4 + rg with row group rg < 4 (shared through LDS); the norms
// of q and k join the k.q sums and are applied where q and k are read, as in the
// single-token kernel.
// Threads per window workgroup, at most.
constexpr int WINDOW_THREADS = 512;

template <int DK, int DV, typename T, bool FX, bool REPLAY, bool CONV = false>
__global__ __launch_bounds__((DecodeShape<DK, DV, WINDOW_THREADS>::NT))
__attribute__((amdgpu_waves_per_eu(CONV ? (DecodeShape<DK, DV, WINDOW_THREADS>::NT + 255) / 256 : (2 * DecodeShape<DK, DV, WINDOW_THREADS>::NT + 255) / 256, 8)))
void decode_window_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ g, const T *__restrict__ beta, float *__restrict__ state,
    float *__restrict__ o, const int32_t *__restrict__ accept, int64_t heads, int32_t H, int32_t Tw,
    DecodeFusion fx, const T *__restrict__ pq, const T *__restrict__ pk, const T *__restrict__ pv,
    const T *__restrict__ pg, const T *__restrict__ pb, const int32_t *__restrict__ replay, int32_t Tp,
    int32_t acc_default) {
    using Sh = DecodeShape<DK, DV, WINDOW_THREADS>;
    constexpr int NC4 = Sh::NC4, RP = Sh::RP, NR = Sh::NR, P = Sh::P, NKW = Sh::NKW;
    const int tid = threadIdx.x;
    const int c4 = tid % NC4;
    const int rg = tid / NC4;
    const int64_t stride = gridDim.x;

    __shared__ float s_k[DK], s_q[DK], s_a[DK];
    __shared__ __attribute__((aligned(16))) float s_red[2][RP][Sh::STRIDE];
    __shared__ __attribute__((aligned(16))) float s_fin[2][DV];
    __shared__ float s_kq[2][NKW];
    __shared__ float s_nq[CONV ? NKW : 1], s_nk[CONV ? NKW : 1];
    __shared__ __attribute__((aligned(16))) float s_vv[CONV ? 2 : 1][CONV ? DV : 4];
    constexpr int RS = 2 * DK + DV;  // pre-convolution row (q | k | v channels)

    struct Tok {
        float k, q, g, b;  // k, q, g of key channel tid (tid < DK)
        f32x4 v;           // v of columns 4 c4 .. +3
    };
    // Replayed tokens of a head's sequence (0 without a replay), uniform per head.
    auto replay_of = [&](int64_t hd) -> int {
        if constexpr (!REPLAY) return 0;
        const int r = replay[hd / H];
        return r < 0 ? 0 : (r > Tp ? Tp : r);
    };
    // Token inputs through buffer resources based at the token's row (uniform),
    // so every lane offset is a loop-invariant 32-bit register.  Head indices
    // stay below 2^31 (B * T * H < 2^31 is checked on the host).  Token t of a
    // head is replayed token t (t < rp, the head's replay count) or window token
    // t - rp.
    auto load_tok = [&](Tok &x, uint32_t hd, int t, int rp) {
        const uint32_t bq = hd / (uint32_t)H;
        const bool rep = REPLAY && t < rp;
        const int64_t row = rep ? ((int64_t)bq * Tp + t) * H + (hd - bq * (uint32_t)H)
                                : ((int64_t)bq * Tw + (t - rp)) * H + (hd - bq * (uint32_t)H);
        const T *kb = rep ? pk : k, *qb = rep ? pq : q, *gb = rep ? pg : g, *vb = rep ? pv : v, *bb = rep ? pb : beta;
        if constexpr (CONV) {
            // q and k channel tid, v column 4 c4 + rg (rg < 4) of the pre-convolution row
            const rsrc_t rx = make_rsrc(qb + row * RS, RS * sizeof(T));
            const rsrc_t rgt = make_rsrc(gb + row * DK, DK * sizeof(T));
            auto elem = [&](const rsrc_t &r, int i) {
                if constexpr (sizeof(T) == 4)
                    return __uint_as_float(buf_load_u32(r, (uint32_t)i * 4u));
                else
                    return bf16_bits_to_f32(buf_load_u16(r, (uint32_t)i * 2u));
            };
            if (tid < DK) {
                x.q = elem(rx, tid);
                x.k = elem(rx, DK + tid);
                x.g = elem(rgt, tid);
            } else {
                x.k = x.q = x.g = 0.f;
            }
            x.v = zero4();
            if (rg < 4) x.v[0] = elem(rx, 2 * DK + 4 * c4 + rg);
            x.b = load_in(bb + row);
            return;
        }
        if (tid < DK) {
            const uint32_t off = tid * (uint32_t)sizeof(T);
            const rsrc_t rk = make_rsrc(kb + row * DK, DK * sizeof(T));
            const rsrc_t rq = make_rsrc(qb + row * DK, DK * sizeof(T));
            const rsrc_t rgt = make_rsrc(gb + row * DK, DK * sizeof(T));
            if constexpr (sizeof(T) == 4) {
                x.k = __uint_as_float(buf_load_u32(rk, off));
                x.q = __uint_as_float(buf_load_u32(rq, off));
                x.g = __uint_as_float(buf_load_u32(rgt, off));
            } else {
                x.k = bf16_bits_to_f32(buf_load_u16(rk, off));
                x.q = bf16_bits_to_f32(buf_load_u16(rq, off));
                x.g = bf16_bits_to_f32(buf_load_u16(rgt, off));
            }
        } else {
            x.k = x.q = x.g = 0.f;
        }
        const rsrc_t rv = make_rsrc(vb + row * DV, DV * sizeof(T));
        if constexpr (sizeof(T) == 4)
            x.v = __builtin_bit_cast(f32x4, buf_load_u32x4(rv, 16u * c4));
        else
            x.v = unpack_bf16x4(buf_load_u32x2(rv, 8u * c4));
        x.b = load_in(bb + row);
    };
    // State rows go through a buffer resource per head: one 32-bit lane offset
    // (row rg, quad c4) serves all NR rows, the row step is the uniform offset.
    const uint32_t soff = (uint32_t)(rg * DV + 4 * c4) * 4u;
    constexpr uint32_t ROW_STEP = RP * DV * 4u, NT_POLICY = 2;  // non-temporal
    auto state_rsrc = [&](int64_t hd) {
        return make_rsrc(state + hd * (int64_t)(DK * DV), DK * DV * 4u);
    };
    auto load_rows = [&](f32x4 (&rows)[NR], int64_t hd) {
        const rsrc_t rs = state_rsrc(hd);
#pragma unroll
        for (int r = 0; r < NR; ++r)
            rows[r] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, soff, r * ROW_STEP, NT_POLICY));
    };

    Tok cur, nxt;
    int par = 0;
    // One (sequence, head): the window's tokens in order, the state rows in
    // registers throughout.  The next head's state rows (into nrows) are
    // loaded during the first token, its first token during the last.
    auto window = [&](f32x4 (&rows)[NR], f32x4 (&nrows)[NR], int64_t head) {
        const int64_t bq = head / H;
        int acc = acc_default;
        if (accept) {
            acc = accept[bq];
            acc = acc < 0 ? 0 : (acc > Tw ? Tw : acc);
        }
        const int rp = replay_of(head), n = rp + Tw;
        acc += rp;  // the state is written back after token acc (not at all when 0)
        const bool more = head + stride < heads;
        const int rp_next = more ? replay_of(head + stride) : 0;
        const rsrc_t rs = state_rsrc(head);
        const float gscale = FX && fx.A_log ? __expf(fx.A_log[head - bq * H]) : 0.f;
        // (layer) the convolution windows (oldest first) and taps of this thread's channels
        float cwq[3] = {0.f, 0.f, 0.f}, cwk[3] = {0.f, 0.f, 0.f}, cwv[3] = {0.f, 0.f, 0.f};
        f32x4 wq4 = zero4(), wk4 = zero4(), wv4 = zero4();
        float *ccache = nullptr;
        const int vcol = 2 * DK + 4 * c4 + rg;  // (rg < 4)
        if constexpr (CONV) {
            ccache = fx.conv_cache + head * (int64_t)(RS * 3);
            const float *wr = fx.conv_w + (head - bq * H) * (int64_t)(RS * 4);
            if (tid < DK) {
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    cwq[j] = ccache[tid * 3 + j];
                    cwk[j] = ccache[(DK + tid) * 3 + j];
                }
                wq4 = *reinterpret_cast<const f32x4 *>(wr + tid * 4);
                wk4 = *reinterpret_cast<const f32x4 *>(wr + (DK + tid) * 4);
            }
            if (rg < 4) {
#pragma unroll
                for (int j = 0; j < 3; ++j) cwv[j] = ccache[vcol * 3 + j];
                wv4 = *reinterpret_cast<const f32x4 *>(wr + vcol * 4);
            }
        }
        // Swish of the 4-tap convolution (w[j] on x_{t-j}), then the window slides
        auto conv_step = [](const f32x4 &w4, float x, float (&c)[3]) {
            const float a = w4[0] * x + w4[1] * c[2] + w4[2] * c[1] + w4[3] * c[0];
            c[0] = c[1];
            c[1] = c[2];
            c[2] = x;
            return a * __builtin_amdgcn_rcpf(1.f + __expf(-a));
        };
        for (int t = 0; t < n; ++t) {
            // LDS reuse across tokens as across heads in the single-token kernel
            float kk = cur.k, qq = cur.q;
            if constexpr (CONV) {
                if (tid < DK) {
                    qq = conv_step(wq4, cur.q, cwq);
                    kk = conv_step(wk4, cur.k, cwk);
                }
                if (rg < 4) s_vv[par][vcol - 2 * DK] = conv_step(wv4, cur.v[0], cwv);
            }
            if (tid < DK) {
                s_k[tid] = kk;
                s_q[tid] = qq;
                s_a[tid] = decay_exp(FX && fx.A_log ? gate_from_logit(cur.g, gscale) : cur.g);
            }
            if (tid < 64 * NKW) {
                float kq = kk * qq, nq = qq * qq, nk = kk * kk;
#pragma unroll
                for (int m = 32; m >= 1; m >>= 1) {
                    kq += __shfl_xor(kq, m);
                    if (CONV) {
                        nq += __shfl_xor(nq, m);
                        nk += __shfl_xor(nk, m);
                    }
                }
                if ((tid & 63) == 0) {
                    s_kq[par][tid >> 6] = kq;
                    if (CONV) {
                        s_nq[tid >> 6] = nq;
                        s_nk[tid >> 6] = nk;
                    }
                }
            }
            f32x4 vv = cur.v;
            const float bb = cur.b;
            if (t == 0 && more) load_rows(nrows, head + stride);
            if (t + 1 < n) {
                load_tok(nxt, head, t + 1, rp);
            } else if (more) {
                load_tok(nxt, head + stride, 0, rp_next);
            }
            __syncthreads();

            // (layer) L2 normalisation of q and k, applied where they are read
            float inv_q = 1.f, inv_k = 1.f;
            if constexpr (CONV) {
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int w = 0; w < NKW; ++w) {
                    sq += s_nq[w];
                    sk += s_nk[w];
                }
                inv_q = __builtin_amdgcn_rsqf(sq + fx.l2eps);
                inv_k = __builtin_amdgcn_rsqf(sk + fx.l2eps);
            }
            f32x4 pv = zero4(), pq = zero4();
            float kr[NR];
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int row = rg + r * RP;
                kr[r] = CONV ? s_k[row] * inv_k : s_k[row];
                rows[r] = rows[r] * s_a[row];  // forget
                pv += kr[r] * rows[r];
                pq += (CONV ? s_q[row] * inv_q : s_q[row]) * rows[r];
            }
            *reinterpret_cast<f32x4 *>(&s_red[0][rg][4 * c4]) = pv;
            *reinterpret_cast<f32x4 *>(&s_red[1][rg][4 * c4]) = pq;
            __syncthreads();
            {
                const int out = tid / P, part = tid % P;
                const int arr = out / DV, col = out % DV;
                float x = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) x += s_red[arr][part + P * j][col];
#pragma unroll
                for (int m = 1; m < P; m <<= 1) x += __shfl_xor(x, m);
                if (part == 0) s_fin[arr][col] = x;
            }
            __syncthreads();

            const f32x4 vhat = *reinterpret_cast<const f32x4 *>(&s_fin[0][4 * c4]);
            const f32x4 rq = *reinterpret_cast<const f32x4 *>(&s_fin[1][4 * c4]);
            float kq = 0.f;
#pragma unroll
            for (int w = 0; w < NKW; ++w) kq += s_kq[par][w];
            if constexpr (CONV) {
                kq *= inv_k * inv_q;
                vv = *reinterpret_cast<const f32x4 *>(&s_vv[par][4 * c4]);
            }
            const f32x4 delta = bb * (vv - vhat);
            const int64_t orow = (bq * Tw + (t - rp)) * H + (head - bq * H);
            if (o && rg == 0 && t >= rp) reinterpret_cast<f32x4 *>(o + orow * DV)[c4] = rq + kq * delta;
#pragma unroll
            for (int r = 0; r < NR; ++r) rows[r] += kr[r] * delta;  // erase + write
            if (t + 1 == acc) {
#pragma unroll
                for (int r = 0; r < NR; ++r)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, rows[r]), rs, soff,
                                                           r * ROW_STEP, NT_POLICY);
                if constexpr (CONV) {  // the convolution cache, committed with the state
                    if (tid < DK) {
#pragma unroll
                        for (int j = 0; j < 3; ++j) {
                            ccache[tid * 3 + j] = cwq[j];
                            ccache[(DK + tid) * 3 + j] = cwk[j];
                        }
                    }
                    if (rg < 4) {
#pragma unroll
                        for (int j = 0; j < 3; ++j) ccache[vcol * 3 + j] = cwv[j];
                    }
                }
            }

            cur = nxt;
            par ^= 1;
        }
    };

    int64_t head = blockIdx.x;
    if (head >= heads) return;
    f32x4 ra[NR], rb[NR];
    load_rows(ra, head);
    load_tok(cur, head, 0, replay_of(head));
    nxt = cur;
    for (;;) {  // two heads per trip so the register sets swap roles without copies
        window(ra, rb, head);
        head += stride;
        if (head >= heads) break;
        window(rb, ra, head);
        head += stride;
        if (head >= heads) break;
    }
}

template <int DK, int DV, typename T>
static hipError_t launch_decode_t(const DecodeArgs &a) {
    using Sh = DecodeShape<DK, DV>;
    const int64_t heads = (int64_t)a.B * a.H;
    const int64_t cap = GRID_THREADS / Sh::NT;
    const int64_t grid = heads < cap ? heads : cap;
    const bool conv = a.fx.conv_w != nullptr;
    const bool fused = conv || a.fx.A_log || a.fx.u;
    auto kern = conv ? decode_kernel<DK, DV, T, true, true>
                     : (fused ? decode_kernel<DK, DV, T, true, false> : decode_kernel<DK, DV, T, false, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Sh::NT), 0, (hipStream_t)a.stream, (const T *)a.q,
                       (const T *)a.k, (const T *)a.v, (const T *)a.g, (const T *)a.beta, a.state, a.o, heads,
                       a.H, a.fx);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_decode_dt(const DecodeArgs &a) {
#define KDA_DEC_CASE(DKV, DVV) \
    if (a.dk == DKV && a.dv == DVV) return launch_decode_t<DKV, DVV, T>(a);
#define KDA_DEC_ROW(DKV) KDA_DEC_CASE(DKV, 16) KDA_DEC_CASE(DKV, 32) KDA_DEC_CASE(DKV, 64) KDA_DEC_CASE(DKV, 128)
    KDA_DEC_ROW(16) KDA_DEC_ROW(32) KDA_DEC_ROW(64) KDA_DEC_ROW(128)
#undef KDA_DEC_ROW
#undef KDA_DEC_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs &a) {
    return a.bf16 ? launch_decode_dt<__bf16>(a) : launch_decode_dt<float>(a);
}

template <int DK, int DV, typename T>
static hipError_t launch_window_t(const DecodeWindowArgs &a) {
    using Sh = DecodeShape<DK, DV, WINDOW_THREADS>;
    const int64_t heads = (int64_t)a.B * a.H;
    const int64_t cap = GRID_THREADS / Sh::NT;
    const int64_t grid = heads < cap ? heads : cap;
    const bool fused = a.fx.A_log != nullptr;
    auto kern = a.fx.conv_w
                    ? (a.replay ? decode_window_kernel<DK, DV, T, true, true, true>
                                : decode_window_kernel<DK, DV, T, true, false, true>)
                    : a.replay ? (fused ? decode_window_kernel<DK, DV, T, true, true> : decode_window_kernel<DK, DV, T, false, true>)
                               : (fused ? decode_window_kernel<DK, DV, T, true, false> : decode_window_kernel<DK, DV, T, false, false>);
    hipLaunchKernelGGL(kern,
                       dim3((unsigned)grid), dim3(Sh::NT), 0, (hipStream_t)a.stream, (const T *)a.q,
                       (const T *)a.k, (const T *)a.v, (const T *)a.g, (const T *)a.beta, a.state, a.o,
                       a.accept, heads, a.H, a.T, a.fx, (const T *)a.pq, (const T *)a.pk, (const T *)a.pv,
                       (const T *)a.pg, (const T *)a.pbeta, a.replay, a.Tp, a.acc_default < 0 ? a.T : a.acc_default);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.fx.u) return e;
    // The epilogue as a second pass over the window's outputs: inside the window
    // kernel its registers pushed the token loop into spills, whose reloads then
    // waited on every prefetch in flight.
    const OutNormGateArgs ep{a.o, a.fx.u, a.fx.w, a.fx.eps, (int64_t)a.B * a.T, a.H, a.dv, a.bf16, a.fx.y, a.stream};
    return launch_out_norm_gate(ep);
}

template <typename T>
static hipError_t launch_window_dt(const DecodeWindowArgs &a) {
#define KDA_WIN_CASE(DKV, DVV) \
    if (a.dk == DKV && a.dv == DVV) return launch_window_t<DKV, DVV, T>(a);
#define KDA_WIN_ROW(DKV) KDA_WIN_CASE(DKV, 16) KDA_WIN_CASE(DKV, 32) KDA_WIN_CASE(DKV, 64) KDA_WIN_CASE(DKV, 128)
    KDA_WIN_ROW(16) KDA_WIN_ROW(32) KDA_WIN_ROW(64) KDA_WIN_ROW(128)
#undef KDA_WIN_ROW
#undef KDA_WIN_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_decode_window(const DecodeWindowArgs &a) {
    const int64_t tokens = (int64_t)a.T + (a.replay ? a.Tp : 0);
    if (a.form == 2 || (a.form == 0 && tokens >= WINDOW_CHUNK_MIN_TOKENS && window_chunk_supported(a)))
        return launch_window_chunk(a);
    return a.bf16 ? launch_window_dt<__bf16>(a) : launch_window_dt<float>(a);
}

}  // namespace kda
