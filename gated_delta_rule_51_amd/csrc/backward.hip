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
// Four kernels, all fp32 on the vector ALUs with the chunk's operands in LDS:
//   1. fwd_ckpt  per (sequence, head, 16-column slice): the forward chunk recurrence,
//      writing S at every chunk start and every chunk's Delta (and the final state);
//   2. adjoint   per (sequence, head, 16-column slice): the adjoint recurrence in
//      reverse chunk order, writing dV, S^ after every chunk, E, and dinit;
//   3. grads     per (chunk, head), all dv columns in 16-column slices: dq, dk, dbeta
//      and the log-decay increments;
//   4. dg_scan   per (sequence, head, key channel): the reverse cumulative sum.
// The column slices of 1 and 2 are independent (the state's columns evolve
// separately), the chunks of 3 too, so only the recurrences in 1 and 2 are serial.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int BWD_THREADS = 256;

// The state-independent quantities of one chunk (n <= 16 tokens; rows past n are
// zero with g = 0, an exact no-op), in fp32.
template <int DK>
struct ChunkOps {
    float Q[16][DK], K[16][DK];        // raw q, k
    float G[16][DK];                   // cumulative log-decay
    float Kp[16][DK], Km[16][DK];      // K e^{G}, K e^{-G}
    float Qp[16][DK], Kt[16][DK];      // Q e^{G}, K e^{G_n - G}
    float gam[DK];                     // e^{G_n}
    float A[16][16], Ap[16][16];       // diag(beta) stril(K+ K-^T), stril(K+ K-^T)
    float Aqk[16][16];                 // tril(Q+ K-^T)
    float T[16][16], Tp[16][16];       // (I + A)^-1, T diag(beta)
    float beta[16];
};

template <int DK, typename T>
__device__ void chunk_prep(ChunkOps<DK> &P, const T *q, const T *k, const T *g, const T *beta, int64_t t0,
                           int n, int32_t H, int h) {
    const int tid = threadIdx.x;
    if (tid < 16) P.beta[tid] = tid < n ? load_in(beta + (t0 + tid) * H + h) : 0.f;
    // One thread per key channel walks the chunk's rows: the cumulative log-decay in
    // registers, one exp per element (e^{-G} and e^{G_n - G} from e^{G} and e^{G_n}).
    for (int ch = tid; ch < DK; ch += BWD_THREADS) {
        float G[16], qv[16], kv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t e = ((t0 + r) * H + h) * DK + ch;
            const bool in = r < n;
            G[r] = in ? load_in(g + e) : 0.f;
            qv[r] = in ? load_in(q + e) : 0.f;
            kv[r] = in ? load_in(k + e) : 0.f;
        }
#pragma unroll
        for (int r = 1; r < 16; ++r) G[r] += G[r - 1];
        const float egn = expf(G[15]);
        P.gam[ch] = egn;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float ep = expf(G[r]), em = 1.f / ep;
            P.Q[r][ch] = qv[r];
            P.K[r][ch] = kv[r];
            P.G[r][ch] = G[r];
            P.Kp[r][ch] = kv[r] * ep;
            P.Km[r][ch] = kv[r] * em;
            P.Qp[r][ch] = qv[r] * ep;
            P.Kt[r][ch] = kv[r] * (egn * em);
        }
    }
    __syncthreads();
    {
        const int r = tid / 16, i = tid % 16;  // 256 threads: one (r, i) entry each
        float kk = 0.f, qk = 0.f;
        for (int ch = 0; ch < DK; ++ch) {
            const float km = P.Km[i][ch];
            kk += P.Kp[r][ch] * km;
            qk += P.Qp[r][ch] * km;
        }
        P.Ap[r][i] = i < r ? kk : 0.f;
        P.A[r][i] = i < r ? P.beta[r] * kk : 0.f;
        P.Aqk[r][i] = i <= r ? qk : 0.f;
    }
    __syncthreads();
    if (tid < 16) {
        // column j of the unit lower triangular inverse by forward substitution, the
        // column in registers (every index compile-time, so nothing goes to scratch)
        const int j = tid;
        float t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float x = i == j ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) x -= (m >= j ? P.A[i][m] : 0.f) * t[m];
            t[i] = i < j ? 0.f : x;
            P.T[i][j] = t[i];
            P.Tp[i][j] = t[i] * P.beta[j];
        }
    }
    __syncthreads();
}

// Chunk c of sequence s occupies slot cu[s]/16 + s + c (the prefill workspace's map).
__device__ __forceinline__ int64_t slot_of(const int32_t *cu, int s, int c) {
    return (int64_t)cu[s] / 16 + s + c;
}

// ------------------------------------------------------------------ 1. forward checkpoints
template <int DK, int DV, typename T>
__global__ __launch_bounds__(BWD_THREADS) void bwd_fwd_ckpt_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ g,
    const T *__restrict__ beta, const float *__restrict__ init, const int32_t *__restrict__ cu, int32_t H,
    float *__restrict__ sck, float *__restrict__ dbuf, float *__restrict__ sfin) {
    constexpr int NSL = DV / 16;
    const int chain = blockIdx.x / NSL, col0 = (blockIdx.x % NSL) * 16;
    const int s = chain / H, h = chain % H;
    const int tid = threadIdx.x;
    __shared__ ChunkOps<DK> P;
    __shared__ float S[DK][16], Y[16][16], D[16][16];
    const int64_t hd = (int64_t)s * H + h;
    for (int idx = tid; idx < DK * 16; idx += BWD_THREADS) {
        const int ch = idx / 16, col = idx % 16;
        S[ch][col] = init ? init[(hd * DK + ch) * DV + col0 + col] : 0.f;
    }
    const int64_t bos = cu[s], len = cu[s + 1] - bos;
    const int nc = (int)((len + 15) / 16);
    for (int c = 0; c < nc; ++c) {
        __syncthreads();
        const int64_t t0 = bos + 16 * c;
        const int n = (int)(len - 16 * c < 16 ? len - 16 * c : 16);
        chunk_prep<DK>(P, q, k, g, beta, t0, n, H, h);
        const int64_t slot = slot_of(cu, s, c);
        for (int idx = tid; idx < DK * 16; idx += BWD_THREADS) {
            const int ch = idx / 16, col = idx % 16;
            sck[((slot * H + h) * DK + ch) * DV + col0 + col] = S[ch][col];
        }
        {
            const int r = tid / 16, col = tid % 16;
            float ks = 0.f;
            for (int ch = 0; ch < DK; ++ch) ks += P.Kp[r][ch] * S[ch][col];
            const float vv = r < n ? load_in(v + ((t0 + r) * H + h) * DV + col0 + col) : 0.f;
            Y[r][col] = vv - ks;
        }
        __syncthreads();
        {
            const int r = tid / 16, col = tid % 16;
            float d = 0.f;
            for (int m = 0; m < 16; ++m) d += P.Tp[r][m] * Y[m][col];
            D[r][col] = d;
            dbuf[((slot * H + h) * 16 + r) * DV + col0 + col] = d;
        }
        __syncthreads();
        for (int idx = tid; idx < DK * 16; idx += BWD_THREADS) {
            const int ch = idx / 16, col = idx % 16;
            float x = P.gam[ch] * S[ch][col];
            for (int r = 0; r < 16; ++r) x += P.Kt[r][ch] * D[r][col];
            S[ch][col] = x;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < DK * 16; idx += BWD_THREADS) {
        const int ch = idx / 16, col = idx % 16;
        sfin[(hd * DK + ch) * DV + col0 + col] = S[ch][col];
    }
}

// ------------------------------------------------------------------ 2. adjoint sweep
template <int DK, int DV, typename T>
__global__ __launch_bounds__(BWD_THREADS) void bwd_adjoint_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ g, const T *__restrict__ beta,
    const float *__restrict__ dO, const float *__restrict__ dfinal, const int32_t *__restrict__ cu, int32_t H,
    float *__restrict__ hck, float *__restrict__ ebuf, float *__restrict__ dv, float *__restrict__ dinit) {
    constexpr int NSL = DV / 16;
    const int chain = blockIdx.x / NSL, col0 = (blockIdx.x % NSL) * 16;
    const int s = chain / H, h = chain % H;
    const int tid = threadIdx.x;
    __shared__ ChunkOps<DK> P;
    __shared__ float Sh[DK][16], Ob[16][16], X[16][16], dV[16][16];
    const int64_t hd = (int64_t)s * H + h;
    for (int idx = tid; idx < DK * 16; idx += BWD_THREADS) {
        const int ch = idx / 16, col = idx % 16;
        Sh[ch][col] = dfinal ? dfinal[(hd * DK + ch) * DV + col0 + col] : 0.f;
    }
    const int64_t bos = cu[s], len = cu[s + 1] - bos;
    const int nc = (int)((len + 15) / 16);
    for (int c = nc - 1; c >= 0; --c) {
        __syncthreads();
        const int64_t t0 = bos + 16 * c;
        const int n = (int)(len - 16 * c < 16 ? len - 16 * c : 16);
        chunk_prep<DK>(P, q, k, g, beta, t0, n, H, h);
        const int64_t slot = slot_of(cu, s, c);
        for (int idx = tid; idx < DK * 16; idx += BWD_THREADS) {
            const int ch = idx / 16, col = idx % 16;
            hck[((slot * H + h) * DK + ch) * DV + col0 + col] = Sh[ch][col];
        }
        {
            const int r = tid / 16, col = tid % 16;
            Ob[r][col] = r < n ? dO[((t0 + r) * H + h) * DV + col0 + col] : 0.f;
        }
        __syncthreads();
        {
            const int r = tid / 16, col = tid % 16;
            float x = 0.f;
            for (int i = 0; i < 16; ++i) x += P.Aqk[i][r] * Ob[i][col];
            for (int ch = 0; ch < DK; ++ch) x += P.Kt[r][ch] * Sh[ch][col];
            X[r][col] = x;
        }
        __syncthreads();
        {
            const int r = tid / 16, col = tid % 16;
            float e = 0.f;
            for (int i = 0; i < 16; ++i) e += P.T[i][r] * X[i][col];
            ebuf[((slot * H + h) * 16 + r) * DV + col0 + col] = e;
            const float d = P.beta[r] * e;
            dV[r][col] = d;
            if (r < n) dv[((t0 + r) * H + h) * DV + col0 + col] = d;
        }
        __syncthreads();
        for (int idx = tid; idx < DK * 16; idx += BWD_THREADS) {
            const int ch = idx / 16, col = idx % 16;
            float x = P.gam[ch] * Sh[ch][col];
            for (int r = 0; r < 16; ++r) x += P.Qp[r][ch] * Ob[r][col] - P.Kp[r][ch] * dV[r][col];
            Sh[ch][col] = x;
        }
    }
    __syncthreads();
    if (dinit)
        for (int idx = tid; idx < DK * 16; idx += BWD_THREADS) {
            const int ch = idx / 16, col = idx % 16;
            dinit[(hd * DK + ch) * DV + col0 + col] = Sh[ch][col];
        }
}

// ------------------------------------------------------------------ 3. per-chunk gradients
template <int DK, int DV, typename T>
__global__ __launch_bounds__(BWD_THREADS) void bwd_grads_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ g,
    const T *__restrict__ beta, const float *__restrict__ dO, const int32_t *__restrict__ cu, int32_t nseq,
    int32_t H, const float *__restrict__ sck, const float *__restrict__ hck, const float *__restrict__ dbuf,
    const float *__restrict__ ebuf, float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ incr,
    float *__restrict__ dbeta) {
    constexpr int NOUT = 16 * DK / BWD_THREADS > 0 ? 16 * DK / BWD_THREADS : 1;  // (r, ch) outputs per thread
    static_assert(16 * DK % BWD_THREADS == 0 || DK == 16, "outputs spread evenly");
    const int64_t slot = blockIdx.x / H;
    const int h = (int)(blockIdx.x % H);
    const int tid = threadIdx.x;
    // the sequence owning this slot: the last s with cu[s]/16 + s <= slot
    int s = 0, hi = nseq - 1;
    while (s < hi) {
        const int mid = (s + hi + 1) >> 1;
        if (slot_of(cu, mid, 0) <= slot) s = mid;
        else hi = mid - 1;
    }
    const int64_t bos = cu[s], len = cu[s + 1] - bos;
    const int c = (int)(slot - slot_of(cu, s, 0));
    if (16 * (int64_t)c >= len) return;  // a slot no chunk uses (the block is uniform)
    const int64_t t0 = bos + 16 * c;
    const int n = (int)(len - 16 * c < 16 ? len - 16 * c : 16);

    __shared__ ChunkOps<DK> P;
    __shared__ float S0[DK][17], Sh[DK][17];          // one 16-column slice of S0 and S^ (padded rows)
    __shared__ float Ob[16][17], Dl[16][17], El[16][17], Vl[16][17];
    __shared__ float M[4][16][16];
    __shared__ float dbp[16][16];
    chunk_prep<DK>(P, q, k, g, beta, t0, n, H, h);

    float QS[NOUT], DS[NOUT], ES[NOUT];
#pragma unroll
    for (int m = 0; m < NOUT; ++m) QS[m] = DS[m] = ES[m] = 0.f;
    float M1 = 0.f, M2 = 0.f, M3 = 0.f, M4 = 0.f, dbacc = 0.f;
    const int mr = tid / 16, mi = tid % 16;  // this thread's (r, i) entry of the 16x16 matrices
    const float *S0g = sck + (slot * H + h) * (int64_t)DK * DV;
    const float *Shg = hck + (slot * H + h) * (int64_t)DK * DV;
    for (int col0 = 0; col0 < DV; col0 += 16) {
        for (int idx = tid; idx < DK * 16; idx += BWD_THREADS) {
            const int ch = idx / 16, col = idx % 16;
            S0[ch][col] = S0g[ch * DV + col0 + col];
            Sh[ch][col] = Shg[ch * DV + col0 + col];
        }
        {
            const int r = tid / 16, col = tid % 16;
            const bool in = r < n;
            Ob[r][col] = in ? dO[((t0 + r) * H + h) * DV + col0 + col] : 0.f;
            Dl[r][col] = dbuf[((slot * H + h) * 16 + r) * DV + col0 + col];
            El[r][col] = ebuf[((slot * H + h) * 16 + r) * DV + col0 + col];
            Vl[r][col] = in ? load_in(v + ((t0 + r) * H + h) * DV + col0 + col) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < NOUT; ++m) {
            const int o = tid + BWD_THREADS * m;
            const int r = o / DK, ch = o % DK;
            if (r >= 16) continue;
            float a = 0.f, b = 0.f, e = 0.f;
            for (int j = 0; j < 16; ++j) {
                a += Ob[r][j] * S0[ch][j];
                b += Dl[r][j] * Sh[ch][j];
                e += El[r][j] * S0[ch][j];
            }
            QS[m] += a;
            DS[m] += b;
            ES[m] += e;
        }
        for (int j = 0; j < 16; ++j) {
            M1 += Dl[mr][j] * Ob[mi][j];
            M2 += Dl[mr][j] * P.beta[mi] * El[mi][j];
            M3 += El[mr][j] * Dl[mi][j];
            M4 += Ob[mr][j] * Dl[mi][j];
        }
        {  // u_r at column col0 + mi, and its part of dbeta_r
            float u = 0.f;
            for (int ch = 0; ch < DK; ++ch) u += P.Kp[mr][ch] * S0[ch][mi];
            for (int i = 0; i < 16; ++i) u += P.Ap[mr][i] * Dl[i][mi];
            dbacc += El[mr][mi] * (Vl[mr][mi] - u);
        }
        __syncthreads();
    }
    M[0][mr][mi] = M1;
    M[1][mr][mi] = M2;
    M[2][mr][mi] = M3;
    M[3][mr][mi] = M4;
    dbp[mr][mi] = dbacc;
    __syncthreads();
    if (tid < 16 && tid < n) {
        float x = 0.f;
        for (int i = 0; i < 16; ++i) x += dbp[tid][i];
        dbeta[(t0 + tid) * H + h] = x;
    }
#pragma unroll
    for (int m = 0; m < NOUT; ++m) {
        const int o = tid + BWD_THREADS * m;
        const int r = o / DK, ch = o % DK;
        if (r >= n) continue;
        float sq = QS[m], sa = 0.f, sb = ES[m];
        for (int i = 0; i <= r; ++i) sq += M[3][r][i] * P.Km[i][ch];
        for (int i = r; i < 16; ++i) sa += M[0][r][i] * P.Qp[i][ch];
        for (int i = r + 1; i < 16; ++i) sa -= M[1][r][i] * P.Kp[i][ch];
        for (int i = 0; i < r; ++i) sb += M[2][r][i] * P.Km[i][ch];
        const float G = P.G[r][ch], ep = expf(G);
        const float dqv = ep * sq;
        const float av = expf(-G) * (sa + P.gam[ch] * DS[m]);
        const float bv = P.beta[r] * ep * sb;
        const int64_t e = ((t0 + r) * H + h) * DK + ch;
        dq[e] = dqv;
        dk[e] = av - bv;
        incr[e] = P.Q[r][ch] * dqv - P.K[r][ch] * (av + bv);
    }
}

// ------------------------------------------------------------------ 4. log-decay scan
template <int DV>
__global__ __launch_bounds__(BWD_THREADS) void bwd_dg_scan_kernel(const int32_t *__restrict__ cu, int32_t nseq,
                                                                   int32_t H, int32_t DK,
                                                                   const float *__restrict__ dfinal,
                                                                   const float *__restrict__ sfin,
                                                                   float *__restrict__ dg) {
    const int64_t i = (int64_t)blockIdx.x * BWD_THREADS + threadIdx.x;
    if (i >= (int64_t)nseq * H * DK) return;
    const int64_t s = i / ((int64_t)H * DK);
    const int64_t hc = i - s * H * DK;
    const int h = (int)(hc / DK), ch = (int)(hc - (int64_t)h * DK);
    float run = 0.f;
    if (dfinal) {
        const float *a = dfinal + i * DV, *b = sfin + i * DV;
        for (int j = 0; j < DV; ++j) run += a[j] * b[j];
    }
    // sixteen tokens per trip, their loads issued before the sums, so they overlap
    const int64_t bos = cu[s];
    int64_t t = cu[s + 1] - 1;
    const int64_t step = (int64_t)H * DK;
    for (; t - 15 >= bos; t -= 16) {
        float x[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) x[m] = dg[((t - m) * H + h) * DK + ch];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            run += x[m];
            dg[((t - m) * H + h) * DK + ch] = run;
        }
    }
    for (; t >= bos; --t) {
        const int64_t e = t * step + (int64_t)h * DK + ch;
        run += dg[e];
        dg[e] = run;
    }
}

// ------------------------------------------------------------------ launch

template <int DK, int DV, typename T>
static hipError_t launch_bwd_t(const BackwardArgs &a) {
    const int64_t slots = chunk_slots(a.N, a.nseq);
    const int64_t blk = slots * a.H * (int64_t)DK * DV;  // floats of one per-chunk state array
    float *sck = a.ws, *hck = sck + blk;
    float *dbuf = hck + blk, *ebuf = dbuf + slots * a.H * 16 * (int64_t)DV;
    float *sfin = ebuf + slots * a.H * 16 * (int64_t)DV;
    const hipStream_t st = (hipStream_t)a.stream;
    const unsigned chains = (unsigned)((int64_t)a.nseq * a.H * (DV / 16));
    hipLaunchKernelGGL((bwd_fwd_ckpt_kernel<DK, DV, T>), dim3(chains), dim3(BWD_THREADS), 0, st,
                       (const T *)a.q, (const T *)a.k, (const T *)a.v, (const T *)a.g, (const T *)a.beta,
                       a.init, a.cu, a.H, sck, dbuf, sfin);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_adjoint_kernel<DK, DV, T>), dim3(chains), dim3(BWD_THREADS), 0, st,
                       (const T *)a.q, (const T *)a.k, (const T *)a.g, (const T *)a.beta, a.dO, a.dfinal, a.cu,
                       a.H, hck, ebuf, a.dv, a.dinit);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.N > 0) {
        hipLaunchKernelGGL((bwd_grads_kernel<DK, DV, T>), dim3((unsigned)(slots * a.H)), dim3(BWD_THREADS), 0, st,
                           (const T *)a.q, (const T *)a.k, (const T *)a.v, (const T *)a.g, (const T *)a.beta, a.dO,
                           a.cu, a.nseq, a.H, sck, hck, dbuf, ebuf, a.dq, a.dk, a.dg, a.dbeta);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int64_t items = (int64_t)a.nseq * a.H * DK;
        hipLaunchKernelGGL((bwd_dg_scan_kernel<DV>), dim3((unsigned)((items + BWD_THREADS - 1) / BWD_THREADS)),
                           dim3(BWD_THREADS), 0, st, a.cu, a.nseq, a.H, DK, a.dfinal, sfin, a.dg);
        e = hipGetLastError();
    }
    return e;
}

template <typename T>
static hipError_t launch_bwd_dt(const BackwardArgs &a) {
#define KDA_BWD_CASE(DKV, DVV) \
    if (a.dk_ == DKV && a.dv_ == DVV) return launch_bwd_t<DKV, DVV, T>(a);
#define KDA_BWD_ROW(DKV) KDA_BWD_CASE(DKV, 16) KDA_BWD_CASE(DKV, 32) KDA_BWD_CASE(DKV, 64) KDA_BWD_CASE(DKV, 128)
    KDA_BWD_ROW(16) KDA_BWD_ROW(32) KDA_BWD_ROW(64) KDA_BWD_ROW(128)
#undef KDA_BWD_ROW
#undef KDA_BWD_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_backward(const BackwardArgs &a) {
    return a.bf16 ? launch_bwd_dt<__bf16>(a) : launch_bwd_dt<float>(a);
}

int64_t backward_workspace_floats(int64_t N, int32_t nseq, int32_t H, int32_t dk, int32_t dv) {
    const int64_t slots = chunk_slots(N, nseq);
    return 2 * slots * H * (int64_t)dk * dv + 2 * slots * H * 16 * (int64_t)dv + (int64_t)nseq * H * dk * dv;
}

}  // namespace kda
