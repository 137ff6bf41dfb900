// Intra-device context parallelism for the KDA prefill (gfx950): one sequence split
// into R chunk-aligned segments that run as independent chains, their exact incoming
// states recovered by a scan.  The algebra is the one the Kimi K3 report digest gives
// for splitting a sequence across devices ("KDA 컨텍스트 병렬화": each segment's state
// map is affine, S_out = M S_in + S~, with M the product of the per-token transitions
// (I - beta k k^T) Diag(alpha)), used here between the compute units of one device
// ("KDA 알고리즘과 시스템의 공동 설계", intra-device CP).
//
// The passes (kda_prefill_cp in api.cpp) reuse the prefill kernels on the segmented
// sequence list:
//   1. cp_segments: segment r of sequence s covers its chunks [nc r / R, nc (r+1) / R);
//   2. chunk_local over the segments (a chunk's T' and A_qk depend only on its tokens, so
//      one pass serves all three recurrences below);
//   3. inter_chunk from zero states: each segment's S~ (outputs not written);
//   4. inter_chunk with v = 0 from the identity (a dk x dk "state"): each segment's M,
//      except for segments whose transition is provably negligible (cp_bound below);
//   5. cp_scan per (sequence, head): S_in,0 = the initial state, S_in,r+1 = M_r S_in,r + S~_r
//      (S~_r alone where M_r was skipped);
//   6. inter_chunk from the exact S_in,r: the outputs, and each segment's final state in
//      place of its S_in (the last one is the sequence's, copied out by cp_final).
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int CP_THREADS = 256;

__global__ __launch_bounds__(CP_THREADS) void cp_segments_kernel(const int32_t *__restrict__ cu, int32_t nseq,
                                                                 int32_t R, int32_t *__restrict__ cu_seg) {
    const int s = blockIdx.x * CP_THREADS + threadIdx.x;
    if (s > nseq) return;
    if (s == nseq) {
        cu_seg[(int64_t)nseq * R] = cu[nseq];
        return;
    }
    const int32_t bos = cu[s], eos = cu[s + 1];
    const int64_t nc = (eos - bos + 15) / 16;
    for (int r = 0; r < R; ++r) {
        const int64_t c0 = nc * r / R;
        const int64_t t = bos + 16 * c0;
        cu_seg[(int64_t)s * R + r] = (int32_t)(t < eos ? t : eos);
    }
}

// A bound on each segment's transition M = prod_t (I - beta_t k_t k_t^T) Diag(alpha_t):
// ||Diag(alpha)||_2 = max_i alpha_i and ||I - beta k k^T||_2 = max(1, |1 - beta ||k||^2|), so
//     log ||M||_2 <= sum_t ( max_i g_t,i + log max(1, |1 - beta_t ||k_t||^2|) )
// (g = log alpha <= 0).  Where it is below log 2^-30 the term M_r S_in,r changes S_in,r+1 by
// less than 2^-30 of S_in,r -- far below fp32 resolution of the state -- so the segment's M
// is not computed and the scan takes S_in,r+1 = S~_r.  At the rates of the pages' workloads
// (channels' largest log-decay around -0.07 per token) this holds for every segment longer
// than a few hundred tokens.  One workgroup per (segment, head), one token row per thread.
constexpr float CP_LOG_NEGLIGIBLE = -20.794415f;  // log 2^-30

template <typename T, int DK>
__global__ __launch_bounds__(CP_THREADS) void cp_bound_kernel(const T *__restrict__ k, const T *__restrict__ g,
                                                              const T *__restrict__ beta,
                                                              const int32_t *__restrict__ cu_seg, int32_t H,
                                                              int32_t *__restrict__ flags) {
    const int64_t sh = blockIdx.x;
    const int64_t seg = sh / H;
    const int h = (int)(sh - seg * H);
    const int64_t t0 = cu_seg[seg], t1 = cu_seg[seg + 1];
    float lsum = 0.f;
    for (int64_t t = t0 + threadIdx.x; t < t1; t += CP_THREADS) {
        const T *gr = g + (t * H + h) * DK, *kr = k + (t * H + h) * DK;
        float gm = -3.4e38f, kk = 0.f;
#pragma unroll 4
        for (int c = 0; c < DK; c += 4) {
            const f32x4 gv = load_in4(gr + c), kv = load_in4(kr + c);
            gm = fmaxf(gm, fmaxf(fmaxf(gv[0], gv[1]), fmaxf(gv[2], gv[3])));
            kk += (kv[0] * kv[0] + kv[1] * kv[1]) + (kv[2] * kv[2] + kv[3] * kv[3]);
        }
        const float e = fabsf(1.f - load_in(beta + t * H + h) * kk);
        lsum += gm + (e > 1.f ? logf(e) : 0.f);
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) lsum += __shfl_xor(lsum, m);
    __shared__ float part[CP_THREADS / 64];
    if (threadIdx.x % 64 == 0) part[threadIdx.x / 64] = lsum;
    __syncthreads();
    if (threadIdx.x == 0) {
        float tot = 0.f;
#pragma unroll
        for (int w = 0; w < CP_THREADS / 64; ++w) tot += part[w];
        flags[sh] = (tot < CP_LOG_NEGLIGIBLE) ? 1 : 0;  // (false for NaN input)
    }
}

__global__ __launch_bounds__(CP_THREADS) void cp_identity_kernel(float *__restrict__ M, int64_t total, int32_t dk) {
    const int64_t i = (int64_t)blockIdx.x * CP_THREADS + threadIdx.x;
    if (i >= total) return;
    const int64_t e = i % ((int64_t)dk * dk);
    M[i] = (e / dk == e % dk) ? 1.f : 0.f;
}

// The columns of the state evolve independently under S_in,r+1 = M_r S_in,r + S~_r (M_r acts
// from the left), so one workgroup serves one (sequence, head, 16-column slice): DK/16 waves,
// wave I owning the 16x16 tile of rows 16I.. of the slice, on the fp32 matrix cores.  The
// slice of the current state stays in LDS (two buffers, one barrier per segment); each wave
// holds its row block of M_r and its tile of S~_r in registers and loads those of the next
// segment before the product, so a step waits on memory only when the product is shorter
// than a load.  Every S_in,r is also written out for the last recurrence pass.
template <int DK, int DV>
__global__ __launch_bounds__(64 * (DK / 16)) void cp_scan_kernel(const float *__restrict__ init,
                                                                const float *__restrict__ M,
                                                                const float *__restrict__ St,
                                                                const int32_t *__restrict__ skip,
                                                                float *__restrict__ Sin, int32_t H, int32_t R) {
    constexpr int NKB = DK / 16, NJ = DV / 16, LD = 20;
    __shared__ __attribute__((aligned(16))) float S[2][DK * LD];
    const int J = blockIdx.x % NJ, sh = blockIdx.x / NJ;
    const int s = sh / H, h = sh % H;
    const int lane = threadIdx.x % 64, I = threadIdx.x / 64, gq = lane / 16, m = lane % 16;
    const int col = 16 * J + m;
    auto seg = [&](int r) { return ((int64_t)s * R + r) * H + h; };
    // this lane's operands of segment r: A = rows 16I + m of M_r, columns 16kb + 4gq ..;
    // the S~_r values at rows 16I + 4gq + j, column col
    auto load_ops = [&](int r, f32x4 (&a)[NKB], f32x4 &t) {
        const float *Mr = M + seg(r) * DK * DK + (16 * I + m) * DK + 4 * gq;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) a[kb] = *reinterpret_cast<const f32x4 *>(Mr + 16 * kb);
        const float *Tr = St + seg(r) * DK * DV + (16 * I + 4 * gq) * DV + col;
#pragma unroll
        for (int j = 0; j < 4; ++j) t[j] = Tr[j * DV];
    };
    {
        const float *I0 = init ? init + ((int64_t)s * H + h) * DK * DV : nullptr;
        float *S0 = Sin + seg(0) * DK * DV;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * I + 4 * gq + j;
            const float x = I0 ? I0[row * DV + col] : 0.f;
            S0[row * DV + col] = x;
            S[0][row * LD + m] = x;
        }
    }
    f32x4 a[NKB], t;
    if (R > 1) load_ops(0, a, t);
    __syncthreads();
    for (int r = 0; r + 1 < R; ++r) {
        // segment r + 1 <= R - 1 exists (M and S~ are kept for every segment)
        f32x4 an[NKB], tn;
        load_ops(r + 1, an, tn);
        const float *Sr = S[r & 1];
        float *Sl = S[(r + 1) & 1];
        f32x4 c = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f32x4 b;
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Sr[(16 * kb + 4 * gq + j) * LD + m];
            c = mma_f32_k16(a[kb], b, c);
        }
        float *Sn = Sin + seg(r + 1) * DK * DV;
        const bool negligible = skip && skip[seg(r)];  // M_r not computed (it holds the identity)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * I + 4 * gq + j;
            const float x = negligible ? t[j] : c[j] + t[j];
            Sn[row * DV + col] = x;
            Sl[row * LD + m] = x;
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) a[kb] = an[kb];
        t = tn;
        __syncthreads();
    }
}

__global__ __launch_bounds__(CP_THREADS) void cp_final_kernel(const float *__restrict__ Sin, float *__restrict__ fin,
                                                              int32_t nseq, int32_t H, int32_t R, int64_t per_head) {
    const int64_t i = (int64_t)blockIdx.x * CP_THREADS + threadIdx.x;
    if (i >= (int64_t)nseq * H * per_head) return;
    const int64_t sh = i / per_head, e = i - sh * per_head;
    const int64_t s = sh / H, h = sh - s * H;
    fin[i] = Sin[((s * R + R - 1) * H + h) * per_head + e];
}

static unsigned blocks_for(int64_t n) { return (unsigned)((n + CP_THREADS - 1) / CP_THREADS); }

hipError_t launch_cp_segments(const int32_t *cu, int32_t nseq, int32_t R, int32_t *cu_seg, void *stream) {
    hipLaunchKernelGGL(cp_segments_kernel, dim3(blocks_for((int64_t)nseq + 1)), dim3(CP_THREADS), 0,
                       (hipStream_t)stream, cu, nseq, R, cu_seg);
    return hipGetLastError();
}

hipError_t launch_cp_identity(float *M, int64_t n_mats, int32_t dk, void *stream) {
    const int64_t total = n_mats * dk * dk;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(cp_identity_kernel, dim3(blocks_for(total)), dim3(CP_THREADS), 0, (hipStream_t)stream, M,
                       total, dk);
    return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_scan_t(const float *init, const float *M, const float *St, const int32_t *skip, float *Sin,
                                int32_t nseq, int32_t H, int32_t R, void *stream) {
    const int64_t grid = (int64_t)nseq * H * (DV / 16);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((cp_scan_kernel<DK, DV>), dim3((unsigned)grid), dim3(64 * (DK / 16)), 0,
                       (hipStream_t)stream, init, M, St, skip, Sin, H, R);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_bound_t(const void *k, const void *g, const void *beta, const int32_t *cu_seg, int32_t nseg,
                                 int32_t H, int32_t dk, int32_t *flags, void *stream) {
    const unsigned grid = (unsigned)((int64_t)nseg * H);
    if (grid == 0) return hipSuccess;
    const hipStream_t st = (hipStream_t)stream;
    const T *kk = (const T *)k, *gg = (const T *)g, *bb = (const T *)beta;
    switch (dk) {
        case 16: hipLaunchKernelGGL((cp_bound_kernel<T, 16>), dim3(grid), dim3(CP_THREADS), 0, st, kk, gg, bb, cu_seg, H, flags); break;
        case 32: hipLaunchKernelGGL((cp_bound_kernel<T, 32>), dim3(grid), dim3(CP_THREADS), 0, st, kk, gg, bb, cu_seg, H, flags); break;
        case 64: hipLaunchKernelGGL((cp_bound_kernel<T, 64>), dim3(grid), dim3(CP_THREADS), 0, st, kk, gg, bb, cu_seg, H, flags); break;
        case 128: hipLaunchKernelGGL((cp_bound_kernel<T, 128>), dim3(grid), dim3(CP_THREADS), 0, st, kk, gg, bb, cu_seg, H, flags); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_cp_bound(const void *k, const void *g, const void *beta, const int32_t *cu_seg, int32_t nseg,
                           int32_t H, int32_t dk, bool bf16, int32_t *flags, void *stream) {
    return bf16 ? launch_bound_t<__bf16>(k, g, beta, cu_seg, nseg, H, dk, flags, stream)
                : launch_bound_t<float>(k, g, beta, cu_seg, nseg, H, dk, flags, stream);
}

hipError_t launch_cp_scan(const float *init, const float *M, const float *St, const int32_t *skip, float *Sin,
                          int32_t nseq, int32_t H, int32_t dk, int32_t dv, int32_t R, void *stream) {
#define KDA_CP_CASE(DKV, DVV) \
    if (dk == DKV && dv == DVV) return launch_scan_t<DKV, DVV>(init, M, St, skip, Sin, nseq, H, R, stream);
#define KDA_CP_ROW(DKV) KDA_CP_CASE(DKV, 16) KDA_CP_CASE(DKV, 32) KDA_CP_CASE(DKV, 64) KDA_CP_CASE(DKV, 128)
    KDA_CP_ROW(16) KDA_CP_ROW(32) KDA_CP_ROW(64) KDA_CP_ROW(128)
#undef KDA_CP_ROW
#undef KDA_CP_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_cp_final(const float *Sin, float *fin, int32_t nseq, int32_t H, int32_t dk, int32_t dv, int32_t R,
                           void *stream) {
    const int64_t per_head = (int64_t)dk * dv, total = (int64_t)nseq * H * per_head;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(cp_final_kernel, dim3(blocks_for(total)), dim3(CP_THREADS), 0, (hipStream_t)stream, Sin, fin,
                       nseq, H, R, per_head);
    return hipGetLastError();
}

}  // namespace kda
