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
// rate: 16-byte vector loads/stores, all of a thread's rows in flight at
// once, column reductions through LDS.  No matrix cores are used (about one
// flop per byte).
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int DK, int DV>
struct DecodeShape {
    static constexpr int NC4 = DV / 4;                                   // column quads per row
    static constexpr int RP = (DK < 256 / NC4) ? DK : 256 / NC4;         // rows per pass
    static constexpr int NT = NC4 * RP;                                  // threads per head
    static constexpr int NR = DK / RP;                                   // rows per thread
};

template <int DK, int DV, typename T>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NT)) void decode_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ g, const T *__restrict__ beta, float *__restrict__ state,
    float *__restrict__ o) {
    using Sh = DecodeShape<DK, DV>;
    constexpr int NC4 = Sh::NC4, RP = Sh::RP, NT = Sh::NT, NR = Sh::NR;
    const int64_t head = blockIdx.x;  // b * H + h
    const int tid = threadIdx.x;
    const int c4 = tid % NC4;
    const int rg = tid / NC4;

    __shared__ float s_k[DK], s_q[DK], s_a[DK];
    __shared__ f32x4 s_red[2][RP][NC4];
    __shared__ float s_kq[RP];

    float *S = state + head * (int64_t)(DK * DV);
    f32x4 rows[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r)
        rows[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (int64_t)(rg + r * RP) * DV) + c4);

    for (int i = tid; i < DK; i += NT) {
        s_k[i] = load_in(k + head * DK + i);
        s_q[i] = load_in(q + head * DK + i);
        s_a[i] = decay_exp(load_in(g + head * DK + i));
    }
    const f32x4 vv = load_in4(v + head * DV + 4 * c4);
    const float b = load_in(beta + head);
    __syncthreads();

    f32x4 pv = zero4(), pq = zero4();
    float pkq = 0.f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int row = rg + r * RP;
        rows[r] = rows[r] * s_a[row];             // forget
        pv += s_k[row] * rows[r];                  // partial S'^T k
        pq += s_q[row] * rows[r];                  // partial S'^T q
        pkq += s_k[row] * s_q[row];
    }
    s_red[0][rg][c4] = pv;
    s_red[1][rg][c4] = pq;
    if (c4 == 0) s_kq[rg] = pkq;
    __syncthreads();

    f32x4 vhat = zero4(), rq = zero4();
    float kq = 0.f;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
        vhat += s_red[0][i][c4];
        rq += s_red[1][i][c4];
        kq += s_kq[i];
    }
    const f32x4 delta = b * (vv - vhat);
    if (rg == 0) reinterpret_cast<f32x4 *>(o + head * DV)[c4] = rq + kq * delta;

#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int row = rg + r * RP;
        const f32x4 nr = rows[r] + s_k[row] * delta;  // erase + write
        __builtin_nontemporal_store(nr, reinterpret_cast<f32x4 *>(S + (int64_t)row * DV) + c4);
    }
}

template <int DK, int DV, typename T>
static hipError_t launch_decode_t(const DecodeArgs &a) {
    using Sh = DecodeShape<DK, DV>;
    const int64_t heads = (int64_t)a.B * a.H;
    hipLaunchKernelGGL((decode_kernel<DK, DV, T>), dim3((unsigned)heads), dim3(Sh::NT), 0,
                       (hipStream_t)a.stream, (const T *)a.q, (const T *)a.k, (const T *)a.v,
                       (const T *)a.g, (const T *)a.beta, a.state, a.o);
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

}  // namespace kda
