// C ABI of the KDA library: argument validation on the host, then launches on
// the caller's stream.  No allocation, no synchronisation, no printing.
#include <hip/hip_runtime.h>

#include "../../include/kda.h"
#include "kda_launch.hpp"

namespace {

thread_local int32_t g_last_hip_error = 0;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dim_ok(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

kda_status hip_status(hipError_t e) {
    if (e == hipSuccess) return KDA_OK;
    g_last_hip_error = static_cast<int32_t>(e);
    return KDA_ERR_HIP;
}

// Launch limits.  A dispatch holds at most 2^32 - 1 work-items per grid dimension, and
// the kernels keep per-chunk buffer extents and row strides in 32 bits.  The bounds
// below follow each prefill-family launch's real work-item count, so a shape that
// passes validation also launches:
//   * recurrence kernels (inter-chunk, backward sweeps, context-parallel scan): at most
//     4096 work-items per (sequence, head) chain -> chains < 2^20;
//   * per-(chunk slot, head) kernels (backward matrices and gradients: 256 work-items,
//     fp32 chunk-local: 64 per slot in x) -> slots * H < 2^24, fp32 slots < 2^26;
//   * 16-token row extents 16 * H * d * 4 bytes in 32 bits -> H * d < 2^24.
constexpr int64_t MAX_CHAINS = int64_t(1) << 20;
constexpr int64_t MAX_SLOT_HEADS = int64_t(1) << 24;

kda_status check_common(int32_t nseq, int64_t total_tokens, int32_t H, int32_t dk, int32_t dv,
                        kda_dtype dt) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
    if (nseq < 1 || H < 1 || total_tokens < 0 || total_tokens >= (int64_t(1) << 31))
        return KDA_ERR_SHAPE;
    if ((int64_t)nseq * H >= MAX_CHAINS) return KDA_ERR_SHAPE;
    if ((int64_t)H * (dk > dv ? dk : dv) >= (int64_t(1) << 24)) return KDA_ERR_SHAPE;
    const int64_t slots = kda::chunk_slots(total_tokens, nseq);
    if (dt == KDA_F32 && slots >= (int64_t(1) << 26)) return KDA_ERR_SHAPE;
    return KDA_OK;
}

// Workspace of kda_prefill_cp: the segments' chunk-local operands, the segment list, and
// per segment and head S~, M and S_in, each region 256-byte aligned.  0 = invalid.
constexpr int32_t CP_MAX_SEGMENTS = 64;
struct CpLayout {
    size_t cl, cu, st, m, sin, flags, total;
};
CpLayout cp_layout(int64_t total_tokens, int32_t nseq, int32_t H, int32_t dk, int32_t dv, int32_t R) {
    auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
    const size_t segs = (size_t)nseq * (size_t)R;
    CpLayout L;
    L.cl = 0;
    L.cu = L.cl + up((size_t)kda::chunk_slots(total_tokens, (int32_t)segs) * H * kda::WS_FLOATS_PER_CHUNK_HEAD * 4);
    L.st = L.cu + up((segs + 1) * 4);
    L.m = L.st + up(segs * H * (size_t)dk * dv * 4);
    L.sin = L.m + up(segs * H * (size_t)dk * dk * 4);
    L.flags = L.sin + up(segs * H * (size_t)dk * dv * 4);
    L.total = L.flags + up(segs * H * 4);
    return L;
}

// kda_prefill's choice of intra-device context parallelism: bf16 with dk >= 32 (the
// warp-specialised kernels), at most 64 (sequence, head) chains -- so the plain pass holds at
// most a quarter of the chip's workgroup slots -- and sequences of 16,384 tokens or more on
// average (the host does not read cu_seqlens), so each of CP's passes is long against its
// fixed cost.  R = 128 / chains segments (2..16): about 240 workgroups in all.  0 = no CP.
bool cp_lengths_ok(int64_t total_tokens, int32_t nseq, int32_t H, int32_t dk, int32_t dv, int32_t R) {
    if (R < 1 || R > CP_MAX_SEGMENTS) return false;
    const int64_t segs = (int64_t)nseq * R;
    if (segs >= (int64_t(1) << 31)) return false;
    if (check_common((int32_t)segs, total_tokens, H, dk, dv, KDA_BF16) != KDA_OK) return false;
    return segs * H * dk * (dk > dv ? dk : dv) < (int64_t(1) << 31);
}
int32_t auto_cp_segments(int64_t total_tokens, int32_t nseq, int32_t H, int32_t dk, int32_t dv, kda_dtype dt) {
    if (dt != KDA_BF16 || dk < 32 || nseq < 1 || H < 1) return 0;
    const int64_t chains = (int64_t)nseq * H;
    if (chains > 64 || total_tokens / nseq < 16384) return 0;
    int64_t R = 128 / chains;
    R = R < 2 ? 2 : (R > 16 ? 16 : R);
    return cp_lengths_ok(total_tokens, nseq, H, dk, dv, (int32_t)R) ? (int32_t)R : 0;
}

size_t workspace_bytes(int64_t total_tokens, int32_t nseq, int32_t H) {
    return static_cast<size_t>(kda::chunk_slots(total_tokens, nseq)) * static_cast<size_t>(H) *
           kda::WS_FLOATS_PER_CHUNK_HEAD * sizeof(float);
}

// Fused layer prefill: the chunk workspace, then the prologue's q, k and log-decay
// (bf16 [3, N, H, 128]).
size_t layer_qkg_offset(int64_t total_tokens, int32_t nseq, int32_t H) {
    return (workspace_bytes(total_tokens, nseq, H) + 255) / 256 * 256;
}
size_t layer_workspace_bytes(int64_t total_tokens, int32_t nseq, int32_t H) {
    return layer_qkg_offset(total_tokens, nseq, H) + (size_t)total_tokens * H * 3 * 128 * 2;
}

kda_status check_ptrs(std::initializer_list<const void *> required,
                      std::initializer_list<const void *> optional) {
    for (const void *p : required)
        if (!p) return KDA_ERR_NULL;
    for (const void *p : required)
        if (!aligned16(p)) return KDA_ERR_ALIGN;
    for (const void *p : optional)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;
    return KDA_OK;
}

// Token-indexed inputs: q, k, v, log_alpha are read four elements at a time (8 bytes
// for bf16, 16 for fp32); beta (when the entry point takes it) is read element by
// element.  With no tokens they may be NULL.
kda_status check_inputs(std::initializer_list<const void *> vec4, bool takes_beta, const void *beta,
                        bool bf16, bool any_tokens) {
    const uintptr_t elem = bf16 ? 2u : 4u;
    for (const void *p : vec4) {
        if (!p) {
            if (any_tokens) return KDA_ERR_NULL;
            continue;
        }
        if (reinterpret_cast<uintptr_t>(p) & (4 * elem - 1)) return KDA_ERR_ALIGN;
    }
    if (!takes_beta) return KDA_OK;
    if (beta) {
        if (reinterpret_cast<uintptr_t>(beta) & (elem - 1)) return KDA_ERR_ALIGN;
    } else if (any_tokens) {
        return KDA_ERR_NULL;
    }
    return KDA_OK;
}

// The layer passes read and write [.., d] rows eight elements at a time: 16-byte
// aligned; with no rows they may be NULL.
kda_status check_rows16(std::initializer_list<const void *> ptrs, bool any_rows) {
    for (const void *p : ptrs) {
        if (!p) {
            if (any_rows) return KDA_ERR_NULL;
            continue;
        }
        if (!aligned16(p)) return KDA_ERR_ALIGN;
    }
    return KDA_OK;
}

// Checks of the fused-work arguments shared by the decode entry points.
kda_status check_fusion(const float *A_log, const void *u, const float *w, float eps, const void *y, bool bf16) {
    if (A_log && (reinterpret_cast<uintptr_t>(A_log) & 3u)) return KDA_ERR_ALIGN;
    if (!u) return KDA_OK;
    if (!w || !y) return KDA_ERR_NULL;
    if (!aligned16(w)) return KDA_ERR_ALIGN;
    const uintptr_t vec = bf16 ? 7u : 15u;
    if ((reinterpret_cast<uintptr_t>(u) & vec) || (reinterpret_cast<uintptr_t>(y) & vec)) return KDA_ERR_ALIGN;
    if (!(eps >= 0.f && eps <= 3.4e38f)) return KDA_ERR_SHAPE;
    return KDA_OK;
}

// The backward's per-(chunk slot, head) kernels: up to 256 work-items each.
kda_status check_backward_shape(int32_t nseq, int64_t total_tokens, int32_t H, int32_t dk, int32_t dv,
                                kda_dtype dt) {
    kda_status st = check_common(nseq, total_tokens, H, dk, dv, dt);
    if (st != KDA_OK) return st;
    if (kda::chunk_slots(total_tokens, nseq) * H >= MAX_SLOT_HEADS) return KDA_ERR_SHAPE;
    return KDA_OK;
}

}  // namespace

namespace kda {
kda_status record_hip_error(hipError_t e) { return hip_status(e); }
}  // namespace kda

extern "C" {

size_t kda_chunk_workspace_bytes(int64_t total_tokens, int32_t nseq, int32_t H, int32_t dk,
                                 int32_t dv, kda_dtype dt) {
    if (check_common(nseq, total_tokens, H, dk, dv, dt) != KDA_OK) return 0;
    return workspace_bytes(total_tokens, nseq, H);
}

size_t kda_prefill_workspace_bytes(int64_t total_tokens, int32_t nseq, int32_t H, int32_t dk,
                                   int32_t dv, kda_dtype dt) {
    if (check_common(nseq, total_tokens, H, dk, dv, dt) != KDA_OK) return 0;
    if (kda::prefill_fused_supported(dk, dv, dt == KDA_BF16, (int64_t)nseq * H)) return 0;  // single pass
    const int32_t R = auto_cp_segments(total_tokens, nseq, H, dk, dv, dt);
    if (R > 0) return cp_layout(total_tokens, nseq, H, dk, dv, R).total;  // context parallelism
    return workspace_bytes(total_tokens, nseq, H);
}

kda_status kda_chunk_local(const void *q, const void *k, const void *log_alpha, const void *beta,
                           const int32_t *cu_seqlens, int32_t nseq, int64_t total_tokens, int32_t H,
                           int32_t dk, kda_dtype dt, void *workspace, size_t ws_bytes, void *stream) {
    kda_status st = check_common(nseq, total_tokens, H, dk, 16, dt);
    if (st != KDA_OK) return st;
    st = check_inputs({q, k, log_alpha}, true, beta, dt == KDA_BF16, total_tokens > 0);
    if (st != KDA_OK) return st;
    st = check_ptrs({cu_seqlens}, {});
    if (st != KDA_OK) return st;
    if (!workspace || ws_bytes < workspace_bytes(total_tokens, nseq, H)) return KDA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KDA_ERR_ALIGN;
    kda::ChunkLocalArgs a{q, k, log_alpha, beta, cu_seqlens, nseq, H, dk, total_tokens,
                          dt == KDA_BF16, static_cast<float *>(workspace), stream};
    return hip_status(kda::launch_chunk_local(a));
}

kda_status kda_inter_chunk(const void *q, const void *k, const void *v, const void *log_alpha,
                           const float *init_state, const int32_t *cu_seqlens, int32_t nseq,
                           int64_t total_tokens, int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                           const void *workspace, size_t ws_bytes, float *o, float *final_state,
                           void *stream) {
    kda_status st = check_common(nseq, total_tokens, H, dk, dv, dt);
    if (st != KDA_OK) return st;
    st = check_inputs({q, k, v, log_alpha}, false, nullptr, dt == KDA_BF16, total_tokens > 0);
    if (st != KDA_OK) return st;
    st = check_ptrs({cu_seqlens}, {init_state, final_state, o});
    if (st != KDA_OK) return st;
    if (!o && total_tokens > 0) return KDA_ERR_NULL;
    if (!workspace || ws_bytes < workspace_bytes(total_tokens, nseq, H)) return KDA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KDA_ERR_ALIGN;
    kda::InterChunkArgs a{q, k, v, log_alpha, init_state, cu_seqlens, nseq, H, dk, dv,
                          total_tokens, dt == KDA_BF16, static_cast<const float *>(workspace), o,
                          final_state, 0, 0, stream};
    return hip_status(kda::launch_inter_chunk(a));
}

kda_status kda_inter_chunk_shaped(const void *q, const void *k, const void *v, const void *log_alpha,
                                  const float *init_state, const int32_t *cu_seqlens, int32_t nseq,
                                  int64_t total_tokens, int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                                  const void *workspace, size_t ws_bytes, int32_t consumers, int32_t producers,
                                  float *o, float *final_state, void *stream) {
    if (consumers == 0 && producers == 0)
        return kda_inter_chunk(q, k, v, log_alpha, init_state, cu_seqlens, nseq, total_tokens, H, dk, dv, dt,
                               workspace, ws_bytes, o, final_state, stream);
    kda_status st = check_common(nseq, total_tokens, H, dk, dv, dt);
    if (st != KDA_OK) return st;
    if (dt != KDA_BF16 || dk < 32 || !kda::inter_chunk_ws_shape_built(dk, dv, consumers, producers))
        return KDA_ERR_UNSUPPORTED;
    st = check_inputs({q, k, v, log_alpha}, false, nullptr, true, total_tokens > 0);
    if (st != KDA_OK) return st;
    st = check_ptrs({cu_seqlens}, {init_state, final_state, o});
    if (st != KDA_OK) return st;
    if (!o && total_tokens > 0) return KDA_ERR_NULL;
    if (!workspace || ws_bytes < workspace_bytes(total_tokens, nseq, H)) return KDA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KDA_ERR_ALIGN;
    kda::InterChunkArgs a{q, k, v, log_alpha, init_state, cu_seqlens, nseq, H, dk, dv,
                          total_tokens, true, static_cast<const float *>(workspace), o,
                          final_state, consumers, producers, stream};
    return hip_status(kda::launch_inter_chunk(a));
}

kda_status kda_prefill(const void *q, const void *k, const void *v, const void *log_alpha,
                       const void *beta, const float *init_state, const int32_t *cu_seqlens,
                       int32_t nseq, int64_t total_tokens, int32_t H, int32_t dk, int32_t dv,
                       kda_dtype dt, float *o, float *final_state, void *workspace, size_t ws_bytes,
                       void *stream) {
    kda_status st = check_common(nseq, total_tokens, H, dk, dv, dt);
    if (st != KDA_OK) return st;
    st = check_inputs({q, k, v, log_alpha}, true, beta, dt == KDA_BF16, total_tokens > 0);
    if (st != KDA_OK) return st;
    st = check_ptrs({cu_seqlens}, {init_state, final_state, o});
    if (st != KDA_OK) return st;
    if (!o && total_tokens > 0) return KDA_ERR_NULL;
    if (kda::prefill_fused_supported(dk, dv, dt == KDA_BF16, (int64_t)nseq * H)) {
        // one kernel: the chunk-local operands stay on chip, the workspace is not used
        kda::PrefillFusedArgs a{q, k, v, log_alpha, beta, init_state, cu_seqlens, nseq, H, dk, dv,
                                true, o, final_state, stream};
        return hip_status(kda::launch_prefill_fused(a, 0, 0));
    }
    // few long chains: intra-device context parallelism
    const int32_t R = auto_cp_segments(total_tokens, nseq, H, dk, dv, dt);
    if (R > 0)
        return kda_prefill_cp(q, k, v, log_alpha, beta, init_state, cu_seqlens, nseq, total_tokens, H, dk, dv, dt, R,
                              o, final_state, workspace, ws_bytes, stream);
    if (!workspace || ws_bytes < workspace_bytes(total_tokens, nseq, H)) return KDA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KDA_ERR_ALIGN;
    st = kda_chunk_local(q, k, log_alpha, beta, cu_seqlens, nseq, total_tokens, H, dk, dt,
                         workspace, ws_bytes, stream);
    if (st != KDA_OK) return st;
    return kda_inter_chunk(q, k, v, log_alpha, init_state, cu_seqlens, nseq, total_tokens, H, dk,
                           dv, dt, workspace, ws_bytes, o, final_state, stream);
}

size_t kda_prefill_layer_workspace_bytes(int64_t total_tokens, int32_t nseq, int32_t H, int32_t dk, int32_t dv,
                                         kda_dtype dt) {
    if (check_common(nseq, total_tokens, H, dk, dv, dt) != KDA_OK) return 0;
    if (dt != KDA_BF16 || dk != 128 || dv != 128) return 0;
    return layer_workspace_bytes(total_tokens, nseq, H);
}

kda_status kda_prefill_layer(const void *q, const void *k, const void *v, const float *conv_w,
                             const float *conv_cache_in, float *conv_cache_out, float l2_eps, const void *z,
                             const float *A_log, const void *beta, const float *init_state,
                             const int32_t *cu_seqlens, int32_t nseq, int64_t total_tokens, int32_t H, int32_t dk,
                             int32_t dv, kda_dtype dt, void *workspace, size_t ws_bytes, float *o,
                             float *final_state, const void *out_gate, const float *norm_w, float norm_eps,
                             void *y, void *stream) {
    kda_status st = check_common(nseq, total_tokens, H, dk, dv, dt);
    if (st != KDA_OK) return st;
    if (dt != KDA_BF16 || dk != 128 || dv != 128) return KDA_ERR_UNSUPPORTED;
    if (!(l2_eps >= 0.f && l2_eps <= 3.4e38f)) return KDA_ERR_SHAPE;
    st = check_inputs({q, k, v, z}, true, beta, true, total_tokens > 0);
    if (st != KDA_OK) return st;
    st = check_ptrs({cu_seqlens, conv_w}, {init_state, final_state, o});
    if (st != KDA_OK) return st;
    if (!A_log) return KDA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(A_log) & 3u) || (conv_cache_in && (reinterpret_cast<uintptr_t>(conv_cache_in) & 3u)) ||
        (conv_cache_out && (reinterpret_cast<uintptr_t>(conv_cache_out) & 3u)))
        return KDA_ERR_ALIGN;
    if (!o && total_tokens > 0) return KDA_ERR_NULL;
    if (out_gate) {
        st = check_rows16({out_gate, y}, total_tokens > 0);
        if (st != KDA_OK) return st;
        st = check_ptrs({norm_w}, {});
        if (st != KDA_OK) return st;
        if (!(norm_eps >= 0.f && norm_eps <= 3.4e38f)) return KDA_ERR_SHAPE;
    }
    if (!workspace || ws_bytes < layer_workspace_bytes(total_tokens, nseq, H)) return KDA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KDA_ERR_ALIGN;
    float *ws = static_cast<float *>(workspace);
    uint16_t *qkg = reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) +
                                                 layer_qkg_offset(total_tokens, nseq, H));
    const size_t plane = (size_t)total_tokens * H * dk;
    const kda::LayerPrologue lp{conv_w, conv_cache_in, A_log, qkg, l2_eps, 2 * dk + dv, total_tokens};
    if (total_tokens > 0) {
        kda::ChunkLocalArgs cl{q, k, z, beta, cu_seqlens, nseq, H, dk, total_tokens, true, ws, stream, &lp};
        st = hip_status(kda::launch_chunk_local(cl));
        if (st != KDA_OK) return st;
    }
    // the recurrence on the prologue's q, k, log-decay; v raw (its prologue is applied on load)
    kda::InterChunkArgs ic{qkg, qkg + plane, v, qkg + 2 * plane, init_state, cu_seqlens, nseq, H, dk, dv,
                           total_tokens, true, ws, o, final_state, 0, 0, stream, &lp};
    st = hip_status(kda::launch_inter_chunk(ic));
    if (st != KDA_OK) return st;
    if (conv_cache_out) {
        st = hip_status(kda::launch_layer_conv_cache(q, k, v, conv_cache_in, conv_cache_out, cu_seqlens, nseq, H,
                                                     dk, dv, stream));
        if (st != KDA_OK) return st;
    }
    if (out_gate && total_tokens > 0) {
        kda::OutNormGateArgs a{o, out_gate, norm_w, norm_eps, total_tokens, H, dv, true, y, stream};
        st = hip_status(kda::launch_out_norm_gate(a));
    }
    return st;
}

kda_status kda_prefill_single_pass(const void *q, const void *k, const void *v, const void *log_alpha,
                                   const void *beta, const float *init_state, const int32_t *cu_seqlens,
                                   int32_t nseq, int64_t total_tokens, int32_t H, int32_t dk, int32_t dv,
                                   kda_dtype dt, int32_t consumers, int32_t slices, float *o, float *final_state,
                                   void *stream) {
    kda_status st = check_common(nseq, total_tokens, H, dk, dv, dt);
    if (st != KDA_OK) return st;
    if (dt != KDA_BF16 || dk != 128 || dv != 128 || !kda::prefill_fused_shape_built(consumers, slices))
        return KDA_ERR_UNSUPPORTED;
    st = check_inputs({q, k, v, log_alpha}, true, beta, true, total_tokens > 0);
    if (st != KDA_OK) return st;
    st = check_ptrs({cu_seqlens}, {init_state, final_state, o});
    if (st != KDA_OK) return st;
    if (!o && total_tokens > 0) return KDA_ERR_NULL;
    kda::PrefillFusedArgs a{q, k, v, log_alpha, beta, init_state, cu_seqlens, nseq, H, dk, dv,
                            true, o, final_state, stream};
    return hip_status(kda::launch_prefill_fused(a, consumers, slices));
}

size_t kda_prefill_cp_workspace_bytes(int64_t total_tokens, int32_t nseq, int32_t H, int32_t dk, int32_t dv,
                                      kda_dtype dt, int32_t segments) {
    if (segments < 1 || segments > CP_MAX_SEGMENTS) return 0;
    if (check_common(nseq, total_tokens, H, dk, dv, dt) != KDA_OK) return 0;
    const int64_t segs = (int64_t)nseq * segments;
    if (check_common((int32_t)segs, total_tokens, H, dk, dv, dt) != KDA_OK) return 0;
    if (segs * H * dk * (dk > dv ? dk : dv) >= (int64_t(1) << 31)) return 0;
    return cp_layout(total_tokens, nseq, H, dk, dv, segments).total;
}

kda_status kda_prefill_cp(const void *q, const void *k, const void *v, const void *log_alpha, const void *beta,
                          const float *init_state, const int32_t *cu_seqlens, int32_t nseq, int64_t total_tokens,
                          int32_t H, int32_t dk, int32_t dv, kda_dtype dt, int32_t segments, float *o,
                          float *final_state, void *workspace, size_t ws_bytes, void *stream) {
    kda_status st = check_common(nseq, total_tokens, H, dk, dv, dt);
    if (st != KDA_OK) return st;
    if (segments < 1 || segments > CP_MAX_SEGMENTS) return KDA_ERR_SHAPE;
    const int64_t segs = (int64_t)nseq * segments;
    if (segs >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;
    st = check_common((int32_t)segs, total_tokens, H, dk, dv, dt);
    if (st != KDA_OK) return st;
    // the identity and final-copy kernels run one work-item per element of the pieces'
    // dk x dk (or dk x dv) matrices in a 1-D grid
    if (segs * H * dk * (dk > dv ? dk : dv) >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;
    st = check_inputs({q, k, v, log_alpha}, true, beta, dt == KDA_BF16, total_tokens > 0);
    if (st != KDA_OK) return st;
    st = check_ptrs({cu_seqlens}, {init_state, final_state, o});
    if (st != KDA_OK) return st;
    if (!o && total_tokens > 0) return KDA_ERR_NULL;
    const CpLayout L = cp_layout(total_tokens, nseq, H, dk, dv, segments);
    if (!workspace || ws_bytes < L.total) return KDA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KDA_ERR_ALIGN;
    char *w = static_cast<char *>(workspace);
    float *cl = reinterpret_cast<float *>(w + L.cl), *St = reinterpret_cast<float *>(w + L.st);
    float *M = reinterpret_cast<float *>(w + L.m), *Sin = reinterpret_cast<float *>(w + L.sin);
    int32_t *cu_seg = reinterpret_cast<int32_t *>(w + L.cu);
    int32_t *negligible = reinterpret_cast<int32_t *>(w + L.flags);
    const bool bf16 = dt == KDA_BF16;
    const int32_t ns = (int32_t)segs;
    hipError_t e = kda::launch_cp_segments(cu_seqlens, nseq, segments, cu_seg, stream);
    if (e != hipSuccess) return hip_status(e);
    // segments whose transition is provably below fp32 resolution skip the M pass
    e = kda::launch_cp_bound(k, log_alpha, beta, cu_seg, ns, H, dk, bf16, negligible, stream);
    if (e != hipSuccess) return hip_status(e);
    if (total_tokens > 0) {
        kda::ChunkLocalArgs c{q, k, log_alpha, beta, cu_seg, ns, H, dk, total_tokens, bf16, cl, stream};
        if ((e = kda::launch_chunk_local(c)) != hipSuccess) return hip_status(e);
    }
    // each segment from a zero state: S~ (outputs not written)
    kda::InterChunkArgs a1{q, k, v, log_alpha, nullptr, cu_seg, ns, H, dk, dv, total_tokens, bf16, cl,
                           nullptr, St, 0, 0, stream};
    if ((e = kda::launch_inter_chunk(a1)) != hipSuccess) return hip_status(e);
    // each segment's transition M: v = 0 from the identity, in place
    if ((e = kda::launch_cp_identity(M, segs * H, dk, stream)) != hipSuccess) return hip_status(e);
    kda::InterChunkArgs a2{q, k, nullptr, log_alpha, M, cu_seg, ns, H, dk, dk, total_tokens, bf16, cl,
                           nullptr, M, 0, 0, stream};
    a2.skip = negligible;
    if ((e = kda::launch_inter_chunk(a2)) != hipSuccess) return hip_status(e);
    if ((e = kda::launch_cp_scan(init_state, M, St, negligible, Sin, nseq, H, dk, dv, segments, stream)) !=
        hipSuccess)
        return hip_status(e);
    // the outputs from the exact incoming states; each segment's final state replaces its S_in
    kda::InterChunkArgs a3{q, k, v, log_alpha, Sin, cu_seg, ns, H, dk, dv, total_tokens, bf16, cl,
                           o, Sin, 0, 0, stream};
    if ((e = kda::launch_inter_chunk(a3)) != hipSuccess) return hip_status(e);
    if (final_state) e = kda::launch_cp_final(Sin, final_state, nseq, H, dk, dv, segments, stream);
    return hip_status(e);
}

kda_status kda_decode_step_fused(const void *q, const void *k, const void *v, const void *gate,
                                 const float *gate_A_log, const void *beta, float *state, float *o,
                                 const void *out_gate, const float *norm_w, float norm_eps, void *y,
                                 int32_t B, int32_t H, int32_t dk, int32_t dv, kda_dtype dt, void *stream) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || (int64_t)B * H >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;
    kda_status st = check_inputs({q, k, v, gate}, true, beta, dt == KDA_BF16, true);
    if (st != KDA_OK) return st;
    st = check_ptrs({state}, {o});
    if (st != KDA_OK) return st;
    if (!o && !out_gate) return KDA_ERR_NULL;
    st = check_fusion(gate_A_log, out_gate, norm_w, norm_eps, y, dt == KDA_BF16);
    if (st != KDA_OK) return st;
    kda::DecodeArgs a{q, k, v, gate, beta, state, o, B, H, dk, dv, dt == KDA_BF16, stream,
                      {gate_A_log, out_gate, norm_w, norm_eps, y}};
    return hip_status(kda::launch_decode(a));
}

kda_status kda_decode_layer_step(const void *qkv, const float *conv_w, float *conv_cache, float l2_eps,
                                 const void *gate, const float *gate_A_log, const void *beta, float *state, float *o,
                                 const void *out_gate, const float *norm_w, float norm_eps, void *y, int32_t B,
                                 int32_t H, int32_t dk, int32_t dv, kda_dtype dt, void *stream) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || (int64_t)B * H >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;
    if (!(l2_eps >= 0.f && l2_eps <= 3.4e38f)) return KDA_ERR_SHAPE;
    // qkv rows are read element-wise (q, k) and four at a time (v): 4-element aligned
    kda_status st = check_inputs({qkv, gate}, true, beta, dt == KDA_BF16, true);
    if (st != KDA_OK) return st;
    st = check_ptrs({state, conv_w}, {o});
    if (st != KDA_OK) return st;
    if (!conv_cache) return KDA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(conv_cache) & 3u) return KDA_ERR_ALIGN;
    if (!o && !out_gate) return KDA_ERR_NULL;
    st = check_fusion(gate_A_log, out_gate, norm_w, norm_eps, y, dt == KDA_BF16);
    if (st != KDA_OK) return st;
    kda::DecodeArgs a{qkv, nullptr, nullptr, gate, beta, state, o, B, H, dk, dv, dt == KDA_BF16, stream,
                      {gate_A_log, out_gate, norm_w, norm_eps, y, conv_w, conv_cache, l2_eps}};
    return hip_status(kda::launch_decode(a));
}

kda_status kda_decode_step(const void *q, const void *k, const void *v, const void *log_alpha,
                           const void *beta, float *state, float *o, int32_t B, int32_t H,
                           int32_t dk, int32_t dv, kda_dtype dt, void *stream) {
    if (!o) return KDA_ERR_NULL;
    return kda_decode_step_fused(q, k, v, log_alpha, nullptr, beta, state, o, nullptr, nullptr, 0.f, nullptr,
                                 B, H, dk, dv, dt, stream);
}

kda_status kda_decode_window_fused(const void *q, const void *k, const void *v, const void *gate,
                                   const float *gate_A_log, const void *beta, float *state, float *o,
                                   const int32_t *accept, const void *out_gate, const float *norm_w,
                                   float norm_eps, void *y, int32_t B, int32_t T, int32_t H, int32_t dk,
                                   int32_t dv, kda_dtype dt, void *stream) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
    if (B < 1 || T < 1 || H < 1 || (int64_t)B * T * H >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;
    kda_status st = check_inputs({q, k, v, gate}, true, beta, dt == KDA_BF16, true);
    if (st != KDA_OK) return st;
    st = check_ptrs({state}, {o});
    if (st != KDA_OK) return st;
    if (accept && (reinterpret_cast<uintptr_t>(accept) & 3u)) return KDA_ERR_ALIGN;
    st = check_fusion(gate_A_log, out_gate, norm_w, norm_eps, y, dt == KDA_BF16);
    if (st != KDA_OK) return st;
    if (out_gate) {  // the window's epilogue runs over o: o is required, rows 16-byte aligned
        if (!o) return KDA_ERR_NULL;
        st = check_rows16({out_gate, y}, true);
        if (st != KDA_OK) return st;
    }
    kda::DecodeWindowArgs a{q, k, v, gate, beta, state, o, accept, B, T, H, dk, dv, dt == KDA_BF16, stream,
                            {gate_A_log, out_gate, norm_w, norm_eps, y}};
    return hip_status(kda::launch_decode_window(a));
}

kda_status kda_decode_window_replay(const void *pq, const void *pk, const void *pv, const void *pgate,
                                    const void *pbeta, const int32_t *replay, int32_t Tp, const void *q,
                                    const void *k, const void *v, const void *gate, const float *gate_A_log,
                                    const void *beta, float *state, float *o, const void *out_gate,
                                    const float *norm_w, float norm_eps, void *y, int32_t B, int32_t T, int32_t H,
                                    int32_t dk, int32_t dv, kda_dtype dt, void *stream) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
    if (B < 1 || T < 1 || H < 1 || Tp < 0 || (int64_t)B * T * H >= (int64_t(1) << 31) ||
        (int64_t)B * Tp * H >= (int64_t(1) << 31))
        return KDA_ERR_SHAPE;
    kda_status st = check_inputs({q, k, v, gate}, true, beta, dt == KDA_BF16, true);
    if (st != KDA_OK) return st;
    if (Tp > 0) {
        if (!replay) return KDA_ERR_NULL;
        if (reinterpret_cast<uintptr_t>(replay) & 3u) return KDA_ERR_ALIGN;
        st = check_inputs({pq, pk, pv, pgate}, true, pbeta, dt == KDA_BF16, true);
        if (st != KDA_OK) return st;
    }
    st = check_ptrs({state}, {o});
    if (st != KDA_OK) return st;
    st = check_fusion(gate_A_log, out_gate, norm_w, norm_eps, y, dt == KDA_BF16);
    if (st != KDA_OK) return st;
    if (out_gate) {  // the epilogue runs over o: o is required, rows 16-byte aligned
        if (!o) return KDA_ERR_NULL;
        st = check_rows16({out_gate, y}, true);
        if (st != KDA_OK) return st;
    }
    kda::DecodeWindowArgs a{q, k, v, gate, beta, state, o, nullptr, B, T, H, dk, dv, dt == KDA_BF16, stream,
                            {gate_A_log, out_gate, norm_w, norm_eps, y}};
    a.acc_default = 0;  // this window's drafts are not committed
    if (Tp > 0) {
        a.pq = pq;
        a.pk = pk;
        a.pv = pv;
        a.pg = pgate;
        a.pbeta = pbeta;
        a.replay = replay;
        a.Tp = Tp;
    }
    return hip_status(kda::launch_decode_window(a));
}

kda_status kda_decode_layer_window_replay(const void *pqkv, const void *pgate, const void *pbeta,
                                          const int32_t *replay, int32_t Tp, const void *qkv, const void *gate,
                                          const void *beta, const float *conv_w, float *conv_cache, float l2_eps,
                                          const float *gate_A_log, float *state, float *o, const void *out_gate,
                                          const float *norm_w, float norm_eps, void *y, int32_t B, int32_t T,
                                          int32_t H, int32_t dk, int32_t dv, kda_dtype dt, void *workspace,
                                          size_t workspace_bytes, void *stream) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
    if (B < 1 || T < 1 || H < 1 || Tp < 0 || (int64_t)B * T * H >= (int64_t(1) << 31) ||
        (int64_t)B * Tp * H >= (int64_t(1) << 31))
        return KDA_ERR_SHAPE;
    if (!(l2_eps >= 0.f && l2_eps <= 3.4e38f)) return KDA_ERR_SHAPE;
    kda_status st = check_inputs({qkv, gate}, true, beta, dt == KDA_BF16, true);
    if (st != KDA_OK) return st;
    if (Tp > 0) {
        if (!replay) return KDA_ERR_NULL;
        if (reinterpret_cast<uintptr_t>(replay) & 3u) return KDA_ERR_ALIGN;
        st = check_inputs({pqkv, pgate}, true, pbeta, dt == KDA_BF16, true);
        if (st != KDA_OK) return st;
    }
    st = check_ptrs({state, conv_w, o}, {});
    if (st != KDA_OK) return st;
    if (!conv_cache) return KDA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(conv_cache) & 3u) return KDA_ERR_ALIGN;
    st = check_fusion(gate_A_log, out_gate, norm_w, norm_eps, y, dt == KDA_BF16);
    if (st != KDA_OK) return st;
    if (out_gate) {  // the epilogue runs over o: rows 16-byte aligned
        st = check_rows16({out_gate, y}, true);
        if (st != KDA_OK) return st;
    }
    kda::DecodeWindowArgs a{qkv, nullptr, nullptr, gate, beta, state, o, nullptr, B, T, H, dk, dv, dt == KDA_BF16,
                            stream, {gate_A_log, out_gate, norm_w, norm_eps, y, conv_w, conv_cache, l2_eps}};
    a.acc_default = 0;  // this window's drafts are not committed
    if (Tp > 0) {
        a.pq = pqkv;
        a.pg = pgate;
        a.pbeta = pbeta;
        a.replay = replay;
        a.Tp = Tp;
    }
    if (workspace && kda::layer_window_chunk_supported(a) && (int64_t)T + Tp >= kda::WINDOW_CHUNK_MIN_TOKENS) {
        if (reinterpret_cast<uintptr_t>(workspace) & 15u) return KDA_ERR_ALIGN;
        if (workspace_bytes < kda::layer_window_chunk_bytes(B, T, Tp, H)) return KDA_ERR_SHAPE;
        return hip_status(kda::launch_layer_window_chunk(a, workspace));
    }
    return hip_status(kda::launch_decode_window(a));
}

size_t kda_decode_layer_window_workspace_bytes(int32_t B, int32_t T, int32_t Tp, int32_t H, int32_t dk,
                                               int32_t dv, kda_dtype dt) {
    if (B < 1 || T < 1 || H < 1 || Tp < 0 || (int64_t)B * T * H >= (int64_t(1) << 31) ||
        (int64_t)B * Tp * H >= (int64_t(1) << 31))
        return 0;
    const int64_t tokens = (int64_t)T + Tp;
    if (!(dt == KDA_BF16 && dk == 128 && dv == 128 && tokens >= kda::WINDOW_CHUNK_MIN_TOKENS && tokens <= 16))
        return 0;
    return kda::layer_window_chunk_bytes(B, T, Tp, H);
}

kda_status kda_decode_window(const void *q, const void *k, const void *v, const void *log_alpha,
                             const void *beta, float *state, float *o, const int32_t *accept,
                             int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                             void *stream) {
    return kda_decode_window_fused(q, k, v, log_alpha, nullptr, beta, state, o, accept, nullptr, nullptr, 0.f,
                                   nullptr, B, T, H, dk, dv, dt, stream);
}

kda_status kda_decode_window_form(const void *q, const void *k, const void *v, const void *log_alpha,
                                  const void *beta, float *state, float *o, const int32_t *accept,
                                  int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                                  int32_t form, void *stream) {
    if (form < 0 || form > 2) return KDA_ERR_SHAPE;
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
    if (B < 1 || T < 1 || H < 1 || (int64_t)B * T * H >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;
    kda_status st = check_inputs({q, k, v, log_alpha}, true, beta, dt == KDA_BF16, true);
    if (st != KDA_OK) return st;
    st = check_ptrs({state}, {o});
    if (st != KDA_OK) return st;
    if (accept && (reinterpret_cast<uintptr_t>(accept) & 3u)) return KDA_ERR_ALIGN;
    kda::DecodeWindowArgs a{q, k, v, log_alpha, beta, state, o, accept, B, T, H, dk, dv, dt == KDA_BF16, stream, {}};
    a.form = form;
    if (form == 2 && !kda::window_chunk_supported(a)) return KDA_ERR_UNSUPPORTED;
    return hip_status(kda::launch_decode_window(a));
}


size_t kda_prefill_backward_workspace_bytes(int64_t total_tokens, int32_t nseq, int32_t H, int32_t dk,
                                            int32_t dv, kda_dtype dt) {
    if (check_backward_shape(nseq, total_tokens, H, dk, dv, dt) != KDA_OK) return 0;
    return static_cast<size_t>(kda::backward_workspace_floats(total_tokens, nseq, H, dk, dv)) * sizeof(float);
}

kda_status kda_prefill_backward(const void *q, const void *k, const void *v, const void *log_alpha,
                                const void *beta, const float *init_state, const int32_t *cu_seqlens, int32_t nseq,
                                int64_t total_tokens, int32_t H, int32_t dk, int32_t dv, kda_dtype dt,
                                const float *d_o, const float *d_final, float *d_q, float *d_k, float *d_v,
                                float *d_log_alpha, float *d_beta, float *d_init, void *workspace, size_t ws_bytes,
                                void *stream) {
    kda_status st = check_backward_shape(nseq, total_tokens, H, dk, dv, dt);
    if (st != KDA_OK) return st;
    const bool any = total_tokens > 0;
    st = check_inputs({q, k, v, log_alpha}, true, beta, dt == KDA_BF16, any);
    if (st != KDA_OK) return st;
    st = check_ptrs({cu_seqlens}, {init_state, d_final, d_init});
    if (st != KDA_OK) return st;
    for (const void *p : {static_cast<const void *>(d_o), static_cast<const void *>(d_q),
                          static_cast<const void *>(d_k), static_cast<const void *>(d_v),
                          static_cast<const void *>(d_log_alpha), static_cast<const void *>(d_beta)}) {
        if (!p && any) return KDA_ERR_NULL;
        if (p && (reinterpret_cast<uintptr_t>(p) & 3u)) return KDA_ERR_ALIGN;
    }
    const size_t need = static_cast<size_t>(kda::backward_workspace_floats(total_tokens, nseq, H, dk, dv)) * 4;
    if (!workspace || ws_bytes < need) return KDA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KDA_ERR_ALIGN;
    kda::BackwardArgs a{q, k, v, log_alpha, beta, init_state, cu_seqlens, nseq, total_tokens, H, dk, dv,
                        dt == KDA_BF16, d_o, d_final, d_q, d_k, d_v, d_log_alpha, d_beta, d_init,
                        static_cast<float *>(workspace), stream};
    return hip_status(kda::launch_backward(a));
}

// Slabbed backward of one sequence (see kda.h): the slabs' {0, length} lists, the state at
// every slab boundary, two adjoint buffers, then one slab's backward workspace.
struct SlabLayout {
    size_t cu, bnd, adj, ws, total;
    int32_t nslab;
};
SlabLayout slab_layout(int64_t N, int32_t H, int32_t dk, int32_t dv, int64_t L) {
    auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
    SlabLayout S{};
    S.nslab = N > L ? (int32_t)((N + L - 1) / L) : 1;
    const size_t state = (size_t)H * dk * dv * 4;
    S.cu = 0;
    S.bnd = up((size_t)S.nslab * 8);
    S.adj = S.bnd + up((size_t)(S.nslab > 1 ? S.nslab - 1 : 0) * state);
    S.ws = S.adj + up(2 * state);
    S.total = S.ws + up((size_t)kda::backward_workspace_floats(L < N ? L : N, 1, H, dk, dv) * 4);
    return S;
}
kda_status check_slab(int64_t N, int32_t H, int32_t dk, int32_t dv, kda_dtype dt, int64_t L) {
    kda_status st = check_backward_shape(1, N, H, dk, dv, dt);
    if (st != KDA_OK) return st;
    if (L < 16 || L % 16 != 0 || L >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;
    if ((N + L - 1) / L >= (int64_t(1) << 24)) return KDA_ERR_SHAPE;
    return KDA_OK;
}

size_t kda_prefill_backward_slabbed_workspace_bytes(int64_t total_tokens, int32_t H, int32_t dk, int32_t dv,
                                                    kda_dtype dt, int64_t slab_tokens) {
    if (check_slab(total_tokens, H, dk, dv, dt, slab_tokens) != KDA_OK) return 0;
    return slab_layout(total_tokens, H, dk, dv, slab_tokens).total;
}

kda_status kda_prefill_backward_slabbed(const void *q, const void *k, const void *v, const void *log_alpha,
                                        const void *beta, const float *init_state, int64_t total_tokens, int32_t H,
                                        int32_t dk, int32_t dv, kda_dtype dt, const float *d_o, const float *d_final,
                                        float *d_q, float *d_k, float *d_v, float *d_log_alpha, float *d_beta,
                                        float *d_init, int64_t slab_tokens, void *workspace, size_t ws_bytes,
                                        void *stream) {
    kda_status st = check_slab(total_tokens, H, dk, dv, dt, slab_tokens);
    if (st != KDA_OK) return st;
    const bool any = total_tokens > 0;
    st = check_inputs({q, k, v, log_alpha}, true, beta, dt == KDA_BF16, any);
    if (st != KDA_OK) return st;
    st = check_ptrs({}, {init_state, d_final, d_init});
    if (st != KDA_OK) return st;
    for (const void *p : {static_cast<const void *>(d_o), static_cast<const void *>(d_q),
                          static_cast<const void *>(d_k), static_cast<const void *>(d_v),
                          static_cast<const void *>(d_log_alpha), static_cast<const void *>(d_beta)}) {
        if (!p && any) return KDA_ERR_NULL;
        if (p && (reinterpret_cast<uintptr_t>(p) & 3u)) return KDA_ERR_ALIGN;
    }
    const SlabLayout S = slab_layout(total_tokens, H, dk, dv, slab_tokens);
    if (!workspace || ws_bytes < S.total) return KDA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KDA_ERR_ALIGN;
    char *w = static_cast<char *>(workspace);
    int32_t *cu = reinterpret_cast<int32_t *>(w + S.cu);
    float *bnd = reinterpret_cast<float *>(w + S.bnd), *adj = reinterpret_cast<float *>(w + S.adj);
    float *ws = reinterpret_cast<float *>(w + S.ws);
    const int64_t state = (int64_t)H * dk * dv;
    const size_t esz = dt == KDA_BF16 ? 2 : 4;
    const bool bf16 = dt == KDA_BF16;
    if (S.nslab <= 1) {  // one slab: the plain backward (also for N = 0, with a one-element list)
        if ((st = hip_status(kda::launch_backward_slab_cu(cu, total_tokens, slab_tokens, 1, stream))) != KDA_OK)
            return st;
        kda::BackwardArgs a{q, k, v, log_alpha, beta, init_state, cu, 1, total_tokens, H, dk, dv, bf16, d_o,
                            d_final, d_q, d_k, d_v, d_log_alpha, d_beta, d_init, ws, stream};
        return hip_status(kda::launch_backward(a));
    }
    if ((st = hip_status(kda::launch_backward_slab_cu(cu, total_tokens, slab_tokens, S.nslab, stream))) != KDA_OK)
        return st;
    // token views and boundary states of slab s (boundary s = the state entering slab s + 1)
    auto in = [&](const void *p, int s, int64_t d) {
        return p ? static_cast<const void *>(static_cast<const char *>(p) + (size_t)s * slab_tokens * H * d * esz)
                 : nullptr;
    };
    auto f32 = [&](const float *p, int s, int64_t d) { return p ? p + (size_t)s * slab_tokens * H * d : nullptr; };
    auto f32w = [&](float *p, int s, int64_t d) { return p ? p + (size_t)s * slab_tokens * H * d : nullptr; };
    auto len_of = [&](int s) {
        const int64_t a = (int64_t)s * slab_tokens;
        return (total_tokens - a < slab_tokens ? total_tokens - a : slab_tokens);
    };
    auto init_of = [&](int s) { return s == 0 ? init_state : bnd + (size_t)(s - 1) * state; };
    // 1. boundary states, slab by slab, by the backward's own fp32 forward sweep
    for (int s = 0; s + 1 < S.nslab; ++s) {
        kda::BackwardArgs a{in(q, s, dk), in(k, s, dk), in(v, s, dv), in(log_alpha, s, dk), in(beta, s, 1),
                            init_of(s), cu + 2 * s, 1, len_of(s), H, dk, dv, bf16, nullptr, nullptr, nullptr,
                            nullptr, nullptr, nullptr, nullptr, nullptr, ws, stream};
        if ((st = hip_status(kda::launch_backward_states(a, bnd + (size_t)s * state))) != KDA_OK) return st;
    }
    // 2. the slabs' gradients in reverse; the adjoint of a slab's initial state is the next
    //    (earlier) slab's final-state adjoint
    for (int s = S.nslab - 1; s >= 0; --s) {
        const float *dfin = s == S.nslab - 1 ? d_final : adj + (size_t)((s + 1) & 1) * state;
        float *dini = s == 0 ? d_init : adj + (size_t)(s & 1) * state;
        kda::BackwardArgs a{in(q, s, dk), in(k, s, dk), in(v, s, dv), in(log_alpha, s, dk), in(beta, s, 1),
                            init_of(s), cu + 2 * s, 1, len_of(s), H, dk, dv, bf16, f32(d_o, s, dv), dfin,
                            f32w(d_q, s, dk), f32w(d_k, s, dk), f32w(d_v, s, dv), f32w(d_log_alpha, s, dk),
                            f32w(d_beta, s, 1), dini, ws, stream};
        if ((st = hip_status(kda::launch_backward(a))) != KDA_OK) return st;
    }
    return KDA_OK;
}

kda_status kda_gate(const void *z, const float *A_log, int64_t N, int32_t H, int32_t dk, kda_dtype dt,
                    void *log_alpha, void *stream) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dim_ok(dk)) return KDA_ERR_UNSUPPORTED;
    // (token, head) rows are indexed in 32 bits
    if (H < 1 || N < 0 || N >= (int64_t(1) << 31) || N * H >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;
    kda_status st = check_rows16({z, log_alpha}, N > 0);
    if (st != KDA_OK) return st;
    if (!A_log) return KDA_ERR_NULL;
    kda::GateArgs a{z, A_log, log_alpha, N, H, dk, dt == KDA_BF16, stream};
    return hip_status(kda::launch_gate(a));
}

kda_status kda_check_cu_seqlens(const int32_t *cu_seqlens, int32_t nseq, int64_t total_tokens, int32_t *result,
                                void *stream) {
    if (!cu_seqlens || !result) return KDA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) || (reinterpret_cast<uintptr_t>(result) & 3u))
        return KDA_ERR_ALIGN;
    if (nseq < 1 || nseq >= (int32_t(1) << 30) || total_tokens < 0 || total_tokens >= (int64_t(1) << 31))
        return KDA_ERR_SHAPE;
    return hip_status(kda::launch_check_cu_seqlens(cu_seqlens, nseq, total_tokens, result, stream));
}

kda_status kda_short_conv(const void *x, const float *w, const float *cache_in, float *cache_out,
                          const int32_t *cu_seqlens, int32_t nseq, int64_t N, int32_t H, int32_t d,
                          int32_t l2norm, float eps, kda_dtype dt, void *y, void *stream) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dim_ok(d)) return KDA_ERR_UNSUPPORTED;
    if (nseq < 1 || H < 1 || N < 0 || N >= (int64_t(1) << 31) || N * H >= (int64_t(1) << 31) ||
        !(eps >= 0.f && eps <= 3.4e38f))
        return KDA_ERR_SHAPE;
    if ((int64_t)nseq * H * d >= (int64_t(1) << 31)) return KDA_ERR_SHAPE;
    kda_status st = check_rows16({x, y}, N > 0);
    if (st != KDA_OK) return st;
    st = check_ptrs({w}, {});
    if (st != KDA_OK) return st;
    if (!cu_seqlens && nseq != N) return KDA_ERR_SHAPE;  // one token per sequence
    if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) return KDA_ERR_ALIGN;
    if ((cache_in && (reinterpret_cast<uintptr_t>(cache_in) & 3u)) ||
        (cache_out && (reinterpret_cast<uintptr_t>(cache_out) & 3u)))
        return KDA_ERR_ALIGN;
    if (N > 0 && x == y) return KDA_ERR_SHAPE;
    kda::ShortConvArgs a{x, w, cache_in, cache_out, cu_seqlens, nseq, N, H, d, l2norm != 0, eps,
                         dt == KDA_BF16, y, stream};
    return hip_status(kda::launch_short_conv(a));
}

kda_status kda_out_norm_gate(const float *o, const void *u, const float *w, float eps, int64_t N, int32_t H,
                             int32_t dv, kda_dtype dt, void *y, void *stream) {
    if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
    if (H < 1 || N < 0 || N >= (int64_t(1) << 31) || N * H >= (int64_t(1) << 31) ||
        !(eps >= 0.f && eps <= 3.4e38f))
        return KDA_ERR_SHAPE;
    kda_status st = check_rows16({u, y}, N > 0);
    if (st != KDA_OK) return st;
    st = check_ptrs({w}, {o});
    if (st != KDA_OK) return st;
    if (N > 0 && !o) return KDA_ERR_NULL;
    kda::OutNormGateArgs a{o, u, w, eps, N, H, dv, dt == KDA_BF16, y, stream};
    return hip_status(kda::launch_out_norm_gate(a));
}

const char *kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
        case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: a pointer is misaligned (fp32 buffers 16 B; q/k/v/log_alpha 4 elements; beta 1 element)";
        case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: nseq, H, B or total_tokens out of range";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: dk/dv not in {16,32,64,128} or unknown dtype";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: kernel launch failed (see kda_last_hip_error)";
        case KDA_ERR_TOO_LARGE: return "KDA_ERR_TOO_LARGE: the problem's workspace exceeds the static scratch of "
                                       "kda_prefill_noalloc (KDA_NOALLOC_SCRATCH_BYTES)";
        default: return "KDA: unknown status";
    }
}

int32_t kda_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
