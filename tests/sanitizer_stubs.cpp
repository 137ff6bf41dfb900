// Host-only test doubles for building the C-ABI validation layer (api.cpp) on the CPU with
// AddressSanitizer and UndefinedBehaviorSanitizer.  The kernel launchers do nothing and report
// success (the ABI tests pass pointers that must never be dereferenced); the shape predicates
// and the workspace formula follow the rules the kernel sources implement; the allocation-free
// entry point follows its documented host behaviour (the size check, then kda_prefill on a
// stand-in workspace).  Test infrastructure only: never linked into the product library.
#include <hip/hip_runtime_api.h>

#include "kda.h"
#include "kda_launch.hpp"

namespace kda {

hipError_t launch_chunk_local(const ChunkLocalArgs &) { return hipSuccess; }
hipError_t launch_inter_chunk(const InterChunkArgs &) { return hipSuccess; }
hipError_t launch_inter_chunk_ws(const InterChunkArgs &, int, int) { return hipSuccess; }
hipError_t launch_decode(const DecodeArgs &) { return hipSuccess; }
hipError_t launch_decode_window(const DecodeWindowArgs &) { return hipSuccess; }
hipError_t launch_window_chunk(const DecodeWindowArgs &) { return hipSuccess; }
hipError_t launch_layer_window_chunk(const DecodeWindowArgs &, void *) { return hipSuccess; }
hipError_t launch_check_cu_seqlens(const int32_t *, int32_t, int64_t, int32_t *, void *) { return hipSuccess; }
size_t layer_window_chunk_bytes(int64_t B, int64_t T, int64_t Tp, int64_t H) {
    return (size_t)1024 * (size_t)(B * H * (T + Tp));  // bf16 q, k, v, log-decay of 128 channels
}
hipError_t launch_backward(const BackwardArgs &) { return hipSuccess; }
hipError_t launch_backward_states(const BackwardArgs &, float *) { return hipSuccess; }
hipError_t launch_backward_slab_cu(int32_t *, int64_t, int64_t, int32_t, void *) { return hipSuccess; }
hipError_t launch_gate(const GateArgs &) { return hipSuccess; }
hipError_t launch_layer_conv_cache(const void *, const void *, const void *, const float *, float *, const int32_t *,
                                   int32_t, int32_t, int32_t, int32_t, void *) {
    return hipSuccess;
}
hipError_t launch_short_conv(const ShortConvArgs &) { return hipSuccess; }
hipError_t launch_out_norm_gate(const OutNormGateArgs &) { return hipSuccess; }
hipError_t launch_prefill_fused(const PrefillFusedArgs &, int, int) { return hipSuccess; }
hipError_t launch_cp_segments(const int32_t *, int32_t, int32_t, int32_t *, void *) { return hipSuccess; }
hipError_t launch_cp_identity(float *, int64_t, int32_t, void *) { return hipSuccess; }
hipError_t launch_cp_scan(const float *, const float *, const float *, const int32_t *, float *, int32_t, int32_t,
                          int32_t, int32_t, int32_t, void *) {
    return hipSuccess;
}
hipError_t launch_cp_bound(const void *, const void *, const void *, const int32_t *, int32_t, int32_t, int32_t, bool,
                           int32_t *, void *) {
    return hipSuccess;
}
hipError_t launch_cp_final(const float *, float *, int32_t, int32_t, int32_t, int32_t, int32_t, void *) {
    return hipSuccess;
}

bool prefill_fused_supported(int dk, int dv, bool bf16, int64_t chains) {
    return bf16 && dk == 128 && dv == 128 && chains >= 256;
}
bool prefill_fused_shape_built(int nc, int sl) {
    return (nc == 0 && sl == 0) || (nc == 4 && (sl == 1 || sl == 2)) || (nc == 2 && sl == 1);
}
bool inter_chunk_ws_shape_built(int dk, int dv, int ncw, int npw) {
    if (dk == 128 && dv == 128 && (ncw == 4 || ncw == 2) && npw == 4) return true;
    const int c4 = dv / 16 < 4 ? dv / 16 : 4, c2 = dv / 16 < 2 ? dv / 16 : 2, p = dk / 16 < 4 ? dk / 16 : 4;
    return dk >= 32 && (ncw == c4 || (dv >= 64 && ncw == c2)) && npw == p;
}
int64_t backward_workspace_floats(int64_t N, int32_t nseq, int32_t H, int32_t dk, int32_t dv) {
    const int64_t slots = chunk_slots(N, nseq);
    return 2 * slots * H * (int64_t)dk * dv + 2 * slots * H * 16 * (int64_t)dv + slots * H * 4 * 256;
}

}  // namespace kda

extern "C" kda_status kda_prefill_noalloc(const void *q, const void *k, const void *v, const void *log_alpha,
                                          const void *beta, const float *init_state, const int32_t *cu_seqlens,
                                          int32_t nseq, int64_t total_tokens, int32_t H, int32_t dk, int32_t dv,
                                          kda_dtype dt, float *o, float *final_state, void *stream) {
    const size_t need = kda_prefill_workspace_bytes(total_tokens, nseq, H, dk, dv, dt);
    if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_TOO_LARGE;
    static unsigned char stand_in[256] __attribute__((aligned(256)));  // never dereferenced
    return kda_prefill(q, k, v, log_alpha, beta, init_state, cu_seqlens, nseq, total_tokens, H, dk, dv, dt, o,
                       final_state, stand_in, (size_t)KDA_NOALLOC_SCRATCH_BYTES, stream);
}
