// Internal launcher interface between the C ABI layer (api.cpp) and the
// kernel translation units.  Arguments are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Workspace per (chunk slot, head): T' = (I + A_kk)^-1 diag(beta), then A_qk,
// each stored as the A-operand fragment of a 16x16 MFMA (64 lanes x 16 bytes:
// lane 16g + m holds row m, columns 4g..4g+3; as {hi[4], lo[4]} bf16 for bf16
// inputs, as 4 fp32 for fp32 inputs).  2 KiB per (chunk slot, head).
constexpr int WS_FLOATS_PER_CHUNK_HEAD = 2 * 16 * 16;

// Chunk slots: sequence s owns slots floor(cu[s]/16) + s + j, j < ceil(len_s/16).
// The map is injective and bounded by floor(N/16) + nseq.
inline int64_t chunk_slots(int64_t total_tokens, int32_t nseq) { return total_tokens / 16 + nseq; }

// Optional work fused into the decode kernels (all NULL: plain decode).
struct DecodeFusion {
    const float *A_log;        // [H]: g holds decay logits z, log-decay = -5 Sigmoid(e^{A_h} z)
    const void *u;             // output-gate logits shaped like o (input dtype): y = Sigmoid(u) RMSNorm(o) w
    const float *w;            // [dv] RMSNorm weight
    float eps;
    void *y;                   // shaped like o, input dtype
    // ShortConv prologue (single-step kernel only): q points at the pre-convolution
    // rows [B, H, 2 dk + dv] (q | k | v channels), k and v are unused
    const float *conv_w;       // [H, 2 dk + dv, 4], tap j on x_{t-j}
    float *conv_cache;         // [B, H, 2 dk + dv, 3], oldest first, updated in place
    float l2eps;               // L2 normalisation of q and k
};

struct DecodeArgs {
    const void *q, *k, *v, *g, *beta;
    float *state, *o;          // o may be NULL when the epilogue writes y
    int32_t B, H, dk, dv;
    bool bf16;
    void *stream;
    DecodeFusion fx;
};

struct DecodeWindowArgs {
    const void *q, *k, *v, *g, *beta;
    float *state, *o;          // o may be NULL (no outputs)
    const int32_t *accept;     // device [B] or NULL (all T tokens accepted)
    int32_t B, T, H, dk, dv;
    bool bf16;
    void *stream;
    DecodeFusion fx;
};

struct ChunkLocalArgs {
    const void *q, *k, *g, *beta;
    const int32_t *cu;
    int32_t nseq, H, dk;
    int64_t total_tokens;
    bool bf16;
    float *ws;
    void *stream;
};

struct InterChunkArgs {
    const void *q, *k, *v, *g;
    const float *init;
    const int32_t *cu;
    int32_t nseq, H, dk, dv;
    int64_t total_tokens;
    bool bf16;
    const float *ws;
    float *o, *fin;
    int32_t waves_per_group;  // 0 = choose automatically
    void *stream;
};

struct GateArgs {
    const void *z;             // decay logits [N, H, dk]
    const float *A_log;        // [H]
    void *g;                   // log-decay out [N, H, dk], input dtype
    int64_t N;
    int32_t H, dk;
    bool bf16;
    void *stream;
};

struct ShortConvArgs {
    const void *x;             // [N, H, d]
    const float *w;            // [H, d, 4]
    const float *cache_in;     // [nseq, H, d, 3] or NULL
    float *cache_out;          // [nseq, H, d, 3] or NULL (may equal cache_in)
    const int32_t *cu;         // [nseq + 1]
    int32_t nseq;
    int64_t N;
    int32_t H, d;
    bool l2norm;
    float eps;
    bool bf16;
    void *y;                   // [N, H, d], input dtype
    void *stream;
};

struct OutNormGateArgs {
    const float *o;            // [N, H, dv]
    const void *u;             // gate logits [N, H, dv], input dtype
    const float *w;            // [dv]
    float eps;
    int64_t N;
    int32_t H, dv;
    bool bf16;
    void *y;                   // [N, H, dv], input dtype
    void *stream;
};

struct BackwardArgs {
    const void *q, *k, *v, *g, *beta;  // forward inputs [N, H, .], input dtype
    const float *init;                 // [nseq, H, dk, dv] or NULL
    const int32_t *cu;
    int32_t nseq;
    int64_t N;
    int32_t H, dk_, dv_;
    bool bf16;
    const float *dO;                   // [N, H, dv]
    const float *dfinal;               // [nseq, H, dk, dv] or NULL
    float *dq, *dk, *dv, *dg, *dbeta;  // [N, H, dk] x3 (dq, dk, dlog_alpha), [N, H, dv], [N, H]
    float *dinit;                      // [nseq, H, dk, dv] or NULL
    float *ws;                         // backward_workspace_floats(...) floats
    void *stream;
};

hipError_t launch_backward(const BackwardArgs &a);
int64_t backward_workspace_floats(int64_t N, int32_t nseq, int32_t H, int32_t dk, int32_t dv);

// Intra-device context parallelism (cp.hip): the small kernels around the prefill passes.
hipError_t launch_cp_segments(const int32_t *cu, int32_t nseq, int32_t R, int32_t *cu_seg, void *stream);
hipError_t launch_cp_identity(float *M, int64_t n_mats, int32_t dk, void *stream);
hipError_t launch_cp_scan(const float *init, const float *M, const float *St, float *Sin, int32_t nseq, int32_t H,
                          int32_t dk, int32_t dv, int32_t R, void *stream);
hipError_t launch_cp_final(const float *Sin, float *fin, int32_t nseq, int32_t H, int32_t dk, int32_t dv, int32_t R,
                           void *stream);

hipError_t launch_gate(const GateArgs &a);
hipError_t launch_short_conv(const ShortConvArgs &a);
hipError_t launch_out_norm_gate(const OutNormGateArgs &a);
hipError_t launch_decode(const DecodeArgs &a);
hipError_t launch_decode_window(const DecodeWindowArgs &a);
hipError_t launch_chunk_local(const ChunkLocalArgs &a);
hipError_t launch_inter_chunk(const InterChunkArgs &a);
// Warp-specialised inter-chunk kernel (bf16, dk >= 32): ncw consumer and npw
// producer waves per workgroup; hipErrorInvalidValue for a shape not built.
hipError_t launch_inter_chunk_ws(const InterChunkArgs &a, int ncw, int npw);

}  // namespace kda
