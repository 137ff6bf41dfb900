// Internal launcher interface between the C ABI layer (api.cpp) and the
// kernel translation units.  Arguments are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

// KDA_OK for hipSuccess; otherwise keeps e for kda_last_hip_error() (per thread) and
// returns KDA_ERR_HIP.  Defined in api.cpp.
kda_status record_hip_error(hipError_t e);

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
    // ShortConv prologue (single-token and token-by-token window kernels): q points at
    // the pre-convolution rows [B, (T,) H, 2 dk + dv] (q | k | v channels), k and v are
    // unused
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
    const int32_t *accept;     // device [B] or NULL (all T tokens accepted; none with a replay)
    int32_t B, T, H, dk, dv;
    bool bf16;
    void *stream;
    DecodeFusion fx;
    // Replay before the window: the previous window's inputs ([B, Tp, H, .]) and, per
    // sequence, how many of its tokens were accepted (replayed and committed first).
    const void *pq = nullptr, *pk = nullptr, *pv = nullptr, *pg = nullptr, *pbeta = nullptr;
    const int32_t *replay = nullptr;
    int32_t Tp = 0;
    int32_t acc_default = -1;  // tokens of this window committed without accept (-1: all T)
    // Evaluation form: 0 automatic, 1 token by token (vector ALUs), 2 the window as one
    // chunk on the matrix cores (decode_chunk.hip).
    int32_t form = 0;
};

// Shapes the one-chunk window form serves: bf16, dk = dv = 128 (with or without the gate
// from logits), no ShortConv prologue, and the window's tokens (with a replay in front)
// within one 16-token chunk.
inline bool window_chunk_supported(const DecodeWindowArgs &a) {
    const int64_t tokens = (int64_t)a.T + (a.replay ? a.Tp : 0);
    return a.bf16 && a.dk == 128 && a.dv == 128 && !a.fx.conv_w && a.T >= 1 && tokens <= 16;
}

// Calls of this many tokens per (sequence, head) on (the window's, plus the replay's at
// most) go through the one-chunk form where it serves the shape: below it the
// token-by-token kernel's arithmetic hides behind its state traffic (B=256 x H=96:
// 0.58 against 0.63 ms at 4 tokens, 0.74 against 0.68 at 6, 0.99 against 0.68 at 8).
constexpr int WINDOW_CHUNK_MIN_TOKENS = 6;

// The layer's window (fx.conv_w set: pre-convolution q | k | v rows) in the one-chunk form:
// a prologue pass writes the chunk kernel's inputs to a workspace of
// layer_window_chunk_bytes(B, T, Tp, H) bytes (decode_chunk.hip).
inline bool layer_window_chunk_supported(const DecodeWindowArgs &a) {
    const int64_t tokens = (int64_t)a.T + (a.replay ? a.Tp : 0);
    return a.bf16 && a.dk == 128 && a.dv == 128 && a.fx.conv_w && a.fx.conv_cache && a.T >= 1 && tokens <= 16;
}
size_t layer_window_chunk_bytes(int64_t B, int64_t T, int64_t Tp, int64_t H);
hipError_t launch_layer_window_chunk(const DecodeWindowArgs &a, void *ws);

// The fused layer prefill's prologue on load (layer_prologue.hpp): what the two
// prefill kernels need besides their usual inputs.
struct LayerPrologue {
    const float *conv_w;  // fp32 [H, 2 dk + dv, 4], tap j multiplies x_{t-j}; channels q, k, v
    const float *cache;   // fp32 [nseq, H, 2 dk + dv, 3]: the 3 inputs before each sequence, oldest first; NULL = 0
    const float *A_log;   // fp32 [H]
    void *qkg;            // bf16 [3, N, H, dk]: the prologue's q, k and log-decay, written by the
                          // chunk-local pass for the inter-chunk pass
    float l2_eps;
    int32_t cw;           // 2 dk + dv: channels per head of conv_w and cache
    int64_t n_tokens;     // N (the planes of qkg)
};

struct ChunkLocalArgs {
    const void *q, *k, *g, *beta;
    const int32_t *cu;
    int32_t nseq, H, dk;
    int64_t total_tokens;
    bool bf16;
    float *ws;
    void *stream;
    const LayerPrologue *layer = nullptr;  // fused layer prologue on load (bf16, dk = 128), or none
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
    int32_t ws_consumers, ws_producers;  // warp-specialised kernel shape; 0, 0 = choose automatically
    void *stream;
    const LayerPrologue *layer = nullptr;  // fused layer prologue on load (bf16, dk = dv = 128), or none
    const int32_t *skip = nullptr;         // per chain (s * H + h): nonzero = leave that chain untouched
};

// Single-pass prefill (prefill_fused.hip): bf16 inputs, dk = dv = 128, many chains; no workspace.
struct PrefillFusedArgs {
    const void *q, *k, *v, *g, *beta;
    const float *init;
    const int32_t *cu;
    int32_t nseq, H, dk, dv;
    bool bf16;
    float *o, *fin;
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
// Only the chunk matrices and the forward sweep of the backward (fp32), which also writes the
// state after each sequence to fin; the workspace is that of launch_backward.
hipError_t launch_backward_states(const BackwardArgs &a, float *fin);
// Per-slab {0, length} sequence lists (2 int32 per slab) of a slabbed backward.
hipError_t launch_backward_slab_cu(int32_t *cu, int64_t N, int64_t L, int32_t nslab, void *stream);
int64_t backward_workspace_floats(int64_t N, int32_t nseq, int32_t H, int32_t dk, int32_t dv);

// Intra-device context parallelism (cp.hip): the small kernels around the prefill passes.
hipError_t launch_cp_segments(const int32_t *cu, int32_t nseq, int32_t R, int32_t *cu_seg, void *stream);
hipError_t launch_cp_identity(float *M, int64_t n_mats, int32_t dk, void *stream);
// Per (segment, head): nonzero when the bound on the segment's transition, ||M||_2 <=
// prod_t max_i alpha_t,i max(1, |1 - beta_t ||k_t||^2|), is below 2^-30.
hipError_t launch_cp_bound(const void *k, const void *g, const void *beta, const int32_t *cu_seg, int32_t nseg,
                           int32_t H, int32_t dk, bool bf16, int32_t *flags, void *stream);
hipError_t launch_cp_scan(const float *init, const float *M, const float *St, const int32_t *skip, float *Sin,
                          int32_t nseq, int32_t H, int32_t dk, int32_t dv, int32_t R, void *stream);
hipError_t launch_cp_final(const float *Sin, float *fin, int32_t nseq, int32_t H, int32_t dk, int32_t dv, int32_t R,
                           void *stream);

bool prefill_fused_supported(int dk, int dv, bool bf16, int64_t chains);
// consumers nc with sl 16-column slices each; (0, 0) = choose from the number of chains;
// hipErrorInvalidValue for a shape that is not built
hipError_t launch_prefill_fused(const PrefillFusedArgs &a, int nc, int sl);
bool prefill_fused_shape_built(int nc, int sl);
bool inter_chunk_ws_shape_built(int dk, int dv, int ncw, int npw);

hipError_t launch_gate(const GateArgs &a);
// The combined q | k | v convolution cache after a fused layer prefill (bf16 inputs).
hipError_t launch_layer_conv_cache(const void *q, const void *k, const void *v, const float *cache_in,
                                   float *cache_out, const int32_t *cu, int32_t nseq, int32_t H, int32_t dk,
                                   int32_t dv, void *stream);
hipError_t launch_short_conv(const ShortConvArgs &a);
hipError_t launch_out_norm_gate(const OutNormGateArgs &a);
hipError_t launch_decode(const DecodeArgs &a);
hipError_t launch_decode_window(const DecodeWindowArgs &a);
hipError_t launch_window_chunk(const DecodeWindowArgs &a);
hipError_t launch_check_cu_seqlens(const int32_t *cu, int32_t nseq, int64_t N, int32_t *result, void *stream);
hipError_t launch_chunk_local(const ChunkLocalArgs &a);
hipError_t launch_inter_chunk(const InterChunkArgs &a);
// Warp-specialised inter-chunk kernel (bf16, dk >= 32): ncw consumer and npw
// producer waves per workgroup; hipErrorInvalidValue for a shape not built.
hipError_t launch_inter_chunk_ws(const InterChunkArgs &a, int ncw, int npw);

}  // namespace kda
