// launch.hpp -- internal host-side launch interface between the C ABI
// (api.cpp, which validates) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

struct DecodeArgs {
    const void *q, *k, *v;
    const float *alpha, *beta;
    float *state, *y;
    int64_t N, H, Dk, Dv;
    bool bf16;
    // elements between consecutive sequences of q, k, v; 0: dense [N, H, D]
    int64_t q_seq_stride = 0, k_seq_stride = 0, v_seq_stride = 0;
};

// Prefill over [B, T, H, *] tensors.  Row strides (elements between
// consecutive tokens) are explicit so that q/k/v may live inside a wider
// fused buffer (the layer passes slices of its in-projection output).
struct PrefillArgs {
    const void *q, *k, *v;
    const float *alpha, *beta;      // [B, T, H]
    const float *s0;                // [B, H, Dk, Dv] or null
    float *y;                       // [B, T, H, Dv]
    float *sT;                      // [B, H, Dk, Dv] or null
    int64_t B, T, H, Dk, Dv, chunk;
    int64_t q_tok_stride, k_tok_stride, v_tok_stride;   // elements per token (all heads)
    bool bf16;
    // fp32: prefill_f32_workspace_bytes(...) bytes, 256-byte aligned; bf16:
    // prefill_bf16_workspace_bytes(...) bytes for the two-kernel form, or null
    // for the single fused kernel
    void *ws;
    // fp32 inputs: the caller's bound is the bf16 one (the layer's core), so the
    // recurrence may run on bf16 MFMA with hi/lo operands (about 16 bits of each
    // operand) instead of fp32 MFMA
    bool hilo_core = false;
    // An independent product C = A B^T (bf16, [M, K] x [N, K] -> [M, N] bf16)
    // that the hi/lo recurrence runs in its own launch, on the compute units its
    // slices leave free; null: none.  prefill_f32_takes_side() says whether the
    // recurrence will take it; if not, the caller runs it itself.
    struct SideGemm {
        const __bf16 *A, *B;
        __bf16 *C;
        int64_t M, N, K, lda, ldb, ldc;
    };
    const SideGemm *side = nullptr;
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

// T tokens per sequence from stored states, every intermediate state written
struct VerifyArgs {
    const void *q, *k, *v;          // [N, T, H, Dk], [N, T, H, Dv]
    const float *alpha, *beta;      // [N, T, H]
    const float *s_in;              // [N, H, Dk, Dv]
    float *s_out;                   // [N, T, H, Dk, Dv]
    float *y;                       // [N, T, H, Dv]
    int64_t N, T, H, Dk, Dv;
    bool bf16;
};
hipError_t launch_verify(const VerifyArgs &a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

// bf16 prefill in one kernel (prefill_fused.hip): chunk quantities formed on chip
hipError_t launch_prefill_fused(const PrefillArgs &a, hipStream_t stream);

// bf16 prefill in two kernels: the state-independent chunk quantities of every
// (b, h, chunk) into per-chunk records (chunk_prep.hip, prep_layout.hpp), then
// the recurrence over 16-column slices reading them (recurrence.hip)
size_t prefill_bf16_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t chunk);
hipError_t launch_chunk_prep(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_recurrence(const PrefillArgs &a, hipStream_t stream);

// Gradients of the prefill (backward.hip): dL/dq, dk, dv, dalpha, dbeta, dS_0
// from dL/dy and dL/dS_T
struct BwdArgs {
    const void *q, *k, *v;          // [B, T, H, Dk], [B, T, H, Dv]
    const float *alpha, *beta;      // [B, T, H]
    const float *s0;                // [B, H, Dk, Dv] or null
    const float *dy;                // [B, T, H, Dv]
    const float *dsT;               // [B, H, Dk, Dv] or null
    float *dq, *dk, *dv, *dalpha, *dbeta;
    float *ds0;                     // [B, H, Dk, Dv] or null
    int64_t B, T, H, Dk, Dv, chunk;
    bool bf16;
    void *ws;                       // prefill_bwd_workspace_bytes(...) bytes, 256-byte aligned
};
int64_t bwd_record_floats(int64_t C);
size_t prefill_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int64_t C);
hipError_t launch_prefill_bwd(const BwdArgs &a, hipStream_t stream);

// fp32 prefill in two kernels (backward.hip): per-chunk preparation into a
// record workspace of prefill_f32_workspace_bytes(...) bytes (a.ws), then the
// state recurrence writing y; q, k, v with token strides
size_t prefill_f32_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t C);
hipError_t launch_prefill_f32_staged(const PrefillArgs &a, hipStream_t stream);
bool prefill_f32_takes_side(const PrefillArgs &a);

// Layer helpers (layer.hip)
struct LayerArgs {
    const void *x;
    const void *W_qkv, *conv_w, *W_ab, *W_gate, *W_o;
    const float *A, *b_alpha, *norm_gamma;
    const float *s0;
    float *sT;
    float *out;
    int64_t B, T, hidden, H, Dk, Dv, conv_k, chunk;
    void *ws;
};
size_t layer_workspace_bytes(int64_t B, int64_t T, int64_t hidden, int64_t H, int64_t Dk, int64_t Dv);
size_t layer_decode_workspace_bytes(int64_t N, int64_t H, int64_t Dk, int64_t Dv);
// the library's own scratch for the allocation-free decode step (layer.hip)
size_t layer_decode_scratch_bytes();
hipError_t layer_decode_scratch(void **out);
hipError_t launch_layer(const LayerArgs &a, hipStream_t stream);

// One token of the layer for N sequences: x [N, hidden]; conv_state [N, conv_k-1,
// H(2Dk+Dv)] and state [N, H, Dk, Dv] updated in place; out [N, hidden]
struct LayerDecodeArgs {
    const void *x;
    const void *W_qkv, *conv_w, *W_ab, *W_gate, *W_o;
    const float *A, *b_alpha, *norm_gamma;
    float *conv_state, *state, *out;
    int64_t N, hidden, H, Dk, Dv, conv_k;
    void *ws;
};
hipError_t launch_layer_decode(const LayerDecodeArgs &a, hipStream_t stream);

}  // namespace gdn
