// prefill.hip -- dispatch of the chunked prefill on gfx950.
//
// Source: "On the Design of Qwen3.8-Next Architecture", picx.dev summary,
// "Theoretical foundations", eqs (1)-(4).  The pages give only the token-by-
// token recurrence; the chunk form the kernels compute is derived from it.
// For one chunk of C tokens r = 1..C entering with state S (Dk x Dv):
//
//   g_r = log2 alpha_r,  G_r = g_1 + ... + g_r,  Gamma_rj = 2^(G_r - G_j) (r >= j)
//   A = strict_lower[ beta_r Gamma_rj (k_r . k_j) ],  T = (I + A)^-1
//   U = T diag(beta) (V - diag(2^G) K S)       (u_r = beta_r e_r of eqs (2)-(3))
//   Y = diag(2^G) Q S + P U,  P = lower_incl[ Gamma_rj (q_r . k_j) ]   (eq (4))
//   S' = 2^{G_C} S + K^T diag(2^{G_C - G}) U                          (eqs (1),(3))
//
// bf16 inputs with a workspace: the chunk quantities of every (b, h, chunk) in
// parallel into per-chunk records (chunk_prep.hip), then the recurrence
// reading them (recurrence.hip).  bf16 inputs without one: a single kernel
// (prefill_fused.hip) that forms every chunk quantity on chip and reads q, k,
// v once.  fp32 inputs (and the layer's core): the per-chunk preparation of
// backward.hip into a caller-provided record workspace, then the recurrence.
// Ragged tails are padded with identity tokens (alpha = 1, beta = 0,
// k = q = v = 0).
#include "common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

// T == 0: the final state is the initial state (or zero).
__global__ void copy_or_zero_state(const float *__restrict__ s0, float *__restrict__ sT, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) sT[i] = s0 ? s0[i] : 0.f;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream)
{
    if (a.B * a.H == 0) return hipSuccess;
    if (a.T == 0) {
        if (!a.sT || a.sT == a.s0) return hipSuccess;
        const int64_t n = a.B * a.H * a.Dk * a.Dv;
        hipLaunchKernelGGL(copy_or_zero_state, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a.s0, a.sT, n);
        return hipGetLastError();
    }
    if (a.bf16) {
        if (!a.ws) return launch_prefill_fused(a, stream);
        const hipError_t e = launch_chunk_prep(a, stream);
        return e != hipSuccess ? e : launch_recurrence(a, stream);
    }
    if (!a.ws) return hipErrorInvalidValue;   // the C ABI checks the workspace first
    return launch_prefill_f32_staged(a, stream);
}

}  // namespace gdn
