/*
 * gdn.h -- C ABI of libgdn.so, the MI355X (gfx950) Gated DeltaNet token mixer.
 *
 * The gated delta rule (source: "On the Design of Qwen3.8-Next Architecture",
 * picx.dev summary page, section "Theoretical foundations", eqs (1)-(4)): per
 * (sequence, head), with state S in R^{Dk x Dv}, decay alpha_t and write
 * strength beta_t,
 *
 *     S~ = alpha_t S_{t-1};  e_t = v_t - S~^T k_t;
 *     S_t = S~ + beta_t k_t e_t^T;  y_t = S_t^T q_t.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer on the current HIP device, to a
 *   dense row-major (last index fastest) buffer, 16-byte aligned.
 * - The caller allocates and frees every buffer.  The library's own state is
 *   a thread-local error string and the scratch array of
 *   gdn_layer_decode_step_noalloc (32 MiB per GPU, part of the code object,
 *   its address looked up once per device under a lock).  Every entry point
 *   other than that one is reentrant.
 * - Calls enqueue work on `stream` and return without synchronising.  A device
 *   fault shows up at the caller's next synchronisation.  With GDN_SYNC_CHECK=1
 *   in the environment (a debugging aid) every call waits for its stream and
 *   returns GDN_ERR_HIP, naming the entry point, if a kernel failed.
 * - Arguments are validated on the host before any HIP call: on a non-OK
 *   status nothing has been launched and no output has been touched.
 *   gdn_last_error() then holds a one-line description.
 * - Value domains are preconditions, not checked on the device:
 *   alpha in [0, 1] for the forward entry points (the pages give the open
 *   interval (0,1); alpha = 1 is accepted as an exact identity decay, and an
 *   alpha below 2^-126 -- zero or subnormal -- acts as 2^-126, which leaves
 *   less than 1.2e-38 of the state), alpha in (0, 1] for gdn_prefill_bwd,
 *   beta in [0, 1], all inputs finite.
 * - Outputs y, out and final_state are always float32.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_API __attribute__((visibility("default")))

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,        /* a required pointer is NULL                      */
    GDN_ERR_SHAPE = 2,       /* a size is negative or the sizes overflow        */
    GDN_ERR_UNSUPPORTED = 3, /* a size/dtype/chunk outside the compiled set     */
    GDN_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                */
    GDN_ERR_ALIAS = 5,       /* an output overlaps an input it must not overlap */
    GDN_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required      */
    GDN_ERR_HIP = 7          /* a HIP runtime call failed (see gdn_last_error)  */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/*
 * gdn_prefill_fwd -- whole sequences through eqs (1)-(4), computed chunk by
 * chunk (C tokens at a time) with the state carried across chunks.
 *
 *   q, k          [B, T, H, Dk]  dtype (GDN_F32: float, GDN_BF16: bf16 bits)
 *   v             [B, T, H, Dv]  dtype
 *   alpha, beta   [B, T, H]      float32 (eq (1) decay, eq (3) write strength)
 *   initial_state [B, H, Dk, Dv] float32, or NULL for S_0 = 0
 *   y             [B, T, H, Dv]  float32 output, y_t of eq (4)
 *   final_state   [B, H, Dk, Dv] float32 output S_T, or NULL if not wanted;
 *                 may be the same pointer as initial_state (in-place resume),
 *                 must not overlap it otherwise.
 *   chunk         C in {16, 32, 64}; Dk, Dv in {16, 32, 64, 128}.
 *   B, H, T >= 0; B*H == 0 or T == 0 launch nothing except, for T == 0,
 *   final_state = initial_state (or zeros).  Any T is accepted: a ragged last
 *   chunk is padded with identity tokens (alpha = 1, beta = 0, k = q = v = 0).
 *   workspace     device scratch of at least gdn_prefill_workspace_bytes(...)
 *                 bytes, 256-byte aligned, owned by the caller and not
 *                 overlapping any other argument: one record per (sequence,
 *                 head, chunk) of the quantities that do not depend on the
 *                 state, computed for every chunk in parallel by a separate
 *                 kernel before the recurrence.  GDN_BF16: the decay prefix,
 *                 decay factors and (I + A)^-1 diag(beta) as bf16 hi/lo MFMA
 *                 fragments (11072 bytes at C = 64; the recurrence forms the
 *                 masked Q K^T block itself); optional:
 *                 NULL selects one kernel that forms every chunk quantity on
 *                 chip and reads q, k, v from memory once (no scratch, less
 *                 memory traffic, longer per-chunk period).  GDN_F32:
 *                 required; (I + A)^-1, P, the masked K K^T, the decay prefix
 *                 and 2^(G_C - G) (49664 bytes at C = 64).  Given but too
 *                 small, or missing where required: GDN_ERR_WORKSPACE.  Its
 *                 contents are overwritten; nothing in it is kept between
 *                 calls.
 * y must not overlap q, k, v, alpha, beta, initial_state or final_state.
 */
GDN_API gdn_status gdn_prefill_fwd(const void *q, const void *k, const void *v,
                           const float *alpha, const float *beta,
                           const float *initial_state,
                           float *y, float *final_state,
                           int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                           int64_t chunk, gdn_dtype dtype,
                           void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Bytes of workspace gdn_prefill_fwd takes for these sizes: B*H*ceil(T/C)
 * records of the dtype's layout; 0 for empty problems and for arguments
 * gdn_prefill_fwd would reject. */
GDN_API size_t gdn_prefill_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                   int64_t Dv, int64_t chunk, gdn_dtype dtype);

/*
 * gdn_prefill_bwd -- gradients of gdn_prefill_fwd: the reverse mode of eqs
 * (1)-(4) ("Theoretical foundations" of the picx.dev summary of "On the Design
 * of Qwen3.8-Next Architecture") for a scalar loss L, given dL/dy of every
 * token and dL/dS_T.  Computed chunk by chunk: the states entering every chunk
 * are recomputed, the state gradient is carried backwards over the chunks, and
 * each chunk's token gradients follow from those two boundary values.
 *
 *   q, k, v, alpha, beta, initial_state   as in gdn_prefill_fwd (the inputs
 *                 of the forward call whose gradients are wanted)
 *   dy            [B, T, H, Dv]  float32, dL/dy
 *   dfinal_state  [B, H, Dk, Dv] float32, dL/dS_T, or NULL for zero
 *   dq, dk        [B, T, H, Dk]  float32 outputs
 *   dv            [B, T, H, Dv]  float32 output
 *   dalpha, dbeta [B, T, H]      float32 outputs
 *   dinitial_state [B, H, Dk, Dv] float32 output dL/dS_0, or NULL if not wanted
 *                 (written also when initial_state is NULL: the gradient at S_0 = 0)
 *   chunk in {16, 32, 64}; Dk, Dv in {16, 32, 64, 128}; B, T, H >= 0.
 *   workspace     at least gdn_prefill_bwd_workspace_bytes(...) bytes,
 *                 256-byte aligned, caller-owned: one record per (sequence,
 *                 head, chunk) holding (I + A)^-1, the masked Q K^T and K K^T
 *                 blocks and the decay prefix (3C^2 + C floats, rounded up to
 *                 64), the state entering and the state gradient leaving
 *                 every chunk (Dk Dv floats each), and the chunk's U,
 *                 V - diag(e^G) K S and dX (C Dv floats each); 0.57 GB for
 *                 B=2, T=4096, H=16, d=128, C=64 and 4.6 GB for B=1,
 *                 T=32768, H=32.  Overwritten; nothing kept between calls.
 * Every output must not overlap any input, another output or the workspace.
 * T == 0 writes dinitial_state = dfinal_state (or zeros) and nothing else.
 * Precision: every product accumulates in fp32.  For bf16 inputs all four
 * kernels multiply on bf16 MFMA, with every operand that is not an input
 * (states, T, P, the chunk matrices, the gradients) split into a bf16 pair
 * hi + lo; for fp32 inputs the products run on fp32 MFMA.
 */
GDN_API size_t gdn_prefill_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                               int64_t Dv, int64_t chunk);
GDN_API gdn_status gdn_prefill_bwd(const void *q, const void *k, const void *v,
                                   const float *alpha, const float *beta,
                                   const float *initial_state, const float *dy,
                                   const float *dfinal_state, float *dq, float *dk, float *dv,
                                   float *dalpha, float *dbeta, float *dinitial_state,
                                   int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                   int64_t chunk, gdn_dtype dtype, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * gdn_decode_step -- one new token for each of N independent sequences: the
 * single-token form of eqs (1)-(4) applied to a stored state, updated in place
 * (the fixed-size state that summarises the prefix).
 *
 *   q, k         [N, H, Dk]      dtype
 *   v            [N, H, Dv]      dtype
 *   alpha, beta  [N, H]          float32
 *   state        [N, H, Dk, Dv]  float32, read and overwritten in place
 *   y            [N, H, Dv]      float32 output
 *   Dk, Dv in {16, 32, 64, 128}; N, H >= 0 (N*H == 0 launches nothing).
 * y must not overlap any input or the state.
 */
GDN_API gdn_status gdn_decode_step(const void *q, const void *k, const void *v,
                           const float *alpha, const float *beta,
                           float *state, float *y,
                           int64_t N, int64_t H, int64_t Dk, int64_t Dv,
                           gdn_dtype dtype, hipStream_t stream);

/*
 * gdn_decode_verify -- T consecutive tokens of each of N sequences from their
 * stored states, eqs (1)-(4) token by token (T calls of gdn_decode_step, in
 * one launch), with the state after every token written out: a caller that
 * checks drafted tokens keeps the state after the prefix it accepts.
 *
 *   q, k        [N, T, H, Dk]  dtype
 *   v           [N, T, H, Dv]  dtype
 *   alpha, beta [N, T, H]      float32
 *   state       [N, H, Dk, Dv] float32, the states before the first token (read only)
 *   states_out  [N, T, H, Dk, Dv] float32: [:, t] is the state after token t
 *   y           [N, T, H, Dv]  float32
 *   Dk, Dv in {16, 32, 64, 128}.  states_out and y must not overlap each
 *   other or any input; state is not modified.
 */
GDN_API gdn_status gdn_decode_verify(const void *q, const void *k, const void *v,
                                     const float *alpha, const float *beta,
                                     const float *state, float *states_out, float *y,
                                     int64_t N, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                     gdn_dtype dtype, hipStream_t stream);

/*
 * gdn_layer_fwd -- the GDN token-mixing layer around the core (picx.dev
 * summary, "1. GDN Hybrid Token Mixing": short causal convolution, L2-normalised
 * queries and keys, eq (9) beta, eq (10) alpha, eq (11) sigmoid-gated
 * zero-centred RMSNorm and output projection):
 *
 *   [q|k|v] = conv(x W_qkv^T);  a = x W_a^T;  b = x W_b^T;  z = x W_gate^T
 *   q, k <- q / sqrt(|q|^2 + 1e-6) per (token, head)
 *   alpha = exp(-exp(A) softplus(a + b_alpha));  beta = sigmoid(b)
 *   y = core(q, k, v, alpha, beta; initial_state)
 *   out = (sigmoid(z) * y / sqrt(mean(y^2) + 1e-6) * (1 + norm_gamma)) W_o^T
 *
 * conv is depthwise and causal over the H*(2Dk+Dv) q|k|v channels,
 * out[t,c] = sum_j conv_w[c,j] * in[t-(conv_k-1)+j, c] (zero history, no bias,
 * no activation).  RMSNorm runs per (token, head) over Dv.
 *
 * The four projections are plain products on this library's GEMM kernel
 * (bf16 operands, fp32 accumulation, every output summed over K in one order
 * whatever the number of rows).
 *
 *   x     [B, T, hidden] bf16;  out [B, T, hidden] float32
 *   initial_state / final_state as in gdn_prefill_fwd (NULL allowed).
 *   hidden % 64 == 0; conv_k in [1, 4]; Dk, Dv, chunk as in gdn_prefill_fwd.
 *   workspace: at least gdn_layer_workspace_bytes(...) bytes, 256-byte aligned.
 */
typedef struct {
    const void  *W_qkv;      /* [H*(2Dk+Dv), hidden] bf16; rows q | k | v, head-major */
    const void  *conv_w;     /* [H*(2Dk+Dv), conv_k] bf16; tap conv_k-1 = current token */
    const void  *W_ab;       /* [2H, hidden] bf16; rows a (eq (10)) | b (eq (9))        */
    const float *A;          /* [H] eq (10) log-scale of the decay rate                 */
    const float *b_alpha;    /* [H] eq (10) bias                                        */
    const void  *W_gate;     /* [H*Dv, hidden] bf16 (W_z of eq (11))                    */
    const float *norm_gamma; /* [Dv] zero-centred RMSNorm gain: scale = 1 + gamma       */
    const void  *W_o;        /* [hidden, H*Dv] bf16                                     */
} gdn_layer_params;

GDN_API gdn_status gdn_layer_fwd(const void *x, const gdn_layer_params *p,
                         const float *initial_state, float *final_state, float *out,
                         int64_t B, int64_t T, int64_t hidden, int64_t H,
                         int64_t Dk, int64_t Dv, int64_t conv_k, int64_t chunk,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

GDN_API size_t gdn_layer_workspace_bytes(int64_t B, int64_t T, int64_t hidden, int64_t H,
                                 int64_t Dk, int64_t Dv, int64_t conv_k, int64_t chunk);

/*
 * gdn_layer_decode_step -- one new token of gdn_layer_fwd for each of N
 * sequences, carrying the layer's two pieces of history: the short
 * convolution's last conv_k-1 inputs and the recurrent state of eqs (1)-(4)
 * (same page and formulas as gdn_layer_fwd, at T = 1 with the history given).
 * Running it T times from a zero history gives gdn_layer_fwd on the T tokens.
 *
 *   x          [N, hidden] bf16: the new token of each sequence
 *   p          as in gdn_layer_fwd
 *   conv_state [N, conv_k-1, H*(2Dk+Dv)] float32, in place: the in-projection
 *              rows x W_qkv^T of the previous conv_k-1 tokens, oldest first
 *              (zeros before a sequence starts); shifted by one token and the
 *              new row appended.  May be NULL when conv_k == 1.
 *   state      [N, H, Dk, Dv] float32, in place: S_{t-1} -> S_t
 *   out        [N, hidden] float32
 *   hidden % 64 == 0; conv_k in [1, 4]; Dk, Dv in {16, 32, 64, 128}.
 *   workspace: at least gdn_layer_decode_workspace_bytes(...) bytes, 256-byte
 *   aligned.  out must not overlap any input, state or conv_state; state and
 *   conv_state must not overlap each other or the inputs.
 */
GDN_API gdn_status gdn_layer_decode_step(const void *x, const gdn_layer_params *p,
                                         float *conv_state, float *state, float *out,
                                         int64_t N, int64_t hidden, int64_t H, int64_t Dk,
                                         int64_t Dv, int64_t conv_k, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream);

GDN_API size_t gdn_layer_decode_workspace_bytes(int64_t N, int64_t hidden, int64_t H,
                                                int64_t Dk, int64_t Dv);

/*
 * gdn_layer_decode_step_noalloc -- gdn_layer_decode_step without a workspace,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Arguments,
 * layouts, in-place updates, results and errors are those of
 * gdn_layer_decode_step; the call allocates nothing, in the library or in HIP.
 * The intermediates live in one 32 MiB scratch array that the library holds on
 * each GPU it runs on until the process ends; a size for which
 * gdn_layer_decode_workspace_bytes() exceeds 32 MiB fails with
 * GDN_ERR_WORKSPACE.  Every call on a GPU shares that GPU's array and writes
 * all of it that it reads, so nothing needs clearing between calls, but two
 * calls that overlap in time on one GPU (other streams, other host threads)
 * race on it and give undefined results.
 */
GDN_API gdn_status gdn_layer_decode_step_noalloc(const void *x, const gdn_layer_params *p,
                                                 float *conv_state, float *state, float *out,
                                                 int64_t N, int64_t hidden, int64_t H, int64_t Dk,
                                                 int64_t Dv, int64_t conv_k, hipStream_t stream);

/* Static description of a status code. */
GDN_API const char *gdn_status_str(gdn_status s);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
GDN_API const char *gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
