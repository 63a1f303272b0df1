// api.cpp -- C ABI of libgdn.so: argument validation and dispatch.
//
// Every check runs on the host before any HIP call, so an invalid call
// launches nothing and leaves every output untouched.
#include <cstdlib>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/gdn.h"
#include "launch.hpp"
#include "prep_layout.hpp"

namespace {

thread_local char g_err[512] = "";

gdn_status fail(gdn_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

gdn_status ok()
{
    g_err[0] = '\0';
    return GDN_OK;
}

bool is_pow2_dim(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// overflow-checked product of non-negative sizes
bool mul_ok(int64_t a, int64_t b, int64_t *out)
{
    if (a == 0 || b == 0) { *out = 0; return true; }
    if (a > INT64_MAX / b) return false;
    *out = a * b;
    return true;
}

bool count(int64_t *out, std::initializer_list<int64_t> dims)
{
    int64_t n = 1;
    for (int64_t d : dims)
        if (!mul_ok(n, d, &n)) return false;
    *out = n;
    return true;
}

struct Range {
    const void *p;
    size_t bytes;
    const char *name;
};

bool overlap(const Range &a, const Range &b)
{
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// The status of a launch.  With GDN_SYNC_CHECK=1 in the environment (a
// debugging aid) the call also waits for the stream and reports any error the
// kernels raised, naming the entry point; otherwise it returns at once.
gdn_status hip_status(hipError_t e, const char *what, hipStream_t stream)
{
    if (e == hipSuccess) {
        const char *sync = getenv("GDN_SYNC_CHECK");
        if (!(sync && sync[0] == '1')) return ok();
        e = hipStreamSynchronize(stream);
        if (e == hipSuccess) e = hipGetLastError();
        if (e == hipSuccess) return ok();
    }
    return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char *gdn_status_str(gdn_status s)
{
    switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL: required pointer is NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: negative or overflowing size";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: size, chunk or dtype not compiled";
    case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: pointer not 16-byte aligned";
    case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS: output overlaps an input";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: HIP runtime error";
    }
    return "unknown gdn_status";
}

const char *gdn_last_error(void) { return g_err; }

size_t gdn_prefill_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int64_t chunk,
                                   gdn_dtype dtype)
{
    if (B <= 0 || T <= 0 || H <= 0 || (dtype != GDN_F32 && dtype != GDN_BF16) || !is_pow2_dim(Dk) ||
        !is_pow2_dim(Dv) || (chunk != 16 && chunk != 32 && chunk != 64))
        return 0;        // nothing for empty or rejected problems
    int64_t n;
    if (dtype == GDN_BF16) {
        if (!count(&n, {B, H, (T + chunk - 1) / chunk, (int64_t)gdn::prep_record_bytes(chunk)})) return 0;
        return gdn::prefill_bf16_workspace_bytes(B, T, H, chunk);
    }
    if (!count(&n, {B, H, (T + chunk - 1) / chunk, gdn::bwd_record_floats(chunk), 4})) return 0;
    return gdn::prefill_f32_workspace_bytes(B, T, H, chunk);
}

namespace {

gdn_status prefill_impl(const char *fn, const void *q, const void *k, const void *v,
                        const float *alpha, const float *beta, const float *initial_state, float *y,
                        float *final_state, int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                        int64_t chunk, gdn_dtype dtype, void *workspace, size_t workspace_bytes,
                        hipStream_t stream)
{
    if (B < 0 || T < 0 || H < 0 || Dk < 0 || Dv < 0 || chunk < 0)
        return fail(GDN_ERR_SHAPE, "%s: negative size (B=%lld T=%lld H=%lld Dk=%lld Dv=%lld chunk=%lld)", fn,
                    (long long)B, (long long)T, (long long)H, (long long)Dk, (long long)Dv, (long long)chunk);
    if (dtype != GDN_F32 && dtype != GDN_BF16)
        return fail(GDN_ERR_UNSUPPORTED, "%s: dtype %d", fn, (int)dtype);
    if (!is_pow2_dim(Dk) || !is_pow2_dim(Dv))
        return fail(GDN_ERR_UNSUPPORTED, "%s: Dk=%lld Dv=%lld (supported: 16, 32, 64, 128)", fn,
                    (long long)Dk, (long long)Dv);
    if (chunk != 16 && chunk != 32 && chunk != 64)
        return fail(GDN_ERR_UNSUPPORTED, "%s: chunk=%lld (supported: 16, 32, 64)", fn, (long long)chunk);
    int64_t n_tok, n_qk, n_v, n_s;
    if (!count(&n_tok, {B, T, H}) || !count(&n_qk, {B, T, H, Dk}) || !count(&n_v, {B, T, H, Dv}) ||
        !count(&n_s, {B, H, Dk, Dv}) || n_qk > INT64_MAX / 4 || n_v > INT64_MAX / 4)
        return fail(GDN_ERR_SHAPE, "%s: sizes overflow", fn);
    if (B * H > (int64_t)1 << 26 || (B * H) * (Dv / 16) > INT32_MAX)
        return fail(GDN_ERR_UNSUPPORTED, "%s: B*H=%lld too large for one launch", fn, (long long)(B * H));
    // bf16 chunks are copied with 32-bit byte offsets within one chunk of rows
    if (dtype == GDN_BF16 && chunk * H * (Dk > Dv ? Dk : Dv) * 2 >= ((int64_t)1 << 31))
        return fail(GDN_ERR_UNSUPPORTED, "%s: H=%lld too large for bf16 (chunk * H * max(Dk, Dv) * 2 must stay below 2^31)", fn,
                    (long long)H);
    if (n_tok > 0 && (!q || !k || !v || !alpha || !beta || !y))
        return fail(GDN_ERR_NULL, "%s: q, k, v, alpha, beta and y are required", fn);
    const void *ptrs[] = {q, k, v, alpha, beta, initial_state, y, final_state};
    const char *names[] = {"q", "k", "v", "alpha", "beta", "initial_state", "y", "final_state"};
    for (int i = 0; i < 8; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(GDN_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, names[i]);
    const size_t esz = dtype == GDN_BF16 ? 2 : 4;
    const Range ry{y, (size_t)n_v * 4, "y"};
    const Range inputs[] = {{q, (size_t)n_qk * esz, "q"}, {k, (size_t)n_qk * esz, "k"},
                            {v, (size_t)n_v * esz, "v"}, {alpha, (size_t)n_tok * 4, "alpha"},
                            {beta, (size_t)n_tok * 4, "beta"}, {initial_state, (size_t)n_s * 4, "initial_state"},
                            {final_state, (size_t)n_s * 4, "final_state"}};
    for (const Range &r : inputs)
        if (overlap(ry, r)) return fail(GDN_ERR_ALIAS, "%s: y overlaps %s", fn, r.name);
    const Range rs{final_state, (size_t)n_s * 4, "final_state"};
    for (int i = 0; i < 5; ++i)
        if (overlap(rs, inputs[i])) return fail(GDN_ERR_ALIAS, "%s: final_state overlaps %s", fn, inputs[i].name);
    if (final_state != initial_state && overlap(rs, inputs[5]))
        return fail(GDN_ERR_ALIAS, "%s: final_state partially overlaps initial_state", fn);
    // bf16: the workspace is optional (none selects the single fused kernel)
    const size_t need = dtype == GDN_BF16 && !workspace ? 0 : gdn_prefill_workspace_bytes(B, T, H, Dk, Dv, chunk, dtype);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                        workspace ? workspace_bytes : (size_t)0);
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(GDN_ERR_ALIGN, "%s: workspace is not 256-byte aligned", fn);
        const Range rw{workspace, need, "workspace"};
        if (overlap(rw, ry)) return fail(GDN_ERR_ALIAS, "%s: workspace overlaps y", fn);
        if (overlap(rw, rs)) return fail(GDN_ERR_ALIAS, "%s: workspace overlaps final_state", fn);
        for (const Range &r : inputs)
            if (overlap(rw, r)) return fail(GDN_ERR_ALIAS, "%s: workspace overlaps %s", fn, r.name);
    }

    gdn::PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta;
    a.s0 = initial_state; a.y = y; a.sT = final_state;
    a.B = B; a.T = T; a.H = H; a.Dk = Dk; a.Dv = Dv; a.chunk = chunk;
    a.q_tok_stride = H * Dk; a.k_tok_stride = H * Dk; a.v_tok_stride = H * Dv;
    a.bf16 = dtype == GDN_BF16;
    a.ws = need > 0 ? workspace : nullptr;
    return hip_status(gdn::launch_prefill(a, stream), fn, stream);
}

}  // namespace

gdn_status gdn_prefill_fwd(const void *q, const void *k, const void *v, const float *alpha,
                           const float *beta, const float *initial_state, float *y,
                           float *final_state, int64_t B, int64_t T, int64_t H, int64_t Dk,
                           int64_t Dv, int64_t chunk, gdn_dtype dtype, void *workspace,
                           size_t workspace_bytes, hipStream_t stream)
{
    return prefill_impl("gdn_prefill_fwd", q, k, v, alpha, beta, initial_state, y, final_state, B, T, H, Dk,
                        Dv, chunk, dtype, workspace, workspace_bytes, stream);
}

gdn_status gdn_decode_step(const void *q, const void *k, const void *v, const float *alpha,
                           const float *beta, float *state, float *y, int64_t N, int64_t H,
                           int64_t Dk, int64_t Dv, gdn_dtype dtype, hipStream_t stream)
{
    if (N < 0 || H < 0 || Dk < 0 || Dv < 0)
        return fail(GDN_ERR_SHAPE, "gdn_decode_step: negative size");
    if (dtype != GDN_F32 && dtype != GDN_BF16)
        return fail(GDN_ERR_UNSUPPORTED, "gdn_decode_step: dtype %d", (int)dtype);
    if (!is_pow2_dim(Dk) || !is_pow2_dim(Dv))
        return fail(GDN_ERR_UNSUPPORTED, "gdn_decode_step: Dk=%lld Dv=%lld (supported: 16, 32, 64, 128)",
                    (long long)Dk, (long long)Dv);
    int64_t n_nh, n_s;
    if (!count(&n_nh, {N, H}) || !count(&n_s, {N, H, Dk, Dv}) || n_s > INT64_MAX / 4)
        return fail(GDN_ERR_SHAPE, "gdn_decode_step: sizes overflow");
    if (n_nh > INT32_MAX)
        return fail(GDN_ERR_UNSUPPORTED, "gdn_decode_step: N*H=%lld too large for one launch", (long long)n_nh);
    if (n_nh > 0 && (!q || !k || !v || !alpha || !beta || !state || !y))
        return fail(GDN_ERR_NULL, "gdn_decode_step: every pointer is required");
    const void *ptrs[] = {q, k, v, alpha, beta, state, y};
    const char *names[] = {"q", "k", "v", "alpha", "beta", "state", "y"};
    for (int i = 0; i < 7; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(GDN_ERR_ALIGN, "gdn_decode_step: %s is not 16-byte aligned", names[i]);
    const size_t esz = dtype == GDN_BF16 ? 2 : 4;
    const Range ry{y, (size_t)(n_nh * Dv) * 4, "y"};
    const Range rs{state, (size_t)n_s * 4, "state"};
    const Range inputs[] = {{q, (size_t)(n_nh * Dk) * esz, "q"}, {k, (size_t)(n_nh * Dk) * esz, "k"},
                            {v, (size_t)(n_nh * Dv) * esz, "v"}, {alpha, (size_t)n_nh * 4, "alpha"},
                            {beta, (size_t)n_nh * 4, "beta"}};
    for (const Range &r : inputs) {
        if (overlap(ry, r)) return fail(GDN_ERR_ALIAS, "gdn_decode_step: y overlaps %s", r.name);
        if (overlap(rs, r)) return fail(GDN_ERR_ALIAS, "gdn_decode_step: state overlaps %s", r.name);
    }
    if (overlap(ry, rs)) return fail(GDN_ERR_ALIAS, "gdn_decode_step: y overlaps state");

    gdn::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.state = state; a.y = y;
    a.N = N; a.H = H; a.Dk = Dk; a.Dv = Dv; a.bf16 = dtype == GDN_BF16;
    return hip_status(gdn::launch_decode(a, stream), "gdn_decode_step launch", stream);
}

gdn_status gdn_decode_verify(const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                             const float *state, float *states_out, float *y, int64_t N, int64_t T, int64_t H,
                             int64_t Dk, int64_t Dv, gdn_dtype dtype, hipStream_t stream)
{
    if (N < 0 || T < 0 || H < 0 || Dk < 0 || Dv < 0)
        return fail(GDN_ERR_SHAPE, "gdn_decode_verify: negative size");
    if (dtype != GDN_F32 && dtype != GDN_BF16)
        return fail(GDN_ERR_UNSUPPORTED, "gdn_decode_verify: dtype %d", (int)dtype);
    if (!is_pow2_dim(Dk) || !is_pow2_dim(Dv))
        return fail(GDN_ERR_UNSUPPORTED, "gdn_decode_verify: Dk=%lld Dv=%lld (supported: 16, 32, 64, 128)",
                    (long long)Dk, (long long)Dv);
    int64_t n_tok, n_s, n_so;
    if (!count(&n_tok, {N, T, H}) || !count(&n_s, {N, H, Dk, Dv}) || !count(&n_so, {N, T, H, Dk, Dv}) ||
        n_so > INT64_MAX / 4 || n_tok > INT64_MAX / (4 * 128))
        return fail(GDN_ERR_SHAPE, "gdn_decode_verify: sizes overflow");
    if (N * H > INT32_MAX || T > INT32_MAX)
        return fail(GDN_ERR_UNSUPPORTED, "gdn_decode_verify: N*H=%lld or T=%lld too large for one launch",
                    (long long)(N * H), (long long)T);
    if (n_tok > 0 && (!q || !k || !v || !alpha || !beta || !state || !states_out || !y))
        return fail(GDN_ERR_NULL, "gdn_decode_verify: every pointer is required");
    const void *ptrs[] = {q, k, v, alpha, beta, state, states_out, y};
    const char *names[] = {"q", "k", "v", "alpha", "beta", "state", "states_out", "y"};
    for (int i = 0; i < 8; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(GDN_ERR_ALIGN, "gdn_decode_verify: %s is not 16-byte aligned", names[i]);
    const size_t esz = dtype == GDN_BF16 ? 2 : 4;
    const Range ry{y, (size_t)(n_tok * Dv) * 4, "y"};
    const Range ro{states_out, (size_t)n_so * 4, "states_out"};
    const Range inputs[] = {{q, (size_t)(n_tok * Dk) * esz, "q"}, {k, (size_t)(n_tok * Dk) * esz, "k"},
                            {v, (size_t)(n_tok * Dv) * esz, "v"}, {alpha, (size_t)n_tok * 4, "alpha"},
                            {beta, (size_t)n_tok * 4, "beta"}, {state, (size_t)n_s * 4, "state"}};
    for (const Range &r : inputs) {
        if (overlap(ry, r)) return fail(GDN_ERR_ALIAS, "gdn_decode_verify: y overlaps %s", r.name);
        if (overlap(ro, r)) return fail(GDN_ERR_ALIAS, "gdn_decode_verify: states_out overlaps %s", r.name);
    }
    if (overlap(ry, ro)) return fail(GDN_ERR_ALIAS, "gdn_decode_verify: y overlaps states_out");

    gdn::VerifyArgs a;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.s_in = state; a.s_out = states_out; a.y = y;
    a.N = N; a.T = T; a.H = H; a.Dk = Dk; a.Dv = Dv; a.bf16 = dtype == GDN_BF16;
    return hip_status(gdn::launch_verify(a, stream), "gdn_decode_verify launch", stream);
}

size_t gdn_layer_workspace_bytes(int64_t B, int64_t T, int64_t hidden, int64_t H, int64_t Dk,
                                 int64_t Dv, int64_t conv_k, int64_t chunk)
{
    (void)conv_k;
    (void)chunk;
    if (B < 0 || T < 0 || hidden < 0 || H < 0 || Dk < 0 || Dv < 0) return 0;
    return gdn::layer_workspace_bytes(B, T, hidden, H, Dk, Dv);
}

gdn_status gdn_layer_fwd(const void *x, const gdn_layer_params *p, const float *initial_state,
                         float *final_state, float *out, int64_t B, int64_t T, int64_t hidden,
                         int64_t H, int64_t Dk, int64_t Dv, int64_t conv_k, int64_t chunk,
                         void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (B < 0 || T < 0 || hidden < 0 || H < 0 || Dk < 0 || Dv < 0 || conv_k < 0 || chunk < 0)
        return fail(GDN_ERR_SHAPE, "gdn_layer_fwd: negative size");
    if (!is_pow2_dim(Dk) || !is_pow2_dim(Dv))
        return fail(GDN_ERR_UNSUPPORTED, "gdn_layer_fwd: Dk=%lld Dv=%lld (supported: 16, 32, 64, 128)",
                    (long long)Dk, (long long)Dv);
    if (chunk != 16 && chunk != 32 && chunk != 64)
        return fail(GDN_ERR_UNSUPPORTED, "gdn_layer_fwd: chunk=%lld (supported: 16, 32, 64)", (long long)chunk);
    if (conv_k < 1 || conv_k > 4)
        return fail(GDN_ERR_UNSUPPORTED, "gdn_layer_fwd: conv_k=%lld (supported: 1..4)", (long long)conv_k);
    if (hidden % 64 != 0 || hidden == 0)
        return fail(GDN_ERR_UNSUPPORTED, "gdn_layer_fwd: hidden=%lld must be a positive multiple of 64",
                    (long long)hidden);
    int64_t n_tok, n_x, n_s, n_w;
    if (!count(&n_tok, {B, T}) || !count(&n_x, {B, T, hidden}) || !count(&n_s, {B, H, Dk, Dv}) ||
        !count(&n_w, {H, 2 * Dk + Dv, hidden}) || n_x > INT64_MAX / 8)
        return fail(GDN_ERR_SHAPE, "gdn_layer_fwd: sizes overflow");
    if (!p) return fail(GDN_ERR_NULL, "gdn_layer_fwd: params is NULL");
    if (n_tok > 0 && H > 0) {
        if (!x || !out || !p->W_qkv || !p->conv_w || !p->W_ab || !p->A || !p->b_alpha || !p->W_gate ||
            !p->norm_gamma || !p->W_o)
            return fail(GDN_ERR_NULL, "gdn_layer_fwd: x, out and every parameter are required");
    }
    const void *ptrs[] = {x, out, initial_state, final_state, p->W_qkv, p->conv_w, p->W_ab, p->A,
                          p->b_alpha, p->W_gate, p->norm_gamma, p->W_o, workspace};
    const char *names[] = {"x", "out", "initial_state", "final_state", "W_qkv", "conv_w", "W_ab", "A",
                           "b_alpha", "W_gate", "norm_gamma", "W_o", "workspace"};
    for (int i = 0; i < 13; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(GDN_ERR_ALIGN, "gdn_layer_fwd: %s is not 16-byte aligned", names[i]);
    const size_t need = gdn::layer_workspace_bytes(B, T, hidden, H, Dk, Dv);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(GDN_ERR_WORKSPACE, "gdn_layer_fwd: workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return fail(GDN_ERR_ALIGN, "gdn_layer_fwd: workspace is not 256-byte aligned");
    const Range ro{out, (size_t)n_x * 4, "out"};
    const Range rw{workspace, need, "workspace"};
    const Range rst{final_state, (size_t)n_s * 4, "final_state"};
    const Range inputs[] = {{x, (size_t)n_x * 2, "x"}, {initial_state, (size_t)n_s * 4, "initial_state"},
                            {p->W_qkv, (size_t)n_w * 2, "W_qkv"}, {p->W_o, (size_t)(hidden * H * Dv) * 2, "W_o"},
                            {p->W_gate, (size_t)(hidden * H * Dv) * 2, "W_gate"},
                            {p->W_ab, (size_t)(2 * H * hidden) * 2, "W_ab"}, {workspace, need, "workspace"}};
    for (const Range &r : inputs) {
        if (overlap(ro, r)) return fail(GDN_ERR_ALIAS, "gdn_layer_fwd: out overlaps %s", r.name);
        if (r.p != workspace && overlap(rw, r)) return fail(GDN_ERR_ALIAS, "gdn_layer_fwd: workspace overlaps %s", r.name);
    }
    if (overlap(rst, ro) || overlap(rst, rw) || overlap(rst, inputs[0]))
        return fail(GDN_ERR_ALIAS, "gdn_layer_fwd: final_state overlaps out, x or workspace");
    if (final_state != initial_state && overlap(rst, inputs[1]))
        return fail(GDN_ERR_ALIAS, "gdn_layer_fwd: final_state partially overlaps initial_state");

    gdn::LayerArgs a;
    a.x = x; a.W_qkv = p->W_qkv; a.conv_w = p->conv_w; a.W_ab = p->W_ab; a.W_gate = p->W_gate;
    a.W_o = p->W_o; a.A = p->A; a.b_alpha = p->b_alpha; a.norm_gamma = p->norm_gamma;
    a.s0 = initial_state; a.sT = final_state; a.out = out;
    a.B = B; a.T = T; a.hidden = hidden; a.H = H; a.Dk = Dk; a.Dv = Dv; a.conv_k = conv_k; a.chunk = chunk;
    a.ws = workspace;
    return hip_status(gdn::launch_layer(a, stream), "gdn_layer_fwd launch", stream);
}

size_t gdn_prefill_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int64_t chunk)
{
    if (B <= 0 || T <= 0 || H <= 0 || !is_pow2_dim(Dk) || !is_pow2_dim(Dv) ||
        (chunk != 16 && chunk != 32 && chunk != 64))
        return 0;
    int64_t n;
    if (!count(&n, {B, H, (T + chunk - 1) / chunk, gdn::bwd_record_floats(chunk) + 2 * Dk * Dv, 4})) return 0;
    return gdn::prefill_bwd_workspace_bytes(B, T, H, Dk, Dv, chunk);
}

gdn_status gdn_prefill_bwd(const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                           const float *initial_state, const float *dy, const float *dfinal_state, float *dq,
                           float *dk, float *dv, float *dalpha, float *dbeta, float *dinitial_state, int64_t B,
                           int64_t T, int64_t H, int64_t Dk, int64_t Dv, int64_t chunk, gdn_dtype dtype,
                           void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    const char *fn = "gdn_prefill_bwd";
    if (B < 0 || T < 0 || H < 0 || Dk < 0 || Dv < 0 || chunk < 0)
        return fail(GDN_ERR_SHAPE, "%s: negative size", fn);
    if (dtype != GDN_F32 && dtype != GDN_BF16) return fail(GDN_ERR_UNSUPPORTED, "%s: dtype %d", fn, (int)dtype);
    if (!is_pow2_dim(Dk) || !is_pow2_dim(Dv))
        return fail(GDN_ERR_UNSUPPORTED, "%s: Dk=%lld Dv=%lld (supported: 16, 32, 64, 128)", fn, (long long)Dk,
                    (long long)Dv);
    if (chunk != 16 && chunk != 32 && chunk != 64)
        return fail(GDN_ERR_UNSUPPORTED, "%s: chunk=%lld (supported: 16, 32, 64)", fn, (long long)chunk);
    int64_t n_tok, n_qk, n_v, n_s, n_ch;
    if (!count(&n_tok, {B, T, H}) || !count(&n_qk, {B, T, H, Dk, 4}) || !count(&n_v, {B, T, H, Dv, 4}) ||
        !count(&n_s, {B, H, Dk, Dv, 4}) || !count(&n_ch, {B, H, (T + chunk - 1) / chunk}))
        return fail(GDN_ERR_SHAPE, "%s: sizes overflow", fn);
    if (n_ch > INT32_MAX || B * H * (Dv / 16) > INT32_MAX)
        return fail(GDN_ERR_UNSUPPORTED, "%s: B*H*chunks=%lld too large for one launch", fn, (long long)n_ch);
    if (n_tok > 0) {
        if (!q || !k || !v || !alpha || !beta || !dy)
            return fail(GDN_ERR_NULL, "%s: q, k, v, alpha, beta and dy are required", fn);
        if (!dq || !dk || !dv || !dalpha || !dbeta)
            return fail(GDN_ERR_NULL, "%s: dq, dk, dv, dalpha and dbeta are required", fn);
    }
    const void *ptrs[] = {q, k, v, alpha, beta, initial_state, dy, dfinal_state,
                          dq, dk, dv, dalpha, dbeta, dinitial_state};
    const char *names[] = {"q", "k", "v", "alpha", "beta", "initial_state", "dy", "dfinal_state",
                           "dq", "dk", "dv", "dalpha", "dbeta", "dinitial_state"};
    for (int i = 0; i < 14; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(GDN_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, names[i]);
    const size_t esz = dtype == GDN_BF16 ? 2 : 4;
    const size_t need = n_tok > 0 ? gdn_prefill_bwd_workspace_bytes(B, T, H, Dk, Dv, chunk) : 0;
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                        workspace ? workspace_bytes : (size_t)0);
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(GDN_ERR_ALIGN, "%s: workspace is not 256-byte aligned", fn);
    }
    const Range inputs[] = {{q, (size_t)n_qk / 4 * esz, "q"}, {k, (size_t)n_qk / 4 * esz, "k"},
                            {v, (size_t)n_v / 4 * esz, "v"}, {alpha, (size_t)n_tok * 4, "alpha"},
                            {beta, (size_t)n_tok * 4, "beta"}, {initial_state, (size_t)n_s, "initial_state"},
                            {dy, (size_t)n_v, "dy"}, {dfinal_state, (size_t)n_s, "dfinal_state"}};
    const Range outputs[] = {{dq, (size_t)n_qk, "dq"}, {dk, (size_t)n_qk, "dk"}, {dv, (size_t)n_v, "dv"},
                             {dalpha, (size_t)n_tok * 4, "dalpha"}, {dbeta, (size_t)n_tok * 4, "dbeta"},
                             {dinitial_state, (size_t)n_s, "dinitial_state"}, {workspace, need, "workspace"}};
    for (int i = 0; i < 7; ++i) {
        for (const Range &r : inputs)
            if (overlap(outputs[i], r)) return fail(GDN_ERR_ALIAS, "%s: %s overlaps %s", fn, outputs[i].name, r.name);
        for (int j = 0; j < i; ++j)
            if (overlap(outputs[i], outputs[j]))
                return fail(GDN_ERR_ALIAS, "%s: %s overlaps %s", fn, outputs[i].name, outputs[j].name);
    }

    gdn::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.s0 = initial_state;
    a.dy = dy; a.dsT = dfinal_state;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dalpha = dalpha; a.dbeta = dbeta; a.ds0 = dinitial_state;
    a.B = B; a.T = T; a.H = H; a.Dk = Dk; a.Dv = Dv; a.chunk = chunk;
    a.bf16 = dtype == GDN_BF16;
    a.ws = need > 0 ? workspace : nullptr;
    return hip_status(gdn::launch_prefill_bwd(a, stream), fn, stream);
}

size_t gdn_layer_decode_workspace_bytes(int64_t N, int64_t hidden, int64_t H, int64_t Dk, int64_t Dv)
{
    if (N < 0 || hidden < 0 || H < 0 || Dk < 0 || Dv < 0) return 0;
    return gdn::layer_decode_workspace_bytes(N, H, Dk, Dv);
}

static gdn_status layer_decode_impl(const char *fn, bool noalloc, const void *x, const gdn_layer_params *p,
                                    float *conv_state, float *state, float *out, int64_t N, int64_t hidden, int64_t H,
                                    int64_t Dk, int64_t Dv, int64_t conv_k, void *workspace, size_t workspace_bytes,
                                    hipStream_t stream)
{
    if (N < 0 || hidden < 0 || H < 0 || Dk < 0 || Dv < 0 || conv_k < 0)
        return fail(GDN_ERR_SHAPE, "%s: negative size", fn);
    if (!is_pow2_dim(Dk) || !is_pow2_dim(Dv))
        return fail(GDN_ERR_UNSUPPORTED, "%s: Dk=%lld Dv=%lld (supported: 16, 32, 64, 128)", fn,
                    (long long)Dk, (long long)Dv);
    if (conv_k < 1 || conv_k > 4)
        return fail(GDN_ERR_UNSUPPORTED, "%s: conv_k=%lld (supported: 1..4)", fn, (long long)conv_k);
    if (hidden % 64 != 0 || hidden == 0)
        return fail(GDN_ERR_UNSUPPORTED, "%s: hidden=%lld must be a positive multiple of 64", fn,
                    (long long)hidden);
    int64_t n_x, n_s, n_w, n_c;
    if (!count(&n_x, {N, hidden}) || !count(&n_s, {N, H, Dk, Dv}) || !count(&n_w, {H, 2 * Dk + Dv, hidden}) ||
        !count(&n_c, {N, conv_k - 1, H, 2 * Dk + Dv}) || n_s > INT64_MAX / 8 || n_c > INT64_MAX / 8)
        return fail(GDN_ERR_SHAPE, "%s: sizes overflow", fn);
    if (N * H > INT32_MAX || N > (int64_t)1 << 31)
        return fail(GDN_ERR_UNSUPPORTED, "%s: N*H=%lld too large for one launch", fn,
                    (long long)(N * H));
    if (!p) return fail(GDN_ERR_NULL, "%s: params is NULL", fn);
    if (N > 0 && H > 0) {
        if (!x || !out || !state || !p->W_qkv || !p->conv_w || !p->W_ab || !p->A || !p->b_alpha || !p->W_gate ||
            !p->norm_gamma || !p->W_o)
            return fail(GDN_ERR_NULL, "%s: x, out, state and every parameter are required", fn);
        if (conv_k > 1 && !conv_state)
            return fail(GDN_ERR_NULL, "%s: conv_state is required when conv_k > 1", fn);
    }
    const void *ptrs[] = {x, out, state, conv_state, p->W_qkv, p->conv_w, p->W_ab, p->A,
                          p->b_alpha, p->W_gate, p->norm_gamma, p->W_o, workspace};
    const char *names[] = {"x", "out", "state", "conv_state", "W_qkv", "conv_w", "W_ab", "A",
                           "b_alpha", "W_gate", "norm_gamma", "W_o", "workspace"};
    for (int i = 0; i < 13; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(GDN_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, names[i]);
    const size_t need = gdn::layer_decode_workspace_bytes(N, H, Dk, Dv);
    if (noalloc) {
        if (need > gdn::layer_decode_scratch_bytes())
            return fail(GDN_ERR_WORKSPACE, "%s: %zu bytes of scratch needed, the library holds %zu", fn, need,
                        gdn::layer_decode_scratch_bytes());
        workspace = nullptr;
        workspace_bytes = 0;
    } else if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    workspace ? workspace_bytes : (size_t)0);
    if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return fail(GDN_ERR_ALIGN, "%s: workspace is not 256-byte aligned", fn);
    const Range ro{out, (size_t)n_x * 4, "out"};
    const Range rs{state, (size_t)n_s * 4, "state"};
    const Range rc{conv_state, (size_t)n_c * 4, "conv_state"};
    const Range rw{workspace, need, "workspace"};
    const Range inputs[] = {{x, (size_t)n_x * 2, "x"}, {p->W_qkv, (size_t)n_w * 2, "W_qkv"},
                            {p->W_o, (size_t)(hidden * H * Dv) * 2, "W_o"},
                            {p->W_gate, (size_t)(hidden * H * Dv) * 2, "W_gate"},
                            {p->W_ab, (size_t)(2 * H * hidden) * 2, "W_ab"}};
    for (const Range &r : inputs) {
        if (overlap(ro, r)) return fail(GDN_ERR_ALIAS, "%s: out overlaps %s", fn, r.name);
        if (overlap(rs, r)) return fail(GDN_ERR_ALIAS, "%s: state overlaps %s", fn, r.name);
        if (overlap(rc, r)) return fail(GDN_ERR_ALIAS, "%s: conv_state overlaps %s", fn, r.name);
        if (overlap(rw, r)) return fail(GDN_ERR_ALIAS, "%s: workspace overlaps %s", fn, r.name);
    }
    if (overlap(ro, rs) || overlap(ro, rc) || overlap(ro, rw))
        return fail(GDN_ERR_ALIAS, "%s: out overlaps state, conv_state or workspace", fn);
    if (overlap(rs, rc) || overlap(rs, rw) || overlap(rc, rw))
        return fail(GDN_ERR_ALIAS, "%s: state, conv_state and workspace must not overlap", fn);

    gdn::LayerDecodeArgs a;
    a.x = x; a.W_qkv = p->W_qkv; a.conv_w = p->conv_w; a.W_ab = p->W_ab; a.W_gate = p->W_gate;
    a.W_o = p->W_o; a.A = p->A; a.b_alpha = p->b_alpha; a.norm_gamma = p->norm_gamma;
    a.conv_state = conv_state; a.state = state; a.out = out;
    a.N = N; a.hidden = hidden; a.H = H; a.Dk = Dk; a.Dv = Dv; a.conv_k = conv_k;
    a.ws = workspace;
    if (noalloc && N > 0 && H > 0) {
        const hipError_t e = gdn::layer_decode_scratch(&a.ws);
        if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s: scratch address: %s", fn, hipGetErrorString(e));
    }
    return hip_status(gdn::launch_layer_decode(a, stream), fn, stream);
}

gdn_status gdn_layer_decode_step(const void *x, const gdn_layer_params *p, float *conv_state, float *state,
                                 float *out, int64_t N, int64_t hidden, int64_t H, int64_t Dk, int64_t Dv,
                                 int64_t conv_k, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return layer_decode_impl("gdn_layer_decode_step", false, x, p, conv_state, state, out, N, hidden, H, Dk, Dv,
                             conv_k, workspace, workspace_bytes, stream);
}

gdn_status gdn_layer_decode_step_noalloc(const void *x, const gdn_layer_params *p, float *conv_state,
                                         float *state, float *out, int64_t N, int64_t hidden, int64_t H,
                                         int64_t Dk, int64_t Dv, int64_t conv_k, hipStream_t stream)
{
    return layer_decode_impl("gdn_layer_decode_step_noalloc", true, x, p, conv_state, state, out, N, hidden, H, Dk,
                             Dv, conv_k, nullptr, 0, stream);
}

}  // extern "C"
