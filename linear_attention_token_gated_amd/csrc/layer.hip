// layer.hip -- the GDN token-mixing layer around the core, on gfx950.
//
// Source: "On the Design of Qwen3.8-Next Architecture", picx.dev summary,
// "Methodology / 1. GDN Hybrid Token Mixing": short causal convolutions,
// L2-normalised queries and keys, eq (9) write strength, eq (10) decay and the
// eq (11) output  o_t = W_o [ sigmoid(W_z x_t) * RMSNorm(y_t) ]  with a
// zero-centred RMSNorm.
//
// Steps (M = B*T tokens):
//   1. projections: qkv_pre = x W_qkv^T (fp32), ab = x W_ab^T (fp32); z = x
//      W_gate^T (bf16), needed only in step 4, runs in the core's launch where
//      the core takes it (step 3), else here
//   2. prologue: depthwise causal conv over the q|k|v channels, L2 norm of
//      every q and k head, alpha (eq (10)) and beta (eq (9)) per (token, head);
//      q, k, v stay fp32
//   3. the chunked core (prefill kernel, fp32 operands) reading q, k, v in place
//   4. epilogue: g = sigmoid(z) * y / sqrt(mean(y^2) + eps) * (1 + gamma) (bf16)
//   5. projection: out = g W_o^T (fp32)
//
// The projections are plain products on this file's gemm_nt_kernel.
//
// Why q, k, v are not rounded to bf16 here: with unit-norm q and k in Dk
// dimensions, y_t = S_t^T q_t is a small projection of the state (|q.k| ~
// 1/sqrt(Dk)), so a relative perturbation of 2^-9 in q, k or v (one bf16
// rounding) becomes several percent of max|err|/RMS in y and in the layer
// output.  The inputs x and the weights are bf16 and the products accumulate in
// fp32, so the projections themselves are exact up to fp32 summation.
#include <cstdlib>
#include <mutex>

#include "common.hpp"
#include "gemm_nt.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr float kL2Eps = 1e-6f;
constexpr float kRmsEps = 1e-6f;


template <typename OutT, int BM, int BN, int ST, int NW>
__global__ __launch_bounds__(64 * NW, BM == 256 ? 1 : 2) void gemm_nt_kernel(const __bf16 *__restrict__ A, const __bf16 *__restrict__ B1,
                                                         OutT *__restrict__ C1, int M, int N1, int K, int64_t lda,
                                                         int64_t ldb1, int64_t ldc1, int tiles_m, int tiles_n, int bn_log,
                                                         const __bf16 *__restrict__ B2, OutT *__restrict__ C2, int N2,
                                                         int64_t ldb2, int64_t ldc2, int tiles_n1)
{
    __shared__ __attribute__((aligned(1024))) char smem[ST * GemmTile<BM, BN, NW>::STAGE];
    gemm_nt_block<OutT, BM, BN, ST, NW>((int)blockIdx.x, smem, A, B1, C1, M, N1, K, lda, ldb1, ldc1, tiles_m, tiles_n,
                                        bn_log, B2, C2, N2, ldb2, ldc2, tiles_n1);
}

template <typename OutT, int BM, int BN, int ST, int NW = 4>
hipError_t gemm_nt_tile(const __bf16 *A, const __bf16 *Bm, OutT *C, int64_t M, int64_t N, int64_t K, int64_t lda,
                        int64_t ldb, int64_t ldc, const __bf16 *B2, OutT *C2, int64_t N2, int64_t ldb2, int64_t ldc2,
                        hipStream_t s)
{
    const GemmGrid<BM, BN> g(M, N, N2);
    hipLaunchKernelGGL((gemm_nt_kernel<OutT, BM, BN, ST, NW>), dim3((unsigned)g.grid), dim3(64 * NW), 0, s, A, Bm, C,
                       (int)M, (int)N, (int)K, lda, ldb, ldc, g.tiles_m, g.tiles_n, g.bn_log, B2 ? B2 : Bm,
                       C2 ? C2 : C, (int)N2, ldb2, ldc2, g.tiles_n1);
    return hipGetLastError();
}

// C[M, N] = A[M, K] B[N, K]^T, and optionally C2[M, N2] = A B2^T in the same
// launch.  The tile is the largest that still gives every compute unit a
// workgroup (256 x 256, 128 x 128, else 64 x 64).  Small tiles do little MFMA
// work per K step, so they keep 7 steps in flight (8 stages, 64 KB of LDS)
// against the memory latency; the larger ones 3.  Where 64 x 64 tiles would
// outnumber the compute units but 64 x 128 tiles would not (a few hundred
// rows, thousands of columns: the decode step's in-projection), the wider
// tile runs the product in one round, one workgroup per CU: its K steps are
// latency-bound, so two workgroups sharing a CU take twice as long.
template <typename OutT>
hipError_t project(const __bf16 *A, const __bf16 *Bm, OutT *C, int64_t M, int64_t N, int64_t K, int64_t lda,
                   int64_t ldb, int64_t ldc, hipStream_t s, const __bf16 *B2 = nullptr, OutT *C2 = nullptr,
                   int64_t N2 = 0, int64_t ldb2 = 0, int64_t ldc2 = 0)
{
    if (M == 0 || N + N2 == 0) return hipSuccess;
    auto tiles = [&](int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn + (N2 + bn - 1) / bn); };
    if (tiles(256, 256) >= 256)
        return gemm_nt_tile<OutT, 256, 256, 4, 8>(A, Bm, C, M, N, K, lda, ldb, ldc, B2, C2, N2, ldb2, ldc2, s);
    if (tiles(128, 128) >= 256)
        return gemm_nt_tile<OutT, 128, 128, 4>(A, Bm, C, M, N, K, lda, ldb, ldc, B2, C2, N2, ldb2, ldc2, s);
    if (tiles(64, 64) > 256 && tiles(64, 128) <= 256)
        return gemm_nt_tile<OutT, 64, 128, 8>(A, Bm, C, M, N, K, lda, ldb, ldc, B2, C2, N2, ldb2, ldc2, s);
    return gemm_nt_tile<OutT, 64, 64, 8>(A, Bm, C, M, N, K, lda, ldb, ldc, B2, C2, N2, ldb2, ldc2, s);
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + expf(-x)); }
__device__ __forceinline__ float softplusf_(float x) { return x > 0.f ? x + log1pf(expf(-x)) : log1pf(expf(x)); }

// ---------------------------------------------------------------------------
// Prologue: one workgroup per tile of PRO_TT consecutive tokens of one
// sequence and 256 vectors of channels.  Each thread owns 8 consecutive
// channels (one 16-byte vector) of the H*(2Dk+Dv) q|k|v channels and walks the
// tile's tokens in order, keeping the last conv_k-1 inputs in registers, so
// every input row is read once (plus conv_k-1 rows before the tile).  A q or
// k head is Dk/8 consecutive lanes, reduced with xor-shuffles for its L2 norm.
// ---------------------------------------------------------------------------
constexpr int PRO_TT = 32;

template <int DK, int KC>
__global__ __launch_bounds__(256) void prologue_kernel(const float *__restrict__ pre, const __bf16 *__restrict__ conv_w,
                                                       const float *__restrict__ ab, const float *__restrict__ Aexp,
                                                       const float *__restrict__ b_alpha, float *__restrict__ post,
                                                       float *__restrict__ alpha, float *__restrict__ beta, int64_t T,
                                                       int H, int nqkv, int conv_k)
{
    const int64_t ntile = (T + PRO_TT - 1) / PRO_TT;
    const int64_t b = blockIdx.x / ntile, t0 = (blockIdx.x % ntile) * PRO_TT;
    const int64_t tend = t0 + PRO_TT < T ? t0 + PRO_TT : T;
    const int nvec = nqkv / 8;
    const int nqk_vec = 2 * H * DK / 8;      // vectors holding q and k channels
    constexpr int HV = DK / 8;               // vectors per q/k head (power of two, <= 16)
    const int vi = blockIdx.y * 256 + threadIdx.x;
    const bool active = vi < nvec;
    const int c0 = active ? vi * 8 : 0;
    const float scale_qk = vi < nqk_vec;     // 1: an L2-normalised q or k channel
    auto load8 = [&](int64_t t, float (&x)[8]) {
        const f32x4 x0 = *reinterpret_cast<const f32x4 *>(pre + (b * T + t) * nqkv + c0);
        const f32x4 x1 = *reinterpret_cast<const f32x4 *>(pre + (b * T + t) * nqkv + c0 + 4);
        x[0] = x0[0]; x[1] = x0[1]; x[2] = x0[2]; x[3] = x0[3];
        x[4] = x1[0]; x[5] = x1[1]; x[6] = x1[2]; x[7] = x1[3];
    };
    // taps (KC = conv_k, a compile-time constant): w[j] multiplies the input
    // of token t - (KC - 1 - j)
    (void)conv_k;
    float w[KC][8];
#pragma unroll
    for (int j = 0; j < KC; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) w[j][e] = (float)conv_w[(int64_t)(c0 + e) * KC + j];
    // win[l - 1] = input of token t - l, zero before the sequence start, so a
    // tap that reaches before it adds an exact zero
    float win[KC > 1 ? KC - 1 : 1][8];
#pragma unroll
    for (int l = 1; l < KC; ++l) {
        if (t0 - l >= 0) {
            load8(t0 - l, win[l - 1]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) win[l - 1][e] = 0.f;
        }
    }
    // tokens in groups of PG: the rows of the next group are in flight while
    // the current group is computed (rows past the tile are not read)
    constexpr int PG = 4;
    static_assert(PRO_TT % PG == 0, "whole groups per tile");
    float cur[PG][8], nxt[PG][8];
    auto load_group = [&](int64_t tg, float (&g)[PG][8]) {
#pragma unroll
        for (int i = 0; i < PG; ++i)
            if (tg + i < tend) load8(tg + i, g[i]);
    };
    load_group(t0, cur);
    for (int64_t tg = t0; tg < tend; tg += PG) {
        if (tg + PG < tend) load_group(tg + PG, nxt);
#pragma unroll
        for (int i = 0; i < PG; ++i) {
            const int64_t t = tg + i;
            if (t >= tend) break;
            const float (&x)[8] = cur[i];
            // taps in the order j = 0 .. KC-1 (oldest input first)
            float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KC; ++j) {
                const int lag = KC - 1 - j;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = fmaf(w[j][e], lag == 0 ? x[e] : win[lag > 0 ? lag - 1 : 0][e], o[e]);
            }
#pragma unroll
            for (int l = KC - 2; l >= 1; --l)
#pragma unroll
                for (int e = 0; e < 8; ++e) win[l][e] = win[l - 1][e];
            if constexpr (KC > 1) {
#pragma unroll
                for (int e = 0; e < 8; ++e) win[0][e] = x[e];
            }
            // L2 normalisation of q and k heads (heads never straddle the q|k / v
            // boundary and vector groups are lane-aligned)
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(o[e], o[e], ss);
#pragma unroll
            for (int off = 1; off < HV; off <<= 1) ss += __shfl_xor(ss, off);
            if (active) {
                const float scale = scale_qk ? 1.f / sqrtf(ss + kL2Eps) : 1.f;
                f32x4 o0, o1;
#pragma unroll
                for (int e = 0; e < 4; ++e) { o0[e] = o[e] * scale; o1[e] = o[4 + e] * scale; }
                *reinterpret_cast<f32x4 *>(post + (b * T + t) * nqkv + c0) = o0;
                *reinterpret_cast<f32x4 *>(post + (b * T + t) * nqkv + c0 + 4) = o1;
            }
        }
#pragma unroll
        for (int i = 0; i < PG; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) cur[i][e] = nxt[i][e];
    }
    // eq (10) decay and eq (9) write strength for every head of the tile's tokens
    if (blockIdx.y == 0) {
        for (int64_t i = threadIdx.x; i < (tend - t0) * H; i += 256) {
            const int64_t row = b * T + t0 + i / H;
            const int hh = (int)(i % H);
            const float a = ab[row * 2 * H + hh];
            const float bb = ab[row * 2 * H + H + hh];
            alpha[row * H + hh] = expf(-expf(Aexp[hh]) * softplusf_(a + b_alpha[hh]));
            beta[row * H + hh] = sigmoidf_(bb);
        }
    }
}

// ---------------------------------------------------------------------------
// Decode prologue: one token per sequence.  conv_state row r of sequence n
// holds the in-projection of token t - (conv_k - 1 - r), oldest first; tap j
// (j < conv_k - 1) reads row j and tap conv_k - 1 the current token.  The
// rows are then shifted by one, in place: each thread reads and writes only
// its own 8 channels.  L2 norm and gates as in the prologue.
// ---------------------------------------------------------------------------
template <int DK, int KC>
__global__ __launch_bounds__(256) void decode_prologue_kernel(const float *__restrict__ pre,
                                                              const __bf16 *__restrict__ conv_w,
                                                              const float *__restrict__ ab,
                                                              const float *__restrict__ Aexp,
                                                              const float *__restrict__ b_alpha,
                                                              float *__restrict__ conv_state, float *__restrict__ post,
                                                              float *__restrict__ alpha, float *__restrict__ beta,
                                                              int H, int nqkv)
{
    const int64_t n = blockIdx.x;
    const int nvec = nqkv / 8;
    const int nqk_vec = 2 * H * DK / 8;
    constexpr int HV = DK / 8;
    const int vi = blockIdx.y * 256 + threadIdx.x;
    const bool active = vi < nvec;
    const int c0 = active ? vi * 8 : 0;
    auto ld8 = [&](const float *src, float (&x)[8]) {
        const f32x4 x0 = *reinterpret_cast<const f32x4 *>(src);
        const f32x4 x1 = *reinterpret_cast<const f32x4 *>(src + 4);
        x[0] = x0[0]; x[1] = x0[1]; x[2] = x0[2]; x[3] = x0[3];
        x[4] = x1[0]; x[5] = x1[1]; x[6] = x1[2]; x[7] = x1[3];
    };
    float rows[KC][8];                       // taps 0 .. KC-1: history rows, then the current token
#pragma unroll
    for (int j = 0; j < KC - 1; ++j) ld8(conv_state + (n * (KC - 1) + j) * nqkv + c0, rows[j]);
    ld8(pre + n * nqkv + c0, rows[KC - 1]);
    // the thread's taps: 8 KC consecutive bf16 (channel-major), in 16-byte pieces
    __bf16 w[8 * KC];
#pragma unroll
    for (int q = 0; q < KC; ++q) {
        const bf16x8 v = *reinterpret_cast<const bf16x8 *>(conv_w + (int64_t)c0 * KC + 8 * q);
#pragma unroll
        for (int e = 0; e < 8; ++e) w[8 * q + e] = v[e];
    }
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KC; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf((float)w[e * KC + j], rows[j][e], o[e]);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(o[e], o[e], ss);
#pragma unroll
    for (int off = 1; off < HV; off <<= 1) ss += __shfl_xor(ss, off);
    if (active) {
        const float scale = vi < nqk_vec ? 1.f / sqrtf(ss + kL2Eps) : 1.f;
        f32x4 o0, o1;
#pragma unroll
        for (int e = 0; e < 4; ++e) { o0[e] = o[e] * scale; o1[e] = o[4 + e] * scale; }
        *reinterpret_cast<f32x4 *>(post + n * nqkv + c0) = o0;
        *reinterpret_cast<f32x4 *>(post + n * nqkv + c0 + 4) = o1;
        // history shifted by one token: row r <- tap r + 1
#pragma unroll
        for (int r = 0; r < KC - 1; ++r) {
            {
                float *dst = conv_state + (n * (KC - 1) + r) * nqkv + c0;
                *reinterpret_cast<f32x4 *>(dst) = f32x4{rows[r + 1][0], rows[r + 1][1], rows[r + 1][2], rows[r + 1][3]};
                *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{rows[r + 1][4], rows[r + 1][5], rows[r + 1][6], rows[r + 1][7]};
            }
        }
    }
    if (blockIdx.y == 0) {
        for (int hh = threadIdx.x; hh < H; hh += 256) {
            const float a = ab[n * 2 * H + hh];
            const float bb = ab[n * 2 * H + H + hh];
            alpha[n * H + hh] = expf(-expf(Aexp[hh]) * softplusf_(a + b_alpha[hh]));
            beta[n * H + hh] = sigmoidf_(bb);
        }
    }
}

// ---------------------------------------------------------------------------
// Epilogue: one workgroup per token; per head, RMSNorm over Dv with gain
// (1 + gamma), times sigmoid(z); written as the bf16 operand of W_o.
// ---------------------------------------------------------------------------
template <int DV>
__global__ __launch_bounds__(256) void epilogue_kernel(const float *__restrict__ y, const __bf16 *__restrict__ z,
                                                       const float *__restrict__ gamma, __bf16 *__restrict__ g,
                                                       int H)
{
    const int64_t row = blockIdx.x;
    const int nvec = H * DV / 8;
    constexpr int HV = DV / 8;
    for (int base = 0; base < nvec; base += 256) {
        const int vi = base + threadIdx.x;
        const bool active = vi < nvec;
        float yv[8];
        float ss = 0.f;
        if (active) {
            const f32x4 y0 = *reinterpret_cast<const f32x4 *>(y + row * H * DV + vi * 8);
            const f32x4 y1 = *reinterpret_cast<const f32x4 *>(y + row * H * DV + vi * 8 + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) { yv[e] = y0[e]; yv[4 + e] = y1[e]; }
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(yv[e], yv[e], ss);
        }
#pragma unroll
        for (int off = 1; off < HV; off <<= 1) ss += __shfl_xor(ss, off);
        if (active) {
            const float inv = 1.f / sqrtf(ss / (float)DV + kRmsEps);
            const f32x4 raw = *reinterpret_cast<const f32x4 *>(z + row * H * DV + vi * 8);
            const __bf16 *zz = reinterpret_cast<const __bf16 *>(&raw);
            const int c0 = (vi * 8) % DV;
            bf16x8 outv;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                outv[e] = (__bf16)(sigmoidf_((float)zz[e]) * yv[e] * inv * (1.f + gamma[c0 + e]));
            *reinterpret_cast<bf16x8 *>(g + row * H * DV + vi * 8) = outv;
        }
    }
}

constexpr size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

struct WsLayout {
    size_t pre, post, z, ab, alpha, beta, y, g, rec, total;
};

// with_core: room for the per-chunk records of the chunked core (the decode
// step runs the token-by-token kernel, which needs none)
WsLayout ws_layout(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, bool with_core = true)
{
    const size_t M = (size_t)(B * T);
    const size_t nqkv = (size_t)(H * (2 * Dk + Dv));
    WsLayout w;
    size_t o = 0;
    w.pre = o;   o += al256(M * nqkv * 4);
    w.post = o;  o += al256(M * nqkv * 4);
    w.z = o;     o += al256(M * (size_t)(H * Dv) * 2);
    w.ab = o;    o += al256(M * (size_t)(2 * H) * 4);
    w.alpha = o; o += al256(M * (size_t)H * 4);
    w.beta = o;  o += al256(M * (size_t)H * 4);
    w.y = o;     o += al256(M * (size_t)(H * Dv) * 4);
    w.g = o;     o += al256(M * (size_t)(H * Dv) * 2);
    // per-chunk records of the fp32 core; chunk 64 needs the most of {16, 32, 64}
    w.rec = o;   o += with_core ? al256(prefill_f32_workspace_bytes(B, T, H, 64)) : 0;
    w.total = o;
    return w;
}

template <int DK>
hipError_t launch_prologue_dk(const float *pre, const __bf16 *conv_w, const float *ab, const float *A,
                              const float *b_alpha, float *post, float *alpha, float *beta, int64_t M, int64_t T,
                              int H, int nqkv, int conv_k, hipStream_t s)
{
    const int64_t tiles = (M / T) * ((T + PRO_TT - 1) / PRO_TT);   // M = B * T, T > 0
    const unsigned slabs = (unsigned)((nqkv / 8 + 255) / 256);
    switch (conv_k) {
    case 1: hipLaunchKernelGGL((prologue_kernel<DK, 1>), dim3((unsigned)tiles, slabs), dim3(256), 0, s, pre, conv_w, ab,
                               A, b_alpha, post, alpha, beta, T, H, nqkv, conv_k); break;
    case 2: hipLaunchKernelGGL((prologue_kernel<DK, 2>), dim3((unsigned)tiles, slabs), dim3(256), 0, s, pre, conv_w, ab,
                               A, b_alpha, post, alpha, beta, T, H, nqkv, conv_k); break;
    case 3: hipLaunchKernelGGL((prologue_kernel<DK, 3>), dim3((unsigned)tiles, slabs), dim3(256), 0, s, pre, conv_w, ab,
                               A, b_alpha, post, alpha, beta, T, H, nqkv, conv_k); break;
    case 4: hipLaunchKernelGGL((prologue_kernel<DK, 4>), dim3((unsigned)tiles, slabs), dim3(256), 0, s, pre, conv_w, ab,
                               A, b_alpha, post, alpha, beta, T, H, nqkv, conv_k); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int DV>
hipError_t launch_epilogue_dv(const float *y, const __bf16 *z, const float *gamma, __bf16 *g, int64_t M, int H,
                              hipStream_t s)
{
    hipLaunchKernelGGL((epilogue_kernel<DV>), dim3((unsigned)M), dim3(256), 0, s, y, z, gamma, g, H);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_decode_prologue_dk(const float *pre, const __bf16 *conv_w, const float *ab, const float *A,
                                     const float *b_alpha, float *conv_state, float *post, float *alpha, float *beta,
                                     int64_t N, int H, int nqkv, int conv_k, hipStream_t s)
{
    const unsigned slabs = (unsigned)((nqkv / 8 + 255) / 256);
    const dim3 grid((unsigned)N, slabs);
    switch (conv_k) {
    case 1: hipLaunchKernelGGL((decode_prologue_kernel<DK, 1>), grid, dim3(256), 0, s, pre, conv_w, ab, A, b_alpha,
                               conv_state, post, alpha, beta, H, nqkv); break;
    case 2: hipLaunchKernelGGL((decode_prologue_kernel<DK, 2>), grid, dim3(256), 0, s, pre, conv_w, ab, A, b_alpha,
                               conv_state, post, alpha, beta, H, nqkv); break;
    case 3: hipLaunchKernelGGL((decode_prologue_kernel<DK, 3>), grid, dim3(256), 0, s, pre, conv_w, ab, A, b_alpha,
                               conv_state, post, alpha, beta, H, nqkv); break;
    case 4: hipLaunchKernelGGL((decode_prologue_kernel<DK, 4>), grid, dim3(256), 0, s, pre, conv_w, ab, A, b_alpha,
                               conv_state, post, alpha, beta, H, nqkv); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

size_t layer_workspace_bytes(int64_t B, int64_t T, int64_t hidden, int64_t H, int64_t Dk, int64_t Dv)
{
    (void)hidden;
    if (B * T == 0 || H == 0) return 0;
    return ws_layout(B, T, H, Dk, Dv).total;
}

size_t layer_decode_workspace_bytes(int64_t N, int64_t H, int64_t Dk, int64_t Dv)
{
    if (N == 0 || H == 0) return 0;
    return ws_layout(N, 1, H, Dk, Dv, false).total;
}

// Scratch memory of the allocation-free layer decode step: the intermediates
// of one call (in-projections, gates, core output, gated norm), each written in
// full before it is read, so no call needs it cleared.  One copy per GPU, held
// until the process ends and shared by every call on that GPU.
constexpr size_t kLayerDecodeScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kLayerDecodeScratchBytes];

size_t layer_decode_scratch_bytes() { return kLayerDecodeScratchBytes; }

// Device address of this GPU's scratch (the current device), looked up once per
// device: in host code the array's name is only a host-side stand-in.
hipError_t layer_decode_scratch(void **out)
{
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

hipError_t launch_layer(const LayerArgs &a, hipStream_t s)
{
    const int64_t M = a.B * a.T;
    const int64_t H = a.H, Dk = a.Dk, Dv = a.Dv, hidden = a.hidden;
    if (a.B * a.H == 0) return hipSuccess;
    if (M == 0 || H == 0) {
        PrefillArgs p{};
        p.B = a.B; p.T = 0; p.H = H; p.Dk = Dk; p.Dv = Dv; p.chunk = a.chunk; p.s0 = a.s0; p.sT = a.sT;
        return launch_prefill(p, s);
    }
    const WsLayout w = ws_layout(a.B, a.T, H, Dk, Dv);
    char *ws = static_cast<char *>(a.ws);
    float *pre = reinterpret_cast<float *>(ws + w.pre);
    float *post = reinterpret_cast<float *>(ws + w.post);
    __bf16 *z = reinterpret_cast<__bf16 *>(ws + w.z);
    float *ab = reinterpret_cast<float *>(ws + w.ab);
    float *alpha = reinterpret_cast<float *>(ws + w.alpha);
    float *beta = reinterpret_cast<float *>(ws + w.beta);
    float *y = reinterpret_cast<float *>(ws + w.y);
    __bf16 *g = reinterpret_cast<__bf16 *>(ws + w.g);
    const __bf16 *x = static_cast<const __bf16 *>(a.x);
    const int64_t nqkv = H * (2 * Dk + Dv);
    hipError_t e;

    // (separate launches: at M = B*T the q|k|v tiles fill whole rounds of the
    // compute units, and the a|b tiles added to that launch would start one more)
    if ((e = project<float>(x, (const __bf16 *)a.W_qkv, pre, M, nqkv, hidden, hidden, hidden, nqkv, s))) return e;
    if ((e = project<float>(x, (const __bf16 *)a.W_ab, ab, M, 2 * H, hidden, hidden, hidden, 2 * H, s))) return e;

    switch (Dk) {
    case 16: e = launch_prologue_dk<16>(pre, (const __bf16 *)a.conv_w, ab, a.A, a.b_alpha, post, alpha, beta, M, a.T, (int)H, (int)nqkv, (int)a.conv_k, s); break;
    case 32: e = launch_prologue_dk<32>(pre, (const __bf16 *)a.conv_w, ab, a.A, a.b_alpha, post, alpha, beta, M, a.T, (int)H, (int)nqkv, (int)a.conv_k, s); break;
    case 64: e = launch_prologue_dk<64>(pre, (const __bf16 *)a.conv_w, ab, a.A, a.b_alpha, post, alpha, beta, M, a.T, (int)H, (int)nqkv, (int)a.conv_k, s); break;
    case 128: e = launch_prologue_dk<128>(pre, (const __bf16 *)a.conv_w, ab, a.A, a.b_alpha, post, alpha, beta, M, a.T, (int)H, (int)nqkv, (int)a.conv_k, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e) return e;

    PrefillArgs p{};
    p.q = post; p.k = post + H * Dk; p.v = post + 2 * H * Dk;
    p.alpha = alpha; p.beta = beta; p.s0 = a.s0; p.y = y; p.sT = a.sT;
    p.B = a.B; p.T = a.T; p.H = H; p.Dk = Dk; p.Dv = Dv; p.chunk = a.chunk;
    p.q_tok_stride = nqkv; p.k_tok_stride = nqkv; p.v_tok_stride = nqkv;
    p.bf16 = false;
    p.ws = ws + w.rec;        // per-chunk records: the two-kernel fp32 core
    p.hilo_core = true;       // the layer's bound is the bf16 one
    // z = x W_gate^T is needed only by the epilogue: its tiles share the core's
    // launch and run on the compute units the core's slices leave free (H * Dv
    // / 16 of them); else it is a launch of its own before the core
    const PrefillArgs::SideGemm gate{x, (const __bf16 *)a.W_gate, z, M, H * Dv, hidden, hidden, hidden, H * Dv};
    if (prefill_f32_takes_side(p)) {
        p.side = &gate;
    } else if ((e = project<__bf16>(x, (const __bf16 *)a.W_gate, z, M, H * Dv, hidden, hidden, hidden, H * Dv, s))) {
        return e;
    }
    if ((e = launch_prefill(p, s))) return e;

    switch (Dv) {
    case 16: e = launch_epilogue_dv<16>(y, z, a.norm_gamma, g, M, (int)H, s); break;
    case 32: e = launch_epilogue_dv<32>(y, z, a.norm_gamma, g, M, (int)H, s); break;
    case 64: e = launch_epilogue_dv<64>(y, z, a.norm_gamma, g, M, (int)H, s); break;
    case 128: e = launch_epilogue_dv<128>(y, z, a.norm_gamma, g, M, (int)H, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e) return e;
    return project<float>(g, (const __bf16 *)a.W_o, a.out, M, hidden, H * Dv, H * Dv, H * Dv, hidden, s);
}

hipError_t launch_layer_decode(const LayerDecodeArgs &a, hipStream_t s)
{
    const int64_t N = a.N, H = a.H, Dk = a.Dk, Dv = a.Dv, hidden = a.hidden;
    if (N == 0 || H == 0) return hipSuccess;
    const WsLayout w = ws_layout(N, 1, H, Dk, Dv, false);
    char *ws = static_cast<char *>(a.ws);
    float *pre = reinterpret_cast<float *>(ws + w.pre);
    float *post = reinterpret_cast<float *>(ws + w.post);
    __bf16 *z = reinterpret_cast<__bf16 *>(ws + w.z);
    float *ab = reinterpret_cast<float *>(ws + w.ab);
    float *alpha = reinterpret_cast<float *>(ws + w.alpha);
    float *beta = reinterpret_cast<float *>(ws + w.beta);
    float *y = reinterpret_cast<float *>(ws + w.y);
    __bf16 *g = reinterpret_cast<__bf16 *>(ws + w.g);
    const __bf16 *x = static_cast<const __bf16 *>(a.x);
    const int64_t nqkv = H * (2 * Dk + Dv);
    hipError_t e;

    // q|k|v and a|b in one launch (the same x, fp32 out): at M = N the launch is
    // one round of small tiles, bound by its K steps, so a|b comes at no cost
    if ((e = project<float>(x, (const __bf16 *)a.W_qkv, pre, N, nqkv, hidden, hidden, hidden, nqkv, s,
                            (const __bf16 *)a.W_ab, ab, 2 * H, hidden, 2 * H)))
        return e;
    if ((e = project<__bf16>(x, (const __bf16 *)a.W_gate, z, N, H * Dv, hidden, hidden, hidden, H * Dv, s)))
        return e;

    const __bf16 *cw = (const __bf16 *)a.conv_w;
    switch (Dk) {
    case 16: e = launch_decode_prologue_dk<16>(pre, cw, ab, a.A, a.b_alpha, a.conv_state, post, alpha, beta, N, (int)H, (int)nqkv, (int)a.conv_k, s); break;
    case 32: e = launch_decode_prologue_dk<32>(pre, cw, ab, a.A, a.b_alpha, a.conv_state, post, alpha, beta, N, (int)H, (int)nqkv, (int)a.conv_k, s); break;
    case 64: e = launch_decode_prologue_dk<64>(pre, cw, ab, a.A, a.b_alpha, a.conv_state, post, alpha, beta, N, (int)H, (int)nqkv, (int)a.conv_k, s); break;
    case 128: e = launch_decode_prologue_dk<128>(pre, cw, ab, a.A, a.b_alpha, a.conv_state, post, alpha, beta, N, (int)H, (int)nqkv, (int)a.conv_k, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e) return e;

    DecodeArgs d{};
    d.q = post; d.k = post + H * Dk; d.v = post + 2 * H * Dk;
    d.alpha = alpha; d.beta = beta; d.state = a.state; d.y = y;
    d.N = N; d.H = H; d.Dk = Dk; d.Dv = Dv; d.bf16 = false;
    d.q_seq_stride = nqkv; d.k_seq_stride = nqkv; d.v_seq_stride = nqkv;
    if ((e = launch_decode(d, s))) return e;

    switch (Dv) {
    case 16: e = launch_epilogue_dv<16>(y, z, a.norm_gamma, g, N, (int)H, s); break;
    case 32: e = launch_epilogue_dv<32>(y, z, a.norm_gamma, g, N, (int)H, s); break;
    case 64: e = launch_epilogue_dv<64>(y, z, a.norm_gamma, g, N, (int)H, s); break;
    case 128: e = launch_epilogue_dv<128>(y, z, a.norm_gamma, g, N, (int)H, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e) return e;
    return project<float>(g, (const __bf16 *)a.W_o, a.out, N, hidden, H * Dv, H * Dv, H * Dv, hidden, s);
}

}  // namespace gdn
