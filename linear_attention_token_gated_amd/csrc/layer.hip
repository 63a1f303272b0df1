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
__global__ __launch_bounds__(64 * NW, BM == 256 ? 1 : 2) void gemm_nt_kernel(const __bf16 *__restrict__ A, int M,
                                                                              int K, int64_t lda,
                                                                              GemmProducts<OutT> P, int tiles_m,
                                                                              int tiles_n, int bn_log, int ksteps)
{
    __shared__ __attribute__((aligned(1024))) char smem[ST * GemmTile<BM, BN, NW>::STAGE];
    GemmSplit sp;
    sp.steps = ksteps;
    sp.split = (int)blockIdx.y;
    gemm_nt_block<OutT, BM, BN, ST, NW>((int)blockIdx.x, smem, A, M, K, lda, P, tiles_m, tiles_n, bn_log, sp);
}

// C_p = A B_p^T for up to three products of one A [M, K] in one launch.
// nsplit = 2: K in two halves of whole K steps (K of at least two steps),
// each writing a partial product, the second at C_p + M * ldc_p; the caller
// adds them (first + second).
template <typename OutT, int BM, int BN, int ST, int NW = 4>
hipError_t gemm_nt_tile(const __bf16 *A, int64_t M, int64_t K, int64_t lda, const GemmOp<OutT> &p0,
                        const GemmOp<OutT> &p1, const GemmOp<OutT> &p2, hipStream_t s, int nsplit = 1)
{
    const GemmGrid<BM, BN> g(M, p0.N, p1.B ? p1.N : 0, p2.B ? p2.N : 0);
    const int ntk = (int)((K + GBK - 1) / GBK);
    const int steps = nsplit == 2 ? (ntk + 1) / 2 : 0;
    if (nsplit == 2 && ntk < 2) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_nt_kernel<OutT, BM, BN, ST, NW>), dim3((unsigned)g.grid, nsplit == 2 ? 2u : 1u),
                       dim3(64 * NW), 0, s, A, (int)M, (int)K, lda, gemm_products(g, p0, p1, p2), g.tiles_m,
                       g.tiles_n, g.bn_log, steps);
    return hipGetLastError();
}

// C[M, N] = A[M, K] B[N, K]^T, with up to two more products of the same A in
// the same launch.  The tile is the largest that still gives every compute
// unit a workgroup (256 x 256, 128 x 128, else 64 x 64).  Small tiles do little
// MFMA work per K step, so they keep 7 steps in flight (8 stages, 64 KB of LDS)
// against the memory latency; the larger ones 3.  Where 64 x 64 tiles would
// outnumber the compute units but 64 x 128 tiles would not (a few hundred
// rows, thousands of columns), the wider tile runs the product in one round,
// one workgroup per CU: its K steps are latency-bound, so two workgroups
// sharing a CU take twice as long.  Where even 64 x 128 tiles outnumber the
// compute units (the decode step's three in-projections at once, 260 tiles),
// they keep 3 steps in flight in 48 KB, so three fit on a CU and the launch
// is still one round.
template <typename OutT>
hipError_t project(const __bf16 *A, int64_t M, int64_t K, int64_t lda, const GemmOp<OutT> &p0, hipStream_t s,
                   const GemmOp<OutT> &p1 = {}, const GemmOp<OutT> &p2 = {})
{
    const int64_t N1 = p0.N, N2 = p1.B ? p1.N : 0, N3 = p2.B ? p2.N : 0;
    if (M == 0 || N1 + N2 + N3 == 0) return hipSuccess;
    auto tiles = [&](int64_t bm, int64_t bn) {
        return ((M + bm - 1) / bm) * ((N1 + bn - 1) / bn + (N2 + bn - 1) / bn + (N3 + bn - 1) / bn);
    };
    if (tiles(256, 256) >= 256) return gemm_nt_tile<OutT, 256, 256, 4, 8>(A, M, K, lda, p0, p1, p2, s);
    if (tiles(128, 128) >= 256) return gemm_nt_tile<OutT, 128, 128, 4>(A, M, K, lda, p0, p1, p2, s);
    if (tiles(64, 64) > 256 && tiles(64, 128) <= 256) return gemm_nt_tile<OutT, 64, 128, 8>(A, M, K, lda, p0, p1, p2, s);
    if (tiles(64, 128) > 256 && tiles(64, 128) <= 3 * 256)
        return gemm_nt_tile<OutT, 64, 128, 4>(A, M, K, lda, p0, p1, p2, s);
    return gemm_nt_tile<OutT, 64, 64, 8>(A, M, K, lda, p0, p1, p2, s);
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
// Layer decode step, everything between the in-projections and the
// out-projection for one (sequence n, head h) in one workgroup:
//   1. causal conv of this head's q, k, v channels over the conv history and
//      this token's in-projection row; the history (conv_state row r of
//      sequence n holds the in-projection of token t - (conv_k - 1 - r), oldest
//      first) shifted by one row in place; L2 norm of q and k; alpha by eq (10)
//      and beta by eq (9)
//   2. eqs (1)-(4) for one token on the stored fp32 state (read once, written
//      once; the same arithmetic as the decode kernel)
//   3. zero-centred RMSNorm of y over Dv with gain (1 + gamma), times
//      sigmoid(z), written as the bf16 operand of W_o (eq (11))
// The state's loads are issued first and land while steps 1 and 2 begin.
// The first (2 Dk + Dv) / 4 threads own 4 channels each (q, then k, then v; a
// q or k head is Dk / 4 aligned lanes of one wavefront, reduced with
// xor-shuffles).
// ---------------------------------------------------------------------------
// Threads of the step: each owns 4 consecutive columns (one float4) of RPT
// rows of the Dk x Dv state, four rows each up to 1024 threads, so a wavefront
// reads and writes whole contiguous rows (the decode kernel's tiling).  WPE:
// waves per SIMD that two resident workgroups need, i.e. the register budget
// that keeps two on a CU, so one's loads stream while the other computes.
template <int DK, int DV> struct LayerDecodeShape {
    static constexpr int CG = DV / 4;
    static constexpr int TOTAL4 = DK * DV / 4;
    static constexpr int NT = TOTAL4 / 4 >= 1024 ? 1024 : (TOTAL4 / 4 < 64 ? (TOTAL4 < 64 ? TOTAL4 : 64) : TOTAL4 / 4);
    static constexpr int RG = NT / CG, RPT = DK / RG, NWAVE = (NT + 63) / 64;
    static constexpr int WPE = NT >= 1024 ? 8 : (NT >= 256 ? NT / 128 : 1);
    static_assert(NT % CG == 0 && DK % RG == 0, "decode tiling");
};

template <int DK, int DV, int KC>
__global__ __launch_bounds__((LayerDecodeShape<DK, DV>::NT), (LayerDecodeShape<DK, DV>::WPE)) void layer_decode_kernel(
    const float *__restrict__ pre, const float *__restrict__ ab, const float *__restrict__ zf,
    const __bf16 *__restrict__ conv_w, const float *__restrict__ Aexp, const float *__restrict__ b_alpha,
    const float *__restrict__ gamma, float *__restrict__ conv_state, float *__restrict__ state,
    __bf16 *__restrict__ g, int H, int nqkv)
{
    using Sh = LayerDecodeShape<DK, DV>;
    constexpr int CG = Sh::CG, RG = Sh::RG, RPT = Sh::RPT, NT = Sh::NT;
    // prologue threads: 4 channels each, in whole wavefronts (PW of them)
    constexpr int HVK = DK / 4, NV = (2 * DK + DV) / 4, PW = (NV + 63) / 64;
    static_assert(64 * PW <= NT && HVK <= 64 && CG <= 64, "prologue threads and y columns");
    const int64_t nh = blockIdx.x, n = nh / H;
    const int hh = (int)(nh % H);
    const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;

    __shared__ __attribute__((aligned(16))) float sk[DK], sq[DK], sv[DV];
    __shared__ f32x4 red_a[Sh::NWAVE][CG], red_b[Sh::NWAVE][CG];
    __shared__ float red_kq[Sh::NWAVE];
    __shared__ float s_ab[2];

    f32x4 *S4 = reinterpret_cast<f32x4 *>(state + nh * (int64_t)(DK * DV));
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = __builtin_nontemporal_load(S4 + (rg + RG * i) * CG + cg);
    f32x4 zv = zero4();
    // the projections arrive as two partial products over halves of K (the
    // second NH rows further on), added first + second
    const int64_t NH = (int64_t)gridDim.x * DV;
    if (rg == 0)
        zv = *reinterpret_cast<const f32x4 *>(zf + nh * DV + 4 * cg) +
             *reinterpret_cast<const f32x4 *>(zf + NH + nh * DV + 4 * cg);

    if (tid < 64 * PW) {
        // step 1: thread tid < NV owns channels c0 .. c0 + 3 of the q|k|v row
        const bool active = tid < NV;
        const int part = tid < HVK ? 0 : (tid < 2 * HVK ? 1 : 2);
        const int local = 4 * (tid - part * HVK);             // channel within this head's q, k or v
        const int c0 = active ? (part < 2 ? part * H * DK + hh * DK : 2 * H * DK + hh * DV) + local : 0;
        f32x4 rows[KC];                                       // taps 0 .. KC-1: history, then this token
#pragma unroll
        for (int j = 0; j < KC - 1; ++j) rows[j] = *reinterpret_cast<const f32x4 *>(conv_state + (n * (KC - 1) + j) * nqkv + c0);
        const int64_t npre = (int64_t)(gridDim.x / H) * nqkv;           // partial stride
        rows[KC - 1] = *reinterpret_cast<const f32x4 *>(pre + n * nqkv + c0) +
                       *reinterpret_cast<const f32x4 *>(pre + npre + n * nqkv + c0);
        __bf16 w[4 * KC];                                     // 4 KC consecutive taps, channel-major
        if constexpr (KC % 2 == 0) {
#pragma unroll
            for (int q = 0; q < KC / 2; ++q) {
                const bf16x8 v = *reinterpret_cast<const bf16x8 *>(conv_w + (int64_t)c0 * KC + 8 * q);
#pragma unroll
                for (int e = 0; e < 8; ++e) w[8 * q + e] = v[e];
            }
        } else {
#pragma unroll
            for (int q = 0; q < KC; ++q) {
                const bf16x4 v = *reinterpret_cast<const bf16x4 *>(conv_w + (int64_t)c0 * KC + 4 * q);
#pragma unroll
                for (int e = 0; e < 4; ++e) w[4 * q + e] = v[e];
            }
        }
        f32x4 o = zero4();
#pragma unroll
        for (int j = 0; j < KC; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = fmaf((float)w[e * KC + j], rows[j][e], o[e]);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) ss = fmaf(o[e], o[e], ss);
#pragma unroll
        for (int off = 1; off < HVK; off <<= 1) ss += __shfl_xor(ss, off);
        if (active) {
            const float scale = part < 2 ? 1.f / sqrtf(ss + kL2Eps) : 1.f;
            float *dst = part == 0 ? sq : (part == 1 ? sk : sv);
            *reinterpret_cast<f32x4 *>(dst + local) = o * scale;
#pragma unroll
            for (int r = 0; r < KC - 1; ++r)
                *reinterpret_cast<f32x4 *>(conv_state + (n * (KC - 1) + r) * nqkv + c0) = rows[r + 1];
        }
        if (tid == 63) {
            const int64_t nab = (int64_t)(gridDim.x / H) * 2 * H;
            const float a = ab[n * 2 * H + hh] + ab[nab + n * 2 * H + hh];
            const float bb = ab[n * 2 * H + H + hh] + ab[nab + n * 2 * H + H + hh];
            s_ab[0] = expf(-expf(Aexp[hh]) * softplusf_(a + b_alpha[hh]));
            s_ab[1] = sigmoidf_(bb);
        }
    }
    __syncthreads();

    // step 2: a = S^T k, b = S^T q, kq = k . q over this thread's rows, reduced
    // inside the wavefront (lanes CG apart), then across wavefronts through LDS
    f32x4 pa = zero4(), pb = zero4();
    float pkq = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        const float kr = sk[r], qr = sq[r];
        pa += s[i] * kr;
        pb += s[i] * qr;
        if (cg == 0) pkq += kr * qr;
    }
#pragma unroll
    for (int off = CG; off < 64 && off < NT; off <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pa[c] += __shfl_xor(pa[c], off);
            pb[c] += __shfl_xor(pb[c], off);
        }
        pkq += __shfl_xor(pkq, off);
    }
    const int lane = tid & 63, wave = tid >> 6;
    if (lane < CG) {
        red_a[wave][lane] = pa;
        red_b[wave][lane] = pb;
        if (lane == 0) red_kq[wave] = pkq;
    }
    __syncthreads();
    f32x4 Av = zero4(), Bq = zero4();
    float kq = 0.f;
#pragma unroll
    for (int w = 0; w < Sh::NWAVE; ++w) {
        Av += red_a[w][cg];
        Bq += red_b[w][cg];
        kq += red_kq[w];
    }
    const float a_t = s_ab[0], b_t = s_ab[1];
    const f32x4 vv = *reinterpret_cast<const f32x4 *>(&sv[4 * cg]);
    const f32x4 e = vv - a_t * Av;                 // eq (2) on the decayed state
    const f32x4 yv = a_t * Bq + (b_t * kq) * e;   // eq (4) on the updated state
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        const f32x4 sn = a_t * s[i] + (b_t * sk[r]) * e;   // eqs (1), (3)
        __builtin_nontemporal_store(sn, S4 + r * CG + cg);
    }

    // step 3: lanes 0 .. CG-1 of wavefront 0 hold y's columns 4 cg .. 4 cg + 3
    if (tid < 64) {
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) ss = fmaf(yv[c], yv[c], ss);
#pragma unroll
        for (int off = 1; off < CG; off <<= 1) ss += __shfl_xor(ss, off);
        if (rg == 0) {
            const float inv = 1.f / sqrtf(ss / (float)DV + kRmsEps);
            bf16x4 outv;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                // z as the layer's gate projection stores it (bf16)
                const float zb = (float)(__bf16)zv[c];
                outv[c] = (__bf16)(sigmoidf_(zb) * yv[c] * inv * (1.f + gamma[4 * cg + c]));
            }
            *reinterpret_cast<bf16x4 *>(g + nh * DV + 4 * cg) = outv;
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

template <int DK, int DV>
hipError_t launch_layer_decode_dv(const LayerDecodeArgs &a, const float *pre, const float *ab, const float *zf,
                                  __bf16 *g, int nqkv, hipStream_t s)
{
    const dim3 grid((unsigned)(a.N * a.H)), block(LayerDecodeShape<DK, DV>::NT);
    const __bf16 *cw = (const __bf16 *)a.conv_w;
    const int H = (int)a.H;
    switch (a.conv_k) {
    case 1: hipLaunchKernelGGL((layer_decode_kernel<DK, DV, 1>), grid, block, 0, s, pre, ab, zf, cw, a.A, a.b_alpha,
                               a.norm_gamma, a.conv_state, a.state, g, H, nqkv); break;
    case 2: hipLaunchKernelGGL((layer_decode_kernel<DK, DV, 2>), grid, block, 0, s, pre, ab, zf, cw, a.A, a.b_alpha,
                               a.norm_gamma, a.conv_state, a.state, g, H, nqkv); break;
    case 3: hipLaunchKernelGGL((layer_decode_kernel<DK, DV, 3>), grid, block, 0, s, pre, ab, zf, cw, a.A, a.b_alpha,
                               a.norm_gamma, a.conv_state, a.state, g, H, nqkv); break;
    case 4: hipLaunchKernelGGL((layer_decode_kernel<DK, DV, 4>), grid, block, 0, s, pre, ab, zf, cw, a.A, a.b_alpha,
                               a.norm_gamma, a.conv_state, a.state, g, H, nqkv); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int DK>
hipError_t launch_layer_decode_dk(const LayerDecodeArgs &a, const float *pre, const float *ab, const float *zf,
                                  __bf16 *g, int nqkv, hipStream_t s)
{
    switch (a.Dv) {
    case 16: return launch_layer_decode_dv<DK, 16>(a, pre, ab, zf, g, nqkv, s);
    case 32: return launch_layer_decode_dv<DK, 32>(a, pre, ab, zf, g, nqkv, s);
    case 64: return launch_layer_decode_dv<DK, 64>(a, pre, ab, zf, g, nqkv, s);
    case 128: return launch_layer_decode_dv<DK, 128>(a, pre, ab, zf, g, nqkv, s);
    }
    return hipErrorInvalidValue;
}

// Workspace of the decode step: the three in-projections (fp32, two partial
// products each over halves of K) and the gated norm (bf16, the
// out-projection's operand)
struct DecodeWs {
    size_t pre, ab, z, g, total;
};
DecodeWs decode_ws_layout(int64_t N, int64_t H, int64_t Dk, int64_t Dv)
{
    const size_t n = (size_t)N, nqkv = (size_t)(H * (2 * Dk + Dv));
    DecodeWs w;
    size_t o = 0;
    w.pre = o; o += al256(2 * n * nqkv * 4);
    w.ab = o;  o += al256(2 * n * (size_t)(2 * H) * 4);
    w.z = o;   o += al256(2 * n * (size_t)(H * Dv) * 4);
    w.g = o;   o += al256(n * (size_t)(H * Dv) * 2);
    w.total = o;
    return w;
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
    return decode_ws_layout(N, H, Dk, Dv).total;
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
    if ((e = project<float>(x, M, hidden, hidden, GemmOp<float>{(const __bf16 *)a.W_qkv, pre, nqkv, hidden, nqkv}, s)))
        return e;
    if ((e = project<float>(x, M, hidden, hidden, GemmOp<float>{(const __bf16 *)a.W_ab, ab, 2 * H, hidden, 2 * H}, s)))
        return e;

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
    } else if ((e = project<__bf16>(x, M, hidden, hidden,
                                    GemmOp<__bf16>{(const __bf16 *)a.W_gate, z, H * Dv, hidden, H * Dv}, s))) {
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
    return project<float>(g, M, H * Dv, H * Dv, GemmOp<float>{(const __bf16 *)a.W_o, a.out, hidden, H * Dv, hidden}, s);
}

hipError_t launch_layer_decode(const LayerDecodeArgs &a, hipStream_t s)
{
    const int64_t N = a.N, H = a.H, Dk = a.Dk, Dv = a.Dv, hidden = a.hidden;
    if (N == 0 || H == 0) return hipSuccess;
    const DecodeWs w = decode_ws_layout(N, H, Dk, Dv);
    char *ws = static_cast<char *>(a.ws);
    float *pre = reinterpret_cast<float *>(ws + w.pre);
    float *ab = reinterpret_cast<float *>(ws + w.ab);
    float *zf = reinterpret_cast<float *>(ws + w.z);
    __bf16 *g = reinterpret_cast<__bf16 *>(ws + w.g);
    const __bf16 *x = static_cast<const __bf16 *>(a.x);
    const int64_t nqkv = H * (2 * Dk + Dv);
    hipError_t e;

    // q|k|v, a|b and the gate z in one launch (the same x, fp32 out), K in two
    // halves: at M = N each product is a few rows of tiles bound by the
    // latency of their K steps (the weights arrive cold from HBM), so halving
    // the steps per workgroup and doubling the workgroups (128 x 128 tiles,
    // two per CU) shortens it; the decode kernel adds the two halves
    if ((e = gemm_nt_tile<float, 128, 128, 4>(x, N, hidden, hidden,
                                              GemmOp<float>{(const __bf16 *)a.W_qkv, pre, nqkv, hidden, nqkv},
                                              GemmOp<float>{(const __bf16 *)a.W_ab, ab, 2 * H, hidden, 2 * H},
                                              GemmOp<float>{(const __bf16 *)a.W_gate, zf, H * Dv, hidden, H * Dv},
                                              s, 2)))
        return e;
    switch (Dk) {
    case 16: e = launch_layer_decode_dk<16>(a, pre, ab, zf, g, (int)nqkv, s); break;
    case 32: e = launch_layer_decode_dk<32>(a, pre, ab, zf, g, (int)nqkv, s); break;
    case 64: e = launch_layer_decode_dk<64>(a, pre, ab, zf, g, (int)nqkv, s); break;
    case 128: e = launch_layer_decode_dk<128>(a, pre, ab, zf, g, (int)nqkv, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e) return e;
    return project<float>(g, N, H * Dv, H * Dv, GemmOp<float>{(const __bf16 *)a.W_o, a.out, hidden, H * Dv, hidden}, s);
}

}  // namespace gdn
