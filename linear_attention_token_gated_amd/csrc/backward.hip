// backward.hip -- reverse mode of the chunkwise gated delta rule on gfx950.
//
// Source: "On the Design of Qwen3.8-Next Architecture", picx.dev summary,
// "Theoretical foundations", eqs (1)-(4).  The forward chunk form (for a chunk
// of C tokens entering with state S, natural-log cumulative decay G, Gamma_rj =
// e^{G_r - G_j}, d_r = e^{G_C - G_r}):
//
//   A = strict_lower[beta_r Gamma_rj k_r.k_j],   T = (I + A)^-1
//   X = diag(beta) (V - diag(e^G) K S),           U = T X
//   Y = diag(e^G) Q S + P U,                       P = lower_incl[Gamma_rj q_r.k_j]
//   S' = e^{G_C} S + K^T diag(d) U
//
// Given dY = dL/dY for every token and dL/dS_T, the gradients come in four
// launches:
//
//   1. prep   (one workgroup per chunk): G, T, P and Ak = strict_lower[Gamma o K K^T]
//             into a per-chunk record;
//   2. states (one workgroup per 16 value columns of a head, chunks in order):
//             the state S_c entering every chunk;
//   3. adjoint states (same grid, chunks in reverse): dS'_c = dL/dS leaving
//             chunk c, from dS = e^{G_C} dS' + Q^T diag(e^G) dY - K^T diag(e^G) dR,
//             dR = diag(beta) T^T (P^T dY + diag(d) K dS');  dS_0 at the end;
//   4. chunk gradients (one workgroup per chunk, value columns in slices of 16):
//             with dU = P^T dY + diag(d) K dS' and dX = T^T dU,
//               dV = diag(beta) dX,   dP = dY U^T,   dA = -(dX U^T)
//               dQ = diag(e^G) dY S^T + (Gamma o dP) K
//               dK = -diag(e^G beta) dX S^T + diag(d) U dS'^T
//                    + (dKK + dKK^T) K + (Gamma o dP)^T Q,  dKK = Gamma o diag(beta) dA
//               dbeta_r = dX_r . W~_r + sum_j dA_rj Ak_rj      (W~ = V - diag(e^G) K S)
//             and the gradient of each G_r from every factor it enters, then
//             d ln alpha_i = sum_{r >= i} dG_r (within the chunk).
//
// Columns of S, dS', V, Y are independent in passes 2 and 3, so those carry a
// 16-column slice of the state in MFMA accumulators, like the forward.  All
// arithmetic is fp32 (16x16x4 fp32 MFMA); bf16 inputs are widened on load.
// Ragged tails are padded with identity tokens (alpha = 1, beta = 0, zeros),
// whose gradients are never written.
#include "common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int NT = 256;   // 4 wavefronts
constexpr int VP = BV + 4;   // LDS pitch of C x 16 slices (fp32)

struct BwdParams {
    const void *q, *k, *v;
    const float *alpha, *beta, *s0, *dy, *dsT;
    float *dq, *dk, *dv, *dalpha, *dbeta, *ds0;
    float *rec, *sc, *dsc;
    int64_t T, H, Dv, NC;
    int64_t rec_floats;
};

// ---- per-chunk record: T [C][C], P [C][C], Ak [C][C], G2 [C] (log2 cumulative decay)
template <int C> struct Rec {
    static constexpr int oT = 0, oP = C * C, oA = 2 * C * C, oG = 3 * C * C;
};

__device__ __forceinline__ f32x4 load4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ f32x4 load4(const __bf16 *p) {
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p);
    return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}

// Rows t = c0 .. c0+C-1 of head h of a [B, T, H, D] tensor into LDS (pitch P
// floats), zeros past T.
template <typename Tin, int C, int D, int P>
__device__ __forceinline__ void stage_rows(float *dst, const Tin *src, int64_t b, int64_t h, int64_t c0, int64_t T,
                                           int64_t H) {
    for (int i = threadIdx.x; i < C * D / 4; i += NT) {
        const int r = i / (D / 4), col = (i % (D / 4)) * 4;
        const int64_t t = c0 + r;
        f32x4 x = zero4();
        if (t < T) x = load4(src + ((b * T + t) * H + h) * D + col);
        *reinterpret_cast<f32x4 *>(dst + r * P + col) = x;
    }
}

// C x 16 slice (columns n0..n0+15) of rows c0.. of head h of a [B, T, H, Dv]
// tensor, into LDS with pitch VP.
template <typename Tin, int C>
__device__ __forceinline__ void stage_slice(float *dst, const Tin *src, int64_t b, int64_t h, int64_t c0, int64_t T,
                                            int64_t H, int64_t Dv, int n0) {
    for (int i = threadIdx.x; i < C * 4; i += NT) {
        const int r = i >> 2, col = (i & 3) * 4;
        const int64_t t = c0 + r;
        f32x4 x = zero4();
        if (t < T) x = load4(src + ((b * T + t) * H + h) * Dv + n0 + col);
        *reinterpret_cast<f32x4 *>(dst + r * VP + col) = x;
    }
}

// C x C matrix (dense, row-major) into LDS with pitch P
template <int C, int P>
__device__ __forceinline__ void stage_cc(float *dst, const float *src) {
    for (int i = threadIdx.x; i < C * C / 4; i += NT) {
        const int r = i / (C / 4), col = (i % (C / 4)) * 4;
        *reinterpret_cast<f32x4 *>(dst + r * P + col) = load4(src + r * C + col);
    }
}

// lower-triangle block index -> (rb, cb), row-major over rb
__device__ __forceinline__ void tri_block(int idx, int &rb, int &cb) {
    rb = 0;
    while ((rb + 1) * (rb + 2) / 2 <= idx) ++rb;
    cb = idx - rb * (rb + 1) / 2;
}

// sum over the 16 lanes of each 16-lane row
__device__ __forceinline__ float row16_sum(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}

// ===========================================================================
// 1. prep: G2, T = (I + A)^-1, P, Ak of one chunk
// ===========================================================================
template <typename Tin, int C, int DK>
__global__ __launch_bounds__(NT) void bwd_prep_kernel(BwdParams p)
{
    constexpr int KP = DK + 4, CP = C + 4, NB = C / 16, KSD = DK % 32 == 0 ? 32 : 16;
    constexpr int NTRI = NB * (NB + 1) / 2;
    __shared__ __attribute__((aligned(16))) float Ks[C * KP];
    __shared__ __attribute__((aligned(16))) float Qs[C * KP];
    __shared__ __attribute__((aligned(16))) float As[C * CP];
    __shared__ __attribute__((aligned(16))) float Ts[C * CP];
    __shared__ float Gs[C], Bs[C];

    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id(), ln = lane & 15, lg = lane >> 4;
    const int64_t bh = blockIdx.x / p.NC, c = blockIdx.x % p.NC;
    const int64_t H = p.H, T = p.T, b = bh / H, h = bh % H, c0 = c * C;
    float *rec = p.rec + (bh * p.NC + c) * p.rec_floats;

    stage_rows<Tin, C, DK, KP>(Ks, static_cast<const Tin *>(p.k), b, h, c0, T, H);
    stage_rows<Tin, C, DK, KP>(Qs, static_cast<const Tin *>(p.q), b, h, c0, T, H);
    if (wave == 0) {
        const int64_t t = c0 + lane;
        const bool ok = lane < C && t < T;
        const float g2 = ok ? __builtin_amdgcn_logf(p.alpha[(b * T + t) * H + h]) : 0.f;
        const float G2 = wave_inclusive_sum(g2, lane);
        if (lane < C) {
            Gs[lane] = G2;
            Bs[lane] = ok ? p.beta[(b * T + t) * H + h] : 0.f;
            rec[Rec<C>::oG + lane] = G2;
        }
    }
    // blocks above the diagonal: zero in the record and in T
    for (int i = tid; i < C * C; i += NT) {
        const int r = i / C, j = i % C;
        if (j / 16 > r / 16) {
            rec[Rec<C>::oP + i] = 0.f;
            rec[Rec<C>::oA + i] = 0.f;
            Ts[r * CP + j] = 0.f;
        }
    }
    __syncthreads();

    // Gram tiles on and below the diagonal: K K^T -> Ak, A;  Q K^T -> P
    for (int tile = wave; tile < 2 * NTRI; tile += 4) {
        const bool isQ = tile >= NTRI;
        int rb, cb;
        tri_block(isQ ? tile - NTRI : tile, rb, cb);
        const float *src = isQ ? Qs : Ks;
        f32x4 acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += KSD) {
            const Frag<float, KSD> a = frag_rows<float, KSD>(src, KP, 16 * rb, k0, lane);
            const Frag<float, KSD> bb = frag_rows<float, KSD>(Ks, KP, 16 * cb, k0, lane);
            acc = Frag<float, KSD>::mma(a, bb, acc);
        }
        const int j = 16 * cb + ln;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * lg + e;
            const float gam = __builtin_amdgcn_exp2f(fminf(Gs[r] - Gs[j], 0.f));
            if (isQ) {
                rec[Rec<C>::oP + r * C + j] = r >= j ? gam * acc[e] : 0.f;
            } else {
                const float ak = r > j ? gam * acc[e] : 0.f;
                rec[Rec<C>::oA + r * C + j] = ak;
                As[r * CP + j] = Bs[r] * ak;
            }
        }
    }
    __syncthreads();

    // diagonal blocks of T by forward substitution
    if (wave < NB) {
        const int blk = wave;
        float Lr[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) Lr[s] = As[(16 * blk + ln) * CP + 16 * blk + s];
        float X[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) X[i] = (ln == lg + 4 * i) ? 1.f : 0.f;
        tri_solve16(X, Lr, ln, std::make_integer_sequence<int, 15>{});
#pragma unroll
        for (int i = 0; i < 4; ++i) Ts[(16 * blk + ln) * CP + 16 * blk + lg + 4 * i] = X[i];
    }
    __syncthreads();

    // blocks below the diagonal, one block row at a time:
    // T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
#pragma unroll
    for (int i = 1; i < NB; ++i) {
        if (wave < i) {
            const int j = wave;
            f32x4 z = zero4();
            for (int kb = j; kb < i; ++kb) {
                const Frag<float, 16> a = frag_rows<float, 16>(As, CP, 16 * i, 16 * kb, lane);
                const Frag<float, 16> t = frag_cols<float, 16>(Ts, CP, 16 * j, 16 * kb, lane);
                z = Frag<float, 16>::mma(a, t, z);
            }
            Frag<float, 16> zf;   // accumulator layout is the B layout for KS = 16
#pragma unroll
            for (int e = 0; e < 4; ++e) zf.v[e] = z[e];
            const Frag<float, 16> tii = frag_rows<float, 16>(Ts, CP, 16 * i, 16 * i, lane);
            const f32x4 o = Frag<float, 16>::mma(tii, zf, zero4());
#pragma unroll
            for (int e = 0; e < 4; ++e) Ts[(16 * i + 4 * lg + e) * CP + 16 * j + ln] = -o[e];
        }
        __syncthreads();
    }

    for (int i = tid; i < C * C / 4; i += NT) {
        const int r = i / (C / 4), col = (i % (C / 4)) * 4;
        *reinterpret_cast<f32x4 *>(rec + Rec<C>::oT + r * C + col) = *reinterpret_cast<const f32x4 *>(Ts + r * CP + col);
    }
}

// ===========================================================================
// 2./3. state passes over a 16-column slice of one head
// ===========================================================================
template <typename Tin, int C, int DK, bool ADJ> struct CarryLay {
    static constexpr int KP = DK + 4, CP = C + 4;
    static constexpr size_t oK = 0;
    static constexpr size_t oQ = oK + 4 * C * KP;
    static constexpr size_t oT = oQ + (ADJ ? 4 * C * KP : 0);
    static constexpr size_t oP = oT + 4 * C * CP;
    static constexpr size_t oST = oP + (ADJ ? 4 * C * CP : 0);
    static constexpr size_t oIn = oST + 4 * BV * KP;
    static constexpr size_t oX = oIn + 4 * C * VP;
    static constexpr size_t oUd = oX + 4 * C * VP;
    static constexpr size_t oYb = oUd + 4 * BV * CP;
    static constexpr size_t oG = oYb + (ADJ ? 4 * BV * CP : 0);
    static constexpr size_t oB = oG + 4 * C;
    static constexpr size_t BYTES = oB + 4 * C;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <typename Tin, int C, int DK, bool ADJ>
__global__ __launch_bounds__(NT) void bwd_carry_kernel(BwdParams p)
{
    using L = CarryLay<Tin, C, DK, ADJ>;
    constexpr int KP = L::KP, CP = L::CP, NB = C / 16, NKB = DK / 16, MS = (NKB + 3) / 4;
    constexpr int KSD = DK % 32 == 0 ? 32 : 16, KSC = C % 32 == 0 ? 32 : 16;
    using FD = Frag<float, KSD>;
    using FC = Frag<float, KSC>;
    using F16 = Frag<float, 16>;

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    float *Ks = reinterpret_cast<float *>(smem + L::oK);
    float *Qs = reinterpret_cast<float *>(smem + L::oQ);
    float *Ts = reinterpret_cast<float *>(smem + L::oT);
    float *Ps = reinterpret_cast<float *>(smem + L::oP);
    float *STs = reinterpret_cast<float *>(smem + L::oST);
    float *Ins = reinterpret_cast<float *>(smem + L::oIn);
    float *Xs = reinterpret_cast<float *>(smem + L::oX);
    float *UdT = reinterpret_cast<float *>(smem + L::oUd);
    float *YbT = reinterpret_cast<float *>(smem + L::oYb);
    float *Gs = reinterpret_cast<float *>(smem + L::oG);
    float *Bs = reinterpret_cast<float *>(smem + L::oB);

    const int lane = lane_id(), wave = wave_id(), ln = lane & 15, lg = lane >> 4;
    const int64_t NS = p.Dv / BV;
    const int64_t bh = blockIdx.x / NS, sl = blockIdx.x % NS;
    const int64_t H = p.H, T = p.T, Dv = p.Dv, NC = p.NC, b = bh / H, h = bh % H;
    const int n0 = (int)sl * BV;

    f32x4 S[MS];
    const float *init = ADJ ? p.dsT : p.s0;
#pragma unroll
    for (int m = 0; m < MS; ++m) {
        S[m] = zero4();
        const int ib = wave + 4 * m;
        if (ib < NKB && init) {
#pragma unroll
            for (int e = 0; e < 4; ++e) S[m][e] = init[(bh * DK + 16 * ib + 4 * lg + e) * Dv + n0 + ln];
        }
    }

    for (int64_t it = 0; it < NC; ++it) {
        const int64_t c = ADJ ? NC - 1 - it : it;
        const int64_t c0 = c * C;
        const float *rec = p.rec + (bh * NC + c) * p.rec_floats;

        // keep the state at this chunk boundary for the chunk-gradient pass,
        // and stage it transposed as the B operand of K S
        float *keep = (ADJ ? p.dsc : p.sc) + (bh * NC + c) * DK * Dv;
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int ib = wave + 4 * m;
            if (ib < NKB) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * ib + 4 * lg + e;
                    keep[row * Dv + n0 + ln] = S[m][e];
                    STs[ln * KP + row] = S[m][e];
                }
            }
        }
        stage_rows<Tin, C, DK, KP>(Ks, static_cast<const Tin *>(p.k), b, h, c0, T, H);
        stage_cc<C, CP>(Ts, rec + Rec<C>::oT);
        if constexpr (ADJ) {
            stage_rows<Tin, C, DK, KP>(Qs, static_cast<const Tin *>(p.q), b, h, c0, T, H);
            stage_cc<C, CP>(Ps, rec + Rec<C>::oP);
            stage_slice<float, C>(Ins, p.dy, b, h, c0, T, H, Dv, n0);
        } else {
            stage_slice<Tin, C>(Ins, static_cast<const Tin *>(p.v), b, h, c0, T, H, Dv, n0);
        }
        for (int i = threadIdx.x; i < C; i += NT) {
            const int64_t t = c0 + i;
            Gs[i] = rec[Rec<C>::oG + i];
            Bs[i] = t < T ? p.beta[(b * T + t) * H + h] : 0.f;
        }
        __syncthreads();
        const float GC = Gs[C - 1];

        // step 1: K S (per 16-token block); forward: X = diag(beta)(V - e^G K S);
        // adjoint: dU = P^T dY + diag(d) K dS'
        if (wave < NB) {
            const int rb = wave;
            f32x4 ks = zero4();
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += KSD)
                ks = FD::mma(frag_rows<float, KSD>(Ks, KP, 16 * rb, k0, lane),
                             frag_rows<float, KSD>(STs, KP, 0, k0, lane), ks);
            if constexpr (ADJ) {
                f32x4 acc;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * lg + e;
                    acc[e] = __builtin_amdgcn_exp2f(GC - Gs[r]) * ks[e];
                    YbT[ln * CP + r] = __builtin_amdgcn_exp2f(Gs[r]) * Ins[r * VP + ln];
                }
                for (int kb = rb; kb < NB; ++kb)
                    acc = F16::mma(frag_cols<float, 16>(Ps, CP, 16 * rb, 16 * kb, lane),
                                   frag_cols<float, 16>(Ins, VP, 0, 16 * kb, lane), acc);
#pragma unroll
                for (int e = 0; e < 4; ++e) Xs[(16 * rb + 4 * lg + e) * VP + ln] = acc[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * lg + e;
                    Xs[r * VP + ln] = Bs[r] * (Ins[r * VP + ln] - __builtin_amdgcn_exp2f(Gs[r]) * ks[e]);
                }
            }
        }
        __syncthreads();

        // step 2: forward: U = T X, stored as d o U (transposed);
        // adjoint: dR = diag(beta) T^T dU, stored as -e^G o dR (transposed)
        if (wave < NB) {
            const int rb = wave;
            f32x4 acc = zero4();
            if constexpr (ADJ) {
                for (int kb = rb; kb < NB; ++kb)
                    acc = F16::mma(frag_cols<float, 16>(Ts, CP, 16 * rb, 16 * kb, lane),
                                   frag_cols<float, 16>(Xs, VP, 0, 16 * kb, lane), acc);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * lg + e;
                    UdT[ln * CP + r] = -__builtin_amdgcn_exp2f(Gs[r]) * Bs[r] * acc[e];
                }
            } else {
                for (int kb = 0; kb <= rb; ++kb)
                    acc = F16::mma(frag_rows<float, 16>(Ts, CP, 16 * rb, 16 * kb, lane),
                                   frag_cols<float, 16>(Xs, VP, 0, 16 * kb, lane), acc);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * lg + e;
                    UdT[ln * CP + r] = __builtin_amdgcn_exp2f(GC - Gs[r]) * acc[e];
                }
            }
        }
        __syncthreads();

        // step 3: S <- e^{G_C} S + K^T UdT (+ Q^T (e^G o dY) for the adjoint)
        const float eGC = __builtin_amdgcn_exp2f(GC);
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int ib = wave + 4 * m;
            if (ib < NKB) {
                f32x4 acc = S[m] * eGC;
#pragma unroll
                for (int j0 = 0; j0 < C; j0 += KSC) {
                    acc = FC::mma(frag_cols<float, KSC>(Ks, KP, 16 * ib, j0, lane),
                                  frag_rows<float, KSC>(UdT, CP, 0, j0, lane), acc);
                    if constexpr (ADJ)
                        acc = FC::mma(frag_cols<float, KSC>(Qs, KP, 16 * ib, j0, lane),
                                      frag_rows<float, KSC>(YbT, CP, 0, j0, lane), acc);
                }
                S[m] = acc;
            }
        }
        __syncthreads();
    }

    if constexpr (ADJ) {
        if (p.ds0) {
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int ib = wave + 4 * m;
                if (ib < NKB) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) p.ds0[(bh * DK + 16 * ib + 4 * lg + e) * Dv + n0 + ln] = S[m][e];
                }
            }
        }
    }
}

// ===========================================================================
// 4. chunk gradients
// ===========================================================================
template <int C, int DK> struct GradLay {
    static constexpr int KP = DK + 4, CP = C + 4, NB = C / 16;
    static constexpr size_t oK = 0;
    static constexpr size_t oQ = oK + 4 * C * KP;
    static constexpr size_t oT = oQ + 4 * C * KP;          // T, then dKK
    static constexpr size_t oP = oT + 4 * C * CP;          // P, then dQK
    // S slice [DK][VP] and dS' slice [DK][VP]; Ak [C][CP] over both after the slices
    static constexpr size_t SREG = 2 * DK * VP > C * CP ? 2 * DK * VP : C * CP;
    static constexpr size_t oS = oP + 4 * C * CP;
    static constexpr size_t oDS = oS + 4 * DK * VP;
    static constexpr size_t oDY = oS + 4 * SREG;
    static constexpr size_t oX = oDY + 4 * C * VP;
    static constexpr size_t oU = oX + 4 * C * VP;
    static constexpr size_t oDU = oU + 4 * C * VP;
    static constexpr size_t oDX = oDU + 4 * C * VP;
    static constexpr size_t oG = oDX + 4 * C * VP;
    static constexpr size_t oB = oG + 4 * C;
    static constexpr size_t oAl = oB + 4 * C;
    static constexpr size_t oTG = oAl + 4 * C;             // per-token dG partials
    static constexpr size_t oTB = oTG + 4 * C;             // per-token dbeta partials
    static constexpr size_t oRP = oTB + 4 * C;                 // [2][NB][NB][16] row sums (P part, A part)
    static constexpr size_t oCP = oRP + 4 * 2 * NB * NB * 16;  // [2][NB][NB][16] column sums
    static constexpr size_t oRB = oCP + 4 * 2 * NB * NB * 16;  // [NB][NB][16] dbeta row sums
    static constexpr size_t oRed = oRB + 4 * NB * NB * 16;
    static constexpr size_t BYTES = oRed + 4 * 8;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <typename Tin, int C, int DK>
__global__ __launch_bounds__(NT) void bwd_chunk_kernel(BwdParams p)
{
    using L = GradLay<C, DK>;
    constexpr int KP = L::KP, CP = L::CP, NB = C / 16, NKB = DK / 16;
    constexpr int KSD = DK % 32 == 0 ? 32 : 16;
    constexpr int NTRI = NB * (NB + 1) / 2;
    constexpr int NCC = (2 * NTRI + 3) / 4;            // C x C tiles per wave (dP, dM)
    constexpr int NTILE = NB * NKB, NCK = (NTILE + 3) / 4;   // C x DK tiles per wave
    using FD = Frag<float, KSD>;
    using F16 = Frag<float, 16>;

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    float *Ks = reinterpret_cast<float *>(smem + L::oK);
    float *Qs = reinterpret_cast<float *>(smem + L::oQ);
    float *Ts = reinterpret_cast<float *>(smem + L::oT);
    float *Ps = reinterpret_cast<float *>(smem + L::oP);
    float *Ss = reinterpret_cast<float *>(smem + L::oS);
    float *dSs = reinterpret_cast<float *>(smem + L::oDS);
    float *dYs = reinterpret_cast<float *>(smem + L::oDY);
    float *Xs = reinterpret_cast<float *>(smem + L::oX);
    float *Us = reinterpret_cast<float *>(smem + L::oU);
    float *dUs = reinterpret_cast<float *>(smem + L::oDU);
    float *dXs = reinterpret_cast<float *>(smem + L::oDX);
    float *Gs = reinterpret_cast<float *>(smem + L::oG);
    float *Bs = reinterpret_cast<float *>(smem + L::oB);
    float *Als = reinterpret_cast<float *>(smem + L::oAl);
    float *tokG = reinterpret_cast<float *>(smem + L::oTG);
    float *tokB = reinterpret_cast<float *>(smem + L::oTB);
    float *rowE = reinterpret_cast<float *>(smem + L::oRP);
    float *colE = reinterpret_cast<float *>(smem + L::oCP);
    float *rowB = reinterpret_cast<float *>(smem + L::oRB);
    float *red = reinterpret_cast<float *>(smem + L::oRed);
    float *Aks = Ss;   // after the slice loop

    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id(), ln = lane & 15, lg = lane >> 4;
    const int64_t bh = blockIdx.x / p.NC, c = blockIdx.x % p.NC;
    const int64_t H = p.H, T = p.T, Dv = p.Dv, b = bh / H, h = bh % H, c0 = c * C;
    const float *rec = p.rec + (bh * p.NC + c) * p.rec_floats;
    const float *Sg = p.sc + (bh * p.NC + c) * DK * Dv;
    const float *dSg = p.dsc + (bh * p.NC + c) * DK * Dv;
    const Tin *vg = static_cast<const Tin *>(p.v);

    stage_rows<Tin, C, DK, KP>(Ks, static_cast<const Tin *>(p.k), b, h, c0, T, H);
    stage_rows<Tin, C, DK, KP>(Qs, static_cast<const Tin *>(p.q), b, h, c0, T, H);
    stage_cc<C, CP>(Ts, rec + Rec<C>::oT);
    stage_cc<C, CP>(Ps, rec + Rec<C>::oP);
    for (int i = tid; i < C; i += NT) {
        const int64_t t = c0 + i;
        const bool ok = t < T;
        Gs[i] = rec[Rec<C>::oG + i];
        Bs[i] = ok ? p.beta[(b * T + t) * H + h] : 0.f;
        Als[i] = ok ? p.alpha[(b * T + t) * H + h] : 1.f;
    }

    // accumulators over the value slices
    f32x4 dQa[NCK], dKa[NCK], dKb[NCK], dPM[NCC];
#pragma unroll
    for (int m = 0; m < NCK; ++m) dQa[m] = dKa[m] = dKb[m] = zero4();
#pragma unroll
    for (int m = 0; m < NCC; ++m) dPM[m] = zero4();
    f32x4 pG = zero4(), pB = zero4();   // per-token partials of this wave's rows
    float pGC = 0.f, pSS = 0.f;

    for (int n0 = 0; n0 < Dv; n0 += BV) {
        // ---- stage S, dS' slices and the dY slice
        for (int i = tid; i < DK * 4; i += NT) {
            const int r = i >> 2, col = (i & 3) * 4;
            const f32x4 s = load4(Sg + r * Dv + n0 + col);
            const f32x4 ds = load4(dSg + r * Dv + n0 + col);
            *reinterpret_cast<f32x4 *>(Ss + r * VP + col) = s;
            *reinterpret_cast<f32x4 *>(dSs + r * VP + col) = ds;
            pSS += s[0] * ds[0] + s[1] * ds[1] + s[2] * ds[2] + s[3] * ds[3];
        }
        stage_slice<float, C>(dYs, p.dy, b, h, c0, T, H, Dv, n0);
        __syncthreads();
        const float GC = Gs[C - 1];

        // ---- A: K S, Q S, K dS' of this wave's token block; X = beta W~
        f32x4 KS = zero4(), QS = zero4(), KD = zero4(), Wt = zero4();
        if (wave < NB) {
            const int rb = wave;
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += KSD) {
                const FD kf = frag_rows<float, KSD>(Ks, KP, 16 * rb, k0, lane);
                const FD qf = frag_rows<float, KSD>(Qs, KP, 16 * rb, k0, lane);
                const FD sf = frag_cols<float, KSD>(Ss, VP, 0, k0, lane);
                const FD df = frag_cols<float, KSD>(dSs, VP, 0, k0, lane);
                KS = FD::mma(kf, sf, KS);
                QS = FD::mma(qf, sf, QS);
                KD = FD::mma(kf, df, KD);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * lg + e;
                const int64_t t = c0 + r;
                const float vv = t < T ? to_f32(vg[((b * T + t) * H + h) * Dv + n0 + ln]) : 0.f;
                Wt[e] = vv - __builtin_amdgcn_exp2f(Gs[r]) * KS[e];
                Xs[r * VP + ln] = Bs[r] * Wt[e];
            }
        }
        __syncthreads();

        // ---- B: U = T X;  dU = P^T dY + d o K dS'
        if (wave < NB) {
            const int rb = wave;
            f32x4 U = zero4(), dU;
            for (int kb = 0; kb <= rb; ++kb)
                U = F16::mma(frag_rows<float, 16>(Ts, CP, 16 * rb, 16 * kb, lane),
                             frag_cols<float, 16>(Xs, VP, 0, 16 * kb, lane), U);
#pragma unroll
            for (int e = 0; e < 4; ++e) dU[e] = __builtin_amdgcn_exp2f(GC - Gs[16 * rb + 4 * lg + e]) * KD[e];
            for (int kb = rb; kb < NB; ++kb)
                dU = F16::mma(frag_cols<float, 16>(Ps, CP, 16 * rb, 16 * kb, lane),
                              frag_cols<float, 16>(dYs, VP, 0, 16 * kb, lane), dU);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * lg + e;
                Us[r * VP + ln] = U[e];
                dUs[r * VP + ln] = dU[e];
                const float dr = __builtin_amdgcn_exp2f(GC - Gs[r]), br = __builtin_amdgcn_exp2f(Gs[r]);
                const float s3 = U[e] * KD[e];
                pG[e] += br * dYs[r * VP + ln] * QS[e] - dr * s3;
                pGC += dr * s3;
            }
        }
        __syncthreads();

        // ---- C: dX = T^T dU;  dV = beta dX
        if (wave < NB) {
            const int rb = wave;
            f32x4 dX = zero4();
            for (int kb = rb; kb < NB; ++kb)
                dX = F16::mma(frag_cols<float, 16>(Ts, CP, 16 * rb, 16 * kb, lane),
                              frag_cols<float, 16>(dUs, VP, 0, 16 * kb, lane), dX);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * lg + e;
                const int64_t t = c0 + r;
                dXs[r * VP + ln] = dX[e];
                const float dW = Bs[r] * dX[e];
                if (t < T) p.dv[((b * T + t) * H + h) * Dv + n0 + ln] = dW;
                pG[e] -= __builtin_amdgcn_exp2f(Gs[r]) * dW * KS[e];
                pB[e] += dX[e] * Wt[e];
            }
        }
        __syncthreads();

        // ---- D: dP += dY U^T, dM += dX U^T (lower blocks);
        //         dQa += dY S^T, dKa += dX S^T, dKb += U dS'^T
#pragma unroll
        for (int m = 0; m < NCC; ++m) {
            const int tile = wave + 4 * m;
            if (tile < 2 * NTRI) {
                const bool isM = tile >= NTRI;
                int rb, jb;
                tri_block(isM ? tile - NTRI : tile, rb, jb);
                dPM[m] = F16::mma(frag_rows<float, 16>(isM ? dXs : dYs, VP, 16 * rb, 0, lane),
                                  frag_rows<float, 16>(Us, VP, 16 * jb, 0, lane), dPM[m]);
            }
        }
#pragma unroll
        for (int m = 0; m < NCK; ++m) {
            const int tile = wave + 4 * m;
            if (tile < NTILE) {
                const int rb = tile / NKB, kb = tile % NKB;
                const F16 sf = frag_rows<float, 16>(Ss, VP, 16 * kb, 0, lane);
                const F16 df = frag_rows<float, 16>(dSs, VP, 16 * kb, 0, lane);
                dQa[m] = F16::mma(frag_rows<float, 16>(dYs, VP, 16 * rb, 0, lane), sf, dQa[m]);
                dKa[m] = F16::mma(frag_rows<float, 16>(dXs, VP, 16 * rb, 0, lane), sf, dKa[m]);
                dKb[m] = F16::mma(frag_rows<float, 16>(Us, VP, 16 * rb, 0, lane), df, dKb[m]);
            }
        }
        __syncthreads();
    }

    // ---- E: per-token partials to LDS; Ak into the freed slice buffers
    if (wave < NB) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float g = row16_sum(pG[e]), bb = row16_sum(pB[e]);
            if (ln == 0) {
                tokG[16 * wave + 4 * lg + e] = g;
                tokB[16 * wave + 4 * lg + e] = bb;
            }
        }
    }
    {
        float x = pGC, y = pSS;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            x += __shfl_xor(x, off);
            y += __shfl_xor(y, off);
        }
        if (lane == 0) {
            red[wave] = x;
            red[4 + wave] = y;
        }
    }
    stage_cc<C, CP>(Aks, rec + Rec<C>::oA);
    __syncthreads();

    // dP tiles -> dQK = Gamma o dP (into Ps); dM tiles -> dA = -dM, dKK =
    // Gamma o diag(beta) dA (into Ts).  E = dP o P + diag(beta) dA o Ak feeds
    // dG_r (+ row sums) and dG_j (- column sums); dA o Ak feeds dbeta.
    // Every (part, block) has exactly one writer, so the sums are deterministic.
#pragma unroll
    for (int m = 0; m < NCC; ++m) {
        const int tile = wave + 4 * m;
        if (tile < 2 * NTRI) {
            const int part = tile >= NTRI ? 1 : 0;
            int rb, jb;
            tri_block(part ? tile - NTRI : tile, rb, jb);
            const int j = 16 * jb + ln;
            float cs = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * lg + e;
                const float gam = __builtin_amdgcn_exp2f(fminf(Gs[r] - Gs[j], 0.f));
                float E, rbeta = 0.f;
                if (part) {
                    const float dA = r > j ? -dPM[m][e] : 0.f;
                    const float ak = Aks[r * CP + j];
                    const float dAk = Bs[r] * dA;
                    Ts[r * CP + j] = gam * dAk;
                    E = dAk * ak;
                    rbeta = dA * ak;
                } else {
                    const float dP = r >= j ? dPM[m][e] : 0.f;
                    E = dP * Ps[r * CP + j];
                    Ps[r * CP + j] = gam * dP;
                }
                cs += E;
                const float rs = row16_sum(E);
                const float rsb = row16_sum(rbeta);
                if (ln == 0) {
                    rowE[((part * NB + rb) * NB + jb) * 16 + 4 * lg + e] = rs;
                    if (part) rowB[(rb * NB + jb) * 16 + 4 * lg + e] = rsb;
                }
            }
            cs += __shfl_xor(cs, 16);
            cs += __shfl_xor(cs, 32);
            if (lg == 0) colE[((part * NB + rb) * NB + jb) * 16 + ln] = cs;
        }
    }
    __syncthreads();

    // ---- F: dQ = e^G o dQa + dQK K;
    //         dK = -e^G beta o dKa + d o dKb + dKK K + dKK^T K + dQK^T Q
#pragma unroll
    for (int m = 0; m < NCK; ++m) {
        const int tile = wave + 4 * m;
        if (tile < NTILE) {
            const int rb = tile / NKB, kb = tile % NKB;
            const float GC = Gs[C - 1];
            f32x4 dq, dk;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * lg + e;
                const float br = __builtin_amdgcn_exp2f(Gs[r]), dr = __builtin_amdgcn_exp2f(GC - Gs[r]);
                dq[e] = br * dQa[m][e];
                dk[e] = dr * dKb[m][e] - br * Bs[r] * dKa[m][e];
            }
            for (int jb = 0; jb <= rb; ++jb) {
                const F16 kf = frag_cols<float, 16>(Ks, KP, 16 * kb, 16 * jb, lane);
                dq = F16::mma(frag_rows<float, 16>(Ps, CP, 16 * rb, 16 * jb, lane), kf, dq);
                dk = F16::mma(frag_rows<float, 16>(Ts, CP, 16 * rb, 16 * jb, lane), kf, dk);
            }
            for (int ib = rb; ib < NB; ++ib) {
                dk = F16::mma(frag_cols<float, 16>(Ts, CP, 16 * rb, 16 * ib, lane),
                              frag_cols<float, 16>(Ks, KP, 16 * kb, 16 * ib, lane), dk);
                dk = F16::mma(frag_cols<float, 16>(Ps, CP, 16 * rb, 16 * ib, lane),
                              frag_cols<float, 16>(Qs, KP, 16 * kb, 16 * ib, lane), dk);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t t = c0 + 16 * rb + 4 * lg + e;
                if (t < T) {
                    const int64_t o = ((b * T + t) * H + h) * DK + 16 * kb + ln;
                    p.dq[o] = dq[e];
                    p.dk[o] = dk[e];
                }
            }
        }
    }

    // ---- G: dG per token, d ln alpha = suffix sums of dG, dalpha, dbeta
    if (wave == 0) {
        const int rr = C - 1 - lane;    // lane l carries token C-1-l (reversed for the scan)
        float g = 0.f;
        if (lane < C) {
            const int rb = rr / 16, ri = rr % 16;
            g = tokG[rr];
            for (int jb = 0; jb <= rb; ++jb)
                g += rowE[(rb * NB + jb) * 16 + ri] + rowE[((NB + rb) * NB + jb) * 16 + ri];
            for (int ib = rb; ib < NB; ++ib)
                g -= colE[(ib * NB + rb) * 16 + ri] + colE[((NB + ib) * NB + rb) * 16 + ri];
            if (rr == C - 1)
                g += (red[0] + red[1]) + (red[2] + red[3]) +
                     __builtin_amdgcn_exp2f(Gs[C - 1]) * ((red[4] + red[5]) + (red[6] + red[7]));
        }
        const float suf = wave_inclusive_sum(g, lane);   // lane l: sum over tokens >= C-1-l
        if (lane < C) {
            const int64_t t = c0 + rr;
            if (t < T) {
                const int rb = rr / 16, ri = rr % 16;
                float db = tokB[rr];
                for (int jb = 0; jb <= rb; ++jb) db += rowB[(rb * NB + jb) * 16 + ri];
                const int64_t o = (b * T + t) * H + h;
                p.dalpha[o] = suf / Als[rr];
                p.dbeta[o] = db;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
template <typename Tin, int C, int DK>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t stream)
{
    BwdParams kp;
    kp.q = a.q; kp.k = a.k; kp.v = a.v;
    kp.alpha = a.alpha; kp.beta = a.beta; kp.s0 = a.s0; kp.dy = a.dy; kp.dsT = a.dsT;
    kp.dq = a.dq; kp.dk = a.dk; kp.dv = a.dv; kp.dalpha = a.dalpha; kp.dbeta = a.dbeta; kp.ds0 = a.ds0;
    kp.T = a.T; kp.H = a.H; kp.Dv = a.Dv;
    kp.NC = (a.T + C - 1) / C;
    kp.rec_floats = bwd_record_floats(C);
    const int64_t bh = a.B * a.H;
    float *ws = static_cast<float *>(a.ws);
    kp.rec = ws;
    kp.sc = kp.rec + bh * kp.NC * kp.rec_floats;
    kp.dsc = kp.sc + bh * kp.NC * DK * a.Dv;
    const unsigned nchunk = (unsigned)(bh * kp.NC), nslice = (unsigned)(bh * (a.Dv / BV));
    hipLaunchKernelGGL((bwd_prep_kernel<Tin, C, DK>), dim3(nchunk), dim3(NT), 0, stream, kp);
    hipLaunchKernelGGL((bwd_carry_kernel<Tin, C, DK, false>), dim3(nslice), dim3(NT), 0, stream, kp);
    hipLaunchKernelGGL((bwd_carry_kernel<Tin, C, DK, true>), dim3(nslice), dim3(NT), 0, stream, kp);
    hipLaunchKernelGGL((bwd_chunk_kernel<Tin, C, DK>), dim3(nchunk), dim3(NT), 0, stream, kp);
    return hipGetLastError();
}

template <typename Tin, int C>
hipError_t launch_bwd_dk(const BwdArgs &a, hipStream_t s)
{
    switch (a.Dk) {
    case 16: return launch_bwd_t<Tin, C, 16>(a, s);
    case 32: return launch_bwd_t<Tin, C, 32>(a, s);
    case 64: return launch_bwd_t<Tin, C, 64>(a, s);
    case 128: return launch_bwd_t<Tin, C, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename Tin>
hipError_t launch_bwd_c(const BwdArgs &a, hipStream_t s)
{
    switch (a.chunk) {
    case 16: return launch_bwd_dk<Tin, 16>(a, s);
    case 32: return launch_bwd_dk<Tin, 32>(a, s);
    case 64: return launch_bwd_dk<Tin, 64>(a, s);
    }
    return hipErrorInvalidValue;
}

// T == 0: dL/dS_0 = dL/dS_T (or zero)
__global__ void copy_or_zero(const float *__restrict__ src, float *__restrict__ dst, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

}  // namespace

int64_t bwd_record_floats(int64_t C) { return (3 * C * C + C + 63) / 64 * 64; }

size_t prefill_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int64_t C)
{
    const int64_t nc = (T + C - 1) / C;
    return (size_t)(4 * B * H * nc * (bwd_record_floats(C) + 2 * Dk * Dv));
}

hipError_t launch_prefill_bwd(const BwdArgs &a, hipStream_t stream)
{
    if (a.B * a.H == 0) return hipSuccess;
    if (a.T == 0) {
        if (!a.ds0) return hipSuccess;
        const int64_t n = a.B * a.H * a.Dk * a.Dv;
        hipLaunchKernelGGL(copy_or_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a.dsT, a.ds0, n);
        return hipGetLastError();
    }
    return a.bf16 ? launch_bwd_c<__bf16>(a, stream) : launch_bwd_c<float>(a, stream);
}

}  // namespace gdn
