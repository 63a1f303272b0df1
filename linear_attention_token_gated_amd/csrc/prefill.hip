// prefill.hip -- chunkwise gated delta rule for whole sequences on gfx950.
//
// Source: "On the Design of Qwen3.8-Next Architecture", picx.dev summary,
// "Theoretical foundations", eqs (1)-(4).  The pages give only the token-by-
// token recurrence; the chunk form below is derived from it.  For one chunk of
// C tokens r = 1..C entering with state S (Dk x Dv):
//
//   g_r = ln alpha_r,  G_r = g_1 + ... + g_r,  Gamma_rj = exp(G_r - G_j) (r >= j)
//   (computed in base 2: G2_r = sum log2 alpha, Gamma_rj = 2^(G2_r - G2_j))
//   A = strict_lower[ beta_r Gamma_rj (k_r . k_j) ]
//   R = diag(beta) (V - diag(e^G) K S)
//   U = (I + A)^-1 R                      (u_r = beta_r e_r of eqs (2)-(3))
//   Y = diag(e^G) Q S + P U,  P = lower_incl[ Gamma_rj (q_r . k_j) ]   (eq (4))
//   S' = e^{G_C} S + K^T diag(e^{G_C - G}) U                           (eqs (1),(3))
//
// Columns of S, V, Y are independent (e_t[j] only involves column j of S and
// v_t[j]), so each workgroup owns one 16-column slice of Dv for one (b, h) and
// carries that slice of S through every chunk in MFMA accumulator registers.
// This file holds the fp32-input path, all of it in one kernel of 4
// wavefronts on fp32 MFMA (16x16x4); within a chunk:
//   1. stage K, Q (Dk wide), the V slice, alpha, beta into LDS; prefix-sum ln alpha
//   2. Gram tiles K K^T and Q K^T -> A and P
//   3. K S and Q S -> R
//   4. (I + A)^-1 of each 16x16 diagonal block by in-register forward
//      substitution (DPP row broadcast), then block forward substitution for U
//   5. Y = diag(e^G) Q S + P U -> y;  S <- e^{G_C} S + K^T (e^{G_C-G} U)
// Ragged tails are padded with identity tokens (alpha = 1, beta = 0, k = q = v = 0).
// bf16 inputs take the two-kernel path of chunk_prep.hip and recurrence.hip;
// launch_prefill below dispatches between them.
#include "common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int NTHREADS = 256;   // 4 wavefronts

template <int C, int DK> struct Lay {
    using OpT = float;
    static constexpr int PAD = 4;
    static constexpr int KP = DK + PAD;     // pitch of K, Q, S^T rows
    static constexpr int CP = C + PAD;      // pitch of C-wide operand rows
    static constexpr int TP = 16 + PAD;     // pitch of diagonal-inverse rows
    static constexpr int AFP = C + 1;       // pitch of fp32 A rows
    static constexpr int NB = C / 16;       // 16-token blocks per chunk
    static constexpr int NSB = DK / 16;     // 16-row blocks of the state slice
    static constexpr int MS = (NSB + 3) / 4;   // state tiles per wavefront
    static constexpr int KS_DK = DK % 32 == 0 ? 32 : 16;
    static constexpr int KS_C = C % 32 == 0 ? 32 : 16;

    static constexpr size_t oK = 0;
    static constexpr size_t oQ = oK + align16(sizeof(OpT) * C * KP);
    static constexpr size_t oST = oQ + align16(sizeof(OpT) * C * KP);
    static constexpr size_t oAf = oST + align16(sizeof(OpT) * BV * KP);
    static constexpr size_t oAn = oAf + align16(4 * C * AFP);
    static constexpr size_t oP = oAn + align16(sizeof(OpT) * C * CP);
    static constexpr size_t oTd = oP + align16(sizeof(OpT) * C * CP);
    static constexpr size_t oRf = oTd + align16(sizeof(OpT) * C * TP);
    static constexpr size_t oUT = oRf + align16(4 * C * BV);
    static constexpr size_t oUdT = oUT + align16(sizeof(OpT) * BV * CP);
    static constexpr size_t oV = oUdT + align16(sizeof(OpT) * BV * CP);
    static constexpr size_t oBe = oV + align16(4 * C * BV);
    static constexpr size_t oG = oBe + align16(4 * C);
    static constexpr size_t oEG = oG + align16(4 * C);
    static constexpr size_t BYTES = oEG + align16(4 * C);
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

struct KParams {
    const void *q, *k, *v;
    const float *alpha, *beta, *s0;
    float *y, *sT;
    int64_t T, H, Dv;
    int64_t qs, ks, vs;      // token strides (elements)
    int nslices;             // Dv / 16
    int xcd_map;             // 1: group the slices of a head on one XCD
};

template <typename Tin, int C, int DK>
__global__ __launch_bounds__(NTHREADS, 1) void gdn_prefill_kernel(KParams p)
{
    using OpT = float;
    using L = Lay<C, DK>;
    constexpr int KP = L::KP, CP = L::CP, TP = L::TP, AFP = L::AFP, NB = L::NB, NSB = L::NSB,
                  MS = L::MS, KS_DK = L::KS_DK, KS_C = L::KS_C;
    using FragDK = Frag<OpT, KS_DK>;
    using FragC = Frag<OpT, KS_C>;
    using Frag16 = Frag<OpT, 16>;

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    OpT *Ks = reinterpret_cast<OpT *>(smem + L::oK);
    OpT *Qs = reinterpret_cast<OpT *>(smem + L::oQ);
    OpT *STs = reinterpret_cast<OpT *>(smem + L::oST);
    float *Af = reinterpret_cast<float *>(smem + L::oAf);
    OpT *An = reinterpret_cast<OpT *>(smem + L::oAn);
    OpT *Ps = reinterpret_cast<OpT *>(smem + L::oP);
    OpT *Td = reinterpret_cast<OpT *>(smem + L::oTd);
    float *Rf = reinterpret_cast<float *>(smem + L::oRf);
    OpT *UT = reinterpret_cast<OpT *>(smem + L::oUT);
    OpT *UdT = reinterpret_cast<OpT *>(smem + L::oUdT);
    float *Vs = reinterpret_cast<float *>(smem + L::oV);
    float *Be = reinterpret_cast<float *>(smem + L::oBe);
    float *Gs = reinterpret_cast<float *>(smem + L::oG);
    float *EG = reinterpret_cast<float *>(smem + L::oEG);

    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int ln = lane & 15, lg = lane >> 4;

    // ---- workgroup -> (b*H + h, slice).  With xcd_map the slices of one head
    // get ids that are equal mod 8, so they run on one XCD and share its L2.
    const int64_t bid = blockIdx.x;
    int64_t bh, sl;
    if (p.xcd_map) {
        const int64_t xcd = bid & 7, local = bid >> 3;
        bh = (local / p.nslices) * 8 + xcd;
        sl = local % p.nslices;
    } else {
        bh = bid / p.nslices;
        sl = bid % p.nslices;
    }
    const int64_t H = p.H, T = p.T, Dv = p.Dv;
    const int64_t b = bh / H, h = bh % H;
    const int n0 = (int)sl * BV;
    const Tin *qg = static_cast<const Tin *>(p.q);
    const Tin *kg = static_cast<const Tin *>(p.k);
    const Tin *vg = static_cast<const Tin *>(p.v);

    // ---- state slice: wavefront w owns 16-row blocks ib = w + 4m
    f32x4 S[MS];
#pragma unroll
    for (int m = 0; m < MS; ++m) {
        S[m] = zero4();
        const int ib = wave + 4 * m;
        if (ib < NSB && p.s0) {
            const float *s0 = p.s0 + bh * (int64_t)DK * Dv;
#pragma unroll
            for (int e = 0; e < 4; ++e) S[m][e] = s0[(int64_t)(16 * ib + 4 * lg + e) * Dv + n0 + ln];
        }
    }

    auto write_state_operand = [&]() {
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int ib = wave + 4 * m;
            if (ib < NSB) {
#pragma unroll
                for (int e = 0; e < 4; ++e) STs[ln * KP + 16 * ib + 4 * lg + e] = S[m][e];
            }
        }
    };
    write_state_operand();

    constexpr int EPV = 16 / sizeof(Tin);        // elements per 16-byte vector
    constexpr int VPR = DK / EPV;                // vectors per K/Q row
    constexpr int VVR = BV / EPV;                // vectors per V-slice row
    constexpr int NKV = (C * VPR + NTHREADS - 1) / NTHREADS;   // K (and Q) vectors per thread

    // Registers holding the next chunk while the current one is computed.
    f32x4 pk[NKV], pq[NKV], pv = zero4();
    float pal = 1.f, pbe = 0.f;
    auto prefetch = [&](int64_t c0) {
#pragma unroll
        for (int it = 0; it < NKV; ++it) {
            const int vi = tid + NTHREADS * it;
            const int r = vi / VPR, col = (vi % VPR) * EPV;
            const int64_t t = c0 + r;
            pk[it] = zero4();
            pq[it] = zero4();
            if (vi < C * VPR && t < T) {
                const int64_t row = b * T + t;
                pk[it] = *reinterpret_cast<const f32x4 *>(kg + row * p.ks + h * DK + col);
                pq[it] = *reinterpret_cast<const f32x4 *>(qg + row * p.qs + h * DK + col);
            }
        }
        if (tid < C * VVR) {
            const int r = tid / VVR, col = (tid % VVR) * EPV;
            const int64_t t = c0 + r;
            pv = zero4();
            if (t < T) pv = *reinterpret_cast<const f32x4 *>(vg + (b * T + t) * p.vs + h * Dv + n0 + col);
        }
        if (tid < C) {
            const int64_t t = c0 + tid;
            const bool ok = t < T;
            pal = ok ? p.alpha[(b * T + t) * H + h] : 1.f;
            pbe = ok ? p.beta[(b * T + t) * H + h] : 0.f;
        }
    };
    prefetch(0);

    // Gram tile table: tiles (rb, cb) with cb <= rb, K-part then Q-part.
    constexpr int NTRI = NB * (NB + 1) / 2;
    constexpr int NGT = (2 * NTRI + 3) / 4;      // Gram tiles per wavefront (upper bound)

    for (int64_t c0 = 0; c0 < T; c0 += C) {
        // ---------------- 1. stage the chunk (from registers), prefetch the next ----------------
#pragma unroll
        for (int it = 0; it < NKV; ++it) {
            const int vi = tid + NTHREADS * it;
            if (vi < C * VPR) {
                const int r = vi / VPR, col = (vi % VPR) * EPV;
                *reinterpret_cast<f32x4 *>(Ks + r * KP + col) = pk[it];
                *reinterpret_cast<f32x4 *>(Qs + r * KP + col) = pq[it];
            }
        }
        if (tid < C * VVR) {
            const int r = tid / VVR, col = (tid % VVR) * EPV;
            const Tin *tv = reinterpret_cast<const Tin *>(&pv);
#pragma unroll
            for (int e = 0; e < EPV; ++e) Vs[r * BV + col + e] = to_f32(tv[e]);
        }
        // log2-decay prefix: wavefront 0 scans it (lane = token) and publishes it
        // before the staging barrier.
        float g2 = 0.f, be_t = 0.f;
        if (tid < C) { g2 = __builtin_amdgcn_logf(pal); be_t = pbe; }
        if (wave == 0) {
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float t = __shfl_up(g2, off);
                if (lane >= off) g2 += t;
            }
            if (lane < C) {
                Gs[lane] = g2;                          // log2 of the cumulative decay
                EG[lane] = __builtin_amdgcn_exp2f(g2);
                Be[lane] = be_t;
            }
        }
        if (c0 + C < T) prefetch(c0 + C);
        __syncthreads();
        const float GC = Gs[C - 1];

        // ---------------- 2. Gram tiles: K K^T -> A, Q K^T -> P ----------------
#pragma unroll
        for (int it = 0; it < NGT; ++it) {
            const int tile = wave + 4 * it;
            if (tile < 2 * NTRI) {
                const bool isQ = tile >= NTRI;
                const int idx = isQ ? tile - NTRI : tile;
                // row-major enumeration of the lower triangle of NB x NB blocks
                const int rb = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
                const int cb = idx - rb * (rb + 1) / 2;
                const OpT *Asrc = isQ ? Qs : Ks;
                f32x4 acc = zero4();
#pragma unroll
                for (int k0 = 0; k0 < DK; k0 += KS_DK) {
                    const FragDK a = frag_rows<OpT, KS_DK>(Asrc, KP, 16 * rb, k0, lane);
                    const FragDK bb = frag_rows<OpT, KS_DK>(Ks, KP, 16 * cb, k0, lane);
                    acc = FragDK::mma(a, bb, acc);
                }
                const int j = 16 * cb + ln;
                const float Gj = Gs[j];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * lg + e;
                    const float gam = __builtin_amdgcn_exp2f(fminf(Gs[r] - Gj, 0.f));
                    if (isQ) {
                        Ps[r * CP + j] = r >= j ? gam * acc[e] : 0.f;
                    } else {
                        const float val = r > j ? Be[r] * gam * acc[e] : 0.f;
                        if (rb == cb) Af[r * AFP + j] = val;
                        else An[r * CP + j] = -val;
                    }
                }
            }
        }

        // ---------------- 3. K S -> R, Q S (kept for Y) ----------------
        f32x4 qs_acc = zero4();
        if (wave < NB) {
            const int rb = wave;
            f32x4 ks_acc = zero4();
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += KS_DK) {
                const FragDK kf = frag_rows<OpT, KS_DK>(Ks, KP, 16 * rb, k0, lane);
                const FragDK qf = frag_rows<OpT, KS_DK>(Qs, KP, 16 * rb, k0, lane);
                const FragDK sf = frag_rows<OpT, KS_DK>(STs, KP, 0, k0, lane);
                ks_acc = FragDK::mma(kf, sf, ks_acc);
                qs_acc = FragDK::mma(qf, sf, qs_acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * lg + e;
                Rf[r * BV + ln] = Be[r] * (Vs[r * BV + ln] - EG[r] * ks_acc[e]);
            }
        }
        __syncthreads();

        // ---------------- 4a. diagonal-block inverses ----------------
        if (wave < NB) {
            const int blk = wave;
            float Lr[16];
#pragma unroll
            for (int s = 0; s < 16; ++s) Lr[s] = Af[(16 * blk + ln) * AFP + 16 * blk + s];
            float X[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) X[i] = (ln == lg + 4 * i) ? 1.f : 0.f;
            tri_solve16(X, Lr, ln, std::make_integer_sequence<int, 15>{});
#pragma unroll
            for (int i = 0; i < 4; ++i) Td[(16 * blk + ln) * TP + lg + 4 * i] = X[i];
        }
        __syncthreads();

        // ---------------- 4b. block forward substitution for U (wavefront 0) ----
        if (wave == 0) {
            // U blocks as B operands (accumulator layout == B layout for KS=16)
            Frag16 Uf[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                f32x4 z;
#pragma unroll
                for (int e = 0; e < 4; ++e) z[e] = Rf[(16 * i + 4 * lg + e) * BV + ln];
#pragma unroll
                for (int kb = 0; kb < i; ++kb) {
                    const Frag16 a = frag_rows<OpT, 16>(An, CP, 16 * i, 16 * kb, lane);
                    z = Frag16::mma(a, Uf[kb], z);
                }
                Frag16 zf;
#pragma unroll
                for (int e = 0; e < 4; ++e) zf.set_raw(e, z[e]);
                const Frag16 ti = frag_rows<OpT, 16>(Td, TP, 16 * i, 0, lane);
                const f32x4 u = Frag16::mma(ti, zf, zero4());
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * i + 4 * lg + e;
                    Uf[i].set_raw(e, u[e]);
                    UT[ln * CP + r] = u[e];
                    UdT[ln * CP + r] = __builtin_amdgcn_exp2f(GC - Gs[r]) * u[e];
                }
            }
        }
        __syncthreads();

        // ---------------- 5a. Y = diag(e^G) Q S + P U ----------------
        if (wave < NB) {
            const int rb = wave;
            f32x4 acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = EG[16 * rb + 4 * lg + e] * qs_acc[e];
            for (int jb = 0; jb <= rb; ++jb) {
                const Frag16 a = frag_rows<OpT, 16>(Ps, CP, 16 * rb, 16 * jb, lane);
                const Frag16 u = frag_rows<OpT, 16>(UT, CP, 0, 16 * jb, lane);
                acc = Frag16::mma(a, u, acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t t = c0 + 16 * rb + 4 * lg + e;
                if (t < T) p.y[((b * T + t) * H + h) * Dv + n0 + ln] = acc[e];
            }
        }

        // ---------------- 5b. S <- e^{G_C} S + K^T (e^{G_C-G} U) ----------------
        const float eGC = __builtin_amdgcn_exp2f(GC);
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int ib = wave + 4 * m;
            if (ib < NSB) {
                f32x4 acc = S[m] * eGC;
#pragma unroll
                for (int j0 = 0; j0 < C; j0 += KS_C) {
                    const FragC a = frag_cols<OpT, KS_C>(Ks, KP, 16 * ib, j0, lane);
                    const FragC u = frag_rows<OpT, KS_C>(UdT, CP, 0, j0, lane);
                    acc = FragC::mma(a, u, acc);
                }
                S[m] = acc;
            }
        }
        write_state_operand();
        __syncthreads();
    }

    if (p.sT) {
        float *sT = p.sT + bh * (int64_t)DK * Dv;
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int ib = wave + 4 * m;
            if (ib < NSB) {
#pragma unroll
                for (int e = 0; e < 4; ++e) sT[(int64_t)(16 * ib + 4 * lg + e) * Dv + n0 + ln] = S[m][e];
            }
        }
    }
}

template <typename Tin, int C, int DK>
hipError_t launch_t(const PrefillArgs &a, hipStream_t stream)
{
    KParams kp;
    kp.q = a.q; kp.k = a.k; kp.v = a.v;
    kp.alpha = a.alpha; kp.beta = a.beta; kp.s0 = a.s0;
    kp.y = a.y; kp.sT = a.sT;
    kp.T = a.T; kp.H = a.H; kp.Dv = a.Dv;
    kp.qs = a.q_tok_stride; kp.ks = a.k_tok_stride; kp.vs = a.v_tok_stride;
    kp.nslices = (int)(a.Dv / BV);
    const int64_t bh = a.B * a.H;
    kp.xcd_map = (bh % 8 == 0) ? 1 : 0;
    const int64_t grid = bh * kp.nslices;
    hipLaunchKernelGGL((gdn_prefill_kernel<Tin, C, DK>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream, kp);
    return hipGetLastError();
}

template <typename Tin, int C>
hipError_t launch_dk(const PrefillArgs &a, hipStream_t s)
{
    switch (a.Dk) {
    case 16: return launch_t<Tin, C, 16>(a, s);
    case 32: return launch_t<Tin, C, 32>(a, s);
    case 64: return launch_t<Tin, C, 64>(a, s);
    case 128: return launch_t<Tin, C, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename Tin>
hipError_t launch_c(const PrefillArgs &a, hipStream_t s)
{
    switch (a.chunk) {
    case 16: return launch_dk<Tin, 16>(a, s);
    case 32: return launch_dk<Tin, 32>(a, s);
    case 64: return launch_dk<Tin, 64>(a, s);
    }
    return hipErrorInvalidValue;
}

// T == 0: the final state is the initial state (or zero).
__global__ void copy_or_zero_state(const float *__restrict__ s0, float *__restrict__ sT, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) sT[i] = s0 ? s0[i] : 0.f;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream, int stages)
{
    if (a.B * a.H == 0) return hipSuccess;
    if (a.T == 0) {
        if (!(stages & 2) || !a.sT || a.sT == a.s0) return hipSuccess;
        const int64_t n = a.B * a.H * a.Dk * a.Dv;
        hipLaunchKernelGGL(copy_or_zero_state, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a.s0, a.sT, n);
        return hipGetLastError();
    }
    if (a.bf16) {
        // per-chunk preparation of every (b, h, chunk), then the recurrence
        if (stages & 1) {
            const hipError_t e = launch_chunk_prep(a, stream);
            if (e != hipSuccess) return e;
        }
        return (stages & 2) ? launch_recurrence(a, stream) : hipSuccess;
    }
    // fp32 with a record workspace: preparation once per chunk, then the
    // recurrence (backward.hip); without one, the single kernel below
    if (a.ws) return launch_prefill_f32_staged(a, stream);
    return launch_c<float>(a, stream);
}

}  // namespace gdn
