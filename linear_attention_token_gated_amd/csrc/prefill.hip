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
// carries that slice of S through every chunk in MFMA accumulator registers
// (fp32 master copy).  Within a chunk:
//   1. stage K, Q (Dk wide), the V slice, alpha, beta into LDS; prefix-sum ln alpha
//   2. Gram tiles K K^T and Q K^T on MFMA -> A (fp32 diagonal blocks, operand
//      precision off-diagonal blocks) and P
//   3. K S and Q S on MFMA -> R
//   4. (I + A)^-1 of each 16x16 diagonal block by in-register forward
//      substitution (DPP row broadcast), then block forward substitution for U
//      on MFMA, chaining accumulator tiles directly as the next B operand
//   5. Y = diag(e^G) Q S + P U -> y (fp32);  S <- e^{G_C} S + K^T (e^{G_C-G} U)
// Ragged tails are padded with identity tokens (alpha = 1, beta = 0, k = q = v = 0).
//
// Precision (bf16 inputs): q, k, v are exact bf16 MFMA operands and every
// product accumulates in fp32.  The operands that are computed in fp32 and
// feed an MFMA -- the state S, P, the substitution right-hand side Z, U and
// the decayed U of the state update -- are carried as a bf16 pair hi + lo with
// hi = bf16(x), lo = bf16(x - hi), and each product with them is summed over
// the pair (hi*hi + hi*lo + lo*hi where both sides are split).  Rounding any of
// them to a single bf16 costs about 1e-2 in max|err|/RMS(y) at the 4K workload;
// the pair keeps the whole path near 2e-3.  The diagonal-block inverses and
// the off-diagonal blocks of A are single bf16 (they contribute ~2e-3).
#include "common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int BV = 16;          // value columns per workgroup
constexpr int NTHREADS = 256;   // 4 wavefronts

constexpr size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

template <typename OpT, int C, int DK> struct Lay {
    static constexpr bool SPLIT = sizeof(OpT) == 2;   // bf16 hi/lo state operand
    static constexpr int PAD = sizeof(OpT) == 2 ? 8 : 4;
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
    static constexpr size_t oSTlo = oST + align16(sizeof(OpT) * BV * KP);
    static constexpr size_t oAf = oSTlo + (SPLIT ? align16(sizeof(OpT) * BV * KP) : 0);
    static constexpr size_t oAn = oAf + align16(4 * C * AFP);
    static constexpr size_t oP = oAn + align16(sizeof(OpT) * C * CP);
    static constexpr size_t oPlo = oP + align16(sizeof(OpT) * C * CP);
    static constexpr size_t oTd = oPlo + (SPLIT ? align16(sizeof(OpT) * C * CP) : 0);
    static constexpr size_t oRf = oTd + align16(sizeof(OpT) * C * TP);
    static constexpr size_t oUT = oRf + align16(4 * C * BV);
    static constexpr size_t oUTlo = oUT + align16(sizeof(OpT) * BV * CP);
    static constexpr size_t oUdT = oUTlo + (SPLIT ? align16(sizeof(OpT) * BV * CP) : 0);
    static constexpr size_t oUdTlo = oUdT + align16(sizeof(OpT) * BV * CP);
    static constexpr size_t oV = oUdTlo + (SPLIT ? align16(sizeof(OpT) * BV * CP) : 0);
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

// Forward substitution of (I + L) X = I for a 16x16 strictly lower L, inside
// one wavefront.  Lane (r = l%16, g = l/16) owns row r of X, columns g+4i.
// Step s: row s is final; every row r > s subtracts L[r][s] * X[s][:].
// X[s][c] lives in lane s of the same 16-lane row (same g) -> DPP broadcast.
template <int S>
__device__ __forceinline__ void tri_step(float (&X)[4], const float (&Lr)[16], int r) {
    // rows r <= S have L[r][S] = 0 (L is strictly lower), so the update is an
    // exact no-op there and needs no select
    (void)r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float xs = row_bcast<S>(X[i]);
        X[i] = fmaf(-Lr[S], xs, X[i]);
    }
}
template <int... S>
__device__ __forceinline__ void tri_solve16(float (&X)[4], const float (&Lr)[16], int r,
                                            std::integer_sequence<int, S...>) {
    (tri_step<S>(X, Lr, r), ...);
}

template <typename Tin, int C, int DK>
__global__ __launch_bounds__(NTHREADS, 1) void gdn_prefill_kernel(KParams p)
{
    using OpT = Tin;
    using L = Lay<OpT, C, DK>;
    constexpr bool SPLIT = L::SPLIT;
    constexpr int KP = L::KP, CP = L::CP, TP = L::TP, AFP = L::AFP, NB = L::NB, NSB = L::NSB,
                  MS = L::MS, KS_DK = L::KS_DK, KS_C = L::KS_C;
    using FragDK = Frag<OpT, KS_DK>;
    using FragC = Frag<OpT, KS_C>;
    using Frag16 = Frag<OpT, 16>;

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    OpT *Ks = reinterpret_cast<OpT *>(smem + L::oK);
    OpT *Qs = reinterpret_cast<OpT *>(smem + L::oQ);
    OpT *STs = reinterpret_cast<OpT *>(smem + L::oST);
    OpT *STlo = reinterpret_cast<OpT *>(smem + L::oSTlo);
    float *Af = reinterpret_cast<float *>(smem + L::oAf);
    OpT *An = reinterpret_cast<OpT *>(smem + L::oAn);
    OpT *Ps = reinterpret_cast<OpT *>(smem + L::oP);
    OpT *Plo = reinterpret_cast<OpT *>(smem + L::oPlo);
    OpT *Td = reinterpret_cast<OpT *>(smem + L::oTd);
    float *Rf = reinterpret_cast<float *>(smem + L::oRf);
    OpT *UT = reinterpret_cast<OpT *>(smem + L::oUT);
    OpT *UTlo = reinterpret_cast<OpT *>(smem + L::oUTlo);
    OpT *UdT = reinterpret_cast<OpT *>(smem + L::oUdT);
    OpT *UdTlo = reinterpret_cast<OpT *>(smem + L::oUdTlo);
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
                for (int e = 0; e < 4; ++e) {
                    const OpT hi = from_f32<OpT>(S[m][e]);
                    STs[ln * KP + 16 * ib + 4 * lg + e] = hi;
                    if constexpr (L::SPLIT) STlo[ln * KP + 16 * ib + 4 * lg + e] = from_f32<OpT>(S[m][e] - to_f32(hi));
                }
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
                        const float pvv = r >= j ? gam * acc[e] : 0.f;
                        const OpT hi = from_f32<OpT>(pvv);
                        Ps[r * CP + j] = hi;
                        if constexpr (SPLIT) Plo[r * CP + j] = from_f32<OpT>(pvv - to_f32(hi));
                    } else {
                        const float val = r > j ? Be[r] * gam * acc[e] : 0.f;
                        if (rb == cb) Af[r * AFP + j] = val;
                        else An[r * CP + j] = from_f32<OpT>(-val);
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
                if constexpr (L::SPLIT) {
                    const FragDK sl2 = frag_rows<OpT, KS_DK>(STlo, KP, 0, k0, lane);
                    ks_acc = FragDK::mma(kf, sl2, ks_acc);
                    qs_acc = FragDK::mma(qf, sl2, qs_acc);
                }
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
            for (int i = 0; i < 4; ++i) Td[(16 * blk + ln) * TP + lg + 4 * i] = from_f32<OpT>(X[i]);
        }
        __syncthreads();

        // ---------------- 4b. block forward substitution for U (wavefront 0) ----
        if (wave == 0) {
            // U blocks as B operands (accumulator layout == B layout for KS=16)
            Frag16 Uh[NB], Ul[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                f32x4 z;
#pragma unroll
                for (int e = 0; e < 4; ++e) z[e] = Rf[(16 * i + 4 * lg + e) * BV + ln];
#pragma unroll
                for (int kb = 0; kb < i; ++kb) {
                    const Frag16 a = frag_rows<OpT, 16>(An, CP, 16 * i, 16 * kb, lane);
                    z = Frag16::mma(a, Uh[kb], z);
                    if constexpr (SPLIT) z = Frag16::mma(a, Ul[kb], z);
                }
                Frag16 zh, zl;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const OpT hi = from_f32<OpT>(z[e]);
                    zh.set_raw(e, hi);
                    if constexpr (SPLIT) zl.set(e, z[e] - to_f32(hi));
                }
                const Frag16 ti = frag_rows<OpT, 16>(Td, TP, 16 * i, 0, lane);
                f32x4 u = Frag16::mma(ti, zh, zero4());
                if constexpr (SPLIT) u = Frag16::mma(ti, zl, u);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * i + 4 * lg + e;
                    const OpT hi = from_f32<OpT>(u[e]);
                    Uh[i].set_raw(e, hi);
                    UT[ln * CP + r] = hi;
                    const float ud = __builtin_amdgcn_exp2f(GC - Gs[r]) * u[e];
                    const OpT dhi = from_f32<OpT>(ud);
                    UdT[ln * CP + r] = dhi;
                    if constexpr (SPLIT) {
                        const OpT lo = from_f32<OpT>(u[e] - to_f32(hi));
                        Ul[i].set_raw(e, lo);
                        UTlo[ln * CP + r] = lo;
                        UdTlo[ln * CP + r] = from_f32<OpT>(ud - to_f32(dhi));
                    }
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
                if constexpr (SPLIT) {
                    const Frag16 alo = frag_rows<OpT, 16>(Plo, CP, 16 * rb, 16 * jb, lane);
                    const Frag16 ulo = frag_rows<OpT, 16>(UTlo, CP, 0, 16 * jb, lane);
                    acc = Frag16::mma(alo, u, acc);
                    acc = Frag16::mma(a, ulo, acc);
                }
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
                    if constexpr (SPLIT) {
                        const FragC ulo = frag_rows<OpT, KS_C>(UdTlo, CP, 0, j0, lane);
                        acc = FragC::mma(a, ulo, acc);
                    }
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

// ===========================================================================
// LDS layout of the bf16 kernel: two chunk buffers (the chunk whose state
// recurrence runs now, and the next chunk being staged and prepared) plus the
// arrays that live for one chunk only.  Packed 16x16 blocks (P, the diagonal
// inverses T_ii, the off-diagonal products N_ik) use a padded row pitch PB.
//
// Bank behaviour of gfx950 LDS, as measured with SQ_LDS_BANK_CONFLICT for a
// lane (ln = l % 16, lg = l / 16) reading or writing row ln at a column set by
// lg, with a row pitch of R dwords:
//   128-bit reads   conflict-free for R = 8 mod 16      (64 banks, 16 lanes/cycle)
//   64-bit reads    conflict-free for R = 4 mod 8       (64 banks, 32 lanes/cycle)
//   128-bit writes  conflict-free for R = 4 mod 8       (32 banks,  8 lanes/cycle)
//   64-bit writes   conflict-free for R = 2 mod 4       (32 banks, 16 lanes/cycle)
// Rows read as MFMA fragments (K, Q, S^T, e^{G_C-G} U^T) take the read pitch
// (frag_pitch).  U^T and the packed blocks are written by 64-bit stores on the
// U chain and in the Gram epilogues; their pitches (C + 4, PB = 20 bf16) keep
// those stores conflict-free at the price of a 2-way conflict on their reads.
// ===========================================================================
template <int KS> constexpr int frag_pitch(int n) {
    int r = n / 2;                                    // dwords
    const int m = KS == 32 ? 16 : 8, want = KS == 32 ? 8 : 4;
    while (r % m != want) ++r;
    return 2 * r;
}

constexpr int PB = 20;                 // pitch of a packed 16x16 bf16 block (16 + 4 pad)
constexpr int BLK = 16 * PB;           // elements per packed block

template <int C, int DK> struct PipeLay {
    static constexpr int NB = C / 16;
    static constexpr int NSB = DK / 16;
    static constexpr int MS = (NSB + 3) / 4;
    static constexpr int NTRI = NB * (NB + 1) / 2;    // lower blocks incl. diagonal
    static constexpr int NOFF = NB * (NB - 1) / 2;    // strictly lower blocks
    static constexpr int KS_DK = DK % 32 == 0 ? 32 : 16;
    static constexpr int KS_C = C % 32 == 0 ? 32 : 16;
    static constexpr int KP = frag_pitch<KS_DK>(DK);  // K, Q, S^T row pitch (bf16)
    static constexpr int CPU = C + 4;                 // U^T row pitch (bf16)
    static constexpr int CPD = frag_pitch<KS_C>(C);   // e^{G_C-G} U^T row pitch (bf16)
    // one chunk buffer
    static constexpr size_t cK = 0;
    static constexpr size_t cQ = cK + align16(2 * C * KP);
    static constexpr size_t cPh = cQ + align16(2 * C * KP);
    static constexpr size_t cPl = cPh + align16(2 * NTRI * BLK);
    static constexpr size_t cTd = cPl + align16(2 * NTRI * BLK);
    static constexpr size_t cNn = cTd + align16(2 * NB * BLK);
    static constexpr size_t cV = cNn + align16(2 * (NOFF > 0 ? NOFF : 1) * BLK);
    static constexpr size_t cG = cV + align16(2 * C * BV);      // V slice, bf16
    static constexpr size_t cEG = cG + align16(4 * C);
    static constexpr size_t cBe = cEG + align16(4 * C);
    static constexpr size_t cEd = cBe + align16(4 * C);
    static constexpr size_t cEa = cEd + align16(4 * C);           // 2^(G_r - G_{16 floor(r/16)})
    static constexpr size_t cEb = cEa + align16(4 * C);           // [NB][C] 2^(G_{16 rb} - G_j), j < 16 rb
    static constexpr size_t CBUF = cEb + align16(4 * NB * C);
    // shared arrays after the two chunk buffers
    static constexpr int AP = 20;                                    // fp32 A block row pitch
    static constexpr size_t oAd = 2 * CBUF;                          // fp32 diagonal A blocks [NB][16][AP]
    // off-diagonal A blocks as bf16 hi/lo, lane order: lane l holds A_ik[4(l/16) + e][l % 16]
    static constexpr size_t oAoh = oAd + align16(4 * NB * 16 * AP);
    static constexpr size_t oAol = oAoh + align16(2 * (NOFF > 0 ? NOFF : 1) * 256);
    static constexpr size_t oSTh = oAol + align16(2 * (NOFF > 0 ? NOFF : 1) * 256);
    static constexpr size_t oSTl = oSTh + align16(2 * BV * KP);
    static constexpr size_t oW = oSTl + align16(2 * BV * KP);        // fp32 W_i exchange [NB][64 lanes][4]
    static constexpr size_t oUh = oW + align16(4 * C * BV);
    static constexpr size_t oUl = oUh + align16(2 * BV * CPU);
    static constexpr size_t oUdh = oUl + align16(2 * BV * CPU);
    static constexpr size_t oUdl = oUdh + align16(2 * BV * CPD);
    static constexpr size_t BYTES = oUdl + align16(2 * BV * CPD);
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// Token order of the decayed U^T rows used by the state update.  Within each
// k-step of KS tokens, lane group g (KS/4 values per lane) takes the tokens
// 2g + 8(e/2) + (e%2), e = 0..KS/4-1: adjacent pairs, 8 tokens apart.  With
// the K row pitch of 4 banks mod 32, the four lane groups then gather K
// columns from rows 2 apart -- 8 banks apart, so the column gather is free of
// bank conflicts.  ud_pos gives the storage position of token t; the B operand
// (e^{G_C-G} U^T) is then an ordinary contiguous fragment read.
template <int KS> __device__ __forceinline__ int ud_pos(int t) {
    constexpr int E = KS / 4;
    const int u = t % KS;
    return (t - u) + ((u & 7) >> 1) * E + (u >> 3) * 2 + (u & 1);
}

// A operand K^T[r0 + ln][tokens of ud_pos order] of one k-step at k0.
template <int KS>
__device__ __forceinline__ Frag<__bf16, KS> k_cols_paired(const __bf16 *Ks, int pitch, int r0, int k0, int lane) {
    Frag<__bf16, KS> f;
    const __bf16 *p = Ks + (k0 + 2 * (lane >> 4)) * pitch + r0 + (lane & 15);
#pragma unroll
    for (int e = 0; e < KS / 4; ++e) f.set_raw(e, p[(8 * (e >> 1) + (e & 1)) * pitch]);
    return f;
}

// Value of v in lane l (l wave-uniform).
__device__ __forceinline__ float lane_value(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// v from N lanes lower in the same 16-lane row; lanes with no such source read 0.
template <int N> __device__ __forceinline__ float row_shr(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + N, 0xF, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes: a scan inside each 16-lane row by
// DPP row shifts, then the totals of the earlier rows added from scalars.
__device__ __forceinline__ float wave_inclusive_sum(float x, int lane) {
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x += row_shr<8>(x);
    const float t0 = lane_value(x, 15), t1 = lane_value(x, 31), t2 = lane_value(x, 47);
    const int row = lane >> 4;
    const float base = row == 0 ? 0.f : row == 1 ? t0 : row == 2 ? t0 + t1 : (t0 + t1) + t2;
    return x + base;
}

// ===========================================================================
// Wide pipelined kernel for bf16 inputs: 16 wavefronts (4 per SIMD).
//
// Only the state recurrence itself sits on the per-chunk critical path; all
// other work runs on other wavefronts in the same three phases:
//
//  waves    phase 1                       phase 2                    phase 3
//  0        K S -> R -> W_0 = T_00 R_0    U chain (right-looking)    S update
//  1-3      K S -> R -> W_i               Gram jobs (chunk c+1)      S update
//  4-7      Q S (row block w-4)           Gram jobs (chunk c+1)      Y = e^G Q S + P U
//  8-11     N_ik = T_ii A_ik of chunk c   diagonal A_ii (c+1)        T_ii (c+1)
//           (9-11); stage c+1
//  12-15    stage c+1; decay scan of      Gram jobs (chunk c+1)      -
//           c+1 (12); prefetch c+2
//
// Gram jobs are the strictly-lower blocks of A = K K^T and the lower blocks
// of P = Q K^T of chunk c+1, spread over eleven wavefronts.  Staging copies
// the K, Q and V rows that were loaded into registers one iteration earlier.
// ===========================================================================
constexpr int WIDE_THREADS = 1024;

struct GTile {
    int kind;   // 0 none, 1 A block (K K^T), 2 P block (Q K^T)
    int rb, cb;
};

template <int C, int DK>
__device__ __forceinline__ GTile gram_job(int job)
{
    using L = PipeLay<C, DK>;
    constexpr int NOFF = L::NOFF, NTRI = L::NTRI;
    GTile t{0, 0, 0};
    if (job < NOFF) {
        const int rb = job >= 3 ? 3 : job >= 1 ? 2 : 1;
        t = GTile{1, rb, job - rb * (rb - 1) / 2};
    } else if (job < NOFF + NTRI) {
        const int idx = job - NOFF;
        const int rb = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
        t = GTile{2, rb, idx - rb * (rb + 1) / 2};
    }
    return t;
}

// Two Gram tiles of chunk buffer nb (kind 0 skips).  P blocks and the diagonal
// A blocks are computed transposed, so that lane (ln, lg) holds row
// r = 16 rb + ln, columns j = 16 cb + 4 lg + e: four contiguous entries of a
// row, stored as the rows later read as MFMA A operands.  Off-diagonal A
// blocks are computed as they stand, lane (ln, lg) holding A[16 rb + 4 lg + e]
// [16 cb + ln]: exactly the A operand of N_ik^T = A_ik^T T_ii^T, so they are
// stored in lane order.
template <int C, int DK>
__device__ __forceinline__ void gram_pair(char *nb, float *Ad, __bf16 *Aoh, __bf16 *Aol, const GTile t0,
                                          const GTile t1, int lane)
{
    using L = PipeLay<C, DK>;
    constexpr int KP = L::KP, AP = L::AP, KS_DK = L::KS_DK, NK = DK / KS_DK;
    using FDK = Frag<__bf16, KS_DK>;
    // keep the per-lane index math inside the caller's loop: hoisting it (and
    // the triangular masks derived from it) out of the loop costs registers
    asm volatile("" : "+v"(lane));
    const int ln = lane & 15, lg = lane >> 4;
    const __bf16 *Ks = reinterpret_cast<const __bf16 *>(nb + L::cK);
    const __bf16 *Qs = reinterpret_cast<const __bf16 *>(nb + L::cQ);
    const float *G = reinterpret_cast<const float *>(nb + L::cG);
    const float *Be = reinterpret_cast<const float *>(nb + L::cBe);
    __bf16 *Ph = reinterpret_cast<__bf16 *>(nb + L::cPh);
    __bf16 *Pl = reinterpret_cast<__bf16 *>(nb + L::cPl);
    const GTile tt[2] = {t0, t1};
    // fragments of two k-steps of both tiles are loaded before their MFMAs
    constexpr int KG = NK < 2 ? NK : 2;
    f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
    for (int k0 = 0; k0 < NK; k0 += KG) {
        FDK fa[2][KG], fb[2][KG];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (tt[u].kind) {
                const __bf16 *Xs = tt[u].kind == 2 ? Qs : Ks;
                const bool direct = tt[u].kind == 1 && tt[u].rb != tt[u].cb;
                const int ra = direct ? tt[u].rb : tt[u].cb, rbb = direct ? tt[u].cb : tt[u].rb;
#pragma unroll
                for (int kk = 0; kk < KG; ++kk) {
                    fa[u][kk] = frag_rows<__bf16, KS_DK>(Ks, KP, 16 * ra, (k0 + kk) * KS_DK, lane);
                    fb[u][kk] = frag_rows<__bf16, KS_DK>(Xs, KP, 16 * rbb, (k0 + kk) * KS_DK, lane);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (tt[u].kind) {
#pragma unroll
                for (int kk = 0; kk < KG; ++kk) acc[u] = FDK::mma(fa[u][kk], fb[u][kk], acc[u]);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        if (tt[u].kind) {
            const int rb = tt[u].rb, cbk = tt[u].cb;
            const bool isP = tt[u].kind == 2;
            const int r = 16 * rb + ln;
            const int j0 = 16 * cbk + 4 * lg;
            f32x4 val;
            if (!isP && rb != cbk) {
                // off-diagonal A block, direct layout: rows r0 + e, column j
                const int r0 = 16 * rb + 4 * lg, j = 16 * cbk + ln;
                const f32x4 ea4 = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(nb + L::cEa) + r0);
                const f32x4 be4 = *reinterpret_cast<const f32x4 *>(Be + r0);
                const float eb = reinterpret_cast<const float *>(nb + L::cEb)[rb * C + j];
                val = acc[u] * eb * ea4 * be4;
                const int oidx = rb * (rb - 1) / 2 + cbk;
                bf16x4 hv, lv;
                split4(val, hv, lv);
                *reinterpret_cast<bf16x4 *>(Aoh + oidx * 256 + lane * 4) = hv;
                *reinterpret_cast<bf16x4 *>(Aol + oidx * 256 + lane * 4) = lv;
                continue;
            }
            if (rb == cbk) {
                // diagonal block: Gamma_rj = 2^(G_r - G_j) per entry, masked to the triangle
                const float Gr = G[r];
                const f32x4 Gj = *reinterpret_cast<const f32x4 *>(G + j0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float gam = __builtin_amdgcn_exp2f(fminf(Gr - Gj[e], 0.f));
                    const float keep = (r > j0 + e || (isP && r == j0 + e)) ? 1.f : 0.f;
                    val[e] = gam * acc[u][e] * keep;
                }
            } else {
                // r > j always: Gamma_rj = 2^(G_r - G_{16 rb}) * 2^(G_{16 rb} - G_j), both <= 1
                const float ea = reinterpret_cast<const float *>(nb + L::cEa)[r];
                const f32x4 eb = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(nb + L::cEb) + rb * C + j0);
                val = acc[u] * eb * ea;
            }
            if (isP) {
                const int idx = rb * (rb + 1) / 2 + cbk;
                bf16x4 hv, lv;
                split4(val, hv, lv);
                *reinterpret_cast<bf16x4 *>(Ph + idx * BLK + ln * PB + 4 * lg) = hv;
                *reinterpret_cast<bf16x4 *>(Pl + idx * BLK + ln * PB + 4 * lg) = lv;
            } else {
                val *= Be[r];
                *reinterpret_cast<f32x4 *>(Ad + (rb * 16 + ln) * AP + 4 * lg) = val;
            }
        }
    }
}

template <int C, int DK>
__global__ __launch_bounds__(WIDE_THREADS, 1) void gdn_prefill_wide_kernel(KParams p)
{
    using L = PipeLay<C, DK>;
    using F16 = Frag<__bf16, 16>;
    using FDK = Frag<__bf16, L::KS_DK>;
    using FC = Frag<__bf16, L::KS_C>;
    constexpr int KP = L::KP, CPU = L::CPU, CPD = L::CPD, NB = L::NB, NSB = L::NSB, MS = L::MS, AP = L::AP;
    constexpr int KS_DK = L::KS_DK, KS_C = L::KS_C, NK = DK / KS_DK;
    constexpr int NJOB = L::NOFF + L::NTRI;     // Gram jobs per chunk
    constexpr int NWORK = 11;                   // wavefronts taking Gram jobs

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    auto cbuf = [&](int parity) { return smem + parity * L::CBUF; };
    float *Ad = reinterpret_cast<float *>(smem + L::oAd);
    __bf16 *Aoh = reinterpret_cast<__bf16 *>(smem + L::oAoh);
    __bf16 *Aol = reinterpret_cast<__bf16 *>(smem + L::oAol);
    __bf16 *STh = reinterpret_cast<__bf16 *>(smem + L::oSTh);
    __bf16 *STl = reinterpret_cast<__bf16 *>(smem + L::oSTl);
    float *Wx = reinterpret_cast<float *>(smem + L::oW);
    __bf16 *UTh = reinterpret_cast<__bf16 *>(smem + L::oUh);
    __bf16 *UTl = reinterpret_cast<__bf16 *>(smem + L::oUl);
    __bf16 *UdTh = reinterpret_cast<__bf16 *>(smem + L::oUdh);
    __bf16 *UdTl = reinterpret_cast<__bf16 *>(smem + L::oUdl);

    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());   // wave-uniform
    const int ln = lane & 15, lg = lane >> 4;

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
    const __bf16 *qg = static_cast<const __bf16 *>(p.q);
    const __bf16 *kg = static_cast<const __bf16 *>(p.k);
    const __bf16 *vg = static_cast<const __bf16 *>(p.v);
    const int64_t NC = (T + C - 1) / C;

    // Gram-job worker index: waves 1-7 -> 0-6, waves 12-15 -> 7-10, others none
    const int work = (wave >= 1 && wave <= 7) ? wave - 1 : (wave >= 12 ? wave - 5 : -1);
    auto gram_jobs = [&](int64_t it) {
        if (work >= 0 && it + 1 < NC) {
            char *nb = cbuf((int)((it + 1) & 1));
            for (int j = work; j < NJOB; j += 2 * NWORK)
                gram_pair<C, DK>(nb, Ad, Aoh, Aol, gram_job<C, DK>(j), gram_job<C, DK>(j + NWORK), lane);
        }
    };

    if (wave < 4) {
        // ===================== S-waves: state slice rows ib = w + 4m =====================
        const int sw = wave;
        f32x4 S[MS];
#pragma unroll
        for (int m = 0; m < MS; ++m) S[m] = zero4();
        auto write_state_operand = [&]() {
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int ib = sw + 4 * m;
                if (ib < NSB) {
                    bf16x4 hv, lv;
                    split4(S[m], hv, lv);
                    *reinterpret_cast<bf16x4 *>(STh + ln * KP + 16 * ib + 4 * lg) = hv;
                    *reinterpret_cast<bf16x4 *>(STl + ln * KP + 16 * ib + 4 * lg) = lv;
                }
            }
        };
        if (p.s0) {
            const float *s0 = p.s0 + bh * (int64_t)DK * Dv;
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int ib = sw + 4 * m;
                if (ib < NSB) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) S[m][e] = s0[(int64_t)(16 * ib + 4 * lg + e) * Dv + n0 + ln];
                }
            }
        }
        write_state_operand();

        for (int64_t it = -1; it < NC; ++it) {
            const bool act = it >= 0;
            const char *cb = cbuf((int)(it & 1));
            const __bf16 *Ks = reinterpret_cast<const __bf16 *>(cb + L::cK);
            // ---- phase 1: R = diag(beta)(V - diag(e^G) K S);  W_i = T_ii R_i
            if (act && sw < NB) {
                const __bf16 *Vs = reinterpret_cast<const __bf16 *>(cb + L::cV);
                const float *EG = reinterpret_cast<const float *>(cb + L::cEG);
                const float *Be = reinterpret_cast<const float *>(cb + L::cBe);
                const __bf16 *Td = reinterpret_cast<const __bf16 *>(cb + L::cTd);
                const int rb = sw;
                FDK kf[NK], sh[NK], slo[NK];
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    kf[kk] = frag_rows<__bf16, KS_DK>(Ks, KP, 16 * rb, kk * KS_DK, lane);
                    sh[kk] = frag_rows<__bf16, KS_DK>(STh, KP, 0, kk * KS_DK, lane);
                    slo[kk] = frag_rows<__bf16, KS_DK>(STl, KP, 0, kk * KS_DK, lane);
                }
                const F16 tf = frag_rows<__bf16, 16>(Td + rb * BLK, PB, 0, 0, lane);
                f32x4 ks_h = zero4(), ks_l = zero4();
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    ks_h = FDK::mma(kf[kk], sh[kk], ks_h);
                    ks_l = FDK::mma(kf[kk], slo[kk], ks_l);
                }
                F16 rh, rl;
                f32x4 rv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * lg + e;
                    rv[e] = Be[r] * ((float)Vs[r * BV + ln] - EG[r] * (ks_h[e] + ks_l[e]));
                }
                split4(rv, rh.v, rl.v);
                f32x4 w = F16::mma(tf, rh, zero4());
                w = F16::mma(tf, rl, w);
                *reinterpret_cast<f32x4 *>(Wx + (rb * 64 + lane) * 4) = w;
            }
            __syncthreads();

            // ---- phase 2: wave 0 runs U_i = W_i + sum_k (-N_ik) U_k; waves 1-3 take Gram jobs
            if (sw == 0) {
                if (act) {
                    const __bf16 *Nn = reinterpret_cast<const __bf16 *>(cb + L::cNn);
                    const float *Ed = reinterpret_cast<const float *>(cb + L::cEd);
                    f32x4 acc[NB], acc2[NB];
#pragma unroll
                    for (int i = 0; i < NB; ++i) {
                        acc[i] = *reinterpret_cast<const f32x4 *>(Wx + (i * 64 + lane) * 4);
                        acc2[i] = zero4();
                    }
#pragma unroll
                    for (int k = 0; k < NB; ++k) {
                        const int r0 = 16 * k + 4 * lg;
                        const f32x4 ed = *reinterpret_cast<const f32x4 *>(Ed + r0);
                        F16 uh, ul;
                        bf16x4 dh, dl;
                        const f32x4 u = acc[k] + acc2[k];
                        split4(u, uh.v, ul.v);
                        split4(ed * u, dh, dl);
#pragma unroll
                        for (int i = k + 1; i < NB; ++i) {
                            const F16 a = frag_rows<__bf16, 16>(Nn + (i * (i - 1) / 2 + k) * BLK, PB, 0, 0, lane);
                            acc[i] = F16::mma(a, uh, acc[i]);
                            acc2[i] = F16::mma(a, ul, acc2[i]);
                        }
                        *reinterpret_cast<bf16x4 *>(UTh + ln * CPU + r0) = uh.v;
                        *reinterpret_cast<bf16x4 *>(UTl + ln * CPU + r0) = ul.v;
                        // tokens (r0, r0 + 1) and (r0 + 2, r0 + 3) stay adjacent in the
                        // permuted order of the decayed U^T
                        const int pa = ln * CPD + ud_pos<KS_C>(r0), pb = ln * CPD + ud_pos<KS_C>(r0 + 2);
                        *reinterpret_cast<bf16x2 *>(UdTh + pa) = bf16x2{dh[0], dh[1]};
                        *reinterpret_cast<bf16x2 *>(UdTh + pb) = bf16x2{dh[2], dh[3]};
                        *reinterpret_cast<bf16x2 *>(UdTl + pa) = bf16x2{dl[0], dl[1]};
                        *reinterpret_cast<bf16x2 *>(UdTl + pb) = bf16x2{dl[2], dl[3]};
                    }
                }
            } else {
                gram_jobs(it);
            }
            __syncthreads();

            // ---- phase 3: S <- e^{G_C} S + K^T (e^{G_C-G} U)
            if (act) {
                const float *EG = reinterpret_cast<const float *>(cb + L::cEG);
                const float EGC = EG[C - 1];
                constexpr int NJ = C / KS_C;
                FC uh[NJ], ul[NJ], ka[MS][NJ];
#pragma unroll
                for (int jj = 0; jj < NJ; ++jj) {
                    uh[jj] = frag_rows<__bf16, KS_C>(UdTh, CPD, 0, jj * KS_C, lane);
                    ul[jj] = frag_rows<__bf16, KS_C>(UdTl, CPD, 0, jj * KS_C, lane);
                }
#pragma unroll
                for (int m = 0; m < MS; ++m) {
                    const int ib = sw + 4 * m;
                    if (ib < NSB) {
#pragma unroll
                        for (int jj = 0; jj < NJ; ++jj) ka[m][jj] = k_cols_paired<KS_C>(Ks, KP, 16 * ib, jj * KS_C, lane);
                    }
                }
#pragma unroll
                for (int m = 0; m < MS; ++m) {
                    const int ib = sw + 4 * m;
                    if (ib < NSB) {
                        f32x4 acc = S[m] * EGC, acc2 = zero4();
#pragma unroll
                        for (int jj = 0; jj < NJ; ++jj) {
                            acc = FC::mma(ka[m][jj], uh[jj], acc);
                            acc2 = FC::mma(ka[m][jj], ul[jj], acc2);
                        }
                        S[m] = acc + acc2;
                    }
                }
                write_state_operand();
            }
            __syncthreads();
        }

        if (p.sT) {
            float *sT = p.sT + bh * (int64_t)DK * Dv;
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int ib = sw + 4 * m;
                if (ib < NSB) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) sT[(int64_t)(16 * ib + 4 * lg + e) * Dv + n0 + ln] = S[m][e];
                }
            }
        }
    } else if (wave < 8) {
        // ===================== Y-waves: row block rb = w - 4 =====================
        const int rb = wave - 4;
        f32x4 qs = zero4();
        for (int64_t it = -1; it < NC; ++it) {
            const bool act = it >= 0 && rb < NB;
            const char *cb = cbuf((int)(it & 1));
            // ---- phase 1: Q S of this row block (state at the chunk's start)
            if (act) {
                const __bf16 *Qs = reinterpret_cast<const __bf16 *>(cb + L::cQ);
                FDK qf[NK], sh[NK], slo[NK];
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    qf[kk] = frag_rows<__bf16, KS_DK>(Qs, KP, 16 * rb, kk * KS_DK, lane);
                    sh[kk] = frag_rows<__bf16, KS_DK>(STh, KP, 0, kk * KS_DK, lane);
                    slo[kk] = frag_rows<__bf16, KS_DK>(STl, KP, 0, kk * KS_DK, lane);
                }
                f32x4 qh = zero4(), ql = zero4();
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    qh = FDK::mma(qf[kk], sh[kk], qh);
                    ql = FDK::mma(qf[kk], slo[kk], ql);
                }
                qs = qh + ql;
            }
            __syncthreads();
            // ---- phase 2: Gram jobs of the next chunk
            gram_jobs(it);
            __syncthreads();
            // ---- phase 3: Y = e^G Q S + P U
            if (act) {
                const float *EG = reinterpret_cast<const float *>(cb + L::cEG);
                const __bf16 *Ph = reinterpret_cast<const __bf16 *>(cb + L::cPh);
                const __bf16 *Pl = reinterpret_cast<const __bf16 *>(cb + L::cPl);
                const int64_t c0 = it * C;
                f32x4 acc, acc2 = zero4();
                const f32x4 eg = *reinterpret_cast<const f32x4 *>(EG + 16 * rb + 4 * lg);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = eg[e] * qs[e];
#pragma unroll
                for (int jb = 0; jb < NB; ++jb) {
                    if (jb <= rb) {
                        const int pidx = rb * (rb + 1) / 2 + jb;
                        const F16 ah = frag_rows<__bf16, 16>(Ph + pidx * BLK, PB, 0, 0, lane);
                        const F16 al = frag_rows<__bf16, 16>(Pl + pidx * BLK, PB, 0, 0, lane);
                        const F16 uh = frag_rows<__bf16, 16>(UTh, CPU, 0, 16 * jb, lane);
                        const F16 ul = frag_rows<__bf16, 16>(UTl, CPU, 0, 16 * jb, lane);
                        acc = F16::mma(ah, uh, acc);
                        acc2 = F16::mma(al, uh, acc2);
                        acc2 = F16::mma(ah, ul, acc2);
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t t = c0 + 16 * rb + 4 * lg + e;
                    if (t < T) p.y[((b * T + t) * H + h) * Dv + n0 + ln] = acc[e] + acc2[e];
                }
            }
            __syncthreads();
        }
    } else {
        // ===================== G-waves (8-15) =====================
        // phase 1: N_ik of chunk it (waves 9-11); stage chunk it+1; decay prefix
        //          and factor tables (wave 12); prefetch chunk it+2
        // phase 2: diagonal A_ii blocks of chunk it+1 (waves 8-11); Gram jobs (12-15)
        // phase 3: T_ii = (I + A_ii)^-1 of chunk it+1 (waves 8-11)
        const int gw = wave - 8;          // 0-7
        const int gtid = tid - 512;       // 0-511
        constexpr int VPR = DK / 8;                         // 16-byte vectors per K/Q row
        constexpr int NKV = (C * VPR + 511) / 512;          // per G thread
        // per-thread global addresses of the chunk-0 rows this thread loads;
        // chunk c adds c * C tokens
        const int64_t rowc = b * T;
        const __bf16 *kp[NKV], *qp[NKV];
        int rr[NKV];
#pragma unroll
        for (int i = 0; i < NKV; ++i) {
            const int vi = gtid + 512 * i;
            rr[i] = vi < C * VPR ? vi / VPR : -1;             // row within the chunk (-1: none)
            const int row0 = rr[i] < 0 ? 0 : rr[i];
            const int col = (vi % VPR) * 8;
            kp[i] = kg + (rowc + row0) * p.ks + h * DK + col;
            qp[i] = qg + (rowc + row0) * p.qs + h * DK + col;
        }
        const int vr = gtid >> 1;
        const __bf16 *vp = vg + (rowc + (gtid < C * 2 ? vr : 0)) * p.vs + h * Dv + n0 + (gtid & 1) * 8;
        const int ar = gtid - 256;         // alpha/beta row held by wave 12 (gtid 256..319)
        const bool has_ab = ar >= 0 && ar < C;
        const float *alp = p.alpha + (rowc + (has_ab ? ar : 0)) * H + h;
        const float *bep = p.beta + (rowc + (has_ab ? ar : 0)) * H + h;
        f32x4 pk[NKV], pq[NKV], pv = zero4();
        float pal = 1.f, pbe = 0.f;
        auto prefetch = [&](int64_t c) {
            const int64_t c0 = c * C;
#pragma unroll
            for (int i = 0; i < NKV; ++i) {
                pk[i] = zero4();
                pq[i] = zero4();
                if (rr[i] >= 0 && c0 + rr[i] < T) {
                    pk[i] = *reinterpret_cast<const f32x4 *>(kp[i] + c0 * p.ks);
                    pq[i] = *reinterpret_cast<const f32x4 *>(qp[i] + c0 * p.qs);
                }
            }
            if (gtid < C * 2) {            // V slice: 16 bf16 = two 16-byte vectors per row
                pv = zero4();
                if (c0 + vr < T) pv = *reinterpret_cast<const f32x4 *>(vp + c0 * p.vs);
            }
            if (has_ab) {
                const bool ok = c0 + ar < T;
                pal = ok ? alp[c0 * H] : 1.f;
                pbe = ok ? bep[c0 * H] : 0.f;
            }
        };
        prefetch(0);
        float X[4] = {0.f, 0.f, 0.f, 0.f};   // T_ii rows (waves 8-11), phase 3 -> next phase 1

        for (int64_t it = -1; it < NC; ++it) {
            const bool act = it + 1 < NC;
            char *nb = cbuf((int)((it + 1) & 1));
            // ---- phase 1
            if (it >= 0 && gw >= 1 && gw < 4 && gw < NB) {
                // N_ik = T_ii A_ik of chunk it (T_ii from the previous phase 3)
                const int i = gw;
                __bf16 *Nn = reinterpret_cast<__bf16 *>(cbuf((int)(it & 1)) + L::cNn);
                // lane (ln, lg) holds T_ii[ln][4 lg + e]: the B operand of
                // N_ik^T = A_ik^T T_ii^T, whose A operand the Gram epilogue stored in
                // lane order; the result row ln, columns 4 lg + e, is a row of N_ik
                F16 th, tl;
                split4(f32x4{X[0], X[1], X[2], X[3]}, th.v, tl.v);
#pragma unroll
                for (int k = 0; k < NB; ++k) {
                    if (k < i) {
                        const int oidx = i * (i - 1) / 2 + k;
                        F16 ah, al;
                        ah.v = *reinterpret_cast<const bf16x4 *>(Aoh + oidx * 256 + lane * 4);
                        al.v = *reinterpret_cast<const bf16x4 *>(Aol + oidx * 256 + lane * 4);
                        f32x4 n = F16::mma(ah, th, zero4());
                        n = F16::mma(al, th, n);
                        n = F16::mma(ah, tl, n);
                        *reinterpret_cast<bf16x4 *>(Nn + oidx * BLK + ln * PB + 4 * lg) =
                            __builtin_convertvector(-n, bf16x4);
                    }
                }
            }
            if (act) {
                __bf16 *Ks = reinterpret_cast<__bf16 *>(nb + L::cK);
                __bf16 *Qs = reinterpret_cast<__bf16 *>(nb + L::cQ);
                __bf16 *Vs = reinterpret_cast<__bf16 *>(nb + L::cV);
#pragma unroll
                for (int i = 0; i < NKV; ++i) {
                    const int vi = gtid + 512 * i;
                    if (vi < C * VPR) {
                        const int r = vi / VPR, col = (vi % VPR) * 8;
                        *reinterpret_cast<f32x4 *>(Ks + r * KP + col) = pk[i];
                        *reinterpret_cast<f32x4 *>(Qs + r * KP + col) = pq[i];
                    }
                }
                if (gtid < C * 2) *reinterpret_cast<f32x4 *>(Vs + (gtid >> 1) * BV + (gtid & 1) * 8) = pv;
                if (gw == 4) {
                    // inclusive prefix of log2 alpha over the chunk (lane = token) and the
                    // decay factors used by the Gram tiles and the state update
                    const float g2 = wave_inclusive_sum(lane < C ? __builtin_amdgcn_logf(pal) : 0.f, lane);
                    const float gC = lane_value(g2, C - 1);
                    const float gblk = row_bcast<0>(g2);      // G at the first row of this lane's block
                    if (lane < C) {
                        reinterpret_cast<float *>(nb + L::cG)[lane] = g2;
                        reinterpret_cast<float *>(nb + L::cEG)[lane] = __builtin_amdgcn_exp2f(g2);
                        reinterpret_cast<float *>(nb + L::cBe)[lane] = pbe;
                        reinterpret_cast<float *>(nb + L::cEd)[lane] = __builtin_amdgcn_exp2f(gC - g2);
                        reinterpret_cast<float *>(nb + L::cEa)[lane] = __builtin_amdgcn_exp2f(g2 - gblk);
                    }
#pragma unroll
                    for (int rb = 1; rb < NB; ++rb) {
                        const float gref = lane_value(g2, 16 * rb);
                        if (lane < C)
                            reinterpret_cast<float *>(nb + L::cEb)[rb * C + lane] =
                                lane < 16 * rb ? __builtin_amdgcn_exp2f(gref - g2) : 0.f;
                    }
                }
                if (it + 2 < NC) prefetch(it + 2);    // consumed by phase 1 of the next iteration
            }
            __syncthreads();

            // ---- phase 2
            if (gw < 4) {
                if (act && gw < NB) gram_pair<C, DK>(nb, Ad, Aoh, Aol, GTile{1, gw, gw}, GTile{0, 0, 0}, lane);
            } else {
                gram_jobs(it);
            }
            __syncthreads();

            // ---- phase 3: T_ii of chunk it+1 (waves 8-11)
            if (act && gw < 4 && gw < NB) {
                const int i = gw;
                float Lr[16];
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const f32x4 v4 = *reinterpret_cast<const f32x4 *>(Ad + (i * 16 + ln) * AP + 4 * s4);
                    Lr[4 * s4] = v4[0]; Lr[4 * s4 + 1] = v4[1]; Lr[4 * s4 + 2] = v4[2]; Lr[4 * s4 + 3] = v4[3];
                }
                // lane (ln, lg) carries row ln of T_ii, columns 4 lg + e
#pragma unroll
                for (int e = 0; e < 4; ++e) X[e] = (ln == 4 * lg + e) ? 1.f : 0.f;
                tri_solve16(X, Lr, ln, std::make_integer_sequence<int, 15>{});
                __bf16 *Td = reinterpret_cast<__bf16 *>(nb + L::cTd);
                *reinterpret_cast<bf16x4 *>(Td + i * BLK + ln * PB + 4 * lg) =
                    __builtin_convertvector((f32x4{X[0], X[1], X[2], X[3]}), bf16x4);
            }
            __syncthreads();
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
    if constexpr (sizeof(Tin) == 2)
        hipLaunchKernelGGL((gdn_prefill_wide_kernel<C, DK>), dim3((unsigned)grid), dim3(WIDE_THREADS), 0, stream, kp);
    else
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

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream)
{
    if (a.B * a.H == 0) return hipSuccess;
    if (a.T == 0) {
        if (!a.sT || a.sT == a.s0) return hipSuccess;
        const int64_t n = a.B * a.H * a.Dk * a.Dv;
        hipLaunchKernelGGL(copy_or_zero_state, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a.s0, a.sT, n);
        return hipGetLastError();
    }
    return a.bf16 ? launch_c<__bf16>(a, stream) : launch_c<float>(a, stream);
}

}  // namespace gdn
