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
// 16-column slice of the state in MFMA accumulators, like the forward.  Every
// product accumulates in fp32.  bf16 inputs: products on bf16 MFMA, with the
// operands that are not inputs (states, T, P, chunk matrices, gradients) split
// into bf16 pairs hi + lo; fp32 inputs: fp32 MFMA (16x16x4).
// Ragged tails are padded with identity tokens (alpha = 1, beta = 0, zeros),
// whose gradients are never written.
#include "common.hpp"
#include "gemm_nt.hpp"
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
    float *ub, *wb, *dxb;      // per chunk [C][Dv]: U, W~ = V - e^G K S (state pass), dX (adjoint pass)
    int64_t T, H, Dv, NC;
    int64_t qs, ks, vs;        // elements between consecutive tokens of q, k, v (H * D when dense)
    float *y, *sT;             // forward path: y [B, T, H, Dv], final state or null
    int64_t rec_floats;
    int xcd_map;               // state passes: the slices of one head on one XCD (B*H % 8 == 0)
};

// ---- per-chunk record: T [C][C], P [C][C], Ak [C][C], G2 [C] (log2 cumulative
// decay), Ed [C] = 2^(G2_{C-1} - G2_r) (formed from the fp64 prefix, so that it
// keeps full precision when G2 itself is large)
template <int C> struct Rec {
    static constexpr int oT = 0, oP = C * C, oA = 2 * C * C, oG = 3 * C * C, oEd = 3 * C * C + C;
};

// Register-staged copies into LDS.  Every load of a tile is issued before any
// of them is used (fixed trip counts, raw input kept in registers), so a tile
// costs one memory latency, and the next chunk's tiles can be in flight while
// the current chunk is computed.  Conversion to fp32 happens at the LDS store.
template <typename Tin> struct Raw4;
template <> struct Raw4<float> {
    using type = f32x4;
    static __device__ __forceinline__ type load(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
    static __device__ __forceinline__ type zero() { return zero4(); }
    static __device__ __forceinline__ f32x4 widen(type x) { return x; }
};
template <> struct Raw4<__bf16> {
    using type = bf16x4;
    static __device__ __forceinline__ type load(const __bf16 *p) { return *reinterpret_cast<const bf16x4 *>(p); }
    static __device__ __forceinline__ type zero() { return bf16x4{(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f}; }
    static __device__ __forceinline__ f32x4 widen(type x) { return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]}; }
};

// Rows t = c0 .. c0+C-1, columns n0 .. n0+W-1 of head h of a [B, T, H, ld]
// tensor whose consecutive tokens are `tok` elements apart (H * ld when dense);
// zeros past T.  Stored with pitch P floats.
template <typename Tin, int C, int W, int NTH = NT> struct RowsTile {
    using R = Raw4<Tin>;
    static constexpr int NU = C * W / 4, NV = (NU + NTH - 1) / NTH;
    typename R::type v[NV];
    __device__ __forceinline__ void load(const Tin *src, int64_t b, int64_t h, int64_t c0, int64_t T, int64_t tok,
                                         int64_t ld, int n0 = 0) {
#pragma unroll
        for (int it = 0; it < NV; ++it) {
            const int vi = threadIdx.x + NTH * it;
            const int r = vi / (W / 4), col = (vi % (W / 4)) * 4;
            const int64_t t = c0 + r;
            v[it] = R::zero();
            if ((NU % NTH == 0 || vi < NU) && t < T) v[it] = R::load(src + (b * T + t) * tok + h * ld + n0 + col);
        }
    }
    template <int P> __device__ __forceinline__ void store(float *dst) const {
#pragma unroll
        for (int it = 0; it < NV; ++it) {
            const int vi = threadIdx.x + NTH * it;
            const int r = vi / (W / 4), col = (vi % (W / 4)) * 4;
            if (NU % NTH == 0 || vi < NU) *reinterpret_cast<f32x4 *>(dst + r * P + col) = R::widen(v[it]);
        }
    }
};

// R x W block of a dense row-major fp32 matrix with row stride `ld`, stored
// with pitch P floats.
template <int R, int W, int NTH = NT> struct DenseTile {
    static constexpr int NU = R * W / 4, NV = (NU + NTH - 1) / NTH;
    f32x4 v[NV];
    __device__ __forceinline__ void load(const float *src, int64_t ld) {
#pragma unroll
        for (int it = 0; it < NV; ++it) {
            const int vi = threadIdx.x + NTH * it;
            const int r = vi / (W / 4), col = (vi % (W / 4)) * 4;
            v[it] = zero4();
            if (NU % NTH == 0 || vi < NU) v[it] = *reinterpret_cast<const f32x4 *>(src + r * ld + col);
        }
    }
    template <int P> __device__ __forceinline__ void store(float *dst) const {
#pragma unroll
        for (int it = 0; it < NV; ++it) {
            const int vi = threadIdx.x + NTH * it;
            const int r = vi / (W / 4), col = (vi % (W / 4)) * 4;
            if (NU % NTH == 0 || vi < NU) *reinterpret_cast<f32x4 *>(dst + r * P + col) = v[it];
        }
    }
};

// lower-triangle block index -> (rb, cb), row-major over rb
__device__ __forceinline__ void tri_block(int idx, int &rb, int &cb) {
    rb = 0;
    while ((rb + 1) * (rb + 2) / 2 <= idx) ++rb;
    cb = idx - rb * (rb + 1) / 2;
}

// Workgroup -> (b*H + h, value slice) for the state passes.  Workgroups are
// dealt to the 8 XCDs round-robin; with xcd_map the NS slices of one head get
// ids equal mod 8, so they run on one XCD and share its L2 copy of the chunk's
// K, Q, T and P.
__device__ __forceinline__ void slice_of(int64_t bid, int64_t NS, int xcd_map, int64_t &bh, int64_t &sl) {
    if (xcd_map) {
        const int64_t xcd = bid & 7, local = bid >> 3;
        bh = (local / NS) * 8 + xcd;
        sl = local % NS;
    } else {
        bh = bid / NS;
        sl = bid % NS;
    }
}

// Sum over the 16 lanes of each 16-lane row, left in the row's last lane
// (ln == 15): an inclusive scan by DPP row shifts, no LDS traffic.
__device__ __forceinline__ float row16_total(float x) {
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x += row_shr<8>(x);
    return x;
}

// four fp32 values as bf16 pairs hi (at hi) + lo (at lo)
__device__ __forceinline__ void store_split4(__bf16 *hi, __bf16 *lo, const f32x4 x) {
    bf16x4 h, l;
    split4(x, h, l);
    *reinterpret_cast<bf16x4 *>(hi) = h;
    *reinterpret_cast<bf16x4 *>(lo) = l;
}

// ===========================================================================
// 1. prep: G2, T = (I + A)^-1, P, Ak of one chunk
// ===========================================================================
template <typename Tin, int C, int DK>
__global__ __launch_bounds__(NT) void bwd_prep_kernel(BwdParams p)
{
    // The Gram runs on bf16 MFMA with fp32 sums: bf16 inputs are exact
    // operands; fp32 inputs are split into bf16 pairs hi + lo (hi = bf16(x),
    // lo = bf16(x - hi)) and each product sums hi*hi + hi*lo + lo*hi.
    // The wavefronts pass values to each other only through LDS, and nothing
    // here reads the record back, so the barriers order LDS only: the record's
    // stores stay in flight across them.
    constexpr bool F32IN = sizeof(Tin) == 4;
    constexpr int NPART = F32IN ? 2 : 1;                 // bf16 parts per K or Q element
    constexpr int KP = DK + 8, CP = C + 4, NB = C / 16, KSD = DK % 32 == 0 ? 32 : 16;
    constexpr int NTRI = NB * (NB + 1) / 2;
    using FG = Frag<__bf16, KSD>;
    // LDS: the K parts; a region holding one Q part at a time (fp32 inputs:
    // the hi part, then the lo part) until the P tiles are done, which A
    // reuses afterwards; T in K's rows once the K K^T tiles are done, where
    // they hold it: three workgroups per CU for fp32 inputs, four for bf16 at
    // C = 64, Dk = 128
    constexpr size_t KQB = (size_t)2 * C * KP;           // one bf16 C x Dk part
    constexpr size_t ATB = (size_t)4 * C * CP;           // one fp32 C x C matrix
    constexpr bool T_IN_K = ATB <= NPART * KQB;
    constexpr size_t oQ = NPART * KQB;
    constexpr size_t QREG = KQB > ATB ? KQB : ATB;
    constexpr size_t oA = oQ, oT = T_IN_K ? 0 : oQ + QREG;
    constexpr size_t oG = oQ + QREG + (T_IN_K ? 0 : ATB), BYTES = oG + 12 * C;   // G (fp64), beta
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) char smem[BYTES];
    __bf16 *Ks = reinterpret_cast<__bf16 *>(smem);                 // part j at Ks + j * C * KP
    __bf16 *Qs = reinterpret_cast<__bf16 *>(smem + oQ);
    float *As = reinterpret_cast<float *>(smem + oA);
    float *Ts = reinterpret_cast<float *>(smem + oT);
    double *Gs = reinterpret_cast<double *>(smem + oG);
    float *Bs = reinterpret_cast<float *>(Gs + C);

    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id(), ln = lane & 15, lg = lane >> 4;
    const int64_t bh = blockIdx.x / p.NC, c = blockIdx.x % p.NC;
    const int64_t H = p.H, T = p.T, b = bh / H, h = bh % H, c0 = c * C;
    float *rec = p.rec + (bh * p.NC + c) * p.rec_floats;

    RowsTile<Tin, C, DK> tq;         // fp32 inputs: kept until the lo part of Q goes to LDS
    // the Q part `lo` (fp32 inputs; 0 = hi) into LDS
    auto write_q = [&](bool lo) {
#pragma unroll
        for (int it = 0; it < RowsTile<Tin, C, DK>::NV; ++it) {
            const int vi = tid + NT * it;
            const int r = vi / (DK / 4), col = (vi % (DK / 4)) * 4;
            if (RowsTile<Tin, C, DK>::NU % NT == 0 || vi < RowsTile<Tin, C, DK>::NU) {
                if constexpr (F32IN) {
                    bf16x4 hv, lv;
                    split4(tq.v[it], hv, lv);
                    *reinterpret_cast<bf16x4 *>(Qs + r * KP + col) = lo ? lv : hv;
                } else {
                    *reinterpret_cast<bf16x4 *>(Qs + r * KP + col) = tq.v[it];
                }
            }
        }
    };
    {
        RowsTile<Tin, C, DK> tk;
        tk.load(static_cast<const Tin *>(p.k), b, h, c0, T, p.ks, DK);
        tq.load(static_cast<const Tin *>(p.q), b, h, c0, T, p.qs, DK);
#pragma unroll
        for (int it = 0; it < RowsTile<Tin, C, DK>::NV; ++it) {
            const int vi = tid + NT * it;
            const int r = vi / (DK / 4), col = (vi % (DK / 4)) * 4;
            if (RowsTile<Tin, C, DK>::NU % NT == 0 || vi < RowsTile<Tin, C, DK>::NU) {
                if constexpr (F32IN) store_split4(Ks + r * KP + col, Ks + C * KP + r * KP + col, tk.v[it]);
                else *reinterpret_cast<bf16x4 *>(Ks + r * KP + col) = tk.v[it];
            }
        }
        write_q(false);
    }
    if (wave == 0) {
        const int64_t t = c0 + lane;
        const bool ok = lane < C && t < T;
        const float g2 = ok ? log2_decay(p.alpha[(b * T + t) * H + h]) : 0.f;
        const double G2 = wave_inclusive_sum_f64((double)g2, lane);
        const double GC = lane_value_f64(G2, C - 1);
        if (lane < C) {
            Gs[lane] = G2;
            Bs[lane] = ok ? p.beta[(b * T + t) * H + h] : 0.f;
            rec[Rec<C>::oG + lane] = (float)G2;
            rec[Rec<C>::oEd + lane] = __builtin_amdgcn_exp2f((float)(GC - G2));
        }
    }
    // blocks above the diagonal: zero in the record
    for (int i = tid; i < C * C; i += NT) {
        const int r = i / C, j = i % C;
        if (j / 16 > r / 16) {
            rec[Rec<C>::oP + i] = 0.f;
            rec[Rec<C>::oA + i] = 0.f;
        }
    }
    lds_barrier();

    // sum over Dk of X_rb Kp_cb^T for one bf16 part of each, added to acc
    auto gram_part = [&](const __bf16 *Xs, const __bf16 *Kp, int rb, int cb, f32x4 acc) {
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += KSD)
            acc = FG::mma(frag_rows<__bf16, KSD>(Xs, KP, 16 * rb, k0, lane), frag_rows<__bf16, KSD>(Kp, KP, 16 * cb, k0, lane), acc);
        return acc;
    };
    // one Gram tile D = X_rb K_cb^T (X = K, all its parts in LDS) on and below the diagonal
    auto gram = [&](const __bf16 *Xs, int rb, int cb) {
        f32x4 acc = zero4(), acc2 = zero4();
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += KSD) {
            const FG xh = frag_rows<__bf16, KSD>(Xs, KP, 16 * rb, k0, lane);
            const FG kh = frag_rows<__bf16, KSD>(Ks, KP, 16 * cb, k0, lane);
            acc = FG::mma(xh, kh, acc);
            if constexpr (F32IN) {
                acc2 = FG::mma(xh, frag_rows<__bf16, KSD>(Ks + C * KP, KP, 16 * cb, k0, lane), acc2);
                acc2 = FG::mma(frag_rows<__bf16, KSD>(Xs + C * KP, KP, 16 * rb, k0, lane), kh, acc2);
            }
        }
        return acc + acc2;
    };
    // Q K^T -> P (the last use of Q).  fp32 inputs: Qh Kh and Qh Kl with the hi
    // part of Q in LDS, then Ql Kh once the lo part has replaced it
    constexpr int NPT = (NTRI + 3) / 4;                  // P tiles per wave
    f32x4 pa[NPT], pb[NPT];
#pragma unroll
    for (int t = 0; t < NPT; ++t) {
        const int tile = wave + 4 * t;
        int rb = 0, cb = 0;
        if (tile < NTRI) tri_block(tile, rb, cb);
        pa[t] = zero4();
        pb[t] = zero4();
        if (tile < NTRI) {
            pa[t] = gram_part(Qs, Ks, rb, cb, pa[t]);
            if constexpr (F32IN) pb[t] = gram_part(Qs, Ks + C * KP, rb, cb, pb[t]);
        }
    }
    if constexpr (F32IN) {
        lds_barrier();                               // every wave is done with Qh
        write_q(true);
        lds_barrier();
#pragma unroll
        for (int t = 0; t < NPT; ++t) {
            const int tile = wave + 4 * t;
            int rb = 0, cb = 0;
            if (tile < NTRI) tri_block(tile, rb, cb);
            if (tile < NTRI) pb[t] = gram_part(Qs, Ks, rb, cb, pb[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < NPT; ++t) {
        const int tile = wave + 4 * t;
        if (tile >= NTRI) continue;
        int rb, cb;
        tri_block(tile, rb, cb);
        const f32x4 acc = pa[t] + pb[t];
        const int j = 16 * cb + ln;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * lg + e;
            const float gam = __builtin_amdgcn_exp2f((float)fmin(Gs[r] - Gs[j], 0.0));
            rec[Rec<C>::oP + r * C + j] = r >= j ? gam * acc[e] : 0.f;
        }
    }
    lds_barrier();                               // A replaces Q
    // K K^T -> Ak (record), A = diag(beta) Ak (LDS)
    for (int tile = wave; tile < NTRI; tile += 4) {
        int rb, cb;
        tri_block(tile, rb, cb);
        const f32x4 acc = gram(Ks, rb, cb);
        const int j = 16 * cb + ln;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * lg + e;
            const float gam = __builtin_amdgcn_exp2f((float)fmin(Gs[r] - Gs[j], 0.0));
            const float ak = r > j ? gam * acc[e] : 0.f;
            rec[Rec<C>::oA + r * C + j] = ak;
            As[r * CP + j] = Bs[r] * ak;
        }
    }
    lds_barrier();                               // T may replace K
    for (int i = tid; i < C * C; i += NT) {
        const int r = i / C, j = i % C;
        if (j / 16 > r / 16) Ts[r * CP + j] = 0.f;
    }

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
    lds_barrier();

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
        lds_barrier();
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
    int64_t bh, sl;
    slice_of(blockIdx.x, NS, p.xcd_map, bh, sl);
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

    // registers holding the next chunk's tiles
    using InT = typename std::conditional<ADJ, float, Tin>::type;
    RowsTile<Tin, C, DK> rk, rq;
    DenseTile<C, C> rt, rp;
    RowsTile<InT, C, BV> ri;
    float rg = 0.f, rbeta = 0.f;
    auto fetch = [&](int64_t c) {
        const int64_t c0 = c * C;
        const float *rec = p.rec + (bh * NC + c) * p.rec_floats;
        rk.load(static_cast<const Tin *>(p.k), b, h, c0, T, H * DK, DK);
        rt.load(rec + Rec<C>::oT, C);
        if constexpr (ADJ) {
            rq.load(static_cast<const Tin *>(p.q), b, h, c0, T, H * DK, DK);
            rp.load(rec + Rec<C>::oP, C);
            ri.load(p.dy, b, h, c0, T, H * Dv, Dv, n0);
        } else {
            ri.load(static_cast<const Tin *>(p.v), b, h, c0, T, H * Dv, Dv, n0);
        }
        if (threadIdx.x < C) {
            const int64_t t = c0 + threadIdx.x;
            rg = rec[Rec<C>::oG + threadIdx.x];
            rbeta = t < T ? p.beta[(b * T + t) * H + h] : 0.f;
        }
    };
    fetch(ADJ ? NC - 1 : 0);

    for (int64_t it = 0; it < NC; ++it) {
        const int64_t c = ADJ ? NC - 1 - it : it;

        rk.template store<KP>(Ks);
        rt.template store<CP>(Ts);
        ri.template store<VP>(Ins);
        if constexpr (ADJ) {
            rq.template store<KP>(Qs);
            rp.template store<CP>(Ps);
        }
        if (threadIdx.x < C) {
            Gs[threadIdx.x] = rg;
            Bs[threadIdx.x] = rbeta;
        }
        if (it + 1 < NC) fetch(ADJ ? c - 1 : c + 1);

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
        lds_barrier();
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
                float *wg = p.wb + (bh * NC + c) * C * Dv + n0 + ln;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * lg + e;
                    const float wt = Ins[r * VP + ln] - __builtin_amdgcn_exp2f(Gs[r]) * ks[e];
                    Xs[r * VP + ln] = Bs[r] * wt;
                    wg[r * Dv] = wt;
                }
            }
        }
        lds_barrier();

        // step 2: forward: U = T X, stored as d o U (transposed);
        // adjoint: dR = diag(beta) T^T dU, stored as -e^G o dR (transposed)
        if (wave < NB) {
            const int rb = wave;
            f32x4 acc = zero4();
            if constexpr (ADJ) {
                for (int kb = rb; kb < NB; ++kb)
                    acc = F16::mma(frag_cols<float, 16>(Ts, CP, 16 * rb, 16 * kb, lane),
                                   frag_cols<float, 16>(Xs, VP, 0, 16 * kb, lane), acc);
                // acc = dX = T^T dU; dV = diag(beta) dX
                float *xg = p.dxb + (bh * NC + c) * C * Dv + n0 + ln;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * lg + e;
                    const int64_t t = c * C + r;
                    UdT[ln * CP + r] = -__builtin_amdgcn_exp2f(Gs[r]) * Bs[r] * acc[e];
                    xg[r * Dv] = acc[e];
                    if (t < T) p.dv[((b * T + t) * H + h) * Dv + n0 + ln] = Bs[r] * acc[e];
                }
            } else {
                for (int kb = 0; kb <= rb; ++kb)
                    acc = F16::mma(frag_rows<float, 16>(Ts, CP, 16 * rb, 16 * kb, lane),
                                   frag_cols<float, 16>(Xs, VP, 0, 16 * kb, lane), acc);
                // acc = U = T X
                float *ug = p.ub + (bh * NC + c) * C * Dv + n0 + ln;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rb + 4 * lg + e;
                    UdT[ln * CP + r] = __builtin_amdgcn_exp2f(GC - Gs[r]) * acc[e];
                    ug[r * Dv] = acc[e];
                }
            }
        }
        lds_barrier();

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
        lds_barrier();
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
// 2./3. state passes, bf16 inputs: bf16 MFMA with hi/lo operands
//
// Same steps as bwd_carry_kernel.  K and Q are exact in bf16; every other
// operand (the state, T, P, X, dY, dU and the decayed products) is split into
// a bf16 pair hi + lo and multiplied as hi*hi + hi*lo + lo*hi (two products
// where one side is exact), which keeps about 16 bits of every operand.
// Transposed operands (K^T, Q^T, T^T, P^T) come from the row-major LDS copies
// through transposing reads (ds_read_tr16_b64).
// ===========================================================================
typedef short i16x4t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4t *lds_i16x4p;

// Lane j of each 16-lane group supplies the address of 4 consecutive bf16;
// lane i of the group receives element i % 4 of the 4-element pieces of
// lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4.
__device__ __forceinline__ bf16x4 tr_read(const __bf16 *p) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                          (lds_i16x4p)(uintptr_t)(uint32_t)(uintptr_t)p));
}

// A operand (16-deep) of M^T, rows r0..r0+15 of M^T = columns of the row-major
// M (pitch P), k = rows k0..k0+15 of M: lane l holds M[k0 + 4(l/16) + e][r0 + l%16].
__device__ __forceinline__ Frag<__bf16, 16> tr_frag16(const __bf16 *M, int P, int r0, int k0, int lane) {
    const int j = lane & 15, g = lane >> 4;
    Frag<__bf16, 16> f;
    f.v = tr_read(M + (k0 + 4 * g + (j >> 2)) * P + r0 + 4 * (j & 3));
    return f;
}

// 32-deep A operand of M^T as two 16-deep pieces: lane group g holds k = k0 +
// 4g..+3 then k0 + 16 + 4g..+3.  B operands for it come from pair_rows32.
__device__ __forceinline__ Frag<__bf16, 32> tr_frag32(const __bf16 *M, int P, int r0, int k0, int lane) {
    const bf16x4 a = tr_frag16(M, P, r0, k0, lane).v, b = tr_frag16(M, P, r0, k0 + 16, lane).v;
    Frag<__bf16, 32> f;
    f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return f;
}

// B operand (rows of B^T, pitch P) with the k order of tr_frag32
__device__ __forceinline__ Frag<__bf16, 32> pair_rows32(const __bf16 *Bt, int P, int r0, int k0, int lane) {
    const int g = lane >> 4;
    const __bf16 *row = Bt + (r0 + (lane & 15)) * P + k0 + 4 * g;
    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(row), b = *reinterpret_cast<const bf16x4 *>(row + 16);
    Frag<__bf16, 32> f;
    f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return f;
}

template <int C, int DK, bool ADJ> struct Carry16Lay {
    static constexpr int KP = DK + 8, CP = C + 8;   // bf16 pitches
    static constexpr size_t KB = 2 * C * KP, CB = 2 * C * CP, SB = 2 * BV * KP, TB = 2 * BV * CP;
    static constexpr size_t oK = 0;                           // K, two buffers
    static constexpr size_t oQ = oK + 2 * KB;                 // Q, two buffers (adjoint)
    static constexpr size_t oTh = oQ + (ADJ ? 2 * KB : 0);
    static constexpr size_t oTl = oTh + CB;
    static constexpr size_t oPh = oTl + CB;                   // P (adjoint)
    static constexpr size_t oPl = oPh + (ADJ ? CB : 0);
    static constexpr size_t oSTh = oPl + (ADJ ? CB : 0);      // state operand, transposed
    static constexpr size_t oSTl = oSTh + SB;
    static constexpr size_t oXh = oSTl + SB;                  // X^T (state pass) or dU^T (adjoint)
    static constexpr size_t oXl = oXh + TB;
    static constexpr size_t oYh = oXl + TB;                   // dY^T (adjoint)
    static constexpr size_t oYl = oYh + (ADJ ? TB : 0);
    static constexpr size_t oUh = oYl + (ADJ ? TB : 0);       // decayed U^T or -e^G dR^T
    static constexpr size_t oUl = oUh + TB;
    static constexpr size_t oBh = oUl + TB;                   // (e^G o dY)^T, two buffers (adjoint)
    static constexpr size_t oBl = oBh + (ADJ ? 2 * TB : 0);
    static constexpr size_t oIn = oBl + (ADJ ? 2 * TB : 0);   // V slice, fp32 (state pass)
    static constexpr size_t oG = oIn + (ADJ ? 0 : 4 * C * VP);   // G2, two buffers
    static constexpr size_t oB = oG + 4 * 2 * C;              // beta, two buffers
    static constexpr size_t BYTES = oB + 4 * 2 * C;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// 8 wavefronts: waves 0-3 carry the chain of every chunk (K S, the C x C
// product, the state update) and the stores of what they produce; waves 4-7
// stage the next chunk into LDS while the chain runs and prefetch the one after
// it into registers.  Per chunk c (barriers A, B, C):
//   A..B  chain: step 1 on chunk c
//   B..C  chain: step 2;  staging: P, dY^T, e^G dY (or V) of the next chunk
//   C..A  chain: step 3;  staging: K, Q, T, G2, beta of the next chunk
// Single-buffered operands are rewritten only after their last read in chunk c.
constexpr int NTC = 512;

template <int C, int DK, bool ADJ>
__global__ __launch_bounds__(NTC) void bwd_carry16_kernel(BwdParams p)
{
    using L = Carry16Lay<C, DK, ADJ>;
    constexpr int KP = L::KP, CP = L::CP, NB = C / 16, NKB = DK / 16, MS = (NKB + 3) / 4;
    using F16 = Frag<__bf16, 16>;
    using F32 = Frag<__bf16, 32>;
    static_assert(DK % 32 == 0 || DK == 16, "Dk");
    constexpr int NST = 256;                                   // staging threads
    constexpr int NUK = C * DK / 8, NVK = (NUK + NST - 1) / NST;   // 8-element units of K or Q
    constexpr int NUT = C * C / 4, NVT = (NUT + NST - 1) / NST;

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    __bf16 *Kb = reinterpret_cast<__bf16 *>(smem + L::oK);
    __bf16 *Qb = reinterpret_cast<__bf16 *>(smem + L::oQ);
    __bf16 *Th = reinterpret_cast<__bf16 *>(smem + L::oTh);
    __bf16 *Tl = reinterpret_cast<__bf16 *>(smem + L::oTl);
    __bf16 *Ph = reinterpret_cast<__bf16 *>(smem + L::oPh);
    __bf16 *Pl = reinterpret_cast<__bf16 *>(smem + L::oPl);
    __bf16 *STh = reinterpret_cast<__bf16 *>(smem + L::oSTh);
    __bf16 *STl = reinterpret_cast<__bf16 *>(smem + L::oSTl);
    __bf16 *Xh = reinterpret_cast<__bf16 *>(smem + L::oXh);
    __bf16 *Xl = reinterpret_cast<__bf16 *>(smem + L::oXl);
    __bf16 *Yh = reinterpret_cast<__bf16 *>(smem + L::oYh);
    __bf16 *Yl = reinterpret_cast<__bf16 *>(smem + L::oYl);
    __bf16 *Uh = reinterpret_cast<__bf16 *>(smem + L::oUh);
    __bf16 *Ul = reinterpret_cast<__bf16 *>(smem + L::oUl);
    __bf16 *Bhb = reinterpret_cast<__bf16 *>(smem + L::oBh);
    __bf16 *Blb = reinterpret_cast<__bf16 *>(smem + L::oBl);
    float *Ins = reinterpret_cast<float *>(smem + L::oIn);
    float *Gb = reinterpret_cast<float *>(smem + L::oG);
    float *Bb = reinterpret_cast<float *>(smem + L::oB);

    const int lane = lane_id(), wave = wave_id(), ln = lane & 15, lg = lane >> 4;
    const bool chain = wave < 4;
    const int ts = threadIdx.x - 256;                          // staging thread index
    const int64_t NS = p.Dv / BV;
    int64_t bh, sl;
    slice_of(blockIdx.x, NS, p.xcd_map, bh, sl);
    const int64_t H = p.H, T = p.T, Dv = p.Dv, NC = p.NC, b = bh / H, h = bh % H;
    const int n0 = (int)sl * BV;
    const __bf16 *kg = static_cast<const __bf16 *>(p.k);
    const __bf16 *qg = static_cast<const __bf16 *>(p.q);
    const __bf16 *vg = static_cast<const __bf16 *>(p.v);

    // ---- staging registers: set A (P, dY or V) and set B (K, Q, T, G2, beta).
    // Every load is issued unconditionally (clamped row and unit indices, the
    // zeros past T applied when the data is written), so the compiler can wait
    // on exact outstanding-load counts instead of draining the prefetch.
    f32x4 rP[NVT], rT[NVT];
    bf16x8 rK[NVK], rQ[NVK];
    f32x4 rY = zero4();                      // dY piece (adjoint)
    bf16x4 rV = Raw4<__bf16>::zero();        // V piece (state pass)
    float rG = 0.f, rBe = 0.f, rGa = 0.f;    // rGa: G2 of this thread's set-A token (e^G o dY)
    int64_t cA = 0, cB = 0;                  // chunk held by set A, set B
    const int ua = ts < C * 4 ? ts : C * 4 - 1;    // clamped set-A unit (row ua/4, columns 4(ua%4)..)
    const int ug = ts < C ? ts : C - 1;            // clamped token of G2 / beta
    auto load_a = [&](int64_t c) {
        cA = c;
        const int64_t c0 = c * C;
        const float *rec = p.rec + (bh * NC + c) * p.rec_floats;
        if constexpr (ADJ) {
#pragma unroll
            for (int i = 0; i < NVT; ++i) {
                int u = ts + NST * i;
                u = (NUT % NST == 0 || u < NUT) ? u : NUT - 1;
                const int r = u / (C / 4), col = (u % (C / 4)) * 4;
                rP[i] = *reinterpret_cast<const f32x4 *>(rec + Rec<C>::oP + r * C + col);
            }
        }
        const int r = ua >> 2, col = (ua & 3) * 4;
        const int64_t t = c0 + r < T ? c0 + r : T - 1;
        if constexpr (ADJ) {
            rY = *reinterpret_cast<const f32x4 *>(p.dy + ((b * T + t) * H + h) * Dv + n0 + col);
            rGa = rec[Rec<C>::oG + r];
        } else {
            rV = *reinterpret_cast<const bf16x4 *>(vg + ((b * T + t) * H + h) * Dv + n0 + col);
        }
    };
    auto load_b = [&](int64_t c) {
        cB = c;
        const int64_t c0 = c * C;
        const float *rec = p.rec + (bh * NC + c) * p.rec_floats;
#pragma unroll
        for (int i = 0; i < NVK; ++i) {
            int u = ts + NST * i;
            u = (NUK % NST == 0 || u < NUK) ? u : NUK - 1;
            const int r = u / (DK / 8), col = (u % (DK / 8)) * 8;
            const int64_t t = c0 + r < T ? c0 + r : T - 1;
            rK[i] = *reinterpret_cast<const bf16x8 *>(kg + ((b * T + t) * H + h) * DK + col);
            if constexpr (ADJ) rQ[i] = *reinterpret_cast<const bf16x8 *>(qg + ((b * T + t) * H + h) * DK + col);
        }
#pragma unroll
        for (int i = 0; i < NVT; ++i) {
            int u = ts + NST * i;
            u = (NUT % NST == 0 || u < NUT) ? u : NUT - 1;
            const int r = u / (C / 4), col = (u % (C / 4)) * 4;
            rT[i] = *reinterpret_cast<const f32x4 *>(rec + Rec<C>::oT + r * C + col);
        }
        const int64_t tg = c0 + ug < T ? c0 + ug : T - 1;
        rG = rec[Rec<C>::oG + ug];
        rBe = p.beta[(b * T + tg) * H + h];
    };
    // set A into LDS: P hi/lo; dY^T hi/lo and (e^G o dY)^T into buffer nb, or V
    auto write_a = [&](int nb) {
        if constexpr (ADJ) {
#pragma unroll
            for (int i = 0; i < NVT; ++i) {
                const int u = ts + NST * i;
                const int r = u / (C / 4), col = (u % (C / 4)) * 4;
                if (NUT % NST == 0 || u < NUT) store_split4(Ph + r * CP + col, Pl + r * CP + col, rP[i]);
            }
        }
        if (C * 4 >= NST || ts < C * 4) {
            const int r = ts >> 2, col = (ts & 3) * 4;
            const bool ok = cA * C + r < T;
            if constexpr (ADJ) {
                // e^G of this token (loaded with set A)
                const float eg = __builtin_amdgcn_exp2f(rGa);
                const f32x4 y = ok ? rY : zero4();
                bf16x4 hh, ll, bh2, bl2;
                split4(y, hh, ll);
                split4(y * eg, bh2, bl2);
                __bf16 *Bh = Bhb + nb * BV * CP, *Bl = Blb + nb * BV * CP;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    Yh[(col + q) * CP + r] = hh[q];
                    Yl[(col + q) * CP + r] = ll[q];
                    Bh[(col + q) * CP + r] = bh2[q];
                    Bl[(col + q) * CP + r] = bl2[q];
                }
            } else {
                *reinterpret_cast<f32x4 *>(Ins + r * VP + col) = ok ? Raw4<__bf16>::widen(rV) : zero4();
            }
        }
    };
    auto write_b = [&](int nb) {
        __bf16 *Kd = Kb + nb * C * KP, *Qd = Qb + nb * C * KP;
#pragma unroll
        for (int i = 0; i < NVK; ++i) {
            const int u = ts + NST * i;
            const int r = u / (DK / 8), col = (u % (DK / 8)) * 8;
            if (NUK % NST == 0 || u < NUK) {
                const bool ok = cB * C + r < T;
                *reinterpret_cast<bf16x8 *>(Kd + r * KP + col) = ok ? rK[i] : bf16x8{};
                if constexpr (ADJ) *reinterpret_cast<bf16x8 *>(Qd + r * KP + col) = ok ? rQ[i] : bf16x8{};
            }
        }
#pragma unroll
        for (int i = 0; i < NVT; ++i) {
            const int u = ts + NST * i;
            const int r = u / (C / 4), col = (u % (C / 4)) * 4;
            if (NUT % NST == 0 || u < NUT) store_split4(Th + r * CP + col, Tl + r * CP + col, rT[i]);
        }
        if (C >= NST || ts < C) {
            Gb[nb * C + ts] = rG;
            Bb[nb * C + ts] = cB * C + ts < T ? rBe : 0.f;
        }
    };

    const int64_t cfirst = ADJ ? NC - 1 : 0;
    const int64_t cstep = ADJ ? -1 : 1;

    // ---- state slice in the chain waves' accumulators
    f32x4 S[MS];
    const float *init = ADJ ? p.dsT : p.s0;
#pragma unroll
    for (int m = 0; m < MS; ++m) {
        S[m] = zero4();
        const int ib = wave + 4 * m;
        if (chain && ib < NKB && init) {
#pragma unroll
            for (int e = 0; e < 4; ++e) S[m][e] = init[(bh * DK + 16 * ib + 4 * lg + e) * Dv + n0 + ln];
        }
    }
    // keep the state at the boundary of chunk c; stage it transposed (hi/lo)
    auto keep_state = [&](int64_t c) {
        float *keep = (ADJ ? p.dsc : p.sc) + (bh * NC + c) * DK * Dv;
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int ib = wave + 4 * m;
            if (ib < NKB) {
                const int row = 16 * ib + 4 * lg;
#pragma unroll
                for (int e = 0; e < 4; ++e) keep[(row + e) * Dv + n0 + ln] = S[m][e];
                store_split4(STh + ln * KP + row, STl + ln * KP + row, S[m]);
            }
        }
    };

    // The two roles run separate loops with the same barrier sequence (one
    // barrier after the prologue, three per chunk), so the chain waves' code
    // holds no global load and never waits on its own stores.
    if (!chain) {
        // ---- staging waves
        // the first chunk (G2 of set B is needed by write_a), then prefetch the
        // second; past the last chunk the last one is fetched again (never read)
        auto clampc = [&](int64_t c) { return c < 0 ? 0 : c >= NC ? NC - 1 : c; };
        load_b(cfirst);
        load_a(cfirst);
        write_b(0);
        write_a(0);
        // same issue order as in the loop (set A, then set B), so the waits in
        // the loop count the same younger loads on both entries
        load_a(clampc(cfirst + cstep));
        __builtin_amdgcn_sched_barrier(0);   // keep the set-A loads ahead of set B
        load_b(clampc(cfirst + cstep));
        lds_barrier();
        for (int64_t it = 0; it < NC; ++it) {
            const int64_t c = cfirst + cstep * it;
            const int nbuf = (int)(it & 1) ^ 1;
            lds_barrier();                  // A..B: step 1 runs
            // set A of the next chunk (single-buffered parts: last read in step 1)
            write_a(nbuf);
            load_a(clampc(c + 2 * cstep));
            lds_barrier();                  // B..C: step 2 runs
            // set B of the next chunk (T: last read in step 2)
            write_b(nbuf);
            load_b(clampc(c + 2 * cstep));
            lds_barrier();                  // C..A: step 3 runs
        }
    } else {
        // ---- chain waves
        keep_state(cfirst);
        lds_barrier();
        for (int64_t it = 0; it < NC; ++it) {
            const int64_t c = cfirst + cstep * it;
            const int buf = (int)(it & 1);
            const bool more = it + 1 < NC;
            const __bf16 *Ks = Kb + buf * C * KP, *Qs = Qb + buf * C * KP;
            const __bf16 *Bh = Bhb + buf * BV * CP, *Bl = Blb + buf * BV * CP;
            const float *Gs = Gb + buf * C, *Bs = Bb + buf * C;
            const float GC = Gs[C - 1];

            // ---- A..B: step 1
            if (wave < NB) {
                const int rb = wave;
                f32x4 ks = zero4(), ks2 = zero4();
                if constexpr (DK % 32 == 0) {
#pragma unroll
                    for (int k0 = 0; k0 < DK; k0 += 32) {
                        const F32 a = frag_rows<__bf16, 32>(Ks, KP, 16 * rb, k0, lane);
                        ks = F32::mma(a, frag_rows<__bf16, 32>(STh, KP, 0, k0, lane), ks);
                        ks2 = F32::mma(a, frag_rows<__bf16, 32>(STl, KP, 0, k0, lane), ks2);
                    }
                } else {
                    const F16 a = frag_rows<__bf16, 16>(Ks, KP, 16 * rb, 0, lane);
                    ks = F16::mma(a, frag_rows<__bf16, 16>(STh, KP, 0, 0, lane), ks);
                    ks2 = F16::mma(a, frag_rows<__bf16, 16>(STl, KP, 0, 0, lane), ks2);
                }
                ks += ks2;
                const int r0 = 16 * rb + 4 * lg;
                if constexpr (ADJ) {
                    f32x4 acc, acc2 = zero4();
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = __builtin_amdgcn_exp2f(GC - Gs[r0 + e]) * ks[e];
                    for (int kb = rb; kb < NB; ++kb) {
                        const F16 ah = tr_frag16(Ph, CP, 16 * rb, 16 * kb, lane);
                        const F16 al = tr_frag16(Pl, CP, 16 * rb, 16 * kb, lane);
                        const F16 yh = frag_rows<__bf16, 16>(Yh, CP, 0, 16 * kb, lane);
                        const F16 yl = frag_rows<__bf16, 16>(Yl, CP, 0, 16 * kb, lane);
                        acc = F16::mma(ah, yh, acc);
                        acc2 = F16::mma(ah, yl, acc2);
                        acc2 = F16::mma(al, yh, acc2);
                    }
                    acc += acc2;
                    store_split4(Xh + ln * CP + r0, Xl + ln * CP + r0, acc);
                } else {
                    float *wg = p.wb + (bh * NC + c) * C * Dv + n0 + ln;
                    f32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float wt = Ins[(r0 + e) * VP + ln] - __builtin_amdgcn_exp2f(Gs[r0 + e]) * ks[e];
                        x[e] = Bs[r0 + e] * wt;
                        wg[(r0 + e) * Dv] = wt;
                    }
                    store_split4(Xh + ln * CP + r0, Xl + ln * CP + r0, x);
                }
            }
            lds_barrier();

            // ---- B..C: step 2
            if (wave < NB) {
                const int rb = wave;
                const int r0 = 16 * rb + 4 * lg;
                f32x4 acc = zero4(), acc2 = zero4();
                if constexpr (ADJ) {
                    for (int kb = rb; kb < NB; ++kb) {
                        const F16 ah = tr_frag16(Th, CP, 16 * rb, 16 * kb, lane);
                        const F16 al = tr_frag16(Tl, CP, 16 * rb, 16 * kb, lane);
                        const F16 xh = frag_rows<__bf16, 16>(Xh, CP, 0, 16 * kb, lane);
                        const F16 xl = frag_rows<__bf16, 16>(Xl, CP, 0, 16 * kb, lane);
                        acc = F16::mma(ah, xh, acc);
                        acc2 = F16::mma(ah, xl, acc2);
                        acc2 = F16::mma(al, xh, acc2);
                    }
                    acc += acc2;
                    float *xg = p.dxb + (bh * NC + c) * C * Dv + n0 + ln;
                    f32x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = r0 + e;
                        const int64_t t = c * C + r;
                        o[e] = -__builtin_amdgcn_exp2f(Gs[r]) * Bs[r] * acc[e];
                        xg[r * Dv] = acc[e];
                        if (t < T) p.dv[((b * T + t) * H + h) * Dv + n0 + ln] = Bs[r] * acc[e];
                    }
                    store_split4(Uh + ln * CP + r0, Ul + ln * CP + r0, o);
                } else {
                    for (int kb = 0; kb <= rb; ++kb) {
                        const F16 ah = frag_rows<__bf16, 16>(Th, CP, 16 * rb, 16 * kb, lane);
                        const F16 al = frag_rows<__bf16, 16>(Tl, CP, 16 * rb, 16 * kb, lane);
                        const F16 xh = frag_rows<__bf16, 16>(Xh, CP, 0, 16 * kb, lane);
                        const F16 xl = frag_rows<__bf16, 16>(Xl, CP, 0, 16 * kb, lane);
                        acc = F16::mma(ah, xh, acc);
                        acc2 = F16::mma(ah, xl, acc2);
                        acc2 = F16::mma(al, xh, acc2);
                    }
                    acc += acc2;
                    float *ug = p.ub + (bh * NC + c) * C * Dv + n0 + ln;
                    f32x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = r0 + e;
                        o[e] = __builtin_amdgcn_exp2f(GC - Gs[r]) * acc[e];
                        ug[r * Dv] = acc[e];
                    }
                    store_split4(Uh + ln * CP + r0, Ul + ln * CP + r0, o);
                }
            }
            lds_barrier();

            // ---- C..A: step 3
            const float eGC = __builtin_amdgcn_exp2f(GC);
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int ib = wave + 4 * m;
                if (ib < NKB) {
                    f32x4 acc = S[m] * eGC, acc2 = zero4();
                    if constexpr (C % 32 == 0) {
#pragma unroll
                        for (int j0 = 0; j0 < C; j0 += 32) {
                            const F32 ka = tr_frag32(Ks, KP, 16 * ib, j0, lane);
                            acc = F32::mma(ka, pair_rows32(Uh, CP, 0, j0, lane), acc);
                            acc2 = F32::mma(ka, pair_rows32(Ul, CP, 0, j0, lane), acc2);
                            if constexpr (ADJ) {
                                const F32 qa = tr_frag32(Qs, KP, 16 * ib, j0, lane);
                                acc = F32::mma(qa, pair_rows32(Bh, CP, 0, j0, lane), acc);
                                acc2 = F32::mma(qa, pair_rows32(Bl, CP, 0, j0, lane), acc2);
                            }
                        }
                    } else {
                        const F16 ka = tr_frag16(Ks, KP, 16 * ib, 0, lane);
                        acc = F16::mma(ka, frag_rows<__bf16, 16>(Uh, CP, 0, 0, lane), acc);
                        acc2 = F16::mma(ka, frag_rows<__bf16, 16>(Ul, CP, 0, 0, lane), acc2);
                        if constexpr (ADJ) {
                            const F16 qa = tr_frag16(Qs, KP, 16 * ib, 0, lane);
                            acc = F16::mma(qa, frag_rows<__bf16, 16>(Bh, CP, 0, 0, lane), acc);
                            acc2 = F16::mma(qa, frag_rows<__bf16, 16>(Bl, CP, 0, 0, lane), acc2);
                        }
                    }
                    S[m] = acc + acc2;
                }
            }
            if (more) keep_state(c + cstep);
            lds_barrier();
        }
    }

    if constexpr (ADJ) {
        if (chain && p.ds0) {
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
//
// U, W~ (state pass) and dX (adjoint pass) of the chunk are read back, so
// every value slice only adds outer products into accumulators:
//   dP += dY U^T, dM += dX U^T (lower blocks),
//   dQa += dY S^T, dKa += dX S^T, dKb += U dS'^T.
// The per-token terms of dG that involve K S, Q S and K dS' are row dot
// products with these sums: sum_j dY_rj (QS)_rj = q_r . dQa_r,
// sum_j dX_rj (KS)_rj = k_r . dKa_r, sum_j U_rj (K dS')_rj = k_r . dKb_r.
// ===========================================================================
template <int C, int DK> struct GradLay {
    static constexpr int KP = DK + 4, CP = C + 4, NB = C / 16, NKB = DK / 16;
    static constexpr size_t oK = 0;
    static constexpr size_t oQ = oK + 4 * C * KP;
    static constexpr size_t oT = oQ + 4 * C * KP;          // dKK
    static constexpr size_t oP = oT + 4 * C * CP;          // P, then dQK
    // S slice [DK][VP] and dS' slice [DK][VP]; Ak [C][CP] over both after the slices
    static constexpr size_t SREG = 2 * DK * VP > C * CP ? 2 * DK * VP : C * CP;
    static constexpr size_t oS = oP + 4 * C * CP;
    static constexpr size_t oDS = oS + 4 * DK * VP;
    static constexpr size_t oDY = oS + 4 * SREG;
    static constexpr size_t oU = oDY + 4 * C * VP;
    static constexpr size_t oDX = oU + 4 * C * VP;
    static constexpr size_t oG = oDX + 4 * C * VP;
    static constexpr size_t oB = oG + 4 * C;
    static constexpr size_t oAl = oB + 4 * C;
    static constexpr size_t oTB = oAl + 4 * C;                 // per-token sum_j dX_rj W~_rj
    static constexpr size_t oSP = oTB + 4 * C;                 // [3][NB*NKB][16] row dot products per tile
    static constexpr size_t oRP = oSP + 4 * 3 * NB * NKB * 16; // [2][NB][NB][16] row sums (P part, A part)
    static constexpr size_t oCP = oRP + 4 * 2 * NB * NB * 16;  // [2][NB][NB][16] column sums
    static constexpr size_t oRB = oCP + 4 * 2 * NB * NB * 16;  // [NB][NB][16] dbeta row sums
    static constexpr size_t oRed = oRB + 4 * NB * NB * 16;
    static constexpr size_t BYTES = oRed + 4 * 16;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

constexpr int NWG = 8, NTG = 64 * NWG;   // chunk-gradient kernel: 8 wavefronts, two per SIMD

template <typename Tin, int C, int DK>
__global__ __launch_bounds__(NTG) void bwd_chunk_kernel(BwdParams p)
{
    using L = GradLay<C, DK>;
    constexpr int KP = L::KP, CP = L::CP, NB = C / 16, NKB = DK / 16;
    constexpr int NTRI = NB * (NB + 1) / 2;
    constexpr int NCC = (2 * NTRI + NWG - 1) / NWG;              // C x C tiles per wave (dP, dM)
    constexpr int NTILE = NB * NKB, NCK = (NTILE + NWG - 1) / NWG; // C x DK tiles per wave
    using F16 = Frag<float, 16>;

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    float *Ks = reinterpret_cast<float *>(smem + L::oK);
    float *Qs = reinterpret_cast<float *>(smem + L::oQ);
    float *Ts = reinterpret_cast<float *>(smem + L::oT);
    float *Ps = reinterpret_cast<float *>(smem + L::oP);
    float *Ss = reinterpret_cast<float *>(smem + L::oS);
    float *dSs = reinterpret_cast<float *>(smem + L::oDS);
    float *dYs = reinterpret_cast<float *>(smem + L::oDY);
    float *Us = reinterpret_cast<float *>(smem + L::oU);
    float *dXs = reinterpret_cast<float *>(smem + L::oDX);
    float *Gs = reinterpret_cast<float *>(smem + L::oG);
    float *Bs = reinterpret_cast<float *>(smem + L::oB);
    float *Als = reinterpret_cast<float *>(smem + L::oAl);
    float *tokB = reinterpret_cast<float *>(smem + L::oTB);
    float *sp = reinterpret_cast<float *>(smem + L::oSP);
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
    const float *Ug = p.ub + (bh * p.NC + c) * C * Dv;
    const float *Wg = p.wb + (bh * p.NC + c) * C * Dv;
    const float *Xg = p.dxb + (bh * p.NC + c) * C * Dv;

    {
        RowsTile<Tin, C, DK, NTG> tk, tq;
        DenseTile<C, C, NTG> tp;
        tk.load(static_cast<const Tin *>(p.k), b, h, c0, T, H * DK, DK);
        tq.load(static_cast<const Tin *>(p.q), b, h, c0, T, H * DK, DK);
        tp.load(rec + Rec<C>::oP, C);
        tk.template store<KP>(Ks);
        tq.template store<KP>(Qs);
        tp.template store<CP>(Ps);
    }
    for (int i = tid; i < C; i += NTG) {
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
    float pW = 0.f, pSS = 0.f;   // sum dX o W~ over this thread's row piece; <S, dS'> piece

    // registers holding the next value slice
    DenseTile<DK, BV, NTG> rs, rds;
    DenseTile<C, BV, NTG> ru, rx, rw;
    RowsTile<float, C, BV, NTG> rdy;
    static_assert(DenseTile<C, BV, NTG>::NV == 1, "one C x 16 slice unit per thread");
    auto fetch_slice = [&](int n0) {
        rs.load(Sg + n0, Dv);
        rds.load(dSg + n0, Dv);
        ru.load(Ug + n0, Dv);
        rx.load(Xg + n0, Dv);
        rw.load(Wg + n0, Dv);
        rdy.load(p.dy, b, h, c0, T, H * Dv, Dv, n0);
    };
    fetch_slice(0);

    for (int n0 = 0; n0 < Dv; n0 += BV) {
        rs.template store<VP>(Ss);
        rds.template store<VP>(dSs);
        ru.template store<VP>(Us);
        rx.template store<VP>(dXs);
        rdy.template store<VP>(dYs);
#pragma unroll
        for (int it = 0; it < DenseTile<DK, BV, NTG>::NV; ++it) {
            const f32x4 a = rs.v[it], d = rds.v[it];
            pSS += a[0] * d[0] + a[1] * d[1] + a[2] * d[2] + a[3] * d[3];
        }
        {
            const f32x4 a = rx.v[0], w = rw.v[0];
            pW += a[0] * w[0] + a[1] * w[1] + a[2] * w[2] + a[3] * w[3];
        }
        if (n0 + BV < Dv) fetch_slice(n0 + BV);
        lds_barrier();

#pragma unroll
        for (int m = 0; m < NCC; ++m) {
            const int tile = wave + NWG * m;
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
            const int tile = wave + NWG * m;
            if (tile < NTILE) {
                const int rb = tile / NKB, kb = tile % NKB;
                const F16 sf = frag_rows<float, 16>(Ss, VP, 16 * kb, 0, lane);
                const F16 df = frag_rows<float, 16>(dSs, VP, 16 * kb, 0, lane);
                dQa[m] = F16::mma(frag_rows<float, 16>(dYs, VP, 16 * rb, 0, lane), sf, dQa[m]);
                dKa[m] = F16::mma(frag_rows<float, 16>(dXs, VP, 16 * rb, 0, lane), sf, dKa[m]);
                dKb[m] = F16::mma(frag_rows<float, 16>(Us, VP, 16 * rb, 0, lane), df, dKb[m]);
            }
        }
        lds_barrier();
    }

    // ---- E: per-token partials to LDS; Ak into the freed slice buffers
    {
        // the 4 consecutive threads of a staged row piece hold one row's 16 columns
        float w = pW;
        w += __shfl_xor(w, 1);
        w += __shfl_xor(w, 2);
        if ((tid & 3) == 0 && tid / 4 < C) tokB[tid / 4] = w;
        float y = pSS;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) y += __shfl_xor(y, off);
        if (lane == 0) red[wave] = y;
    }
    // row dot products q . dQa, k . dKa, k . dKb of every C x DK tile
#pragma unroll
    for (int m = 0; m < NCK; ++m) {
        const int tile = wave + NWG * m;
        if (tile < NTILE) {
            const int rb = tile / NKB, kb = tile % NKB;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * lg + e, col = 16 * kb + ln;
                const float qv = Qs[r * KP + col], kv = Ks[r * KP + col];
                const float a1 = row16_total(qv * dQa[m][e]);
                const float a2 = row16_total(kv * dKa[m][e]);
                const float a3 = row16_total(kv * dKb[m][e]);
                if (ln == 15) {
                    sp[(0 * NTILE + tile) * 16 + 4 * lg + e] = a1;
                    sp[(1 * NTILE + tile) * 16 + 4 * lg + e] = a2;
                    sp[(2 * NTILE + tile) * 16 + 4 * lg + e] = a3;
                }
            }
        }
    }
    {
        DenseTile<C, C, NTG> ta;
        ta.load(rec + Rec<C>::oA, C);
        ta.template store<CP>(Aks);
    }
    lds_barrier();

    // dP tiles -> dQK = Gamma o dP (into Ps); dM tiles -> dA = -dM, dKK =
    // Gamma o diag(beta) dA (into Ts).  E = dP o P + diag(beta) dA o Ak feeds
    // dG_r (+ row sums) and dG_j (- column sums); dA o Ak feeds dbeta.
    // Every (part, block) has exactly one writer, so the sums are deterministic.
#pragma unroll
    for (int m = 0; m < NCC; ++m) {
        const int tile = wave + NWG * m;
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
                const float rs = row16_total(E);
                const float rsb = row16_total(rbeta);
                if (ln == 15) {
                    rowE[((part * NB + rb) * NB + jb) * 16 + 4 * lg + e] = rs;
                    if (part) rowB[(rb * NB + jb) * 16 + 4 * lg + e] = rsb;
                }
            }
            cs += __shfl_xor(cs, 16);
            cs += __shfl_xor(cs, 32);
            if (lg == 0) colE[((part * NB + rb) * NB + jb) * 16 + ln] = cs;
        }
    }
    lds_barrier();

    // ---- F: dQ = e^G o dQa + dQK K;
    //         dK = -e^G beta o dKa + d o dKb + dKK K + dKK^T K + dQK^T Q
#pragma unroll
    for (int m = 0; m < NCK; ++m) {
        const int tile = wave + NWG * m;
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
        const float GC = Gs[C - 1];
        float g = 0.f, d3 = 0.f;
        if (lane < C) {
            const int rb = rr / 16, ri = rr % 16;
            float s1 = 0.f, s2 = 0.f, s3 = 0.f;
            for (int kb = 0; kb < NKB; ++kb) {
                const int tile = rb * NKB + kb;
                s1 += sp[(0 * NTILE + tile) * 16 + ri];
                s2 += sp[(1 * NTILE + tile) * 16 + ri];
                s3 += sp[(2 * NTILE + tile) * 16 + ri];
            }
            const float br = __builtin_amdgcn_exp2f(Gs[rr]), dr = __builtin_amdgcn_exp2f(GC - Gs[rr]);
            d3 = dr * s3;
            g = br * s1 - br * Bs[rr] * s2 - d3;
            for (int jb = 0; jb <= rb; ++jb)
                g += rowE[(rb * NB + jb) * 16 + ri] + rowE[((NB + rb) * NB + jb) * 16 + ri];
            for (int ib = rb; ib < NB; ++ib)
                g -= colE[(ib * NB + rb) * 16 + ri] + colE[((NB + ib) * NB + rb) * 16 + ri];
        }
        // e^{G_C} and the d_r factors all depend on G_C: their terms go to the last token
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) d3 += __shfl_xor(d3, off);
        {
            float ss = 0.f;
#pragma unroll
            for (int w = 0; w < NWG; ++w) ss += red[w];
            if (lane == 0) g += d3 + __builtin_amdgcn_exp2f(GC) * ss;
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

// ===========================================================================
// 4'. chunk gradients, bf16 inputs: bf16 MFMA with hi/lo operands
//
// The steps of bwd_chunk_kernel with 32 value columns per pass: S, dS', U, dX
// and dY enter as bf16 pairs (three 16x16x32 products per fp32 product); the
// final products take K and Q exactly and dQK, dKK as pairs, with K^T, Q^T and
// dKK^T, dQK^T from transposing reads.
// ===========================================================================
template <int C, int DK> struct Grad16Lay {
    static constexpr int KP = DK + 8, CP = C + 4, HP = C + 8;   // K/Q bf16, P fp32, dQK/dKK bf16
    static constexpr int SW = 32, SP = SW + 16;                  // value columns per pass, bf16 pitch
    static constexpr int NB = C / 16, NKB = DK / 16;
    static constexpr size_t oK = 0;
    static constexpr size_t oQ = oK + 2 * C * KP;
    static constexpr size_t oP = oQ + 2 * C * KP;             // P (fp32)
    // value-slice operands (hi, lo); after the passes: Ak (fp32) and dQK, dKK (hi, lo)
    static constexpr size_t SLICE = 2 * 2 * (2 * DK * SP + 3 * C * SP);
    static constexpr size_t AFTER = 4 * C * CP + 4 * 2 * C * HP;
    static constexpr size_t oR = oP + 4 * C * CP;
    static constexpr size_t oSh = oR, oSl = oSh + 2 * DK * SP, oDSh = oSl + 2 * DK * SP, oDSl = oDSh + 2 * DK * SP;
    static constexpr size_t oUh = oDSl + 2 * DK * SP, oUl = oUh + 2 * C * SP;
    static constexpr size_t oXh = oUl + 2 * C * SP, oXl = oXh + 2 * C * SP;
    static constexpr size_t oYh = oXl + 2 * C * SP, oYl = oYh + 2 * C * SP;
    static constexpr size_t oAk = oR;
    static constexpr size_t oQKh = oAk + 4 * C * CP, oQKl = oQKh + 2 * C * HP;
    static constexpr size_t oKKh = oQKl + 2 * C * HP, oKKl = oKKh + 2 * C * HP;
    static constexpr size_t oG = oR + (SLICE > AFTER ? SLICE : AFTER);
    static constexpr size_t oB = oG + 4 * C;
    static constexpr size_t oAl = oB + 4 * C;
    static constexpr size_t oTB = oAl + 4 * C;
    static constexpr size_t oSP = oTB + 4 * C;
    static constexpr size_t oRP = oSP + 4 * 3 * NB * NKB * 16;
    static constexpr size_t oCP = oRP + 4 * 2 * NB * NB * 16;
    static constexpr size_t oRB = oCP + 4 * 2 * NB * NB * 16;
    static constexpr size_t oRed = oRB + 4 * NB * NB * 16;
    static constexpr size_t BYTES = oRed + 4 * 16;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int C, int DK>
__global__ __launch_bounds__(NTG) void bwd_chunk16_kernel(BwdParams p)
{
    using L = Grad16Lay<C, DK>;
    constexpr int KP = L::KP, CP = L::CP, HP = L::HP, SW = L::SW, SP = L::SP, NB = C / 16, NKB = DK / 16;
    constexpr int NTRI = NB * (NB + 1) / 2;
    constexpr int NCC = (2 * NTRI + NWG - 1) / NWG;
    constexpr int NTILE = NB * NKB, NCK = (NTILE + NWG - 1) / NWG;
    using F16 = Frag<__bf16, 16>;
    using F32 = Frag<__bf16, 32>;

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    __bf16 *Ks = reinterpret_cast<__bf16 *>(smem + L::oK);
    __bf16 *Qs = reinterpret_cast<__bf16 *>(smem + L::oQ);
    float *Ps = reinterpret_cast<float *>(smem + L::oP);
    __bf16 *Sh = reinterpret_cast<__bf16 *>(smem + L::oSh), *Sl = reinterpret_cast<__bf16 *>(smem + L::oSl);
    __bf16 *DSh = reinterpret_cast<__bf16 *>(smem + L::oDSh), *DSl = reinterpret_cast<__bf16 *>(smem + L::oDSl);
    __bf16 *Uh = reinterpret_cast<__bf16 *>(smem + L::oUh), *Ul = reinterpret_cast<__bf16 *>(smem + L::oUl);
    __bf16 *Xh = reinterpret_cast<__bf16 *>(smem + L::oXh), *Xl = reinterpret_cast<__bf16 *>(smem + L::oXl);
    __bf16 *Yh = reinterpret_cast<__bf16 *>(smem + L::oYh), *Yl = reinterpret_cast<__bf16 *>(smem + L::oYl);
    float *Aks = reinterpret_cast<float *>(smem + L::oAk);
    __bf16 *QKh = reinterpret_cast<__bf16 *>(smem + L::oQKh), *QKl = reinterpret_cast<__bf16 *>(smem + L::oQKl);
    __bf16 *KKh = reinterpret_cast<__bf16 *>(smem + L::oKKh), *KKl = reinterpret_cast<__bf16 *>(smem + L::oKKl);
    float *Gs = reinterpret_cast<float *>(smem + L::oG);
    float *Bs = reinterpret_cast<float *>(smem + L::oB);
    float *Als = reinterpret_cast<float *>(smem + L::oAl);
    float *tokB = reinterpret_cast<float *>(smem + L::oTB);
    float *sp = reinterpret_cast<float *>(smem + L::oSP);
    float *rowE = reinterpret_cast<float *>(smem + L::oRP);
    float *colE = reinterpret_cast<float *>(smem + L::oCP);
    float *rowB = reinterpret_cast<float *>(smem + L::oRB);
    float *red = reinterpret_cast<float *>(smem + L::oRed);

    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id(), ln = lane & 15, lg = lane >> 4;
    const int64_t bh = blockIdx.x / p.NC, c = blockIdx.x % p.NC;
    const int64_t H = p.H, T = p.T, Dv = p.Dv, b = bh / H, h = bh % H, c0 = c * C;
    const float *rec = p.rec + (bh * p.NC + c) * p.rec_floats;
    const float *Sg = p.sc + (bh * p.NC + c) * DK * Dv;
    const float *dSg = p.dsc + (bh * p.NC + c) * DK * Dv;
    const float *Ug = p.ub + (bh * p.NC + c) * C * Dv;
    const float *Wg = p.wb + (bh * p.NC + c) * C * Dv;
    const float *Xg = p.dxb + (bh * p.NC + c) * C * Dv;

    {
        using R = Raw4<__bf16>;
        RowsTile<__bf16, C, DK, NTG> tk, tq;
        DenseTile<C, C, NTG> tp;
        tk.load(static_cast<const __bf16 *>(p.k), b, h, c0, T, H * DK, DK);
        tq.load(static_cast<const __bf16 *>(p.q), b, h, c0, T, H * DK, DK);
        tp.load(rec + Rec<C>::oP, C);
#pragma unroll
        for (int it = 0; it < RowsTile<__bf16, C, DK, NTG>::NV; ++it) {
            const int vi = tid + NTG * it;
            const int r = vi / (DK / 4), col = (vi % (DK / 4)) * 4;
            if (RowsTile<__bf16, C, DK, NTG>::NU % NTG == 0 || vi < RowsTile<__bf16, C, DK, NTG>::NU) {
                *reinterpret_cast<R::type *>(Ks + r * KP + col) = tk.v[it];
                *reinterpret_cast<R::type *>(Qs + r * KP + col) = tq.v[it];
            }
        }
        tp.template store<CP>(Ps);
    }
    for (int i = tid; i < C; i += NTG) {
        const int64_t t = c0 + i;
        const bool ok = t < T;
        Gs[i] = rec[Rec<C>::oG + i];
        Bs[i] = ok ? p.beta[(b * T + t) * H + h] : 0.f;
        Als[i] = ok ? p.alpha[(b * T + t) * H + h] : 1.f;
    }

    f32x4 dQa[NCK], dKa[NCK], dKb[NCK], dPM[NCC];
#pragma unroll
    for (int m = 0; m < NCK; ++m) dQa[m] = dKa[m] = dKb[m] = zero4();
#pragma unroll
    for (int m = 0; m < NCC; ++m) dPM[m] = zero4();
    float pW = 0.f, pSS = 0.f;   // sum dX o W~ over this thread's row piece; <S, dS'> piece

    DenseTile<DK, SW, NTG> rs, rds;
    DenseTile<C, SW, NTG> ru, rx, rw;
    RowsTile<float, C, SW, NTG> rdy;
    static_assert(DenseTile<C, SW, NTG>::NV == 1, "one C x 32 slice unit per thread");
    auto fetch_slice = [&](int n0) {
        rs.load(Sg + n0, Dv);
        rds.load(dSg + n0, Dv);
        ru.load(Ug + n0, Dv);
        rx.load(Xg + n0, Dv);
        rw.load(Wg + n0, Dv);
        rdy.load(p.dy, b, h, c0, T, H * Dv, Dv, n0);
    };
    fetch_slice(0);

    for (int n0 = 0; n0 < Dv; n0 += SW) {
#pragma unroll
        for (int it = 0; it < DenseTile<DK, SW, NTG>::NV; ++it) {
            const int vi = tid + NTG * it;
            const int r = vi / (SW / 4), col = (vi % (SW / 4)) * 4;
            if (DenseTile<DK, SW, NTG>::NU % NTG == 0 || vi < DenseTile<DK, SW, NTG>::NU) {
                store_split4(Sh + r * SP + col, Sl + r * SP + col, rs.v[it]);
                store_split4(DSh + r * SP + col, DSl + r * SP + col, rds.v[it]);
            }
            const f32x4 a = rs.v[it], d = rds.v[it];
            pSS += a[0] * d[0] + a[1] * d[1] + a[2] * d[2] + a[3] * d[3];
        }
        {
            const int vi = tid;
            const int r = vi / (SW / 4), col = (vi % (SW / 4)) * 4;
            if (DenseTile<C, SW, NTG>::NU % NTG == 0 || vi < DenseTile<C, SW, NTG>::NU) {
                store_split4(Uh + r * SP + col, Ul + r * SP + col, ru.v[0]);
                store_split4(Xh + r * SP + col, Xl + r * SP + col, rx.v[0]);
                store_split4(Yh + r * SP + col, Yl + r * SP + col, rdy.v[0]);
            }
            const f32x4 a = rx.v[0], w = rw.v[0];
            pW += a[0] * w[0] + a[1] * w[1] + a[2] * w[2] + a[3] * w[3];
        }
        if (n0 + SW < Dv) fetch_slice(n0 + SW);
        lds_barrier();

#pragma unroll
        for (int m = 0; m < NCC; ++m) {
            const int tile = wave + NWG * m;
            if (tile < 2 * NTRI) {
                const bool isM = tile >= NTRI;
                int rb, jb;
                tri_block(isM ? tile - NTRI : tile, rb, jb);
                const F32 ah = frag_rows<__bf16, 32>(isM ? Xh : Yh, SP, 16 * rb, 0, lane);
                const F32 al = frag_rows<__bf16, 32>(isM ? Xl : Yl, SP, 16 * rb, 0, lane);
                const F32 bh2 = frag_rows<__bf16, 32>(Uh, SP, 16 * jb, 0, lane);
                const F32 bl2 = frag_rows<__bf16, 32>(Ul, SP, 16 * jb, 0, lane);
                dPM[m] = F32::mma(ah, bh2, dPM[m]);
                dPM[m] = F32::mma(ah, bl2, dPM[m]);
                dPM[m] = F32::mma(al, bh2, dPM[m]);
            }
        }
#pragma unroll
        for (int m = 0; m < NCK; ++m) {
            const int tile = wave + NWG * m;
            if (tile < NTILE) {
                const int rb = tile / NKB, kb = tile % NKB;
                const F32 sh = frag_rows<__bf16, 32>(Sh, SP, 16 * kb, 0, lane);
                const F32 sl = frag_rows<__bf16, 32>(Sl, SP, 16 * kb, 0, lane);
                const F32 dh = frag_rows<__bf16, 32>(DSh, SP, 16 * kb, 0, lane);
                const F32 dl = frag_rows<__bf16, 32>(DSl, SP, 16 * kb, 0, lane);
                const F32 yh = frag_rows<__bf16, 32>(Yh, SP, 16 * rb, 0, lane);
                const F32 yl = frag_rows<__bf16, 32>(Yl, SP, 16 * rb, 0, lane);
                const F32 xh = frag_rows<__bf16, 32>(Xh, SP, 16 * rb, 0, lane);
                const F32 xl = frag_rows<__bf16, 32>(Xl, SP, 16 * rb, 0, lane);
                const F32 uh = frag_rows<__bf16, 32>(Uh, SP, 16 * rb, 0, lane);
                const F32 ul = frag_rows<__bf16, 32>(Ul, SP, 16 * rb, 0, lane);
                dQa[m] = F32::mma(yh, sh, dQa[m]);
                dKa[m] = F32::mma(xh, sh, dKa[m]);
                dKb[m] = F32::mma(uh, dh, dKb[m]);
                dQa[m] = F32::mma(yh, sl, dQa[m]);
                dKa[m] = F32::mma(xh, sl, dKa[m]);
                dKb[m] = F32::mma(uh, dl, dKb[m]);
                dQa[m] = F32::mma(yl, sh, dQa[m]);
                dKa[m] = F32::mma(xl, sh, dKa[m]);
                dKb[m] = F32::mma(ul, dh, dKb[m]);
            }
        }
        lds_barrier();
    }

    // ---- E: per-token partials to LDS; Ak into the freed slice buffers
    {
        float w = pW;
        // the 8 consecutive threads of a staged row piece hold one row's 32 columns
        w += __shfl_xor(w, 1);
        w += __shfl_xor(w, 2);
        w += __shfl_xor(w, 4);
        if ((tid & 7) == 0 && tid / 8 < C) tokB[tid / 8] = w;
        float y = pSS;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) y += __shfl_xor(y, off);
        if (lane == 0) red[wave] = y;
    }
#pragma unroll
    for (int m = 0; m < NCK; ++m) {
        const int tile = wave + NWG * m;
        if (tile < NTILE) {
            const int rb = tile / NKB, kb = tile % NKB;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * lg + e, col = 16 * kb + ln;
                const float qv = (float)Qs[r * KP + col], kv = (float)Ks[r * KP + col];
                const float a1 = row16_total(qv * dQa[m][e]);
                const float a2 = row16_total(kv * dKa[m][e]);
                const float a3 = row16_total(kv * dKb[m][e]);
                if (ln == 15) {
                    sp[(0 * NTILE + tile) * 16 + 4 * lg + e] = a1;
                    sp[(1 * NTILE + tile) * 16 + 4 * lg + e] = a2;
                    sp[(2 * NTILE + tile) * 16 + 4 * lg + e] = a3;
                }
            }
        }
    }
    {
        DenseTile<C, C, NTG> ta;
        ta.load(rec + Rec<C>::oA, C);
        ta.template store<CP>(Aks);
    }
    lds_barrier();

    // dP tiles -> dQK = Gamma o dP; dM tiles -> dA = -dM, dKK = Gamma o diag(beta) dA;
    // both as bf16 pairs for the final products.  Row/column sums as in the fp32 kernel.
#pragma unroll
    for (int m = 0; m < NCC; ++m) {
        const int tile = wave + NWG * m;
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
                float E, rbeta = 0.f, outv;
                if (part) {
                    const float dA = r > j ? -dPM[m][e] : 0.f;
                    const float ak = Aks[r * CP + j];
                    const float dAk = Bs[r] * dA;
                    outv = gam * dAk;
                    E = dAk * ak;
                    rbeta = dA * ak;
                } else {
                    const float dP = r >= j ? dPM[m][e] : 0.f;
                    E = dP * Ps[r * CP + j];
                    outv = gam * dP;
                }
                const __bf16 hi = (__bf16)outv;
                const __bf16 lo = (__bf16)(outv - (float)hi);
                __bf16 *dh = part ? KKh : QKh, *dl = part ? KKl : QKl;
                dh[r * HP + j] = hi;
                dl[r * HP + j] = lo;
                cs += E;
                const float rs = row16_total(E);
                const float rsb = row16_total(rbeta);
                if (ln == 15) {
                    rowE[((part * NB + rb) * NB + jb) * 16 + 4 * lg + e] = rs;
                    if (part) rowB[(rb * NB + jb) * 16 + 4 * lg + e] = rsb;
                }
            }
            cs += __shfl_xor(cs, 16);
            cs += __shfl_xor(cs, 32);
            if (lg == 0) colE[((part * NB + rb) * NB + jb) * 16 + ln] = cs;
        }
    }
    lds_barrier();

    // ---- F: dQ = e^G o dQa + dQK K;
    //         dK = -e^G beta o dKa + d o dKb + dKK K + dKK^T K + dQK^T Q
#pragma unroll
    for (int m = 0; m < NCK; ++m) {
        const int tile = wave + NWG * m;
        if (tile < NTILE) {
            const int rb = tile / NKB, kb = tile % NKB;
            const float GC = Gs[C - 1];
            f32x4 dq, dk, dq2 = zero4(), dk2 = zero4();
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * lg + e;
                const float br = __builtin_amdgcn_exp2f(Gs[r]), dr = __builtin_amdgcn_exp2f(GC - Gs[r]);
                dq[e] = br * dQa[m][e];
                dk[e] = dr * dKb[m][e] - br * Bs[r] * dKa[m][e];
            }
            for (int jb = 0; jb <= rb; ++jb) {
                // K block jb as the B operand: B[k = token][n = dk column]
                const F16 kf = tr_frag16(Ks, KP, 16 * kb, 16 * jb, lane);
                dq = F16::mma(frag_rows<__bf16, 16>(QKh, HP, 16 * rb, 16 * jb, lane), kf, dq);
                dq2 = F16::mma(frag_rows<__bf16, 16>(QKl, HP, 16 * rb, 16 * jb, lane), kf, dq2);
                dk = F16::mma(frag_rows<__bf16, 16>(KKh, HP, 16 * rb, 16 * jb, lane), kf, dk);
                dk2 = F16::mma(frag_rows<__bf16, 16>(KKl, HP, 16 * rb, 16 * jb, lane), kf, dk2);
            }
            for (int ib = rb; ib < NB; ++ib) {
                const F16 kf = tr_frag16(Ks, KP, 16 * kb, 16 * ib, lane);
                const F16 qf = tr_frag16(Qs, KP, 16 * kb, 16 * ib, lane);
                dk = F16::mma(tr_frag16(KKh, HP, 16 * rb, 16 * ib, lane), kf, dk);
                dk2 = F16::mma(tr_frag16(KKl, HP, 16 * rb, 16 * ib, lane), kf, dk2);
                dk = F16::mma(tr_frag16(QKh, HP, 16 * rb, 16 * ib, lane), qf, dk);
                dk2 = F16::mma(tr_frag16(QKl, HP, 16 * rb, 16 * ib, lane), qf, dk2);
            }
            dq += dq2;
            dk += dk2;
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
        const float GC = Gs[C - 1];
        float g = 0.f, d3 = 0.f;
        if (lane < C) {
            const int rb = rr / 16, ri = rr % 16;
            float s1 = 0.f, s2 = 0.f, s3 = 0.f;
            for (int kb = 0; kb < NKB; ++kb) {
                const int tile = rb * NKB + kb;
                s1 += sp[(0 * NTILE + tile) * 16 + ri];
                s2 += sp[(1 * NTILE + tile) * 16 + ri];
                s3 += sp[(2 * NTILE + tile) * 16 + ri];
            }
            const float br = __builtin_amdgcn_exp2f(Gs[rr]), dr = __builtin_amdgcn_exp2f(GC - Gs[rr]);
            d3 = dr * s3;
            g = br * s1 - br * Bs[rr] * s2 - d3;
            for (int jb = 0; jb <= rb; ++jb)
                g += rowE[(rb * NB + jb) * 16 + ri] + rowE[((NB + rb) * NB + jb) * 16 + ri];
            for (int ib = rb; ib < NB; ++ib)
                g -= colE[(ib * NB + rb) * 16 + ri] + colE[((NB + ib) * NB + rb) * 16 + ri];
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) d3 += __shfl_xor(d3, off);
        {
            float ss = 0.f;
#pragma unroll
            for (int w = 0; w < NWG; ++w) ss += red[w];
            if (lane == 0) g += d3 + __builtin_amdgcn_exp2f(GC) * ss;
        }
        const float suf = wave_inclusive_sum(g, lane);
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

// ===========================================================================
// Forward prefill for fp32 inputs in two kernels: bwd_prep_kernel<float> (T, P
// and the decay prefix of every chunk, once per chunk) and fwd32_carry_kernel,
// the state recurrence over 16-column slices that also writes y:
//   X = diag(beta)(V - diag(e^G) K S),  U = T X,
//   Y = diag(e^G) Q S + P U,  S' = e^{G_C} S + K^T diag(d) U.
// q, k, v may be slices of a wider buffer (token strides).
// ===========================================================================
template <int C, int DK> struct Fwd32Lay {
    static constexpr int KP = DK + 4, CP = C + 4;
    static constexpr size_t oK = 0;
    static constexpr size_t oQ = oK + 4 * C * KP;
    static constexpr size_t oT = oQ + 4 * C * KP;
    static constexpr size_t oP = oT + 4 * C * CP;
    static constexpr size_t oST = oP + 4 * C * CP;
    static constexpr size_t oIn = oST + 4 * BV * KP;
    static constexpr size_t oX = oIn + 4 * C * VP;
    static constexpr size_t oU = oX + 4 * C * VP;
    static constexpr size_t oUd = oU + 4 * C * VP;
    static constexpr size_t oG = oUd + 4 * BV * CP;
    static constexpr size_t oB = oG + 4 * C;
    static constexpr size_t oEd = oB + 4 * C;
    static constexpr size_t BYTES = oEd + 4 * C;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

template <int C, int DK>
__global__ __launch_bounds__(NT) void fwd32_carry_kernel(BwdParams p)
{
    using L = Fwd32Lay<C, DK>;
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
    float *Us = reinterpret_cast<float *>(smem + L::oU);
    float *UdT = reinterpret_cast<float *>(smem + L::oUd);
    float *Gs = reinterpret_cast<float *>(smem + L::oG);
    float *Bs = reinterpret_cast<float *>(smem + L::oB);
    float *Eds = reinterpret_cast<float *>(smem + L::oEd);

    const int lane = lane_id(), wave = wave_id(), ln = lane & 15, lg = lane >> 4;
    const int64_t NS = p.Dv / BV;
    int64_t bh, sl;
    slice_of(blockIdx.x, NS, p.xcd_map, bh, sl);
    const int64_t H = p.H, T = p.T, Dv = p.Dv, NC = p.NC, b = bh / H, h = bh % H;
    const int n0 = (int)sl * BV;

    f32x4 S[MS];
#pragma unroll
    for (int m = 0; m < MS; ++m) {
        S[m] = zero4();
        const int ib = wave + 4 * m;
        if (ib < NKB && p.s0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) S[m][e] = p.s0[(bh * DK + 16 * ib + 4 * lg + e) * Dv + n0 + ln];
        }
    }

    RowsTile<float, C, DK> rk, rq;
    DenseTile<C, C> rt, rp;
    RowsTile<float, C, BV> ri;
    float rg = 0.f, rbeta = 0.f, red = 0.f;
    auto fetch = [&](int64_t c) {
        const int64_t c0 = c * C;
        const float *rec = p.rec + (bh * NC + c) * p.rec_floats;
        rk.load(static_cast<const float *>(p.k), b, h, c0, T, p.ks, DK);
        rq.load(static_cast<const float *>(p.q), b, h, c0, T, p.qs, DK);
        rt.load(rec + Rec<C>::oT, C);
        rp.load(rec + Rec<C>::oP, C);
        ri.load(static_cast<const float *>(p.v), b, h, c0, T, p.vs, Dv, n0);
        if (threadIdx.x < C) {
            const int64_t t = c0 + threadIdx.x;
            rg = rec[Rec<C>::oG + threadIdx.x];
            red = rec[Rec<C>::oEd + threadIdx.x];
            rbeta = t < T ? p.beta[(b * T + t) * H + h] : 0.f;
        }
    };
    fetch(0);

    for (int64_t c = 0; c < NC; ++c) {
        const int64_t c0 = c * C;
        rk.template store<KP>(Ks);
        rq.template store<KP>(Qs);
        rt.template store<CP>(Ts);
        rp.template store<CP>(Ps);
        ri.template store<VP>(Ins);
        if (threadIdx.x < C) {
            Gs[threadIdx.x] = rg;
            Bs[threadIdx.x] = rbeta;
            Eds[threadIdx.x] = red;
        }
        if (c + 1 < NC) fetch(c + 1);
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int ib = wave + 4 * m;
            if (ib < NKB) {
#pragma unroll
                for (int e = 0; e < 4; ++e) STs[ln * KP + 16 * ib + 4 * lg + e] = S[m][e];
            }
        }
        lds_barrier();
        const float GC = Gs[C - 1];

        // step 1: K S -> X = diag(beta)(V - e^G K S); Q S kept for y
        f32x4 qsv = zero4();
        if (wave < NB) {
            const int rb = wave;
            f32x4 ks = zero4();
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += KSD) {
                const FD sf = frag_rows<float, KSD>(STs, KP, 0, k0, lane);
                ks = FD::mma(frag_rows<float, KSD>(Ks, KP, 16 * rb, k0, lane), sf, ks);
                qsv = FD::mma(frag_rows<float, KSD>(Qs, KP, 16 * rb, k0, lane), sf, qsv);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * lg + e;
                Xs[r * VP + ln] = Bs[r] * (Ins[r * VP + ln] - __builtin_amdgcn_exp2f(Gs[r]) * ks[e]);
            }
        }
        lds_barrier();

        // step 2: U = T X (row-major for P U, decayed and transposed for the update)
        if (wave < NB) {
            const int rb = wave;
            f32x4 acc = zero4();
            for (int kb = 0; kb <= rb; ++kb)
                acc = F16::mma(frag_rows<float, 16>(Ts, CP, 16 * rb, 16 * kb, lane),
                               frag_cols<float, 16>(Xs, VP, 0, 16 * kb, lane), acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rb + 4 * lg + e;
                Us[r * VP + ln] = acc[e];
                UdT[ln * CP + r] = Eds[r] * acc[e];
            }
        }
        lds_barrier();

        // step 3: Y = diag(e^G) Q S + P U;  S <- e^{G_C} S + K^T (d o U)
        if (wave < NB) {
            const int rb = wave;
            f32x4 acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = __builtin_amdgcn_exp2f(Gs[16 * rb + 4 * lg + e]) * qsv[e];
            for (int jb = 0; jb <= rb; ++jb)
                acc = F16::mma(frag_rows<float, 16>(Ps, CP, 16 * rb, 16 * jb, lane),
                               frag_cols<float, 16>(Us, VP, 0, 16 * jb, lane), acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t t = c0 + 16 * rb + 4 * lg + e;
                if (t < T) p.y[((b * T + t) * H + h) * Dv + n0 + ln] = acc[e];
            }
        }
        const float eGC = __builtin_amdgcn_exp2f(GC);
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int ib = wave + 4 * m;
            if (ib < NKB) {
                f32x4 acc = S[m] * eGC;
#pragma unroll
                for (int j0 = 0; j0 < C; j0 += KSC)
                    acc = FC::mma(frag_cols<float, KSC>(Ks, KP, 16 * ib, j0, lane),
                                  frag_rows<float, KSC>(UdT, CP, 0, j0, lane), acc);
                S[m] = acc;
            }
        }
        lds_barrier();
    }

    if (p.sT) {
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int ib = wave + 4 * m;
            if (ib < NKB) {
#pragma unroll
                for (int e = 0; e < 4; ++e) p.sT[(bh * DK + 16 * ib + 4 * lg + e) * Dv + n0 + ln] = S[m][e];
            }
        }
    }
}

// The same recurrence on bf16 MFMA: every fp32 operand (K, Q, the state, T, P,
// X, U and the decayed U) enters as a bf16 pair hi + lo, and each product sums
// hi*hi + hi*lo + lo*hi (about 16 bits of every operand).  Same LDS bytes as
// the fp32 form; the MFMA chain per chunk is a quarter as long.
template <int C, int DK> struct Fwd16Lay {
    static constexpr int KP = DK + 8, CP = C + 8;   // bf16 pitches
    static constexpr size_t KB = 2 * C * KP, CB = 2 * C * CP, SB = 2 * BV * KP, TB = 2 * BV * CP;
    static constexpr size_t oKh = 0, oKl = oKh + KB, oQh = oKl + KB, oQl = oQh + KB;
    static constexpr size_t oTh = oQl + KB, oTl = oTh + CB, oPh = oTl + CB, oPl = oPh + CB;
    static constexpr size_t oSTh = oPl + CB, oSTl = oSTh + SB;
    static constexpr size_t oXh = oSTl + SB, oXl = oXh + TB;       // X^T
    static constexpr size_t oUh = oXl + TB, oUl = oUh + TB;        // U^T (for P U)
    static constexpr size_t oDh = oUl + TB, oDl = oDh + TB;        // (d o U)^T (for the update)
    static constexpr size_t oIn = oDl + TB;
    static constexpr size_t oG = oIn + 4 * C * VP;                 // G2, two buffers
    static constexpr size_t oB = oG + 2 * 4 * C;                   // beta, two buffers
    static constexpr size_t oEd = oB + 2 * 4 * C;                  // 2^(G2_{C-1} - G2), two buffers
    static constexpr size_t BYTES = oEd + 2 * 4 * C;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// 8 wavefronts: waves 0-3 carry the chain of every chunk, waves 4-7 stage the
// operands into LDS (as bf16 pairs) while it runs, each array in the window
// after its last read, and prefetch the next chunk's into registers.  The
// chain reads the K^T operands of the state update in step 1, so K (like Q
// and V) is free after step 1.  Per chunk c (barriers B1, B2, B3):
//   B1..B2  chain: step 1 (K S, Q S, X);    staging: P and T of chunk c
//   B2..B3  chain: step 2 (U = T X);        staging: 3/4 of K, V, G2, beta of chunk c+1
//   B3..B1  chain: step 3 (y, update);      staging: the rest of K, Q of chunk c+1
// (the K and Q conversions to bf16 pairs are the staging's largest part, so
// they are spread over the two windows after step 1)
constexpr int NTF = 512;

// One workgroup of the recurrence: slice bid of the grid, LDS of
// Fwd16Lay<C, DK>::BYTES at smem.
template <int C, int DK>
__device__ __forceinline__ void fwd16_carry_block(const BwdParams &p, int64_t bid, char *smem)
{
    using L = Fwd16Lay<C, DK>;
    constexpr int KP = L::KP, CP = L::CP, NB = C / 16, NKB = DK / 16, MS = (NKB + 3) / 4, NJ = C / 32;
    using F16 = Frag<__bf16, 16>;
    using F32 = Frag<__bf16, 32>;
    static_assert(DK % 32 == 0 && C % 32 == 0, "32-deep fragments over Dk and C");
    constexpr int NST = 256;                                       // staging threads
    constexpr int NUK = C * DK / 4, NVK = (NUK + NST - 1) / NST;   // float4 units of K or Q
    constexpr int NUT = C * C / 4, NVT = (NUT + NST - 1) / NST;    // of T or P
    constexpr int NUV = C * BV / 4;                                // of the V slice
    static_assert(NUV <= NST && C <= NST, "one V unit and one gate per staging thread");

    __bf16 *Kh = reinterpret_cast<__bf16 *>(smem + L::oKh), *Kl = reinterpret_cast<__bf16 *>(smem + L::oKl);
    __bf16 *Qh = reinterpret_cast<__bf16 *>(smem + L::oQh), *Ql = reinterpret_cast<__bf16 *>(smem + L::oQl);
    __bf16 *Th = reinterpret_cast<__bf16 *>(smem + L::oTh), *Tl = reinterpret_cast<__bf16 *>(smem + L::oTl);
    __bf16 *Ph = reinterpret_cast<__bf16 *>(smem + L::oPh), *Pl = reinterpret_cast<__bf16 *>(smem + L::oPl);
    __bf16 *STh = reinterpret_cast<__bf16 *>(smem + L::oSTh), *STl = reinterpret_cast<__bf16 *>(smem + L::oSTl);
    __bf16 *Xh = reinterpret_cast<__bf16 *>(smem + L::oXh), *Xl = reinterpret_cast<__bf16 *>(smem + L::oXl);
    __bf16 *Uh = reinterpret_cast<__bf16 *>(smem + L::oUh), *Ul = reinterpret_cast<__bf16 *>(smem + L::oUl);
    __bf16 *Dh = reinterpret_cast<__bf16 *>(smem + L::oDh), *Dl = reinterpret_cast<__bf16 *>(smem + L::oDl);
    float *Ins = reinterpret_cast<float *>(smem + L::oIn);
    float *Gb = reinterpret_cast<float *>(smem + L::oG);
    float *Bb = reinterpret_cast<float *>(smem + L::oB);
    float *Edb = reinterpret_cast<float *>(smem + L::oEd);

    const int lane = lane_id(), wave = wave_id(), ln = lane & 15, lg = lane >> 4;
    const bool chain = wave < 4;
    const int64_t NS = p.Dv / BV;
    int64_t bh, sl;
    slice_of(bid, NS, p.xcd_map, bh, sl);
    const int64_t H = p.H, T = p.T, Dv = p.Dv, NC = p.NC, b = bh / H, h = bh % H;
    const int n0 = (int)sl * BV;

    // The two roles run separate loops with the same barrier sequence (one
    // barrier after the prologue, three per chunk).
    if (!chain) {
        // ---- staging waves.  Every load is issued unconditionally (clamped
        // unit and row indices, the zeros past T applied when the data is
        // written), so the compiler waits on exact outstanding-load counts.
        const int ts = threadIdx.x - 256;
        const float *kg = static_cast<const float *>(p.k);
        const float *qg = static_cast<const float *>(p.q);
        const float *vg = static_cast<const float *>(p.v);
        auto clampc = [&](int64_t c) { return c >= NC ? NC - 1 : c; };
        auto rec_of = [&](int64_t c) { return p.rec + (bh * NC + c) * p.rec_floats; };
        f32x4 rK[NVK], rQ[NVK], rT[NVT], rP[NVT], rV = zero4();
        float rG = 0.f, rBe = 0.f, rEd = 0.f;
        int64_t cK = 0;                                    // chunk held by rV, rG, rBe
        const int uv = ts < NUV ? ts : NUV - 1, ug = ts < C ? ts : C - 1;
        // unit u = ts + NST i of a K or Q tile: row ts / (DK/4) + i NST / (DK/4),
        // columns 4 (ts mod DK/4) ..; byte offsets inside a chunk's rows, 32-bit
        constexpr int RPI = NST / (DK / 4);                 // rows between units i and i+1
        static_assert(NUK % NST == 0, "whole K/Q tiles per staging pass");
        const int kr0 = ts / (DK / 4), kc0 = (ts % (DK / 4)) * 4;
        const uint32_t kstep = (uint32_t)(RPI * p.ks * 4), qstep = (uint32_t)(RPI * p.qs * 4);
        const uint32_t koff0 = (uint32_t)((kr0 * p.ks + kc0) * 4), qoff0 = (uint32_t)((kr0 * p.qs + kc0) * 4);
        // rows of a K or Q tile at or past T (the last chunk only) read token
        // T-1: their beta is 0 and their outputs are not stored, so the rows
        // need no zeros (finite values suffice)
        auto tile_off = [&](int64_t c0, int i, int64_t stride, uint32_t off0, uint32_t step) {
            if (c0 + C <= T) return off0 + (uint32_t)i * step;
            const int64_t r = kr0 + (int64_t)i * RPI;
            return (uint32_t)(((c0 + r < T ? r : T - 1 - c0) * stride + kc0) * 4);
        };
        // K units [i0, i1) of chunk c
        auto load_k = [&](int64_t c, int i0, int i1) {
            const int64_t c0 = c * C;
            const char *kb = reinterpret_cast<const char *>(kg + (b * T + c0) * p.ks + h * DK);
#pragma unroll
            for (int i = i0; i < i1; ++i)
                rK[i] = *reinterpret_cast<const f32x4 *>(kb + tile_off(c0, i, p.ks, koff0, kstep));
        };
        auto load_vg = [&](int64_t c) {
            cK = c;
            const int64_t c0 = c * C;
            const int rv = uv / (BV / 4), cv = (uv % (BV / 4)) * 4;
            const int64_t tv = c0 + rv < T ? c0 + rv : T - 1;
            rV = *reinterpret_cast<const f32x4 *>(vg + (b * T + tv) * p.vs + h * Dv + n0 + cv);
            const int64_t tg = c0 + ug < T ? c0 + ug : T - 1;
            rG = rec_of(c)[Rec<C>::oG + ug];
            rEd = rec_of(c)[Rec<C>::oEd + ug];
            rBe = p.beta[(b * T + tg) * H + h];
        };
        auto load_q = [&](int64_t c) {
            const int64_t c0 = c * C;
            const char *qb = reinterpret_cast<const char *>(qg + (b * T + c0) * p.qs + h * DK);
#pragma unroll
            for (int i = 0; i < NVK; ++i)
                rQ[i] = *reinterpret_cast<const f32x4 *>(qb + tile_off(c0, i, p.qs, qoff0, qstep));
        };
        auto load_cc = [&](f32x4 (&rr)[NVT], int64_t c, int off) {
            const float *rec = rec_of(c) + off;
#pragma unroll
            for (int i = 0; i < NVT; ++i) {
                int u = ts + NST * i;
                u = (NUT % NST == 0 || u < NUT) ? u : NUT - 1;
                const int r = u / (C / 4), col = (u % (C / 4)) * 4;
                rr[i] = *reinterpret_cast<const f32x4 *>(rec + r * C + col);
            }
        };
        auto write_k = [&](int i0, int i1) {
#pragma unroll
            for (int i = i0; i < i1; ++i) {
                const int r = kr0 + RPI * i;
                store_split4(Kh + r * KP + kc0, Kl + r * KP + kc0, rK[i]);
            }
        };
        auto write_vg = [&](int gb) {
            if (ts < NUV) {
                const int r = ts / (BV / 4), col = (ts % (BV / 4)) * 4;
                *reinterpret_cast<f32x4 *>(Ins + r * VP + col) = cK * C + r < T ? rV : zero4();
            }
            if (ts < C) {
                Gb[gb * C + ts] = rG;
                Edb[gb * C + ts] = rEd;
                Bb[gb * C + ts] = cK * C + ts < T ? rBe : 0.f;
            }
        };
        auto write_q = [&]() {
#pragma unroll
            for (int i = 0; i < NVK; ++i) {
                const int r = kr0 + RPI * i;
                store_split4(Qh + r * KP + kc0, Ql + r * KP + kc0, rQ[i]);
            }
        };
        auto write_cc = [&](const f32x4 (&rr)[NVT], __bf16 *hi, __bf16 *lo) {
#pragma unroll
            for (int i = 0; i < NVT; ++i) {
                const int u = ts + NST * i;
                const int r = u / (C / 4), col = (u % (C / 4)) * 4;
                if (NUT % NST == 0 || u < NUT) store_split4(hi + r * CP + col, lo + r * CP + col, rr[i]);
            }
        };
        // chunk 0 into LDS (P(0) and T(0) are written in its first window),
        // then chunk 1 in flight, in the issue order of the loop
        constexpr int NK1 = (3 * NVK + 2) / 4;          // K units staged in B2..B3, the rest in B3..B1
        load_k(0, 0, NVK);
        load_vg(0);
        load_q(0);
        load_cc(rP, 0, Rec<C>::oP);
        load_cc(rT, 0, Rec<C>::oT);
        write_k(0, NVK);
        write_vg(0);
        write_q();
        load_k(clampc(1), 0, NK1);
        load_vg(clampc(1));
        __builtin_amdgcn_sched_barrier(0);
        load_k(clampc(1), NK1, NVK);
        load_q(clampc(1));
        lds_barrier();                                  // B1 of chunk 0
        for (int64_t c = 0; c < NC; ++c) {
            write_cc(rP, Ph, Pl);                       // P(c): P(c-1) last read in step 3
            write_cc(rT, Th, Tl);                       // T(c): T(c-1) last read in step 2
            load_cc(rP, clampc(c + 1), Rec<C>::oP);
            load_cc(rT, clampc(c + 1), Rec<C>::oT);
            lds_barrier();                              // B2
            write_k(0, NK1);                            // chunk c+1: K and V last read in step 1
            write_vg((int)((c + 1) & 1));
            load_k(clampc(c + 2), 0, NK1);
            load_vg(clampc(c + 2));
            lds_barrier();                              // B3
            write_k(NK1, NVK);
            write_q();                                  // Q(c+1): Q(c) last read in step 1
            load_k(clampc(c + 2), NK1, NVK);
            load_q(clampc(c + 2));
            lds_barrier();                              // B1 of chunk c+1
        }
    } else {
        // ---- chain waves: the state slice in accumulators
        f32x4 S[MS];
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            S[m] = zero4();
            const int ib = wave + 4 * m;
            if (ib < NKB && p.s0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) S[m][e] = p.s0[(bh * DK + 16 * ib + 4 * lg + e) * Dv + n0 + ln];
            }
        }
        auto write_state_operand = [&]() {
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int ib = wave + 4 * m;
                if (ib < NKB) {
                    const int row = 16 * ib + 4 * lg;
                    store_split4(STh + ln * KP + row, STl + ln * KP + row, S[m]);
                }
            }
        };
        write_state_operand();
        lds_barrier();                                  // B1 of chunk 0
        for (int64_t c = 0; c < NC; ++c) {
            const int64_t c0 = c * C;
            const float *Gs = Gb + (c & 1) * C, *Bs = Bb + (c & 1) * C, *Eds = Edb + (c & 1) * C;
            const float GC = Gs[C - 1];

            // ---- step 1: K S, Q S;  X = diag(beta)(V - e^G K S); the K^T
            // operands of the update (K is restaged after this step)
            F32 kth[MS][NJ], ktl[MS][NJ];
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int ib = wave + 4 * m;
                if (ib < NKB) {
#pragma unroll
                    for (int jj = 0; jj < NJ; ++jj) {
                        kth[m][jj] = tr_frag32(Kh, KP, 16 * ib, 32 * jj, lane);
                        ktl[m][jj] = tr_frag32(Kl, KP, 16 * ib, 32 * jj, lane);
                    }
                }
            }
            f32x4 qsv = zero4();
            if (wave < NB) {
                const int rb = wave;
                f32x4 ks = zero4(), ks2 = zero4(), qs2 = zero4();
#pragma unroll
                for (int k0 = 0; k0 < DK; k0 += 32) {
                    const F32 sh = frag_rows<__bf16, 32>(STh, KP, 0, k0, lane);
                    const F32 sl2 = frag_rows<__bf16, 32>(STl, KP, 0, k0, lane);
                    const F32 kh = frag_rows<__bf16, 32>(Kh, KP, 16 * rb, k0, lane);
                    const F32 kl = frag_rows<__bf16, 32>(Kl, KP, 16 * rb, k0, lane);
                    const F32 qh = frag_rows<__bf16, 32>(Qh, KP, 16 * rb, k0, lane);
                    const F32 ql = frag_rows<__bf16, 32>(Ql, KP, 16 * rb, k0, lane);
                    ks = F32::mma(kh, sh, ks);
                    qsv = F32::mma(qh, sh, qsv);
                    ks2 = F32::mma(kh, sl2, ks2);
                    qs2 = F32::mma(qh, sl2, qs2);
                    ks2 = F32::mma(kl, sh, ks2);
                    qs2 = F32::mma(ql, sh, qs2);
                }
                ks += ks2;
                qsv += qs2;
                const int r0 = 16 * rb + 4 * lg;
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    x[e] = Bs[r0 + e] * (Ins[(r0 + e) * VP + ln] - __builtin_amdgcn_exp2f(Gs[r0 + e]) * ks[e]);
                store_split4(Xh + ln * CP + r0, Xl + ln * CP + r0, x);
            }
            lds_barrier();                              // B2

            // ---- step 2: U = T X, kept transposed (for P U) and decayed (for the update)
            if (wave < NB) {
                const int rb = wave;
                const int r0 = 16 * rb + 4 * lg;
                f32x4 acc = zero4(), acc2 = zero4();
                for (int kb = 0; kb <= rb; ++kb) {
                    const F16 ah = frag_rows<__bf16, 16>(Th, CP, 16 * rb, 16 * kb, lane);
                    const F16 al = frag_rows<__bf16, 16>(Tl, CP, 16 * rb, 16 * kb, lane);
                    const F16 xh = frag_rows<__bf16, 16>(Xh, CP, 0, 16 * kb, lane);
                    const F16 xl = frag_rows<__bf16, 16>(Xl, CP, 0, 16 * kb, lane);
                    acc = F16::mma(ah, xh, acc);
                    acc2 = F16::mma(ah, xl, acc2);
                    acc2 = F16::mma(al, xh, acc2);
                }
                acc += acc2;
                store_split4(Uh + ln * CP + r0, Ul + ln * CP + r0, acc);
                f32x4 d;
#pragma unroll
                for (int e = 0; e < 4; ++e) d[e] = Eds[r0 + e] * acc[e];
                store_split4(Dh + ln * CP + r0, Dl + ln * CP + r0, d);
            }
            lds_barrier();                              // B3

            // ---- step 3: Y = diag(e^G) Q S + P U;  S <- e^{G_C} S + K^T (d o U)
            if (wave < NB) {
                const int rb = wave;
                f32x4 acc, acc2 = zero4();
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = __builtin_amdgcn_exp2f(Gs[16 * rb + 4 * lg + e]) * qsv[e];
                for (int jb = 0; jb <= rb; ++jb) {
                    const F16 ah = frag_rows<__bf16, 16>(Ph, CP, 16 * rb, 16 * jb, lane);
                    const F16 al = frag_rows<__bf16, 16>(Pl, CP, 16 * rb, 16 * jb, lane);
                    const F16 uh = frag_rows<__bf16, 16>(Uh, CP, 0, 16 * jb, lane);
                    const F16 ul = frag_rows<__bf16, 16>(Ul, CP, 0, 16 * jb, lane);
                    acc = F16::mma(ah, uh, acc);
                    acc2 = F16::mma(ah, ul, acc2);
                    acc2 = F16::mma(al, uh, acc2);
                }
                acc += acc2;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t t = c0 + 16 * rb + 4 * lg + e;
                    if (t < T) p.y[((b * T + t) * H + h) * Dv + n0 + ln] = acc[e];
                }
            }
            const float eGC = __builtin_amdgcn_exp2f(GC);
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int ib = wave + 4 * m;
                if (ib < NKB) {
                    f32x4 acc = S[m] * eGC, acc2 = zero4();
#pragma unroll
                    for (int jj = 0; jj < NJ; ++jj) {
                        const F32 dh = pair_rows32(Dh, CP, 0, 32 * jj, lane);
                        const F32 dl = pair_rows32(Dl, CP, 0, 32 * jj, lane);
                        acc = F32::mma(kth[m][jj], dh, acc);
                        acc2 = F32::mma(kth[m][jj], dl, acc2);
                        acc2 = F32::mma(ktl[m][jj], dh, acc2);
                    }
                    S[m] = acc + acc2;
                }
            }
            write_state_operand();                      // S^T of chunk c+1: last read in step 1
            lds_barrier();                              // B1 of chunk c+1
        }

        if (p.sT) {
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int ib = wave + 4 * m;
                if (ib < NKB) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) p.sT[(bh * DK + 16 * ib + 4 * lg + e) * Dv + n0 + ln] = S[m][e];
                }
            }
        }
    }
}

template <int C, int DK>
__global__ __launch_bounds__(NTF) void fwd16_carry_kernel(BwdParams p)
{
    __shared__ __attribute__((aligned(16))) char smem[Fwd16Lay<C, DK>::BYTES];
    fwd16_carry_block<C, DK>(p, blockIdx.x, smem);
}

// The recurrence and an independent bf16 product in one launch: workgroups
// below nslice are the recurrence's slices (placed as in fwd16_carry_kernel),
// those from ncore (nslice rounded up to a multiple of 8; the ones between end
// at once) the product's 256 x 256 tiles, which the hardware then places on
// the compute units the slices leave free.  Every output of the product sums its K in the
// same order as in a launch of its own, so it is the same bits.
constexpr int SIDE_BM = 256, SIDE_BN = 256, SIDE_ST = 4, SIDE_NW = 8;
static_assert(SIDE_NW * 64 == NTF, "one block size for both roles");

struct SideArgs {
    const __bf16 *A;
    GemmProducts<__bf16> P;
    int M, K;
    int64_t lda;
    int tiles_m, tiles_n, bn_log;
    int64_t nslice, ncore;
};

template <int C, int DK>
__global__ __launch_bounds__(NTF, 1) void fwd16_carry_side_kernel(BwdParams p, SideArgs g)
{
    constexpr size_t GB = (size_t)SIDE_ST * GemmTile<SIDE_BM, SIDE_BN, SIDE_NW>::STAGE;
    constexpr size_t FB = Fwd16Lay<C, DK>::BYTES;
    __shared__ __attribute__((aligned(1024))) char smem[FB > GB ? FB : GB];
    const int64_t bid = blockIdx.x;
    if (bid < g.nslice) {
        fwd16_carry_block<C, DK>(p, bid, smem);
    } else if (bid >= g.ncore) {
        gemm_nt_block<__bf16, SIDE_BM, SIDE_BN, SIDE_ST, SIDE_NW>((int)(bid - g.ncore), smem, g.A, g.M, g.K, g.lda,
                                                                  g.P, g.tiles_m, g.tiles_n, g.bn_log);
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
    kp.qs = a.H * DK; kp.ks = a.H * DK; kp.vs = a.H * a.Dv;
    kp.y = nullptr; kp.sT = nullptr;
    kp.xcd_map = (a.B * a.H) % 8 == 0 ? 1 : 0;
    const int64_t bh = a.B * a.H;
    float *ws = static_cast<float *>(a.ws);
    kp.rec = ws;
    kp.sc = kp.rec + bh * kp.NC * kp.rec_floats;
    kp.dsc = kp.sc + bh * kp.NC * DK * a.Dv;
    kp.ub = kp.dsc + bh * kp.NC * DK * a.Dv;
    kp.wb = kp.ub + bh * kp.NC * C * a.Dv;
    kp.dxb = kp.wb + bh * kp.NC * C * a.Dv;
    const unsigned nchunk = (unsigned)(bh * kp.NC), nslice = (unsigned)(bh * (a.Dv / BV));
    hipLaunchKernelGGL((bwd_prep_kernel<Tin, C, DK>), dim3(nchunk), dim3(NT), 0, stream, kp);
    if constexpr (std::is_same<Tin, __bf16>::value) {
        hipLaunchKernelGGL((bwd_carry16_kernel<C, DK, false>), dim3(nslice), dim3(NTC), 0, stream, kp);
        hipLaunchKernelGGL((bwd_carry16_kernel<C, DK, true>), dim3(nslice), dim3(NTC), 0, stream, kp);
    } else {
        hipLaunchKernelGGL((bwd_carry_kernel<Tin, C, DK, false>), dim3(nslice), dim3(NT), 0, stream, kp);
        hipLaunchKernelGGL((bwd_carry_kernel<Tin, C, DK, true>), dim3(nslice), dim3(NT), 0, stream, kp);
    }
    // the bf16 chunk-gradient kernel takes the value columns 32 at a time
    if (std::is_same<Tin, __bf16>::value && a.Dv % 32 == 0)
        hipLaunchKernelGGL((bwd_chunk16_kernel<C, DK>), dim3(nchunk), dim3(NTG), 0, stream, kp);
    else
        hipLaunchKernelGGL((bwd_chunk_kernel<Tin, C, DK>), dim3(nchunk), dim3(NTG), 0, stream, kp);
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

template <int C, int DK>
hipError_t launch_fwd32_t(const PrefillArgs &a, hipStream_t stream)
{
    BwdParams kp{};
    kp.q = a.q; kp.k = a.k; kp.v = a.v;
    kp.alpha = a.alpha; kp.beta = a.beta; kp.s0 = a.s0;
    kp.y = a.y; kp.sT = a.sT;
    kp.T = a.T; kp.H = a.H; kp.Dv = a.Dv;
    kp.NC = (a.T + C - 1) / C;
    kp.rec_floats = bwd_record_floats(C);
    kp.xcd_map = (a.B * a.H) % 8 == 0 ? 1 : 0;
    kp.qs = a.q_tok_stride; kp.ks = a.k_tok_stride; kp.vs = a.v_tok_stride;
    kp.rec = static_cast<float *>(a.ws);
    const int64_t bh = a.B * a.H;
    const unsigned nchunk = (unsigned)(bh * kp.NC), nslice = (unsigned)(bh * (a.Dv / BV));
    hipLaunchKernelGGL((bwd_prep_kernel<float, C, DK>), dim3(nchunk), dim3(NT), 0, stream, kp);
    // fp32 MFMA unless the caller's bound is the bf16 one (hi/lo operands carry
    // about 16 bits, which an fp32-input run with a small RMS(y) can exceed)
    if constexpr (DK % 32 == 0 && C % 32 == 0) {
        // (its staging addresses a chunk's q and k rows by 32-bit byte offsets)
        const int64_t wide = a.q_tok_stride > a.k_tok_stride ? a.q_tok_stride : a.k_tok_stride;
        if (a.hilo_core && (int64_t)C * wide * 4 < ((int64_t)1 << 32)) {
            if (!a.side) {
                hipLaunchKernelGGL((fwd16_carry_kernel<C, DK>), dim3(nslice), dim3(NTF), 0, stream, kp);
                return hipGetLastError();
            }
            const PrefillArgs::SideGemm &sg = *a.side;
            const GemmGrid<SIDE_BM, SIDE_BN> gg(sg.M, sg.N, 0);
            SideArgs g;
            g.A = sg.A;
            g.P = gemm_products(gg, GemmOp<__bf16>{sg.B, sg.C, sg.N, sg.ldb, sg.ldc});
            g.M = (int)sg.M; g.K = (int)sg.K; g.lda = sg.lda;
            g.tiles_m = gg.tiles_m; g.tiles_n = gg.tiles_n; g.bn_log = gg.bn_log;
            // the product's workgroups start on a multiple of 8, so its XCD
            // placement is the one of a launch of its own
            g.nslice = nslice;
            g.ncore = ((int64_t)nslice + 7) / 8 * 8;
            hipLaunchKernelGGL((fwd16_carry_side_kernel<C, DK>), dim3((unsigned)(g.ncore + gg.grid)), dim3(NTF), 0,
                               stream, kp, g);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((fwd32_carry_kernel<C, DK>), dim3(nslice), dim3(NT), 0, stream, kp);
    return hipGetLastError();
}

template <int C>
hipError_t launch_fwd32_dk(const PrefillArgs &a, hipStream_t s)
{
    switch (a.Dk) {
    case 16: return launch_fwd32_t<C, 16>(a, s);
    case 32: return launch_fwd32_t<C, 32>(a, s);
    case 64: return launch_fwd32_t<C, 64>(a, s);
    case 128: return launch_fwd32_t<C, 128>(a, s);
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

int64_t bwd_record_floats(int64_t C) { return (3 * C * C + 2 * C + 63) / 64 * 64; }

size_t prefill_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int64_t C)
{
    const int64_t nc = (T + C - 1) / C;
    return (size_t)(4 * B * H * nc * (bwd_record_floats(C) + 2 * Dk * Dv + 3 * C * Dv));
}

size_t prefill_f32_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t C)
{
    return (size_t)(4 * B * H * ((T + C - 1) / C) * bwd_record_floats(C));
}

hipError_t launch_prefill_f32_staged(const PrefillArgs &a, hipStream_t stream)
{
    switch (a.chunk) {
    case 16: return launch_fwd32_dk<16>(a, stream);
    case 32: return launch_fwd32_dk<32>(a, stream);
    case 64: return launch_fwd32_dk<64>(a, stream);
    }
    return hipErrorInvalidValue;
}

// Whether launch_prefill_f32_staged runs the hi/lo recurrence for these
// arguments (and with it a.side): the same conditions as launch_fwd32_t, after
// launch_prefill's early returns.
bool prefill_f32_takes_side(const PrefillArgs &a)
{
    const int64_t wide = a.q_tok_stride > a.k_tok_stride ? a.q_tok_stride : a.k_tok_stride;
    return !a.bf16 && a.ws && a.hilo_core && a.B * a.H > 0 && a.T > 0 && a.Dk % 32 == 0 && a.Dk <= 128 &&
           a.chunk % 32 == 0 && a.chunk <= 64 && a.chunk * wide * 4 < ((int64_t)1 << 32);
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
