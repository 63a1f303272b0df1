// recurrence.hip -- the state recurrence of the chunkwise gated delta rule for
// bf16 inputs, consuming the per-chunk records of the preparation kernel.
//
// Source: "On the Design of Qwen3.8-Next Architecture", picx.dev summary,
// "Theoretical foundations", eqs (1)-(4).  With the chunk quantities of the
// record (EG, Ed, EGC, T' = (I + A)^-1 diag(beta), P) one chunk entering with
// state S is
//
//   R  = V - diag(EG) K S
//   U  = T' R                         (u_r = beta_r e_r of eqs (2)-(3))
//   Y  = diag(EG) Q S + P U           (eq (4))
//   S' = EGC S + K^T diag(Ed) U       (eqs (1), (3))
//
// Columns of S, V, U, Y are independent, so each workgroup carries one
// 16-column slice of S for one (b, h) through all chunks (fp32 master copy in
// MFMA accumulators).  Twelve wavefronts, three phases per chunk:
//
//  waves   phase 1                        phase 2                 phase 3
//  0-3     K S of row block w -> R_w      U_w = sum_k T'_wk R_k    S update (rows 16w, 16(w+4))
//  4-7     Q S of row block w-4           -                       Y = EG Q S + P U
//  8-11    -                              stage chunk c+1 into    -
//                                         LDS; load chunk c+2
//
// Only the staging waves touch global memory inside the loop (K, Q, V and the
// chunk's record, loaded one chunk ahead into registers): the compute waves
// never wait on the vector-memory counter, which on this architecture also
// counts the output stores.
//
// Precision: q, k, v are exact bf16 MFMA operands, every product accumulates
// in fp32.  Operands computed in fp32 -- S, R, U, the decayed U, and from the
// record T' and P -- enter the MFMAs as bf16 pairs hi + lo (hi = bf16(x),
// lo = bf16(x - hi)); products sum hi*hi + hi*lo + lo*hi.
#include "common.hpp"
#include "launch.hpp"
#include "prep_layout.hpp"

namespace gdn {

namespace {

constexpr int REC_THREADS = 768;   // 12 wavefronts

struct RecParams {
    const void *q, *k, *v;
    const float *s0;
    float *y, *sT;
    const char *ws;
    int64_t T, H, Dv;
    int64_t qs, ks, vs;      // token strides (elements)
    int nslices;             // Dv / 16
    int xcd_map;             // 1: group the slices of a head on one XCD
};

template <int C, int DK> struct RecLay {
    static constexpr int NB = C / 16;
    static constexpr int NSB = DK / 16;
    static constexpr int MS = (NSB + 3) / 4;           // state row blocks per S-wave
    static constexpr int KS_DK = DK % 32 == 0 ? 32 : 16;
    static constexpr int KS_C = C % 32 == 0 ? 32 : 16;
    static constexpr int KP = frag_pitch<KS_DK>(DK);   // K, Q, S^T rows (bf16)
    static constexpr int CPU = C + 4;                  // U^T rows: 64-bit stores and reads
    static constexpr int CPD = frag_pitch<KS_C>(C);    // e^{G_C-G} U^T rows
    // one chunk buffer
    static constexpr size_t cK = 0;
    static constexpr size_t cQ = cK + align16(2 * C * KP);
    static constexpr size_t cV = cQ + align16(2 * C * KP);     // V slice [C][16] bf16
    static constexpr size_t cRec = cV + align16(2 * C * BV);   // copy of the chunk's record
    static constexpr size_t CBUF = cRec + align16(PrepRecord<C>::BYTES);
    // shared by the phases of one chunk
    static constexpr size_t oSTh = 2 * CBUF;
    static constexpr size_t oSTl = oSTh + align16(2 * BV * KP);
    static constexpr size_t oRh = oSTl + align16(2 * BV * KP);   // R blocks [NB][64 lanes] bf16x4
    static constexpr size_t oRl = oRh + (size_t)NB * 512;
    static constexpr size_t oUh = oRl + (size_t)NB * 512;
    static constexpr size_t oUl = oUh + align16(2 * BV * CPU);
    static constexpr size_t oUdh = oUl + align16(2 * BV * CPU);
    static constexpr size_t oUdl = oUdh + align16(2 * BV * CPD);
    static constexpr size_t BYTES = oUdl + align16(2 * BV * CPD);
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ int tri_idx(int i, int k) { return i * (i + 1) / 2 + k; }

// Token order of the decayed U^T rows used by the state update.  Within each
// k-step of KS tokens, lane group g (KS/4 values per lane) takes the tokens
// 2g + 8(e/2) + (e%2), e = 0..KS/4-1: adjacent pairs, 8 tokens apart.  The
// column gather of K then reads rows two tokens apart in the four lane groups,
// which fall on distinct LDS banks.  ud_pos gives the storage position of
// token t; the B operand is then an ordinary contiguous fragment read.
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

template <int C, int DK>
__global__ __launch_bounds__(REC_THREADS, 1) void gdn_recurrence_kernel(RecParams p)
{
    using L = RecLay<C, DK>;
    using Rec = PrepRecord<C>;
    using F16 = Frag<__bf16, 16>;
    using FDK = Frag<__bf16, L::KS_DK>;
    using FC = Frag<__bf16, L::KS_C>;
    constexpr int KP = L::KP, CPU = L::CPU, CPD = L::CPD, NB = L::NB, NSB = L::NSB, MS = L::MS;
    constexpr int KS_DK = L::KS_DK, KS_C = L::KS_C, NK = DK / KS_DK;

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    auto cbuf = [&](int64_t c) { return smem + (c & 1) * L::CBUF; };
    __bf16 *STh = reinterpret_cast<__bf16 *>(smem + L::oSTh);
    __bf16 *STl = reinterpret_cast<__bf16 *>(smem + L::oSTl);
    bf16x4 *Rh = reinterpret_cast<bf16x4 *>(smem + L::oRh);
    bf16x4 *Rl = reinterpret_cast<bf16x4 *>(smem + L::oRl);
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
    const int64_t NC = (T + C - 1) / C;
    const char *recs = p.ws + bh * NC * (int64_t)Rec::BYTES;

    // S-waves: row block rb = w; state rows ib = w + 4m.  The row block is a
    // compile-time constant in each copy, so the block sums are fully unrolled.
    auto s_wave = [&](auto rb_c) {
        constexpr int rb = decltype(rb_c)::value;
        constexpr bool has_rb = rb < NB;
        f32x4 S[MS];
#pragma unroll
        for (int m = 0; m < MS; ++m) S[m] = zero4();
        if (p.s0) {
            const float *s0 = p.s0 + bh * (int64_t)DK * Dv;
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int ib = rb + 4 * m;
                if (ib < NSB) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) S[m][e] = s0[(int64_t)(16 * ib + 4 * lg + e) * Dv + n0 + ln];
                }
            }
        }
        auto write_state_operand = [&]() {
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int ib = rb + 4 * m;
                if (ib < NSB) {
                    bf16x4 hv, lv;
                    split4(S[m], hv, lv);
                    *reinterpret_cast<bf16x4 *>(STh + ln * KP + 16 * ib + 4 * lg) = hv;
                    *reinterpret_cast<bf16x4 *>(STl + ln * KP + 16 * ib + 4 * lg) = lv;
                }
            }
        };
        write_state_operand();

        __syncthreads();                        // chunk 0 staged, S^T written

        for (int64_t c = 0; c < NC; ++c) {
            const char *cb = cbuf(c);
            const __bf16 *Ks = reinterpret_cast<const __bf16 *>(cb + L::cK);
            const float *dec = reinterpret_cast<const float *>(cb + L::cRec + Rec::oDec);
            const bf16x4 *tf = reinterpret_cast<const bf16x4 *>(cb + L::cRec + Rec::oT);
            // ---- phase 1: R_rb = V_rb - diag(EG) K_rb S
            if constexpr (has_rb) {
                const __bf16 *Vs = reinterpret_cast<const __bf16 *>(cb + L::cV);
                const f32x4 eg = *reinterpret_cast<const f32x4 *>(dec + 16 * rb + 4 * lg);
                FDK kf[NK], sh[NK], slo[NK];
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    kf[kk] = frag_rows<__bf16, KS_DK>(Ks, KP, 16 * rb, kk * KS_DK, lane);
                    sh[kk] = frag_rows<__bf16, KS_DK>(STh, KP, 0, kk * KS_DK, lane);
                    slo[kk] = frag_rows<__bf16, KS_DK>(STl, KP, 0, kk * KS_DK, lane);
                }
                f32x4 ks_h = zero4(), ks_l = zero4();
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    ks_h = FDK::mma(kf[kk], sh[kk], ks_h);
                    ks_l = FDK::mma(kf[kk], slo[kk], ks_l);
                }
                f32x4 rv;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    rv[e] = (float)Vs[(16 * rb + 4 * lg + e) * BV + ln] - eg[e] * (ks_h[e] + ks_l[e]);
                bf16x4 hv, lv;
                split4(rv, hv, lv);
                Rh[rb * 64 + lane] = hv;
                Rl[rb * 64 + lane] = lv;
            }
            __syncthreads();

            // ---- phase 2: U_rb = sum_{k <= rb} T'_rb,k R_k
            if constexpr (has_rb) {
                f32x4 u = zero4(), u2 = zero4();
                const int r0 = 16 * rb + 4 * lg;
                const f32x4 ed = *reinterpret_cast<const f32x4 *>(dec + C + r0);
                F16 rh[rb + 1], rl[rb + 1], ah[rb + 1], al[rb + 1];
                static_for<rb + 1>([&](auto k_c) {
                    constexpr int k = decltype(k_c)::value;
                    rh[k].v = Rh[k * 64 + lane];
                    rl[k].v = Rl[k * 64 + lane];
                    ah[k].v = tf[tri_idx(rb, k) * 128 + lane];
                    al[k].v = tf[tri_idx(rb, k) * 128 + 64 + lane];
                });
                static_for<rb + 1>([&](auto k_c) {
                    constexpr int k = decltype(k_c)::value;
                    u = F16::mma(ah[k], rh[k], u);
                    u2 = F16::mma(ah[k], rl[k], u2);
                    u2 = F16::mma(al[k], rh[k], u2);
                });
                u += u2;
                bf16x4 uh, ul, dh, dl;
                split4(u, uh, ul);
                split4(ed * u, dh, dl);
                *reinterpret_cast<bf16x4 *>(UTh + ln * CPU + r0) = uh;
                *reinterpret_cast<bf16x4 *>(UTl + ln * CPU + r0) = ul;
                // tokens (r0, r0 + 1) and (r0 + 2, r0 + 3) stay adjacent in the
                // permuted order of the decayed U^T
                const int pa = ln * CPD + ud_pos<KS_C>(r0), pb = ln * CPD + ud_pos<KS_C>(r0 + 2);
                *reinterpret_cast<bf16x2 *>(UdTh + pa) = bf16x2{dh[0], dh[1]};
                *reinterpret_cast<bf16x2 *>(UdTh + pb) = bf16x2{dh[2], dh[3]};
                *reinterpret_cast<bf16x2 *>(UdTl + pa) = bf16x2{dl[0], dl[1]};
                *reinterpret_cast<bf16x2 *>(UdTl + pb) = bf16x2{dl[2], dl[3]};
            }
            __syncthreads();

            // ---- phase 3: S <- EGC S + K^T (diag(Ed) U)
            {
                constexpr int NJ = C / KS_C;
                const float egc = dec[2 * C];
                FC uh[NJ], ul[NJ], ka[MS][NJ];
#pragma unroll
                for (int jj = 0; jj < NJ; ++jj) {
                    uh[jj] = frag_rows<__bf16, KS_C>(UdTh, CPD, 0, jj * KS_C, lane);
                    ul[jj] = frag_rows<__bf16, KS_C>(UdTl, CPD, 0, jj * KS_C, lane);
                }
#pragma unroll
                for (int m = 0; m < MS; ++m) {
                    const int ib = rb + 4 * m;
                    if (ib < NSB) {
#pragma unroll
                        for (int jj = 0; jj < NJ; ++jj) ka[m][jj] = k_cols_paired<KS_C>(Ks, KP, 16 * ib, jj * KS_C, lane);
                    }
                }
#pragma unroll
                for (int m = 0; m < MS; ++m) {
                    const int ib = rb + 4 * m;
                    if (ib < NSB) {
                        f32x4 acc = S[m] * egc, acc2 = zero4();
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
                const int ib = rb + 4 * m;
                if (ib < NSB) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) sT[(int64_t)(16 * ib + 4 * lg + e) * Dv + n0 + ln] = S[m][e];
                }
            }
        }
    };

    // Y-waves: row block rb = w - 4, compile-time in each copy.
    auto y_wave = [&](auto rb_c) {
        constexpr int rb = decltype(rb_c)::value;
        constexpr bool has_rb = rb < NB;
        __syncthreads();

        f32x4 qs = zero4();
        for (int64_t c = 0; c < NC; ++c) {
            const char *cb = cbuf(c);
            // ---- phase 1: Q S of this row block (state at the chunk's start)
            if constexpr (has_rb) {
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
                // keep the sum next to its MFMAs: an MFMA result read right after
                // a branch can miss its wait states
                asm volatile("" : "+v"(qs));
            }
            __syncthreads();
            __syncthreads();
            // ---- phase 3: Y = diag(EG) Q S + P U
            if constexpr (has_rb) {
                const float *dec = reinterpret_cast<const float *>(cb + L::cRec + Rec::oDec);
                const bf16x4 *pf = reinterpret_cast<const bf16x4 *>(cb + L::cRec + Rec::oP);
                const f32x4 eg = *reinterpret_cast<const f32x4 *>(dec + 16 * rb + 4 * lg);
                f32x4 acc = eg * qs, acc2 = zero4();
                F16 ah[rb + 1], al[rb + 1], uh[rb + 1], ul[rb + 1];
                static_for<rb + 1>([&](auto j_c) {
                    constexpr int jb = decltype(j_c)::value;
                    ah[jb].v = pf[tri_idx(rb, jb) * 128 + lane];
                    al[jb].v = pf[tri_idx(rb, jb) * 128 + 64 + lane];
                    uh[jb] = frag_rows<__bf16, 16>(UTh, CPU, 0, 16 * jb, lane);
                    ul[jb] = frag_rows<__bf16, 16>(UTl, CPU, 0, 16 * jb, lane);
                });
                static_for<rb + 1>([&](auto j_c) {
                    constexpr int jb = decltype(j_c)::value;
                    acc = F16::mma(ah[jb], uh[jb], acc);
                    acc2 = F16::mma(al[jb], uh[jb], acc2);
                    acc2 = F16::mma(ah[jb], ul[jb], acc2);
                });
                const int64_t c0 = c * C;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t t = c0 + 16 * rb + 4 * lg + e;
                    if (t < T) p.y[((b * T + t) * H + h) * Dv + n0 + ln] = acc[e] + acc2[e];
                }
            }
            __syncthreads();
        }
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    switch (wave) {
    case 0: s_wave(I0{}); break;
    case 1: s_wave(I1{}); break;
    case 2: s_wave(I2{}); break;
    case 3: s_wave(I3{}); break;
    case 4: y_wave(I0{}); break;
    case 5: y_wave(I1{}); break;
    case 6: y_wave(I2{}); break;
    case 7: y_wave(I3{}); break;
    default: {
        // ===================== L-waves (8-11): staging =====================
        const int lt = tid - 512;                          // 0-255
        constexpr int VPR = DK / 8;                        // 16-byte vectors per K/Q row
        constexpr int NKV = (C * VPR + 255) / 256;         // per thread
        const __bf16 *qg = static_cast<const __bf16 *>(p.q);
        const __bf16 *kg = static_cast<const __bf16 *>(p.k);
        const __bf16 *vg = static_cast<const __bf16 *>(p.v);
        const int64_t rowc = b * T;
        const __bf16 *kp[NKV], *qp[NKV];
        int rr[NKV];
#pragma unroll
        for (int i = 0; i < NKV; ++i) {
            const int vi = lt + 256 * i;
            rr[i] = vi < C * VPR ? vi / VPR : -1;          // row within the chunk (-1: none)
            const int row0 = rr[i] < 0 ? 0 : rr[i];
            const int col = (vi % VPR) * 8;
            kp[i] = kg + (rowc + row0) * p.ks + h * DK + col;
            qp[i] = qg + (rowc + row0) * p.qs + h * DK + col;
        }
        const int vr = lt >> 1;                            // V slice: two 16-byte vectors per row
        const bool has_v = lt < C * 2;
        const __bf16 *vp = vg + (rowc + (has_v ? vr : 0)) * p.vs + h * Dv + n0 + (lt & 1) * 8;
        constexpr int RECV = (int)(Rec::BYTES / 16);              // 16-byte vectors per record
        constexpr int NRV = (RECV + 255) / 256;
        const f32x4 *recv = reinterpret_cast<const f32x4 *>(recs);
        f32x4 pk[NKV], pq[NKV], pr[NRV], pv = zero4();
        // Loads are issued unconditionally (rows past the end read row 0 of the
        // sequence and are zeroed when staged), so the compiler can count them
        // and each wait covers exactly the data being staged.
        auto row_ok = [&](int64_t c0, int r) { return r >= 0 && c0 + r < T; };
        auto load_k = [&](int64_t c) {
            const int64_t c0 = c * C;
#pragma unroll
            for (int i = 0; i < NKV; ++i)
                pk[i] = *reinterpret_cast<const f32x4 *>(row_ok(c0, rr[i]) ? kp[i] + c0 * p.ks : kp[i]);
        };
        auto load_qv = [&](int64_t c) {
            const int64_t c0 = c * C;
#pragma unroll
            for (int i = 0; i < NKV; ++i)
                pq[i] = *reinterpret_cast<const f32x4 *>(row_ok(c0, rr[i]) ? qp[i] + c0 * p.qs : qp[i]);
            pv = *reinterpret_cast<const f32x4 *>(has_v && c0 + vr < T ? vp + c0 * p.vs : vp);
        };
        auto load_rec = [&](int64_t c) {
#pragma unroll
            for (int i = 0; i < NRV; ++i) {
                const int j = lt + 256 * i < RECV ? lt + 256 * i : RECV - 1;
                pr[i] = recv[c * RECV + j];
            }
        };
        // staging is split over the three phases: K rows, then Q rows and V, then
        // the record (buffer c+1 is free for the whole of iteration c)
        auto stage_k = [&](int64_t c) {
            __bf16 *Ks = reinterpret_cast<__bf16 *>(cbuf(c) + L::cK);
            const int64_t c0 = c * C;
#pragma unroll
            for (int i = 0; i < NKV; ++i)
                if (rr[i] >= 0)
                    *reinterpret_cast<f32x4 *>(Ks + rr[i] * KP + ((lt + 256 * i) % VPR) * 8) =
                        row_ok(c0, rr[i]) ? pk[i] : zero4();
        };
        auto stage_qv = [&](int64_t c) {
            __bf16 *Qs = reinterpret_cast<__bf16 *>(cbuf(c) + L::cQ);
            __bf16 *Vs = reinterpret_cast<__bf16 *>(cbuf(c) + L::cV);
            const int64_t c0 = c * C;
#pragma unroll
            for (int i = 0; i < NKV; ++i)
                if (rr[i] >= 0)
                    *reinterpret_cast<f32x4 *>(Qs + rr[i] * KP + ((lt + 256 * i) % VPR) * 8) =
                        row_ok(c0, rr[i]) ? pq[i] : zero4();
            if (has_v) *reinterpret_cast<f32x4 *>(Vs + vr * BV + (lt & 1) * 8) = c0 + vr < T ? pv : zero4();
        };
        auto stage_rec = [&](int64_t c) {
            f32x4 *rd = reinterpret_cast<f32x4 *>(cbuf(c) + L::cRec);
#pragma unroll
            for (int i = 0; i < NRV; ++i)
                if (lt + 256 * i < RECV) rd[lt + 256 * i] = pr[i];
        };
        load_k(0);
        load_qv(0);
        load_rec(0);
        stage_k(0);
        stage_qv(0);
        stage_rec(0);
        const int64_t c1 = NC > 1 ? 1 : 0;
        load_k(c1);
        load_qv(c1);
        load_rec(c1);
        __syncthreads();
        // The loop body is straight-line: every iteration stages and loads (the
        // last chunk's data again near the end, staged as zeros into the buffer
        // nothing reads any more), so the wait before each staging step can let
        // everything loaded after that piece stay in flight.
        for (int64_t c = 0; c < NC; ++c) {
            // chunk c+1 (loaded one iteration ago) is staged piece by piece; each
            // piece's registers are reloaded with chunk c+2 right after
            const int64_t cn = c + 2 < NC ? c + 2 : NC - 1;
            stage_k(c + 1);
            load_k(cn);
            __syncthreads();
            stage_qv(c + 1);
            load_qv(cn);
            __syncthreads();
            stage_rec(c + 1 < NC ? c + 1 : NC - 1);
            load_rec(cn);
            __syncthreads();
        }
        break;
    }
    }
}

template <int C, int DK>
hipError_t launch_rec_t(const PrefillArgs &a, hipStream_t stream)
{
    RecParams rp;
    rp.q = a.q; rp.k = a.k; rp.v = a.v;
    rp.s0 = a.s0; rp.y = a.y; rp.sT = a.sT;
    rp.ws = static_cast<const char *>(a.ws);
    rp.T = a.T; rp.H = a.H; rp.Dv = a.Dv;
    rp.qs = a.q_tok_stride; rp.ks = a.k_tok_stride; rp.vs = a.v_tok_stride;
    rp.nslices = (int)(a.Dv / BV);
    const int64_t bh = a.B * a.H;
    rp.xcd_map = (bh % 8 == 0) ? 1 : 0;
    const int64_t grid = bh * rp.nslices;
    hipLaunchKernelGGL((gdn_recurrence_kernel<C, DK>), dim3((unsigned)grid), dim3(REC_THREADS), 0, stream, rp);
    return hipGetLastError();
}

template <int C>
hipError_t launch_rec_dk(const PrefillArgs &a, hipStream_t s)
{
    switch (a.Dk) {
    case 16: return launch_rec_t<C, 16>(a, s);
    case 32: return launch_rec_t<C, 32>(a, s);
    case 64: return launch_rec_t<C, 64>(a, s);
    case 128: return launch_rec_t<C, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t prefill_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t chunk, bool bf16)
{
    if (!bf16 || chunk <= 0) return 0;
    const size_t rec = prep_record_bytes(chunk);
    return (size_t)B * (size_t)H * (size_t)((T + chunk - 1) / chunk) * rec;
}

hipError_t launch_recurrence(const PrefillArgs &a, hipStream_t stream)
{
    switch (a.chunk) {
    case 16: return launch_rec_dk<16>(a, stream);
    case 32: return launch_rec_dk<32>(a, stream);
    case 64: return launch_rec_dk<64>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
