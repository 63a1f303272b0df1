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
//  waves   phase 1                     phase 2                 phase 3
//  0-3     K S of row block w -> R_w   U_w = sum_k T'_wk R_k    S update (rows 16w, 16(w+4))
//  4-7     Y of chunk c-1: + P U       EG Q S of row block w-4  -
//  8-11    copy chunk c+2 into LDS, a third in each phase; wait for chunk c+1
//
// Three LDS chunk buffers hold K, Q, the V slice and the decay vectors.  The
// staging waves fill them with buffer loads that write LDS directly (no
// registers, no LDS store instructions), two chunks ahead; the only wait is one
// exact count of those loads before the barrier that hands a buffer over.
// Rows past the end of the sequence lie outside the buffer range of the load
// and arrive as zeros.  K and Q rows are stored unpadded with their 16-byte
// granules permuted by row (granule g of row r at position g ^ (r mod G)):
// fragment reads and the column gather of the state update then hit distinct
// LDS banks.  The T' and P fragments of the record go straight into the
// registers of the wavefronts that use them, one chunk ahead.
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
constexpr int NBUF = 3;            // LDS chunk buffers

typedef __attribute__((address_space(3))) void *lds_ptr;
__device__ __forceinline__ lds_ptr as_lds(const void *p) { return (lds_ptr)(uintptr_t)(uint32_t)(uintptr_t)p; }
// fourth word of a raw (unswizzled, byte-addressed) buffer resource: 32-bit data format
constexpr int RAW_RSRC_W3 = 0x00020000;
constexpr uint32_t OOB_OFFSET = 0x7FFFFFF0u;   // beyond every buffer range used here

// One 64-lane load of 16 bytes per lane written straight into LDS at dst +
// 16 * lane: the source is byte offset voff of a raw buffer of nrec bytes at
// base; lanes whose 16 bytes lie outside it read zeros.
__device__ __forceinline__ void load_to_lds(const void *base, uint32_t nrec, uint32_t voff, void *dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)nrec, RAW_RSRC_W3), as_lds(dst), 16,
        voff, 0, 0, 0);
}

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

constexpr size_t round1k(size_t x) { return (x + 1023) & ~size_t(1023); }

template <int C, int DK> struct RecLay {
    static constexpr int NB = C / 16;
    static constexpr int NSB = DK / 16;
    static constexpr int MS = (NSB + 3) / 4;           // state row blocks per S-wave
    static constexpr int KS_DK = DK % 32 == 0 ? 32 : 16;
    static constexpr int KS_C = C % 32 == 0 ? 32 : 16;
    static constexpr int G = DK / 8;                   // 16-byte granules per K/Q row
    static constexpr int KPS = frag_pitch<KS_DK>(DK);  // S^T rows (bf16)
    static constexpr int CPU = C + 4;                  // U^T rows: 64-bit stores and reads
    static constexpr int CPD = frag_pitch<KS_C>(C);    // e^{G_C-G} U^T rows
    static constexpr int DEC = 2 * C + 16;             // floats of EG, Ed, EGC (+ padding)
    // one chunk buffer; every region a whole number of 1 KB blocks (one wave's load)
    static constexpr size_t cK = 0;                    // [C][DK] bf16, granules permuted
    static constexpr size_t cQ = cK + round1k(2 * C * DK);
    static constexpr size_t cV = cQ + round1k(2 * C * DK);     // [C][16] bf16
    static constexpr size_t cDec = cV + round1k(2 * C * BV);
    static constexpr size_t CBUF = cDec + round1k(4 * DEC);
    // shared by the phases of one chunk
    static constexpr size_t oSTh = NBUF * CBUF;
    static constexpr size_t oSTl = oSTh + align16(2 * BV * KPS);
    static constexpr size_t oRh = oSTl + align16(2 * BV * KPS);  // R blocks [NB][64 lanes] bf16x4
    static constexpr size_t oRl = oRh + (size_t)NB * 512;
    static constexpr size_t oUh = oRl + (size_t)NB * 512;
    static constexpr size_t oUl = oUh + align16(2 * BV * CPU);
    static constexpr size_t oUdh = oUl + align16(2 * BV * CPU);
    static constexpr size_t oUdl = oUdh + align16(2 * BV * CPD);
    static constexpr size_t oJunk = round1k(oUdl + align16(2 * BV * CPD));   // target of padding loads
    static constexpr size_t BYTES = oJunk + 1024;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    // staging loads per chunk (one 64-lane, 16-byte-per-lane load each)
    static constexpr int NIK = (C * G + 63) / 64;      // per K or Q array
    static constexpr int NIV = (2 * C + 63) / 64;      // V slice: two granules per row
    static constexpr int NID = (DEC * 4 / 16 + 63) / 64;
    static constexpr int NJOB = 2 * NIK + NIV + NID;
    static constexpr int JW = (NJOB + 3) / 4;          // per staging wavefront
    static_assert(JW <= 31, "vector-memory counter range for two chunks in flight");
};

__device__ __forceinline__ int tri_idx(int i, int k) { return i * (i + 1) / 2 + k; }

// Position of element (row, col) of a K or Q chunk in LDS: 16-byte granule
// col/8 of row r sits at granule position (col/8) ^ (r mod G).
template <int DK> __device__ __forceinline__ int kq_idx(int row, int col) {
    constexpr int G = DK / 8;
    return row * DK + ((((col >> 3) ^ row) & (G - 1)) << 3) + (col & 7);
}

// MFMA fragment of rows r0.. of a K or Q chunk (see frag_rows)
template <int KS, int DK>
__device__ __forceinline__ Frag<__bf16, KS> frag_kq(const __bf16 *base, int r0, int k0, int lane) {
    Frag<__bf16, KS> f;
    f.load(base + kq_idx<DK>(r0 + (lane & 15), k0 + (lane >> 4) * (KS / 4)));
    return f;
}

// Token order of the decayed U^T rows used by the state update.  Within each
// k-step of KS tokens, lane group g (KS/4 values per lane) takes the tokens
// 2g + 8(e/2) + (e%2), e = 0..KS/4-1: adjacent pairs, 8 tokens apart, so the
// K column gather reads rows two tokens apart in the four lane groups.
// ud_pos gives the storage position of token t; the B operand is then an
// ordinary contiguous fragment read.
template <int KS> __device__ __forceinline__ int ud_pos(int t) {
    constexpr int E = KS / 4;
    const int u = t % KS;
    return (t - u) + ((u & 7) >> 1) * E + (u >> 3) * 2 + (u & 1);
}

// A operand K^T[r0 + ln][tokens of ud_pos order] of one k-step at k0.  The
// token of element e is t = k0 + 2g + 8(e/2) + (e%2); k0 is a multiple of the
// granule count G, and 2g + (e%2) < 8, so t mod G = (2g + e%2) ^ (8(e/2) mod G):
// the permuted granule takes two lane-dependent values per e%2, and the rest
// of the address is a compile-time row offset.
template <int KS, int DK>
__device__ __forceinline__ Frag<__bf16, KS> k_cols_paired(const __bf16 *Ks, int r0, int k0, int lane) {
    constexpr int G = DK / 8;
    Frag<__bf16, KS> f;
    const int col = r0 + (lane & 15), g2 = 2 * (lane >> 4);
    const int base = g2 * DK + (col & 7);
    int off[2][2];                                   // [e % 2][(e / 2) % 2]
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int x = (col >> 3) ^ ((g2 + i) & (G - 1));
        off[i][0] = base + i * DK + x * 8;
        off[i][1] = base + i * DK + (x ^ (8 & (G - 1))) * 8;
    }
#pragma unroll
    for (int e = 0; e < KS / 4; ++e) f.set_raw(e, Ks[(k0 + 8 * (e >> 1)) * DK + off[e & 1][(e >> 1) & 1]]);
    return f;
}

// s_waitcnt vmcnt(N) leaving the other counters alone
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int C, int DK>
__global__ __launch_bounds__(REC_THREADS, 1) void gdn_recurrence_kernel(RecParams p)
{
    using L = RecLay<C, DK>;
    using Rec = PrepRecord<C>;
    using F16 = Frag<__bf16, 16>;
    using FDK = Frag<__bf16, L::KS_DK>;
    using FC = Frag<__bf16, L::KS_C>;
    constexpr int KPS = L::KPS, CPU = L::CPU, CPD = L::CPD, NB = L::NB, NSB = L::NSB, MS = L::MS;
    constexpr int KS_DK = L::KS_DK, KS_C = L::KS_C, NK = DK / KS_DK;

    __shared__ __attribute__((aligned(1024))) char smem[L::BYTES];
    auto cbuf = [&](int64_t c) { return smem + (c % NBUF) * L::CBUF; };
    __bf16 *STh = reinterpret_cast<__bf16 *>(smem + L::oSTh);
    __bf16 *STl = reinterpret_cast<__bf16 *>(smem + L::oSTl);
    bf16x4 *Rh = reinterpret_cast<bf16x4 *>(smem + L::oRh);
    bf16x4 *Rl = reinterpret_cast<bf16x4 *>(smem + L::oRl);
    __bf16 *UTh = reinterpret_cast<__bf16 *>(smem + L::oUh);
    __bf16 *UTl = reinterpret_cast<__bf16 *>(smem + L::oUl);
    __bf16 *UdTh = reinterpret_cast<__bf16 *>(smem + L::oUdh);
    __bf16 *UdTl = reinterpret_cast<__bf16 *>(smem + L::oUdl);

    const int lane = lane_id();
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
    auto clampc = [&](int64_t c) { return c < NC ? c : NC - 1; };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;

    // S-waves: row block rb = w; state rows ib = w + 4m.  The row block is a
    // compile-time constant in each copy, so the block sums are fully unrolled.
    auto s_wave = [&](auto rb_c) {
        constexpr int rb = decltype(rb_c)::value;
        constexpr bool has_rb = rb < NB;
        constexpr int NT = has_rb ? rb + 1 : 1;     // T' blocks of this row block
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
                    *reinterpret_cast<bf16x4 *>(STh + ln * KPS + 16 * ib + 4 * lg) = hv;
                    *reinterpret_cast<bf16x4 *>(STl + ln * KPS + 16 * ib + 4 * lg) = lv;
                }
            }
        };
        write_state_operand();

        // T' fragments of this row block, two register sets (chunk j in set j % 2)
        bf16x4 tfh[2][NT], tfl[2][NT];
        auto load_t = [&](auto set_c, int64_t c) {
            constexpr int s_ = decltype(set_c)::value;
            if constexpr (has_rb) {
                const bf16x4 *tf = reinterpret_cast<const bf16x4 *>(recs + c * (int64_t)Rec::BYTES + Rec::oT);
#pragma unroll
                for (int k = 0; k <= rb; ++k) {
                    tfh[s_][k] = tf[tri_idx(rb, k) * 128 + lane];
                    tfl[s_][k] = tf[tri_idx(rb, k) * 128 + 64 + lane];
                }
            }
        };
        load_t(S0{}, 0);
        __syncthreads();                        // chunk 0 staged, S^T written

        auto iter = [&](auto set_c, int64_t c) {
            constexpr int s_ = decltype(set_c)::value;
            const char *cb = cbuf(c);
            const __bf16 *Ks = reinterpret_cast<const __bf16 *>(cb + L::cK);
            const float *dec = reinterpret_cast<const float *>(cb + L::cDec);
            // ---- phase 1: R_rb = V_rb - diag(EG) K_rb S
            if constexpr (has_rb) {
                const __bf16 *Vs = reinterpret_cast<const __bf16 *>(cb + L::cV);
                const f32x4 eg = *reinterpret_cast<const f32x4 *>(dec + 16 * rb + 4 * lg);
                FDK kf[NK], sh[NK], slo[NK];
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    kf[kk] = frag_kq<KS_DK, DK>(Ks, 16 * rb, kk * KS_DK, lane);
                    sh[kk] = frag_rows<__bf16, KS_DK>(STh, KPS, 0, kk * KS_DK, lane);
                    slo[kk] = frag_rows<__bf16, KS_DK>(STl, KPS, 0, kk * KS_DK, lane);
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
            // the next chunk's T' (the last chunk's again at the end: no branch)
            load_t(std::integral_constant<int, 1 - s_>{}, clampc(c + 1));
            __syncthreads();

            // ---- phase 2: U_rb = sum_{k <= rb} T'_rb,k R_k
            if constexpr (has_rb) {
                f32x4 u = zero4(), u2 = zero4();
                const int r0 = 16 * rb + 4 * lg;
                const f32x4 ed = *reinterpret_cast<const f32x4 *>(dec + C + r0);
                F16 rh[NT], rl[NT];
                static_for<NT>([&](auto k_c) {
                    constexpr int k = decltype(k_c)::value;
                    rh[k].v = Rh[k * 64 + lane];
                    rl[k].v = Rl[k * 64 + lane];
                });
                static_for<NT>([&](auto k_c) {
                    constexpr int k = decltype(k_c)::value;
                    F16 ah, al;
                    ah.v = tfh[s_][k];
                    al.v = tfl[s_][k];
                    u = F16::mma(ah, rh[k], u);
                    u2 = F16::mma(ah, rl[k], u2);
                    u2 = F16::mma(al, rh[k], u2);
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
                        for (int jj = 0; jj < NJ; ++jj) ka[m][jj] = k_cols_paired<KS_C, DK>(Ks, 16 * ib, jj * KS_C, lane);
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
        };
        int64_t c = 0;
        for (; c + 1 < NC; c += 2) {
            iter(S0{}, c);
            iter(S1{}, c + 1);
        }
        if (c < NC) iter(S0{}, c);

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

    // Y-waves: row block rb = w - 4, compile-time in each copy.  The output
    // of a chunk is off the critical path of the recurrence, so it is spread
    // over the phases the S-waves leave light: Q S of chunk c in phase 2 of
    // iteration c (the state operand still holds the chunk's initial state),
    // and P U of chunk c with the store of its rows in phase 1 of iteration
    // c + 1 (U of chunk c stays in LDS until phase 2 of that iteration).
    auto y_wave = [&](auto rb_c) {
        constexpr int rb = decltype(rb_c)::value;
        constexpr bool has_rb = rb < NB;
        constexpr int NP = has_rb ? rb + 1 : 1;     // P blocks of this row block
        // P fragments of this row block for the chunk whose output is pending
        bf16x4 pfh[NP], pfl[NP];
        auto load_p = [&](int64_t c) {
            if constexpr (has_rb) {
                const bf16x4 *pf = reinterpret_cast<const bf16x4 *>(recs + c * (int64_t)Rec::BYTES + Rec::oP);
#pragma unroll
                for (int k = 0; k <= rb; ++k) {
                    pfh[k] = pf[tri_idx(rb, k) * 128 + lane];
                    pfl[k] = pf[tri_idx(rb, k) * 128 + 64 + lane];
                }
            }
        };
        f32x4 eqs = zero4();                        // diag(EG) Q S of the pending chunk
        // Y rows of chunk c: diag(EG) Q S + P U, U read from LDS
        auto finish = [&](int64_t c) {
            if constexpr (has_rb) {
                f32x4 acc = eqs, acc2 = zero4();
                F16 uh[NP], ul[NP];
                static_for<NP>([&](auto j_c) {
                    constexpr int jb = decltype(j_c)::value;
                    uh[jb] = frag_rows<__bf16, 16>(UTh, CPU, 0, 16 * jb, lane);
                    ul[jb] = frag_rows<__bf16, 16>(UTl, CPU, 0, 16 * jb, lane);
                });
                static_for<NP>([&](auto j_c) {
                    constexpr int jb = decltype(j_c)::value;
                    F16 ah, al;
                    ah.v = pfh[jb];
                    al.v = pfl[jb];
                    acc = F16::mma(ah, uh[jb], acc);
                    acc2 = F16::mma(al, uh[jb], acc2);
                    acc2 = F16::mma(ah, ul[jb], acc2);
                });
                f32x4 yv = acc + acc2;
                // keep the sum next to its MFMAs: an MFMA result read right after
                // a branch can miss its wait states
                asm volatile("" : "+v"(yv));
                const int64_t c0 = c * C;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t t = c0 + 16 * rb + 4 * lg + e;
                    if (t < T) p.y[((b * T + t) * H + h) * Dv + n0 + ln] = yv[e];
                }
            }
        };
        load_p(0);
        __syncthreads();

        for (int64_t c = 0; c < NC; ++c) {
            const char *cb = cbuf(c);
            // ---- phase 1: output of chunk c - 1, then the P fragments of chunk c
            if (c > 0) finish(c - 1);
            if (c > 0) load_p(c);
            __syncthreads();
            // ---- phase 2: diag(EG) Q S of this row block (state at the chunk's start)
            if constexpr (has_rb) {
                const __bf16 *Qs = reinterpret_cast<const __bf16 *>(cb + L::cQ);
                const float *dec = reinterpret_cast<const float *>(cb + L::cDec);
                FDK qf[NK], sh[NK], slo[NK];
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    qf[kk] = frag_kq<KS_DK, DK>(Qs, 16 * rb, kk * KS_DK, lane);
                    sh[kk] = frag_rows<__bf16, KS_DK>(STh, KPS, 0, kk * KS_DK, lane);
                    slo[kk] = frag_rows<__bf16, KS_DK>(STl, KPS, 0, kk * KS_DK, lane);
                }
                const f32x4 eg = *reinterpret_cast<const f32x4 *>(dec + 16 * rb + 4 * lg);
                f32x4 qh = zero4(), ql = zero4();
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    qh = FDK::mma(qf[kk], sh[kk], qh);
                    ql = FDK::mma(qf[kk], slo[kk], ql);
                }
                eqs = eg * (qh + ql);
                asm volatile("" : "+v"(eqs));
            }
            __syncthreads();
            // ---- phase 3: the S-waves update the state
            __syncthreads();
        }
        // U of the last chunk was written before the last phase 2 barrier
        if (NC > 0) finish(NC - 1);
    };

    // Staging waves: JW loads of 64 lanes x 16 bytes per chunk each, written
    // straight into the chunk buffer.  Load j of the chunk (j = lw + 4 i) is the
    // j-th 1 KB block of K, Q, V, the decay vectors, or a padding load into a
    // scratch block when the count does not divide evenly.  The wave index is a
    // compile-time constant in each copy, so the source array and the LDS block
    // of every load are too.
    auto l_wave = [&](auto lw_c) {
        constexpr int lw = decltype(lw_c)::value;
        const __bf16 *qg = static_cast<const __bf16 *>(p.q);
        const __bf16 *kg = static_cast<const __bf16 *>(p.k);
        const __bf16 *vg = static_cast<const __bf16 *>(p.v);
        constexpr int G = L::G, NIK = L::NIK, NIV = L::NIV, JW = L::JW;
        // 0 K, 1 Q, 2 V, 3 decay vectors, 4 padding
        auto kind_of = [](int i) constexpr {
            const int j = lw + 4 * i;
            return j < 2 * NIK ? j / NIK : j < 2 * NIK + NIV ? 2 : j < 2 * NIK + NIV + L::NID ? 3 : 4;
        };
        // byte offset of the 1 KB block of load i in a chunk buffer
        auto block_of = [](int i) constexpr -> uint32_t {
            const int j = lw + 4 * i;
            return j < 2 * NIK ? (uint32_t)((j < NIK ? L::cK : L::cQ) + (size_t)(j % NIK) * 1024)
                 : j < 2 * NIK + NIV ? (uint32_t)(L::cV + (size_t)(j - 2 * NIK) * 1024)
                 : j < 2 * NIK + NIV + L::NID ? (uint32_t)(L::cDec + (size_t)(j - 2 * NIK - NIV) * 1024)
                 : 0u;
        };
        // per-lane byte offsets of each load (chunk independent)
        uint32_t voff[JW];
        static_for<JW>([&](auto i_c) {
            constexpr int i = decltype(i_c)::value;
            constexpr int kd = kind_of(i);
            constexpr int j = lw + 4 * i;
            if constexpr (kd <= 1) {
                const int q = (j % NIK) * 64 + lane, row = q / G, phys = q % G, logi = phys ^ (row & (G - 1));
                const int64_t st = kd ? p.qs : p.ks;
                voff[i] = q < C * G ? (uint32_t)(row * st * 2 + logi * 16) : OOB_OFFSET;
            } else if constexpr (kd == 2) {
                const int q = (j - 2 * NIK) * 64 + lane, row = q >> 1;
                voff[i] = q < 2 * C ? (uint32_t)(row * p.vs * 2 + (q & 1) * 16) : OOB_OFFSET;
            } else if constexpr (kd == 3) {
                const int q = (j - 2 * NIK - NIV) * 64 + lane;
                voff[i] = q * 16 < L::DEC * 4 ? (uint32_t)(Rec::oDec + q * 16) : OOB_OFFSET;
            } else {
                voff[i] = OOB_OFFSET;
            }
        });
        // loads [I0, I1) of chunk c into chunk buffer cb_idx % 3
        auto stage = [&](int64_t c, int64_t cb_idx, auto i0_c, auto i1_c) {
            constexpr int I0 = decltype(i0_c)::value, I1 = decltype(i1_c)::value;
            const int64_t c0 = c * C;
            const int64_t valid = T - c0 < C ? T - c0 : C;                 // rows of this chunk
            const int64_t tok = b * T + c0;
            const uint32_t nk = (uint32_t)((valid - 1) * p.ks * 2 + DK * 2);
            const uint32_t nq = (uint32_t)((valid - 1) * p.qs * 2 + DK * 2);
            const uint32_t nv = (uint32_t)((valid - 1) * p.vs * 2 + BV * 2);
            const void *bk = kg + tok * p.ks + h * DK;
            const void *bq = qg + tok * p.qs + h * DK;
            const void *bv = vg + tok * p.vs + h * Dv + n0;
            const void *br = recs + c * (int64_t)Rec::BYTES;
            char *nb = cbuf(cb_idx);
            static_for<JW>([&](auto i_c) {
                constexpr int i = decltype(i_c)::value;
                constexpr int kd = kind_of(i);
                if constexpr (i < I0 || i >= I1) {
                } else if constexpr (kd == 0) load_to_lds(bk, nk, voff[i], nb + block_of(i));
                else if constexpr (kd == 1) load_to_lds(bq, nq, voff[i], nb + block_of(i));
                else if constexpr (kd == 2) load_to_lds(bv, nv, voff[i], nb + block_of(i));
                else if constexpr (kd == 3) load_to_lds(br, (uint32_t)Rec::BYTES, voff[i], nb + block_of(i));
                else load_to_lds(br, (uint32_t)Rec::BYTES, voff[i], smem + L::oJunk);
            });
        };
        // The barriers of this wave carry no memory fence: a workgroup fence
        // would wait for every load in flight, the prefetch included.  The
        // explicit counter waits order the LDS writes of the loads instead.
        using Z = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, JW / 3>;
        using P2 = std::integral_constant<int, 2 * JW / 3>;
        using PJ = std::integral_constant<int, JW>;
        // chunks 0 and 1 in flight; chunk 0 complete before the first barrier
        stage(0, 0, Z{}, PJ{});
        stage(clampc(1), 1, Z{}, PJ{});
        wait_vmcnt<JW>();
        __builtin_amdgcn_s_barrier();
        for (int64_t c = 0; c < NC; ++c) {
            // chunk c+2 two iterations ahead into buffer (c+2) % 3, whose last reader
            // was iteration c-1 (past the end, the last chunk again: that buffer is
            // never read).  The loads are spread over the three phases so that
            // their issue overlaps the computation.
            const int64_t cn = clampc(c + 2);
            stage(cn, c + 2, Z{}, P1{});
            __builtin_amdgcn_s_barrier();
            stage(cn, c + 2, P1{}, P2{});
            __builtin_amdgcn_s_barrier();
            stage(cn, c + 2, P2{}, PJ{});
            // chunk c+1 must be complete before the barrier that starts iteration
            // c+1; chunk c+2 may still be in flight
            wait_vmcnt<JW>();
            __builtin_amdgcn_s_barrier();
        }
        // no LDS write may land after the workgroup ends
        wait_vmcnt<0>();
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
    case 8: l_wave(I0{}); break;
    case 9: l_wave(I1{}); break;
    case 10: l_wave(I2{}); break;
    default: l_wave(I3{}); break;
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
