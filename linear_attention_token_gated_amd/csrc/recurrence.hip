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
//  0-3     K S, Q S of row block w     U_w = sum_k T'_wk R_k    S update (rows 16w, 16(w+4))
//          -> R_w, EG Q S
//  4-7     store Y of chunk c-1        -                       Y = EG Q S + P U
//  8-11    T' of chunk c+1 and chunk c+2 into LDS, spread over the phases;
//          wait for chunk c+1
//
// Three LDS chunk buffers hold K, Q, the V slice and the decay vectors.  The
// staging waves fill them with buffer loads that write LDS directly (no
// registers, no LDS store instructions), two chunks ahead; the only wait is one
// exact count of those loads before the barrier that hands a buffer over.
// T' of the next chunk goes the same way into a ring of two slots.
// Rows past the end of the sequence lie outside the buffer range of the load
// and arrive as zeros.  K and Q rows are stored unpadded with their 16-byte
// granules permuted by row (granule g of row r at position g ^ (r mod G)):
// fragment reads and the column gather of the state update then hit distinct
// LDS banks.  The P fragments of the record go straight into the registers
// of the wavefronts that use them, one chunk ahead.
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
    static constexpr int DEC = PrepRecord<C>::DEC;     // floats of EG, Ed, EGC (+ padding), G
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
    // T' of two chunks (chunk c in slot c % 2), the record's 1 KB blocks as they are
    static constexpr int NTRI = NB * (NB + 1) / 2;
    static constexpr size_t oTr = round1k(oUdl + align16(2 * BV * CPD));
    static constexpr size_t oEq = oTr + (size_t)2 * NTRI * 1024;    // diag(EG) Q S [NB][64 lanes] f32x4
    static constexpr size_t oJunk = round1k(oEq + (size_t)NB * 1024);   // target of padding loads
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
// k-step of KS tokens, lane group g takes the tokens 4g..4g+3 and, for KS = 32,
// 16+4g..16+4g+3 (the order in which the transposing reads below deliver K^T).
// ud_pos gives the storage position of token t, so that the B operand is an
// ordinary contiguous fragment read and four consecutive tokens stay adjacent.
template <int KS> __device__ __forceinline__ int ud_pos(int t) {
    if constexpr (KS == 16) {
        return t;
    } else {
        const int u = t % 32;
        return (t - u) + 8 * ((u & 15) >> 2) + 4 * (u >> 4) + (u & 3);
    }
}

typedef short i16x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4v *lds_i16x4;

// Transposing LDS read of 16-bit elements (gfx950): lane j of each group of 16
// supplies the address of 4 consecutive elements; lane i of the group receives
// element i % 4 of the rows supplied by lanes i/4, 4 + i/4, 8 + i/4, 12 + i/4.
__device__ __forceinline__ bf16x4 read_tr16(const __bf16 *p) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                          (lds_i16x4)(uintptr_t)(uint32_t)(uintptr_t)p));
}

// A operand K^T[r0 + m][tokens of ud_pos order] of one k-step at k0 from the
// row-major (granule-permuted) K chunk: lane j of group g points at row
// k0 + 4g + j/4 (and 16 rows further for KS = 32), columns r0 + 4(j%4)..+3;
// lane m of the group then holds column r0 + m at the four tokens.  Each read
// covers 16 consecutive rows, whose permuted granules fall on distinct banks.
template <int KS, int DK>
__device__ __forceinline__ Frag<__bf16, KS> k_cols_tr(const __bf16 *Ks, int r0, int k0, int lane) {
    const int j = lane & 15, g = lane >> 4;
    const int row = k0 + 4 * g + (j >> 2), col = r0 + 4 * (j & 3);
    Frag<__bf16, KS> f;
    if constexpr (KS == 16) {
        f.v = read_tr16(Ks + kq_idx<DK>(row, col));
    } else {
        const bf16x4 a = read_tr16(Ks + kq_idx<DK>(row, col));
        const bf16x4 b = read_tr16(Ks + kq_idx<DK>(row + 16, col));
        f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
    return f;
}

// Two 16-deep MFMA fragments (k-blocks a and b) as one 32-deep fragment.  Used
// on both operands of a product, the pairing only reorders the terms of the
// k-sum: A[m][a-block k], A[m][b-block k] meet B[a-block k][n], B[b-block k][n].
__device__ __forceinline__ Frag<__bf16, 32> pair16(bf16x4 a, bf16x4 b) {
    Frag<__bf16, 32> f;
    f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return f;
}

// sum over the blocks k < NK2 of A_k B_k (hi/lo pairs, three products each),
// two blocks per 32-deep MFMA and a 16-deep one for an odd last block.  The
// 16-deep products of an odd last block after pairs accumulate apart and are
// added at the end: a 32-deep result is never the accumulator input of a
// 16-deep MFMA.
template <int NK2>
__device__ __forceinline__ void pair_products(const bf16x4 *ah, const bf16x4 *al, const bf16x4 *bh, const bf16x4 *bl,
                                              f32x4 &acc, f32x4 &acc2) {
    using F16 = Frag<__bf16, 16>;
    using F32 = Frag<__bf16, 32>;
    static_for<NK2 / 2>([&](auto i_c) {
        constexpr int k = 2 * decltype(i_c)::value;
        const F32 a = pair16(ah[k], ah[k + 1]), a2 = pair16(al[k], al[k + 1]);
        const F32 b = pair16(bh[k], bh[k + 1]), b2 = pair16(bl[k], bl[k + 1]);
        acc = F32::mma(a, b, acc);
        acc2 = F32::mma(a, b2, acc2);
        acc2 = F32::mma(a2, b, acc2);
    });
    if constexpr (NK2 % 2) {
        F16 a, a2, b, b2;
        a.v = ah[NK2 - 1]; a2.v = al[NK2 - 1]; b.v = bh[NK2 - 1]; b2.v = bl[NK2 - 1];
        if constexpr (NK2 == 1) {
            acc = F16::mma(a, b, acc);
            acc2 = F16::mma(a, b2, acc2);
            acc2 = F16::mma(a2, b, acc2);
        } else {
            f32x4 o = F16::mma(a, b, zero4()), o2 = F16::mma(a, b2, zero4());
            o2 = F16::mma(a2, b, o2);
            acc += o;
            acc2 += o2;
        }
    }
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
    using FDK = Frag<__bf16, L::KS_DK>;
    using FC = Frag<__bf16, L::KS_C>;
    constexpr int KPS = L::KPS, CPU = L::CPU, CPD = L::CPD, NB = L::NB, NSB = L::NSB, MS = L::MS;
    constexpr int KS_DK = L::KS_DK, KS_C = L::KS_C, NK = DK / KS_DK;

    __shared__ __attribute__((aligned(1024))) char smem[L::BYTES];
    // chunk buffer i (chunk c lives in buffer c % NBUF; the loops track the index)
    auto cbuf = [&](int i) { return smem + i * L::CBUF; };
    auto next_buf = [](int i) { return i == NBUF - 1 ? 0 : i + 1; };
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

        lds_barrier();                        // chunk 0 staged, S^T written

        auto iter = [&](auto set_c, int64_t c, int cbi) {
            constexpr int s_ = decltype(set_c)::value;
            const char *cb = cbuf(cbi);
            const __bf16 *Ks = reinterpret_cast<const __bf16 *>(cb + L::cK);
            const float *dec = reinterpret_cast<const float *>(cb + L::cDec);
            // ---- phase 1: R_rb = V_rb - diag(EG) K_rb S, and diag(EG) Q_rb S for
            // the output (the state operand is read once for both)
            if constexpr (has_rb) {
                const __bf16 *Vs = reinterpret_cast<const __bf16 *>(cb + L::cV);
                const __bf16 *Qs = reinterpret_cast<const __bf16 *>(cb + L::cQ);
                const f32x4 eg = *reinterpret_cast<const f32x4 *>(dec + 16 * rb + 4 * lg);
                // V[16 rb + 4 lg + e][ln], e = 0..3, in one transposing read issued
                // ahead of the products (lane j of the group points at row j/4,
                // columns 4 (j%4)..+3)
                const bf16x4 vv = read_tr16(Vs + (16 * rb + 4 * lg + (ln >> 2)) * BV + 4 * (ln & 3));
                // software-pipelined: the fragments of k-step kk + 2 are read while
                // the MFMAs of step kk run (the scheduling barriers keep that order)
                FDK kf[NK], qf[NK], sh[NK], slo[NK];
                auto ld = [&](int kk) {
                    kf[kk] = frag_kq<KS_DK, DK>(Ks, 16 * rb, kk * KS_DK, lane);
                    sh[kk] = frag_rows<__bf16, KS_DK>(STh, KPS, 0, kk * KS_DK, lane);
                    slo[kk] = frag_rows<__bf16, KS_DK>(STl, KPS, 0, kk * KS_DK, lane);
                    qf[kk] = frag_kq<KS_DK, DK>(Qs, 16 * rb, kk * KS_DK, lane);
                };
                ld(0);
                if constexpr (NK > 1) ld(1);
                f32x4 ks_h = zero4(), ks_l = zero4(), qs_h = zero4(), qs_l = zero4();
                static_for<NK>([&](auto kk_c) {
                    constexpr int kk = decltype(kk_c)::value;
                    __builtin_amdgcn_sched_barrier(0);
                    ks_h = FDK::mma(kf[kk], sh[kk], ks_h);
                    ks_l = FDK::mma(kf[kk], slo[kk], ks_l);
                    qs_h = FDK::mma(qf[kk], sh[kk], qs_h);
                    qs_l = FDK::mma(qf[kk], slo[kk], qs_l);
                    if constexpr (kk + 2 < NK) ld(kk + 2);
                });
                __builtin_amdgcn_sched_barrier(0);
                f32x4 rv;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    rv[e] = (float)vv[e] - eg[e] * (ks_h[e] + ks_l[e]);
                bf16x4 hv, lv;
                split4(rv, hv, lv);
                Rh[rb * 64 + lane] = hv;
                Rl[rb * 64 + lane] = lv;
                reinterpret_cast<f32x4 *>(smem + L::oEq)[rb * 64 + lane] = eg * (qs_h + qs_l);
            }
            lds_barrier();

            // ---- phase 2: U_rb = sum_{k <= rb} T'_rb,k R_k.  The K^T operands of
            // the phase-3 update are read first: K of the chunk is unchanged
            // since the iteration began, so their latency overlaps this phase.
            constexpr int NJ = C / KS_C;
            FC ka[MS][NJ];
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int ib = rb + 4 * m;
                if (ib < NSB) {
#pragma unroll
                    for (int jj = 0; jj < NJ; ++jj) ka[m][jj] = k_cols_tr<KS_C, DK>(Ks, 16 * ib, jj * KS_C, lane);
                }
            }
            if constexpr (has_rb) {
                f32x4 u = zero4(), u2 = zero4();
                const int r0 = 16 * rb + 4 * lg;
                const f32x4 ed = *reinterpret_cast<const f32x4 *>(dec + C + r0);
                // T' of this chunk: slot c % 2 (s_ == c % 2)
                const bf16x4 *Tp = reinterpret_cast<const bf16x4 *>(smem + L::oTr + (size_t)s_ * L::NTRI * 1024);
                bf16x4 rh[NT], rl[NT], ah[NT], al[NT];
                static_for<NT>([&](auto k_c) {
                    constexpr int k = decltype(k_c)::value;
                    rh[k] = Rh[k * 64 + lane];
                    rl[k] = Rl[k * 64 + lane];
                    ah[k] = Tp[tri_idx(rb, k) * 128 + lane];
                    al[k] = Tp[tri_idx(rb, k) * 128 + 64 + lane];
                });
                pair_products<NT>(ah, al, rh, rl, u, u2);
                u += u2;
                bf16x4 uh, ul, dh, dl;
                split4(u, uh, ul);
                split4(ed * u, dh, dl);
                *reinterpret_cast<bf16x4 *>(UTh + ln * CPU + r0) = uh;
                *reinterpret_cast<bf16x4 *>(UTl + ln * CPU + r0) = ul;
                // tokens r0..r0+3 stay adjacent in the order of the decayed U^T
                const int pd = ln * CPD + ud_pos<KS_C>(r0);
                *reinterpret_cast<bf16x4 *>(UdTh + pd) = dh;
                *reinterpret_cast<bf16x4 *>(UdTl + pd) = dl;
            }
            lds_barrier();

            // ---- phase 3: S <- EGC S + K^T (diag(Ed) U)
            {
                const float egc = dec[2 * C];
                FC uh[NJ], ul[NJ];
#pragma unroll
                for (int jj = 0; jj < NJ; ++jj) {
                    uh[jj] = frag_rows<__bf16, KS_C>(UdTh, CPD, 0, jj * KS_C, lane);
                    ul[jj] = frag_rows<__bf16, KS_C>(UdTl, CPD, 0, jj * KS_C, lane);
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
            lds_barrier();
        };
        int64_t c = 0;
        int cbi = 0;
        for (; c + 1 < NC; c += 2) {
            iter(S0{}, c, cbi);
            cbi = next_buf(cbi);
            iter(S1{}, c + 1, cbi);
            cbi = next_buf(cbi);
        }
        if (c < NC) iter(S0{}, c, cbi);

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

    // Y-waves: row block rb = 7 - w, compile-time in each copy (the wave of the
    // largest row block of P and of P U shares its SIMD with the S-wave that has
    // the smallest U product).  The output of a chunk is off the critical path
    // of the recurrence: the causal scores P of the row block in phase 2, from
    // the chunk's K and Q rows already in LDS (D = K_cb Q_rb^T, so that lane
    // (ln, lg) holds P[16 rb + ln][16 cb + 4 lg + e], the A operand of P U),
    // decayed by 2^(G_r - G_j) and kept in registers as hi/lo pairs; then P U in
    // phase 3 (U is complete; diag(EG) Q S comes from the S-wave of the row
    // block), and the stores of the rows in phase 1 of the next iteration.
    auto y_wave = [&](auto rb_c) {
        constexpr int rb = decltype(rb_c)::value;
        constexpr bool has_rb = rb < NB;
        constexpr int NP = has_rb ? rb + 1 : 1;     // P blocks of this row block
        bf16x4 pfh[NP], pfl[NP];                    // P fragments of this row block
        auto form_p = [&](int cbi) {
            if constexpr (has_rb) {
                const char *cb = cbuf(cbi);
                const __bf16 *Ks = reinterpret_cast<const __bf16 *>(cb + L::cK);
                const __bf16 *Qs = reinterpret_cast<const __bf16 *>(cb + L::cQ);
                const float *Gv = reinterpret_cast<const float *>(cb + L::cDec) + Rec::DEC_G;
                FDK qf[NK];
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) qf[kk] = frag_kq<KS_DK, DK>(Qs, 16 * rb, kk * KS_DK, lane);
                const int r = 16 * rb + ln;
                const float Gr = Gv[r], Grb = Gv[16 * rb];
                const float Ear = __builtin_amdgcn_exp2f(Gr - Grb);
                static_for<NP>([&](auto cb_c) {
                    constexpr int cbk = decltype(cb_c)::value;
                    f32x4 acc = zero4();
#pragma unroll
                    for (int kk = 0; kk < NK; ++kk)
                        acc = FDK::mma(frag_kq<KS_DK, DK>(Ks, 16 * cbk, kk * KS_DK, lane), qf[kk], acc);
                    const int j0 = 16 * cbk + 4 * lg;
                    const f32x4 Gj = *reinterpret_cast<const f32x4 *>(Gv + j0);
                    f32x4 val;
                    if constexpr (cbk == rb) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            val[e] = r >= j0 + e ? __builtin_amdgcn_exp2f(Gr - Gj[e]) * acc[e] : 0.f;
                    } else {
                        // r > j: 2^(G_r - G_j) = 2^(G_r - G_{16 rb}) 2^(G_{16 rb} - G_j), both <= 1
                        f32x4 eb;
#pragma unroll
                        for (int e = 0; e < 4; ++e) eb[e] = __builtin_amdgcn_exp2f(Grb - Gj[e]);
                        val = acc * eb * Ear;
                    }
                    split4(val, pfh[cbk], pfl[cbk]);
                });
            }
        };
        f32x4 yv = zero4();                         // output rows waiting to be stored
        auto store_y = [&](int64_t c) {
            if constexpr (has_rb) {
                const int64_t c0 = c * C;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t t = c0 + 16 * rb + 4 * lg + e;
                    if (t < T) p.y[((b * T + t) * H + h) * Dv + n0 + ln] = yv[e];
                }
            }
        };
        lds_barrier();

        int cbi = 0;
        for (int64_t c = 0; c < NC; ++c) {
            // ---- phase 1: rows of chunk c - 1
            if (c > 0) store_y(c - 1);
            lds_barrier();
            // ---- phase 2: P of chunk c
            form_p(cbi);
            lds_barrier();
            // ---- phase 3: Y = diag(EG) Q S + P U
            if constexpr (has_rb) {
                f32x4 acc = reinterpret_cast<const f32x4 *>(smem + L::oEq)[rb * 64 + lane], acc2 = zero4();
                bf16x4 uh[NP], ul[NP];
                static_for<NP>([&](auto j_c) {
                    constexpr int jb = decltype(j_c)::value;
                    uh[jb] = *reinterpret_cast<const bf16x4 *>(UTh + ln * CPU + 16 * jb + 4 * lg);
                    ul[jb] = *reinterpret_cast<const bf16x4 *>(UTl + ln * CPU + 16 * jb + 4 * lg);
                });
                pair_products<NP>(pfh, pfl, uh, ul, acc, acc2);
                yv = acc + acc2;
                // keep the sum next to its MFMAs: an MFMA result read right after
                // a branch can miss its wait states
                asm volatile("" : "+v"(yv));
            }
            lds_barrier();
            cbi = next_buf(cbi);
        }
        if (NC > 0) store_y(NC - 1);
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
        // T' of chunk c into slot c % 2: record blocks t = lw, lw + 4, ...
        constexpr int NTW = (L::NTRI - lw + 3) / 4;
        auto stage_t = [&](int64_t c, int64_t slot) {
            const void *br = recs + c * (int64_t)Rec::BYTES + Rec::oT;
            char *dst = smem + L::oTr + (size_t)(slot & 1) * L::NTRI * 1024;
            static_for<NTW>([&](auto i_c) {
                constexpr int t = lw + 4 * decltype(i_c)::value;
                load_to_lds(br, (uint32_t)(L::NTRI * 1024), (uint32_t)(t * 1024 + lane * 16), dst + t * 1024);
            });
        };
        // loads [I0, I1) of chunk c into chunk buffer cb_idx
        auto stage = [&](int64_t c, int cb_idx, auto i0_c, auto i1_c) {
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
        // T' of chunk 0 and chunks 0 and 1 in flight; all but chunk 1 complete
        // before the first barrier
        stage_t(0, 0);
        stage(0, 0, Z{}, PJ{});
        stage(clampc(1), 1, Z{}, PJ{});
        wait_vmcnt<JW>();
        __builtin_amdgcn_s_barrier();
        int nbi = 2 % NBUF;                         // buffer of chunk c + 2
        for (int64_t c = 0; c < NC; ++c) {
            // chunk c+2 two iterations ahead into buffer (c+2) % 3, whose last reader
            // was iteration c-1 (past the end, the last chunk again: that buffer is
            // never read).  The loads are spread over the three phases so that
            // their issue overlaps the computation.
            // T' of chunk c+1 first, into slot (c+1) % 2, last read in phase 2 of
            // iteration c-1
            stage_t(clampc(c + 1), c + 1);
            const int64_t cn = clampc(c + 2);
            stage(cn, nbi, Z{}, P1{});
            __builtin_amdgcn_s_barrier();
            stage(cn, nbi, P1{}, P2{});
            __builtin_amdgcn_s_barrier();
            stage(cn, nbi, P2{}, PJ{});
            nbi = next_buf(nbi);
            // T' of chunk c+1 and chunk c+1 must be complete before the barrier
            // that starts iteration c+1; chunk c+2 (the last JW loads) may still
            // be in flight
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
    case 4: y_wave(I3{}); break;
    case 5: y_wave(I2{}); break;
    case 6: y_wave(I1{}); break;
    case 7: y_wave(I0{}); break;
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

size_t prefill_bf16_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t chunk)
{
    if (chunk <= 0) return 0;
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
