// prefill_fused.hip -- the chunked prefill of the gated delta rule for bf16
// inputs in a single kernel: every chunk quantity is formed on chip, q, k and v
// are read from HBM once, and y and the final state are written once.
//
// Source: "On the Design of Qwen3.8-Next Architecture", picx.dev summary,
// "Theoretical foundations", eqs (1)-(4).  For one chunk of C tokens entering
// with state S (G_r = sum_{i<=r} log2 alpha_i within the chunk):
//
//   A  = strict_lower[ beta_r 2^(G_r - G_j) (k_r . k_j) ],  T = (I + A)^-1
//   T' = T diag(beta),  P = lower_incl[ 2^(G_r - G_j) (q_r . k_j) ]
//   R  = V - diag(2^G) K S,   U = T' R          (u_r = beta_r e_r of eqs (2)-(3))
//   Y  = diag(2^G) Q S + P U                     (eq (4))
//   S' = 2^(G_C) S + K^T diag(2^(G_C - G)) U      (eqs (1), (3))
//
// Columns of S, V, U, Y are independent, so one workgroup carries one
// 16-column slice of S of one (b, h) through every chunk; the slices of a head
// are placed on one XCD, whose L2 then serves the eight reads of K and Q.
// Eight wavefronts, two barriers (X, Y) per chunk c:
//
//   chain waves 0-3 (wave w owns state rows 16 (w + 4m))
//     X-phase: K_w S (S as one bf16), Q_w S (S as bf16 hi + lo) for token block
//              w; R_w = V_w - 2^G K_w S  -> LDS
//     Y-phase: U = T' R for all token blocks (each chain wave, from LDS); its
//              own state rows S <- 2^G_C S + K^T (2^(G_C-G) U); the S operand,
//              U_w and 2^G Q_w S -> LDS
//   preparation waves 4-7 (wave p = w - 4; chunk c + 1; outputs of chunk c - 1)
//     X-phase: Y_p of chunk c-1 = 2^G Q_p S + P_p U (P_p kept in registers)
//              -> y; decay prefix of chunk c+1 (fp64); Gram blocks (P row p,
//              A_pp and some blocks of A below the diagonal); T_pp =
//              (I + A_pp)^-1 by forward substitution -> LDS
//     Y-phase: column p of T from the blocks of all waves,
//              T_mp = -T_mm sum_{j=p}^{m-1} A_mj T_jp; T' column p -> LDS
//
// The chain waves also stage the inputs: the q, k, v rows and gates of token
// block w of chunk c + 2 are loaded into registers at the start of iteration c
// and written to LDS at its end.  Rows past the end of the sequence are zeros
// with alpha = 1 and beta = 0 (identity tokens).
//
// Precision: q, k, v are exact bf16 operands and every product accumulates in
// fp32.  Operands computed in fp32 (S in Q S, R, U, T, T', P, the level
// products of T) enter as bf16 pairs hi + lo, each product summing hi*hi +
// hi*lo + lo*hi.  S enters K S as a single bf16 (the state recurrence damps
// that rounding: 2e-3 of the bound-relevant max|err|/RMS at T = 32768 in a CPU
// simulation of these rounding points, against 1e-2 for Q S).  Decay
// prefixes are summed in fp64 so that 2^(G_r - G_j) keeps its precision after
// decays near 0.
#include "common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int FT = 512;   // 8 wavefronts

struct FusedParams {
    const __bf16 *q, *k, *v;
    const float *alpha, *beta, *s0;
    float *y, *sT;
    int64_t T, H, Dv;
    int64_t qs, ks, vs;      // token strides (elements)
    int nslices;             // Dv / 16
    int xcd_map;             // 1: the slices of a head on one XCD
};

template <int C, int DK> struct FL {
    static constexpr int NB = C / 16, NSB = DK / 16, MS = (NSB + 3) / 4;
    static constexpr int NTRI = NB * (NB + 1) / 2, NOFF = NB * (NB - 1) / 2;
    static constexpr int KSD = DK % 32 == 0 ? 32 : 16, NK = DK / KSD;   // k-steps over Dk
    static constexpr int KSC = C % 32 == 0 ? 32 : 16, NJ = C / KSC;     // k-steps over the chunk
    static constexpr int KPS = frag_pitch<KSD>(DK);                     // S^T row pitch (bf16)
    static constexpr size_t KQB = (size_t)2 * C * DK;                   // one K or Q chunk
    static constexpr size_t VB = (size_t)2 * C * BV;                    // one V slice
    static constexpr size_t ABB = (size_t)8 * C;                        // alpha[C] | beta[C]
    // decay table of one chunk: G[C] (fp64) | 2^G[C] | 2^(G_C - G)[C] | HC[C] |
    // FR[NB - 1][C] | 2^G_C, with HC and FR the column and row factors of the
    // decay ratios of the blocks below the diagonal
    static constexpr size_t DT_EG = 8 * C, DT_ED = 12 * C, DT_HC = 16 * C, DT_FR = 20 * C;
    static constexpr size_t DT_EGC = DT_FR + (size_t)4 * (NB - 1) * C;
    static constexpr size_t DTB = align16(DT_EGC + 16);
    static constexpr size_t oK = 0;                                     // [3] K chunks
    static constexpr size_t oQ = oK + 3 * KQB;                          // [2] Q chunks
    static constexpr size_t oV = oQ + 2 * KQB;                          // [2] V slices [C][16]
    static constexpr size_t oAB = oV + 2 * VB;                          // [4] gates
    static constexpr size_t oSTh = align16(oAB + 4 * ABB);              // S^T operand, hi
    static constexpr size_t oSTl = oSTh + align16(2 * BV * KPS);        // S^T operand, lo
    static constexpr size_t oR = oSTl + align16(2 * BV * KPS);          // R [NB][hi|lo][64] bf16x4
    static constexpr size_t oTP = oR + (size_t)NB * 1024;               // [2][NTRI] T'^T blocks, hi|lo
    static constexpr size_t TPB = (size_t)NTRI * 1024;
    static constexpr size_t oDT = oTP + 2 * TPB;                        // [4] decay tables
    static constexpr size_t oXT = oDT + 4 * DTB;                        // [NB] T_mm row-major, hi|lo
    static constexpr size_t oXA = oXT + (size_t)NB * 1024;              // [NOFF] A_mj row-major, hi|lo
    static constexpr size_t oUQ = oXA + (size_t)(NOFF > 0 ? NOFF : 1) * 1024;   // U_w [NB][hi|lo][64] bf16x4
    static constexpr size_t oQS = oUQ + (size_t)NB * 1024;              // 2^G Q_w S [NB][64] f32x4
    static constexpr size_t oUD = oQS + (size_t)NB * 1024;              // 2^(G_C-G) U [hi|lo][64][NB] bf16x4
    static constexpr size_t oTX = oUD + (size_t)NB * 1024;              // T_10 (accumulator layout) | T_32^T, hi|lo
    static constexpr size_t BYTES = oTX + 2048;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ int tri_idx(int i, int k) { return i * (i + 1) / 2 + k; }
__device__ __forceinline__ int off_idx(int m, int j) { return m * (m - 1) / 2 + j; }
constexpr int off_idx_c(int m, int j) { return m * (m - 1) / 2 + j; }

// Which preparation wave forms the Gram block A_mj (m > j).  With four token
// blocks the assignment evens out the X-phase: every wave forms five blocks
// (its P row, A_pp and the ones listed here); otherwise the owner of column j.
template <int NB> constexpr int a_owner(int m, int j) {
    if constexpr (NB == 4) {
        return (m == 1 && j == 0) || (m == 2 && j == 0) || (m == 3 && j == 2) ? 0
             : (m == 3 && j == 0) || (m == 2 && j == 1) ? 1 : 2;
    } else {
        return j;
    }
}

// Element (row, col) of a K or Q chunk in LDS: 16-byte granule col/8 of row r
// sits at granule position (col/8) ^ (r mod G), which spreads fragment reads and
// the column reads of the state update over distinct banks.
template <int DK> __device__ __forceinline__ int kq_idx(int row, int col) {
    constexpr int G = DK / 8;
    return row * DK + ((((col >> 3) ^ row) & (G - 1)) << 3) + (col & 7);
}

template <int KS, int DK>
__device__ __forceinline__ Frag<__bf16, KS> frag_kq(const __bf16 *base, int r0, int k0, int lane) {
    Frag<__bf16, KS> f;
    f.load(base + kq_idx<DK>(r0 + (lane & 15), k0 + (lane >> 4) * (KS / 4)));
    return f;
}

typedef __attribute__((address_space(3))) void *lds_ptr;

// Copy of 16 (4) bytes per lane from global memory straight into LDS (gfx950
// global_load_lds): lane L writes at l + 16 L (4 L); completion is tracked by
// vmcnt.  The host pass of this file sees an empty body: the builtin exists only
// for the device target.
__device__ __forceinline__ void load_lds16(const void *g, lds_ptr l) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
#endif
}
__device__ __forceinline__ void load_lds4(const void *g, lds_ptr l) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
#endif
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

// Column-ordered read of a row-major 16 x 16 bf16 block M: lane (n, g) receives
// M[4g + s][n], s = 0..3 -- the MFMA accumulator layout of M, which is the B
// operand of a 16-deep product with k = row.
__device__ __forceinline__ bf16x4 read_cols16(const __bf16 *blk, int lane) {
    const int ln = lane & 15, lg = lane >> 4;
    return read_tr16(blk + (4 * lg + (ln >> 2)) * 16 + 4 * (ln & 3));
}
// Row-ordered read: lane (r, g) receives M[r][4g + s] -- the A operand layout.
__device__ __forceinline__ bf16x4 read_rows16(const __bf16 *blk, int lane) {
    return *reinterpret_cast<const bf16x4 *>(blk + (lane & 15) * 16 + 4 * (lane >> 4));
}
// The lane's four values of a block held in accumulator layout (lane (n, g):
// M[4g + s][n]) written row-major as the transpose: position n * 16 + 4g + s.
__device__ __forceinline__ void write_acc_transposed(__bf16 *blk, bf16x4 v, int lane) {
    *reinterpret_cast<bf16x4 *>(blk + (lane & 15) * 16 + 4 * (lane >> 4)) = v;
}

// A operand K^T[r0 + m][tokens k0 ..] of the state update from the row-major
// (granule-permuted) K chunk: lane j of group g points at row k0 + 4g + j/4
// (and 16 rows further for KS = 32), columns r0 + 4 (j % 4)..+3; lane m of the
// group then holds column r0 + m at tokens k0 + 4g + s (and k0 + 16 + 4g + s).
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

// Two 16-deep fragments (k-blocks a and b) as one 32-deep fragment.  Used on
// both operands of a product, the pairing only reorders the terms of the k-sum.
__device__ __forceinline__ Frag<__bf16, 32> pair16(bf16x4 a, bf16x4 b) {
    Frag<__bf16, 32> f;
    f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return f;
}

// acc += A B for one 16 x 16 block pair held as bf16 hi/lo parts: the three
// products hi*hi + hi*lo + lo*hi on 16-deep MFMAs into the one accumulator.
// Accumulators that pass through here only ever meet 16x16x16 MFMAs: a 16x16x16
// MFMA that takes the result of a 16x16x32 one as its accumulator input at once
// reads a stale value on gfx950 (the compiler inserts no wait states between the
// two shapes).
__device__ __forceinline__ f32x4 mma_hl(bf16x4 ah, bf16x4 al, bf16x4 bh, bf16x4 bl, f32x4 acc) {
    using F16 = Frag<__bf16, 16>;
    F16 a, a2, b, b2;
    a.v = ah; a2.v = al; b.v = bh; b2.v = bl;
    acc = F16::mma(a, b, acc);
    acc = F16::mma(a, b2, acc);
    return F16::mma(a2, b, acc);
}

// One step of X <- (I - nL)^-1 X for a 16 x 16 block by forward substitution,
// lane (r, g) holding X[r][4g + e] and nL[r][:] = -L[r][:] (strictly lower):
// step S adds nL[r][S] X[S][:] to every row r (a no-op for r <= S), with n =
// nL[r][S].  X[S][:] sits in lane S of the same 16-lane row and is read
// through a DPP row broadcast folded into the multiply-add.  Each step is one
// asm statement led by s_nop 1: a DPP read of a VGPR needs two wait states
// after a VALU write of it, and the compiler may place its own instructions (a
// copy of X among them) between the steps; inside a step the four columns are
// independent.  The compiler schedules nothing across an asm statement, so
// what the caller writes between two steps runs between them.
template <int S> __device__ __forceinline__ void fsub_step(float (&X)[4], float n);
#define GDN_FS1(S, E) "v_fmac_f32_dpp %" #E ", %" #E ", %4 row_newbcast:" #S " row_mask:0xf bank_mask:0xf\n"
#define GDN_FSTEP(S)                                                                                   \
    template <> __device__ __forceinline__ void fsub_step<S>(float (&X)[4], float n) {               \
        asm volatile("s_nop 1\n" GDN_FS1(S, 0) GDN_FS1(S, 1) GDN_FS1(S, 2) GDN_FS1(S, 3)              \
                     : "+v"(X[0]), "+v"(X[1]), "+v"(X[2]), "+v"(X[3])                                 \
                     : "v"(n));                                                                       \
    }
GDN_FSTEP(0) GDN_FSTEP(1) GDN_FSTEP(2) GDN_FSTEP(3) GDN_FSTEP(4) GDN_FSTEP(5) GDN_FSTEP(6) GDN_FSTEP(7)
GDN_FSTEP(8) GDN_FSTEP(9) GDN_FSTEP(10) GDN_FSTEP(11) GDN_FSTEP(12) GDN_FSTEP(13) GDN_FSTEP(14)
#undef GDN_FSTEP
#undef GDN_FS1

// Blocks A_mj (m > j) that preparation wave pw forms in X, in order (m, then j)
template <int NB> constexpr int own_count(int pw) {
    int n = 0;
    for (int m = 1; m < NB; ++m)
        for (int j = 0; j < m; ++j) n += a_owner<NB>(m, j) == pw;
    return n;
}
template <int NB> constexpr int own_blk(int pw, int k, bool row) {
    for (int m = 1; m < NB; ++m)
        for (int j = 0; j < m; ++j)
            if (a_owner<NB>(m, j) == pw && k-- == 0) return row ? m : j;
    return 0;
}

template <int C, int DK>
__global__ __launch_bounds__(FT, 1) void gdn_prefill_fused_kernel(FusedParams p)
{
    using L = FL<C, DK>;
    using FDK = Frag<__bf16, L::KSD>;
    using FC = Frag<__bf16, L::KSC>;
    using F16 = Frag<__bf16, 16>;
    constexpr int NB = L::NB, NSB = L::NSB, MS = L::MS, NTRI = L::NTRI, KSD = L::KSD, NK = L::NK;
    constexpr int KSC = L::KSC, NJ = L::NJ, KPS = L::KPS;
    constexpr int NBO = NB > 1 ? NB - 1 : 1;     // register blocks of P below the diagonal
    static_assert(NTRI >= 1, "chunk");

    __shared__ __attribute__((aligned(1024))) char smem[L::BYTES];
    auto Kb = [&](int i) { return reinterpret_cast<__bf16 *>(smem + L::oK + (size_t)i * L::KQB); };
    auto Qb = [&](int i) { return reinterpret_cast<__bf16 *>(smem + L::oQ + (size_t)i * L::KQB); };
    auto Vb = [&](int i) { return reinterpret_cast<__bf16 *>(smem + L::oV + (size_t)i * L::VB); };
    auto ABb = [&](int i) { return reinterpret_cast<float *>(smem + L::oAB + (size_t)i * L::ABB); };
    auto TPb = [&](int s, int blk) { return reinterpret_cast<__bf16 *>(smem + L::oTP + (size_t)s * L::TPB + (size_t)blk * 1024); };
    auto DTb = [&](int s) { return smem + L::oDT + (size_t)s * L::DTB; };
    auto XTb = [&](int m) { return reinterpret_cast<__bf16 *>(smem + L::oXT + (size_t)m * 1024); };
    auto XAb = [&](int o) { return reinterpret_cast<__bf16 *>(smem + L::oXA + (size_t)o * 1024); };
    __bf16 *STh = reinterpret_cast<__bf16 *>(smem + L::oSTh);
    __bf16 *STl = reinterpret_cast<__bf16 *>(smem + L::oSTl);
    bf16x4 *Rs = reinterpret_cast<bf16x4 *>(smem + L::oR);       // [NB][hi 64 | lo 64]
    bf16x4 *UQs = reinterpret_cast<bf16x4 *>(smem + L::oUQ);     // [NB][hi 64 | lo 64]
    f32x4 *QSs = reinterpret_cast<f32x4 *>(smem + L::oQS);       // [NB][64]
    bf16x4 *UDs = reinterpret_cast<bf16x4 *>(smem + L::oUD);     // [hi | lo][64][NB]
    __bf16 *TX = reinterpret_cast<__bf16 *>(smem + L::oTX);

    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());
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

    // lane offsets (elements) of the K / Q fragments of block 0 of a chunk in LDS;
    // block j adds 16 j DK, since 16 j leaves the granule permutation unchanged
    int kqo[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) kqo[kk] = kq_idx<DK>(ln, kk * KSD + lg * (KSD / 4));
    auto frag_blk = [&](const __bf16 *X, int blk, int kk) {
        FDK f;
        f.load(X + blk * 16 * DK + kqo[kk]);
        return f;
    };

    // ======================= chain waves =======================
    auto chain_wave = [&](auto w_c) {
        constexpr int w = decltype(w_c)::value;
        constexpr bool has_rb = w < NB;
        f32x4 S[MS];
#pragma unroll
        for (int m = 0; m < MS; ++m) S[m] = zero4();
        if (p.s0) {
            const float *s0 = p.s0 + bh * (int64_t)DK * Dv;
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int ib = w + 4 * m;
                if (ib < NSB) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) S[m][e] = s0[(int64_t)(16 * ib + 4 * lg + e) * Dv + n0 + ln];
                }
            }
        }
        // Inputs go straight from global memory into LDS (global_load_lds): lane L
        // of a load writes the 16 bytes at the load's LDS base + 16 L, so each lane
        // fetches the granule that the row permutation of kq_idx puts there.  Rows
        // past the end of the sequence read token T-1 and are overwritten once the
        // data has landed: zeros, alpha = 1, beta = 0 (identity tokens).
        constexpr int G = DK / 8;                        // 16-byte granules per K / Q row
        constexpr int NLD = (DK + 31) / 32;              // 1 KB loads per 16-row block
        const __bf16 *kg = p.k + b * T * p.ks + h * DK;
        const __bf16 *qg = p.q + b * T * p.qs + h * DK;
        const __bf16 *vg = p.v + b * T * p.vs + h * Dv + n0;
        const float *ag = p.alpha + b * T * H + h;
        const float *bg = p.beta + b * T * H + h;
        int rbl[NLD], colg[NLD];                         // row in the block and column of lane's granule
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int byte = i * 1024 + 16 * lane;
            rbl[i] = byte / (2 * DK);
            const int gp = (byte % (2 * DK)) / 16;
            colg[i] = 8 * (gp ^ (rbl[i] & (G - 1)));
        }
        const int rv = lane >> 1;                        // V row of lane (lanes 0..31)
        auto tok = [&](int64_t c0, int r) -> int64_t {   // token row r of the block, clamped
            const int64_t t = c0 + 16 * w + r;
            return t < T ? t : T - 1;
        };
        // element offsets of the lane's data from token 0 of a chunk (no clamping)
        uint32_t ofk[NLD], ofq[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            ofk[i] = (uint32_t)((16 * w + rbl[i]) * p.ks + colg[i]);
            ofq[i] = (uint32_t)((16 * w + rbl[i]) * p.qs + colg[i]);
        }
        const uint32_t ofv = (uint32_t)((16 * w + rv) * p.vs + (lane & 1) * 8);
        const uint32_t ofg = (uint32_t)((16 * w + (lane & 15)) * H);
        auto lds = [&](const void *x) { return (lds_ptr)(uintptr_t)(uint32_t)(uintptr_t)x; };
        auto issue_k = [&](int64_t j) {
            if constexpr (has_rb) {
                const int64_t c0 = j * C;
                __bf16 *dst = Kb((int)(j % 3)) + 16 * w * DK;
                const __bf16 *kc = kg + c0 * p.ks;
                const bool full = c0 + C <= T;
#pragma unroll
                for (int i = 0; i < NLD; ++i)
                    if (rbl[i] < 16)
                        load_lds16(full ? kc + ofk[i] : kg + tok(c0, rbl[i]) * p.ks + colg[i], lds(dst + i * 512));
            }
        };
        auto issue_qv = [&](int64_t j) {
            if constexpr (has_rb) {
                const int64_t c0 = j * C;
                __bf16 *dst = Qb((int)(j & 1)) + 16 * w * DK;
                const __bf16 *qc = qg + c0 * p.qs, *vc = vg + c0 * p.vs;
                const bool full = c0 + C <= T;
#pragma unroll
                for (int i = 0; i < NLD; ++i)
                    if (rbl[i] < 16)
                        load_lds16(full ? qc + ofq[i] : qg + tok(c0, rbl[i]) * p.qs + colg[i], lds(dst + i * 512));
                if (lane < 32)
                    load_lds16(full ? vc + ofv : vg + tok(c0, rv) * p.vs + (lane & 1) * 8,
                               lds(Vb((int)(j & 1)) + 16 * w * BV));
            }
        };
        auto issue_gates = [&](int64_t j) {
            if constexpr (has_rb) {
                const int64_t c0 = j * C;
                float *dst = ABb((int)(j & 3));
                if (lane < 16) {
                    const bool full = c0 + C <= T;
                    const float *ac = full ? ag + c0 * H + ofg : ag + tok(c0, lane) * H;
                    const float *bc = full ? bg + c0 * H + ofg : bg + tok(c0, lane) * H;
                    load_lds4(ac, lds(dst + 16 * w));
                    load_lds4(bc, lds(dst + C + 16 * w));
                }
            }
        };
        // after the loads of chunk j (inputs) and jg (gates) have landed
        auto fill_tail = [&](int64_t j, int64_t jg) {
            if constexpr (has_rb) {
                if (j < NC && j * C + C > T) {
                    const int64_t c0 = j * C;
                    __bf16 *kd = Kb((int)(j % 3)) + 16 * w * DK, *qd = Qb((int)(j & 1)) + 16 * w * DK;
#pragma unroll
                    for (int i = 0; i < NLD; ++i)
                        if (rbl[i] < 16 && c0 + 16 * w + rbl[i] >= T) {
                            *reinterpret_cast<bf16x8 *>(kd + i * 512 + 8 * lane) = bf16x8{};
                            *reinterpret_cast<bf16x8 *>(qd + i * 512 + 8 * lane) = bf16x8{};
                        }
                    if (lane < 32 && c0 + 16 * w + rv >= T)
                        *reinterpret_cast<bf16x8 *>(Vb((int)(j & 1)) + 16 * w * BV + 8 * lane) = bf16x8{};
                }
                if (jg < NC && jg * C + C > T && lane < 16 && jg * C + 16 * w + lane >= T) {
                    float *ab = ABb((int)(jg & 3));
                    ab[16 * w + lane] = 1.f;
                    ab[C + 16 * w + lane] = 0.f;
                }
            }
        };
        auto wait_loads = [&]() {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0)
            asm volatile("" ::: "memory");
        };

        auto write_state_operand = [&]() {
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int ib = w + 4 * m;
                if (ib < NSB) {
                    bf16x4 hv, lv;
                    split4(S[m], hv, lv);
                    *reinterpret_cast<bf16x4 *>(STh + ln * KPS + 16 * ib + 4 * lg) = hv;
                    *reinterpret_cast<bf16x4 *>(STl + ln * KPS + 16 * ib + 4 * lg) = lv;
                }
            }
        };
        // chunk 0 and the gates of chunks 0 and 1 into LDS, then the decay table of
        // chunk 0 (preparation wave 3)
        issue_k(0);
        issue_qv(0);
        issue_gates(0);
        if (NC > 1) issue_gates(1);
        wait_loads();
        fill_tail(0, 0);
        if (NC > 1) fill_tail(NC, 1);
        lds_barrier();
        lds_barrier();

        // iteration c (c = -1 .. NC), three barriers:
        //   X:  K_w S, Q_w S, R_w of chunk c; copies of chunk c+2 (gates of c+3)
        //       into LDS are issued once this wave has read its Q and V rows of
        //       chunk c (no other wave reads those rows in this iteration)
        //   Y1: U_w = sum_k T'_wk R_k; U_w, 2^(G_C-G) U_w and 2^G Q_w S -> LDS
        //   Y2: state rows S <- 2^G_C S + K^T (2^(G_C-G) U), the S operand -> LDS
        int kb = 0;                                  // c % 3 for c >= 0
#pragma unroll 1
        for (int64_t c = -1; c <= NC; ++c) {
            const bool work = c >= 0 && c < NC;
            const int qb = (int)(c & 1);
            const __bf16 *Ks = Kb(kb);
            const char *dt = DTb((int)(c & 3));
            const float *EG = reinterpret_cast<const float *>(dt + L::DT_EG);
            const float *Ed = reinterpret_cast<const float *>(dt + L::DT_ED);
            // ---- X-phase: K_w S, Q_w S -> R_w
            f32x4 egqs = zero4();
            if (c + 2 < NC) issue_k(c + 2);
            if (c + 3 < NC) issue_gates(c + 3);
            if (has_rb && work) {
                const __bf16 *Qs = Qb(qb);
                FDK kf[NK], qf[NK], sh[NK], sl[NK];
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    kf[kk] = frag_blk(Ks, w, kk);
                    qf[kk] = frag_blk(Qs, w, kk);
                    sh[kk] = frag_rows<__bf16, KSD>(STh, KPS, 0, kk * KSD, lane);
                    sl[kk] = frag_rows<__bf16, KSD>(STl, KPS, 0, kk * KSD, lane);
                }
                const bf16x4 vv = read_cols16(Vb(qb) + 16 * w * BV, lane);
                const f32x4 eg = *reinterpret_cast<const f32x4 *>(EG + 16 * w + 4 * lg);
                f32x4 ks = zero4(), qs = zero4();
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    ks = FDK::mma(kf[kk], sh[kk], ks);
                    qs = FDK::mma(qf[kk], sh[kk], qs);
                    qs = FDK::mma(qf[kk], sl[kk], qs);
                }
                // the rows of Q_w and V_w of chunk c are in registers before the
                // copies of chunk c+2 into the same rows are issued
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                if (c + 2 < NC) issue_qv(c + 2);
                f32x4 rv;
#pragma unroll
                for (int e = 0; e < 4; ++e) rv[e] = (float)vv[e] - eg[e] * ks[e];
                bf16x4 hv, lv;
                split4(rv, hv, lv);
                Rs[w * 128 + lane] = hv;
                Rs[w * 128 + 64 + lane] = lv;
                egqs = eg * qs;
            } else {
                if (c + 2 < NC) issue_qv(c + 2);
            }
            lds_barrier();
            // ---- Y1: U_w = T'_w. R (token block w)
            if (has_rb && work) {
                const int ts = qb;
                f32x4 u = zero4();
#pragma unroll
                for (int k = 0; k <= w; ++k) {
                    const __bf16 *tb = TPb(ts, tri_idx(w, k));
                    u = mma_hl(read_cols16(tb, lane), read_cols16(tb + 256, lane), Rs[k * 128 + lane],
                               Rs[k * 128 + 64 + lane], u);
                }
                const f32x4 ed = *reinterpret_cast<const f32x4 *>(Ed + 16 * w + 4 * lg);
                bf16x4 dh, dl, uh, ul;
                split4(ed * u, dh, dl);
                split4(u, uh, ul);
                UDs[lane * NB + w] = dh;
                UDs[64 * NB + lane * NB + w] = dl;
                UQs[w * 128 + lane] = uh;
                UQs[w * 128 + 64 + lane] = ul;
                QSs[w * 64 + lane] = egqs;
            }
            lds_barrier();
            // ---- Y2: state update
            if (work) {
                const float egc = *reinterpret_cast<const float *>(dt + L::DT_EGC);
#pragma unroll
                for (int m = 0; m < MS; ++m) {
                    const int ib = w + 4 * m;
                    if (ib < NSB) {
                        f32x4 acc = S[m] * egc;
#pragma unroll
                        for (int jj = 0; jj < NJ; ++jj) {
                            const FC ka = k_cols_tr<KSC, DK>(Ks, 16 * ib, jj * KSC, lane);
                            FC bhf, blf;
                            if constexpr (KSC == 32) {
                                bhf.v = *reinterpret_cast<const bf16x8 *>(UDs + lane * NB + 2 * jj);
                                blf.v = *reinterpret_cast<const bf16x8 *>(UDs + 64 * NB + lane * NB + 2 * jj);
                            } else {
                                bhf.v = UDs[lane * NB + jj];
                                blf.v = UDs[64 * NB + lane * NB + jj];
                            }
                            acc = FC::mma(ka, bhf, acc);
                            acc = FC::mma(ka, blf, acc);
                        }
                        S[m] = acc;
                    }
                }
            }
            if (c < NC) write_state_operand();       // c = -1: the initial state
            wait_loads();
            fill_tail(c + 2, c + 3);
            lds_barrier();
            if (c >= 0) kb = kb == 2 ? 0 : kb + 1;
        }
        if (p.sT) {
            float *sT = p.sT + bh * (int64_t)DK * Dv;
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                const int ib = w + 4 * m;
                if (ib < NSB) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) sT[(int64_t)(16 * ib + 4 * lg + e) * Dv + n0 + ln] = S[m][e];
                }
            }
        }
    };

    // ======================= preparation waves =======================
    auto prep_wave = [&](auto p_c) {
        constexpr int pw = decltype(p_c)::value;
        constexpr bool has_rb = pw < NB;

        // P row pw of a chunk as bf16 hi/lo A operands (lane (r, g): P[r][4g + e]):
        // the blocks left of the diagonal and the diagonal block, kept from the
        // chunk's preparation until its output is formed; register set j & 1
        // holds chunk j
        bf16x4 Ph[2][NBO], Pl[2][NBO], Pdh[2], Pdl[2];

        // decay ratios 2^(G_r - G_j) on a diagonal block (r >= j, or r > j), 0 above
        auto decay_diag = [&](f32x4 d, int blk, bool incl, const char *dt) {
            const double *Gd = reinterpret_cast<const double *>(dt) + 16 * blk;
            const double Gr = Gd[ln];
            double Gc[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) Gc[e] = Gd[4 * lg + e];
            f32x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int jc = 4 * lg + e;
                const bool keep = incl ? ln >= jc : ln > jc;
                // above the diagonal the exponent is positive and the product discarded
                const float g = __builtin_amdgcn_exp2f((float)fmin(Gr - Gc[e], 0.0)) * d[e];
                out[e] = keep ? g : 0.f;
            }
            return out;
        };
        // decay ratios on block (m, jb), m > jb: row factor f (of row 16 m + ln)
        // times the column factors of block jb
        auto decay_off = [&](f32x4 d, float f, int jb, const char *dt) {
            const f32x4 hc = *reinterpret_cast<const f32x4 *>(dt + L::DT_HC + 4 * (16 * jb + 4 * lg));
            return d * (hc * f);
        };
        auto row_factor = [&](const char *dt, int jb, int m) {
            return reinterpret_cast<const float *>(dt + L::DT_FR)[jb * C + 16 * m + ln];
        };

        // decay table of chunk j from its gates: fp64 prefix G of log2 alpha, then
        // 2^G, 2^(G_C - G), 2^G_C; with anchor a_jb = G at the last token of block
        // jb, HC_t = 2^(a_blk(t) - G_t) and FR_jb,t = 2^(G_t - a_jb) (used for
        // t in later blocks), so that 2^(G_r - G_t) = FR_jb,r HC_t with both
        // factors at most 1
        auto decay_table = [&](int64_t j) {
            const float *ab = ABb((int)(j & 3));
            char *dt = DTb((int)(j & 3));
            const float al = lane < C ? ab[lane] : 1.f;
            const double G = wave_inclusive_sum_f64(lane < C ? (double)log2_decay(al) : 0.0, lane);
            const double GC = lane_value_f64(G, C - 1);
            double anc[NB];
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) anc[jb] = lane_value_f64(G, 16 * jb + 15);
            if (lane < C) {
                float *f = reinterpret_cast<float *>(dt);
                reinterpret_cast<double *>(dt)[lane] = G;
                f[L::DT_EG / 4 + lane] = __builtin_amdgcn_exp2f((float)G);
                f[L::DT_ED / 4 + lane] = __builtin_amdgcn_exp2f((float)(GC - G));
                const int blk = lane >> 4;
                double a = anc[0];
#pragma unroll
                for (int jb = 1; jb < NB; ++jb) a = blk == jb ? anc[jb] : a;
                f[L::DT_HC / 4 + lane] = __builtin_amdgcn_exp2f((float)(a - G));
#pragma unroll
                for (int jb = 0; jb < NB - 1; ++jb)
                    f[L::DT_FR / 4 + jb * C + lane] = blk > jb ? __builtin_amdgcn_exp2f((float)(G - anc[jb])) : 0.f;
            }
            if (lane == 0) *reinterpret_cast<float *>(dt + L::DT_EGC) = __builtin_amdgcn_exp2f((float)GC);
        };

        // X-phase work of chunk j; its P row goes to register set par.  The
        // fragments of every K block and of Q block pw are read once; the Gram
        // blocks are formed from registers.
        auto prep_x = [&](auto par_c, int64_t j) {
            constexpr int par = decltype(par_c)::value;
            if constexpr (!has_rb) return;
            const __bf16 *Ks = Kb((int)(j % 3));
            const __bf16 *Qs = Qb((int)(j & 1));
            const float *ab = ABb((int)(j & 3));
            const char *dt = DTb((int)(j & 3));
            FDK kf[NB][NK], qf[NK];
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) qf[kk] = frag_blk(Qs, pw, kk);
#pragma unroll
            for (int jb = 0; jb < NB; ++jb)
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) kf[jb][kk] = frag_blk(Ks, jb, kk);
            // X_r K_jb^T in row layout from fragments
            auto gramr = [&](const FDK (&xr)[NK], int jb) {
                f32x4 acc = zero4();
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) acc = FDK::mma(kf[jb][kk], xr[kk], acc);
                return acc;
            };
            // every Gram block at once (A_pp first: its substitution is the long
            // chain), then the decay factors, so that the substitution steps
            // below have only registers to wait for
            constexpr int NOWN = own_count<NB>(pw);
            const f32x4 gpp = gramr(kf[pw], pw);
            f32x4 gp[NB], ga[NOWN > 0 ? NOWN : 1], fp[NB], fa[NOWN > 0 ? NOWN : 1];
            static_for<NB>([&](auto jb_c) {
                constexpr int jb = decltype(jb_c)::value;
                if constexpr (jb <= pw) gp[jb] = gramr(qf, jb);
            });
            static_for<NOWN>([&](auto k_c) {
                constexpr int k = decltype(k_c)::value;
                ga[k] = gramr(kf[own_blk<NB>(pw, k, true)], own_blk<NB>(pw, k, false));
            });
            const float nbet = -ab[C + 16 * pw + ln];
            const f32x4 one4 = {1.f, 1.f, 1.f, 1.f};
            static_for<NB>([&](auto jb_c) {
                constexpr int jb = decltype(jb_c)::value;
                if constexpr (jb < pw) fp[jb] = decay_off(one4, row_factor(dt, jb, pw), jb, dt);
                else if constexpr (jb == pw) fp[jb] = decay_diag(one4, pw, true, dt);
            });
            static_for<NOWN>([&](auto k_c) {
                constexpr int k = decltype(k_c)::value;
                constexpr int m = own_blk<NB>(pw, k, true), jj = own_blk<NB>(pw, k, false);
                fa[k] = decay_off(one4, row_factor(dt, jj, m) * ab[C + 16 * m + ln], jj, dt);
            });
            // A_pp: -A_pp rows through the T_pp slot (scratch)
            float nL[16];
            {
                const f32x4 d = decay_diag(gpp, pw, false, dt) * nbet;
                float *scr = reinterpret_cast<float *>(XTb(pw));
                *reinterpret_cast<f32x4 *>(scr + ln * 16 + 4 * lg) = d;
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const f32x4 v4 = *reinterpret_cast<const f32x4 *>(scr + ln * 16 + 4 * s4);
                    nL[4 * s4] = v4[0]; nL[4 * s4 + 1] = v4[1]; nL[4 * s4 + 2] = v4[2]; nL[4 * s4 + 3] = v4[3];
                }
            }
            // the other blocks, one between each pair of substitution steps: P
            // row pw (left of the diagonal, then the diagonal block), then the
            // owned blocks of A below the diagonal
            auto task = [&](auto t_c) {
                constexpr int t = decltype(t_c)::value;
                if constexpr (t < pw) {
                    split4(gp[t] * fp[t], Ph[par][t], Pl[par][t]);
                } else if constexpr (t == pw) {
                    split4(gp[pw] * fp[pw], Pdh[par], Pdl[par]);
                } else if constexpr (t - pw - 1 < NOWN) {
                    constexpr int k = t - pw - 1;
                    constexpr int o = off_idx_c(own_blk<NB>(pw, k, true), own_blk<NB>(pw, k, false));
                    bf16x4 hv, lv;
                    split4(ga[k] * fa[k], hv, lv);
                    *reinterpret_cast<bf16x4 *>(XAb(o) + ln * 16 + 4 * lg) = hv;
                    *reinterpret_cast<bf16x4 *>(XAb(o) + 256 + ln * 16 + 4 * lg) = lv;
                }
            };
            static_assert(NB + NOWN <= 15, "one block a step");
            float X[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) X[e] = ln == 4 * lg + e ? 1.f : 0.f;
            static_for<15>([&](auto s_c) {
                constexpr int S = decltype(s_c)::value;
                fsub_step<S>(X, nL[S]);
                task(s_c);
            });
            {
                bf16x4 hv, lv;
                split4(f32x4{X[0], X[1], X[2], X[3]}, hv, lv);
                // the scratch rows were read above (same wavefront, LDS in order)
                *reinterpret_cast<bf16x4 *>(XTb(pw) + ln * 16 + 4 * lg) = hv;
                *reinterpret_cast<bf16x4 *>(XTb(pw) + 256 + ln * 16 + 4 * lg) = lv;
            }
        };

        // T = (I + A)^-1 from the diagonal inverses T_mm (in XT) by halves of the
        // chunk: T_10 = -T_11 A_10 T_00 and T_32 = -T_33 A_32 T_22 (Y1), then the
        // lower-left quarter -T_lower (A_lower-left T_upper) (Y2):
        //   T_20 = -T_22 (A_20 T_00 + A_21 T_10),  T_21 = -T_22 A_21 T_11,
        //   T_30 = -(T_32 W_20 + T_33 W_30),        T_31 = -(T_32 W_21 + T_33 W_31),
        //   W_m0 = A_m0 T_00 + A_m1 T_10,  W_m1 = A_m1 T_11.
        // Every block of T' = T diag(beta) goes to slot j % 2 as its transpose.
        // B operands (right factors) are in accumulator layout, A operands in row
        // layout; every product is hi/lo.
        bf16x4 t10h = {}, t10l = {};                     // T_10 (wave 0, from Y1 to Y2)
        auto xa_rows = [&](int m, int jj, bf16x4 &h, bf16x4 &l) {
            const __bf16 *x = XAb(off_idx(m, jj));
            h = read_rows16(x, lane);
            l = read_rows16(x + 256, lane);
        };
        auto write_tp = [&](int ts, int m, int k, f32x4 t, float bk) {
            bf16x4 hv, lv;
            split4(t * bk, hv, lv);
            write_acc_transposed(TPb(ts, tri_idx(m, k)), hv, lane);
            write_acc_transposed(TPb(ts, tri_idx(m, k)) + 256, lv, lane);
        };
        // -T_mm Z for Z in accumulator layout
        auto neg_tmm = [&](int m, f32x4 z) {
            bf16x4 zh, zl;
            split4(-z, zh, zl);
            return mma_hl(read_rows16(XTb(m), lane), read_rows16(XTb(m) + 256, lane), zh, zl, zero4());
        };
        auto prep_y1 = [&](int64_t j) {
            if constexpr (!has_rb) return;
            const int ts = (int)(j & 1);
            const float bk = ABb((int)(j & 3))[C + 16 * pw + ln];     // beta of column block pw
            const bf16x4 dh = read_cols16(XTb(pw), lane), dl = read_cols16(XTb(pw) + 256, lane);
            {
                f32x4 t;
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] = (float)dh[e] + (float)dl[e];
                write_tp(ts, pw, pw, t, bk);
            }
            if constexpr (NB >= 2 && (pw == 0 || (NB == 4 && pw == 2))) {
                bf16x4 ah, al;
                xa_rows(pw + 1, pw, ah, al);
                const f32x4 t = neg_tmm(pw + 1, mma_hl(ah, al, dh, dl, zero4()));
                write_tp(ts, pw + 1, pw, t, bk);
                if constexpr (NB == 4) {
                    bf16x4 h, l;
                    split4(t, h, l);
                    if constexpr (pw == 0) {
                        t10h = h;
                        t10l = l;
                        reinterpret_cast<bf16x4 *>(TX)[lane] = h;
                        reinterpret_cast<bf16x4 *>(TX)[64 + lane] = l;
                    } else {
                        write_acc_transposed(TX + 512, h, lane);
                        write_acc_transposed(TX + 768, l, lane);
                    }
                }
            }
        };
        auto prep_y2 = [&](int64_t j) {
            if constexpr (NB == 4 && has_rb) {
                const int ts = (int)(j & 1);
                constexpr int k = pw & 1;                 // column block of this wave's result
                const float bk = ABb((int)(j & 3))[C + 16 * k + ln];
                // T_kk (B operand) and, for column 0, T_10
                const bf16x4 th = read_cols16(XTb(k), lane), tl = read_cols16(XTb(k) + 256, lane);
                bf16x4 a1h, a1l, a2h, a2l;
                if constexpr (pw == 0) {                  // T_20
                    xa_rows(2, 0, a1h, a1l);
                    xa_rows(2, 1, a2h, a2l);
                    f32x4 z = mma_hl(a1h, a1l, th, tl, zero4());
                    z = mma_hl(a2h, a2l, t10h, t10l, z);
                    write_tp(ts, 2, 0, neg_tmm(2, z), bk);
                } else if constexpr (pw == 1) {           // T_21
                    xa_rows(2, 1, a1h, a1l);
                    write_tp(ts, 2, 1, neg_tmm(2, mma_hl(a1h, a1l, th, tl, zero4())), bk);
                } else {                                  // T_3k
                    f32x4 wa, wb;                         // W_2k, W_3k
                    if constexpr (k == 0) {
                        const bf16x4 uh = reinterpret_cast<const bf16x4 *>(TX)[lane];
                        const bf16x4 ul = reinterpret_cast<const bf16x4 *>(TX)[64 + lane];
                        xa_rows(2, 0, a1h, a1l);
                        xa_rows(2, 1, a2h, a2l);
                        wa = mma_hl(a2h, a2l, uh, ul, mma_hl(a1h, a1l, th, tl, zero4()));
                        xa_rows(3, 0, a1h, a1l);
                        xa_rows(3, 1, a2h, a2l);
                        wb = mma_hl(a2h, a2l, uh, ul, mma_hl(a1h, a1l, th, tl, zero4()));
                    } else {
                        xa_rows(2, 1, a1h, a1l);
                        xa_rows(3, 1, a2h, a2l);
                        wa = mma_hl(a1h, a1l, th, tl, zero4());
                        wb = mma_hl(a2h, a2l, th, tl, zero4());
                    }
                    bf16x4 wah, wal, wbh, wbl;
                    split4(-wa, wah, wal);
                    split4(-wb, wbh, wbl);
                    f32x4 t = mma_hl(read_cols16(TX + 512, lane), read_cols16(TX + 768, lane), wah, wal, zero4());
                    t = mma_hl(read_rows16(XTb(3), lane), read_rows16(XTb(3) + 256, lane), wbh, wbl, t);
                    write_tp(ts, 3, k, t, bk);
                }
            }
        };

        // output rows of token block pw of chunk j from P register set par
        float *yg = p.y + ((b * T) * H + h) * Dv + n0;
        uint32_t yo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) yo[e] = (uint32_t)((16 * pw + 4 * lg + e) * H * Dv) + ln;
        auto out_y = [&](auto par_c, int64_t j) {
            constexpr int par = decltype(par_c)::value;
            if constexpr (!has_rb) return;
            f32x4 acc = QSs[pw * 64 + lane];
            static_for<NB - 1>([&](auto jb_c) {
                constexpr int jb = decltype(jb_c)::value;
                if constexpr (jb < pw) acc = mma_hl(Ph[par][jb], Pl[par][jb], UQs[jb * 128 + lane], UQs[jb * 128 + 64 + lane], acc);
            });
            acc = mma_hl(Pdh[par], Pdl[par], UQs[pw * 128 + lane], UQs[pw * 128 + 64 + lane], acc);
            const int64_t c0 = j * C;
            float *yc = yg + c0 * H * Dv;
            if (c0 + C <= T) {
#pragma unroll
                for (int e = 0; e < 4; ++e) yc[yo[e]] = acc[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c0 + 16 * pw + 4 * lg + e < T) yc[yo[e]] = acc[e];
            }
        };

        constexpr int TBL = NB == 4 ? 1 : 3;        // the wave that builds the decay tables
        lds_barrier();                              // chunk 0 and gates 0, 1 staged
        if constexpr (pw == TBL) decay_table(0);
        lds_barrier();

        // iteration c: X (outputs of c-1, preparation of c+1), Y1 and Y2 (T' of
        // c+1, decay table of c+2).  Set (c+1) & 1 holds P of chunk c-1 until its
        // output is formed, then P of chunk c+1.
        auto iter = [&](auto par_c, int64_t c) {
            if (c >= 1) out_y(par_c, c - 1);
            if (c + 1 < NC) prep_x(par_c, c + 1);
            lds_barrier();
            if (c + 1 < NC) prep_y1(c + 1);
            if constexpr (pw == TBL) {
                if (c + 2 < NC) decay_table(c + 2);
            }
            lds_barrier();
            if (c + 1 < NC) prep_y2(c + 1);
            lds_barrier();
        };
#pragma unroll 1
        for (int64_t c = -1; c <= NC; c += 2) {
            iter(std::integral_constant<int, 0>{}, c);
            if (c + 1 <= NC) iter(std::integral_constant<int, 1>{}, c + 1);
        }
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    switch (wave) {
    case 0: chain_wave(I0{}); break;
    case 1: chain_wave(I1{}); break;
    case 2: chain_wave(I2{}); break;
    case 3: chain_wave(I3{}); break;
    case 4: prep_wave(I0{}); break;
    case 5: prep_wave(I1{}); break;
    case 6: prep_wave(I2{}); break;
    default: prep_wave(I3{}); break;
    }
}

template <int C, int DK>
hipError_t launch_fused_t(const PrefillArgs &a, hipStream_t stream)
{
    FusedParams fp;
    fp.q = static_cast<const __bf16 *>(a.q);
    fp.k = static_cast<const __bf16 *>(a.k);
    fp.v = static_cast<const __bf16 *>(a.v);
    fp.alpha = a.alpha; fp.beta = a.beta; fp.s0 = a.s0;
    fp.y = a.y; fp.sT = a.sT;
    fp.T = a.T; fp.H = a.H; fp.Dv = a.Dv;
    fp.qs = a.q_tok_stride; fp.ks = a.k_tok_stride; fp.vs = a.v_tok_stride;
    fp.nslices = (int)(a.Dv / BV);
    const int64_t bh = a.B * a.H;
    fp.xcd_map = (bh % 8 == 0) ? 1 : 0;
    const int64_t grid = bh * fp.nslices;
    hipLaunchKernelGGL((gdn_prefill_fused_kernel<C, DK>), dim3((unsigned)grid), dim3(FT), 0, stream, fp);
    return hipGetLastError();
}

template <int C>
hipError_t launch_fused_dk(const PrefillArgs &a, hipStream_t s)
{
    switch (a.Dk) {
    case 16: return launch_fused_t<C, 16>(a, s);
    case 32: return launch_fused_t<C, 32>(a, s);
    case 64: return launch_fused_t<C, 64>(a, s);
    case 128: return launch_fused_t<C, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill_fused(const PrefillArgs &a, hipStream_t stream)
{
    switch (a.chunk) {
    case 16: return launch_fused_dk<16>(a, stream);
    case 32: return launch_fused_dk<32>(a, stream);
    case 64: return launch_fused_dk<64>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
