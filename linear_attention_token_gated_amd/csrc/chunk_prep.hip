// chunk_prep.hip -- the part of the chunkwise gated delta rule that does not
// depend on the state or on V, computed for every (sequence, head, chunk) in
// parallel ahead of the recurrence.
//
// Source: "On the Design of Qwen3.8-Next Architecture", picx.dev summary,
// "Theoretical foundations", eqs (1)-(4); the chunk form is derived from the
// token recurrence.  For one chunk of C tokens r = 0..C-1 with gates
// alpha_r, beta_r (base-2 decay prefix G_r = sum_{j<=r} log2 alpha_j):
//
//   EG_r = 2^G_r,  Ed_r = 2^(G_{C-1} - G_r),  EGC = 2^G_{C-1}
//   A    = strict_lower[ beta_r 2^(G_r - G_j) (k_r . k_j) ]
//   T'   = (I + A)^-1 diag(beta)        (so that U = T' (V - diag(EG) K S))
//
// The recurrence kernel then needs K S, one dense product U = T' R per chunk,
// the state update and the output; it forms the output's causal scores P =
// lower_incl[ 2^(G_r - G_j) (q_r . k_j) ] itself from the K and Q rows it
// stages anyway, so this kernel reads only K and the gates.  T' is written as
// bf16 hi/lo pairs in MFMA operand order (one 8-byte fragment per lane and
// 16x16 block), and G beside the decay vectors.
//
// (I + A)^-1 is formed in fp32: each diagonal block by forward substitution
// inside one wavefront (DPP row broadcast), the blocks below it level by level
//   T_ik = -T_ii sum_{m=k}^{i-1} A_im T_mk
// on fp32 MFMA.  Ragged tails are padded with identity tokens (alpha = 1,
// beta = 0, k = q = 0), which leave every real entry unchanged.
#include "common.hpp"
#include "launch.hpp"
#include "prep_layout.hpp"

namespace gdn {

namespace {

constexpr int PREP_THREADS = 256;   // 4 wavefronts
// resident workgroups per CU: four fit the LDS (33 KB each at C = 64, d = 128)
// and the register file (one wavefront per SIMD each, at most 128 VGPRs)
constexpr int PREP_PER_CU = 4;

template <int C, int DK> struct PrepLds {
    using R = PrepRecord<C>;
    static constexpr int NB = C / 16, NTRI = R::NTRI;
    static constexpr int KS_DK = DK % 32 == 0 ? 32 : 16;
    static constexpr int KP = frag_pitch<KS_DK>(DK);
    static constexpr int AP = 20;                               // fp32 block row pitch
    static constexpr size_t oK = 0;
    static constexpr size_t oA = oK + align16(2 * C * KP);      // A blocks [NTRI][16][AP], row-major
    // (I + A)^-1 blocks, row-major: written only after the Gram blocks are done,
    // so they reuse the space of the K rows where that is large enough
    static constexpr bool T_IN_KQ = 4 * NTRI * 16 * AP <= 2 * C * KP;
    static constexpr size_t oT = T_IN_KQ ? oK : oA + align16(4 * NTRI * 16 * AP);
    static constexpr size_t oG = (T_IN_KQ ? oA : oT) + align16(4 * NTRI * 16 * AP);
    static constexpr size_t oBe = oG + align16(4 * C);
    static constexpr size_t oEa = oBe + align16(4 * C);         // 2^(G_r - G_{16 floor(r/16)})
    static constexpr size_t oEb = oEa + align16(4 * C);         // [NB][C] 2^(G_{16 rb} - G_j), j < 16 rb
    static constexpr size_t BYTES = oEb + align16(4 * NB * C);
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ int tri_idx(int i, int k) { return i * (i + 1) / 2 + k; }

template <int S>
__device__ __forceinline__ void fsub_step(float (&X)[4], const float (&Lr)[16]) {
    // rows r <= S have L[r][S] = 0 (strictly lower): the update is an exact no-op there
#pragma unroll
    for (int e = 0; e < 4; ++e) X[e] = fmaf(-Lr[S], row_bcast<S>(X[e]), X[e]);
}
template <int... S>
__device__ __forceinline__ void fsub16(float (&X)[4], const float (&Lr)[16], std::integer_sequence<int, S...>) {
    (fsub_step<S>(X, Lr), ...);
}

template <int C, int DK>
__global__ __launch_bounds__(PREP_THREADS, PREP_PER_CU) void gdn_chunk_prep_kernel(PrepParams p)
{
    using L = PrepLds<C, DK>;
    using Rec = PrepRecord<C>;
    using FDK = Frag<__bf16, L::KS_DK>;
    using F32 = Frag<float, 16>;
    constexpr int KP = L::KP, AP = L::AP, NB = L::NB, NTRI = L::NTRI, KS_DK = L::KS_DK, NK = DK / KS_DK;
    constexpr int VPR = DK / 8;                  // 16-byte vectors per K/Q row

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    __bf16 *Ks = reinterpret_cast<__bf16 *>(smem + L::oK);
    float *As = reinterpret_cast<float *>(smem + L::oA);
    float *Ts = reinterpret_cast<float *>(smem + L::oT);
    float *Gs = reinterpret_cast<float *>(smem + L::oG);
    float *Bes = reinterpret_cast<float *>(smem + L::oBe);
    float *Eas = reinterpret_cast<float *>(smem + L::oEa);
    float *Ebs = reinterpret_cast<float *>(smem + L::oEb);

    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(wave_id());
    const int ln = lane & 15, lg = lane >> 4;
    const __bf16 *kg = static_cast<const __bf16 *>(p.k);
    const int64_t NC = (p.T + C - 1) / C;
    const int64_t BH = p.BH, nwork = BH * NC;

    // Work items are taken chunk-major, so the workgroups running at one time
    // share the rows of K and the gates.  With a grid that is a multiple of
    // 8, the items of chunk c go to the workgroups with id = c mod 8, which the
    // hardware places on one XCD: every gate row is then fetched into one L2.
    // The rows of the next item are loaded into registers while the current
    // one is computed.
    const bool xcd = gridDim.x % 8 == 0;
    const int64_t gx = xcd ? blockIdx.x & 7 : 0;                   // chunk residue of this workgroup
    const int64_t stride = xcd ? gridDim.x >> 3 : gridDim.x;       // workgroups per residue
    const int64_t mine = xcd ? (NC > gx ? (NC - gx + 7) / 8 : 0) * BH : nwork;   // items of this residue
    // item i of this residue -> (chunk, bh)
    auto item_c = [&](int64_t i) { return xcd ? gx + 8 * (i / BH) : i / BH; };
    constexpr int NLD = (C * VPR + PREP_THREADS - 1) / PREP_THREADS;
    f32x4 kv[NLD];
    float al = 1.f, be = 0.f;
    auto fetch = [&](int64_t i) {
        const int64_t c = item_c(i), bh = i % BH, b = bh / p.H, h = bh % p.H, t0 = c * C;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int vi = tid + i * PREP_THREADS;
            const int r = (vi < C * VPR ? vi : 0) / VPR, col = (vi % VPR) * 8;
            const int64_t tok = b * p.T + (t0 + r < p.T ? t0 + r : p.T - 1);   // rows past the end: zeroed later
            kv[i] = *reinterpret_cast<const f32x4 *>(kg + tok * p.ks + h * DK + col);
        }
        if (wave == 0) {
            const int64_t gi = (b * p.T + (lane < C && t0 + lane < p.T ? t0 + lane : 0)) * p.H + h;
            al = p.alpha[gi];
            be = p.beta[gi];
        }
    };
    const int64_t first = xcd ? blockIdx.x >> 3 : blockIdx.x;
    if (first < mine) fetch(first);

    for (int64_t i = first; i < mine; i += stride) {
    const int64_t c = item_c(i), bh = i % BH;
    const int64_t t0 = c * C;
    char *out = static_cast<char *>(p.ws) + (bh * NC + c) * Rec::BYTES;

    // ---- 1. K rows of the chunk (zero past the end), gates and decay scan
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int vi = tid + i * PREP_THREADS;
        const int r = vi / VPR, col = (vi % VPR) * 8;
        if (vi < C * VPR) {
            const bool in = t0 + r < p.T;
            *reinterpret_cast<f32x4 *>(Ks + r * KP + col) = in ? kv[i] : zero4();
        }
    }
    if (wave == 0) {
        const bool real = lane < C && t0 + lane < p.T;
        al = real ? al : 1.f;
        be = real ? be : 0.f;
        const float g2 = wave_inclusive_sum(lane < C ? log2_decay(al) : 0.f, lane);
        const float gC = lane_value(g2, C - 1);
        const float gblk = row_bcast<0>(g2);
        float *dec = reinterpret_cast<float *>(out + Rec::oDec);
        if (lane < C) {
            Gs[lane] = g2;
            Bes[lane] = be;
            Eas[lane] = __builtin_amdgcn_exp2f(g2 - gblk);
            dec[lane] = __builtin_amdgcn_exp2f(g2);                 // EG
            dec[C + lane] = __builtin_amdgcn_exp2f(gC - g2);        // Ed
            dec[Rec::DEC_G + lane] = g2;                            // G
        }
        if (lane == 0) dec[2 * C] = __builtin_amdgcn_exp2f(gC);     // EGC
#pragma unroll
        for (int rb = 1; rb < NB; ++rb) {
            const float gref = lane_value(g2, 16 * rb);
            if (lane < C) Ebs[rb * C + lane] = lane < 16 * rb ? __builtin_amdgcn_exp2f(gref - g2) : 0.f;
        }
    }
    // the next item's rows (the registers of this one are consumed); the
    // barriers below order LDS only, so these loads stay in flight until the
    // next item stores them
    if (i + stride < mine) fetch(i + stride);
    lds_barrier();

    // ---- 2. Gram blocks of A (NTRI blocks, fp32 into LDS), computed transposed,
    //         D = K_cb K_rb^T, so lane (ln, lg) holds row r = 16 rb + ln, columns
    //         j = 16 cb + 4 lg + e: the A-operand fragment of that block.  Wave w
    //         takes block row w (its K_rb fragments are loaded once).
    auto gram_row = [&](auto rb_c) {
        constexpr int rb = decltype(rb_c)::value;
        FDK fb[NK];
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) fb[kk] = frag_rows<__bf16, KS_DK>(Ks, KP, 16 * rb, kk * KS_DK, lane);
        const int r = 16 * rb + ln;
        const float Gr = Gs[r], Ear = Eas[r], ber = Bes[r];
        static_for<rb + 1>([&](auto cb_c) {
            constexpr int cb = decltype(cb_c)::value;
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < NK; ++kk)
                acc = FDK::mma(frag_rows<__bf16, KS_DK>(Ks, KP, 16 * cb, kk * KS_DK, lane), fb[kk], acc);
            const int j0 = 16 * cb + 4 * lg;
            f32x4 val;
            if constexpr (rb == cb) {
                const f32x4 Gj = *reinterpret_cast<const f32x4 *>(Gs + j0);
#pragma unroll
                for (int e = 0; e < 4; ++e) val[e] = r > j0 + e ? __builtin_amdgcn_exp2f(Gr - Gj[e]) * acc[e] : 0.f;
            } else {
                // r > j: 2^(G_r - G_j) = 2^(G_r - G_{16 rb}) 2^(G_{16 rb} - G_j), both factors <= 1
                const f32x4 eb = *reinterpret_cast<const f32x4 *>(Ebs + rb * C + j0);
                val = acc * eb * Ear;
            }
            constexpr int idx = rb * (rb + 1) / 2 + cb;
            *reinterpret_cast<f32x4 *>(As + (idx * 16 + ln) * AP + 4 * lg) = val * ber;
        });
    };
    switch (wave) {
    case 0: gram_row(std::integral_constant<int, 0>{}); break;
    case 1: if constexpr (NB > 1) gram_row(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (NB > 2) gram_row(std::integral_constant<int, 2>{}); break;
    default: if constexpr (NB > 3) gram_row(std::integral_constant<int, 3>{}); break;
    }
    lds_barrier();

    // ---- 3. diagonal blocks T_ii = (I + A_ii)^-1; lane (ln, lg) carries row ln,
    //         columns 4 lg + e
    float X[4];
    if (wave < NB) {
        const int ii = tri_idx(wave, wave);
        float Lr[16];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const f32x4 v4 = *reinterpret_cast<const f32x4 *>(As + (ii * 16 + ln) * AP + 4 * s4);
            Lr[4 * s4] = v4[0]; Lr[4 * s4 + 1] = v4[1]; Lr[4 * s4 + 2] = v4[2]; Lr[4 * s4 + 3] = v4[3];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) X[e] = ln == 4 * lg + e ? 1.f : 0.f;
        fsub16(X, Lr, std::make_integer_sequence<int, 15>{});
        *reinterpret_cast<f32x4 *>(Ts + (ii * 16 + ln) * AP + 4 * lg) = f32x4{X[0], X[1], X[2], X[3]};
    }
    lds_barrier();

    // ---- 4. blocks below the diagonal, one distance d = i - k per level; wave i
    //         owns row block i.  M = sum_m A_im T_mk, then T_ik = -T_ii M.  The MFMA
    //         accumulator layout (lane holds M[4 lg + e][ln]) is the B operand of the
    //         second product as it stands.
    for (int d = 1; d < NB; ++d) {
        const int i = wave, k = wave - d;
        if (i < NB && k >= 0) {
            f32x4 m = zero4();
            for (int mm = k; mm < i; ++mm) {
                const F32 a = frag_rows<float, 16>(As + tri_idx(i, mm) * 16 * AP, AP, 0, 0, lane);
                F32 t;
                const float *tc = Ts + tri_idx(mm, k) * 16 * AP;
#pragma unroll
                for (int e = 0; e < 4; ++e) t.v[e] = tc[(4 * lg + e) * AP + ln];
                m = F32::mma(a, t, m);
            }
            F32 ti, mb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ti.v[e] = X[e];
                mb.v[e] = m[e];
            }
            const f32x4 tik = F32::mma(ti, mb, zero4());
            float *dst = Ts + tri_idx(i, k) * 16 * AP;
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[(4 * lg + e) * AP + ln] = -tik[e];
        }
        lds_barrier();
    }

    // ---- 5. T' = T diag(beta) as bf16 hi/lo fragments: lane (ln, lg) holds
    //         T'_ik[ln][4 lg + e], the A operand of U_i = sum_k T'_ik R_k
    for (int idx = wave; idx < NTRI; idx += 4) {
        int i = 0;
        while (tri_idx(i + 1, 0) <= idx) ++i;
        const int k = idx - tri_idx(i, 0);
        const f32x4 t = *reinterpret_cast<const f32x4 *>(Ts + (idx * 16 + ln) * AP + 4 * lg);
        const f32x4 bj = *reinterpret_cast<const f32x4 *>(Bes + 16 * k + 4 * lg);
        bf16x4 hv, lv;
        split4(t * bj, hv, lv);
        bf16x4 *tf = reinterpret_cast<bf16x4 *>(out + Rec::oT) + idx * 128;
        tf[lane] = hv;
        tf[64 + lane] = lv;
    }
    // T reuses the K/Q rows: the next item's rows go there after this barrier
    lds_barrier();
    }
}

// Workgroups of the persistent preparation grid: PREP_PER_CU per CU, never
// more than there are records.
int prep_grid(int64_t nrec)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const int64_t g = (int64_t)cus * PREP_PER_CU;
    return (int)(nrec < g ? nrec : g);
}

template <int C, int DK>
hipError_t launch_prep_t(const PrepParams &p, int64_t nrec, hipStream_t stream)
{
    hipLaunchKernelGGL((gdn_chunk_prep_kernel<C, DK>), dim3((unsigned)prep_grid(nrec)), dim3(PREP_THREADS), 0,
                       stream, p);
    return hipGetLastError();
}

template <int C>
hipError_t launch_prep_dk(const PrepParams &p, int64_t Dk, int64_t nrec, hipStream_t s)
{
    switch (Dk) {
    case 16: return launch_prep_t<C, 16>(p, nrec, s);
    case 32: return launch_prep_t<C, 32>(p, nrec, s);
    case 64: return launch_prep_t<C, 64>(p, nrec, s);
    case 128: return launch_prep_t<C, 128>(p, nrec, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_prep(const PrefillArgs &a, hipStream_t stream)
{
    PrepParams p;
    p.k = a.k; p.alpha = a.alpha; p.beta = a.beta; p.ws = a.ws;
    p.T = a.T; p.H = a.H; p.BH = a.B * a.H;
    p.ks = a.k_tok_stride;
    const int64_t nrec = a.B * a.H * ((a.T + a.chunk - 1) / a.chunk);
    switch (a.chunk) {
    case 16: return launch_prep_dk<16>(p, a.Dk, nrec, stream);
    case 32: return launch_prep_dk<32>(p, a.Dk, nrec, stream);
    case 64: return launch_prep_dk<64>(p, a.Dk, nrec, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
