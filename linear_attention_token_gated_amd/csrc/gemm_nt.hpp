// gemm_nt.hpp -- the library's bf16 GEMM tile, C = A B^T with fp32
// accumulation, as a device function: the layer's projections launch it on
// its own (layer.hip), and the layer's fp32 core shares a launch with one
// projection (backward.hip), its tiles on the compute units the core leaves
// free.
#pragma once

#include "common.hpp"

namespace gdn {

namespace {

// ---------------------------------------------------------------------------
// C[M, N] = A[M, K] * B[N, K]^T, bf16 operands, fp32 accumulation.
// A BM x BN workgroup tile, NW wavefronts in a (NW/2) x 2 grid of
// (2 BM/NW) x (BN/2), K steps of 32 on 16x16x32 MFMAs.  The K-step tiles of A and B reach LDS
// through buffer loads that write LDS directly, three steps ahead into four
// stages; the fragments of step k+1 are read while the MFMAs of step k run.
// Every output element sums its K in the same order (32-wide steps, ascending)
// whatever the tile size, so a product of a few rows equals, bit for bit, the
// same rows of a taller product.
// Rows (64 bytes) are stored unpadded, 16-byte granule g of row r at position
// g ^ s(r), s(r) = ((r / 2) ^ (r / 4)) mod 4: any 8 consecutive rows of a
// fragment read then cover 128 bytes of banks once and the 16 rows of it 256
// bytes once, so the read is conflict-free whether the LDS serves 8 or 16
// lanes of a 16-byte read per pass.  Rows past M / N lie outside the
// buffer range of the load and k past K gets an offset outside it: both read
// as zeros.  K must be a multiple of 8.
// ---------------------------------------------------------------------------
constexpr int GBK = 32;
constexpr uint32_t G_OOB = 0x7FFFFFF0u;

typedef __attribute__((address_space(3))) void *glds_ptr;
__device__ __forceinline__ void gload_lds(const void *base, uint32_t nrec, uint32_t voff, void *dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)nrec, 0x00020000),
        (glds_ptr)(uintptr_t)(uint32_t)(uintptr_t)dst, 16, voff, 0, 0, 0);
}

// NW wavefronts in a (NW / 2) x 2 grid over the BM x BN tile
template <int BM, int BN, int NW> struct GemmTile {
    static constexpr int WGM = NW / 2;
    static constexpr int MI = BM / (16 * WGM), NJ = BN / 32;  // 16 x 16 tiles per wave
    static constexpr int ATILE = BM * GBK * 2, BTILE = BN * GBK * 2;
    static constexpr int STAGE = ATILE + BTILE;
    static constexpr int LA = BM / (16 * NW), LB = BN / (16 * NW);   // 1 KB loads per thread per stage
    static constexpr int LOADS = LA + LB;
    static_assert(LA >= 1 && LB >= 1, "every wave loads rows of both tiles");
};

// Up to three products of one A in one launch, C_p = A B_p^T: column tiles
// [0, tile_end[0]) belong to product 0, [tile_end[0], tile_end[1]) to product
// 1, [tile_end[1], tile_end[2]) to product 2 (an absent product has no tiles).
template <typename OutT> struct GemmProducts {
    const __bf16 *B[3];
    OutT *C[3];
    int N[3];
    int64_t ldb[3], ldc[3];
    int tile_end[3];
};

// K cut into splits of whole K steps: split s sums K steps s * steps ..
// s * steps + steps - 1 and writes its partial product at C_p + s * M * ldc_p
// (steps = 0: one split, all of K).  The consumer adds the partials in split
// order.
struct GemmSplit {
    int steps = 0, split = 0;
};

// One workgroup's tile (pid: its index in the GEMM's grid, smem: ST * STAGE
// bytes of LDS, 1024-byte aligned).  ST stages of K steps in LDS (a power of
// two >= 4), ST - 1 of them in flight; NW wavefronts.  tiles_n: column tiles of
// every product together.
template <typename OutT, int BM, int BN, int ST, int NW>
__device__ __forceinline__ void gemm_nt_block(int pid, char *smem, const __bf16 *__restrict__ A, int M, int K,
                                              int64_t lda, const GemmProducts<OutT> &P, int tiles_m, int tiles_n,
                                              int bn_log, GemmSplit sp = GemmSplit{})
{
    using G = GemmTile<BM, BN, NW>;
    constexpr int WGM = G::WGM;
    constexpr int MI = G::MI, NJ = G::NJ, LA = G::LA, LB = G::LB;
    static_assert(ST >= 4 && (ST & (ST - 1)) == 0 && (ST - 2) * G::LOADS < 64, "stages");
    const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(wave_id());
    const int ln = lane & 15, lg = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;

    // Tile order: workgroups are dispatched to the 8 XCDs in turn, so workgroup
    // 8 j + x runs on XCD x; XCD x takes blocks of 32 / bn x bn tiles (rows x
    // columns, bn = 2^bn_log <= 8), block 8 (j / 32) + x, tile j % 32 of it.  The
    // 32 workgroups of an XCD then share a few rows of A tiles and columns of B
    // tiles in its L2.  Tiles past the grid (blocks padded to a multiple of 8)
    // end at once.
    int tm, tn;
    {
        const int x = pid & 7, j = pid >> 3;
        const int blk = 8 * (j >> 5) + x, t = j & 31;
        const int bn = 1 << bn_log, bm = 32 >> bn_log;
        const int bpr = (tiles_n + bn - 1) / bn;                // blocks per block-row
        tm = (blk / bpr) * bm + (t >> bn_log);
        tn = (blk % bpr) * bn + (t & (bn - 1));
        if (tm >= tiles_m || tn >= tiles_n) return;
    }
    const int pi = tn < P.tile_end[0] ? 0 : (tn < P.tile_end[1] ? 1 : 2);
    const __bf16 *Bm = P.B[pi];
    OutT *Cm = P.C[pi];
    const int N = P.N[pi];
    const int64_t ldb = P.ldb[pi], ldc = P.ldc[pi];
    if (pi > 0) tn -= P.tile_end[pi - 1];
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t mrows = M - m0 < BM ? M - m0 : BM, nrows = N - n0 < BN ? N - n0 : BN;
    // this split's K steps: kbase .. kbase + ntk - 1
    const int ntk_all = (K + GBK - 1) / GBK;
    const int kbase = sp.steps ? sp.split * sp.steps : 0;
    const int ntk = sp.steps ? (ntk_all - kbase < sp.steps ? ntk_all - kbase : sp.steps) : ntk_all;
    Cm += (int64_t)sp.split * M * ldc;

    // load t of this wave moves tile rows 16 i .. 16 i + 15 (i = wave + 4 t): lane
    // -> row 16 i + lane / 4, LDS granule position lane % 4, which holds granule
    // (lane % 4) ^ s(lane / 4) of the row
    const int gk = 8 * ((lane & 3) ^ (((lane >> 3) ^ (lane >> 4)) & 3));   // k offset of the lane's granule
    uint32_t roff_a[LA], roff_b[LB];
#pragma unroll
    for (int t = 0; t < LA; ++t) roff_a[t] = (uint32_t)((16 * (wave + NW * t) + (lane >> 2)) * lda * 2 + gk * 2);
#pragma unroll
    for (int t = 0; t < LB; ++t) roff_b[t] = (uint32_t)((16 * (wave + NW * t) + (lane >> 2)) * ldb * 2 + gk * 2);
    auto issue = [&](int kt, int stage) {
        const int k0 = (kbase + kt) * GBK;
        char *sa = smem + stage * G::STAGE, *sb = sa + G::ATILE;
        const __bf16 *ba = A + m0 * lda + k0, *bb = Bm + n0 * ldb + k0;
        const uint32_t na = (uint32_t)((mrows * lda - k0) * 2), nb = (uint32_t)((nrows * ldb - k0) * 2);
        // granules past K: an offset outside the range (a select, not a branch)
        const uint32_t oob = k0 + gk < K ? 0u : G_OOB;
#pragma unroll
        for (int t = 0; t < LA; ++t) gload_lds(ba, na, roff_a[t] | oob, sa + (wave + NW * t) * 1024);
#pragma unroll
        for (int t = 0; t < LB; ++t) gload_lds(bb, nb, roff_b[t] | oob, sb + (wave + NW * t) * 1024);
    };
    // fragment of rows r0 + ln, k 8 lg .. 8 lg + 7 (r0 a multiple of 16)
    const int fpos = 8 * (lg ^ (((ln >> 1) ^ (ln >> 2)) & 3));
    using F = Frag<__bf16, 32>;
    auto read_frags = [&](int stage, F (&af)[MI], F (&bf)[NJ]) {
        const __bf16 *As = reinterpret_cast<const __bf16 *>(smem + stage * G::STAGE);
        const __bf16 *Bs = reinterpret_cast<const __bf16 *>(smem + stage * G::STAGE + G::ATILE);
#pragma unroll
        for (int i = 0; i < MI; ++i) af[i].load(As + (wm * (BM / WGM) + 16 * i + ln) * GBK + fpos);
#pragma unroll
        for (int j = 0; j < NJ; ++j) bf[j].load(Bs + (wn * (BN / 2) + 16 * j + ln) * GBK + fpos);
    };

    f32x4 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = zero4();
    auto mmas = [&](const F (&af)[MI], const F (&bf)[NJ]) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[i][j] = F::mma(af[i], bf[j], acc[i][j]);
    };
    // vmcnt(n) with expcnt and lgkmcnt left alone
    auto wait_vm = [&](auto n_c) {
        constexpr int n = decltype(n_c)::value;
        __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
    };
    auto barrier = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    constexpr int L = G::LOADS;
    auto last = [&](int kt) { return kt < ntk ? kt : ntk - 1; };   // past the end: the last tile again

    // tiles 0 .. ST-2 in flight; tile 0 landed for every wave, its fragments read
    static_for<ST - 1>([&](auto t_c) {
        constexpr int t = decltype(t_c)::value;
        issue(last(t), t);
    });
    wait_vm(std::integral_constant<int, (ST - 2) * L>{});
    barrier();
    F fa[2][MI], fb[2][NJ];
    read_frags(0, fa[0], fb[0]);
    // step kt: tile kt+1 landed for every wave (tiles kt+2 .. kt+ST-2 may be in
    // flight); tile kt+ST-1 goes to the stage of tile kt-1, read before the
    // barrier of step kt-1; the fragments of kt+1 are read while the MFMAs of
    // kt run
    auto step = [&](int kt, auto cur_c) {
        constexpr int cur = decltype(cur_c)::value;
        wait_vm(std::integral_constant<int, (ST - 3) * L>{});
        barrier();
        issue(last(kt + ST - 1), (kt + ST - 1) & (ST - 1));
        if (kt + 1 < ntk) read_frags((kt + 1) & (ST - 1), fa[cur ^ 1], fb[cur ^ 1]);
        mmas(fa[cur], fb[cur]);
        // interleave: the loads into LDS and the fragment reads between the MFMAs
        // (with one wavefront per SIMD; with two the SIMD interleaves them)
        if constexpr (NW == 4) static_for<L>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      // VMEM read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
        });
        if constexpr (NW == 4) static_for<MI + NJ>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // DS read
            __builtin_amdgcn_sched_group_barrier(0x008, (MI * NJ - L) / (MI + NJ), 0);
        });
    };
    int kt = 0;
    for (; kt + 1 < ntk; kt += 2) {
        step(kt, std::integral_constant<int, 0>{});
        step(kt + 1, std::integral_constant<int, 1>{});
    }
    if (kt < ntk) step(kt, std::integral_constant<int, 0>{});
    // no LDS write may land after the workgroup ends
    wait_vm(std::integral_constant<int, 0>{});

#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int64_t col = n0 + wn * (BN / 2) + 16 * j + ln;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = m0 + wm * (BM / WGM) + 16 * i + 4 * lg + e;
                if (row < M && col < N) Cm[row * ldc + col] = from_f32<OutT>(acc[i][j][e]);
            }
        }
}

// Grid of a GEMM launch: tiles_m x tiles_n tiles of BM x BN, XCD blocks of
// 32 tiles (bn_log: log2 of the columns of a block), a multiple of 8 blocks.
template <int BM, int BN> struct GemmGrid {
    int tiles_m, tiles_n, bn_log;
    int tile_end[3];
    int64_t grid;
    GemmGrid(int64_t M, int64_t N, int64_t N2 = 0, int64_t N3 = 0) {
        tiles_m = (int)((M + BM - 1) / BM);
        tile_end[0] = (int)((N + BN - 1) / BN);
        tile_end[1] = tile_end[0] + (int)((N2 + BN - 1) / BN);
        tile_end[2] = tile_end[1] + (int)((N3 + BN - 1) / BN);
        tiles_n = tile_end[2];
        bn_log = 0;
        while (bn_log < 3 && (2 << bn_log) <= tiles_n) ++bn_log;
        const int bn = 1 << bn_log, bm = 32 >> bn_log;
        const int64_t blocks = (int64_t)((tiles_m + bm - 1) / bm) * ((tiles_n + bn - 1) / bn);
        grid = (blocks + 7) / 8 * 8 * 32;                 // 32 tiles a block, blocks a multiple of 8
    }
};

// One product of a launch: C[M, N] = A B^T with B [N, K] (rows ldb apart)
// and C rows ldc apart
template <typename OutT> struct GemmOp {
    const __bf16 *B = nullptr;
    OutT *C = nullptr;
    int64_t N = 0, ldb = 0, ldc = 0;
};

// The products of a launch on grid g (built with the same N, N2, N3); an
// absent product keeps the first one's pointers and has no tiles.
template <typename OutT, int BM, int BN>
GemmProducts<OutT> gemm_products(const GemmGrid<BM, BN> &g, const GemmOp<OutT> &p0, GemmOp<OutT> p1 = {},
                                 GemmOp<OutT> p2 = {})
{
    if (!p1.B) { p1 = p0; p1.N = 0; }
    if (!p2.B) { p2 = p0; p2.N = 0; }
    const GemmOp<OutT> *ops[3] = {&p0, &p1, &p2};
    GemmProducts<OutT> P;
    for (int i = 0; i < 3; ++i) {
        P.B[i] = ops[i]->B; P.C[i] = ops[i]->C; P.N[i] = (int)ops[i]->N;
        P.ldb[i] = ops[i]->ldb; P.ldc[i] = ops[i]->ldc; P.tile_end[i] = g.tile_end[i];
    }
    return P;
}

}  // namespace

}  // namespace gdn
