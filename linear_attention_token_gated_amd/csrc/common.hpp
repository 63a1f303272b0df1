// common.hpp -- shared device helpers for the gfx950 (CDNA4) kernels:
// bf16 conversion, 16x16 MFMA fragments, DPP row broadcast.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// float -> bf16 conversion is round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// Split four floats into bf16 pairs hi = bf16(x), lo = bf16(x - hi), both
// round-to-nearest-even.  Two packed conversions give hi; the widened hi is
// rebuilt from the packed word by a shift (low half) and a mask (high half).
__device__ __forceinline__ void split4(const f32x4 x, bf16x4 &hi, bf16x4 &lo) {
    const bf16x2 h01 = __builtin_convertvector((f32x2{x[0], x[1]}), bf16x2);
    const bf16x2 h23 = __builtin_convertvector((f32x2{x[2], x[3]}), bf16x2);
    const uint32_t u01 = __builtin_bit_cast(uint32_t, h01), u23 = __builtin_bit_cast(uint32_t, h23);
    const f32x2 r01 = f32x2{x[0] - __uint_as_float(u01 << 16), x[1] - __uint_as_float(u01 & 0xffff0000u)};
    const f32x2 r23 = f32x2{x[2] - __uint_as_float(u23 << 16), x[3] - __uint_as_float(u23 & 0xffff0000u)};
    const bf16x2 l01 = __builtin_convertvector(r01, bf16x2);
    const bf16x2 l23 = __builtin_convertvector(r23, bf16x2);
    hi = bf16x4{h01[0], h01[1], h23[0], h23[1]};
    lo = bf16x4{l01[0], l01[1], l23[0], l23[1]};
}

// ---------------------------------------------------------------------------
// 16x16 MFMA tiles.
//
// A tile product D[16x16] += A[16 x KS] * B[KS x 16].  Lane l supplies row
// (l % 16) of A and column (l % 16) of B, each as KS/4 consecutive k values
// starting at k = (l / 16) * KS/4.  Any k-permutation that is the same for A
// and B gives the same sum, so only the row/column ownership matters.  The
// accumulator layout is the hardware one: lane l holds D[4*(l/16) + i][l % 16],
// i = 0..3.
//
//   bf16, KS=32: v_mfma_f32_16x16x32_bf16      (8 bf16 per lane)
//   bf16, KS=16: v_mfma_f32_16x16x16_bf16      (4 bf16 per lane)
//   f32,  KS=16: 4 x v_mfma_f32_16x16x4_f32    (4 f32 per lane)
//   f32,  KS=32: 8 x v_mfma_f32_16x16x4_f32    (8 f32 per lane)
// ---------------------------------------------------------------------------
template <typename OpT, int KS> struct Frag;

template <> struct Frag<__bf16, 32> {
    bf16x8 v;
    __device__ __forceinline__ void load(const __bf16 *p) { v = *reinterpret_cast<const bf16x8 *>(p); }
    __device__ __forceinline__ void set(int e, float x) { v[e] = (__bf16)x; }
    __device__ __forceinline__ void set_raw(int e, __bf16 x) { v[e] = x; }
    static __device__ __forceinline__ f32x4 mma(const Frag &a, const Frag &b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
    }
};

template <> struct Frag<__bf16, 16> {
    bf16x4 v;
    __device__ __forceinline__ void load(const __bf16 *p) { v = *reinterpret_cast<const bf16x4 *>(p); }
    __device__ __forceinline__ void set(int e, float x) { v[e] = (__bf16)x; }
    __device__ __forceinline__ void set_raw(int e, __bf16 x) { v[e] = x; }
    static __device__ __forceinline__ f32x4 mma(const Frag &a, const Frag &b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a.v),
                                                         __builtin_bit_cast(i16x4, b.v), c, 0, 0, 0);
    }
};

template <int KS> struct FragF32 {
    static constexpr int N = KS / 4;
    float v[N];
    __device__ __forceinline__ void load(const float *p) {
#pragma unroll
        for (int e = 0; e < N; e += 4) {
            f32x4 t = *reinterpret_cast<const f32x4 *>(p + e);
            v[e] = t[0]; v[e + 1] = t[1]; v[e + 2] = t[2]; v[e + 3] = t[3];
        }
    }
    __device__ __forceinline__ void set(int e, float x) { v[e] = x; }
    __device__ __forceinline__ void set_raw(int e, float x) { v[e] = x; }
    static __device__ __forceinline__ f32x4 mma(const FragF32 &a, const FragF32 &b, f32x4 c) {
#pragma unroll
        for (int e = 0; e < N; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
        return c;
    }
};
template <> struct Frag<float, 32> : FragF32<32> {};
template <> struct Frag<float, 16> : FragF32<16> {};

// Fragment of rows r0..r0+15 (lane -> row r0 + l%16) and k-range k0..k0+KS-1
// of a row-major matrix with `pitch` elements per row.  Used both for A
// operands (rows of A) and for B operands stored transposed (rows of B^T).
template <typename OpT, int KS>
__device__ __forceinline__ Frag<OpT, KS> frag_rows(const OpT *base, int pitch, int r0, int k0, int lane) {
    Frag<OpT, KS> f;
    f.load(base + (r0 + (lane & 15)) * pitch + k0 + (lane >> 4) * (KS / 4));
    return f;
}

// Same fragment taken from the transpose of a row-major matrix: row r of the
// operand is column r of `base`, so the KS/4 values are gathered down a column.
template <typename OpT, int KS>
__device__ __forceinline__ Frag<OpT, KS> frag_cols(const OpT *base, int pitch, int r0, int k0, int lane) {
    Frag<OpT, KS> f;
    const OpT *p = base + (k0 + (lane >> 4) * (KS / 4)) * pitch + r0 + (lane & 15);
#pragma unroll
    for (int e = 0; e < KS / 4; ++e) f.set_raw(e, p[e * pitch]);
    return f;
}

// Calls f(std::integral_constant<int, i>{}) for i = 0..N-1: loops whose
// index must be a constant expression (if constexpr on it).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F> __device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// log2 of a decay alpha in [0, 1], floored at -126: alpha = 0 (or a subnormal
// alpha) acts as 2^-126, a decay that leaves less than 1.2e-38 of the state,
// instead of -inf, which would turn the decay ratios 2^(G_r - G_j) into NaN.
__device__ __forceinline__ float log2_decay(float alpha) {
    return fmaxf(__builtin_amdgcn_logf(alpha), -126.f);
}

// Broadcast lane S of every 16-lane row to the whole row (DPP row_newbcast).
// Every lane has a valid source, so no old value is needed (bound_ctrl set):
// the move then carries no extra copy and no wait state of its own.
template <int S> __device__ __forceinline__ float row_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + S, 0xF, 0xF, true));
}

constexpr int BV = 16;   // value columns carried by one prefill workgroup

constexpr size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

// LDS row pitch (bf16 elements) for rows of n elements read as 16x16 MFMA
// fragments: 128-bit reads (KS = 32) are free of bank conflicts on gfx950 when
// the pitch is 8 mod 16 dwords, 64-bit reads (KS = 16) when it is 4 mod 8.
template <int KS> constexpr int frag_pitch(int n) {
    int r = n / 2;                                    // dwords
    const int m = KS == 32 ? 16 : 8, want = KS == 32 ? 8 : 4;
    while (r % m != want) ++r;
    return 2 * r;
}

// Value of v in lane l (l wave-uniform).
__device__ __forceinline__ float lane_value(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// v from N lanes lower in the same 16-lane row; lanes with no such source read 0.
template <int N> __device__ __forceinline__ float row_shr(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + N, 0xF, 0xF, false));
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

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


// The same inclusive prefix sum in fp64.  The decay prefixes G_r of a chunk
// are summed in fp64 so that differences G_r - G_j keep their precision when
// the prefix itself is large (several alpha near 0 in one chunk); DPP moves
// 32 bits, so each shift moves the two halves of the double.
template <int N> __device__ __forceinline__ double row_shr_f64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, 0x110 + N, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), 0x110 + N, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double lane_value_f64(double v, int l) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double wave_inclusive_sum_f64(double x, int lane) {
    x += row_shr_f64<1>(x);
    x += row_shr_f64<2>(x);
    x += row_shr_f64<4>(x);
    x += row_shr_f64<8>(x);
    const double t0 = lane_value_f64(x, 15), t1 = lane_value_f64(x, 31), t2 = lane_value_f64(x, 47);
    const int row = lane >> 4;
    const double base = row == 0 ? 0.0 : row == 1 ? t0 : row == 2 ? t0 + t1 : (t0 + t1) + t2;
    return x + base;
}

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

// Workgroup barrier that orders LDS only: this wave's LDS accesses complete
// (lgkmcnt(0)), then s_barrier.  Unlike __syncthreads() it carries no memory
// fence, so global loads in flight (prefetch) and global stores (outputs) are
// not waited for; for kernels whose wavefronts pass values to each other only
// through LDS.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt and expcnt at their maximum, lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace gdn
