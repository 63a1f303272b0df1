// decode.hip -- single-token gated delta rule on stored fp32 states.
//
// Source: "On the Design of Qwen3.8-Next Architecture", picx.dev summary,
// "Theoretical foundations", eqs (1)-(4), applied to one new token per
// sequence; the fixed-size state is the whole memory of the prefix.
//
// Eqs (1)-(4) for one token rewritten so that the state is read once and
// written once:
//     a = S^T k,  b = S^T q,  kq = k . q            (one pass over S)
//     e = v - alpha a                               (eq (2), decayed state)
//     y = S_t^T q = alpha b + beta kq e             (eq (4) after eq (3))
//     S <- alpha S + beta k e^T                     (eqs (1), (3))
//
// One workgroup per (sequence, head).  Each thread owns 4 consecutive
// columns (one float4) of RPT rows of the Dk x Dv state (RPT = 4 for states of
// 64 float4 or more), so a wavefront reads and writes whole contiguous rows
// (coalesced dwordx4).  The state is streamed
// with non-temporal loads/stores: every element is touched once per step.
#include "common.hpp"
#include "launch.hpp"

namespace gdn {

template <int DK, int DV> struct DecodeShape {
    static constexpr int CG = DV / 4;                       // float4 columns per row
    static constexpr int TOTAL4 = DK * DV / 4;              // float4 per state
    // four float4 rows per thread: measured fastest for 128x128 states on
    // MI355X (1024 threads, 5.8 TB/s of state traffic vs 5.6 at 256 threads)
    static constexpr int NT = TOTAL4 / 4 >= 1024 ? 1024 : (TOTAL4 / 4 < 64 ? (TOTAL4 < 64 ? TOTAL4 : 64) : TOTAL4 / 4);
    static constexpr int RG = NT / CG;                      // row groups
    static constexpr int RPT = DK / RG;                     // rows per thread
    static constexpr int NWAVE = (NT + 63) / 64;
    static_assert(NT % CG == 0 && DK % RG == 0, "decode tiling");
};

template <typename Tin, int DK, int DV>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NT)) void gdn_decode_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta,
    float *__restrict__ state, float *__restrict__ y, int H, int64_t qn, int64_t kn, int64_t vn)
{
    using Sh = DecodeShape<DK, DV>;
    constexpr int CG = Sh::CG, RG = Sh::RG, RPT = Sh::RPT, NT = Sh::NT;
    const int64_t nh = blockIdx.x;
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;

    __shared__ float sk[DK], sq[DK], sv[DV];
    __shared__ f32x4 red_a[Sh::NWAVE][CG], red_b[Sh::NWAVE][CG];
    __shared__ float red_kq[Sh::NWAVE];

    f32x4 *S4 = reinterpret_cast<f32x4 *>(state + nh * (int64_t)(DK * DV));
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = __builtin_nontemporal_load(S4 + (rg + RG * i) * CG + cg);

    // sequence n = nh / H, head nh % H; qn, kn, vn: elements between sequences
    const int64_t n = nh / H, hh = nh % H;
    for (int i = tid; i < DK; i += NT) {
        sk[i] = to_f32(k[n * kn + hh * DK + i]);
        sq[i] = to_f32(q[n * qn + hh * DK + i]);
    }
    for (int i = tid; i < DV; i += NT) sv[i] = to_f32(v[n * vn + hh * DV + i]);
    const float a_t = alpha[nh];
    const float b_t = beta[nh];
    __syncthreads();

    // partial S^T k, S^T q over this thread's rows; k.q over rows (column group 0 only)
    f32x4 pa = zero4(), pb = zero4();
    float pkq = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        const float kr = sk[r], qr = sq[r];
        pa += s[i] * kr;
        pb += s[i] * qr;
        if (cg == 0) pkq += kr * qr;
    }
    // reduce over row groups: first inside the wavefront (lanes CG apart)...
#pragma unroll
    for (int off = CG; off < 64 && off < NT; off <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pa[c] += __shfl_xor(pa[c], off);
            pb[c] += __shfl_xor(pb[c], off);
        }
        pkq += __shfl_xor(pkq, off);
    }
    // ...then across wavefronts through LDS
    const int lane = tid & 63, wave = tid >> 6;
    if (lane < CG) {
        red_a[wave][lane] = pa;
        red_b[wave][lane] = pb;
        if (lane == 0) red_kq[wave] = pkq;
    }
    __syncthreads();
    f32x4 A = zero4(), Bq = zero4();
    float kq = 0.f;
#pragma unroll
    for (int w = 0; w < Sh::NWAVE; ++w) {
        A += red_a[w][cg];
        Bq += red_b[w][cg];
        kq += red_kq[w];
    }

    const f32x4 vv = *reinterpret_cast<const f32x4 *>(&sv[4 * cg]);
    const f32x4 e = vv - a_t * A;                 // eq (2) on the decayed state
    const f32x4 yv = a_t * Bq + (b_t * kq) * e;   // eq (4) on the updated state
    if (rg == 0) *reinterpret_cast<f32x4 *>(y + nh * DV + 4 * cg) = yv;

#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        const f32x4 sn = a_t * s[i] + (b_t * sk[r]) * e;   // eqs (1), (3)
        __builtin_nontemporal_store(sn, S4 + r * CG + cg);
    }
}

// T consecutive tokens of one (sequence, head) from a stored state, with the
// state after every token written out (verification of drafted tokens: the
// caller keeps the state after the accepted prefix).  The same step as
// gdn_decode_kernel, token after token, the state held in registers: read
// once, written T times (one snapshot per token).
//   q, k [N, T, H, DK]; v [N, T, H, DV]; alpha, beta [N, T, H]
//   s_in [N, H, DK, DV] (not modified); s_out [N, T, H, DK, DV]; y [N, T, H, DV]
template <typename Tin, int DK, int DV>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NT)) void gdn_verify_kernel(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
    const float *__restrict__ alpha, const float *__restrict__ beta, const float *__restrict__ s_in,
    float *__restrict__ s_out, float *__restrict__ y, int H, int T)
{
    using Sh = DecodeShape<DK, DV>;
    constexpr int CG = Sh::CG, RG = Sh::RG, RPT = Sh::RPT, NT = Sh::NT;
    const int64_t nh = blockIdx.x, n = nh / H, hh = nh % H;
    const int tid = threadIdx.x;
    const int cg = tid % CG;
    const int rg = tid / CG;
    const int lane = tid & 63, wave = tid >> 6;

    __shared__ float sk[DK], sq[DK], sv[DV];
    __shared__ f32x4 red_a[Sh::NWAVE][CG], red_b[Sh::NWAVE][CG];
    __shared__ float red_kq[Sh::NWAVE];

    const f32x4 *S4 = reinterpret_cast<const f32x4 *>(s_in + nh * (int64_t)(DK * DV));
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = __builtin_nontemporal_load(S4 + (rg + RG * i) * CG + cg);

    for (int t = 0; t < T; ++t) {
        const int64_t tok = (n * T + t) * H + hh;          // (n, t, h)
        // barriers order LDS only: the previous token's state and y stores
        // stay in flight across them (no wavefront reads what another stored)
        lds_barrier();                                     // the previous token's k, q, v are consumed
        for (int i = tid; i < DK; i += NT) {
            sk[i] = to_f32(k[tok * DK + i]);
            sq[i] = to_f32(q[tok * DK + i]);
        }
        for (int i = tid; i < DV; i += NT) sv[i] = to_f32(v[tok * DV + i]);
        const float a_t = alpha[tok];
        const float b_t = beta[tok];
        lds_barrier();

        f32x4 pa = zero4(), pb = zero4();
        float pkq = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + RG * i;
            const float kr = sk[r], qr = sq[r];
            pa += s[i] * kr;
            pb += s[i] * qr;
            if (cg == 0) pkq += kr * qr;
        }
#pragma unroll
        for (int off = CG; off < 64 && off < NT; off <<= 1) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                pa[c] += __shfl_xor(pa[c], off);
                pb[c] += __shfl_xor(pb[c], off);
            }
            pkq += __shfl_xor(pkq, off);
        }
        if (lane < CG) {
            red_a[wave][lane] = pa;
            red_b[wave][lane] = pb;
            if (lane == 0) red_kq[wave] = pkq;
        }
        lds_barrier();
        f32x4 A = zero4(), Bq = zero4();
        float kq = 0.f;
#pragma unroll
        for (int w = 0; w < Sh::NWAVE; ++w) {
            A += red_a[w][cg];
            Bq += red_b[w][cg];
            kq += red_kq[w];
        }
        const f32x4 vv = *reinterpret_cast<const f32x4 *>(&sv[4 * cg]);
        const f32x4 e = vv - a_t * A;
        const f32x4 yv = a_t * Bq + (b_t * kq) * e;
        if (rg == 0) *reinterpret_cast<f32x4 *>(y + tok * DV + 4 * cg) = yv;
        f32x4 *O4 = reinterpret_cast<f32x4 *>(s_out + tok * (int64_t)(DK * DV));
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = rg + RG * i;
            s[i] = a_t * s[i] + (b_t * sk[r]) * e;
            __builtin_nontemporal_store(s[i], O4 + r * CG + cg);
        }
    }
}

template <typename Tin, int DK, int DV>
static hipError_t launch_verify_t(const VerifyArgs &a, hipStream_t stream)
{
    using Sh = DecodeShape<DK, DV>;
    hipLaunchKernelGGL((gdn_verify_kernel<Tin, DK, DV>), dim3((unsigned)(a.N * a.H)), dim3(Sh::NT), 0, stream,
                       (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v, a.alpha, a.beta, a.s_in, a.s_out, a.y,
                       (int)a.H, (int)a.T);
    return hipGetLastError();
}

template <typename Tin, int DK>
static hipError_t launch_verify_dv(const VerifyArgs &a, hipStream_t s)
{
    switch (a.Dv) {
    case 16: return launch_verify_t<Tin, DK, 16>(a, s);
    case 32: return launch_verify_t<Tin, DK, 32>(a, s);
    case 64: return launch_verify_t<Tin, DK, 64>(a, s);
    case 128: return launch_verify_t<Tin, DK, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename Tin>
static hipError_t launch_verify_dk(const VerifyArgs &a, hipStream_t s)
{
    switch (a.Dk) {
    case 16: return launch_verify_dv<Tin, 16>(a, s);
    case 32: return launch_verify_dv<Tin, 32>(a, s);
    case 64: return launch_verify_dv<Tin, 64>(a, s);
    case 128: return launch_verify_dv<Tin, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename Tin, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream)
{
    using Sh = DecodeShape<DK, DV>;
    const int64_t grid = a.N * a.H;
    hipLaunchKernelGGL((gdn_decode_kernel<Tin, DK, DV>), dim3((unsigned)grid), dim3(Sh::NT), 0, stream,
                       (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v, a.alpha, a.beta,
                       a.state, a.y, (int)a.H, a.q_seq_stride ? a.q_seq_stride : a.H * DK,
                       a.k_seq_stride ? a.k_seq_stride : a.H * DK, a.v_seq_stride ? a.v_seq_stride : a.H * DV);
    return hipGetLastError();
}

template <typename Tin, int DK>
static hipError_t launch_decode_dv(const DecodeArgs &a, hipStream_t s)
{
    switch (a.Dv) {
    case 16: return launch_decode_t<Tin, DK, 16>(a, s);
    case 32: return launch_decode_t<Tin, DK, 32>(a, s);
    case 64: return launch_decode_t<Tin, DK, 64>(a, s);
    case 128: return launch_decode_t<Tin, DK, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename Tin>
static hipError_t launch_decode_dk(const DecodeArgs &a, hipStream_t s)
{
    switch (a.Dk) {
    case 16: return launch_decode_dv<Tin, 16>(a, s);
    case 32: return launch_decode_dv<Tin, 32>(a, s);
    case 64: return launch_decode_dv<Tin, 64>(a, s);
    case 128: return launch_decode_dv<Tin, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream)
{
    if (a.N * a.H == 0) return hipSuccess;
    return a.bf16 ? launch_decode_dk<__bf16>(a, stream) : launch_decode_dk<float>(a, stream);
}

hipError_t launch_verify(const VerifyArgs &a, hipStream_t stream)
{
    if (a.N * a.H == 0 || a.T == 0) return hipSuccess;
    return a.bf16 ? launch_verify_dk<__bf16>(a, stream) : launch_verify_dk<float>(a, stream);
}

}  // namespace gdn
