// prep_layout.hpp -- layout of the per-chunk records written by the chunk
// preparation kernel and read by the bf16 recurrence kernel.
//
// One record per (sequence b, head h, chunk c), at index (b * H + h) * NC + c
// of the prefill workspace.  NTRI = NB (NB + 1) / 2 lower-triangular 16x16
// blocks (row block i, column block k <= i) at index i (i + 1) / 2 + k:
//   oT   [NTRI][hi, lo][64 lanes] bf16x4   T' = (I + A)^-1 diag(beta):
//                                           lane (ln, lg) holds T'_ik[ln][4 lg + e]
//                                           (the A-operand fragments of 16x16x16
//                                           bf16 MFMAs)
//   oDec float EG[C], Ed[C], EGC, 15 floats of padding, G[C] (the base-2 decay
//        prefix itself, from which the recurrence forms the decay ratios of P)
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace gdn {

template <int C> struct PrepRecord {
    static constexpr int NB = C / 16;
    static constexpr int NTRI = NB * (NB + 1) / 2;
    static constexpr int DEC = 3 * C + 16;          // floats of the decay block
    static constexpr int DEC_G = 2 * C + 16;        // offset of G in it
    static constexpr size_t oT = 0;
    static constexpr size_t oDec = oT + (size_t)NTRI * 2 * 64 * 8;
    static constexpr size_t BYTES = oDec + (size_t)DEC * 4;
    static_assert(BYTES % 64 == 0, "records stay 64-byte aligned");
};

inline size_t prep_record_bytes(int64_t chunk) {
    switch (chunk) {
    case 16: return PrepRecord<16>::BYTES;
    case 32: return PrepRecord<32>::BYTES;
    case 64: return PrepRecord<64>::BYTES;
    }
    return 0;
}

struct PrepParams {
    const void *k;
    const float *alpha, *beta;
    void *ws;
    int64_t T, H;
    int64_t BH;              // B * H
    int64_t ks;              // token stride (elements)
};

}  // namespace gdn
