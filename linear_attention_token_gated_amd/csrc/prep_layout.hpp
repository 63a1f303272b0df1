// prep_layout.hpp -- layout of the per-chunk records written by the chunk
// preparation kernel and read by the bf16 recurrence kernel.
//
// One record per (sequence b, head h, chunk c), at index (b * H + h) * NC + c
// of the prefill workspace.  NTRI = NB (NB + 1) / 2 lower-triangular 16x16
// blocks (row block i, column block k <= i) at index i (i + 1) / 2 + k:
//   oT   [NTRI][hi, lo][64 lanes] bf16x4   T' = (I + A)^-1 diag(beta):
//                                           lane (ln, lg) holds T'_ik[ln][4 lg + e]
//   oP   [NTRI][hi, lo][64 lanes] bf16x4   P: lane (ln, lg) holds P_ik[ln][4 lg + e]
//   oDec float EG[C], Ed[C], EGC, 15 floats of padding
// Both block arrays hold the A-operand fragments of 16x16x16 bf16 MFMAs.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace gdn {

template <int C> struct PrepRecord {
    static constexpr int NB = C / 16;
    static constexpr int NTRI = NB * (NB + 1) / 2;
    static constexpr size_t oT = 0;
    static constexpr size_t oP = oT + (size_t)NTRI * 2 * 64 * 8;
    static constexpr size_t oDec = oP + (size_t)NTRI * 2 * 64 * 8;
    static constexpr size_t BYTES = oDec + (size_t)(2 * C + 16) * 4;
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
    const void *q, *k;
    const float *alpha, *beta;
    void *ws;
    int64_t T, H;
    int64_t BH;              // B * H
    int64_t qs, ks;          // token strides (elements)
};

}  // namespace gdn
