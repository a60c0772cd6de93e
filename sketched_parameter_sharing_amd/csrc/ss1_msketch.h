// The sketch of two signed sources formed on the matrix cores (the band
// kernel at c = 2 and the group kernel), as a 16x16x32 bf16 MFMA against a
// signed one-hot selection.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace ss1 {
namespace dev {

// ------------------------------------------- sketch on the matrix cores
// The sketch of two signed sources as one 16x16x32 bf16 MFMA,
// D[i][m] = sum_k A[i][k] X[k][m]: the X operand of lane l holds 16 inputs of
// token l%16 from source (l/16)/2, at offsets 16*((l/16)%2) + {0..3, 8..11}
// (first MFMA) or + {4..7, 12..15} (second) of a 32-wide half-step, and A is
// the signed selection that puts input offset o at row i with
// o = 8*(i/4) + i%4 (+4 in the second MFMA).  Row i of lane group q then holds
// sketch column 8q + i%4 (+4), so the two results together are columns
// 8q..8q+7 of the lane's token: the contraction's operand layout.  For lane
// l (row li = l%16, quarter q = l/16) the selection row has one non-zero, at
// element li%8, when li/8 == q%2.  `one` holds bf16 1.0 there, `neg` its sign
// bit.
//
// With `swapped`, lanes of the second source take the other offset half
// (16*((q%2) ^ (q/2))), so that quarter-waves 0 and 2 (and 1 and 3), which may
// be served in the same LDS cycle, read different 16-byte pieces when the two
// sources' rows sit on the same banks; the non-zero then sits where
// li/8 == (q%2) ^ (q/2).
__device__ __forceinline__ void sketch_selector_base(int li, int q, uint4& one, uint4& neg, bool swapped = false) {
    uint32_t o[4] = {0u, 0u, 0u, 0u}, n[4] = {0u, 0u, 0u, 0u};
    if ((li >> 3) == ((q & 1) ^ (swapped ? (q >> 1) : 0))) {
        const int e = li & 7;
        o[e >> 1] = 0x3F80u << (16 * (e & 1));
        n[e >> 1] = 0x8000u << (16 * (e & 1));
    }
    one = make_uint4(o[0], o[1], o[2], o[3]);
    neg = make_uint4(n[0], n[1], n[2], n[3]);
}

// The selection for a source of sign-XOR word sx (0x80008000 for a negative
// sign, else 0) and sign sg (0 for a source a malformed plan leaves absent).
__device__ __forceinline__ uint4 sketch_selector(const uint4& one, const uint4& neg, uint32_t sx, float sg) {
    const uint32_t keep = sg != 0.0f ? 0xFFFFFFFFu : 0u;
    return make_uint4((one.x ^ (neg.x & sx)) & keep, (one.y ^ (neg.y & sx)) & keep,
                      (one.z ^ (neg.z & sx)) & keep, (one.w ^ (neg.w & sx)) & keep);
}

}  // namespace dev
}  // namespace ss1
