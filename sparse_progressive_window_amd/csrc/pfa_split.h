// Three-way bf16 split of fp32 operands for the bf16 matrix cores (gfx950).
//
// x = hi + mid + lo, each part the round-to-nearest-even bf16 of what is left
// (the subtractions are exact in fp32), so |x - (hi + mid + lo)| <= 2^-24 |x|.
// A dot product of two split vectors keeps the six part products down to order
// 2^-16 (lo.hi, mid.mid, hi.lo, mid.hi, hi.mid, hi.hi, smallest first); each
// bf16 x bf16 product is exact in fp32 and the dropped ones (mid.lo, lo.mid,
// lo.lo) are below 2^-26 of |x_c y_c|, so the result is as accurate as fp32
// products, at 6 v_mfma_f32_16x16x32_bf16 per 16x16 tile of 32-long dot
// products instead of 8 v_mfma_f32_16x16x4_f32.
#pragma once

#include "pfa_device.h"

namespace pfa {

typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

template <int NE, class V>
__device__ __forceinline__ void split3(const float* x, V& hi, V& mid, V& lo) {
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        hi[i] = (__bf16)x[i];
        const float r = x[i] - (float)hi[i];
        mid[i] = (__bf16)r;
        lo[i] = (__bf16)(r - (float)mid[i]);
    }
}

// 16x16 tile of 32-long dot products from split operands (A rows a*, B columns b*),
// accumulated onto acc, the small products first.
__device__ __forceinline__ v4f_t dot_split3(const bf8& ah, const bf8& am, const bf8& al, const bf8& bh,
                                            const bf8& bm, const bf8& bl, v4f_t acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, bm, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bm, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
    return acc;
}

// bytes per row of one bf16 plane of a 32-wide tile (64 + 16 pad: the 16-byte
// operand reads of 16 consecutive rows hit distinct banks)
constexpr int kSplitRow = 80;

}  // namespace pfa
