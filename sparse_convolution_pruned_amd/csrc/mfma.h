// CDNA4 matrix-core helpers: v_mfma_f32_32x32x16_bf16 operand fragments.
//
// Operand layouts of the 32x32x16 bf16 instruction (64 lanes, l = lane):
//   A (32 rows x 16 k):   lane l holds row (l & 31), k = 8*(l >> 5) .. +7
//   B (16 k x 32 cols):   lane l holds col (l & 31), k = 8*(l >> 5) .. +7
//   D (32 x 32, fp32):    lane l holds col (l & 31); acc[4*g + r] is
//                         row 8*g + 4*(l >> 5) + r,  g, r in 0..3
// Only the pairing of A's and B's k slots matters for the product, and both
// are built with the same k order here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ floatx16_t mfma32(bf16x8_t a, bf16x8_t b, floatx16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx16_t zero16() {
    floatx16_t z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// 8 consecutive bf16 along a contiguous LDS row (16-byte aligned).
__device__ __forceinline__ bf16x8_t frag_row(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

}  // namespace svc
