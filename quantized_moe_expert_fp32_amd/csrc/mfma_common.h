// Matrix-core helpers shared by the grouped expert GEMMs and the router GEMM.
//
// v_mfma_f32_16x16x32_bf16: lane l supplies A[m = l % 16][8 k values] and
// B[8 k values][n = l % 16] for the k block 8 * (l / 16) .. +8, and receives
// D[m = 4 * (l / 16) + r][n = l % 16] for r = 0..3. The int4 and int8 conversions
// produce B values in natural k order, so activations are used as stored.
#pragma once

#include "moe_internal.h"

namespace moe {

constexpr int A_STRIDE = 72;  // LDS row stride in bf16 of a staged 64 x 64 activation group (64 + 8 padding)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

// B fragment of one 16x32 k-half: four packed int4 bytes -> eight bf16 (1 + q/16).
__device__ __forceinline__ uint4 bfrag(uint32_t qd) {
    uint32_t p[4];
    int4x8_to_bf16_pairs(qd, p);
    return make_uint4(p[0], p[1], p[2], p[3]);
}

// Stages one 64x64 activation group into LDS and its row sums (fp32, fixed
// order). Thread tid covers row tid/4, columns 16*(tid%4) .. +16.
__device__ __forceinline__ void stage_store(uint16_t* __restrict__ a_lds, float* __restrict__ x_lds, int tid,
                                            const uint4& v0, const uint4& v1) {
    const int row = tid >> 2, qq = tid & 3;
    const uint32_t i0[4] = {v0.x, v0.y, v0.z, v0.w};
    const uint32_t i1[4] = {v1.x, v1.y, v1.z, v1.w};
    uint4* dst = reinterpret_cast<uint4*>(a_lds + row * A_STRIDE + 16 * qq);
    dst[0] = v0;
    dst[1] = v1;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        s += bf16_to_f32(i0[j] & 0xFFFFu);
        s += bf16_to_f32(i0[j] >> 16);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        s += bf16_to_f32(i1[j] & 0xFFFFu);
        s += bf16_to_f32(i1[j] >> 16);
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (qq == 0) x_lds[row] = s;
}

// Eight int8 codes (two dwords) as four bf16 pairs in natural order; every code
// 0..255 is exact in bf16.
__device__ __forceinline__ uint4 int8x8_to_bf16_pairs(uint32_t d0, uint32_t d1) {
    const uint32_t f0 = __float_as_uint((float)((d0 >> 0) & 0xFFu));
    const uint32_t f1 = __float_as_uint((float)((d0 >> 8) & 0xFFu));
    const uint32_t f2 = __float_as_uint((float)((d0 >> 16) & 0xFFu));
    const uint32_t f3 = __float_as_uint((float)((d0 >> 24) & 0xFFu));
    const uint32_t f4 = __float_as_uint((float)((d1 >> 0) & 0xFFu));
    const uint32_t f5 = __float_as_uint((float)((d1 >> 8) & 0xFFu));
    const uint32_t f6 = __float_as_uint((float)((d1 >> 16) & 0xFFu));
    const uint32_t f7 = __float_as_uint((float)((d1 >> 24) & 0xFFu));
    // high halves of two floats: low16 = hi(a), high16 = hi(b)
    return make_uint4(__builtin_amdgcn_perm(f1, f0, 0x07060302u), __builtin_amdgcn_perm(f3, f2, 0x07060302u),
                      __builtin_amdgcn_perm(f5, f4, 0x07060302u), __builtin_amdgcn_perm(f7, f6, 0x07060302u));
}

}  // namespace moe
