// q8_block.h -- the per-block and per-group arithmetic of the m = 1 matvec,
// shared by its two tile layouts (q8_gemv.hip: a lane per super-row, for
// widths that are not a multiple of 256; q8_gemv_rc.hip: lanes over rows and
// group slots).  Included inside an anonymous namespace by each, so every
// kernel source keeps its own copy.
//
// What is computed (page "IV.4: One command buffer per token", section
// "Eight kernels", q8_matvec): y[r] = sum_b d(r,b) * sum_j q(r,b,j) x[32b+j],
// accumulated within a block and scaled once per block.  The order of every
// sum is fixed here, so all tile layouts round alike:
//   block  S_b = (a0 + a1) + (a2 + a3), chain a_i over quants j = i mod 4;
//   group  g   = fma(d_7, S_7, ... fma(d_1, S_1, fma(d_0, S_0, 0)));
//   row    the groups of a row meet in per-row slots (see kRowSlots).
#pragma once

#include "q8_device.h"

namespace q8 {
namespace {

// Block K (0..7) of a group held in D: d and S = sum_j q_j x_j.  xs is the
// group's x slice in LDS (the same address for every lane of a slice).
template <int K>
__device__ __forceinline__ void block_terms(const uint32_t (&D)[68], const float4 *xs, float &d, float &s) {
    constexpr int sb = K * kBlockBytes;
    d = half_to_float(D[sb >> 2] >> ((sb & 3) * 8));
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int j = 0; j < kQuants; j += 4) {
        const float4 xv = xs[(K * kQuants + j) / 4];
        a0 = fmaf(quant(D, sb + 2 + j + 0), xv.x, a0);
        a1 = fmaf(quant(D, sb + 2 + j + 1), xv.y, a1);
        a2 = fmaf(quant(D, sb + 2 + j + 2), xv.z, a2);
        a3 = fmaf(quant(D, sb + 2 + j + 3), xv.w, a3);
    }
    s = (a0 + a1) + (a2 + a3);
}

// The whole group (eight blocks of one row): its subtotal.
__device__ __forceinline__ float group_sum(const uint32_t (&D)[68], const float4 *xs) {
    float sub = 0.f, d, s;
    block_terms<0>(D, xs, d, s); sub = fmaf(d, s, sub);
    block_terms<1>(D, xs, d, s); sub = fmaf(d, s, sub);
    block_terms<2>(D, xs, d, s); sub = fmaf(d, s, sub);
    block_terms<3>(D, xs, d, s); sub = fmaf(d, s, sub);
    block_terms<4>(D, xs, d, s); sub = fmaf(d, s, sub);
    block_terms<5>(D, xs, d, s); sub = fmaf(d, s, sub);
    block_terms<6>(D, xs, d, s); sub = fmaf(d, s, sub);
    block_terms<7>(D, xs, d, s); sub = fmaf(d, s, sub);
    return sub;
}

// ---------------------------------------------------------------- x as Q8_0
// A group's x slice (256 floats at xa, lane l holding floats 4l..4l+3, of
// block l/8) becomes Q8_0 in place: 32 code bytes per block at xa + 32 b and
// the eight binary16 scales, as floats, at xa + 256.  One wave, no barrier:
// the wave's LDS reads and writes are performed in program order.
__device__ __forceinline__ void quantize_slice(uint8_t *xa, int lane) {
    const float4 v = reinterpret_cast<const float4 *>(xa)[lane];
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = fmaxf(a, __shfl_xor(a, 1, kWave));
    a = fmaxf(a, __shfl_xor(a, 2, kWave));
    a = fmaxf(a, __shfl_xor(a, 4, kWave));
    const float d = xq_scale(a);
    reinterpret_cast<uint32_t *>(xa)[lane] =
        pack4(xq_code(v.x, d), xq_code(v.y, d), xq_code(v.z, d), xq_code(v.w, d));
    if ((lane & 7) == 0) reinterpret_cast<float *>(xa + 256)[lane >> 3] = xq_f16_value(d);
}

// Block K (0..7) of a group with x as Q8_0: the integer dot of the 32 quant
// pairs (eight v_dot4), times the two scales.  Quants of an even block start
// 2 bytes into a dword and are realigned with v_alignbyte.
template <int K>
__device__ __forceinline__ float block_terms_xq(const uint32_t (&D)[68], const uint8_t *xa) {
    constexpr int sb = K * kBlockBytes;
    constexpr int qb = sb + 2;
    const float dw = half_to_float(D[sb >> 2] >> ((sb & 3) * 8));
    const uint4 x0 = reinterpret_cast<const uint4 *>(xa)[2 * K];
    const uint4 x1 = reinterpret_cast<const uint4 *>(xa)[2 * K + 1];
    const float dx = reinterpret_cast<const float *>(xa + 256)[K];
    const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    int isum = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        constexpr int w0 = qb >> 2;
        uint32_t wq;
        if constexpr ((qb & 3) == 0) wq = D[w0 + k];
        else wq = __builtin_amdgcn_alignbyte(D[w0 + k + 1], D[w0 + k], qb & 3);
        isum = __builtin_amdgcn_sdot4((int)wq, (int)xw[k], isum, false);
    }
    return (float)isum * (dw * dx);
}

// The whole group with x as Q8_0: its subtotal (block shares added in order).
__device__ __forceinline__ float group_sum_xq(const uint32_t (&D)[68], const uint8_t *xa) {
    float sub = 0.f;
    sub += block_terms_xq<0>(D, xa);
    sub += block_terms_xq<1>(D, xa);
    sub += block_terms_xq<2>(D, xa);
    sub += block_terms_xq<3>(D, xa);
    sub += block_terms_xq<4>(D, xa);
    sub += block_terms_xq<5>(D, xa);
    sub += block_terms_xq<6>(D, xa);
    sub += block_terms_xq<7>(D, xa);
    return sub;
}

}  // namespace
}  // namespace q8
