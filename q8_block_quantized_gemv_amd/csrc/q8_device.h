// q8_device.h -- device helpers shared by the matvec (q8_gemv.hip) and the
// small-batch kernels (q8_gemm.hip): lane bookkeeping, the direct
// HBM -> LDS loads, the 17-chunk group layout, the per-row summation slots
// and the generic path for tail rows.  Included by one kernel source each,
// inside an anonymous namespace, so each keeps its own copy.
#pragma once

#include "q8_internal.h"

namespace q8 {
namespace {

typedef const __attribute__((address_space(1))) uint16_t GHalf;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

// binary16 bit pattern in the low half of v -> float (v_cvt_f32_f16; exact,
// subnormals included, Inf/NaN propagate).
__device__ __forceinline__ float half_to_float(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}

// Signed quant at byte `idx` of the group held in D (idx is a constant after
// unrolling, so this is one v_cvt_f32_i32 with an SDWA sign-extended byte).
__device__ __forceinline__ float quant(const uint32_t (&D)[68], int idx) {
    return (float)(int8_t)(D[idx >> 2] >> ((idx & 3) * 8));
}

// Per-lane byte offsets (from the wave's first super-row) of the 17 chunks
// this lane moves for each group: load i of lane l carries chunk c of local
// super-row s where 17*s + c = 64*i + l, so that lane l later finds its own
// super-row's 272 bytes at LDS offset 272*l.  Super-rows past `last` are
// clamped to `last` (their results are never stored).
__device__ __forceinline__ void chunk_offsets(uint32_t (&off)[kGroupChunks], int lane,
                                              int last, int64_t sr_bytes) {
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i) {
        const int slot = kWave * i + lane;
        int s = slot / kGroupChunks;
        const int c = slot - s * kGroupChunks;
        s = s < last ? s : last;
        off[i] = (uint32_t)((int64_t)s * sr_bytes + 16 * c);
    }
}

// A pointer that is the same in every lane, made visibly so for the
// compiler (it goes into a scalar register pair).
__device__ __forceinline__ const uint8_t *uniform_ptr(const uint8_t *p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const uint8_t *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// The kernels issue their direct loads from inline asm.  The compiler tracks
// LDS-DMA it emits itself and, unable to tell the two stages apart, waits
// for ALL outstanding loads before any LDS read -- which would stall every
// compute phase on the next group's loads.  Issued from asm, the loads are
// invisible to that tracking, and the kernel orders them itself: wait_vm_asm
// (a memory barrier for the compiler) before a stage is read, and a stage is
// refilled only after its last read.  m0 carries the LDS address; nothing
// else in these kernels uses m0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane: global (sbase + voff) -> LDS (m0 + 16 * lane).  sbase
// must be the same in every lane (it is taken from the first).
__device__ __forceinline__ void dma16_s(const uint8_t *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds), "v"(voff), "s"(uniform_ptr(sbase)) : "memory", "m0");
}
// the same with the non-temporal hint (streaming data read once)
__device__ __forceinline__ void dma16_s_nt(const uint8_t *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :: "s"(lds), "v"(voff), "s"(uniform_ptr(sbase)) : "memory", "m0");
}
// 16 bytes per lane: global (per-lane address) -> LDS (m0 + 16 * lane)
__device__ __forceinline__ void dma16_v(const void *addr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(lds), "v"(addr) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vm_asm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}

// This lane's 272 bytes of a staged group -> 68 dwords.
__device__ __forceinline__ void read_group(const uint8_t *st, int lane, uint32_t (&D)[68]) {
    const uint4 *src = reinterpret_cast<const uint4 *>(st + kGroupBytes * lane);
#pragma unroll
    for (int c = 0; c < kGroupChunks; ++c) {
        const uint4 v = src[c];
        D[4 * c + 0] = v.x;
        D[4 * c + 1] = v.y;
        D[4 * c + 2] = v.z;
        D[4 * c + 3] = v.w;
    }
}

// direct loads per group of the matvec: 17 of W and one of x
constexpr int kLoadsPerGroup = kGroupChunks + 1;

// Where lane `lane` finds its 16 bytes of the x slice of group kk: floats
// 4*(lane%8) .. +3 of block lane/8 of the group, i.e. of column block
// (8*kk + lane/8) mod nb (a group of a super-row wraps past the row end).
template <int RS>
__device__ __forceinline__ const float *x_slice_src(const OpDesc &op, const float *base, int kk,
                                                    int lane) {
    int b = kk * kGroupBlocks + (lane >> 3);
    if (RS > 1) b %= op.nb;
    return base + (int64_t)b * kQuants + 4 * (lane & 7);
}

// One group: 17 loads of W and one load of its x slice (at st + kStageW).
template <int RS>
__device__ __forceinline__ void dma_group_x(const uint8_t *g, const uint32_t (&off)[kGroupChunks],
                                            uint8_t *st, const OpDesc &op, int kk, int lane) {
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(st));
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i) dma16_s(g, off[i], l0 + kWave * 16 * i);
    dma16_v(x_slice_src<RS>(op, op.x, kk, lane), l0 + kStageW);
}

// The SwiGLU product, as the step's silu_hadamard kernel computes it.
__device__ __forceinline__ float silu_up(float g, float u) { return (g / (1.0f + expf(-g))) * u; }

// kXNormAdd: the squared norm of s = x + x_res over the op's n columns is
// summed in kNormParts contiguous parts of its float4s; within a part lane l
// takes float4s lo + l, lo + l + 64, ... in increasing order and the lanes
// meet in a fixed butterfly; the parts are then added in part order.  Each
// part's sum is the same bits whichever wave computes it and however many
// loads it keeps in flight, so inv does not depend on the launch shape.
constexpr int kNormParts = 4;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;   // the same in every lane: each step adds a pair in both lanes
}

// Part `part` of kNormParts (and, with `write`, that part of s stored to
// x_out); returns the part's sum in every lane.
__device__ __forceinline__ float norm_add_part(const OpDesc &op, int lane, int part, int nparts, bool write) {
    constexpr int B = 8;   // float4 pairs in flight per lane
    const int n = op.nb * kQuants, nv = n / 4;
    const int lo = (int)((int64_t)nv * part / nparts), hi = (int)((int64_t)nv * (part + 1) / nparts);
    const float4 *a4 = reinterpret_cast<const float4 *>(op.x);
    const float4 *r4 = reinterpret_cast<const float4 *>(op.x_res);
    float4 *o4 = reinterpret_cast<float4 *>(op.x_out);
    float ss = 0.f;
    for (int i0 = lo; i0 < hi; i0 += kWave * B) {
        float4 a[B], r[B];
#pragma unroll
        for (int e = 0; e < B; ++e) {
            const int i = i0 + lane + kWave * e;
            a[e] = make_float4(0.f, 0.f, 0.f, 0.f);
            r[e] = a[e];
            if (i < hi) {
                a[e] = a4[i];
                r[e] = r4[i];
            }
        }
#pragma unroll
        for (int e = 0; e < B; ++e) {
            const int i = i0 + lane + kWave * e;
            const float4 v = make_float4(a[e].x + r[e].x, a[e].y + r[e].y, a[e].z + r[e].z, a[e].w + r[e].w);
            ss = fmaf(v.x, v.x, ss);
            ss = fmaf(v.y, v.y, ss);
            ss = fmaf(v.z, v.z, ss);
            ss = fmaf(v.w, v.w, ss);
            if (write && i < hi) o4[i] = v;
        }
    }
    return wave_sum(ss);
}

// All kNormParts parts by one wave, their loads issued together.
__device__ __forceinline__ void norm_add_parts(const OpDesc &op, int lane, bool write,
                                               float (&part)[kNormParts]) {
    constexpr int B = 2;   // float4 pairs in flight per lane and part
    const int n = op.nb * kQuants, nv = n / 4;
    const float4 *a4 = reinterpret_cast<const float4 *>(op.x);
    const float4 *r4 = reinterpret_cast<const float4 *>(op.x_res);
    float4 *o4 = reinterpret_cast<float4 *>(op.x_out);
    int lo[kNormParts], hi[kNormParts];
    float ss[kNormParts];
    int len = 0;
#pragma unroll
    for (int k = 0; k < kNormParts; ++k) {
        lo[k] = (int)((int64_t)nv * k / kNormParts);
        hi[k] = (int)((int64_t)nv * (k + 1) / kNormParts);
        len = max(len, hi[k] - lo[k]);
        ss[k] = 0.f;
    }
    for (int e0 = 0; e0 < len; e0 += kWave * B) {
        float4 a[kNormParts][B], r[kNormParts][B];
#pragma unroll
        for (int k = 0; k < kNormParts; ++k)
#pragma unroll
            for (int e = 0; e < B; ++e) {
                const int i = lo[k] + e0 + lane + kWave * e;
                a[k][e] = make_float4(0.f, 0.f, 0.f, 0.f);
                r[k][e] = a[k][e];
                if (i < hi[k]) {
                    a[k][e] = a4[i];
                    r[k][e] = r4[i];
                }
            }
#pragma unroll
        for (int k = 0; k < kNormParts; ++k)
#pragma unroll
            for (int e = 0; e < B; ++e) {
                const int i = lo[k] + e0 + lane + kWave * e;
                const float4 v = make_float4(a[k][e].x + r[k][e].x, a[k][e].y + r[k][e].y,
                                             a[k][e].z + r[k][e].z, a[k][e].w + r[k][e].w);
                ss[k] = fmaf(v.x, v.x, ss[k]);
                ss[k] = fmaf(v.y, v.y, ss[k]);
                ss[k] = fmaf(v.z, v.z, ss[k]);
                ss[k] = fmaf(v.w, v.w, ss[k]);
                if (write && i < hi[k]) o4[i] = v;
            }
    }
#pragma unroll
    for (int k = 0; k < kNormParts; ++k) part[k] = wave_sum(ss[k]);
}

// 1 / rms of s from its parts.
__device__ __forceinline__ float norm_inv_from(const float (&part)[kNormParts], const OpDesc &op) {
    float ss = part[0];
#pragma unroll
    for (int k = 1; k < kNormParts; ++k) ss += part[k];
    return 1.0f / sqrtf(ss / (float)(op.nb * kQuants) + op.norm_eps);
}

// One normalised value of the kXNormAdd input.
__device__ __forceinline__ float norm_add(float a, float r, float inv, float w) { return (a + r) * inv * w; }

// acc[slot][r] += v for a uniform slot and row index (unrolled selects).
template <int RS>
__device__ __forceinline__ void flush_row(float (&acc)[kSlots][RS], int slot, int r, float v) {
#pragma unroll
    for (int q = 0; q < kSlots; ++q)
#pragma unroll
        for (int k = 0; k < RS; ++k)
            if (q == slot && k == r) acc[q][k] += v;
}

__device__ __forceinline__ float combine_slots(float s0, float s1, float s2, float s3) {
    return (s0 + s1) + (s2 + s3);
}

// ---------------------------------------------------------------- activations as Q8_0
// The integer path quantizes x to Q8_0 blocks the way the pages' CPU path is
// read here: per 32 values d = amax / 127 (float32 division), code =
// x / d rounded half away from zero (0 when d == 0), and the scale kept as
// binary16 (nearest, ties to even).  Every step is an IEEE float32 operation,
// so every implementation doing the same operations gets the same codes.
__device__ __forceinline__ float xq_scale(float amax) { return amax / 127.0f; }
__device__ __forceinline__ int xq_code(float x, float d) {
    return d != 0.f ? (int)roundf(x / d) : 0;
}
__device__ __forceinline__ uint16_t xq_f16_bits(float d) {
    return __builtin_bit_cast(uint16_t, (_Float16)d);
}
__device__ __forceinline__ float xq_f16_value(float d) { return (float)(_Float16)d; }
__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)(d & 0xff) << 24);
}

// ---------------------------------------------------------------- tail rows
// Generic path for the last p % rs rows: one wave per row, lane l takes
// blocks l, l+64, ...; blocks are read with 2-byte loads (a block is only
// 2-byte aligned in general).  Per-lane sums are flushed every 8 blocks and
// the 64 lanes meet in a fixed butterfly.
template <int XM = kXFloat>
__device__ void tail_tile(const OpDesc &op, uint32_t tile, int waves) {
    const int lane = lane_id();
    const int wave = wave_id();
    const int64_t row = (int64_t)op.tail_row0 + (int64_t)tile * waves + wave;
    if (row >= op.p) return;
    float inv = 0.f;
    if constexpr (XM == kXNormAdd) {
        float part[kNormParts];
        norm_add_parts(op, lane, false, part);
        inv = norm_inv_from(part, op);
    }
    const int nb = op.nb;
    const uint8_t *wr = op.w + row * (int64_t)nb * kBlockBytes;
    for (int i = 0; i < op.m; ++i) {
        const __attribute__((address_space(1))) float *x =
            (const __attribute__((address_space(1))) float *)(op.x + (int64_t)i * op.x_stride);
        float acc = 0.f, sub = 0.f;
        int cnt = 0;
        for (int b = lane; b < nb; b += kWave) {
            GHalf *blk = (GHalf *)(wr + (int64_t)b * kBlockBytes);
            const float d = half_to_float(blk[0]);
            const __attribute__((address_space(1))) float *xb = x + (int64_t)b * kQuants;
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int j = 0; j < kQuants / 2; ++j) {
                const uint32_t v = blk[1 + j];
                float x0 = xb[2 * j], x1 = xb[2 * j + 1];
                if constexpr (XM == kXSiluUp) {
                    const float *ub = op.x_up + (int64_t)b * kQuants;
                    x0 = silu_up(x0, ub[2 * j]);
                    x1 = silu_up(x1, ub[2 * j + 1]);
                } else if constexpr (XM == kXNormAdd) {
                    const float *rb = op.x_res + (int64_t)b * kQuants;
                    const float *wb = op.norm_w + (int64_t)b * kQuants;
                    x0 = norm_add(x0, rb[2 * j], inv, wb[2 * j]);
                    x1 = norm_add(x1, rb[2 * j + 1], inv, wb[2 * j + 1]);
                }
                a0 = fmaf((float)(int8_t)(v & 0xffu), x0, a0);
                a1 = fmaf((float)(int8_t)(v >> 8), x1, a1);
            }
            sub = fmaf(d, a0 + a1, sub);
            if (++cnt == 8) { acc += sub; sub = 0.f; cnt = 0; }
        }
        acc += sub;
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
        if (lane == 0) op.y[(int64_t)i * op.y_stride + row] = acc;
    }
    // Settle this path's loads and stores here: the structurizer can merge
    // its flow into the fast path's, and the compiler's wait tracking would
    // otherwise carry them into the fast path's streaming loop as waits.
    __builtin_amdgcn_s_waitcnt(0);
}

}  // namespace
}  // namespace q8
