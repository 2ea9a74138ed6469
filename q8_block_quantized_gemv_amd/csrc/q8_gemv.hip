// q8_gemv.hip -- gfx950 kernels for the Q8_0 decode matvec (m = 1) on
// widths that are not a multiple of 256, and fused launches that mix them
// with the others.
//
// What is computed (page "IV.4: One command buffer per token", section
// "Eight kernels", q8_matvec): y[r] = sum_b d(r,b) * sum_j q(r,b,j) x[32b+j],
// accumulated within a block, scaled once per block (q8_block.h).
//
// When n/32 is not a multiple of 8 a row is not a whole number of 272-byte
// groups, so rows are taken rs at a time ("super-rows", OpDesc), and:
//
//  * One lane owns one super-row.  All lanes of a wave walk the same columns
//    at the same time, so x is wave-uniform: one x value feeds 64 super-rows.
//  * W moves HBM -> LDS with gfx950's direct global_load_lds_dwordx4: a
//    wave's 64 super-rows of one group are 17 fully used 16-byte loads per
//    lane, and inside a group every scale and quant sits at a compile-time
//    byte offset.  The group's 256 x values ride along as an 18th direct
//    load; the compute reads them back with LDS broadcast reads.  Each wave
//    double-buffers its own groups.
//  * Every row sums its groups into four slots (group kk into slot kk % 4)
//    and finishes with (s0 + s1) + (s2 + s3).  When the waves of a workgroup
//    split one row tile's groups (ks = 2 or 4) each slot still has exactly
//    one owner and the slots meet in LDS: every launch shape rounds alike.
//  * Rows that do not fill a whole super-row take a generic path (one wave
//    per row, lanes across blocks, 2-byte loads).
//
// Rows that are whole groups (n a multiple of 256) are computed by the
// rows-and-group-slots tile of q8_rc.h; a fused launch of independent ops of
// both kinds runs each tile in its own layout.
#include "q8_rc.h"

namespace q8 {
namespace {

// One group (8 blocks) of this lane's super-row, accumulated into acc.  A
// group may cross row boundaries inside the super-row; where it does is the
// same for every lane (uniform branches).
template <int RS>
__device__ __forceinline__ void group_dot(const uint32_t (&D)[68], const float4 *xs,
                                          const OpDesc &op, int kk, float (&acc)[kSlots][RS]) {
    const int slot = kk & (kSlots - 1);
    float sub = 0.f, d, s;
    const int bp = kk * kGroupBlocks;
    int r = bp / op.nb;
    int cb = bp - r * op.nb;
#define Q8_STEP(K)                                                   \
    block_terms<K>(D, xs, d, s);                                     \
    sub = fmaf(d, s, sub);                                           \
    if (++cb == op.nb) { flush_row<RS>(acc, slot, r, sub); sub = 0.f; cb = 0; ++r; }
    Q8_STEP(0) Q8_STEP(1) Q8_STEP(2) Q8_STEP(3)
    Q8_STEP(4) Q8_STEP(5) Q8_STEP(6) Q8_STEP(7)
#undef Q8_STEP
    flush_row<RS>(acc, slot, r, sub);
}

template <int RS>
__device__ __forceinline__ void group_dot_xq(const uint32_t (&D)[68], const uint8_t *xa,
                                             const OpDesc &op, int kk, float (&acc)[kSlots][RS]) {
    const int slot = kk & (kSlots - 1);
    float sub = 0.f;
    const int bp = kk * kGroupBlocks;
    int r = bp / op.nb;
    int cb = bp - r * op.nb;
#define Q8_STEP(K)                                                   \
    sub += block_terms_xq<K>(D, xa);                                 \
    if (++cb == op.nb) { flush_row<RS>(acc, slot, r, sub); sub = 0.f; cb = 0; ++r; }
    Q8_STEP(0) Q8_STEP(1) Q8_STEP(2) Q8_STEP(3)
    Q8_STEP(4) Q8_STEP(5) Q8_STEP(6) Q8_STEP(7)
#undef Q8_STEP
    flush_row<RS>(acc, slot, r, sub);
}

// The same rows with x quantized to Q8_0 (the integer path, m = 1): each
// lane quantizes the x blocks it needs itself and multiplies the codes.
__device__ void tail_tile_xq(const OpDesc &op, uint32_t tile, int waves) {
    const int lane = lane_id();
    const int wave = wave_id();
    const int64_t row = (int64_t)op.tail_row0 + (int64_t)tile * waves + wave;
    if (row >= op.p) return;
    const int nb = op.nb;
    const uint8_t *wr = op.w + row * (int64_t)nb * kBlockBytes;
    float acc = 0.f, sub = 0.f;
    int cnt = 0;
    for (int b = lane; b < nb; b += kWave) {
        const float4 *xb = reinterpret_cast<const float4 *>(op.x + (int64_t)b * kQuants);
        float4 xv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) xv[k] = xb[k];
        float amax = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(xv[k].x), fabsf(xv[k].y)),
                                     fmaxf(fabsf(xv[k].z), fabsf(xv[k].w))));
        const float d = xq_scale(amax);
        GHalf *blk = (GHalf *)(wr + (int64_t)b * kBlockBytes);
        const float dw = half_to_float(blk[0]);
        int isum = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t lo = blk[1 + 2 * k], hi = blk[2 + 2 * k];
            const int wq = (int)(lo | (hi << 16));
            const int xq = (int)pack4(xq_code(xv[k].x, d), xq_code(xv[k].y, d), xq_code(xv[k].z, d),
                                      xq_code(xv[k].w, d));
            isum = __builtin_amdgcn_sdot4(wq, xq, isum, false);
        }
        sub = fmaf((float)isum, dw * xq_f16_value(d), sub);
        if (++cnt == 8) { acc += sub; sub = 0.f; cnt = 0; }
    }
    acc += sub;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
    if (lane == 0) op.y[row] = acc;
    __builtin_amdgcn_s_waitcnt(0);
}

// Bytes of one stage: W, the x slice and, for kXSiluUp, the up slice.
template <int XM>
constexpr int stage_bytes() { return kStageBytes + (XM == kXSiluUp ? kStageX : 0); }

// One workgroup tile of NW waves: NW/ks row tiles of 64 super-rows, each row
// tile's groups split over ks waves (group kk = ksl + ks*t to wave ksl, so
// slot kk % 4 has one owner).  Each wave keeps one group in flight ahead of
// the one it computes.  writer (kXNormAdd): this workgroup also writes
// x + x_res to op.x_out.
template <int RS, int NW, int XM>
__device__ __forceinline__ void superrow_tile(const OpDesc &op, int64_t wtile, uint8_t *stage, bool writer) {
    constexpr int SB = stage_bytes<XM>();
    const int lane = lane_id();
    const int wave = wave_id();
    const int ks = op.ks;
    const int rt = wave / ks;                 // row tile within the workgroup
    const int ksl = wave - rt * ks;           // this wave's share of the groups
    const int64_t row_tile = wtile * (NW / ks) + rt;
    const int64_t sr0 = row_tile * kWave;
    const int nsr = op.nsr;
    uint8_t *st0 = stage + (size_t)wave * (kBufs * SB);

    float acc[kSlots][RS];
#pragma unroll
    for (int q = 0; q < kSlots; ++q)
#pragma unroll
        for (int k = 0; k < RS; ++k) acc[q][k] = 0.f;

    // kXNormAdd: the norm in its fixed parts (every wave of the workgroup
    // reaches the barrier when NW > 1); one wave computes it while its first
    // group streams in
    float ninv = 0.f;
    auto norm = [&]() {
        float part[kNormParts];
        const bool wr = op.x_out && writer;
        if constexpr (NW > 1) {
            __shared__ float parts[kNormParts];
#pragma unroll
            for (int k = 0; k < kNormParts; ++k)
                if (k % NW == wave) {
                    const float v = norm_add_part(op, lane, k, kNormParts, wr);
                    if (lane == 0) parts[k] = v;
                }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < kNormParts; ++k) part[k] = parts[k];
        } else {
            norm_add_parts(op, lane, wr, part);
        }
        return norm_inv_from(part, op);
    };
    if constexpr (XM == kXNormAdd && NW > 1) ninv = norm();

    if (sr0 < nsr) {
        const int G = op.gsr;
        const int64_t srb = op.sr_bytes;
        const uint8_t *wt = uniform_ptr(op.w + sr0 * srb);   // the direct loads' scalar base
        const int last = (int)min((int64_t)nsr - 1 - sr0, (int64_t)kWave - 1);
        uint32_t off[kGroupChunks];
        chunk_offsets(off, lane, last, srb);
        const int ng = G > ksl ? (G - ksl + ks - 1) / ks : 0;
        float4 na = make_float4(0.f, 0.f, 0.f, 0.f), nr = na, nw = na;   // kXNormAdd prefetch
        auto issue = [&](int t) {
            const int kk = ksl + ks * t;
            uint8_t *st = st0 + (t & 1) * SB;
            if constexpr (XM == kXNormAdd) {
                // W by direct loads; this lane's four x, x_res and gain values
                // of the group into registers, used before the next issue
                const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(st));
                const uint8_t *g = wt + (int64_t)kk * kGroupBytes;
#pragma unroll
                for (int i = 0; i < kGroupChunks; ++i) dma16_s(g, off[i], l0 + kWave * 16 * i);
                na = *reinterpret_cast<const float4 *>(x_slice_src<RS>(op, op.x, kk, lane));
                nr = *reinterpret_cast<const float4 *>(x_slice_src<RS>(op, op.x_res, kk, lane));
                nw = *reinterpret_cast<const float4 *>(x_slice_src<RS>(op, op.norm_w, kk, lane));
            } else {
                dma_group_x<RS>(wt + (int64_t)kk * kGroupBytes, off, st, op, kk, lane);
                if constexpr (XM == kXSiluUp)
                    dma16_v(x_slice_src<RS>(op, op.x_up, kk, lane),
                            __builtin_amdgcn_readfirstlane(lds_addr(st)) + kStageBytes);
            }
        };
        if (ng > 0) issue(0);
        if constexpr (XM == kXNormAdd && NW == 1) ninv = norm();
        for (int t = 0; t < ng; ++t) {
            uint8_t *cur = st0 + (t & 1) * SB;
            uint32_t D[68];
            wait_vm_asm<0>();   // this group's W and x have landed
            read_group(cur, lane, D);
            if constexpr (XM == kXNormAdd)   // this group's normalised x slice into the stage
                reinterpret_cast<float4 *>(cur + kStageW)[lane] =
                    make_float4(norm_add(na.x, nr.x, ninv, nw.x), norm_add(na.y, nr.y, ninv, nw.y),
                                norm_add(na.z, nr.z, ninv, nw.z), norm_add(na.w, nr.w, ninv, nw.w));
            if (t + 1 < ng) issue(t + 1);
            const int kk = ksl + ks * t;
            if constexpr (XM == kXQuant) {
                quantize_slice(cur + kStageW, lane);
                group_dot_xq<RS>(D, cur + kStageW, op, kk, acc);
            } else {
                if constexpr (XM == kXSiluUp) {   // the x slice becomes silu(gate) * up in place
                    float4 *xs = reinterpret_cast<float4 *>(cur + kStageW);
                    const float4 g = xs[lane];
                    const float4 u = reinterpret_cast<const float4 *>(cur + kStageBytes)[lane];
                    xs[lane] = make_float4(silu_up(g.x, u.x), silu_up(g.y, u.y), silu_up(g.z, u.z),
                                           silu_up(g.w, u.w));
                }
                group_dot<RS>(D, reinterpret_cast<const float4 *>(cur + kStageW), op, kk, acc);
            }
        }
    }

    if (ks > 1) {
        // Slot q belongs to wave (q % ks) of the row tile, which parks it in
        // its own (now idle) first stage: red_w[(q / ks) * RS + k][lane].
        // Its last direct load completed before its last group was read.
        float *mine = reinterpret_cast<float *>(st0);
#pragma unroll
        for (int q = 0; q < kSlots; ++q)
            if (q % ks == ksl)
#pragma unroll
                for (int k = 0; k < RS; ++k) mine[((q / ks) * RS + k) * kWave + lane] = acc[q][k];
        __syncthreads();
        if (ksl == 0) {
#pragma unroll
            for (int q = 1; q < kSlots; ++q) {
                const int owner = rt * ks + q % ks;
                const float *theirs = reinterpret_cast<const float *>(
                    stage + (size_t)owner * (kBufs * SB));
                if (owner != wave)
#pragma unroll
                    for (int k = 0; k < RS; ++k) acc[q][k] = theirs[((q / ks) * RS + k) * kWave + lane];
            }
        }
    }
    if (ksl == 0 && sr0 + lane < nsr) {
        float *yr = op.y + (sr0 + lane) * RS;
#pragma unroll
        for (int k = 0; k < RS; ++k) yr[k] = combine_slots(acc[0][k], acc[1][k], acc[2][k], acc[3][k]);
    }
}

template <int NW, int XM>
__device__ __forceinline__ void run_superrow(const OpDesc &op, uint32_t t, uint8_t *stage) {
    if (t & kTailBit) {
        if constexpr (XM == kXQuant) tail_tile_xq(op, t & ~kTailBit, NW);
        else tail_tile<XM>(op, t & ~kTailBit, NW);
        return;
    }
    switch (op.rs) {
        case 2: superrow_tile<2, NW, XM>(op, t, stage, t == 0); break;
        case 4: superrow_tile<4, NW, XM>(op, t, stage, t == 0); break;
        default: superrow_tile<8, NW, XM>(op, t, stage, t == 0); break;
    }
}

template <int NW, int XM>
__global__ __launch_bounds__(NW * kWave) void k_q8_gemv(OpDesc op) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[NW * kBufs * stage_bytes<XM>()];
    uint32_t t = blockIdx.x;
    if (t >= (uint32_t)op.fast_tiles) t = (t - op.fast_tiles) | kTailBit;
    run_superrow<NW, XM>(op, t, stage);
}

// A fused launch of one-wave workgroups over a table of tiles of
// independent ops: rows of whole groups take the rows-and-group-slots tile
// with kMixC lanes per row and kMixNst W stages, the others the super-row
// tile; the LDS is the larger of the two.
template <int XM>
constexpr int mixed_lds_bytes() {
    return kBufs * stage_bytes<XM>() > rc_lds_bytes<kMixC, 1, XM, kMixNst>() ? kBufs * stage_bytes<XM>()
                                                                            : rc_lds_bytes<kMixC, 1, XM, kMixNst>();
}

template <int XM>
__global__ __launch_bounds__(kWave) void k_q8_gemv_mixed(const OpDesc *__restrict__ ops,
                                                         const Tile *__restrict__ tiles) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[mixed_lds_bytes<XM>()];
    const Tile tl = tiles[blockIdx.x];
    const OpDesc op = ops[tl.op];
    if (op.rs == 1) rc_tile<kMixC, 1, XM, kMixNst>(op, tl.tile, stage, tl.tile == 0);
    else run_superrow<1, XM>(op, tl.tile, stage);
}

// x (n floats) -> n/32 Q8_0 blocks of 34 bytes: 32 lanes per block, eight
// blocks per 256-thread workgroup.
__global__ __launch_bounds__(256) void k_quantize_x(const float *x, uint8_t *xq, int64_t nb) {
    const int64_t b = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
    const int j = threadIdx.x & 31;
    const bool live = b < nb;
    const float v = live ? x[b * kQuants + j] : 0.f;
    float a = fabsf(v);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, kWave));
    if (!live) return;
    const float d = xq_scale(a);
    uint8_t *blk = xq + b * kBlockBytes;
    blk[2 + j] = (uint8_t)(int8_t)xq_code(v, d);
    if (j == 0) {
        const uint16_t bits = xq_f16_bits(d);
        blk[0] = (uint8_t)(bits & 0xff);
        blk[1] = (uint8_t)(bits >> 8);
    }
}

}  // namespace

namespace {
template <int NW, int XM>
hipError_t launch_single_t(const OpDesc &op, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((k_q8_gemv<NW, XM>), dim3((unsigned)grid), dim3(NW * kWave), 0, s, op);
    return hipGetLastError();
}
template <int XM>
hipError_t launch_mixed_t(const OpDesc *d_ops, const Tile *d_tiles, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((k_q8_gemv_mixed<XM>), dim3((unsigned)grid), dim3(kWave), 0, s, d_ops, d_tiles);
    return hipGetLastError();
}
template <int XM>
hipError_t launch_single_v(const OpDesc &op, const Variant &v, int64_t grid, hipStream_t s) {
    if (v.pf != 1) return hipErrorInvalidValue;
    switch (v.nw) {
        case 1: return launch_single_t<1, XM>(op, grid, s);
        case 4: return launch_single_t<4, XM>(op, grid, s);
        default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t launch_gemv_single(const OpDesc &op, const Variant &v, int64_t grid, hipStream_t s,
                              int xmode) {
    if (grid <= 0 || op.rs <= 1) return hipErrorInvalidValue;
    switch (xmode) {
        case kXFloat: return launch_single_v<kXFloat>(op, v, grid, s);
        case kXQuant: return launch_single_v<kXQuant>(op, v, grid, s);
        case kXSiluUp: return launch_single_v<kXSiluUp>(op, v, grid, s);
        case kXNormAdd: return launch_single_v<kXNormAdd>(op, v, grid, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_fused(const OpDesc *d_ops, const Tile *d_tiles, const Variant &v,
                             int64_t grid, hipStream_t s, int xmode) {
    if (grid <= 0 || v.nw != 1 || v.pf != 1) return hipErrorInvalidValue;
    switch (xmode) {
        case kXFloat: return launch_mixed_t<kXFloat>(d_ops, d_tiles, grid, s);
        case kXQuant: return launch_mixed_t<kXQuant>(d_ops, d_tiles, grid, s);
        case kXSiluUp: return launch_mixed_t<kXSiluUp>(d_ops, d_tiles, grid, s);
        case kXNormAdd: return launch_mixed_t<kXNormAdd>(d_ops, d_tiles, grid, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_quantize_x(const float *x, void *xq, int64_t n, hipStream_t s) {
    const int64_t nb = n / kQuants;
    hipLaunchKernelGGL(k_quantize_x, dim3((unsigned)((nb + 7) / 8)), dim3(256), 0, s, x,
                       (uint8_t *)xq, nb);
    return hipGetLastError();
}

}  // namespace q8
