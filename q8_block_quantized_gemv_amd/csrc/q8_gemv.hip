// q8_gemv.hip -- gfx950 kernels for the Q8_0 decode matvec (m = 1): the
// standalone launch and the fused launch of a chain.
//
// What is computed (page "IV.4: One command buffer per token", section
// "Eight kernels", q8_matvec): y[r] = sum_b d(r,b) * sum_j q(r,b,j) x[32b+j],
// accumulated within a block, scaled once per block.
//
// How, on CDNA4 (the page's one-SIMD-group-per-row layout is not used):
//
//  * One lane owns one output row (or one "super-row" of rs rows, see
//    OpDesc).  All lanes of a wave walk the same columns at the same time,
//    so x is wave-uniform: one x value feeds 64 rows.
//  * W moves HBM -> LDS with gfx950's direct global_load_lds_dwordx4: eight
//    blocks are 272 bytes = 17 aligned 16-byte chunks, so a wave's 64 rows
//    of one "group" are 17 fully used 16-byte loads per lane, and inside a
//    group every scale and quant sits at a compile-time byte offset.  The
//    group's 256 x values (1 KB, L2-resident) ride along as an 18th direct
//    load, so x never waits on its own trip through a saturated memory
//    system; the compute reads it back with LDS broadcast reads.  Each
//    wave double-buffers its own groups (the next group streams in while the
//    current one is computed), so there are no workgroup barriers on the
//    streaming path.
//  * Quant bytes become float with one SDWA conversion each; products go
//    into four independent float32 chains per block; the block sum is scaled
//    once; per-group and per-row subtotals keep every summation chain short
//    (<= ~100 roundings at the largest shapes, so the accuracy bound of
//    1e-5 * sum|w x| holds for all finite inputs, not only random ones).
//  * Every row sums its groups into four slots (group kk into slot kk % 4)
//    and finishes with (s0 + s1) + (s2 + s3).  When the waves of a workgroup
//    split one row tile's groups (ks = 2 or 4) each slot still has exactly
//    one owner, and the slots meet in LDS: the rounding of every output is
//    the same whatever ks, launch or batch size, so results are bitwise
//    reproducible and a chain's outputs equal standalone calls' bit for bit.
//    There are no atomics.
//  * Rows that do not fill a whole super-row take a simple generic path
//    (one wave per row, lanes across blocks, 2-byte loads).
#include "q8_device.h"

namespace q8 {
namespace {

// Block K (0..7) of a group: d and S = sum_j q_j x_j (four chains of eight).
// xs is the group's x slice in LDS (the same address for every lane).
template <int K>
__device__ __forceinline__ void block_terms(const uint32_t (&D)[68], const float4 *xs,
                                            float &d, float &s) {
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

// ---------------------------------------------------------------- m = 1
// One group (8 blocks) of this lane's super-row, accumulated into acc.
template <int RS>
__device__ __forceinline__ void group_dot(const uint32_t (&D)[68], const float4 *xs,
                                          const OpDesc &op, int kk, float (&acc)[kSlots][RS]) {
    const int slot = kk & (kSlots - 1);
    float sub = 0.f, d, s;
    if constexpr (RS == 1) {
        // rows are whole groups: group kk is blocks 8kk .. 8kk+7 of the row
        block_terms<0>(D, xs, d, s); sub = fmaf(d, s, sub);
        block_terms<1>(D, xs, d, s); sub = fmaf(d, s, sub);
        block_terms<2>(D, xs, d, s); sub = fmaf(d, s, sub);
        block_terms<3>(D, xs, d, s); sub = fmaf(d, s, sub);
        block_terms<4>(D, xs, d, s); sub = fmaf(d, s, sub);
        block_terms<5>(D, xs, d, s); sub = fmaf(d, s, sub);
        block_terms<6>(D, xs, d, s); sub = fmaf(d, s, sub);
        block_terms<7>(D, xs, d, s); sub = fmaf(d, s, sub);
        flush_row<1>(acc, slot, 0, sub);
    } else {
        // a group may cross row boundaries inside the super-row; where it
        // does is the same for every lane (uniform branches)
        const int bp = kk * kGroupBlocks;
        int r = bp / op.nb;
        int cb = bp - r * op.nb;
#define Q8_STEP(K)                                                   \
        block_terms<K>(D, xs, d, s);                                 \
        sub = fmaf(d, s, sub);                                       \
        if (++cb == op.nb) { flush_row<RS>(acc, slot, r, sub); sub = 0.f; cb = 0; ++r; }
        Q8_STEP(0) Q8_STEP(1) Q8_STEP(2) Q8_STEP(3)
        Q8_STEP(4) Q8_STEP(5) Q8_STEP(6) Q8_STEP(7)
#undef Q8_STEP
        flush_row<RS>(acc, slot, r, sub);
    }
}

// ---------------------------------------------------------------- m = 1, integer
// The group's x slice (256 floats at xa, lane l holding floats 4l..4l+3, of
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

template <int RS>
__device__ __forceinline__ void group_dot_xq(const uint32_t (&D)[68], const uint8_t *xa,
                                             const OpDesc &op, int kk, float (&acc)[kSlots][RS]) {
    const int slot = kk & (kSlots - 1);
    float sub = 0.f;
    if constexpr (RS == 1) {
        sub += block_terms_xq<0>(D, xa);
        sub += block_terms_xq<1>(D, xa);
        sub += block_terms_xq<2>(D, xa);
        sub += block_terms_xq<3>(D, xa);
        sub += block_terms_xq<4>(D, xa);
        sub += block_terms_xq<5>(D, xa);
        sub += block_terms_xq<6>(D, xa);
        sub += block_terms_xq<7>(D, xa);
        flush_row<1>(acc, slot, 0, sub);
    } else {
        const int bp = kk * kGroupBlocks;
        int r = bp / op.nb;
        int cb = bp - r * op.nb;
#define Q8_STEP(K)                                                   \
        sub += block_terms_xq<K>(D, xa);                             \
        if (++cb == op.nb) { flush_row<RS>(acc, slot, r, sub); sub = 0.f; cb = 0; ++r; }
        Q8_STEP(0) Q8_STEP(1) Q8_STEP(2) Q8_STEP(3)
        Q8_STEP(4) Q8_STEP(5) Q8_STEP(6) Q8_STEP(7)
#undef Q8_STEP
        flush_row<RS>(acc, slot, r, sub);
    }
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

// One workgroup tile of NW waves: NW/ks row tiles of 64 super-rows, each
// row tile's groups split over ks waves.  PF is how many groups each wave
// keeps in flight ahead of the one it computes (1 or 2; each stage holds one
// group, and with PF = 2 the stage a group was computed from is refilled
// right after that group's compute, so two groups stream while one waits).
constexpr int kGatherBatch = 8;

// With K slices (op.slices > 1), or a stream-K row tile shared by several
// workgroups, the ksl == 0 wave of each row tile parks its rows' partial
// sums in its slot and counts in; the last of the nslices to arrive adds the
// slots in order.  The partials travel through device-scope stores and
// loads (they come from other workgroups, possibly on other XCDs).
template <int RS>
__device__ __forceinline__ void slice_arrive(const OpDesc &op, int64_t row_tile, int slice, int nslices,
                                          int64_t sr0, const float (&acc)[kSlots][RS], int lane) {
    const int64_t P = (int64_t)op.nsr * RS;
    const bool live = sr0 + lane < op.nsr;
    const int64_t r0 = (sr0 + lane) * RS;
    if (live)
#pragma unroll
        for (int k = 0; k < RS; ++k)
            __hip_atomic_store(op.part + slice * P + r0 + k,
                               combine_slots(acc[0][k], acc[1][k], acc[2][k], acc[3][k]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    uint32_t prev = 0;
    if (lane == 0)
        prev = __hip_atomic_fetch_add(op.cnt + row_tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != (uint32_t)nslices - 1) return;
    asm volatile("" ::: "memory");
    if (live) {
#pragma unroll
        for (int k = 0; k < RS; ++k) {
            float sum = 0.f;
            for (int q0 = 0; q0 < nslices; q0 += kGatherBatch) {   // loads eight at a time
                float v[kGatherBatch];
#pragma unroll
                for (int b = 0; b < kGatherBatch; ++b) {
                    v[b] = 0.f;
                    if (q0 + b < nslices)
                        v[b] = __hip_atomic_load(op.part + (q0 + b) * P + r0 + k, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
                }
#pragma unroll
                for (int b = 0; b < kGatherBatch; ++b)
                    if (q0 + b < nslices) sum += v[b];
            }
            op.y[r0 + k] = sum;
        }
    }
    if (lane == 0)   // ready for the next launch
        __hip_atomic_store(op.cnt + row_tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bytes of one stage: W, the x slice and, for kXSiluUp, the up slice.
template <int XM>
constexpr int stage_bytes() { return kStageBytes + (XM == kXSiluUp ? kStageX : 0); }

// What one workgroup does with an op: groups [g0, g1) of each of its row
// tiles (wtile * (NW / ks) onward); nslots > 1: the row tiles are shared by
// nslots workgroups and this one parks its partial sums in slot `slot`.
struct TileJob {
    int64_t wtile;
    int g0, g1;
    int slot, nslots;
    bool writer;   // kXNormAdd: this workgroup's first wave writes x + x_res to x_out
};

template <int RS, int NW, int PF, int XM>
__device__ __forceinline__ void fast_job(const OpDesc &op, const TileJob &job, uint8_t *stage) {
    constexpr int SB = stage_bytes<XM>();
    // memory operations per group: 17 direct loads of W, then the x slice
    // (one more direct load; two for kXSiluUp; three vector loads for kXNormAdd)
    constexpr int LPG = kGroupChunks + (XM == kXSiluUp ? 2 : XM == kXNormAdd ? 3 : 1);
    const int lane = lane_id();
    const int wave = wave_id();
    const int ks = op.ks;
    const int rt = wave / ks;                 // row tile within the workgroup
    const int ksl = wave - rt * ks;           // this wave's share of the groups
    const int tiles_per_wg = NW / ks;
    const int64_t row_tile = job.wtile * tiles_per_wg + rt;
    const int64_t sr0 = row_tile * kWave;
    const int nsr = op.nsr;
    uint8_t *st0 = stage + (size_t)wave * (kBufs * SB);

    float acc[kSlots][RS];
#pragma unroll
    for (int q = 0; q < kSlots; ++q)
#pragma unroll
        for (int k = 0; k < RS; ++k) acc[q][k] = 0.f;

    // kXNormAdd with several waves: they share one op, so each sums the
    // squares of a quarter of x + x_res (the writer workgroup's waves also
    // store their share of it) and the parts meet in LDS, added in wave
    // order by every wave.  Every wave of the workgroup reaches the barrier.
    // (This runs before the first group's loads are issued; with one wave
    // the norm is computed while they stream, below.)
    float norm_inv_shared = 0.f;
    if constexpr (XM == kXNormAdd && NW > 1) {
        __shared__ float norm_part[NW];
        const float part = norm_add_part(op, lane, wave, NW, op.x_out && job.writer);
        if (lane == 0) norm_part[wave] = part;
        __syncthreads();
        float ss = norm_part[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) ss += norm_part[w];
        norm_inv_shared = 1.0f / sqrtf(ss / (float)(op.nb * kQuants) + op.norm_eps);
    }

    if (sr0 < nsr) {
        const int G = op.gsr;
        const int64_t srb = op.sr_bytes;
        const uint8_t *wt = uniform_ptr(op.w + sr0 * srb);   // the direct loads' scalar base
        const int last = (int)min((int64_t)nsr - 1 - sr0, (int64_t)kWave - 1);
        uint32_t off[kGroupChunks];
        chunk_offsets(off, lane, last, srb);
        // the job's groups [g0, g1); with ks > 1, g0 is a multiple of kSlots,
        // so group kk = g0 + ksl + ks*t still falls in slot kk % 4 owned by
        // wave ksl
        const int g0 = job.g0;
        const int g1 = min(G, job.g1);
        const int ng = g1 - g0 > ksl ? (g1 - g0 - ksl + ks - 1) / ks : 0;
        float4 na = make_float4(0.f, 0.f, 0.f, 0.f), nr = na, nw = na;   // kXNormAdd prefetch
        auto issue = [&](int t) {
            const int kk = g0 + ksl + ks * t;
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
        float ninv = 0.f;
        if constexpr (XM == kXNormAdd) {
            if constexpr (NW > 1) ninv = norm_inv_shared;
            else ninv = norm_add_inv(op, lane, op.x_out && job.writer && wave == 0);
        }
        if (PF == 2 && ng > 1) issue(1);
        for (int t = 0; t < ng; ++t) {
            uint8_t *cur = st0 + (t & 1) * SB;
            uint32_t D[68];
            // this group's W and x have landed in LDS (loads complete in order)
            if (PF == 2 && t + 1 < ng) wait_vm_asm<LPG>();
            else wait_vm_asm<0>();
            read_group(cur, lane, D);
            if constexpr (XM == kXNormAdd)   // this group's normalised x slice into the stage
                reinterpret_cast<float4 *>(cur + kStageW)[lane] =
                    make_float4(norm_add(na.x, nr.x, ninv, nw.x), norm_add(na.y, nr.y, ninv, nw.y),
                                norm_add(na.z, nr.z, ninv, nw.z), norm_add(na.w, nr.w, ninv, nw.w));
            if (PF == 1 && t + 1 < ng) issue(t + 1);
            if constexpr (XM == kXQuant) {
                quantize_slice(cur + kStageW, lane);
                group_dot_xq<RS>(D, cur + kStageW, op, g0 + ksl + ks * t, acc);
            } else {
                if constexpr (XM == kXSiluUp) {   // the x slice becomes silu(gate) * up in place
                    float4 *xs = reinterpret_cast<float4 *>(cur + kStageW);
                    const float4 g = xs[lane];
                    const float4 u = reinterpret_cast<const float4 *>(cur + kStageBytes)[lane];
                    xs[lane] = make_float4(silu_up(g.x, u.x), silu_up(g.y, u.y), silu_up(g.z, u.z),
                                           silu_up(g.w, u.w));
                }
                group_dot<RS>(D, reinterpret_cast<const float4 *>(cur + kStageW), op, g0 + ksl + ks * t,
                              acc);
            }
            if (PF == 2 && t + 2 < ng) issue(t + 2);   // into the stage just consumed
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
    if (job.nslots > 1) {
        if (ksl == 0 && sr0 < nsr) slice_arrive<RS>(op, row_tile, job.slot, job.nslots, sr0, acc, lane);
        return;
    }
    if (ksl == 0 && sr0 + lane < nsr) {
        float *yr = op.y + (sr0 + lane) * RS;
#pragma unroll
        for (int k = 0; k < RS; ++k) yr[k] = combine_slots(acc[0][k], acc[1][k], acc[2][k], acc[3][k]);
    }
}

// Fast tile `tile` of a launch: with K slices, tile = row-tile group * slices + slice.
template <int RS, int NW, int PF, int XM>
__device__ __forceinline__ void fast_tile(const OpDesc &op, uint32_t tile, uint8_t *stage) {
    const int S = op.slices;
    TileJob job;
    job.wtile = S > 1 ? tile / (uint32_t)S : tile;
    job.slot = (int)(tile - (uint32_t)job.wtile * (uint32_t)S);
    job.nslots = S;
    job.g0 = S > 1 ? job.slot * op.slice_groups : 0;
    job.g1 = S > 1 ? job.g0 + op.slice_groups : op.gsr;
    job.writer = tile == 0;
    fast_job<RS, NW, PF, XM>(op, job, stage);
}

template <int NW, int PF, int XM>
__device__ __forceinline__ void run_tile(const OpDesc &op, uint32_t t, uint8_t *stage) {
    if (t & kTailBit) {
        if constexpr (XM == kXQuant) tail_tile_xq(op, t & ~kTailBit, NW);
        else tail_tile<XM>(op, t & ~kTailBit, NW);
        return;
    }
    switch (op.rs) {
        case 1: fast_tile<1, NW, PF, XM>(op, t, stage); break;
        case 2: fast_tile<2, NW, PF, XM>(op, t, stage); break;
        case 4: fast_tile<4, NW, PF, XM>(op, t, stage); break;
        default: fast_tile<8, NW, PF, XM>(op, t, stage); break;
    }
}

template <int NW, int PF, int XM>
__global__ __launch_bounds__(NW * kWave) void k_q8_gemv(OpDesc op) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[NW * kBufs * stage_bytes<XM>()];
    uint32_t t = blockIdx.x;
    if (t >= (uint32_t)op.fast_tiles) t = (t - op.fast_tiles) | kTailBit;
    run_tile<NW, PF, XM>(op, t, stage);
}

template <int NW, int PF, int XM>
__global__ __launch_bounds__(NW * kWave) void k_q8_gemv_fused(const OpDesc *__restrict__ ops,
                                                              const Tile *__restrict__ tiles) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[NW * kBufs * stage_bytes<XM>()];
    const Tile tl = tiles[blockIdx.x];
    const OpDesc op = ops[tl.op];
    run_tile<NW, PF, XM>(op, tl.tile, stage);
}

// Stream-K: workgroup b (one wave) walks its pieces, contiguous runs of an
// equal share of all (row tile, group) items of the launch's ops, in order.
template <int PF, int XM>
__device__ __forceinline__ void run_pieces(const OpDesc *__restrict__ ops, const Piece *__restrict__ pieces,
                                           const uint32_t *__restrict__ begin, uint32_t b, uint8_t *stage) {
    const uint32_t e = begin[b + 1];
    for (uint32_t i = begin[b]; i < e; ++i) {
        const Piece pc = pieces[i];
        const OpDesc op = ops[pc.op];
        TileJob job;
        job.wtile = pc.tile;
        job.g0 = (int)pc.g0;
        job.g1 = (int)pc.g1;
        job.slot = (int)pc.slot;
        job.nslots = (int)pc.nslots;
        job.writer = pc.tile == 0 && pc.g0 == 0;
        switch (op.rs) {
            case 1: fast_job<1, 1, PF, XM>(op, job, stage); break;
            case 2: fast_job<2, 1, PF, XM>(op, job, stage); break;
            case 4: fast_job<4, 1, PF, XM>(op, job, stage); break;
            default: fast_job<8, 1, PF, XM>(op, job, stage); break;
        }
    }
}

template <int XM>
__device__ __forceinline__ void run_tail(const OpDesc &op, uint32_t t) {
    if constexpr (XM == kXQuant) tail_tile_xq(op, t & ~kTailBit, 1);
    else tail_tile<XM>(op, t & ~kTailBit, 1);
}

// The workgroups after the first n_sk run tail tiles.
template <int PF, int XM>
__global__ __launch_bounds__(kWave) void k_q8_gemv_sk(const OpDesc *__restrict__ ops,
                                                      const Piece *__restrict__ pieces,
                                                      const uint32_t *__restrict__ begin,
                                                      const Tile *__restrict__ tails, uint32_t n_sk) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[kBufs * stage_bytes<XM>()];
    const uint32_t b = blockIdx.x;
    if (b >= n_sk) {
        const Tile tl = tails[b - n_sk];
        run_tail<XM>(ops[tl.op], tl.tile);
        return;
    }
    run_pieces<PF, XM>(ops, pieces, begin, b, stage);
}

// ---------------------------------------------------------------- one launch, many phases
// A chain of dependent matvecs in one launch: every workgroup takes its
// stream-K share of phase s, then waits until all workgroups have finished
// phase s before it starts phase s + 1.  All workgroups are resident at
// once (the host sizes the grid by occupancy), so every wait ends; a wait
// still gives up after kSpinLimit polls (about a second) and flags err, and
// once err is set the waits of the launch give up at once, so that no wave
// can spin for long.
//
// The barrier is two-level, by XCD (each has its own L2): a workgroup
// counts in on its XCD's counter once its own memory operations are done
// (its stores are then in that L2); the last of the XCD's `per` workgroups
// writes the L2 back (agent-scope release), counts the XCD in on the global
// counter, waits for all `nx` XCDs, invalidates the L2 (acquire) and raises
// the XCD's flag; the others wait for the flag and invalidate their CU's L1.
// One release and one acquire per XCD instead of per wave, and no counter
// that every wave hits: measured 3.6 us per barrier against 39 us for one
// counter and per-wave fences.  Counts run on across launches (generation
// g = the flag's value at launch start + s), compared modulo 2^32, so
// nothing has to be cleared between launches.
//
// A CU's L1 is only dropped by a wave's own agent-scope acquire (9.9 us per
// barrier when every wave does it).  The L1 holds only lines this launch
// has read (each launch starts with it clean), so it can only be stale for
// memory that an earlier phase read and a later one rewrote; the host marks
// the phases that read such memory (PhaseDesc::acquire) and only their
// barriers pay for the per-wave acquire.
constexpr uint32_t kSpinLimit = 1u << 20;
// sync words, one 256-B line each: global counter, per-XCD counters,
// per-XCD flags, err
constexpr int kSyncLine = 64;
constexpr int kMaxXcc = 16;
__device__ __forceinline__ uint32_t *sync_global(uint32_t *sy) { return sy; }
__device__ __forceinline__ uint32_t *sync_local(uint32_t *sy, uint32_t x) { return sy + kSyncLine * (1 + x); }
__device__ __forceinline__ uint32_t *sync_flag(uint32_t *sy, uint32_t x) { return sy + kSyncLine * (1 + kMaxXcc + x); }
__device__ __forceinline__ uint32_t *sync_err(uint32_t *sy) { return sy + kSyncLine * (1 + 2 * kMaxXcc); }

__device__ __forceinline__ uint32_t xcc_id() {
    uint32_t v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(v));
    return v & (kMaxXcc - 1);
}

__device__ __forceinline__ uint32_t load_agent(uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Spin (lane 0) until *p has reached `target` (modulo 2^32).
__device__ __forceinline__ void spin_to(uint32_t *p, uint32_t target, uint32_t *err) {
    uint32_t polls = 0;
    while ((int32_t)(load_agent(p) - target) < 0) {
        __builtin_amdgcn_s_sleep(1);
        if ((++polls & 1023u) == 0 && load_agent(err)) break;
        if (polls == kSpinLimit) {
            __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
    }
}

// Barrier generation g among all workgroups (per on each of nx XCDs);
// all: every wave takes an agent-scope acquire after it.
__device__ __forceinline__ void phase_sync(uint32_t *sy, uint32_t x, uint32_t g, uint32_t per, uint32_t nx,
                                           bool all) {
    if (lane_id() == 0) {
        uint32_t *err = sync_err(sy);
        __builtin_amdgcn_s_waitcnt(0);   // this wave's loads and stores are done
        const uint32_t prev =
            __hip_atomic_fetch_add(sync_local(sy, x), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == g * per - 1u) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __hip_atomic_fetch_add(sync_global(sy), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            spin_to(sync_global(sy), g * nx, err);
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            // the invalidation completes before the flag lets the XCD's
            // other waves load through this L2
            __builtin_amdgcn_s_waitcnt(0);
            __hip_atomic_store(sync_flag(sy, x), g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            spin_to(sync_flag(sy, x), g, err);
            if (all) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
    }
    asm volatile("" ::: "memory");
}

template <int PF, int XM>
__device__ __forceinline__ void phase_work(const PhaseDesc &ph, uint32_t b, uint32_t wgs, uint8_t *stage) {
    if (b < (uint32_t)ph.n_sk) run_pieces<PF, XM>(ph.ops, ph.pieces, ph.begin, b, stage);
    for (uint32_t t = b; t < (uint32_t)ph.n_tail; t += wgs) {
        const Tile tl = ph.tails[t];
        run_tail<XM>(ph.ops[tl.op], tl.tile);
    }
}

// The largest stage of the modes a phase can have.
constexpr int kPhasedStage = stage_bytes<kXSiluUp>();

// n_phases == 0: census -- each workgroup writes its XCD to census[b].
template <int PF>
__global__ __launch_bounds__(kWave) void k_q8_gemv_phased(const PhaseDesc *__restrict__ phases, int n_phases,
                                                          uint32_t *sy, uint32_t per, uint32_t nx,
                                                          uint32_t *census) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[kBufs * kPhasedStage];
    const uint32_t b = blockIdx.x, wgs = gridDim.x;
    const uint32_t x = xcc_id();
    if (n_phases == 0) {
        if (lane_id() == 0) census[b] = x;
        return;
    }
    // the generation before this launch: the XCD's flag cannot move until
    // every workgroup of the XCD has arrived at this launch's first barrier
    const uint32_t g0 = __builtin_amdgcn_readfirstlane(load_agent(sync_flag(sy, x)));
    for (int s = 0; s < n_phases; ++s) {
        const PhaseDesc ph = phases[s];
        if (s > 0) phase_sync(sy, x, g0 + (uint32_t)s, per, nx, ph.acquire != 0);
        switch (ph.xmode) {
            case kXSiluUp: phase_work<PF, kXSiluUp>(ph, b, wgs, stage); break;
            case kXNormAdd: phase_work<PF, kXNormAdd>(ph, b, wgs, stage); break;
            default: phase_work<PF, kXFloat>(ph, b, wgs, stage); break;
        }
    }
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
template <int NW, int PF, int XM>
hipError_t launch_single_t(const OpDesc &op, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((k_q8_gemv<NW, PF, XM>), dim3((unsigned)grid), dim3(NW * kWave), 0, s, op);
    return hipGetLastError();
}
template <int NW, int PF, int XM>
hipError_t launch_fused_t(const OpDesc *d_ops, const Tile *d_tiles, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((k_q8_gemv_fused<NW, PF, XM>), dim3((unsigned)grid), dim3(NW * kWave), 0, s,
                       d_ops, d_tiles);
    return hipGetLastError();
}
template <int PF, int XM>
hipError_t launch_sk_t(const OpDesc *d_ops, const Piece *d_pieces, const uint32_t *d_begin,
                       const Tile *d_tails, int64_t n_sk, int64_t n_tail, hipStream_t s) {
    hipLaunchKernelGGL((k_q8_gemv_sk<PF, XM>), dim3((unsigned)(n_sk + n_tail)), dim3(kWave), 0, s, d_ops,
                       d_pieces, d_begin, d_tails, (uint32_t)n_sk);
    return hipGetLastError();
}
// Every launch shape for the float and integer paths; the decode step's
// input modes (SiLU·up, residual add + norm) in the shapes its plans use.
template <int XM>
hipError_t launch_single_v(const OpDesc &op, const Variant &v, int64_t grid, hipStream_t s) {
    switch (v.nw * 10 + v.pf) {
        case 11: return launch_single_t<1, 1, XM>(op, grid, s);
        case 41: return launch_single_t<4, 1, XM>(op, grid, s);
        default: break;
    }
    if constexpr (XM == kXFloat || XM == kXQuant) {
        switch (v.nw * 10 + v.pf) {
            case 12: return launch_single_t<1, 2, XM>(op, grid, s);
            case 21: return launch_single_t<2, 1, XM>(op, grid, s);
            case 22: return launch_single_t<2, 2, XM>(op, grid, s);
            case 42: return launch_single_t<4, 2, XM>(op, grid, s);
            default: break;
        }
    }
    return hipErrorInvalidValue;
}
template <int XM>
hipError_t launch_fused_v(const OpDesc *d_ops, const Tile *d_tiles, const Variant &v, int64_t grid,
                          hipStream_t s) {
    switch (v.nw * 10 + v.pf) {
        case 11: return launch_fused_t<1, 1, XM>(d_ops, d_tiles, grid, s);
        case 41: return launch_fused_t<4, 1, XM>(d_ops, d_tiles, grid, s);
        default: break;
    }
    if constexpr (XM == kXFloat || XM == kXQuant) {
        switch (v.nw * 10 + v.pf) {
            case 12: return launch_fused_t<1, 2, XM>(d_ops, d_tiles, grid, s);
            case 21: return launch_fused_t<2, 1, XM>(d_ops, d_tiles, grid, s);
            case 22: return launch_fused_t<2, 2, XM>(d_ops, d_tiles, grid, s);
            case 42: return launch_fused_t<4, 2, XM>(d_ops, d_tiles, grid, s);
            default: break;
        }
    }
    return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_gemv_single(const OpDesc &op, const Variant &v, int64_t grid, hipStream_t s,
                              int xmode) {
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
    switch (xmode) {
        case kXFloat: return launch_fused_v<kXFloat>(d_ops, d_tiles, v, grid, s);
        case kXQuant: return launch_fused_v<kXQuant>(d_ops, d_tiles, v, grid, s);
        case kXSiluUp: return launch_fused_v<kXSiluUp>(d_ops, d_tiles, v, grid, s);
        case kXNormAdd: return launch_fused_v<kXNormAdd>(d_ops, d_tiles, v, grid, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_streamk(const OpDesc *d_ops, const Piece *d_pieces, const uint32_t *d_begin,
                               const Tile *d_tails, int64_t n_sk, int64_t n_tail, int pf,
                               hipStream_t s, int xmode) {
    if (n_sk + n_tail <= 0) return hipErrorInvalidValue;
#define Q8_SK(XM)                                                                                 \
    return pf == 2 ? launch_sk_t<2, XM>(d_ops, d_pieces, d_begin, d_tails, n_sk, n_tail, s)       \
                   : launch_sk_t<1, XM>(d_ops, d_pieces, d_begin, d_tails, n_sk, n_tail, s);
    switch (xmode) {
        case kXFloat: Q8_SK(kXFloat)
        case kXQuant: Q8_SK(kXQuant)
        case kXSiluUp: Q8_SK(kXSiluUp)
        case kXNormAdd: Q8_SK(kXNormAdd)
        default: return hipErrorInvalidValue;
    }
#undef Q8_SK
}

hipError_t launch_gemv_phased(const PhaseDesc *d_phases, int n_phases, uint32_t *d_sync, uint32_t per,
                              uint32_t nx, int64_t wgs, int pf, hipStream_t s) {
    if (n_phases <= 0 || wgs <= 0 || pf != 1 || nx == 0 || nx > (uint32_t)kMaxXcc || (uint64_t)per * nx != (uint64_t)wgs)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_q8_gemv_phased<1>), dim3((unsigned)wgs), dim3(kWave), 0, s, d_phases, n_phases,
                       d_sync, per, nx, (uint32_t *)nullptr);
    return hipGetLastError();
}

hipError_t launch_gemv_phased_census(uint32_t *d_census, int64_t wgs, hipStream_t s) {
    if (wgs <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_q8_gemv_phased<1>), dim3((unsigned)wgs), dim3(kWave), 0, s,
                       (const PhaseDesc *)nullptr, 0, (uint32_t *)nullptr, 0u, 0u, d_census);
    return hipGetLastError();
}

int gemv_phased_blocks_per_cu(int pf) {
    int n = 0;
    if (pf != 1) return 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_q8_gemv_phased<1>, kWave, 0);
    return e == hipSuccess ? n : 0;
}

hipError_t launch_quantize_x(const float *x, void *xq, int64_t n, hipStream_t s) {
    const int64_t nb = n / kQuants;
    hipLaunchKernelGGL(k_quantize_x, dim3((unsigned)((nb + 7) / 8)), dim3(256), 0, s, x,
                       (uint8_t *)xq, nb);
    return hipGetLastError();
}

}  // namespace q8
