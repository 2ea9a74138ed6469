// q8_kernels.hip -- gfx950 kernels for the Q8_0 decode matvec.
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
#include "q8_internal.h"

namespace q8 {
namespace {

typedef __attribute__((address_space(3))) void LdsVoid;
// x (X) is read-only for a kernel's lifetime (outputs never overlap inputs
// and dependent ops never share a launch), so it is read through the
// constant address space: wave-uniform reads then become scalar loads.
typedef const __attribute__((address_space(4))) float CFloat;
typedef const __attribute__((address_space(1))) uint16_t GHalf;

__device__ __forceinline__ CFloat *cptr(const float *p) { return (CFloat *)p; }

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

// The 32 quants of block K as floats.
template <int K>
__device__ __forceinline__ void block_quants(const uint32_t (&D)[68], float (&qf)[kQuants],
                                             float &d) {
    constexpr int sb = K * kBlockBytes;
    d = half_to_float(D[sb >> 2] >> ((sb & 3) * 8));
#pragma unroll
    for (int j = 0; j < kQuants; ++j) qf[j] = quant(D, sb + 2 + j);
}

// s_waitcnt vmcnt(N), leaving expcnt and lgkmcnt unconstrained (gfx9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_vm0() { wait_vm<0>(); }
// direct loads per group of the matvec: 17 of W and one of x
constexpr int kLoadsPerGroup = kGroupChunks + 1;

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

// Issue the 17 direct HBM -> LDS loads of one group into stage `st`.
__device__ __forceinline__ void dma_group(const uint8_t *g, const uint32_t (&off)[kGroupChunks],
                                          uint8_t *st) {
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i)
        __builtin_amdgcn_global_load_lds((const void *)(g + off[i]),
                                         (LdsVoid *)(st + kWave * 16 * i), 16, 0, 0);
}

// Where lane `lane` finds its 16 bytes of the x slice of group kk: floats
// 4*(lane%8) .. +3 of block lane/8 of the group, i.e. of column block
// (8*kk + lane/8) mod nb (a group of a super-row wraps past the row end).
template <int RS>
__device__ __forceinline__ const float *x_slice_src(const OpDesc &op, int kk, int lane) {
    int b = kk * kGroupBlocks + (lane >> 3);
    if (RS > 1) b %= op.nb;
    return op.x + (int64_t)b * kQuants + 4 * (lane & 7);
}

// The matvec issues its direct loads from inline asm.  The compiler tracks
// LDS-DMA it emits itself and, unable to tell the two stages apart, waits
// for ALL outstanding loads before any LDS read -- which would stall every
// compute phase on the next group's loads.  Issued from asm, the loads are
// invisible to that tracking, and the kernel orders them itself: wait_vm_asm
// (a memory barrier for the compiler) before a stage is read, and a stage is
// refilled only after its last read.  m0 carries the LDS address; nothing
// else in the matvec kernels uses m0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane: global (sbase + voff) -> LDS (m0 + 16 * lane)
__device__ __forceinline__ void dma16_s(const uint8_t *sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds), "v"(voff), "s"(sbase) : "memory", "m0");
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

// One group: 17 loads of W and one load of its x slice (at st + kStageW).
template <int RS>
__device__ __forceinline__ void dma_group_x(const uint8_t *g, const uint32_t (&off)[kGroupChunks],
                                            uint8_t *st, const OpDesc &op, int kk, int lane) {
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(st));
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i) dma16_s(g, off[i], l0 + kWave * 16 * i);
    dma16_v(x_slice_src<RS>(op, kk, lane), l0 + kStageW);
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

constexpr int kSlots = 4;

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

// One workgroup tile of NW waves: NW/ks row tiles of 64 super-rows, each
// row tile's groups split over ks waves.  PF is how many groups each wave
// keeps in flight ahead of the one it computes (1 or 2; each stage holds one
// group, and with PF = 2 the stage a group was computed from is refilled
// right after that group's compute, so two groups stream while one waits).
template <int RS, int NW, int PF>
__device__ void fast_tile(const OpDesc &op, uint32_t tile, uint8_t *stage) {
    const int lane = lane_id();
    const int wave = wave_id();
    const int ks = op.ks;
    const int rt = wave / ks;                 // row tile within the workgroup
    const int ksl = wave - rt * ks;           // this wave's share of the groups
    const int tiles_per_wg = NW / ks;
    const int64_t sr0 = ((int64_t)tile * tiles_per_wg + rt) * kWave;
    const int nsr = op.nsr;
    uint8_t *st0 = stage + (size_t)wave * (kBufs * kStageBytes);

    float acc[kSlots][RS];
#pragma unroll
    for (int q = 0; q < kSlots; ++q)
#pragma unroll
        for (int k = 0; k < RS; ++k) acc[q][k] = 0.f;

    if (sr0 < nsr) {
        const int G = op.gsr;
        const int64_t srb = op.sr_bytes;
        const uint8_t *wt = op.w + sr0 * srb;
        const int last = (int)min((int64_t)nsr - 1 - sr0, (int64_t)kWave - 1);
        uint32_t off[kGroupChunks];
        chunk_offsets(off, lane, last, srb);
        const int ng = (G - ksl + ks - 1) / ks;  // groups kk = ksl + ks*t, t < ng
        auto issue = [&](int t) {
            const int kk = ksl + ks * t;
            dma_group_x<RS>(wt + (int64_t)kk * kGroupBytes, off, st0 + (t & 1) * kStageBytes, op,
                            kk, lane);
        };
        if (ng > 0) issue(0);
        if (PF == 2 && ng > 1) issue(1);
        for (int t = 0; t < ng; ++t) {
            uint8_t *cur = st0 + (t & 1) * kStageBytes;
            uint32_t D[68];
            // this group's W and x have landed in LDS (loads complete in order)
            if (PF == 2 && t + 1 < ng) wait_vm_asm<kLoadsPerGroup>();
            else wait_vm_asm<0>();
            read_group(cur, lane, D);
            if (PF == 1 && t + 1 < ng) issue(t + 1);
            group_dot<RS>(D, reinterpret_cast<const float4 *>(cur + kStageW), op, ksl + ks * t, acc);
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
                    stage + (size_t)owner * (kBufs * kStageBytes));
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

// ---------------------------------------------------------------- m > 1
// Small batch: the same stream of W, M activation rows (rows of X past
// op.m are clamped to the last one and never stored).
template <int M, int RS>
__device__ __forceinline__ void group_dot_m(const uint32_t (&D)[68], const OpDesc &op, int kk,
                                            float (&acc)[M][kSlots][RS]) {
    const int slot = kk & (kSlots - 1);
    const int bp = kk * kGroupBlocks;
    int r = (RS == 1) ? 0 : bp / op.nb;
    int cb = bp - r * op.nb;
    float sub[M];
#pragma unroll
    for (int i = 0; i < M; ++i) sub[i] = 0.f;
    float qf[kQuants];
    float d;
#define Q8_STEPM(K)                                                              \
    block_quants<K>(D, qf, d);                                                   \
    _Pragma("unroll") for (int i = 0; i < M; ++i) {                              \
        const int xi = i < op.m ? i : op.m - 1;                                  \
        CFloat *xb = cptr(op.x) + (int64_t)xi * op.x_stride + (int64_t)cb * kQuants; \
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;                            \
        _Pragma("unroll") for (int j = 0; j < kQuants; j += 4) {                 \
            a0 = fmaf(qf[j + 0], xb[j + 0], a0);                                 \
            a1 = fmaf(qf[j + 1], xb[j + 1], a1);                                 \
            a2 = fmaf(qf[j + 2], xb[j + 2], a2);                                 \
            a3 = fmaf(qf[j + 3], xb[j + 3], a3);                                 \
        }                                                                        \
        sub[i] = fmaf(d, (a0 + a1) + (a2 + a3), sub[i]);                         \
    }                                                                            \
    if (++cb == op.nb) {                                                         \
        _Pragma("unroll") for (int i = 0; i < M; ++i) {                          \
            flush_row<RS>(acc[i], slot, r, sub[i]); sub[i] = 0.f;                \
        }                                                                        \
        cb = 0; ++r;                                                             \
    }
    Q8_STEPM(0) Q8_STEPM(1) Q8_STEPM(2) Q8_STEPM(3)
    Q8_STEPM(4) Q8_STEPM(5) Q8_STEPM(6) Q8_STEPM(7)
#undef Q8_STEPM
#pragma unroll
    for (int i = 0; i < M; ++i) flush_row<RS>(acc[i], slot, r, sub[i]);
}

template <int M, int RS>
__device__ void fast_tile_m(const OpDesc &op, uint32_t tile, uint8_t *stage) {
    const int lane = lane_id();
    const int wave = wave_id();
    const int64_t sr0 = ((int64_t)tile * kWaves + wave) * kWave;  // no K split
    const int nsr = op.nsr;
    uint8_t *st0 = stage + (size_t)wave * (kBufs * kStageBytesM);
    if (sr0 >= nsr) return;

    float acc[M][kSlots][RS];
#pragma unroll
    for (int i = 0; i < M; ++i)
#pragma unroll
        for (int q = 0; q < kSlots; ++q)
#pragma unroll
            for (int k = 0; k < RS; ++k) acc[i][q][k] = 0.f;

    const int G = op.gsr;
    const int64_t srb = op.sr_bytes;
    const uint8_t *wt = op.w + sr0 * srb;
    const int last = (int)min((int64_t)nsr - 1 - sr0, (int64_t)kWave - 1);
    uint32_t off[kGroupChunks];
    chunk_offsets(off, lane, last, srb);
    dma_group(wt, off, st0);
    for (int t = 0; t < G; ++t) {
        uint8_t *cur = st0 + (t & 1) * kStageBytesM;
        uint32_t D[68];
        wait_vm0();
        read_group(cur, lane, D);
        if (t + 1 < G)
            dma_group(wt + (int64_t)(t + 1) * kGroupBytes, off, st0 + ((t + 1) & 1) * kStageBytesM);
        group_dot_m<M, RS>(D, op, t, acc);
    }
    if (sr0 + lane < nsr) {
        const int64_t row0 = (sr0 + lane) * RS;
#pragma unroll
        for (int i = 0; i < M; ++i) {
            if (i < op.m) {
                float *yr = op.y + (int64_t)i * op.y_stride + row0;
#pragma unroll
                for (int k = 0; k < RS; ++k)
                    yr[k] = combine_slots(acc[i][0][k], acc[i][1][k], acc[i][2][k], acc[i][3][k]);
            }
        }
    }
}

// ---------------------------------------------------------------- tail rows
// Generic path for the last p % rs rows: one wave per row, lane l takes
// blocks l, l+64, ...; blocks are read with 2-byte loads (a block is only
// 2-byte aligned in general).  Per-lane sums are flushed every 8 blocks and
// the 64 lanes meet in a fixed butterfly.
__device__ void tail_tile(const OpDesc &op, uint32_t tile, int waves) {
    const int lane = lane_id();
    const int wave = wave_id();
    const int64_t row = (int64_t)op.tail_row0 + (int64_t)tile * waves + wave;
    if (row >= op.p) return;
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
                a0 = fmaf((float)(int8_t)(v & 0xffu), xb[2 * j], a0);
                a1 = fmaf((float)(int8_t)(v >> 8), xb[2 * j + 1], a1);
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

template <int NW, int PF>
__device__ __forceinline__ void run_tile(const OpDesc &op, uint32_t t, uint8_t *stage) {
    if (t & kTailBit) {
        tail_tile(op, t & ~kTailBit, NW);
        return;
    }
    switch (op.rs) {
        case 1: fast_tile<1, NW, PF>(op, t, stage); break;
        case 2: fast_tile<2, NW, PF>(op, t, stage); break;
        case 4: fast_tile<4, NW, PF>(op, t, stage); break;
        default: fast_tile<8, NW, PF>(op, t, stage); break;
    }
}

template <int NW, int PF>
__global__ __launch_bounds__(NW * kWave) void k_q8_gemv(OpDesc op) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[NW * kBufs * kStageBytes];
    uint32_t t = blockIdx.x;
    if (t >= (uint32_t)op.fast_tiles) t = (t - op.fast_tiles) | kTailBit;
    run_tile<NW, PF>(op, t, stage);
}

template <int NW, int PF>
__global__ __launch_bounds__(NW * kWave) void k_q8_gemv_fused(const OpDesc *__restrict__ ops,
                                                              const Tile *__restrict__ tiles) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[NW * kBufs * kStageBytes];
    const Tile tl = tiles[blockIdx.x];
    const OpDesc op = ops[tl.op];
    run_tile<NW, PF>(op, tl.tile, stage);
}

template <int M>
__global__ __launch_bounds__(kThreads) void k_q8_gemm(OpDesc op) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[kWaves * kBufs * kStageBytesM];
    uint32_t t = blockIdx.x;
    if (t >= (uint32_t)op.fast_tiles) {
        tail_tile(op, t - op.fast_tiles, kWaves);
        return;
    }
    // the host sends widths whose super-rows exceed 2 rows to the m = 1 path
    if (op.rs == 1) fast_tile_m<M, 1>(op, t, stage);
    else fast_tile_m<M, 2>(op, t, stage);
}

}  // namespace

namespace {
template <int NW, int PF>
hipError_t launch_single_t(const OpDesc &op, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((k_q8_gemv<NW, PF>), dim3((unsigned)grid), dim3(NW * kWave), 0, s, op);
    return hipGetLastError();
}
template <int NW, int PF>
hipError_t launch_fused_t(const OpDesc *d_ops, const Tile *d_tiles, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((k_q8_gemv_fused<NW, PF>), dim3((unsigned)grid), dim3(NW * kWave), 0, s,
                       d_ops, d_tiles);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_gemv_single(const OpDesc &op, const Variant &v, int64_t grid, hipStream_t s) {
    switch (v.nw * 10 + v.pf) {
        case 11: return launch_single_t<1, 1>(op, grid, s);
        case 12: return launch_single_t<1, 2>(op, grid, s);
        case 21: return launch_single_t<2, 1>(op, grid, s);
        case 22: return launch_single_t<2, 2>(op, grid, s);
        case 41: return launch_single_t<4, 1>(op, grid, s);
        case 42: return launch_single_t<4, 2>(op, grid, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_fused(const OpDesc *d_ops, const Tile *d_tiles, const Variant &v,
                             int64_t grid, hipStream_t s) {
    switch (v.nw * 10 + v.pf) {
        case 11: return launch_fused_t<1, 1>(d_ops, d_tiles, grid, s);
        case 12: return launch_fused_t<1, 2>(d_ops, d_tiles, grid, s);
        case 21: return launch_fused_t<2, 1>(d_ops, d_tiles, grid, s);
        case 22: return launch_fused_t<2, 2>(d_ops, d_tiles, grid, s);
        case 41: return launch_fused_t<4, 1>(d_ops, d_tiles, grid, s);
        case 42: return launch_fused_t<4, 2>(d_ops, d_tiles, grid, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_single(const OpDesc &op, int mpad, int64_t grid, hipStream_t s) {
    switch (mpad) {
        case 2: hipLaunchKernelGGL(k_q8_gemm<2>, dim3((unsigned)grid), dim3(kThreads), 0, s, op); break;
        case 4: hipLaunchKernelGGL(k_q8_gemm<4>, dim3((unsigned)grid), dim3(kThreads), 0, s, op); break;
        case 8: hipLaunchKernelGGL(k_q8_gemm<8>, dim3((unsigned)grid), dim3(kThreads), 0, s, op); break;
        case 16: hipLaunchKernelGGL(k_q8_gemm<16>, dim3((unsigned)grid), dim3(kThreads), 0, s, op); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace q8
