// q8_gemm.hip -- gfx950 kernels for the small-batch product Y = X W^T
// (2 <= m <= 16 rows of X in one pass over W): on the matrix cores, with X
// split into exact bfloat16 parts, and on the vector units in the matvec's
// layout; both split their (row tile, group) items stream-K style.
#include "q8_device.h"
#include "q8_gemm.h"

namespace q8 {
namespace {

// ---------------------------------------------------------------- m > 1
// Small batch, Y = X W^T for m <= 16 rows of X, on the matrix cores.
//
// At m = 16 the contraction needs 16 FMAs per weight: over the FP32 vector
// units that is ~3x slower than HBM delivers weights, so it runs on
// v_mfma_f32_16x16x32_bf16 instead, exactly:
//   * A (16 x 32) is X: row i = activation row, k = column in the block.
//     Each x is split into three bfloat16 parts, h + m + l == x exactly
//     (8 + 8 + 8 significant bits; non-finite x keeps only h).
//   * B (32 x 16) is the block's int8 quants, which bfloat16 holds exactly;
//     column j = weight row.  Every product is exact in float32.
//   * C (16 x 16) collects one block; the lane that holds C[i][j] also read
//     the quants of row j, so it scales its four C values by that row's
//     block scale and adds them to per-group subtotals.
// Lane layout (gfx950, checked on the device): A[i][k] is element k%8 of
// lane i + 16*(k/8), B[k][j] element k%8 of lane j + 16*(k/8), and C[i][j]
// element i%4 of lane j + 16*(i/4).
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_as_float(__bf16 h) {
    return __builtin_bit_cast(float, (uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}

// x = h + m + l exactly, each part bfloat16 (round to nearest even).
__device__ __forceinline__ void split3(const float (&x)[8], bf16x8 &h, bf16x8 &m, bf16x8 &l) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 hh = (__bf16)x[e];
        float r = x[e] - bf16_as_float(hh);
        r = __builtin_isfinite(x[e]) ? r : 0.f;
        const __bf16 mm = (__bf16)r;
        const float r2 = r - bf16_as_float(mm);
        h[e] = hh;
        m[e] = mm;
        l[e] = (__bf16)r2;
    }
}

// The A operands of X, split once per call by k_split_x into
// xs[b][part][i][g]: for block b and part (h, m, l), the bf16x8 of columns
// 32b + 8g .. 32b + 8g + 7 of row i, 16 rows x 4 column groups in a
// contiguous 1 KiB, so that one load instruction of a wave (lane = i + 16 g
// reads entry 4i + g) covers whole cache lines.  Rows i >= m are never
// written or read.
__device__ __forceinline__ int64_t xpart_index(int b, int part, int i, int g) {
    return ((int64_t)b * 3 + part) * 64 + i * 4 + g;
}

__global__ __launch_bounds__(256) void k_split_x(const float *__restrict__ X,
                                                 bf16x8 *__restrict__ xs, int m, int n) {
    const int nb = n / kQuants;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;   // (i, b, g)
    if (t >= (int64_t)m * nb * 4) return;
    const int g = (int)(t & 3), b = (int)((t >> 2) % nb), i = (int)((t >> 2) / nb);
    const float4 *src = reinterpret_cast<const float4 *>(X) + 2 * t;
    const float4 v0 = src[0], v1 = src[1];
    const float x[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    XParts o;
    split3(x, o.h, o.m, o.l);
    xs[xpart_index(b, 0, i, g)] = o.h;
    xs[xpart_index(b, 1, i, g)] = o.m;
    xs[xpart_index(b, 2, i, g)] = o.l;
}

__global__ __launch_bounds__(256) void k_zero_u32(uint32_t *__restrict__ p, int64_t n) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t < n) p[t] = 0u;
}

// The A operand of block K of group kk for lane (i, g).  Rows i >= m load
// row m - 1 again: the matrix core keeps rows of A apart, so those C rows
// are never looked at, and no lane needs a branch or a zero fill.
template <int RS>
__device__ __forceinline__ XParts load_parts(const GemmDesc &d, int kk, int K, int i, int g) {
    int b = kk * kGroupBlocks + K;
    if (RS > 1) b %= d.nb;
    const int ii = i < d.m ? i : d.m - 1;
    XParts r;
    r.h = d.xs[xpart_index(b, 0, ii, g)];
    r.m = d.xs[xpart_index(b, 1, ii, g)];
    r.l = d.xs[xpart_index(b, 2, ii, g)];
    return r;
}

// All eight blocks' A operands of group kk (96 VGPRs), loaded together so
// that their latency overlaps the group's W loads instead of stalling every
// block.
template <int RS>
__device__ __forceinline__ void load_xgroup(const GemmDesc &d, int kk, int lane,
                                            XParts (&xg)[kGroupBlocks]) {
    const int i = lane & 15, g = lane >> 4;
#pragma unroll
    for (int K = 0; K < kGroupBlocks; ++K) xg[K] = load_parts<RS>(d, kk, K, i, g);
}

template <int RS>
__device__ __forceinline__ void flush_tile(f32x4 (&acc)[4][RS], f32x4 (&sub)[4], int r) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int k = 0; k < RS; ++k)
            if (k == r) acc[t][k] += sub[t];
        sub[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// The LDS words a lane needs for block K of tile t: the 8 quants it feeds
// (two dwords, or three when they start 2 bytes past a dword) and its row's
// scale.
struct BRaw {
    uint32_t a0, a1, a2;
    uint32_t dh;
};

template <int K>
__device__ __forceinline__ void read_braw(const uint8_t *stage, int j, int g, BRaw (&r)[4]) {
    constexpr int q0 = K * kBlockBytes + 2;   // first quant byte of the block
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint8_t *grp = stage + kGroupBytes * (16 * t + j);
        if constexpr ((q0 & 3) == 0) {
            const uint32_t *p = reinterpret_cast<const uint32_t *>(grp + q0 + 8 * g);
            r[t].a0 = p[0];
            r[t].a1 = p[1];
        } else {
            const uint32_t *p = reinterpret_cast<const uint32_t *>(grp + q0 - 2 + 8 * g);
            r[t].a0 = p[0];
            r[t].a1 = p[1];
            r[t].a2 = p[2];
        }
        r[t].dh = *reinterpret_cast<const uint16_t *>(grp + K * kBlockBytes);
    }
}

// Raw words -> the B operands (bf16 quants) and the scales of block K.
template <int K>
__device__ __forceinline__ void convert_b(const BRaw (&r)[4], bf16x8 (&bq)[4], float (&dsc)[4]) {
    constexpr int q0 = K * kBlockBytes + 2;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t w0 = r[t].a0, w1 = r[t].a1;
        if constexpr ((q0 & 3) != 0) {
            w0 = __builtin_amdgcn_alignbyte(r[t].a1, r[t].a0, 2);
            w1 = __builtin_amdgcn_alignbyte(r[t].a2, r[t].a1, 2);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bq[t][e] = (__bf16)(float)(int8_t)(w0 >> (8 * e));
            bq[t][4 + e] = (__bf16)(float)(int8_t)(w1 >> (8 * e));
        }
        dsc[t] = half_to_float(r[t].dh);
    }
}

// One group of the wave's 64 super-rows (4 MFMA tiles of 16), all blocks;
// xg holds the group's A operands.  A three-deep software pipeline over the
// blocks: while block K's MFMAs run, block K+1's quants are converted, block
// K+2's words are read from LDS, and block K-1's results are scaled and
// added, so the vector and matrix units and the LDS work side by side.
template <int RS>
__device__ __forceinline__ void group_mfma(const uint8_t *stage, const GemmDesc &d, int kk,
                                           int lane, const XParts (&xg)[kGroupBlocks],
                                           f32x4 (&acc)[4][RS]) {
    const int j = lane & 15, g = lane >> 4;
    f32x4 sub[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) sub[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    int r = 0, cb = kk * kGroupBlocks;
    if (RS > 1) { r = cb / d.nb; cb -= r * d.nb; }
    BRaw R0[4], R1[4];
    bf16x8 B0[4], B1[4];
    float D0[4], D1[4];
    f32x4 C0[4], C1[4];
    auto accumulate = [&](const float (&dd)[4], const f32x4 (&cc)[4]) {
#pragma unroll
        for (int t = 0; t < 4; ++t) sub[t] += dd[t] * cc[t];
        if (RS > 1 && ++cb == d.nb) { flush_tile<RS>(acc, sub, r); cb = 0; ++r; }
    };
    auto mfma3 = [&](const XParts &x, const bf16x8 (&bb)[4], f32x4 (&cc)[4]) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
            cc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.h, bb[t], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int t = 0; t < 4; ++t) cc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.m, bb[t], cc[t], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < 4; ++t) cc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.l, bb[t], cc[t], 0, 0, 0);
    };
    read_braw<0>(stage, j, g, R0);
    read_braw<1>(stage, j, g, R1);
    convert_b<0>(R0, B0, D0);
    // step K: A = block K's parity, Bp = the other one
#define Q8_MSTEP(K, RA, RB, BA, BB, DA, DB, CA, CB)                                     \
    {                                                                                   \
        asm volatile("" ::: "memory"); /* bounds the registers the steps hold */       \
        if constexpr ((K) >= 1) accumulate(DB, CB);                                     \
        if constexpr ((K) + 2 < kGroupBlocks) read_braw<((K) + 2) % kGroupBlocks>(stage, j, g, RA); \
        if constexpr ((K) + 1 < kGroupBlocks) convert_b<((K) + 1) % kGroupBlocks>(RB, BB, DB); \
        mfma3(xg[K], BA, CA);                                                           \
    }
    Q8_MSTEP(0, R0, R1, B0, B1, D0, D1, C0, C1)
    Q8_MSTEP(1, R1, R0, B1, B0, D1, D0, C1, C0)
    Q8_MSTEP(2, R0, R1, B0, B1, D0, D1, C0, C1)
    Q8_MSTEP(3, R1, R0, B1, B0, D1, D0, C1, C0)
    Q8_MSTEP(4, R0, R1, B0, B1, D0, D1, C0, C1)
    Q8_MSTEP(5, R1, R0, B1, B0, D1, D0, C1, C0)
    Q8_MSTEP(6, R0, R1, B0, B1, D0, D1, C0, C1)
    Q8_MSTEP(7, R1, R0, B1, B0, D1, D0, C1, C0)
#undef Q8_MSTEP
    accumulate(D1, C1);   // block 7
    flush_tile<RS>(acc, sub, RS == 1 ? 0 : r);
}

// Groups [g0, g1) of row tile rt (64 super-rows = 4 MFMA tiles), added
// into acc: two W stages and two register sets of A operands, used in turn,
// so the next group's loads stream while this one computes (one wave per
// SIMD; a single-stage variant with two waves per SIMD measured no faster).
template <int RS>
__device__ void gemm_run(const GemmDesc &d, int rt, int g0, int g1, uint8_t *stage,
                         f32x4 (&acc)[4][RS]) {
    const int lane = lane_id();
    const int64_t sr0 = (int64_t)rt * kWave;
    const int last = (int)min((int64_t)d.nsr - 1 - sr0, (int64_t)kWave - 1);
    const uint8_t *wt = d.w + sr0 * d.sr_bytes;
    uint32_t off[kGroupChunks];
    chunk_offsets(off, lane, last, d.sr_bytes);
    auto issue_w = [&](int kk, uint8_t *st) {
        const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(st));
        const uint8_t *gb = wt + (int64_t)kk * kGroupBytes;
#pragma unroll
        for (int c = 0; c < kGroupChunks; ++c) dma16_s(gb, off[c], l0 + kWave * 16 * c);
    };
    // Every wait is vmcnt(0) through the builtin, so the compiler knows that
    // the A operands it loaded (ordinary loads) have landed as well.
    XParts xa[kGroupBlocks], xb[kGroupBlocks];
    uint8_t *st1 = stage + kStageBytesM;
    if (g0 < g1) {
        issue_w(g0, stage);
        load_xgroup<RS>(d, g0, lane, xa);
    }
    for (int kk = g0; kk < g1; kk += 2) {
        __builtin_amdgcn_s_waitcnt(0x0F70);
        asm volatile("" ::: "memory");
        if (kk + 1 < g1) {
            issue_w(kk + 1, st1);
            load_xgroup<RS>(d, kk + 1, lane, xb);
        }
        group_mfma<RS>(stage, d, kk, lane, xa, acc);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // stage 0 fully read
        asm volatile("" ::: "memory");
        if (kk + 1 >= g1) break;
        __builtin_amdgcn_s_waitcnt(0x0F70);
        asm volatile("" ::: "memory");
        if (kk + 2 < g1) {
            issue_w(kk + 2, stage);
            load_xgroup<RS>(d, kk + 2, lane, xa);
        }
        group_mfma<RS>(st1, d, kk + 1, lane, xb, acc);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // stage 1 fully read
        asm volatile("" ::: "memory");
    }
}

// Stream-K split of the small-batch product: the row_tiles * G (row tile,
// group) items, row tile major, are cut into gridDim-many equal contiguous
// ranges, one per workgroup.  Workgroup b owns items [b*N/W, (b+1)*N/W).
__device__ __forceinline__ int64_t sk_first_item(int64_t b, int64_t N, int64_t W) {
    return b * N / W;
}
// The workgroup whose range holds item i.
__device__ __forceinline__ int64_t sk_owner(int64_t i, int64_t N, int64_t W) {
    return ((i + 1) * W - 1) / N;
}

// lane holds C[i = 4g + e][super-row 16t + j], row-in-super-row k
template <int RS>
__device__ __forceinline__ void store_tile(const GemmDesc &d, int64_t sr0, int lane,
                                           const f32x4 (&acc)[4][RS]) {
    const int j = lane & 15, g = lane >> 4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int64_t sr = sr0 + 16 * t + j;
        if (sr >= d.nsr) continue;
#pragma unroll
        for (int k = 0; k < RS; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ii = 4 * g + e;
                if (ii < d.m) d.Y[(int64_t)ii * d.p + sr * RS + k] = acc[t][k][e];
            }
    }
}

// A row tile shared by several workgroups: each parks its share (m X rows x
// 64 * RS W rows of floats) in a slot of its own and counts its arrival; the
// last of `contributors` to arrive adds the shares in workgroup order and
// stores Y.  A workgroup's items are contiguous, so only its first and last
// row tiles can be shared: workgroup q owns slots 2q (its first tile) and
// 2q + 1 (its last).  Of a tile's contributors only the first can hold it as
// its last tile.  Partials are written and read with device-scope (sc1)
// accesses, coherent across the XCDs' L2s by themselves (no fence has to
// write back or invalidate a whole L2); the wait before the counter makes
// this share's stores complete before its arrival is counted.
template <int RS>
__device__ __forceinline__ float *partial_slot(const GemmDesc &d, int64_t q, int last) {
    return d.ws + (2 * q + last) * ((int64_t)d.m * kWave * RS);
}

__device__ __forceinline__ void store_partial(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival at tile rt's counter: 64 bits, the call's epoch above the count of
// arrivals.  An arrival adds one; if the counter held another epoch (an
// earlier call's, or whatever the workspace held), this call's epoch with no
// arrivals is swapped in -- unless another arrival of the call already did
// -- and the arrival is made again.  So no call has to clear the counters
// and the last to arrive needs no reset; only arrivals that meet an old
// epoch take the extra round trips.  Returns the call's arrivals before this
// one.  (Only this call's arrivals set its epoch, so the second add always
// meets it.)
__device__ __forceinline__ uint32_t arrive(const GemmDesc &d, int rt) {
    unsigned long long *c = d.cnt + rt;
    constexpr unsigned long long kHi = 0xFFFFFFFF00000000ull;
    const unsigned long long tag = (unsigned long long)d.epoch << 32;
    for (;;) {
        const unsigned long long old = __hip_atomic_fetch_add(c, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((old & kHi) == tag) return (uint32_t)old;
        unsigned long long cur = old + 1ull;
        while ((cur & kHi) != tag &&
               !__hip_atomic_compare_exchange_strong(c, &cur, tag, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT)) {
        }
    }
}

// Called by every lane once this share's partial is stored; `first` is the
// tile's first contributing workgroup.
template <int RS>
__device__ void arrive_reduce(const GemmDesc &d, int rt, int64_t first, int contributors, int lane) {
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
    uint32_t prev = 0;
    if (lane == 0) prev = arrive(d, rt);
    prev = __shfl(prev, 0, kWave);
    if (prev != (uint32_t)contributors - 1) return;
    asm volatile("" ::: "memory");
    const int64_t sr0 = (int64_t)rt * kWave;
    // the first contributor's share is in its last-tile slot when its range
    // began before this tile
    const int64_t N = (int64_t)d.row_tiles * d.gsr;
    const int first_last = sk_first_item(first, N, d.fast_wgs) < (int64_t)rt * d.gsr ? 1 : 0;
    // A lane sums kIdx outputs at a time, kBatch shares of each in flight
    // (32 loads per round trip); every sum still runs in workgroup order.
    // Past the last contributor the share index is clamped and the value
    // dropped; rows past the matrix's last row are loaded (in the slot) but
    // not stored.
    constexpr int kBatch = 8, kIdx = 4;
    const int total = d.m * (kWave * RS);
    for (int idx0 = lane; idx0 < total; idx0 += kIdx * kWave) {
        float v[kIdx];
#pragma unroll
        for (int k = 0; k < kIdx; ++k) v[k] = 0.f;
        for (int q0 = 0; q0 < contributors; q0 += kBatch) {
            const float *src[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int q = min(q0 + u, contributors - 1);
                src[u] = partial_slot<RS>(d, first + q, q == 0 ? first_last : 0);
            }
            float t[kIdx][kBatch];
#pragma unroll
            for (int k = 0; k < kIdx; ++k) {
                const int idx = idx0 + k * kWave;
#pragma unroll
                for (int u = 0; u < kBatch; ++u)
                    t[k][u] = idx < total ? __hip_atomic_load(src[u] + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                          : 0.f;
            }
#pragma unroll
            for (int k = 0; k < kIdx; ++k)
#pragma unroll
                for (int u = 0; u < kBatch; ++u)
                    if (q0 + u < contributors) v[k] = (q0 + u == 0) ? t[k][u] : v[k] + t[k][u];
        }
#pragma unroll
        for (int k = 0; k < kIdx; ++k) {
            const int idx = idx0 + k * kWave;
            const int ii = idx / (kWave * RS);
            const int rr = idx - ii * (kWave * RS);
            if (idx < total && sr0 + rr / RS < d.nsr) d.Y[(int64_t)ii * d.p + sr0 * RS + rr] = v[k];
        }
    }
}

// The matrix-core share: lane (j, g) holds C[4g + e][16t + j] of tile t.
template <int RS>
__device__ void partial_tile(const GemmDesc &d, int rt, int64_t b, int last, int64_t first, int contributors,
                             int lane, const f32x4 (&acc)[4][RS]) {
    const int j = lane & 15, g = lane >> 4;
    float *mine = partial_slot<RS>(d, b, last);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int k = 0; k < RS; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * g + e < d.m)
                    store_partial(mine + (4 * g + e) * (kWave * RS) + (16 * t + j) * RS + k,
                                  acc[t][k][e]);
    arrive_reduce<RS>(d, rt, first, contributors, lane);
}

// Workgroup b's range of (row tile, group) items.
template <int RS>
__device__ void gemm_streamk(const GemmDesc &d, int64_t b, uint8_t *stage) {
    const int lane = lane_id();
    const int64_t G = d.gsr, N = (int64_t)d.row_tiles * G, W = d.fast_wgs;
    const int64_t it0 = sk_first_item(b, N, W);
    int64_t it = it0;
    const int64_t end = sk_first_item(b + 1, N, W);
    while (it < end) {
        const int rt = (int)(it / G);
        const int g0 = (int)(it - (int64_t)rt * G);
        const int g1 = (int)min(G, (int64_t)g0 + (end - it));
        f32x4 acc[4][RS];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int k = 0; k < RS; ++k) acc[t][k] = f32x4{0.f, 0.f, 0.f, 0.f};
        gemm_run<RS>(d, rt, g0, g1, stage, acc);
        if (g0 == 0 && g1 == G) {
            store_tile<RS>(d, (int64_t)rt * kWave, lane, acc);
        } else {
            const int64_t first = sk_owner((int64_t)rt * G, N, W);
            const int64_t contributors = sk_owner((int64_t)rt * G + G - 1, N, W) - first + 1;
            partial_tile<RS>(d, rt, b, it != it0, first, (int)contributors, lane, acc);
        }
        it += g1 - g0;
    }
}

// ---------------------------------------------------------------- small m, vector units
// Y = X W^T for m = M rows of X (2 <= M <= 4) in the matvec's layout: one
// lane per super-row, the group's 17 chunks of W and the x slices of all M
// rows arrive by the same direct loads, and every quant is converted once and
// then used for each row.  Per row, the arithmetic is the matvec's (four
// chains of eight per block, the block sum scaled once, groups into four
// slots).  Work is split stream-K style like the matrix-core kernel's.
// One stage: the group's W, then its x slices of all M rows.
template <int M>
struct VStage {
    static constexpr int kBytes = kStageW + M * kStageX;
};

// d and S_i = sum_j q_j x_i[j] for block K and each row i of X.
template <int K, int M>
__device__ __forceinline__ void block_terms_m(const uint32_t (&D)[68], const uint8_t *xst,
                                              float &d, float (&s)[M]) {
    constexpr int sb = K * kBlockBytes;
    d = half_to_float(D[sb >> 2] >> ((sb & 3) * 8));
    float q[kQuants];
#pragma unroll
    for (int j = 0; j < kQuants; ++j) q[j] = quant(D, sb + 2 + j);
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const float4 *xs = reinterpret_cast<const float4 *>(xst + i * kStageX);
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
        for (int j = 0; j < kQuants; j += 4) {
            const float4 xv = xs[(K * kQuants + j) / 4];
            a0 = fmaf(q[j + 0], xv.x, a0);
            a1 = fmaf(q[j + 1], xv.y, a1);
            a2 = fmaf(q[j + 2], xv.z, a2);
            a3 = fmaf(q[j + 3], xv.w, a3);
        }
        s[i] = (a0 + a1) + (a2 + a3);
    }
}

template <int RS, int M>
__device__ __forceinline__ void group_dot_m(const uint32_t (&D)[68], const uint8_t *xst,
                                            const GemmDesc &gd, int kk,
                                            float (&acc)[M][kSlots][RS]) {
    const int slot = kk & (kSlots - 1);
    float sub[M], s[M], d;
#pragma unroll
    for (int i = 0; i < M; ++i) sub[i] = 0.f;
    int r = 0, cb = 0;
    if (RS > 1) {
        const int bp = kk * kGroupBlocks;
        r = bp / gd.nb;
        cb = bp - r * gd.nb;
    }
    // A block's sums are finished before the next block's x is read: the
    // compiler would otherwise read all eight blocks' x (8 * M * 32 floats)
    // up front and run out of registers.
#define Q8_VSTEP(K)                                                             \
    block_terms_m<K, M>(D, xst, d, s);                                          \
    _Pragma("unroll") for (int i = 0; i < M; ++i) {                             \
        sub[i] = fmaf(d, s[i], sub[i]);                                         \
        asm volatile("" : "+v"(sub[i]) :: "memory");                            \
    }                                                                           \
    if (RS > 1 && ++cb == gd.nb) {                                              \
        _Pragma("unroll") for (int i = 0; i < M; ++i) {                         \
            flush_row<RS>(acc[i], slot, r, sub[i]);                             \
            sub[i] = 0.f;                                                       \
        }                                                                       \
        cb = 0;                                                                 \
        ++r;                                                                    \
    }
    Q8_VSTEP(0) Q8_VSTEP(1) Q8_VSTEP(2) Q8_VSTEP(3)
    Q8_VSTEP(4) Q8_VSTEP(5) Q8_VSTEP(6) Q8_VSTEP(7)
#undef Q8_VSTEP
#pragma unroll
    for (int i = 0; i < M; ++i) flush_row<RS>(acc[i], slot, RS == 1 ? 0 : r, sub[i]);
}

// Groups [g0, g1) of row tile rt, double-buffered: the next group's loads
// stream while this one is computed.  (Two groups in flight, with a ring of
// three x stages, measured no faster: the x reads, not the loads, bound it.)
template <int RS, int M>
__device__ void vsmall_run(const GemmDesc &d, int rt, int g0, int g1, uint8_t *stage,
                           float (&acc)[M][kSlots][RS]) {
    constexpr int SB = VStage<M>::kBytes;
    const int lane = lane_id();
    const int64_t sr0 = (int64_t)rt * kWave;
    const int last = (int)min((int64_t)d.nsr - 1 - sr0, (int64_t)kWave - 1);
    const uint8_t *wt = d.w + sr0 * d.sr_bytes;
    uint32_t off[kGroupChunks];
    chunk_offsets(off, lane, last, d.sr_bytes);
    // lane l carries floats 4(l%8) .. +3 of block l/8 of the group
    const int xb = lane >> 3, xo = 4 * (lane & 7);
    auto issue = [&](int kk, uint8_t *st) {
        const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(st));
        const uint8_t *gb = uniform_ptr(wt + (int64_t)kk * kGroupBytes);
#pragma unroll
        for (int c = 0; c < kGroupChunks; ++c) dma16_s(gb, off[c], l0 + kWave * 16 * c);
        int b = kk * kGroupBlocks + xb;
        if (RS > 1) b %= d.nb;
#pragma unroll
        for (int i = 0; i < M; ++i)
            dma16_v(d.X + (int64_t)i * d.n + (int64_t)b * kQuants + xo, l0 + kStageW + i * kStageX);
    };
    if (g0 < g1) issue(g0, stage);
    for (int kk = g0; kk < g1; ++kk) {
        uint8_t *cur = stage + ((kk - g0) & 1) * SB;
        uint32_t D[68];
        wait_vm_asm<0>();   // this group's W and x have landed
        read_group(cur, lane, D);
        // the other stage was last read by the previous group, whose reads
        // have all returned (their values are used)
        if (kk + 1 < g1) issue(kk + 1, stage + ((kk + 1 - g0) & 1) * SB);
        group_dot_m<RS, M>(D, cur + kStageW, d, kk, acc);
    }
}

template <int RS, int M>
__device__ void vsmall_streamk(const GemmDesc &d, int64_t b, uint8_t *stage) {
    const int lane = lane_id();
    const int64_t G = d.gsr, N = (int64_t)d.row_tiles * G, W = d.fast_wgs;
    const int64_t it0 = sk_first_item(b, N, W);
    int64_t it = it0;
    const int64_t end = sk_first_item(b + 1, N, W);
    while (it < end) {
        const int rt = (int)(it / G);
        const int g0 = (int)(it - (int64_t)rt * G);
        const int g1 = (int)min(G, (int64_t)g0 + (end - it));
        float acc[M][kSlots][RS];
#pragma unroll
        for (int i = 0; i < M; ++i)
#pragma unroll
            for (int q = 0; q < kSlots; ++q)
#pragma unroll
                for (int k = 0; k < RS; ++k) acc[i][q][k] = 0.f;
        vsmall_run<RS, M>(d, rt, g0, g1, stage, acc);
        const int64_t sr = (int64_t)rt * kWave + lane;
        if (g0 == 0 && g1 == G) {
            if (sr < d.nsr)
#pragma unroll
                for (int i = 0; i < M; ++i)
#pragma unroll
                    for (int k = 0; k < RS; ++k)
                        d.Y[(int64_t)i * d.p + sr * RS + k] =
                            combine_slots(acc[i][0][k], acc[i][1][k], acc[i][2][k], acc[i][3][k]);
        } else {
            const int64_t first = sk_owner((int64_t)rt * G, N, W);
            const int64_t contributors = sk_owner((int64_t)rt * G + G - 1, N, W) - first + 1;
            float *mine = partial_slot<RS>(d, b, it != it0);
#pragma unroll
            for (int i = 0; i < M; ++i)
#pragma unroll
                for (int k = 0; k < RS; ++k)
                    store_partial(mine + i * (kWave * RS) + lane * RS + k,
                                  combine_slots(acc[i][0][k], acc[i][1][k], acc[i][2][k], acc[i][3][k]));
            arrive_reduce<RS>(d, rt, first, (int)contributors, lane);
        }
        it += g1 - g0;
    }
}

// ---------------------------------------------------------------- small m, lanes over rows and blocks
// Y = X W^T for m = M (2 or 3) rows of X where every row is one super-row
// (n a multiple of 256).  A group's W tile and its x slices arrive by direct
// loads as in k_q8_gemm_valu, but lane (r, c) = (lane / 4, lane % 4) takes
// blocks 2c and 2c + 1 of the tile's rows r, r + 16, r + 32 and r + 48.  So
// it needs the x values of two blocks per row of X (64 floats), read from
// LDS into registers once per block and used for its four rows, where a
// lane per row needs every x value of the group through broadcast reads.
// The x slices are staged transposed (LDS slot 4k + c holds floats 64c + 4k
// .. +3 of the slice), so that the four lanes' reads of one instruction hit
// distinct banks.  Each block's sum is the matvec's (four chains of eight,
// scaled once); a lane's two blocks of a row go into that row's slot kk % 4,
// and when the row tile is done the four lanes of a row meet in a butterfly.
// No bf16 split of X is needed, so a call is one launch.  Two waves per
// workgroup share the stages, each taking half of every group's rows.

// Block PAR (0: 2c, 1: 2c + 1) of a local row: D holds the 9 dwords from
// the 4-byte boundary at or before the block's first byte (the block starts
// 2 * PAR bytes in), xv[i] the block's 32 x values of row i of X.  Returns d
// and the sums S_i = sum_j q_j x_i[j], each as four chains of eight.
template <int PAR, int M>
__device__ __forceinline__ void vrow_block(const uint32_t (&D)[68], const float4 (&xv)[M][8],
                                           float &d, float (&s)[M]) {
    constexpr int sb = 2 * PAR;   // the block's first byte in D
    d = half_to_float(D[sb >> 2] >> ((sb & 3) * 8));
    float a[M][4];
#pragma unroll
    for (int i = 0; i < M; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) a[i][t] = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        float q[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) q[t] = quant(D, sb + 2 + 4 * u + t);
#pragma unroll
        for (int i = 0; i < M; ++i) {
            const float4 x = xv[i][u];
            a[i][0] = fmaf(q[0], x.x, a[i][0]);
            a[i][1] = fmaf(q[1], x.y, a[i][1]);
            a[i][2] = fmaf(q[2], x.z, a[i][2]);
            a[i][3] = fmaf(q[3], x.w, a[i][3]);
        }
    }
#pragma unroll
    for (int i = 0; i < M; ++i) s[i] = (a[i][0] + a[i][1]) + (a[i][2] + a[i][3]);
}

// Groups [g0, g1) of row tile rt, double-buffered like vsmall_run.  NW
// waves share the stages: wave w takes local rows HW*w .. HW*w + HW - 1
// (HW = 4 / NW), the group's direct loads are split between the waves, and
// with NW > 1 a barrier per group makes every wave's loads visible and
// every wave done with the other stage before it is refilled.
template <int M, int NW>
__device__ void vrow_run(const GemmDesc &d, int rt, int g0, int g1, uint8_t *stage,
                         float (&acc)[4 / NW][M][kSlots]) {
    constexpr int SB = VStage<M>::kBytes;
    constexpr int HW = 4 / NW;
    const int lane = lane_id();
    const int wave = NW > 1 ? wave_id() : 0;
    const int r = lane >> 2, c = lane & 3;
    const int64_t sr0 = (int64_t)rt * kWave;
    const int last = (int)min((int64_t)d.nsr - 1 - sr0, (int64_t)kWave - 1);
    const uint8_t *wt = d.w + sr0 * d.sr_bytes;
    uint32_t off[kGroupChunks];
    chunk_offsets(off, lane, last, d.sr_bytes);
    // this lane's 16 bytes of a group's x slice (LDS slot `lane`): floats
    // 64c + 4r .. +3, i.e. float4 r of the 16 that lane (., c) reads
    const float *xsrc = d.X + 64 * c + 4 * r;
    // loads [k_lo, k_hi) of the group's 17 W loads, and the x slices, are this wave's
    const int k_lo = kGroupChunks * wave / NW;
    const int k_hi = kGroupChunks * (wave + 1) / NW;
    const bool does_x = NW == 1 || wave == NW - 1;
    auto issue = [&](int kk, uint8_t *st) {
        const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(st));
        const uint8_t *gb = uniform_ptr(wt + (int64_t)kk * kGroupBytes);
#pragma unroll
        for (int k = 0; k < kGroupChunks; ++k)
            if (k >= k_lo && k < k_hi) dma16_s(gb, off[k], l0 + kWave * 16 * k);
        if (does_x) {
            const float *xk = xsrc + (int64_t)kk * (kGroupBlocks * kQuants);
#pragma unroll
            for (int i = 0; i < M; ++i) dma16_v(xk + (int64_t)i * d.n, l0 + kStageW + i * kStageX);
        }
    };
    if (g0 < g1) issue(g0, stage);
    for (int kk = g0; kk < g1; ++kk) {
        uint8_t *cur = stage + ((kk - g0) & 1) * SB;
        wait_vm_asm<0>();   // this wave's loads of the group have landed
        if constexpr (NW > 1) __syncthreads();   // and every other wave's
        // the other stage was last read by the previous group, whose reads
        // have all returned (their values are used) in every wave
        if (kk + 1 < g1) issue(kk + 1, stage + ((kk + 1 - g0) & 1) * SB);
        const int slot = kk & (kSlots - 1);
        // One block of the pair at a time: its x values for all M rows (8
        // float4 per row) serve the wave's local rows; W is read from this
        // stage one block (9 dwords) at a time while the next group streams
        // into the other stage.
        float sub[HW][M];
        auto half = [&](auto pc) {
            constexpr int PAR = decltype(pc)::value;
            float4 xv[M][8];
#pragma unroll
            for (int i = 0; i < M; ++i) {
                const float4 *xs = reinterpret_cast<const float4 *>(cur + kStageW + i * kStageX);
#pragma unroll
                for (int u = 0; u < 8; ++u) xv[i][u] = xs[4 * (8 * PAR + u) + c];
            }
#pragma unroll
            for (int hh = 0; hh < HW; ++hh) {
                // the block's 34 bytes start 2 * PAR bytes into these 9 dwords
                uint32_t D[68];
                const uint32_t *src = reinterpret_cast<const uint32_t *>(
                    cur + kGroupBytes * (16 * (HW * wave + hh) + r) + 2 * kBlockBytes * c + 32 * PAR);
#pragma unroll
                for (int w = 0; w < 9; ++w) D[w] = src[w];
                float dd, sv[M];
                vrow_block<PAR, M>(D, xv, dd, sv);
#pragma unroll
                for (int i = 0; i < M; ++i)
                    sub[hh][i] = PAR == 0 ? dd * sv[i] : fmaf(dd, sv[i], sub[hh][i]);
            }
        };
        half(std::integral_constant<int, 0>{});
        half(std::integral_constant<int, 1>{});
#pragma unroll
        for (int h = 0; h < HW; ++h)
#pragma unroll
            for (int i = 0; i < M; ++i)
#pragma unroll
                for (int q = 0; q < kSlots; ++q)
                    if (q == slot) acc[h][i][q] += sub[h][i];
    }
}

template <int M, int NW>
__device__ void vrow_streamk(const GemmDesc &d, int64_t b, uint8_t *stage) {
    constexpr int HW = 4 / NW;
    const int lane = lane_id();
    const int wave = NW > 1 ? wave_id() : 0;
    const int r = lane >> 2, c = lane & 3;
    const int64_t G = d.gsr, N = (int64_t)d.row_tiles * G, W = d.fast_wgs;
    const int64_t it0 = sk_first_item(b, N, W);
    int64_t it = it0;
    const int64_t end = sk_first_item(b + 1, N, W);
    while (it < end) {
        const int rt = (int)(it / G);
        const int g0 = (int)(it - (int64_t)rt * G);
        const int g1 = (int)min(G, (int64_t)g0 + (end - it));
        float acc[HW][M][kSlots];
#pragma unroll
        for (int h = 0; h < HW; ++h)
#pragma unroll
            for (int i = 0; i < M; ++i)
#pragma unroll
                for (int q = 0; q < kSlots; ++q) acc[h][i][q] = 0.f;
        vrow_run<M, NW>(d, rt, g0, g1, stage, acc);
        // the four lanes of a row meet; lane (r, c) then holds local row
        // 16 (HW wave + c) + r, for c < HW
        float out[M];
#pragma unroll
        for (int h = 0; h < HW; ++h)
#pragma unroll
            for (int i = 0; i < M; ++i) {
                float v = combine_slots(acc[h][i][0], acc[h][i][1], acc[h][i][2], acc[h][i][3]);
                v += __shfl_xor(v, 1, kWave);
                v += __shfl_xor(v, 2, kWave);
                if (h == 0 || c == h) out[i] = v;
            }
        const bool holder = c < HW;
        const int row = 16 * (HW * wave + c) + r;
        const int64_t sr = (int64_t)rt * kWave + row;
        if (g0 == 0 && g1 == G) {
            if (holder && sr < d.nsr)
#pragma unroll
                for (int i = 0; i < M; ++i) d.Y[(int64_t)i * d.p + sr] = out[i];
            // with NW > 1 no wave refills a stage of the next item before
            // every wave has finished reading this one's
            if constexpr (NW > 1) __syncthreads();
        } else {
            const int64_t first = sk_owner((int64_t)rt * G, N, W);
            const int64_t contributors = sk_owner((int64_t)rt * G + G - 1, N, W) - first + 1;
            float *mine = partial_slot<1>(d, b, it != it0);
            if (holder)
#pragma unroll
                for (int i = 0; i < M; ++i) store_partial(mine + i * kWave + row, out[i]);
            if constexpr (NW > 1) {
                // every wave's share is stored before wave 0 counts the arrival
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (wave == 0) arrive_reduce<1>(d, rt, first, (int)contributors, lane);
            } else {
                arrive_reduce<1>(d, rt, first, (int)contributors, lane);
            }
        }
        it += g1 - g0;
    }
}

// ---------------------------------------------------------------- m > 1, matrix cores, X held in LDS
// Y = X W^T for 2 <= m <= 16 where every row is one super-row (n a multiple
// of 256), on v_mfma_f32_16x16x32_bf16 with X split exactly into bf16 parts
// as in k_q8_gemm_mfma.  The columns are cut into d.ks_ranges ranges of
// d.ks_groups groups, and a workgroup owns one range and a block of
// d.ks_rows rows:
//  * at its start it reads the range's x values (m rows) and splits them
//    into their parts in LDS (1.5 KiB per row of X and group), and keeps them
//    there: every wave reads its A operands from them, so X crosses from L2
//    once per workgroup and needs no launch of its own;
//  * its NW waves take the block's 32-row sub-tiles in turn (wave w:
//    sub-tiles w, w + NW, ...), each walking the range's groups.  A step
//    (sub-tile, group) moves 32 rows of W HBM -> LDS by the matvec tile's
//    direct loads into the wave's one stage (row r at LDS offset 272 r); once
//    landed, each lane copies the words it feeds the matrix cores -- for
//    MFMA tile t and block K the quants 8g .. 8g+7 of row 16t + j and the
//    block's scale -- into registers, the next step's loads go into the
//    stage at once, and the step is computed from registers.
// A sub-tile's sums over the range go to Y (one range) or to the range's
// slice of d.yp; the ranges' slices are then added in range order, by the
// last of a row block's workgroups to arrive on its counter (d.ks_sum_here)
// or by a second launch, k_ks_reduce.
template <int NW>
struct Ks {
    static constexpr int kWaveRows = 32;
    static constexpr int kChunks = kWaveRows * kGroupChunks;      // 16-byte chunks of a step's W
    static constexpr int kLoads = (kChunks + kWave - 1) / kWave;   // direct loads per lane (the last one half)
    static constexpr int kStage = kWaveRows * kGroupBytes;          // 8704
    // the parts of X: whatever LDS the stages leave for this many
    // workgroups per CU (1 with eight waves, 2 with four)
    static constexpr int kWgsPerCu = NW >= 8 ? 1 : 2;
    static constexpr int kA = ((160 * 1024 / kWgsPerCu - NW * kStage - 64) / 1536) * 1536;
};

// One lane's words of a step: quants of tile t, block K, and the scales
// (binary16 bits) of blocks 2h and 2h + 1 in the low and high halves of
// s[t][h].
struct McHeld {
    uint32_t q[2][kGroupBlocks][2];
    uint32_t s[2][kGroupBlocks / 2];
};

// Block K of tile t (rows 16t .. 16t + 15 of the stage) for lane (j, g):
// the eight quants 8g .. 8g+7 of row 16t + j.
template <int K>
__device__ __forceinline__ void mc_hold_quants(const uint8_t *grp, int g, uint32_t (&q)[2]) {
    constexpr int q0 = K * kBlockBytes + 2;   // the block's first quant byte
    if constexpr ((q0 & 3) == 0) {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(grp + q0 + 8 * g);
        q[0] = p[0];
        q[1] = p[1];
    } else {   // the quants start two bytes into a dword
        const uint32_t *p = reinterpret_cast<const uint32_t *>(grp + q0 - 2 + 8 * g);
        const uint32_t a0 = p[0], a1 = p[1], a2 = p[2];
        q[0] = __builtin_amdgcn_alignbyte(a1, a0, 2);
        q[1] = __builtin_amdgcn_alignbyte(a2, a1, 2);
    }
}

__device__ __forceinline__ void mc_hold(const uint8_t *stage, int j, int g, McHeld &H) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const uint8_t *grp = stage + kGroupBytes * (16 * t + j);
        mc_hold_quants<0>(grp, g, H.q[t][0]);
        mc_hold_quants<1>(grp, g, H.q[t][1]);
        mc_hold_quants<2>(grp, g, H.q[t][2]);
        mc_hold_quants<3>(grp, g, H.q[t][3]);
        mc_hold_quants<4>(grp, g, H.q[t][4]);
        mc_hold_quants<5>(grp, g, H.q[t][5]);
        mc_hold_quants<6>(grp, g, H.q[t][6]);
        mc_hold_quants<7>(grp, g, H.q[t][7]);
#pragma unroll
        for (int h = 0; h < kGroupBlocks / 2; ++h) {
            const uint32_t lo = *reinterpret_cast<const uint16_t *>(grp + 2 * h * kBlockBytes);
            const uint32_t hi = *reinterpret_cast<const uint16_t *>(grp + (2 * h + 1) * kBlockBytes);
            H.s[t][h] = lo | (hi << 16);
        }
    }
}

// Eight int8 quants -> the B operand (bfloat16 holds every int8 exactly).
__device__ __forceinline__ bf16x8 mc_bq(const uint32_t (&q)[2]) {
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        b[e] = (__bf16)(float)(int8_t)(q[0] >> (8 * e));
        b[4 + e] = (__bf16)(float)(int8_t)(q[1] >> (8 * e));
    }
    return b;
}

// Block K of the held step; `ab` points at its first block's parts in LDS
// (layout of k_split_x with rows = m): for each tile t, C_t = sum over the
// parts (h, then m, then l) of A_part B_t, then acc_t += d_t C_t.
template <int K>
__device__ __forceinline__ void mc_block(const McHeld &H, const bf16x8 *ab, int ii, int g, int m, f32x4 (&acc)[2]) {
    const bf16x8 ah = ab[((K * 3 + 0) * m + ii) * 4 + g];
    const bf16x8 am = ab[((K * 3 + 1) * m + ii) * 4 + g];
    const bf16x8 al = ab[((K * 3 + 2) * m + ii) * 4 + g];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const bf16x8 b = mc_bq(H.q[t][K]);
        f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, b, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b, c, 0, 0, 0);
        acc[t] += half_to_float(H.s[t][K / 2] >> (16 * (K & 1))) * c;
    }
}

template <int NW>
__global__ __launch_bounds__(NW * kWave, 1) void k_q8_gemm_ks(GemmDesc d) {
    using P = Ks<NW>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[P::kA + NW * P::kStage];
    const int lane = lane_id();
    const int wk = NW > 1 ? wave_id() : 0;
    const int j = lane & 15, g = lane >> 4;
    const int m = d.m;
    const int ii = min(j, m - 1);   // A: lane (i, g) with i = lane & 15; rows i >= m read row m - 1
    const int nkr = d.ks_ranges;
    const int kr = (int)(blockIdx.x % (uint32_t)nkr);
    const int64_t row_lo = (int64_t)(blockIdx.x / (uint32_t)nkr) * d.ks_rows;
    const int G = d.gsr;
    const int k0 = kr * d.ks_groups, k1 = min(G, k0 + d.ks_groups);
    const int64_t rows = min((int64_t)d.ks_rows, (int64_t)d.p - row_lo);
    const int nst = (int)((rows + P::kWaveRows - 1) / P::kWaveRows);
    uint8_t *wst = lds + P::kA + wk * P::kStage;
    const bf16x8 *abase = reinterpret_cast<const bf16x8 *>(lds);
    const uint8_t *wt = uniform_ptr(d.w + row_lo * d.sr_bytes);
    const uint32_t lw = __builtin_amdgcn_readfirstlane(lds_addr(wst));
    const int last = (int)(rows - 1);   // the block's last row
    // load c of lane l carries chunk q = 64c + l of a step: row q / 17 of
    // the sub-tile (clamped to the block's last row), chunk q % 17
    uint32_t off[P::kLoads];
    auto offsets = [&](int st) {
#pragma unroll
        for (int c = 0; c < P::kLoads; ++c) {
            const int q = kWave * c + lane;
            const int r = q / kGroupChunks;
            off[c] = (uint32_t)((int64_t)min(P::kWaveRows * st + r, last) * d.sr_bytes + 16 * (q - kGroupChunks * r));
        }
    };
    auto issue = [&](int kk) {
#pragma unroll
        for (int c = 0; c < P::kLoads; ++c) {
            if (c + 1 < P::kLoads || P::kChunks % kWave == 0 || lane < P::kChunks % kWave)
                dma16_s(wt, off[c] + (uint32_t)kk * kGroupBytes, lw + kWave * 16 * c);
        }
    };
    int st = wk, kk = k0;
    if (st < nst && k0 < k1) {
        offsets(st);
        issue(kk);
    }
    // The range's x values, split into their parts in LDS (layout of
    // k_split_x with rows = m, blocks counted from the range's first): thread
    // q takes pieces q, q + 64 NW, ... of (row i, block b, column group g),
    // eight floats each.  (Their loads are waited for together with the
    // first step's, which the step needs anyway.)
    {
        bf16x8 *ab = reinterpret_cast<bf16x8 *>(lds);
        const int nbk = (k1 - k0) * kGroupBlocks;
        for (int c = threadIdx.x; c < m * nbk * 4; c += NW * kWave) {
            const int i = c / (nbk * 4), b = (c >> 2) % nbk, gg = c & 3;
            const float4 *src = reinterpret_cast<const float4 *>(d.X + (int64_t)i * d.n +
                                                                 (int64_t)(k0 * kGroupBlocks + b) * kQuants + 8 * gg);
            const float4 v0 = src[0], v1 = src[1];
            const float x[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            XParts o;
            split3(x, o.h, o.m, o.l);
            ab[((b * 3 + 0) * m + i) * 4 + gg] = o.h;
            ab[((b * 3 + 1) * m + i) * 4 + gg] = o.m;
            ab[((b * 3 + 2) * m + i) * 4 + gg] = o.l;
        }
    }
    __syncthreads();
    f32x4 acc[2];
    acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[1] = acc[0];
    while (st < nst) {   // (the launcher refuses empty ranges)
        __builtin_amdgcn_s_waitcnt(0x0F70);   // this step's W has landed
        asm volatile("" ::: "memory");
        McHeld H;
        mc_hold(wst, j, g, H);
        // the stage is refilled only after every read of it has returned
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        int nst_next = st, nkk = kk + 1;
        if (nkk == k1) {
            nkk = k0;
            nst_next = st + NW;
        }
        if (nst_next < nst) {
            if (nst_next != st) offsets(nst_next);
            issue(nkk);
        }
        const bf16x8 *ab = abase + (kk - k0) * kGroupBlocks * 3 * m * 4;
        mc_block<0>(H, ab, ii, g, m, acc);
        mc_block<1>(H, ab, ii, g, m, acc);
        mc_block<2>(H, ab, ii, g, m, acc);
        mc_block<3>(H, ab, ii, g, m, acc);
        mc_block<4>(H, ab, ii, g, m, acc);
        mc_block<5>(H, ab, ii, g, m, acc);
        mc_block<6>(H, ab, ii, g, m, acc);
        mc_block<7>(H, ab, ii, g, m, acc);
        if (kk + 1 == k1) {
            // lane (j, g) holds Y[4g + e][row_lo + 32 st + 16t + j] in acc[t][e]
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * g + e, r = P::kWaveRows * st + 16 * t + j;
                    if (i < m && r <= last) {
                        float *o = nkr == 1 ? d.Y + (int64_t)i * d.p + row_lo + r
                                            : d.yp + ((int64_t)kr * m + i) * d.p + row_lo + r;
                        if (d.ks_sum_here) store_partial(o, acc[t][e]);   // read by another workgroup
                        else *o = acc[t][e];
                    }
                }
            acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc[1] = acc[0];
        }
        st = nst_next;
        kk = nkk;
    }
    if (nkr == 1 || !d.ks_sum_here) return;
    // The ranges' sums meet here: every wave's share is stored before wave 0
    // counts the workgroup's arrival on the row block's counter, and the last
    // of the block's ranges to arrive adds them, in range order, with all its
    // threads.
    __shared__ uint32_t last_flag;
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
    __syncthreads();
    const int rb = (int)(blockIdx.x / (uint32_t)nkr);
    if (wk == 0) {
        uint32_t prev = 0;
        if (lane == 0) prev = arrive(d, rb);
        prev = __shfl(prev, 0, kWave);
        if (lane == 0) last_flag = prev == (uint32_t)nkr - 1 ? 1u : 0u;
    }
    __syncthreads();
    if (!last_flag) return;
    asm volatile("" ::: "memory");
    const int64_t slice = (int64_t)m * d.p;
    for (int o = threadIdx.x; o < m * (int)rows; o += NW * kWave) {
        const int i = o / (int)rows, r = o - i * (int)rows;
        const float *src = d.yp + (int64_t)i * d.p + row_lo + r;
        float v = 0.f;
        for (int q0 = 0; q0 < nkr; q0 += 8) {
            float t8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                t8[u] = q0 + u < nkr ? __hip_atomic_load(src + (int64_t)(q0 + u) * slice, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT)
                                     : 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (q0 + u < nkr) v = (q0 + u == 0) ? t8[u] : v + t8[u];
        }
        d.Y[(int64_t)i * d.p + row_lo + r] = v;
    }
}

// Y = the sum over the ranges of d.yp, in range order.  Where p is a
// multiple of 4 a thread takes four consecutive outputs (16-byte loads of
// the slices, up to 16 ranges' loads in flight before they are added),
// else one output; either way every output is v_0 + v_1 + ... in range
// order, the same bits as the last-arriver sum in k_q8_gemm_ks.  Y is
// stored a float at a time (it need only be 4-byte aligned).
constexpr int kReduceBatch = 16;
__global__ __launch_bounds__(256) void k_ks_reduce(GemmDesc d) {
    const int64_t total = (int64_t)d.m * d.p;
    const int nkr = d.ks_ranges;
    if (d.p % 4 == 0) {
        const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
        if (i4 >= total) return;
        const float4 *src = reinterpret_cast<const float4 *>(d.yp + i4);
        const int64_t slice4 = total / 4;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int q0 = 0; q0 < nkr; q0 += kReduceBatch) {
            float4 t[kReduceBatch];
#pragma unroll
            for (int u = 0; u < kReduceBatch; ++u)
                t[u] = q0 + u < nkr ? src[(int64_t)(q0 + u) * slice4] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int u = 0; u < kReduceBatch; ++u)
                if (q0 + u < nkr) {
                    if (q0 + u == 0) v = t[u];
                    else v = make_float4(v.x + t[u].x, v.y + t[u].y, v.z + t[u].z, v.w + t[u].w);
                }
        }
        d.Y[i4] = v.x;
        d.Y[i4 + 1] = v.y;
        d.Y[i4 + 2] = v.z;
        d.Y[i4 + 3] = v.w;
        return;
    }
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const float *src = d.yp + i;
    float v = 0.f;
    for (int q0 = 0; q0 < nkr; q0 += kReduceBatch) {
        float t[kReduceBatch];
#pragma unroll
        for (int u = 0; u < kReduceBatch; ++u) t[u] = q0 + u < nkr ? src[(int64_t)(q0 + u) * total] : 0.f;
#pragma unroll
        for (int u = 0; u < kReduceBatch; ++u)
            if (q0 + u < nkr) v = (q0 + u == 0) ? t[u] : v + t[u];
    }
    d.Y[i] = v;
}

template <int RS>
__global__ __launch_bounds__(kWave, 1) void k_q8_gemm_mfma(GemmDesc d) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[2 * kStageBytesM];
    const uint32_t bid = blockIdx.x;
    if (bid < (uint32_t)d.fast_wgs) {
        gemm_streamk<RS>(d, bid, stage);
    } else {
        OpDesc t;
        t.x = d.X; t.w = d.w; t.y = d.Y; t.nb = d.nb; t.p = d.p; t.m = d.m;
        t.x_stride = d.n; t.y_stride = d.p; t.tail_row0 = d.tail_row0;
        tail_tile<kXFloat>(t, bid - d.fast_wgs, 1);
    }
}

template <int RS, int M>
__global__ __launch_bounds__(kWave) void k_q8_gemm_valu(GemmDesc d) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[2 * VStage<M>::kBytes];
    const uint32_t bid = blockIdx.x;
    if (bid < (uint32_t)d.fast_wgs) {
        vsmall_streamk<RS, M>(d, bid, stage);
    } else {
        OpDesc t;
        t.x = d.X; t.w = d.w; t.y = d.Y; t.nb = d.nb; t.p = d.p; t.m = d.m;
        t.x_stride = d.n; t.y_stride = d.p; t.tail_row0 = d.tail_row0;
        tail_tile<kXFloat>(t, bid - d.fast_wgs, 1);
    }
}


template <int M, int NW>
__global__ __launch_bounds__(NW * kWave) void k_q8_gemm_vrow(GemmDesc d) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[2 * VStage<M>::kBytes];
    vrow_streamk<M, NW>(d, blockIdx.x, stage);
}

}  // namespace

hipError_t launch_split_x(const float *X, void *xs, int m, int n, hipStream_t s) {
    const int64_t items = (int64_t)m * (n / kQuants) * 4;
    hipLaunchKernelGGL(k_split_x, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, X,
                       (bf16x8 *)xs, m, n);
    return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t *p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_gemm_mfma(const GemmDesc &d, int64_t grid, hipStream_t s) {
    const dim3 gr((unsigned)grid), bl(kWave);
    switch (d.rs) {
        case 1: hipLaunchKernelGGL((k_q8_gemm_mfma<1>), gr, bl, 0, s, d); break;
        case 2: hipLaunchKernelGGL((k_q8_gemm_mfma<2>), gr, bl, 0, s, d); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int ks_a_bytes(int nw) { return nw == 8 ? Ks<8>::kA : nw == 4 ? Ks<4>::kA : 0; }

hipError_t launch_gemm_ks(const GemmDesc &d, int nw, hipStream_t s) {
    if (d.rs != 1 || d.m < 2 || d.m > 16 || d.ks_ranges < 1 || d.ks_groups < 1 || d.ks_rows < 32 ||
        d.ks_rows % 32 || (int64_t)d.ks_ranges * d.ks_groups < d.gsr ||
        (int64_t)(d.ks_ranges - 1) * d.ks_groups >= d.gsr ||   // no empty range
        (int64_t)d.ks_groups * kGroupBlocks * d.m * 192 > ks_a_bytes(nw))
        return hipErrorInvalidValue;
    const int64_t blocks = (int64_t)d.ks_ranges * ((d.p + d.ks_rows - 1) / d.ks_rows);
    const dim3 gr((unsigned)blocks), bl((unsigned)(nw * kWave));
    switch (nw) {
        case 4: hipLaunchKernelGGL((k_q8_gemm_ks<4>), gr, bl, 0, s, d); break;
        case 8: hipLaunchKernelGGL((k_q8_gemm_ks<8>), gr, bl, 0, s, d); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || d.ks_ranges == 1 || d.ks_sum_here) return e;
    const int64_t total = (int64_t)d.m * d.p;
    const int64_t threads = d.p % 4 == 0 ? total / 4 : total;   // four outputs a thread where p allows
    hipLaunchKernelGGL(k_ks_reduce, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, d);
    return hipGetLastError();
}

int gemm_valu_stage_bytes(int m) {
    switch (m) {
        case 2: return 2 * VStage<2>::kBytes;
        case 3: return 2 * VStage<3>::kBytes;
        case 4: return 2 * VStage<4>::kBytes;
        default: return 0;
    }
}

namespace {
template <int RS>
hipError_t launch_valu_rs(const GemmDesc &d, const dim3 &gr, hipStream_t s) {
    const dim3 bl(kWave);
    switch (d.m) {
        case 2: hipLaunchKernelGGL((k_q8_gemm_valu<RS, 2>), gr, bl, 0, s, d); break;
        case 3: hipLaunchKernelGGL((k_q8_gemm_valu<RS, 3>), gr, bl, 0, s, d); break;
        case 4: hipLaunchKernelGGL((k_q8_gemm_valu<RS, 4>), gr, bl, 0, s, d); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_vrow(const GemmDesc &d, int nw, hipStream_t s) {
    if (d.rs != 1 || d.tail_row0 != d.p) return hipErrorInvalidValue;
    const dim3 gr((unsigned)d.fast_wgs), bl(nw * kWave);
    if (nw == 1 && d.m == 2) hipLaunchKernelGGL((k_q8_gemm_vrow<2, 1>), gr, bl, 0, s, d);
    else if (nw == 1 && d.m == 3) hipLaunchKernelGGL((k_q8_gemm_vrow<3, 1>), gr, bl, 0, s, d);
    else if (nw == 2 && d.m == 2) hipLaunchKernelGGL((k_q8_gemm_vrow<2, 2>), gr, bl, 0, s, d);
    else if (nw == 2 && d.m == 3) hipLaunchKernelGGL((k_q8_gemm_vrow<3, 2>), gr, bl, 0, s, d);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_gemm_valu(const GemmDesc &d, int64_t grid, hipStream_t s) {
    const dim3 gr((unsigned)grid);
    switch (d.rs) {
        case 1: return launch_valu_rs<1>(d, gr, s);
        case 2: return launch_valu_rs<2>(d, gr, s);
        case 4: return launch_valu_rs<4>(d, gr, s);
        case 8: return launch_valu_rs<8>(d, gr, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace q8
