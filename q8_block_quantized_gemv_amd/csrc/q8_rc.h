// q8_rc.h -- the m = 1 matvec tile for matrices whose rows are whole
// 272-byte groups (n a multiple of 256): lanes over rows and group slots.
// Included inside an anonymous namespace by q8_gemv_rc.hip (its own
// launches) and q8_gemv.hip (fused launches that mix in other widths).
//
// What is computed (page "IV.4: One command buffer per token", section
// "Eight kernels", q8_matvec) for rows [row0, row0 + 64/C):
//   y[r] = sum_b d(r,b) * sum_j q(r,b,j) x[32b+j].
//
// Layout, for a launch shape (C, NWK):
//  * A wave covers R = 64/C rows; lane (r, c) = (lane / C, lane % C).  The
//    row's groups (8 blocks, 272 bytes) are taken C at a time, in "group
//    columns" j = 0, 1, ...: column j is groups C*j .. C*j + C-1 of each of
//    the R rows, and lane (r, c) computes group C*j + c of row r.
//  * Each column moves HBM -> LDS as 17 direct 16-byte loads per lane
//    (non-temporal where op.w_once: latency and fused launches)
//    (global_load_lds_dwordx4): load i of lane l carries chunk (64i + l) of
//    the column's R runs of C*272 contiguous bytes, so every load
//    instruction reads whole contiguous KiB, and lane l finds its own group
//    at LDS offset 272*l.  The lane copies it into registers and the next
//    column's loads are issued while the current one is computed: with
//    NST = 2 W stages into the other stage at once, with NST = 1 into the
//    same stage once its reads have completed (17 KiB of LDS per wave
//    instead of 34, so twice the waves fit on a CU).
//  * The column's C x slices (1 KiB each) ride along as C more direct loads
//    into a double-buffered x stage; a lane reads its slice with LDS
//    broadcast reads.
//  * The NWK waves of a workgroup share its R rows: wave w takes columns
//    j = w, w + NWK, ...  Group kk = C*j + c lands in row slot kk % 16, which
//    is lane c's local slot j % (16/C) -- so every slot has exactly one
//    owner (a lane of one wave), and slots meet in LDS at the end.
//  * The 16 slots combine in the fixed tree of kRowSlots; with C lanes per
//    row the last steps run across the row's lanes in a fixed butterfly.
// The arithmetic (q8_block.h), the slot of every group and the final tree
// do not depend on (C, NWK): every launch shape gives the same bits.
//
// Input mode kXNormScale: x arrives already multiplied by the norm's gain
// (the producer wrote it so), and the norm's 1 / rms, a scalar, multiplies
// each row result instead of each x element: rms_norm(x) * g . w =
// inv * ((x * g) . w).  Its tiles are the float tiles plus one multiply.
//
// Output modes (YMode): y = W x; a residual add (y = x_res + W x, with the
// sums of y^2 over fixed 16-row blocks for the norm the next matvec applies,
// and, if x_out is set, y * norm_w there: the next matvec's input); and the
// SwiGLU pair, where the workgroup's waves come in two halves that compute
// the same rows of W (gate) and W2 (up) and the first half writes
// silu(gate) * up.
#pragma once

#include "q8_block.h"

namespace q8 {
namespace {

// One x slice (1 KiB) plus 16 bytes, so the C slices of a stage start in
// different LDS banks.
constexpr int kXSlice = kStageX + 16;

template <int C, int XM, int NST>
struct RcLds {
    static constexpr int kX = C * kXSlice;                  // one x stage
    // its up slices (kXSiluUp)
    static constexpr int kUp = XM == kXSiluUp ? kX : 0;
    static constexpr int kWaveBytes = NST * kStageW + 2 * (kX + kUp);
};

// waves of a workgroup: NWK, twice that for the SwiGLU pair
template <int NWK, int YM>
constexpr int rc_waves() { return YM == kYSwiGLU ? 2 * NWK : NWK; }

template <int C, int NWK, int XM, int NST, int YM = kYPlain>
constexpr int rc_lds_bytes() { return rc_waves<NWK, YM>() * RcLds<C, XM, NST>::kWaveBytes; }
// LDS a workgroup may have on gfx950
constexpr int kMaxLds = 160 * 1024;

// kXNormAdd with NWK waves: wave w sums the squares of parts w, w + NWK, ...
// of x + x_res (and, in the writer workgroup, stores those parts to x_out);
// the parts meet in LDS and are added in part order by every wave.  One
// wave computes all parts in one pass.  Either way each part's sum runs in
// the same fixed order (norm_add_part), so inv is the same bits for every
// launch shape.  Every wave of the workgroup must call this.
template <int NWK>
__device__ __forceinline__ float rc_norm_inv(const OpDesc &op, int lane, int wave, bool write) {
    float part[kNormParts];
    if constexpr (NWK == 1) {
        norm_add_parts(op, lane, write, part);
    } else {
        __shared__ float parts[kNormParts];
#pragma unroll
        for (int k = 0; k < kNormParts; ++k)
            if (k % NWK == wave) {
                const float v = norm_add_part(op, lane, k, kNormParts, write);
                if (lane == 0) parts[k] = v;
            }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kNormParts; ++k) part[k] = parts[k];
    }
    return norm_inv_from(part, op);
}

// kXNormScale: 1 / rms of the op's x from the producer's block sums of x^2
// (op.psum_n floats, a multiple of 4, 16-byte aligned), added in a fixed
// order: lane l takes the float4s l, l + 64, ... in turn (each as
// (a + b) + (c + d)), then the lanes meet in the fixed butterfly.
__device__ __forceinline__ float psum_inv(const OpDesc &op, int lane) {
    const float4 *p4 = reinterpret_cast<const float4 *>(op.psum);
    const int n4 = op.psum_n / 4;
    float ss = 0.f;
    for (int i = lane; i < n4; i += kWave) {
        const float4 v = p4[i];
        ss += (v.x + v.y) + (v.z + v.w);
    }
    ss = wave_sum(ss);
    return 1.0f / sqrtf(ss / (float)(op.nb * kQuants) + op.norm_eps);
}

// Tile `tile` (rows tile*R ..) of op, all its groups, on a workgroup of NWK
// waves whose LDS is `lds` (rc_lds_bytes).  writer (kXNormAdd): this
// workgroup also writes x + x_res to op.x_out.
template <int C, int NWK, int XM, int NST, int YM = kYPlain>
__device__ __forceinline__ void rc_tile(const OpDesc &op, int64_t tile, uint8_t *lds, bool writer) {
    using L = RcLds<C, XM, NST>;
    static_assert(NST == 1 || NST == 2, "W stages per wave");
    static_assert(YM != kYSwiGLU || XM != kXNormAdd, "the pair does not take the norm-add input");
    constexpr int R = kWave / C;          // rows of the tile
    constexpr int U = kRowSlots / C;      // slots a lane owns in its row
    static_assert(C == 1 || C == 2 || C == 4, "lanes per row");
    static_assert(U % NWK == 0, "every slot needs exactly one owner wave");
    const int lane = lane_id();
    const int wave = wave_id();
    // kYSwiGLU: waves [0, NWK) take the rows of W (gate), [NWK, 2 NWK) of W2 (up)
    const int half = YM == kYSwiGLU ? wave / NWK : 0;
    const int wk = wave - half * NWK;    // the wave's place among the NWK sharing its rows
    const int r = lane / C, c = lane % C;
    // a tile covers TR <= R rows (lanes past them compute a copy of the
    // last row and store nothing)
    const int TR = op.tile_rows > 0 && op.tile_rows < R ? op.tile_rows : R;
    const int64_t row0 = tile * TR;
    if (row0 >= op.p) return;   // a grid past the op's tiles (every wave of the workgroup leaves)
    const int last = (int)min((int64_t)op.p - 1 - row0, (int64_t)TR - 1);   // rows past p re-read this one
    const int G = op.gsr;                 // groups per row
    const int J = (G + C - 1) / C;        // group columns
    const int64_t RB = op.sr_bytes;       // bytes per row
    uint8_t *wst = lds + wave * L::kWaveBytes;   // NST W stages
    uint8_t *xst = wst + NST * kStageW;          // two x stages, then (kXSiluUp) two up stages
    const uint8_t *wbase = uniform_ptr((half ? op.w2 : op.w) + row0 * RB);

    // Per load i: the owner lane s = (64i + lane) / 17 of the chunk this lane
    // carries, as (row part of the byte offset + chunk offset) and the
    // owner's lane-in-row c_s.
    uint32_t base[kGroupChunks];
    uint32_t cs[kGroupChunks];
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i) {
        const int q = kWave * i + lane;
        const int s = q / kGroupChunks;
        const int rs = s / C;
        base[i] = (uint32_t)((int64_t)min(rs, last) * RB + 16 * (q - kGroupChunks * s));
        cs[i] = (uint32_t)(s % C);
    }
    float acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = 0.f;

    // this wave's group columns j = wk + NWK * t, t < nt
    const int nt = J > wk ? (J - wk + NWK - 1) / NWK : 0;
    float4 na[C], nr[C], nw[C];   // kXNormAdd: x, x_res and gain of the column, prefetched
    const bool w_once = op.w_once != 0;
    auto issue = [&](int t) {
        const int j = wk + NWK * t;
        const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(wst + (t % NST) * kStageW));
        if (w_once) {
#pragma unroll
            for (int i = 0; i < kGroupChunks; ++i) {
                const uint32_t kk = min((uint32_t)(C * j) + cs[i], (uint32_t)(G - 1));
                dma16_s_nt(wbase, base[i] + kk * kGroupBytes, l0 + kWave * 16 * i);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kGroupChunks; ++i) {
                const uint32_t kk = min((uint32_t)(C * j) + cs[i], (uint32_t)(G - 1));
                dma16_s(wbase, base[i] + kk * kGroupBytes, l0 + kWave * 16 * i);
            }
        }
        uint8_t *xs = xst + (t & 1) * L::kX;
#pragma unroll
        for (int cc = 0; cc < C; ++cc) {
            const int kk = min(C * j + cc, G - 1);
            const int64_t xo = (int64_t)kk * (kGroupBlocks * kQuants) + 4 * lane;
            if constexpr (XM == kXNormAdd) {
                na[cc] = *reinterpret_cast<const float4 *>(op.x + xo);
                nr[cc] = *reinterpret_cast<const float4 *>(op.x_res + xo);
                nw[cc] = *reinterpret_cast<const float4 *>(op.norm_w + xo);
            } else {
                const uint32_t x0 = __builtin_amdgcn_readfirstlane(lds_addr(xs)) + cc * kXSlice;
                dma16_v(op.x + xo, x0);
                if constexpr (XM == kXSiluUp) dma16_v(op.x_up + xo, x0 + 2 * L::kX);
            }
        }
    };

    // kXNormAdd, kXNormScale: the norm is computed while the first column
    // streams in (kXNormScale: by the waves that write the rows)
    float ninv = 0.f;
    if (nt > 0) issue(0);
    // kYResAdd: the row's residual and gain, read while the first column
    // streams in (not after the sums, a round trip later)
    float xres = 0.f, ngain = 0.f;
    if constexpr (YM == kYResAdd)
        if (wk == 0 && c == 0 && r <= last) {
            xres = op.x_res[row0 + r];
            if (op.x_out) ngain = op.norm_w[row0 + r];
        }
    if constexpr (XM == kXNormAdd) ninv = rc_norm_inv<NWK>(op, lane, wave, op.x_out && writer);
    if constexpr (XM == kXNormScale)
        if (wk == 0) ninv = psum_inv(op, lane);
    for (int t = 0; t < nt; ++t) {
        const int j = wk + NWK * t;
        uint8_t *xs = xst + (t & 1) * L::kX;
        wait_vm_asm<0>();   // this column's W and x have landed (nothing else is in flight)
        if constexpr (XM == kXNormAdd) {
#pragma unroll
            for (int cc = 0; cc < C; ++cc)
                reinterpret_cast<float4 *>(xs + cc * kXSlice)[lane] = make_float4(
                    norm_add(na[cc].x, nr[cc].x, ninv, nw[cc].x), norm_add(na[cc].y, nr[cc].y, ninv, nw[cc].y),
                    norm_add(na[cc].z, nr[cc].z, ninv, nw[cc].z), norm_add(na[cc].w, nr[cc].w, ninv, nw[cc].w));
        }
        uint32_t D[68];
        read_group(wst + (t % NST) * kStageW, lane, D);
        // the next column: into the other stage at once, or into this one
        // once its reads (and the LDS writes above) have completed
        if constexpr (NST == 1) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (t + 1 < nt) issue(t + 1);
        if constexpr (XM == kXSiluUp) {   // the x slices become silu(gate) * up in place
#pragma unroll
            for (int cc = 0; cc < C; ++cc) {
                float4 *g4 = reinterpret_cast<float4 *>(xs + cc * kXSlice);
                const float4 g = g4[lane];
                const float4 u = reinterpret_cast<const float4 *>(xs + 2 * L::kX + cc * kXSlice)[lane];
                g4[lane] = make_float4(silu_up(g.x, u.x), silu_up(g.y, u.y), silu_up(g.z, u.z), silu_up(g.w, u.w));
            }
        } else if constexpr (XM == kXQuant) {
#pragma unroll
            for (int cc = 0; cc < C; ++cc) quantize_slice(xs + cc * kXSlice, lane);
        }
        const int kk = C * j + c;
        float sub;
        if constexpr (XM == kXQuant) sub = group_sum_xq(D, xs + c * kXSlice);
        else sub = group_sum(D, reinterpret_cast<const float4 *>(xs + c * kXSlice));
        const int u = j % U;
        if (kk < G) {
#pragma unroll
            for (int q = 0; q < U; ++q)
                if (q == u) acc[q] += sub;
        }
    }

    // slots of other waves meet in the half's first wave: slot u of lane l
    // of its owner wave (u % NWK) is parked at float u*64 + l of that wave's
    // first W stage, idle now (its last column was read into registers, and
    // those reads have completed, before it was computed)
    if constexpr (NWK > 1) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        float *mine = reinterpret_cast<float *>(wst);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u % NWK == wk) mine[u * kWave + lane] = acc[u];
        __syncthreads();
        if (wk == 0) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (u % NWK != 0)
                    acc[u] = reinterpret_cast<const float *>(lds + (half * NWK + u % NWK) * L::kWaveBytes)
                        [u * kWave + lane];
        }
    }
    // lane c holds slots C*u + c
    float row = 0.f;
    if (wk == 0) {
        if constexpr (C == 1) {
            float La[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) La[a] = (acc[a] + acc[a + 4]) + (acc[a + 8] + acc[a + 12]);
            row = (La[0] + La[1]) + (La[2] + La[3]);
        } else if constexpr (C == 2) {
            // L_c from u = 0, 2, 4, 6 and L_{c+2} from u = 1, 3, 5, 7
            const float La = (acc[0] + acc[2]) + (acc[4] + acc[6]);
            const float Lb = (acc[1] + acc[3]) + (acc[5] + acc[7]);
            const float La1 = __shfl_xor(La, 1, kWave), Lb1 = __shfl_xor(Lb, 1, kWave);
            row = (La + La1) + (Lb + Lb1);   // used by c == 0: (L0 + L1) + (L2 + L3)
        } else {
            const float La = (acc[0] + acc[1]) + (acc[2] + acc[3]);   // L_c
            const float pair = La + __shfl_xor(La, 1, kWave);           // c = 0: L0 + L1, c = 2: L2 + L3
            row = pair + __shfl_xor(pair, 2, kWave);
        }
        if constexpr (XM == kXNormScale) row *= ninv;
    }
    if constexpr (YM == kYSwiGLU) {
        // the up half's first wave hands its rows to the gate half's
        __shared__ float up_rows[kWave];
        if (half == 1 && wk == 0 && c == 0) up_rows[r] = row;
        __syncthreads();
        if (half == 0 && wk == 0 && c == 0 && r <= last) op.y[row0 + r] = silu_up(row, up_rows[r]);
        return;
    }
    if (wk != 0) return;
    if constexpr (YM == kYResAdd) {
        // y = x_res + W x (and y * norm_w, the next matvec's input); the
        // squares of a 16-row block meet in a fixed butterfly over the row
        // index (lanes C apart), the same tree for every C, and the block's
        // first row stores the sum
        float out = 0.f;
        if (c == 0 && r <= last) {
            out = xres + row;
            op.y[row0 + r] = out;
            if (op.x_out) op.x_out[row0 + r] = out * ngain;
        }
        float sq = out * out;
#pragma unroll
        for (int o = 1; o < kPsumRows; o <<= 1) sq += __shfl_xor(sq, o * C, kWave);
        if (c == 0 && r % kPsumRows == 0 && r <= last) op.psum[(row0 + r) / kPsumRows] = sq;
        return;
    }
    if (c == 0 && r <= last) op.y[row0 + r] = row;
}

}  // namespace
}  // namespace q8
