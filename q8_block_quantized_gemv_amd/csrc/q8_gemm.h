// q8_gemm.h -- the small-batch product's descriptor and launchers, shared
// between q8_gemm.hip and the host side of the library.
#pragma once

#include "q8_internal.h"

namespace q8 {

// Three bf16x8 (48 bytes): one lane's A operand of X for one block, split
// exactly into bfloat16 parts h + m + l (see k_split_x).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
struct XParts {
    bf16x8 h, m, l;
};

// A small-batch product (2 <= m <= 16) as its kernels see it.  Workgroups
// are one wave.  The work is row_tiles (64 super-rows each) x gsr groups of
// items, split stream-K style into fast_wgs equal contiguous ranges; a row
// tile shared by several workgroups goes through partial slots of the
// workspace `ws` (two per workgroup, m * 64 * rs floats each: its first and
// its last tile) and the per-row-tile arrival counters `cnt`, tagged with the
// call's epoch so that they need no clearing.
struct GemmDesc {
    const float *X;
    const bf16x8 *xs;    // X split into exact bf16 parts, 3 KiB per block (k_split_x)
    const uint8_t *w;
    float *Y;
    float *ws;
    unsigned long long *cnt;   // per row tile: the epoch (high 32 bits) and the arrivals
    int64_t sr_bytes;
    int32_t n, nb, p, m;
    int32_t rs, nsr, gsr;
    int32_t row_tiles;   // ceil(nsr / 64)
    int32_t fast_wgs;    // stream-K workgroups; the tail rows follow, one per workgroup
    int32_t tail_row0;
    uint32_t epoch;      // this call's tag on the arrival counters (never 0)
    int32_t ks_groups;   // k_q8_gemm_ks: groups per column range
    int32_t ks_ranges;   // column ranges
    int32_t ks_rows;     // rows per workgroup (a multiple of 32)
    float *yp;           // per-range sums (ks_ranges > 1)
    int32_t ks_sum_here; // the last workgroup of a row block adds the ranges (counters in cnt)
};

hipError_t launch_gemm_mfma(const GemmDesc &d, int64_t grid, hipStream_t s);
// the matrix cores with X held in LDS (k_q8_gemm_ks): rs == 1, 2 <= m <= 16,
// ks_ranges * ceil(p / ks_rows) workgroups of nw (4 or 8) waves (each splits
// its range of X itself; d.xs is not used), d.yp (ks_ranges * m * p floats,
// 16-byte aligned) when ks_ranges > 1 (then the row blocks' last workgroups
// add the ranges, with d.cnt one counter per row block, or a second launch
// does, as d.ks_sum_here says)
hipError_t launch_gemm_ks(const GemmDesc &d, int nw, hipStream_t s);
int ks_a_bytes(int nw);   // LDS a workgroup keeps for the parts of X (0: no such nw)
// the vector-unit small batch for m = 2..4 (any rs); d.xs is not used
hipError_t launch_gemm_valu(const GemmDesc &d, int64_t grid, hipStream_t s);
int gemm_valu_stage_bytes(int m);   // LDS bytes per workgroup (0 if m is not 2..4)
// m = 2..3 on the vector units with lanes over (row, block pair); one row per
// super-row only (rs == 1, so no tail rows); the same LDS bytes as the above
hipError_t launch_gemm_vrow(const GemmDesc &d, int nw, hipStream_t s);   // nw: waves per workgroup, 1 or 2
constexpr int kVrowMaxM = 3;
constexpr int kValuMaxM = 4;
// X (m x n) -> the bf16 parts the matrix-core kernel reads: kXPartsBytesPerBlock
// bytes per block of 32 columns, for up to 16 rows
hipError_t launch_split_x(const float *X, void *xs, int m, int n, hipStream_t s);
// p[0 .. n) = 0 (a fill kernel: no memset node, so it may be captured)
hipError_t launch_zero_u32(uint32_t *p, int64_t n, hipStream_t s);
constexpr int64_t kXPartsBytesPerBlock = 3 * 16 * 4 * 16;   // parts x rows x column groups x bf16x8

}  // namespace q8
