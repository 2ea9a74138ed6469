// q8_internal.h -- shared between the HIP kernels and the host side of the
// library: the Q8_0 geometry, the matvec's op and tile descriptors and its
// launchers (the small batch's are in q8_gemm.h).  Not installed; the public
// interface is include/q8gemv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

// Q8_0 geometry (page "IV.4: One command buffer per token", section "Eight
// kernels": 32 quants and a 2-byte binary16 scale per block).
constexpr int kQuants = 32;
constexpr int kBlockBytes = 34;
// Eight consecutive blocks are 272 bytes = 17 aligned 16-byte chunks: the
// unit the fast path moves from HBM to LDS.
constexpr int kGroupBlocks = 8;
constexpr int kGroupBytes = kGroupBlocks * kBlockBytes;  // 272
constexpr int kGroupChunks = kGroupBytes / 16;           // 17

constexpr int kWave = 64;
constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = kWave * kWaves;  // 256
constexpr int kBufs = 2;                  // LDS stages per wave
// One stage holds a group of 64 lanes (17408 B of W) and, for the matvec,
// the group's 256 x values (1 KB), which arrive by the same direct loads.
constexpr int kStageW = kWave * kGroupBytes;       // 17408
constexpr int kStageX = kGroupBlocks * kQuants * 4;  // 1024
constexpr int kStageBytes = kStageW + kStageX;     // 18432
constexpr int kStageBytesM = kStageW;              // small batch: W only

// One matvec (or small-batch product) as the kernels see it.  A "super-row"
// is `rs` consecutive rows whose bytes, taken together, are a whole number of
// 272-byte groups: rs = 8 / gcd(n/32, 8).  rs == 1 (n a multiple of 256):
// every row is whole groups and the rows-and-group-slots kernel takes the op
// (q8_gemv_rc.hip).  rs > 1: lane l of a wave owns one super-row
// (q8_gemv.hip); rows that do not fill a last super-row are "tail" rows and
// take the generic path.
struct OpDesc {
    const float *x;      // x, or X row 0 for small batches
    const uint8_t *w;
    float *y;            // y, or Y row 0
    int64_t sr_bytes;    // bytes of one super-row = rs * nb * 34
    int64_t x_stride;    // floats between rows of X (= n)
    int64_t y_stride;    // floats between rows of Y (= p)
    int32_t nb;          // blocks per row = n / 32
    int32_t p;           // rows
    int32_t rs;          // rows per super-row: 1, 2, 4 or 8
    int32_t nsr;         // super-rows handled by the fast path = p / rs
    int32_t gsr;         // groups per super-row = rs * nb / 8
    int32_t ks;          // rs > 1: waves that split one super-row's groups (1, 2 or 4)
    int32_t fast_tiles;  // workgroup tiles of the fast path
    int32_t tail_row0;   // first tail row = nsr * rs
    int32_t m;           // activation rows (1 for a matvec)
    int32_t tile_rows;   // rows-and-group-slots tiles: rows per tile, 1 .. 64 / C (0: 64 / C)
    const float *x_up;   // kXSiluUp: the input is silu(x) * x_up, elementwise
    // kXNormAdd: the input is rms_norm(x + x_res) * norm_w over the op's n
    // columns; the op-local tile 0's workgroup also writes x + x_res to x_out
    const float *x_res;
    const float *norm_w;
    float *x_out;        // may be null
    float norm_eps;
    // kXNormScale: x holds v * g (a gain applied by the producer) and the
    // input is x * inv, inv = 1 / sqrt(ss / n + norm_eps), ss the sum of the
    // psum_n floats at psum (the block sums of v^2, as kYResAdd writes them);
    // inv scales each row result.
    // kYResAdd: y = x_res + W x, psum[row / 16] = sum of y^2 over each
    // 16-row block, and (x_out not null) x_out = y * norm_w, p floats.
    // kYSwiGLU: rows of w2 too; y = silu(W x) * (W2 x).
    int32_t psum_n;
    // rows-and-group-slots tiles: W's lines are loaded with the non-temporal
    // hint (a launch that waits on the one before and is waited on by the
    // next: its weights, read once, then do not push out of L2 the
    // activations, norm sums and KV cache the next launches read)
    int32_t w_once;
    float *psum;
    const uint8_t *w2;
};

// How a matvec reads its activations (a compile-time mode of the kernels).
enum XMode : int {
    kXFloat = 0,    // x as float32
    kXQuant = 1,    // x quantized to Q8_0 per group, integer dots
    kXSiluUp = 2,   // silu(x) * x_up formed per group (the SwiGLU product feeding a down projection)
    kXNormAdd = 3,  // rms_norm(x + x_res) * norm_w formed per group (a residual add and the norm after it)
    kXNormScale = 4,  // x * inv, x gain-scaled by the producer, inv from the block sums it left in psum
};
// What a matvec writes (a compile-time mode of the rows-and-group-slots kernel).
enum YMode : int {
    kYPlain = 0,    // y = W x
    kYResAdd = 1,   // y = x_res + W x, 16-row block sums of y^2 in psum, y * norm_w in x_out (a residual add)
    kYSwiGLU = 2,   // y = silu(W x) * (W2 x): gate and up rows computed together
};
// Rows per block of the squared-norm partial sums (kYResAdd / kXNormScale).
constexpr int kPsumRows = 16;
// rs > 1: every row sums its groups into kSlots partial sums (group kk into
// slot kk % kSlots, in increasing kk) and combines them as
// (s0 + s1) + (s2 + s3).
constexpr int kSlots = 4;
// rs == 1: kRowSlots partial sums per row (group kk into slot kk % 16, in
// increasing kk), combined as (L0 + L1) + (L2 + L3) with
// L_a = (s_a + s_{a+4}) + (s_{a+8} + s_{a+12}).  Every launch shape of the
// rs == 1 kernel computes exactly this tree.
constexpr int kRowSlots = 16;

// One workgroup's work in a fused launch.
struct Tile {
    uint32_t op;    // index into the op table
    uint32_t tile;  // tile within the op; kTailBit set: tail tile
};
constexpr uint32_t kTailBit = 0x80000000u;

// rs > 1 kernel shape: waves per workgroup (1 or 4); each wave keeps one
// group in flight ahead of the one it computes.
struct Variant {
    int nw;
    int pf;
};

// Shape of a launch of the rs == 1 kernel: C lanes per row (1, 2 or 4) so a
// wave covers 64 / C rows, NWK waves per workgroup (1, 2 or 4) that share a
// tile's rows and split its groups by slot (wave w takes the group columns
// j = w, w + NWK, ...), and NST W stages per wave (1 or 2).
struct RcShape {
    int c;
    int nwk;
    int nst;
    int tr = 0;   // rows per tile, 1 .. 64 / c (0: 64 / c); one-op launches only
};
// rows of a tile of shape sh
inline int rc_rows(RcShape sh) { return sh.tr > 0 ? sh.tr : kWave / sh.c; }

// rs > 1: fast tiles cover (nw / ks) * 64 super-rows each.
inline int64_t fast_tiles_for(int64_t nsr, int ks, int nw = kWaves) {
    const int64_t per = (int64_t)(nw / ks) * kWave;
    return (nsr + per - 1) / per;
}
// Tail tiles take one row per wave.
inline int64_t tail_tiles_for(int64_t tail_rows, int nw = kWaves) {
    return (tail_rows + nw - 1) / nw;
}
// rs == 1: tiles of 64 / C rows, or of the shape's rc_rows.
// The mixed-width fused launch (k_q8_gemv_mixed): rows of whole groups take
// the rows-and-group-slots tile with kMixC lanes per row and kMixNst W
// stages, W loaded non-temporal (measured on the Qwen2.5-0.5B chain, whose
// whole-group rows are its 24 down projections: 97.4-97.6 us per token
// against 98.6-98.7 with plain loads, 97.9-98.1 with four lanes and the
// hint, 101.2-101.5 with four lanes and plain loads, 99.5 with {1 lane,
// 2 stages}), the other widths the super-row tile.  (The super-row tile
// with one W stage and two x stages measured no faster there: 99.7-107.6
// us.)
constexpr int kMixC = 2, kMixNst = 1;

inline int64_t rc_tiles_for(int64_t p, int c) {
    const int64_t rows = kWave / c;
    return (p + rows - 1) / rows;
}
inline int64_t rc_tiles_for(int64_t p, RcShape sh) {
    const int64_t rows = rc_rows(sh);
    return (p + rows - 1) / rows;
}

// Matvec launchers.  All return the hipError_t of the launch.  xmode: how
// the activations are read (XMode).
// rs > 1 ops (q8_gemv.hip): one op on workgroups of v.nw waves (1 or 4).
hipError_t launch_gemv_single(const OpDesc &op, const Variant &v, int64_t grid, hipStream_t s,
                              int xmode = kXFloat);
// A table of tiles of independent ops of any width, on one-wave workgroups
// (v = {1, 1}): rs == 1 tiles in RcShape {1, 1, 2}, the others as super-rows.
hipError_t launch_gemv_fused(const OpDesc *d_ops, const Tile *d_tiles, const Variant &v,
                             int64_t grid, hipStream_t s, int xmode = kXFloat);
// rs == 1 ops (q8_gemv_rc.hip, built once per build mode M -- a pair of
// input and output modes, kBuildModes -- with the entry points below with
// the mode's number appended).  One op: grid =
// rc_tiles_for(p, sh) workgroups, tiles of sh.tr rows when it is set (a
// multiple of 16 for the residual-add output).  A table of tiles of independent rs == 1
// ops read in one mode.  LDS bytes of a workgroup (0: no such shape, or one
// whose LDS does not fit a workgroup).
// build mode -> (XMode, YMode)
constexpr int kBuildModes = 7;
constexpr int kBuildX[kBuildModes] = {kXFloat, kXQuant, kXSiluUp, kXNormAdd, kXNormScale, kXFloat, kXNormScale};
constexpr int kBuildY[kBuildModes] = {kYPlain, kYPlain, kYPlain, kYPlain, kYPlain, kYResAdd, kYSwiGLU};
inline int build_mode(int xmode, int ymode) {
    for (int m = 0; m < kBuildModes; ++m)
        if (kBuildX[m] == xmode && kBuildY[m] == ymode) return m;
    return -1;
}
#define Q8_RC_DECLARE(M)                                                                              \
    hipError_t launch_gemv_rc_##M(const OpDesc &op, RcShape sh, int64_t grid, hipStream_t s);         \
    hipError_t launch_gemv_rc_fused_##M(const OpDesc *d_ops, const Tile *d_tiles, RcShape sh,         \
                                        int64_t grid, hipStream_t s);                                 \
    int gemv_rc_lds_bytes_##M(RcShape sh);
Q8_RC_DECLARE(0)
Q8_RC_DECLARE(1)
Q8_RC_DECLARE(2)
Q8_RC_DECLARE(3)
Q8_RC_DECLARE(4)
Q8_RC_DECLARE(5)
Q8_RC_DECLARE(6)
#undef Q8_RC_DECLARE

#define Q8_RC_SWITCH(F, ...)                            \
    switch (build_mode(xmode, ymode)) {                 \
        case 0: return F##0(__VA_ARGS__);               \
        case 1: return F##1(__VA_ARGS__);               \
        case 2: return F##2(__VA_ARGS__);               \
        case 3: return F##3(__VA_ARGS__);               \
        case 4: return F##4(__VA_ARGS__);               \
        case 5: return F##5(__VA_ARGS__);               \
        case 6: return F##6(__VA_ARGS__);               \
        default: break;                                 \
    }
inline hipError_t launch_gemv_rc(const OpDesc &op, RcShape sh, int64_t grid, hipStream_t s, int xmode,
                                 int ymode = kYPlain) {
    Q8_RC_SWITCH(launch_gemv_rc_, op, sh, grid, s)
    return hipErrorInvalidValue;
}
inline hipError_t launch_gemv_rc_fused(const OpDesc *d_ops, const Tile *d_tiles, RcShape sh, int64_t grid,
                                       hipStream_t s, int xmode, int ymode = kYPlain) {
    Q8_RC_SWITCH(launch_gemv_rc_fused_, d_ops, d_tiles, sh, grid, s)
    return hipErrorInvalidValue;
}
inline int gemv_rc_lds_bytes(RcShape sh, int xmode, int ymode = kYPlain) {
    Q8_RC_SWITCH(gemv_rc_lds_bytes_, sh)
    return 0;
}
#undef Q8_RC_SWITCH
// x (n floats, n % 32 == 0) -> n/32 Q8_0 blocks of 34 bytes at xq.
hipError_t launch_quantize_x(const float *x, void *xq, int64_t n, hipStream_t s);

}  // namespace q8
