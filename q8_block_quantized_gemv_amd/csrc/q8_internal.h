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
// 272-byte groups: rs = 8 / gcd(n/32, 8).  Lane l of a wave owns one
// super-row; rows that do not fill a last super-row are "tail" rows and take
// the generic path.
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
    int32_t ks;          // waves that split one super-row's groups: 1, 2 or 4
    int32_t fast_tiles;  // workgroup tiles of the fast path
    int32_t tail_row0;   // first tail row = nsr * rs
    int32_t m;           // activation rows (1 for a matvec)
    // K split across workgroups (matvec only): `slices` workgroups share a
    // row tile, slice s taking groups [s * slice_groups, (s+1) * slice_groups).
    // Each parks its per-row partial sums in part[s][row]; the last of them
    // to arrive (counted in cnt[row tile]) adds the slices in order into y
    // and clears the counter.  slices == 1: no split, part and cnt unused.
    int32_t slices;
    int32_t slice_groups;  // a multiple of kSlots
    // Stream-K launches (Piece): the most workgroups sharing one row tile;
    // part then holds sk_slots slots of nsr * rs floats.  0: not stream-K.
    int32_t sk_slots;
    float *part;         // max(slices, sk_slots) * nsr * rs floats
    uint32_t *cnt;       // one per row tile of 64 super-rows, zero between launches
    const float *x_up;   // kXSiluUp: the input is silu(x) * x_up, elementwise
    // kXNormAdd: the input is rms_norm(x + x_res) * norm_w over the op's n
    // columns; the op-local tile 0's first wave also writes x + x_res to x_out
    const float *x_res;
    const float *norm_w;
    float *x_out;        // may be null
    float norm_eps;
    int32_t pad2_;
};

// How a matvec reads its activations (a compile-time mode of the kernels).
enum XMode : int {
    kXFloat = 0,    // x as float32
    kXQuant = 1,    // x quantized to Q8_0 per group, integer dots
    kXSiluUp = 2,   // silu(x) * x_up formed per group (the SwiGLU product feeding a down projection)
    kXNormAdd = 3,  // rms_norm(x + x_res) * norm_w formed per group (a residual add and the norm after it)
};
constexpr int kMaxSlices = 32;
// Every row sums its groups into kSlots partial sums (group kk into slot
// kk % kSlots) and combines them in a fixed tree at the end.
constexpr int kSlots = 4;

// One workgroup's work in a fused launch.
struct Tile {
    uint32_t op;    // index into the op table
    uint32_t tile;  // tile within the op; kTailBit set: tail tile
};
constexpr uint32_t kTailBit = 0x80000000u;

// Stream-K work of a one-wave workgroup: groups [g0, g1) of row tile `tile`
// (64 super-rows) of op `op`.  A row tile that several workgroups share
// (nslots > 1) has each park its partial sums in slot `slot` of the op's
// partials; the last of them to arrive adds the slots in slot order.
struct Piece {
    uint32_t op;
    uint32_t tile;
    uint32_t g0, g1;
    uint32_t slot, nslots;
};

// One phase of a one-launch chain: a stream-K schedule (pieces, then tail
// tiles) of mutually independent ops that read their activations in one
// mode.  The phases run in order, separated by device-wide barriers.
struct PhaseDesc {
    const OpDesc *ops;
    const Piece *pieces;
    const uint32_t *begin;   // n_sk + 1 piece offsets
    const Tile *tails;
    int32_t n_sk;            // workgroups with pieces (the first n_sk of the launch)
    int32_t n_tail;          // tail tiles, taken round robin by all workgroups
    int32_t xmode;           // XMode (kXFloat, kXSiluUp or kXNormAdd)
    // 1: this phase reads memory that an earlier phase of the launch read
    // and a later one rewrote, so every wave drops its CU's cached lines at
    // the barrier before it (an agent-scope acquire) -- otherwise only the
    // XCD leaders do, for the L2s
    int32_t acquire;
};

// Matvec kernel shape: waves per workgroup (1, 2 or 4) and groups each wave
// keeps in flight ahead of the one it computes (1 or 2).
struct Variant {
    int nw;
    int pf;
};

// Fast tiles cover (nw / ks) * 64 super-rows each (times the K slices).
inline int64_t fast_tiles_for(int64_t nsr, int ks, int nw = kWaves, int slices = 1) {
    const int64_t per = (int64_t)(nw / ks) * kWave;
    return (nsr + per - 1) / per * slices;
}
// Tail tiles take one row per wave.
inline int64_t tail_tiles_for(int64_t tail_rows, int nw = kWaves) {
    return (tail_rows + nw - 1) / nw;
}

// Matvec launchers (q8_gemv.hip).  All return the hipError_t of the launch.
// xmode: how the activations are read (XMode).
hipError_t launch_gemv_single(const OpDesc &op, const Variant &v, int64_t grid, hipStream_t s,
                              int xmode = kXFloat);
hipError_t launch_gemv_fused(const OpDesc *d_ops, const Tile *d_tiles, const Variant &v,
                             int64_t grid, hipStream_t s, int xmode = kXFloat);
// Stream-K launch of one-wave workgroups: workgroup b < n_sk walks pieces
// [begin[b], begin[b+1]); the n_tail workgroups after them run tails[b - n_sk]
// (tail tiles).  pf: groups in flight per wave (1 or 2).
hipError_t launch_gemv_streamk(const OpDesc *d_ops, const Piece *d_pieces, const uint32_t *d_begin,
                               const Tile *d_tails, int64_t n_sk, int64_t n_tail, int pf,
                               hipStream_t s, int xmode = kXFloat);
// One launch of a whole chain of dependent phases on `wgs` one-wave
// workgroups, all of which must be resident at once (wgs <= the CUs times
// gemv_phased_blocks_per_cu()), `per` of them on each of `nx` XCDs
// (per * nx == wgs, as the census found).  d_sync: kPhasedSyncBytes of
// barrier state, zero when first used and kept between launches; its word
// kPhasedSyncErr is set to 1 if a barrier wait gave up.
constexpr int kPhasedSyncBytes = 64 * 4 * 34;
constexpr int kPhasedSyncErr = 64 * 33;
hipError_t launch_gemv_phased(const PhaseDesc *d_phases, int n_phases, uint32_t *d_sync, uint32_t per,
                              uint32_t nx, int64_t wgs, int pf, hipStream_t s);
// The same kernel with no phases: workgroup b writes the XCD it runs on to
// d_census[b] (wgs words).
hipError_t launch_gemv_phased_census(uint32_t *d_census, int64_t wgs, hipStream_t s);
// Workgroups of the one-launch kernel that fit on one CU at once (0 on error
// or for a pf it is not built with; it has pf = 1 only).
int gemv_phased_blocks_per_cu(int pf);
// x (n floats, n % 32 == 0) -> n/32 Q8_0 blocks of 34 bytes at xq.
hipError_t launch_quantize_x(const float *x, void *xq, int64_t n, hipStream_t s);

}  // namespace q8
