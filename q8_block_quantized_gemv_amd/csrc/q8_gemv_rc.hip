// q8_gemv_rc.hip -- launches of the rows-and-group-slots matvec tile
// (q8_rc.h) for matrices whose rows are whole 272-byte groups (n a multiple
// of 256): one op, or a table of tiles of independent ops read in one mode.
//
// This file is compiled once per build mode, with Q8_RC_MODE set to its
// number (0 .. kBuildModes-1: a pair of input and output modes, see
// q8_internal.h); each build defines that mode's entry points
// (launch_gemv_rc_<mode>, ...).
#include "q8_rc.h"

#ifndef Q8_RC_MODE
#error "build with -DQ8_RC_MODE=<build mode>"
#endif

namespace q8 {
namespace {

constexpr int XM = kBuildX[Q8_RC_MODE];
constexpr int YM = kBuildY[Q8_RC_MODE];

// Every launch shape whose LDS fits is built: (C, NWK) in {1, 2, 4}^2 and
// NST in {1, 2}.  (The build mode is a template argument too, so that
// profiles tell the builds apart.)
constexpr int kThreadsOf(int nwk) { return (YM == kYSwiGLU ? 2 : 1) * nwk * kWave; }

template <int C, int NWK, int NST, int MODE>
__global__ __launch_bounds__(kThreadsOf(NWK)) void k_q8_gemv_rc(OpDesc op) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[rc_lds_bytes<C, NWK, XM, NST, YM>()];
    rc_tile<C, NWK, XM, NST, YM>(op, blockIdx.x, lds, blockIdx.x == 0);
}

template <int C, int NWK, int NST, int MODE>
__global__ __launch_bounds__(kThreadsOf(NWK)) void k_q8_gemv_rc_fused(const OpDesc *__restrict__ ops,
                                                                      const Tile *__restrict__ tiles) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[rc_lds_bytes<C, NWK, XM, NST, YM>()];
    const Tile tl = tiles[blockIdx.x];
    const OpDesc op = ops[tl.op];
    rc_tile<C, NWK, XM, NST, YM>(op, tl.tile, lds, tl.tile == 0);
}

template <int C, int NWK, int NST>
constexpr bool fits() { return rc_lds_bytes<C, NWK, XM, NST, YM>() <= kMaxLds; }

template <int C, int NWK, int NST>
hipError_t single_t(const OpDesc &op, int64_t grid, hipStream_t s) {
    if constexpr (fits<C, NWK, NST>()) {
        hipLaunchKernelGGL((k_q8_gemv_rc<C, NWK, NST, Q8_RC_MODE>), dim3((unsigned)grid), dim3(kThreadsOf(NWK)),
                           0, s, op);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

template <int C, int NWK, int NST>
hipError_t fused_t(const OpDesc *d_ops, const Tile *d_tiles, int64_t grid, hipStream_t s) {
    if constexpr (fits<C, NWK, NST>()) {
        hipLaunchKernelGGL((k_q8_gemv_rc_fused<C, NWK, NST, Q8_RC_MODE>), dim3((unsigned)grid),
                           dim3(kThreadsOf(NWK)), 0, s, d_ops, d_tiles);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

template <int C, int NWK, int NST>
constexpr int lds_of() { return fits<C, NWK, NST>() ? rc_lds_bytes<C, NWK, XM, NST, YM>() : 0; }

}  // namespace

#define Q8_CAT2(a, b) a##b
#define Q8_CAT(a, b) Q8_CAT2(a, b)

// case labels: 100 * C + 10 * NWK + NST
#define Q8_RC_CASES(F, ...)                                                   \
    case 111: return F<1, 1, 1>(__VA_ARGS__);                                 \
    case 112: return F<1, 1, 2>(__VA_ARGS__);                                 \
    case 121: return F<1, 2, 1>(__VA_ARGS__);                                 \
    case 122: return F<1, 2, 2>(__VA_ARGS__);                                 \
    case 141: return F<1, 4, 1>(__VA_ARGS__);                                 \
    case 142: return F<1, 4, 2>(__VA_ARGS__);                                 \
    case 211: return F<2, 1, 1>(__VA_ARGS__);                                 \
    case 212: return F<2, 1, 2>(__VA_ARGS__);                                 \
    case 221: return F<2, 2, 1>(__VA_ARGS__);                                 \
    case 222: return F<2, 2, 2>(__VA_ARGS__);                                 \
    case 241: return F<2, 4, 1>(__VA_ARGS__);                                 \
    case 242: return F<2, 4, 2>(__VA_ARGS__);                                 \
    case 411: return F<4, 1, 1>(__VA_ARGS__);                                 \
    case 412: return F<4, 1, 2>(__VA_ARGS__);                                 \
    case 421: return F<4, 2, 1>(__VA_ARGS__);                                 \
    case 422: return F<4, 2, 2>(__VA_ARGS__);                                 \
    case 441: return F<4, 4, 1>(__VA_ARGS__);                                 \
    case 442: return F<4, 4, 2>(__VA_ARGS__);

static int shape_key(RcShape sh) { return 100 * sh.c + 10 * sh.nwk + sh.nst; }

hipError_t Q8_CAT(launch_gemv_rc_, Q8_RC_MODE)(const OpDesc &op, RcShape sh, int64_t grid, hipStream_t s) {
    if (grid <= 0 || op.rs != 1 || sh.tr < 0 || sh.tr > kWave / sh.c) return hipErrorInvalidValue;
    // the residual-add output sums squares over whole 16-row blocks of a tile
    if (YM == kYResAdd && sh.tr % kPsumRows) return hipErrorInvalidValue;
    OpDesc o = op;
    o.tile_rows = sh.tr;
    switch (shape_key(sh)) {
        Q8_RC_CASES(single_t, o, grid, s)
        default: return hipErrorInvalidValue;
    }
}

hipError_t Q8_CAT(launch_gemv_rc_fused_, Q8_RC_MODE)(const OpDesc *d_ops, const Tile *d_tiles, RcShape sh,
                                                      int64_t grid, hipStream_t s) {
    if (grid <= 0) return hipErrorInvalidValue;
    switch (shape_key(sh)) {
        Q8_RC_CASES(fused_t, d_ops, d_tiles, grid, s)
        default: return hipErrorInvalidValue;
    }
}

int Q8_CAT(gemv_rc_lds_bytes_, Q8_RC_MODE)(RcShape sh) {
    switch (shape_key(sh)) {
        Q8_RC_CASES(lds_of)
        default: return 0;
    }
}

}  // namespace q8
