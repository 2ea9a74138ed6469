// q8_gemv_rc.hip -- launches of the rows-and-group-slots matvec tile
// (q8_rc.h) for matrices whose rows are whole 272-byte groups (n a multiple
// of 256): one op, or a table of tiles of independent ops read in one mode.
//
// This file is compiled once per activation mode, with Q8_RC_XMODE set to
// the XMode (0..3); each build defines that mode's entry points
// (launch_gemv_rc_<mode>, ...), declared in q8_internal.h.
#include "q8_rc.h"

#ifndef Q8_RC_XMODE
#error "build with -DQ8_RC_XMODE=<XMode>"
#endif

namespace q8 {
namespace {

constexpr int XM = Q8_RC_XMODE;

// Every launch shape is built: (C, NWK) in {1, 2, 4} x {1, 2, 4}.  (The
// mode is a template argument too, so that profiles tell the builds apart.)
template <int C, int NWK, int MODE>
__global__ __launch_bounds__(NWK * kWave) void k_q8_gemv_rc(OpDesc op) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[rc_lds_bytes<C, NWK, MODE>()];
    rc_tile<C, NWK, MODE>(op, blockIdx.x, lds, blockIdx.x == 0);
}

template <int C, int NWK, int MODE>
__global__ __launch_bounds__(NWK * kWave) void k_q8_gemv_rc_fused(const OpDesc *__restrict__ ops,
                                                                  const Tile *__restrict__ tiles) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[rc_lds_bytes<C, NWK, MODE>()];
    const Tile tl = tiles[blockIdx.x];
    const OpDesc op = ops[tl.op];
    rc_tile<C, NWK, MODE>(op, tl.tile, lds, tl.tile == 0);
}

template <int C, int NWK>
hipError_t single_t(const OpDesc &op, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((k_q8_gemv_rc<C, NWK, XM>), dim3((unsigned)grid), dim3(NWK * kWave), 0, s, op);
    return hipGetLastError();
}

template <int C, int NWK>
hipError_t fused_t(const OpDesc *d_ops, const Tile *d_tiles, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((k_q8_gemv_rc_fused<C, NWK, XM>), dim3((unsigned)grid), dim3(NWK * kWave), 0, s, d_ops,
                       d_tiles);
    return hipGetLastError();
}

template <int C, int NWK>
constexpr int lds_of() { return rc_lds_bytes<C, NWK, XM>(); }

}  // namespace

#define Q8_CAT2(a, b) a##b
#define Q8_CAT(a, b) Q8_CAT2(a, b)

hipError_t Q8_CAT(launch_gemv_rc_, Q8_RC_XMODE)(const OpDesc &op, RcShape sh, int64_t grid, hipStream_t s) {
    if (grid <= 0 || op.rs != 1) return hipErrorInvalidValue;
    switch (sh.c * 10 + sh.nwk) {
        case 11: return single_t<1, 1>(op, grid, s);
        case 12: return single_t<1, 2>(op, grid, s);
        case 14: return single_t<1, 4>(op, grid, s);
        case 21: return single_t<2, 1>(op, grid, s);
        case 22: return single_t<2, 2>(op, grid, s);
        case 24: return single_t<2, 4>(op, grid, s);
        case 41: return single_t<4, 1>(op, grid, s);
        case 42: return single_t<4, 2>(op, grid, s);
        case 44: return single_t<4, 4>(op, grid, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t Q8_CAT(launch_gemv_rc_fused_, Q8_RC_XMODE)(const OpDesc *d_ops, const Tile *d_tiles, RcShape sh,
                                                      int64_t grid, hipStream_t s) {
    if (grid <= 0) return hipErrorInvalidValue;
    switch (sh.c * 10 + sh.nwk) {
        case 11: return fused_t<1, 1>(d_ops, d_tiles, grid, s);
        case 12: return fused_t<1, 2>(d_ops, d_tiles, grid, s);
        case 14: return fused_t<1, 4>(d_ops, d_tiles, grid, s);
        case 21: return fused_t<2, 1>(d_ops, d_tiles, grid, s);
        case 22: return fused_t<2, 2>(d_ops, d_tiles, grid, s);
        case 24: return fused_t<2, 4>(d_ops, d_tiles, grid, s);
        case 41: return fused_t<4, 1>(d_ops, d_tiles, grid, s);
        case 42: return fused_t<4, 2>(d_ops, d_tiles, grid, s);
        case 44: return fused_t<4, 4>(d_ops, d_tiles, grid, s);
        default: return hipErrorInvalidValue;
    }
}

int Q8_CAT(gemv_rc_lds_bytes_, Q8_RC_XMODE)(RcShape sh) {
    switch (sh.c * 10 + sh.nwk) {
        case 11: return lds_of<1, 1>();
        case 12: return lds_of<1, 2>();
        case 14: return lds_of<1, 4>();
        case 21: return lds_of<2, 1>();
        case 22: return lds_of<2, 2>();
        case 24: return lds_of<2, 4>();
        case 41: return lds_of<4, 1>();
        case 42: return lds_of<4, 2>();
        case 44: return lds_of<4, 4>();
        default: return 0;
    }
}

}  // namespace q8
