// q8_api.hip -- the C ABI of include/q8gemv.h: validation, launch planning,
// decode chains (hipGraph record/replay) and the bounded stream wait.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <random>
#include <string>
#include <thread>
#include <vector>

#include "q8gemv.h"
#include "q8_internal.h"
#include "q8_gemm.h"
#include "q8_host.h"

using namespace q8;

namespace q8 {

thread_local std::string g_last_error;

int fail(int code, const std::string &msg) {
    g_last_error = msg;
    return code;
}

int fail_hip(hipError_t e, const char *where) {
    std::string m = std::string(where) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
    return fail(Q8_ERR_HIP, m);
}

bool overlaps(const void *a, int64_t na, const void *b, int64_t nb) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

// The current device must exist and be gfx950 (checked once per device).
int check_device(int *dev_out) {
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return fail(Q8_ERR_NO_DEVICE, "no HIP device is visible");
    }
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return fail_hip(e, "hipGetDevice");
    static std::mutex mu;
    static std::vector<int> arch_ok;  // -1 unknown, 0 unsupported, 1 ok
    std::lock_guard<std::mutex> lk(mu);
    if ((int)arch_ok.size() <= dev) arch_ok.resize(dev + 1, -1);
    if (arch_ok[dev] < 0) {
        hipDeviceProp_t prop;
        if ((e = hipGetDeviceProperties(&prop, dev)) != hipSuccess)
            return fail_hip(e, "hipGetDeviceProperties");
        arch_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
        if (!arch_ok[dev])
            return fail(Q8_ERR_UNSUPPORTED,
                        std::string("device is ") + prop.gcnArchName + ", this library is built for gfx950");
    }
    if (!arch_ok[dev]) return fail(Q8_ERR_UNSUPPORTED, "device is not gfx950");
    if (dev_out) *dev_out = dev;
    return Q8_OK;
}

int cu_count(int dev) {
    static std::mutex mu;
    static std::vector<int> cus;
    std::lock_guard<std::mutex> lk(mu);
    if ((int)cus.size() <= dev) cus.resize(dev + 1, 0);
    if (cus[dev] <= 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        cus[dev] = v;
    }
    return cus[dev];
}


}  // namespace q8

namespace {

constexpr int kLdsPerCu = 160 * 1024;

int64_t w_bytes(int64_t n, int64_t p) { return p * (n / kQuants) * kBlockBytes; }

// Argument checks shared by every entry point; touches no device state.
int validate(const float *x, const void *w, const float *y, int64_t m, int64_t n, int64_t p,
             const char *what) {
    std::string tag(what);
    if (!x || !w || !y) return fail(Q8_ERR_INVALID_ARG, tag + ": null pointer");
    if (n <= 0 || n % kQuants != 0 || n > Q8_MAX_N)
        return fail(Q8_ERR_SHAPE, tag + ": n=" + std::to_string(n) +
                                      " must be a positive multiple of 32 and <= 1048576");
    if (p <= 0 || p > Q8_MAX_P)
        return fail(Q8_ERR_SHAPE, tag + ": p=" + std::to_string(p) + " out of range");
    if (m < 1 || m > Q8_MAX_M)
        return fail(Q8_ERR_SHAPE, tag + ": m=" + std::to_string(m) + " must be in 1..16");
    if ((uintptr_t)w % 16 || (uintptr_t)x % 16)
        return fail(Q8_ERR_ALIGN, tag + ": w and x must be 16-byte aligned");
    if ((uintptr_t)y % 4) return fail(Q8_ERR_ALIGN, tag + ": y must be 4-byte aligned");
    const int64_t yb = 4 * m * p;
    if (overlaps(y, yb, x, 4 * m * n)) return fail(Q8_ERR_ALIAS, tag + ": y overlaps x");
    if (overlaps(y, yb, w, w_bytes(n, p))) return fail(Q8_ERR_ALIAS, tag + ": y overlaps w");
    return Q8_OK;
}

int64_t gcd64(int64_t a, int64_t b) {
    while (b) { int64_t t = a % b; a = b; b = t; }
    return a;
}

// rs > 1: waves that split one row tile's groups (ks <= nw).  A standalone
// launch wants many workgroups; inside a fused launch the other ops fill the
// GPU, so the choice only has to keep the waves of a workgroup evenly loaded.
int choose_ks(int64_t gsr, int64_t nsr, bool standalone, int nw) {
    auto eff = [&](int ks) {
        const int64_t per = (gsr + ks - 1) / ks;
        return (double)gsr / (double)(ks * per);
    };
    if (standalone) {
        for (int ks : {4, 2}) {
            if (ks > nw || gsr < ks) continue;
            if (fast_tiles_for(nsr, 1, nw) < 512 || eff(ks) >= 0.95) return ks;
        }
        return 1;
    }
    int best = 1;
    double be = eff(1);
    for (int ks : {2, 4}) {
        if (ks > nw || gsr < ks) continue;
        const double e = eff(ks);
        if (e >= 0.95 || e > be + 1e-9) { best = ks; be = e; }
    }
    return best;
}

// The op's shape fields.  rs > 1: planned for workgroups of nw waves.
OpDesc plan_op(const float *x, const void *w, float *y, int64_t m, int64_t n, int64_t p,
               bool standalone, int nw) {
    OpDesc d;
    std::memset(&d, 0, sizeof d);
    const int64_t nb = n / kQuants;
    const int64_t rs = kGroupBlocks / gcd64(nb, kGroupBlocks);
    d.x = x;
    d.w = (const uint8_t *)w;
    d.y = y;
    d.nb = (int32_t)nb;
    d.p = (int32_t)p;
    d.rs = (int32_t)rs;
    d.nsr = (int32_t)(p / rs);
    d.gsr = (int32_t)(rs * nb / kGroupBlocks);
    d.sr_bytes = rs * nb * kBlockBytes;
    d.m = (int32_t)m;
    d.x_stride = n;
    d.y_stride = p;
    if (rs == 1) {
        d.ks = 1;
        d.fast_tiles = (int32_t)rc_tiles_for(p, 1);
        d.tail_row0 = (int32_t)p;
    } else {
        d.ks = choose_ks(d.gsr, d.nsr, standalone, nw);
        d.fast_tiles = (int32_t)fast_tiles_for(d.nsr, d.ks, nw);
        d.tail_row0 = (int32_t)(d.nsr * rs);
    }
    return d;
}

// rs > 1: every workgroup of a launch, fast tiles then tail tiles.
int64_t tiles_of(const OpDesc &d, int nw) {
    return (int64_t)d.fast_tiles + tail_tiles_for((int64_t)d.p - d.tail_row0, nw);
}

// Launch shape of the rows-and-group-slots kernel for a launch that waits
// on the one before it: `rows` rows of G groups (one op, or independent ops
// of one width) read in mode xmode, on `cus` CUs.  From a sweep of lone
// launches at the decode shapes (0.6B and 7B projections, lm_heads, in each
// input mode):
//  * tiles of 16 rows (C = 4) with the groups split over NWK waves by slot,
//    as many waves as there are group columns (up to 4), when one wave of
//    such workgroups covers the rows (a row-poor op: every wave then streams
//    its columns at once, e.g. 7B q/o/down, every 0.6B projection);
//  * tiles of 32 rows with four waves when that still fits (7B q|k|v);
//  * otherwise one-wave tiles of 16 rows (7B gate; the lm_heads, with the
//    weights read non-temporal: 7B 98.2 us against 102.3 with two-wave
//    tiles, 0.6B 34.6 us against 53.9) -- except where every workgroup
//    first sums the squares of x + x_res over the whole row (kXNormAdd), and
//    for the gate|up pair (kYSwiGLU, two waves per tile already): there
//    one-wave tiles of 32 rows, half the workgroups, are fastest.
// One W stage per wave: twice the waves fit, which measured faster than a
// second stage at every one of these shapes.
//
// One op (`single`): where the tiles are all resident but come two or more
// to a CU, some CUs get one tile more than others and finish last; tiles of
// fewer rows, ceil(rows / (k * cus)) for k tiles a CU, even the CUs out.
// Measured on lone launches: the 7B gate|up pair 30.0 -> 28.3 us (32 -> 26
// rows a tile), and the 7B gate alone 18.9 us in one-wave tiles of 16 rows
// -> 18.1 us in two-wave tiles of 25 (of 32) rows.  Where one round of tiles
// leaves CUs idle (k = 1) smaller tiles measured no faster (7B q, k, down:
// latency, not rows, sets their time), and for many rounds (lm_heads) the
// rule gives whole tiles anyway.  Not for the residual-add output, whose
// tiles hold whole 16-row blocks.
RcShape plan_rc_latency(int64_t rows, int64_t G, int xmode, int ymode, int64_t cus, bool single) {
    auto resident = [&](RcShape sh) {
        const int b = gemv_rc_lds_bytes(sh, xmode, ymode);
        return b > 0 ? cus * std::max(1, kLdsPerCu / b) : 0;
    };
    auto balanced = [&](RcShape sh) {
        const int R = kWave / sh.c;
        const int64_t t = (rows + R - 1) / R, k = (t + cus - 1) / cus;
        if (!single || ymode == kYResAdd || k < 2 || t > resident(sh)) return sh;
        const int64_t tr = (rows + k * cus - 1) / (k * cus);
        if (tr < R) sh.tr = (int)tr;
        return sh;
    };
    const int64_t J4 = (G + 3) / 4;
    const int n4 = J4 >= 3 ? 4 : (int)J4;
    const int64_t t4 = (rows + 15) / 16;
    if (t4 <= resident({4, n4, 1})) return balanced({4, n4, 1});
    if ((G + 1) / 2 >= 4 && (rows + 31) / 32 <= resident({2, 4, 1})) return balanced({2, 4, 1});
    if (xmode == kXNormAdd || ymode == kYSwiGLU) return balanced({2, 1, 1});
    if (single && (G + 1) / 2 >= 2) {
        const int64_t t2 = (rows + 31) / 32;
        if (t2 > cus && t2 <= resident({2, 2, 1})) return balanced({2, 2, 1});
    }
    return balanced({4, 1, 1});
}

// Launch shape of a fused launch of independent ops (a throughput launch),
// and whether its weights are loaded non-temporal (each is read once).
//  * Float x: one-wave 16-row tiles, four lanes per row, one W stage,
//    non-temporal.  A group column is then 16 runs of 1088 contiguous bytes
//    (whole rows where n = 1024), so few 128-byte lines are split between
//    two columns, and the hint pays.  Measured (kernel time per token): 7B
//    chain 1180-1182 us against 1189-1193 with the shape below; 0.6B chain
//    102.5-106.3 against 107.3-107.4 (box to box), 111.6 with four lanes and
//    plain loads, 104.0 with the hint only where a column holds whole rows;
//    with two lanes (runs of 544 bytes) the hint lost (7B chain 1360 us:
//    every line two runs share came in twice).
//  * x quantized per column (kXQuant): two lanes per row, plain loads, two
//    W stages where the launch's byte-weighted mean row is 8 groups or more,
//    else one: a tile quantizes each column's x slices, and 16-row tiles
//    would do that twice as often per weight byte (7B chain 1261 us against
//    1190).  The 7B chain (mean ~20 groups) 1190 us with {2, 1, 2}, 1226 with
//    one lane; the 0.6B shape (mean ~5.6) 107.3 us with {2, 1, 1}, 109.1
//    with {1, 1, 2}, 115 with {2, 1, 2}.
struct FusePlan {
    RcShape shape;
    bool w_once;
};
FusePlan fuse_plan(int xmode, double mean_groups) {
    if (xmode == kXQuant) return {mean_groups >= 8.0 ? RcShape{2, 1, 2} : RcShape{2, 1, 1}, false};
    return {RcShape{4, 1, 1}, true};
}

bool shape_ok(int c, int nwk, int nst) {
    return (c == 1 || c == 2 || c == 4) && (nwk == 1 || nwk == 2 || nwk == 4) && (nst == 1 || nst == 2);
}

// One matvec: rs == 1 on the rows-and-group-slots kernel in `sh` (or its
// latency plan when sh.c == 0); rs > 1 on four-wave super-row workgroups.
int gemv_launch(const float *x, const void *w, float *y, int64_t n, int64_t p, hipStream_t s,
                int xmode, RcShape sh, const char *what) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    OpDesc d = plan_op(x, w, y, 1, n, p, true, kWaves);
    if (d.rs == 1) {
        if (sh.c == 0) sh = plan_rc_latency(p, d.gsr, xmode, kYPlain, cu_count(dev), true);
        d.w_once = 1;
        e = launch_gemv_rc(d, sh, rc_tiles_for(p, sh), s, xmode);
    } else {
        e = launch_gemv_single(d, Variant{kWaves, 1}, tiles_of(d, kWaves), s, xmode);
    }
    if (e != hipSuccess) return fail_hip(e, what);
    return Q8_OK;
}

// Shape fields of a small-batch product (validated arguments).
GemmDesc plan_gemm(const float *X, const void *w, float *Y, int64_t m, int64_t n, int64_t p) {
    GemmDesc d;
    std::memset(&d, 0, sizeof d);
    const int64_t nb = n / kQuants;
    const int64_t rs = kGroupBlocks / gcd64(nb, kGroupBlocks);
    d.X = X;
    d.w = (const uint8_t *)w;
    d.Y = Y;
    d.n = (int32_t)n;
    d.nb = (int32_t)nb;
    d.p = (int32_t)p;
    d.m = (int32_t)m;
    d.rs = (int32_t)rs;
    d.nsr = (int32_t)(p / rs);
    d.gsr = (int32_t)(rs * nb / kGroupBlocks);
    d.sr_bytes = rs * nb * kBlockBytes;
    d.row_tiles = (int32_t)((d.nsr + kWave - 1) / kWave);
    d.tail_row0 = d.nsr * (int32_t)rs;
    return d;
}

// Stream-K split: up to `wpc` one-wave workgroups per CU, each an equal
// contiguous range of at least `min_items` (row tile, group) items, so that
// short ranges do not multiply the partial sums.  Sets fast_wgs and returns
// the bytes of partial slots the split needs (two per workgroup).
size_t plan_streamk(GemmDesc &d, int64_t cus, int wpc, int min_items) {
    const int64_t items = (int64_t)d.row_tiles * d.gsr;
    const int64_t slots = (int64_t)wpc * cus;
    const int64_t wgs = std::max<int64_t>(1, std::min({items, slots, items / min_items}));
    d.fast_wgs = (int32_t)wgs;
    return (size_t)(2 * wgs) * d.m * kWave * d.rs * sizeof(float);
}

// The column ranges and row blocks of the matrix cores with X held in LDS
// (k_q8_gemm_ks, eight waves, one workgroup per CU): as many groups per
// range as the LDS left by the waves' stages holds parts of X for (1.5 KiB
// per row of X and group), ranges evened out; then the shortest row blocks
// (a multiple of 32 rows) whose workgroups all fit on the CUs at once
// (measured: one round of workgroups, 25.2 us for gate at m = 16, against
// 31-35 us for blocks that leave a second, partial round).
void plan_ks(GemmDesc &d, int64_t cus) {
    const int64_t gk_max = std::max<int64_t>(1, ks_a_bytes(8) / ((int64_t)kGroupBlocks * d.m * 192));
    const int64_t nkr = (d.gsr + gk_max - 1) / gk_max;
    d.ks_ranges = (int32_t)nkr;
    d.ks_groups = (int32_t)((d.gsr + nkr - 1) / nkr);
    const int64_t blocks = std::max<int64_t>(1, cus / nkr);
    int64_t rows = (d.p + blocks - 1) / blocks;
    d.ks_rows = (int32_t)std::max<int64_t>(32, (rows + 31) / 32 * 32);
    // The ranges' sums: added by each row block's last workgroup (no second
    // launch) where that is at most 32 loads a thread and the ranges hold at
    // most 512K sums, else by k_ks_reduce.  The in-kernel sum has its sums
    // stored device-coherent, one by one: measured 1.1 us faster for down at
    // m = 4 and 8, but 4.2 us slower for gate at m = 16 (1.5M sums, 60
    // loads a thread) and 10.9 us for the lm_head at m = 8 (2.4M sums).
    d.ks_sum_here = nkr > 1 && nkr * d.m * (int64_t)d.ks_rows <= 32 * 8 * kWave &&
                    nkr * d.m * (int64_t)d.p <= ((int64_t)1 << 19) ? 1 : 0;
}

// A small-batch product's workspace, every piece 256-byte aligned: the
// per-row-tile arrival counters (8 bytes each, tagged with the call's epoch,
// so they need no clearing), then (matrix cores) X split into bf16 parts,
// then the partial slots.
struct SmallmWs {
    size_t cnt = 0, xs = 0, part = 0, bytes = 0;   // offsets and total
};
size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// A resolved kernel (never Q8_SMALLM_AUTO) for m rows: its plan and
// workspace.  m = 1 needs none.
SmallmWs smallm_plan(GemmDesc &d, int kernel, int64_t cus) {
    SmallmWs L;
    if (d.m == 1) return L;
    size_t part = 0, xs = 0;
    if (kernel == Q8_SMALLM_KS) {
        plan_ks(d, cus);
        part = d.ks_ranges > 1 ? (size_t)d.ks_ranges * d.m * d.p * sizeof(float) : 0;
        const size_t cnt = d.ks_sum_here ? (size_t)((d.p + d.ks_rows - 1) / d.ks_rows) * 8 : 0;
        L.cnt = 0;
        L.part = align256(cnt);
        L.bytes = L.part + align256(part);
        return L;
    }
    if (kernel == Q8_SMALLM_MFMA) {
        part = plan_streamk(d, cus, 4, 4);   // four double-buffered one-wave workgroups fill a CU's LDS
        xs = (size_t)d.nb * kXPartsBytesPerBlock;
    } else {
        // as many workgroups per CU as their double-buffered stages fit in 160 KiB of LDS
        part = plan_streamk(d, cus, (160 * 1024) / gemm_valu_stage_bytes(d.m), 4);
    }
    L.cnt = 0;
    L.xs = align256((size_t)d.row_tiles * sizeof(unsigned long long));
    L.part = L.xs + align256(xs);
    L.bytes = L.part + align256(part);
    return L;
}

// A small-batch call's kernel argument checked against (m, n): the kernel
// (Q8_SMALLM_AUTO stays so; smallm_resolve picks once the device is known),
// or an error status (negative).
int smallm_kernel(int kernel, int64_t m, int64_t n, const char *what) {
    if (kernel < Q8_SMALLM_AUTO || kernel > Q8_SMALLM_KS)
        return fail(Q8_ERR_INVALID_ARG, std::string(what) + ": unknown kernel");
    const int64_t rs = kGroupBlocks / gcd64(n / kQuants, kGroupBlocks);
    const bool mfma_ok = rs <= 2, vrow_ok = rs == 1 && m >= 2 && m <= kVrowMaxM;
    if ((kernel == Q8_SMALLM_MFMA && !(mfma_ok && m >= 2)) || (kernel == Q8_SMALLM_KS && !(rs == 1 && m >= 2)) ||
        ((kernel == Q8_SMALLM_VROW || kernel == Q8_SMALLM_VROW1) && !vrow_ok) ||
        (kernel == Q8_SMALLM_VALU && m < 2))
        return fail(Q8_ERR_SHAPE, std::string(what) + ": this kernel does not take m=" + std::to_string(m) +
                                       ", n=" + std::to_string(n));
    return kernel;
}

// Most bytes of per-range sums Q8_SMALLM_AUTO lets the held-X kernel take:
// with a caller's workspace, and within the library's scratch (the
// allocation-free entry point, whose choice must fit what it has).
constexpr int64_t kKsPartCap = int64_t(64) << 20;
constexpr int64_t kKsPartCapNoAlloc = int64_t(16) << 20;

// The kernel Q8_SMALLM_AUTO runs for a validated (m, n, p) on a device of
// `cus` CUs; a named kernel is returned as it is.
int smallm_resolve(int kernel, int64_t m, int64_t n, int64_t p, int64_t cus, int64_t part_cap = kKsPartCap) {
    if (kernel != Q8_SMALLM_AUTO) return kernel;
    const int64_t rs = kGroupBlocks / gcd64(n / kQuants, kGroupBlocks);
    const bool mfma_ok = rs <= 2, vrow_ok = rs == 1 && m >= 2 && m <= kVrowMaxM;
    // Rows of whole groups (n a multiple of 256) run on the matrix cores with
    // each column range's parts of X held in LDS (one copy of X per
    // workgroup, not per wave): at the 7B shapes 26-32 us for down and gate
    // at m = 4..16 against 30-44 us for the stream-K matrix-core kernel, and
    // 109-161 us for the lm_head at m = 2..16 against 115-172 us -- except
    // m = 2..3 at fewer than 65536 rows, where the vector units with lanes
    // over (row, block pair) keep each lane's x values in registers and need
    // no split of X (down 26.5-26.9 us, gate 22.5 us at m = 2, against 39.1
    // and 25.3 on the stream-K matrix cores and 36.0-36.2 and 23.4 with X
    // held in LDS), and shapes whose per-range sums would pass part_cap, which stay
    // on the stream-K kernel (the 7B lm_head at m = 16, 48.7 MB of sums:
    // 149.3-149.5 us held-X against 164.1-164.6 stream-K, so a caller's
    // workspace may hold them; the library's scratch may not).  Where rows fill
    // super-rows of 1 or 2 (n a multiple of 128) the stream-K matrix cores
    // take m >= 2.  Other widths run on the vector units with a lane per
    // row, kValuMaxM rows of X per pass over W.
    if (rs == 1 && m >= 2 && !(m <= kVrowMaxM && p < 65536)) {
        static const float kShapeOnly[4] = {0.f, 0.f, 0.f, 0.f};   // the plan reads only shapes
        GemmDesc d = plan_gemm(kShapeOnly, kShapeOnly, nullptr, m, n, p);
        plan_ks(d, cus);
        const int64_t part = d.ks_ranges > 1 ? (int64_t)d.ks_ranges * m * p * (int64_t)sizeof(float) : 0;
        if (part <= part_cap) return Q8_SMALLM_KS;
    }
    return vrow_ok ? Q8_SMALLM_VROW : mfma_ok ? Q8_SMALLM_MFMA : Q8_SMALLM_VALU;
}

// Workspace bytes of a call (the largest of its launches; they run in order
// on one stream and share it).
size_t smallm_bytes(const float *X, const void *w, float *Y, int64_t m, int64_t n, int64_t p, int kernel,
                    int64_t cus) {
    if (m == 1) return 0;
    const int64_t mi = kernel == Q8_SMALLM_VALU ? std::min<int64_t>(kValuMaxM, m) : m;
    GemmDesc d = plan_gemm(X, w, Y, mi, n, p);
    return smallm_plan(d, kernel, cus).bytes;
}

// A call's tag for its arrival counters: distinct for 2^32 - 1 calls of the
// process, from a start that differs between processes, never 0.
uint32_t next_epoch() {
    static std::atomic<uint32_t> e{(uint32_t)std::random_device{}() | 1u};
    uint32_t v;
    do v = e.fetch_add(1u, std::memory_order_relaxed); while (v == 0u);
    return v;
}

// One launch of a resolved kernel for mi rows on the workspace ws.
int smallm_launch(const float *X, const void *w, float *Y, int64_t mi, int64_t n, int64_t p, int kernel,
                  uint8_t *ws, int64_t cus, hipStream_t s) {
    GemmDesc d = plan_gemm(X, w, Y, mi, n, p);
    const SmallmWs L = smallm_plan(d, kernel, cus);
    d.cnt = (unsigned long long *)(ws + L.cnt);
    d.ws = (float *)(ws + L.part);
    d.epoch = next_epoch();
    hipError_t e;
    if (kernel == Q8_SMALLM_KS) {
        d.yp = (float *)(ws + L.part);
        e = launch_gemm_ks(d, 8, s);   // (d.cnt and d.epoch are set above)
    } else if (kernel == Q8_SMALLM_MFMA) {
        d.xs = (const bf16x8 *)(ws + L.xs);
        e = launch_split_x(X, ws + L.xs, (int)mi, (int)n, s);
        if (e != hipSuccess) return fail_hip(e, "q8_0_gemm_smallm split launch");
        e = launch_gemm_mfma(d, (int64_t)d.fast_wgs + (p - d.tail_row0), s);
    } else {
        if (kernel == Q8_SMALLM_VROW || kernel == Q8_SMALLM_VROW1)
            // two waves per workgroup (the default) share its stages, each
            // taking half the rows of every group -- two waves per SIMD where
            // one wave's stages fill a quarter of the LDS (measured 5-10 %
            // faster than one wave; four waves, held to two per SIMD by their
            // registers, slower)
            e = launch_gemm_vrow(d, kernel == Q8_SMALLM_VROW ? 2 : 1, s);
        else
            e = launch_gemm_valu(d, (int64_t)d.fast_wgs + (p - d.tail_row0), s);
    }
    if (e != hipSuccess) return fail_hip(e, "q8_0_gemm_smallm launch");
    return Q8_OK;
}

// The whole call: m = 1 is the matvec; the vector-unit kernel takes
// kValuMaxM rows of X per pass over W; the others take all m at once.
int smallm_run(const float *X, const void *w, float *Y, int64_t m, int64_t n, int64_t p, int kernel,
               uint8_t *ws, int64_t cus, hipStream_t s) {
    if (m == 1)
        return gemv_launch(X, w, Y, n, p, s, kXFloat, RcShape{0, 0, 0}, "q8_0_gemm_smallm launch");
    if (kernel != Q8_SMALLM_VALU) return smallm_launch(X, w, Y, m, n, p, kernel, ws, cus, s);
    for (int64_t i0 = 0; i0 < m; i0 += kValuMaxM) {
        const int64_t mi = std::min<int64_t>(kValuMaxM, m - i0);
        const int rc = mi == 1 ? gemv_launch(X + i0 * n, w, Y + i0 * p, n, p, s, kXFloat, RcShape{0, 0, 0},
                                             "q8_0_gemm_smallm launch")
                               : smallm_launch(X + i0 * n, w, Y + i0 * p, mi, n, p, kernel, ws, cus, s);
        if (rc) return rc;
    }
    return Q8_OK;
}

}  // namespace

// ===================================================================== static scratch
// The allocation-free small-batch entry point's scratch: a file-scope device
// array, kScratchBytes on every GPU the library runs on, held until the
// process ends.  In host code `scratch` is only a host-side stand-in; the
// device address of each GPU's copy comes from hipGetSymbolAddress, once per
// device with that device current, and is the only form passed to kernels.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

int scratch_for(int dev, uint8_t **out) {
    static std::mutex mu;
    static std::vector<uint8_t *> ptrs;
    std::lock_guard<std::mutex> lk(mu);
    if ((int)ptrs.size() <= dev) ptrs.resize(dev + 1, nullptr);
    if (!ptrs[dev]) {
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return fail_hip(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                                   "hipGetSymbolAddress(scratch)");
        ptrs[dev] = (uint8_t *)p;
    }
    *out = ptrs[dev];
    return Q8_OK;
}

}  // namespace

// ===================================================================== ABI
extern "C" {

const char *q8_0_status_string(int status) {
    switch (status) {
        case Q8_OK: return "ok";
        case Q8_ERR_INVALID_ARG: return "invalid argument";
        case Q8_ERR_SHAPE: return "shape out of range";
        case Q8_ERR_ALIGN: return "misaligned pointer";
        case Q8_ERR_ALIAS: return "output overlaps an input";
        case Q8_ERR_NO_DEVICE: return "no HIP device";
        case Q8_ERR_HIP: return "HIP runtime error";
        case Q8_ERR_TIMEOUT: return "timed out";
        case Q8_ERR_UNSUPPORTED: return "unsupported device";
        default: return "unknown status";
    }
}

const char *q8_0_last_error(void) { return g_last_error.c_str(); }

int q8_0_gemv(const float *x, const void *w, float *y, int64_t n, int64_t p, void *stream) {
    int rc = validate(x, w, y, 1, n, p, "q8_0_gemv");
    if (rc) return rc;
    if ((rc = check_device())) return rc;
    return gemv_launch(x, w, y, n, p, (hipStream_t)stream, kXFloat, RcShape{0, 0, 0}, "q8_0_gemv launch");
}

int q8_0_gemv_shaped(const float *x, const void *w, float *y, int64_t n, int64_t p, int lanes_per_row,
                     int waves, int stages, void *stream) {
    int rc = validate(x, w, y, 1, n, p, "q8_0_gemv_shaped");
    if (rc) return rc;
    const RcShape sh{lanes_per_row, waves, stages};
    if (!shape_ok(lanes_per_row, waves, stages) || gemv_rc_lds_bytes(sh, kXFloat) == 0)
        return fail(Q8_ERR_INVALID_ARG, "q8_0_gemv_shaped: lanes_per_row and waves must each be 1, 2 or 4, "
                                        "stages 1 or 2, and the workgroup's LDS must fit in 160 KiB");
    if (n % (kQuants * kGroupBlocks))
        return fail(Q8_ERR_SHAPE, "q8_0_gemv_shaped: n must be a multiple of 256 for an explicit launch shape");
    if ((rc = check_device())) return rc;
    return gemv_launch(x, w, y, n, p, (hipStream_t)stream, kXFloat, sh, "q8_0_gemv_shaped launch");
}

int q8_0_gemv_q8q8(const float *x, const void *w, float *y, int64_t n, int64_t p, void *stream) {
    int rc = validate(x, w, y, 1, n, p, "q8_0_gemv_q8q8");
    if (rc) return rc;
    if ((rc = check_device())) return rc;
    return gemv_launch(x, w, y, n, p, (hipStream_t)stream, kXQuant, RcShape{0, 0, 0}, "q8_0_gemv_q8q8 launch");
}

int q8_0_quantize(const float *x, void *xq, int64_t n, void *stream) {
    if (!x || !xq) return fail(Q8_ERR_INVALID_ARG, "q8_0_quantize: null pointer");
    if (n <= 0 || n % kQuants || n > ((int64_t)1 << 31))
        return fail(Q8_ERR_SHAPE, "q8_0_quantize: n must be a positive multiple of 32, at most 2^31");
    if ((uintptr_t)x & 3u) return fail(Q8_ERR_ALIGN, "q8_0_quantize: x must be 4-byte aligned");
    if (overlaps(xq, n / kQuants * kBlockBytes, x, 4 * n))
        return fail(Q8_ERR_ALIAS, "q8_0_quantize: xq overlaps x");
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_quantize_x(x, xq, n, (hipStream_t)stream);
    return e == hipSuccess ? Q8_OK : fail_hip(e, "q8_0_quantize launch");
}

int q8_0_gemm_smallm_workspace(int64_t m, int64_t n, int64_t p, int kernel, size_t *bytes) {
    if (!bytes) return fail(Q8_ERR_INVALID_ARG, "q8_0_gemm_smallm_workspace: bytes is null");
    *bytes = 0;
    if (n <= 0 || n % kQuants != 0 || n > Q8_MAX_N || p <= 0 || p > Q8_MAX_P || m < 1 || m > Q8_MAX_M)
        return fail(Q8_ERR_SHAPE, "q8_0_gemm_smallm_workspace: shape out of range");
    int k = smallm_kernel(kernel, m, n, "q8_0_gemm_smallm_workspace");
    if (k < 0) return k;
    int dev = 0;
    int rc = check_device(&dev);
    if (rc) return rc;
    k = smallm_resolve(k, m, n, p, cu_count(dev));
    // (the plan reads only shapes; these pointers are never dereferenced)
    static const float kDummyX[4] = {0.f, 0.f, 0.f, 0.f};
    *bytes = smallm_bytes(kDummyX, kDummyX, nullptr, m, n, p, k, cu_count(dev));
    return Q8_OK;
}

int q8_0_gemm_smallm_choice(int64_t m, int64_t n, int64_t p, int *kernel) {
    if (!kernel) return fail(Q8_ERR_INVALID_ARG, "q8_0_gemm_smallm_choice: kernel is null");
    *kernel = Q8_SMALLM_AUTO;
    if (n <= 0 || n % kQuants != 0 || n > Q8_MAX_N || p <= 0 || p > Q8_MAX_P || m < 2 || m > Q8_MAX_M)
        return fail(Q8_ERR_SHAPE, "q8_0_gemm_smallm_choice: shape out of range (m = 2..16)");
    int dev = 0;
    const int rc = check_device(&dev);
    if (rc) return rc;
    *kernel = smallm_resolve(Q8_SMALLM_AUTO, m, n, p, cu_count(dev));
    return Q8_OK;
}

int q8_0_gemm_smallm_kernel(const float *X, const void *w, float *Y, int64_t m, int64_t n, int64_t p,
                            int kernel, void *workspace, size_t workspace_bytes, void *stream) {
    int rc = validate(X, w, Y, m, n, p, "q8_0_gemm_smallm");
    if (rc) return rc;
    int k = smallm_kernel(kernel, m, n, "q8_0_gemm_smallm_kernel");
    if (k < 0) return k;
    int dev = 0;
    if ((rc = check_device(&dev))) return rc;
    const int64_t cus = cu_count(dev);
    k = smallm_resolve(k, m, n, p, cus);
    const size_t need = smallm_bytes(X, w, Y, m, n, p, k, cus);
    if (need > 0) {
        if (!workspace || ((uintptr_t)workspace & 255u))
            return fail(Q8_ERR_ALIGN, "q8_0_gemm_smallm: the workspace must be a 256-byte aligned device buffer");
        if (workspace_bytes < need)
            return fail(Q8_ERR_INVALID_ARG, "q8_0_gemm_smallm: the workspace holds " + std::to_string(workspace_bytes) +
                                                " bytes, the call needs " + std::to_string(need) +
                                                " (q8_0_gemm_smallm_workspace)");
        const int64_t nb = (int64_t)need;
        if (overlaps(workspace, nb, X, 4 * m * n) || overlaps(workspace, nb, w, w_bytes(n, p)) ||
            overlaps(workspace, nb, Y, 4 * m * p))
            return fail(Q8_ERR_ALIAS, "q8_0_gemm_smallm: the workspace overlaps X, w or Y");
    }
    return smallm_run(X, w, Y, m, n, p, k, (uint8_t *)workspace, cus, (hipStream_t)stream);
}

int q8_0_gemm_smallm(const float *X, const void *w, float *Y, int64_t m, int64_t n, int64_t p,
                     void *workspace, size_t workspace_bytes, void *stream) {
    return q8_0_gemm_smallm_kernel(X, w, Y, m, n, p, Q8_SMALLM_AUTO, workspace, workspace_bytes, stream);
}

int q8_0_gemm_smallm_noalloc(const float *X, const void *w, float *Y, int64_t m, int64_t n, int64_t p,
                             void *stream) {
    int rc = validate(X, w, Y, m, n, p, "q8_0_gemm_smallm_noalloc");
    if (rc) return rc;
    int k = smallm_kernel(Q8_SMALLM_AUTO, m, n, "q8_0_gemm_smallm_noalloc");
    if (k < 0) return k;
    int dev = 0;
    if ((rc = check_device(&dev))) return rc;
    const int64_t cus = cu_count(dev);
    k = smallm_resolve(k, m, n, p, cus, kKsPartCapNoAlloc);
    const size_t need = smallm_bytes(X, w, Y, m, n, p, k, cus);
    if (need > kScratchBytes)
        return fail(Q8_ERR_SHAPE, "q8_0_gemm_smallm_noalloc: m=" + std::to_string(m) + ", n=" + std::to_string(n) +
                                      ", p=" + std::to_string(p) + " needs " + std::to_string(need) +
                                      " bytes of scratch, more than the library's " +
                                      std::to_string(kScratchBytes) +
                                      "; call q8_0_gemm_smallm with a workspace instead");
    uint8_t *ptr = nullptr;
    if (need > 0 && (rc = scratch_for(dev, &ptr))) return rc;
    return smallm_run(X, w, Y, m, n, p, k, ptr, cus, (hipStream_t)stream);
}

int q8_0_stream_wait(void *stream, int64_t timeout_ms) {
    const auto t0 = std::chrono::steady_clock::now();
    for (;;) {
        hipError_t e = hipStreamQuery((hipStream_t)stream);
        if (e == hipSuccess) return Q8_OK;
        if (e != hipErrorNotReady) return fail_hip(e, "hipStreamQuery");
        if (timeout_ms >= 0) {
            const auto el = std::chrono::duration_cast<std::chrono::milliseconds>(
                std::chrono::steady_clock::now() - t0).count();
            if (el >= timeout_ms)
                return fail(Q8_ERR_TIMEOUT, "stream still busy after " + std::to_string(timeout_ms) + " ms");
        }
        std::this_thread::sleep_for(std::chrono::microseconds(50));
    }
}

}  // extern "C"

// ===================================================================== chains
struct q8_0_chain {
    int device = -1;
    uint32_t flags = 0;
    std::vector<q8_0_op> ops;
    // one entry per kernel launch of a token
    struct Launch {
        enum Kind { kSingleRc, kSingleSuperrow, kFusedRc, kFusedMixed } kind;
        int xmode;            // XMode: how the activations are read
        int ymode;            // YMode: what is written
        RcShape shape;        // kSingleRc, kFusedRc
        OpDesc single;        // single-op launches
        const OpDesc *d_ops;  // fused launches: op table and tiles
        const Tile *d_tiles;
        int64_t grid;
    };
    std::vector<Launch> launches;
    void *d_table = nullptr;
    hipStream_t capture = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

namespace {

hipError_t issue(const q8_0_chain::Launch &L, hipStream_t s) {
    switch (L.kind) {
        case q8_0_chain::Launch::kSingleRc: return launch_gemv_rc(L.single, L.shape, L.grid, s, L.xmode, L.ymode);
        case q8_0_chain::Launch::kSingleSuperrow:
            return launch_gemv_single(L.single, Variant{kWaves, 1}, L.grid, s, L.xmode);
        case q8_0_chain::Launch::kFusedRc:
            return launch_gemv_rc_fused(L.d_ops, L.d_tiles, L.shape, L.grid, s, L.xmode, L.ymode);
        case q8_0_chain::Launch::kFusedMixed: return launch_gemv_fused(L.d_ops, L.d_tiles, Variant{1, 1}, L.grid, s, L.xmode);
    }
    return hipErrorInvalidValue;
}

void chain_free(q8_0_chain *c) {
    if (!c) return;
    if (c->exec) (void)hipGraphExecDestroy(c->exec);
    if (c->graph) (void)hipGraphDestroy(c->graph);
    if (c->capture) (void)hipStreamDestroy(c->capture);
    if (c->d_table) (void)hipFree(c->d_table);
    delete c;
}

// The memory an op reads and writes, as (pointer, bytes) ranges.
struct Ranges {
    const void *r[7];
    int64_t rn[7];
    int nr = 0;
    const void *w[3];
    int64_t wn[3];
    int nw = 0;
};

Ranges ranges_of(const q8_0_op &o, const OpExtra *e) {
    Ranges g;
    auto rd = [&](const void *p, int64_t n) { if (p) { g.r[g.nr] = p; g.rn[g.nr++] = n; } };
    auto wr = [&](const void *p, int64_t n) { if (p) { g.w[g.nw] = p; g.wn[g.nw++] = n; } };
    rd(o.x, 4 * o.n);
    rd(o.w, w_bytes(o.n, o.p));
    wr(o.y, 4 * o.p);
    if (e) {
        rd(e->x_up, 4 * o.n);
        const int64_t en = 4 * (e->out_mode == kYResAdd ? o.p : o.n);   // residual vectors are outputs' length
        rd(e->x_res, en);
        rd(e->norm_w, en);
        wr(e->x_out, en);
        rd(e->w2, w_bytes(o.n, o.p));
        if (e->out_mode == kYResAdd) wr(e->psum, 4 * (o.p / kPsumRows));
        else if (e->mode == kXNormScale) rd(e->psum, 4 * (o.n / kPsumRows));
    }
    return g;
}

// Does op b have to wait for op a (a earlier)?  Any write of one that
// touches memory the other reads or writes.
bool depends(const q8_0_op &a, const q8_0_op &b, const OpExtra *ea = nullptr,
             const OpExtra *eb = nullptr) {
    const Ranges A = ranges_of(a, ea), B = ranges_of(b, eb);
    for (int i = 0; i < B.nw; ++i) {
        for (int j = 0; j < A.nr; ++j)
            if (overlaps(B.w[i], B.wn[i], A.r[j], A.rn[j])) return true;
        for (int j = 0; j < A.nw; ++j)
            if (overlaps(B.w[i], B.wn[i], A.w[j], A.wn[j])) return true;
    }
    for (int i = 0; i < A.nw; ++i)
        for (int j = 0; j < B.nr; ++j)
            if (overlaps(A.w[i], A.wn[i], B.r[j], B.rn[j])) return true;
    return false;
}

void set_extra(OpDesc &d, const OpExtra *e) {
    if (!e) return;
    d.x_up = e->x_up;
    d.x_res = e->x_res;
    d.norm_w = e->norm_w;
    d.x_out = e->x_out;
    d.norm_eps = e->eps;
    d.psum = e->psum;
    d.psum_n = e->mode == kXNormScale ? (int32_t)(d.nb * kQuants / kPsumRows) : 0;
    d.w2 = (const uint8_t *)e->w2;
}

struct ChainPlan {
    struct SegInfo {
        q8_0_chain::Launch L;
        size_t op0, tile0;   // the launch's op descriptors and tiles in h_ops, h_tiles
        int64_t first, n;    // its ops: ops[first .. first + n)
    };
    std::vector<OpDesc> h_ops;
    std::vector<Tile> h_tiles;
    std::vector<SegInfo> info;
};

// Argument checks of a chain (touch no device state).
int validate_chain(const q8_0_op *ops, int64_t n_ops, uint32_t flags, const OpExtra *extra, const char *what) {
    if (!ops || n_ops <= 0 || n_ops > Q8_MAX_CHAIN_OPS)
        return fail(Q8_ERR_INVALID_ARG, std::string(what) + ": need 1..65535 ops");
    if (flags & ~(uint32_t)(Q8_CHAIN_PER_OP | Q8_CHAIN_SPLIT_K | Q8_CHAIN_XQ))
        return fail(Q8_ERR_INVALID_ARG, std::string(what) + ": unknown flags");
    const int emode = extra ? extra[0].mode : kXFloat;
    const int eout = extra ? extra[0].out_mode : kYPlain;
    if (extra && (flags & Q8_CHAIN_XQ))
        return fail(Q8_ERR_INVALID_ARG, std::string(what) + ": these inputs have no integer form");
    auto a16 = [](const void *p) { return p && ((uintptr_t)p & 15u) == 0; };
    auto a4 = [](const void *p) { return p && ((uintptr_t)p & 3u) == 0; };
    for (int64_t i = 0; i < n_ops; ++i) {
        const std::string tag = std::string(what) + " op " + std::to_string(i);
        int rc = validate(ops[i].x, ops[i].w, ops[i].y, 1, ops[i].n, ops[i].p, tag.c_str());
        if (rc) return rc;
        if (!extra) continue;
        const OpExtra &e = extra[i];
        const int64_t n = ops[i].n, p = ops[i].p, xb = 4 * n, yb = 4 * p;
        const bool whole = n % (kQuants * kGroupBlocks) == 0;   // rows of whole groups
        bool ok = e.mode == emode && e.out_mode == eout;
        if (e.mode == kXSiluUp) ok = ok && a16(e.x_up) && !overlaps(ops[i].y, yb, e.x_up, xb);
        else if (e.mode == kXNormAdd)   // (the writer of x_out needs a fast tile: p >= 8)
            ok = ok && a16(e.x_res) && a16(e.norm_w) && (!e.x_out || (a16(e.x_out) && p >= 8)) &&
                 !overlaps(ops[i].y, yb, e.x_res, xb) &&
                 !(e.x_out && (overlaps(e.x_out, xb, ops[i].x, xb) || overlaps(e.x_out, xb, e.x_res, xb) ||
                               overlaps(e.x_out, xb, ops[i].y, yb)));
        else if (e.mode == kXNormScale)
            ok = ok && whole && a16(e.psum) && !overlaps(ops[i].y, yb, e.psum, 4 * (n / kPsumRows));
        else ok = ok && e.mode == kXFloat;
        if (e.out_mode == kYResAdd) {
            const int64_t sb = 4 * (p / kPsumRows);
            ok = ok && whole && p % kPsumRows == 0 && a4(e.x_res) && a4(e.psum) && e.mode == kXFloat &&
                 !overlaps(ops[i].y, yb, e.x_res, yb) && !overlaps(e.psum, sb, ops[i].y, yb) &&
                 !overlaps(e.psum, sb, ops[i].x, xb) && !overlaps(e.psum, sb, e.x_res, yb) &&
                 (!e.x_out == !e.norm_w) &&
                 !(e.x_out && (!a4(e.x_out) || !a4(e.norm_w) || overlaps(e.x_out, yb, ops[i].x, xb) ||
                               overlaps(e.x_out, yb, ops[i].y, yb) || overlaps(e.x_out, yb, e.x_res, yb) ||
                               overlaps(e.x_out, yb, e.psum, sb)));
        }
        else if (e.out_mode == kYSwiGLU)
            ok = ok && whole && a16(e.w2) && (e.mode == kXFloat || e.mode == kXNormScale) &&
                 !overlaps(ops[i].y, yb, e.w2, w_bytes(n, p));
        else ok = ok && e.out_mode == kYPlain;
        if (!ok) return fail(Q8_ERR_INVALID_ARG, tag + ": extra inputs missing, misaligned, aliased or not "
                                                        "supported for this width");
    }
    return Q8_OK;
}

// The launches of a chain on a GPU of `cus` compute units: the op
// descriptors and tile tables of fused launches, and each launch with its
// kind, shape and grid (device pointers left unset).  Host only.
int plan_chain(const q8_0_op *ops, int64_t n_ops, uint32_t flags, const OpExtra *extra, int64_t cus,
               const char *what, ChainPlan &plan) {
    // Runs of mutually independent ops (or single ops).  Every plan
    // computes each op's outputs in the same fixed order, so the chain gives
    // the bits of standalone calls whatever the launch shapes.
    const int emode = extra ? extra[0].mode : kXFloat;
    const int xmode = (flags & Q8_CHAIN_XQ) ? kXQuant : emode;
    const int ymode = extra ? extra[0].out_mode : kYPlain;
    const bool per_op = (flags & Q8_CHAIN_PER_OP) != 0;
    const bool latency = (flags & Q8_CHAIN_SPLIT_K) != 0;
    const auto segs = chain_segments(ops, n_ops, per_op, extra);
    std::vector<OpDesc> &h_ops = plan.h_ops;
    std::vector<Tile> &h_tiles = plan.h_tiles;
    auto &info = plan.info;
    for (auto &sg : segs) {
        ChainPlan::SegInfo si;
        std::memset(&si, 0, sizeof si);
        si.first = sg.first;
        si.n = sg.second - sg.first;
        si.L.xmode = xmode;
        si.L.ymode = ymode;
        si.op0 = h_ops.size();
        si.tile0 = h_tiles.size();
        const auto ex = [&](int64_t i) { return extra ? &extra[i] : nullptr; };
        if (sg.second - sg.first == 1) {
            // one op: planned as a standalone call (a latency launch)
            const q8_0_op &o = ops[sg.first];
            OpDesc d = plan_op(o.x, o.w, o.y, 1, o.n, o.p, true, kWaves);
            set_extra(d, ex(sg.first));
            si.L.single = d;
            if (d.rs == 1) {
                si.L.kind = q8_0_chain::Launch::kSingleRc;
                si.L.single.w_once = 1;
                si.L.shape = plan_rc_latency(d.p, d.gsr, xmode, ymode, cus, true);
                si.L.grid = rc_tiles_for(d.p, si.L.shape);
            } else {
                si.L.kind = q8_0_chain::Launch::kSingleSuperrow;
                si.L.grid = tiles_of(d, kWaves);
            }
            info.push_back(si);
            continue;
        }
        // several independent ops in one launch
        bool all_rc = true, one_width = true;
        int64_t rows = 0;
        double wsum = 0.0, wg = 0.0;   // bytes, and bytes x groups per row
        for (int64_t i = sg.first; i < sg.second; ++i) {
            all_rc = all_rc && ops[i].n % (kQuants * kGroupBlocks) == 0;
            one_width = one_width && ops[i].n == ops[sg.first].n;
            rows += ops[i].p;
            const double bytes = (double)w_bytes(ops[i].n, ops[i].p);
            wsum += bytes;
            wg += bytes * (double)(ops[i].n / (kQuants * kGroupBlocks));
        }
        if (all_rc) {
            // SPLIT_K (ops that wait on the launch before): the latency plan
            // over all the launch's rows when they share a width; otherwise
            // the steady-state one-wave tiles, largest tiles first so that
            // the smallest finish the launch
            const bool lat = latency && one_width;
            const FusePlan fp = fuse_plan(xmode, wg / wsum);
            const RcShape sh = lat ? plan_rc_latency(rows, ops[sg.first].n / (kQuants * kGroupBlocks), xmode, ymode, cus, false)
                                   : fp.shape;
            struct Item { Tile t; int64_t bytes; };
            std::vector<Item> items;
            for (int64_t i = sg.first; i < sg.second; ++i) {
                const q8_0_op &o = ops[i];
                OpDesc d = plan_op(o.x, o.w, o.y, 1, o.n, o.p, false, 1);
                set_extra(d, ex(i));
                d.w_once = lat || fp.w_once ? 1 : 0;
                const uint32_t oi = (uint32_t)(h_ops.size() - si.op0);
                h_ops.push_back(d);
                const int64_t tb = (int64_t)(kWave / sh.c) * d.sr_bytes;
                const int64_t nt = rc_tiles_for(d.p, sh.c);
                for (int64_t t = 0; t < nt; ++t) items.push_back({{oi, (uint32_t)t}, tb});
            }
            if (!lat)
                std::stable_sort(items.begin(), items.end(),
                                 [](const Item &a, const Item &b) { return a.bytes > b.bytes; });
            for (auto &it : items) h_tiles.push_back(it.t);
            si.L.kind = q8_0_chain::Launch::kFusedRc;
            si.L.shape = sh;
            si.L.grid = (int64_t)items.size();
        } else {
            // widths that are not all multiples of 256: one-wave workgroups,
            // each tile in its own layout, largest tiles first (plain output)
            if (ymode != kYPlain)
                return fail(Q8_ERR_INVALID_ARG, std::string(what) + ": output modes need n % 256 == 0");
            struct Item { Tile t; int64_t bytes; };
            std::vector<Item> items;
            for (int64_t i = sg.first; i < sg.second; ++i) {
                const q8_0_op &o = ops[i];
                OpDesc d = plan_op(o.x, o.w, o.y, 1, o.n, o.p, false, 1);
                set_extra(d, ex(i));
                // rows of whole groups: the rows-and-group-slots tile of the
                // mixed launch (kMixC lanes per row, W loaded non-temporal);
                // others: 64 super-rows
                const bool rc = d.rs == 1;
                d.w_once = rc ? 1 : 0;
                const uint32_t oi = (uint32_t)(h_ops.size() - si.op0);
                h_ops.push_back(d);
                const int64_t nf = rc ? rc_tiles_for(d.p, kMixC) : d.fast_tiles;
                const int64_t fb = (rc ? kWave / kMixC : kWave) * d.sr_bytes;
                for (int64_t t = 0; t < nf; ++t) items.push_back({{oi, (uint32_t)t}, fb});
                const int64_t tt = tail_tiles_for((int64_t)d.p - d.tail_row0, 1);
                for (int64_t t = 0; t < tt; ++t)
                    items.push_back({{oi, (uint32_t)t | kTailBit}, (int64_t)d.nb * kBlockBytes});
            }
            std::stable_sort(items.begin(), items.end(),
                             [](const Item &a, const Item &b) { return a.bytes > b.bytes; });
            for (auto &it : items) h_tiles.push_back(it.t);
            si.L.kind = q8_0_chain::Launch::kFusedMixed;
            si.L.grid = (int64_t)items.size();
        }
        info.push_back(si);
    }
    return Q8_OK;
}
}  // namespace

int q8::chain_issue(const q8_0_chain *c, hipStream_t s) {
    for (const auto &L : c->launches) {
        hipError_t e = issue(L, s);
        if (e != hipSuccess) return fail_hip(e, "chain launch");
    }
    return Q8_OK;
}

std::vector<std::pair<int64_t, int64_t>> q8::chain_segments(const q8_0_op *ops, int64_t n_ops, bool per_op,
                                                            const OpExtra *extra) {
    std::vector<std::pair<int64_t, int64_t>> segs;
    if (per_op) {
        for (int64_t i = 0; i < n_ops; ++i) segs.push_back({i, i + 1});
        return segs;
    }
    int64_t b = 0;
    for (int64_t i = 1; i <= n_ops; ++i) {
        bool cut = (i == n_ops);
        for (int64_t j = b; !cut && j < i; ++j)
            cut = depends(ops[j], ops[i], extra ? &extra[j] : nullptr, extra ? &extra[i] : nullptr);
        if (cut) { segs.push_back({b, i}); b = i; }
    }
    return segs;
}

extern "C" {

int q8_0_chain_create(const q8_0_op *ops, int64_t n_ops, uint32_t flags, q8_0_chain **out) {
    return q8::chain_create_ex(ops, n_ops, flags, nullptr, out);
}

int q8_0_chain_plan(const q8_0_op *ops, int64_t n_ops, uint32_t flags, int64_t cus, q8_0_launch_plan *launches,
                    int64_t max_launches, int64_t *n_launches, int64_t *tile_op, uint32_t *tile_id,
                    int64_t max_tiles, int64_t *n_tiles) {
    if (!n_launches || !n_tiles) return fail(Q8_ERR_INVALID_ARG, "q8_0_chain_plan: n_launches and n_tiles are needed");
    *n_launches = 0;
    *n_tiles = 0;
    if (cus < 1 || cus > 4096) return fail(Q8_ERR_INVALID_ARG, "q8_0_chain_plan: cus must be in 1..4096");
    int rc = validate_chain(ops, n_ops, flags, nullptr, "q8_0_chain_plan");
    if (rc) return rc;
    ChainPlan plan;
    if ((rc = plan_chain(ops, n_ops, flags, nullptr, cus, "q8_0_chain_plan", plan))) return rc;
    *n_launches = (int64_t)plan.info.size();
    *n_tiles = (int64_t)plan.h_tiles.size();
    if (launches && max_launches >= *n_launches) {
        for (size_t k = 0; k < plan.info.size(); ++k) {
            const auto &si = plan.info[k];
            q8_0_launch_plan &o = launches[k];
            std::memset(&o, 0, sizeof o);
            o.first_op = si.first;
            o.n_ops = si.n;
            o.workgroups = si.L.grid;
            o.first_tile = -1;
            switch (si.L.kind) {
                case q8_0_chain::Launch::kSingleRc:
                    o.kind = Q8_LAUNCH_ROWS;
                    break;
                case q8_0_chain::Launch::kSingleSuperrow:
                    o.kind = Q8_LAUNCH_SUPERROWS;
                    o.waves = kWaves;
                    break;
                case q8_0_chain::Launch::kFusedRc:
                    o.kind = Q8_LAUNCH_FUSED;
                    o.first_tile = (int64_t)si.tile0;
                    break;
                case q8_0_chain::Launch::kFusedMixed:
                    o.kind = Q8_LAUNCH_FUSED_MIXED;
                    o.first_tile = (int64_t)si.tile0;
                    o.lanes_per_row = 1;   // rc tiles of one lane per row, one wave, two stages
                    o.waves = 1;
                    o.stages = 2;
                    break;
            }
            if (si.L.kind == q8_0_chain::Launch::kSingleRc || si.L.kind == q8_0_chain::Launch::kFusedRc) {
                o.lanes_per_row = si.L.shape.c;
                o.waves = si.L.shape.nwk;
                o.stages = si.L.shape.nst;
                o.tile_rows = rc_rows(si.L.shape);
            }
            if (si.L.kind == q8_0_chain::Launch::kFusedMixed) o.tile_rows = kWave;
        }
    }
    if (tile_op && tile_id && max_tiles >= *n_tiles) {
        for (const auto &si : plan.info) {
            if (si.L.kind != q8_0_chain::Launch::kFusedRc && si.L.kind != q8_0_chain::Launch::kFusedMixed) continue;
            for (int64_t g = 0; g < si.L.grid; ++g) {
                const Tile &t = plan.h_tiles[si.tile0 + g];
                tile_op[si.tile0 + g] = si.first + (int64_t)t.op;
                tile_id[si.tile0 + g] = t.tile;
            }
        }
    }
    return Q8_OK;
}

int q8_0_gemv_plan(int64_t n, int64_t p, int64_t cus, int *lanes_per_row, int *waves, int *stages,
                   int *tile_rows, int64_t *workgroups) {
    if (!lanes_per_row || !waves || !stages || !tile_rows || !workgroups)
        return fail(Q8_ERR_INVALID_ARG, "q8_0_gemv_plan: null output");
    if (n <= 0 || n % kQuants != 0 || n > Q8_MAX_N || p <= 0 || p > Q8_MAX_P)
        return fail(Q8_ERR_SHAPE, "q8_0_gemv_plan: shape out of range");
    if (cus < 1 || cus > 4096) return fail(Q8_ERR_INVALID_ARG, "q8_0_gemv_plan: cus must be in 1..4096");
    // (the plan reads only shapes; these pointers are never dereferenced)
    static const float kDummy[4] = {0.f, 0.f, 0.f, 0.f};
    OpDesc d = plan_op(kDummy, kDummy, nullptr, 1, n, p, true, kWaves);
    if (d.rs == 1) {
        const RcShape sh = plan_rc_latency(p, d.gsr, kXFloat, kYPlain, cus, true);
        *lanes_per_row = sh.c;
        *waves = sh.nwk;
        *stages = sh.nst;
        *tile_rows = rc_rows(sh);
        *workgroups = rc_tiles_for(p, sh);
    } else {
        *lanes_per_row = 0;
        *waves = kWaves;
        *stages = 0;
        *tile_rows = 0;
        *workgroups = tiles_of(d, kWaves);
    }
    return Q8_OK;
}

}  // extern "C"

int q8::chain_create_ex(const q8_0_op *ops, int64_t n_ops, uint32_t flags, const OpExtra *extra,
                        q8_0_chain **out) {
    if (!out) return fail(Q8_ERR_INVALID_ARG, "q8_0_chain_create: out is null");
    *out = nullptr;
    int rc = validate_chain(ops, n_ops, flags, extra, "q8_0_chain_create");
    if (rc) return rc;
    int dev = 0;
    if ((rc = check_device(&dev))) return rc;
    ChainPlan plan;
    if ((rc = plan_chain(ops, n_ops, flags, extra, cu_count(dev), "q8_0_chain_create", plan))) return rc;
    const std::vector<OpDesc> &h_ops = plan.h_ops;
    const std::vector<Tile> &h_tiles = plan.h_tiles;
    const auto &info = plan.info;

    q8_0_chain *c = new q8_0_chain();
    c->device = dev;
    c->flags = flags;
    c->ops.assign(ops, ops + n_ops);
    // device block: op descriptors, then tiles
    const size_t ob = h_ops.size() * sizeof(OpDesc);
    const size_t t_at = (ob + 255) / 256 * 256;
    const size_t total = h_tiles.empty() ? ob : t_at + h_tiles.size() * sizeof(Tile);
    if (total) {
        hipError_t e = hipMalloc(&c->d_table, total);
        if (e != hipSuccess) { chain_free(c); return fail_hip(e, "q8_0_chain_create hipMalloc"); }
        std::vector<char> host(total, 0);
        if (ob) std::memcpy(host.data(), h_ops.data(), ob);
        if (!h_tiles.empty()) std::memcpy(host.data() + t_at, h_tiles.data(), h_tiles.size() * sizeof(Tile));
        if ((e = hipMemcpy(c->d_table, host.data(), host.size(), hipMemcpyHostToDevice)) != hipSuccess) {
            chain_free(c);
            return fail_hip(e, "q8_0_chain_create hipMemcpy");
        }
    }
    const OpDesc *d_ops = (const OpDesc *)c->d_table;
    const Tile *d_tiles = (const Tile *)((const char *)c->d_table + t_at);
    for (auto &si : info) {
        q8_0_chain::Launch L = si.L;
        if (L.kind == q8_0_chain::Launch::kFusedRc || L.kind == q8_0_chain::Launch::kFusedMixed) {
            L.d_ops = d_ops + si.op0;
            L.d_tiles = d_tiles + si.tile0;
        }
        c->launches.push_back(L);
    }

    // ---- record one token into a graph on a private stream
    hipError_t e = hipStreamCreateWithFlags(&c->capture, hipStreamNonBlocking);
    if (e != hipSuccess) { chain_free(c); return fail_hip(e, "hipStreamCreateWithFlags"); }
    if ((e = hipStreamBeginCapture(c->capture, hipStreamCaptureModeThreadLocal)) != hipSuccess) {
        chain_free(c);
        return fail_hip(e, "hipStreamBeginCapture");
    }
    hipError_t le = hipSuccess;
    for (auto &L : c->launches)
        if (le == hipSuccess) le = issue(L, c->capture);
    e = hipStreamEndCapture(c->capture, &c->graph);
    if (le != hipSuccess) { chain_free(c); return fail_hip(le, "chain launch during capture"); }
    if (e != hipSuccess) { chain_free(c); return fail_hip(e, "hipStreamEndCapture"); }
    if ((e = hipGraphInstantiate(&c->exec, c->graph, nullptr, nullptr, 0)) != hipSuccess) {
        chain_free(c);
        return fail_hip(e, "hipGraphInstantiate");
    }
    *out = c;
    return Q8_OK;
}

extern "C" {

int q8_0_decode_chain(q8_0_chain *c, int mode, void *stream) {
    if (!c) return fail(Q8_ERR_INVALID_ARG, "q8_0_decode_chain: null chain");
    if (mode != Q8_MODE_GRAPH && mode != Q8_MODE_EAGER && mode != Q8_MODE_SYNC_EACH)
        return fail(Q8_ERR_INVALID_ARG, "q8_0_decode_chain: unknown mode");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    if (dev != c->device)
        return fail(Q8_ERR_INVALID_ARG, "q8_0_decode_chain: chain was created on device " +
                                            std::to_string(c->device) + ", current is " + std::to_string(dev));
    hipStream_t s = (hipStream_t)stream;
    // GRAPH: the recorded graph -- unless it holds one launch, which is issued
    // directly (replaying a one-node graph measured ~4 us slower than the
    // launch itself: 113.5 against 109.1 us per Qwen3-0.6B-shaped token)
    if (mode == Q8_MODE_GRAPH && c->launches.size() != 1) {
        if ((e = hipGraphLaunch(c->exec, s)) != hipSuccess) return fail_hip(e, "hipGraphLaunch");
        return Q8_OK;
    }
    for (auto &L : c->launches) {
        if ((e = issue(L, s)) != hipSuccess) return fail_hip(e, "chain launch");
        if (mode == Q8_MODE_SYNC_EACH && (e = hipStreamSynchronize(s)) != hipSuccess)
            return fail_hip(e, "hipStreamSynchronize");
    }
    return Q8_OK;
}

int q8_0_chain_launches(const q8_0_chain *c) {
    if (!c) return fail(Q8_ERR_INVALID_ARG, "q8_0_chain_launches: null chain");
    return (int)c->launches.size();
}

int q8_0_chain_destroy(q8_0_chain *c) {
    chain_free(c);
    return Q8_OK;
}

}  // extern "C"
