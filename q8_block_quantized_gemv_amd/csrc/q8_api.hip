// q8_api.hip -- the C ABI of include/q8gemv.h: validation, launch planning,
// decode chains (hipGraph record/replay) and the bounded stream wait.
#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
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

// Split-K workspace of the small-batch product, one per (device, stream):
// calls on one stream run in order and may share it; calls on different
// streams get different ones.  Grown on demand (hipFree synchronizes the
// device first), kept until the process ends.  The arrival counters are
// zeroed once here and left at zero by every launch.
struct Workspace {
    float *ws = nullptr;
    size_t ws_bytes = 0;
    uint32_t *cnt = nullptr;
    size_t cnt_n = 0;
};

int workspace_for(int dev, hipStream_t s, size_t ws_bytes, size_t cnt_n, float **ws_out,
                  uint32_t **cnt_out) {
    static std::mutex mu;
    static std::map<std::pair<int, hipStream_t>, Workspace> pool;
    std::lock_guard<std::mutex> lk(mu);
    Workspace &W = pool[{dev, s}];
    hipError_t e;
    if (W.ws_bytes < ws_bytes) {
        if (W.ws && (e = hipFree(W.ws)) != hipSuccess) return fail_hip(e, "hipFree");
        W.ws = nullptr;
        W.ws_bytes = 0;
        if ((e = hipMalloc(&W.ws, ws_bytes)) != hipSuccess) return fail_hip(e, "workspace hipMalloc");
        W.ws_bytes = ws_bytes;
    }
    if (W.cnt_n < cnt_n) {
        if (W.cnt && (e = hipFree(W.cnt)) != hipSuccess) return fail_hip(e, "hipFree");
        W.cnt = nullptr;
        W.cnt_n = 0;
        if ((e = hipMalloc(&W.cnt, cnt_n * sizeof(uint32_t))) != hipSuccess)
            return fail_hip(e, "counter hipMalloc");
        if ((e = hipMemset(W.cnt, 0, cnt_n * sizeof(uint32_t))) != hipSuccess ||
            (e = hipDeviceSynchronize()) != hipSuccess)
            return fail_hip(e, "counter hipMemset");
        W.cnt_n = cnt_n;
    }
    *ws_out = W.ws;
    *cnt_out = W.cnt;
    return Q8_OK;
}

}  // namespace q8

namespace {

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

// Kernel shape per launch kind.  Q8GEMV_VARIANT=nw<1|2|4>pf<1|2> (read at
// each planning call) overrides it for A/B measurements.
Variant pick_variant(bool fused) {
    Variant v = fused ? Variant{1, 1} : Variant{4, 1};
    if (const char *e = std::getenv("Q8GEMV_VARIANT")) {
        int nw = 0, pf = 0;
        if (std::sscanf(e, "nw%dpf%d", &nw, &pf) == 2 && (nw == 1 || nw == 2 || nw == 4) &&
            (pf == 1 || pf == 2))
            v = Variant{nw, pf};
    }
    return v;
}

// Waves that split one row tile's groups (ks <= nw).  A standalone launch
// wants many workgroups; inside a fused chain the other ops fill the GPU, so
// the choice only has to keep the waves of a workgroup evenly loaded.
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

// K slices across workgroups (SPLIT_K chains): up to `target` slices, at
// least one group each, at most kMaxSlices.  With one wave per row tile
// (ks == 1) the wave owns all kSlots slots and any run of groups can be a
// slice; with ks > 1 a slice holds a multiple of kSlots groups.
void plan_slices(OpDesc &d, int64_t target) {
    if (target <= 1 || d.gsr <= 1) return;
    const bool any_run = d.ks == 1;
    int64_t S = std::min<int64_t>(std::min<int64_t>(target, kMaxSlices), d.gsr);
    if (!any_run) S = std::min<int64_t>(S, (d.gsr + kSlots - 1) / kSlots);
    if (S <= 1) return;
    int64_t per = (d.gsr + S - 1) / S;
    if (!any_run) per = (per + kSlots - 1) / kSlots * kSlots;
    S = (d.gsr + per - 1) / per;
    if (S <= 1) return;
    d.slices = (int32_t)S;
    d.slice_groups = (int32_t)per;
}

OpDesc plan_op(const float *x, const void *w, float *y, int64_t m, int64_t n, int64_t p,
               bool standalone, int nw = kWaves, int64_t slices = 1) {
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
    d.ks = choose_ks(d.gsr, d.nsr, standalone, nw);
    d.slices = 1;
    d.slice_groups = d.gsr;
    plan_slices(d, slices);
    d.fast_tiles = (int32_t)fast_tiles_for(d.nsr, d.ks, nw, d.slices);
    d.tail_row0 = (int32_t)(d.nsr * rs);
    d.m = (int32_t)m;
    d.x_stride = n;
    d.y_stride = p;
    return d;
}

int64_t tiles_of(const OpDesc &d, int nw = kWaves) {
    return (int64_t)d.fast_tiles + tail_tiles_for((int64_t)d.p - d.tail_row0, nw);
}

int gemv_launch(const float *x, const void *w, float *y, int64_t n, int64_t p, hipStream_t s,
                bool xq = false) {
    const Variant v = pick_variant(false);
    const OpDesc d = plan_op(x, w, y, 1, n, p, true, v.nw);
    hipError_t e = launch_gemv_single(d, v, tiles_of(d, v.nw), s, xq ? kXQuant : kXFloat);
    if (e != hipSuccess) return fail_hip(e, xq ? "q8_0_gemv_q8q8 launch" : "q8_0_gemv launch");
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

int env_int(const char *name, int dflt) {
    const char *ev = std::getenv(name);
    return ev ? std::atoi(ev) : dflt;
}

// Stream-K split: up to `wpc` one-wave workgroups per CU, each an equal
// contiguous range of at least `min_items` (row tile, group) items, so that
// short ranges do not multiply the partial sums.  Sets fast_wgs and maxc
// and returns the bytes of partial slots the split needs.
size_t plan_streamk(GemmDesc &d, int dev, int wpc, int min_items) {
    wpc = std::max(1, env_int("Q8GEMV_SMALLM_WPC", wpc));
    min_items = std::max(1, env_int("Q8GEMV_SMALLM_MINIT", min_items));
    const int64_t items = (int64_t)d.row_tiles * d.gsr;
    const int64_t slots = (int64_t)wpc * cu_count(dev);
    const int64_t wgs = std::max<int64_t>(1, std::min({items, slots, items / min_items}));
    d.fast_wgs = (int32_t)wgs;
    // a row tile's contributors: at most ceil(G / per) + 1, per = items per workgroup
    const int64_t per = std::max<int64_t>(1, items / wgs);
    d.maxc = (int32_t)std::min<int64_t>(wgs, (d.gsr + per - 1) / per + 1);
    return (size_t)d.row_tiles * d.maxc * 16 * kWave * d.rs * sizeof(float);
}

// m = 2..4 rows on the vector units.
int smallm_valu(const float *X, const void *w, float *Y, int64_t m, int64_t n, int64_t p,
                hipStream_t s) {
    GemmDesc d = plan_gemm(X, w, Y, m, n, p);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    // as many workgroups per CU as their double-buffered stages fit in 160 KiB of LDS
    const int wpc = (160 * 1024) / gemm_valu_stage_bytes((int)m);
    const size_t part_bytes = plan_streamk(d, dev, wpc, 4);
    float *ws = nullptr;
    int rc = workspace_for(dev, s, std::max<size_t>(part_bytes, 256), (size_t)d.row_tiles, &ws, &d.cnt);
    if (rc) return rc;
    d.ws = ws;
    e = launch_gemm_valu(d, (int64_t)d.fast_wgs + (p - d.tail_row0), s);
    if (e != hipSuccess) return fail_hip(e, "q8_0_gemm_smallm launch");
    return Q8_OK;
}

// m = 2..3 rows where every row is one super-row: the vector units, lanes
// over (row, block pair); one launch, no split of X.
int smallm_vrow(const float *X, const void *w, float *Y, int64_t m, int64_t n, int64_t p,
                hipStream_t s) {
    GemmDesc d = plan_gemm(X, w, Y, m, n, p);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    const int wpc = (160 * 1024) / gemm_valu_stage_bytes((int)m);
    const size_t part_bytes = plan_streamk(d, dev, wpc, 4);
    float *ws = nullptr;
    int rc = workspace_for(dev, s, std::max<size_t>(part_bytes, 256), (size_t)d.row_tiles, &ws, &d.cnt);
    if (rc) return rc;
    d.ws = ws;
    // Two waves per workgroup share its stages, each taking half the rows of
    // every group: two waves per SIMD where one wave's stages fill a quarter
    // of the LDS (measured 5-10 % faster than one wave; four waves, held to
    // two per SIMD by their registers, slower).  Q8GEMV_SMALLM_VROW_NW=1
    // selects one wave for A/B runs.
    const int nw = env_int("Q8GEMV_SMALLM_VROW_NW", 2) == 1 ? 1 : 2;
    e = launch_gemm_vrow(d, nw, s);
    if (e != hipSuccess) return fail_hip(e, "q8_0_gemm_smallm launch");
    return Q8_OK;
}

// m = 2..16 rows on the matrix cores (rows of 1 or 2 per super-row).
int smallm_mfma(const float *X, const void *w, float *Y, int64_t m, int64_t n, int64_t p,
                hipStream_t s) {
    GemmDesc d = plan_gemm(X, w, Y, m, n, p);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    // four double-buffered one-wave workgroups fill a CU's LDS
    const size_t part_bytes = plan_streamk(d, dev, 4, 4);
    // workspace: the split X (3 KiB per block of 32 columns, 256-B aligned), then the
    // partial slots
    const size_t xs_bytes = ((size_t)(n / kQuants) * kXPartsBytesPerBlock + 255) / 256 * 256;
    float *ws = nullptr;
    int rc = workspace_for(dev, s, xs_bytes + part_bytes, (size_t)d.row_tiles, &ws, &d.cnt);
    if (rc) return rc;
    d.xs = (const bf16x8 *)ws;
    d.ws = (float *)((char *)ws + xs_bytes);
    e = launch_split_x(X, ws, (int)m, (int)n, s);
    if (e != hipSuccess) return fail_hip(e, "q8_0_gemm_smallm split launch");
    e = launch_gemm_mfma(d, (int64_t)d.fast_wgs + (p - d.tail_row0), s);
    if (e != hipSuccess) return fail_hip(e, "q8_0_gemm_smallm launch");
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
    return gemv_launch(x, w, y, n, p, (hipStream_t)stream);
}

int q8_0_gemv_q8q8(const float *x, const void *w, float *y, int64_t n, int64_t p, void *stream) {
    int rc = validate(x, w, y, 1, n, p, "q8_0_gemv_q8q8");
    if (rc) return rc;
    if ((rc = check_device())) return rc;
    return gemv_launch(x, w, y, n, p, (hipStream_t)stream, true);
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

int q8_0_gemm_smallm(const float *X, const void *w, float *Y, int64_t m, int64_t n, int64_t p,
                     void *stream) {
    int rc = validate(X, w, Y, m, n, p, "q8_0_gemm_smallm");
    if (rc) return rc;
    if ((rc = check_device())) return rc;
    hipStream_t s = (hipStream_t)stream;
    if (m == 1) return gemv_launch(X, w, Y, n, p, s);
    const int64_t rs = kGroupBlocks / gcd64(n / kQuants, kGroupBlocks);
    // m = 2..3 with rows of one super-row (n a multiple of 256) run on the
    // vector units with lanes over (row, block pair): each lane holds the x
    // values of its two blocks in registers, the quants are converted once
    // for all rows of X, and no split of X is needed (measured 16-24 % faster
    // than the matrix cores at m = 2 on the 7B shapes, 9-17 % at m = 3,
    // slower from m = 4).  Where rows fill super-rows of 1 or 2 (n a multiple
    // of 128) the matrix cores take the other m >= 2: on the vector units
    // with a lane per row, the x values every lane needs come through LDS
    // broadcast reads, m of them per quant and lane.  Other widths run on the
    // vector units with a lane per row, kValuMaxM rows of X per pass over W.
    // Q8GEMV_SMALLM_PATH=valu|mfma|vrow overrides.
    bool mfma = rs <= 2;
    bool vrow = rs == 1 && m <= kVrowMaxM;
    if (const char *ev = std::getenv("Q8GEMV_SMALLM_PATH")) {
        if (!std::strcmp(ev, "valu")) mfma = vrow = false;
        else if (!std::strcmp(ev, "mfma") && rs <= 2) mfma = true, vrow = false;
        else if (!std::strcmp(ev, "vrow")) vrow = rs == 1 && m <= kVrowMaxM;
    }
    if (vrow) return smallm_vrow(X, w, Y, m, n, p, s);
    if (mfma) return smallm_mfma(X, w, Y, m, n, p, s);
    // vector units: one pass over W per kValuMaxM rows of X
    for (int64_t i0 = 0; i0 < m; i0 += kValuMaxM) {
        const int64_t mi = std::min<int64_t>(kValuMaxM, m - i0);
        rc = mi == 1 ? gemv_launch(X + i0 * n, w, Y + i0 * p, n, p, s)
                     : smallm_valu(X + i0 * n, w, Y + i0 * p, mi, n, p, s);
        if (rc) return rc;
    }
    return Q8_OK;
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
        bool fused;
        bool sk;              // stream-K launch (d_ops, d_pieces, d_begin; d_tiles = tail tiles)
        bool phased;          // one launch of n_phases phases (d_phases, d_bar, d_err)
        int xmode;            // XMode: how the activations are read
        Variant v;
        OpDesc single;        // per-op launch
        const OpDesc *d_ops;  // fused launch
        const Tile *d_tiles;
        const Piece *d_pieces;
        const uint32_t *d_begin;
        int64_t n_sk;         // stream-K workgroups (the tail tiles' follow)
        const PhaseDesc *d_phases;
        int n_phases;
        uint32_t *d_sync;     // barrier state (kPhasedSyncBytes)
        uint32_t per, nx;     // workgroups per XCD, XCDs
        int64_t grid;
    };
    std::vector<Launch> launches;
    void *d_table = nullptr;
    uint32_t *d_err = nullptr;   // one-launch chains: the barrier timeout flag
    hipStream_t capture = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

namespace {

hipError_t issue(const q8_0_chain::Launch &L, hipStream_t s) {
    if (L.phased) return launch_gemv_phased(L.d_phases, L.n_phases, L.d_sync, L.per, L.nx, L.grid, L.v.pf, s);
    if (L.sk)
        return launch_gemv_streamk(L.d_ops, L.d_pieces, L.d_begin, L.d_tiles, L.n_sk, L.grid - L.n_sk,
                                   L.v.pf, s, L.xmode);
    if (L.fused) return launch_gemv_fused(L.d_ops, L.d_tiles, L.v, L.grid, s, L.xmode);
    return launch_gemv_single(L.single, L.v, L.grid, s, L.xmode);
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
    const void *r[5];
    int64_t rn[5];
    int nr = 0;
    const void *w[2];
    int64_t wn[2];
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
        rd(e->x_res, 4 * o.n);
        rd(e->norm_w, 4 * o.n);
        wr(e->x_out, 4 * o.n);
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

// How the one-launch kernel's `wgs` workgroups spread over the XCDs of
// device `dev`: a census launch of the same kernel and grid, once per
// (device, wgs).  Sets *per and *nx and returns true when every XCD holds
// the same number (the two-level barrier counts on it).
bool phased_split(int dev, int64_t wgs, uint32_t *per, uint32_t *nx) {
    static std::mutex mu;
    static std::map<std::pair<int, int64_t>, std::pair<uint32_t, uint32_t>> known;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_pair(dev, wgs);
    auto it = known.find(key);
    if (it == known.end()) {
        uint32_t p = 0, n = 0;
        uint32_t *d = nullptr;
        if (hipMalloc(&d, (size_t)wgs * sizeof(uint32_t)) == hipSuccess) {
            std::vector<uint32_t> h((size_t)wgs, 0xFFFFFFFFu);
            if (launch_gemv_phased_census(d, wgs, nullptr) == hipSuccess &&
                hipMemcpy(h.data(), d, h.size() * sizeof(uint32_t), hipMemcpyDeviceToHost) == hipSuccess) {
                std::map<uint32_t, int64_t> count;
                for (uint32_t x : h) count[x]++;
                bool even = !count.empty() && count.size() <= 16 && count.rbegin()->first < 16;
                for (auto &kv : count) even = even && kv.second * (int64_t)count.size() == wgs;
                if (even) { n = (uint32_t)count.size(); p = (uint32_t)(wgs / n); }
            }
            (void)hipFree(d);
        }
        it = known.emplace(key, std::make_pair(p, n)).first;
    }
    *per = it->second.first;
    *nx = it->second.second;
    return *nx > 0;
}

// Stream-K schedule of a launch's ops on `wgs` one-wave workgroups: all
// (op, row tile, group) items, in that order, are cut into wgs equal
// contiguous ranges (workgroup b takes [b*N/wgs, (b+1)*N/wgs)), and each
// range into pieces where it crosses a row tile.  The pieces of one row tile
// are numbered in workgroup order (their partial slots); maxc[i] is op i's
// largest number of pieces on one row tile.  begin holds wgs + 1 offsets.
void plan_pieces(const std::vector<OpDesc> &ds, int64_t wgs, std::vector<Piece> &pieces,
                 std::vector<uint32_t> &begin, std::vector<int32_t> &maxc) {
    const size_t n_ops = ds.size();
    std::vector<int64_t> off(n_ops + 1, 0);
    std::vector<std::vector<uint32_t>> count(n_ops);
    for (size_t i = 0; i < n_ops; ++i) {
        const int64_t tiles = ((int64_t)ds[i].nsr + kWave - 1) / kWave;
        off[i + 1] = off[i] + tiles * ds[i].gsr;
        count[i].assign((size_t)tiles, 0u);
    }
    const int64_t N = off[n_ops];
    pieces.clear();
    begin.assign((size_t)wgs + 1, 0u);
    size_t i = 0;
    for (int64_t b = 0; b < wgs; ++b) {
        begin[(size_t)b] = (uint32_t)pieces.size();
        int64_t lo = b * N / wgs;
        const int64_t hi = (b + 1) * N / wgs;
        while (lo < hi) {
            while (off[i + 1] <= lo) ++i;
            const int64_t G = ds[i].gsr;
            const int64_t local = lo - off[i];
            const int64_t tile = local / G;
            const int64_t g0 = local - tile * G;
            const int64_t g1 = std::min<int64_t>(G, g0 + (hi - lo));
            Piece pc;
            pc.op = (uint32_t)i;
            pc.tile = (uint32_t)tile;
            pc.g0 = (uint32_t)g0;
            pc.g1 = (uint32_t)g1;
            pc.slot = count[i][(size_t)tile]++;
            pc.nslots = 0;
            pieces.push_back(pc);
            lo += g1 - g0;
        }
    }
    begin[(size_t)wgs] = (uint32_t)pieces.size();
    maxc.assign(n_ops, 1);
    for (auto &pc : pieces) {
        pc.nslots = count[pc.op][pc.tile];
        maxc[pc.op] = std::max<int32_t>(maxc[pc.op], (int32_t)pc.nslots);
    }
}

// Does phase k (segment k) of a one-launch chain read memory that an earlier
// phase j read and a phase in [j, k) wrote?  Then a CU may still hold
// phase j's copy in its L1.  Ranges are widened to whole 128-byte lines.
bool phase_rereads(const q8_0_op *ops, const OpExtra *extra,
                   const std::vector<std::pair<int64_t, int64_t>> &segs, size_t k) {
    auto line = [](const void *p, int64_t n, uintptr_t &a, uintptr_t &b) {
        a = (uintptr_t)p & ~(uintptr_t)127;
        b = ((uintptr_t)p + (uintptr_t)n + 127) & ~(uintptr_t)127;
    };
    auto meet = [&](const void *p, int64_t n, const void *q, int64_t m) {
        uintptr_t a0, a1, b0, b1;
        line(p, n, a0, a1);
        line(q, m, b0, b1);
        return a0 < b1 && b0 < a1;
    };
    auto ex = [&](int64_t i) { return extra ? &extra[i] : nullptr; };
    if (segs.back().second > 512) return k > 0;   // long chains: every barrier acquires
    for (int64_t i = segs[k].first; i < segs[k].second; ++i) {
        const Ranges R = ranges_of(ops[i], ex(i));
        for (int r = 0; r < R.nr; ++r)
            for (size_t j = 0; j < k; ++j)
                for (int64_t a = segs[j].first; a < segs[j].second; ++a) {
                    const Ranges A = ranges_of(ops[a], ex(a));
                    for (int ra = 0; ra < A.nr; ++ra) {
                        if (!meet(R.r[r], R.rn[r], A.r[ra], A.rn[ra])) continue;
                        for (size_t w = j; w < k; ++w)
                            for (int64_t b = segs[w].first; b < segs[w].second; ++b) {
                                const Ranges B = ranges_of(ops[b], ex(b));
                                for (int wb = 0; wb < B.nw; ++wb)
                                    if (meet(R.r[r], R.rn[r], B.w[wb], B.wn[wb])) return true;
                            }
                    }
                }
    }
    return false;
}

void set_extra(OpDesc &d, const OpExtra *e) {
    if (!e) return;
    d.x_up = e->x_up;
    d.x_res = e->x_res;
    d.norm_w = e->norm_w;
    d.x_out = e->x_out;
    d.norm_eps = e->eps;
}

}  // namespace

int q8::chain_issue(const q8_0_chain *c, hipStream_t s) {
    for (const auto &L : c->launches) {
        hipError_t e = issue(L, s);
        if (e != hipSuccess) return fail_hip(e, "chain launch");
    }
    return Q8_OK;
}

extern "C" {

int q8_0_chain_create(const q8_0_op *ops, int64_t n_ops, uint32_t flags, q8_0_chain **out) {
    return q8::chain_create_ex(ops, n_ops, flags, nullptr, out);
}

}  // extern "C"

int q8::chain_create_ex(const q8_0_op *ops, int64_t n_ops, uint32_t flags, const OpExtra *extra,
                        q8_0_chain **out) {
    if (!out) return fail(Q8_ERR_INVALID_ARG, "q8_0_chain_create: out is null");
    *out = nullptr;
    if (!ops || n_ops <= 0 || n_ops > Q8_MAX_CHAIN_OPS)
        return fail(Q8_ERR_INVALID_ARG, "q8_0_chain_create: need 1..65535 ops");
    if (flags & ~(uint32_t)(Q8_CHAIN_PER_OP | Q8_CHAIN_SPLIT_K | Q8_CHAIN_XQ | Q8_CHAIN_ONE_LAUNCH))
        return fail(Q8_ERR_INVALID_ARG, "q8_0_chain_create: unknown flags");
    const bool one = (flags & Q8_CHAIN_ONE_LAUNCH) != 0;
    if (one && (flags & (Q8_CHAIN_XQ | Q8_CHAIN_PER_OP)))
        return fail(Q8_ERR_INVALID_ARG, "q8_0_chain_create: Q8_CHAIN_ONE_LAUNCH takes neither XQ nor PER_OP");
    const int emode = extra ? extra[0].mode : kXFloat;
    if (extra && (flags & Q8_CHAIN_XQ))
        return fail(Q8_ERR_INVALID_ARG, "q8_0_chain_create: these inputs have no integer form");
    auto a16 = [](const void *p) { return p && ((uintptr_t)p & 15u) == 0; };
    for (int64_t i = 0; i < n_ops; ++i) {
        const std::string what = "q8_0_chain_create op " + std::to_string(i);
        int rc = validate(ops[i].x, ops[i].w, ops[i].y, 1, ops[i].n, ops[i].p, what.c_str());
        if (rc) return rc;
        if (!extra) continue;
        const OpExtra &e = extra[i];
        const int64_t xb = 4 * ops[i].n, yb = 4 * ops[i].p;
        // one-launch chains take a mode per phase (kXFloat: none)
        bool ok = one || e.mode == emode;
        if (e.mode == kXFloat) ok = one;
        else if (e.mode == kXSiluUp) ok = ok && a16(e.x_up) && !overlaps(ops[i].y, yb, e.x_up, xb);
        else if (e.mode == kXNormAdd)   // (the writer of x_out needs a fast tile: p >= 8)
            ok = ok && a16(e.x_res) && a16(e.norm_w) && (!e.x_out || (a16(e.x_out) && ops[i].p >= 8)) &&
                 !overlaps(ops[i].y, yb, e.x_res, xb) &&
                 !(e.x_out && (overlaps(e.x_out, xb, ops[i].x, xb) || overlaps(e.x_out, xb, e.x_res, xb) ||
                               overlaps(e.x_out, xb, ops[i].y, yb)));
        else ok = false;
        if (!ok) return fail(Q8_ERR_INVALID_ARG, what + ": extra inputs missing, misaligned or aliased");
    }
    int dev = 0;
    int rc = check_device(&dev);
    if (rc) return rc;

    q8_0_chain *c = new q8_0_chain();
    c->device = dev;
    c->flags = flags;
    c->ops.assign(ops, ops + n_ops);

    // ---- plan: runs of mutually independent ops (or single ops)
    const bool per_op = (flags & Q8_CHAIN_PER_OP) != 0;
    const bool split = (flags & Q8_CHAIN_SPLIT_K) != 0;
    std::vector<std::pair<int64_t, int64_t>> segs;  // [begin, end)
    if (per_op) {
        for (int64_t i = 0; i < n_ops; ++i) segs.push_back({i, i + 1});
    } else {
        int64_t b = 0;
        for (int64_t i = 1; i <= n_ops; ++i) {
            bool cut = (i == n_ops);
            // (a one-launch chain's phase reads its activations in one mode)
            if (one && extra && extra[i].mode != extra[b].mode) cut = true;
            for (int64_t j = b; !cut && j < i; ++j)
                cut = depends(ops[j], ops[i], extra ? &extra[j] : nullptr, extra ? &extra[i] : nullptr);
            if (cut) { segs.push_back({b, i}); b = i; }
        }
    }

    // ---- fused segments: op table + tile schedule in one device block;
    // with SPLIT_K every op is planned like a standalone launch (four-wave
    // workgroups, groups split over the waves) and row-poor ops are split
    // across workgroups too, their partial sums in the same device block
    // SPLIT_K (ops that wait on each other).  Measured on the decode step's
    // shapes: while a launch's row tiles (64 super-rows) fit on the CUs, four-
    // wave workgroups splitting a tile's groups in LDS, with K further sliced
    // across workgroups until there is one workgroup per CU, are fastest (a
    // workgroup's stages fill a CU's LDS); launches with more row tiles than
    // CUs (an lm_head, a 7B gate|up) are fastest on unsplit one-wave tiles.
    const Variant v_single = pick_variant(false), v_fused = pick_variant(true);
    const int64_t cus = cu_count(dev);
    // Stream-K for split launches with more row tiles than CUs whose one-wave
    // tiles would leave a long tail (below):
    // Q8GEMV_STREAMK=0 turns it off, 2 uses it for every split launch (A/B
    // runs); Q8GEMV_SK_PF sets its groups in flight (1 or 2).
    const int sk_mode = env_int("Q8GEMV_STREAMK", 1);
    // Q8GEMV_SK_TAIL overrides the tail threshold below (0: every row-rich launch)
    const double sk_tail_groups = env_int("Q8GEMV_SK_TAIL", 4);
    const int sk_pf = env_int("Q8GEMV_SK_PF", 1) == 2 ? 2 : 1;
    // a one-launch chain: every phase stream-K on the same workgroups, as
    // many as the CUs hold at once (four one-wave workgroups fill a CU's LDS)
    // (where the census finds the workgroups unevenly spread over the XCDs,
    // the phases become launches of their own, planned like SPLIT_K)
    int64_t one_wgs = 0;
    uint32_t xcc_per = 0, xcc_n = 0;
    bool phased = false;
    if (one) {
        const int per_cu = std::min(4, gemv_phased_blocks_per_cu(1));
        if (per_cu < 1) { chain_free(c); return fail(Q8_ERR_HIP, "q8_0_chain_create: occupancy query failed"); }
        one_wgs = per_cu * cus;
        phased = phased_split(dev, one_wgs, &xcc_per, &xcc_n);
    }
    std::vector<OpDesc> h_ops;
    std::vector<Tile> h_tiles;
    std::vector<Piece> h_pieces;
    std::vector<uint32_t> h_begin;
    struct SegInfo {
        size_t op0, tile0;
        int64_t ntiles;
        bool fused;
        OpDesc single;
        Variant v;
        bool sk;
        size_t piece0, begin0;
        int64_t n_sk;
        int xmode;   // one-launch phases
    };
    std::vector<SegInfo> info;
    for (auto &sg : segs) {
        const bool fused = !per_op && (sg.second - sg.first > 1);
        int64_t target = 1;
        Variant v = fused ? v_fused : v_single;
        bool sk = false;
        if (phased) {
            sk = true;
            v = Variant{1, 1};
        } else if (split || one) {
            int64_t row_tiles = 0, tile_groups = 0;
            for (int64_t i = sg.first; i < sg.second; ++i) {
                const OpDesc d = plan_op(ops[i].x, ops[i].w, ops[i].y, 1, ops[i].n, ops[i].p, false, 1);
                row_tiles += d.fast_tiles;
                tile_groups = std::max<int64_t>(tile_groups, d.gsr);
            }
            if (row_tiles > cus) {
                v = Variant{1, 1};
            } else {
                v = Variant{kWaves, 1};
                target = std::max<int64_t>(1, cus / std::max<int64_t>(1, row_tiles));
            }
            // Row-rich launches: one-wave tiles, four per CU, run in waves of
            // 4 * cus tiles; the last wave's idle slots cost (ceil(w) - w)
            // tile times, w = row_tiles / (4 * cus).  Stream-K spreads the
            // (tile, group) items evenly but pays partial sums where tiles
            // are shared.  It is taken where the one-wave tail would idle
            // the slots for at least sk_tail_groups group times (measured:
            // the 7B gate|up, 592 tiles of 14 groups, 5.9 group times, and
            // lm_head, 2376 of 14, 9.5, are faster on stream-K; the 0.6B
            // lm_head, 2374 tiles of 4 groups, 2.7, is 5 us faster on tiles).
            const double waves = (double)row_tiles / (double)(4 * cus);
            const double tail_groups = (std::ceil(waves) - waves) * (double)tile_groups;
            sk = sk_mode == 2 || (sk_mode == 1 && row_tiles > cus && tail_groups >= sk_tail_groups);
            // A/B overrides: Q8GEMV_SPLIT_SLICES (slices per row tile), Q8GEMV_VARIANT
            if (const int forced = env_int("Q8GEMV_SPLIT_SLICES", 0); forced > 0) target = forced;
            if (std::getenv("Q8GEMV_VARIANT")) v = v_single;
            if (sk) v = Variant{1, sk_pf};
        }
        // four-wave split workgroups take the standalone K split inside the workgroup
        const bool standalone = (!(split || one) && !fused) || ((split || one) && v.nw > 1);
        SegInfo si{h_ops.size(), h_tiles.size(), 0, fused, OpDesc{}, v, sk, h_pieces.size(), h_begin.size(), 0,
                   extra ? extra[sg.first].mode : kXFloat};
        if (sk) {
            // one-wave workgroups, four per CU (their two stages fill its LDS),
            // each at least kSkMinItems (row tile, group) items
            constexpr int64_t kSkMinItems = 2;
            std::vector<OpDesc> ds;
            int64_t items = 0;
            for (int64_t i = sg.first; i < sg.second; ++i) {
                const q8_0_op &o = ops[i];
                OpDesc d = plan_op(o.x, o.w, o.y, 1, o.n, o.p, false, 1);
                set_extra(d, extra ? &extra[i] : nullptr);
                items += (int64_t)d.fast_tiles * d.gsr;
                ds.push_back(d);
            }
            const int64_t wgs = std::min<int64_t>(phased ? one_wgs : 4 * cus, std::max<int64_t>(1, items / kSkMinItems));
            std::vector<Piece> pcs;
            std::vector<uint32_t> bg;
            std::vector<int32_t> maxc;
            plan_pieces(ds, items > 0 ? wgs : 0, pcs, bg, maxc);
            for (size_t i = 0; i < ds.size(); ++i) {
                if (maxc[i] > 1) ds[i].sk_slots = maxc[i];
                h_ops.push_back(ds[i]);
                const int64_t tt = tail_tiles_for((int64_t)ds[i].p - ds[i].tail_row0, 1);
                for (int64_t t = 0; t < tt; ++t) h_tiles.push_back({(uint32_t)i, (uint32_t)t | kTailBit});
            }
            h_pieces.insert(h_pieces.end(), pcs.begin(), pcs.end());
            h_begin.insert(h_begin.end(), bg.begin(), bg.end());
            si.n_sk = items > 0 ? wgs : 0;
            si.ntiles = (int64_t)(h_tiles.size() - si.tile0);
        } else if (fused) {
            // tiles sorted by decreasing weight bytes so that the smallest
            // tiles finish the launch (ties keep encode order)
            struct Item { Tile t; int64_t bytes; };
            std::vector<Item> items;
            for (int64_t i = sg.first; i < sg.second; ++i) {
                const q8_0_op &o = ops[i];
                OpDesc d = plan_op(o.x, o.w, o.y, 1, o.n, o.p, standalone, v.nw, target);
                set_extra(d, extra ? &extra[i] : nullptr);
                const uint32_t oi = (uint32_t)(h_ops.size() - si.op0);
                h_ops.push_back(d);
                const int64_t fb = (int64_t)(v.nw / d.ks) * kWave *
                                   (d.slices > 1 ? (int64_t)d.slice_groups * kGroupBytes : d.sr_bytes);
                for (int64_t t = 0; t < d.fast_tiles; ++t) items.push_back({{oi, (uint32_t)t}, fb});
                const int64_t tt = tail_tiles_for((int64_t)d.p - d.tail_row0, v.nw);
                for (int64_t t = 0; t < tt; ++t)
                    items.push_back({{oi, (uint32_t)t | kTailBit}, (int64_t)v.nw * d.nb * kBlockBytes});
            }
            std::stable_sort(items.begin(), items.end(),
                             [](const Item &a, const Item &b) { return a.bytes > b.bytes; });
            for (auto &it : items) h_tiles.push_back(it.t);
            si.ntiles = (int64_t)items.size();
        } else {
            const q8_0_op &o = ops[sg.first];
            si.single = plan_op(o.x, o.w, o.y, 1, o.n, o.p, standalone, v.nw, target);
            set_extra(si.single, extra ? &extra[sg.first] : nullptr);
        }
        info.push_back(si);
    }
    // device block: op descriptors, tiles, pieces, piece offsets, then the
    // K-split partials and counters
    auto up256 = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t ob = h_ops.size() * sizeof(OpDesc);
    const size_t tb = h_tiles.size() * sizeof(Tile);
    const size_t pb = h_pieces.size() * sizeof(Piece);
    const size_t bb = h_begin.size() * sizeof(uint32_t);
    const size_t t_at = ob, p_at = up256(ob + tb), b_at = up256(p_at + pb);
    // one-launch chains: the phase table, a barrier counter per phase, the
    // timeout flag
    const size_t nph = phased ? segs.size() : 0;
    const size_t ph_at = up256(b_at + bb), sync_at = up256(ph_at + nph * sizeof(PhaseDesc));
    size_t wb = phased ? up256(sync_at + kPhasedSyncBytes) : up256(b_at + bb);   // running end of the block
    std::vector<std::pair<OpDesc *, size_t>> ws;  // (op, offset of its partials)
    auto part_bytes = [](const OpDesc &d) {
        return (size_t)std::max(d.slices, d.sk_slots) * d.nsr * d.rs * sizeof(float);
    };
    auto reserve = [&](OpDesc &d) {
        if (d.slices <= 1 && d.sk_slots <= 1) return;
        ws.push_back({&d, wb});
        const size_t cnt = (size_t)((d.nsr + kWave - 1) / kWave) * sizeof(uint32_t);
        wb += up256(part_bytes(d)) + up256(cnt);
    };
    for (auto &d : h_ops) reserve(d);
    for (auto &si : info)
        if (!si.fused && !si.sk) reserve(si.single);
    const size_t total = wb;
    if (total) {
        hipError_t e = hipMalloc(&c->d_table, total);
        if (e != hipSuccess) { chain_free(c); return fail_hip(e, "q8_0_chain_create hipMalloc"); }
        char *base = (char *)c->d_table;
        for (auto &pw : ws) {
            OpDesc &d = *pw.first;
            d.part = (float *)(base + pw.second);
            d.cnt = (uint32_t *)(base + pw.second + up256(part_bytes(d)));
        }
        std::vector<char> host(total, 0);   // counters start at zero
        if (ob) std::memcpy(host.data(), h_ops.data(), ob);
        if (tb) std::memcpy(host.data() + t_at, h_tiles.data(), tb);
        if (pb) std::memcpy(host.data() + p_at, h_pieces.data(), pb);
        if (bb) std::memcpy(host.data() + b_at, h_begin.data(), bb);
        for (size_t k = 0; k < nph; ++k) {
            PhaseDesc ph;
            std::memset(&ph, 0, sizeof ph);
            ph.ops = (const OpDesc *)base + info[k].op0;
            ph.pieces = (const Piece *)(base + p_at) + info[k].piece0;
            ph.begin = (const uint32_t *)(base + b_at) + info[k].begin0;
            ph.tails = (const Tile *)(base + t_at) + info[k].tile0;
            ph.n_sk = (int32_t)info[k].n_sk;
            ph.n_tail = (int32_t)info[k].ntiles;
            ph.xmode = info[k].xmode;
            ph.acquire = phase_rereads(ops, extra, segs, k) ? 1 : 0;
            std::memcpy(host.data() + ph_at + k * sizeof(PhaseDesc), &ph, sizeof ph);
        }
        if ((e = hipMemcpy(c->d_table, host.data(), host.size(), hipMemcpyHostToDevice)) != hipSuccess) {
            chain_free(c);
            return fail_hip(e, "q8_0_chain_create hipMemcpy");
        }
    }
    const OpDesc *d_ops = (const OpDesc *)c->d_table;
    const Tile *d_tiles = (const Tile *)((const char *)c->d_table + t_at);
    const Piece *d_pieces = (const Piece *)((const char *)c->d_table + p_at);
    const uint32_t *d_begin = (const uint32_t *)((const char *)c->d_table + b_at);
    if (phased) {
        q8_0_chain::Launch L;
        std::memset(&L, 0, sizeof L);
        L.phased = true;
        L.v = Variant{1, 1};
        L.d_phases = (const PhaseDesc *)((const char *)c->d_table + ph_at);
        L.n_phases = (int)nph;
        L.d_sync = (uint32_t *)((char *)c->d_table + sync_at);
        L.per = xcc_per;
        L.nx = xcc_n;
        L.grid = one_wgs;
        c->d_err = L.d_sync + kPhasedSyncErr;
        c->launches.push_back(L);
    }
    for (size_t k = 0; k < segs.size() && !phased; ++k) {
        q8_0_chain::Launch L;
        std::memset(&L, 0, sizeof L);
        L.xmode = (flags & Q8_CHAIN_XQ) ? kXQuant : info[k].xmode;
        L.v = info[k].v;
        if (info[k].sk) {
            L.sk = true;
            L.d_ops = d_ops + info[k].op0;
            L.d_tiles = d_tiles + info[k].tile0;
            L.d_pieces = d_pieces + info[k].piece0;
            L.d_begin = d_begin + info[k].begin0;
            L.n_sk = info[k].n_sk;
            L.grid = info[k].n_sk + info[k].ntiles;
        } else if (info[k].fused) {
            L.fused = true;
            L.d_ops = d_ops + info[k].op0;
            L.d_tiles = d_tiles + info[k].tile0;
            L.grid = info[k].ntiles;
        } else {
            L.fused = false;
            L.single = info[k].single;
            L.grid = tiles_of(L.single, L.v.nw);
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
    if (mode == Q8_MODE_GRAPH) {
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

int q8_0_chain_check(const q8_0_chain *c) {
    if (!c) return fail(Q8_ERR_INVALID_ARG, "q8_0_chain_check: null chain");
    if (!c->d_err) return Q8_OK;
    uint32_t err = 0;
    const hipError_t e = hipMemcpy(&err, c->d_err, sizeof err, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail_hip(e, "q8_0_chain_check hipMemcpy");
    if (err) return fail(Q8_ERR_TIMEOUT, "q8_0_chain_check: a barrier wait of the one-launch chain gave up");
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
