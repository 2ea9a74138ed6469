// q8_host.h -- host-side helpers shared by the library's entry points
// (q8_api.hip, q8_step_api.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <utility>
#include <vector>

#include "q8gemv.h"

#define Q8_HIDDEN __attribute__((visibility("hidden")))

namespace q8 {

// Record `msg` as this thread's last error and return `code`.
Q8_HIDDEN int fail(int code, const std::string &msg);
Q8_HIDDEN int fail_hip(hipError_t e, const char *where);
Q8_HIDDEN bool overlaps(const void *a, int64_t na, const void *b, int64_t nb);
// The current device exists and is gfx950 (Q8_OK), else a status.
Q8_HIDDEN int check_device(int *dev_out = nullptr);
Q8_HIDDEN int cu_count(int dev);
// A scratch buffer of at least ws_bytes and cnt_n zeroed counters for
// stream s on device dev, kept across calls (grown when too small).
Q8_HIDDEN int workspace_for(int dev, hipStream_t s, size_t ws_bytes, size_t cnt_n, float **ws_out,
                            uint32_t **cnt_out);
// Per-op inputs of the decode step's chains (internal): how the op reads its
// activations (XMode) and the extra vectors that takes, n floats each,
// 16-byte aligned.
struct OpExtra {
    int mode = 0;                  // kXSiluUp or kXNormAdd, the same for every op of a chain
    const float *x_up = nullptr;   // kXSiluUp: input silu(x) * x_up
    const float *x_res = nullptr;  // kXNormAdd: input rms_norm(x + x_res) * norm_w
    const float *norm_w = nullptr;
    float *x_out = nullptr;        // kXNormAdd: x + x_res written here (may be null)
    float eps = 0.f;
};
// q8_0_chain_create with per-op extras (null: plain ops).
Q8_HIDDEN int chain_create_ex(const q8_0_op *ops, int64_t n_ops, uint32_t flags,
                              const OpExtra *extra, q8_0_chain **out);
// The launches of a chain before planning: maximal runs [begin, end) of
// ops that do not depend on one another (one op per run with per_op).
Q8_HIDDEN std::vector<std::pair<int64_t, int64_t>> chain_segments(const q8_0_op *ops, int64_t n_ops,
                                                                  bool per_op, const OpExtra *extra);
// Issue a chain's launches on s, without its graph.
Q8_HIDDEN int chain_issue(const q8_0_chain *c, hipStream_t s);

}  // namespace q8
