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
// Per-op inputs and outputs of the decode step's chains (internal): how
// the op reads its activations (XMode) and writes its result (YMode), and
// the extra vectors those take (n floats each for the inputs, 16-byte
// aligned).  Every op of one chain reads and writes in the same modes.
struct OpExtra {
    int mode = 0;                  // XMode: kXSiluUp, kXNormAdd or kXNormScale (kXFloat: none)
    int out_mode = 0;              // YMode: kYResAdd or kYSwiGLU (kYPlain: none)
    const float *x_up = nullptr;   // kXSiluUp: input silu(x) * x_up
    const float *x_res = nullptr;  // kXNormAdd: input rms_norm(x + x_res) * norm_w;
                                   // kYResAdd: output x_res + W x (p floats)
    const float *norm_w = nullptr; // kXNormAdd: the gain (n floats); kYResAdd: the gain for x_out (p)
    float *x_out = nullptr;        // kXNormAdd: x + x_res written here; kYResAdd: y * norm_w (may be null)
    float eps = 0.f;               // kXNormAdd, kXNormScale
    float *psum = nullptr;         // kYResAdd: p/16 block sums of y^2 out; kXNormScale: n/16 in
                                   // (kXNormScale: x is the producer's x_out, gain already applied)
    const void *w2 = nullptr;      // kYSwiGLU: the up matrix (as w); y = silu(W x) * (W2 x)
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
