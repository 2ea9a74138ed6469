// q8_step.h -- the decode-step kernels' descriptors and launchers (q8_step.hip),
// shared with the host side of the library.
#pragma once

#include "q8_internal.h"

namespace q8 {

// Cached rows per attention workgroup; a head's rows [0, seq) are split into
// ceil(seq / kAttnChunk) chunks whose partial softmaxes are merged in order.
constexpr int kAttnChunk = 128;
// contexts of at most kAttnShort rows are one chunk of a body sized for them
constexpr int kAttnShort = 32;

struct AttnDesc {
    const float *q;      // n_heads x head_dim
    const float *kc;     // cache rows of kv_width floats
    const float *vc;
    float *out;          // n_heads x head_dim
    const int *pos_dev;  // if set, seq = min(*pos_dev + 1, seq) (a recorded step); else seq
    float *ws;           // n_heads * max_chunks * (head_dim + 2) floats
    uint32_t *cnt;       // n_heads arrival counters, zero between launches
    int seq, kv_width, head_dim, n_heads, kv_group, max_chunks;
};

// The step's per-head q/k work folded into attention (see k_attention):
// raw q (n_heads heads), k and v (KV heads) of this token, the norm gains,
// and the caches to store the token's row into (the same as AttnDesc's).
struct AttnFuse {
    const float *q, *k, *v;
    const float *q_norm, *k_norm;
    float *kc_w, *vc_w;
    float eps, theta;
    // (cos, sin) of every rotation angle, [position][pair], as
    // launch_rope_table leaves them (required)
    const double2 *rope;
};

struct ArgmaxDesc {
    const float *x;
    int64_t n;
    uint32_t *out;       // the winning index (0xFFFFFFFF if every value is NaN)
    float *ws_val;       // one (value, index) per workgroup
    uint32_t *ws_idx;
    uint32_t *cnt;       // arrival counter, zero between launches
    int *pos_dev;        // if set, incremented once the index is written
};

// (cos, sin) of pos * theta^(-i / half) for every pos < rows and i < half,
// computed exactly as the rotation kernels compute them, into t[pos][i]
hipError_t launch_rope_table(double2 *t, int rows, int half, float theta, hipStream_t s);

// pos_dev, when not null, overrides pos (a recorded step reads it per replay)
hipError_t launch_rms_norm(const float *x, const float *w, float *out, int dim, int rows, float eps,
                           hipStream_t s);
hipError_t launch_rope(float *x, int head_dim, int heads, const int *pos_dev, int pos, float theta,
                       hipStream_t s);
// rows: the caches' length; a position at or past it writes nothing.
hipError_t launch_append_kv(const float *k, const float *v, float *kc, float *vc, int width,
                            const int *pos_dev, int pos, int rows, hipStream_t s);
// head_dim 64, 128, 192 or 256; q, kc, vc 16-byte aligned, kv_width % 4 == 0
hipError_t launch_attention(const AttnDesc &d, hipStream_t s);
// The recorded token's attention: d.q is unused (the query comes raw from
// f.q); needs d.pos_dev.  Also stores the token's K/V row into the caches.
hipError_t launch_attention_fused(const AttnDesc &d, const AttnFuse &f, hipStream_t s);
hipError_t launch_add(float *x, const float *y, int n, hipStream_t s);
hipError_t launch_silu(const float *g, const float *u, float *out, int n, hipStream_t s);
hipError_t launch_argmax(const ArgmaxDesc &d, int wgs, hipStream_t s);
// x = row *token of table (zeros if *token >= vocab), then xn = rms_norm(x) * w
hipError_t launch_embed_rms(const float *table, const uint32_t *token, uint32_t vocab, float *x,
                            const float *w, float *xn, int dim, float eps, hipStream_t s);
// *pos_dev = pos, *token_dev = token, ordered on s (a kernel, so it may be recorded).
hipError_t launch_set_state(int *pos_dev, uint32_t *token_dev, int pos, uint32_t token, hipStream_t s);

}  // namespace q8
