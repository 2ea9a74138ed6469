/*
 * q8step.h -- C ABI of the rest of a Q8_0 decode step on MI355X (gfx950).
 *
 * The page "IV.4: One command buffer per token" (section "Eight kernels")
 * defines, next to q8_matvec, the seven kernels one decode step needs, and
 * its section "One command buffer" wires them into the step of a
 * Qwen3-style model.  This header exposes each kernel on its own and the
 * whole step recorded once and replayed per token.
 *
 * Conventions are those of q8gemv.h: device pointers owned by the caller,
 * `stream` a hipStream_t as void* (NULL = the legacy default stream),
 * arguments validated before anything is enqueued (negative q8_status on
 * failure, detail in q8_0_last_error()), asynchronous calls, no fallback.
 * Float data is float32 and 4-byte aligned.
 */
#ifndef Q8STEP_H
#define Q8STEP_H

#include <stdint.h>

#include "q8gemv.h"

#ifdef __cplusplus
extern "C" {
#endif

#define Q8_MAX_HEAD_DIM 256    /* head_dim is 64, 128, 192 or 256 */
#define Q8_MAX_SEQ 65536       /* cached positions an attention call may read */

/*
 * rms_norm_row: for each of `rows` rows of x (rows x dim, row-major)
 *   out = x * (sum_i x_i^2 / dim + eps)^(-1/2) * w      (w: dim floats)
 * out may equal x (in place); otherwise they must not overlap.
 * The layer norms use rows = 1; the per-head q/k norms rows = heads,
 * dim = head_dim.  1 <= dim <= 65536, 1 <= rows <= 65536.
 */
Q8_API int q8_0_rms_norm(const float *x, const float *w, float *out, int64_t dim, int64_t rows,
                  float eps, void *stream);

/*
 * rope_row, in place: in each of `heads` heads of x (heads x head_dim), the
 * pair (x[i], x[i + head_dim/2]) is turned by the angle
 * pos * theta^(-i / (head_dim/2)) (angle, sine and cosine in double
 * precision; the result rounds once to float).  head_dim even, <= 65536;
 * 0 <= pos < 2^31; theta > 0.
 */
Q8_API int q8_0_rope(float *x, int64_t head_dim, int64_t heads, int64_t pos, float theta, void *stream);

/*
 * append_kv: row `pos` of the caches (kc, vc: rows of `width` floats, at
 * least pos + 1 rows) becomes k (resp. v).
 */
Q8_API int q8_0_append_kv(const float *k, const float *v, float *kc, float *vc, int64_t width,
                   int64_t pos, void *stream);

/*
 * attention_decode: for query head h (q: n_heads x head_dim) on KV head
 * h / kv_group (row t of the caches holds all KV heads, kv_width floats):
 *   out[h] = sum_{t < seq} softmax_t(q_h . k_t / sqrt(head_dim)) v_t
 * n_heads a multiple of kv_group; kv_width >= (n_heads / kv_group) *
 * head_dim and a multiple of 4; q, kc and vc 16-byte aligned (Q8_ERR_ALIGN
 * otherwise); 1 <= seq <= Q8_MAX_SEQ.  workspace: a 256-byte aligned device
 * buffer of at least q8_0_attention_workspace's bytes, not overlapping q or
 * out, its contents before the call immaterial (the chunks' partial
 * softmaxes and arrival counters).  Bitwise reproducible for the same inputs
 * and shape.
 */
Q8_API int q8_0_attention_decode(const float *q, const float *kc, const float *vc, float *out,
                          int64_t seq, int64_t kv_width, int64_t head_dim, int64_t n_heads,
                          int64_t kv_group, void *workspace, size_t workspace_bytes, void *stream);

/* *bytes = the workspace q8_0_attention_decode needs (host only). */
Q8_API int q8_0_attention_workspace(int64_t seq, int64_t head_dim, int64_t n_heads, size_t *bytes);

/* add_inplace: x[i] += y[i] for i < n. */
Q8_API int q8_0_add_inplace(float *x, const float *y, int64_t n, void *stream);

/* silu_hadamard: out[i] = gate[i] / (1 + e^-gate[i]) * up[i] for i < n. */
Q8_API int q8_0_silu_hadamard(const float *gate, const float *up, float *out, int64_t n, void *stream);

/*
 * argmax_row: *out (device uint32) = the index of the largest of x[0..n):
 * ties to the lowest index, NaN never wins, 0xFFFFFFFF if every value is
 * NaN.  Exact.  workspace: a 256-byte aligned device buffer of at least
 * q8_0_argmax_workspace's bytes, not overlapping x or out, its contents
 * before the call immaterial (the workgroups' winners and a counter).
 */
Q8_API int q8_0_argmax(const float *x, int64_t n, uint32_t *out, void *workspace,
                       size_t workspace_bytes, void *stream);

/* *bytes = the workspace q8_0_argmax needs (host only). */
Q8_API int q8_0_argmax_workspace(int64_t n, size_t *bytes);

/*
 * A whole decode step of a Qwen3-style model (section "One command buffer"):
 *   x = embed[token]
 *   per layer: xn = rms_norm(x, attn_norm); q, k, v = Wq xn, Wk xn, Wv xn;
 *     q, k = per-head rms_norm(q, q_norm), (k, k_norm); rope(q), rope(k) at
 *     pos; append k, v at pos; a = attention(q, caches, seq = pos + 1);
 *     x += Wo a; xn = rms_norm(x, ffn_norm); h = silu(Wgate xn) * (Wup xn);
 *     x += Wdown h
 *   logits = lm_head rms_norm(x, out_norm); token = argmax(logits); pos += 1
 * Independent matvecs (q, k, v; gate, up) share one fused launch, and the
 * small kernels are fused where one feeds the next: the embedding row with
 * the first norm, each residual add with the norm after it, the per-head
 * q/k norms with the rotary embedding and the cache append, and argmax with
 * the position advance.  A token is 5 n_layers + 3 launches.  Every matvec
 * launch is planned for latency (Q8_CHAIN_SPLIT_K); its outputs are bitwise
 * those of q8_0_gemv on the same inputs.
 */
typedef struct q8_0_layer_w {
    const void *wq, *wk, *wv, *wo;   /* Q8_0, 16-B aligned, as q8_0_gemv's w */
    const void *wgate, *wup, *wdown;
    const float *attn_norm, *ffn_norm;   /* hidden floats, 16-B aligned */
    const float *q_norm, *k_norm;        /* head_dim floats */
} q8_0_layer_w;

typedef struct q8_0_model {
    int64_t n_layers, hidden, n_heads, n_kv_heads, head_dim, inter, vocab, max_seq;
    float eps, theta;
    const float *embed;       /* vocab x hidden, 16-B aligned */
    const float *out_norm;    /* hidden, 16-B aligned */
    const void *lm_head;      /* Q8_0, vocab rows of hidden */
    const q8_0_layer_w *layers;   /* n_layers entries, copied at create */
} q8_0_model;

typedef struct q8_0_step q8_0_step; /* opaque */

/*
 * Validate the model, allocate the step's device state (activations, the
 * KV caches: n_layers x max_seq x n_kv_heads*head_dim floats each for K
 * and V, the rotation angles' (cos, sin) as doubles for every position and
 * pair: max_seq x head_dim/2 x 16 bytes, workspaces, the position and token
 * words) and record one token's launches into a hipGraph.  Weight pointers are baked into the recording
 * and must stay valid until q8_0_step_destroy.  The position starts at 0
 * and the token at 0.  max_seq <= Q8_MAX_SEQ.
 */
Q8_API int q8_0_step_create(const q8_0_model *m, q8_0_step **out);

/* Set the position and the input token (ordered on `stream`). */
Q8_API int q8_0_step_reset(q8_0_step *s, int64_t pos, uint32_t token, void *stream);

/*
 * One token on `stream`: mode Q8_MODE_GRAPH (replay the recording) or
 * Q8_MODE_EAGER (issue the same launches).  Reads the token and position
 * the previous step (or q8_0_step_reset) left on the device, writes the next
 * token there and advances the position; refuses to run past max_seq (the
 * check uses the host's count of steps since the last reset).
 */
Q8_API int q8_0_step_run(q8_0_step *s, int mode, void *stream);

/* Kernel launches one token costs. */
Q8_API int q8_0_step_launches(const q8_0_step *s);


/* Device buffers of the step, for reading results. */
typedef struct q8_0_step_bufs {
    const uint32_t *token;   /* the last argmax */
    const int32_t *pos;      /* the next position */
    const float *x;          /* hidden: the residual stream after the last layer */
    const float *logits;     /* vocab */
    const float *k_cache, *v_cache;   /* n_layers x max_seq x kv_width each */
} q8_0_step_bufs;
Q8_API int q8_0_step_buffers(const q8_0_step *s, q8_0_step_bufs *out);

Q8_API int q8_0_step_destroy(q8_0_step *s);

#ifdef __cplusplus
}
#endif

#endif /* Q8STEP_H */
