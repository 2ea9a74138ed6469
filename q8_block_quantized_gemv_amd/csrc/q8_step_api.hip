// q8_step_api.hip -- the C ABI of include/q8step.h: the decode-step kernels
// one at a time, and a whole step recorded into a hipGraph (page "IV.4: One
// command buffer per token", section "One command buffer": every dispatch of
// a token encoded once, one wait, the next token id the only result).
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "q8step.h"
#include "q8_gemm.h"
#include "q8_host.h"
#include "q8_step.h"

using namespace q8;

namespace {

constexpr int64_t kMaxDim = 65536;
constexpr int kArgmaxPerWg = 4096;   // values per argmax workgroup before more are added
constexpr int kArgmaxMaxWgs = 256;

bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int argmax_wgs(int64_t n) {
    return (int)std::max<int64_t>(1, std::min<int64_t>(kArgmaxMaxWgs, (n + kArgmaxPerWg - 1) / kArgmaxPerWg));
}

int attn_chunks(int64_t seq) { return (int)((seq + kAttnChunk - 1) / kAttnChunk); }

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// The standalone calls' workspaces, 256-byte aligned pieces: attention's
// per-head arrival counters, then each (head, chunk)'s (m, s, acc[head_dim]);
// argmax's arrival counter, then each workgroup's winning value and index.
size_t attn_ws_bytes(int64_t seq, int64_t head_dim, int64_t n_heads) {
    return align256(4 * (size_t)n_heads) +
           align256((size_t)n_heads * attn_chunks(seq) * (head_dim + 2) * sizeof(float));
}
size_t argmax_ws_bytes(int64_t n) {
    const size_t wgs = (size_t)argmax_wgs(n);
    return 256 + align256(4 * wgs) + align256(4 * wgs);
}

int check_workspace(const void *ws, size_t have, size_t need, const char *what) {
    if (!ws || ((uintptr_t)ws & 255u))
        return fail(Q8_ERR_ALIGN, std::string(what) + ": the workspace must be a 256-byte aligned device buffer");
    if (have < need)
        return fail(Q8_ERR_INVALID_ARG, std::string(what) + ": the workspace holds " + std::to_string(have) +
                                            " bytes, the call needs " + std::to_string(need));
    return Q8_OK;
}

bool head_dim_ok(int64_t hd) { return hd == 64 || hd == 128 || hd == 192 || hd == 256; }

int check_attention(const float *q, const float *kc, const float *vc, const float *out, int64_t seq,
                    int64_t kv_width, int64_t head_dim, int64_t n_heads, int64_t kv_group,
                    const char *what) {
    const std::string tag(what);
    if (!q || !kc || !vc || !out) return fail(Q8_ERR_INVALID_ARG, tag + ": null pointer");
    if (!aligned16(q) || !aligned16(kc) || !aligned16(vc) || !aligned4(out) || kv_width % 4)
        return fail(Q8_ERR_ALIGN, tag + ": q, kc, vc must be 16-byte aligned, kv_width a multiple of 4, "
                                        "out 4-byte aligned");
    if (!head_dim_ok(head_dim))
        return fail(Q8_ERR_SHAPE, tag + ": head_dim must be 64, 128, 192 or 256");
    if (n_heads < 1 || n_heads > 4096 || kv_group < 1 || n_heads % kv_group)
        return fail(Q8_ERR_SHAPE, tag + ": n_heads must be a positive multiple of kv_group");
    if (kv_width < (n_heads / kv_group) * head_dim || kv_width > (int64_t)1 << 24)
        return fail(Q8_ERR_SHAPE, tag + ": kv_width must hold every KV head");
    if (seq < 1 || seq > Q8_MAX_SEQ) return fail(Q8_ERR_SHAPE, tag + ": seq out of range");
    const int64_t ob = 4 * n_heads * head_dim;
    if (overlaps(out, ob, q, ob) || overlaps(out, ob, kc, 4 * seq * kv_width) ||
        overlaps(out, ob, vc, 4 * seq * kv_width))
        return fail(Q8_ERR_ALIAS, tag + ": out overlaps an input");
    return Q8_OK;
}

}  // namespace

extern "C" {

int q8_0_rms_norm(const float *x, const float *w, float *out, int64_t dim, int64_t rows, float eps,
                  void *stream) {
    if (!x || !w || !out) return fail(Q8_ERR_INVALID_ARG, "q8_0_rms_norm: null pointer");
    if (dim < 1 || dim > kMaxDim || rows < 1 || rows > kMaxDim)
        return fail(Q8_ERR_SHAPE, "q8_0_rms_norm: dim and rows must be in 1..65536");
    if (!aligned4(x) || !aligned4(w) || !aligned4(out))
        return fail(Q8_ERR_ALIGN, "q8_0_rms_norm: buffers must be 4-byte aligned");
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(Q8_ERR_INVALID_ARG, "q8_0_rms_norm: eps");
    const int64_t nb = 4 * dim * rows;
    if (out != x && overlaps(out, nb, x, nb))
        return fail(Q8_ERR_ALIAS, "q8_0_rms_norm: out overlaps x without being x");
    if (overlaps(out, nb, w, 4 * dim)) return fail(Q8_ERR_ALIAS, "q8_0_rms_norm: out overlaps w");
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_rms_norm(x, w, out, (int)dim, (int)rows, eps, (hipStream_t)stream);
    return e == hipSuccess ? Q8_OK : fail_hip(e, "q8_0_rms_norm launch");
}

int q8_0_rope(float *x, int64_t head_dim, int64_t heads, int64_t pos, float theta, void *stream) {
    if (!x) return fail(Q8_ERR_INVALID_ARG, "q8_0_rope: null pointer");
    if (head_dim < 2 || head_dim % 2 || head_dim > kMaxDim || heads < 1 || heads > kMaxDim)
        return fail(Q8_ERR_SHAPE, "q8_0_rope: head_dim must be even, heads positive, both <= 65536");
    if (pos < 0 || pos > INT32_MAX) return fail(Q8_ERR_SHAPE, "q8_0_rope: pos out of range");
    if (!(theta > 0.f) || !std::isfinite(theta)) return fail(Q8_ERR_INVALID_ARG, "q8_0_rope: theta");
    if (!aligned4(x)) return fail(Q8_ERR_ALIGN, "q8_0_rope: x must be 4-byte aligned");
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_rope(x, (int)head_dim, (int)heads, nullptr, (int)pos, theta, (hipStream_t)stream);
    return e == hipSuccess ? Q8_OK : fail_hip(e, "q8_0_rope launch");
}

int q8_0_append_kv(const float *k, const float *v, float *kc, float *vc, int64_t width, int64_t pos,
                   void *stream) {
    if (!k || !v || !kc || !vc) return fail(Q8_ERR_INVALID_ARG, "q8_0_append_kv: null pointer");
    if (width < 1 || width > (int64_t)1 << 24 || pos < 0 || pos >= Q8_MAX_SEQ)
        return fail(Q8_ERR_SHAPE, "q8_0_append_kv: width or pos out of range");
    if (!aligned4(k) || !aligned4(v) || !aligned4(kc) || !aligned4(vc))
        return fail(Q8_ERR_ALIGN, "q8_0_append_kv: buffers must be 4-byte aligned");
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_append_kv(k, v, kc, vc, (int)width, nullptr, (int)pos, (int)pos + 1,
                                    (hipStream_t)stream);
    return e == hipSuccess ? Q8_OK : fail_hip(e, "q8_0_append_kv launch");
}

int q8_0_attention_workspace(int64_t seq, int64_t head_dim, int64_t n_heads, size_t *bytes) {
    if (!bytes) return fail(Q8_ERR_INVALID_ARG, "q8_0_attention_workspace: bytes is null");
    *bytes = 0;
    if (seq < 1 || seq > INT32_MAX / 2 || head_dim < 1 || head_dim > 256 || n_heads < 1 || n_heads > 65536)
        return fail(Q8_ERR_SHAPE, "q8_0_attention_workspace: shape out of range");
    *bytes = attn_ws_bytes(seq, head_dim, n_heads);
    return Q8_OK;
}

int q8_0_attention_decode(const float *q, const float *kc, const float *vc, float *out, int64_t seq,
                          int64_t kv_width, int64_t head_dim, int64_t n_heads, int64_t kv_group,
                          void *workspace, size_t workspace_bytes, void *stream) {
    int rc = check_attention(q, kc, vc, out, seq, kv_width, head_dim, n_heads, kv_group,
                             "q8_0_attention_decode");
    if (rc) return rc;
    const size_t need = attn_ws_bytes(seq, head_dim, n_heads);
    if ((rc = check_workspace(workspace, workspace_bytes, need, "q8_0_attention_decode"))) return rc;
    if (overlaps(workspace, (int64_t)need, out, 4 * n_heads * head_dim) ||
        overlaps(workspace, (int64_t)need, q, 4 * n_heads * head_dim))
        return fail(Q8_ERR_ALIAS, "q8_0_attention_decode: the workspace overlaps q or out");
    if ((rc = check_device())) return rc;
    hipStream_t s = (hipStream_t)stream;
    AttnDesc d;
    std::memset(&d, 0, sizeof d);
    d.q = q; d.kc = kc; d.vc = vc; d.out = out; d.pos_dev = nullptr;
    d.seq = (int)seq; d.kv_width = (int)kv_width; d.head_dim = (int)head_dim;
    d.n_heads = (int)n_heads; d.kv_group = (int)kv_group; d.max_chunks = attn_chunks(seq);
    d.cnt = (uint32_t *)workspace;
    d.ws = (float *)((uint8_t *)workspace + align256(4 * (size_t)n_heads));
    hipError_t e = hipSuccess;
    if (d.max_chunks > 1) e = launch_zero_u32(d.cnt, n_heads, s);   // the chunks' arrival counters
    if (e == hipSuccess) e = launch_attention(d, s);
    return e == hipSuccess ? Q8_OK : fail_hip(e, "q8_0_attention_decode launch");
}

int q8_0_add_inplace(float *x, const float *y, int64_t n, void *stream) {
    if (!x || !y) return fail(Q8_ERR_INVALID_ARG, "q8_0_add_inplace: null pointer");
    if (n < 1 || n > INT32_MAX - 256) return fail(Q8_ERR_SHAPE, "q8_0_add_inplace: n out of range");
    if (!aligned4(x) || !aligned4(y)) return fail(Q8_ERR_ALIGN, "q8_0_add_inplace: alignment");
    if (x != y && overlaps(x, 4 * n, y, 4 * n))
        return fail(Q8_ERR_ALIAS, "q8_0_add_inplace: x and y partly overlap");
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_add(x, y, (int)n, (hipStream_t)stream);
    return e == hipSuccess ? Q8_OK : fail_hip(e, "q8_0_add_inplace launch");
}

int q8_0_silu_hadamard(const float *gate, const float *up, float *out, int64_t n, void *stream) {
    if (!gate || !up || !out) return fail(Q8_ERR_INVALID_ARG, "q8_0_silu_hadamard: null pointer");
    if (n < 1 || n > INT32_MAX - 256) return fail(Q8_ERR_SHAPE, "q8_0_silu_hadamard: n out of range");
    if (!aligned4(gate) || !aligned4(up) || !aligned4(out))
        return fail(Q8_ERR_ALIGN, "q8_0_silu_hadamard: alignment");
    if ((out != gate && overlaps(out, 4 * n, gate, 4 * n)) || (out != up && overlaps(out, 4 * n, up, 4 * n)))
        return fail(Q8_ERR_ALIAS, "q8_0_silu_hadamard: out partly overlaps an input");
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_silu(gate, up, out, (int)n, (hipStream_t)stream);
    return e == hipSuccess ? Q8_OK : fail_hip(e, "q8_0_silu_hadamard launch");
}

int q8_0_argmax_workspace(int64_t n, size_t *bytes) {
    if (!bytes) return fail(Q8_ERR_INVALID_ARG, "q8_0_argmax_workspace: bytes is null");
    *bytes = 0;
    if (n < 1 || n > INT32_MAX) return fail(Q8_ERR_SHAPE, "q8_0_argmax_workspace: n out of range");
    *bytes = argmax_ws_bytes(n);
    return Q8_OK;
}

int q8_0_argmax(const float *x, int64_t n, uint32_t *out, void *workspace, size_t workspace_bytes,
                void *stream) {
    if (!x || !out) return fail(Q8_ERR_INVALID_ARG, "q8_0_argmax: null pointer");
    if (n < 1 || n > INT32_MAX) return fail(Q8_ERR_SHAPE, "q8_0_argmax: n out of range");
    if (!aligned4(x) || !aligned4(out)) return fail(Q8_ERR_ALIGN, "q8_0_argmax: alignment");
    if (overlaps(out, 4, x, 4 * n)) return fail(Q8_ERR_ALIAS, "q8_0_argmax: out overlaps x");
    const size_t need = argmax_ws_bytes(n);
    int rc = check_workspace(workspace, workspace_bytes, need, "q8_0_argmax");
    if (rc) return rc;
    if (overlaps(workspace, (int64_t)need, out, 4) || overlaps(workspace, (int64_t)need, x, 4 * n))
        return fail(Q8_ERR_ALIAS, "q8_0_argmax: the workspace overlaps x or out");
    if ((rc = check_device())) return rc;
    hipStream_t s = (hipStream_t)stream;
    const int wgs = argmax_wgs(n);
    ArgmaxDesc d;
    d.x = x; d.n = n; d.out = out; d.pos_dev = nullptr;
    d.cnt = (uint32_t *)workspace;
    d.ws_val = (float *)((uint8_t *)workspace + 256);
    d.ws_idx = (uint32_t *)((uint8_t *)workspace + 256 + align256(4 * (size_t)wgs));
    hipError_t e = launch_zero_u32(d.cnt, 1, s);   // the arrival counter
    if (e == hipSuccess) e = launch_argmax(d, wgs, s);
    return e == hipSuccess ? Q8_OK : fail_hip(e, "q8_0_argmax launch");
}

}  // extern "C"

// ===================================================================== the step
struct q8_0_step {
    int device = -1;
    q8_0_model m{};
    std::vector<q8_0_layer_w> layers;
    int64_t q_width = 0, kv_width = 0, kv_group = 0;
    void *mem = nullptr;      // one device allocation for everything below
    float *x = nullptr, *xn = nullptr, *q = nullptr, *k = nullptr, *v = nullptr, *attn = nullptr;
    float *xa = nullptr, *xb = nullptr;   // the residual stream, alternating between layers
    // fused residual path (widths multiples of 256): the squared norm's
    // 16-row block sums, left by o and by down for the matvecs after them,
    // and the residual stream times the next norm's gain (their input)
    float *psum_o = nullptr, *psum_d = nullptr, *xg = nullptr;
    bool fused_residual = false;
    float *resid = nullptr, *gate = nullptr, *up = nullptr, *logits = nullptr;
    float *kcache = nullptr, *vcache = nullptr, *attn_ws = nullptr, *amax_ws = nullptr;
    uint32_t *cnt = nullptr;  // n_heads attention counters, then the argmax counter
    int32_t *pos = nullptr;
    uint32_t *token = nullptr;
    double2 *rope = nullptr;  // (cos, sin) of every rotation angle, [position][pair]
    int max_chunks = 0, amax_wgs = 0, launches = 0;
    // per layer q|k|v, o, gate|up, down; then the lm_head
    std::vector<q8_0_chain *> chains;
    int64_t steps_since_reset = 0, reset_pos = 0;
    hipStream_t capture = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

namespace {

void step_free(q8_0_step *s) {
    if (!s) return;
    if (s->exec) (void)hipGraphExecDestroy(s->exec);
    if (s->graph) (void)hipGraphDestroy(s->graph);
    if (s->capture) (void)hipStreamDestroy(s->capture);
    for (q8_0_chain *c : s->chains) (void)q8_0_chain_destroy(c);
    if (s->mem) (void)hipFree(s->mem);
    delete s;
}

// Every launch of one token, in order, on stream st.
int issue_step(const q8_0_step *s, hipStream_t st) {
    const q8_0_model &m = s->m;
    const int hid = (int)m.hidden, nh = (int)m.n_heads;
    const int64_t cache_stride = m.max_seq * s->kv_width;
    hipError_t e = hipSuccess;
    auto ok = [&](hipError_t err) {
        if (err != hipSuccess && e == hipSuccess) e = err;
    };
    int rc = Q8_OK;
    ok(launch_embed_rms(m.embed, s->token, (uint32_t)m.vocab, s->xa, s->layers[0].attn_norm, s->xn,
                        hid, m.eps, st));
    for (int64_t l = 0; l < m.n_layers && e == hipSuccess; ++l) {
        const q8_0_layer_w &L = s->layers[l];
        float *kc = s->kcache + l * cache_stride, *vc = s->vcache + l * cache_stride;
        q8_0_chain *const *ch = &s->chains[4 * l];
        if ((rc = chain_issue(ch[0], st))) return rc;
        AttnDesc d;
        std::memset(&d, 0, sizeof d);
        d.q = nullptr; d.kc = kc; d.vc = vc; d.out = s->attn; d.pos_dev = s->pos;
        d.ws = s->attn_ws; d.cnt = s->cnt; d.seq = (int)m.max_seq; d.kv_width = (int)s->kv_width;
        d.head_dim = (int)m.head_dim; d.n_heads = nh; d.kv_group = (int)s->kv_group;
        d.max_chunks = s->max_chunks;
        AttnFuse f;
        f.q = s->q; f.k = s->k; f.v = s->v; f.q_norm = L.q_norm; f.k_norm = L.k_norm;
        f.kc_w = kc; f.vc_w = vc; f.eps = m.eps; f.theta = m.theta; f.rope = s->rope;
        ok(launch_attention_fused(d, f, st));
        if ((rc = chain_issue(ch[1], st))) return rc;
        if ((rc = chain_issue(ch[2], st))) return rc;
        if ((rc = chain_issue(ch[3], st))) return rc;
    }
    if (e != hipSuccess) return fail_hip(e, "decode step launch");
    if ((rc = chain_issue(s->chains.back(), st))) return rc;
    ArgmaxDesc a;
    a.x = s->logits; a.n = m.vocab; a.out = s->token; a.ws_val = s->amax_ws;
    a.ws_idx = (uint32_t *)(s->amax_ws + s->amax_wgs); a.cnt = s->cnt + m.n_heads;
    a.pos_dev = s->pos;
    ok(launch_argmax(a, s->amax_wgs, st));
    return e == hipSuccess ? Q8_OK : fail_hip(e, "decode step launch");
}

int check_model(const q8_0_model *m) {
    if (!m || !m->embed || !m->out_norm || !m->lm_head || !m->layers)
        return fail(Q8_ERR_INVALID_ARG, "q8_0_step_create: null model pointer");
    if (m->n_layers < 1 || m->n_layers > 4096)
        return fail(Q8_ERR_SHAPE, "q8_0_step_create: n_layers out of range");
    if (!head_dim_ok(m->head_dim))
        return fail(Q8_ERR_SHAPE, "q8_0_step_create: head_dim must be 64, 128, 192 or 256");
    if (m->n_kv_heads < 1 || m->n_heads < 1 || m->n_heads % m->n_kv_heads || m->n_heads > 4096)
        return fail(Q8_ERR_SHAPE, "q8_0_step_create: n_heads must be a multiple of n_kv_heads");
    if (m->hidden < 32 || m->hidden % 32 || m->hidden > kMaxDim || m->inter < 32 || m->inter % 32 ||
        m->inter > Q8_MAX_N)
        return fail(Q8_ERR_SHAPE, "q8_0_step_create: hidden and inter must be multiples of 32");
    if (m->vocab < 1 || m->vocab > INT32_MAX || m->max_seq < 1 || m->max_seq > Q8_MAX_SEQ)
        return fail(Q8_ERR_SHAPE, "q8_0_step_create: vocab or max_seq out of range");
    if (!(m->eps >= 0.f) || !std::isfinite(m->eps) || !(m->theta > 0.f) || !std::isfinite(m->theta))
        return fail(Q8_ERR_INVALID_ARG, "q8_0_step_create: eps or theta");
    if (!aligned16(m->embed) || !aligned16(m->out_norm))
        return fail(Q8_ERR_ALIGN, "q8_0_step_create: embed and out_norm must be 16-byte aligned");
    for (int64_t l = 0; l < m->n_layers; ++l) {
        const q8_0_layer_w &L = m->layers[l];
        if (!L.wq || !L.wk || !L.wv || !L.wo || !L.wgate || !L.wup || !L.wdown || !L.attn_norm ||
            !L.ffn_norm || !L.q_norm || !L.k_norm)
            return fail(Q8_ERR_INVALID_ARG, "q8_0_step_create: null weight in layer " + std::to_string(l));
        if (!aligned16(L.attn_norm) || !aligned16(L.ffn_norm) || !aligned4(L.q_norm) ||
            !aligned4(L.k_norm))
            return fail(Q8_ERR_ALIGN, "q8_0_step_create: norm weights of layer " + std::to_string(l) +
                                          " misaligned (attn/ffn 16 bytes, q/k 4 bytes)");
    }
    return Q8_OK;
}

}  // namespace

extern "C" {

int q8_0_step_create(const q8_0_model *m, q8_0_step **out) {
    if (!out) return fail(Q8_ERR_INVALID_ARG, "q8_0_step_create: out is null");
    *out = nullptr;
    int rc = check_model(m);
    if (rc) return rc;
    int dev = 0;
    if ((rc = check_device(&dev))) return rc;
    q8_0_step *s = new q8_0_step();
    s->device = dev;
    s->m = *m;
    s->layers.assign(m->layers, m->layers + m->n_layers);
    s->m.layers = nullptr;
    s->q_width = m->n_heads * m->head_dim;
    s->kv_width = m->n_kv_heads * m->head_dim;
    s->kv_group = m->n_heads / m->n_kv_heads;
    s->max_chunks = attn_chunks(m->max_seq);
    s->amax_wgs = argmax_wgs(m->vocab);
    if (s->q_width % 32) { step_free(s); return fail(Q8_ERR_SHAPE, "q8_0_step_create: n_heads * head_dim must be a multiple of 32"); }
    // one allocation, every piece 256-B aligned
    std::vector<size_t> sizes = {
        (size_t)m->hidden, (size_t)m->hidden, (size_t)m->hidden, (size_t)m->hidden,
        (size_t)s->q_width, (size_t)s->kv_width,
        (size_t)s->kv_width, (size_t)s->q_width, (size_t)m->hidden, (size_t)m->inter,
        (size_t)m->inter, (size_t)m->vocab,
        (size_t)(m->n_layers * m->max_seq * s->kv_width), (size_t)(m->n_layers * m->max_seq * s->kv_width),
        (size_t)(m->n_heads * s->max_chunks * (m->head_dim + 2)), (size_t)(2 * s->amax_wgs),
        (size_t)(m->n_heads + 1), 1, 1,
        (size_t)(m->max_seq * (m->head_dim / 2) * 4),   // double2 per (position, pair)
        (size_t)(m->hidden / kPsumRows + 1), (size_t)(m->hidden / kPsumRows + 1), (size_t)m->hidden};
    std::vector<size_t> offs;
    size_t total = 0;
    for (size_t n : sizes) {
        offs.push_back(total);
        total += (n * 4 + 255) / 256 * 256;
    }
    hipError_t e = hipMalloc(&s->mem, total);
    if (e != hipSuccess) { step_free(s); return fail_hip(e, "q8_0_step_create hipMalloc"); }
    if ((e = hipMemset(s->mem, 0, total)) != hipSuccess || (e = hipDeviceSynchronize()) != hipSuccess) {
        step_free(s);
        return fail_hip(e, "q8_0_step_create hipMemset");
    }
    char *b = (char *)s->mem;
    float **fl[] = {&s->x, &s->xn, &s->xa, &s->xb, &s->q, &s->k, &s->v, &s->attn, &s->resid, &s->gate, &s->up,
                    &s->logits, &s->kcache, &s->vcache, &s->attn_ws, &s->amax_ws};
    const size_t nf = sizeof fl / sizeof fl[0];
    for (size_t i = 0; i < nf; ++i) *fl[i] = (float *)(b + offs[i]);
    s->cnt = (uint32_t *)(b + offs[nf]);
    s->pos = (int32_t *)(b + offs[nf + 1]);
    s->token = (uint32_t *)(b + offs[nf + 2]);
    s->rope = (double2 *)(b + offs[nf + 3]);
    s->psum_o = (float *)(b + offs[nf + 4]);
    s->psum_d = (float *)(b + offs[nf + 5]);
    s->xg = (float *)(b + offs[nf + 6]);
    // the rotation angles of every position, once: attention reads them
    // instead of evaluating pow and sincos in double precision per token
    if ((e = launch_rope_table(s->rope, (int)m->max_seq, (int)(m->head_dim / 2), m->theta, nullptr)) !=
            hipSuccess ||
        (e = hipDeviceSynchronize()) != hipSuccess) {
        step_free(s);
        return fail_hip(e, "q8_0_step_create rotation table");
    }
    // the matvecs: fused where independent.  Each residual add and the norm
    // after it are folded into the next matvec's activation staging
    // (kXNormAdd): it reads the residual stream and the block's output,
    // normalises their sum, and its first workgroup writes the sum to the
    // other stream buffer.  The down projections read silu(gate) * up
    // (kXSiluUp).  The embedding row and the first norm come from embed+norm.
    auto mk = [&](std::vector<q8_0_op> ops, const OpExtra *e = nullptr) {
        q8_0_chain *c = nullptr;
        std::vector<OpExtra> ex;
        if (e) {
            ex.assign(ops.size(), *e);
            for (size_t i = 1; i < ex.size(); ++i) ex[i].x_out = nullptr;   // one writer per launch
        }
        int r = chain_create_ex(ops.data(), (int64_t)ops.size(), Q8_CHAIN_FUSE | Q8_CHAIN_SPLIT_K,
                                e ? ex.data() : nullptr, &c);
        if (!r) s->chains.push_back(c);
        return r;
    };
    auto norm_add = [&](const float *gain, float *x_out, const float *res = nullptr) {
        OpExtra e;
        e.mode = kXNormAdd;
        e.x_res = res ? res : s->resid;
        e.norm_w = gain;
        e.x_out = x_out;
        e.eps = m->eps;
        return e;
    };
    float *cur = s->xa, *oth = s->xb;
    // Where every projection's rows are whole 272-byte groups (hidden, inter
    // and the query width multiples of 256), the residual adds move into the
    // matvecs that produce them: o and down write the new residual stream
    // v = x_res + W x, the sums of v^2 over 16-row blocks and v times the
    // next norm's gain (kYResAdd); the matvecs after them read that product
    // and scale each row result by 1 / rms(v) from those sums (kXNormScale)
    // -- no workgroup re-reads the whole stream for its norm.  gate and up run as one pair whose workgroups
    // compute the same rows of both and write silu(gate) * up (kYSwiGLU), so
    // down reads a plain input.  Other widths take the inputs apart in each
    // consumer instead (kXNormAdd, kXSiluUp).
    const auto whole = [](int64_t v) { return v % (kQuants * kGroupBlocks) == 0; };
    s->fused_residual = whole(m->hidden) && whole(m->inter) && whole(s->q_width);
    if (s->fused_residual) {
        auto norm_scale = [&](float *psum) {
            OpExtra e;
            e.mode = kXNormScale;
            e.psum = psum;
            e.eps = m->eps;
            return e;
        };
        // out = res + W x, and xg = out * gain for the next matvec
        auto res_add = [&](const float *res, float *psum, const float *gain) {
            OpExtra e;
            e.out_mode = kYResAdd;
            e.x_res = res;
            e.psum = psum;
            e.norm_w = gain;
            e.x_out = s->xg;
            return e;
        };
        for (int64_t l = 0; l < m->n_layers && !rc; ++l) {
            const q8_0_layer_w &L = s->layers[l];
            if (l == 0) {
                rc = mk({{s->xn, L.wq, s->q, m->hidden, s->q_width}, {s->xn, L.wk, s->k, m->hidden, s->kv_width},
                         {s->xn, L.wv, s->v, m->hidden, s->kv_width}});
            } else {
                const OpExtra e = norm_scale(s->psum_d);   // attn_norm(cur), from xg = cur * attn_norm
                rc = mk({{s->xg, L.wq, s->q, m->hidden, s->q_width}, {s->xg, L.wk, s->k, m->hidden, s->kv_width},
                         {s->xg, L.wv, s->v, m->hidden, s->kv_width}}, &e);
            }
            if (rc) break;
            const OpExtra eo = res_add(cur, s->psum_o, L.ffn_norm);   // oth = cur + Wo attn
            if ((rc = mk({{s->attn, L.wo, oth, s->q_width, m->hidden}}, &eo))) break;
            OpExtra eg = norm_scale(s->psum_o);   // gate = silu(Wg n) * (Wu n), n = ffn_norm(oth)
            eg.out_mode = kYSwiGLU;
            eg.w2 = L.wup;
            if ((rc = mk({{s->xg, L.wgate, s->gate, m->hidden, m->inter}}, &eg))) break;
            const float *next = l + 1 < m->n_layers ? s->layers[l + 1].attn_norm : m->out_norm;
            const OpExtra ed = res_add(oth, s->psum_d, next);          // cur = oth + Wd gate
            if ((rc = mk({{s->gate, L.wdown, cur, m->inter, m->hidden}}, &ed))) break;
        }
        if (!rc) {
            const OpExtra e = norm_scale(s->psum_d);   // out_norm(cur)
            rc = mk({{s->xg, m->lm_head, s->logits, m->hidden, m->vocab}}, &e);
        }
    } else {
        OpExtra silu;
        silu.mode = kXSiluUp;
        silu.x_up = s->up;
        for (int64_t l = 0; l < m->n_layers && !rc; ++l) {
            const q8_0_layer_w &L = s->layers[l];
            if (l == 0) {
                rc = mk({{s->xn, L.wq, s->q, m->hidden, s->q_width}, {s->xn, L.wk, s->k, m->hidden, s->kv_width},
                         {s->xn, L.wv, s->v, m->hidden, s->kv_width}});
            } else {
                const OpExtra e = norm_add(L.attn_norm, oth);
                rc = mk({{cur, L.wq, s->q, m->hidden, s->q_width}, {cur, L.wk, s->k, m->hidden, s->kv_width},
                         {cur, L.wv, s->v, m->hidden, s->kv_width}}, &e);
                std::swap(cur, oth);
            }
            if (rc) break;
            if ((rc = mk({{s->attn, L.wo, s->resid, s->q_width, m->hidden}}))) break;
            const OpExtra e = norm_add(L.ffn_norm, oth);
            if ((rc = mk({{cur, L.wgate, s->gate, m->hidden, m->inter}, {cur, L.wup, s->up, m->hidden, m->inter}},
                         &e)))
                break;
            std::swap(cur, oth);
            if ((rc = mk({{s->gate, L.wdown, s->resid, m->inter, m->hidden}}, &silu))) break;
        }
        if (!rc) {
            const OpExtra e = norm_add(m->out_norm, s->x);
            rc = mk({{cur, m->lm_head, s->logits, m->hidden, m->vocab}}, &e);
        }
    }
    if (rc) { std::string why = "q8_0_step_create: " + std::string(q8_0_last_error()); step_free(s); return fail(rc, why); }
    s->launches = 0;
    for (q8_0_chain *c : s->chains) s->launches += q8_0_chain_launches(c);
    s->launches += (int)(m->n_layers + 2);   // embed+norm, attention per layer, argmax
    // record one token
    if ((e = hipStreamCreateWithFlags(&s->capture, hipStreamNonBlocking)) != hipSuccess) {
        step_free(s);
        return fail_hip(e, "hipStreamCreateWithFlags");
    }
    if ((e = hipStreamBeginCapture(s->capture, hipStreamCaptureModeThreadLocal)) != hipSuccess) {
        step_free(s);
        return fail_hip(e, "hipStreamBeginCapture");
    }
    int irc = issue_step(s, s->capture);
    e = hipStreamEndCapture(s->capture, &s->graph);
    if (irc) { std::string why = q8_0_last_error(); step_free(s); return fail(irc, why); }
    if (e != hipSuccess) { step_free(s); return fail_hip(e, "hipStreamEndCapture"); }
    if ((e = hipGraphInstantiate(&s->exec, s->graph, nullptr, nullptr, 0)) != hipSuccess) {
        step_free(s);
        return fail_hip(e, "hipGraphInstantiate");
    }
    *out = s;
    return Q8_OK;
}

int q8_0_step_reset(q8_0_step *s, int64_t pos, uint32_t token, void *stream) {
    if (!s) return fail(Q8_ERR_INVALID_ARG, "q8_0_step_reset: null step");
    if (pos < 0 || pos >= s->m.max_seq) return fail(Q8_ERR_SHAPE, "q8_0_step_reset: pos out of range");
    hipError_t e = launch_set_state(s->pos, s->token, (int)pos, token, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "q8_0_step_reset launch");
    s->reset_pos = pos;
    s->steps_since_reset = 0;
    return Q8_OK;
}

int q8_0_step_run(q8_0_step *s, int mode, void *stream) {
    if (!s) return fail(Q8_ERR_INVALID_ARG, "q8_0_step_run: null step");
    if (mode != Q8_MODE_GRAPH && mode != Q8_MODE_EAGER)
        return fail(Q8_ERR_INVALID_ARG, "q8_0_step_run: mode must be GRAPH or EAGER");
    if (s->reset_pos + s->steps_since_reset >= s->m.max_seq)
        return fail(Q8_ERR_SHAPE, "q8_0_step_run: the KV cache is full (max_seq)");
    hipStream_t st = (hipStream_t)stream;
    int rc = Q8_OK;
    if (mode == Q8_MODE_GRAPH) {
        hipError_t e = hipGraphLaunch(s->exec, st);
        if (e != hipSuccess) return fail_hip(e, "hipGraphLaunch");
    } else if ((rc = issue_step(s, st))) {
        return rc;
    }
    ++s->steps_since_reset;
    return Q8_OK;
}

int q8_0_step_launches(const q8_0_step *s) {
    if (!s) return fail(Q8_ERR_INVALID_ARG, "q8_0_step_launches: null step");
    return s->launches;
}

int q8_0_step_buffers(const q8_0_step *s, q8_0_step_bufs *out) {
    if (!s || !out) return fail(Q8_ERR_INVALID_ARG, "q8_0_step_buffers: null pointer");
    out->token = s->token;
    out->pos = s->pos;
    out->x = s->fused_residual ? s->xa : s->x;   // the residual stream after the last layer
    out->logits = s->logits;
    out->k_cache = s->kcache;
    out->v_cache = s->vcache;
    return Q8_OK;
}

int q8_0_step_destroy(q8_0_step *s) {
    step_free(s);
    return Q8_OK;
}

}  // extern "C"
