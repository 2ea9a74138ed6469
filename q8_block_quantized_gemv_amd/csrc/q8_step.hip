// q8_step.hip -- gfx950 kernels for the rest of a decode step: the seven
// kernels the page "IV.4: One command buffer per token" (section "Eight
// kernels") puts around q8_matvec -- rms_norm_row, rope_row, append_kv,
// attention_decode, add_inplace, silu_hadamard, argmax_row -- and the fused
// forms a recorded token uses.
//
// Designed for CDNA4 rather than taken over from the page's threadgroups.
// These kernels move kilobytes, so their time is memory latency, not
// bandwidth: every kernel issues all of a lane's loads before it uses any
// (float4 loads into register arrays), so a kernel costs about one trip to
// HBM instead of one trip per loop iteration.
//  * a row (a norm, a head) belongs to one 64-lane wave and is reduced with
//    a fixed butterfly (no LDS, no atomics);
//  * attention splits each head's cached rows into chunks of kAttnChunk
//    handled by separate workgroups (a 16-head step uses many CUs, not 16);
//    the last chunk to arrive merges the partial softmaxes in chunk order --
//    deterministic, like every reduction here;
//  * argmax scans with many workgroups and merges their winners the same
//    way, with the page's comparison (greater, or equal at a lower index).
// The fused kernels of a recorded token (the page encodes each of its
// kernels separately; fewer, larger launches suit a hipGraph better):
//  * embed_rms: x = embedding row of the token, xn = rms_norm(x);
//  * (the residual adds and the norms after them are folded into the next
//    matvec's activation staging, see q8_gemv.hip);
//  * attention takes the per-head q and k norms, the rotary embedding of q
//    and k and the K/V cache append into its own prologue;
//  * argmax also advances the position.
// Kernels a recorded token replays read the position from device memory
// (pos_dev), so one recording serves every token.
#include <cstring>

#include "q8_step.h"

namespace q8 {
namespace {

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// A whole-wave reduction of v by op, the result in every lane, in a fixed
// order: pairs, quads, 8- and 16-lane rows through DPP (no LDS), the two
// rows of each 32-lane half through one swizzle, the halves through two
// reads of lanes 0 and 32.
template <typename Op>
__device__ __forceinline__ float dpp_reduce(float v, Op op) {
    auto dpp = [](float x, int ctrl) -> float {
        switch (ctrl) {   // (the control must be a constant of the instruction)
            case 0: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
            case 1: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
            case 2: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
            default: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
        }
    };
    v = op(v, dpp(v, 0));   // quad_perm [1,0,3,2]: lane ^ 1
    v = op(v, dpp(v, 1));   // quad_perm [2,3,0,1]: lane ^ 2
    v = op(v, dpp(v, 2));   // row_half_mirror: the other quad of 8
    v = op(v, dpp(v, 3));   // row_mirror: the other 8 of 16
    v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F)));   // lane ^ 16
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    return op(lo, hi);
}
__device__ __forceinline__ float dpp_sum(float v) {
    return dpp_reduce(v, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ float dpp_max(float v) {
    return dpp_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}

__device__ __forceinline__ int position(const int *pos_dev, int pos) {
    return pos_dev ? *pos_dev : pos;
}

__device__ __forceinline__ float sq4(float4 v, float acc) {
    acc = fmaf(v.x, v.x, acc);
    acc = fmaf(v.y, v.y, acc);
    acc = fmaf(v.z, v.z, acc);
    return fmaf(v.w, v.w, acc);
}

__device__ __forceinline__ float4 scale4(float4 x, float inv, float4 w) {
    return make_float4(x.x * inv * w.x, x.y * inv * w.y, x.z * inv * w.z, x.w * inv * w.w);
}

// ---------------------------------------------------------------- rms_norm_row
// out = x * (sum(x^2)/dim + eps)^(-1/2) * w, one wave per row.
constexpr int kNormRegs = 16;                           // float4 a lane holds
constexpr int kNormMaxInRegs = kWave * kNormRegs * 4;   // 4096 floats

__device__ __forceinline__ float rms_inv(float ss, int dim, float eps) {
    return 1.0f / sqrtf(ss / (float)dim + eps);
}

// A row of nv float4 (dim = 4 nv <= kNormMaxInRegs) into registers; returns
// its sum of squares through the butterfly.
__device__ __forceinline__ float load_row4(const float4 *xr, int nv, float4 (&xv)[kNormRegs]) {
    const int lane = lane_id();
#pragma unroll
    for (int e = 0; e < kNormRegs; ++e) {
        const int i = lane + kWave * e;
        xv[e] = i < nv ? xr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < kNormRegs; ++e) ss = sq4(xv[e], ss);
    return wave_sum(ss);
}

__device__ __forceinline__ void store_row4(float4 *orow, const float4 *w4, int nv, float inv,
                                           const float4 (&xv)[kNormRegs]) {
    const int lane = lane_id();
    float4 wv[kNormRegs];
#pragma unroll
    for (int e = 0; e < kNormRegs; ++e) {
        const int i = lane + kWave * e;
        wv[e] = i < nv ? w4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int e = 0; e < kNormRegs; ++e) {
        const int i = lane + kWave * e;
        if (i < nv) orow[i] = scale4(xv[e], inv, wv[e]);
    }
}

// One row by one wave, any dim (float4 path when V).
template <bool V>
__device__ __forceinline__ void rms_row(const float *xr, const float *w, float *orow, int dim,
                                        float eps) {
    const int lane = lane_id();
    if (V && dim <= kNormMaxInRegs) {
        float4 xv[kNormRegs];
        const int nv = dim / 4;
        const float ss = load_row4((const float4 *)xr, nv, xv);
        store_row4((float4 *)orow, (const float4 *)w, nv, rms_inv(ss, dim, eps), xv);
        return;
    }
    if (V) {   // long rows: batches of kNormRegs float4 per lane, then a second pass
        const int nv = dim / 4;
        const float4 *x4 = (const float4 *)xr;
        float ss = 0.f;
        for (int b = 0; b < nv; b += kWave * kNormRegs) {
            float4 xv[kNormRegs];
#pragma unroll
            for (int e = 0; e < kNormRegs; ++e) {
                const int i = b + lane + kWave * e;
                xv[e] = i < nv ? x4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int e = 0; e < kNormRegs; ++e) ss = sq4(xv[e], ss);
        }
        const float inv = rms_inv(wave_sum(ss), dim, eps);
        for (int b = 0; b < nv; b += kWave * kNormRegs) {
            float4 xv[kNormRegs], wv[kNormRegs];
#pragma unroll
            for (int e = 0; e < kNormRegs; ++e) {
                const int i = b + lane + kWave * e;
                xv[e] = i < nv ? x4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
                wv[e] = i < nv ? ((const float4 *)w)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int e = 0; e < kNormRegs; ++e) {
                const int i = b + lane + kWave * e;
                if (i < nv) ((float4 *)orow)[i] = scale4(xv[e], inv, wv[e]);
            }
        }
        return;
    }
    float ss = 0.f;
    for (int i = lane; i < dim; i += kWave) ss = fmaf(xr[i], xr[i], ss);
    const float inv = rms_inv(wave_sum(ss), dim, eps);
    for (int i = lane; i < dim; i += kWave) orow[i] = xr[i] * inv * w[i];
}

template <bool V>
__global__ __launch_bounds__(kThreads) void k_rms_norm(const float *x, const float *w, float *out,
                                                       int dim, int rows, float eps) {
    const int row = blockIdx.x * kWaves + (int)(threadIdx.x / kWave);
    if (row >= rows) return;
    rms_row<V>(x + (int64_t)row * dim, w, out + (int64_t)row * dim, dim, eps);
}

// ---------------------------------------------------------------- fused residual + norm
// EMBED: x = row `token` of the table y (zeros past the table: a row of only
// NaN logits has no argmax); else x += y.  Then xn = rms_norm(x) * w.
// A recorded step uses the EMBED form for its first norm.
// One 256-thread workgroup (four float4 per thread in flight for rows up to
// 4096); dim % 4 == 0 and x, y, w, xn 16-byte aligned.
template <bool EMBED>
__device__ __forceinline__ float4 residual4(const float4 *x4, const float4 *src, bool zero, int i) {
    if (EMBED) return zero ? make_float4(0.f, 0.f, 0.f, 0.f) : src[i];
    const float4 a = x4[i], b = src[i];
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

template <bool EMBED>
__global__ __launch_bounds__(kThreads) void k_add_rms(float *x, const float *y, const uint32_t *token,
                                                      uint32_t vocab, const float *w, float *xn,
                                                      int dim, float eps) {
    constexpr int R = 4;   // float4 a thread holds: rows up to kThreads * R * 4 = 4096 floats
    __shared__ float red[kWaves];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const int nv = dim / 4;
    float4 *x4 = (float4 *)x;
    const float4 *w4 = (const float4 *)w;
    const float4 *src = (const float4 *)y;
    bool zero = false;
    if (EMBED) {
        const uint32_t t = *token;
        zero = t >= vocab;
        src = (const float4 *)(y + (int64_t)(zero ? 0u : t) * dim);
    }
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (nv <= kThreads * R) {   // the row stays in registers
        float4 xv[R], wq[R];
#pragma unroll
        for (int e = 0; e < R; ++e) {
            const int i = tid + kThreads * e;
            xv[e] = z4;
            wq[e] = z4;
            if (i < nv) {
                xv[e] = residual4<EMBED>(x4, src, zero, i);
                wq[e] = w4[i];
            }
        }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < R; ++e) {
            const int i = tid + kThreads * e;
            if (i < nv) x4[i] = xv[e];
            ss = sq4(xv[e], ss);
        }
        ss = wave_sum(ss);
        if (lane == 0) red[wv] = ss;
        __syncthreads();
        const float inv = rms_inv((red[0] + red[1]) + (red[2] + red[3]), dim, eps);
#pragma unroll
        for (int e = 0; e < R; ++e) {
            const int i = tid + kThreads * e;
            if (i < nv) ((float4 *)xn)[i] = scale4(xv[e], inv, wq[e]);
        }
        return;
    }
    // long rows: write x batch by batch, then normalise it (each thread
    // re-reads only what it wrote itself)
    float ss = 0.f;
    for (int b = 0; b < nv; b += kThreads * R) {
        float4 xv[R];
#pragma unroll
        for (int e = 0; e < R; ++e) {
            const int i = b + tid + kThreads * e;
            xv[e] = z4;
            if (i < nv) xv[e] = residual4<EMBED>(x4, src, zero, i);
        }
#pragma unroll
        for (int e = 0; e < R; ++e) {
            const int i = b + tid + kThreads * e;
            if (i < nv) x4[i] = xv[e];
            ss = sq4(xv[e], ss);
        }
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wv] = ss;
    __syncthreads();
    const float inv = rms_inv((red[0] + red[1]) + (red[2] + red[3]), dim, eps);
    for (int b = 0; b < nv; b += kThreads * R) {
        float4 xv[R], wq[R];
#pragma unroll
        for (int e = 0; e < R; ++e) {
            const int i = b + tid + kThreads * e;
            xv[e] = z4;
            wq[e] = z4;
            if (i < nv) {
                xv[e] = x4[i];
                wq[e] = w4[i];
            }
        }
#pragma unroll
        for (int e = 0; e < R; ++e) {
            const int i = b + tid + kThreads * e;
            if (i < nv) ((float4 *)xn)[i] = scale4(xv[e], inv, wq[e]);
        }
    }
}

// ---------------------------------------------------------------- rope_row
// Pair (i, i + half) of each head turns by pos * theta^(-i / half); the angle
// and its sine and cosine are taken in double precision (the page's float32
// angle loses ~pos * 2^-24 rad), the rotation rounds once to float.
__device__ __forceinline__ void rope_sincos(int i, int half, int pos, float theta, double &s, double &c) {
    const double ang = (double)pos * pow((double)theta, -(double)i / half);
    sincos(ang, &s, &c);
}

__device__ __forceinline__ void rotate_by(double a, double b, double s, double c, float &ra, float &rb) {
    ra = (float)(a * c - b * s);
    rb = (float)(a * s + b * c);
}

__device__ __forceinline__ void rotate(double a, double b, int i, int half, int pos, float theta,
                                       float &ra, float &rb) {
    double s, c;
    rope_sincos(i, half, pos, theta, s, c);
    rotate_by(a, b, s, c, ra, rb);
}

// The step's table of every angle's (cos, sin): t[pos * half + i].
__global__ __launch_bounds__(256) void k_rope_table(double2 *t, int rows, int half, float theta) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= (int64_t)rows * half) return;
    const int pos = (int)(j / half), i = (int)(j - (int64_t)pos * half);
    double s, c;
    rope_sincos(i, half, pos, theta, s, c);
    t[j] = make_double2(c, s);
}

__global__ __launch_bounds__(256) void k_rope(float *x, int head_dim, int heads, const int *pos_dev,
                                              int pos0, float theta) {
    const int half = head_dim / 2;
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= heads * half) return;
    const int h = t / half, i = t - h * half;
    float *xh = x + (int64_t)h * head_dim;
    float ra, rb;
    rotate(xh[i], xh[i + half], i, half, position(pos_dev, pos0), theta, ra, rb);
    xh[i] = ra;
    xh[i + half] = rb;
}

// ---------------------------------------------------------------- append_kv
// A position at or past `rows` (the cache's length) writes nothing.
__global__ __launch_bounds__(256) void k_append_kv(const float *k, const float *v, float *kc,
                                                   float *vc, int width, const int *pos_dev,
                                                   int pos0, int rows) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int pos = position(pos_dev, pos0);
    if (i >= width || pos < 0 || pos >= rows) return;
    const int64_t row = (int64_t)pos * width;
    kc[row + i] = k[i];
    vc[row + i] = v[i];
}

// ---------------------------------------------------------------- attention_decode
// Workgroup (chunk c, head h) of 256 threads: the scores of cached rows
// [c*CHUNK, min(seq, (c+1)*CHUNK)) on KV head h / kv_group, their
// local softmax (max m, sum s of e^(score - m)) and acc[j] = sum e * v[j].
// A head of one chunk writes acc / s; otherwise the last chunk of a head to
// arrive merges the parts in chunk order.
// Scores: a row is read by L lanes with float4 loads (L = HD/4 rounded up
// to a power of two), 64/L rows per wave at a time, every row of a lane's
// share loaded before any is reduced.  Values: thread (column float4,
// row group) accumulates its rows, the row groups meet in LDS.  Once the
// position is read, every load of the chunk that depends on nothing else
// (keys, the first batch of values, q/k/v, norm gains, rotation angles)
// is issued at once, so a short chunk costs two memory round trips.
// FUSED (a recorded token): the q head arrives raw and is normed (q_norm)
// and rotated here; the chunk holding the token's own row (pos = seq - 1)
// norms and rotates that row's key from the raw k and takes its value from
// the raw v instead of reading them from the caches, and the first query
// head of each KV group stores them into cache row pos for later tokens.
constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int kMergeBatch = 8;

template <int HD, bool FUSED, int CHUNK>
__device__ __forceinline__ void attention_part(const AttnDesc &d, const AttnFuse &f, const int seq) {
    constexpr int NV = HD / 4;                                   // float4 per row
    constexpr int HALF = HD / 2;
    constexpr int L = NV <= 16 ? 16 : NV <= 32 ? 32 : 64;        // lanes per row
    constexpr int RPW = kWave / L;                               // rows per wave per pass
    constexpr int RPP = kAttnWaves * RPW;                        // rows per pass
    constexpr int PASSES = CHUNK / RPP;
    constexpr int SB = PASSES < 16 ? PASSES : 16;                // score loads in flight
    constexpr int RG = kAttnThreads / NV;                        // value row groups
    constexpr int RPT = (CHUNK + RG - 1) / RG;                   // rows per thread
    constexpr int VB = RPT < 16 ? RPT : 16;                      // value loads in flight
    __shared__ float sc[CHUNK];
    __shared__ float pt[kAttnWaves * SB * 65];   // each wave's partial-dot tile
    __shared__ float red[2 * kAttnWaves];
    __shared__ float4 accp[kAttnThreads];
    __shared__ uint32_t prev;
    __shared__ __attribute__((aligned(16))) float qs[FUSED ? kAttnWaves * HD : 4];   // per wave
    __shared__ __attribute__((aligned(16))) float kn[FUSED ? kAttnWaves * HD : 4];
    const int head = blockIdx.x % d.n_heads;
    const int c = blockIdx.x / d.n_heads;
    const int n_chunks = (seq + CHUNK - 1) / CHUNK;
    if (c >= n_chunks) return;   // the whole workgroup: no part, no arrival
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const int t0 = c * CHUNK, rows = min(CHUNK, seq - t0);
    const int kvh = head / d.kv_group;
    const int64_t kv_off = (int64_t)kvh * HD;
    const int pos = seq - 1;
    const bool cur = FUSED && pos >= t0 && pos < t0 + rows;   // this chunk holds the token's row
    const int rcur = pos - t0;
    const bool writer = cur && head % d.kv_group == 0;        // stores the row into the caches
    const int64_t crow = (int64_t)pos * d.kv_width + kv_off;
    // ---- every read of the chunk that depends only on the position is
    // issued here at once: keys, the first batch of values, the raw q/k/v,
    // the norm gains and the rotation angles.  The token's own row is not in
    // the caches yet: its key and value are skipped here (they read as zero)
    // and enter once, from the raw k and v.
    const int g = lane / L, col = lane % L;
    const bool colv = col < NV;
    const float *kbase = d.kc + (int64_t)t0 * d.kv_width + kv_off + 4 * col;
    float4 kv[SB];
    auto load_keys = [&](int p0) {
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            const int r = (p0 + b) * RPP + wv * RPW + g;
            kv[b] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (colv && r < rows && !(cur && r == rcur))
                kv[b] = *(const float4 *)(kbase + (int64_t)r * d.kv_width);
        }
    };
    const int vcol = tid % NV, rg = tid / NV;
    const float *vbase = d.vc + (int64_t)t0 * d.kv_width + kv_off + 4 * vcol;
    float4 vv[VB];
    auto load_vals = [&](int r0) {
#pragma unroll
        for (int b = 0; b < VB; ++b) {
            const int r = rg + (r0 + b) * RG;
            vv[b] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (rg < RG && r < rows && !(cur && r == rcur))
                vv[b] = *(const float4 *)(vbase + (int64_t)r * d.kv_width);
        }
    };
    load_keys(0);
    load_vals(0);
    // FUSED: each wave norms and rotates its own copy of q (and k): lane l
    // holds the pairs (i, i + HALF), i = l + 64 j < HALF
    constexpr int NP = (HALF + kWave - 1) / kWave;
    float qa[NP], qb[NP], ka[NP], kb[NP], qga[NP], qgb[NP], kga[NP], kgb[NP];
    double2 cs[NP];
    float4 vn4 = make_float4(0.f, 0.f, 0.f, 0.f);   // the token's raw value, column vcol
    float4 q4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (FUSED) {
        const float *qh = f.q + (int64_t)head * HD;
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int i = lane + kWave * j;
            qa[j] = qb[j] = ka[j] = kb[j] = qga[j] = qgb[j] = kga[j] = kgb[j] = 0.f;
            cs[j] = make_double2(1.0, 0.0);
            if (i < HALF) {
                qa[j] = qh[i];
                qb[j] = qh[i + HALF];
                qga[j] = f.q_norm[i];
                qgb[j] = f.q_norm[i + HALF];
                cs[j] = f.rope[(int64_t)pos * HALF + i];
                if (cur) {
                    ka[j] = f.k[kv_off + i];
                    kb[j] = f.k[kv_off + i + HALF];
                    kga[j] = f.k_norm[i];
                    kgb[j] = f.k_norm[i + HALF];
                }
            }
        }
        if (cur) vn4 = *(const float4 *)(f.v + kv_off + 4 * vcol);
    } else if (colv) {
        q4 = ((const float4 *)(d.q + (int64_t)head * HD))[col];
    }
    // ---- scores
    float s_cur = 0.f;   // the token's own score (FUSED)
    {
        if (FUSED) {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                sq = fmaf(qa[j], qa[j], sq);
                sq = fmaf(qb[j], qb[j], sq);
                sk = fmaf(ka[j], ka[j], sk);
                sk = fmaf(kb[j], kb[j], sk);
            }
            const float iq = rms_inv(dpp_sum(sq), HD, f.eps);
            const float ik = cur ? rms_inv(dpp_sum(sk), HD, f.eps) : 0.f;
            float *qw = qs + wv * HD, *kw = kn + wv * HD;   // this wave's copies
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                const int i = lane + kWave * j;
                if (i < HALF) {
                    float ra, rb;
                    rotate_by(qa[j] * iq * qga[j], qb[j] * iq * qgb[j], cs[j].y, cs[j].x, ra, rb);
                    qw[i] = ra;
                    qw[i + HALF] = rb;
                    if (cur) {
                        rotate_by(ka[j] * ik * kga[j], kb[j] * ik * kgb[j], cs[j].y, cs[j].x, ra, rb);
                        kw[i] = ra;
                        kw[i + HALF] = rb;
                        if (writer && wv == 0) {
                            f.kc_w[crow + i] = ra;
                            f.kc_w[crow + i + HALF] = rb;
                        }
                    }
                }
            }
            if (writer && tid < NV) *(float4 *)(f.vc_w + crow + 4 * vcol) = vn4;
            __builtin_amdgcn_wave_barrier();
            if (colv) q4 = ((const float4 *)qw)[col];
            if (cur) {   // q . k of the token's row: every group of L lanes holds it whole
                const float4 k4 = colv ? ((const float4 *)kw)[col] : make_float4(0.f, 0.f, 0.f, 0.f);
                float dc = q4.x * k4.x;
                dc = fmaf(q4.y, k4.y, dc);
                dc = fmaf(q4.z, k4.z, dc);
                dc = fmaf(q4.w, k4.w, dc);
                s_cur = dpp_sum(dc) * (1.0f / RPW);   // the RPW equal group sums, an exact multiple
            }
        }
        const float scale = 1.0f / sqrtf((float)HD);
        // A lane's SB partial dots (one per pass of the batch) go to the
        // wave's tile P[b][lane] (rows of 65 floats: both the writes and the
        // transposed reads below hit distinct banks); lane j then adds the SB
        // partials of row (pass b, group g), columns [h SB, h SB + SB), for
        // j = (g LG + h) SB + b, and the LG lanes of a row meet in a
        // butterfly over h.
        constexpr int LG = L / SB;
        static_assert(SB <= L && L % SB == 0, "passes per batch within a row's lanes");
        float *P = pt + wv * (SB * 65);
        const int rb = lane % SB, rgh = lane / SB;   // (b, g LG + h) of the row part this lane adds
        for (int p0 = 0; p0 < PASSES; p0 += SB) {
            if (p0 > 0) load_keys(p0);
#pragma unroll
            for (int b = 0; b < SB; ++b) {
                float dot = q4.x * kv[b].x;
                dot = fmaf(q4.y, kv[b].y, dot);
                dot = fmaf(q4.z, kv[b].z, dot);
                P[b * 65 + lane] = fmaf(q4.w, kv[b].w, dot);
            }
            __builtin_amdgcn_wave_barrier();
            float part = 0.f;
#pragma unroll
            for (int k = 0; k < SB; ++k) part += P[rb * 65 + rgh * SB + k];
#pragma unroll
            for (int o = SB; o < LG * SB; o <<= 1) part += __shfl_xor(part, o, kWave);
            __builtin_amdgcn_wave_barrier();   // (the tile is rewritten by the next batch)
            const int gg = rgh / LG;
            const int r = (p0 + rb) * RPP + wv * RPW + gg;
            if (rgh % LG == 0 && r < rows) sc[r] = (cur && r == rcur ? s_cur : part) * scale;
        }
    }
    __syncthreads();
    // ---- local max and sum over the chunk
    float m = -INFINITY;
    for (int r = tid; r < rows; r += kAttnThreads) m = fmaxf(m, sc[r]);
    m = dpp_max(m);
    if (lane == 0) red[wv] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float s = 0.f;
    for (int r = tid; r < rows; r += kAttnThreads) {
        const float e = expf(sc[r] - m);
        sc[r] = e;
        s += e;
    }
    s = dpp_sum(s);
    if (lane == 0) red[wv] = s;
    __syncthreads();
    s = (red[0] + red[1]) + (red[2] + red[3]);
    // ---- acc over the chunk's values (thread (vcol, rg) takes rows rg, rg + RG, ...)
    {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (rg < RG) {
            for (int r0 = 0; r0 < RPT; r0 += VB) {
                if (r0 > 0) load_vals(r0);
                float ee[VB];
#pragma unroll
                for (int b = 0; b < VB; ++b) {
                    const int r = rg + (r0 + b) * RG;
                    const float e = sc[min(r, CHUNK - 1)];
                    ee[b] = r < rows ? e : 0.f;
                }
#pragma unroll
                for (int b = 0; b < VB; ++b) {
                    acc.x = fmaf(ee[b], vv[b].x, acc.x);
                    acc.y = fmaf(ee[b], vv[b].y, acc.y);
                    acc.z = fmaf(ee[b], vv[b].z, acc.z);
                    acc.w = fmaf(ee[b], vv[b].w, acc.w);
                }
            }
            if (cur && rg == rcur % RG) {   // the token's own value, after the cached rows
                const float e = sc[rcur];
                acc.x = fmaf(e, vn4.x, acc.x);
                acc.y = fmaf(e, vn4.y, acc.y);
                acc.z = fmaf(e, vn4.z, acc.z);
                acc.w = fmaf(e, vn4.w, acc.w);
            }
        }
        accp[tid] = acc;
    }
    __syncthreads();
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid < NV) {
        t = accp[tid];
        for (int q = 1; q < RG; ++q) {
            const float4 u = accp[q * NV + tid];
            t = make_float4(t.x + u.x, t.y + u.y, t.z + u.z, t.w + u.w);
        }
    }
    if (n_chunks == 1) {   // the whole head in this chunk: no merge
        if (tid < NV)
            ((float4 *)(d.out + (int64_t)head * HD))[tid] =
                make_float4(t.x / s, t.y / s, t.z / s, t.w / s);
        return;
    }
    // ---- park (m, s, acc[0..HD)) of this chunk, device-scope, then count in
    float *mine = d.ws + ((int64_t)head * d.max_chunks + c) * (HD + 2);
    if (tid < NV) {
        __hip_atomic_store(mine + 2 + 4 * tid, t.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(mine + 3 + 4 * tid, t.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(mine + 4 + 4 * tid, t.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(mine + 5 + 4 * tid, t.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0) {
        __hip_atomic_store(mine, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(mine + 1, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
        prev = __hip_atomic_fetch_add(d.cnt + head, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (prev != (uint32_t)n_chunks - 1) return;
    asm volatile("" ::: "memory");
    // ---- merge: M = max m_c, S = sum s_c e^(m_c - M), out = sum acc_c e^(m_c - M) / S
    const float *parts0 = d.ws + (int64_t)head * d.max_chunks * (HD + 2);
    float M = -INFINITY;
    for (int q0 = 0; q0 < n_chunks; q0 += kMergeBatch) {
        float mv[kMergeBatch];
#pragma unroll
        for (int b = 0; b < kMergeBatch; ++b) {
            mv[b] = -INFINITY;
            if (q0 + b < n_chunks)
                mv[b] = __hip_atomic_load(parts0 + (int64_t)(q0 + b) * (HD + 2), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int b = 0; b < kMergeBatch; ++b) M = fmaxf(M, mv[b]);
    }
    if (tid < HD) {
        float S = 0.f, A = 0.f;
        for (int q0 = 0; q0 < n_chunks; q0 += kMergeBatch) {
            float mv[kMergeBatch], sv[kMergeBatch], av[kMergeBatch];
#pragma unroll
            for (int b = 0; b < kMergeBatch; ++b) {
                const bool ok = q0 + b < n_chunks;
                const float *pq = parts0 + (int64_t)(ok ? q0 + b : 0) * (HD + 2);
                mv[b] = __hip_atomic_load(pq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                sv[b] = __hip_atomic_load(pq + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                av[b] = __hip_atomic_load(pq + 2 + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int b = 0; b < kMergeBatch; ++b) {
                if (q0 + b < n_chunks) {
                    const float fct = expf(mv[b] - M);
                    S = fmaf(sv[b], fct, S);
                    A = fmaf(av[b], fct, A);
                }
            }
        }
        d.out[(int64_t)head * HD + tid] = A / S;
    }
    if (tid == 0)   // ready for the next launch
        __hip_atomic_store(d.cnt + head, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Contexts of at most kAttnShort rows take one chunk of that many rows: the
// same arithmetic in a body whose loads and loops are sized for it (a chunk
// of kAttnChunk rows issues and masks that many rows' loads however few
// rows there are).  Measured per token at position 0 against one body of
// 128-row chunks: 7B 2171 -> 2125 us, Qwen3-0.6B 809 -> 774 us.
template <int HD, bool FUSED>
__global__ __launch_bounds__(kAttnThreads) void k_attention(AttnDesc d, AttnFuse f) {
    const int seq = d.pos_dev ? min(*d.pos_dev + 1, d.seq) : d.seq;
    if (seq <= kAttnShort) attention_part<HD, FUSED, kAttnShort>(d, f, seq);
    else attention_part<HD, FUSED, kAttnChunk>(d, f, seq);
}

// ---------------------------------------------------------------- add_inplace, silu_hadamard
__global__ __launch_bounds__(256) void k_add(float *x, const float *y, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) x[i] += y[i];
}

__global__ __launch_bounds__(256) void k_silu(const float *g, const float *u, float *out, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float v = g[i];
    out[i] = (v / (1.0f + expf(-v))) * u[i];
}

// ---------------------------------------------------------------- argmax_row
// (value, index) wins over (best, besti) if greater, or equal at a lower
// index; NaN never wins.  This order does not depend on how the scan is
// split, so the parallel result is the linear scan's.
__device__ __forceinline__ void better(float v, uint32_t i, float &best, uint32_t &besti) {
    if (v > best || (v == best && i < besti)) {
        best = v;
        besti = i;
    }
}

__device__ __forceinline__ void wave_best(float &best, uint32_t &besti) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const float ov = __shfl_xor(best, o, kWave);
        const uint32_t oi = __shfl_xor(besti, o, kWave);
        better(ov, oi, best, besti);
    }
}

constexpr int kArgmaxLoads = 8;   // values a thread has in flight

__global__ __launch_bounds__(256) void k_argmax(ArgmaxDesc d) {
    __shared__ float bv[4];
    __shared__ uint32_t bi[4];
    __shared__ uint32_t prev;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    float best = -INFINITY;
    uint32_t besti = 0xFFFFFFFFu;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i0 = (int64_t)blockIdx.x * 256 + tid; i0 < d.n; i0 += stride * kArgmaxLoads) {
        float v[kArgmaxLoads];
#pragma unroll
        for (int b = 0; b < kArgmaxLoads; ++b) {
            const int64_t i = i0 + b * stride;
            v[b] = i < d.n ? d.x[i] : __builtin_nanf("");
        }
#pragma unroll
        for (int b = 0; b < kArgmaxLoads; ++b) better(v[b], (uint32_t)(i0 + b * stride), best, besti);
    }
    wave_best(best, besti);
    if (lane == 0) { bv[wv] = best; bi[wv] = besti; }
    __syncthreads();
    if (tid == 0) {
        for (int q = 1; q < 4; ++q) better(bv[q], bi[q], best, besti);
        __hip_atomic_store(d.ws_val + blockIdx.x, best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(d.ws_idx + blockIdx.x, besti, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        prev = __hip_atomic_fetch_add(d.cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (prev != gridDim.x - 1) return;
    asm volatile("" ::: "memory");
    if (tid < kWave) {
        best = -INFINITY;
        besti = 0xFFFFFFFFu;
        for (int q = tid; q < (int)gridDim.x; q += kWave)
            better(__hip_atomic_load(d.ws_val + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                   __hip_atomic_load(d.ws_idx + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                   best, besti);
        wave_best(best, besti);
        if (tid == 0) {
            d.out[0] = besti;
            if (d.pos_dev) d.pos_dev[0] += 1;   // the token loop's next position
            __hip_atomic_store(d.cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------- token loop
__global__ void k_set_state(int *pos_dev, uint32_t *token_dev, int pos, uint32_t token) {
    if (threadIdx.x == 0) {
        pos_dev[0] = pos;
        token_dev[0] = token;
    }
}

unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

hipError_t launch_rms_norm(const float *x, const float *w, float *out, int dim, int rows, float eps,
                           hipStream_t s) {
    const dim3 grid((unsigned)((rows + kWaves - 1) / kWaves));
    if (dim % 4 == 0 && aligned16(x) && aligned16(w) && aligned16(out))
        hipLaunchKernelGGL(k_rms_norm<true>, grid, dim3(kThreads), 0, s, x, w, out, dim, rows, eps);
    else
        hipLaunchKernelGGL(k_rms_norm<false>, grid, dim3(kThreads), 0, s, x, w, out, dim, rows, eps);
    return hipGetLastError();
}

hipError_t launch_embed_rms(const float *table, const uint32_t *token, uint32_t vocab, float *x,
                            const float *w, float *xn, int dim, float eps, hipStream_t s) {
    hipLaunchKernelGGL(k_add_rms<true>, dim3(1), dim3(kThreads), 0, s, x, table, token, vocab, w, xn,
                       dim, eps);
    return hipGetLastError();
}

hipError_t launch_rope(float *x, int head_dim, int heads, const int *pos_dev, int pos, float theta,
                       hipStream_t s) {
    hipLaunchKernelGGL(k_rope, dim3(blocks_for((int64_t)heads * head_dim / 2)), dim3(256), 0, s, x,
                       head_dim, heads, pos_dev, pos, theta);
    return hipGetLastError();
}

hipError_t launch_append_kv(const float *k, const float *v, float *kc, float *vc, int width,
                            const int *pos_dev, int pos, int rows, hipStream_t s) {
    hipLaunchKernelGGL(k_append_kv, dim3(blocks_for(width)), dim3(256), 0, s, k, v, kc, vc, width,
                       pos_dev, pos, rows);
    return hipGetLastError();
}

template <bool FUSED>
hipError_t launch_attention_t(const AttnDesc &d, const AttnFuse &f, hipStream_t s) {
    const dim3 grid((unsigned)(d.n_heads * d.max_chunks));
    switch (d.head_dim) {
        case 64: hipLaunchKernelGGL((k_attention<64, FUSED>), grid, dim3(kAttnThreads), 0, s, d, f); break;
        case 128: hipLaunchKernelGGL((k_attention<128, FUSED>), grid, dim3(kAttnThreads), 0, s, d, f); break;
        case 192: hipLaunchKernelGGL((k_attention<192, FUSED>), grid, dim3(kAttnThreads), 0, s, d, f); break;
        case 256: hipLaunchKernelGGL((k_attention<256, FUSED>), grid, dim3(kAttnThreads), 0, s, d, f); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_attention(const AttnDesc &d, hipStream_t s) {
    AttnFuse f;
    std::memset(&f, 0, sizeof f);
    return launch_attention_t<false>(d, f, s);
}

hipError_t launch_rope_table(double2 *t, int rows, int half, float theta, hipStream_t s) {
    hipLaunchKernelGGL(k_rope_table, dim3(blocks_for((int64_t)rows * half)), dim3(256), 0, s, t, rows,
                       half, theta);
    return hipGetLastError();
}

hipError_t launch_attention_fused(const AttnDesc &d, const AttnFuse &f, hipStream_t s) {
    if (!f.rope) return hipErrorInvalidValue;
    return launch_attention_t<true>(d, f, s);
}

hipError_t launch_add(float *x, const float *y, int n, hipStream_t s) {
    hipLaunchKernelGGL(k_add, dim3(blocks_for(n)), dim3(256), 0, s, x, y, n);
    return hipGetLastError();
}

hipError_t launch_silu(const float *g, const float *u, float *out, int n, hipStream_t s) {
    hipLaunchKernelGGL(k_silu, dim3(blocks_for(n)), dim3(256), 0, s, g, u, out, n);
    return hipGetLastError();
}

hipError_t launch_argmax(const ArgmaxDesc &d, int wgs, hipStream_t s) {
    hipLaunchKernelGGL(k_argmax, dim3((unsigned)wgs), dim3(256), 0, s, d);
    return hipGetLastError();
}

hipError_t launch_set_state(int *pos_dev, uint32_t *token_dev, int pos, uint32_t token, hipStream_t s) {
    hipLaunchKernelGGL(k_set_state, dim3(1), dim3(kWave), 0, s, pos_dev, token_dev, pos, token);
    return hipGetLastError();
}

}  // namespace q8
