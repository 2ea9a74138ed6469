// q8_step.hip -- gfx950 kernels for the rest of a decode step: the seven
// kernels the page "IV.4: One command buffer per token" (section "Eight
// kernels") puts around q8_matvec -- rms_norm_row, rope_row, append_kv,
// attention_decode, add_inplace, silu_hadamard, argmax_row -- plus the two
// a device-resident token loop needs (the embedding row of the previous
// token, and advancing the position).
//
// Designed for CDNA4 rather than taken over from the page's threadgroups:
//  * rows are reduced by one 64-lane wave with a fixed butterfly (no LDS);
//  * attention splits each head's cached rows into chunks of kAttnChunk
//    handled by separate workgroups (so a 16-head step uses hundreds of CUs,
//    not 16) and the last chunk to arrive merges the partial softmaxes in
//    chunk order -- deterministic, like every other reduction here;
//  * argmax scans with many workgroups and merges their winners the same
//    way, with the page's comparison (greater, or equal at a lower index).
// Kernels that a recorded token replays read the position from device
// memory (pos_dev), so one recording serves every token.
#include "q8_step.h"

namespace q8 {
namespace {

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ int position(const int *pos_dev, int pos) {
    return pos_dev ? *pos_dev : pos;
}

// ---------------------------------------------------------------- rms_norm_row
// One wave per row: out = x * (sum(x^2)/dim + eps)^(-1/2) * w.  out may be x.
__global__ __launch_bounds__(kWave) void k_rms_norm(const float *x, const float *w, float *out,
                                                    int dim, float eps) {
    const int lane = lane_id();
    const float *xr = x + (int64_t)blockIdx.x * dim;
    float *orow = out + (int64_t)blockIdx.x * dim;
    float ss = 0.f;
    for (int i = lane; i < dim; i += kWave) ss = fmaf(xr[i], xr[i], ss);
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)dim + eps);
    for (int i = lane; i < dim; i += kWave) orow[i] = xr[i] * inv * w[i];
}

// ---------------------------------------------------------------- rope_row
// Pair (i, i + half) of each head turns by pos * theta^(-i / half); the angle
// and its sine and cosine are taken in double precision (the page's float32
// angle loses ~pos * 2^-24 rad), the rotation rounds once to float.
__global__ __launch_bounds__(256) void k_rope(float *x, int head_dim, int heads, const int *pos_dev,
                                              int pos0, float theta) {
    const int half = head_dim / 2;
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= heads * half) return;
    const int h = t / half, i = t - h * half;
    const double ang = (double)position(pos_dev, pos0) * pow((double)theta, -(double)i / half);
    double s, c;
    sincos(ang, &s, &c);
    float *xh = x + (int64_t)h * head_dim;
    const double a = xh[i], b = xh[i + half];
    xh[i] = (float)(a * c - b * s);
    xh[i + half] = (float)(a * s + b * c);
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
// [c*kAttnChunk, min(seq, (c+1)*kAttnChunk)) on KV head h / kv_group, their
// local softmax (max m, sum s of e^(score - m)) and acc[j] = sum e * v[j];
// the last chunk of a head to arrive merges the parts in chunk order.
// Rows are scored one per wave: 64 lanes read a key row together (coalesced)
// and reduce the dot product with a butterfly.
constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;

__global__ __launch_bounds__(kAttnThreads) void k_attention(AttnDesc d) {
    __shared__ float sc[kAttnChunk];
    __shared__ float red[kAttnWaves];
    __shared__ float accp[kAttnThreads];
    const int head = blockIdx.x % d.n_heads;
    const int c = blockIdx.x / d.n_heads;
    const int seq = d.pos_dev ? min(*d.pos_dev + 1, d.seq) : d.seq;
    const int n_chunks = (seq + kAttnChunk - 1) / kAttnChunk;
    if (c >= n_chunks) return;   // the whole workgroup: no part, no arrival
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const int hd = d.head_dim, per = hd / kWave;   // elements per lane (1..4)
    const int t0 = c * kAttnChunk, rows = min(kAttnChunk, seq - t0);
    const int64_t kv_off = (int64_t)(head / d.kv_group) * hd;
    const float *qh = d.q + (int64_t)head * hd;
    float qv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) qv[e] = e < per ? qh[e * kWave + lane] : 0.f;
    const float scale = 1.0f / sqrtf((float)hd);
    for (int r = wv; r < rows; r += kAttnWaves) {
        const float *kr = d.kc + (int64_t)(t0 + r) * d.kv_width + kv_off;
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e < per) dot = fmaf(qv[e], kr[e * kWave + lane], dot);
        dot = wave_sum(dot);
        if (lane == 0) sc[r] = dot * scale;
    }
    __syncthreads();
    // local max and sum over the chunk
    float m = -INFINITY;
    for (int r = tid; r < rows; r += kAttnThreads) m = fmaxf(m, sc[r]);
    m = wave_max(m);
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
    s = wave_sum(s);
    if (lane == 0) red[wv] = s;
    __syncthreads();
    s = (red[0] + red[1]) + (red[2] + red[3]);
    // acc[j]: thread (j, part) sums rows part, part + parts, ... of the chunk
    const int parts = kAttnThreads / hd;
    const int j = tid % hd, part = tid / hd;
    float a = 0.f;
    if (part < parts)
        for (int r = part; r < rows; r += parts)
            a = fmaf(sc[r], d.vc[(int64_t)(t0 + r) * d.kv_width + kv_off + j], a);
    accp[tid] = a;
    __syncthreads();
    // park (m, s, acc[0..hd)) of this chunk, device-scope, then count in
    float *mine = d.ws + ((int64_t)head * d.max_chunks + c) * (hd + 2);
    if (tid < hd) {
        float t = accp[tid];
        for (int q = 1; q < parts; ++q) t += accp[q * hd + tid];
        __hip_atomic_store(mine + 2 + tid, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0) {
        __hip_atomic_store(mine, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(mine + 1, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __shared__ uint32_t prev;
    if (tid == 0)
        prev = __hip_atomic_fetch_add(d.cnt + head, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (prev != (uint32_t)n_chunks - 1) return;
    asm volatile("" ::: "memory");
    // merge: M = max m_c, S = sum s_c e^(m_c - M), out = sum acc_c e^(m_c - M) / S
    const float *parts0 = d.ws + (int64_t)head * d.max_chunks * (hd + 2);
    float M = -INFINITY;
    for (int q = 0; q < n_chunks; ++q)
        M = fmaxf(M, __hip_atomic_load(parts0 + (int64_t)q * (hd + 2), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT));
    if (tid < hd) {
        float S = 0.f, A = 0.f;
        for (int q = 0; q < n_chunks; ++q) {
            const float *pq = parts0 + (int64_t)q * (hd + 2);
            const float f = expf(__hip_atomic_load(pq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - M);
            S = fmaf(__hip_atomic_load(pq + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), f, S);
            A = fmaf(__hip_atomic_load(pq + 2 + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), f, A);
        }
        d.out[(int64_t)head * hd + tid] = A / S;
    }
    if (tid == 0)   // ready for the next launch
        __hip_atomic_store(d.cnt + head, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

__global__ __launch_bounds__(256) void k_argmax(ArgmaxDesc d) {
    __shared__ float bv[4];
    __shared__ uint32_t bi[4];
    __shared__ uint32_t prev;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    float best = -INFINITY;
    uint32_t besti = 0xFFFFFFFFu;
    for (int64_t i = (int64_t)blockIdx.x * 256 + tid; i < d.n; i += (int64_t)gridDim.x * 256)
        better(d.x[i], (uint32_t)i, best, besti);
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
            __hip_atomic_store(d.cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------- token loop
// x = row `token` of the embedding table (zeros for a token past the table:
// a row of only NaN logits has no argmax).
__global__ __launch_bounds__(256) void k_embed(const float *table, const uint32_t *token,
                                               uint32_t vocab, float *x, int dim) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= dim) return;
    const uint32_t t = *token;
    x[i] = t < vocab ? table[(int64_t)t * dim + i] : 0.f;
}

__global__ void k_advance(int *pos_dev) {
    if (threadIdx.x == 0) pos_dev[0] += 1;
}

__global__ void k_set_state(int *pos_dev, uint32_t *token_dev, int pos, uint32_t token) {
    if (threadIdx.x == 0) {
        pos_dev[0] = pos;
        token_dev[0] = token;
    }
}

unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_rms_norm(const float *x, const float *w, float *out, int dim, int rows, float eps,
                           hipStream_t s) {
    hipLaunchKernelGGL(k_rms_norm, dim3((unsigned)rows), dim3(kWave), 0, s, x, w, out, dim, eps);
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

hipError_t launch_attention(const AttnDesc &d, hipStream_t s) {
    hipLaunchKernelGGL(k_attention, dim3((unsigned)(d.n_heads * d.max_chunks)), dim3(kAttnThreads),
                       0, s, d);
    return hipGetLastError();
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

hipError_t launch_embed(const float *table, const uint32_t *token, uint32_t vocab, float *x, int dim,
                        hipStream_t s) {
    hipLaunchKernelGGL(k_embed, dim3(blocks_for(dim)), dim3(256), 0, s, table, token, vocab, x, dim);
    return hipGetLastError();
}

hipError_t launch_advance(int *pos_dev, hipStream_t s) {
    hipLaunchKernelGGL(k_advance, dim3(1), dim3(kWave), 0, s, pos_dev);
    return hipGetLastError();
}

hipError_t launch_set_state(int *pos_dev, uint32_t *token_dev, int pos, uint32_t token, hipStream_t s) {
    hipLaunchKernelGGL(k_set_state, dim3(1), dim3(kWave), 0, s, pos_dev, token_dev, pos, token);
    return hipGetLastError();
}

}  // namespace q8
