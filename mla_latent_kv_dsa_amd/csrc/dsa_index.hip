// dsa_index.hip -- DSA lightning-indexer scores.
// colibri-analysis 06 "MLA attention and KV cache", sec. 2.2: each causal key t gets a
// ReLU-gated, per-head-weighted score  I[t] = sum_h w[h] * ReLU(q[h] . Ic[t]);
// "Ch.7 sec. 03 ... faithful DSA", sec. 2: Ic is fp32 (index_hd x 4 bytes per token).
//
// Fixed evaluation order (the contract that makes the selected set exact): s = +0; for h
// ascending { a = +0; for d ascending a = fma(q[h][d], Ic[t][d], a); s = fma(w[h], max(a,+0), s) }.
// Every kernel below performs exactly this sequence of fp32 operations per key.
#include "common.h"

namespace mla {

// One lane per key.  The query (n_ih x HD fp32) is uniform across the block and is read
// with scalar loads; the key row lives in VGPRs.  Heads run four at a time as independent
// fma chains; their weighted sum is still folded into s in ascending head order.
template <int HD>
__global__ __launch_bounds__(256) void index_scores_lane_per_key(const float *__restrict__ q,
                                                                 const float *__restrict__ w, int n_ih,
                                                                 KvView kv, int64_t t_max,
                                                                 float *__restrict__ scores)
{
    const int b = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= t_max) return;
    float *out = scores + (int64_t)b * t_max;
    const int64_t n = seq_len_of(kv, b);
    if (t >= n) {
        out[t] = -INFINITY;
        return;
    }
    const int64_t row = kv_row(kv, b, t);
    if (row < 0) {
        out[t] = -INFINITY;
        return;
    }
    const float4 *kp = reinterpret_cast<const float4 *>(kv.ic + row * HD);
    float k[HD];
#pragma unroll
    for (int i = 0; i < HD / 4; ++i) {
        const float4 v = kp[i];
        k[4 * i + 0] = v.x;
        k[4 * i + 1] = v.y;
        k[4 * i + 2] = v.z;
        k[4 * i + 3] = v.w;
    }
    const float *qb = q + (int64_t)b * n_ih * HD;
    const float *wb = w + (int64_t)b * n_ih;
    float s = 0.0f;
    int h = 0;
    for (; h + 4 <= n_ih; h += 4) {
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
        const float *q0 = qb + h * HD;
#pragma unroll
        for (int d = 0; d < HD; ++d) {
            a0 = __builtin_fmaf(q0[d], k[d], a0);
            a1 = __builtin_fmaf(q0[HD + d], k[d], a1);
            a2 = __builtin_fmaf(q0[2 * HD + d], k[d], a2);
            a3 = __builtin_fmaf(q0[3 * HD + d], k[d], a3);
        }
        s = __builtin_fmaf(wb[h + 0], a0 > 0.f ? a0 : 0.f, s);
        s = __builtin_fmaf(wb[h + 1], a1 > 0.f ? a1 : 0.f, s);
        s = __builtin_fmaf(wb[h + 2], a2 > 0.f ? a2 : 0.f, s);
        s = __builtin_fmaf(wb[h + 3], a3 > 0.f ? a3 : 0.f, s);
    }
    for (; h < n_ih; ++h) {
        float a = 0.f;
        const float *q0 = qb + h * HD;
#pragma unroll
        for (int d = 0; d < HD; ++d) a = __builtin_fmaf(q0[d], k[d], a);
        s = __builtin_fmaf(wb[h], a > 0.f ? a : 0.f, s);
    }
    out[t] = s;
}

// Any index_hd (multiple of 4, <= 256): the key row is re-read per head from cache.
__global__ __launch_bounds__(256) void index_scores_generic(const float *__restrict__ q,
                                                           const float *__restrict__ w, int n_ih, int hd,
                                                           KvView kv, int64_t t_max,
                                                           float *__restrict__ scores)
{
    const int b = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= t_max) return;
    float *out = scores + (int64_t)b * t_max;
    const int64_t n = seq_len_of(kv, b);
    const int64_t row = t < n ? kv_row(kv, b, t) : -1;
    if (row < 0) {
        out[t] = -INFINITY;
        return;
    }
    const float *k = kv.ic + row * hd;
    const float *qb = q + (int64_t)b * n_ih * hd;
    const float *wb = w + (int64_t)b * n_ih;
    float s = 0.0f;
    for (int h = 0; h < n_ih; ++h) {
        float a = 0.f;
        for (int d = 0; d < hd; ++d) a = __builtin_fmaf(qb[h * hd + d], k[d], a);
        s = __builtin_fmaf(wb[h], a > 0.f ? a : 0.f, s);
    }
    out[t] = s;
}

mla_status launch_index_scores(const float *q, const float *w, int32_t B, int32_t n_ih, int32_t hd,
                               const KvView &kv, int64_t t_max, float *scores, hipStream_t s)
{
    const int64_t gx = (t_max + 255) / 256;
    if (gx > 0x7fffffff || B > 65535) return fail(MLA_ERR_UNSUPPORTED, "index: grid too large");
    dim3 grid((unsigned)gx, (unsigned)B);
    if (hd == 128)
        hipLaunchKernelGGL(index_scores_lane_per_key<128>, grid, dim3(256), 0, s, q, w, n_ih, kv, t_max, scores);
    else
        hipLaunchKernelGGL(index_scores_generic, grid, dim3(256), 0, s, q, w, n_ih, hd, kv, t_max, scores);
    return check_launch("index_scores");
}

}  // namespace mla
