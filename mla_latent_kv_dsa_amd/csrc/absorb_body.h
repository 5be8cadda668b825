// absorb_body.h -- one workgroup of the query absorption of the matrix-core decode
// (kv_lora 512, 64 heads), shared by the absorb kernel and the fused decode step.
// colibri-analysis 06 "MLA attention and KV cache", sec. 2.3: the absorbed path folds W_UK into
// the query, q_abs[b][h][:] = W_UK[h]^T q_nope[b][h], with W_UK[h] the first qk_nope rows of
// head h's block of kv_b.
//
// Job (cb, h), 256 threads, covers columns 128 cb .. 128 cb + 127 of head h for queries 0..B-1.
// A workgroup may run several jobs side by side (tid = thread index inside the job, sh_abs = the
// job's own LDS); they then pass the same barriers, since every job loops over the same B.
// Thread t: row group rg = t/16 (rows rg, rg+16, ...) and column group cg = t%16 (8 of
// the 128 columns).  The W_UK rows go out first, then the queries of head h are staged in LDS
// (sh_abs: B * qk_nope + 4 * AB_QB * 128 floats), so both latencies overlap.  Queries are
// handled eight at a time; row-group partial sums are reduced with lane shuffles inside a
// wave, then across the four waves through LDS in a fixed order (fp32 FMA, bf16 out).
#pragma once
#include "common.h"

namespace mla {

constexpr int AB_L = 512, AB_H = 64;
constexpr int AB_QB = 8;

template <int NR>   // qk_nope / 16
__device__ __forceinline__ void absorb_block(const bf16_t *__restrict__ q_nope, const bf16_t *__restrict__ kv_b,
                                             int B, int v, bf16_t *__restrict__ q_abs, int cb, int h,
                                             float *__restrict__ sh_abs, int tid)
{
    constexpr int nope = 16 * NR;
    const int rg = tid >> 4, cg = tid & 15, lane = tid & 63, wave = tid >> 6;
    const int cbase = cb * 128;
    const bf16_t *W = kv_b + ((int64_t)h * (nope + v) + rg) * AB_L + cbase + cg * 8;
    uint4 w[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) w[k] = *reinterpret_cast<const uint4 *>(W + (int64_t)k * 16 * AB_L);
    float *sq = sh_abs;
    float *red = sh_abs + B * nope;
    for (int i = tid; i < B * nope; i += 256) {
        const int b = i / nope, r = i - b * nope;
        sq[i] = bf2f(q_nope[((int64_t)b * AB_H + h) * nope + r]);
    }
    __syncthreads();
    for (int b0 = 0; b0 < B; b0 += AB_QB) {
        const int nb = B - b0 < AB_QB ? B - b0 : AB_QB;
        float acc[AB_QB][8];
#pragma unroll
        for (int q = 0; q < AB_QB; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[q][e] = 0.f;
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            float wf[8];
            wf[0] = __uint_as_float(w[k].x << 16); wf[1] = __uint_as_float(w[k].x & 0xffff0000u);
            wf[2] = __uint_as_float(w[k].y << 16); wf[3] = __uint_as_float(w[k].y & 0xffff0000u);
            wf[4] = __uint_as_float(w[k].z << 16); wf[5] = __uint_as_float(w[k].z & 0xffff0000u);
            wf[6] = __uint_as_float(w[k].w << 16); wf[7] = __uint_as_float(w[k].w & 0xffff0000u);
#pragma unroll
            for (int q = 0; q < AB_QB; ++q) {
                if (q < nb) {
                    const float qv = sq[(b0 + q) * nope + rg + 16 * k];
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[q][e] = fmaf(qv, wf[e], acc[q][e]);
                }
            }
        }
        // the four row groups of a wave sit 16 lanes apart
#pragma unroll
        for (int q = 0; q < AB_QB; ++q) {
            if (q < nb) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float x = acc[q][e];
                    x += __shfl_xor(x, 16, 64);
                    x += __shfl_xor(x, 32, 64);
                    acc[q][e] = x;
                }
            }
        }
        if (lane < 16) {
#pragma unroll
            for (int q = 0; q < AB_QB; ++q) {
                if (q < nb) {
                    float *dst = &red[(wave * AB_QB + q) * 128 + cg * 8];
                    *reinterpret_cast<float4 *>(dst) = make_float4(acc[q][0], acc[q][1], acc[q][2], acc[q][3]);
                    *reinterpret_cast<float4 *>(dst + 4) = make_float4(acc[q][4], acc[q][5], acc[q][6], acc[q][7]);
                }
            }
        }
        __syncthreads();
        for (int i = tid; i < nb * 128; i += 256) {
            const int q = i >> 7, c = i & 127;
            const float s = ((red[(0 * AB_QB + q) * 128 + c] + red[(1 * AB_QB + q) * 128 + c]) +
                             red[(2 * AB_QB + q) * 128 + c]) + red[(3 * AB_QB + q) * 128 + c];
            q_abs[((int64_t)(b0 + q) * AB_H + h) * AB_L + cbase + c] = f2bf(s);
        }
        __syncthreads();
    }
}

}  // namespace mla
