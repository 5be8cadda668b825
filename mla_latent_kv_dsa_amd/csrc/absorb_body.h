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
#include "qformat.h"

namespace mla {

constexpr int AB_L = 512, AB_H = 64;
constexpr int AB_QB = 8;

// FMT: 0 for the bf16 kv_b, else its quantized format (qformat.h; kv_b then holds the codes and
// scales their scales).
template <int NR, int FMT = 0>   // qk_nope / 16
__device__ __forceinline__ void absorb_block(const bf16_t *__restrict__ q_nope, const void *__restrict__ kv_b,
                                             const void *__restrict__ scales, int B, int v, bf16_t *__restrict__ q_abs,
                                             int cb, int h, float *__restrict__ sh_abs, int tid)
{
    constexpr int nope = 16 * NR;
    const int rg = tid >> 4, cg = tid & 15, lane = tid & 63, wave = tid >> 6;
    const int cbase = cb * 128;
    const int64_t row0 = (int64_t)h * (nope + v) + rg;
    QRaw8<FMT> raw[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) raw[k] = q_raw8<FMT>(kv_b, scales, row0 + 16 * k, AB_L, cbase + cg * 8);
    float *sq = sh_abs;
    float *red = sh_abs + B * nope;
    for (int i = tid; i < B * nope; i += 256) {
        const int b = i / nope, r = i - b * nope;
        sq[i] = bf2f(q_nope[((int64_t)b * AB_H + h) * nope + r]);
    }
    __syncthreads();
    // the weights as exact bf16 values and a factor per row (the row scale of the byte formats,
    // applied to the query element instead of every weight)
    uint4 w[NR];
    float wsc[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) q_bf16x8<FMT>(raw[k], w[k], wsc[k]);
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
                    const float qv = (FMT == MLA_Q_FP8_E4M3 || FMT == MLA_Q_INT8)
                                         ? sq[(b0 + q) * nope + rg + 16 * k] * wsc[k]
                                         : sq[(b0 + q) * nope + rg + 16 * k];
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

// Batches of at least AB_MFMA_B queries: the same job on v_mfma_f32_16x16x32_bf16.  The job's
// W_UK block (qk_nope rows x 128 columns) is staged in LDS once (rows padded to AB_WROWB bytes
// so the transposed reads of four rows fall in distinct banks); the queries go straight from
// memory into registers as the A operand (16 queries x 32 dims per product), the transposed LDS
// reads of W_UK give the B operand, and wave w produces columns 32w .. 32w+31 for every query
// (fp32 products summed in the matrix core, bf16 out).  sh: nope * AB_WROWB bytes.
constexpr int AB_MFMA_B = 4;
constexpr int AB_WROWB = 288;

typedef short ab_v4s __attribute__((ext_vector_type(4)));
typedef short ab_v8s __attribute__((ext_vector_type(8)));
typedef __bf16 ab_bf16x8 __attribute__((ext_vector_type(8)));
typedef float ab_f32x4 __attribute__((ext_vector_type(4)));

template <int NR>   // qk_nope / 16
__device__ __forceinline__ void absorb_block_mfma(const bf16_t *__restrict__ q_nope, const bf16_t *__restrict__ kv_b,
                                                  int B, int v, bf16_t *__restrict__ q_abs, int cb, int h,
                                                  char *__restrict__ sh, int tid)
{
    constexpr int nope = 16 * NR, KS = nope / 32;
    static_assert(nope % 32 == 0, "qk_nope must be a multiple of 32");
    const int lane = tid & 63, wave = tid >> 6, jj = lane & 15, quad = lane >> 4;
    // stage W_UK[h][:, 128 cb .. 128 cb + 127]: nope rows x 16 pieces of 16 B, NR pieces per thread
    {
        const bf16_t *W = kv_b + (int64_t)h * (nope + v) * AB_L + cb * 128;
        uint4 t[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int pcs = tid + 256 * i, r = pcs >> 4, pc = pcs & 15;
            t[i] = *reinterpret_cast<const uint4 *>(W + (int64_t)r * AB_L + 8 * pc);
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int pcs = tid + 256 * i, r = pcs >> 4, pc = pcs & 15;
            *reinterpret_cast<uint4 *>(sh + r * AB_WROWB + 16 * pc) = t[i];
        }
    }
    __syncthreads();
    // B operand of dims 32 ks + 8 quad + e, column jj of tile nt: rows 32 ks + 8 quad + (0..3 | 4..7)
    const char *wb = sh + (8 * quad + (jj >> 2)) * AB_WROWB + 2 * (32 * wave + 4 * (jj & 3));
    for (int b0 = 0; b0 < B; b0 += 16) {
        const int bq = b0 + jj < B ? b0 + jj : B - 1;
        const bf16_t *qa = q_nope + ((int64_t)bq * AB_H + h) * nope + 8 * quad;
        uint4 a[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a[ks] = *reinterpret_cast<const uint4 *>(qa + 32 * ks);
        ab_f32x4 acc[2] = {ab_f32x4{0.f, 0.f, 0.f, 0.f}, ab_f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const char *p = wb + 32 * ks * AB_WROWB + 32 * nt;
                const ab_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) ab_v4s *)p);
                const ab_v4s hi =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) ab_v4s *)(p + 4 * AB_WROWB));
                const ab_v8s bt = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(ab_bf16x8, a[ks]),
                                                                  __builtin_bit_cast(ab_bf16x8, bt), acc[nt], 0, 0, 0);
            }
        // result register r of lane (jj, quad): query b0 + 4 quad + r, column 16 nt + jj of the wave
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int b = b0 + 4 * quad + r;
                if (b < B) q_abs[((int64_t)b * AB_H + h) * AB_L + cb * 128 + 32 * wave + 16 * nt + jj] = f2bf(acc[nt][r]);
            }
    }
}

}  // namespace mla
