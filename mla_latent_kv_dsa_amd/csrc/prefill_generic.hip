// prefill_generic.hip -- non-absorbed causal prefill for any head geometry (fp32 or bf16
// inputs, fp32 arithmetic).  colibri-analysis 06 "MLA attention and KV cache", sec. 2.3,
// non-absorbed path: one kv_b matmul rebuilds k_nope and v of every token, then causal
// attention with score = q_pass . k_nope + q_rot . k_rot, softmax and value accumulation.
//   1. kvb_gemm_generic  KV[t][h*(nope+v) + r] = kv_b[h*(nope+v) + r] . Lc(t)   (fp32 scratch)
//   2. attn_generic      per (query, head): online softmax over keys t <= pos_base + i
#include "common.h"
#include "prefill_plan.h"

namespace mla {

template <typename T>
__global__ __launch_bounds__(256) void kvb_gemm_generic(KvView kv, const T *__restrict__ kv_b, int64_t Tn, int N,
                                                        int L, float *__restrict__ out)
{
    __shared__ float As[16][64 + 1];
    __shared__ float Bs[16][64 + 1];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int64_t m0 = (int64_t)blockIdx.y * 64;
    const int n0 = blockIdx.x * 64;
    const T *lc = reinterpret_cast<const T *>(kv.lc);
    float acc[4][4] = {};
    for (int k0 = 0; k0 < L; k0 += 16) {
        for (int e = tid; e < 1024; e += 256) {
            const int r = e >> 4, kk = e & 15;
            const int64_t t = m0 + r;
            float a = 0.f;
            if (t < Tn && k0 + kk < L) {
                const int64_t row = kv_row(kv, 0, t);
                if (row >= 0) a = ld(lc + row * L + k0 + kk);
            }
            As[kk][r] = a;
            const int nn = e >> 4;
            float w = 0.f;
            if (n0 + nn < N && k0 + kk < L) w = ld(kv_b + (int64_t)(n0 + nn) * L + k0 + kk);
            Bs[kk][nn] = w;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float a[4], w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = m0 + ty * 4 + i;
        if (t >= Tn) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n < N) out[t * N + n] = acc[i][j];
        }
    }
}

constexpr int kPChunk = 256;

// mask (optional): query i attends key t only if bit t % 32 of mask[(t / 32) * mask_stride + i] is set
template <typename T, typename O>
__global__ __launch_bounds__(256) void attn_generic(const T *__restrict__ q, const float *__restrict__ kvw, KvView kv,
                                                    int H, int nope, int rope, int v, int pos_base,
                                                    float sm_scale, O *__restrict__ out,
                                                    const uint32_t *__restrict__ mask, int mask_stride)
{
    extern __shared__ int64_t sh_rows[];
    int64_t *srow = sh_rows;                                   // [kPChunk] pool rows
    float *ss = reinterpret_cast<float *>(srow + kPChunk);    // [kPChunk]
    float *sq = ss + kPChunk;                                  // [nope + rope]
    __shared__ float red[8];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i = blockIdx.x, h = blockIdx.y;
    const int qh = nope + rope;
    const int N = H * (nope + v);
    const T *rc = reinterpret_cast<const T *>(kv.rc);
    const int64_t nk = (int64_t)pos_base + i + 1;
    for (int c = tid; c < qh; c += 256) sq[c] = ld(q + ((int64_t)i * H + h) * qh + c);
    float m = -INFINITY, l = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};   // v <= 1024
    for (int64_t jc = 0; jc < nk; jc += kPChunk) {
        const int cnt = (int)(nk - jc < kPChunk ? nk - jc : kPChunk);
        __syncthreads();
        for (int e = tid; e < cnt; e += 256) srow[e] = kv_row(kv, 0, jc + e);
        __syncthreads();
        for (int e = wave; e < cnt; e += 4) {
            const int64_t t = jc + e;
            const int64_t row = srow[e];
            const float *kt = kvw + t * N + (int64_t)h * (nope + v);
            float p = 0.f;
            for (int c = lane; c < nope; c += 64) p = fmaf(sq[c], kt[c], p);
            if (row >= 0)
                for (int c = lane; c < rope; c += 64) p = fmaf(sq[nope + c], ld(rc + row * rope + c), p);
            p = wave_sum(p);
            // a key without a pool row (a block-table hole) is not attended, as in the decode
            const bool keep = row >= 0 && (!mask || ((mask[(t >> 5) * (int64_t)mask_stride + i] >> (t & 31)) & 1u));
            if (lane == 0) ss[e] = keep ? p * sm_scale : -INFINITY;
        }
        __syncthreads();
        float x = tid < cnt ? ss[tid] : -INFINITY;
        x = wave_max(x);
        if (lane == 0) red[wave] = x;
        __syncthreads();
        const float nm = fmaxf(m, fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
        const float ns = nm == -INFINITY ? 0.f : nm;   // no attended key yet (a key mask): P = 0
        const float scale = __expf(m - ns);
        __syncthreads();
        float pv = 0.f;
        if (tid < cnt) {
            pv = __expf(ss[tid] - ns);
            ss[tid] = pv;
        }
        pv = wave_sum(pv);
        if (lane == 0) red[4 + wave] = pv;
        __syncthreads();
        l = l * scale + ((red[4] + red[5]) + (red[6] + red[7]));
        m = nm;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = tid + 256 * r;
            if (j < v) {
                float a = acc[r] * scale;
                const float *vt = kvw + jc * N + (int64_t)h * (nope + v) + nope + j;
                for (int e = 0; e < cnt; ++e) a = fmaf(ss[e], vt[(int64_t)e * N], a);
                acc[r] = a;
            }
        }
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int j = tid + 256 * r;
        if (j < v) st(out + ((int64_t)i * H + h) * v + j, acc[r] * inv);
    }
}

size_t prefill_generic_ws(const mla_dims &d, int32_t, int64_t T)
{
    return (size_t)T * d.n_heads * (d.qk_nope + d.v_head) * 4 + 256;
}

template <typename T>
static mla_status run_prefill_generic(const void *q, const void *kv_b, const mla_dims &d, const KvView &kv, int32_t S,
                                      int32_t pos_base, float sm_scale, void *out, mla_dtype out_dt, void *ws,
                                      hipStream_t s, const uint32_t *mask, int mask_stride)
{
    const int H = d.n_heads, nope = d.qk_nope, rope = d.qk_rope, v = d.v_head, L = d.kv_lora;
    const int64_t Tn = (int64_t)pos_base + S;
    const int N = H * (nope + v);
    float *kvw = reinterpret_cast<float *>(ws);
    const int64_t gy = (Tn + 63) / 64;
    if (gy > 65535) return fail(MLA_ERR_UNSUPPORTED, "prefill: too many tokens for the generic path");
    hipLaunchKernelGGL(kvb_gemm_generic<T>, dim3((N + 63) / 64, (unsigned)gy), dim3(256), 0, s, kv, (const T *)kv_b, Tn,
                       N, L, kvw);
    mla_status st = check_launch("kvb_gemm_generic");
    if (st) return st;
    const size_t shm = (size_t)(nope + rope + kPChunk) * 4 + (size_t)kPChunk * 8;
    if (H > 65535) return fail(MLA_ERR_UNSUPPORTED, "prefill: too many heads");
    if (out_dt == MLA_FP32)
        hipLaunchKernelGGL((attn_generic<T, float>), dim3(S, H), dim3(256), shm, s, (const T *)q, kvw, kv, H, nope, rope,
                           v, pos_base, sm_scale, (float *)out, mask, mask_stride);
    else
        hipLaunchKernelGGL((attn_generic<T, bf16_t>), dim3(S, H), dim3(256), shm, s, (const T *)q, kvw, kv, H, nope,
                           rope, v, pos_base, sm_scale, (bf16_t *)out, mask, mask_stride);
    return check_launch("attn_generic");
}

mla_status launch_prefill_generic(const void *q, const void *kv_b, mla_dtype dt, const mla_dims &d, const KvView &kv,
                                  int32_t S, int32_t pos_base, float sm_scale, void *out, mla_dtype out_dt, void *ws,
                                  hipStream_t s, const uint32_t *mask, int mask_stride)
{
    if (dt == MLA_FP32)
        return run_prefill_generic<float>(q, kv_b, d, kv, S, pos_base, sm_scale, out, out_dt, ws, s, mask, mask_stride);
    return run_prefill_generic<bf16_t>(q, kv_b, d, kv, S, pos_base, sm_scale, out, out_dt, ws, s, mask, mask_stride);
}

}  // namespace mla
