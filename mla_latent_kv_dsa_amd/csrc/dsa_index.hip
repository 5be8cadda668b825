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

// ------------------------------------------------------------------------------------------
// Matrix-core path for 32 heads x 128 dims.  v_mfma_f32_32x32x1_2b_f32 multiplies a 32x1
// column by a 1x32 row and adds it to a 32x32 accumulator, in two independent blocks; with
// one product per output element it rounds exactly like fmaf (checked against fmaf on the
// host for 16.7M random triples).  Chaining it over d = 0..127 therefore reproduces the
// fixed fp32 order bit for bit, at twice the rate of the vector ALU.
//   lane L supplies a = q[L % 32][d] (head) and b = Ic[key L][d]; block 0 covers keys
//   0..31 of the tile, block 1 keys 32..63.  Accumulator register r (0..15) of lane L holds
//   block 0, key L % 32, head 8*(r/4) + 4*(L/32) + r%4; registers 16..31 hold block 1.
// A wave owns a 64-key tile; the key rows are staged through LDS in 32-wide d slices so
// that each lane can read its own key's row (rows padded to avoid bank conflicts), with
// the next slice prefetched into registers while the current one is consumed.
typedef float v32f __attribute__((ext_vector_type(32)));

constexpr int IXM_WAVES = 4;
constexpr int IXM_ROW = 32 + 4;      // floats per staged key row (32 d + pad)
constexpr int IXM_QROW = 128 + 4;    // floats per query row in LDS

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(64 * IXM_WAVES) void index_scores_mfma(const float *__restrict__ q,
                                                                     const float *__restrict__ w, KvView kv,
                                                                     int64_t t_max, int tiles_per_wave,
                                                                     float *__restrict__ scores)
{
    __shared__ float sq[32 * IXM_QROW];
    __shared__ float sw[32];
    __shared__ float sk[IXM_WAVES][64 * IXM_ROW];
    const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n = seq_len_of(kv, b) < t_max ? seq_len_of(kv, b) : t_max;
    const int64_t ntiles = (t_max + 63) / 64;
    const int64_t waves_total = (int64_t)gridDim.x * IXM_WAVES;
    float *out = scores + (int64_t)b * t_max;

    const float4 *qb = reinterpret_cast<const float4 *>(q + (int64_t)b * 32 * 128);
    for (int i = tid; i < 32 * 32; i += 64 * IXM_WAVES) {
        const float4 v = qb[i];
        *reinterpret_cast<float4 *>(&sq[(i >> 5) * IXM_QROW + (i & 31) * 4]) = v;
    }
    if (tid < 32) sw[tid] = w[(int64_t)b * 32 + tid];
    __syncthreads();

    float *skw = sk[wave];
    const int lrow = lane >> 3;          // rows lrow + 8*i of the tile are loaded by this lane
    const int lcol = (lane & 7) * 4;     // float offset inside the 32-wide slice
    const float *qrow = &sq[(lane & 31) * IXM_QROW];
    const bool lo_half = lane < 32;

    for (int it = 0; it < tiles_per_wave; ++it) {
        const int64_t tile = (int64_t)blockIdx.x * IXM_WAVES + wave + (int64_t)it * waves_total;
        if (tile >= ntiles) break;
        const int64_t t0 = tile * 64;
        if (t0 >= n) {
            const int64_t t = t0 + lane;
            if (t < t_max) out[t] = -INFINITY;
            continue;
        }
        const float *src[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t t = t0 + lrow + 8 * i;
            const int64_t row = t < n ? kv_row(kv, b, t) : -1;
            src[i] = row >= 0 ? kv.ic + row * 128 + lcol : nullptr;
        }
        float4 stg[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            stg[i] = src[i] ? *reinterpret_cast<const float4 *>(src[i]) : make_float4(0.f, 0.f, 0.f, 0.f);
        v32f acc;
#pragma unroll
        for (int r = 0; r < 32; ++r) acc[r] = 0.f;
#pragma unroll
        for (int st_ = 0; st_ < 4; ++st_) {
            wave_lds_sync();   // every lane is done reading the previous slice
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<float4 *>(&skw[(lrow + 8 * i) * IXM_ROW + lcol]) = stg[i];
            wave_lds_sync();
            if (st_ < 3) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    stg[i] = src[i] ? *reinterpret_cast<const float4 *>(src[i] + (st_ + 1) * 32)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float4 kk = *reinterpret_cast<const float4 *>(&skw[lane * IXM_ROW + 4 * j]);
                const float4 qq = *reinterpret_cast<const float4 *>(&qrow[st_ * 32 + 4 * j]);
                acc = __builtin_amdgcn_mfma_f32_32x32x1f32(qq.x, kk.x, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x1f32(qq.y, kk.y, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x1f32(qq.z, kk.z, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x1f32(qq.w, kk.w, acc, 0, 0, 0);
            }
        }
        // lanes L and L^32 hold complementary head groups of the same two keys: swap so that
        // lane L holds all 32 heads of key L, then fold them in ascending head order
        float y[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) y[r] = __shfl_xor(lo_half ? acc[16 + r] : acc[r], 32, 64);
        float s = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float a = lo_half ? acc[4 * g + r4] : y[4 * g + r4];
                s = __builtin_fmaf(sw[8 * g + r4], a > 0.f ? a : 0.f, s);
            }
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const float a = lo_half ? y[4 * g + r4] : acc[16 + 4 * g + r4];
                s = __builtin_fmaf(sw[8 * g + 4 + r4], a > 0.f ? a : 0.f, s);
            }
        }
        const int64_t t = t0 + lane;
        if (t < t_max) out[t] = t < n ? s : -INFINITY;
    }
}

mla_status launch_index_scores(const float *q, const float *w, int32_t B, int32_t n_ih, int32_t hd,
                               const KvView &kv, int64_t t_max, float *scores, hipStream_t s)
{
    const int64_t gx = (t_max + 255) / 256;
    if (gx > 0x7fffffff || B > 65535) return fail(MLA_ERR_UNSUPPORTED, "index: grid too large");
    dim3 grid((unsigned)gx, (unsigned)B);
    const bool aligned = ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(kv.ic)) & 15u) == 0;
    if (hd == 128 && n_ih == 32 && aligned) {
        // enough waves for two resident blocks per CU (256 CUs); each wave loops over tiles
        const int64_t ntiles = (t_max + 63) / 64;
        const int64_t want_waves = 2 * 256 * IXM_WAVES;
        int64_t tpw = (ntiles * B + want_waves - 1) / want_waves;
        if (tpw < 1) tpw = 1;
        const int64_t bx = (ntiles + IXM_WAVES * tpw - 1) / (IXM_WAVES * tpw);
        hipLaunchKernelGGL(index_scores_mfma, dim3((unsigned)bx, (unsigned)B), dim3(64 * IXM_WAVES), 0, s, q, w, kv,
                           t_max, (int)tpw, scores);
    } else if (hd == 128 && aligned)
        hipLaunchKernelGGL(index_scores_lane_per_key<128>, grid, dim3(256), 0, s, q, w, n_ih, kv, t_max, scores);
    else
        hipLaunchKernelGGL(index_scores_generic, grid, dim3(256), 0, s, q, w, n_ih, hd, kv, t_max, scores);
    return check_launch("index_scores");
}

}  // namespace mla
