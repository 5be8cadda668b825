// cache_write.hip -- writes new tokens into the compressed cache.
// colibri-analysis 06 "MLA attention and KV cache", sec. 2.1 (KV path): the kv_a output comp
// splits into a kv_lora part, RMS-normalised (kv_a_ln) into the latent row Lc[pos], and a
// qk_rope part, rotated by the interleaved RoPE into the shared key row Rc[pos]; sec. 2.2: the
// indexer key (the ix_wk output) is LayerNorm'd (eps 1e-6 on the page) and rotated into Ic[pos].
//
// One wave per token.  Sums of squares and the LayerNorm moments are wave reductions in fp32
// (two passes for the variance); the rotations use the same rope_pair as mla_rope_interleave, so
// a token's Rc row equals that call's output on the same tail, bit for bit.
#include "common.h"

namespace mla {

// Pool row of (sequence b, position p), or -1 outside the view (seq, position or pool bounds).
__device__ __forceinline__ int64_t cw_row(const KvView &v, int b, int n_seq, int64_t p)
{
    if (b < 0 || b >= n_seq || p < 0) return -1;
    if (v.bt) {
        if (p >= (int64_t)v.max_blocks * v.bs) return -1;
        return kv_row(v, b, p);
    }
    const int64_t r = (int64_t)b * v.seq_stride + p;
    return r < v.rows ? r : -1;
}

template <typename TIN, typename TKV>
__global__ __launch_bounds__(64) void cache_write_kernel(const TIN *__restrict__ comp, const TIN *__restrict__ ik,
                                                         const int32_t *__restrict__ seq,
                                                         const int32_t *__restrict__ pos, int n_seq, KvView kv,
                                                         int L, int rope, int hd, const float *__restrict__ kv_gain,
                                                         const float *__restrict__ gamma,
                                                         const float *__restrict__ beta, int ix_off, int ix_rdim,
                                                         float eps_kv, float eps_ix, double theta)
{
    __shared__ float ys[256];
    const int64_t j = blockIdx.x;
    const int lane = threadIdx.x;
    const int b = seq[j];
    const int64_t p = pos[j];
    const int64_t row = cw_row(kv, b, n_seq, p);
    if (row < 0) return;   // wave-uniform
    const TIN *cj = comp + j * (int64_t)(L + rope);
    // Lc = comp[0:L] / sqrt(mean(comp[0:L]^2) + eps) * gain
    float ss = 0.f;
    for (int c = lane; c < L; c += 64) {
        const float x = ld(cj + c);
        ss = __builtin_fmaf(x, x, ss);
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / __builtin_sqrtf(ss / (float)L + eps_kv);
    TKV *lc = const_cast<TKV *>(reinterpret_cast<const TKV *>(kv.lc)) + row * L;
    for (int c = lane; c < L; c += 64) {
        const float g = kv_gain ? kv_gain[c] : 1.f;
        st(lc + c, ld(cj + c) * inv * g);
    }
    // Rc = RoPE(comp[L:L+rope]) at the token's position
    const int half = rope >> 1;
    TKV *rc = const_cast<TKV *>(reinterpret_cast<const TKV *>(kv.rc)) + row * rope;
    for (int q = lane; q < half; q += 64) {
        float lo, hi;
        rope_pair(ld(cj + L + 2 * q), ld(cj + L + 2 * q + 1), q, rope, (double)p, theta, lo, hi);
        st(rc + q, lo);
        st(rc + half + q, hi);
    }
    if (!ik) return;
    // Ic = RoPE over [ix_off, ix_off + ix_rdim) of LayerNorm(ik)
    const TIN *kj = ik + j * (int64_t)hd;
    float s1 = 0.f;
    for (int c = lane; c < hd; c += 64) s1 += ld(kj + c);
    const float mean = wave_sum(s1) / (float)hd;
    float s2 = 0.f;
    for (int c = lane; c < hd; c += 64) {
        const float d = ld(kj + c) - mean;
        s2 = __builtin_fmaf(d, d, s2);
    }
    const float is = 1.0f / __builtin_sqrtf(wave_sum(s2) / (float)hd + eps_ix);
    for (int c = lane; c < hd; c += 64) {
        const float y = (ld(kj + c) - mean) * is;
        ys[c] = __builtin_fmaf(y, gamma ? gamma[c] : 1.f, beta ? beta[c] : 0.f);
    }
    __syncthreads();
    float *ic = const_cast<float *>(kv.ic);
    const int rh = ix_rdim >> 1;
    for (int c = lane; c < hd; c += 64) {
        float o = ys[c];
        const int sidx = c - ix_off;
        if (sidx >= 0 && sidx < ix_rdim) {
            const int q = sidx < rh ? sidx : sidx - rh;
            float lo, hi;
            rope_pair(ys[ix_off + 2 * q], ys[ix_off + 2 * q + 1], q, ix_rdim, (double)p, theta, lo, hi);
            o = sidx < rh ? lo : hi;
        }
        float *dst = kv.ic_tiled ? ic + ((row >> 6) * (hd >> 2) + (c >> 2)) * 256 + (row & 63) * 4 + (c & 3)
                                 : ic + row * hd + c;
        *dst = o;
    }
}

mla_status launch_cache_write(const void *comp, const void *ik, mla_dtype in_dt, int64_t n, const int32_t *seq,
                              const int32_t *pos, int32_t n_seq, const KvView &kv, mla_dtype kv_dt, int32_t L,
                              int32_t rope, int32_t hd, const float *kv_gain, const float *gamma, const float *beta,
                              int32_t ix_off, int32_t ix_rdim, float eps_kv, float eps_ix, double theta,
                              hipStream_t s)
{
    if (n == 0) return MLA_OK;
    if (n > 0x7fffffff) return fail(MLA_ERR_UNSUPPORTED, "cache write: too many tokens");
    const dim3 g((unsigned)n), blk(64);
#define MLA_CW(TI, TK)                                                                                            \
    hipLaunchKernelGGL((cache_write_kernel<TI, TK>), g, blk, 0, s, (const TI *)comp, (const TI *)ik, seq, pos, n_seq, \
                       kv, L, rope, hd, kv_gain, gamma, beta, ix_off, ix_rdim, eps_kv, eps_ix, theta)
    if (in_dt == MLA_FP32 && kv_dt == MLA_FP32) MLA_CW(float, float);
    else if (in_dt == MLA_FP32) MLA_CW(float, bf16_t);
    else if (kv_dt == MLA_FP32) MLA_CW(bf16_t, float);
    else MLA_CW(bf16_t, bf16_t);
#undef MLA_CW
    return check_launch("cache_write_kernel");
}

}  // namespace mla
