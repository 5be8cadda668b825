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

// One wave per token.  Every load of the token (the kv_a row, the indexer key row, the gains) is
// issued before the first reduction waits on any of them; lane l holds columns l, l + 64, .. .
constexpr int CW_LC = 2048 / 64, CW_RP = 512 / 2 / 64, CW_IC = 256 / 64;   // per-lane capacities

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
    const TIN *cj = comp + j * (int64_t)(L + rope);
    const TIN *kj = ik ? ik + j * (int64_t)hd : nullptr;
    const int half = rope >> 1;
    // all loads first (clamped addresses, masked on use)
    float xl[CW_LC], gl[CW_LC], ra[CW_RP], rb[CW_RP], xk[CW_IC], gk[CW_IC], bk[CW_IC];
#pragma unroll
    for (int u = 0; u < CW_LC; ++u) {
        const int c = lane + 64 * u;
        xl[u] = c < L ? ld(cj + c) : 0.f;
        gl[u] = (c < L && kv_gain) ? kv_gain[c] : 1.f;
    }
#pragma unroll
    for (int u = 0; u < CW_RP; ++u) {
        const int q = lane + 64 * u;
        ra[u] = q < half ? ld(cj + L + 2 * q) : 0.f;
        rb[u] = q < half ? ld(cj + L + 2 * q + 1) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < CW_IC; ++u) {
        const int c = lane + 64 * u;
        xk[u] = (kj && c < hd) ? ld(kj + c) : 0.f;
        gk[u] = (gamma && c < hd) ? gamma[c] : 1.f;
        bk[u] = (beta && c < hd) ? beta[c] : 0.f;
    }
    const int64_t row = cw_row(kv, b, n_seq, p);
    if (row < 0) return;   // wave-uniform
    // Lc = comp[0:L] / sqrt(mean(comp[0:L]^2) + eps) * gain
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < CW_LC; ++u) ss = __builtin_fmaf(xl[u], xl[u], ss);
    ss = wave_sum(ss);
    const float inv = 1.0f / __builtin_sqrtf(ss / (float)L + eps_kv);
    TKV *lc = const_cast<TKV *>(reinterpret_cast<const TKV *>(kv.lc)) + row * L;
#pragma unroll
    for (int u = 0; u < CW_LC; ++u) {
        const int c = lane + 64 * u;
        if (c < L) st(lc + c, xl[u] * inv * gl[u]);
    }
    // Rc = RoPE(comp[L:L+rope]) at the token's position
    TKV *rc = const_cast<TKV *>(reinterpret_cast<const TKV *>(kv.rc)) + row * rope;
#pragma unroll
    for (int u = 0; u < CW_RP; ++u) {
        const int q = lane + 64 * u;
        if (q < half) {
            float lo, hi;
            rope_pair(ra[u], rb[u], q, rope, (double)p, theta, lo, hi);
            st(rc + q, lo);
            st(rc + half + q, hi);
        }
    }
    if (!kj) return;
    // Ic = RoPE over [ix_off, ix_off + ix_rdim) of LayerNorm(ik)
    float s1 = 0.f;
#pragma unroll
    for (int u = 0; u < CW_IC; ++u) s1 += xk[u];
    const float mean = wave_sum(s1) / (float)hd;
    float s2 = 0.f;
#pragma unroll
    for (int u = 0; u < CW_IC; ++u) {
        const int c = lane + 64 * u;
        const float dlt = c < hd ? xk[u] - mean : 0.f;
        s2 = __builtin_fmaf(dlt, dlt, s2);
    }
    const float is = 1.0f / __builtin_sqrtf(wave_sum(s2) / (float)hd + eps_ix);
#pragma unroll
    for (int u = 0; u < CW_IC; ++u) {
        const int c = lane + 64 * u;
        if (c < hd) ys[c] = __builtin_fmaf((xk[u] - mean) * is, gk[u], bk[u]);
    }
    __syncthreads();
    float *ic = const_cast<float *>(kv.ic);
    const int rh = ix_rdim >> 1;
#pragma unroll
    for (int u = 0; u < CW_IC; ++u) {
        const int c = lane + 64 * u;
        if (c >= hd) continue;
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
