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

// One wave per token, CW_TPW tokens per workgroup.  Every load of the token (the kv_a row, the indexer key row, the gains) is
// issued before the first reduction waits on any of them; lane l holds columns l, l + 64, .. .
constexpr int CW_LC = 2048 / 64, CW_RP = 512 / 2 / 64, CW_IC = 256 / 64;   // per-lane capacities

constexpr int CW_TPW = 4;   // tokens (waves) per workgroup

template <typename TIN, typename TKV>
__global__ __launch_bounds__(64 * CW_TPW) void cache_write_kernel(const TIN *__restrict__ comp,
                                                                  const TIN *__restrict__ ik,
                                                                  const int32_t *__restrict__ seq,
                                                                  const int32_t *__restrict__ pos, int64_t n_tok,
                                                                  int n_seq, KvView kv, int L, int rope, int hd,
                                                                  const float *__restrict__ kv_gain,
                                                                  const float *__restrict__ gamma,
                                                                  const float *__restrict__ beta, int ix_off,
                                                                  int ix_rdim, float eps_kv, float eps_ix, double theta)
{
    __shared__ float ys_all[CW_TPW][256];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float *ys = ys_all[wave];
    const int64_t jt = (int64_t)blockIdx.x * CW_TPW + wave;
    const bool live = jt < n_tok;              // waves past the last token only pass the barrier
    const int64_t j = live ? jt : n_tok - 1;
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
    const int64_t row = live ? cw_row(kv, b, n_seq, p) : -1;
    const bool ok = row >= 0;   // wave-uniform; a wave without a row writes nothing
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
        if (ok && c < L) st(lc + c, xl[u] * inv * gl[u]);
    }
    TKV *rc = const_cast<TKV *>(reinterpret_cast<const TKV *>(kv.rc)) + row * rope;
    // Ic = RoPE over [ix_off, ix_off + ix_rdim) of LayerNorm(ik)
    float *ic = const_cast<float *>(kv.ic);
    const int rh = kj ? ix_rdim >> 1 : 0;
    auto ic_at = [&](int c) {
        return kv.ic_tiled ? ic + ((row >> 6) * (hd >> 2) + (c >> 2)) * 256 + (row & 63) * 4 + (c & 3)
                           : ic + row * hd + c;
    };
    if (kj) {
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
            if (c < hd) {
                const float y = __builtin_fmaf((xk[u] - mean) * is, gk[u], bk[u]);
                ys[c] = y;
                if (ok && (c < ix_off || c >= ix_off + ix_rdim)) *ic_at(c) = y;   // dims outside the rotated slice
            }
        }
        __syncthreads();
    }
    // the rotations: pair job i < half is pair i of the Rc tail (comp[L:L+rope], held in ra/rb by
    // lane i % 64), job half + q pair q of the Ic slice; every lane takes jobs lane, lane + 64, .. so
    // each pair's angle (fp64) is formed once
    for (int u = 0; ok && u * 64 < half + rh; ++u) {
        const int pi = lane + 64 * u;
        if (pi >= half + rh) break;
        const bool is_rc = pi < half;
        const int q = is_rc ? pi : pi - half;
        float a = 0.f, bb = 0.f;
        if (is_rc) {
#pragma unroll
            for (int v = 0; v < CW_RP; ++v)
                if (v == u) {
                    a = ra[v];
                    bb = rb[v];
                }
        } else {
            a = ys[ix_off + 2 * q];
            bb = ys[ix_off + 2 * q + 1];
        }
        float lo, hi;
        rope_pair(a, bb, q, is_rc ? rope : ix_rdim, (double)p, theta, lo, hi);
        if (is_rc) {
            st(rc + q, lo);
            st(rc + half + q, hi);
        } else {
            *ic_at(ix_off + q) = lo;
            *ic_at(ix_off + rh + q) = hi;
        }
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
    const dim3 g((unsigned)((n + CW_TPW - 1) / CW_TPW)), blk(64 * CW_TPW);
#define MLA_CW(TI, TK)                                                                                            \
    hipLaunchKernelGGL((cache_write_kernel<TI, TK>), g, blk, 0, s, (const TI *)comp, (const TI *)ik, seq, pos, n, \
                       n_seq, kv, L, rope, hd, kv_gain, gamma, beta, ix_off, ix_rdim, eps_kv, eps_ix, theta)
    if (in_dt == MLA_FP32 && kv_dt == MLA_FP32) MLA_CW(float, float);
    else if (in_dt == MLA_FP32) MLA_CW(float, bf16_t);
    else if (kv_dt == MLA_FP32) MLA_CW(bf16_t, float);
    else MLA_CW(bf16_t, bf16_t);
#undef MLA_CW
    return check_launch("cache_write_kernel");
}

}  // namespace mla
