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

// The same for the GLM-5.2 geometry (kv_lora 512, qk_rope 64, index_hd 128 or no indexer key,
// an even rotated slice): lane l holds latent columns 8 l .. 8 l + 7 (one or two 16-byte loads and
// stores), the Rc pair l (l < 32) and indexer columns 2 l, 2 l + 1, so that an indexer pair of the
// rotated slice is already in one lane and nothing goes through LDS.  The generic kernel above
// unrolls its loops for kv_lora up to 2048 with guards, and spends most of its time issuing them.
// The rotations are the same rope_pair calls (Rc equals mla_rope_interleave bit for bit); the sums
// run in another order than the generic kernel's.
template <typename T> struct CwVec;
template <> struct CwVec<float> {
    static __device__ __forceinline__ void ld8(const float *p, float *x)
    {
        const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
    static __device__ __forceinline__ void st8(float *p, const float *x)
    {
        *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
        *reinterpret_cast<float4 *>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
    }
    static __device__ __forceinline__ void ld2(const float *p, float &a, float &b)
    {
        const float2 v = *reinterpret_cast<const float2 *>(p);
        a = v.x;
        b = v.y;
    }
};
template <> struct CwVec<bf16_t> {
    static __device__ __forceinline__ void ld8(const bf16_t *p, float *x)
    {
        const uint4 v = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void st8(bf16_t *p, const float *x)
    {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f2bf(x[2 * i]) | ((uint32_t)f2bf(x[2 * i + 1]) << 16);
        *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    static __device__ __forceinline__ void ld2(const bf16_t *p, float &a, float &b)
    {
        const uint32_t v = *reinterpret_cast<const uint32_t *>(p);
        a = __uint_as_float(v << 16);
        b = __uint_as_float(v & 0xffff0000u);
    }
};

constexpr int CWF_L = 512, CWF_R = 64, CWF_HD = 128;

template <typename TIN, typename TKV, bool IX>
__global__ __launch_bounds__(64 * CW_TPW) void cache_write_fast(const TIN *__restrict__ comp, const TIN *__restrict__ ik,
                                                                const int32_t *__restrict__ seq,
                                                                const int32_t *__restrict__ pos, int64_t n_tok,
                                                                int n_seq, KvView kv,
                                                                const float *__restrict__ kv_gain,
                                                                const float *__restrict__ gamma,
                                                                const float *__restrict__ beta, int ix_off, int ix_rdim,
                                                                float eps_kv, float eps_ix, double theta)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t j = (int64_t)blockIdx.x * CW_TPW + wave;
    if (j >= n_tok) return;   // (no barrier in this kernel)
    const int b = seq[j];
    const int64_t p = pos[j];
    const TIN *cj = comp + j * (int64_t)(CWF_L + CWF_R);
    // every load first
    float x[8], g[8], ra = 0.f, rb = 0.f, k0 = 0.f, k1 = 0.f, g0 = 1.f, g1 = 1.f, b0 = 0.f, b1 = 0.f;
    CwVec<TIN>::ld8(cj + 8 * lane, x);
    if (kv_gain) CwVec<float>::ld8(kv_gain + 8 * lane, g);
    else
#pragma unroll
        for (int i = 0; i < 8; ++i) g[i] = 1.f;
    if (lane < CWF_R / 2) CwVec<TIN>::ld2(cj + CWF_L + 2 * lane, ra, rb);
    if (IX) {
        CwVec<TIN>::ld2(ik + j * (int64_t)CWF_HD + 2 * lane, k0, k1);
        if (gamma) CwVec<float>::ld2(gamma + 2 * lane, g0, g1);
        if (beta) CwVec<float>::ld2(beta + 2 * lane, b0, b1);
    }
    const int64_t row = cw_row(kv, b, n_seq, p);
    if (row < 0) return;   // wave-uniform: no row, nothing written
    // Lc = comp[0:L] / sqrt(mean(comp[0:L]^2) + eps) * gain
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(x[i], x[i], ss);
    ss = wave_sum(ss);
    const float inv = 1.0f / __builtin_sqrtf(ss / (float)CWF_L + eps_kv);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = x[i] * inv * g[i];
    CwVec<TKV>::st8(const_cast<TKV *>(reinterpret_cast<const TKV *>(kv.lc)) + row * CWF_L + 8 * lane, x);
    // Ic = RoPE over [ix_off, ix_off + ix_rdim) of LayerNorm(ik)
    float y0 = 0.f, y1 = 0.f;
    const int c0 = 2 * lane;
    const bool ic_rot = IX && c0 >= ix_off && c0 < ix_off + ix_rdim;   // pair (c0, c0 + 1) is pair qi of the slice
    const int qi = (c0 - ix_off) >> 1;
    float *ic = const_cast<float *>(kv.ic);
    auto ic_at = [&](int c) {
        return kv.ic_tiled ? ic + ((row >> 6) * (CWF_HD >> 2) + (c >> 2)) * 256 + (row & 63) * 4 + (c & 3)
                           : ic + row * CWF_HD + c;
    };
    if (IX) {
        const float mean = wave_sum(k0 + k1) / (float)CWF_HD;
        const float d0 = k0 - mean, d1 = k1 - mean;
        const float is = 1.0f / __builtin_sqrtf(wave_sum(__builtin_fmaf(d0, d0, d1 * d1)) / (float)CWF_HD + eps_ix);
        y0 = __builtin_fmaf(d0 * is, g0, b0);
        y1 = __builtin_fmaf(d1 * is, g1, b1);
        if (!ic_rot) {
            *ic_at(c0) = y0;
            *ic_at(c0 + 1) = y1;
        }
    }
    // The rotations, one rope_pair per lane: lane l < 32 takes Rc pair l, a lane >= 32 the indexer
    // pair it holds (with the rotated slice in the upper half of the key, the usual place, every
    // lane has exactly one).  A single call site keeps the wave on one pass through the fp64 angle
    // and sincos, which dominate the kernel; as two calls under lane conditions the wave ran both.
    const bool rc_job = lane < CWF_R / 2;
    float lo, hi;
    rope_pair(rc_job ? ra : y0, rc_job ? rb : y1, rc_job ? lane : qi, rc_job ? CWF_R : ix_rdim, (double)p, theta,
              lo, hi);
    if (rc_job) {
        TKV *rc = const_cast<TKV *>(reinterpret_cast<const TKV *>(kv.rc)) + row * CWF_R;
        st(rc + lane, lo);
        st(rc + CWF_R / 2 + lane, hi);
    } else if (ic_rot) {
        *ic_at(ix_off + qi) = lo;
        *ic_at(ix_off + (ix_rdim >> 1) + qi) = hi;
    }
    if (rc_job && ic_rot) {   // a rotated slice reaching into the lower half of the key
        rope_pair(y0, y1, qi, ix_rdim, (double)p, theta, lo, hi);
        *ic_at(ix_off + qi) = lo;
        *ic_at(ix_off + (ix_rdim >> 1) + qi) = hi;
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
    const uintptr_t al = reinterpret_cast<uintptr_t>(comp) | reinterpret_cast<uintptr_t>(ik) |
                         reinterpret_cast<uintptr_t>(kv.lc) | reinterpret_cast<uintptr_t>(kv.rc) |
                         reinterpret_cast<uintptr_t>(kv.ic) | reinterpret_cast<uintptr_t>(kv_gain) |
                         reinterpret_cast<uintptr_t>(gamma) | reinterpret_cast<uintptr_t>(beta);
    const bool fast = L == CWF_L && rope == CWF_R && (!ik || (hd == CWF_HD && ix_off % 2 == 0)) && (al & 15u) == 0;
    if (fast) {
#define MLA_CWF(TI, TK)                                                                                            \
    do {                                                                                                           \
        if (ik)                                                                                                    \
            hipLaunchKernelGGL((cache_write_fast<TI, TK, true>), g, blk, 0, s, (const TI *)comp, (const TI *)ik, seq, \
                               pos, n, n_seq, kv, kv_gain, gamma, beta, ix_off, ix_rdim, eps_kv, eps_ix, theta);   \
        else                                                                                                       \
            hipLaunchKernelGGL((cache_write_fast<TI, TK, false>), g, blk, 0, s, (const TI *)comp, (const TI *)ik,  \
                               seq, pos, n, n_seq, kv, kv_gain, gamma, beta, ix_off, ix_rdim, eps_kv, eps_ix,      \
                               theta);                                                                             \
    } while (0)
        if (in_dt == MLA_FP32 && kv_dt == MLA_FP32) MLA_CWF(float, float);
        else if (in_dt == MLA_FP32) MLA_CWF(float, bf16_t);
        else if (kv_dt == MLA_FP32) MLA_CWF(bf16_t, float);
        else MLA_CWF(bf16_t, bf16_t);
#undef MLA_CWF
        return check_launch("cache_write_fast");
    }
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
