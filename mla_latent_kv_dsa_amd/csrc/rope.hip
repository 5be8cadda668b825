// rope.hip -- interleaved partial RoPE, in place.
// colibri-analysis 06 "MLA attention and KV cache", sec. 2.1: only the qk_rope tail of a
// head rotates; input pair (a, b) = (x[2j], x[2j+1]) of the tail becomes
// out[j] = a cos - b sin and out[half + j] = b cos + a sin.  The angle pos * theta^(-2j/rope)
// is formed and reduced in double (an fp32 angle at position ~1e5 is off by ~1e-2 rad); the
// rotation itself runs in fp32.
#include "common.h"

namespace mla {

// One (token, head) tail is a "unit"; a block of 256 threads handles 256/half units, one
// thread per rotation pair.  Every thread reads its pair before any thread writes, because
// the half-split output slots of one unit overlap the interleaved input slots of others.
template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(T *__restrict__ x, int64_t n_units, int32_t n_heads,
                                                   int64_t tok_stride, int64_t head_stride,
                                                   int32_t rope_off, int32_t half,
                                                   const int32_t *__restrict__ pos, double theta,
                                                   int32_t units_per_block)
{
    const int tid = threadIdx.x;
    const int u_local = tid / half;
    const int j = tid - u_local * half;
    const int64_t unit = (int64_t)blockIdx.x * units_per_block + u_local;
    const bool active = u_local < units_per_block && unit < n_units;
    T *tail = nullptr;
    float lo = 0.f, hi = 0.f;
    if (active) {
        const int64_t n = unit / n_heads;
        const int32_t h = (int32_t)(unit - n * n_heads);
        tail = x + n * tok_stride + (int64_t)h * head_stride + rope_off;
        rope_pair(ld(tail + 2 * j), ld(tail + 2 * j + 1), j, 2 * half, (double)pos[n], theta, lo, hi);
    }
    __syncthreads();
    if (active) {
        st(tail + j, lo);
        st(tail + half + j, hi);
    }
}

// Tokens with several heads: every head of a token rotates by the same angles, so a block takes one
// token (grid.x) and a run of its heads (grid.y: all of them when there are many tokens, else one
// chunk of 256 / half heads per block so that a few tokens still spread over the chip), forms the
// half (cos, sin) pairs once (threads j < half) and rotates its heads in chunks of whole tails (half
// divides 256): each thread reads its pair, the block syncs (the in-place hazard of one tail), then
// writes.  The same rope_cs / rope_apply arithmetic as rope_pair, so the values equal the per-pair
// kernel's bit for bit; the double-precision angles are formed half times per block instead of once
// per pair.
template <typename T>
__global__ __launch_bounds__(256) void rope_token_kernel(T *__restrict__ x, int32_t n_heads, int64_t tok_stride,
                                                         int64_t head_stride, int32_t rope_off, int32_t half,
                                                         const int32_t *__restrict__ pos, double theta)
{
    __shared__ float s_c[256], s_s[256];
    const int tid = threadIdx.x;
    const int64_t n = blockIdx.x;
    if (tid < half) rope_cs(tid, 2 * half, (double)pos[n], theta, s_c[tid], s_s[tid]);
    __syncthreads();
    T *tok = x + n * tok_stride + rope_off;
    const int upc = 256 / half;                                        // tails per chunk
    const int hpb = (n_heads + (int)gridDim.y - 1) / (int)gridDim.y;   // heads of this block's run
    const int hb = (int)blockIdx.y * hpb, he = hb + hpb < n_heads ? hb + hpb : n_heads;
    const int j = tid % half, hl = tid / half;
    const float c = s_c[j], sn = s_s[j];
    for (int h0 = hb; h0 < he; h0 += upc) {
        const int h = h0 + hl;
        T *tail = tok + (int64_t)h * head_stride;
        float lo = 0.f, hi = 0.f;
        if (h < he) rope_apply(ld(tail + 2 * j), ld(tail + 2 * j + 1), c, sn, lo, hi);
        __syncthreads();
        if (h < he) {
            st(tail + j, lo);
            st(tail + half + j, hi);
        }
    }
}

mla_status launch_rope(void *x, mla_dtype dt, int64_t n_tok, int32_t n_heads, int64_t tok_stride,
                       int64_t head_stride, int32_t rope_off, int32_t rope_dim, const int32_t *pos,
                       double theta, hipStream_t s)
{
    const int32_t half = rope_dim / 2;
    if (n_heads > 1 && half > 0 && 256 % half == 0 && n_tok <= 0x7fffffff) {
        if (n_tok == 0) return MLA_OK;
        // a block per token when the tokens fill the chip, else a block per chunk of heads
        const int upc = 256 / half, nchunk = (n_heads + upc - 1) / upc;
        const int gy = n_tok >= 512 || nchunk > 65535 ? 1 : nchunk;
        const dim3 g((unsigned)n_tok, (unsigned)gy);
        if (dt == MLA_FP32)
            hipLaunchKernelGGL(rope_token_kernel<float>, g, dim3(256), 0, s, (float *)x, n_heads, tok_stride,
                               head_stride, rope_off, half, pos, theta);
        else
            hipLaunchKernelGGL(rope_token_kernel<bf16_t>, g, dim3(256), 0, s, (bf16_t *)x, n_heads, tok_stride,
                               head_stride, rope_off, half, pos, theta);
        return check_launch("rope_token_kernel");
    }
    const int32_t upb = 256 / half;
    const int64_t n_units = n_tok * n_heads;
    const int64_t blocks = (n_units + upb - 1) / upb;
    if (blocks > 0x7fffffff) return fail(MLA_ERR_UNSUPPORTED, "rope: too many units");
    if (dt == MLA_FP32)
        hipLaunchKernelGGL(rope_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, (float *)x, n_units,
                           n_heads, tok_stride, head_stride, rope_off, half, pos, theta, upb);
    else
        hipLaunchKernelGGL(rope_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, s, (bf16_t *)x, n_units,
                           n_heads, tok_stride, head_stride, rope_off, half, pos, theta, upb);
    return check_launch("rope_kernel");
}

// Decode queries: y[b][h] = RoPE of the tail x[b][h][0..rope) at position seq_len[b] - 1 (the
// query's own position, the last cached token), out of place.  grid (ceil(B * H * half / 256)).
template <typename T>
__global__ __launch_bounds__(256) void rope_decode_kernel(const T *__restrict__ x, T *__restrict__ y, int32_t B,
                                                          int32_t n_heads, int32_t half, KvView kv, double theta)
{
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= (int64_t)B * n_heads * half) return;
    const int64_t unit = p / half;
    const int j = (int)(p - unit * half);
    const int b = (int)(unit / n_heads);
    const int64_t sl = seq_len_of(kv, b);
    float lo, hi;
    rope_pair(ld(x + unit * 2 * half + 2 * j), ld(x + unit * 2 * half + 2 * j + 1), j, 2 * half,
              (double)(sl > 0 ? sl - 1 : 0), theta, lo, hi);
    st(y + unit * 2 * half + j, lo);
    st(y + unit * 2 * half + half + j, hi);
}

mla_status launch_rope_decode(const void *x, void *y, mla_dtype dt, int32_t B, int32_t n_heads, int32_t rope_dim,
                              const KvView &kv, double theta, hipStream_t s)
{
    const int32_t half = rope_dim / 2;
    const int64_t n = (int64_t)B * n_heads * half;
    if (n == 0) return MLA_OK;
    const int64_t blocks = (n + 255) / 256;
    if (blocks > 0x7fffffff) return fail(MLA_ERR_UNSUPPORTED, "rope: too many units");
    if (dt == MLA_FP32)
        hipLaunchKernelGGL(rope_decode_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, (const float *)x,
                           (float *)y, B, n_heads, half, kv, theta);
    else
        hipLaunchKernelGGL(rope_decode_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, s, (const bf16_t *)x,
                           (bf16_t *)y, B, n_heads, half, kv, theta);
    return check_launch("rope_decode_kernel");
}

}  // namespace mla
