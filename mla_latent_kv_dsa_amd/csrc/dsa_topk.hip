// dsa_topk.hip -- top-k causal key selection without a full sort.
// colibri-analysis 06 "MLA attention and KV cache", sec. 2.2: keep the top-2048 causal keys
// (sort + threshold scan into dsa_sel / dsa_nsel).  Here the threshold is found by radix
// select on order-preserving uint32 keys, and the kept positions are compacted in position
// order, which yields the same set and order as sorting.
//
// Order: score descending, then position ascending; -0.0 equals +0.0.
#include "common.h"

namespace mla {

// Order-preserving map fp32 -> uint32 (larger score -> larger key).  -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-wide exclusive scan of one uint32 per thread (blockDim.x == 1024, 16 waves).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *sh_wave, uint32_t *total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh_wave[wave] = x;
    __syncthreads();
    if (wave == 0) {
        uint32_t wv = lane < 16 ? sh_wave[lane] : 0u;
        uint32_t z = wv;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            uint32_t y = __shfl_up(z, o, 64);
            if (lane >= o) z += y;
        }
        if (lane < 16) sh_wave[16 + lane] = z - wv;   // exclusive wave offsets
        if (lane == 15) *total = z;
    }
    __syncthreads();
    const uint32_t r = sh_wave[16 + wave] + x - v;
    __syncthreads();
    return r;
}

// One workgroup of 1024 threads per row.
__global__ __launch_bounds__(1024) void topk_rowwise_kernel(const float *__restrict__ scores, int64_t t_max,
                                                           const int32_t *__restrict__ n_valid, int k,
                                                           int32_t *__restrict__ sel, int32_t *__restrict__ nsel)
{
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh_wave[32];
    __shared__ uint32_t sh_total;
    __shared__ uint32_t sh_prefix, sh_remaining;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const float *s = scores + (int64_t)b * t_max;
    int64_t n = n_valid[b];
    if (n < 0) n = 0;
    if (n > t_max) n = t_max;
    int32_t *out = sel + (int64_t)b * k;
    if (n <= k) {
        for (int i = tid; i < k; i += 1024) out[i] = i < n ? i : -1;
        if (tid == 0) nsel[b] = (int32_t)n;
        return;
    }
    // radix select of the k-th largest key, 8 bits per pass from the top
    uint32_t prefix = 0u, mask = 0u, remaining = (uint32_t)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0u;
        __syncthreads();
        for (int64_t t = tid; t < n; t += 1024) {
            const uint32_t key = order_key(s[t]);
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid == 0) {
            uint32_t cum = 0u;
            int bin = 255;
            for (; bin > 0; --bin) {
                if (cum + hist[bin] >= remaining) break;
                cum += hist[bin];
            }
            sh_remaining = remaining - cum;
            sh_prefix = prefix | ((uint32_t)bin << shift);
        }
        __syncthreads();
        remaining = sh_remaining;
        prefix = sh_prefix;
        mask |= 255u << shift;
    }
    // prefix is the k-th largest key; keep every key above it and the first `remaining`
    // (lowest positions) equal to it.  Each thread owns a contiguous segment.
    const int64_t seg = (n + 1023) / 1024;
    const int64_t t0 = (int64_t)tid * seg;
    const int64_t t1 = t0 + seg < n ? t0 + seg : n;
    uint32_t gt = 0u, eq = 0u;
    for (int64_t t = t0; t < t1; ++t) {
        const uint32_t key = order_key(s[t]);
        gt += key > prefix;
        eq += key == prefix;
    }
    const uint32_t gt_before = block_excl_scan(gt, sh_wave, &sh_total);
    const uint32_t eq_before = block_excl_scan(eq, sh_wave, &sh_total);
    uint32_t e = eq_before;
    uint32_t o = gt_before + (eq_before < remaining ? eq_before : remaining);
    for (int64_t t = t0; t < t1; ++t) {
        const uint32_t key = order_key(s[t]);
        bool take = key > prefix;
        if (key == prefix) {
            take = e < remaining;
            ++e;
        }
        if (take) out[o++] = (int32_t)t;
    }
    if (tid == 0) nsel[b] = k;
}

size_t topk_workspace_bytes(int32_t, int64_t, int32_t) { return 0; }

mla_status launch_topk(const float *scores, int32_t B, int64_t t_max, const int32_t *n_valid, int32_t k,
                       int32_t *sel, int32_t *nsel, void *, size_t, hipStream_t s)
{
    hipLaunchKernelGGL(topk_rowwise_kernel, dim3(B), dim3(1024), 0, s, scores, t_max, n_valid, k, sel, nsel);
    return check_launch("topk_rowwise_kernel");
}

}  // namespace mla
