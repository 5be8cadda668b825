// attention.hip -- attention of S queries of one sequence at positions pos_base .. pos_base + S - 1
// (colibri-analysis 06 "MLA attention and KV cache", sec. 2: Tk = pos_base + S), on either path of
// sec. 2.3 as the g_absorb rule picks it: -1 absorbs when S <= 4 (decode, draft verification), 0
// never, 1 always.  Query i sees keys 0 .. pos_base + i, optionally restricted to its own
// selection (sec. 2.2, the DSA top-k of that query).
//   absorbed      the decode kernels over S launch rows of the same sequence (KvView.qps = S):
//                 q split into its nope and rope parts, W_UK folded into every query, scores against
//                 Lc / Rc, softmax, latent accumulation, W_UV
//   non-absorbed  the prefill kernels (kv_b GEMM rebuilding k_nope and v, causal attention); a
//                 selection becomes a per-query key bitmap that the attention applies tile by tile
#include "common.h"

namespace mla {

bool attention_absorbs(int32_t S, int32_t g_absorb) { return g_absorb > 0 || (g_absorb < 0 && S <= 4); }

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// mask geometry for T keys and S queries: words per query column (two per 64-key tile), and the
// padded column count (query blocks of 128 read whole blocks)
static int64_t mask_groups(int64_t T) { return 2 * ((T + 63) / 64); }
static int64_t mask_cols(int32_t S) { return ((int64_t)S + 127) / 128 * 128; }

size_t attention_workspace_bytes(const mla_dims &d, int32_t S, int64_t T, int32_t sel_stride, bool absorbed,
                                 mla_dtype dt)
{
    const size_t esz = dt == MLA_FP32 ? 4 : 2;
    if (absorbed) {
        const int64_t max_keys = sel_stride > 0 ? sel_stride : T;
        return 256 + al256((size_t)S * d.n_heads * (d.qk_nope + d.qk_rope) * esz) +
               al256(decode_workspace_bytes(d, S, max_keys, dt));
    }
    size_t m = sel_stride > 0 ? al256((size_t)mask_groups(T) * mask_cols(S) * 4) : 0;
    return 256 + m + al256(prefill_workspace_bytes(d, S, T, dt));
}

// q [S][H][nope + rope] -> qn [S][H][nope], qr [S][H][rope] (element copies)
template <typename E>
__global__ __launch_bounds__(256) void split_q_kernel(const E *__restrict__ q, E *__restrict__ qn, E *__restrict__ qr,
                                                      int64_t units, int nope, int rope)
{
    const int qh = nope + rope;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= units * qh) return;
    const int64_t u = e / qh;
    const int c = (int)(e - u * qh);
    if (c < nope) qn[u * nope + c] = q[e];
    else qr[u * rope + (c - nope)] = q[e];
}

// Key bitmap of the selections: column i (query i), word g holds keys 32 g .. 32 g + 31.  Workgroup
// (c, r) builds the words g in [MASK_GCH r, MASK_GCH (r + 1)) of the MASK_QB columns c MASK_QB ..
// in LDS, then writes them out row by row, MASK_QB consecutive words at a time, so every word of the
// mask is written.  The selection rows of its MASK_QB queries are one contiguous range of sel; the
// workgroup reads it flat, MASK_LD entries per thread in flight, and sets the bits of the kept
// positions in its key range with LDS atomics.
constexpr int MASK_QB = 32, MASK_GCH = 256, MASK_NT = 512, MASK_LD = 8;

__global__ __launch_bounds__(MASK_NT) void sel_mask_kernel(const int32_t *__restrict__ sel,
                                                           const int32_t *__restrict__ nsel, int sel_stride, int S,
                                                           int64_t T, int64_t groups, int64_t cols,
                                                           uint32_t *__restrict__ mask)
{
    __shared__ uint32_t m[MASK_GCH * MASK_QB];
    __shared__ int ns[MASK_QB];
    const int tid = threadIdx.x;
    const int64_t c0 = (int64_t)blockIdx.x * MASK_QB, g0 = (int64_t)blockIdx.y * MASK_GCH;
    const int64_t ng = groups - g0 < MASK_GCH ? groups - g0 : MASK_GCH;
    for (int e = tid; e < MASK_GCH * MASK_QB; e += MASK_NT) m[e] = 0u;
    if (tid < MASK_QB) {
        int n = c0 + tid < S ? nsel[c0 + tid] : 0;
        ns[tid] = n < 0 ? 0 : (n > sel_stride ? sel_stride : n);
    }
    __syncthreads();
    const int64_t t_lo = 32 * g0, t_hi = (32 * (g0 + ng) < T) ? 32 * (g0 + ng) : T;
    const int64_t qn = S - c0 < MASK_QB ? S - c0 : MASK_QB;
    // entries of the workgroup's rows of sel: below MASK_QB * 2^19 = 2^24 (the entry point bounds
    // sel_stride), so 32-bit indices, and the row of entry f from an fp32 reciprocal (exact below
    // 2^24) corrected by one step
    const int total = qn > 0 ? (int)qn * sel_stride : 0;
    const float rcp = 1.0f / (float)sel_stride;
    const int32_t *base = sel + c0 * sel_stride;
    for (int f0 = 0; f0 < total; f0 += MASK_NT * MASK_LD) {
        int32_t v[MASK_LD];
#pragma unroll
        for (int u = 0; u < MASK_LD; ++u) {
            const int f = f0 + u * MASK_NT + tid;
            v[u] = f < total ? base[f] : -1;
        }
#pragma unroll
        for (int u = 0; u < MASK_LD; ++u) {
            const int f = f0 + u * MASK_NT + tid;
            if (f >= total) continue;
            int q = (int)((float)f * rcp), j = f - q * sel_stride;
            if (j < 0) {
                --q;
                j += sel_stride;
            } else if (j >= sel_stride) {
                ++q;
                j -= sel_stride;
            }
            const int32_t t = v[u];
            if (j < ns[q] && t >= t_lo && t < t_hi)
                atomicOr(&m[(int)((t >> 5) - g0) * MASK_QB + q], 1u << (t & 31));
        }
    }
    __syncthreads();
    for (int e = tid; e < ng * MASK_QB; e += MASK_NT) {
        const int g = e / MASK_QB, q = e % MASK_QB;
        mask[(g0 + g) * cols + c0 + q] = m[e];
    }
}

mla_status launch_attention(const void *q, mla_dtype dt, const void *kv_b, const mla_dims &d, const KvView &kv0,
                            int32_t S, int32_t pos_base, const int32_t *sel, const int32_t *nsel, int32_t sel_stride,
                            float sm_scale, bool absorbed, float *out, void *ws, hipStream_t s)
{
    const int64_t T = (int64_t)pos_base + S;
    char *p = reinterpret_cast<char *>((reinterpret_cast<uintptr_t>(ws) + 255) & ~(uintptr_t)255);
    KvView kv = kv0;
    kv.seq_len = nullptr;    // one sequence of T tokens
    kv.max_seq_len = T;
    if (absorbed) {
        kv.qps = S;          // launch row i = query i, keys 0 .. pos_base + i
        const size_t esz = dt == MLA_FP32 ? 4 : 2;
        const int64_t units = (int64_t)S * d.n_heads;
        char *qn = p;
        char *qr = p + (size_t)units * d.qk_nope * esz;
        void *dec_ws = p + al256((size_t)units * (d.qk_nope + d.qk_rope) * esz);
        const int64_t n = units * (d.qk_nope + d.qk_rope);
        const int64_t blocks = (n + 255) / 256;
        if (blocks > 0x7fffffff) return fail(MLA_ERR_UNSUPPORTED, "attention: too many queries");
        if (esz == 4)
            hipLaunchKernelGGL(split_q_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, s, (const uint32_t *)q,
                               (uint32_t *)qn, (uint32_t *)qr, units, d.qk_nope, d.qk_rope);
        else
            hipLaunchKernelGGL(split_q_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s, (const uint16_t *)q,
                               (uint16_t *)qn, (uint16_t *)qr, units, d.qk_nope, d.qk_rope);
        mla_status st = check_launch("split_q_kernel");
        if (st) return st;
        const int64_t max_keys = sel ? (int64_t)sel_stride : T;
        return launch_decode(qn, qr, kv_b, dt, d, S, kv, sel, nsel, sel ? sel_stride : 0, max_keys, sm_scale, out,
                             dec_ws, 0, s);
    }
    uint32_t *mask = nullptr;
    const int64_t cols = mask_cols(S);
    if (sel) {
        mask = reinterpret_cast<uint32_t *>(p);
        p += al256((size_t)mask_groups(T) * cols * 4);
        const int64_t gy = (mask_groups(T) + MASK_GCH - 1) / MASK_GCH;
        if (gy > 65535) return fail(MLA_ERR_UNSUPPORTED, "attention: key range too long for the selection mask");
        hipLaunchKernelGGL(sel_mask_kernel, dim3((unsigned)(cols / MASK_QB), (unsigned)gy), dim3(MASK_NT), 0, s, sel,
                           nsel, sel_stride, S, T, mask_groups(T), cols, mask);
        mla_status st = check_launch("sel_mask_kernel");
        if (st) return st;
    }
    return launch_prefill(q, kv_b, dt, d, kv, S, pos_base, sm_scale, out, MLA_FP32, p, 0, s, mask, (int)cols);
}

}  // namespace mla
