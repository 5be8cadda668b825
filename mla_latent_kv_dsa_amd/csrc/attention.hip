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
// mask is written.  A thread takes runs of MASK_RUN consecutive entries of one query's selection
// (run r of row q: entries MASK_RUN r ..); the bits of consecutive entries in the same word are
// merged in a register and set with one LDS atomic per change of word.  A selection in position
// order (as the DSA selection is) then gives each lane of a wave its own words, entries 16 apart,
// instead of 64 lanes setting bits of the same word; any order stays correct.
constexpr int MASK_QB = 32, MASK_GCH = 256, MASK_NT = 512, MASK_RUN = 16;

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
    const int qn = S - c0 < MASK_QB ? (int)(S - c0) : MASK_QB;
    const int rpr = (sel_stride + MASK_RUN - 1) / MASK_RUN;   // runs per row (sel_stride < 2^19)
    const int nruns = qn > 0 ? qn * rpr : 0;
    const int32_t *base = sel + c0 * sel_stride;
    const bool vec = sel_stride % 4 == 0 && (reinterpret_cast<uintptr_t>(base) & 15u) == 0;
    for (int rr = tid; rr < nruns; rr += MASK_NT) {
        const int q = rr / rpr, j0 = (rr - q * rpr) * MASK_RUN;
        const int n = ns[q];
        if (j0 >= n) continue;
        const int32_t *src = base + (int64_t)q * sel_stride + j0;
        int32_t v[MASK_RUN];
        if (vec && j0 + MASK_RUN <= sel_stride) {
#pragma unroll
            for (int k = 0; k < MASK_RUN / 4; ++k) {
                const int4 x = reinterpret_cast<const int4 *>(src)[k];
                v[4 * k] = x.x;
                v[4 * k + 1] = x.y;
                v[4 * k + 2] = x.z;
                v[4 * k + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < MASK_RUN; ++k) v[k] = j0 + k < sel_stride ? src[k] : -1;
        }
        int wcur = -1;
        uint32_t bits = 0u;
#pragma unroll
        for (int k = 0; k < MASK_RUN; ++k) {
            const int32_t t = v[k];
            const bool ok = j0 + k < n && t >= t_lo && t < t_hi;
            const int w = ok ? (int)((t >> 5) - g0) : -1;
            if (w != wcur) {
                if (wcur >= 0) atomicOr(&m[wcur * MASK_QB + q], bits);
                wcur = w;
                bits = 0u;
            }
            if (ok) bits |= 1u << (t & 31);
        }
        if (wcur >= 0) atomicOr(&m[wcur * MASK_QB + q], bits);
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
