// dsa_topk.hip -- top-k causal key selection without a full sort.
// colibri-analysis 06 "MLA attention and KV cache", sec. 2.2: keep the top-2048 causal keys
// (the page's engine sorts and scans for the threshold into dsa_sel / dsa_nsel).  Here the
// threshold is found by radix selection on order-preserving uint32 keys and the kept
// positions are emitted in position order, which yields exactly the set and order that
// sorting would: score descending, then position ascending; -0.0 equals +0.0.
//
// Three launches per call, all rows of the batch at once:
//   1. topk_hist    grid (chunks, B): 2048-bin histogram of the top 11 key bits per chunk
//   2. topk_filter  grid (chunks, B): every workgroup reduces the chunk histograms to find
//                   the threshold bin; keys above it are kept for sure (written as a bitmap
//                   over positions), keys inside it are candidates (written in position
//                   order to the chunk's candidate region)
//   3. topk_final   grid (B): radix-selects the remaining 21 bits among the candidates,
//                   marks the kept candidates in the bitmap, then emits the kept positions in
//                   ascending order from the bitmap
// Rows with n_valid <= k keep every position (0..n-1) and skip the first two phases.
#include "common.h"

namespace mla {

constexpr int TK_CH = 8192;        // positions per chunk
constexpr int TK_THREADS = 256;    // threads of the chunk kernels
constexpr int TK_PER = TK_CH / TK_THREADS;   // 32 consecutive positions (one bitmap word) per thread
constexpr int TK_BINS = 2048;      // top 11 bits of the key
constexpr int TK_FINAL_THREADS = 1024;
static_assert(TK_PER == 32, "one bitmap word per thread");

// Block-wide exclusive scan of one uint32 per thread (NW waves of 64).  sh needs 2*NW+1 words.
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *sh, uint32_t *total = nullptr)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    if (wave == 0) {
        const uint32_t wv = lane < NW ? sh[lane] : 0u;
        uint32_t z = wv;
#pragma unroll
        for (int o = 1; o < NW; o <<= 1) {
            const uint32_t y = __shfl_up(z, o, 64);
            if (lane >= o) z += y;
        }
        if (lane < NW) sh[NW + lane] = z - wv;
        if (lane == NW - 1) sh[2 * NW] = z;
    }
    __syncthreads();
    const uint32_t r = sh[NW + wave] + x - v;
    if (total) *total = sh[2 * NW];
    __syncthreads();
    return r;
}

// Row length: n_valid[b] clamped to [0, max_len], or max_len when there is no n_valid.
__device__ __forceinline__ int64_t row_len(const int32_t *n_valid, int b, int64_t max_len)
{
    int64_t n = n_valid ? (int64_t)n_valid[b] : max_len;
    if (n < 0) n = 0;
    if (n > max_len) n = max_len;
    return n;
}

// Loads the 32 keys of positions [t0, t0+32) (invalid positions -> valid bit clear).
__device__ __forceinline__ uint32_t load_keys32(const float *s, int64_t t0, int64_t n, uint32_t key[32])
{
    uint32_t valid = 0u;
    if (t0 + 32 <= n && ((reinterpret_cast<uintptr_t>(s + t0) & 15u) == 0)) {
        const float4 *p = reinterpret_cast<const float4 *>(s + t0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 v = p[i];
            key[4 * i + 0] = order_key(v.x);
            key[4 * i + 1] = order_key(v.y);
            key[4 * i + 2] = order_key(v.z);
            key[4 * i + 3] = order_key(v.w);
        }
        valid = 0xffffffffu;
    } else {
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            const bool ok = t0 + e < n;
            key[e] = ok ? order_key(s[t0 + e]) : 0u;
            valid |= (ok ? 1u : 0u) << e;
        }
    }
    return valid;
}

__global__ __launch_bounds__(TK_THREADS) void topk_hist(const float *__restrict__ scores, int64_t t_max,
                                                        const int32_t *__restrict__ n_valid, int64_t max_len, int k,
                                                        int nch,
                                                        uint32_t *__restrict__ hist)
{
    __shared__ uint32_t h[TK_BINS];
    const int b = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    const int64_t n = row_len(n_valid, b, max_len);
    if (n <= k) return;
    for (int i = tid; i < TK_BINS; i += TK_THREADS) h[i] = 0u;
    __syncthreads();
    const int64_t t0 = (int64_t)c * TK_CH + (int64_t)tid * TK_PER;
    if (t0 < n) {
        uint32_t key[32];
        const uint32_t valid = load_keys32(scores + (int64_t)b * t_max, t0, n, key);
#pragma unroll
        for (int e = 0; e < 32; ++e)
            if (valid >> e & 1u) atomicAdd(&h[key[e] >> 21], 1u);
    }
    __syncthreads();
    uint32_t *out = hist + ((int64_t)b * nch + c) * TK_BINS;
    for (int i = tid; i < TK_BINS; i += TK_THREADS) out[i] = h[i];
}

__global__ __launch_bounds__(TK_THREADS) void topk_filter(const float *__restrict__ scores, int64_t t_max,
                                                          const int32_t *__restrict__ n_valid, int64_t max_len, int k,
                                                          int nch,
                                                          const uint32_t *__restrict__ hist,
                                                          uint32_t *__restrict__ bitmap, int64_t nwords,
                                                          uint2 *__restrict__ cand, uint32_t *__restrict__ meta)
{
    __shared__ uint32_t tot[TK_BINS];
    __shared__ uint32_t sh[2 * (TK_THREADS / 64) + 1];
    __shared__ uint32_t s_tb, s_above;
    const int b = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    const int64_t n = row_len(n_valid, b, max_len);
    if (n <= k) return;
    // 1. row histogram: thread t owns the 8 bins [2040-8t, 2048-8t) (so thread order is
    //    descending bin order) and sums them over the chunks, several chunks in flight
    constexpr int BPT = TK_BINS / TK_THREADS;
    static_assert(BPT == 8, "two uint4 per thread and chunk");
    const int lo_bin = TK_BINS - BPT * (tid + 1);
    const uint32_t *hb = hist + (int64_t)b * nch * TK_BINS + lo_bin;
    uint32_t bin8[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll 4
    for (int cc = 0; cc < nch; ++cc) {
        const uint4 *p = reinterpret_cast<const uint4 *>(hb + (int64_t)cc * TK_BINS);
        const uint4 x0 = p[0], x1 = p[1];
        bin8[0] += x0.x; bin8[1] += x0.y; bin8[2] += x0.z; bin8[3] += x0.w;
        bin8[4] += x1.x; bin8[5] += x1.y; bin8[6] += x1.z; bin8[7] += x1.w;
    }
#pragma unroll
    for (int j = 0; j < BPT; ++j) tot[lo_bin + j] = bin8[j];
    // 2. threshold bin
    const int hi = lo_bin + BPT - 1;
    uint32_t local = 0u;
#pragma unroll
    for (int j = 0; j < BPT; ++j) local += bin8[j];
    const uint32_t before = block_excl_scan<TK_THREADS / 64>(local, sh);
    if (before < (uint32_t)k && before + local >= (uint32_t)k) {
        uint32_t cum = before;
        for (int j = 0; j < BPT; ++j) {
            const uint32_t cnt = tot[hi - j];
            if (cum + cnt >= (uint32_t)k) {
                s_tb = (uint32_t)(hi - j);
                s_above = cum;
                break;
            }
            cum += cnt;
        }
    }
    __syncthreads();
    const uint32_t tb = s_tb;
    if (c == 0 && tid == 0) {
        meta[2 * b + 0] = tb;
        meta[2 * b + 1] = s_above;
    }
    // 3. this chunk: bitmap of sure keeps, ordered candidates
    const int64_t t0 = (int64_t)c * TK_CH + (int64_t)tid * TK_PER;
    uint32_t key[32];
    uint32_t valid = 0u;
    if (t0 < n) valid = load_keys32(scores + (int64_t)b * t_max, t0, n, key);
    uint32_t bits = 0u, ncand = 0u;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        if (valid >> e & 1u) {
            const uint32_t kb = key[e] >> 21;
            bits |= (kb > tb ? 1u : 0u) << e;
            ncand += kb == tb ? 1u : 0u;
        }
    }
    const int64_t w = t0 / 32;
    if (w < nwords) bitmap[(int64_t)b * nwords + w] = bits;
    const uint32_t off = block_excl_scan<TK_THREADS / 64>(ncand, sh);
    if (ncand) {
        uint2 *dst = cand + (int64_t)b * nch * TK_CH + (int64_t)c * TK_CH + off;
        uint32_t j = 0u;
#pragma unroll
        for (int e = 0; e < 32; ++e)
            if ((valid >> e & 1u) && (key[e] >> 21) == tb) dst[j++] = make_uint2(key[e], (uint32_t)(t0 + e));
    }
}

constexpr int TK_LDS_CAND = 6144;   // candidates staged in LDS (48 KB); more are read from memory

__global__ __launch_bounds__(TK_FINAL_THREADS) void topk_final(const int32_t *__restrict__ n_valid, int64_t max_len,
                                                              int k, int nch, const uint32_t *__restrict__ hist,
                                                              uint32_t *__restrict__ bitmap, int64_t nwords,
                                                              const uint2 *__restrict__ cand,
                                                              const uint32_t *__restrict__ meta,
                                                              int32_t *__restrict__ sel, int32_t *__restrict__ nsel)
{
    constexpr int NW = TK_FINAL_THREADS / 64;
    __shared__ uint32_t h[256];
    __shared__ uint32_t sh[2 * NW + 1];
    __shared__ uint32_t s_prefix, s_remaining;
    __shared__ uint2 sc[TK_LDS_CAND];
    extern __shared__ uint32_t cc[];   // [nch + 1]: exclusive prefix of candidates per chunk
    const int b = blockIdx.x, tid = threadIdx.x;
    const int64_t n = row_len(n_valid, b, max_len);
    int32_t *out = sel + (int64_t)b * k;
    if (n <= k) {
        for (int64_t i = tid; i < k; i += TK_FINAL_THREADS) out[i] = i < n ? (int32_t)i : -1;
        if (tid == 0) nsel[b] = (int32_t)n;
        return;
    }
    const uint32_t tb = meta[2 * b + 0];
    const uint32_t above = meta[2 * b + 1];
    const uint32_t need = (uint32_t)k - above;   // >= 1 by construction of tb
    const uint32_t *hb = hist + (int64_t)b * nch * TK_BINS;
    // candidates per chunk -> exclusive prefix (chunks handled 1024 at a time)
    uint32_t run = 0u;
    for (int c0 = 0; c0 < nch; c0 += TK_FINAL_THREADS) {
        const int c = c0 + tid;
        const uint32_t v = c < nch ? hb[(int64_t)c * TK_BINS + tb] : 0u;
        uint32_t tot_c;
        const uint32_t ex = block_excl_scan<NW>(v, sh, &tot_c);
        if (c < nch) cc[c] = run + ex;
        run += tot_c;
    }
    if (tid == 0) cc[nch] = run;
    __syncthreads();
    const uint32_t E = run;
    const uint2 *cb = cand + (int64_t)b * nch * TK_CH;
    // candidate j (position order) lives in chunk region c at index j - cc[c]
    auto cand_mem = [&](uint32_t j) -> uint2 {
        int lo = 0, hi2 = nch - 1;   // last c with cc[c] <= j
        while (lo < hi2) {
            const int mid = (lo + hi2 + 1) >> 1;
            if (cc[mid] <= j) lo = mid;
            else hi2 = mid - 1;
        }
        return cb[(int64_t)lo * TK_CH + (j - cc[lo])];
    };
    const bool in_lds = E <= (uint32_t)TK_LDS_CAND;
    if (in_lds) {
        for (uint32_t j = tid; j < E; j += TK_FINAL_THREADS) sc[j] = cand_mem(j);
        __syncthreads();
    }
    auto cand_at = [&](uint32_t j) -> uint2 { return in_lds ? sc[j] : cand_mem(j); };
    // radix select of the need-th largest low-21-bit value among the candidates
    uint32_t prefix = tb << 21, mask = 0xFFE00000u, remaining = need;
    const int shifts[3] = {13, 5, 0};
    const int widths[3] = {8, 8, 5};
    for (int p = 0; p < 3; ++p) {
        const int sh_ = shifts[p];
        const uint32_t dm = (1u << widths[p]) - 1u;
        if (tid < 256) h[tid] = 0u;
        __syncthreads();
        for (uint32_t j = tid; j < E; j += TK_FINAL_THREADS) {
            const uint32_t key = cand_at(j).x;
            if ((key & mask) == prefix) atomicAdd(&h[(key >> sh_) & dm], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            // wave 0 scans the (at most 256) bins from the top: lane owns 4 consecutive bins
            const int nb = (int)dm + 1;
            const int top = nb - 1 - 4 * tid;
            uint32_t c4 = 0u;
#pragma unroll
            for (int q = 0; q < 4; ++q) c4 += (top - q >= 0) ? h[top - q] : 0u;
            uint32_t inc = c4;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_up(inc, o, 64);
                if (tid >= o) inc += y;
            }
            const uint32_t exc = inc - c4;
            if (top >= 0 && exc < remaining && inc >= remaining) {
                uint32_t cum = exc;
                int bin = top;
                for (int q = 0; q < 4 && top - q >= 0; ++q) {
                    bin = top - q;
                    if (cum + h[bin] >= remaining) break;
                    cum += h[bin];
                }
                s_remaining = remaining - cum;
                s_prefix = prefix | ((uint32_t)bin << sh_);
            }
        }
        __syncthreads();
        remaining = s_remaining;
        prefix = s_prefix;
        mask |= dm << sh_;
    }
    // prefix is the exact threshold key; keep candidates above it and the first `remaining`
    // equal to it in position order
    const uint32_t kth = prefix;
    uint32_t eq_run = 0u;
    for (uint32_t j0 = 0; j0 < E; j0 += TK_FINAL_THREADS) {
        const uint32_t j = j0 + tid;
        uint2 cv = make_uint2(0u, 0u);
        const bool in = j < E;
        if (in) cv = cand_at(j);
        const uint32_t is_eq = (in && cv.x == kth) ? 1u : 0u;
        uint32_t tot_eq;
        const uint32_t eq_before = eq_run + block_excl_scan<NW>(is_eq, sh, &tot_eq);
        if (in && (cv.x > kth || (is_eq && eq_before < remaining)))
            atomicOr(&bitmap[(int64_t)b * nwords + (cv.y >> 5)], 1u << (cv.y & 31u));
        eq_run += tot_eq;
    }
    __threadfence();
    __syncthreads();
    // emit kept positions in ascending order from the bitmap, four words per thread per round
    const int64_t words = (n + 31) / 32;
    uint32_t base = 0u;
    const uint32_t *bm = bitmap + (int64_t)b * nwords;
    for (int64_t w0 = 0; w0 < words; w0 += 4 * TK_FINAL_THREADS) {
        const int64_t w = w0 + 4 * (int64_t)tid;
        uint32_t bits[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            bits[q] = w + q < words ? __hip_atomic_load(bm + w + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
        const uint32_t cnt = __popc(bits[0]) + __popc(bits[1]) + __popc(bits[2]) + __popc(bits[3]);
        uint32_t tot_c;
        uint32_t o = base + block_excl_scan<NW>(cnt, sh, &tot_c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t x = bits[q];
            while (x) {
                const int e = __ffs(x) - 1;
                x &= x - 1u;
                if (o < (uint32_t)k) out[o] = (int32_t)((w + q) * 32 + e);
                ++o;
            }
        }
        base += tot_c;
    }
    if (tid == 0) nsel[b] = k;
}

static inline int tk_chunks(int64_t t_max) { return (int)((t_max + TK_CH - 1) / TK_CH); }

size_t topk_workspace_bytes(int32_t B, int64_t t_max, int32_t)
{
    const int nch = tk_chunks(t_max);
    const int64_t nwords = (t_max + 31) / 32;
    size_t bytes = 0;
    bytes += (size_t)B * nch * TK_BINS * 4;          // hist
    bytes += (size_t)B * nwords * 4;                 // bitmap
    bytes = (bytes + 15) & ~(size_t)15;
    bytes += (size_t)B * nch * TK_CH * 8;            // candidates
    bytes += (size_t)B * 2 * 4;                      // meta
    return bytes + 256;
}

mla_status launch_topk(const float *scores, int32_t B, int64_t t_max, const int32_t *n_valid, int64_t max_len,
                       int32_t k, int32_t *sel, int32_t *nsel, void *ws, size_t, hipStream_t s)
{
    const int nch = tk_chunks(t_max);
    const int64_t nwords = (t_max + 31) / 32;
    if (B > 65535) return fail(MLA_ERR_UNSUPPORTED, "topk: B > 65535");
    if (nch > 2047) return fail(MLA_ERR_UNSUPPORTED, "topk: t_max above %d", 2047 * TK_CH);
    char *p = reinterpret_cast<char *>(ws);
    uint32_t *hist = reinterpret_cast<uint32_t *>(p);
    p += (size_t)B * nch * TK_BINS * 4;
    uint32_t *bitmap = reinterpret_cast<uint32_t *>(p);
    p += (size_t)B * nwords * 4;
    p = reinterpret_cast<char *>((reinterpret_cast<uintptr_t>(p) + 15) & ~(uintptr_t)15);
    uint2 *cand = reinterpret_cast<uint2 *>(p);
    p += (size_t)B * nch * TK_CH * 8;
    uint32_t *meta = reinterpret_cast<uint32_t *>(p);
    if (nch > 0) {
        hipLaunchKernelGGL(topk_hist, dim3(nch, B), dim3(TK_THREADS), 0, s, scores, t_max, n_valid, max_len, k, nch,
                           hist);
        mla_status st = check_launch("topk_hist");
        if (st) return st;
        hipLaunchKernelGGL(topk_filter, dim3(nch, B), dim3(TK_THREADS), 0, s, scores, t_max, n_valid, max_len, k, nch, hist,
                           bitmap, nwords, cand, meta);
        st = check_launch("topk_filter");
        if (st) return st;
    }
    hipLaunchKernelGGL(topk_final, dim3(B), dim3(TK_FINAL_THREADS), (size_t)(nch + 1) * 4, s, n_valid, max_len, k, nch,
                       hist, bitmap, nwords, cand, meta, sel, nsel);
    return check_launch("topk_final");
}

}  // namespace mla
