// dsa_select.hip -- DSA key selection fused with the indexer: scores and the top-k of every
// row in one call.  colibri-analysis 06 "MLA attention and KV cache", sec. 2.2: score every
// causal key with the lightning indexer and keep the top-2048.  The result is that of
// dsa_index_scores followed by dsa_topk_select with n_valid = seq_len: score descending, then
// position ascending (-0.0 equals +0.0), kept positions in ascending order, nsel = min(k, n).
//
// Launches (all rows of the batch together):
//   1. sel_zero     clears the row histograms and counters of the workspace
//   2. indexer      writes the scores and, in the same pass, a histogram of the top 11
//                   order-key bits of every score of a key t < n (per workgroup in LDS, then
//                   added into the row histogram with atomics)
//   3. sel_filter   grid (t_max / 1024, B): finds the threshold bin from the row histogram,
//                   counts its keys above the bin and appends its keys inside the bin to the
//                   row's candidate list
//   4. sel_resolve  grid (B): the exact k-th key (two radix passes over the candidates'
//                   remaining 21 bits) and the output offset of every filter workgroup
//   5. sel_emit     grid (t_max / 1024, B): every workgroup re-reads its scores, keeps the
//                   keys above the k-th key and the leading keys equal to it (position order),
//                   and writes their positions at its offset -- ascending across the row
// Rows longer than SEL_TMAX positions take the general top-k (three launches, any length).
#include "common.h"
#include "absorb_body.h"

namespace mla {

constexpr int SEL_BINS = 2048;             // top 11 key bits
constexpr int SEL_CH = 1024;               // positions per filter workgroup
constexpr int SEL_TMAX = 262144;           // longest row the LDS-resident final step handles

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (row shifts inside rows of 16
// lanes, then row broadcasts of lanes 15 and 31), no LDS traffic.
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t x)
{
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);   // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return x;
}

// Block-wide exclusive scan (NW waves) on DPP wave scans; sh needs NW words.
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan_dpp(uint32_t v, uint32_t *sh, uint32_t *total = nullptr)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t inc = wave_incl_scan_dpp(v);
    if (lane == 63) sh[wave] = inc;
    __syncthreads();
    uint32_t before = 0u, all = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t t = sh[w];
        before += w < wave ? t : 0u;
        all += t;
    }
    if (total) *total = all;
    __syncthreads();
    return before + inc - v;
}

// ------------------------------------------------------------------------------ 1. zero
__global__ __launch_bounds__(256) void sel_zero(uint32_t *__restrict__ ghist, uint32_t *__restrict__ cnt)
{
    const int b = blockIdx.x;
    for (int i = threadIdx.x; i < SEL_BINS; i += 256) ghist[(int64_t)b * SEL_BINS + i] = 0u;
    if (threadIdx.x == 0) cnt[b] = 0u;
}

// ------------------------------------------------------------------------------ 2'. histogram
// For indexer kernels without a built-in histogram: grid (ceil(t_max/1024), B).
__global__ __launch_bounds__(256) void sel_hist(const float *__restrict__ scores, int64_t t_max, KvView kv,
                                                uint32_t *__restrict__ ghist)
{
    __shared__ uint32_t hs[SEL_BINS];
    const int b = blockIdx.y, tid = threadIdx.x;
    const int64_t n = seq_len_of(kv, b);
    for (int i = tid; i < SEL_BINS; i += 256) hs[i] = 0u;
    __syncthreads();
    const float *row = scores + (int64_t)b * t_max;
    if (n > 0) {
        float v[SEL_CH / 256];
#pragma unroll
        for (int j = 0; j < SEL_CH / 256; ++j) {
            const int64_t t = (int64_t)blockIdx.x * SEL_CH + 256 * j + tid;
            v[j] = row[t < n ? t : n - 1];
        }
#pragma unroll
        for (int j = 0; j < SEL_CH / 256; ++j) {
            const int64_t t = (int64_t)blockIdx.x * SEL_CH + 256 * j + tid;
            if (t < n) atomicAdd(&hs[order_key(v[j]) >> 21], 1u);
        }
    }
    __syncthreads();
    for (int i = tid; i < SEL_BINS; i += 256) {
        const uint32_t c = hs[i];
        if (c) atomicAdd(&ghist[(int64_t)b * SEL_BINS + i], c);
    }
}

mla_status launch_score_hist(const float *scores, int32_t B, int64_t t_max, const KvView &kv, uint32_t *ghist,
                             hipStream_t s)
{
    const int64_t nch = (t_max + SEL_CH - 1) / SEL_CH;
    if (nch == 0) return MLA_OK;
    hipLaunchKernelGGL(sel_hist, dim3((unsigned)nch, B), dim3(256), 0, s, scores, t_max, kv, ghist);
    return check_launch("sel_hist");
}

// ------------------------------------------------------------------------------ 3. filter
// 256 threads; thread t of workgroup c handles positions c*1024 + 256 j + t (j = 0..3), so the
// ballot of wave w for step j covers the 64 consecutive positions c*1024 + 256 j + 64 w ...
// Every workgroup finds the threshold bin tb from the row histogram, counts its keys above the
// bin and appends its keys inside the bin to the row's candidate list.
constexpr int SEL_MAXCH = SEL_TMAX / SEL_CH;   // workgroups per row (256)
constexpr int SEL_CPT = 16;                    // candidates per thread held in registers

struct SelRow {           // per-row results of the filter (uint32 words)
    uint32_t tb, kth, remaining, pad;
};

// One workgroup of 256 threads per row b: resolves the exact k-th key of the row among its
// candidates and the output offset of every filter workgroup.
__device__ __forceinline__ void resolve_row(int b, KvView kv, int nch, int k, const uint2 *__restrict__ cand,
                                            int64_t cap, const uint32_t *__restrict__ cnt,
                                            const uint32_t *__restrict__ blkabove, uint32_t *__restrict__ outpfx,
                                            uint32_t *__restrict__ eqpfx, SelRow *__restrict__ row_out)
{
    constexpr int NW = 4;
    __shared__ uint32_t h[SEL_BINS];
    __shared__ uint32_t gtc[SEL_MAXCH], eqc[SEL_MAXCH];
    __shared__ uint32_t sh[NW];
    __shared__ uint32_t s_bc[2];
    const int tid = threadIdx.x;
    if (seq_len_of(kv, b) <= k) return;
    const SelRow rin = row_out[b];   // tb and the count above its bin, from the filter
    uint32_t E = cnt[b];
    // issued before anything waits: the filter workgroups' counts above the bin, and the first
    // 256 * SEL_CPT candidates (thread t holds t + 256 i), as unconditional loads clamped into
    // the buffers and masked on use
    const uint32_t above_blk = blkabove[(int64_t)b * SEL_MAXCH + (tid < nch ? tid : 0)];
    const uint2 *cb = cand + (int64_t)b * cap;
    uint2 cr[SEL_CPT];
#pragma unroll
    for (int i = 0; i < SEL_CPT; ++i) {
        const int64_t j = tid + 256 * i;
        cr[i] = cb[j < cap ? j : cap - 1];
    }
    const uint32_t tb = rin.tb, above_total = rin.kth;
    if (E > cap) E = (uint32_t)cap;
    // every candidate once: those held in registers, then the rest from memory in batches of
    // eight independent loads per thread
    auto for_each = [&](auto f) {
#pragma unroll
        for (int i = 0; i < SEL_CPT; ++i)
            if (tid + 256u * i < E) f(cr[i]);
        for (uint32_t base = 256u * SEL_CPT; base < E; base += 2048u) {
            uint2 t[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t j = base + tid + 256u * i;
                t[i] = cb[j < E ? j : E - 1u];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (base + tid + 256u * i < E) f(t[i]);
        }
    };
    // radix select of the need-th largest key: digits of bits 20..10, then 9..0
    uint32_t prefix = tb << 21, mask = 0xFFE00000u, remaining = (uint32_t)k - above_total;   // >= 1
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int shift = p == 0 ? 10 : 0;
        const int nb = p == 0 ? 2048 : 1024;
        const uint32_t dm = (uint32_t)nb - 1u;
#pragma unroll
        for (int q = 0; q < 8; ++q) h[tid + 256 * q] = 0u;
        __syncthreads();
        const uint32_t pf = prefix, mk = mask;
        for_each([&](uint2 c) {
            if ((c.x & mk) == pf) atomicAdd(&h[(c.x >> shift) & dm], 1u);
        });
        __syncthreads();
        const int per = nb / 256;   // 8 or 4 bins per thread, thread order = descending bins
        const int top = nb - 1 - per * tid;
        uint32_t hv[8], local = 0u;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            hv[q] = q < per ? h[top - q] : 0u;
            local += hv[q];
        }
        const uint32_t before = block_excl_scan_dpp<NW>(local, sh);
        if (before < remaining && before + local >= remaining) {
            uint32_t cum = before;
            int bin = top;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (q < per && cum + hv[q] >= remaining) {
                    bin = top - q;
                    break;
                }
                cum += hv[q];
            }
            s_bc[0] = remaining - cum;
            s_bc[1] = prefix | ((uint32_t)bin << shift);
        }
        __syncthreads();
        remaining = s_bc[0];
        prefix = s_bc[1];
        mask |= dm << shift;
    }
    const uint32_t kth = prefix;
    // per workgroup: candidates above the k-th key, and equal to it
    gtc[tid] = 0u;
    eqc[tid] = 0u;
    __syncthreads();
    for_each([&](uint2 c) {
        if (c.x > kth) atomicAdd(&gtc[c.y / SEL_CH], 1u);
        else if (c.x == kth) atomicAdd(&eqc[c.y / SEL_CH], 1u);
    });
    __syncthreads();
    // thread t = workgroup t: keys equal to the k-th one are taken in position order, i.e. in
    // workgroup order
    const uint32_t ec = tid < nch ? eqc[tid] : 0u;
    const uint32_t epf = block_excl_scan_dpp<NW>(ec, sh);
    uint32_t take = remaining > epf ? remaining - epf : 0u;
    if (take > ec) take = ec;
    const uint32_t kept = tid < nch ? above_blk + gtc[tid] + take : 0u;
    const uint32_t opf = block_excl_scan_dpp<NW>(kept, sh);
    if (tid < nch) {
        outpfx[(int64_t)b * SEL_MAXCH + tid] = opf;
        eqpfx[(int64_t)b * SEL_MAXCH + tid] = epf;
    }
    if (tid == 0) {
        SelRow r;
        r.tb = tb;
        r.kth = kth;
        r.remaining = remaining;
        r.pad = 0u;
        row_out[b] = r;
    }
}

// grid (B), 256 threads
__global__ __launch_bounds__(256) void sel_resolve(KvView kv, int nch, int k, const uint2 *__restrict__ cand,
                                                   int64_t cap, const uint32_t *__restrict__ cnt,
                                                   const uint32_t *__restrict__ blkabove, uint32_t *__restrict__ outpfx,
                                                   uint32_t *__restrict__ eqpfx, SelRow *__restrict__ row_out)
{
    resolve_row(blockIdx.x, kv, nch, k, cand, cap, cnt, blkabove, outpfx, eqpfx, row_out);
}

// The resolve step leaves all but B workgroups of the chip idle; the decode step fills them with
// work that does not depend on the selection: the query absorption (absorb_body.h) and the RoPE
// rotation of the query tails at each row's query position seq_len - 1 (into a separate buffer).
// grid (nres + 4 * 64): workgroups nres.. are absorb workgroup (cb, h) = (a % 4, a / 4); the
// cb == 0 one of head h also rotates that head's query tails.
template <int NR>
__global__ __launch_bounds__(256) void sel_resolve_absorb(KvView kv, int nch, int k, const uint2 *__restrict__ cand,
                                                          int64_t cap, const uint32_t *__restrict__ cnt,
                                                          const uint32_t *__restrict__ blkabove,
                                                          uint32_t *__restrict__ outpfx, uint32_t *__restrict__ eqpfx,
                                                          SelRow *__restrict__ row_out, int nres, SideAbsorb sa)
{
    extern __shared__ float sh_abs[];
    if ((int)blockIdx.x < nres) {
        resolve_row(blockIdx.x, kv, nch, k, cand, cap, cnt, blkabove, outpfx, eqpfx, row_out);
        return;
    }
    const int a = blockIdx.x - nres, cb = a & 3, h = a >> 2;
    absorb_block<NR>(sa.q_nope, sa.kv_b, sa.B, sa.v, sa.q_abs, cb, h, sh_abs);
    if (cb != 0) return;
    const int half = sa.rope / 2;
    for (int p = threadIdx.x; p < sa.B * half; p += 256) {
        const int b = p / half, j = p - b * half;
        const bf16_t *x = sa.q_rope + ((int64_t)b * AB_H + h) * sa.rope;
        bf16_t *y = sa.q_rope_out + ((int64_t)b * AB_H + h) * sa.rope;
        const int64_t sl = seq_len_of(kv, b);
        float lo, hi;
        rope_pair(bf2f(x[2 * j]), bf2f(x[2 * j + 1]), j, sa.rope, (double)(sl > 0 ? sl - 1 : 0), sa.theta, lo, hi);
        y[j] = f2bf(lo);
        y[half + j] = f2bf(hi);
    }
}

__global__ __launch_bounds__(256) void sel_filter(const float *__restrict__ scores, int64_t t_max, KvView kv, int k,
                                                  const uint32_t *__restrict__ ghist, uint2 *__restrict__ cand,
                                                  int64_t cap, uint32_t *__restrict__ cnt,
                                                  uint32_t *__restrict__ blkabove, SelRow *__restrict__ rows)
{
    constexpr int NW = 4;
    __shared__ uint32_t tot[SEL_BINS];
    __shared__ uint32_t sh[NW];
    __shared__ uint32_t s_tb, s_above, s_base;
    __shared__ uint32_t s_wcnt[NW], s_wab[NW];
    const int b = blockIdx.y, c = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n = seq_len_of(kv, b);
    if (n <= k) return;
    // threshold bin: thread t owns the 8 bins [2040-8t, 2048-8t) (thread order = descending bins)
    const int lo_bin = SEL_BINS - 8 * (tid + 1);
    const uint4 *hp = reinterpret_cast<const uint4 *>(ghist + (int64_t)b * SEL_BINS + lo_bin);
    const uint4 x0 = hp[0], x1 = hp[1];
    const uint32_t bin8[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    // the scores of this workgroup's positions go out while the histogram is scanned
    const float *row = scores + (int64_t)b * t_max;
    uint32_t key[SEL_CH / 256];
    float sv[SEL_CH / 256];
#pragma unroll
    for (int j = 0; j < SEL_CH / 256; ++j) {   // unconditional loads (clamped into the row), masked after
        const int64_t t = (int64_t)c * SEL_CH + 256 * j + tid;
        sv[j] = row[t < n ? t : n - 1];
    }
    __builtin_amdgcn_sched_barrier(0);   // all four loads in flight together
#pragma unroll
    for (int j = 0; j < SEL_CH / 256; ++j) {
        const int64_t t = (int64_t)c * SEL_CH + 256 * j + tid;
        key[j] = t < n ? order_key(sv[j]) : 0u;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) tot[lo_bin + j] = bin8[j];
    uint32_t local = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) local += bin8[j];
    const uint32_t before = block_excl_scan_dpp<NW>(local, sh);
    if (before < (uint32_t)k && before + local >= (uint32_t)k) {
        uint32_t cum = before;
        const int hi = lo_bin + 7;
        for (int j = 0; j < 8; ++j) {
            const uint32_t ct = tot[hi - j];
            if (cum + ct >= (uint32_t)k) {
                s_tb = (uint32_t)(hi - j);
                s_above = cum;
                break;
            }
            cum += ct;
        }
    }
    __syncthreads();
    const uint32_t tb = s_tb;
    // classify
    uint64_t cm[SEL_CH / 256];
    uint32_t wtot = 0u, wab = 0u;
#pragma unroll
    for (int j = 0; j < SEL_CH / 256; ++j) {
        const int64_t t = (int64_t)c * SEL_CH + 256 * j + tid;
        const uint32_t kb = key[j] >> 21;
        const bool ok = t < n;
        wab += (uint32_t)__popcll(__ballot(ok && kb > tb));
        cm[j] = __ballot(ok && kb == tb);
        wtot += (uint32_t)__popcll(cm[j]);
    }
    if (lane == 0) {
        s_wcnt[wave] = wtot;
        s_wab[wave] = wab;
    }
    __syncthreads();
    if (tid == 0) {
        const uint32_t all = s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
        s_base = all ? atomicAdd(&cnt[b], all) : 0u;
        blkabove[(int64_t)b * SEL_MAXCH + c] = s_wab[0] + s_wab[1] + s_wab[2] + s_wab[3];
    }
    __syncthreads();
    uint32_t off = s_base;
    for (int w = 0; w < wave; ++w) off += s_wcnt[w];
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int j = 0; j < SEL_CH / 256; ++j) {
        if ((cm[j] >> lane) & 1ull) {
            const uint32_t at = off + (uint32_t)__popcll(cm[j] & below);
            const int64_t t = (int64_t)c * SEL_CH + 256 * j + tid;
            if (at < (uint64_t)cap) cand[(int64_t)b * cap + at] = make_uint2(key[j], (uint32_t)t);
        }
        off += (uint32_t)__popcll(cm[j]);
    }
    if (c == 0 && tid == 0) {
        SelRow r;   // threshold bin and the count above it (sel_resolve replaces the row)
        r.tb = tb;
        r.kth = s_above;
        r.remaining = 0u;
        r.pad = 0u;
        rows[b] = r;
    }
}

// ------------------------------------------------------------------------------ 4. emit
// grid (max(nch, 1), B), 256 threads, same position mapping as the filter.  Rows with n <= k keep
// every position; otherwise a position is kept when its key lies above the k-th key, or equals
// it and ranks (in position order, across the row) below the number of equal keys still needed.
// Kept positions are written at the workgroup's output offset plus their rank in the workgroup.
__global__ __launch_bounds__(256) void sel_emit(const float *__restrict__ scores, int64_t t_max, KvView kv, int k,
                                                const uint32_t *__restrict__ outpfx, const uint32_t *__restrict__ eqpfx,
                                                const SelRow *__restrict__ rows, int32_t *__restrict__ sel,
                                                int32_t *__restrict__ nsel)
{
    __shared__ uint32_t s_eq[SEL_CH / 64], s_kp[SEL_CH / 64];   // per (step, wave), position order
    const int b = blockIdx.y, c = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n = seq_len_of(kv, b);
    int32_t *out = sel + (int64_t)b * k;
    if (n <= k) {
        for (int64_t base = (int64_t)c * SEL_CH; base < k; base += (int64_t)gridDim.x * SEL_CH) {
#pragma unroll
            for (int j = 0; j < SEL_CH / 256; ++j) {
                const int64_t u = base + 256 * j + tid;
                if (u < k) out[u] = u < n ? (int32_t)u : -1;
            }
        }
        if (c == 0 && tid == 0) nsel[b] = (int32_t)n;
        return;
    }
    const SelRow r = rows[b];
    const uint32_t opf = outpfx[(int64_t)b * SEL_MAXCH + c], epf = eqpfx[(int64_t)b * SEL_MAXCH + c];
    const float *row = scores + (int64_t)b * t_max;
    bool gt[SEL_CH / 256], eq[SEL_CH / 256];
    float sv[SEL_CH / 256];
#pragma unroll
    for (int j = 0; j < SEL_CH / 256; ++j) {   // n > k >= 1 here; loads clamped into the row
        const int64_t t = (int64_t)c * SEL_CH + 256 * j + tid;
        sv[j] = row[t < n ? t : n - 1];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < SEL_CH / 256; ++j) {
        const int64_t t = (int64_t)c * SEL_CH + 256 * j + tid;
        const uint32_t key = t < n ? order_key(sv[j]) : 0u;
        const uint32_t kb = key >> 21;
        gt[j] = t < n && (kb > r.tb || (kb == r.tb && key > r.kth));
        eq[j] = t < n && key == r.kth;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // ranks among the equal keys of the workgroup, in position order
    uint64_t em[SEL_CH / 256];
#pragma unroll
    for (int j = 0; j < SEL_CH / 256; ++j) {
        em[j] = __ballot(eq[j]);
        if (lane == 0) s_eq[4 * j + wave] = (uint32_t)__popcll(em[j]);
    }
    __syncthreads();
    uint64_t km[SEL_CH / 256];
    bool kp[SEL_CH / 256];
#pragma unroll
    for (int j = 0; j < SEL_CH / 256; ++j) {
        uint32_t before = 0u;
        for (int i = 0; i < 4 * j + wave; ++i) before += s_eq[i];
        const uint32_t erank = epf + before + (uint32_t)__popcll(em[j] & below);
        kp[j] = gt[j] || (eq[j] && erank < r.remaining);
        km[j] = __ballot(kp[j]);
        if (lane == 0) s_kp[4 * j + wave] = (uint32_t)__popcll(km[j]);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SEL_CH / 256; ++j) {
        if (kp[j]) {
            uint32_t before = 0u;
            for (int i = 0; i < 4 * j + wave; ++i) before += s_kp[i];
            const uint32_t o = opf + before + (uint32_t)__popcll(km[j] & below);
            if (o < (uint32_t)k) out[o] = (int32_t)((int64_t)c * SEL_CH + 256 * j + tid);
        }
    }
    if (c == 0 && tid == 0) nsel[b] = k;
}

// ------------------------------------------------------------------------------ host side
struct SelWs {
    uint32_t *ghist, *cnt, *blkabove, *outpfx, *eqpfx;
    SelRow *rows;
    uint2 *cand;
    int64_t nch, cap;
};

static size_t sal(size_t x) { return (x + 255) & ~(size_t)255; }

static SelWs sel_ws(void *ws, int32_t B, int64_t t_max, size_t *bytes)
{
    SelWs w;
    w.nch = (t_max + SEL_CH - 1) / SEL_CH;
    w.cap = w.nch * SEL_CH;
    char *p = reinterpret_cast<char *>(ws);
    size_t off = 0;
    auto take = [&](size_t sz) {
        char *q = p + off;
        off += sal(sz);
        return q;
    };
    w.ghist = reinterpret_cast<uint32_t *>(take((size_t)B * SEL_BINS * 4));
    w.cnt = reinterpret_cast<uint32_t *>(take((size_t)B * 4));
    w.blkabove = reinterpret_cast<uint32_t *>(take((size_t)B * SEL_MAXCH * 4));
    w.outpfx = reinterpret_cast<uint32_t *>(take((size_t)B * SEL_MAXCH * 4));
    w.eqpfx = reinterpret_cast<uint32_t *>(take((size_t)B * SEL_MAXCH * 4));
    w.rows = reinterpret_cast<SelRow *>(take((size_t)B * sizeof(SelRow)));
    w.cand = reinterpret_cast<uint2 *>(take((size_t)B * w.cap * 8));
    if (bytes) *bytes = off;
    return w;
}

size_t index_select_workspace_bytes(int32_t B, int64_t t_max, int32_t k)
{
    size_t fast = 0;
    sel_ws(nullptr, B, t_max, &fast);
    const size_t general = topk_workspace_bytes(B, t_max, k);
    return t_max <= SEL_TMAX ? fast : general;
}

mla_status launch_index_select(const float *q, const float *w, int32_t B, int32_t n_ih, int32_t hd, const KvView &kv,
                               int64_t t_max, int32_t k, float *scores, int32_t *sel, int32_t *nsel, void *ws,
                               size_t ws_bytes, hipStream_t s, const SideAbsorb *side, bool *side_done)
{
    if (side_done) *side_done = false;
    if (B > 65535) return fail(MLA_ERR_UNSUPPORTED, "select: B > 65535");
    mla_status st;
    if (t_max > SEL_TMAX) {
        // general path: the scores, then the stand-alone top-k of every row (n_valid = seq_len)
        st = launch_index_scores(q, w, B, n_ih, hd, kv, t_max, scores, nullptr, s);
        if (st) return st;
        return launch_topk(scores, B, t_max, kv.seq_len, kv.max_seq_len, k, sel, nsel, ws, ws_bytes, s);
    }
    const SelWs sw = sel_ws(ws, B, t_max, nullptr);
    hipLaunchKernelGGL(sel_zero, dim3(B), dim3(256), 0, s, sw.ghist, sw.cnt);
    st = check_launch("sel_zero");
    if (st) return st;
    const bool with_side = side && side->B == B && B <= SIDE_MAXB &&
                           (side->nope == 128 || side->nope == 192 || side->nope == 256);
    const int nres = t_max > 0 ? B : 0;
    if (t_max > 0) {
        st = launch_index_scores(q, w, B, n_ih, hd, kv, t_max, scores, sw.ghist, s);
        if (st) return st;
        hipLaunchKernelGGL(sel_filter, dim3((unsigned)sw.nch, B), dim3(256), 0, s, scores, t_max, kv, k, sw.ghist,
                           sw.cand, sw.cap, sw.cnt, sw.blkabove, sw.rows);
        st = check_launch("sel_filter");
        if (st) return st;
        if (!with_side) {
            hipLaunchKernelGGL(sel_resolve, dim3(B), dim3(256), 0, s, kv, (int)sw.nch, k, sw.cand, sw.cap, sw.cnt,
                               sw.blkabove, sw.outpfx, sw.eqpfx, sw.rows);
            st = check_launch("sel_resolve");
            if (st) return st;
        }
    }
    if (with_side) {
        const dim3 g((unsigned)(nres + 4 * AB_H));
        const size_t shm = (size_t)B * side->nope * 4 + 4 * AB_QB * 128 * 4;
        const int nch = (int)sw.nch;
        if (side->nope == 128)
            hipLaunchKernelGGL(sel_resolve_absorb<8>, g, dim3(256), shm, s, kv, nch, k, sw.cand, sw.cap, sw.cnt,
                               sw.blkabove, sw.outpfx, sw.eqpfx, sw.rows, nres, *side);
        else if (side->nope == 192)
            hipLaunchKernelGGL(sel_resolve_absorb<12>, g, dim3(256), shm, s, kv, nch, k, sw.cand, sw.cap, sw.cnt,
                               sw.blkabove, sw.outpfx, sw.eqpfx, sw.rows, nres, *side);
        else
            hipLaunchKernelGGL(sel_resolve_absorb<16>, g, dim3(256), shm, s, kv, nch, k, sw.cand, sw.cap, sw.cnt,
                               sw.blkabove, sw.outpfx, sw.eqpfx, sw.rows, nres, *side);
        st = check_launch("sel_resolve_absorb");
        if (st) return st;
        if (side_done) *side_done = true;
    }
    const unsigned ge = sw.nch > 0 ? (unsigned)sw.nch : 1u;
    hipLaunchKernelGGL(sel_emit, dim3(ge, B), dim3(256), 0, s, scores, t_max, kv, k, sw.outpfx, sw.eqpfx, sw.rows, sel,
                       nsel);
    return check_launch("sel_emit");
}

}  // namespace mla
