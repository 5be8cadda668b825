// dsa_select.hip -- DSA key selection fused with the indexer: scores and the top-k of every
// row in one call.  colibri-analysis 06 "MLA attention and KV cache", sec. 2.2: score every
// causal key with the lightning indexer and keep the top-2048.  The result is that of
// dsa_index_scores followed by dsa_topk_select with n_valid = seq_len: score descending, then
// position ascending (-0.0 equals +0.0), kept positions in ascending order, nsel = min(k, n).
//
// Launches (all rows of the batch together); no step accumulates into memory with atomics, so the
// workspace needs no clearing between calls:
//   1. indexer      writes the scores and, in the same pass, a histogram of the top 11
//                   order-key bits of its keys t < n (per workgroup in LDS), written as that
//                   workgroup's list of nonzero bins (common.h)
//   2. sel_filter   grid (t_max / 1024, B): sums the lists into the row histogram (only as deep
//                   as the threshold needs), finds the threshold bin, writes the row bitmask words
//                   of its keys above the bin and its keys inside the bin into its own slot
//   3. sel_resolve  grid (B x SR_PARTS): the exact k-th key (two radix passes over the candidates'
//                   remaining 21 bits), the kept candidates' bits, ties resolved in position
//                   order, and the kept positions written out of the bitmask in ascending order
//                   (each of a row's SR_PARTS workgroups writes those of one part of the bitmask)
// Rows longer than SEL_TMAX positions take the general top-k (three launches, any length).
#include "common.h"
#include "absorb_body.h"

namespace mla {

constexpr int SEL_BINS = HIST_BINS;        // top 11 key bits
constexpr int SEL_CH = 1024;               // positions per filter workgroup (one candidate slot)
constexpr int SEL_TMAX = 262144;           // longest row whose bitmasks the resolve step holds in LDS

// ------------------------------------------------------------------------------ 1'. histogram
// For indexer kernels without a built-in histogram: grid (ceil(t_max/1024), B), one list part per
// workgroup.
__global__ __launch_bounds__(256) void sel_hist(const float *__restrict__ scores, int64_t t_max, KvView kv,
                                                uint32_t *__restrict__ hl, uint32_t *__restrict__ hcnt,
                                                int parts_max)
{
    __shared__ uint32_t hs[SEL_BINS];
    __shared__ uint32_t sh[4];
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
    hist_write_list<256>(hs, hl + (int64_t)b * HL_CAP * parts_max + blockIdx.x, parts_max, (int)blockIdx.x,
                         hcnt + (int64_t)b * parts_max + blockIdx.x, sh);
}

mla_status launch_score_hist(const float *scores, int32_t B, int64_t t_max, const KvView &kv, HistOut *hist,
                             hipStream_t s)
{
    const int64_t nch = (t_max + SEL_CH - 1) / SEL_CH;
    if (nch == 0) return MLA_OK;
    if (nch > hist->parts_max) return fail(MLA_ERR_UNSUPPORTED, "select: histogram parts exceed the workspace");
    hist->parts = (int)nch;
    hipLaunchKernelGGL(sel_hist, dim3((unsigned)nch, B), dim3(256), 0, s, scores, t_max, kv, hist->hl, hist->hcnt,
                       hist->parts_max);
    return check_launch("sel_hist");
}

// ------------------------------------------------------------------------------ 2. filter
// 256 threads; thread t of workgroup c handles positions c*1024 + 256 j + t (j = 0..3), so the
// ballot of wave w for step j covers the 64 consecutive positions c*1024 + 256 j + 64 w ..., the
// word 16 c + 4 j + w of the row's bitmask.
//
// Row histogram: thread t reads parts t, t + 256, .. (PPT of them): the part's length and its
// first HL_TOP entries (the highest bins), added into an LDS histogram.  For a part longer than
// that, every bin at or above its last entry read is complete; the histogram is therefore exact
// from F = the highest such bin over the truncated parts upwards.  When the threshold lies below F
// the remaining entries of the truncated parts are added as well (then it is exact everywhere).
constexpr int SEL_CPT = 8;                     // candidates per thread held in registers (resolve)
constexpr int SR_NT = 512, SR_NW = SR_NT / 64; // threads / waves of the resolve workgroup
constexpr int SR_WPT = 8;                      // bitmask words per resolve thread (SEL_TMAX)
// The resolve code is compiled for at most WPT words per thread, WPT = 4 (rows up to 131072
// positions) or SR_WPT: its per-word steps are unrolled straight-line code, so that rows of
// 128k keys do not run the instructions of eight words per thread (~400 per wave after the scans).
constexpr int sr_wpt_of(int wp) { return wp / 512 <= 4 ? 4 : SR_WPT; }
// Workgroups per row of the resolve step.  Each finds the k-th key and the output offsets on its
// own (the same loads, passes and scans) and then writes the positions of one part of the row's
// bitmask words: the bit loop that turns words into positions costs ~2 us of one workgroup's ALU
// time at k = 2048, and split this way each thread handles one word instead of four.
constexpr int SR_PARTS = 4;
constexpr int SR_STATIC = SEL_BINS * 6 + 2048; // static LDS of the resolve workgroup (bytes)
constexpr int SR_DYN_MAX = 160 * 1024 - SR_STATIC;

struct SelRow {           // per-row results of the filter (uint32 words)
    uint32_t tb, above, pad0, pad1;
};

// words per row bitmask: ceil(t_max / 64) rounded up to a multiple of SR_NT
__host__ __device__ inline int sel_words(int64_t t_max)
{
    return (int)(((t_max + 63) / 64 + SR_NT - 1) / SR_NT * SR_NT);
}

template <int PPT>   // list parts per thread: parts <= 256 PPT
__global__ __launch_bounds__(256) void sel_filter(const float *__restrict__ scores, int64_t t_max, KvView kv, int k,
                                                  const uint32_t *__restrict__ hl, const uint32_t *__restrict__ hcnt,
                                                  int parts_max, int parts, uint2 *__restrict__ cand,
                                                  uint32_t *__restrict__ fcnt, uint64_t *__restrict__ gkeep, int wp,
                                                  SelRow *__restrict__ rows)
{
    constexpr int NW = 4;
    __shared__ uint32_t hs[SEL_BINS];
    __shared__ uint32_t sh[NW];
    __shared__ uint32_t s_tb, s_above, s_floor, s_found;
    __shared__ uint32_t s_wcnt[NW];
    const int b = blockIdx.y, c = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n = seq_len_of(kv, b);
    if (n <= k) return;
    if ((int64_t)c * SEL_CH >= n) {   // past the row's last key (a shorter row of a batch): an empty slot
        if (tid == 0) fcnt[(int64_t)b * gridDim.x + c] = 0u;
        return;
    }
    // this workgroup's scores and the top of every list part go out together
    const float *row = scores + (int64_t)b * t_max;
    float sv[SEL_CH / 256];
#pragma unroll
    for (int j = 0; j < SEL_CH / 256; ++j) {   // unconditional loads (clamped into the row), masked after
        const int64_t t = (int64_t)c * SEL_CH + 256 * j + tid;
        sv[j] = row[t < n ? t : n - 1];
    }
    // Row i of the list heads: register i of the thread of part p holds entry (i - p) % HL_TOP of
    // that part (the heads are stored rotated, common.h), so the lanes of one LDS atomic below add
    // bins of 16 different depths.
    const uint32_t *hlb = hl + (int64_t)b * HL_CAP * parts_max;
    uint32_t pc[PPT], pe[PPT][HL_TOP], pl[PPT];
#pragma unroll
    for (int r = 0; r < PPT; ++r) {   // clamped to the last part; parts past the end are skipped
        const int p = tid + 256 * r < parts ? tid + 256 * r : parts - 1;
        pc[r] = hcnt[(int64_t)b * parts_max + p];
#pragma unroll
        for (int i = 0; i < HL_TOP; ++i) pe[r][i] = hlb[(int64_t)i * parts_max + p];
        pl[r] = hlb[(int64_t)hl_row(HL_TOP - 1, p) * parts_max + p];   // entry HL_TOP - 1: a truncated part's floor
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < SEL_BINS / 256; ++i) hs[tid + 256 * i] = 0u;
    if (tid == 0) {
        s_floor = 0u;
        s_found = 0u;
    }
    __syncthreads();
    uint32_t key[SEL_CH / 256];
#pragma unroll
    for (int j = 0; j < SEL_CH / 256; ++j) {
        const int64_t t = (int64_t)c * SEL_CH + 256 * j + tid;
        key[j] = t < n ? order_key(sv[j]) : 0u;
    }
    uint32_t fl = 0u;   // this thread's highest floor bin over its truncated parts
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
        if (tid + 256 * r >= parts) break;
        const uint32_t ne = pc[r] < HL_TOP ? pc[r] : HL_TOP;
#pragma unroll
        for (int i = 0; i < HL_TOP; ++i)
            if ((uint32_t)((i - tid - 256 * r) & (HL_TOP - 1)) < ne) atomicAdd(&hs[pe[r][i] >> 21], pe[r][i] & 0x1FFFFFu);
        if (pc[r] > HL_TOP && (pl[r] >> 21) > fl) fl = pl[r] >> 21;
    }
    // one LDS atomic per wave for the floor (all lanes on one address would serialize)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t x = (uint32_t)__shfl_xor((int)fl, o);
        fl = x > fl ? x : fl;
    }
    if (lane == 0 && fl > 0u) atomicMax(&s_floor, fl);
    __syncthreads();
    // threshold bin: thread t owns the 8 bins [2040-8t, 2048-8t) (thread order = descending bins)
    for (int pass = 0; pass < 2; ++pass) {
        const int lo_bin = SEL_BINS - 8 * (tid + 1), hi = lo_bin + 7;
        uint32_t bin8[8], local = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            bin8[j] = hs[hi - j];
            local += bin8[j];
        }
        const uint32_t before = block_excl_scan_dpp<NW>(local, sh);
        const uint32_t fl = pass == 0 ? s_floor : 0u;
        if (before < (uint32_t)k && before + local >= (uint32_t)k) {
            uint32_t cum = before;
            for (int j = 0; j < 8; ++j) {
                if (cum + bin8[j] >= (uint32_t)k) {
                    if ((uint32_t)(hi - j) >= fl) {   // counts at and above this bin are complete
                        s_tb = (uint32_t)(hi - j);
                        s_above = cum;
                        s_found = 1u;
                    }
                    break;
                }
                cum += bin8[j];
            }
        }
        __syncthreads();
        if (s_found) break;
        // the threshold lies below the complete range: add the rest of the truncated parts
#pragma unroll
        for (int r = 0; r < PPT; ++r) {
            if (tid + 256 * r >= parts) break;
            const uint32_t *lp = hlb + tid + 256 * r;
            for (uint32_t i = HL_TOP; i < pc[r]; ++i) {
                const uint32_t e = lp[(int64_t)i * parts_max];
                atomicAdd(&hs[e >> 21], e & 0x1FFFFFu);
            }
        }
        __syncthreads();
    }
    const uint32_t tb = s_tb;
    // classify: the words of keys above the bin go straight to the row bitmask
    uint64_t cm[SEL_CH / 256];
    uint32_t wtot = 0u;
    uint64_t *kw = gkeep + (int64_t)b * wp + 16 * c + wave;
#pragma unroll
    for (int j = 0; j < SEL_CH / 256; ++j) {
        const int64_t t = (int64_t)c * SEL_CH + 256 * j + tid;
        const uint32_t kb = key[j] >> 21;
        const bool ok = t < n;
        const uint64_t am = __ballot(ok && kb > tb);
        if (lane == 0) kw[4 * j] = am;
        cm[j] = __ballot(ok && kb == tb);
        wtot += (uint32_t)__popcll(cm[j]);
    }
    if (lane == 0) s_wcnt[wave] = wtot;
    __syncthreads();
    // the keys inside the bin, in this workgroup's own slot
    const int64_t slot = (int64_t)b * gridDim.x + c;
    if (tid == 0) fcnt[slot] = s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
    uint32_t off = 0u;
    for (int w = 0; w < wave; ++w) off += s_wcnt[w];
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint2 *cs = cand + slot * SEL_CH;
#pragma unroll
    for (int j = 0; j < SEL_CH / 256; ++j) {
        if ((cm[j] >> lane) & 1ull) {
            const uint32_t at = off + (uint32_t)__popcll(cm[j] & below);
            const int64_t t = (int64_t)c * SEL_CH + 256 * j + tid;
            cs[at] = make_uint2(key[j], (uint32_t)t);
        }
        off += (uint32_t)__popcll(cm[j]);
    }
    if (c == 0 && tid == 0) {
        SelRow r;   // threshold bin and the count of keys above it
        r.tb = tb;
        r.above = s_above;
        r.pad0 = r.pad1 = 0u;
        rows[b] = r;
    }
}

// ------------------------------------------------------------------------------ 3. resolve + emit
// SR_PARTS workgroups of SR_NT threads per row b, each doing all of the following but writing only
// the positions of its part of the bitmask words:
//   - the candidates sit in nch slots (one per filter workgroup, fcnt[c] each).  The tps = SR_NT /
//     nch consecutive threads t of slot c = t / tps take its entries in pairs: thread r = t % tps
//     the pairs r + tps i, i < SEL_CPT / 2 (the first D = SEL_CPT tps entries, loaded before
//     anything waits); entries past D (long slots) are spread evenly over all threads through a
//     prefix of the slots' overflow counts
//   - the exact k-th key among the candidates (two radix digits, bits 20..10 and 9..0)
//   - candidates above it set their bit in the row bitmask (held in LDS), candidates equal to it
//     their bit in an eq bitmask
//   - thread t owns the bitmask words [t wpt, (t+1) wpt), a run of positions: the first
//     `remaining` eq bits in position order join the kept bits.  One pair of block scans gives both
//     the eq keys before a thread's run (erank) and the kept keys above the threshold before it; its
//     output offset is the latter plus min(remaining, erank), the eq keys taken before it.  The
//     final words and each word's output offset go to LDS, and the set bits of the part's words are
//     written out as positions -- ascending across the row.
// Every histogram and scan has LDS of its own, cleared or written once, so a phase needs only the
// barrier that publishes its inputs (10 barriers with the one that publishes the final words).
// (Writing the positions through LDS as one contiguous run instead of the scattered 4-byte stores
// changed nothing.)
// dyn: keep[wp], eq[wp] (uint64; the final words and their output offsets at the end), then staged
// overflow candidates.
template <int WPT>
__device__ __forceinline__ void resolve_emit_row(int b, int part, const KvView &kv, int k,
                                                 const uint2 *__restrict__ cand,
                                                 const uint32_t *__restrict__ fcnt, int nch,
                                                 const uint64_t *__restrict__ gkeep, int wp,
                                                 const SelRow *__restrict__ rows, int32_t *__restrict__ sel,
                                                 int32_t *__restrict__ nsel, uint64_t *__restrict__ dyn, int ov_cap)
{
    __shared__ uint32_t h[SEL_BINS], h2[SEL_BINS / 2];   // radix histograms, bits 20..10 and 9..0
    __shared__ uint32_t sh[5 * SR_NW];
    __shared__ uint32_t s_bc[4];
    __shared__ uint32_t s_ov[SEL_TMAX / SEL_CH + 1];   // overflow prefix over the slots
    const int tid = threadIdx.x;
    const int64_t n = seq_len_of(kv, b);
    int32_t *out = sel + (int64_t)b * k;
    if (n <= k) {   // every position is kept
        for (int u = part * SR_NT + tid; u < k; u += SR_PARTS * SR_NT) out[u] = u < n ? u : -1;
        if (part == 0 && tid == 0) nsel[b] = (int32_t)n;
        return;
    }
    // issued before anything waits: the row's threshold, the slot counts, bitmask words and the
    // first SEL_CPT entries of this thread in its slot, as unconditional loads clamped into the
    // buffers and masked on use
    const SelRow rin = rows[b];
    const int tps = SR_NT / nch;                     // threads per slot (nch <= 256: at least 2)
    const bool active = tid < tps * nch;             // threads past tps nch idle
    const int my_c = active ? tid / tps : 0, my_r = tid % tps;
    const uint32_t *fc = fcnt + (int64_t)b * nch;
    const uint32_t cnt_mine = fc[my_c];
    const uint32_t cnt_t = fc[tid < nch ? tid : 0];  // thread t < nch: slot t, for the overflow prefix
    const int wpt = wp / SR_NT;
    const int nw = (int)((n + 63) / 64);   // words that hold positions < n
    const uint64_t *gk = gkeep + (int64_t)b * wp + tid * wpt;
    uint64_t kw[WPT];
#pragma unroll
    for (int i = 0; i < WPT; ++i) kw[i] = gk[i < wpt ? i : 0];
    const uint2 *cb = cand + (int64_t)b * nch * SEL_CH;
    const uint4 *cmine = reinterpret_cast<const uint4 *>(cb + (int64_t)my_c * SEL_CH);
    uint2 cr[SEL_CPT];
#pragma unroll
    for (int i = 0; i < SEL_CPT / 2; ++i) {   // pair my_r + tps i: entries 2 (my_r + tps i), +1
        const int pr = my_r + tps * i;
        const uint4 v = cmine[pr < SEL_CH / 2 ? pr : SEL_CH / 2 - 1];
        cr[2 * i] = make_uint2(v.x, v.y);
        cr[2 * i + 1] = make_uint2(v.z, v.w);
    }
    uint64_t *keep = dyn, *eqm = dyn + wp;
    // cleared or filled before the first barrier: eq bits, the filter's words of keys above the
    // threshold bin, both radix histograms
    for (int i = tid; i < wp; i += SR_NT) eqm[i] = 0ull;
#pragma unroll
    for (int i = 0; i < WPT; ++i)
        if (i < wpt) keep[tid * wpt + i] = tid * wpt + i < nw ? kw[i] : 0ull;
#pragma unroll
    for (int q = 0; q < SEL_BINS / SR_NT; ++q) h[tid + SR_NT * q] = 0u;
#pragma unroll
    for (int q = 0; q < SEL_BINS / 2 / SR_NT; ++q) h2[tid + SR_NT * q] = 0u;
    const uint32_t tb = rin.tb, above_total = rin.above;
    // entries past the first D of each slot: prefix over the slots (thread t < nch: slot t)
    const uint32_t D = (uint32_t)tps * SEL_CPT;
    const uint32_t ov_t = tid < nch && cnt_t > D ? cnt_t - D : 0u;
    uint32_t OV = 0u;
    const uint32_t ov_pre = block_excl_scan_once<SR_NW>(ov_t, sh, &OV);   // (publishes the clears)
    if (tid < nch) s_ov[tid] = ov_pre;
    if (tid == 0) s_ov[nch] = OV;
    // the overflow entries (item i: slot c with s_ov[c] <= i < s_ov[c+1]) are read from memory
    // once into LDS behind the bitmasks when they fit (ov_cap entries), else in every pass
    uint2 *ovs = reinterpret_cast<uint2 *>(dyn + 2 * wp);
    const bool ov_lds = OV <= (uint32_t)ov_cap;
    auto ov_item = [&](uint32_t ic) {
        int lo = 0, hi = nch - 1;   // last slot with s_ov[slot] <= ic
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_ov[mid] <= ic) lo = mid;
            else hi = mid - 1;
        }
        return cb[(int64_t)lo * SEL_CH + D + (ic - s_ov[lo])];
    };
    if (OV > 0u) {
        __syncthreads();   // s_ov
        if (ov_lds) {
            for (uint32_t base = 0u; base < OV; base += 8u * SR_NT) {
                uint2 t[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t it = base + tid + (uint32_t)SR_NT * i;
                    t[i] = ov_item(it < OV ? it : OV - 1u);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t it = base + tid + (uint32_t)SR_NT * i;
                    if (it < OV) ovs[it] = t[i];
                }
            }
            __syncthreads();   // ovs
        }
    }
    // every candidate once: those held in registers, then the overflow entries (from LDS, or in
    // batches of eight independent loads per thread)
    auto for_each = [&](auto f) {
#pragma unroll
        for (int i = 0; i < SEL_CPT; ++i)
            if (active && (uint32_t)(2 * (my_r + tps * (i >> 1)) + (i & 1)) < cnt_mine) f(cr[i]);
        if (ov_lds) {
            for (uint32_t it = tid; it < OV; it += SR_NT) f(ovs[it]);
            return;
        }
        for (uint32_t base = 0u; base < OV; base += 8u * SR_NT) {
            uint2 t[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t it = base + tid + (uint32_t)SR_NT * i;
                t[i] = ov_item(it < OV ? it : OV - 1u);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (base + tid + (uint32_t)SR_NT * i < OV) f(t[i]);
        }
    };
    // radix select of the need-th largest key: digits of bits 20..10, then 9..0
    uint32_t prefix = tb << 21, mask = 0xFFE00000u, remaining = (uint32_t)k - above_total;   // >= 1
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int shift = p == 0 ? 10 : 0;
        const int nb = p == 0 ? SEL_BINS : SEL_BINS / 2;
        const uint32_t dm = (uint32_t)nb - 1u;
        uint32_t *hp = p == 0 ? h : h2;
        const uint32_t pf = prefix, mk = mask;
        for_each([&](uint2 c) {
            if ((c.x & mk) == pf) atomicAdd(&hp[(c.x >> shift) & dm], 1u);
        });
        __syncthreads();
        const int per = nb / SR_NT;   // 4 or 2 bins per thread, thread order = descending bins
        const int top = nb - 1 - per * tid;
        uint32_t hv[4], local = 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            hv[q] = q < per ? hp[top - q] : 0u;
            local += hv[q];
        }
        const uint32_t before = block_excl_scan_once<SR_NW>(local, sh + (1 + p) * SR_NW);
        if (before < remaining && before + local >= remaining) {
            uint32_t cum = before;
            int bin = top;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q < per && cum + hv[q] >= remaining) {
                    bin = top - q;
                    break;
                }
                cum += hv[q];
            }
            s_bc[2 * p] = remaining - cum;
            s_bc[2 * p + 1] = prefix | ((uint32_t)bin << shift);
        }
        __syncthreads();
        remaining = s_bc[2 * p];
        prefix = s_bc[2 * p + 1];
        mask |= dm << shift;
    }
    const uint32_t kth = prefix;
    // the candidates' bits: above the k-th key into the kept bitmask, equal to it into eq
    for_each([&](uint2 c) {
        if (c.x > kth) atomicOr(reinterpret_cast<unsigned long long *>(&keep[c.y >> 6]), 1ull << (c.y & 63));
        else if (c.x == kth) atomicOr(reinterpret_cast<unsigned long long *>(&eqm[c.y >> 6]), 1ull << (c.y & 63));
    });
    __syncthreads();
    uint64_t ew[WPT];
    uint32_t ec = 0u, kc = 0u;
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
        kw[i] = i < wpt ? keep[tid * wpt + i] : 0ull;
        ew[i] = i < wpt ? eqm[tid * wpt + i] : 0ull;
        ec += (uint32_t)__popcll(ew[i]);
        kc += (uint32_t)__popcll(kw[i]);
    }
    uint32_t erank, o;   // equal keys before this run; kept keys above the k-th before it
    block_excl_scan2_once<SR_NW>(ec, kc, sh + 3 * SR_NW, erank, o);
    o += erank < remaining ? erank : remaining;
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
        uint64_t e = ew[i];
        const uint32_t c = (uint32_t)__popcll(e);
        if (erank >= remaining) e = 0ull;
        else if (erank + c > remaining) {   // only the first remaining - erank of them
            uint64_t take = 0ull;
            for (uint32_t m = remaining - erank; m; --m) {
                const uint64_t low = e & (~e + 1ull);
                take |= low;
                e ^= low;
            }
            e = take;
        }
        erank += c;
        kw[i] |= e;
    }
    // the final words and the output offset of each word go to LDS (over the bitmasks: every
    // thread read its own words before the scans' barriers), then this part's words are emitted,
    // one word per thread and pass, in ascending positions
    uint32_t *woff = reinterpret_cast<uint32_t *>(eqm);
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
        if (i < wpt) {
            keep[tid * wpt + i] = kw[i];
            woff[tid * wpt + i] = o;
            o += (uint32_t)__popcll(kw[i]);
        }
    }
    __syncthreads();
    const int wpp = wp / SR_PARTS;   // (wp is a multiple of SR_NT)
    for (int w = part * wpp + tid; w < (part + 1) * wpp; w += SR_NT) {
        uint64_t x = keep[w];
        uint32_t ow = woff[w];
        while (x) {
            const int bit = __builtin_ctzll(x);
            x &= x - 1ull;
            if (ow < (uint32_t)k) out[ow] = 64 * w + bit;
            ++ow;
        }
    }
    if (part == 0 && tid == 0) nsel[b] = k;
}

// grid (B SR_PARTS), SR_NT threads, dynamic LDS 16 wp bytes + overflow room
template <int WPT>
__global__ __launch_bounds__(SR_NT) void sel_resolve(KvView kv, int k, const uint2 *__restrict__ cand,
                                                     const uint32_t *__restrict__ fcnt, int nch,
                                                     const uint64_t *__restrict__ gkeep, int wp,
                                                     const SelRow *__restrict__ rows, int32_t *__restrict__ sel,
                                                     int32_t *__restrict__ nsel, int ov_cap)
{
    extern __shared__ uint64_t sr_dyn[];
    resolve_emit_row<WPT>((int)blockIdx.x / SR_PARTS, (int)blockIdx.x % SR_PARTS, kv, k, cand, fcnt, nch, gkeep, wp,
                          rows,
                     sel, nsel, sr_dyn, ov_cap);
}

// Side job j (SR_NT threads): two absorb jobs a = 2 j + half, (cb, h) = (a % 4, a / 4), one per 256
// threads; the cb == 0 job of head h also rotates that head's query tails at each row's query
// position seq_len - 1 (into a separate buffer; no rotation when there is none).  FMT: 0 for the
// bf16 kv_b, else its quantized format (always the vector-ALU absorption: the fp32 row scales are
// not exact in the bf16 operands of the matrix-core one).
template <int NR, int FMT>
__device__ __forceinline__ void side_absorb_job(const KvView &kv, const SideAbsorb &sa, int job, uint64_t *sr_dyn)
{
    const int half = threadIdx.x >> 8, jt = threadIdx.x & 255;
    const int a = 2 * job + half, cb = a & 3, h = a >> 2;
    if (FMT == 0 && sa.B >= AB_MFMA_B) {
        absorb_block_mfma<NR>(sa.q_nope, reinterpret_cast<const bf16_t *>(sa.kv_b), sa.B, sa.v, sa.q_abs, cb, h,
                              reinterpret_cast<char *>(sr_dyn) + half * 16 * NR * AB_WROWB, jt);
    } else {
        float *shj = reinterpret_cast<float *>(sr_dyn) + half * (sa.B * 16 * NR + 4 * AB_QB * 128);
        absorb_block<NR, FMT>(sa.q_nope, sa.kv_b, sa.scales, sa.B, sa.v, sa.q_abs, cb, h, shj, jt);
    }
    if (cb != 0 || !sa.q_rope_out) return;
    const int hr = sa.rope / 2;
    for (int p = jt; p < sa.B * hr; p += 256) {
        const int b = p / hr, j = p - b * hr;
        const bf16_t *x = sa.q_rope + ((int64_t)b * AB_H + h) * sa.rope;
        bf16_t *y = sa.q_rope_out + ((int64_t)b * AB_H + h) * sa.rope;
        const int64_t sl = seq_len_of(kv, b);
        float lo, hi;
        rope_pair(bf2f(x[2 * j]), bf2f(x[2 * j + 1]), j, sa.rope, (double)(sl > 0 ? sl - 1 : 0), sa.theta, lo, hi);
        y[j] = f2bf(lo);
        y[hr + j] = f2bf(hi);
    }
}

// The resolve step leaves all but B SR_PARTS workgroups of the chip idle; the decode step fills them with
// work that does not depend on the selection: the query absorption (absorb_body.h) and the RoPE
// rotation of the query tails at each row's query position seq_len - 1 (into a separate buffer).
// grid (nres + 2 * 64): workgroups nres.. run two absorb jobs a = 2 (blockIdx - nres) + half,
// (cb, h) = (a % 4, a / 4), one per 256 threads; the cb == 0 job of head h also rotates that
// head's query tails.
template <int NR, int FMT, int WPT>
__global__ __launch_bounds__(SR_NT) void sel_resolve_absorb(KvView kv, int k, const uint2 *__restrict__ cand,
                                                            const uint32_t *__restrict__ fcnt, int nch,
                                                            const uint64_t *__restrict__ gkeep, int wp,
                                                            const SelRow *__restrict__ rows,
                                                            int32_t *__restrict__ sel, int32_t *__restrict__ nsel,
                                                            int nres, SideAbsorb sa, int ov_cap)
{
    extern __shared__ uint64_t sr_dyn[];
    if ((int)blockIdx.x < nres) {
        resolve_emit_row<WPT>((int)blockIdx.x / SR_PARTS, (int)blockIdx.x % SR_PARTS, kv, k, cand, fcnt, nch, gkeep,
                              wp, rows, sel, nsel, sr_dyn, ov_cap);
        return;
    }
    side_absorb_job<NR, FMT>(kv, sa, (int)blockIdx.x - nres, sr_dyn);
}

// The same side work as a launch of its own (2 * 64 workgroups of SR_NT threads), for decode steps
// whose selection is given (the shared layer) or that run no selection.
template <int NR, int FMT>
__global__ __launch_bounds__(SR_NT) void absorb_rope(KvView kv, SideAbsorb sa)
{
    extern __shared__ uint64_t sr_dyn[];
    side_absorb_job<NR, FMT>(kv, sa, blockIdx.x, sr_dyn);
}

static size_t side_lds(const SideAbsorb &sa)
{
    return sa.fmt == 0 && sa.B >= AB_MFMA_B ? 2 * (size_t)sa.nope * AB_WROWB
                                            : 2 * ((size_t)sa.B * sa.nope + 4 * AB_QB * 128) * 4;
}

bool side_absorb_ok(const SideAbsorb &sa)
{
    return sa.B <= SIDE_MAXB && (sa.nope == 128 || sa.nope == 192 || sa.nope == 256) && sa.fmt >= 0 &&
           sa.fmt <= MLA_Q_MXFP4;
}

// f(NR, FMT) for the side job's template arguments
#define SIDE_DISPATCH(sa, f)                                              \
    do {                                                                  \
        if ((sa).nope == 128) SIDE_DISPATCH_F((sa), f, 8);                \
        else if ((sa).nope == 192) SIDE_DISPATCH_F((sa), f, 12);          \
        else SIDE_DISPATCH_F((sa), f, 16);                                \
    } while (0)
#define SIDE_DISPATCH_F(sa, f, NR)                                        \
    do {                                                                  \
        if ((sa).fmt == MLA_Q_FP8_E4M3) f(NR, MLA_Q_FP8_E4M3);            \
        else if ((sa).fmt == MLA_Q_INT8) f(NR, MLA_Q_INT8);               \
        else if ((sa).fmt == MLA_Q_MXFP4) f(NR, MLA_Q_MXFP4);             \
        else f(NR, 0);                                                    \
    } while (0)

template <int NR, int FMT> static hipError_t side_attr()
{
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&absorb_rope<NR, FMT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, SR_DYN_MAX);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&sel_resolve_absorb<NR, FMT, 4>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, SR_DYN_MAX);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&sel_resolve_absorb<NR, FMT, SR_WPT>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, SR_DYN_MAX);
    return e;
}

static mla_status enable_side_lds()
{
    static bool done = false;
    if (!done) {
        hipError_t e = hipSuccess;
        for (int nope : {128, 192, 256})
            for (int fmt = 0; fmt <= MLA_Q_MXFP4; ++fmt) {
                SideAbsorb t{};
                t.nope = nope;
                t.fmt = fmt;
#define SIDE_ATTR(NR, FMT) e = e == hipSuccess ? side_attr<NR, FMT>() : e
                SIDE_DISPATCH(t, SIDE_ATTR);
#undef SIDE_ATTR
            }
        if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
        done = true;
    }
    return MLA_OK;
}

mla_status launch_absorb_rope(const SideAbsorb &sa, const KvView &kv, hipStream_t s)
{
    mla_status st = enable_side_lds();
    if (st) return st;
    const size_t dyn = side_lds(sa);
    const dim3 g(2 * AB_H);
#define AR_LAUNCH(NR, FMT) hipLaunchKernelGGL((absorb_rope<NR, FMT>), g, dim3(SR_NT), dyn, s, kv, sa)
    SIDE_DISPATCH(sa, AR_LAUNCH);
#undef AR_LAUNCH
    return check_launch("absorb_rope");
}

// ------------------------------------------------------------------------------ host side
struct SelWs {
    HistOut hist;
    uint32_t *fcnt;
    SelRow *rows;
    uint64_t *keep;
    uint2 *cand;
    int64_t nch;
    int wp;
};

static size_t sal(size_t x) { return (x + 255) & ~(size_t)255; }

static SelWs sel_ws(void *ws, int32_t B, int64_t t_max, size_t *bytes)
{
    SelWs w;
    w.nch = (t_max + SEL_CH - 1) / SEL_CH;
    w.wp = sel_words(t_max);
    w.hist.parts_max = hist_parts_max(B, t_max);
    w.hist.parts = 0;
    char *p = reinterpret_cast<char *>(ws);
    size_t off = 0;
    auto take = [&](size_t sz) {
        char *q = p + off;
        off += sal(sz);
        return q;
    };
    w.hist.hl = reinterpret_cast<uint32_t *>(take((size_t)B * w.hist.parts_max * HL_CAP * 4));
    w.hist.hcnt = reinterpret_cast<uint32_t *>(take((size_t)B * w.hist.parts_max * 4));
    w.fcnt = reinterpret_cast<uint32_t *>(take((size_t)B * w.nch * 4));
    w.rows = reinterpret_cast<SelRow *>(take((size_t)B * sizeof(SelRow)));
    w.keep = reinterpret_cast<uint64_t *>(take((size_t)B * w.wp * 8));
    w.cand = reinterpret_cast<uint2 *>(take((size_t)B * w.nch * SEL_CH * 8));
    if (bytes) *bytes = off;
    return w;
}

size_t index_select_workspace_bytes(int32_t B, int64_t t_max, int32_t k)
{
    if (t_max > SEL_TMAX) return topk_workspace_bytes(B, t_max, k);
    size_t fast = 0;
    sel_ws(nullptr, B, t_max, &fast);
    return fast;
}

static mla_status enable_sel_lds()
{
    static bool done = false;
    if (!done) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&sel_resolve<4>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, SR_DYN_MAX);
        if (e == hipSuccess)
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(&sel_resolve<SR_WPT>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, SR_DYN_MAX);
        if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
        done = true;
    }
    return enable_side_lds();
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
    st = enable_sel_lds();
    if (st) return st;
    SelWs sw = sel_ws(ws, B, t_max, nullptr);
    if (t_max > 0) {
        st = launch_index_scores(q, w, B, n_ih, hd, kv, t_max, scores, &sw.hist, s);
        if (st) return st;
        const int P = sw.hist.parts;
        const dim3 gf((unsigned)sw.nch, B);
#define SF_LAUNCH(PPT)                                                                                         \
    hipLaunchKernelGGL(sel_filter<PPT>, gf, dim3(256), 0, s, scores, t_max, kv, k, sw.hist.hl, sw.hist.hcnt, \
                       sw.hist.parts_max, P, sw.cand, sw.fcnt, sw.keep, sw.wp, sw.rows)
        if (P <= 256) SF_LAUNCH(1);
        else if (P <= 512) SF_LAUNCH(2);
        else if (P <= 768) SF_LAUNCH(3);
        else return fail(MLA_ERR_UNSUPPORTED, "select: more than 768 histogram parts");
#undef SF_LAUNCH
        st = check_launch("sel_filter");
        if (st) return st;
    }
    const int nch = sw.nch > 0 ? (int)sw.nch : 1;
    // the bitmasks, then room for staged overflow candidates (at least 64 KB or what is left)
    const size_t dyn_masks = (size_t)sw.wp * 16;
    const size_t dyn_sel = dyn_masks + 65536 < (size_t)SR_DYN_MAX ? dyn_masks + 65536 : (size_t)SR_DYN_MAX;
    const bool with_side = side && side->B == B && side_absorb_ok(*side);
    if (!with_side) {
        if (sr_wpt_of(sw.wp) == 4)
            hipLaunchKernelGGL((sel_resolve<4>), dim3(B * SR_PARTS), dim3(SR_NT), dyn_sel, s, kv, k, sw.cand, sw.fcnt, nch, sw.keep,
                               sw.wp, sw.rows, sel, nsel, (int)((dyn_sel - dyn_masks) / 8));
        else
            hipLaunchKernelGGL((sel_resolve<SR_WPT>), dim3(B * SR_PARTS), dim3(SR_NT), dyn_sel, s, kv, k, sw.cand, sw.fcnt, nch, sw.keep,
                               sw.wp, sw.rows, sel, nsel, (int)((dyn_sel - dyn_masks) / 8));
        return check_launch("sel_resolve");
    }
    const size_t dyn_abs = side_lds(*side);
    const size_t dyn = dyn_sel > dyn_abs ? dyn_sel : dyn_abs;
    const dim3 g((unsigned)(B * SR_PARTS + 2 * AB_H));
#define SRA_LAUNCH(NR, FMT, W)                                                                                  \
    hipLaunchKernelGGL((sel_resolve_absorb<NR, FMT, W>), g, dim3(SR_NT), dyn, s, kv, k, sw.cand, sw.fcnt, nch, sw.keep, \
                       sw.wp, sw.rows, sel, nsel, B * SR_PARTS, *side, (int)((dyn - dyn_masks) / 8))
#define SRA_LAUNCH4(NR, FMT) SRA_LAUNCH(NR, FMT, 4)
#define SRA_LAUNCH8(NR, FMT) SRA_LAUNCH(NR, FMT, SR_WPT)
    if (sr_wpt_of(sw.wp) == 4) SIDE_DISPATCH(*side, SRA_LAUNCH4);
    else SIDE_DISPATCH(*side, SRA_LAUNCH8);
#undef SRA_LAUNCH8
#undef SRA_LAUNCH4
#undef SRA_LAUNCH
    st = check_launch("sel_resolve_absorb");
    if (st) return st;
    if (side_done) *side_done = true;
    return MLA_OK;
}

}  // namespace mla
