// common.h -- internal helpers shared by the HIP kernels of libmla_dsa (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla_dsa.h"

namespace mla {

// ------------------------------------------------------------------ error reporting
void set_error(const char *fmt, ...);
mla_status fail(mla_status s, const char *fmt, ...);
// Check the last launch; returns MLA_ERR_HIP (with the HIP message) on failure.
mla_status check_launch(const char *what);

// ------------------------------------------------------------------ bf16 as raw bits
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// round to nearest even (inputs here are finite)
__device__ __forceinline__ bf16_t f2bf(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float ld(const T *p);
template <> __device__ __forceinline__ float ld<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float ld<bf16_t>(const bf16_t *p) { return bf2f(*p); }

template <typename T> __device__ __forceinline__ void st(T *p, float v);
template <> __device__ __forceinline__ void st<float>(float *p, float v) { *p = v; }
template <> __device__ __forceinline__ void st<bf16_t>(bf16_t *p, float v) { *p = f2bf(v); }

// ------------------------------------------------------------------ KV cache addressing
// Device-side copy of mla_kv_view (passed by value to kernels).
struct KvView {
    const void *lc;
    const void *rc;
    const float *ic;
    int64_t rows;
    const int32_t *bt;
    int32_t bs;
    int32_t max_blocks;
    int64_t seq_stride;
    const int32_t *seq_len;
    int64_t max_seq_len;
    int32_t ic_tiled;   // indexer pool in 64-row tiles (MLA_IC_TILE64)
    // queries per sequence: row b of a launch is query b % qps of sequence b / qps, at position
    // len - qps + b % qps where len is that sequence's length (seq_len or max_seq_len); it sees
    // keys 0 .. that position.  1 for one query per sequence at len - 1.
    int32_t qps;
};

inline KvView to_view(const mla_kv_view &v)
{
    KvView k;
    k.lc = v.lc;
    k.rc = v.rc;
    k.ic = v.ic;
    k.rows = v.rows;
    k.bt = v.block_table;
    k.bs = v.block_size > 0 ? v.block_size : 1;
    k.max_blocks = v.max_blocks;
    k.seq_stride = v.seq_stride;
    k.seq_len = v.seq_len;
    k.max_seq_len = v.max_seq_len;
    k.ic_tiled = v.ic_layout == MLA_IC_TILE64;
    k.qps = 1;
    return k;
}

// The sequence that launch row b belongs to.
__device__ __forceinline__ int kv_seq(const KvView &v, int b) { return v.qps > 1 ? b / v.qps : b; }

// Dims 4g .. 4g+3 of indexer row `row` (hd dims per row), in either pool layout.
__device__ __forceinline__ const float *ic_quad(const KvView &v, int64_t row, int g, int hd)
{
    return v.ic_tiled ? v.ic + ((row >> 6) * (hd >> 2) + g) * 256 + (row & 63) * 4 : v.ic + row * hd + 4 * g;
}

// Pool row of logical token t of launch row b, or -1 if it falls outside the pools.
// t must satisfy 0 <= t < max_seq_len (callers clamp), so the table index is in range.
__device__ __forceinline__ int64_t kv_row(const KvView &v, int b, int64_t t)
{
    b = kv_seq(v, b);
    int64_t r;
    if (v.bt) {
        int32_t blk = v.bt[(int64_t)b * v.max_blocks + t / v.bs];
        r = (int64_t)blk * v.bs + t % v.bs;
    } else {
        r = (int64_t)b * v.seq_stride + t;
    }
    return (r >= 0 && r < v.rows) ? r : -1;
}

// Keys launch row b sees (its query's position + 1), clamped to [0, max_seq_len]: seq_len[b] for one
// query per sequence.
__device__ __forceinline__ int64_t seq_len_of(const KvView &v, int b)
{
    const int sb = kv_seq(v, b);
    int64_t s = v.seq_len ? (int64_t)v.seq_len[sb] : v.max_seq_len;
    if (v.qps > 1) s -= v.qps - 1 - (b - sb * v.qps);
    if (s < 0) s = 0;
    if (s > v.max_seq_len) s = v.max_seq_len;
    return s;
}

// ------------------------------------------------------------------ RoPE
// Pair j of a rope_dim-wide interleaved tail at position pos: (a, b) -> (a cos - b sin,
// b cos + a sin) with angle pos * theta^(-2j/rope_dim) formed in double.  The rotation uses
// explicit fused multiply-adds so that every kernel that rotates produces the same bits.
// cos and sin of pair j's angle at pos, formed in double and rounded to float
__device__ __forceinline__ void rope_cs(int j, int rope_dim, double pos, double theta, float &c, float &sn)
{
    const double inv = pow(theta, -2.0 * (double)j / (double)rope_dim);
    double sd, cd;
    sincos(pos * inv, &sd, &cd);
    c = (float)cd;
    sn = (float)sd;
}

__device__ __forceinline__ void rope_apply(float a, float b, float c, float sn, float &lo, float &hi)
{
    lo = __builtin_fmaf(a, c, -(b * sn));
    hi = __builtin_fmaf(b, c, a * sn);
}

__device__ __forceinline__ void rope_pair(float a, float b, int j, int rope_dim, double pos, double theta,
                                          float &lo, float &hi)
{
    float c, sn;
    rope_cs(j, rope_dim, pos, theta, c, sn);
    rope_apply(a, b, c, sn, lo, hi);
}

// ------------------------------------------------------------------ selection keys
// Order-preserving map fp32 -> uint32 (larger score -> larger key); -0.0 maps like +0.0.
// Histogram of the top 11 order-key bits used by the key selection, written without atomics:
// every workgroup p of a producing kernel (the indexer, or the histogram kernel) writes the
// nonzero bins of its own keys as a list: entry i of part p, i < hcnt[b][p], in descending bin
// order, is hl[b][hl_row(i, p)][p] = (bin << 21) | count (entry-major, so that one row of
// consecutive parts is contiguous for the reader).  The first HL_TOP entries of part p sit in rows
// rotated by p: the lists of different parts are much alike (entry i of every part is a bin near
// the top of the row's range, often the same one), and a reader that loads one row for 64
// consecutive parts then holds 16 different depths across its lanes, so its LDS histogram atomics
// spread over many bins instead of piling onto one.  The row histogram is the sum of its parts'
// lists.
constexpr int HIST_BINS = 2048;
constexpr int HL_CAP = HIST_BINS;          // entries per part (every bin nonzero at most)
constexpr int HL_TOP = 16;                 // rotated head of every list (the entries a reader takes first)
static_assert((HL_TOP & (HL_TOP - 1)) == 0, "list heads rotate modulo HL_TOP");
__device__ __forceinline__ uint32_t hl_entry(uint32_t bin, uint32_t count) { return (bin << 21) | count; }
__device__ __forceinline__ int hl_row(int i, int part) { return i < HL_TOP ? ((i + part) & (HL_TOP - 1)) : i; }

__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------------ wave helpers (wave64)
__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

// ------------------------------------------------------------------ scans (wave64)
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

// The same without the closing barrier, for a caller that gives every call its own sh (NW words)
// within one pass of the block, so that no later write can meet a slower thread's read.
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan_once(uint32_t v, uint32_t *sh, uint32_t *total = nullptr)
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
    return before + inc - v;
}

// Two exclusive scans behind one barrier (sh: 2 NW words, used once as above); ta, tb: totals.
template <int NW>
__device__ __forceinline__ void block_excl_scan2_once(uint32_t a, uint32_t b, uint32_t *sh, uint32_t &ea, uint32_t &eb,
                                                      uint32_t *ta = nullptr, uint32_t *tb = nullptr)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t ia = wave_incl_scan_dpp(a), ib = wave_incl_scan_dpp(b);
    if (lane == 63) {
        sh[wave] = ia;
        sh[NW + wave] = ib;
    }
    __syncthreads();
    uint32_t ba = 0u, bb = 0u, sa = 0u, sb = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t x = sh[w], y = sh[NW + w];
        ba += w < wave ? x : 0u;
        bb += w < wave ? y : 0u;
        sa += x;
        sb += y;
    }
    ea = ba + ia - a;
    eb = bb + ib - b;
    if (ta) *ta = sa;
    if (tb) *tb = sb;
}

// Writes the nonzero bins of the complete LDS histogram hs (HIST_BINS, every thread of an NT-thread
// block calls it) as the list of part `part` (descending bins; entry i at list[hl_row(i, part) *
// stride]) and its length `count`; sh: NT / 64 words.
template <int NT>
__device__ __forceinline__ void hist_write_list(const uint32_t *hs, uint32_t *__restrict__ list, int64_t stride,
                                                int part, uint32_t *__restrict__ count, uint32_t *sh)
{
    constexpr int PER = HIST_BINS / NT;   // bins per thread, thread order = descending bins
    const int top = HIST_BINS - 1 - PER * (int)threadIdx.x;
    uint32_t c[PER], nz = 0u;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        c[q] = hs[top - q];
        nz += c[q] ? 1u : 0u;
    }
    uint32_t total;
    uint32_t off = block_excl_scan_dpp<NT / 64>(nz, sh, &total);
#pragma unroll
    for (int q = 0; q < PER; ++q)
        if (c[q]) list[(int64_t)hl_row((int)(off++), part) * stride] = hl_entry((uint32_t)(top - q), c[q]);
    if (threadIdx.x == 0) *count = total;
}

// ------------------------------------------------------------------ internal launchers
mla_status launch_rope(void *x, mla_dtype dt, int64_t n_tok, int32_t n_heads, int64_t tok_stride,
                       int64_t head_stride, int32_t rope_off, int32_t rope_dim, const int32_t *pos,
                       double theta, hipStream_t s);
mla_status launch_rope_decode(const void *x, void *y, mla_dtype dt, int32_t B, int32_t n_heads, int32_t rope_dim,
                              const KvView &kv, double theta, hipStream_t s);

// hl, hcnt (optional): the histogram lists of the scores of keys t < seq_len (format above), one
// part per workgroup of the launch; *parts receives the number of parts per row, at most
// hist_parts_max(B, t_max).
struct HistOut {
    uint32_t *hl;     // [B][HL_CAP][parts_max]
    uint32_t *hcnt;   // [B][parts_max]
    int parts_max;    // row stride in parts
    int parts;        // set by the launch
};
int hist_parts_max(int32_t B, int64_t t_max);
mla_status launch_index_scores(const float *q, const float *w, int32_t B, int32_t n_ih, int32_t hd,
                               const KvView &kv, int64_t t_max, float *scores, HistOut *hist, hipStream_t s);

mla_status launch_score_hist(const float *scores, int32_t B, int64_t t_max, const KvView &kv, HistOut *hist,
                             hipStream_t s);
size_t index_select_workspace_bytes(int32_t B, int64_t t_max, int32_t k);
// Work that the fused decode step runs beside the select's resolve step (matrix-core decode
// geometry: 64 heads, kv_lora 512, bf16): q_abs = W_UK^T q_nope, and the query tails rotated
// by RoPE at position seq_len - 1 into q_rope_out.
constexpr int SIDE_MAXB = 32;
struct SideAbsorb {
    const bf16_t *q_nope;   // [B][64][nope]
    const void *kv_b;       // [64 (nope + v)][512]: bf16, or the codes of a quantized kv_b
    const void *scales;     // the scales of a quantized kv_b (qformat.h)
    int fmt;                // 0 for bf16, else an mla_qformat
    bf16_t *q_abs;          // [B][64][512]
    const bf16_t *q_rope;   // [B][64][rope], before rotation
    bf16_t *q_rope_out;     // [B][64][rope]; nullptr: no rotation
    int B, nope, v, rope;
    double theta;
};
// The side work as a launch of its own (when no selection runs beside it)
bool side_absorb_ok(const SideAbsorb &sa);
mla_status launch_absorb_rope(const SideAbsorb &sa, const KvView &kv, hipStream_t s);
mla_status launch_index_select(const float *q, const float *w, int32_t B, int32_t n_ih, int32_t hd, const KvView &kv,
                               int64_t t_max, int32_t k, float *scores, int32_t *sel, int32_t *nsel, void *ws,
                               size_t ws_bytes, hipStream_t s,
                               const SideAbsorb *side = nullptr, bool *side_done = nullptr);
size_t topk_workspace_bytes(int32_t B, int64_t t_max, int32_t k);
// n_valid (optional): row lengths, clamped to [0, max_len]; without it every row has max_len
mla_status launch_topk(const float *scores, int32_t B, int64_t t_max, const int32_t *n_valid, int64_t max_len,
                       int32_t k, int32_t *sel, int32_t *nsel, void *ws, size_t ws_bytes, hipStream_t s);

size_t decode_workspace_bytes(const mla_dims &d, int32_t B, int64_t max_keys, mla_dtype dt);
size_t decode_absorb_workspace_bytes(const mla_dims &d, int32_t B, mla_dtype dt);
mla_status launch_decode_absorb(const void *q_nope, const void *kv_b, mla_dtype dt, const mla_dims &d, int32_t B,
                                void *ws, hipStream_t s);
mla_status launch_decode_attend(const void *q_rope, const void *kv_b, mla_dtype dt, const mla_dims &d, int32_t B,
                                const KvView &kv, const int32_t *sel, const int32_t *nsel, int32_t sel_stride,
                                int64_t max_keys, float sm_scale, float *out, void *ws, hipStream_t s);
mla_status launch_decode(const void *q_nope, const void *q_rope, const void *kv_b, mla_dtype dt,
                         const mla_dims &d, int32_t B, const KvView &kv, const int32_t *sel,
                         const int32_t *nsel, int32_t sel_stride, int64_t max_keys,
                         float sm_scale, float *out, void *ws, size_t ws_bytes, hipStream_t s);
size_t dsa_decode_workspace_bytes(const mla_dims &d, int32_t B, int64_t t_max, int32_t k, mla_dtype dt);
mla_status launch_dsa_decode(const void *q_nope, const void *q_rope, mla_dtype dt, double theta, const float *q_idx,
                             const float *w_idx, int32_t n_ih, int32_t hd, const void *kv_b, const mla_dims &d,
                             int32_t B, const KvView &kv_sel, const KvView &kv, int64_t t_max, int32_t k,
                             float sm_scale, float *scores, int32_t *sel, int32_t *nsel, float *out, void *ws,
                             hipStream_t s);

mla_status launch_cache_write(const void *comp, const void *ik, mla_dtype in_dt, int64_t n, const int32_t *seq,
                              const int32_t *pos, int32_t n_seq, const KvView &kv, mla_dtype kv_dt, int32_t L,
                              int32_t rope, int32_t hd, const float *kv_gain, const float *gamma, const float *beta,
                              int32_t ix_off, int32_t ix_rdim, float eps_kv, float eps_ix, double theta,
                              hipStream_t s);

// absorbed decode with quantized kv_b rows (quant.hip); workspace as decode_workspace_bytes
bool decode_quant_supported(const mla_dims &d, mla_dtype dt);
mla_status launch_decode_quant(const void *q_nope, const void *q_rope, const uint8_t *codes, const void *scales,
                               int32_t fmt, const mla_dims &d, int32_t B, const KvView &kv, const int32_t *sel,
                               const int32_t *nsel, int32_t sel_stride, int64_t max_keys, float sm_scale, float *out,
                               void *ws, hipStream_t s);

mla_status launch_dsa_decode_quant(const void *q_nope, const void *q_rope, double theta, const float *q_idx,
                                   const float *w_idx, int32_t n_ih, int32_t hd, const uint8_t *codes,
                                   const void *scales, int32_t fmt, const mla_dims &d, int32_t B, const KvView &kv_sel,
                                   const KvView &kv, int64_t t_max, int32_t k, float sm_scale, float *scores,
                                   int32_t *sel, int32_t *nsel, float *out, void *ws, hipStream_t s);

// The library's static device scratch (noalloc.hip): its size, and its address on the calling
// thread's current device (looked up once per device).
constexpr size_t NOALLOC_SCRATCH_BYTES = MLA_NOALLOC_SCRATCH_BYTES;
mla_status noalloc_scratch(void **ptr);

size_t dsa_shared_workspace_bytes(const mla_dims &d, int32_t B, int32_t k, mla_dtype dt);
mla_status launch_dsa_shared(const void *q_nope, const void *q_rope, mla_dtype dt, double theta, const void *kv_b,
                             const mla_dims &d, int32_t B, const KvView &kv, const int32_t *sel, const int32_t *nsel,
                             int32_t k, float sm_scale, float *out, void *ws, hipStream_t s);

size_t prefill_workspace_bytes(const mla_dims &d, int32_t S, int64_t T, mla_dtype dt);
// mask (optional): keys further restricted per query, bit t % 32 of mask[(t / 32) * mask_stride + i];
// mask_stride >= S rounded up to 128, 2 * ceil((pos_base + S) / 64) words per query column
mla_status launch_prefill(const void *q, const void *kv_b, mla_dtype dt, const mla_dims &d,
                          const KvView &kv, int32_t S, int32_t pos_base, float sm_scale,
                          void *out, mla_dtype out_dt, void *ws, size_t ws_bytes, hipStream_t s,
                          const uint32_t *mask = nullptr, int mask_stride = 0);

// S queries of one sequence ([MLA] sec. 2.3 g_absorb rule) and their selections
bool attention_absorbs(int32_t S, int32_t g_absorb);
size_t attention_workspace_bytes(const mla_dims &d, int32_t S, int64_t T, int32_t sel_stride, bool absorbed,
                                 mla_dtype dt);
mla_status launch_attention(const void *q, mla_dtype dt, const void *kv_b, const mla_dims &d, const KvView &kv,
                            int32_t S, int32_t pos_base, const int32_t *sel, const int32_t *nsel, int32_t sel_stride,
                            float sm_scale, bool absorbed, float *out, void *ws, hipStream_t s);

}  // namespace mla
