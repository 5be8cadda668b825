// dsa_index.hip -- DSA lightning-indexer scores.
// colibri-analysis 06 "MLA attention and KV cache", sec. 2.2: each causal key t gets a
// ReLU-gated, per-head-weighted score  I[t] = sum_h w[h] * ReLU(q[h] . Ic[t]);
// "Ch.7 sec. 03 ... faithful DSA", sec. 2: Ic is fp32 (index_hd x 4 bytes per token).
//
// Fixed evaluation order (the contract that makes the selected set exact): s = +0; for h
// ascending { a = +0; for d ascending a = fma(q[h][d], Ic[t][d], a); s = fma(w[h], max(a,+0), s) }.
// Every kernel below performs exactly this sequence of fp32 operations per key.
#include "common.h"

namespace mla {

// One lane per key.  The query (n_ih x HD fp32) is uniform across the block and is read
// with scalar loads; the key row lives in VGPRs.  Heads run four at a time as independent
// fma chains; their weighted sum is still folded into s in ascending head order.
template <int HD>
__global__ __launch_bounds__(256) void index_scores_lane_per_key(const float *__restrict__ q,
                                                                 const float *__restrict__ w, int n_ih,
                                                                 KvView kv, int64_t t_max,
                                                                 float *__restrict__ scores)
{
    const int b = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= t_max) return;
    float *out = scores + (int64_t)b * t_max;
    const int64_t n = seq_len_of(kv, b);
    if (t >= n) {
        out[t] = -INFINITY;
        return;
    }
    const int64_t row = kv_row(kv, b, t);
    if (row < 0) {
        out[t] = -INFINITY;
        return;
    }
    float k[HD];
#pragma unroll
    for (int i = 0; i < HD / 4; ++i) {
        const float4 v = *reinterpret_cast<const float4 *>(ic_quad(kv, row, i, HD));
        k[4 * i + 0] = v.x;
        k[4 * i + 1] = v.y;
        k[4 * i + 2] = v.z;
        k[4 * i + 3] = v.w;
    }
    const float *qb = q + (int64_t)b * n_ih * HD;
    const float *wb = w + (int64_t)b * n_ih;
    float s = 0.0f;
    int h = 0;
    for (; h + 4 <= n_ih; h += 4) {
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
        const float *q0 = qb + h * HD;
#pragma unroll
        for (int d = 0; d < HD; ++d) {
            a0 = __builtin_fmaf(q0[d], k[d], a0);
            a1 = __builtin_fmaf(q0[HD + d], k[d], a1);
            a2 = __builtin_fmaf(q0[2 * HD + d], k[d], a2);
            a3 = __builtin_fmaf(q0[3 * HD + d], k[d], a3);
        }
        s = __builtin_fmaf(wb[h + 0], a0 > 0.f ? a0 : 0.f, s);
        s = __builtin_fmaf(wb[h + 1], a1 > 0.f ? a1 : 0.f, s);
        s = __builtin_fmaf(wb[h + 2], a2 > 0.f ? a2 : 0.f, s);
        s = __builtin_fmaf(wb[h + 3], a3 > 0.f ? a3 : 0.f, s);
    }
    for (; h < n_ih; ++h) {
        float a = 0.f;
        const float *q0 = qb + h * HD;
#pragma unroll
        for (int d = 0; d < HD; ++d) a = __builtin_fmaf(q0[d], k[d], a);
        s = __builtin_fmaf(wb[h], a > 0.f ? a : 0.f, s);
    }
    out[t] = s;
}

// Any index_hd (multiple of 4, <= 256): the key row is re-read per head from cache.
__global__ __launch_bounds__(256) void index_scores_generic(const float *__restrict__ q,
                                                           const float *__restrict__ w, int n_ih, int hd,
                                                           KvView kv, int64_t t_max,
                                                           float *__restrict__ scores)
{
    const int b = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= t_max) return;
    float *out = scores + (int64_t)b * t_max;
    const int64_t n = seq_len_of(kv, b);
    const int64_t row = t < n ? kv_row(kv, b, t) : -1;
    if (row < 0) {
        out[t] = -INFINITY;
        return;
    }
    const float *qb = q + (int64_t)b * n_ih * hd;
    const float *wb = w + (int64_t)b * n_ih;
    float s = 0.0f;
    for (int h = 0; h < n_ih; ++h) {
        float a = 0.f;
        for (int d = 0; d < hd; ++d) a = __builtin_fmaf(qb[h * hd + d], ic_quad(kv, row, d >> 2, hd)[d & 3], a);
        s = __builtin_fmaf(wb[h], a > 0.f ? a : 0.f, s);
    }
    out[t] = s;
}

// ------------------------------------------------------------------------------------------
// Matrix-core path for 32 heads x 128 dims.  v_mfma_f32_32x32x1_2b_f32 multiplies a 32x1
// column by a 1x32 row and adds it to a 32x32 accumulator, in two independent blocks; with
// one product per output element it rounds exactly like fmaf (checked against fmaf on the
// host for 16.7M random triples).  Chaining it over d = 0..127 therefore reproduces the
// fixed fp32 order bit for bit, at twice the rate of the vector ALU.
//   lane L supplies a = q[L % 32][d] (head) and b = Ic[key L][d]; block 0 covers keys
//   0..31 of the tile, block 1 keys 32..63.  Accumulator register r (0..15) of lane L holds
//   block 0, key L % 32, head 8*(r/4) + 4*(L/32) + r%4; registers 16..31 hold block 1.
// A wave owns 64-key tiles.  Lane L loads key L's row straight into registers, 32 dims
// (one slice, 8 x 16 B) at a time, through a ring of one slice refilled group by group (the
// single-query kernel) or of two slices (the multi-query kernel): while slice s feeds its
// MFMAs, the next slice is already in flight.  No LDS staging is needed because
// the B operand of this MFMA is exactly "key L's value at dim d" in lane L.  The query
// (32 x 128) is staged in LDS once per block, before any key load is issued, so that the
// block barrier does not wait on the key stream.
typedef float v32f __attribute__((ext_vector_type(32)));

constexpr int IXM_WAVES = 4;
constexpr int IXM_QROW = 128 + 4;    // floats per query row in LDS (pad against bank conflicts)

// Pointer for the lane-private loads of key (tile * 64 + lane).  A key with no score (past the
// sequence or outside the pools) reads from `dummy` instead (any readable range of the right
// size), so that every load is unconditional; its lane's result is replaced by -inf.
//   MODE 0: contiguous rows (no block table);
//   MODE 1: block table with block_size % 64 == 0 -- the whole tile sits in one block, so the
//           table entry is wave-uniform and is fetched with a scalar load, which leaves the
//           vector-memory counter (and the key stream waiting on it) alone;
//   MODE 2: any block size, one table lookup per lane (row layout only).
// Row layout: the key's 512-byte row.  TILED (64-row tiles, 128 dims): the lane's first quad in
// its tile, tile + 4 lane; the tile holds all 64 keys in dims-major quads.
template <int MODE, bool TILED>
__device__ __forceinline__ const float *ix_key_ptr(const KvView &kv, int b, int64_t tile, int lane, int64_t n,
                                                   const float *dummy, bool &valid)
{
    const int64_t t = tile * 64 + lane;
    int64_t row;
    if (MODE == 0) {
        row = (int64_t)kv_seq(kv, b) * kv.seq_stride + t;
    } else if (MODE == 1) {
        const int64_t t0 = tile * 64;
        // read through the constant address space, so that the uniform entry is a scalar load: a
        // vector load here is counted with the key slices in flight, and waiting for it drains them
        typedef const __attribute__((address_space(4))) int32_t cbt_t;
        cbt_t *bt = (cbt_t *)kv.bt;
        const int64_t blk = bt[(int64_t)kv_seq(kv, b) * kv.max_blocks + t0 / kv.bs];
        row = blk < 0 ? -1 : blk * kv.bs + t0 % kv.bs + lane;
    } else {
        row = t < n ? kv_row(kv, b, t) : -1;
    }
    valid = t < n && row >= 0 && row < kv.rows;
    if (TILED) return valid ? kv.ic + (row >> 6) * 64 * 128 + 4 * lane : dummy;
    return valid ? kv.ic + row * 128 : dummy;
}

// The key stream is read once per call: nontemporal loads (the nt bit) keep it from displacing
// what the following launches read from the caches (the scores and lists just written, the
// weights), and stream faster themselves (alone 17.1 -> 15.7 us, decode step 47.0 -> 43.7 us,
// same box, alternating).
typedef float ix_f4 __attribute__((ext_vector_type(4)));

// acc += q x K^T over one 64-key tile, one MFMA per dim, d ascending.
// A tile's 128 products per output over a ring of IX_LAG four-dim groups, refilled group by
// group: once the four MFMAs of group g (dims 4g .. 4g+3) are issued, its ring slot is reloaded
// with group g + IX_LAG (of this tile at p, or of the next tile at pn), so a wave keeps IX_LAG
// groups in flight all the time and its products run as the groups arrive.  The query group is
// read from LDS one group ahead: qq holds group 0 on entry and on exit (the query rows are the
// same for every tile).  Eight groups (one slice, 8 KB per wave) stream best: four took the
// T = 131072 indexer from 13.7-13.9 to 14.2-14.3 us and two to 17.9 us (same box, alternating).
constexpr int IX_LAG = 8;
typedef float ixk_t __attribute__((ext_vector_type(4 * IX_LAG)));
static_assert(32 % IX_LAG == 0, "a tile's groups must fill whole rings");

template <bool TILED>
__device__ __forceinline__ void ix_load_ring(ixk_t &K, const float *p)
{
#pragma unroll
    for (int g = 0; g < IX_LAG; ++g) {
        const ix_f4 x = __builtin_nontemporal_load(reinterpret_cast<const ix_f4 *>(TILED ? p + g * 256 : p + 4 * g));
        K[4 * g + 0] = x.x;
        K[4 * g + 1] = x.y;
        K[4 * g + 2] = x.z;
        K[4 * g + 3] = x.w;
    }
}

template <bool TILED>
__device__ __forceinline__ void ix_tile_refill(v32f &acc, ixk_t &K, const float *qrow, float4 &qq, const float *p,
                                               const float *pn)
{
#pragma unroll
    for (int g = 0; g < 32; ++g) {
        const int sl = 4 * (g % IX_LAG);
        const float4 qn = *reinterpret_cast<const float4 *>(&qrow[4 * ((g + 1) & 31)]);
        acc = __builtin_amdgcn_mfma_f32_32x32x1f32(qq.x, K[sl + 0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x1f32(qq.y, K[sl + 1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x1f32(qq.z, K[sl + 2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x1f32(qq.w, K[sl + 3], acc, 0, 0, 0);
        const int gl = (g + IX_LAG) & 31;
        const float *src = g + IX_LAG < 32 ? p : pn;
        const ix_f4 x =
            __builtin_nontemporal_load(reinterpret_cast<const ix_f4 *>(TILED ? src + gl * 256 : src + 4 * gl));
        K[sl + 0] = x.x;
        K[sl + 1] = x.y;
        K[sl + 2] = x.z;
        K[sl + 3] = x.w;
        qq = qn;
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The same for QB queries against each key group (the multi-query kernel): each group's products
// of every query are issued before its ring slot is refilled; qq[qi] holds group 0 of query qi's
// rows on entry and on exit.
template <bool TILED, int QB>
__device__ __forceinline__ void ix_tile_refill_mq(v32f (&acc)[QB], ixk_t &K, const float *qrow, float4 (&qq)[QB],
                                                  const float *p, const float *pn)
{
#pragma unroll
    for (int g = 0; g < 32; ++g) {
        const int sl = 4 * (g % IX_LAG);
        float4 qn[QB];
#pragma unroll
        for (int qi = 0; qi < QB; ++qi)
            qn[qi] = *reinterpret_cast<const float4 *>(&qrow[qi * 32 * IXM_QROW + 4 * ((g + 1) & 31)]);
#pragma unroll
        for (int qi = 0; qi < QB; ++qi) {
            acc[qi] = __builtin_amdgcn_mfma_f32_32x32x1f32(qq[qi].x, K[sl + 0], acc[qi], 0, 0, 0);
            acc[qi] = __builtin_amdgcn_mfma_f32_32x32x1f32(qq[qi].y, K[sl + 1], acc[qi], 0, 0, 0);
            acc[qi] = __builtin_amdgcn_mfma_f32_32x32x1f32(qq[qi].z, K[sl + 2], acc[qi], 0, 0, 0);
            acc[qi] = __builtin_amdgcn_mfma_f32_32x32x1f32(qq[qi].w, K[sl + 3], acc[qi], 0, 0, 0);
        }
        const int gl = (g + IX_LAG) & 31;
        const float *src = g + IX_LAG < 32 ? p : pn;
        const ix_f4 x =
            __builtin_nontemporal_load(reinterpret_cast<const ix_f4 *>(TILED ? src + gl * 256 : src + 4 * gl));
        K[sl + 0] = x.x;
        K[sl + 1] = x.y;
        K[sl + 2] = x.z;
        K[sl + 3] = x.w;
#pragma unroll
        for (int qi = 0; qi < QB; ++qi) qq[qi] = qn[qi];
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Score of key L in lane L from the accumulator: lanes L and L^32 hold complementary head
// groups of the same two keys, so one v_permlane32_swap per register pair leaves every lane
// with heads 8g..8g+3 of its key in lo[] and heads 8g+4..8g+7 in hi[]; the heads are then folded
// in ascending order.  (Selecting acc[r] or acc[16 + r] by lane half would index the register
// array per lane, which compiles to long chains of selects.)
__device__ __forceinline__ float ix_fold(const v32f &acc, const float *__restrict__ w)
{
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        float lo[4], hi[4];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int r = 4 * g + r4;
            const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[r]), __float_as_uint(acc[16 + r]),
                                                            false, false);
            lo[r4] = __uint_as_float(p[0]);
            hi[r4] = __uint_as_float(p[1]);
        }
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) s = __builtin_fmaf(w[8 * g + r4], lo[r4] > 0.f ? lo[r4] : 0.f, s);
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) s = __builtin_fmaf(w[8 * g + 4 + r4], hi[r4] > 0.f ? hi[r4] : 0.f, s);
    }
    return s;
}

// HIST: also count the top 11 order-key bits of every score with t < n in an LDS histogram and
// write its nonzero bins as this workgroup's list (part blockIdx.x of row b) -- the first pass of
// the top-k selection.
constexpr int IX_BINS = HIST_BINS;

template <int MODE, bool HIST, bool TILED>
__global__ __launch_bounds__(64 * IXM_WAVES) void index_scores_mfma(const float *__restrict__ q,
                                                                     const float *__restrict__ w, KvView kv,
                                                                     int64_t t_max, float *__restrict__ scores,
                                                                     uint32_t *__restrict__ hl,
                                                                     uint32_t *__restrict__ hcnt, int parts_max)
{
    __shared__ float sq[32 * IXM_QROW];
    __shared__ uint32_t hs[HIST ? IX_BINS : 1];
    __shared__ uint32_t sh_scan[IXM_WAVES];
    const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: tile math stays scalar
    const int64_t n = seq_len_of(kv, b) < t_max ? seq_len_of(kv, b) : t_max;
    const int64_t ntv = (n + 63) / 64;   // tiles holding at least one scored key
    const int64_t waves_total = (int64_t)gridDim.x * IXM_WAVES;
    float *out = scores + (int64_t)b * t_max;
    const float *wb = w + (int64_t)b * 32;

    // whole tiles past the last scored key
    for (int64_t t = ntv * 64 + (int64_t)blockIdx.x * 64 * IXM_WAVES + tid; t < t_max; t += waves_total * 64)
        out[t] = -INFINITY;
    if ((int64_t)blockIdx.x * IXM_WAVES >= ntv) {   // no tile of a shorter row: an empty list, no query staging
        if (HIST && tid == 0) hcnt[(int64_t)b * parts_max + blockIdx.x] = 0u;
        return;
    }

    if (HIST)
        for (int i = tid; i < IX_BINS; i += 64 * IXM_WAVES) hs[i] = 0u;
    // The query's loads go out first and the wave's first key slice right behind them; the query
    // is then staged in LDS while the key data is still on its way (loads return in issue order,
    // so the stores wait for the query only), and the barrier waits for LDS alone.  The key
    // pointer is formed before the query's loads (its branches would otherwise let the compiler
    // sink them behind the key slice), and the slices are loaded unconditionally, from the
    // stand-in for a wave without a tile.  One slice in flight per wave, kept full by the
    // group-by-group refill, streams faster than two (a wave then folds a slice in while the
    // next arrives, and the chip holds 8 MB of requests in flight instead of up to 16 MB).
    int64_t tile = (int64_t)blockIdx.x * IXM_WAVES + wave;
    const float *qrow = &sq[(lane & 31) * IXM_QROW];
    // stand-in for keys without a row: the query block (512 B rows), or the pool's first tile
    const float *qraw = TILED ? kv.ic + 4 * lane : q + (int64_t)b * 32 * 128;
    bool valid = false, valid_n = false;
    const float *p = qraw;
    if (tile < ntv) p = ix_key_ptr<MODE, TILED>(kv, b, tile, lane, n, qraw, valid);
    // (native vectors: a struct copy from memory to LDS would become one memcpy at the store)
    const ix_f4 *qb = reinterpret_cast<const ix_f4 *>(q + (int64_t)b * 32 * 128);
    ix_f4 qv[32 * 32 / (64 * IXM_WAVES)];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 32 * 32 / (64 * IXM_WAVES); ++k) qv[k] = qb[tid + k * 64 * IXM_WAVES];
    __builtin_amdgcn_sched_barrier(0);
    ixk_t K;
    v32f acc;
    ix_load_ring<TILED>(K, p);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 32 * 32 / (64 * IXM_WAVES); ++k) {
        const int i = tid + k * 64 * IXM_WAVES;
        *reinterpret_cast<ix_f4 *>(&sq[(i >> 5) * IXM_QROW + (i & 31) * 4]) = qv[k];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // the query and the cleared histogram

    if (tile < ntv) {   // (no early return: the histogram flush below needs every wave at the barrier)
    float4 qq = *reinterpret_cast<const float4 *>(&qrow[0]);
    for (; tile < ntv; tile += waves_total) {
        // the next tile's first slice is loaded unconditionally (from the stand-in when there
        // is no next tile) so every iteration leaves the same loads in flight
        const int64_t nxt = tile + waves_total;
        const float *pn = qraw;
        valid_n = false;
        if (nxt < ntv) pn = ix_key_ptr<MODE, TILED>(kv, b, nxt, lane, n, qraw, valid_n);
#pragma unroll
        for (int r = 0; r < 32; ++r) acc[r] = 0.f;
        ix_tile_refill<TILED>(acc, K, qrow, qq, p, pn);
        const float s = ix_fold(acc, wb);
        const int64_t t = tile * 64 + lane;
        const float sc = valid ? s : -INFINITY;
        if (t < t_max) out[t] = sc;
        if (HIST && t < n) atomicAdd(&hs[order_key(sc) >> 21], 1u);
        p = pn;
        valid = valid_n;
    }
    }
    if (HIST) {
        __syncthreads();
        hist_write_list<64 * IXM_WAVES>(hs, hl + (int64_t)b * HL_CAP * parts_max + blockIdx.x, parts_max,
                                        (int)blockIdx.x, hcnt + (int64_t)b * parts_max + blockIdx.x, sh_scan);
    }
}

// The same for launch rows that are queries of one sequence (KvView.qps > 1): a workgroup scores
// the QB consecutive queries r0 .. r0 + nb - 1 of one sequence against each key tile it loads, so
// a key row is read once for all of them; each query keeps its own accumulators and its own
// causal length (t < n of that row), and the products of each query are the same chain as above.
// grid.y = sequences x nbps blocks of QB queries (the last block of a sequence may hold fewer).
// Queries per workgroup of the multi-query indexer.  Two (50 KB of LDS, three workgroups per CU)
// beat four (100 KB, one per CU): 0.81-0.84 against 0.83-0.85 ms for the selection of 4096
// prefill queries, 65.5 against 69 us for 4 queries at 131072 keys (one query per workgroup:
// 1.11 ms and 73 us).
constexpr int IX_QB = 2;

template <int MODE, bool HIST, bool TILED, int QB>
__global__ __launch_bounds__(64 * IXM_WAVES) void index_scores_mfma_mq(const float *__restrict__ q,
                                                                     const float *__restrict__ w, KvView kv,
                                                                     int64_t t_max, float *__restrict__ scores,
                                                                     uint32_t *__restrict__ hl,
                                                                     uint32_t *__restrict__ hcnt, int parts_max,
                                                                     int nbps)
{
    __shared__ float sq[QB * 32 * IXM_QROW];
    __shared__ uint32_t hs[HIST ? QB * IX_BINS : 1];
    __shared__ uint32_t sh_scan[IXM_WAVES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: tile math stays scalar
    const int by = gridDim.y - 1 - blockIdx.y;   // the longest query blocks start first
    const int sqn = by / nbps, jb = by - sqn * nbps;
    const int r0 = sqn * kv.qps + jb * QB;
    const int nb = kv.qps - jb * QB < QB ? kv.qps - jb * QB : QB;
    int64_t nq[QB];
    int64_t n = 0;   // the longest causal range of the block
#pragma unroll
    for (int qi = 0; qi < QB; ++qi) {
        const int64_t l = qi < nb ? seq_len_of(kv, r0 + qi) : 0;
        nq[qi] = l < t_max ? l : t_max;
        n = nq[qi] > n ? nq[qi] : n;
    }
    const int64_t ntv = (n + 63) / 64;   // tiles holding at least one scored key
    const int64_t waves_total = (int64_t)gridDim.x * IXM_WAVES;

    // whole tiles past the last scored key
    for (int qi = 0; qi < nb; ++qi) {
        float *out = scores + (int64_t)(r0 + qi) * t_max;
        for (int64_t t = ntv * 64 + (int64_t)blockIdx.x * 64 * IXM_WAVES + tid; t < t_max; t += waves_total * 64)
            out[t] = -INFINITY;
    }
    if ((int64_t)blockIdx.x * IXM_WAVES >= ntv) {   // no tile of a shorter row: an empty list, no query staging
        if (HIST && tid < nb) hcnt[(int64_t)(r0 + tid) * parts_max + blockIdx.x] = 0u;
        return;
    }

    if (HIST)
        for (int i = tid; i < QB * IX_BINS; i += 64 * IXM_WAVES) hs[i] = 0u;
    // queries to LDS: all loads in flight before the first store (rows past nb repeat the last)
    constexpr int QL = 32 * 32 / (64 * IXM_WAVES);
    float4 qv[QB * QL];
#pragma unroll
    for (int qi = 0; qi < QB; ++qi) {
        const float4 *qb = reinterpret_cast<const float4 *>(q + (int64_t)(r0 + (qi < nb ? qi : nb - 1)) * 32 * 128);
#pragma unroll
        for (int k = 0; k < QL; ++k) qv[qi * QL + k] = qb[tid + k * 64 * IXM_WAVES];
    }
#pragma unroll
    for (int qi = 0; qi < QB; ++qi)
#pragma unroll
        for (int k = 0; k < QL; ++k) {
            const int i = tid + k * 64 * IXM_WAVES;
            *reinterpret_cast<float4 *>(&sq[(qi * 32 + (i >> 5)) * IXM_QROW + (i & 31) * 4]) = qv[qi * QL + k];
        }
    __syncthreads();

    int64_t tile = (int64_t)blockIdx.x * IXM_WAVES + wave;
    if (tile < ntv) {   // (no early return: the histogram flush below needs every wave at the barrier)
    const float *qrow = &sq[(lane & 31) * IXM_QROW];

    // stand-in for keys without a row: the query block (512 B rows), or the pool's first tile
    const float *qraw = TILED ? kv.ic + 4 * lane : q + (int64_t)r0 * 32 * 128;
    bool valid, valid_n = false;
    const float *p = ix_key_ptr<MODE, TILED>(kv, r0, tile, lane, n, qraw, valid);
    ixk_t K;
    v32f acc[QB];
    ix_load_ring<TILED>(K, p);
    float4 qq[QB];
#pragma unroll
    for (int qi = 0; qi < QB; ++qi) qq[qi] = *reinterpret_cast<const float4 *>(&qrow[qi * 32 * IXM_QROW]);
    for (; tile < ntv; tile += waves_total) {
        // the next tile's first slice is loaded unconditionally (from the stand-in when there is
        // no next tile) so every iteration leaves the same loads in flight
        const int64_t nxt = tile + waves_total;
        const float *pn = qraw;
        valid_n = false;
        if (nxt < ntv) pn = ix_key_ptr<MODE, TILED>(kv, r0, nxt, lane, n, qraw, valid_n);
#pragma unroll
        for (int qi = 0; qi < QB; ++qi)
#pragma unroll
            for (int r = 0; r < 32; ++r) acc[qi][r] = 0.f;
        // (a block with nb < QB queries repeats its last query's rows: the spare products are
        // discarded, and the group loop stays free of branches)
        ix_tile_refill_mq<TILED, QB>(acc, K, qrow, qq, p, pn);
        const int64_t t = tile * 64 + lane;
#pragma unroll
        for (int qi = 0; qi < QB; ++qi) {
            if (qi < nb) {
                const float s = ix_fold(acc[qi], w + (int64_t)(r0 + qi) * 32);
                const bool in = t < nq[qi];
                const float sc = valid && in ? s : -INFINITY;
                if (t < t_max) scores[(int64_t)(r0 + qi) * t_max + t] = sc;
                if (HIST && in) atomicAdd(&hs[qi * IX_BINS + (order_key(sc) >> 21)], 1u);
            }
        }
        p = pn;
        valid = valid_n;
    }
    }
    if (HIST) {
        __syncthreads();
        for (int qi = 0; qi < nb; ++qi)
            hist_write_list<64 * IXM_WAVES>(hs + qi * IX_BINS,
                                            hl + (int64_t)(r0 + qi) * HL_CAP * parts_max + blockIdx.x, parts_max,
                                            (int)blockIdx.x, hcnt + (int64_t)(r0 + qi) * parts_max + blockIdx.x, sh_scan);
    }
}

// workgroups per row of index_scores_mfma (the histogram parts of a row)
static int64_t ixm_grid_x(int32_t B, int64_t t_max, bool tiled)
{
    const int64_t ntiles = (t_max + 63) / 64;
    int64_t bx;
    if (tiled) {
        // tiled keys: two tiles or more per wave, so that a wave requests its next tile while it
        // finishes the current one, and at most 256 workgroups per row (one per CU for a single
        // row).  Rows of a batch differ in length: the workgroups past a row's last key exit at
        // once and the many short workgroups keep every CU busy until the longest rows are done.
        bx = (ntiles + 2 * IXM_WAVES - 1) / (2 * IXM_WAVES);
        if (bx > 256) bx = 256;
    } else {
        // row keys: about 3 resident waves per SIMD over the chip; each wave strides over the tiles
        bx = 768 / B;
        const int64_t need = (ntiles + IXM_WAVES - 1) / IXM_WAVES;
        if (bx > need) bx = need;
    }
    return bx < 1 ? 1 : bx;
}

int hist_parts_max(int32_t B, int64_t t_max)
{
    int64_t m = (t_max + 1023) / 1024;   // the histogram kernel: one part per 1024 positions
    const int64_t a = ixm_grid_x(B, t_max, false), c = ixm_grid_x(B, t_max, true);
    if (a > m) m = a;
    if (c > m) m = c;
    return (int)(m < 1 ? 1 : m);
}

mla_status launch_index_scores(const float *q, const float *w, int32_t B, int32_t n_ih, int32_t hd,
                               const KvView &kv, int64_t t_max, float *scores, HistOut *hist, hipStream_t s)
{
    const int64_t gx = (t_max + 255) / 256;
    if (gx > 0x7fffffff || B > 65535) return fail(MLA_ERR_UNSUPPORTED, "index: grid too large");
    dim3 grid((unsigned)gx, (unsigned)B);
    const bool aligned = ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(kv.ic)) & 15u) == 0;
    if (hd == 128 && n_ih == 32 && aligned) {
        const int mode = !kv.bt ? 0 : (kv.bs % 64 == 0 ? 1 : 2);
        if (kv.ic_tiled && mode == 2) return fail(MLA_ERR_UNSUPPORTED, "index: tiled keys need block_size % 64 == 0");
        // queries of one sequence (qps > 1) share their key tiles, IX_QB per workgroup
        const bool multi = kv.qps > 1 && B % kv.qps == 0;
        const int nbps = multi ? (kv.qps + IX_QB - 1) / IX_QB : 1;
        const int64_t gy = multi ? (int64_t)(B / kv.qps) * nbps : B;
        int64_t bx = ixm_grid_x(multi ? (int32_t)gy : B, t_max, kv.ic_tiled != 0);
        if (multi) {
            // about four workgroups per CU over the launch (query blocks of a prefill differ in length
            // by up to the whole range, so many short workgroups even out the tail), at least one
            // tile per wave
            const int64_t want = (1024 + gy - 1) / gy, most = ((t_max + 63) / 64 + IXM_WAVES - 1) / IXM_WAVES;
            bx = want < most ? want : most;
            if (bx < 1) bx = 1;
        }
        uint32_t *hl = nullptr, *hc = nullptr;
        int pm = 0;
        if (hist) {
            if (multi && bx > hist->parts_max) bx = hist->parts_max;
            if (bx > hist->parts_max) return fail(MLA_ERR_UNSUPPORTED, "index: histogram parts exceed the workspace");
            hist->parts = (int)bx;
            hl = hist->hl;
            hc = hist->hcnt;
            pm = hist->parts_max;
        }
        const dim3 g((unsigned)bx, (unsigned)gy), blk(64 * IXM_WAVES);
#define IX_LAUNCH(M, H, TL)                                                                                         \
    do {                                                                                                            \
        if (multi)                                                                                                  \
            hipLaunchKernelGGL((index_scores_mfma_mq<M, H, TL, IX_QB>), g, blk, 0, s, q, w, kv, t_max, scores, hl,  \
                               hc, pm, nbps);                                                                       \
        else                                                                                                        \
            hipLaunchKernelGGL((index_scores_mfma<M, H, TL>), g, blk, 0, s, q, w, kv, t_max, scores, hl, hc, pm);   \
    } while (0)
        const bool h = hist != nullptr;
        if (kv.ic_tiled) {
            if (mode == 0) { if (h) IX_LAUNCH(0, true, true); else IX_LAUNCH(0, false, true); }
            else { if (h) IX_LAUNCH(1, true, true); else IX_LAUNCH(1, false, true); }
        } else if (mode == 0) { if (h) IX_LAUNCH(0, true, false); else IX_LAUNCH(0, false, false); }
        else if (mode == 1) { if (h) IX_LAUNCH(1, true, false); else IX_LAUNCH(1, false, false); }
        else { if (h) IX_LAUNCH(2, true, false); else IX_LAUNCH(2, false, false); }
#undef IX_LAUNCH
        return check_launch("index_scores");
    } else if (hd == 128 && aligned)
        hipLaunchKernelGGL(index_scores_lane_per_key<128>, grid, dim3(256), 0, s, q, w, n_ih, kv, t_max, scores);
    else
        hipLaunchKernelGGL(index_scores_generic, grid, dim3(256), 0, s, q, w, n_ih, hd, kv, t_max, scores);
    mla_status st = check_launch("index_scores");
    if (st || !hist) return st;
    return launch_score_hist(scores, B, t_max, kv, hist, s);   // kernels without a built-in histogram
}

}  // namespace mla
