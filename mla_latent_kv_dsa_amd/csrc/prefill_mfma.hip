// prefill_mfma.hip -- non-absorbed causal prefill on bf16 matrix cores for 64 heads, kv_lora
// 512, qk_rope 64, v_head 256 and qk_nope 128/192 (the GLM-5.2 geometry).  colibri-analysis 06
// "MLA attention and KV cache", sec. 2.3, non-absorbed path: one kv_b matmul rebuilds k_nope
// and v of every cached token, then causal softmax attention with
// score = q_nope . k_nope + q_rope . Rc over the keys t <= pos_base + i.
//
//   pf_kvb    C[t][n] = sum_l kv_b[n][l] Lc(t)[l], bf16 out ([T][H (nope + v)], head h's k_nope
//             then v in columns h (nope + v) ..).  Computed as C^T = kv_b . Lc^T in 256 x 256
//             tiles (wave: 128 x 128) on v_mfma_f32_32x32x16_bf16, K = 512 in steps of 64 copied
//             straight into LDS through a two-slot ring (16-byte chunks XOR-swizzled: conflict-free
//             operand reads); one v_permlane32_swap per register pair gives every lane eight
//             consecutive columns of one token: 16-byte stores.
//   pf_attn   per (128-query block, head), 64-key tiles of K (k_nope and Rc, 256 dims) and V (256
//             dims) staged in LDS, two waves per SIMD with split roles:
//               S-wave  S^T = K Q^T (A = K rows from LDS, B = its 32 queries held in registers),
//                       masks, online softmax (lane l owns query l % 32 with lane l ^ 32), P to LDS
//               O-wave  O^T += V^T P^T one tile later (A = V^T by transposed LDS reads, B = P^T
//                       from LDS), the output at the end
//             blocks of late queries (the most keys) are dispatched first.
//
// MFMA operand layouts (gfx950): v_mfma_f32_32x32x16_bf16 lane l supplies A[l%32][8(l/32)+e]
// and B[8(l/32)+e][l%32], e = 0..7; result register r of lane l is D[8(r/4)+4(l/32)+r%4][l%32].
// ds_read_b64_tr_b16: in each group of 16 lanes, element e of lane j is element j%4 of the
// 8-byte word addressed by lane 4e + j/4.
#include "common.h"
#include "prefill_plan.h"

namespace mla {

typedef __bf16 pbf16x8 __attribute__((ext_vector_type(8)));
typedef float pf32x16 __attribute__((ext_vector_type(16)));
typedef short pv4s __attribute__((ext_vector_type(4)));
typedef short pv8s __attribute__((ext_vector_type(8)));

constexpr int PF_H = 64, PF_L = 512, PF_R = 64, PF_V = 256;

__device__ __forceinline__ pbf16x8 pf_bf16x8(uint4 v) { return __builtin_bit_cast(pbf16x8, v); }

__device__ __forceinline__ uint32_t pf_pack(float a, float b)
{
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    const bf2 v = {(__bf16)a, (__bf16)b};   // v_cvt_pk_bf16_f32, round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

// ------------------------------------------------------------------------------ kv_b GEMM
__device__ __forceinline__ uint32_t pf_lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// One 64-lane global_load_lds_dwordx4 (16 B per lane from g, lane i's to LDS byte lds + 16 i; lds
// wave-uniform), from inline assembly so that the compiler does not make every later LDS access
// wait for it; completion is awaited with an explicit s_waitcnt vmcnt.  M0 is restored.
__device__ __forceinline__ void pf_dma16(const void *g, uint32_t lds)
{
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(keep)
                 : "v"(g), "s"(lds)
                 : "memory");
}

constexpr int KG_BM = 256, KG_BN = 256, KG_BK = 64;   // rows of C^T (n), columns (tokens), K step
constexpr int KG_NS = 2;                               // K steps staged at a time
constexpr int KG_RB = KG_BK * 2;                       // bytes per staged row (one 128-byte line)
constexpr size_t KG_LDS = (size_t)KG_NS * (KG_BM + KG_BN) * KG_RB;   // 128 KB

// grid (ceil(N / 256), ceil(T / 256)), 256 threads; wave w: n rows 128 (w&1) .., tokens 128 (w>>1) ..
// A K step of a tile is 256 rows x 128 B in LDS, the eight 16-byte chunks of row r stored at
// positions c ^ ((r >> 1) & 7): sixteen consecutive rows read at one chunk hit distinct banks.
// Wave w copies rows 64 w .. 64 w + 63 of both tiles, 8 rows (1 KB, whole lines) per DMA: lane L
// moves chunk (L % 8) ^ ((r >> 1) & 7) of row r = 8 j + L / 8 into position L % 8.
__global__ __launch_bounds__(256) void pf_kvb(KvView kv, const bf16_t *__restrict__ kv_b, int64_t T, int N,
                                              bf16_t *__restrict__ C)
{
    extern __shared__ __attribute__((aligned(16))) char kg_smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * KG_BM;
    const int64_t t0 = (int64_t)blockIdx.y * KG_BN;
    const bf16_t *lc = reinterpret_cast<const bf16_t *>(kv.lc);
    const bf16_t *ga[8];
    const bf16_t *gb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = 64 * wave + 8 * j + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        const int n = n0 + r;
        ga[j] = kv_b + (int64_t)(n < N ? n : N - 1) * PF_L + 8 * c;
        const int64_t t = t0 + r;
        const int64_t row = kv_row(kv, 0, t < T ? t : T - 1);
        gb[j] = lc + (row >= 0 ? row : 0) * PF_L + 8 * c;
    }
    auto stage = [&](int ks) {   // K step ks into ring slot ks % KG_NS
        char *base = kg_smem + (ks % KG_NS) * (KG_BM + KG_BN) * KG_RB;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            pf_dma16(ga[j] + KG_BK * ks, pf_lds_addr(base + (64 * wave + 8 * j) * KG_RB));
            pf_dma16(gb[j] + KG_BK * ks, pf_lds_addr(base + KG_BM * KG_RB + (64 * wave + 8 * j) * KG_RB));
        }
    };
    pf32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    const int wm = 128 * (wave & 1), wn = 128 * (wave >> 1);
    const int l32 = lane & 31, hi = lane >> 5;
    constexpr int NK = PF_L / KG_BK;   // 8 K steps
    stage(0);
    for (int ks = 0; ks < NK; ++ks) {
        // step ks has landed everywhere, and every wave is done with step ks - 1, whose slot the
        // copies of step ks + 1 fill
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        if (ks + 1 < NK) stage(ks + 1);
        const char *base = kg_smem + (ks % KG_NS) * (KG_BM + KG_BN) * KG_RB;
#pragma unroll
        for (int kk = 0; kk < KG_BK / 16; ++kk) {
            uint4 a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ra = wm + 32 * i + l32, rb = wn + 32 * i + l32, c = 2 * kk + hi;
                a[i] = *reinterpret_cast<const uint4 *>(base + ra * KG_RB + 16 * (c ^ ((ra >> 1) & 7)));
                b[i] = *reinterpret_cast<const uint4 *>(base + KG_BM * KG_RB + rb * KG_RB + 16 * (c ^ ((rb >> 1) & 7)));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf_bf16x8(a[i]), pf_bf16x8(b[j]), acc[i][j],
                                                                        0, 0, 0);
        }
    }
    // Register r of tile (i, j): n = n0 + wm + 32 i + 8 (r/4) + 4 hi + r%4, token t0 + wn + 32 j + l32.
    // Per pair of register groups (g = 2 gp, 2 gp + 1), one v_permlane32_swap of the packed values
    // trades lane half hi = 1's group 2 gp for half 0's group 2 gp + 1: lane (l32, hi) then holds
    // n = 32 i + 16 gp + 8 hi .. + 7 and stores 16 bytes, 32 contiguous bytes per token and pair.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t t = t0 + wn + 32 * j + l32;
        bf16_t *crow = C + (t < T ? t : 0) * (int64_t)N;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int gp = 0; gp < 2; ++gp) {
                const pf32x16 &r = acc[i][j];
                const int q = 8 * gp;
                const auto x = __builtin_amdgcn_permlane32_swap(pf_pack(r[q], r[q + 1]), pf_pack(r[q + 4], r[q + 5]),
                                                                false, false);
                const auto y = __builtin_amdgcn_permlane32_swap(pf_pack(r[q + 2], r[q + 3]),
                                                                pf_pack(r[q + 6], r[q + 7]), false, false);
                const int n = n0 + wm + 32 * i + 16 * gp + 8 * hi;
                if (t < T && n < N) *reinterpret_cast<uint4 *>(crow + n) = make_uint4(x[0], y[0], x[1], y[1]);
            }
    }
}

// ------------------------------------------------------------------------------ attention
constexpr int PA_BQ = 128, PA_BK = 64;
// A staged tile holds the 64 K rows, then the 64 V rows, 512 B each and unpadded.  The 16-byte
// chunks of a row are placed through the copies' source addresses: chunk c of K row r sits at
// c ^ (r % 32), so the 16-byte score-operand reads of 16 consecutive rows hit distinct banks;
// chunk c of V row r at c ^ 4 (r % 4), so each transposed read (rows r .. r+3, 64 bytes of
// columns) covers all 64 banks once.
constexpr int PA_KROW = 256;                              // bf16 per staged K or V row
constexpr int PA_TILE = 2 * PA_BK * PA_KROW;              // bf16 per staged tile
constexpr size_t PA_LDS = (size_t)2 * PA_TILE * 2;        // two tiles
// With a key mask (a selection per query): per staged tile, the mask words of its two 32-key
// groups for the block's 128 queries ([group][query], 1 KB), double-buffered behind the rest.
constexpr size_t PA_MASK_LDS = 2 * 2 * PA_BQ * 4;
constexpr int PA_PF = 6;       // score operand reads in flight

// grid (ceil(S / 128) * H), 512 threads.  NOPE: qk_nope (128 or 192).  OUT: float or bf16_t.
// Workgroups go to the 8 XCDs round-robin (id % 8); XCD x runs heads x, x + 8, .. one after the
// other, each as all of its query blocks at once (late ones first), so the head's K and V (4 MB
// at 4096 tokens) are fetched into that XCD's L2 once and shared by its 32 CUs.
// MODE 0: Rc rows contiguous (row = position); 1: block table with block_size % 64 == 0 (a tile's
// keys in one block, looked up once per tile with a scalar load); 2: any block table (one lookup
// per key, a vector load whose wait also lands the copies in flight).
// MASK: keys are further restricted per query by a bitmap (bit t % 32 of word
// mask[(t / 32) * mask_stride + i] set = key t attended by query i); wave 0 copies a tile's words
// into LDS with its K rows, so the same waits cover them.
//
// The work of a tile is split between two waves per SIMD: wave w < 4 (an S-wave) and wave w + 4
// (its O-wave) share SIMD w and the queries 32 w .. 32 w + 31 of the block.  The S-wave forms
// S^T = K Q^T of a tile, masks it and runs the online softmax; it hands P (bf16, [query][key]) and
// the tile's rescale factor to its O-wave through LDS, and the O-wave forms O^T += V^T P^T one
// tile later, so that one wave's value products run while the other computes the next tile's
// scores.  Two barriers per iteration it = 0 .. ntile:
//   B_it   K(it), its mask words, and V(it - 1) have landed
//          S-wave: scores and softmax of tile it (P kept in registers)
//          O-wave: reads P(it - 1) and its factors, rescales, value products of tile it - 1
//   B'_it  every P(it - 1) read is done, K(it) and V(it - 1) are consumed
//          all waves: copies of K(it + 2) (into K(it)'s buffer) and V(it + 1) (into V(it - 1)'s)
//          S-wave: writes P(it) and its factors
// so a tile's copies have one and a half iterations to land.  Each wave copies keys 8 w .. 8 w + 7
// of a tile (K or V halves of two keys per copy, chunks placed as above).
constexpr int PW_PROW = 72;                                      // bf16 per P row (64 keys + pad)
constexpr size_t PW_P_LDS = (size_t)4 * 32 * PW_PROW * 2;         // P of the four wave pairs
constexpr size_t PW_LDS = PA_LDS + PW_P_LDS + 2 * PA_BQ * 4;      // + rescale factors and final sums
constexpr size_t PW_VALID = 16;                                   // + key validity words of the two tiles
constexpr int PW_PV = 8;   // value-operand reads in flight (4: +1%, none: +2% prefill time, same box)

template <int NOPE, typename OUT, int MODE, bool MASK>
__global__ __launch_bounds__(512) void pf_attn(const bf16_t *__restrict__ q, const bf16_t *__restrict__ C,
                                               KvView kv, int S, int pos_base, float scale_log2,
                                               OUT *__restrict__ out, const uint32_t *__restrict__ mask,
                                               int mask_stride)
{
    extern __shared__ __attribute__((aligned(16))) char pa_smem[];
    bf16_t *sT = reinterpret_cast<bf16_t *>(pa_smem);   // [2 buffers][K rows, V rows][64][PA_KROW]
    bf16_t *sP = reinterpret_cast<bf16_t *>(pa_smem + PA_LDS);           // [4 pairs][32 queries][PW_PROW]
    float *sAl = reinterpret_cast<float *>(pa_smem + PA_LDS + PW_P_LDS);   // [128] rescale factor of P
    float *sL = sAl + PA_BQ;                                               // [128] final sums
    uint8_t *sValid = reinterpret_cast<uint8_t *>(pa_smem + PW_LDS);     // [2 tiles][8 waves]: bit i of byte w =
                                                                           // key 8 w + i of the tile has a pool row
    char *sMask = pa_smem + PW_LDS + PW_VALID;                             // [2][2 groups][128 queries]
    constexpr int QD = NOPE + PF_R;
    constexpr int KS = QD / 16;
    constexpr int N = PF_H * (NOPE + PF_V);
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pw = wave & 3;                   // the wave pair (SIMD) and its 32 queries
    const int l32 = lane & 31, hi = lane >> 5;
    const int nqb = (S + PA_BQ - 1) / PA_BQ;
    const int xcd = (int)blockIdx.x & 7, idx = (int)blockIdx.x >> 3;
    const int h = xcd + 8 * (idx / nqb);
    const int qb = nqb - 1 - idx % nqb;        // late query blocks (most keys) first
    const int i0 = qb * PA_BQ;
    const int iq = i0 + 32 * pw + l32;         // this lane's query
    const bf16_t *rc = reinterpret_cast<const bf16_t *>(kv.rc);
    const int i_last = i0 + PA_BQ - 1 < S - 1 ? i0 + PA_BQ - 1 : S - 1;
    const int64_t kend = (int64_t)pos_base + i_last + 1;
    const int ntile = (int)((kend + PA_BK - 1) / PA_BK);
    const int pp = lane & 31, kh = lane >> 5;

    // Rc rows of the wave's 8 keys of tile kt: lane i < 8 resolves key 64 kt + 8 wave + i.  In a paged
    // view, whether each has a pool row (none: a block-table hole) goes into the wave's byte of the
    // tile's validity word, and a key without one scores -inf, as in the decode (a contiguous view
    // has a row for every key: the view's checks require (B - 1) seq_stride + max_seq_len <= rows).
    auto rows_of = [&](int kt) -> int64_t {
        const int64_t t0 = (int64_t)kt * PA_BK + 8 * wave + (lane & 7);
        const int64_t t = t0 < kend ? t0 : kend - 1;
        int64_t row;
        if (MODE == 0) {
            row = t < kv.rows ? t : -1;
        } else if (MODE == 1) {
            const int32_t *pb = kv.bt + (int)((int64_t)kt * PA_BK / kv.bs);
            int32_t blk;
            asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(blk) : "s"(pb) : "memory");
            row = blk < 0 ? -1 : (int64_t)blk * kv.bs + t % kv.bs;
            if (row >= kv.rows) row = -1;
        } else {
            row = kv_row(kv, 0, t);
        }
        if (MODE != 0) {
            const uint32_t vb = (uint32_t)__builtin_amdgcn_ballot_w64(row >= 0) & 0xffu;
            if (lane == 0) sValid[(kt & 1) * 8 + wave] = (uint8_t)vb;
        }
        return row >= 0 ? row : 0;
    };
    auto settle = [](int64_t x) { asm volatile("" ::"v"((uint32_t)x), "v"((uint32_t)(x >> 32))); };
    // K rows (k_nope from C, then Rc) of tile kt, and wave 0's copy of its mask words first
    auto stage_k = [&](int kt, int64_t rrow) {
        bf16_t *dst = sT + (kt & 1) * PA_TILE;
        if (MASK && wave == 0) {
            const uint32_t *src = mask + (int64_t)(2 * kt + (lane >> 5)) * mask_stride + i0 + 4 * (lane & 31);
            pf_dma16(src, pf_lds_addr(sMask + (kt & 1) * 1024));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r0 = 8 * wave + 2 * i, key = r0 + kh;
            const int64_t t0 = (int64_t)kt * PA_BK + key;
            const int64_t t = t0 < kend ? t0 : kend - 1;
            const int64_t ra = ((int64_t)__builtin_amdgcn_readlane((int)(rrow >> 32), 2 * i) << 32) |
                               (uint32_t)__builtin_amdgcn_readlane((int)rrow, 2 * i);
            const int64_t rb = ((int64_t)__builtin_amdgcn_readlane((int)(rrow >> 32), 2 * i + 1) << 32) |
                               (uint32_t)__builtin_amdgcn_readlane((int)rrow, 2 * i + 1);
            const int64_t rrc = kh ? rb : ra;
            const bf16_t *crow = C + t * (int64_t)N + h * (NOPE + PF_V);
            const int ck = pp ^ (key & 31);
            const bf16_t *sk = ck < NOPE / 8 ? crow + 8 * ck : (ck < QD / 8 ? rc + rrc * PF_R + 8 * ck - NOPE : crow);
            pf_dma16(sk, pf_lds_addr(dst + r0 * PA_KROW));
        }
    };
    // V rows of tile kt
    auto stage_v = [&](int kt) {
        bf16_t *dst = sT + (kt & 1) * PA_TILE;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r0 = 8 * wave + 2 * i, key = r0 + kh;
            const int64_t t0 = (int64_t)kt * PA_BK + key;
            const int64_t t = t0 < kend ? t0 : kend - 1;
            const bf16_t *crow = C + t * (int64_t)N + h * (NOPE + PF_V);
            const int cv = pp ^ (4 * (key & 3));
            pf_dma16(crow + NOPE + 8 * cv, pf_lds_addr(dst + (PA_BK + r0) * PA_KROW));
        }
    };
    // K(it + 2) and V(it + 1) after B'_it (it = -1: the prologue's second half)
    auto stage_point = [&](int it) {
        if (it + 2 < ntile) {
            const int64_t rr = rows_of(it + 2);
            settle(rr);
            stage_k(it + 2, rr);
        }
        if (it + 1 < ntile) stage_v(it + 1);
    };
    // B_it: K(it) (with its mask words) and V(it - 1) landed; younger than them are the copies of
    // stage point it - 1 (wave 0's mask copy among them only makes it wait longer)
    auto top_wait = [&](int it) {
        const int young = (it + 1 < ntile ? 4 : 0) + (it < ntile ? 4 : 0);
        if (young == 8) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
        else if (young == 4) asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    };

    if (wave < 4) {
        // ---------------------------------------------------------------- S-wave
        uint4 bq[KS];
        {
            const bf16_t *qr = q + ((int64_t)(iq < S ? iq : S - 1) * PF_H + h) * QD + 8 * hi;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) bq[ks] = *reinterpret_cast<const uint4 *>(qr + 16 * ks);
        }
        const int64_t qpos = (int64_t)pos_base + iq;
        float m_run = -INFINITY, l_run = 0.f;
        {
            const int64_t rr = rows_of(0);
            settle(rr);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(bq[ks].x), "v"(bq[ks].y), "v"(bq[ks].z), "v"(bq[ks].w));
            stage_k(0, rr);
            stage_point(-1);
        }
        bf16_t *prow = sP + (pw * 32 + l32) * PW_PROW;
        for (int it = 0; it <= ntile; ++it) {
            top_wait(it);
            uint2 pk[2][4];
            float alpha = 1.f;
            if (it < ntile) {
                const int64_t k0 = (int64_t)it * PA_BK;
                const bf16_t *tk = sT + (it & 1) * PA_TILE;
                pf32x16 s[2];
                {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) s[mt][r] = 0.f;
                    const bf16_t *ka = tk + l32 * PA_KROW;
                    auto a_op = [&](int i) {
                        return *reinterpret_cast<const uint4 *>(ka + (i & 1) * 32 * PA_KROW +
                                                                8 * ((2 * (i >> 1) + hi) ^ l32));
                    };
                    uint4 ring[PA_PF];
#pragma unroll
                    for (int i = 0; i < PA_PF; ++i) ring[i] = a_op(i);
#pragma unroll
                    for (int i = 0; i < 2 * KS; ++i) {
                        const uint4 a = ring[i % PA_PF];
                        if (i + PA_PF < 2 * KS) ring[i % PA_PF] = a_op(i + PA_PF);
                        s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf_bf16x8(a), pf_bf16x8(bq[i >> 1]), s[i & 1],
                                                                           0, 0, 0);
                    }
#pragma unroll
                    for (int i = 0; i < PA_PF; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
                    for (int i = 0; i < 2 * KS - PA_PF; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
#pragma unroll
                    for (int i = 0; i < PA_PF; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
                if (MASK) {
                    const uint32_t *mw = reinterpret_cast<const uint32_t *>(sMask + (it & 1) * 1024);
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        const uint32_t w = mw[PA_BQ * mt + 32 * pw + l32];
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            if (!((w >> (8 * (r >> 2) + 4 * hi + (r & 3))) & 1u)) s[mt][r] = -INFINITY;
                    }
                }
                if (MODE != 0) {   // keys without a pool row (the word is the same for the whole wave)
                    const uint64_t vw = *reinterpret_cast<const uint64_t *>(sValid + (it & 1) * 8);
                    if (__builtin_amdgcn_readfirstlane((uint32_t)vw) != 0xffffffffu ||
                        __builtin_amdgcn_readfirstlane((uint32_t)(vw >> 32)) != 0xffffffffu) {
#pragma unroll
                        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                            for (int r = 0; r < 16; ++r)
                                if (!((vw >> (32 * mt + 8 * (r >> 2) + 4 * hi + (r & 3))) & 1ull)) s[mt][r] = -INFINITY;
                    }
                }
                const int qpos32 = (int)qpos;
                if (k0 + PA_BK - 1 > (int64_t)pos_base + i0 + 32 * pw) {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int t = (int)k0 + 32 * mt + 8 * (r >> 2) + 4 * hi + (r & 3);
                            if (t > qpos32) s[mt][r] = -INFINITY;
                        }
                }
                float mx = -INFINITY;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
                {
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                    mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2;
                }
                // lazy reference: it moves only when the tile's maximum exceeds it by more than 8
                // (log2 units), so P = exp2(s - m_run) < 2^8 and the accumulators are rescaled only
                // on the tiles where it moves; a masked score (-inf) gives P = 0, and until the
                // query's first attended key (key 0 unless it is masked or has no row) the reference
                // stays -inf and its P are 0
                const bool move = mx > m_run + 8.f;
                const float m_new = move ? mx : m_run;
                alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
                const float m_sub = m_new == -INFINITY ? 0.f : m_new;
                float psum = 0.f;
                typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
                const bf2 one2 = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        float pv[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][4 * g + e], scale_log2, -m_sub));
                        pk[mt][g].x = pf_pack(pv[0], pv[1]);
                        pk[mt][g].y = pf_pack(pv[2], pv[3]);
                        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, pk[mt][g].x), one2, psum, false);
                        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, pk[mt][g].y), one2, psum, false);
                    }
                {
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(psum), __float_as_uint(psum), false, false);
                    psum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                }
                l_run = l_run * alpha + psum;
                m_run = m_new;
            }
            asm volatile("s_barrier" ::: "memory");   // B'_it: the O-waves hold P(it - 1)
            stage_point(it);
            if (it < ntile) {
                // P(it): lane (l32, hi) holds keys 32 mt + 8 g + 4 hi .. + 3 of query l32
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *reinterpret_cast<uint2 *>(prow + 32 * mt + 8 * g + 4 * hi) = pk[mt][g];
                if (hi == 0) sAl[32 * pw + l32] = alpha;
                if (it == ntile - 1 && hi == 0) sL[32 * pw + l32] = l_run;
            }
        }
    } else {
        // ---------------------------------------------------------------- O-wave
        pf32x16 o[PF_V / 32];
#pragma unroll
        for (int dt = 0; dt < PF_V / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
        {
            const int64_t rr = rows_of(0);
            settle(rr);
            stage_k(0, rr);
            stage_point(-1);
        }
        const int G = lane >> 4, j16 = lane & 15;
        const int r3 = j16 >> 2;
        const int tr_off = PA_BK * PA_KROW + (8 * (G >> 1) + r3) * PA_KROW + 8 * (2 * (G & 1) + ((j16 & 3) >> 1)) +
                           4 * (j16 & 1);
        const bf16_t *prow = sP + (pw * 32 + l32) * PW_PROW + 8 * hi;
        for (int it = 0; it <= ntile; ++it) {
            top_wait(it);
            if (it >= 1) {
                const int kt = it - 1;
                uint4 pb[PA_BK / 16];
#pragma unroll
                for (int kb = 0; kb < PA_BK / 16; ++kb) pb[kb] = *reinterpret_cast<const uint4 *>(prow + 16 * kb);
                const float alpha = sAl[32 * pw + l32];
                if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
                    for (int dt = 0; dt < PF_V / 32; ++dt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
                }
                const bf16_t *tk = sT + (kt & 1) * PA_TILE;
                // step i = 8 kb + dt: the two transposed V reads run PW_PV steps ahead of the product
                auto v_op = [&](int i) {
                    const bf16_t *vb = tk + 16 * (i >> 3) * PA_KROW + tr_off + 32 * ((i & 7) ^ r3);
                    const pv4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) pv4s *)vb);
                    const pv4s hi4 =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) pv4s *)(vb + 4 * PA_KROW));
                    return __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                };
                constexpr int NSTEP = (PA_BK / 16) * (PF_V / 32);
                pv8s vring[PW_PV];
#pragma unroll
                for (int i = 0; i < PW_PV; ++i) vring[i] = v_op(i);
#pragma unroll
                for (int i = 0; i < NSTEP; ++i) {
                    const pv8s vt = vring[i % PW_PV];
                    if (i + PW_PV < NSTEP) vring[i % PW_PV] = v_op(i + PW_PV);
                    o[i & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(pbf16x8, vt),
                                                                       pf_bf16x8(pb[i >> 3]), o[i & 7], 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 2 * PW_PV; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
                for (int i = 0; i < NSTEP - PW_PV; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
#pragma unroll
                for (int i = 0; i < PW_PV; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            asm volatile("s_barrier" ::: "memory");   // B'_it
            stage_point(it);
        }
        if (iq >= S) return;
        const float l = sL[32 * pw + l32];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        OUT *orow = out + ((int64_t)iq * PF_H + h) * PF_V;
#pragma unroll
        for (int dt = 0; dt < PF_V / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dim = 32 * dt + 8 * g + 4 * hi;
                const float a = o[dt][4 * g] * inv, b = o[dt][4 * g + 1] * inv, c = o[dt][4 * g + 2] * inv,
                            d = o[dt][4 * g + 3] * inv;
                if constexpr (sizeof(OUT) == 4) {
                    *reinterpret_cast<float4 *>(orow + dim) = make_float4(a, b, c, d);
                } else {
                    uint2 v;
                    v.x = pf_pack(a, b);
                    v.y = pf_pack(c, d);
                    *reinterpret_cast<uint2 *>(orow + dim) = v;
                }
            }
    }
}

// ------------------------------------------------------------------------------ host side
bool prefill_mfma_supported(const mla_dims &d, mla_dtype dt)
{
    return dt == MLA_BF16 && d.n_heads == PF_H && d.kv_lora == PF_L && d.qk_rope == PF_R && d.v_head == PF_V &&
           (d.qk_nope == 128 || d.qk_nope == 192);
}

size_t prefill_mfma_ws(const mla_dims &d, int64_t T)
{
    return 256 + (size_t)T * d.n_heads * (d.qk_nope + d.v_head) * 2;
}

template <int NOPE, typename OUT, int MODE, bool MASK>
static mla_status launch_attn_mode(const void *q, const bf16_t *C, const KvView &kv, int32_t S, int32_t pos_base,
                                   float scale_log2, void *out, const uint32_t *mask, int mask_stride, hipStream_t s)
{
    constexpr size_t lds = PW_LDS + PW_VALID + (MASK ? PA_MASK_LDS : 0);
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&pf_attn<NOPE, OUT, MODE, MASK>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
        attr = true;
    }
    const dim3 g((unsigned)((S + PA_BQ - 1) / PA_BQ * PF_H));
    hipLaunchKernelGGL((pf_attn<NOPE, OUT, MODE, MASK>), g, dim3(512), lds, s, (const bf16_t *)q, C, kv, S, pos_base,
                       scale_log2, (OUT *)out, mask, mask_stride);
    return check_launch("pf_attn");
}

template <int NOPE, typename OUT, bool MASK>
static mla_status launch_attn(const void *q, const bf16_t *C, const KvView &kv, int32_t S, int32_t pos_base,
                              float scale_log2, void *out, const uint32_t *mask, int mask_stride, hipStream_t s)
{
    if (!kv.bt)
        return launch_attn_mode<NOPE, OUT, 0, MASK>(q, C, kv, S, pos_base, scale_log2, out, mask, mask_stride, s);
    if (kv.bs % PA_BK == 0)
        return launch_attn_mode<NOPE, OUT, 1, MASK>(q, C, kv, S, pos_base, scale_log2, out, mask, mask_stride, s);
    return launch_attn_mode<NOPE, OUT, 2, MASK>(q, C, kv, S, pos_base, scale_log2, out, mask, mask_stride, s);
}

template <int NOPE, typename OUT>
static mla_status launch_attn_any(const void *q, const bf16_t *C, const KvView &kv, int32_t S, int32_t pos_base,
                                  float scale_log2, void *out, const uint32_t *mask, int mask_stride, hipStream_t s)
{
    if (mask) return launch_attn<NOPE, OUT, true>(q, C, kv, S, pos_base, scale_log2, out, mask, mask_stride, s);
    return launch_attn<NOPE, OUT, false>(q, C, kv, S, pos_base, scale_log2, out, nullptr, 0, s);
}

mla_status launch_prefill_mfma(const void *q, const void *kv_b, const mla_dims &d, const KvView &kv, int32_t S,
                               int32_t pos_base, float sm_scale, void *out, mla_dtype out_dt, void *ws, hipStream_t s,
                               const uint32_t *mask, int mask_stride)
{
    const int64_t T = (int64_t)pos_base + S;
    const int N = d.n_heads * (d.qk_nope + d.v_head);
    bf16_t *C = reinterpret_cast<bf16_t *>((reinterpret_cast<uintptr_t>(ws) + 255) & ~(uintptr_t)255);
    const int64_t gy = (T + KG_BN - 1) / KG_BN;
    if (gy > 65535) return fail(MLA_ERR_UNSUPPORTED, "prefill: too many tokens");
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&pf_kvb),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)KG_LDS);
        if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
        attr = true;
    }
    hipLaunchKernelGGL(pf_kvb, dim3((unsigned)((N + KG_BM - 1) / KG_BM), (unsigned)gy), dim3(256), KG_LDS, s, kv,
                       (const bf16_t *)kv_b, T, N, C);
    mla_status st = check_launch("pf_kvb");
    if (st) return st;
    const float sl2 = sm_scale * 1.4426950408889634f;
    if (d.qk_nope == 192)
        return out_dt == MLA_FP32 ? launch_attn_any<192, float>(q, C, kv, S, pos_base, sl2, out, mask, mask_stride, s)
                                  : launch_attn_any<192, bf16_t>(q, C, kv, S, pos_base, sl2, out, mask, mask_stride, s);
    return out_dt == MLA_FP32 ? launch_attn_any<128, float>(q, C, kv, S, pos_base, sl2, out, mask, mask_stride, s)
                              : launch_attn_any<128, bf16_t>(q, C, kv, S, pos_base, sl2, out, mask, mask_stride, s);
}

}  // namespace mla
