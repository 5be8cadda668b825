// decode_mfma.hip -- absorbed MLA decode on bf16 matrix cores for 64 heads, kv_lora 512,
// qk_rope 64 (the GLM-5.2 geometry).  colibri-analysis 06 "MLA attention and KV cache",
// sec. 2.3, absorbed path: fold W_UK into the query, score against Lc/Rc directly,
// accumulate the softmax-weighted latent, apply W_UV per head.
//
// Launches (all asynchronous on the caller's stream):
//   absorb_rows   q_abs[b][h][c] = sum_i q_nope[b][h][i] W_UK[h][i][c]    (fp32 FMA, bf16 out)
//   core_mfma     per (split, b): the 64 heads x 576 score contraction and the 64 x 512 latent
//                 accumulation on v_mfma_f32_32x32x16_bf16 with an online softmax; each
//                 32-key tile of Lc/Rc is read from HBM once and shared by all heads
//   combine       log-sum-exp merge of the split partials -> clat[b][h][:] (bf16)
//   unabsorb_mfma out[b][h][j] = W_UV[h][j] . clat[b][h]  on v_mfma_f32_16x16x32_bf16
//
// MFMA operand layouts used (gfx950, checked on the device):
//   32x32x16: lane l supplies A[l%32][8*(l/32)+e] and B[8*(l/32)+e][l%32], e = 0..7;
//             result register r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l%32].
//   16x16x32: lane l supplies A[l%16][8*(l/16)+e] and B[8*(l/16)+e][l%16];
//             result register r of lane l is D[4*(l/16) + r][l%16].
#include "common.h"
#include "decode_plan.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int DM_H = 64, DM_L = 512, DM_R = 64, DM_QK = DM_L + DM_R;
constexpr int DM_KT = 32;                 // keys per tile
constexpr int DM_KROW = DM_QK + 8;        // bf16 per row of the key tile / query block in LDS
constexpr int DM_VROW = DM_KT + 4;        // bf16 per row of the transposed latent tile (72 B)
constexpr size_t DM_SQ_BYTES = (size_t)DM_H * DM_KROW * 2;
constexpr size_t DM_SK_BYTES = (size_t)DM_KT * DM_KROW * 2;
constexpr size_t DM_SV_BYTES = (size_t)DM_L * DM_VROW * 2;
constexpr size_t DM_CORE_LDS = DM_SQ_BYTES + DM_SK_BYTES + DM_SV_BYTES + 64;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// ------------------------------------------------------------------------------ absorb
// grid (L/64, H), 256 threads: thread (rg = t/8, cg = t%8) owns columns cb*64 + 8cg .. +8 and
// rows rg, rg+32, ...; partial sums over row groups are reduced through LDS.  Queries are
// processed four at a time (W_UK rows are re-read from cache for later groups).
__global__ __launch_bounds__(256) void absorb_rows(const bf16_t *__restrict__ q_nope, const bf16_t *__restrict__ kv_b,
                                                  int B, int nope, int v, bf16_t *__restrict__ q_abs)
{
    extern __shared__ float sh_abs[];                 // q values [B][nope], then reduction [32][4][64]
    float *sq = sh_abs;
    float *red = sh_abs + B * nope;
    const int tid = threadIdx.x, cg = tid & 7, rg = tid >> 3;
    const int h = blockIdx.y, c0 = blockIdx.x * 64 + cg * 8;
    for (int i = tid; i < B * nope; i += 256) {
        const int b = i / nope, r = i - b * nope;
        sq[i] = bf2f(q_nope[((int64_t)b * DM_H + h) * nope + r]);
    }
    __syncthreads();
    const bf16_t *W = kv_b + (int64_t)h * (nope + v) * DM_L + c0;
    for (int b0 = 0; b0 < B; b0 += 4) {
        const int nb = B - b0 < 4 ? B - b0 : 4;
        float acc[4][8];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[q][e] = 0.f;
#pragma unroll 6
        for (int i = rg; i < nope; i += 32) {
            const uint4 wv = *reinterpret_cast<const uint4 *>(W + (int64_t)i * DM_L);
            float wf[8];
            wf[0] = __uint_as_float(wv.x << 16); wf[1] = __uint_as_float(wv.x & 0xffff0000u);
            wf[2] = __uint_as_float(wv.y << 16); wf[3] = __uint_as_float(wv.y & 0xffff0000u);
            wf[4] = __uint_as_float(wv.z << 16); wf[5] = __uint_as_float(wv.z & 0xffff0000u);
            wf[6] = __uint_as_float(wv.w << 16); wf[7] = __uint_as_float(wv.w & 0xffff0000u);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q < nb) {
                    const float qv = sq[(b0 + q) * nope + i];
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[q][e] = fmaf(qv, wf[e], acc[q][e]);
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[(rg * 4 + q) * 64 + cg * 8 + e] = acc[q][e];
        __syncthreads();
        {
            const int q = tid >> 6, c = tid & 63;
            if (q < nb) {
                float s = 0.f;
                for (int r = 0; r < 32; ++r) s += red[(r * 4 + q) * 64 + c];
                q_abs[((int64_t)(b0 + q) * DM_H + h) * DM_L + blockIdx.x * 64 + c] = f2bf(s);
            }
        }
    }
}

// ------------------------------------------------------------------------------ core
// grid (NS, B), 256 threads = 4 waves.  Wave w: head block hb = w&1 (heads 32hb..32hb+31) and
// latent half cq = w>>1 (columns 256cq..256cq+255).  Per 32-key tile:
//   S^T[key][head] = K Q^T  (36 MFMAs over the 576 dims; both waves of a head block compute
//                    it, which costs less than exchanging it)
//   online softmax per head (the head of lane l is 32hb + l%32 in every register)
//   O^T[c][head] += Vt P^T  (16 MFMAs: 8 column blocks x 2 key steps), where the P^T operand
//                    comes straight from the S^T registers: for key step ks the lanes of half
//                    g hold keys 16ks + {4g..4g+3, 8+4g..8+4g+3}, and the transposed latent
//                    tile is read in that same key order.
__global__ __launch_bounds__(256) void core_mfma(const bf16_t *__restrict__ q_abs, const bf16_t *__restrict__ q_rope,
                                                KvView kv, const int32_t *__restrict__ sel,
                                                const int32_t *__restrict__ nsel, int sel_stride, float scale_log2,
                                                int NS, float *__restrict__ part_ml, float *__restrict__ part_o)
{
    extern __shared__ __attribute__((aligned(16))) char smem[];
    bf16_t *sQ = reinterpret_cast<bf16_t *>(smem);
    bf16_t *sK = reinterpret_cast<bf16_t *>(smem + DM_SQ_BYTES);
    bf16_t *sV = reinterpret_cast<bf16_t *>(smem + DM_SQ_BYTES + DM_SK_BYTES);
    uint8_t *sValid = reinterpret_cast<uint8_t *>(smem + DM_SQ_BYTES + DM_SK_BYTES + DM_SV_BYTES);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hb = wave & 1, cq = wave >> 1, g = lane >> 5, l32 = lane & 31;
    const int split = blockIdx.x, b = blockIdx.y;
    const bf16_t *lc = reinterpret_cast<const bf16_t *>(kv.lc);
    const bf16_t *rc = reinterpret_cast<const bf16_t *>(kv.rc);

    const int64_t sl = seq_len_of(kv, b);
    int64_t nk = sl;
    if (sel) {
        nk = nsel[b];
        if (nk < 0) nk = 0;
        if (nk > sel_stride) nk = sel_stride;
    }
    int64_t kps = (nk + NS - 1) / NS;
    kps = (kps + DM_KT - 1) / DM_KT * DM_KT;
    const int64_t j0 = (int64_t)split * kps;
    const int64_t j1 = j0 + kps < nk ? j0 + kps : nk;

    // query block -> LDS: sQ[h][0..512) = q_abs, sQ[h][512..576) = q_rope
#pragma unroll 6
    for (int i = tid; i < DM_H * (DM_QK / 8); i += 256) {
        const int h = i / (DM_QK / 8), ch = i - h * (DM_QK / 8);
        const bf16_t *src = ch < DM_L / 8 ? q_abs + ((int64_t)b * DM_H + h) * DM_L + ch * 8
                                          : q_rope + ((int64_t)b * DM_H + h) * DM_R + (ch - DM_L / 8) * 8;
        *reinterpret_cast<uint4 *>(sQ + h * DM_KROW + ch * 8) = *reinterpret_cast<const uint4 *>(src);
    }

    // loader roles: latent quad kq = tid&7 (keys 4kq..4kq+3) x column group cg = tid>>3 (16 cols);
    // rope-key row kr = tid>>3, part pr = tid&7 (8 cols)
    const int kq = tid & 7, cg = tid >> 3;
    const int kr = tid >> 3, pr = tid & 7;
    auto key_row = [&](int64_t j) -> int64_t {
        if (j >= j1) return -1;
        const int64_t t = sel ? (int64_t)sel[(int64_t)b * sel_stride + j] : j;
        if (t < 0 || t >= sl) return -1;
        return kv_row(kv, b, t);
    };
    uint4 ldL[8];   // 4 keys x 2 x 16 B of latent
    uint4 ldR;      // 16 B of rope key
    bool vR = false;
    auto load_tile = [&](int64_t jt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = key_row(jt + 4 * kq + r);
            if (row >= 0) {
                const uint4 *p = reinterpret_cast<const uint4 *>(lc + row * DM_L + cg * 16);
                ldL[2 * r] = p[0];
                ldL[2 * r + 1] = p[1];
            } else {
                ldL[2 * r] = make_uint4(0u, 0u, 0u, 0u);
                ldL[2 * r + 1] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
        const int64_t row = key_row(jt + kr);
        vR = row >= 0;
        ldR = vR ? *reinterpret_cast<const uint4 *>(rc + row * DM_R + pr * 8) : make_uint4(0u, 0u, 0u, 0u);
    };

    f32x16 acc[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
    float m = -INFINITY, lsum = 0.f;

    if (j0 < j1) load_tile(j0);
    for (int64_t jt = j0; jt < j1; jt += DM_KT) {
        __syncthreads();   // previous tile fully consumed (and, first time, sQ written)
        // key tile, row-major (latent | rope key)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uint4 *dst = reinterpret_cast<uint4 *>(sK + (4 * kq + r) * DM_KROW + cg * 16);
            dst[0] = ldL[2 * r];
            dst[1] = ldL[2 * r + 1];
        }
        *reinterpret_cast<uint4 *>(sK + kr * DM_KROW + DM_L + pr * 8) = ldR;
        if (pr == 0) sValid[kr] = vR ? 1 : 0;
        // latent tile transposed: sV[c][key], written one key quad (8 B) per column
        {
            const uint32_t *w0 = reinterpret_cast<const uint32_t *>(&ldL[0]);
            const uint32_t *w1 = reinterpret_cast<const uint32_t *>(&ldL[2]);
            const uint32_t *w2 = reinterpret_cast<const uint32_t *>(&ldL[4]);
            const uint32_t *w3 = reinterpret_cast<const uint32_t *>(&ldL[6]);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int wi = j >> 1;
                uint32_t a0 = w0[wi], a1 = w1[wi], a2 = w2[wi], a3 = w3[wi];
                uint2 pk;
                if (j & 1) {
                    pk.x = (a0 >> 16) | (a1 & 0xffff0000u);
                    pk.y = (a2 >> 16) | (a3 & 0xffff0000u);
                } else {
                    pk.x = (a0 & 0xffffu) | (a1 << 16);
                    pk.y = (a2 & 0xffffu) | (a3 << 16);
                }
                *reinterpret_cast<uint2 *>(sV + (cg * 16 + j) * DM_VROW + 4 * kq) = pk;
            }
        }
        __syncthreads();
        if (jt + DM_KT < j1) load_tile(jt + DM_KT);   // prefetch the next tile

        // S^T = K Q^T for this wave's head block
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
        const bf16_t *ka = sK + l32 * DM_KROW + 8 * g;
        const bf16_t *qb = sQ + (32 * hb + l32) * DM_KROW + 8 * g;
#pragma unroll 12
        for (int ks = 0; ks < DM_QK / 16; ++ks) {
            const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4 *>(ka + 16 * ks));
            const bf16x8 bq = as_bf16x8(*reinterpret_cast<const uint4 *>(qb + 16 * ks));
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq, s, 0, 0, 0);
        }
        // online softmax (log2 domain); key of register r is 8*(r/4) + 4g + r%4
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = 8 * (r >> 2) + 4 * g + (r & 3);
            s[r] = sValid[key] ? s[r] * scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, s[r]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float mn = fmaxf(m, tmax);
        if (mn == -INFINITY) continue;   // no valid key yet (same for every lane)
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        uint32_t pw[8];
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const bf16_t p0 = f2bf(__builtin_amdgcn_exp2f(s[r] - mn));
            const bf16_t p1 = f2bf(__builtin_amdgcn_exp2f(s[r + 1] - mn));
            psum += bf2f(p0) + bf2f(p1);
            pw[r >> 1] = (uint32_t)p0 | ((uint32_t)p1 << 16);
        }
        psum += __shfl_xor(psum, 32, 64);
        lsum = lsum * alpha + psum;
        m = mn;
        if (alpha != 1.0f) {
#pragma unroll
            for (int cb = 0; cb < 8; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
        }
        const bf16x8 p0 = as_bf16x8(make_uint4(pw[0], pw[1], pw[2], pw[3]));   // keys 0..15
        const bf16x8 p1 = as_bf16x8(make_uint4(pw[4], pw[5], pw[6], pw[7]));   // keys 16..31
        // O^T += Vt P^T
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
            const bf16_t *vrow = sV + (256 * cq + 32 * cb + l32) * DM_VROW + 4 * g;
            const uint2 a00 = *reinterpret_cast<const uint2 *>(vrow);
            const uint2 a01 = *reinterpret_cast<const uint2 *>(vrow + 8);
            const uint2 a10 = *reinterpret_cast<const uint2 *>(vrow + 16);
            const uint2 a11 = *reinterpret_cast<const uint2 *>(vrow + 24);
            acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(make_uint4(a00.x, a00.y, a01.x, a01.y)), p0,
                                                              acc[cb], 0, 0, 0);
            acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(make_uint4(a10.x, a10.y, a11.x, a11.y)), p1,
                                                              acc[cb], 0, 0, 0);
        }
    }
    // partials: m (log2 domain), l, unnormalised O for this split
    const int h = 32 * hb + l32;
    const int64_t slot = ((int64_t)b * NS + split) * DM_H + h;
    if (cq == 0 && g == 0) {
        part_ml[2 * slot] = m;
        part_ml[2 * slot + 1] = lsum;
    }
    float *po = part_o + slot * DM_L;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = 256 * cq + 32 * cb + 8 * q + 4 * g;
            *reinterpret_cast<float4 *>(po + c) =
                make_float4(acc[cb][4 * q], acc[cb][4 * q + 1], acc[cb][4 * q + 2], acc[cb][4 * q + 3]);
        }
}

// ------------------------------------------------------------------------------ combine
// grid (4, H, B), one wave per (b, h, column quarter); NS <= 64 so lane s holds the statistics
// of split s; the lane then owns two latent columns of the quarter.
__global__ __launch_bounds__(64) void combine_splits(const float *__restrict__ part_ml, const float *__restrict__ part_o,
                                                    int NS, bf16_t *__restrict__ clat)
{
    const int lane = threadIdx.x, quarter = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    float ms = -INFINITY, ls = 0.f;
    if (lane < NS) {
        const int64_t slot = ((int64_t)b * NS + lane) * DM_H + h;
        ms = part_ml[2 * slot];
        ls = part_ml[2 * slot + 1];
    }
    const float M = wave_max(ms);
    const float wgt = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    const float den = wave_sum(wgt * ls);
    const int c = quarter * 128 + 2 * lane;
    const float *po = part_o + ((int64_t)b * NS * DM_H + h) * DM_L + c;
    float o0 = 0.f, o1 = 0.f;
    for (int s0 = 0; s0 < NS; s0 += 8) {
        float2 x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            x[u] = s0 + u < NS ? *reinterpret_cast<const float2 *>(po + (int64_t)(s0 + u) * DM_H * DM_L)
                               : make_float2(0.f, 0.f);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float w_s = __shfl(wgt, (s0 + u) & 63, 64);
            o0 = fmaf(w_s, x[u].x, o0);
            o1 = fmaf(w_s, x[u].y, o1);
        }
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    *reinterpret_cast<uint32_t *>(clat + ((int64_t)b * DM_H + h) * DM_L + c) =
        (uint32_t)f2bf(o0 * inv) | ((uint32_t)f2bf(o1 * inv) << 16);
}

// ------------------------------------------------------------------------------ unabsorb
// grid (v/32, H), 128 threads: wave w computes output columns j0 + 16w .. +16 of head h for
// every query, 16 queries per MFMA row block, contracting the 512 latent columns in 16 steps.
__global__ __launch_bounds__(128) void unabsorb_mfma(const bf16_t *__restrict__ clat, const bf16_t *__restrict__ kv_b,
                                                    int B, int nope, int v, float *__restrict__ out)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.y, j0 = blockIdx.x * 32 + wave * 16;
    const int r16 = lane & 15, q4 = lane >> 4;
    const bf16_t *wrow = kv_b + ((int64_t)h * (nope + v) + nope + j0 + r16) * DM_L + 8 * q4;
    for (int b0 = 0; b0 < B; b0 += 16) {
        const int bq = b0 + r16;
        const bf16_t *arow = clat + ((int64_t)bq * DM_H + h) * DM_L + 8 * q4;
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DM_L / 32; ++ks) {
            const uint4 av = bq < B ? *reinterpret_cast<const uint4 *>(arow + 32 * ks) : make_uint4(0u, 0u, 0u, 0u);
            const uint4 wv = *reinterpret_cast<const uint4 *>(wrow + 32 * ks);
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(wv), d, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int bb = b0 + 4 * q4 + r;
            if (bb < B) out[((int64_t)bb * DM_H + h) * v + j0 + r16] = d[r];
        }
    }
}

// ------------------------------------------------------------------------------ host side
bool decode_mfma_supported(const mla_dims &d, mla_dtype dt)
{
    return dt == MLA_BF16 && d.n_heads == DM_H && d.kv_lora == DM_L && d.qk_rope == DM_R && d.qk_nope % 32 == 0 &&
           d.v_head % 32 == 0;
}

int mfma_splits(int32_t B, int64_t max_keys)
{
    // at least two 32-key tiles per split (a split's partials are as large as ~110 keys of
    // cache), and about one (split, b) block per CU
    int64_t by_keys = (max_keys + 63) / 64;
    int64_t by_cus = (256 + B - 1) / B;
    int64_t ns = by_keys < by_cus ? by_keys : by_cus;
    if (ns < 1) ns = 1;
    if (ns > 64) ns = 64;
    return (int)ns;
}

size_t decode_mfma_ws(const mla_dims &d, int32_t B, int64_t max_keys)
{
    const int NS = mfma_splits(B, max_keys);
    size_t bytes = 0;
    bytes += (size_t)B * DM_H * DM_L * 2;             // q_abs
    bytes += (size_t)B * DM_H * DM_L * 2;             // clat
    bytes += (size_t)B * NS * DM_H * 2 * 4;           // m, l
    bytes += (size_t)B * NS * DM_H * DM_L * 4;        // partial O
    (void)d;
    return bytes + 1024;
}

static mla_status enable_big_lds()
{
    static bool done = false;
    if (!done) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&core_mfma),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)DM_CORE_LDS);
        if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
        done = true;
    }
    return MLA_OK;
}

mla_status launch_decode_mfma(const void *q_nope, const void *q_rope, const void *kv_b, const mla_dims &d, int32_t B,
                              const KvView &kv, const int32_t *sel, const int32_t *nsel, int32_t sel_stride,
                              int64_t max_keys, float sm_scale, float *out, void *ws, hipStream_t s)
{
    const int NS = mfma_splits(B, max_keys);
    if (B > 65535) return fail(MLA_ERR_UNSUPPORTED, "decode: B > 65535");
    char *p = reinterpret_cast<char *>(ws);
    p = reinterpret_cast<char *>((reinterpret_cast<uintptr_t>(p) + 255) & ~(uintptr_t)255);
    bf16_t *q_abs = reinterpret_cast<bf16_t *>(p);
    p += (size_t)B * DM_H * DM_L * 2;
    bf16_t *clat = reinterpret_cast<bf16_t *>(p);
    p += (size_t)B * DM_H * DM_L * 2;
    float *part_ml = reinterpret_cast<float *>(p);
    p += (size_t)B * NS * DM_H * 2 * 4;
    float *part_o = reinterpret_cast<float *>(p);

    mla_status st = enable_big_lds();
    if (st) return st;
    // absorb: queries staged in LDS (at most 32 KB of them per launch)
    int per = (int)((32 * 1024) / ((size_t)d.qk_nope * 4));
    if (per > 32) per = 32;
    if (per < 1) return fail(MLA_ERR_UNSUPPORTED, "decode: qk_nope too large for the matrix-core path");
    for (int b0 = 0; b0 < B; b0 += per) {
        const int nb = B - b0 < per ? B - b0 : per;
        const size_t shm = (size_t)nb * d.qk_nope * 4 + 32 * 4 * 64 * 4;
        hipLaunchKernelGGL(absorb_rows, dim3(DM_L / 64, DM_H), dim3(256), shm, s,
                           (const bf16_t *)q_nope + (int64_t)b0 * DM_H * d.qk_nope, (const bf16_t *)kv_b, nb,
                           d.qk_nope, d.v_head, q_abs + (int64_t)b0 * DM_H * DM_L);
        st = check_launch("absorb_rows");
        if (st) return st;
    }
    const float scale_log2 = sm_scale * 1.4426950408889634f;
    hipLaunchKernelGGL(core_mfma, dim3(NS, B), dim3(256), DM_CORE_LDS, s, q_abs, (const bf16_t *)q_rope, kv, sel, nsel,
                       sel_stride, scale_log2, NS, part_ml, part_o);
    st = check_launch("core_mfma");
    if (st) return st;
    hipLaunchKernelGGL(combine_splits, dim3(4, DM_H, B), dim3(64), 0, s, part_ml, part_o, NS, clat);
    st = check_launch("combine_splits");
    if (st) return st;
    hipLaunchKernelGGL(unabsorb_mfma, dim3(d.v_head / 32, DM_H), dim3(128), 0, s, clat, (const bf16_t *)kv_b, B,
                       d.qk_nope, d.v_head, out);
    return check_launch("unabsorb_mfma");
}

}  // namespace mla
