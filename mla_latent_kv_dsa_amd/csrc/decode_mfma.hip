// decode_mfma.hip -- absorbed MLA decode on bf16 matrix cores for 64 heads, kv_lora 512,
// qk_rope 64 (the GLM-5.2 geometry).  colibri-analysis 06 "MLA attention and KV cache",
// sec. 2.3, absorbed path: fold W_UK into the query, score against Lc/Rc directly, weight the
// latent rows by the softmax, apply W_UV per head.
//
// Four launches, asynchronous on the caller's stream, each spread over the whole chip even
// at batch 1:
//   absorb_q         q_abs[b][h][:] = W_UK[h]^T q_nope[b][h]       (fp32 FMA, bf16 out); also
//                    resets the per-head running maxima used below
//   dec_scores       S[b][h][j] = scale * log2(e) * (q_abs . Lc[t_j] + q_rope . Rc[t_j]) for
//                    16-key tiles x all 64 heads on v_mfma_f32_16x16x32_bf16; the per-head
//                    maximum over all keys is kept with an integer atomicMax on an
//                    order-preserving encoding (max is order independent, so the result is
//                    deterministic)
//   dec_pv           P = exp2(S - max) (bf16) and O_part[b][split][h][c] = sum_j P V[j][c] for
//                    (64-column chunk, key split) blocks on v_mfma_f32_32x32x16_bf16; V is
//                    staged row-major in LDS and read transposed with ds_read_b64_tr_b16;
//                    l_part = sum_j P
//   combine_unabsorb clat = sum_split O_part / sum_split l_part (bf16), then
//                    out[b][h][:] = W_UV[h] clat on v_mfma_f32_16x16x32_bf16
// The softmax needs no rescaling between splits because every split subtracts the same
// global maximum, so the split partials are plain sums.
//
// MFMA operand layouts used (gfx950, checked on the device):
//   32x32x16: lane l supplies A[l%32][8*(l/32)+e] and B[8*(l/32)+e][l%32], e = 0..7;
//             result register r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l%32].
//   16x16x32: lane l supplies A[l%16][8*(l/16)+e] and B[8*(l/16)+e][l%16];
//             result register r of lane l is D[4*(l/16) + r][l%16].
//   ds_read_b64_tr_b16: in each group of 16 lanes, element e of lane j is element j%4 of the
//             8-byte word addressed by lane 4e + j/4.
#include "common.h"
#include "decode_plan.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int DM_H = 64, DM_L = 512, DM_R = 64;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Integer encoding of a float whose signed-integer order is the float order (for atomicMax).
__device__ __forceinline__ int f2ord(float f)
{
    const int i = __float_as_int(f);
    return i >= 0 ? i : i ^ 0x7fffffff;
}
__device__ __forceinline__ float ord2f(int i) { return __int_as_float(i >= 0 ? i : i ^ 0x7fffffff); }

// Keys attended by sequence b: the selected ones, or every cached token.
__device__ __forceinline__ int64_t dec_nkeys(const KvView &kv, int b, const int32_t *sel, const int32_t *nsel,
                                             int sel_stride)
{
    int64_t nk = seq_len_of(kv, b);
    if (sel) {
        nk = nsel[b];
        if (nk < 0) nk = 0;
        if (nk > sel_stride) nk = sel_stride;
    }
    return nk;
}

// Cache row of the j-th attended key of sequence b, or -1 when it has none.
__device__ __forceinline__ int64_t dec_row(const KvView &kv, int b, int64_t j, int64_t sl, const int32_t *sel,
                                           int sel_stride)
{
    const int64_t t = sel ? (int64_t)sel[(int64_t)b * sel_stride + j] : j;
    if (t < 0 || t >= sl) return -1;
    return kv_row(kv, b, t);
}

// ------------------------------------------------------------------------------ absorb
// grid (DM_L / 128, H), 256 threads.  Thread t: row group rg = t/16 (rows rg, rg+16, ...) and
// column group cg = t%16 (8 of the block's 128 columns).  The W_UK rows go out first, then the
// queries of head h are staged in LDS, so both latencies overlap.  Queries are handled eight at
// a time; row-group partial sums are reduced with lane shuffles inside a wave, then across
// the four waves through LDS in a fixed order.
constexpr int AB_QB = 8;

template <int NR>   // qk_nope / 16
__global__ __launch_bounds__(256) void absorb_q(const bf16_t *__restrict__ q_nope, const bf16_t *__restrict__ kv_b,
                                                int B, int v, bf16_t *__restrict__ q_abs, int *__restrict__ m2)
{
    constexpr int nope = 16 * NR;
    extern __shared__ float sh_abs[];   // q [B][nope] fp32, then partials [4][AB_QB][128]
    const int tid = threadIdx.x, rg = tid >> 4, cg = tid & 15, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.y, cbase = blockIdx.x * 128;
    const bf16_t *W = kv_b + ((int64_t)h * (nope + v) + rg) * DM_L + cbase + cg * 8;
    uint4 w[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) w[k] = *reinterpret_cast<const uint4 *>(W + (int64_t)k * 16 * DM_L);
    if (blockIdx.x == 0)
        for (int b = tid; b < B; b += 256) m2[(int64_t)b * DM_H + h] = f2ord(-INFINITY);
    float *sq = sh_abs;
    float *red = sh_abs + B * nope;
    for (int i = tid; i < B * nope; i += 256) {
        const int b = i / nope, r = i - b * nope;
        sq[i] = bf2f(q_nope[((int64_t)b * DM_H + h) * nope + r]);
    }
    __syncthreads();
    for (int b0 = 0; b0 < B; b0 += AB_QB) {
        const int nb = B - b0 < AB_QB ? B - b0 : AB_QB;
        float acc[AB_QB][8];
#pragma unroll
        for (int q = 0; q < AB_QB; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[q][e] = 0.f;
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            float wf[8];
            wf[0] = __uint_as_float(w[k].x << 16); wf[1] = __uint_as_float(w[k].x & 0xffff0000u);
            wf[2] = __uint_as_float(w[k].y << 16); wf[3] = __uint_as_float(w[k].y & 0xffff0000u);
            wf[4] = __uint_as_float(w[k].z << 16); wf[5] = __uint_as_float(w[k].z & 0xffff0000u);
            wf[6] = __uint_as_float(w[k].w << 16); wf[7] = __uint_as_float(w[k].w & 0xffff0000u);
#pragma unroll
            for (int q = 0; q < AB_QB; ++q) {
                if (q < nb) {
                    const float qv = sq[(b0 + q) * nope + rg + 16 * k];
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[q][e] = fmaf(qv, wf[e], acc[q][e]);
                }
            }
        }
        // the four row groups of a wave sit 16 lanes apart
#pragma unroll
        for (int q = 0; q < AB_QB; ++q) {
            if (q < nb) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float x = acc[q][e];
                    x += __shfl_xor(x, 16, 64);
                    x += __shfl_xor(x, 32, 64);
                    acc[q][e] = x;
                }
            }
        }
        if (lane < 16) {
#pragma unroll
            for (int q = 0; q < AB_QB; ++q) {
                if (q < nb) {
                    float *dst = &red[(wave * AB_QB + q) * 128 + cg * 8];
                    *reinterpret_cast<float4 *>(dst) = make_float4(acc[q][0], acc[q][1], acc[q][2], acc[q][3]);
                    *reinterpret_cast<float4 *>(dst + 4) = make_float4(acc[q][4], acc[q][5], acc[q][6], acc[q][7]);
                }
            }
        }
        __syncthreads();
        for (int i = tid; i < nb * 128; i += 256) {
            const int q = i >> 7, c = i & 127;
            const float s = ((red[(0 * AB_QB + q) * 128 + c] + red[(1 * AB_QB + q) * 128 + c]) +
                             red[(2 * AB_QB + q) * 128 + c]) + red[(3 * AB_QB + q) * 128 + c];
            q_abs[((int64_t)(b0 + q) * DM_H + h) * DM_L + cbase + c] = f2bf(s);
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------ scores
// grid (ceil(max_keys / 16), B), 256 threads; wave w scores heads 16w..16w+15 against the
// block's 16 keys over the 576 dims (16 MFMA steps over Lc, 2 over Rc).  Operands come straight
// from memory: lane l reads 16 B of key l%16 and of head 16w + l%16 at dims 32ks + 8(l/16).
// Keys without a cache row read the query row instead and score -inf.
__global__ __launch_bounds__(256) void dec_scores(const bf16_t *__restrict__ q_abs, const bf16_t *__restrict__ q_rope,
                                                  KvView kv, const int32_t *__restrict__ sel,
                                                  const int32_t *__restrict__ nsel, int sel_stride, float scale_log2,
                                                  int nkp, float *__restrict__ S2, int *__restrict__ m2,
                                                  int64_t *__restrict__ rows)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.y, jj = lane & 15, quad = lane >> 4;
    const int64_t j0 = (int64_t)blockIdx.x * 16;
    const int h = 16 * wave + jj;
    const bf16_t *qa = q_abs + ((int64_t)b * DM_H + h) * DM_L + 8 * quad;
    const bf16_t *qr = q_rope + ((int64_t)b * DM_H + h) * DM_R + 8 * quad;
    // query operands first: they depend on nothing, so they are in flight during the key lookups
    uint4 A[18], Bq[18];
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) Bq[ks] = *reinterpret_cast<const uint4 *>(qa + 32 * ks);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) Bq[16 + ks] = *reinterpret_cast<const uint4 *>(qr + 32 * ks);
    // the selection entry is read before the key count is known (clamped into the row of sel)
    const int64_t jq = j0 + jj;
    int64_t t = jq;
    if (sel) t = sel[(int64_t)b * sel_stride + (jq < sel_stride ? jq : sel_stride - 1)];
    const int64_t sl = seq_len_of(kv, b);
    const int64_t nk = dec_nkeys(kv, b, sel, nsel, sel_stride);
    if (j0 >= nk) return;
    const int64_t row = (jq < nk && t >= 0 && t < sl) ? kv_row(kv, b, t) : -1;
    const bool valid = row >= 0;
    const uint64_t vmask = __ballot(valid);   // bit k (k < 16): key j0 + k has a row
    if (tid < 16) rows[(int64_t)b * nkp + j0 + jj] = row;   // for the P V step
    const bf16_t *ka = valid ? reinterpret_cast<const bf16_t *>(kv.lc) + row * DM_L + 8 * quad : qa;
    const bf16_t *kr = valid ? reinterpret_cast<const bf16_t *>(kv.rc) + row * DM_R + 8 * quad : qr;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) A[ks] = *reinterpret_cast<const uint4 *>(ka + 32 * ks);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) A[16 + ks] = *reinterpret_cast<const uint4 *>(kr + 32 * ks);
    __builtin_amdgcn_sched_barrier(0);   // every operand load in flight before the first MFMA
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(A[ks]), as_bf16x8(Bq[ks]), d, 0, 0, 0);
    // register r holds key 4*quad + r of head h
    float s[4], mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        s[r] = ((vmask >> (4 * quad + r)) & 1) ? d[r] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[r]);
    }
    *reinterpret_cast<float4 *>(S2 + ((int64_t)b * DM_H + h) * nkp + j0 + 4 * quad) = make_float4(s[0], s[1], s[2], s[3]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (quad == 0 && mx > -INFINITY) atomicMax(&m2[(int64_t)b * DM_H + h], f2ord(mx));
}

// ------------------------------------------------------------------------------ P V
// grid (DM_L / 64, NS, B), 256 threads; wave w: heads 32(w&1) .. +32, columns
// 64 bx + 32 (w>>1) .. +32.  Keys of split s: [s*kps, min((s+1)*kps, nk)), in chunks of four
// 32-key tiles.  The chunk's cache rows (resolved by dec_scores) and scores are requested
// before the key count is known (it only masks).  P = exp2(S - max) is computed once per
// block (thread t: head t/4, keys 8(t%4) .. +8 of each tile) and staged in LDS with the
// latent tile; then each wave runs
//   A = P[32 heads][16 keys] (one 16-byte LDS read per lane)
//   B = V[16 keys][32 columns] (two transposed LDS reads)
constexpr int PV_KT = 32, PV_CH = 4;
constexpr int PV_VROW = 80;   // bf16 per staged V row: 64 columns + pad (160 B: the 4 rows of a
                              // transposed read fall in distinct banks)
constexpr int PV_PROW = 40;   // bf16 per staged P row: 32 keys + pad (80 B: conflict-free reads)

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float a, float b, float &sum)
{
    const bf16x2 v = {(__bf16)a, (__bf16)b};   // v_cvt_pk_bf16_f32, round to nearest even
    sum += (float)v[0] + (float)v[1];
    return __builtin_bit_cast(uint32_t, v);
}

__global__ __launch_bounds__(256) void dec_pv(const float *__restrict__ S2, const int *__restrict__ m2, KvView kv,
                                              const int64_t *__restrict__ rows, const int32_t *__restrict__ sel,
                                              const int32_t *__restrict__ nsel, int sel_stride, int nkp, int kps,
                                              float *__restrict__ o_part, float *__restrict__ l_part)
{
    __shared__ __attribute__((aligned(16))) bf16_t sV[PV_CH][PV_KT * PV_VROW];
    __shared__ __attribute__((aligned(16))) bf16_t sP[PV_CH][DM_H * PV_PROW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hb = wave & 1, cb = wave >> 1;
    const int cc = blockIdx.x, s = blockIdx.y, b = blockIdx.z, NS = gridDim.y;
    const int64_t k0 = (int64_t)s * kps;
    // keys of the split as far as the buffers go; the true bound only masks
    const int64_t ks1 = k0 + kps < nkp ? k0 + kps : nkp;
    const int ph = tid >> 2, pk = tid & 3;     // P role
    const float *srow = S2 + ((int64_t)b * DM_H + ph) * nkp + 8 * pk;
    const int64_t *rrow = rows + (int64_t)b * nkp;
    const bf16_t *lc = reinterpret_cast<const bf16_t *>(kv.lc) + 64 * cc;
    const int lk = tid >> 3, lch = tid & 7;    // V loader role: key lk, 16-byte chunk lch
    const int G = lane >> 4, i16 = lane & 15;  // transposed-read address inside a 16-key step
    const int tr_off = (8 * (G >> 1) + (i16 >> 2)) * PV_VROW + 32 * cb + 16 * (G & 1) + 4 * (i16 & 3);
    const int pa_off = (32 * hb + (lane & 31)) * PV_PROW + 8 * (lane >> 5);

    int64_t rw[PV_CH];
    float4 sp[PV_CH][2];
    auto prefetch = [&](int64_t c0) {
#pragma unroll
        for (int m = 0; m < PV_CH; ++m) {
            const int64_t j = c0 + PV_KT * m + lk;
            rw[m] = j < ks1 ? rrow[j] : -1;
#pragma unroll
            for (int u = 0; u < 2; ++u)
                sp[m][u] = c0 + PV_KT * m < ks1 ? *reinterpret_cast<const float4 *>(srow + c0 + PV_KT * m + 4 * u)
                                                : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    if (k0 < ks1) prefetch(k0);
    const int64_t nk = dec_nkeys(kv, b, sel, nsel, sel_stride);
    const int64_t k1 = k0 + kps < nk ? k0 + kps : nk;
    const float mh = ord2f(m2[(int64_t)b * DM_H + ph]);
    const bool live = mh > -INFINITY;

    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    float psum = 0.f;
    for (int64_t c0 = k0; c0 < k1; c0 += PV_KT * PV_CH) {
        uint4 vv[PV_CH];
#pragma unroll
        for (int m = 0; m < PV_CH; ++m)
            vv[m] = (rw[m] >= 0 && c0 + PV_KT * m + lk < k1)
                        ? *reinterpret_cast<const uint4 *>(lc + rw[m] * DM_L + 8 * lch)
                        : make_uint4(0u, 0u, 0u, 0u);
        // P of this thread's 8 keys in each tile
        uint4 pv[PV_CH];
#pragma unroll
        for (int m = 0; m < PV_CH; ++m) {
            const int64_t kb = c0 + PV_KT * m + 8 * pk;
            const float sv[8] = {sp[m][0].x, sp[m][0].y, sp[m][0].z, sp[m][0].w,
                                 sp[m][1].x, sp[m][1].y, sp[m][1].z, sp[m][1].w};
            float p[8];
            if (live && kb + 8 <= k1) {
#pragma unroll
                for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(sv[e] - mh);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) p[e] = (live && kb + e < k1) ? __builtin_amdgcn_exp2f(sv[e] - mh) : 0.f;
            }
            pv[m].x = pack_bf16(p[0], p[1], psum);
            pv[m].y = pack_bf16(p[2], p[3], psum);
            pv[m].z = pack_bf16(p[4], p[5], psum);
            pv[m].w = pack_bf16(p[6], p[7], psum);
        }
        if (c0 + PV_KT * PV_CH < k1) prefetch(c0 + PV_KT * PV_CH);
        __syncthreads();   // the previous chunk's tiles are no longer read
#pragma unroll
        for (int m = 0; m < PV_CH; ++m) {
            *reinterpret_cast<uint4 *>(&sV[m][lk * PV_VROW + 8 * lch]) = vv[m];
            *reinterpret_cast<uint4 *>(&sP[m][ph * PV_PROW + 8 * pk]) = pv[m];
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < PV_CH; ++m) {
            if (c0 + PV_KT * m >= k1) break;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const uint4 pa = *reinterpret_cast<const uint4 *>(&sP[m][pa_off + 16 * kk]);
                const bf16_t *vb = &sV[m][16 * kk * PV_VROW + tr_off];
                const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)vb);
                const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4s *)(vb + 4 * PV_VROW));
                const v8s vt = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(pa), __builtin_bit_cast(bf16x8, vt), acc, 0,
                                                              0, 0);
            }
        }
    }
    // register r: head 32hb + 8(r/4) + 4(l/32) + r%4, column 64cc + 32cb + l%32
    float *po = o_part + ((int64_t)b * NS + s) * DM_H * DM_L + 64 * cc + 32 * cb + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int hr = 32 * hb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        po[(int64_t)hr * DM_L] = acc[r];
    }
    if (cc == 0) {
        psum += __shfl_xor(psum, 1, 64);
        psum += __shfl_xor(psum, 2, 64);
        if (pk == 0) l_part[((int64_t)b * NS + s) * DM_H + ph] = psum;
    }
}

// ------------------------------------------------------------------------------ combine + W_UV
// grid (v / 64, H, ceil(B / 16)), 256 threads.  Wave w owns rows 64 bx + 16 w .. +16 of W_UV[h].
// They are requested first, one whole 1 KB row per instruction straight into LDS
// (global_load_lds_dwordx4; rows padded to 1040 B so the later operand reads are
// conflict-free).  The softmax denominators of the block's queries and the first batch of
// split partials follow; the latent rows (sum of the partials over the splits, in split
// order, divided by the denominator) are staged in LDS as bf16, then the 512 latent columns
// are contracted in 16 MFMA steps.
constexpr int CU_ROW = DM_L + 8;
constexpr int CU_WROW = DM_L + 8;          // bf16 per staged W_UV row (1040 B)
constexpr int CU_QB = 4, CU_SB = 16;
constexpr size_t CU_LDS = (size_t)(64 * CU_WROW + 16 * CU_ROW) * 2 + 16 * 4;

__global__ __launch_bounds__(256) void combine_unabsorb(const float *__restrict__ o_part,
                                                        const float *__restrict__ l_part, int NS,
                                                        const bf16_t *__restrict__ kv_b, int B, int nope, int v,
                                                        float *__restrict__ out)
{
    extern __shared__ __attribute__((aligned(16))) char cu_smem[];
    bf16_t *sW = reinterpret_cast<bf16_t *>(cu_smem);
    bf16_t *sC = sW + 64 * CU_WROW;
    float *sInv = reinterpret_cast<float *>(sC + 16 * CU_ROW);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.y, j0 = 64 * blockIdx.x + 16 * wave, b0 = 16 * blockIdx.z;
    const int nb = B - b0 < 16 ? B - b0 : 16;
    const int r16 = lane & 15, q4 = lane >> 4;
    {
        const bf16_t *wsrc = kv_b + ((int64_t)h * (nope + v) + nope + j0) * DM_L + 8 * lane;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(wsrc + (int64_t)i * DM_L),
                                             (__attribute__((address_space(3))) void *)(sW + (16 * wave + i) * CU_WROW),
                                             16, 0, 0);
    }

    float2 x[CU_QB][CU_SB];
    // unconditional loads (query and split clamped into range), zeroed after: conditional loads
    // would each wait for the previous ones
    auto load_batch = [&](int q0, int s0) {
#pragma unroll
        for (int qq = 0; qq < CU_QB; ++qq)
#pragma unroll
            for (int u = 0; u < CU_SB; ++u) {
                const int qc = q0 + qq < nb ? q0 + qq : nb - 1;
                const int sc = s0 + u < NS ? s0 + u : NS - 1;
                const float2 v = *reinterpret_cast<const float2 *>(
                    o_part + (((int64_t)(b0 + qc) * NS + sc) * DM_H + h) * DM_L + 2 * tid);
                x[qq][u] = (q0 + qq < nb && s0 + u < NS) ? v : make_float2(0.f, 0.f);
            }
    };
    load_batch(0, 0);
    if (tid < nb) {
        float l = 0.f;
#pragma unroll
        for (int s = 0; s < 64; ++s)
            if (s < NS) l += l_part[((int64_t)(b0 + tid) * NS + s) * DM_H + h];
        sInv[tid] = l > 0.f ? 1.f / l : 0.f;
    }
    __syncthreads();
    for (int q0 = 0; q0 < nb; q0 += CU_QB) {
        float o[CU_QB][2];
#pragma unroll
        for (int qq = 0; qq < CU_QB; ++qq) o[qq][0] = o[qq][1] = 0.f;
        for (int s0 = 0; s0 < NS; s0 += CU_SB) {
            if (q0 + s0 > 0) load_batch(q0, s0);
#pragma unroll
            for (int qq = 0; qq < CU_QB; ++qq)
#pragma unroll
                for (int u = 0; u < CU_SB; ++u) {
                    o[qq][0] += x[qq][u].x;
                    o[qq][1] += x[qq][u].y;
                }
        }
#pragma unroll
        for (int qq = 0; qq < CU_QB; ++qq) {
            if (q0 + qq < nb) {
                const float inv = sInv[q0 + qq];
                const bf16x2 c = {(__bf16)(o[qq][0] * inv), (__bf16)(o[qq][1] * inv)};
                *reinterpret_cast<uint32_t *>(&sC[(q0 + qq) * CU_ROW + 2 * tid]) = __builtin_bit_cast(uint32_t, c);
            }
        }
    }
    __syncthreads();
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
    const bf16_t *wl = sW + (16 * wave + r16) * CU_WROW + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4 *>(&sC[r16 * CU_ROW + 32 * ks + 8 * q4]);
        const uint4 wq = *reinterpret_cast<const uint4 *>(wl + 32 * ks);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(wq), d, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int bq = 4 * q4 + r;
        if (bq < nb) out[((int64_t)(b0 + bq) * DM_H + h) * v + j0 + r16] = d[r];
    }
}

// ------------------------------------------------------------------------------ host side
bool decode_mfma_supported(const mla_dims &d, mla_dtype dt)
{
    return dt == MLA_BF16 && d.n_heads == DM_H && d.kv_lora == DM_L && d.qk_rope == DM_R &&
           (d.qk_nope == 128 || d.qk_nope == 192 || d.qk_nope == 256) && d.v_head % 64 == 0;
}

struct DecPlan {
    int ns;        // key splits of the P V step
    int64_t kps;   // keys per split (multiple of 32)
    int64_t nkp;   // row stride of the score buffer (multiple of 32)
};

static DecPlan dec_plan(int32_t B, int64_t max_keys)
{
    DecPlan p;
    const int64_t by_keys = (max_keys + 127) / 128;                 // >= 128 keys per split
    const int64_t by_fill = ((1024 / 8) + B - 1) / (int64_t)B;     // ~1024 (chunk, split, b) blocks
    int64_t ns = by_keys < by_fill ? by_keys : by_fill;
    if (ns > 64) ns = 64;
    if (ns < 1) ns = 1;
    p.ns = (int)ns;
    int64_t kps = (max_keys + ns - 1) / ns;
    p.kps = (kps + PV_KT - 1) / PV_KT * PV_KT;
    if (p.kps < PV_KT) p.kps = PV_KT;
    p.nkp = (max_keys + 31) / 32 * 32;
    if (p.nkp < 32) p.nkp = 32;
    return p;
}

// combine_unabsorb stages 64 rows of W_UV (65 KB) besides the latent rows
static mla_status enable_big_lds()
{
    static bool done = false;
    if (!done) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&combine_unabsorb),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)CU_LDS);
        if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
        done = true;
    }
    return MLA_OK;
}

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_mfma_ws(const mla_dims &d, int32_t B, int64_t max_keys)
{
    const DecPlan p = dec_plan(B, max_keys);
    size_t bytes = 256;
    bytes += al256((size_t)B * DM_H * DM_L * 2);                // q_abs
    bytes += al256((size_t)B * DM_H * 4);                       // running maxima
    bytes += al256((size_t)B * DM_H * p.nkp * 4);               // scores
    bytes += al256((size_t)B * p.nkp * 8);                      // cache rows of the attended keys
    bytes += al256((size_t)B * p.ns * DM_H * DM_L * 4);         // P V partials
    bytes += al256((size_t)B * p.ns * DM_H * 4);                // softmax denominators
    (void)d;
    return bytes;
}

// Workspace layout (the first two parts depend on B only, so the absorb step can run without
// knowing the key count): q_abs | running maxima | scores | key rows | P V partials | denominators
struct DecWs {
    bf16_t *q_abs;
    int *m2;
    float *S2;
    int64_t *rows;
    float *o_part;
    float *l_part;
};

static DecWs dec_ws(void *ws, int32_t B, const DecPlan &p)
{
    DecWs w;
    char *c = reinterpret_cast<char *>((reinterpret_cast<uintptr_t>(ws) + 255) & ~(uintptr_t)255);
    w.q_abs = reinterpret_cast<bf16_t *>(c);
    c += al256((size_t)B * DM_H * DM_L * 2);
    w.m2 = reinterpret_cast<int *>(c);
    c += al256((size_t)B * DM_H * 4);
    w.S2 = reinterpret_cast<float *>(c);
    c += al256((size_t)B * DM_H * p.nkp * 4);
    w.rows = reinterpret_cast<int64_t *>(c);
    c += al256((size_t)B * p.nkp * 8);
    w.o_part = reinterpret_cast<float *>(c);
    c += al256((size_t)B * p.ns * DM_H * DM_L * 4);
    w.l_part = reinterpret_cast<float *>(c);
    return w;
}

size_t decode_mfma_absorb_ws(int32_t B) { return 256 + al256((size_t)B * DM_H * DM_L * 2) + al256((size_t)B * DM_H * 4); }

mla_status launch_absorb_mfma(const void *q_nope, const void *kv_b, const mla_dims &d, int32_t B, void *ws,
                              hipStream_t s)
{
    if (B > 65535) return fail(MLA_ERR_UNSUPPORTED, "decode: B > 65535");
    const DecWs w = dec_ws(ws, B, dec_plan(B, 0));
    // at most 32 queries' worth of q staged in LDS per launch
    for (int b0 = 0; b0 < B; b0 += 32) {
        const int nb = B - b0 < 32 ? B - b0 : 32;
        const size_t shm = (size_t)nb * d.qk_nope * 4 + 4 * AB_QB * 128 * 4;
        const dim3 g(DM_L / 128, DM_H), blk(256);
        const bf16_t *qn = (const bf16_t *)q_nope + (int64_t)b0 * DM_H * d.qk_nope;
        bf16_t *qa = w.q_abs + (int64_t)b0 * DM_H * DM_L;
        int *mm = w.m2 + (int64_t)b0 * DM_H;
        if (d.qk_nope == 128)
            hipLaunchKernelGGL(absorb_q<8>, g, blk, shm, s, qn, (const bf16_t *)kv_b, nb, d.v_head, qa, mm);
        else if (d.qk_nope == 192)
            hipLaunchKernelGGL(absorb_q<12>, g, blk, shm, s, qn, (const bf16_t *)kv_b, nb, d.v_head, qa, mm);
        else
            hipLaunchKernelGGL(absorb_q<16>, g, blk, shm, s, qn, (const bf16_t *)kv_b, nb, d.v_head, qa, mm);
        mla_status st = check_launch("absorb_q");
        if (st) return st;
    }
    return MLA_OK;
}

mla_status launch_attend_mfma(const void *q_rope, const void *kv_b, const mla_dims &d, int32_t B, const KvView &kv,
                              const int32_t *sel, const int32_t *nsel, int32_t sel_stride, int64_t max_keys,
                              float sm_scale, float *out, void *ws, hipStream_t s)
{
    if (B > 65535) return fail(MLA_ERR_UNSUPPORTED, "decode: B > 65535");
    const DecPlan p = dec_plan(B, max_keys);
    if (p.nkp > 0x7fffffff) return fail(MLA_ERR_UNSUPPORTED, "decode: too many keys");
    const DecWs w = dec_ws(ws, B, p);
    const int64_t gk = (max_keys + 15) / 16;
    const float scale_log2 = sm_scale * 1.4426950408889634f;
    if (gk > 0) {
        hipLaunchKernelGGL(dec_scores, dim3((unsigned)gk, B), dim3(256), 0, s, w.q_abs, (const bf16_t *)q_rope, kv,
                           sel, nsel, sel_stride, scale_log2, (int)p.nkp, w.S2, w.m2, w.rows);
        mla_status st = check_launch("dec_scores");
        if (st) return st;
    }
    hipLaunchKernelGGL(dec_pv, dim3(DM_L / 64, p.ns, B), dim3(256), 0, s, w.S2, w.m2, kv, w.rows, sel, nsel,
                       sel_stride, (int)p.nkp, (int)p.kps, w.o_part, w.l_part);
    mla_status st = check_launch("dec_pv");
    if (st) return st;
    st = enable_big_lds();
    if (st) return st;
    hipLaunchKernelGGL(combine_unabsorb, dim3(d.v_head / 64, DM_H, (B + 15) / 16), dim3(256), CU_LDS, s, w.o_part,
                       w.l_part, p.ns, (const bf16_t *)kv_b, B, d.qk_nope, d.v_head, out);
    return check_launch("combine_unabsorb");
}

}  // namespace mla
