// decode_mfma.hip -- absorbed MLA decode on bf16 matrix cores for 64 heads, kv_lora 512,
// qk_rope 64 (the GLM-5.2 geometry).  colibri-analysis 06 "MLA attention and KV cache",
// sec. 2.3, absorbed path: fold W_UK into the query, score against Lc/Rc directly, weight the
// latent rows by the softmax, apply W_UV per head.
//
// Three launches, asynchronous on the caller's stream, each spread over the whole chip even
// at batch 1:
//   absorb_q         q_abs[b][h][:] = W_UK[h]^T q_nope[b][h]       (fp32 FMA, bf16 out)
//   dec_core         per (key split, group of 16 heads): scores S = q_abs . Lc + q_rope . Rc on
//                    v_mfma_f32_16x16x32_bf16, an online softmax over the split's keys in 64-key
//                    chunks, and O = sum_j P_j Lc[t_j] on the same instruction; the split's O,
//                    running maximum and sum are written as partials.  When the chip has CUs
//                    to spare, an extra slice of workgroups reads W_UV meanwhile (into an LDS
//                    sink), so that the next launch finds it in the Infinity Cache.
//   combine_unabsorb clat = sum_s f_s O_s / sum_s f_s l_s with f_s = exp2(m_s - max m), then
//                    out[b][h][:] = W_UV[h] clat on v_mfma_f32_16x16x32_bf16
// Each split keeps its own maximum, so the splits need no common pass before the values.

// MFMA operand layouts used (gfx950, checked on the device):
//   32x32x16: lane l supplies A[l%32][8*(l/32)+e] and B[8*(l/32)+e][l%32], e = 0..7;
//             result register r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l%32].
//   16x16x32: lane l supplies A[l%16][8*(l/16)+e] and B[8*(l/16)+e][l%16];
//             result register r of lane l is D[4*(l/16) + r][l%16].
//   ds_read_b64_tr_b16: in each group of 16 lanes, element e of lane j is element j%4 of the
//             8-byte word addressed by lane 4e + j/4.
#include "common.h"
#include "decode_plan.h"
#include "absorb_body.h"
#include "qformat.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int DM_H = 64, DM_L = 512, DM_R = 64;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

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
// grid (DM_L / 128, H): one absorb_block per workgroup (absorb_body.h).
template <int NR>   // qk_nope / 16
__global__ __launch_bounds__(256) void absorb_q(const bf16_t *__restrict__ q_nope, const bf16_t *__restrict__ kv_b,
                                                int B, int v, bf16_t *__restrict__ q_abs)
{
    extern __shared__ float sh_abs[];   // q [B][nope] fp32, then partials [4][AB_QB][128]
    absorb_block<NR>(q_nope, kv_b, nullptr, B, v, q_abs, blockIdx.x, blockIdx.y, sh_abs, threadIdx.x);
}

// grid (DM_L / 128, H): the matrix-core job for batches (absorb_block_mfma).
template <int NR>
__global__ __launch_bounds__(256) void absorb_q_mfma(const bf16_t *__restrict__ q_nope,
                                                     const bf16_t *__restrict__ kv_b, int B, int v,
                                                     bf16_t *__restrict__ q_abs)
{
    extern __shared__ __attribute__((aligned(16))) char sh_w[];   // W_UK block, nope rows of AB_WROWB bytes
    absorb_block_mfma<NR>(q_nope, kv_b, B, v, q_abs, blockIdx.x, blockIdx.y, sh_w, threadIdx.x);
}

// ------------------------------------------------------------------------------ attention core
// grid (NS, DM_H / 16, B), 256 threads: split s of sequence b (keys [s*kps, min((s+1)*kps, nk)))
// against heads 16g .. 16g+15.  Up to 128 keys at a time are staged in LDS: every wave copies
// the latent rows of 16 of them straight from memory (one 1 KB row per global_load_lds_dwordx4,
// rows padded to 1072 B so that both the row reads of the score product and the transposed
// reads of the value product fall in distinct banks); the query operands (B of the score
// product) and the rope rows (A, read straight into registers) are requested before that.
// Per 64-key chunk:
//   S[key][head] = q_abs . Lc + q_rope . Rc   wave w: keys 16w..16w+15, v_mfma_f32_16x16x32_bf16
//   chunk max per head across the waves (LDS); m_new = max(m_run, chunk max);
//   P = exp2(S * scale_log2 - m_new) rounded to bf16, staged in LDS as [head][key];
//   O = O * exp2(m_run - m_new) + P Lc        wave w: columns 128w .. 128w+127, transposed reads
// The split's O, running maximum m (log2 units) and sum l (of the rounded P) go to the partials;
// the combine step rescales the splits to their common maximum.
constexpr int DC_KC = 64;                        // keys per chunk (four waves x 16)
constexpr int DC_SUP = 2;                        // chunks staged at a time
constexpr int DC_ROWB = 1024;                    // bytes per staged latent row (unpadded, dc_swz)

// Position of chunk c of staged latent row r is c ^ dc_swz(r % 16): the score-operand reads (16
// consecutive rows, one chunk) and the transposed value reads (rows 0-3 with 8-11, or 4-7 with
// 12-15, two chunks, per pass of 32 lanes) then hit distinct banks.
__device__ __forceinline__ int dc_swz(int r) { return 2 * (r & 3) + ((r >> 2) & 1) + 8 * ((r >> 3) & 1); }
constexpr int DC_PROW = 72;                      // bf16 per P row (64 keys + pad: 144 B)
constexpr size_t DC_QOFF = (size_t)DC_SUP * DC_KC * DC_ROWB + 16 * DC_PROW * 2 + (64 + 64 + 16) * 4;
// + q_abs of the workgroup's 16 heads (16 rows of 1 KB, chunks placed by dc_swz like the latent rows)
constexpr size_t DC_LDS = DC_QOFF + 16 * DC_ROWB;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float a, float b, float &sum)
{
    const bf16x2 v = {(__bf16)a, (__bf16)b};   // v_cvt_pk_bf16_f32, round to nearest even
    sum += (float)v[0] + (float)v[1];
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// One 64-lane global_load_lds_dwordx4 (16 B per lane from g, lane i's to LDS byte lds + 16 i;
// lds must be wave-uniform), issued from inline assembly: the compiler's wait-count pass would
// otherwise treat every later LDS access as dependent on it and wait for all outstanding memory
// traffic.  Completion is awaited explicitly (s_waitcnt vmcnt) before the staged data is read.
// M0 (the LDS base of the copy) is saved and restored around it.
__device__ __forceinline__ void lds_dma16(const void *g, uint32_t lds)
{
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(keep)
                 : "v"(g), "s"(lds)
                 : "memory");
}

// grid (NS, 4, B + pf): slice z == B (present when pf = 1) only reads W_UV (wuv = row 0 of
// head 0's W_UV block, rph rows per head block, v W_UV rows per head): workgroup (x, y) takes
// rows 128 x .. 128 x + 127 of the 16 v rows of heads 16 y .. 16 y + 15.
// ONE: every split fits in one staged chunk (kps <= DC_SUP * DC_KC); the chunk's selection entries
// are then requested before the query operands, so resolving them into cache rows waits for
// nothing else (loads complete in issue order).
// PB16: the split outputs are stored as bf16 (for combine_one), else fp32.
template <bool ONE, bool PB16 = false>
__global__ __launch_bounds__(256) void dec_core(const bf16_t *__restrict__ q_abs, const bf16_t *__restrict__ q_rope,
                                                KvView kv, const int32_t *__restrict__ sel,
                                                const int32_t *__restrict__ nsel, int sel_stride, float scale_log2,
                                                int kps, float *__restrict__ o_part, float *__restrict__ m_part,
                                                float *__restrict__ l_part, int B, const bf16_t *__restrict__ wuv,
                                                int rph, int v)
{
    extern __shared__ __attribute__((aligned(16))) char dc_smem[];
    if ((int)blockIdx.z == B) {
        const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), ln = threadIdx.x & 63;
        const int rows = 16 * v, lr0 = 128 * (int)blockIdx.x + 32 * wv;
        if (lr0 < rows) {
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const int lr = lr0 + i < rows ? lr0 + i : rows - 1;
                const int hh = 16 * (int)blockIdx.y + lr / v;
                lds_dma16(wuv + ((int64_t)hh * rph + lr % v) * DM_L + 8 * ln, lds_addr(dc_smem + 1024 * wv));
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy may outlive the workgroup's LDS
        return;
    }
    char *sL = dc_smem;
    bf16_t *sP = reinterpret_cast<bf16_t *>(dc_smem + DC_SUP * DC_KC * DC_ROWB);
    float *sMx = reinterpret_cast<float *>(sP + 16 * DC_PROW);   // [wave][head] chunk maxima
    float *sSum = sMx + 64;                                      // [wave][head] sums of P
    float *sAl = sSum + 64;                                      // [head] rescale factor
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = blockIdx.x, NS = gridDim.x, h0 = 16 * blockIdx.y, b = blockIdx.z;
    const int jj = lane & 15, quad = lane >> 4;
    const int h = h0 + jj;
    const bf16_t *qr = q_rope + ((int64_t)b * DM_H + h) * DM_R + 8 * quad;
    const bf16_t *dummy = q_abs + ((int64_t)b * DM_H + h0) * DM_L + 8 * lane;   // any readable 1 KB
    const int64_t k0 = (int64_t)s * kps;
    int32_t t_first[DC_SUP];
    if (ONE) {
#pragma unroll
        for (int u = 0; u < DC_SUP; ++u) {
            const int64_t j = k0 + 64 * u + 16 * wave + jj;
            t_first[u] = sel ? sel[(int64_t)b * sel_stride + (j < sel_stride ? j : sel_stride - 1)] : (int32_t)j;
        }
    }
    // The score product's B operand: q_abs of the 16 heads is copied into LDS once per workgroup
    // (below, behind the first chunk's rows) and read from there; loaded by every wave into
    // registers it was 64 KB of requests per workgroup queued ahead of the rows.  The rope part
    // (2 KB per wave) is loaded straight into registers.
    char *sQ = dc_smem + DC_QOFF;
    uint4 Bq[18];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) Bq[16 + ks] = *reinterpret_cast<const uint4 *>(qr + 32 * ks);
    const int64_t sl = seq_len_of(kv, b);
    const int64_t nk = dec_nkeys(kv, b, sel, nsel, sel_stride);
    const int64_t k1 = k0 + kps < nk ? k0 + kps : nk;
    const bf16_t *lc = reinterpret_cast<const bf16_t *>(kv.lc);
    const bf16_t *rc = reinterpret_cast<const bf16_t *>(kv.rc);

    float m_run = -INFINITY, l_run = 0.f;   // head h (the same in every lane with this jj)
    f32x4 acc[8];                            // column tile ct: heads 4 quad + r, column 128 wave + 16 ct + jj
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t c0 = k0; c0 < k1; c0 += DC_SUP * DC_KC) {
        // cache rows: lane jj of wave w resolves key c0 + 64 u + 16 w + jj (the selection entry
        // is read unconditionally, clamped into its row)
        int64_t row[DC_SUP];
        uint4 Arc[DC_SUP][2];
#pragma unroll
        for (int u = 0; u < DC_SUP; ++u) {
            const int64_t j = c0 + 64 * u + 16 * wave + jj;
            int64_t t = j;
            if (ONE) t = t_first[u];
            else if (sel) t = sel[(int64_t)b * sel_stride + (j < sel_stride ? j : sel_stride - 1)];
            row[u] = (j < k1 && t >= 0 && t < sl) ? kv_row(kv, b, t) : -1;
            const bf16_t *kr = row[u] >= 0 ? rc + row[u] * DM_R + 8 * quad : qr;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) Arc[u][ks] = *reinterpret_cast<const uint4 *>(kr + 32 * ks);
        }
#pragma unroll
        for (int u = 0; u < DC_SUP; ++u) {
            if (c0 + 64 * u >= k1) break;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int64_t r = ((int64_t)__builtin_amdgcn_readlane((int)(row[u] >> 32), i) << 32) |
                                  (uint32_t)__builtin_amdgcn_readlane((int)row[u], i);
                const bf16_t *src = r >= 0 ? lc + r * DM_L + 8 * (lane ^ dc_swz(i)) : dummy;
                lds_dma16(src, lds_addr(sL + (64 * u + 16 * wave + i) * DC_ROWB));
            }
        }
        if (c0 == k0) {   // q_abs rows of heads h0 + 4 wave .. + 3
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int hr = 4 * wave + i;
                lds_dma16(q_abs + ((int64_t)b * DM_H + h0 + hr) * DM_L + 8 * (lane ^ dc_swz(hr)),
                          lds_addr(sQ + hr * DC_ROWB));
            }
        }
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        if (c0 == k0) {
            const int fq = dc_swz(jj);
#pragma unroll
            for (int ks = 0; ks < 16; ++ks)
                Bq[ks] = *reinterpret_cast<const uint4 *>(sQ + jj * DC_ROWB + 16 * ((4 * ks + quad) ^ fq));
        }
#pragma unroll
        for (int u = 0; u < DC_SUP; ++u) {
            if (c0 + 64 * u >= k1) break;
            // scores: register r is key 16 wave + 4 quad + r of the chunk, head h
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
            const char *ka = sL + (64 * u + 16 * wave + jj) * DC_ROWB;
            const int fj = dc_swz(jj);
#pragma unroll
            for (int ks = 0; ks < 16; ++ks)
                d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(*reinterpret_cast<const uint4 *>(ka + 16 * ((4 * ks + quad) ^ fj))), as_bf16x8(Bq[ks]), d, 0,
                    0, 0);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(Arc[u][ks]), as_bf16x8(Bq[16 + ks]), d, 0, 0, 0);
            const uint64_t vmask = __ballot(row[u] >= 0);   // bit k < 16: key 16 wave + k has a row
            float sv[4], mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sv[r] = ((vmask >> (4 * quad + r)) & 1) ? d[r] * scale_log2 : -INFINITY;
                mx = fmaxf(mx, sv[r]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            if (quad == 0) sMx[16 * wave + jj] = mx;
            __syncthreads();
            const float cm = fmaxf(fmaxf(sMx[jj], sMx[16 + jj]), fmaxf(sMx[32 + jj], sMx[48 + jj]));
            const float m_new = fmaxf(m_run, cm);
            const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
            float p[4], psum = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = sv[r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[r] - m_new);
            uint2 pw;
            pw.x = pack_bf16(p[0], p[1], psum);
            pw.y = pack_bf16(p[2], p[3], psum);
            *reinterpret_cast<uint2 *>(&sP[jj * DC_PROW + 16 * wave + 4 * quad]) = pw;
            psum += __shfl_xor(psum, 16, 64);
            psum += __shfl_xor(psum, 32, 64);
            if (quad == 0) sSum[16 * wave + jj] = psum;
            if (wave == 0 && quad == 0) sAl[jj] = alpha;
            __syncthreads();
            l_run = l_run * alpha + ((sSum[jj] + sSum[16 + jj]) + sSum[32 + jj]) + sSum[48 + jj];
            m_run = m_new;
            // values: rescale, then two 32-key steps over eight column tiles
            float al[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) al[r] = sAl[4 * quad + r];
#pragma unroll
            for (int ct = 0; ct < 8; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[ct][r] *= al[r];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const uint4 pa = *reinterpret_cast<const uint4 *>(&sP[jj * DC_PROW + 32 * kk + 8 * quad]);
                // rows 8 quad + jj/4 (and 4 on) of this 32-key step, columns 128 wave + 16 ct + 4 (jj % 4) ..:
                // chunk 16 wave + 2 ct + (jj % 4) / 2
                const int rl = (8 * quad + (jj >> 2)) & 15, flo = dc_swz(rl), fhi = dc_swz(rl + 4);
                const char *vb = sL + (64 * u + 32 * kk + 8 * quad + (jj >> 2)) * DC_ROWB + 8 * (jj & 1);
                const int c0 = 16 * wave + ((jj & 3) >> 1);
#pragma unroll
                for (int ct = 0; ct < 8; ++ct) {
                    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4s *)(vb + 16 * ((c0 + 2 * ct) ^ flo)));
                    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4s *)(vb + 4 * DC_ROWB + 16 * ((c0 + 2 * ct) ^ fhi)));
                    const v8s vt = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pa), __builtin_bit_cast(bf16x8, vt),
                                                                      acc[ct], 0, 0, 0);
                }
            }
        }
        __syncthreads();   // the staged rows are no longer read
        if (ONE) break;
    }
    const int64_t po0 = (((int64_t)b * NS + s) * DM_H + h0 + 4 * quad) * DM_L + 128 * wave + jj;
    if (PB16) {
        bf16_t *po = reinterpret_cast<bf16_t *>(o_part) + po0;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) po[(int64_t)r * DM_L + 16 * ct] = f2bf(acc[ct][r]);
    } else {
        float *po = o_part + po0;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) po[(int64_t)r * DM_L + 16 * ct] = acc[ct][r];
    }
    if (wave == 0 && quad == 0) {
        m_part[((int64_t)b * NS + s) * DM_H + h] = m_run;
        l_part[((int64_t)b * NS + s) * DM_H + h] = l_run;
    }
}

// ------------------------------------------------------------------------------ attention core, batches
// grid (NS, B), 256 threads: split s of sequence b against all 64 heads, wave w owning heads
// 16w .. 16w+15, so every key reaches the CU once for all heads (dec_core above brings it in once
// per group of 16 heads, which only pays when a single query leaves CUs idle).  The split's keys
// go in groups of 256: thread t resolves key g0 + t to its cache row (LDS), then 32-key chunks
// are staged through four LDS buffers, three chunks in flight while one is computed.  Wave w
// copies the latent rows of keys 8w .. 8w+7 of a chunk (one 1 KB row per DMA) and their rope
// rows (eight 128 B rows in one DMA; the 16-byte pieces of key t's row are stored in the order
// piece ^ (t % 8), which spreads the operand reads over the banks).  Per chunk, in every wave:
//   S[key][head] = q_abs . Lc + q_rope . Rc over two 16-key tiles, v_mfma_f32_16x16x32_bf16;
//   the online softmax of the chunk is wave-local (all keys of the chunk are in the wave), with
//   a lazy reference maximum: it moves only when a chunk exceeds it by more than 2^MH_LAZY, so
//   the O rows are rescaled rarely and P stays below 2^MH_LAZY (the partials carry that
//   reference, which is all the combine needs);
//   P stays in registers as the A operand of O += P Lc: the k slots of lane (j, q) are keys
//   4q .. 4q+3 of the two key tiles, and the transposed reads of Lc fetch the same keys for the
//   B operand, so P needs no pass through LDS.
// O (16 heads x 512 columns per wave), the reference maximum and the sum of the rounded P go to
// the same partials as dec_core's.
constexpr int MH_ROWB = 1024;   // bytes per staged latent row (unpadded; 16-byte chunks swizzled, mh_swz)
constexpr int MH_RCB = 128;     // bytes per staged rope row
constexpr int MH_KC = 32;       // keys per chunk
constexpr int MH_NBUF = 4;      // chunk buffers
constexpr int MH_DMA = MH_KC / 4 + 1;   // DMAs per wave and chunk
constexpr float MH_LAZY = 8.f;  // slack of the reference maximum (log2 units)
constexpr int MH_PF = 6;        // score operand reads in flight
constexpr int MH_PV = 4;        // value column tiles read ahead
constexpr size_t MH_LDS = (size_t)MH_NBUF * MH_KC * (MH_ROWB + MH_RCB) + 256 * sizeof(int64_t);

// Position of chunk c of staged latent row r is c ^ mh_swz(r): the score-operand reads (16
// consecutive rows, one chunk) and the transposed value reads (8 rows, two chunks per pass of 32
// lanes) then hit distinct banks.
__device__ __forceinline__ int mh_swz(int r) { return 2 * (r & 7) + ((r >> 3) & 1); }

__device__ __forceinline__ int64_t readlane64(int64_t x, int i)
{
    return ((int64_t)__builtin_amdgcn_readlane((int)(x >> 32), i) << 32) | (uint32_t)__builtin_amdgcn_readlane((int)x, i);
}

// Maximum and sum over the four 16-lane rows (lanes j, j+16, j+32, j+48), left in every lane:
// v_permlane32_swap and v_permlane16_swap on two copies exchange the halves and rows (no LDS).
__device__ __forceinline__ float mh_max4(float x)
{
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float mh_sum4(float x)
{
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// s_waitcnt vmcnt(n * MH_DMA) for a wave-uniform n in 0..MH_NBUF-1, then the block barrier
__device__ __forceinline__ void mh_wait_chunks(int n)
{
    static_assert(MH_NBUF == 4 && MH_DMA == 9, "wait counts below");
    if (n >= 3) asm volatile("s_waitcnt vmcnt(27)\n\ts_barrier" ::: "memory");
    else if (n == 2) asm volatile("s_waitcnt vmcnt(18)\n\ts_barrier" ::: "memory");
    else if (n == 1) asm volatile("s_waitcnt vmcnt(9)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

__global__ __launch_bounds__(256) void dec_core_mh(const bf16_t *__restrict__ q_abs, const bf16_t *__restrict__ q_rope,
                                                   KvView kv, const int32_t *__restrict__ sel,
                                                   const int32_t *__restrict__ nsel, int sel_stride, float scale_log2,
                                                   int kps, float *__restrict__ o_part, float *__restrict__ m_part,
                                                   float *__restrict__ l_part)
{
    extern __shared__ __attribute__((aligned(16))) char mh_smem[];
    char *sL = mh_smem;                                                          // [NBUF][KC][MH_ROWB]
    char *sR = mh_smem + MH_NBUF * MH_KC * MH_ROWB;                              // [NBUF][KC][MH_RCB]
    int64_t *sRow = reinterpret_cast<int64_t *>(sR + MH_NBUF * MH_KC * MH_RCB);  // [256]
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = blockIdx.x, NS = gridDim.x, b = blockIdx.y;
    const int jj = lane & 15, quad = lane >> 4;
    const int h = 16 * wave + jj;
    const bf16_t *qa = q_abs + ((int64_t)b * DM_H + h) * DM_L + 8 * quad;
    const bf16_t *qr = q_rope + ((int64_t)b * DM_H + h) * DM_R + 8 * quad;
    const bf16_t *dummy = q_abs + (int64_t)b * DM_H * DM_L + 8 * lane;   // any readable 1 KB
    uint4 Bq[18];
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) Bq[ks] = *reinterpret_cast<const uint4 *>(qa + 32 * ks);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) Bq[16 + ks] = *reinterpret_cast<const uint4 *>(qr + 32 * ks);
    const int64_t sl = seq_len_of(kv, b);
    const int64_t nk = dec_nkeys(kv, b, sel, nsel, sel_stride);
    const int64_t k0 = (int64_t)s * kps;
    const int64_t k1 = k0 + kps < nk ? k0 + kps : nk;
    const bf16_t *lc = reinterpret_cast<const bf16_t *>(kv.lc);
    const bf16_t *rc = reinterpret_cast<const bf16_t *>(kv.rc);

    float m_run = -INFINITY, l_run = 0.f;   // head h
    f32x4 acc[32];                           // column tile ct: heads 16 wave + 4 quad + r, column 16 ct + jj
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    // latent and rope rows of chunk c (keys MH_KC c .. of the group) into buffer buf
    auto issue = [&](int c, int buf) {
        const int64_t rw = sRow[MH_KC * c + 8 * wave + (lane & 7)];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t r = readlane64(rw, i);
            const bf16_t *src = r >= 0 ? lc + r * DM_L + 8 * (lane ^ mh_swz(8 * wave + i)) : dummy;
            lds_dma16(src, lds_addr(sL + (MH_KC * buf + 8 * wave + i) * MH_ROWB));
        }
        const int kc = 8 * wave + (lane >> 3);   // key of the chunk whose rope piece this lane copies
        const int64_t r = sRow[MH_KC * c + kc];
        const int pc = (lane & 7) ^ (kc & 7);
        const bf16_t *src = r >= 0 ? rc + r * DM_R + 8 * pc : dummy;
        lds_dma16(src, lds_addr(sR + (MH_KC * buf + 8 * wave) * MH_RCB));
    };

    for (int64_t g0 = k0; g0 < k1; g0 += 256) {
        const int64_t j = g0 + tid;
        sRow[tid] = j < k1 ? dec_row(kv, b, j, sl, sel, sel_stride) : -1;
        __syncthreads();
        const int nc = (int)(((k1 - g0 < 256 ? k1 - g0 : 256) + MH_KC - 1) / MH_KC);
        // the query operands are complete before the first DMA: the compiler's own wait for them
        // would otherwise count the DMAs (which it does not see) and wait for later chunks too
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) asm volatile("" ::"v"(Bq[ks].x), "v"(Bq[ks].y), "v"(Bq[ks].z), "v"(Bq[ks].w));
        for (int c = 0; c < MH_NBUF - 1 && c < nc; ++c) issue(c, c);
        for (int c = 0; c < nc; ++c) {
            const int buf = c % MH_NBUF;
            if (c + MH_NBUF - 1 < nc) issue(c + MH_NBUF - 1, (c + MH_NBUF - 1) % MH_NBUF);
            mh_wait_chunks(nc - 1 - c);   // the chunks issued after c may stay in flight
            const uint64_t vmask = __ballot(lane < MH_KC && sRow[MH_KC * c + (lane & (MH_KC - 1))] >= 0);
            const char *bL = sL + MH_KC * buf * MH_ROWB;
            const char *bR = sR + MH_KC * buf * MH_RCB;
            // scores: register r of tile kt is key 16 kt + 4 quad + r, head h.  Step i of 36 takes
            // tile i % 2, operand slice i / 2 (16 latent slices, then 2 rope slices); the LDS
            // reads run MH_PF steps ahead of their products.
            f32x4 d[2];
            {
                // four accumulator chains: tile i % 2, even or odd slice (i / 2) % 2
                f32x4 dd[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) dd[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                auto a_op = [&](int i) -> uint4 {
                    const int kt = i & 1, ks = i >> 1, key = 16 * kt + jj;
                    if (ks < 16)
                        return *reinterpret_cast<const uint4 *>(bL + key * MH_ROWB + 16 * ((4 * ks + quad) ^ mh_swz(key)));
                    return *reinterpret_cast<const uint4 *>(bR + key * MH_RCB + 16 * ((4 * (ks - 16) + quad) ^ (key & 7)));
                };
                uint4 ring[MH_PF];
#pragma unroll
                for (int i = 0; i < MH_PF; ++i) ring[i] = a_op(i);
#pragma unroll
                for (int i = 0; i < 36; ++i) {
                    const uint4 a = ring[i % MH_PF];
                    if (i + MH_PF < 36) ring[i % MH_PF] = a_op(i + MH_PF);
                    dd[i & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(Bq[i >> 1]), dd[i & 3], 0, 0, 0);
                }
                d[0] = dd[0] + dd[2];
                d[1] = dd[1] + dd[3];
#pragma unroll
                for (int i = 0; i < MH_PF; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS reads
#pragma unroll
                for (int i = 0; i < 36 - MH_PF; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
#pragma unroll
                for (int i = 0; i < MH_PF; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            float sv[2][4], mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sv[kt][r] = ((vmask >> (16 * kt + 4 * quad + r)) & 1) ? d[kt][r] * scale_log2 : -INFINITY;
                    mx = fmaxf(mx, sv[kt][r]);
                }
            mx = mh_max4(mx);
            const bool move = mx > m_run + MH_LAZY;
            const float m_new = move ? mx : m_run;
            const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
            float psum = 0.f;
            uint4 pa;   // A operand: keys 4 quad .. 4 quad + 3 of tile 0, then of tile 1
            {
                float p[2][4];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        p[kt][r] = sv[kt][r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[kt][r] - m_new);
                pa.x = pack_bf16(p[0][0], p[0][1], psum);
                pa.y = pack_bf16(p[0][2], p[0][3], psum);
                pa.z = pack_bf16(p[1][0], p[1][1], psum);
                pa.w = pack_bf16(p[1][2], p[1][3], psum);
            }
            psum = mh_sum4(psum);
            l_run = l_run * alpha + psum;
            m_run = m_new;
            // values: output rows are heads 4 quad + r, whose factors sit in lanes 4 quad + r
            if (__ballot(move) != 0) {
                float al[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * quad + r, 64);
#pragma unroll
                for (int ct = 0; ct < 32; ++ct) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[ct][r] *= al[r];
                    __builtin_amdgcn_sched_barrier(0);   // one tile at a time: no VGPR copy of all of O
                }
            }
            {
                // values: the transposed reads of column tile ct run MH_PV tiles ahead of its product
                // row 4 quad + jj/4 (and 16 rows on), columns 16 ct + 4 (jj % 4) ..: chunk 2 ct + (jj % 4) / 2
                const int vrow = 4 * quad + (jj >> 2), vsw = mh_swz(vrow);
                const char *vb = bL + vrow * MH_ROWB + 8 * (jj & 1);
                auto b_op = [&](int ct) -> v8s {
                    const int pos = (2 * ct + ((jj & 3) >> 1)) ^ vsw;
                    const v4s lo =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(vb + 16 * pos));
                    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4s *)(vb + 16 * MH_ROWB + 16 * pos));
                    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                };
                v8s ring[MH_PV];
#pragma unroll
                for (int i = 0; i < MH_PV; ++i) ring[i] = b_op(i);
#pragma unroll
                for (int ct = 0; ct < 32; ++ct) {
                    const v8s vt = ring[ct % MH_PV];
                    if (ct + MH_PV < 32) ring[ct % MH_PV] = b_op(ct + MH_PV);
                    acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pa), __builtin_bit_cast(bf16x8, vt),
                                                                      acc[ct], 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 2 * MH_PV; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
                for (int i = 0; i < 32 - MH_PV; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
#pragma unroll
                for (int i = 0; i < MH_PV; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            __syncthreads();   // buffer buf is free for chunk c + MH_NBUF; sRow is free after the last chunk
        }
    }
    float *po = o_part + (((int64_t)b * NS + s) * DM_H + 16 * wave + 4 * quad) * DM_L + jj;
#pragma unroll
    for (int ct = 0; ct < 32; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) po[(int64_t)r * DM_L + 16 * ct] = acc[ct][r];
    if (quad == 0) {
        m_part[((int64_t)b * NS + s) * DM_H + h] = m_run;
        l_part[((int64_t)b * NS + s) * DM_H + h] = l_run;
    }
}

// ------------------------------------------------------------------------------ combine + W_UV
// Maximum and sum over the 64 lanes of a wave with DPP moves (row shifts inside rows of 16 lanes,
// then row broadcasts), read back from the last lane: no LDS traffic.
__device__ __forceinline__ float wave_max_dpp(float x)
{
    const int ninf = __float_as_int(-INFINITY);
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(x), 0x111, 0xf, 0xf, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(x), 0x112, 0xf, 0xf, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(x), 0x114, 0xf, 0xf, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(x), 0x118, 0xf, 0xf, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(x), 0x142, 0xa, 0xf, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(x), 0x143, 0xc, 0xf, false)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ float wave_sum_dpp(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xa, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xc, 0xf, false));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// grid (v / 64, H, ceil(B / 16)), 256 threads; QB queries and SB splits per batch of partials
// (QB = 1, SB >= NS when the launch holds one query: a single batch).  Wave w owns rows
// 64 bx + 16 w .. +16 of W_UV[h]; they are requested first, one whole 1 KB row per DMA straight
// into LDS (rows padded to 1040 B so the operand reads are conflict-free), then the first batch
// of split partials and the splits' maxima and sums.  Wave w reduces queries w, w+4, .. over
// the splits (one split per lane) into the factors
//   f_s = exp2(m_s - max_s m_s) / sum_s exp2(m_s - max_s m_s) l_s,
// the latent rows clat = sum_s f_s O_s (in split order) are staged in LDS as bf16, and the 512
// latent columns are contracted in 16 MFMA steps.
constexpr int CU_ROW = DM_L + 8;
constexpr int CU_WROW = DM_L + 8;          // bf16 per staged W_UV row (1040 B)
constexpr int CU_MAXNS = 64;
constexpr size_t CU_LDS = (size_t)(64 * CU_WROW + 16 * CU_ROW) * 2 + (size_t)16 * CU_MAXNS * 4;

template <int QB, int SB>
__global__ __launch_bounds__(256) void combine_unabsorb(const float *__restrict__ o_part,
                                                        const float *__restrict__ m_part,
                                                        const float *__restrict__ l_part, int NS,
                                                        const bf16_t *__restrict__ kv_b, int B, int nope, int v,
                                                        float *__restrict__ out)
{
    extern __shared__ __attribute__((aligned(16))) char cu_smem[];
    bf16_t *sW = reinterpret_cast<bf16_t *>(cu_smem);
    bf16_t *sC = sW + 64 * CU_WROW;
    float *sF = reinterpret_cast<float *>(sC + 16 * CU_ROW);   // [query][split] factors
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = blockIdx.y, j0 = 64 * blockIdx.x + 16 * wave, b0 = 16 * blockIdx.z;
    const int nb = B - b0 < 16 ? B - b0 : 16;
    const int r16 = lane & 15, q4 = lane >> 4;
    {
        const bf16_t *wsrc = kv_b + ((int64_t)h * (nope + v) + nope + j0) * DM_L + 8 * lane;
#pragma unroll
        for (int i = 0; i < 16; ++i) lds_dma16(wsrc + (int64_t)i * DM_L, lds_addr(sW + (16 * wave + i) * CU_WROW));
    }

    float2 x[QB][SB];
    // unconditional loads (query and split clamped into range), zeroed after: conditional loads
    // would each wait for the previous ones
    auto load_batch = [&](int q0, int s0) {
#pragma unroll
        for (int qq = 0; qq < QB; ++qq)
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                const int qc = q0 + qq < nb ? q0 + qq : nb - 1;
                const int sc = s0 + u < NS ? s0 + u : NS - 1;
                const float2 val = *reinterpret_cast<const float2 *>(
                    o_part + (((int64_t)(b0 + qc) * NS + sc) * DM_H + h) * DM_L + 2 * tid);
                x[qq][u] = (q0 + qq < nb && s0 + u < NS) ? val : make_float2(0.f, 0.f);
            }
    };
    load_batch(0, 0);
    // maxima and sums: wave w, lane = split, queries w + 4k
    float mv[4], lv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int q = wave + 4 * k;
        const int qc = q < nb ? q : nb - 1, sc = lane < NS ? lane : NS - 1;
        const int64_t o = ((int64_t)(b0 + qc) * NS + sc) * DM_H + h;
        mv[k] = m_part[o];
        lv[k] = l_part[o];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int q = wave + 4 * k;
        if (q < nb) {
            const float m = lane < NS ? mv[k] : -INFINITY;
            const float M = wave_max_dpp(m);
            const float e = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
            const float L = wave_sum_dpp(e * (lane < NS ? lv[k] : 0.f));
            sF[q * CU_MAXNS + lane] = L > 0.f ? e / L : 0.f;
        }
    }
    __syncthreads();
    for (int q0 = 0; q0 < nb; q0 += QB) {
        float o[QB][2];
#pragma unroll
        for (int qq = 0; qq < QB; ++qq) o[qq][0] = o[qq][1] = 0.f;
        for (int s0 = 0; s0 < NS; s0 += SB) {
            if (q0 + s0 > 0) load_batch(q0, s0);
#pragma unroll
            for (int qq = 0; qq < QB; ++qq) {
                const int qc = q0 + qq < nb ? q0 + qq : 0;
#pragma unroll
                for (int u = 0; u < SB; ++u) {
                    // factors past the last split are zero; the index only stays inside the row
                    const float f = sF[qc * CU_MAXNS + (s0 + u < CU_MAXNS ? s0 + u : CU_MAXNS - 1)];
                    o[qq][0] = fmaf(f, x[qq][u].x, o[qq][0]);
                    o[qq][1] = fmaf(f, x[qq][u].y, o[qq][1]);
                }
            }
        }
#pragma unroll
        for (int qq = 0; qq < QB; ++qq) {
            if (q0 + qq < nb) {
                const bf16x2 c = {(__bf16)o[qq][0], (__bf16)o[qq][1]};
                *reinterpret_cast<uint32_t *>(&sC[(q0 + qq) * CU_ROW + 2 * tid]) = __builtin_bit_cast(uint32_t, c);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the W_UV rows have landed
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

// ------------------------------------------------------------------------------ combine, batches
// Batches of at least MH_MIN_B queries combine in two launches, so that every split partial
// and every W_UV row is read once (combine_unabsorb re-reads the partials for each 64-row slice
// of W_UV):
//   combine_reduce  grid (ceil(B H / 8)), 256 threads: eight (query, head) pairs per workgroup;
//                   wave w reduces the split maxima and sums of pairs 2w, 2w + 1 into the
//                   factors f_s (as combine_unabsorb), then thread t forms columns 2t, 2t + 1 of
//                   clat = sum_s f_s O_s (in split order) for the eight pairs, stored as bf16;
//   unabsorb        grid (v / 64, H), 256 threads: wave w holds rows 64 bx + 16 w .. +16 of W_UV[h]
//                   as the A operand (read straight from memory, K = 512 latent columns) and
//                   multiplies them with clat of 16 queries at a time (B operand, also straight
//                   from memory): out[b][h][j] on v_mfma_f32_16x16x32_bf16.
constexpr int CR_PAIRS = 8;
constexpr int CR_SB = 8;   // splits loaded per batch (all of them at once for up to 8 splits)

__global__ __launch_bounds__(256) void combine_reduce(const float *__restrict__ o_part, const float *__restrict__ m_part,
                                                      const float *__restrict__ l_part, int NS, int npairs,
                                                      bf16_t *__restrict__ clat)
{
    __shared__ float sF[CR_PAIRS][CU_MAXNS];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p0 = CR_PAIRS * blockIdx.x;
    // pair p = b * DM_H + h; its split s partials sit at ((b * NS + s) * DM_H + h)
    auto part = [&](int p, int s) { return ((int64_t)(p / DM_H) * NS + s) * DM_H + p % DM_H; };
    float2 x[CR_PAIRS][CR_SB];
    auto load = [&](int s0) {
#pragma unroll
        for (int q = 0; q < CR_PAIRS; ++q)
#pragma unroll
            for (int u = 0; u < CR_SB; ++u) {
                const int p = p0 + q < npairs ? p0 + q : npairs - 1, s = s0 + u < NS ? s0 + u : NS - 1;
                x[q][u] = *reinterpret_cast<const float2 *>(o_part + part(p, s) * DM_L + 2 * tid);
            }
    };
    load(0);
#pragma unroll
    for (int k = 0; k < CR_PAIRS / 4; ++k) {
        const int q = 2 * wave + k;
        const int p = p0 + q < npairs ? p0 + q : npairs - 1;
        const int sc = lane < NS ? lane : NS - 1;
        const float m = lane < NS ? m_part[part(p, sc)] : -INFINITY;
        const float l = lane < NS ? l_part[part(p, sc)] : 0.f;
        const float M = wave_max_dpp(m);
        const float e = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
        const float L = wave_sum_dpp(e * l);
        sF[q][lane] = L > 0.f ? e / L : 0.f;
    }
    __syncthreads();
    float o[CR_PAIRS][2];
#pragma unroll
    for (int q = 0; q < CR_PAIRS; ++q) o[q][0] = o[q][1] = 0.f;
    for (int s0 = 0; s0 < NS; s0 += CR_SB) {
        if (s0 > 0) load(s0);
#pragma unroll
        for (int q = 0; q < CR_PAIRS; ++q)
#pragma unroll
            for (int u = 0; u < CR_SB; ++u) {
                // factors past the last split are zero (sF holds CU_MAXNS >= NS entries)
                const float f = s0 + u < NS ? sF[q][s0 + u] : 0.f;
                o[q][0] = fmaf(f, x[q][u].x, o[q][0]);
                o[q][1] = fmaf(f, x[q][u].y, o[q][1]);
            }
    }
#pragma unroll
    for (int q = 0; q < CR_PAIRS; ++q)
        if (p0 + q < npairs) {
            const bf16x2 c = {(__bf16)o[q][0], (__bf16)o[q][1]};
            *reinterpret_cast<uint32_t *>(clat + (int64_t)(p0 + q) * DM_L + 2 * tid) = __builtin_bit_cast(uint32_t, c);
        }
}

__global__ __launch_bounds__(256) void unabsorb(const bf16_t *__restrict__ clat, const bf16_t *__restrict__ kv_b, int B,
                                                int nope, int v, float *__restrict__ out)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = blockIdx.y, j0 = 64 * blockIdx.x + 16 * wave;
    const int jj = lane & 15, quad = lane >> 4;
    const bf16_t *wr = kv_b + ((int64_t)h * (nope + v) + nope + j0 + jj) * DM_L + 8 * quad;
    uint4 a[16];
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) a[ks] = *reinterpret_cast<const uint4 *>(wr + 32 * ks);
    // B operand of the query tile starting at b0: clat of query b0 + jj (clamped), 32 ks + 8 quad
    auto load_c = [&](uint4 (&c)[16], int b0) {
        const int bq = b0 + jj < B ? b0 + jj : B - 1;
        const bf16_t *cr = clat + ((int64_t)bq * DM_H + h) * DM_L + 8 * quad;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) c[ks] = *reinterpret_cast<const uint4 *>(cr + 32 * ks);
    };
    uint4 cn[16];
    load_c(cn, 0);
    for (int b0 = 0; b0 < B; b0 += 16) {
        uint4 c[16];
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) c[ks] = cn[ks];
        if (b0 + 16 < B) load_c(cn, b0 + 16);   // the next tile is in flight during this one
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 16; ++ks)
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[ks]), as_bf16x8(c[ks]), d, 0, 0, 0);
        // register r of lane (jj, quad): row j0 + 4 quad + r of W_UV, query b0 + jj
        if (b0 + jj < B) {
            float *o = out + ((int64_t)(b0 + jj) * DM_H + h) * v + j0 + 4 * quad;   // 4-byte aligned only
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = d[r];
        }
    }
}

// ------------------------------------------------------------------------------ combine, one query
// B = 1: grid (v / 128, H), 512 threads.  Waves 4..7 copy the workgroup's 128 W_UV rows of head h
// (rows 128 bx ..) into LDS, 32 rows each, and only wait for them; waves 0..3 load the split
// maxima and sums (lane = split) and the split partials of head h (thread t: columns 2t, 2t + 1
// of every split), so their waits never include the W_UV copies (wait counts are per wave).
// Wave 0 reduces the factors f_s as in combine_unabsorb, waves 0..3 form clat = sum_s f_s O_s
// (split order) as bf16 in LDS, and then all eight waves contract 16 W_UV rows each with clat on
// v_mfma_f32_16x16x32_bf16 (A rows other than 0 are never read into an output).
constexpr int C1_ROWS = 128;
constexpr size_t C1_LDS = (size_t)(C1_ROWS * CU_WROW + 16 * CU_ROW) * 2 + (size_t)CU_MAXNS * 4;

//
// FMT != 0: kv_b holds the codes of a quantized kv_b (qformat.h).  Waves 4..7 then load the codes
// of their W_UV rows into registers and write them to LDS as bf16 in the same layout: the byte
// codes without their row scale, which multiplies the row's product at the end, and MXFP4 weights
// with their block scale; all of these are exact in bf16.
template <int FMT>
__device__ __forceinline__ void c1_stage_quant(const uint8_t *__restrict__ codes, const void *__restrict__ scales,
                                               int64_t row0, bf16_t *__restrict__ sW, int t)
{
    // 128 rows x 32 pieces of 16 columns; piece p = t + 256 i: row p / 32, columns 16 (p % 32) ..
    uint4 c[16];
    float sc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int p = t + 256 * i, r = p >> 5, c16 = p & 31;
        if constexpr (FMT == MLA_Q_MXFP4) {
            const uint2 x = *reinterpret_cast<const uint2 *>(codes + (row0 + r) * (DM_L / 2) + 8 * c16);
            c[i] = make_uint4(x.x, x.y, 0u, 0u);
            sc[i] = q_scale_e8m0(reinterpret_cast<const uint8_t *>(scales)[(row0 + r) * (DM_L / 32) + (c16 >> 1)]);
        } else {
            c[i] = *reinterpret_cast<const uint4 *>(codes + (row0 + r) * DM_L + 16 * c16);
            sc[i] = 1.f;
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int p = t + 256 * i, r = p >> 5, c16 = p & 31;
        uint4 lo, hi;
        q_bf16x16<FMT>(c[i], sc[i], lo, hi);
        uint4 *d = reinterpret_cast<uint4 *>(sW + r * CU_WROW + 16 * c16);
        d[0] = lo;
        d[1] = hi;
    }
}

template <int SB, bool PB16 = false, int FMT = 0>   // splits held per thread, NS <= SB; PB16: bf16 split outputs
__global__ __launch_bounds__(512) void combine_one(const float *__restrict__ o_part, const float *__restrict__ m_part,
                                                   const float *__restrict__ l_part, int NS,
                                                   const void *__restrict__ kv_b, const void *__restrict__ scales,
                                                   int nope, int v, float *__restrict__ out)
{
    extern __shared__ __attribute__((aligned(16))) char c1_smem[];
    bf16_t *sW = reinterpret_cast<bf16_t *>(c1_smem);
    bf16_t *sC = sW + C1_ROWS * CU_WROW;
    float *sF = reinterpret_cast<float *>(sC + 16 * CU_ROW);
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = blockIdx.y, jb = C1_ROWS * blockIdx.x;
    const int64_t row0 = (int64_t)h * (nope + v) + nope + jb;   // first W_UV row of the workgroup
    if (wave >= 4) {
        if constexpr (FMT == 0) {
            const int w4 = wave - 4;
            const bf16_t *wsrc = reinterpret_cast<const bf16_t *>(kv_b) + (row0 + 32 * w4) * DM_L + 8 * lane;
#pragma unroll
            for (int i = 0; i < 32; ++i) lds_dma16(wsrc + (int64_t)i * DM_L, lds_addr(sW + (32 * w4 + i) * CU_WROW));
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's copies have landed
        } else {
            c1_stage_quant<FMT>(reinterpret_cast<const uint8_t *>(kv_b), scales, row0, sW, tid - 256);
        }
        __syncthreads();
        __syncthreads();
    } else {
        const int sc = lane < NS ? lane : NS - 1;
        float m = 0.f, l = 0.f;
        if (wave == 0) {
            m = m_part[(int64_t)sc * DM_H + h];
            l = l_part[(int64_t)sc * DM_H + h];
        }
        float2 x[SB];
#pragma unroll
        for (int u = 0; u < SB; ++u) {   // unconditional loads, the split clamped into range
            const int uc = u < NS ? u : NS - 1;
            if (PB16) {
                const uint32_t pv = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const bf16_t *>(o_part) +
                                                                         ((int64_t)uc * DM_H + h) * DM_L + 2 * tid);
                x[u] = make_float2(__uint_as_float(pv << 16), __uint_as_float(pv & 0xffff0000u));
            } else {
                x[u] = *reinterpret_cast<const float2 *>(o_part + ((int64_t)uc * DM_H + h) * DM_L + 2 * tid);
            }
        }
        if (wave == 0) {
            const float mm = lane < NS ? m : -INFINITY;
            const float M = wave_max_dpp(mm);
            const float e = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mm - M);
            const float L = wave_sum_dpp(e * (lane < NS ? l : 0.f));
            sF[lane] = L > 0.f ? e / L : 0.f;
        }
        __syncthreads();
        float o0 = 0.f, o1 = 0.f;
#pragma unroll
        for (int u = 0; u < SB; ++u) {   // factors past the last split are zero
            const float f = sF[u < CU_MAXNS ? u : CU_MAXNS - 1];
            o0 = fmaf(f, x[u].x, o0);
            o1 = fmaf(f, x[u].y, o1);
        }
        const bf16x2 c = {(__bf16)o0, (__bf16)o1};
        *reinterpret_cast<uint32_t *>(&sC[2 * tid]) = __builtin_bit_cast(uint32_t, c);
        __syncthreads();
    }
    const int r16 = lane & 15, q4 = lane >> 4;
    float rs = 1.f;   // the row scale of the byte formats
    if (FMT == MLA_Q_FP8_E4M3 || FMT == MLA_Q_INT8) rs = reinterpret_cast<const float *>(scales)[row0 + 16 * wave + r16];
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
    const bf16_t *wl = sW + (16 * wave + r16) * CU_WROW + 8 * q4;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4 *>(&sC[r16 * CU_ROW + 32 * ks + 8 * q4]);
        const uint4 wq = *reinterpret_cast<const uint4 *>(wl + 32 * ks);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(wq), d, 0, 0, 0);
    }
    if (q4 == 0) out[(int64_t)h * v + jb + 16 * wave + r16] = (FMT == MLA_Q_FP8_E4M3 || FMT == MLA_Q_INT8) ? d[0] * rs : d[0];
}

// ------------------------------------------------------------------------------ host side
bool decode_mfma_supported(const mla_dims &d, mla_dtype dt)
{
    return dt == MLA_BF16 && d.n_heads == DM_H && d.kv_lora == DM_L && d.qk_rope == DM_R &&
           (d.qk_nope == 128 || d.qk_nope == 192 || d.qk_nope == 256) && d.v_head % 64 == 0;
}

struct DecPlan {
    int ns;        // key splits
    int64_t kps;   // keys per split (multiple of 64)
};

// Batches of at least MH_MIN_B queries run dec_core_mh (all heads per workgroup).  Four queries
// over 2048 selected keys each: 27-30 us on dec_core (16 splits x 4 head groups) + combine_unabsorb
// against 36-39 us on dec_core_mh, whose 32 splits write 16 MB of fp32 partials; from five queries
// on dec_core_mh is the faster (B = 6: 38 against 46 us, B = 16: 43 against 60 us).
constexpr int MH_MIN_B = 5;

// Splits: at most 256 keys per split, enough splits for ~256 workgroups (dec_core: 4 head groups
// each; dec_core_mh: ~128, since each of its splits writes 64 heads' fp32 partials -- 2048 keys per
// query, same box: B = 8 35.5 against 40.9 us with ~256, B = 12 40.4 against 44.9, B = 24 48.2
// against 61.7, B = 5 39.9 against 37.2), at least 64 keys per split and at most CU_MAXNS splits.
static DecPlan dec_plan(int32_t B, int64_t max_keys)
{
    DecPlan p;
    const int64_t by_len = (max_keys + 255) / 256;
    const int64_t by_fill = ((B >= MH_MIN_B ? 128 : 64) + B - 1) / (int64_t)B;
    const int64_t most = (max_keys + DC_KC - 1) / DC_KC;
    int64_t ns = by_len > by_fill ? by_len : by_fill;
    if (B >= MH_MIN_B) {
        // at most ~256 workgroups' worth of length splits: a large batch fills the chip by itself,
        // and every split adds 64 heads' fp32 partials (2048 keys per query, same box: B = 64 95.9
        // -> 79.7 us, B = 256 368 -> 264 us, 4096 queries 5.0 -> 3.4 ms; B = 32 keeps 8 splits)
        const int64_t cap = (256 + B - 1) / B;
        const int64_t l = by_len < cap ? by_len : cap;
        ns = l > by_fill ? l : by_fill;
    }
    // two to four queries: the fewest splits whose keys fit one staged set (DC_SUP chunks), so
    // that every split takes dec_core<true> (2048 keys: 16 splits; same box, B = 2 / 3: 27.0 /
    // 29.5 us against 31.4 / 35.3 with 32 / 22 splits)
    if (B > 1 && B < MH_MIN_B) ns = (max_keys + DC_SUP * DC_KC - 1) / (DC_SUP * DC_KC);
    // one query over more than 2048 keys: likewise one staged set per split, up to CU_MAXNS splits
    // (dense T = 4096: 32 splits of 128, 20.7 against 22.7 us with 64 of 64; 2048 keys keep 32
    // splits of 64, faster than 16 of 128; from 8192 keys on CU_MAXNS decides)
    if (B == 1 && max_keys > 2048) ns = (max_keys + DC_SUP * DC_KC - 1) / (DC_SUP * DC_KC);
    if (ns > most) ns = most;
    if (ns > CU_MAXNS) ns = CU_MAXNS;
    if (ns < 1) ns = 1;
    p.ns = (int)ns;
    int64_t kps = (max_keys + ns - 1) / ns;
    p.kps = (kps + DC_KC - 1) / DC_KC * DC_KC;
    if (p.kps < DC_KC) p.kps = DC_KC;
    return p;
}

template <int FMT> static hipError_t c1_attrs()
{
    const void *c1[3] = {reinterpret_cast<const void *>(&combine_one<16, true, FMT>),
                         reinterpret_cast<const void *>(&combine_one<32, true, FMT>),
                         reinterpret_cast<const void *>(&combine_one<64, true, FMT>)};
    hipError_t e = hipSuccess;
    for (int i = 0; i < 3 && e == hipSuccess; ++i)
        e = hipFuncSetAttribute(c1[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)C1_LDS);
    return e;
}

// dec_core stages 128 latent rows (134 KB), combine_unabsorb 64 rows of W_UV (65 KB)
static mla_status enable_big_lds()
{
    static bool done = false;
    if (!done) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&dec_core<true>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)DC_LDS);
        if (e == hipSuccess)
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(&dec_core<true, true>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)DC_LDS);
        if (e == hipSuccess)
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(&dec_core<false, true>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)DC_LDS);
        if (e == hipSuccess)
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(&dec_core<false>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)DC_LDS);
        if (e == hipSuccess)
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(&dec_core_mh),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)MH_LDS);
        const void *am[3] = {reinterpret_cast<const void *>(&absorb_q_mfma<8>),
                             reinterpret_cast<const void *>(&absorb_q_mfma<12>),
                             reinterpret_cast<const void *>(&absorb_q_mfma<16>)};
        for (int i = 0; i < 3 && e == hipSuccess; ++i)
            e = hipFuncSetAttribute(am[i], hipFuncAttributeMaxDynamicSharedMemorySize, 16 * 16 * AB_WROWB);
        const void *cu[4] = {reinterpret_cast<const void *>(&combine_unabsorb<1, 16>),
                             reinterpret_cast<const void *>(&combine_unabsorb<1, 32>),
                             reinterpret_cast<const void *>(&combine_unabsorb<1, 64>),
                             reinterpret_cast<const void *>(&combine_unabsorb<4, 16>)};
        for (int i = 0; i < 4 && e == hipSuccess; ++i)
            e = hipFuncSetAttribute(cu[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)CU_LDS);
        if (e == hipSuccess) e = c1_attrs<0>();
        if (e == hipSuccess) e = c1_attrs<MLA_Q_FP8_E4M3>();
        if (e == hipSuccess) e = c1_attrs<MLA_Q_INT8>();
        if (e == hipSuccess) e = c1_attrs<MLA_Q_MXFP4>();
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
    bytes += al256((size_t)B * p.ns * DM_H * 4);                // split maxima
    bytes += al256((size_t)B * p.ns * DM_H * 4);                // split sums
    bytes += al256((size_t)B * p.ns * DM_H * DM_L * 4);         // split outputs
    bytes += al256((size_t)B * DM_H * DM_L * 2);                // combined latent rows (batches)
    (void)d;
    return bytes;
}

// Workspace layout (the first part depends on B only, so the absorb step can run without
// knowing the key count): q_abs | split maxima | split sums | split outputs | combined latent rows
struct DecWs {
    bf16_t *q_abs;
    float *m_part;
    float *l_part;
    float *o_part;
    bf16_t *clat;
};

static DecWs dec_ws(void *ws, int32_t B, const DecPlan &p)
{
    DecWs w;
    char *c = reinterpret_cast<char *>((reinterpret_cast<uintptr_t>(ws) + 255) & ~(uintptr_t)255);
    w.q_abs = reinterpret_cast<bf16_t *>(c);
    c += al256((size_t)B * DM_H * DM_L * 2);
    w.m_part = reinterpret_cast<float *>(c);
    c += al256((size_t)B * p.ns * DM_H * 4);
    w.l_part = reinterpret_cast<float *>(c);
    c += al256((size_t)B * p.ns * DM_H * 4);
    w.o_part = reinterpret_cast<float *>(c);
    c += al256((size_t)B * p.ns * DM_H * DM_L * 4);
    w.clat = reinterpret_cast<bf16_t *>(c);
    return w;
}

size_t decode_mfma_absorb_ws(int32_t B) { return 256 + al256((size_t)B * DM_H * DM_L * 2); }

bf16_t *decode_mfma_qabs(void *ws) { return dec_ws(ws, 1, DecPlan{1, DC_KC}).q_abs; }

mla_status launch_absorb_mfma(const void *q_nope, const void *kv_b, const mla_dims &d, int32_t B, void *ws,
                              hipStream_t s)
{
    if (B > 65535) return fail(MLA_ERR_UNSUPPORTED, "decode: B > 65535");
    const DecWs w = dec_ws(ws, B, dec_plan(B, 0));
    if (B >= AB_MFMA_B) {
        mla_status st = enable_big_lds();
        if (st) return st;
        const dim3 g(DM_L / 128, DM_H), blk(256);
        const size_t shm = (size_t)d.qk_nope * AB_WROWB;
        const bf16_t *qn = (const bf16_t *)q_nope, *kb = (const bf16_t *)kv_b;
        if (d.qk_nope == 128) hipLaunchKernelGGL(absorb_q_mfma<8>, g, blk, shm, s, qn, kb, B, d.v_head, w.q_abs);
        else if (d.qk_nope == 192) hipLaunchKernelGGL(absorb_q_mfma<12>, g, blk, shm, s, qn, kb, B, d.v_head, w.q_abs);
        else hipLaunchKernelGGL(absorb_q_mfma<16>, g, blk, shm, s, qn, kb, B, d.v_head, w.q_abs);
        return check_launch("absorb_q_mfma");
    }
    // at most 32 queries' worth of q staged in LDS per launch
    for (int b0 = 0; b0 < B; b0 += 32) {
        const int nb = B - b0 < 32 ? B - b0 : 32;
        const size_t shm = (size_t)nb * d.qk_nope * 4 + 4 * AB_QB * 128 * 4;
        const dim3 g(DM_L / 128, DM_H), blk(256);
        const bf16_t *qn = (const bf16_t *)q_nope + (int64_t)b0 * DM_H * d.qk_nope;
        bf16_t *qa = w.q_abs + (int64_t)b0 * DM_H * DM_L;
        if (d.qk_nope == 128)
            hipLaunchKernelGGL(absorb_q<8>, g, blk, shm, s, qn, (const bf16_t *)kv_b, nb, d.v_head, qa);
        else if (d.qk_nope == 192)
            hipLaunchKernelGGL(absorb_q<12>, g, blk, shm, s, qn, (const bf16_t *)kv_b, nb, d.v_head, qa);
        else
            hipLaunchKernelGGL(absorb_q<16>, g, blk, shm, s, qn, (const bf16_t *)kv_b, nb, d.v_head, qa);
        mla_status st = check_launch("absorb_q");
        if (st) return st;
    }
    return MLA_OK;
}

mla_status launch_attend_mfma(const void *q_rope, const void *kv_b, const mla_dims &d, int32_t B, const KvView &kv,
                              const int32_t *sel, const int32_t *nsel, int32_t sel_stride, int64_t max_keys,
                              float sm_scale, float *out, void *ws, hipStream_t s, const void *scales, int fmt)
{
    if (B > 65535) return fail(MLA_ERR_UNSUPPORTED, "decode: B > 65535");
    if (max_keys > 0x7fffffff) return fail(MLA_ERR_UNSUPPORTED, "decode: too many keys");
    if (fmt < 0 || fmt > MLA_Q_MXFP4) return fail(MLA_ERR_ARG, "decode: unknown weight format %d", fmt);
    const DecPlan p = dec_plan(B, max_keys);
    const DecWs w = dec_ws(ws, B, p);
    const float scale_log2 = sm_scale * 1.4426950408889634f;
    mla_status st = enable_big_lds();
    if (st) return st;
    // the W_UV slice when the decode leaves at least as many CUs idle
    const int pf = (int64_t)B * p.ns * (DM_H / 16) <= 128 ? 1 : 0;
    // one query: the split outputs go to combine_one as bf16 (half the bytes each way)
    const bool one_b16 = B == 1 && d.v_head % C1_ROWS == 0;
    // W_UV in 1 KB units for the read-ahead slice: a bf16 row, two byte-code rows, or four MXFP4 rows
    const int upr = fmt == 0 ? 1 : fmt == MLA_Q_MXFP4 ? 4 : 2;
    const int64_t w_row_bytes = fmt == 0 ? 2 * DM_L : fmt == MLA_Q_MXFP4 ? DM_L / 2 : DM_L;
    const bf16_t *wuv = reinterpret_cast<const bf16_t *>(reinterpret_cast<const char *>(kv_b) +
                                                         (int64_t)d.qk_nope * w_row_bytes);
    const int rph = (d.qk_nope + d.v_head) / upr, vpf = d.v_head / upr;
    if (B >= MH_MIN_B)
        hipLaunchKernelGGL(dec_core_mh, dim3(p.ns, B), dim3(256), MH_LDS, s, w.q_abs, (const bf16_t *)q_rope, kv, sel,
                           nsel, sel_stride, scale_log2, (int)p.kps, w.o_part, w.m_part, w.l_part);
    else if (one_b16 && p.kps <= DC_SUP * DC_KC)
        hipLaunchKernelGGL((dec_core<true, true>), dim3(p.ns, DM_H / 16, B + pf), dim3(256), DC_LDS, s, w.q_abs,
                           (const bf16_t *)q_rope, kv, sel, nsel, sel_stride, scale_log2, (int)p.kps, w.o_part, w.m_part,
                           w.l_part, B, wuv, rph, vpf);
    else if (one_b16)
        hipLaunchKernelGGL((dec_core<false, true>), dim3(p.ns, DM_H / 16, B + pf), dim3(256), DC_LDS, s, w.q_abs,
                           (const bf16_t *)q_rope, kv, sel, nsel, sel_stride, scale_log2, (int)p.kps, w.o_part, w.m_part,
                           w.l_part, B, wuv, rph, vpf);
    else if (p.kps <= DC_SUP * DC_KC)
        hipLaunchKernelGGL(dec_core<true>, dim3(p.ns, DM_H / 16, B + pf), dim3(256), DC_LDS, s, w.q_abs,
                           (const bf16_t *)q_rope, kv, sel, nsel, sel_stride, scale_log2, (int)p.kps, w.o_part, w.m_part,
                           w.l_part, B, wuv, rph, vpf);
    else
        hipLaunchKernelGGL(dec_core<false>, dim3(p.ns, DM_H / 16, B + pf), dim3(256), DC_LDS, s, w.q_abs,
                           (const bf16_t *)q_rope, kv, sel, nsel, sel_stride, scale_log2, (int)p.kps, w.o_part, w.m_part,
                           w.l_part, B, wuv, rph, vpf);
    st = check_launch("dec_core");
    if (st) return st;
    const dim3 gc(d.v_head / 64, DM_H, (B + 15) / 16);
    const bf16_t *kb = (const bf16_t *)kv_b;
    if (B >= MH_MIN_B || (fmt != 0 && !one_b16)) {
        const int npairs = B * DM_H;
        hipLaunchKernelGGL(combine_reduce, dim3((npairs + CR_PAIRS - 1) / CR_PAIRS), dim3(256), 0, s, w.o_part, w.m_part,
                           w.l_part, p.ns, npairs, w.clat);
        st = check_launch("combine_reduce");
        if (st) return st;
        if (fmt != 0)
            return launch_unabsorb_quant(w.clat, (const uint8_t *)kv_b, scales, fmt, d, B, out, s);
        hipLaunchKernelGGL(unabsorb, dim3(d.v_head / 64, DM_H), dim3(256), 0, s, w.clat, kb, B, d.qk_nope, d.v_head, out);
        return check_launch("unabsorb");
    }
    if (one_b16) {
        const dim3 g1(d.v_head / C1_ROWS, DM_H);
#define C1_LAUNCH(SB, FMT)                                                                                       \
    hipLaunchKernelGGL((combine_one<SB, true, FMT>), g1, dim3(512), C1_LDS, s, w.o_part, w.m_part, w.l_part, p.ns, \
                       kv_b, scales, d.qk_nope, d.v_head, out)
#define C1_FMT(SB)                                                  \
    do {                                                            \
        if (fmt == MLA_Q_FP8_E4M3) C1_LAUNCH(SB, MLA_Q_FP8_E4M3);   \
        else if (fmt == MLA_Q_INT8) C1_LAUNCH(SB, MLA_Q_INT8);      \
        else if (fmt == MLA_Q_MXFP4) C1_LAUNCH(SB, MLA_Q_MXFP4);    \
        else C1_LAUNCH(SB, 0);                                      \
    } while (0)
        if (p.ns <= 16) C1_FMT(16);
        else if (p.ns <= 32) C1_FMT(32);
        else C1_FMT(64);
#undef C1_FMT
#undef C1_LAUNCH
        return check_launch("combine_one");
    }
    if (B == 1 && p.ns <= 16)
        hipLaunchKernelGGL((combine_unabsorb<1, 16>), gc, dim3(256), CU_LDS, s, w.o_part, w.m_part, w.l_part, p.ns,
                           kb, B, d.qk_nope, d.v_head, out);
    else if (B == 1 && p.ns <= 32)
        hipLaunchKernelGGL((combine_unabsorb<1, 32>), gc, dim3(256), CU_LDS, s, w.o_part, w.m_part, w.l_part, p.ns,
                           kb, B, d.qk_nope, d.v_head, out);
    else if (B == 1)
        hipLaunchKernelGGL((combine_unabsorb<1, 64>), gc, dim3(256), CU_LDS, s, w.o_part, w.m_part, w.l_part, p.ns,
                           kb, B, d.qk_nope, d.v_head, out);
    else
        hipLaunchKernelGGL((combine_unabsorb<4, 16>), gc, dim3(256), CU_LDS, s, w.o_part, w.m_part, w.l_part, p.ns,
                           kb, B, d.qk_nope, d.v_head, out);
    return check_launch("combine_unabsorb");
}

}  // namespace mla
