// decode_generic.hip -- absorbed MLA decode for any head geometry (fp32 or bf16 inputs,
// fp32 arithmetic).  colibri-analysis 06 "MLA attention and KV cache", sec. 2.3, absorbed
// path: fold W_UK into the query, score against Lc/Rc directly, accumulate the softmax-
// weighted latent, then apply W_UV per head.
//
// Three launches:
//   absorb   q_abs[b][h][c] = sum_i q_nope[b][h][i] * W_UK[h][i][c]
//   core     split-K over the attended keys; each (b, h, split) keeps an online softmax
//            (running max m, running sum l, latent accumulator clat[L])
//   combine  log-sum-exp merge of the splits, then out[b][h] = W_UV[h] clat
#include "common.h"
#include "decode_plan.h"

namespace mla {

template <typename T>
__global__ __launch_bounds__(256) void absorb_generic(const T *__restrict__ q_nope, const T *__restrict__ kv_b,
                                                      int H, int nope, int v, int L, float *__restrict__ q_abs)
{
    const int bh = blockIdx.x;
    const int h = bh % H;
    const int c = blockIdx.y * 256 + threadIdx.x;
    if (c >= L) return;
    const T *qn = q_nope + (int64_t)bh * nope;
    const T *W = kv_b + (int64_t)h * (nope + v) * L;
    float acc = 0.f;
    for (int i = 0; i < nope; ++i) acc = fmaf(ld(qn + i), ld(W + (int64_t)i * L + c), acc);
    q_abs[(int64_t)bh * L + c] = acc;
}

constexpr int kChunk = 256;   // keys scored per round inside one split
constexpr int kMaxLPerThread = 8;   // L <= 2048 with 256 threads

template <typename T>
__global__ __launch_bounds__(256) void decode_core_generic(const float *__restrict__ q_abs,
                                                           const T *__restrict__ q_rope, int H, int rope, int L,
                                                           KvView kv, const int32_t *__restrict__ sel,
                                                           const int32_t *__restrict__ nsel, int sel_stride,
                                                           float sm_scale, int NS, float *__restrict__ part_m,
                                                           float *__restrict__ part_l, float *__restrict__ part_c)
{
    extern __shared__ int64_t sh_rows[];
    int64_t *srow = sh_rows;                                   // [kChunk] pool rows
    float *ss = reinterpret_cast<float *>(srow + kChunk);     // [kChunk] scores, then probabilities
    float *sq = ss + kChunk;                                   // [L]
    float *sr = sq + L;                                        // [rope]
    __shared__ float red[8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int split = blockIdx.x, bh = blockIdx.y, b = bh / H;
    const T *lc = reinterpret_cast<const T *>(kv.lc);
    const T *rc = reinterpret_cast<const T *>(kv.rc);
    const int64_t sl = seq_len_of(kv, b);
    int64_t nk = sl;
    if (sel) {
        nk = nsel[b];
        if (nk < 0) nk = 0;
        if (nk > sel_stride) nk = sel_stride;
    }
    const int64_t kps = (nk + NS - 1) / NS;
    const int64_t j0 = (int64_t)split * kps;
    const int64_t j1 = j0 + kps < nk ? j0 + kps : nk;

    for (int c = tid; c < L; c += 256) sq[c] = q_abs[(int64_t)bh * L + c];
    for (int c = tid; c < rope; c += 256) sr[c] = ld(q_rope + (int64_t)bh * rope + c);

    float m = -INFINITY, l = 0.f;
    float acc[kMaxLPerThread];
#pragma unroll
    for (int i = 0; i < kMaxLPerThread; ++i) acc[i] = 0.f;

    for (int64_t jc = j0; jc < j1; jc += kChunk) {
        const int cnt = (int)(j1 - jc < kChunk ? j1 - jc : kChunk);
        __syncthreads();
        for (int i = tid; i < cnt; i += 256) {
            const int64_t t = sel ? (int64_t)sel[(int64_t)b * sel_stride + jc + i] : jc + i;
            srow[i] = (t >= 0 && t < sl) ? kv_row(kv, b, t) : -1;
        }
        __syncthreads();
        for (int i = wave; i < cnt; i += 4) {
            const int64_t row = srow[i];
            float p = 0.f;
            if (row >= 0) {
                for (int c = lane; c < L; c += 64) p = fmaf(sq[c], ld(lc + row * L + c), p);
                for (int c = lane; c < rope; c += 64) p = fmaf(sr[c], ld(rc + row * rope + c), p);
            }
            p = wave_sum(p);
            if (lane == 0) ss[i] = row >= 0 ? p * sm_scale : -INFINITY;
        }
        __syncthreads();
        // chunk maximum
        float x = tid < cnt ? ss[tid] : -INFINITY;
        x = wave_max(x);
        if (lane == 0) red[wave] = x;
        __syncthreads();
        const float cm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        const float nm = fmaxf(m, cm);
        if (nm == -INFINITY) continue;   // nothing valid yet (uniform across the block)
        const float scale = __expf(m - nm);
        __syncthreads();
        float pv = 0.f;
        if (tid < cnt) {
            pv = ss[tid] == -INFINITY ? 0.f : __expf(ss[tid] - nm);
            ss[tid] = pv;
        }
        pv = wave_sum(pv);
        if (lane == 0) red[4 + wave] = pv;
        __syncthreads();
        l = l * scale + ((red[4] + red[5]) + (red[6] + red[7]));
        m = nm;
#pragma unroll
        for (int i = 0; i < kMaxLPerThread; ++i) {
            const int c = tid + 256 * i;
            if (c < L) {
                float a = acc[i] * scale;
                for (int j = 0; j < cnt; ++j) {
                    const int64_t row = srow[j];
                    if (row >= 0) a = fmaf(ss[j], ld(lc + row * L + c), a);
                }
                acc[i] = a;
            }
        }
    }
    const int64_t slot = (int64_t)bh * NS + split;
    if (tid == 0) {
        part_m[slot] = m;
        part_l[slot] = l;
    }
#pragma unroll
    for (int i = 0; i < kMaxLPerThread; ++i) {
        const int c = tid + 256 * i;
        if (c < L) part_c[slot * L + c] = acc[i];
    }
}

template <typename T>
__global__ __launch_bounds__(256) void combine_unabsorb_generic(const float *__restrict__ part_m,
                                                                const float *__restrict__ part_l,
                                                                const float *__restrict__ part_c, int NS,
                                                                const T *__restrict__ kv_b, int H, int nope, int v,
                                                                int L, float *__restrict__ out)
{
    extern __shared__ float clat[];   // [L]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x, h = bh % H;
    const float *pm = part_m + (int64_t)bh * NS;
    const float *pl = part_l + (int64_t)bh * NS;
    float M = -INFINITY;
    for (int s = 0; s < NS; ++s) M = fmaxf(M, pm[s]);
    float den = 0.f;
    if (M != -INFINITY)
        for (int s = 0; s < NS; ++s)
            if (pm[s] != -INFINITY) den += __expf(pm[s] - M) * pl[s];
    const float inv = den > 0.f ? 1.f / den : 0.f;
    for (int c = tid; c < L; c += 256) {
        float a = 0.f;
        if (M != -INFINITY)
            for (int s = 0; s < NS; ++s)
                if (pm[s] != -INFINITY) a = fmaf(__expf(pm[s] - M), part_c[((int64_t)bh * NS + s) * L + c], a);
        clat[c] = a * inv;
    }
    __syncthreads();
    const T *W = kv_b + ((int64_t)h * (nope + v) + nope) * L;
    for (int jj = wave; jj < 64; jj += 4) {
        const int j = blockIdx.y * 64 + jj;
        if (j >= v) break;
        float a = 0.f;
        for (int c = lane; c < L; c += 64) a = fmaf(ld(W + (int64_t)j * L + c), clat[c], a);
        a = wave_sum(a);
        if (lane == 0) out[(int64_t)bh * v + j] = a;
    }
}

size_t decode_generic_ws(const mla_dims &d, int32_t B, int64_t max_keys)
{
    const int NS = generic_splits(max_keys);
    const size_t BH = (size_t)B * d.n_heads;
    return BH * d.kv_lora * 4 + BH * NS * 8 + BH * NS * (size_t)d.kv_lora * 4 + 256;
}

size_t decode_generic_absorb_ws(const mla_dims &d, int32_t B) { return (size_t)B * d.n_heads * d.kv_lora * 4; }

// Workspace layout: q_abs (fp32, depends on B only) | split maxima | split sums | split latents
mla_status launch_absorb_generic(const void *q_nope, const void *kv_b, mla_dtype dt, const mla_dims &d, int32_t B,
                                 void *ws, hipStream_t s)
{
    const int H = d.n_heads, nope = d.qk_nope, v = d.v_head, L = d.kv_lora;
    const int64_t BH = (int64_t)B * H;
    if (BH > 0x7fffffff) return fail(MLA_ERR_UNSUPPORTED, "decode: B*H too large");
    float *q_abs = reinterpret_cast<float *>(ws);
    const dim3 g((unsigned)BH, (L + 255) / 256);
    if (dt == MLA_FP32)
        hipLaunchKernelGGL(absorb_generic<float>, g, dim3(256), 0, s, (const float *)q_nope, (const float *)kv_b, H,
                           nope, v, L, q_abs);
    else
        hipLaunchKernelGGL(absorb_generic<bf16_t>, g, dim3(256), 0, s, (const bf16_t *)q_nope, (const bf16_t *)kv_b,
                           H, nope, v, L, q_abs);
    return check_launch("absorb_generic");
}

template <typename T>
static mla_status attend_generic(const void *q_rope, const void *kv_b, const mla_dims &d, int32_t B, const KvView &kv,
                                 const int32_t *sel, const int32_t *nsel, int32_t sel_stride, int64_t max_keys,
                                 float sm_scale, float *out, void *ws, hipStream_t s)
{
    const int H = d.n_heads, nope = d.qk_nope, rope = d.qk_rope, v = d.v_head, L = d.kv_lora;
    const int NS = generic_splits(max_keys);
    const int64_t BH = (int64_t)B * H;
    if (BH > 0x7fffffff) return fail(MLA_ERR_UNSUPPORTED, "decode: B*H too large");
    float *q_abs = reinterpret_cast<float *>(ws);
    float *pm = q_abs + BH * L;
    float *pl = pm + BH * NS;
    float *pc = pl + BH * NS;
    const size_t shm = (size_t)(L + rope + kChunk) * 4 + (size_t)kChunk * 8;
    hipLaunchKernelGGL(decode_core_generic<T>, dim3(NS, (unsigned)BH), dim3(256), shm, s, q_abs,
                       (const T *)q_rope, H, rope, L, kv, sel, nsel, sel_stride, sm_scale, NS, pm, pl, pc);
    mla_status st = check_launch("decode_core_generic");
    if (st) return st;
    hipLaunchKernelGGL(combine_unabsorb_generic<T>, dim3((unsigned)BH, (v + 63) / 64), dim3(256), (size_t)L * 4, s,
                       pm, pl, pc, NS, (const T *)kv_b, H, nope, v, L, out);
    return check_launch("combine_unabsorb_generic");
}

mla_status launch_attend_generic(const void *q_rope, const void *kv_b, mla_dtype dt, const mla_dims &d, int32_t B,
                                 const KvView &kv, const int32_t *sel, const int32_t *nsel, int32_t sel_stride,
                                 int64_t max_keys, float sm_scale, float *out, void *ws, hipStream_t s)
{
    if (dt == MLA_FP32)
        return attend_generic<float>(q_rope, kv_b, d, B, kv, sel, nsel, sel_stride, max_keys, sm_scale, out, ws, s);
    return attend_generic<bf16_t>(q_rope, kv_b, d, B, kv, sel, nsel, sel_stride, max_keys, sm_scale, out, ws, s);
}

}  // namespace mla
