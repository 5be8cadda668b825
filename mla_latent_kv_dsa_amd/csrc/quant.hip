// quant.hip -- absorbed decode with a quantized kv_b.
// colibri-analysis 06 "MLA attention and KV cache", sec. 2.3: the absorbed path reads kv_b only
// in the two per-head products (qt_addrow folds W_UK into the query, qt_matvec_rows applies W_UV to
// the combined latent), over quantized rows.  aiknowledge.cn Ch.7 sec. 03, sec. 3 and 5: int8 /
// FP8 / MXFP4 weight formats, each a bounded-loss form of the same weights.  At batch 1 these two
// products stream all of kv_b (29.4 MB in bf16 at the GLM geometry) against 2.4 MB of selected
// cache; 8-bit codes halve that, MXFP4 quarters it.
//
// Formats (a row of kv_b = kv_lora columns):
//   MLA_Q_FP8_E4M3  one byte per weight, OCP E4M3 (no infinities), one fp32 scale per row
//   MLA_Q_INT8      one signed byte per weight, one fp32 scale per row
//   MLA_Q_MXFP4     OCP MX: FP4 E2M1, two per byte (even column in the low nibble), an E8M0
//                   scale byte per 32 columns
// The codes are decoded by the chip's scaled conversion instructions (qformat.h); every product and
// sum is fp32, so the only loss against the bf16 path is the weights' own.
//   absorption        q_abs[b][h][:] = W_UK[h]^T q_nope[b][h] (bf16 out, as the bf16 path): the
//                     decode step's side job over the codes (absorb_body.h), or absorb_q_quant for
//                     batches beyond it
//   attention         the matrix-core key splits; at batch 1 combine_one decodes W_UV into LDS and
//                     contracts it on the matrix cores (decode_mfma), otherwise the split
//                     reduction into clat and unabsorb_quant
//   unabsorb_quant    out[b][h][j] = W_UV[h][j] . clat[b][h]
#include "common.h"
#include "decode_plan.h"
#include "qformat.h"

namespace mla {

constexpr int QA_QB = 8;   // queries per pass

// grid (L / 128, H), 256 threads: thread t holds columns 128 bx + 4 (t % 32) .. + 3 over the W_UK rows
// t / 32, t / 32 + 8, ..; the eight row groups are summed through LDS in a fixed order.
template <int FMT>
__global__ __launch_bounds__(256) void absorb_q_quant(const bf16_t *__restrict__ q_nope, const uint8_t *__restrict__ codes,
                                                      const void *__restrict__ scales, int B, int nope, int v, int L,
                                                      bf16_t *__restrict__ q_abs)
{
    __shared__ float sq[QA_QB][256];
    __shared__ float red[8][QA_QB][128];
    const int tid = threadIdx.x, cg = tid & 31, rg = tid >> 5;
    const int h = blockIdx.y, H = gridDim.y, c = 128 * blockIdx.x + 4 * cg;
    const int64_t row0 = (int64_t)h * (nope + v);
    for (int b0 = 0; b0 < B; b0 += QA_QB) {
        const int nb = B - b0 < QA_QB ? B - b0 : QA_QB;
        for (int e = tid; e < QA_QB * nope; e += 256) {
            const int bb = e / nope, i = e - bb * nope;
            sq[bb][i] = bb < nb ? bf2f(q_nope[((int64_t)(b0 + bb) * H + h) * nope + i]) : 0.f;
        }
        __syncthreads();
        float acc[QA_QB][4] = {};
        for (int i = rg; i < nope; i += 8) {
            float w[4];
            q_load4<FMT>(codes, scales, row0 + i, L, c, w);
#pragma unroll
            for (int bb = 0; bb < QA_QB; ++bb) {
                const float a = sq[bb][i];
#pragma unroll
                for (int k = 0; k < 4; ++k) acc[bb][k] = __builtin_fmaf(a, w[k], acc[bb][k]);
            }
        }
#pragma unroll
        for (int bb = 0; bb < QA_QB; ++bb)
#pragma unroll
            for (int k = 0; k < 4; ++k) red[rg][bb][4 * cg + k] = acc[bb][k];
        __syncthreads();
        for (int o = tid; o < QA_QB * 128; o += 256) {
            const int bb = o >> 7, col = o & 127;
            float sum = 0.f;
#pragma unroll
            for (int g = 0; g < 8; ++g) sum += red[g][bb][col];
            if (bb < nb) q_abs[((int64_t)(b0 + bb) * H + h) * L + 128 * blockIdx.x + col] = f2bf(sum);
        }
        __syncthreads();
    }
}

// grid (v / 32, H), 256 threads: eight threads per W_UV row (thread t: row 32 bx + t / 8, columns
// 4 (t % 8) + 32 k), summed across the eight with lane exchanges.
template <int FMT>
__global__ __launch_bounds__(256) void unabsorb_quant(const bf16_t *__restrict__ clat, const uint8_t *__restrict__ codes,
                                                      const void *__restrict__ scales, int B, int nope, int v, int L,
                                                      float *__restrict__ out)
{
    __shared__ float sc[QA_QB][512];
    const int tid = threadIdx.x, pr = tid & 7;
    const int h = blockIdx.y, H = gridDim.y, j = 32 * blockIdx.x + (tid >> 3);
    const int64_t row = (int64_t)h * (nope + v) + nope + j;
    for (int b0 = 0; b0 < B; b0 += QA_QB) {
        const int nb = B - b0 < QA_QB ? B - b0 : QA_QB;
        for (int e = tid; e < QA_QB * L; e += 256) {
            const int bb = e / L, c = e - bb * L;
            sc[bb][c] = bb < nb ? bf2f(clat[((int64_t)(b0 + bb) * H + h) * L + c]) : 0.f;
        }
        __syncthreads();
        float acc[QA_QB] = {};
        for (int c = 4 * pr; c < L; c += 32) {
            float w[4];
            q_load4<FMT>(codes, scales, row, L, c, w);
#pragma unroll
            for (int bb = 0; bb < QA_QB; ++bb)
#pragma unroll
                for (int k = 0; k < 4; ++k) acc[bb] = __builtin_fmaf(w[k], sc[bb][c + k], acc[bb]);
        }
#pragma unroll
        for (int bb = 0; bb < QA_QB; ++bb) {
            float x = acc[bb];
            x += __shfl_xor(x, 1, 64);
            x += __shfl_xor(x, 2, 64);
            x += __shfl_xor(x, 4, 64);
            if (pr == 0 && bb < nb) out[((int64_t)(b0 + bb) * H + h) * v + j] = x;
        }
        __syncthreads();
    }
}

bool decode_quant_supported(const mla_dims &d, mla_dtype dt)
{
    return decode_mfma_supported(d, dt) && d.qk_nope % 8 == 0 && d.qk_nope <= 256 && d.v_head % 32 == 0;
}

mla_status launch_unabsorb_quant(const bf16_t *clat, const uint8_t *codes, const void *scales, int32_t fmt,
                                 const mla_dims &d, int32_t B, float *out, hipStream_t s)
{
    const int L = d.kv_lora, H = d.n_heads;
#define MLA_UQ(F) hipLaunchKernelGGL(unabsorb_quant<F>, dim3(d.v_head / 32, H), dim3(256), 0, s, clat, codes, scales, \
                                     B, d.qk_nope, d.v_head, L, out)
    if (fmt == MLA_Q_FP8_E4M3) MLA_UQ(MLA_Q_FP8_E4M3);
    else if (fmt == MLA_Q_INT8) MLA_UQ(MLA_Q_INT8);
    else MLA_UQ(MLA_Q_MXFP4);
#undef MLA_UQ
    return check_launch("unabsorb_quant");
}

// The absorption over the quantized W_UK (the side job of the decode step as a launch of its own,
// up to SIDE_MAXB queries; absorb_q_quant beyond), then the matrix-core attention with the
// quantized W_UV (decode_mfma).
mla_status launch_decode_quant(const void *q_nope, const void *q_rope, const uint8_t *codes, const void *scales,
                               int32_t fmt, const mla_dims &d, int32_t B, const KvView &kv, const int32_t *sel,
                               const int32_t *nsel, int32_t sel_stride, int64_t max_keys, float sm_scale, float *out,
                               void *ws, hipStream_t s)
{
    const int L = d.kv_lora, H = d.n_heads;
    bf16_t *qa = decode_mfma_qabs(ws);
    const bf16_t *qn = (const bf16_t *)q_nope;
    SideAbsorb sa{};
    sa.q_nope = qn;
    sa.kv_b = codes;
    sa.scales = scales;
    sa.fmt = fmt;
    sa.q_abs = qa;
    sa.q_rope = (const bf16_t *)q_rope;
    sa.q_rope_out = nullptr;   // the query tails come rotated
    sa.B = B;
    sa.nope = d.qk_nope;
    sa.v = d.v_head;
    sa.rope = d.qk_rope;
    mla_status st;
    if (side_absorb_ok(sa)) {
        st = launch_absorb_rope(sa, kv, s);
    } else {
#define MLA_QA(F) hipLaunchKernelGGL(absorb_q_quant<F>, dim3(L / 128, H), dim3(256), 0, s, qn, codes, scales, B, \
                                     d.qk_nope, d.v_head, L, qa)
        if (fmt == MLA_Q_FP8_E4M3) MLA_QA(MLA_Q_FP8_E4M3);
        else if (fmt == MLA_Q_INT8) MLA_QA(MLA_Q_INT8);
        else MLA_QA(MLA_Q_MXFP4);
#undef MLA_QA
        st = check_launch("absorb_q_quant");
    }
    if (st) return st;
    return launch_attend_mfma(q_rope, codes, d, B, kv, sel, nsel, sel_stride, max_keys, sm_scale, out, ws, s, scales,
                              fmt);
}

}  // namespace mla
