// decode_plan.h -- split-K planning and internal launchers of the absorbed decode.
#pragma once
#include "common.h"

namespace mla {

// Splits of the attended keys for the generic decode: enough (b, h, split) blocks to fill
// the chip at batch 1, at most 64 so the partial buffers stay small.
inline int generic_splits(int64_t max_keys)
{
    int64_t ns = (max_keys + 127) / 128;
    if (ns < 1) ns = 1;
    if (ns > 64) ns = 64;
    return (int)ns;
}

size_t decode_generic_ws(const mla_dims &d, int32_t B, int64_t max_keys);
size_t decode_generic_absorb_ws(const mla_dims &d, int32_t B);
mla_status launch_absorb_generic(const void *q_nope, const void *kv_b, mla_dtype dt, const mla_dims &d, int32_t B,
                                 void *ws, hipStream_t s);
mla_status launch_attend_generic(const void *q_rope, const void *kv_b, mla_dtype dt, const mla_dims &d, int32_t B,
                                 const KvView &kv, const int32_t *sel, const int32_t *nsel, int32_t sel_stride,
                                 int64_t max_keys, float sm_scale, float *out, void *ws, hipStream_t s);

bool decode_mfma_supported(const mla_dims &d, mla_dtype dt);
size_t decode_mfma_ws(const mla_dims &d, int32_t B, int64_t max_keys);
size_t decode_mfma_absorb_ws(int32_t B);
mla_status launch_absorb_mfma(const void *q_nope, const void *kv_b, const mla_dims &d, int32_t B, void *ws,
                              hipStream_t s);
bf16_t *decode_mfma_qabs(void *ws);   // where the absorb step leaves q_abs in a decode workspace
// fmt != 0: kv_b holds the codes of a quantized kv_b with the given scales (qformat.h)
mla_status launch_attend_mfma(const void *q_rope, const void *kv_b, const mla_dims &d, int32_t B, const KvView &kv,
                              const int32_t *sel, const int32_t *nsel, int32_t sel_stride, int64_t max_keys,
                              float sm_scale, float *out, void *ws, hipStream_t s, const void *scales = nullptr,
                              int fmt = 0);
// out[b][h][:] = W_UV[h] clat[b][h] over a quantized kv_b (bf16 clat [B][64][512])
mla_status launch_unabsorb_quant(const bf16_t *clat, const uint8_t *codes, const void *scales, int32_t fmt,
                                 const mla_dims &d, int32_t B, float *out, hipStream_t s);

}  // namespace mla
