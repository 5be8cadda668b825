// prefill_plan.h -- internal launchers of the non-absorbed prefill.
#pragma once
#include "common.h"

namespace mla {

size_t prefill_generic_ws(const mla_dims &d, int32_t S, int64_t T);
// mask (optional): keys further restricted per query, bit t % 32 of mask[(t / 32) * mask_stride + i]
mla_status launch_prefill_generic(const void *q, const void *kv_b, mla_dtype dt, const mla_dims &d, const KvView &kv,
                                  int32_t S, int32_t pos_base, float sm_scale, void *out, mla_dtype out_dt, void *ws,
                                  hipStream_t s, const uint32_t *mask = nullptr, int mask_stride = 0);

bool prefill_mfma_supported(const mla_dims &d, mla_dtype dt);
size_t prefill_mfma_ws(const mla_dims &d, int64_t T);
mla_status launch_prefill_mfma(const void *q, const void *kv_b, const mla_dims &d, const KvView &kv, int32_t S,
                               int32_t pos_base, float sm_scale, void *out, mla_dtype out_dt, void *ws, hipStream_t s,
                               const uint32_t *mask = nullptr, int mask_stride = 0);

}  // namespace mla
