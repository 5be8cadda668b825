// decode.hip -- chooses the kernels of mla_absorbed_decode for a given shape and dtype:
// the matrix-core kernels for bf16 caches with 64 heads, kv_lora 512 and qk_rope 64 (and
// 16-byte aligned tensors), the generic kernels for every other geometry.
#include "decode_plan.h"

namespace mla {

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t decode_workspace_bytes(const mla_dims &d, int32_t B, int64_t max_keys, mla_dtype dt)
{
    size_t g = decode_generic_ws(d, B, max_keys);
    if (decode_mfma_supported(d, dt)) {
        size_t m = decode_mfma_ws(d, B, max_keys);
        return m > g ? m : g;
    }
    return g;
}

mla_status launch_decode(const void *q_nope, const void *q_rope, const void *kv_b, mla_dtype dt,
                         const mla_dims &d, int32_t B, const KvView &kv, const int32_t *sel,
                         const int32_t *nsel, int32_t sel_stride, int64_t max_keys, float sm_scale,
                         float *out, void *ws, size_t, hipStream_t s)
{
    if (decode_mfma_supported(d, dt) && aligned16(q_nope) && aligned16(q_rope) && aligned16(kv_b) &&
        aligned16(kv.lc) && aligned16(kv.rc))
        return launch_decode_mfma(q_nope, q_rope, kv_b, d, B, kv, sel, nsel, sel_stride, max_keys, sm_scale, out,
                                  ws, s);
    return launch_decode_generic(q_nope, q_rope, kv_b, dt, d, B, kv, sel, nsel, sel_stride, max_keys,
                                 sm_scale, out, ws, s);
}

}  // namespace mla
