// decode.hip -- chooses the kernels of mla_absorbed_decode for a given shape and dtype.
#include "decode_plan.h"

namespace mla {

size_t decode_workspace_bytes(const mla_dims &d, int32_t B, int64_t max_keys, mla_dtype)
{
    return decode_generic_ws(d, B, max_keys);
}

mla_status launch_decode(const void *q_nope, const void *q_rope, const void *kv_b, mla_dtype dt,
                         const mla_dims &d, int32_t B, const KvView &kv, const int32_t *sel,
                         const int32_t *nsel, int32_t sel_stride, int64_t max_keys, float sm_scale,
                         float *out, void *ws, size_t, hipStream_t s)
{
    return launch_decode_generic(q_nope, q_rope, kv_b, dt, d, B, kv, sel, nsel, sel_stride, max_keys,
                                 sm_scale, out, ws, s);
}

}  // namespace mla
