// prefill.hip -- chooses the kernels of mla_prefill_nonabsorbed for a given shape and dtype.
#include "prefill_plan.h"

namespace mla {

size_t prefill_workspace_bytes(const mla_dims &d, int32_t S, int64_t T, mla_dtype)
{
    return prefill_generic_ws(d, S, T);
}

mla_status launch_prefill(const void *q, const void *kv_b, mla_dtype dt, const mla_dims &d, const KvView &kv,
                          int32_t S, int32_t pos_base, float sm_scale, void *out, mla_dtype out_dt, void *ws,
                          size_t, hipStream_t s)
{
    return launch_prefill_generic(q, kv_b, dt, d, kv, S, pos_base, sm_scale, out, out_dt, ws, s);
}

}  // namespace mla
