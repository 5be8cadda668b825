// prefill.hip -- chooses the kernels of mla_prefill_nonabsorbed for a given shape and dtype:
// the matrix-core kernels (prefill_mfma.hip) for bf16 with 64 heads, kv_lora 512, qk_rope 64,
// v_head 256 and qk_nope 128/192 (16-byte aligned operands required), the generic kernels for
// every other geometry and for fp32.
#include "prefill_plan.h"

namespace mla {

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t prefill_workspace_bytes(const mla_dims &d, int32_t S, int64_t T, mla_dtype dt)
{
    const size_t g = prefill_generic_ws(d, S, T);
    if (prefill_mfma_supported(d, dt)) {
        const size_t m = prefill_mfma_ws(d, T);
        return m > g ? m : g;
    }
    return g;
}

mla_status launch_prefill(const void *q, const void *kv_b, mla_dtype dt, const mla_dims &d, const KvView &kv,
                          int32_t S, int32_t pos_base, float sm_scale, void *out, mla_dtype out_dt, void *ws,
                          size_t, hipStream_t s, const uint32_t *mask, int mask_stride)
{
    if (prefill_mfma_supported(d, dt)) {
        // the matrix-core kernels read and write in 16-byte pieces: on their geometry a tensor
        // that is not 16-byte aligned is rejected, never routed to other kernels
        if (!aligned16(q) || !aligned16(kv_b) || !aligned16(kv.lc) || !aligned16(kv.rc) || !aligned16(out))
            return fail(MLA_ERR_UNSUPPORTED, "prefill: on the matrix-core geometry (bf16, 64 heads, kv_lora 512, "
                        "qk_rope 64, v_head 256) every tensor must be 16-byte aligned");
        return launch_prefill_mfma(q, kv_b, d, kv, S, pos_base, sm_scale, out, out_dt, ws, s, mask, mask_stride);
    }
    return launch_prefill_generic(q, kv_b, dt, d, kv, S, pos_base, sm_scale, out, out_dt, ws, s, mask, mask_stride);
}

}  // namespace mla
