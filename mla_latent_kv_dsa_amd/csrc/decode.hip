// decode.hip -- chooses the kernels of the absorbed decode for a given shape and dtype: the
// matrix-core kernels for bf16 caches with 64 heads, kv_lora 512 and qk_rope 64, the generic
// kernels for every other geometry.  The decode runs in two steps that share one workspace:
// absorb (W_UK folded into the query; needs only q_nope and kv_b) and attend (scores,
// softmax, latent accumulation, W_UV).  The absorb step can therefore be issued early, e.g.
// on a second stream while the indexer and the top-k run.
#include "decode_plan.h"

namespace mla {

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The path both steps take: decided from what the absorb step sees (shape, dtype, kv_b).
static bool use_mfma(const mla_dims &d, mla_dtype dt, const void *kv_b)
{
    return decode_mfma_supported(d, dt) && aligned16(kv_b);
}

size_t decode_workspace_bytes(const mla_dims &d, int32_t B, int64_t max_keys, mla_dtype dt)
{
    size_t g = decode_generic_ws(d, B, max_keys);
    if (decode_mfma_supported(d, dt)) {
        size_t m = decode_mfma_ws(d, B, max_keys);
        return m > g ? m : g;
    }
    return g;
}

size_t decode_absorb_workspace_bytes(const mla_dims &d, int32_t B, mla_dtype dt)
{
    size_t g = decode_generic_absorb_ws(d, B);
    if (decode_mfma_supported(d, dt)) {
        size_t m = decode_mfma_absorb_ws(B);
        return m > g ? m : g;
    }
    return g;
}

mla_status launch_decode_absorb(const void *q_nope, const void *kv_b, mla_dtype dt, const mla_dims &d, int32_t B,
                                void *ws, hipStream_t s)
{
    if (use_mfma(d, dt, kv_b)) return launch_absorb_mfma(q_nope, kv_b, d, B, ws, s);
    return launch_absorb_generic(q_nope, kv_b, dt, d, B, ws, s);
}

mla_status launch_decode_attend(const void *q_rope, const void *kv_b, mla_dtype dt, const mla_dims &d, int32_t B,
                                const KvView &kv, const int32_t *sel, const int32_t *nsel, int32_t sel_stride,
                                int64_t max_keys, float sm_scale, float *out, void *ws, hipStream_t s)
{
    if (use_mfma(d, dt, kv_b)) {
        if (!aligned16(q_rope) || !aligned16(kv.lc) || !aligned16(kv.rc))
            return fail(MLA_ERR_UNSUPPORTED,
                        "decode: the matrix-core path needs 16-byte aligned q_rope, Lc and Rc (the fused call "
                        "mla_absorbed_decode falls back to the generic kernels instead)");
        return launch_attend_mfma(q_rope, kv_b, d, B, kv, sel, nsel, sel_stride, max_keys, sm_scale, out, ws, s);
    }
    return launch_attend_generic(q_rope, kv_b, dt, d, B, kv, sel, nsel, sel_stride, max_keys, sm_scale, out, ws, s);
}

mla_status launch_decode(const void *q_nope, const void *q_rope, const void *kv_b, mla_dtype dt,
                         const mla_dims &d, int32_t B, const KvView &kv, const int32_t *sel,
                         const int32_t *nsel, int32_t sel_stride, int64_t max_keys, float sm_scale,
                         float *out, void *ws, size_t, hipStream_t s)
{
    mla_status st;
    if (use_mfma(d, dt, kv_b) && aligned16(q_rope) && aligned16(kv.lc) && aligned16(kv.rc)) {
        st = launch_absorb_mfma(q_nope, kv_b, d, B, ws, s);
        if (st) return st;
        return launch_attend_mfma(q_rope, kv_b, d, B, kv, sel, nsel, sel_stride, max_keys, sm_scale, out, ws, s);
    }
    st = launch_absorb_generic(q_nope, kv_b, dt, d, B, ws, s);
    if (st) return st;
    return launch_attend_generic(q_rope, kv_b, dt, d, B, kv, sel, nsel, sel_stride, max_keys, sm_scale, out, ws, s);
}

}  // namespace mla
